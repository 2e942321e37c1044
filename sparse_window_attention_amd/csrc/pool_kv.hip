// Mean pooling of K and V into the global memory tokens.
//
// Source: BASA discussion reply, paragraph on the method's four parts (a
// global memory made by pooling K/V, since shifted windows stay local);
// Scale-Free Attention abstract (summaries by mean pooling).  Cell g of the
// pooled grid averages the pt x py x px tokens of the unshifted grid it
// covers; memory tokens are stored [B, H, G, D] in raster order of the pooled
// grid.
//
// A streaming reduction bound by HBM bandwidth: each thread owns one 16-byte
// chunk of one memory token for both K and V and walks the tokens of its
// cell.  The lanes of a wave cover whole 16-byte-chunk rows of neighbouring
// cells, so every load instruction reads full token rows.  fp32 accumulation;
// bf16 results rounded to nearest even.
#include "basa_common.h"
#include "basa_internal.h"

namespace basa {

namespace {

constexpr int kThreads = 256;

template <bool BF16>
__global__ void __launch_bounds__(kThreads) pool_kernel(PoolParams p, int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= total) return;
  constexpr int EPC = BF16 ? 8 : 4;           // elements per 16B chunk
  const int cpr = p.head_dim / EPC;           // chunks per row
  const int chunk = (int)(gid % cpr);
  const int64_t rest = gid / cpr;
  const int g = (int)(rest % p.G);
  const int bh = (int)(rest / p.G);
  const int b = bh / p.heads, h = bh - b * p.heads;
  const int gx = g % p.Gx;
  const int gy = (g / p.Gx) % p.Gy;
  const int gt = g / (p.Gx * p.Gy);
  const int64_t base = (int64_t)b * p.stride_b + (int64_t)h * p.stride_h;
  const int esz = BF16 ? 2 : 4;
  const char* kb = reinterpret_cast<const char*>(p.k) + (base + chunk * EPC) * esz;
  const char* vb = reinterpret_cast<const char*>(p.v) + (base + chunk * EPC) * esz;
  const int64_t tokb = (int64_t)p.stride_tok * esz;

  float ks[8] = {0, 0, 0, 0, 0, 0, 0, 0}, vs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int a = 0; a < p.pt; ++a) {
    for (int c = 0; c < p.py; ++c) {
      const int64_t row = ((int64_t)(gt * p.pt + a) * p.Hg + (gy * p.py + c)) * p.Wg + gx * p.px;
      const char* kr = kb + row * tokb;
      const char* vr = vb + row * tokb;
      int x = 0;
      for (; x + 4 <= p.px; x += 4) {
        u32x4 kk[4], vv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kk[u] = *reinterpret_cast<const u32x4*>(kr + (x + u) * tokb);
          vv[u] = *reinterpret_cast<const u32x4*>(vr + (x + u) * tokb);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if constexpr (BF16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ks[2 * e] += bf16_lo(kk[u][e]);
              ks[2 * e + 1] += bf16_hi(kk[u][e]);
              vs[2 * e] += bf16_lo(vv[u][e]);
              vs[2 * e + 1] += bf16_hi(vv[u][e]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ks[e] += __uint_as_float(kk[u][e]);
              vs[e] += __uint_as_float(vv[u][e]);
            }
          }
        }
      }
      for (; x < p.px; ++x) {
        const u32x4 kk = *reinterpret_cast<const u32x4*>(kr + x * tokb);
        const u32x4 vv = *reinterpret_cast<const u32x4*>(vr + x * tokb);
        if constexpr (BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ks[2 * e] += bf16_lo(kk[e]);
            ks[2 * e + 1] += bf16_hi(kk[e]);
            vs[2 * e] += bf16_lo(vv[e]);
            vs[2 * e + 1] += bf16_hi(vv[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ks[e] += __uint_as_float(kk[e]);
            vs[e] += __uint_as_float(vv[e]);
          }
        }
      }
    }
  }
  const float cnt = (float)(p.pt * p.py * p.px);
  const int64_t obase = ((int64_t)bh * p.G + g) * p.head_dim + chunk * EPC;
  if constexpr (BF16) {
    u32x4 ko, vo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ko[e] = pack_bf16x2(ks[2 * e] / cnt, ks[2 * e + 1] / cnt);
      vo[e] = pack_bf16x2(vs[2 * e] / cnt, vs[2 * e + 1] / cnt);
    }
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.kmem) + obase) = ko;
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.vmem) + obase) = vo;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.kmem) + obase) =
        f32x4{ks[0] / cnt, ks[1] / cnt, ks[2] / cnt, ks[3] / cnt};
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.vmem) + obase) =
        f32x4{vs[0] / cnt, vs[1] / cnt, vs[2] / cnt, vs[3] / cnt};
  }
}

}  // namespace

int launch_pool(const PoolParams& p, int dtype, hipStream_t stream) {
  const bool bf16 = dtype == BASA_BF16;
  const int64_t total = (int64_t)p.batch_heads * p.G * (p.head_dim / (bf16 ? 8 : 4));
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > INT32_MAX) return BASA_ERR_UNSUPPORTED;
  if (bf16)
    hipLaunchKernelGGL(pool_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, total);
  else
    hipLaunchKernelGGL(pool_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, total);
  return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

}  // namespace basa
