// Mean pooling of K and V into the global memory tokens.
//
// Source: BASA discussion reply, paragraph on the method's four parts (a
// global memory made by pooling K/V, since shifted windows stay local);
// Scale-Free Attention abstract (summaries by mean pooling).  Cell g of the
// pooled grid averages the pt x py x px tokens of the unshifted grid it
// covers; memory tokens are stored [B, H, G, D] in raster order of the pooled
// grid.
//
// A streaming reduction bound by HBM bandwidth.  One wave per (batch, head,
// cell): the CPR lanes of a lane group hold the 16-byte chunks of one token
// row, and the 64 / CPR lane groups take interleaved tokens of each grid row
// of the cell, so every load instruction reads consecutive tokens.  Rows and
// frames are walked by pointer steps, with no integer division per token.
// Each lane accumulates its tokens of K and V, then the groups' partial sums
// are added with lane exchanges.  fp32 accumulation; bf16 results rounded to
// nearest even.
#include "basa_common.h"
#include "basa_internal.h"

namespace basa {

namespace {

constexpr int kWavesPerBlock = 4;

template <bool BF16>
__device__ __forceinline__ void accumulate(float (&acc)[8], const u32x4& x) {
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(x[e]);
      acc[2 * e + 1] += bf16_hi(x[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(x[e]);
  }
}

template <bool BF16, int CPR>
__global__ void __launch_bounds__(kWavesPerBlock * 64) pool_kernel(PoolParams p, int64_t cells) {
  constexpr int EPC = BF16 ? 8 : 4;   // elements per 16B chunk
  constexpr int NG = 64 / CPR;        // lane groups (row splits) per wave
  constexpr int NA = EPC;             // live accumulators per tensor
  const int64_t cell = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (cell >= cells) return;          // whole wave exits together
  const int lane = threadIdx.x & 63;
  const int chunk = lane % CPR;
  const int grp = lane / CPR;
  const int g = (int)(cell % p.G);
  const int bh = (int)(cell / p.G);
  const int b = bh / p.heads, h = bh - b * p.heads;
  const int gx = g % p.Gx;
  const int gy = (g / p.Gx) % p.Gy;
  const int gt = g / (p.Gx * p.Gy);
  const int64_t base = (int64_t)b * p.stride_b + (int64_t)h * p.stride_h;
  constexpr int ES = BF16 ? 2 : 4;
  const char* kb = reinterpret_cast<const char*>(p.k) + (base + chunk * EPC) * ES;
  const char* vb = reinterpret_cast<const char*>(p.v) + (base + chunk * EPC) * ES;
  const int64_t tokb = (int64_t)p.stride_tok * ES;

  float ks[8], vs[8];  // the first NA are live
#pragma unroll
  for (int e = 0; e < 8; ++e) ks[e] = vs[e] = 0.0f;
  // Lane group grp takes the tokens x = grp, grp + NG, ... of every grid row
  // of the cell, so one load instruction reads NG consecutive tokens of one
  // row.  Rows and frames advance by pointer steps: no division per token.
  const int64_t rowstep = (int64_t)p.Wg * tokb;           // next grid row
  const int64_t framestep = (int64_t)p.Hg * p.Wg * tokb;  // next frame
  const int64_t cell0 = ((int64_t)(gt * p.pt) * p.Hg + gy * p.py) * p.Wg + gx * p.px;
  const char* kf = kb + cell0 * tokb;
  const char* vf = vb + cell0 * tokb;
  for (int a = 0; a < p.pt; ++a, kf += framestep, vf += framestep) {
    const char* kr = kf;
    const char* vr = vf;
    for (int c = 0; c < p.py; ++c, kr += rowstep, vr += rowstep) {
      int x = grp;
      for (; x + NG < p.px; x += 2 * NG) {
        const u32x4 k0 = *reinterpret_cast<const u32x4*>(kr + x * tokb);
        const u32x4 v0 = *reinterpret_cast<const u32x4*>(vr + x * tokb);
        const u32x4 k1 = *reinterpret_cast<const u32x4*>(kr + (x + NG) * tokb);
        const u32x4 v1 = *reinterpret_cast<const u32x4*>(vr + (x + NG) * tokb);
        accumulate<BF16>(ks, k0);
        accumulate<BF16>(vs, v0);
        accumulate<BF16>(ks, k1);
        accumulate<BF16>(vs, v1);
      }
      if (x < p.px) {
        accumulate<BF16>(ks, *reinterpret_cast<const u32x4*>(kr + x * tokb));
        accumulate<BF16>(vs, *reinterpret_cast<const u32x4*>(vr + x * tokb));
      }
    }
  }
  // add the lane groups' partial sums: groups differ in the lane bits above CPR
#pragma unroll
  for (int off = CPR; off < 64; off *= 2) {
#pragma unroll
    for (int e = 0; e < NA; ++e) {
      ks[e] += __shfl_xor(ks[e], off);
      vs[e] += __shfl_xor(vs[e], off);
    }
  }
  if (grp != 0) return;
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

template <bool BF16, int CPR>
int launch_cpr(const PoolParams& p, hipStream_t stream) {
  const int64_t cells = (int64_t)p.batch_heads * p.G;
  const int64_t blocks = (cells + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > INT32_MAX) return BASA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((pool_kernel<BF16, CPR>), dim3((unsigned)blocks), dim3(kWavesPerBlock * 64), 0,
                     stream, p, cells);
  return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

// Row gather for a shared key region (HilbertA catalogue record, abstract: a
// small central region shared by every tile): one thread per 16-byte chunk.
__global__ void __launch_bounds__(256) gather_kernel(GatherParams p, int cpr, int es) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.batch_heads * p.n_idx * cpr;
  if (i >= total) return;
  const int c = (int)(i % cpr);
  const int64_t row = i / cpr;                  // bh * n_idx + j
  const int bh = (int)(row / p.n_idx);
  const int j = (int)(row - (int64_t)bh * p.n_idx);
  int t = p.idx[j];
  t = t < 0 ? 0 : (t >= p.n ? p.n - 1 : t);
  const int b = bh / p.heads, h = bh - b * p.heads;
  const int64_t src = ((int64_t)b * p.stride_b + (int64_t)h * p.stride_h + (int64_t)t * p.stride_tok) * es + c * 16;
  const int64_t dst = row * (int64_t)p.head_dim * es + c * 16;
  *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(p.kout) + dst) =
      *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(p.k) + src);
  *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(p.vout) + dst) =
      *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(p.v) + src);
}

}  // namespace

int launch_gather(const GatherParams& p, int dtype, hipStream_t stream) {
  const int es = dtype == BASA_BF16 ? 2 : 4;
  const int cpr = p.head_dim * es / 16;
  const int64_t total = (int64_t)p.batch_heads * p.n_idx * cpr;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > INT32_MAX) return BASA_ERR_UNSUPPORTED;
  if (blocks == 0) return BASA_OK;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, cpr, es);
  return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

int launch_pool(const PoolParams& p, int dtype, hipStream_t stream) {
  const bool bf16 = dtype == BASA_BF16;
  const int cpr = p.head_dim * (bf16 ? 2 : 4) / 16;  // 16B chunks per token row
  if (bf16) {
    if (cpr == 16) return launch_cpr<true, 16>(p, stream);
    if (cpr == 8) return launch_cpr<true, 8>(p, stream);
  } else {
    if (cpr == 32) return launch_cpr<false, 32>(p, stream);
    if (cpr == 16) return launch_cpr<false, 16>(p, stream);
  }
  return BASA_ERR_UNSUPPORTED;
}

}  // namespace basa
