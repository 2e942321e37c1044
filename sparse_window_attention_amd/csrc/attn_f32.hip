// fp32 window / full attention (vector ALU, no down-conversion anywhere).
//
// The same virtual key sequence [window keys; memory keys] and the same LDS
// table of shifted-window raster offsets as the bf16 kernel; each thread owns
// one query row, keeps q and its output accumulator in registers, and walks
// the key tiles staged in LDS (every thread reads the same key row, an LDS
// broadcast).  Softmax in natural-log units with expf, exact rescale per
// group of 2 (D = 128) or 8 (D = 64) keys.  Built for accuracy on small fp32
// workloads, not for speed.
#include "basa_common.h"
#include "basa_internal.h"

namespace basa {

namespace {

constexpr int kThreads = 128;
constexpr int kKT = 32;   // keys per LDS tile
// keys scored and folded in at a time: q and the accumulator already hold
// 2*D registers per thread
template <int D>
constexpr int kSub = D >= 128 ? 2 : 8;

template <int D, bool FULL>
__global__ void __launch_bounds__(kThreads) attn_f32_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* sK = reinterpret_cast<float*>(smem);
  float* sV = sK + kKT * D;
  int32_t* sOff = reinterpret_cast<int32_t*>(sV + kKT * D);

  const int unit = blockIdx.x;
  if (unit >= p.units) return;
  const int qt = unit % p.nQT;
  const int rest = unit / p.nQT;
  const int win = rest % p.nW;
  const int bh = rest / p.nW;
  const int b = bh / p.heads, h = bh - b * p.heads;
  const int64_t base = (int64_t)b * p.stride_b + (int64_t)h * p.stride_h;
  const float* __restrict__ gq = reinterpret_cast<const float*>(p.q) + base;
  const int64_t kvbase = FULL ? (int64_t)b * p.kv_stride_b + (int64_t)h * p.kv_stride_h : base;
  const float* __restrict__ gk = reinterpret_cast<const float*>(p.k) + kvbase;
  const float* __restrict__ gv = reinterpret_cast<const float*>(p.v) + kvbase;
  float* __restrict__ go = reinterpret_cast<float*>(p.out) + base;
  const float* __restrict__ gkm = reinterpret_cast<const float*>(p.kmem) + (int64_t)bh * p.G * D;
  const float* __restrict__ gvm = reinterpret_cast<const float*>(p.vmem) + (int64_t)bh * p.G * D;

  const int tid = threadIdx.x;
  const int m = p.m;
  const int L = FULL ? p.n_kv : m + p.G;
  const int nwin = FULL ? L : m;  // keys read through the token map
  const int stok = p.stride_tok;
  if (!FULL) {
    for (int r = tid; r < m; r += kThreads) sOff[r] = slot_token(p, win, r) * stok;
    __syncthreads();
  }
  auto tokoff = [&](int r) -> int32_t { return FULL ? r * stok : sOff[r]; };

  const int qrow = qt * kThreads + tid;
  const bool qvalid = qrow < m;
  const int32_t qoff = qvalid ? tokoff(qrow) : 0;
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const f32x4 x = qvalid ? *reinterpret_cast<const f32x4*>(gq + qoff + d) : f32x4{0, 0, 0, 0};
    q[d] = x[0]; q[d + 1] = x[1]; q[d + 2] = x[2]; q[d + 3] = x[3];
    acc[d] = acc[d + 1] = acc[d + 2] = acc[d + 3] = 0.0f;
  }
  float mrun = -INFINITY, lsum = 0.0f;
  const float scale = p.scale;

  constexpr int C4 = D / 4;  // 16B chunks per row
  for (int k0 = 0; k0 < L; k0 += kKT) {
    __syncthreads();  // previous tile fully consumed
    for (int i = tid; i < kKT * C4; i += kThreads) {
      const int r = i / C4, c = i % C4;
      const int key = k0 + r;
      f32x4 kx{0, 0, 0, 0}, vx{0, 0, 0, 0};
      if (key < nwin) {
        const int32_t o = tokoff(key);
        kx = *reinterpret_cast<const f32x4*>(gk + o + 4 * c);
        vx = *reinterpret_cast<const f32x4*>(gv + o + 4 * c);
      } else if (key < L) {
        const int64_t o = (int64_t)(key - m) * D;
        kx = *reinterpret_cast<const f32x4*>(gkm + o + 4 * c);
        vx = *reinterpret_cast<const f32x4*>(gvm + o + 4 * c);
      }
      *reinterpret_cast<f32x4*>(sK + r * D + 4 * c) = kx;
      *reinterpret_cast<f32x4*>(sV + r * D + 4 * c) = vx;
    }
    __syncthreads();
    const int nk = min(kKT, L - k0);
    // groups of kSub keys: scores, the exact rescale of the running sum and
    // accumulator to the new max, then P V; a group of padding keys only is
    // skipped (keys past L come last, so one of them ends the tile)
#pragma unroll 1
    for (int j0 = 0; j0 < nk; j0 += kSub<D>) {
      float s[kSub<D>];
      float mt = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < kSub<D>; ++jj) {
        const int j = j0 + jj;
        // four independent partial sums of the dot product
        float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int d = 0; d < D; d += 4) {
          const f32x4 kv = *reinterpret_cast<const f32x4*>(sK + j * D + d);
#pragma unroll
          for (int e = 0; e < 4; ++e) d4[e] = __builtin_fmaf(q[d + e], kv[e], d4[e]);
        }
        float x = ((d4[0] + d4[1]) + (d4[2] + d4[3])) * scale;
        if (k0 + j >= nwin) x += p.mem_bias;
        s[jj] = (j < nk) ? x : -INFINITY;
        mt = fmaxf(mt, s[jj]);
      }
      const float mnew = fmaxf(mrun, mt);   // finite: the group holds a valid key
      const float alpha = expf(mrun - mnew);
      mrun = mnew;
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
      for (int jj = 0; jj < kSub<D>; ++jj) {
        const float pj = expf(s[jj] - mnew);
        lsum += pj;
        const float* vr = sV + (j0 + jj) * D;
#pragma unroll
        for (int d = 0; d < D; d += 4) {
          const f32x4 vv = *reinterpret_cast<const f32x4*>(vr + d);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[d + e] = __builtin_fmaf(pj, vv[e], acc[d + e]);
        }
      }
    }
  }
  if (qvalid) {
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int d = 0; d < D; d += 4)
      *reinterpret_cast<f32x4*>(go + qoff + d) =
          f32x4{acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv};
  }
}

template <int D, bool FULL>
int launch(const AttnParams& p0, hipStream_t stream) {
  AttnParams p = p0;
  p.nQT = (p.m + kThreads - 1) / kThreads;
  const int64_t units = (int64_t)p.batch_heads * p.nW * p.nQT;
  if (units > (int64_t)INT32_MAX) return BASA_ERR_UNSUPPORTED;
  p.units = (int32_t)units;
  const size_t lds = 2 * kKT * D * sizeof(float) + (FULL ? 0 : (size_t)p.m * 4);
  if (lds > 160 * 1024) return BASA_ERR_UNSUPPORTED;
  static bool attr_set[64] = {};  // per device; benign race: the call is idempotent
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BASA_ERR_HIP;
  if (dev < 0 || dev >= 64 || !attr_set[dev]) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_f32_kernel<D, FULL>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return BASA_ERR_HIP;
    if (dev >= 0 && dev < 64) attr_set[dev] = true;
  }
  hipLaunchKernelGGL((attn_f32_kernel<D, FULL>), dim3((unsigned)p.units), dim3(kThreads), lds,
                     stream, p);
  return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

}  // namespace

int launch_attn_f32(const AttnParams& p, bool full, hipStream_t stream) {
  if (p.head_dim == 128) return full ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  if (p.head_dim == 64) return full ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return BASA_ERR_UNSUPPORTED;
}

}  // namespace basa
