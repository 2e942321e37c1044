// bf16 window / full attention on gfx950 matrix cores.
//
// One workgroup computes QT query rows of one window of one (batch, head).
// The window's keys and the pooled memory keys form one virtual key sequence
// [window keys; memory keys] of length L = m + G, streamed through LDS in
// tiles of KT keys.  Per tile and wave:
//   S^T = K Q^T        (32x32x16 bf16 MFMA, keys x queries, fp32 accumulate)
//   online softmax     (fp32, base 2; the row max needs one lane swap since a
//                       lane holds 16 keys of one query)
//   O^T += V^T P^T     (32x32x16 bf16 MFMA, P rounded to bf16)
// Computing S transposed puts every query in one lane pair, so the softmax
// reductions stay in registers, and the fp32 scores already sit in the
// operand layout the P V product needs (no shuffles).
//
// The cyclic shift and the window gather are address arithmetic: a table of
// the window's raster offsets is built in LDS once per workgroup and every
// Q/K/V/O row is addressed through it (BASA forum summary, "The BASA
// Method": shift, partition, attend, shift back -- here without any copy).
// Memory keys (BASA discussion reply, the four parts of the method: a global
// memory of pooled K/V) are plain rows of the [B,H,G,D] memory tensors.
#include "basa_common.h"
#include "basa_internal.h"

namespace basa {

namespace {

constexpr int kWaves = 4;
constexpr int kQPW = 32;              // query rows per wave
constexpr int kQT = kWaves * kQPW;    // query rows per workgroup
constexpr int kKT = 64;               // keys per tile
constexpr int kThreads = kWaves * 64;
constexpr float kRescaleSlack = 8.0f; // log2 units the stale max may lag

template <int D>
struct Tiles {
  static constexpr int KS = D + 8;    // K tile row stride (bf16), 16B aligned, skewed banks
  static constexpr int VS = kKT + 8;  // transposed V tile row stride (bf16)
  static constexpr int kBytes = kKT * KS * 2;
  static constexpr int vBytes = D * VS * 2;
  static constexpr int bufBytes = kBytes + vBytes;
  static constexpr int CPR = D / 8;               // 16B chunks per row
  static constexpr int RPP = kThreads / CPR;      // K rows per load pass
  static constexpr int KPASS = kKT / RPP;         // K load passes per tile
  static constexpr int KPT = kKT * D / (kThreads * 8);  // V keys per thread
};

// Slot of key `key` (0..kKT-1) in the transposed V tile: within each group of
// 16 keys, the order matches how the S^T accumulator registers map onto the
// k index of the P V product's operand.
__device__ __forceinline__ int vslot(int key) {
  const int a = key >> 2, i = key & 3;
  return (a >> 2) * 16 + (a & 1) * 8 + ((a >> 1) & 1) * 4 + i;
}

template <int D, bool FULL>
__global__ void __launch_bounds__(kThreads, 2) attn_bf16_kernel(AttnParams p) {
  using TL = Tiles<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* sOff = reinterpret_cast<int32_t*>(smem + 2 * TL::bufBytes);

  // ---- work unit (XCD-aware: consecutive units run on one XCD's L2)
  const int xcd = blockIdx.x & 7;
  const int kidx = blockIdx.x >> 3;
  const int unit = xcd * p.units_per_xcd + kidx;
  if (kidx >= p.units_per_xcd || unit >= p.units) return;
  const int qt = unit % p.nQT;
  const int rest = unit / p.nQT;
  const int win = rest % p.nW;
  const int bh = rest / p.nW;
  const int b = bh / p.heads, h = bh - b * p.heads;
  const int64_t base = (int64_t)b * p.stride_b + (int64_t)h * p.stride_h;
  const uint16_t* __restrict__ gq = p.q + base;
  const uint16_t* __restrict__ gk = p.k + base;
  const uint16_t* __restrict__ gv = p.v + base;
  uint16_t* __restrict__ go = p.out + base;
  const uint16_t* __restrict__ gkm = p.kmem + (int64_t)bh * p.G * D;
  const uint16_t* __restrict__ gvm = p.vmem + (int64_t)bh * p.G * D;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int m = p.m;
  const int L = m + p.G;
  const int stok = p.stride_tok;

  if (!FULL) {
    for (int r = tid; r < m; r += kThreads) sOff[r] = window_token(p.geo, win, r) * stok;
    __syncthreads();
  }
  auto tokoff = [&](int r) -> int32_t { return FULL ? r * stok : sOff[r]; };

  // ---- Q rows of this wave, kept in registers as the B operand of K Q^T:
  // step s, lane half hf holds d = hf*D/2 + 8s .. +7
  constexpr int QS = D / 16;
  u32x4 qreg[QS];
  const int qrow = qt * kQT + wave * kQPW + l32;
  const bool qvalid = qrow < m;
  const int32_t qoff = qvalid ? tokoff(qrow) : 0;
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    qreg[s] = qvalid ? *reinterpret_cast<const u32x4*>(gq + qoff + hf * (D / 2) + s * 8)
                     : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- tile loader (global -> registers -> LDS)
  const int kc = tid % TL::CPR;                // K: chunk within a row
  const int kr0 = tid / TL::CPR;               // K: first row
  const int va = tid % (kKT / TL::KPT);        // V: key group
  const int vc = tid / (kKT / TL::KPT);        // V: 8-wide d chunk
  u32x4 kreg[TL::KPASS];
  u32x4 vreg[TL::KPT];

  auto row_src = [&](int key, const uint16_t* g, const uint16_t* gm) -> const uint16_t* {
    if (key < m) return g + tokoff(key);
    if (key < L) return gm + (int64_t)(key - m) * D;
    return nullptr;
  };
  auto load_tile = [&](int t) {
    const int k0 = t * kKT;
#pragma unroll
    for (int i = 0; i < TL::KPASS; ++i) {
      const uint16_t* src = row_src(k0 + kr0 + i * TL::RPP, gk, gkm);
      kreg[i] = src ? *reinterpret_cast<const u32x4*>(src + kc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < TL::KPT; ++i) {
      const uint16_t* src = row_src(k0 + va * TL::KPT + i, gv, gvm);
      vreg[i] = src ? *reinterpret_cast<const u32x4*>(src + vc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* sK = reinterpret_cast<uint16_t*>(smem + buf * TL::bufBytes);
    uint16_t* sV = reinterpret_cast<uint16_t*>(smem + buf * TL::bufBytes + TL::kBytes);
#pragma unroll
    for (int i = 0; i < TL::KPASS; ++i)
      *reinterpret_cast<u32x4*>(sK + (kr0 + i * TL::RPP) * TL::KS + kc * 8) = kreg[i];
    // transpose: for each of the 8 d of this chunk, the KPT keys side by side
    const int slot = vslot(va * TL::KPT);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (TL::KPT == 4) {
        const uint32_t lo0 = (vreg[0][e] & 0xffffu) | (vreg[1][e] << 16);
        const uint32_t lo1 = (vreg[2][e] & 0xffffu) | (vreg[3][e] << 16);
        const uint32_t hi0 = (vreg[0][e] >> 16) | (vreg[1][e] & 0xffff0000u);
        const uint32_t hi1 = (vreg[2][e] >> 16) | (vreg[3][e] & 0xffff0000u);
        *reinterpret_cast<u32x2*>(sV + (vc * 8 + 2 * e) * TL::VS + slot) = u32x2{lo0, lo1};
        *reinterpret_cast<u32x2*>(sV + (vc * 8 + 2 * e + 1) * TL::VS + slot) = u32x2{hi0, hi1};
      } else {
        const uint32_t lo = (vreg[0][e] & 0xffffu) | (vreg[1][e] << 16);
        const uint32_t hi = (vreg[0][e] >> 16) | (vreg[1][e] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(sV + (vc * 8 + 2 * e) * TL::VS + slot) = lo;
        *reinterpret_cast<uint32_t*>(sV + (vc * 8 + 2 * e + 1) * TL::VS + slot) = hi;
      }
    }
  };

  // ---- online softmax state (one query per lane pair)
  constexpr int DB = D / 32;
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
  float m_used = -INFINITY;   // running max in log2 units (may lag by < slack)
  float l_part = 0.0f;        // this lane's share of the row sum
  const float c1 = p.c1;
  const bool has_bias = p.mem_bias_raw != 0.0f;

  const int nkt = (L + kKT - 1) / kKT;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < nkt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nkt) load_tile(t + 1);
    const uint16_t* sK = reinterpret_cast<const uint16_t*>(smem + buf * TL::bufBytes);
    const uint16_t* sV = reinterpret_cast<const uint16_t*>(smem + buf * TL::bufBytes + TL::kBytes);

    // S^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
      for (int ss = 0; ss < QS; ++ss) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(
            sK + (kb * 32 + l32) * TL::KS + hf * (D / 2) + ss * 8);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qreg[ss]), s[kb], 0, 0, 0);
      }
    }
    // padding keys -> -inf; memory keys get the logit bias
    const int k0 = t * kKT;
    if (k0 + kKT > L || (has_bias && k0 + kKT > m)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= L) s[kb][r] = -INFINITY;
          else if (key >= m) s[kb][r] += p.mem_bias_raw;
        }
    }
    // row max over the tile (16 keys in registers x 2 blocks, then the lane pair)
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float m_new = mx * c1;
    const bool need = m_new > m_used + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_tgt = need ? m_new : m_used;
      const float alpha = exp2f(m_used - m_tgt);
      m_used = m_tgt;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
    }
    // P = exp2(S*c1 - m), row sum, bf16 operands of the P V product
    u32x4 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * u + j], c1, -m_used));
          l_part += e[j];
        }
        pb[2 * kb + u] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                               pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
      }
    }
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(
            sV + (db * 32 + l32) * TL::VS + sl * 16 + hf * 8);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pb[sl]), acc[db], 0, 0, 0);
      }
    }
    if (t + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and scatter back to raster order
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part),
                                                     __float_as_uint(l_part), false, false);
    const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const float inv = 1.0f / l;
    if (qvalid) {
      uint16_t* dst = go + qoff;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * hf;
          const u32x2 w{pack_bf16x2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv),
                        pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(dst + d) = w;
        }
    }
  }
}

template <int D, bool FULL>
int launch(const AttnParams& p0, hipStream_t stream) {
  using TL = Tiles<D>;
  AttnParams p = p0;
  p.nQT = (p.m + kQT - 1) / kQT;
  const int64_t units = (int64_t)p.batch_heads * p.nW * p.nQT;
  if (units > (int64_t)INT32_MAX / 2) return BASA_ERR_UNSUPPORTED;
  p.units = (int32_t)units;
  p.units_per_xcd = (p.units + 7) / 8;
  const size_t lds = 2 * TL::bufBytes + (FULL ? 0 : (size_t)p.m * 4);
  if (lds > 160 * 1024) return BASA_ERR_UNSUPPORTED;
  static bool attr_set = false;  // benign race: the call is idempotent
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16_kernel<D, FULL>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return BASA_ERR_HIP;
    attr_set = true;
  }
  const dim3 grid((unsigned)(8 * p.units_per_xcd));
  hipLaunchKernelGGL((attn_bf16_kernel<D, FULL>), grid, dim3(kThreads), lds, stream, p);
  return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

}  // namespace

int launch_attn_bf16(const AttnParams& p, bool full, hipStream_t stream) {
  if (p.head_dim == 128) return full ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  if (p.head_dim == 64) return full ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return BASA_ERR_UNSUPPORTED;
}

}  // namespace basa
