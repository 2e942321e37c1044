// bf16 window / full attention on gfx950 matrix cores.
//
// One workgroup computes kQT query rows of one window of one (batch, head).
// The window's keys and the pooled memory keys form one virtual key sequence
// [window keys; memory keys] of length L = m + G, streamed through LDS in
// tiles of kKT keys.  Per tile and wave:
//   S^T = K Q^T        (32x32x16 bf16 MFMA, keys x queries, fp32 accumulate)
//   online softmax     (fp32, base 2; the row max needs one lane swap since a
//                       lane holds 16 keys of one query)
//   O^T += V^T P^T     (32x32x16 bf16 MFMA, P rounded to bf16)
// Computing S transposed puts every query in one lane pair, so the softmax
// reductions stay in registers, and the fp32 scores already sit in the
// operand layout the P V product needs (no shuffles).
//
// The loop is software-pipelined inside each wave: while the exponentials of
// tile t are computed on the vector ALU, the matrix core already runs
// K(t+1) Q^T, and the row max of tile t+1 overlaps the P V product of tile
// t.  K runs one tile ahead of V through two LDS buffers each.
//
// The cyclic shift and the window gather are address arithmetic: a table of
// the window's raster offsets is built in LDS once per workgroup and every
// Q/K/V/O row is addressed through it (BASA forum summary, "The BASA
// Method": shift, partition, attend, shift back -- here without any copy).
// Memory keys (BASA discussion reply, the four parts of the method: a global
// memory of pooled K/V) are plain rows of the [B,H,G,D] memory tensors.
#include <type_traits>

#include "basa_common.h"
#include "basa_internal.h"

namespace basa {

namespace {

constexpr int kQPW = 32;              // query rows per wave
constexpr int kKT = 64;               // keys per tile
constexpr float kRescaleSlack = 8.0f; // log2 units the stale max may lag

template <int D, int NW>
struct Tiles {
  static constexpr int kThreads = NW * 64;
  static constexpr int kQT = NW * kQPW;           // query rows per workgroup
  static constexpr int KS = D + 8;    // K tile row stride (bf16), 16B aligned, skewed banks
  static constexpr int VS = kKT + 8;  // transposed V tile row stride (bf16)
  static constexpr int kBytes = kKT * KS * 2;
  static constexpr int vBytes = D * VS * 2;
  static constexpr int ldsBytes = 2 * kBytes + 2 * vBytes;
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

template <bool B>
using bool_c = std::integral_constant<bool, B>;

template <int D, bool FULL, int NW>
__global__ void __launch_bounds__(NW * 64, 8 / NW) attn_bf16_kernel(AttnParams p) {
  using TL = Tiles<D, NW>;
  constexpr int kThreads = TL::kThreads;
  constexpr int kQT = TL::kQT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* sOff = reinterpret_cast<int32_t*>(smem + TL::ldsBytes);
  auto sK = [&](int buf) __attribute__((always_inline)) { return reinterpret_cast<uint16_t*>(smem + buf * TL::kBytes); };
  auto sV = [&](int buf) __attribute__((always_inline)) {
    return reinterpret_cast<uint16_t*>(smem + 2 * TL::kBytes + buf * TL::vBytes);
  };

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

  // ---- Q rows of this wave, kept in registers as the B operand of K Q^T:
  // step s, lane half hf holds d = hf*D/2 + 8s .. +7
  constexpr int QS = D / 16;
  u32x4 qreg[QS];
  const int qrow = qt * kQT + wave * kQPW + l32;
  const bool qvalid = qrow < m;
  const int32_t qoff = qvalid ? (FULL ? __mul24(qrow, stok) : sOff[qrow]) : 0;
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    qreg[s] = qvalid ? *reinterpret_cast<const u32x4*>(gq + qoff + hf * (D / 2) + s * 8)
                     : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- tile loader (global -> registers -> LDS).  Key indices past the end
  // are clamped to the last key: those rows load valid data that the score
  // mask removes, so the loader has no branches.
  const int kc = tid % TL::CPR;                // K: chunk within a row
  const int kr0 = tid / TL::CPR;               // K: first row
  const int va = tid % (kKT / TL::KPT);        // V: key group
  const int vc = tid / (kKT / TL::KPT);        // V: 8-wide d chunk
  u32x4 kreg[TL::KPASS];
  u32x4 vreg[TL::KPT];
  const int Lm1 = L - 1;

  // Keys stay below 2^24 and token offsets below 2^31 (checked on the host),
  // so a full-rate 24-bit multiply forms the row offsets.
  auto row_ptr = [&](int key, const uint16_t* g, const uint16_t* gm) __attribute__((always_inline)) -> const uint16_t* {
    key = min(key, Lm1);
    if constexpr (FULL) {
      return g + __mul24(key, stok);
    } else {
      const bool inwin = key < m;
      const int32_t off = sOff[inwin ? key : 0];
      const int64_t moff = (int64_t)__mul24(inwin ? 0 : key - m, D);
      return inwin ? g + off : gm + moff;
    }
  };
  auto load_k = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TL::KPASS; ++i)
      kreg[i] = *reinterpret_cast<const u32x4*>(row_ptr(t * kKT + kr0 + i * TL::RPP, gk, gkm) + kc * 8);
  };
  auto load_v = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TL::KPT; ++i)
      vreg[i] = *reinterpret_cast<const u32x4*>(row_ptr(t * kKT + va * TL::KPT + i, gv, gvm) + vc * 8);
  };
  auto store_k = [&](int buf) __attribute__((always_inline)) {
    uint16_t* dst = sK(buf);
#pragma unroll
    for (int i = 0; i < TL::KPASS; ++i)
      *reinterpret_cast<u32x4*>(dst + (kr0 + i * TL::RPP) * TL::KS + kc * 8) = kreg[i];
  };
  auto store_v = [&](int buf) __attribute__((always_inline)) {
    // transpose: for each of the 8 d of this chunk, the KPT keys side by side
    uint16_t* dst = sV(buf);
    const int slot = vslot(va * TL::KPT);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (TL::KPT == 4) {
        const uint32_t lo0 = (vreg[0][e] & 0xffffu) | (vreg[1][e] << 16);
        const uint32_t lo1 = (vreg[2][e] & 0xffffu) | (vreg[3][e] << 16);
        const uint32_t hi0 = (vreg[0][e] >> 16) | (vreg[1][e] & 0xffff0000u);
        const uint32_t hi1 = (vreg[2][e] >> 16) | (vreg[3][e] & 0xffff0000u);
        *reinterpret_cast<u32x2*>(dst + (vc * 8 + 2 * e) * TL::VS + slot) = u32x2{lo0, lo1};
        *reinterpret_cast<u32x2*>(dst + (vc * 8 + 2 * e + 1) * TL::VS + slot) = u32x2{hi0, hi1};
      } else if constexpr (TL::KPT == 2) {
        const uint32_t lo = (vreg[0][e] & 0xffffu) | (vreg[1][e] << 16);
        const uint32_t hi = (vreg[0][e] >> 16) | (vreg[1][e] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(dst + (vc * 8 + 2 * e) * TL::VS + slot) = lo;
        *reinterpret_cast<uint32_t*>(dst + (vc * 8 + 2 * e + 1) * TL::VS + slot) = hi;
      } else {
        dst[(vc * 8 + 2 * e) * TL::VS + slot] = (uint16_t)(vreg[0][e] & 0xffffu);
        dst[(vc * 8 + 2 * e + 1) * TL::VS + slot] = (uint16_t)(vreg[0][e] >> 16);
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
  float l_part = 0.0f;        // this lane's share of the row sum (two partial sums)
  float l_part1 = 0.0f;
  const float c1 = p.c1;
  const float bias = p.mem_bias_raw;
  const f32x16 zero16 = {};

  auto compute_s = [&](const uint16_t* kt, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ss = 0; ss < QS; ++ss) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(
            kt + (kb * 32 + l32) * TL::KS + hf * (D / 2) + ss * 8);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qreg[ss]),
            ss == 0 ? zero16 : s[kb], 0, 0, 0);
      }
    }
  };
  // padding keys -> -inf; memory keys get the logit bias (selects, no branches)
  auto mask_s = [&](f32x16 (&s)[2], int k0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        const float x = s[kb][r] + (key >= m ? bias : 0.0f);
        s[kb][r] = key < L ? x : -INFINITY;
      }
  };
  auto rowmax = [&](const f32x16 (&s)[2]) -> float {
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };
  // lagging max: rescale O only when the max has grown by more than the slack
  auto update_max = [&](float mx) __attribute__((always_inline)) {
    const float m_new = mx * c1;
    const bool need = m_new > m_used + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_tgt = need ? m_new : m_used;
      const float alpha = exp2f(m_used - m_tgt);
      m_used = m_tgt;
      l_part *= alpha;
      l_part1 *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
    }
  };
  // P = exp2(S*c1 - m): row sum (two partial sums) and the bf16 operands of
  // the P V product
  auto make_p = [&](const f32x16 (&s)[2], u32x4 (&pb)[4]) {
    const float nm = -m_used;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * u + j], c1, nm));
        u32x4 w{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
        float& lp = u ? l_part1 : l_part;
        lp += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
        pb[2 * kb + u] = w;
      }
    }
  };
  // O^T += V^T P^T
  auto pv = [&](const uint16_t* vt, const u32x4 (&pb)[4]) {
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(
            vt + (db * 32 + l32) * TL::VS + sl * 16 + hf * 8);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pb[sl]), acc[db], 0, 0, 0);
      }
    }
  };

  // first tile whose scores need the mask (memory-key bias or padding)
  const int nkt = (L + kKT - 1) / kKT;
  int tmask = nkt;
  if (bias != 0.0f) tmask = m / kKT;
  if (L % kKT) tmask = min(tmask, nkt - 1);

  // ---- prologue: K(0), V(0), K(1) in LDS; V(1), K(2) in flight
  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  load_k(1);
  store_k(1);
  __syncthreads();
  load_v(1);
  load_k(2);
  f32x16 sA[2], sB[2];
  compute_s(sK(0), sA);
  if (tmask == 0) mask_s(sA, 0);
  update_max(rowmax(sA));

  // ---- steady state.  Iteration t: S(t+1) from K buffer (t+1)&1 while P(t)
  // is formed; P(t) V(t) from V buffer t&1 while max S(t+1) is taken; then
  // V(t+1) and K(t+2) go to the buffers that iteration t-1 finished with.
  // The two score buffers alternate roles, so the loop runs in pairs.
  auto iter = [&](int t, f32x16 (&sc)[2], f32x16 (&sn)[2], auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    u32x4 pb[4];
    compute_s(sK((t + 1) & 1), sn);
    make_p(sc, pb);
    pv(sV(t & 1), pb);
    if constexpr (MASK) mask_s(sn, (t + 1) * kKT);
    const float mx = rowmax(sn);
    store_v((t + 1) & 1);
    store_k(t & 1);
    __syncthreads();
    load_v(t + 2);
    load_k(t + 3);
    update_max(mx);
  };
  int t = 0;
  const int t1 = min(nkt, tmask);  // iterations t < t1 - 1 need no mask on S(t+1)
  for (; t + 2 < t1; t += 2) {
    iter(t, sA, sB, bool_c<false>{});
    iter(t + 1, sB, sA, bool_c<false>{});
  }
  if (t + 1 < t1) {
    iter(t, sA, sB, bool_c<false>{});
    ++t;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sA[kb] = sB[kb];
  }
  for (; t + 2 < nkt; t += 2) {
    iter(t, sA, sB, bool_c<true>{});
    iter(t + 1, sB, sA, bool_c<true>{});
  }
  if (t + 1 < nkt) {
    iter(t, sA, sB, bool_c<true>{});
    ++t;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sA[kb] = sB[kb];
  }
  {
    u32x4 pb[4];
    make_p(sA, pb);
    pv(sV(t & 1), pb);
  }

  // ---- normalise and scatter back to raster order
  {
    const float lp = l_part + l_part1;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lp), __float_as_uint(lp),
                                                     false, false);
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

template <int D, bool FULL, int NW>
int launch(const AttnParams& p0, hipStream_t stream) {
  using TL = Tiles<D, NW>;
  AttnParams p = p0;
  p.nQT = (p.m + TL::kQT - 1) / TL::kQT;
  const int64_t units = (int64_t)p.batch_heads * p.nW * p.nQT;
  if (units > (int64_t)INT32_MAX / 2) return BASA_ERR_UNSUPPORTED;
  p.units = (int32_t)units;
  p.units_per_xcd = (p.units + 7) / 8;
  const size_t lds = TL::ldsBytes + (FULL ? 0 : (size_t)p.m * 4);
  if (lds > 160 * 1024) return BASA_ERR_UNSUPPORTED;
  static bool attr_set = false;  // benign race: the call is idempotent
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16_kernel<D, FULL, NW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return BASA_ERR_HIP;
    attr_set = true;
  }
  const dim3 grid((unsigned)(8 * p.units_per_xcd));
  hipLaunchKernelGGL((attn_bf16_kernel<D, FULL, NW>), grid, dim3(TL::kThreads), lds, stream, p);
  return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

#ifndef BASA_ATTN_WAVES
#define BASA_ATTN_WAVES 8
#endif

template <int D>
int launch_d(const AttnParams& p, bool full, hipStream_t stream) {
  return full ? launch<D, true, BASA_ATTN_WAVES>(p, stream)
              : launch<D, false, BASA_ATTN_WAVES>(p, stream);
}

}  // namespace

int launch_attn_bf16(const AttnParams& p, bool full, hipStream_t stream) {
  if (p.head_dim == 128) return launch_d<128>(p, full, stream);
  if (p.head_dim == 64) return launch_d<64>(p, full, stream);
  return BASA_ERR_UNSUPPORTED;
}

}  // namespace basa
