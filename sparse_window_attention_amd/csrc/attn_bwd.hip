// Backward of shifted-window attention with pooled K/V memory (bf16, gfx950).
//
// The forward (BASA forum summary, "The BASA Method": attention inside
// shifted windows; BASA discussion reply, the four parts of the method: a
// global memory of pooled K/V appended to every window's keys under one
// softmax) is differentiated exactly.  Per window, with S = scale Q Kc^T +
// bias over Kc = [window keys; memory keys], P = softmax(S), O = P Vc:
//   Dv_i  = sum_d dO_id O_id
//   dS    = P * (dO Vc^T - Dv)
//   dQ    = scale dS Kc,   dKc = scale dS^T Q,   dVc = P^T dO
// P is recomputed from the forward's log-sum-exp.  A window key belongs to
// one window; a memory key collects the gradient of every query of its
// (batch, head), which mean pooling hands on to each token of its cell
// divided by the cell size.
//
// Kernels (one workgroup per unit, 32 rows per wave, XCD-aware unit order):
//   dvec     Dv for every token
//   dq       query-stationary: 128 queries of a window (4 waves, two
//            workgroups per CU) against the key sequence [window keys;
//            memory keys] in tiles of 64 keys loaded straight into LDS:
//            S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T (K^T by
//            transposing LDS reads)
//   dkdv     key-stationary: 128 window keys (4 waves, two workgroups per
//            CU) or 256 memory keys (8 waves) against blocks of 32
//            queries: S = Q K^T, P; pass 0: dV^T += dO^T P; pass 1:
//            dP = dO V^T, dS, dK^T += Q^T dS.  Both passes run in one grid
//            (one launch for memory keys, one for window keys).  Memory-key
//            units cover one chunk of the head's queries each and write fp32
//            partial sums; window-key units write the final dK, dV of their
//            tokens, adding the pooled memory gradient of the token's cell.
//            Windows of 129 to 256 tokens at head dim 128 instead take
//            8-wave workgroups, one per CU, each walking windows of its
//            XCD: a window's query tiles sit in LDS for both passes, and the
//            next window's tiles are loaded while the dK pass runs.
//   memsum   sums the memory partials and divides by the cell size
// All products are 32x32x16 bf16 MFMA with fp32 accumulation; P and dS are
// rounded to bf16 as operands.  Tiles are loaded straight into LDS row-major;
// the transposed operands (K^T, dO^T, Q^T) are read with the transposing LDS
// read, whose lane addresses give the k index the key (or query) order in
// which the S accumulators hold P and dS.
#include "basa_common.h"
#include "basa_internal.h"

namespace basa {

namespace {

constexpr int kNW = 8;                 // waves per workgroup unless a kernel chooses
constexpr int kBlk = 32;               // rows of one MFMA block: keys (dq), queries (dkdv)

// Waves per workgroup of the dQ kernel and of the dK/dV kernel for window
// keys and for memory keys: 8, or 4 with two workgroups per CU, so that one
// workgroup's first loads and last stores overlap the other's products
// (the short units of dQ and of window keys gain; the memory keys' units,
// four times longer, do not).
#ifndef BASA_BWD_DQ_WAVES
#define BASA_BWD_DQ_WAVES 4
#endif
#ifndef BASA_BWD_DKDV_WAVES
#define BASA_BWD_DKDV_WAVES 4
#endif
#ifndef BASA_BWD_DKDV_MEM_WAVES
#define BASA_BWD_DKDV_MEM_WAVES 8
#endif
// Window keys of windows of more than BASA_BWD_DKDV_WAVES * 32 and at most
// 256 tokens, head dim 128: one 8-wave workgroup per window with the
// window's query tiles resident in LDS (both passes in one unit); 0 turns
// it off.  (At head dim 64 the two-buffer kernel measured faster.)
#ifndef BASA_BWD_DKDV_RESIDENT
#define BASA_BWD_DKDV_RESIDENT 1
#endif

template <int D>
struct BT {
  static constexpr int CPR = D / 8;             // 16B chunks per row
  static constexpr int QS = D / 16;             // MFMA steps over the head dim
  static constexpr int DB = D / 32;             // 32-row blocks of a head-dim accumulator
};

__device__ __forceinline__ int64_t slice_base(const BwdParams& p, int bh) {
  const int b = bh / p.heads, h = bh - b * p.heads;
  return (int64_t)b * p.stride_b + (int64_t)h * p.stride_h;
}

// Unit of workgroup `blk` with consecutive units on one XCD; -1 past the
// end.  Workgroups are dealt to the XCDs round robin, so blk & 7 is the XCD
// as long as blk differs from the block index by a multiple of 8.
__device__ __forceinline__ int xcd_unit(int units, int blk) {
  const int upx = (units + 7) / 8;
  const int slot = blk >> 3;
  const int u = (blk & 7) * upx + slot;
  return (slot < upx && u < units) ? u : -1;
}

// Register r of an S accumulator holds row 8*(r/4) + 4*hf + r%4 of the tile.
__device__ __forceinline__ int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// Position of row i (0..31) in a per-lane-half permuted array of 32 floats:
// lane half hf reads its 16 rows (in register order) at hf*16.
__device__ __forceinline__ int perm32(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }

__device__ __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Writes a head-dim accumulator (lane = row of the output, registers = 4
// consecutive d of each 8-d group) as bf16 rows of 16 bytes per lane after a
// lane-pair exchange.  `add` (fp32 [D] per row, may be null) is added first.
template <int D>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[BT<D>::DB], float mul,
                                           const float* add, uint16_t* dst_slice, uint32_t off,
                                           bool valid, int hf) {
  const Rsrc rs = make_rsrc(dst_slice);
#pragma unroll
  for (int db = 0; db < BT<D>::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; g += 2) {
      float a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = acc[db][4 * g + i] * mul;
      if (add != nullptr && valid) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(add + db * 32 + 8 * g + 4 * hf);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(add + db * 32 + 8 * (g + 1) + 4 * hf);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] += x0[i];
          a[4 + i] += x1[i];
        }
      }
      const uint32_t a0 = pack_bf16x2(a[0], a[1]), a1 = pack_bf16x2(a[2], a[3]);
      const uint32_t b0 = pack_bf16x2(a[4], a[5]), b1 = pack_bf16x2(a[6], a[7]);
      // lanes 0-31 end with group g+1 (own half first), lanes 32-63 with group g
      const auto x0 = __builtin_amdgcn_permlane32_swap(b0, a0, false, false);
      const auto x1 = __builtin_amdgcn_permlane32_swap(b1, a1, false, false);
      const u32x4 w{x0[0], x1[0], x0[1], x1[1]};
      const int d = db * 32 + 8 * (g + 1 - hf);
      if (valid) __builtin_amdgcn_raw_buffer_store_b128(w, rs, off + d * 2, 0, 0);
    }
}

// store_rows for a kernel that loops over units: the row's byte offset and
// `add` pass through an empty asm, so that each store and load adds a
// constant to them in its offset field (rather than the compiler holding
// every per-lane offset plus constant in a register of its own across the
// loop), and the `add` values of two d blocks are loaded together, one wait
// for eight loads.
template <int D>
__device__ __forceinline__ void store_rows_u(const f32x16 (&acc)[BT<D>::DB], float mul,
                                             const float* add, uint16_t* dst_slice,
                                             uint32_t off, bool valid, int hf) {
  using gf4 = const __attribute__((address_space(1))) f32x4;
  const Rsrc rs = make_rsrc(dst_slice);
  off -= 16 * hf;   // the lane half's part of d
  asm("" : "+v"(off));
  const __attribute__((address_space(1))) float* ag = nullptr;
  if (add != nullptr) {
    const float* a4 = add + 4 * hf;
    asm("" : "+v"(a4));
    ag = (const __attribute__((address_space(1))) float*)a4;
  }
#pragma unroll
  for (int db0 = 0; db0 < BT<D>::DB; db0 += 2) {
    f32x4 x[2][4] = {};
    if (ag != nullptr && valid) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int g = 0; g < 4; ++g) x[u][g] = *(gf4*)(ag + (db0 + u) * 32 + 8 * g);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g = 0; g < 4; g += 2) {
        const int db = db0 + u;
        float a[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = acc[db][4 * g + i] * mul + x[u][g][i];
          a[4 + i] = acc[db][4 * g + 4 + i] * mul + x[u][g + 1][i];
        }
        const uint32_t a0 = pack_bf16x2(a[0], a[1]), a1 = pack_bf16x2(a[2], a[3]);
        const uint32_t b0 = pack_bf16x2(a[4], a[5]), b1 = pack_bf16x2(a[6], a[7]);
        const auto x0 = __builtin_amdgcn_permlane32_swap(b0, a0, false, false);
        const auto x1 = __builtin_amdgcn_permlane32_swap(b1, a1, false, false);
        const u32x4 w{x0[0], x1[0], x0[1], x1[1]};
        if (valid)
          __builtin_amdgcn_raw_buffer_store_b128(w, rs, off + (db * 32 + 8 * (g + 1)) * 2, 0, 0);
      }
  }
}

// ---------------------------------------------------------------- dvec
template <int D>
__global__ void __launch_bounds__(256) bwd_dvec_kernel(BwdParams p) {
  constexpr int CPR = D / 8, RPW = 64 / CPR;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / CPR;
  if (row >= (int64_t)p.batch_heads * p.n) return;   // whole row groups exit together
  const int bh = (int)(row / p.n);
  const int tok = (int)(row - (int64_t)bh * p.n);
  const int c = lane % CPR;
  const int64_t off = slice_base(p, bh) + (int64_t)tok * p.stride_tok + c * 8;
  const u32x4 o = *reinterpret_cast<const u32x4*>(p.out + off);
  const u32x4 g = *reinterpret_cast<const u32x4*>(p.dout + off);
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s += bf16_lo(o[e]) * bf16_lo(g[e]) + bf16_hi(o[e]) * bf16_hi(g[e]);
#pragma unroll
  for (int w = 1; w < CPR; w *= 2) s += __shfl_xor(s, w);
  if (c == 0) p.dvec[row] = s;
}

// A wave-uniform pointer held in vector registers, read into scalar ones.
template <class P>
__device__ __forceinline__ P* uniform_ptr(P* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (P*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------- dq
// dQ with the key tiles loaded straight into LDS: 64 keys per iteration, K
// and V tiles row-major (16-byte chunks XOR-swizzled per row), K rows and V
// rows read as MFMA operands and K^T read with the transposing LDS read.  One
// swizzle serves both reads of the K tile: chunk c of row r sits at slot
// c ^ f(r), f a bijection of r mod 16 whose bits 2-3 separate any 4
// consecutive rows, so the 16 rows of a quarter-wave row read and the
// 4 rows x 4 chunks of a half-wave transposing read fall in distinct banks.
template <int D, int NW = kNW>
struct DqDma {
  using T = BT<D>;
  static constexpr int kKeys = 64;                  // keys per iteration
  static constexpr int CPR = D / 8;
  static constexpr int RowB = CPR * 16;             // bytes per row
  static constexpr int kTileB = kKeys * RowB;       // one K or V tile
  static constexpr int kIpw = kTileB / 1024 / NW;   // 1 KB loads per wave and tile
  static_assert(kIpw >= 1 && kIpw * NW * 1024 == kTileB, "tile must split over the waves");
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
};

// NW waves of 32 queries per workgroup; with 4, two workgroups share a CU.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 8 / NW) bwd_dq_kernel(BwdParams p) {
  using T = BT<D>;
  using Q = DqDma<D, NW>;
  constexpr int kUnit = NW * 32;        // queries per unit
  constexpr int kThreads = NW * 64;
  constexpr int CPR = Q::CPR, RowB = Q::RowB, KTB = Q::kTileB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // K buffer b at b * KTB, V buffer b at (2 + b) * KTB, then the table
  const int nQT = (p.m + kUnit - 1) / kUnit;
  const int unit = xcd_unit(p.batch_heads * p.nW * nQT, blockIdx.x);
  if (unit < 0) return;
  const int qt = unit % nQT;
  const int rest = unit / nQT;
  const int win = rest % p.nW;
  const int bh = rest / p.nW;
  const int64_t base = slice_base(p, bh);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const uint32_t stb = (uint32_t)p.stride_tok * 2u;
  int32_t* tab = reinterpret_cast<int32_t*>(smem + 4 * KTB);
  for (int r = tid; r < p.m; r += kThreads) tab[r] = window_token(p.geo, win, r);
  __syncthreads();

  const int qr = qt * kUnit + wave * 32 + l32;
  const bool qvalid = qr < p.m;
  const int qtok = qvalid ? tab[qr] : 0;
  const uint32_t qoff = (uint32_t)qtok * stb;
  u32x4 qreg[T::QS], dreg[T::QS];
  {
    const Rsrc rq = make_rsrc(p.q + base), rd = make_rsrc(p.dout + base);
#pragma unroll
    for (int s = 0; s < T::QS; ++s) {
      const u32x4 a = buf_load16(rq, qoff + hf * D + s * 16, 0);
      const u32x4 b = buf_load16(rd, qoff + hf * D + s * 16, 0);
      qreg[s] = qvalid ? a : u32x4{0u, 0u, 0u, 0u};
      dreg[s] = qvalid ? b : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const float lse2 = qvalid ? p.lse[(int64_t)bh * p.n + qtok] * kLog2e : INFINITY;
  const float dval = qvalid ? p.dvec[(int64_t)bh * p.n + qtok] : 0.0f;
  f32x16 acc[T::DB];
#pragma unroll
  for (int i = 0; i < T::DB; ++i) acc[i] = f32x16{};

  const int L = p.m + p.G;
  const int nit = (L + Q::kKeys - 1) / Q::kKeys;
  const uint16_t* kmem = p.kmem + (int64_t)bh * p.G * D;
  const uint16_t* vmem = p.vmem + (int64_t)bh * p.G * D;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // this wave's share of the loads of iteration it's K and V tiles; the tile
  // kind (window rows through the table, memory rows, mixed) and the buffer
  // resources are decided once per tile
  auto dma = [&](int it) __attribute__((always_inline)) {
    const int k0 = it * Q::kKeys;
    unsigned char* bk = smem + (it & 1) * KTB;
    unsigned char* bv = smem + (2 + (it & 1)) * KTB;
    const bool winT = k0 + Q::kKeys <= p.m;
    const bool memT = k0 >= p.m && k0 + Q::kKeys <= L;
    int r[Q::kIpw];
    uint32_t cb[Q::kIpw];
#pragma unroll
    for (int i = 0; i < Q::kIpw; ++i) {
      r[i] = ((wv * Q::kIpw + i) * 64 + lane) / CPR;
      cb[i] = (uint32_t)(((lane % CPR) ^ Q::swz(r[i])) * 16);
    }
    // LDS destinations of instruction i: bk / bv + (wv * kIpw + i) KB.  Macros,
    // and offsets named before the builtin calls: with a lambda returning the
    // LDS pointer, or an offset expression inside the call, the compiler's
    // host pass silently drops this kernel's launch stub (the library then
    // fails to load).
#define BASA_DQ_LK(i) ((__attribute__((address_space(3))) void*)(bk + (wv * Q::kIpw + (i)) * 1024))
#define BASA_DQ_LV(i) ((__attribute__((address_space(3))) void*)(bv + (wv * Q::kIpw + (i)) * 1024))
    if (winT) {
      // all table reads first (one LDS wait), then the loads
      uint32_t toff[Q::kIpw];
#pragma unroll
      for (int i = 0; i < Q::kIpw; ++i) toff[i] = (uint32_t)tab[k0 + r[i]] * stb;
      const Rsrc rk = make_rsrc(p.k + base), rvs = make_rsrc(p.v + base);
#pragma unroll
      for (int i = 0; i < Q::kIpw; ++i) {
        const uint32_t off = toff[i] + cb[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, BASA_DQ_LK(i), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rvs, BASA_DQ_LV(i), 16, off, 0, 0, 0);
      }
    } else if (memT) {
      // scalar copies: the mixed-tile path keeps kmem / vmem in vector
      // registers, and a resource built from those would wrap every load in
      // a loop over its lanes' values
      const Rsrc rk = make_rsrc(uniform_ptr(kmem)), rvs = make_rsrc(uniform_ptr(vmem));
#pragma unroll
      for (int i = 0; i < Q::kIpw; ++i) {
        const uint32_t off = (uint32_t)(k0 - p.m + r[i]) * (D * 2) + cb[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, BASA_DQ_LK(i), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rvs, BASA_DQ_LV(i), 16, off, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < Q::kIpw; ++i) {
        const int key = min(k0 + r[i], L - 1);   // rows past the end: clamped, masked below
        const char* gk;
        const char* gvp;
        if (key < p.m) {
          const int64_t o = (int64_t)tab[key] * stb + cb[i];
          gk = reinterpret_cast<const char*>(p.k + base) + o;
          gvp = reinterpret_cast<const char*>(p.v + base) + o;
        } else {
          const int64_t o = (int64_t)(key - p.m) * (D * 2) + cb[i];
          gk = reinterpret_cast<const char*>(kmem) + o;
          gvp = reinterpret_cast<const char*>(vmem) + o;
        }
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gk, BASA_DQ_LK(i), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gvp, BASA_DQ_LV(i), 16, 0, 0);
      }
    }
#undef BASA_DQ_LK
#undef BASA_DQ_LV
  };
  dma(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads are in LDS
  __syncthreads();
  const float c1 = p.c1;
  const int x = Q::swz(l32);
  const int sq = (lane & 15) >> 2;
  const int d0 = 16 * (l32 >> 4) + 4 * (lane & 3);
  for (int it = 0; it < nit; ++it) {
    if (it + 1 < nit) dma(it + 1);
    const unsigned char* sk = smem + (it & 1) * KTB;
    const unsigned char* sv = smem + (2 + (it & 1)) * KTB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s{}, dp{};
#pragma unroll
      for (int ss = 0; ss < T::QS; ++ss) {
        const int off = (kb * 32 + l32) * RowB + (((hf * (CPR / 2) + ss) ^ x) * 16);
        const u32x4 a = *reinterpret_cast<const u32x4*>(sk + off);
        const u32x4 b = *reinterpret_cast<const u32x4*>(sv + off);
        s = mfma(a, qreg[ss], s);
        dp = mfma(b, dreg[ss], dp);
      }
      u32x4 dsb[2];
      // A tile of window keys only or of memory keys only, with no key past
      // the end, takes the memory bias as one offset; other tiles select
      // per key (bias for memory keys, -inf past the end).
      const int k0 = it * Q::kKeys;
      const bool whole = k0 + Q::kKeys <= p.m || (k0 >= p.m && k0 + Q::kKeys <= L);
      const float nb = (k0 >= p.m ? p.mem_bias_raw * c1 : 0.0f) - lse2;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
        if (whole) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = 8 * u + j;
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c1, nb));
            e[j] = pr * (dp[r] - dval);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = 8 * u + j;
            const int key = k0 + kb * 32 + acc_row(r, hf);
            float xv = s[r] + (key >= p.m ? p.mem_bias_raw : 0.0f);
            xv = key < L ? xv : -INFINITY;
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(xv, c1, -lse2));
            e[j] = pr * (dp[r] - dval);
          }
        }
        dsb[u] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                       pack_bf16x2(e[6], e[7])};
      }
      // dQ^T += K^T dS^T: K^T of slice sl = 2kb + u by transposing reads
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int sl = 2 * kb + u;
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          bf16x4 h2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int key = 16 * sl + 8 * h + 4 * hf + sq;
            const int d = 32 * db + d0;
            h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(
                sk + key * RowB + (((d >> 3) ^ Q::swz(key)) * 16) + (d & 7) * 2));
          }
          const bf16x8 av = {h2[0][0], h2[0][1], h2[0][2], h2[0][3],
                             h2[1][0], h2[1][1], h2[1][2], h2[1][3]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, dsb[u]),
                                                           acc[db], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's loads of the next tiles
    __syncthreads();
  }
  store_rows<D>(acc, p.scale, nullptr, p.dq + base, qoff, qvalid, hf);
}

// ---------------------------------------------------------------- dk, dv
// MEM: memory-key units (b*h, memory chunk of 256 keys, query chunk) writing
// fp32 partials; otherwise window-key units (b*h, window, key chunk of 256)
// writing the final gradients.  PASS 0: dV; PASS 1: dK.  Each iteration
// takes 64 queries (two blocks of 32, one barrier): the Q and dO tiles are
// loaded straight into LDS (the dQ kernel's row swizzle); Q rows and dO rows
// are read as MFMA operands, and dO^T (pass 0) and Q^T (pass 1) with the
// transposing LDS read.
// The products of one query tile (Q rows at sqt, dO rows at sqt + TB, lse
// and Dv at slp) for its 32-query blocks KB0 .. KB0 + NKB - 1, against
// this wave's 32 keys (K and V rows in registers), accumulated into acc:
// pass PS = 0: dV^T += dO^T P; PS = 1: dK^T += Q^T dS.  With NKB = 2 the
// accumulation chains of the two blocks are interleaved and every LDS
// operand is read two products before its MFMA; with NKB = 1 each operand
// is read right before its MFMA.  Each accumulator sums its terms in the
// same order either way.
using lds_cu8 = const __attribute__((address_space(3))) unsigned char;

// base + off as an LDS address; with FA, formed in a register the compiler
// cannot see through (an asm without side effects: loads still move freely
// around it).  In a loop over LDS buffers each address is then one such sum
// per iteration, with its constant part in the instruction's offset field;
// otherwise every (per-lane offset + constant) may be hoisted out of the
// loop into a register of its own and the buffer base added at each read.
template <bool FA>
__device__ __forceinline__ lds_cu8* lds_at(const unsigned char* base, uint32_t off) {
  uint32_t a = (uint32_t)(uintptr_t)(lds_cu8*)base + off;
  if constexpr (FA) asm("" : "+v"(a));
  return (lds_cu8*)(uintptr_t)a;
}

template <int D, int NW, int PS, int KB0, int NKB, bool FA = false>
__device__ __forceinline__ void dkdv_blocks(const unsigned char* sqt, const unsigned char* slp,
                                            const u32x4* kreg,
                                            const u32x4* vreg, f32x16 (&acc)[BT<D>::DB],
                                            float c1, int l32, int hf, int lane) {
  using T = BT<D>;
  using Q = DqDma<D, NW>;
  using lds_v4 = const __attribute__((address_space(3))) u32x4;
  using lds_f4 = const __attribute__((address_space(3))) f32x4;
  using lds_h4 = __attribute__((address_space(3))) bf16x4;
  constexpr int CPR = Q::CPR, RowB = Q::RowB, TB = Q::kTileB;
  const int x = Q::swz(l32);
  const int sq = (lane & 15) >> 2;
  const int d0 = 16 * (l32 >> 4) + 4 * (lane & 3);
  constexpr int AH = NKB == 2 ? 2 : 0;   // operand reads ahead
  // With FA, each address is the per-lane part formed on the tile's base
  // (lds_at) plus a constant (block, row slice, dO tile).
  // chunk ss of row l32 (S = Q K^T and dP = dO V^T A operands)
  lds_cu8* ra[T::QS];
  // lse of this lane's rows (Dv 32 floats further)
  lds_cu8* rl = nullptr;
  // transposing reads: row 8h + 4hf + sq of each 16-row slice, d block db
  // (the swizzle depends on the row modulo 16 only)
  lds_cu8* rt[2][T::DB];
  if constexpr (FA) {
#pragma unroll
    for (int ss = 0; ss < T::QS; ++ss)
      ra[ss] = lds_at<FA>(sqt, l32 * RowB + (((hf * (CPR / 2) + ss) ^ x) * 16));
    rl = lds_at<FA>(slp, hf * 64);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const int row = 8 * h + 4 * hf + sq;
        const int d = 32 * db + d0;
        rt[h][db] = lds_at<FA>(sqt, row * RowB + (((d >> 3) ^ Q::swz(row)) * 16) + (d & 7) * 2);
      }
  }
  // A operand chunk ss of row l32 of block KB0 + j, tile at toff
  auto rda = [&](int toff, int ss, int j) __attribute__((always_inline)) {
    if constexpr (FA) return *(lds_v4*)(ra[ss] + toff + (KB0 + j) * 32 * RowB);
    else
      return *reinterpret_cast<const u32x4*>(sqt + toff + ((KB0 + j) * 32 + l32) * RowB +
                                             (((hf * (CPR / 2) + ss) ^ x) * 16));
  };
  // 4 floats of the lse / Dv array at float offset o (+ this lane's rows)
  auto rdl = [&](int o) __attribute__((always_inline)) {
    if constexpr (FA) return *(lds_f4*)(rl + o * 4);
    else return *reinterpret_cast<const f32x4*>(slp + (o + hf * 16) * 4);
  };
  // S = Q K^T (tile at toff 0, b = K rows) or dP = dO V^T (toff TB, b = V rows)
  auto rowprod = [&](int toff, const u32x4* b, f32x16 (&o)[NKB])
      __attribute__((always_inline)) {
    u32x4 a[AH + 1][NKB];
    auto rd = [&](int ss) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NKB; ++j)
        a[ss % (AH + 1)][j] = rda(toff, ss, j);
    };
#pragma unroll
    for (int ss = 0; ss < AH; ++ss) rd(ss);
#pragma unroll
    for (int ss = 0; ss < T::QS; ++ss) {
      if (ss + AH < T::QS) rd(ss + AH);
#pragma unroll
      for (int j = 0; j < NKB; ++j)
        o[j] = mfma(a[ss % (AH + 1)][j], b[ss], ss == 0 ? f32x16{} : o[j]);
    }
  };
  f32x16 sc[NKB];
  rowprod(0, kreg, sc);
  float w[NKB][16];   // P, then (pass 1) dS
#pragma unroll
  for (int j = 0; j < NKB; ++j)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 l4 = rdl((KB0 + j) * 64 + r4 * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[j][4 * r4 + i] =
            __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j][4 * r4 + i], c1, -l4[i]));
    }
  if constexpr (PS == 1) {
    f32x16 dp[NKB];
    rowprod(TB, vreg, dp);
#pragma unroll
    for (int j = 0; j < NKB; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 d4 = rdl((KB0 + j) * 64 + 32 + r4 * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[j][4 * r4 + i] *= dp[j][4 * r4 + i] - d4[i];
      }
  }
  // pass 0: dV^T += dO^T P; pass 1: dK^T += Q^T dS -- the transposed
  // operand by transposing reads of the row-major tile.  Product i is
  // (key slice i / DB of these blocks, d block i % DB), so consecutive
  // products update different accumulators.
  constexpr int tto = PS == 0 ? TB : 0;
  u32x4 pb[2 * NKB];
#pragma unroll
  for (int u = 0; u < 2 * NKB; ++u) {
    const float* v = w[u >> 1] + 8 * (u & 1);
    pb[u] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
  constexpr int NP = 2 * NKB * T::DB;
  auto rdt = [&](int i) __attribute__((always_inline)) {
    const int slc = 2 * KB0 + i / T::DB, db = i % T::DB;
    bf16x4 h2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (FA) {
        h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_h4*)(rt[h][db] + tto + 16 * slc * RowB));
      } else {
        const int row = 16 * slc + 8 * h + 4 * hf + sq;
        const int d = 32 * db + d0;
        h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_h4*)(
            sqt + tto + row * RowB + (((d >> 3) ^ Q::swz(row)) * 16) + (d & 7) * 2));
      }
    }
    return bf16x8{h2[0][0], h2[0][1], h2[0][2], h2[0][3], h2[1][0], h2[1][1], h2[1][2], h2[1][3]};
  };
  bf16x8 av[AH + 1];
#pragma unroll
  for (int i = 0; i < AH; ++i) av[i] = rdt(i);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (i + AH < NP) av[(i + AH) % (AH + 1)] = rdt(i + AH);
    acc[i % T::DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        av[i % (AH + 1)], __builtin_bit_cast(bf16x8, pb[i / T::DB]), acc[i % T::DB], 0, 0, 0);
  }
}

template <int P>
struct pass_c {
  static constexpr int value = P;
};

// RES: a window-key unit holding all of its window's keys (m <= NW * 32)
// loads every query tile of the window (Q, dO, lse, Dv) into LDS once, then
// runs pass 0 and pass 1 over the resident tiles with no loads or barriers
// in the loop.  Otherwise the unit runs pass PASS with two tile buffers in
// turn, loading the next query tile during each iteration.
template <int D, bool MEM, int PASS, int NW, bool RES = false>
__device__ __forceinline__ void dkdv_body(const BwdParams& p, int blk) {
  using T = BT<D>;
  using Q = DqDma<D, NW>;
  constexpr int kUnit = NW * 32;               // keys per unit
  constexpr int kThreads = NW * 64;
  constexpr int CPR = Q::CPR, RowB = Q::RowB, TB = Q::kTileB;
  constexpr int kQ = Q::kKeys;                 // queries per iteration
  constexpr int kBufB = 2 * TB + 2 * kQ * 4;   // Q tile, dO tile, lse and Dv
  constexpr int kNB = RES ? kUnit / kQ : 2;    // tile buffers
  static_assert(!(RES && MEM), "resident query tiles are for window keys");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int bh, kbase, nq, qbase = 0, win = 0;
  if constexpr (MEM) {
    const int nmc = (p.G + kUnit - 1) / kUnit;
    const int unit = xcd_unit(p.batch_heads * nmc * p.nqc, blk);
    if (unit < 0) return;
    const int qc = unit % p.nqc;
    const int rest = unit / p.nqc;
    kbase = (rest % nmc) * kUnit;
    bh = rest / nmc;
    qbase = qc * p.qchunk;
    nq = min(p.qchunk, p.n - qbase);
  } else {
    const int nkc = (p.m + kUnit - 1) / kUnit;
    const int unit = xcd_unit(p.batch_heads * p.nW * nkc, blk);
    if (unit < 0) return;
    kbase = (unit % nkc) * kUnit;
    const int rest = unit / nkc;
    win = rest % p.nW;
    bh = rest / p.nW;
    nq = p.m;
  }
  const int64_t base = slice_base(p, bh);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const uint32_t stb = (uint32_t)p.stride_tok * 2u;
  const int nkeys = MEM ? p.G : p.m;
  int32_t* tab = reinterpret_cast<int32_t*>(smem + kNB * kBufB);
  if constexpr (!MEM) {
    for (int r = tid; r < p.m; r += kThreads) tab[r] = window_token(p.geo, win, r);
    __syncthreads();
  }
  auto buf = [&](int it) __attribute__((always_inline)) {
    return smem + (RES ? it : (it & 1)) * kBufB;
  };

  // this lane's key: K (and V) rows as B operands
  const int key = kbase + wave * 32 + l32;
  const bool kvalid = key < nkeys;
  const int kcl = min(key, nkeys - 1);
  u32x4 kreg[T::QS], vreg[(PASS == 1 || RES) ? T::QS : 1];
  {
    const uint16_t* ks = MEM ? p.kmem + (int64_t)bh * p.G * D : p.k + base;
    const uint16_t* vs = MEM ? p.vmem + (int64_t)bh * p.G * D : p.v + base;
    const uint32_t koff = MEM ? (uint32_t)kcl * (D * 2) : (uint32_t)tab[kcl] * stb;
    const Rsrc rk = make_rsrc(ks), rv = make_rsrc(vs);
#pragma unroll
    for (int s = 0; s < T::QS; ++s) {
      kreg[s] = buf_load16(rk, koff + hf * D + s * 16, 0);
      if constexpr (PASS == 1 || RES) vreg[s] = buf_load16(rv, koff + hf * D + s * 16, 0);
    }
  }
  const int nit = (nq + kQ - 1) / kQ;
  auto token_of = [&](int q) __attribute__((always_inline)) {
    return MEM ? qbase + q : tab[q];
  };
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  float lx = INFINITY, dvx = 0.0f;
  // this wave's share of the Q and dO tile loads of iteration it; lse and Dv
  // of the iteration's queries into registers (stored by `put`)
  auto get = [&](int it) __attribute__((always_inline)) {
    unsigned char* b = buf(it);
    // all row tokens first (one LDS wait for the window table), then the loads
    int tok[Q::kIpw];
#pragma unroll
    for (int i = 0; i < Q::kIpw; ++i) {
      const int r = ((wv * Q::kIpw + i) * 64 + lane) / CPR;
      tok[i] = token_of(min(it * kQ + r, nq - 1));
    }
#pragma unroll
    for (int i = 0; i < Q::kIpw; ++i) {
      const int ins = wv * Q::kIpw + i;
      const int r = (ins * 64 + lane) / CPR;
      const uint32_t off = (uint32_t)tok[i] * stb + (uint32_t)(((lane % CPR) ^ Q::swz(r)) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p.q + base),
          (__attribute__((address_space(3))) void*)(b + ins * 1024), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p.dout + base),
          (__attribute__((address_space(3))) void*)(b + TB + ins * 1024), 16, off, 0, 0, 0);
    }
    if (tid < kQ) {
      const int q = it * kQ + tid;
      const bool ok = q < nq;
      const int64_t idx = (int64_t)bh * p.n + token_of(ok ? q : nq - 1);
      // log2-scale log-sum-exp less the memory keys' bias (P = exp2(S c1 -
      // lx) with the bias folded in); a missing query gets P = 0
      lx = ok ? p.lse[idx] * kLog2e - (MEM ? p.mem_bias_raw * p.c1 : 0.0f) : INFINITY;
      dvx = ok ? p.dvec[idx] : 0.0f;
    }
  };
  auto put = [&](int it) __attribute__((always_inline)) {
    if (tid < kQ) {
      float* sl = reinterpret_cast<float*>(buf(it) + 2 * TB);
      sl[(tid / kBlk) * 64 + perm32(tid % kBlk)] = lx;
      sl[(tid / kBlk) * 64 + 32 + perm32(tid % kBlk)] = dvx;
    }
  };
  if constexpr (RES) {
    // every tile's loads first, then the stores of lse and Dv (each waits
    // for its own global loads, so storing between the tile loads would
    // hold back the next tile's issue)
    float lxs[kNB], dvs[kNB];
#pragma unroll
    for (int it = 0; it < kNB; ++it)
      if (it < nit) {
        get(it);
        lxs[it] = lx;
        dvs[it] = dvx;
      }
#pragma unroll
    for (int it = 0; it < kNB; ++it)
      if (it < nit) {
        lx = lxs[it];
        dvx = dvs[it];
        put(it);
      }
  } else {
    get(0);
    put(0);
  }
  // window keys: the pooled-memory cell of the key's token, whose gradient
  // the epilogue adds; its divisions run while the unit's first loads are
  // in flight, off the epilogue's path
  int cell = 0;
  if constexpr (!MEM) {
    if (p.G > 0) {
      const int tok = tab[kcl];
      const int xx = tok % p.geo.Wg;
      const int y = (tok / p.geo.Wg) % p.geo.Hg;
      const int t = tok / (p.geo.Wg * p.geo.Hg);
      cell = ((t / p.pt) * p.Gy + y / p.py) * p.Gx + xx / p.px;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's tile loads are in LDS
  __syncthreads();
  const float c1 = p.c1;
  auto run = [&](auto pc) __attribute__((always_inline)) {
    constexpr int PS = decltype(pc)::value;
    f32x16 acc[T::DB];
#pragma unroll
    for (int i = 0; i < T::DB; ++i) acc[i] = f32x16{};
    for (int it = 0; it < nit; ++it) {
      if (!RES && it + 1 < nit) get(it + 1);
      const unsigned char* sqt = buf(it);   // Q tile, dO tile, lse and Dv
      if constexpr (RES) {
        dkdv_blocks<D, NW, PS, 0, 2>(sqt, sqt + 2 * TB, kreg, vreg, acc, c1, l32, hf, lane);
      } else {
        // the interleaved order fits beside the next tile's load state only
        // with the addresses formed per tile
        dkdv_blocks<D, NW, PS, 0, 2, true>(sqt, sqt + 2 * TB, kreg, vreg, acc, c1, l32, hf, lane);
      }
      if constexpr (!RES) {
        if (it + 1 < nit) put(it + 1);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's loads of the next tiles
        __syncthreads();
      }
    }

    if constexpr (MEM) {
      // fp32 partials [bh][qc][key][d]; lane = key, registers = 4 consecutive d
      if (kvalid) {
        const int qc = qbase / p.qchunk;
        float* dst = (PS == 0 ? p.pv : p.pk) + (((int64_t)bh * p.nqc + qc) * p.G + key) * D;
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(dst + db * 32 + 8 * g + 4 * hf) =
                f32x4{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
      }
    } else {
      const int tok = tab[kcl];
      const float* add = nullptr;
      if (p.G > 0) add = (PS == 0 ? p.gv : p.gk) + ((int64_t)bh * p.G + cell) * D;
      store_rows<D>(acc, PS == 0 ? 1.0f : p.scale, add, (PS == 0 ? p.dv : p.dk) + base,
                    (uint32_t)tok * stb, kvalid, hf);
    }
  };
  if constexpr (RES) {
    run(pass_c<0>{});
    run(pass_c<1>{});
  } else {
    run(pass_c<PASS>{});
  }
}

// Both passes in one grid: workgroups [0, split) run pass 0 (dV), the rest
// pass 1 (dK); split is a multiple of 8.  One launch lets the second pass
// fill the CUs the first leaves idle at its end.
// NW waves of 32 keys per workgroup; with 4, two workgroups share a CU.
template <int D, bool MEM, int NW>
__global__ void __launch_bounds__(NW * 64, 8 / NW) bwd_dkdv_kernel(BwdParams p, int split) {
  if ((int)blockIdx.x < split) dkdv_body<D, MEM, 0, NW>(p, blockIdx.x);
  else dkdv_body<D, MEM, 1, NW>(p, blockIdx.x - split);
}

// x, wave-uniform, through an empty asm the compiler cannot see through: the
// set-up of a division by x (its reciprocal) is then recomputed where the
// division is, instead of hoisted out of an outer loop and held in registers
// across it.
__device__ __forceinline__ int32_t opaque_s(int32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}
// The same for a per-lane value: what is computed from it is recomputed
// where it is used rather than held in registers across a loop.
__device__ __forceinline__ int32_t opaque_v(int32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Window keys of windows of at most 256 tokens, one 8-wave workgroup per
// CU walking the (batch, head, window) units of one XCD.  A unit holds all
// of its window's query tiles (Q, dO) and their lse and Dv in LDS and runs
// pass 0 (dV) and pass 1 (dK) over them.  The next unit's tiles are loaded
// while pass 1 runs, tile it into buffer it as soon as every wave is done
// with it (BASA_BWD_RES_PREFETCH 2: the last wave to finish the tile, told
// by a count in LDS, issues the whole tile's loads, and no wave waits; 1: a
// barrier after each tile, then each wave its share; 0: no prefetch, the
// loads after the unit).  The next unit's K and V rows, lse and Dv are
// loaded after the dK epilogue.  The window token tables and the lse / Dv
// arrays alternate between two slots by unit parity.  Wave w writes and
// reads rows w*32 .. w*32+31 of each table (its keys, and the same tokens
// as queries for their lse and Dv); only whole-tile loads read the rows of
// other waves, after the count or barrier that follows every wave's rows.
#ifndef BASA_BWD_RES_PREFETCH
#define BASA_BWD_RES_PREFETCH 2
#endif
template <int D>
__device__ __forceinline__ void dkdv_res_body(const BwdParams& p) {
  constexpr int NW = kNW;
  constexpr int PF = BASA_BWD_RES_PREFETCH;
  using T = BT<D>;
  using Q = DqDma<D, NW>;
  constexpr int CPR = Q::CPR, TB = Q::kTileB;
  constexpr int kQ = Q::kKeys;                 // queries per tile
  constexpr int kMaxM = NW * 32;               // window tokens at most (keys of the unit)
  constexpr int kNB = kMaxM / kQ;              // tile buffers
  constexpr int kSlB = 2 * kQ * 4;             // lse and Dv of one tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int units = p.batch_heads * p.nW;
  const int upx = (units + 7) / 8;
  const int S = (int)(gridDim.x >> 3);
  const int ubeg = (int)(blockIdx.x & 7) * upx, uend = min(ubeg + upx, units);
  const int first = ubeg + (int)(blockIdx.x >> 3);
  if (first >= uend) return;                   // whole workgroup exits together
  const int J = (uend - first + S - 1) / S;    // units of this workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t stb = (uint32_t)p.stride_tok * 2u;
  const int m = p.m;
  const int nit = (m + kQ - 1) / kQ;
  const int key = wave * 32 + l32;             // this lane's key of the window
  const bool kvalid = key < m;
  const int kcl = min(key, m - 1);
  const float c1 = p.c1;
  // LDS: kNB Q/dO tile buffers, two slots of kNB lse/Dv arrays, two table
  // slots, kNB finish counts
  auto buf = [&](int it) __attribute__((always_inline)) { return smem + it * (2 * TB); };
  auto slb = [&](int j, int it) __attribute__((always_inline)) {
    return smem + kNB * (2 * TB) + ((j & 1) * kNB + it) * kSlB;
  };
  auto tab_of = [&](int j) __attribute__((always_inline)) {
    return reinterpret_cast<int32_t*>(smem + kNB * (2 * TB) + 2 * kNB * kSlB) + (j & 1) * kMaxM;
  };
  int32_t* cnt = reinterpret_cast<int32_t*>(smem + kNB * (2 * TB) + 2 * kNB * kSlB) + 2 * kMaxM;
  // unit j's window and (batch, head) slice, wave-uniform (scalar registers:
  // the buffer resources built from them stay scalar)
  auto win_of = [&](int j) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane((first + j * S) % opaque_s(p.nW));
  };
  auto bh_of = [&](int j) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane((first + j * S) / opaque_s(p.nW));
  };
  // this wave's rows of a table (kMaxM = 32 rows per wave)
  auto build_rows = [&](int32_t* tab, int win) __attribute__((always_inline)) {
    Geometry g = p.geo;
    g.nwx = opaque_s(g.nwx);
    g.nwy = opaque_s(g.nwy);
    if (hf == 0 && kvalid) tab[key] = window_token(g, win, key);
  };
  // Q and dO loads of query tile it into buffer it: 1 KB instructions i0,
  // i0 + 1, ..., i0 + n - 1 of the tile
  auto tile_part = [&](int it, int i0, int n, int64_t base, const int32_t* tab)
      __attribute__((always_inline)) {
    unsigned char* b = buf(it);
    const int ln = opaque_v(lane);   // addresses computed here, not held across pass 1
    const Rsrc rq = make_rsrc(p.q + base), rd = make_rsrc(p.dout + base);
#pragma unroll 1
    for (int i4 = 0; i4 < n; i4 += 4) {
      int tok[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = ((i0 + i4 + i) * 64 + ln) / CPR;
        tok[i] = (i4 + i < n) ? tab[min(it * kQ + r, m - 1)] : 0;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i4 + i < n) {
          const int ins = i0 + i4 + i;
          const int r = (ins * 64 + ln) / CPR;
          const uint32_t off =
              (uint32_t)tok[i] * stb + (uint32_t)(((ln % CPR) ^ Q::swz(r)) * 16);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rq,
              (__attribute__((address_space(3))) void*)(b + ins * 1024), 16, off, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rd,
              (__attribute__((address_space(3))) void*)(b + TB + ins * 1024), 16, off, 0, 0, 0);
        }
      }
    }
  };
  // this wave's share of tile it
  auto tiles = [&](int it, int64_t base, const int32_t* tab) __attribute__((always_inline)) {
    tile_part(it, wv * Q::kIpw, Q::kIpw, base, tab);
  };
  // The wave's 32 queries (its keys' tokens): lanes 0-31 the log2-scale
  // log-sum-exp, lanes 32-63 Dv; a missing query gets P = 0.
  auto vec = [&](int bh, const int32_t* tab) __attribute__((always_inline)) {
    float x = hf ? 0.0f : INFINITY;
    if (kvalid) {
      const int64_t idx = (int64_t)bh * p.n + tab[key];
      x = hf ? p.dvec[idx] : p.lse[idx] * kLog2e;
    }
    return x;
  };
  // query `key` is row key % 64 of tile key / 64: block (wave & 1) of tile
  // wave / 2; tiles past the window's last hold only missing queries
  auto put = [&](int j, float x) __attribute__((always_inline)) {
    float* sl = reinterpret_cast<float*>(slb(j, wave >> 1));
    sl[(wave & 1) * 64 + hf * 32 + perm32(l32)] = x;
  };
  u32x4 kreg[T::QS], vreg[T::QS];   // this lane's K and V rows (B operands)
  // (a key past the window's end loads token 0's rows, never stored)
  auto rows = [&](int64_t base, const int32_t* tab) __attribute__((always_inline)) {
    const uint32_t koff = kvalid ? (uint32_t)tab[key] * stb : 0u;
    const Rsrc rk = make_rsrc(p.k + base), rv = make_rsrc(p.v + base);
#pragma unroll
    for (int s = 0; s < T::QS; ++s) {
      kreg[s] = buf_load16(rk, koff + hf * D + s * 16, 0);
      vreg[s] = buf_load16(rv, koff + hf * D + s * 16, 0);
    }
  };
  // the pooled-memory cell of this lane's key token, whose gradient the
  // epilogues add
  auto cell_of = [&](const int32_t* tab) __attribute__((always_inline)) {
    if (p.G == 0) return 0;
    const int tok = tab[kcl];
    const int Wg = opaque_s(p.geo.Wg), Hg = opaque_s(p.geo.Hg);
    const int xx = tok % Wg;
    const int y = (tok / Wg) % Hg;
    const int t = tok / opaque_s(Wg * Hg);
    return ((t / opaque_s(p.pt)) * p.Gy + y / opaque_s(p.py)) * p.Gx + xx / opaque_s(p.px);
  };

  // unit 0: its table, rows, tiles, lse and Dv
  build_rows(tab_of(0), win_of(0));
  if (tid < kNB) cnt[tid] = 0;
  __syncthreads();   // the whole table, for the tile loads
  float lsd;         // the next unit's lse / Dv of this lane (vec)
  {
    const int bh = bh_of(0);
    const int64_t base = slice_base(p, bh);
    rows(base, tab_of(0));
#pragma unroll
    for (int it = 0; it < kNB; ++it)
      if (it < nit) tiles(it, base, tab_of(0));
    lsd = vec(bh, tab_of(0));
  }
  for (int j = 0; j < J; ++j) {
    const bool has_next = j + 1 < J;
    const int32_t* tab = tab_of(j);
    const int bh = bh_of(j);
    const int64_t base = slice_base(p, bh);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of the unit have landed
    put(j, lsd);
    // Every wave's tiles, lse and Dv are in LDS; every wave is done with the
    // previous unit (its table and lse / Dv slots are free for the next unit's).
    __syncthreads();
    const int bhn = has_next ? bh_of(j + 1) : bh;
    const int64_t basen = slice_base(p, bhn);
    if (has_next) build_rows(tab_of(j + 1), win_of(j + 1));
    {  // pass 0: dV
      f32x16 acc[T::DB];
#pragma unroll
      for (int i = 0; i < T::DB; ++i) acc[i] = f32x16{};
      for (int it = 0; it < nit; ++it)
        dkdv_blocks<D, NW, 0, 0, 2, true>(buf(it), slb(j, it), kreg, vreg, acc, c1, l32, hf,
                                          lane);
      const float* add = p.G > 0 ? p.gv + ((int64_t)bh * p.G + cell_of(tab)) * D : nullptr;
      store_rows_u<D>(acc, 1.0f, add, p.dv + base, (uint32_t)tab[kcl] * stb, kvalid, hf);
    }
    {  // pass 1: dK; the next unit's tiles go into the buffers it leaves
      f32x16 acc[T::DB];
#pragma unroll
      for (int i = 0; i < T::DB; ++i) acc[i] = f32x16{};
      bool last_tile = false;   // PF 2: this wave loads the last tile after the epilogue
      for (int it = 0; it < nit; ++it) {
        dkdv_blocks<D, NW, 1, 0, 2, true>(buf(it), slb(j, it), kreg, vreg, acc, c1, l32, hf,
                                          lane);
        if (PF == 1 && has_next && it + 1 < nit) {
          __syncthreads();   // every wave is done with buffer it (and the next table is built)
          tiles(it, basen, tab_of(j + 1));
        }
        if (PF == 2 && has_next) {
          // This wave's reads of buffer it precede the count (LDS operations
          // of a wave run in order; the empty asm keeps the compiler from
          // moving them past it).  The wave whose count completes the tile
          // loads all of it; every wave built its rows of the next table
          // before its pass 0, and so before its count.
          asm volatile("" ::: "memory");
          int old = 0;
          if (lane == 0)
            old = __hip_atomic_fetch_add(cnt + it, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_WORKGROUP);
          old = __builtin_amdgcn_readfirstlane(old);
          if (old % NW == NW - 1) {
            if (it + 1 < nit) tile_part(it, 0, NW * Q::kIpw, basen, tab_of(j + 1));
            else last_tile = true;
          }
        }
      }
      // the epilogue's loads wait only for tile loads issued a tile earlier
      const float* add = p.G > 0 ? p.gk + ((int64_t)bh * p.G + cell_of(tab)) * D : nullptr;
      store_rows_u<D>(acc, p.scale, add, p.dk + base, (uint32_t)tab[kcl] * stb, kvalid, hf);
      if (last_tile) tile_part(nit - 1, 0, NW * Q::kIpw, basen, tab_of(j + 1));
    }
    if (has_next) {   // the next unit's tiles (without prefetch: all, PF 1: the last), K and
                      // V rows, lse and Dv
      if (PF == 0) {
        __syncthreads();   // every wave is done with the buffers
#pragma unroll
        for (int it = 0; it < kNB; ++it)
          if (it < nit) tiles(it, basen, tab_of(j + 1));
      }
      if (PF == 1) {
        __syncthreads();   // every wave is done with the last buffer
        tiles(nit - 1, basen, tab_of(j + 1));
      }
      rows(basen, tab_of(j + 1));   // this wave's own rows of the next table
      lsd = vec(bhn, tab_of(j + 1));
    }
  }
}

#ifndef BASA_BWD_RES_PERSISTENT
#define BASA_BWD_RES_PERSISTENT 1
#endif
template <int D>
__global__ void __launch_bounds__(kNW * 64, 1) bwd_dkdv_res_kernel(BwdParams p) {
  if constexpr (BASA_BWD_RES_PERSISTENT) dkdv_res_body<D>(p);
  else dkdv_body<D, false, 0, kNW, true>(p, blockIdx.x);
}

// ---------------------------------------------------------------- memsum
template <int D>
__global__ void __launch_bounds__(256) bwd_memsum_kernel(BwdParams p, float inv_cell) {
  // four consecutive d of one (b*h, memory key) per thread (G * D is a
  // multiple of 4, the buffers 16-byte aligned); the loads of four query
  // chunks go out together, and each element still sums the chunks in order
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;   // over bh, g, d
  const int64_t per = (int64_t)p.G * D;
  if (i >= (int64_t)p.batch_heads * per) return;
  const int64_t bh = i / per, rest = i - bh * per;
  const f32x4* pk = reinterpret_cast<const f32x4*>(p.pk + bh * p.nqc * per + rest);
  const f32x4* pv = reinterpret_cast<const f32x4*>(p.pv + bh * p.nqc * per + rest);
  const int64_t cs = per / 4;   // one query chunk's partials, in 4-float steps
  f32x4 sk = {}, sv = {};
  int c = 0;
  for (; c + 4 <= p.nqc; c += 4) {
    f32x4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = pk[(c + u) * cs];
      b[u] = pv[(c + u) * cs];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sk += a[u];
      sv += b[u];
    }
  }
  for (; c < p.nqc; ++c) {
    sk += pk[c * cs];
    sv += pv[c * cs];
  }
  *reinterpret_cast<f32x4*>(p.gk + i) = sk * p.scale * inv_cell;
  *reinterpret_cast<f32x4*>(p.gv + i) = sv * inv_cell;
}

template <typename K>
int set_lds(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return BASA_OK;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess
             ? BASA_OK
             : BASA_ERR_HIP;
}

template <int D, bool MEM>
int launch_dkdv(const BwdParams& p, hipStream_t stream) {
  if constexpr (!MEM && BASA_BWD_DKDV_RESIDENT && D == 128) {
    if (p.m > BASA_BWD_DKDV_WAVES * 32 && p.m <= kNW * 32) {
      constexpr int kNB = kNW * 32 / DqDma<D, kNW>::kKeys;
      // tile buffers with their lse / Dv, then one table; persistent: tile
      // buffers, two slots of lse / Dv arrays and of tables, finish counts
      const size_t lds = BASA_BWD_RES_PERSISTENT
          ? kNB * (2 * (size_t)DqDma<D, kNW>::kTileB + 2 * 2 * 64 * 4) + 2 * (size_t)kNW * 32 * 4 +
                kNB * 4
          : kNB * (2 * (size_t)DqDma<D, kNW>::kTileB + 2 * 64 * 4) + (size_t)p.m * 4;
      if (lds > 160 * 1024) return BASA_ERR_UNSUPPORTED;
      const int64_t units = (int64_t)p.batch_heads * p.nW;
      if (units > INT32_MAX / 4) return BASA_ERR_UNSUPPORTED;
      if (set_lds(&bwd_dkdv_res_kernel<D>, lds)) return BASA_ERR_HIP;
      // persistent: at most 32 workgroups per XCD (one per CU of an MI355X);
      // any count is correct, the workgroups share nothing
      const int64_t upx = (units + 7) / 8;
      const int64_t per_xcd = BASA_BWD_RES_PERSISTENT ? std::min<int64_t>(upx, 32) : upx;
      hipLaunchKernelGGL((bwd_dkdv_res_kernel<D>), dim3((unsigned)(8 * per_xcd)),
                         dim3(kNW * 64), lds, stream, p);
      return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
    }
  }
  constexpr int NW = MEM ? BASA_BWD_DKDV_MEM_WAVES : BASA_BWD_DKDV_WAVES, U = NW * 32;
  const size_t lds = 2 * (2 * (size_t)DqDma<D, NW>::kTileB + 2 * 64 * 4) + (MEM ? 0 : (size_t)p.m * 4);
  if (lds > 160 * 1024) return BASA_ERR_UNSUPPORTED;
  const int64_t units = MEM ? (int64_t)p.batch_heads * ((p.G + U - 1) / U) * p.nqc
                            : (int64_t)p.batch_heads * p.nW * ((p.m + U - 1) / U);
  if (units > INT32_MAX / 4) return BASA_ERR_UNSUPPORTED;
  if (set_lds(&bwd_dkdv_kernel<D, MEM, NW>, lds)) return BASA_ERR_HIP;
  const int64_t per_pass = 8 * ((units + 7) / 8);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, MEM, NW>), dim3((unsigned)(2 * per_pass)), dim3(NW * 64),
                     lds, stream, p, (int)per_pass);
  return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

template <int D>
int launch_d(const BwdParams& p, hipStream_t stream) {
  using T = BT<D>;
  {
    constexpr int CPR = D / 8, RPW = 64 / CPR;
    const int64_t rows = (int64_t)p.batch_heads * p.n;
    const int64_t blocks = (rows + 4 * RPW - 1) / (4 * RPW);
    hipLaunchKernelGGL((bwd_dvec_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return BASA_ERR_HIP;
  }
  int rc;
  if (p.G > 0) {
    if ((rc = launch_dkdv<D, true>(p, stream))) return rc;
    const int64_t total = (int64_t)p.batch_heads * p.G * D;
    hipLaunchKernelGGL((bwd_memsum_kernel<D>), dim3((unsigned)((total / 4 + 255) / 256)), dim3(256), 0,
                       stream, p, 1.0f / (float)(p.pt * p.py * p.px));
    if (hipGetLastError() != hipSuccess) return BASA_ERR_HIP;
  }
  if ((rc = launch_dkdv<D, false>(p, stream))) return rc;
  {
    constexpr int NW = BASA_BWD_DQ_WAVES;
    const int64_t units = (int64_t)p.batch_heads * p.nW * ((p.m + NW * 32 - 1) / (NW * 32));
    const int64_t upx = (units + 7) / 8;
    const size_t lds = 4 * (size_t)DqDma<D, NW>::kTileB + (size_t)p.m * 4;
    if (lds > 160 * 1024) return BASA_ERR_UNSUPPORTED;
    if (set_lds(&bwd_dq_kernel<D, NW>, lds)) return BASA_ERR_HIP;
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW>), dim3((unsigned)(8 * upx)), dim3(NW * 64), lds,
                       stream, p);
    if (hipGetLastError() != hipSuccess) return BASA_ERR_HIP;
  }
  return BASA_OK;
}

}  // namespace

int launch_attn_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.head_dim == 128) return launch_d<128>(p, stream);
  if (p.head_dim == 64) return launch_d<64>(p, stream);
  return BASA_ERR_UNSUPPORTED;
}

}  // namespace basa
