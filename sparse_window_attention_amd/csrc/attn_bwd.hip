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
// Kernels (one workgroup of 8 waves per unit, XCD-aware unit order):
//   dvec     Dv for every token
//   dq       query-stationary: 256 queries of a window against the key
//            sequence [window keys; memory keys] in tiles of 64 keys loaded
//            straight into LDS: S^T = K Q^T, dP^T = V dO^T, dS^T,
//            dQ^T += K^T dS^T (K^T by transposing LDS reads)
//   dkdv     key-stationary: 256 keys (32 per wave) against blocks of 32
//            queries: S = Q K^T, P; pass 0: dV^T += dO^T P; pass 1:
//            dP = dO V^T, dS, dK^T += Q^T dS.  Both passes run in one grid
//            (one launch for memory keys, one for window keys).  Memory-key
//            units cover one chunk of the head's queries each and write fp32
//            partial sums; window-key units write the final dK, dV of their
//            tokens, adding the pooled memory gradient of the token's cell.
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

constexpr int kNW = 8;                 // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr int kBlk = 32;               // rows of one MFMA block: keys (dq), queries (dkdv)
constexpr int kUnit = kNW * 32;        // queries per dq unit, keys per dkdv unit

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

// ---------------------------------------------------------------- dq
// dQ with the key tiles loaded straight into LDS: 64 keys per iteration, K
// and V tiles row-major (16-byte chunks XOR-swizzled per row), K rows and V
// rows read as MFMA operands and K^T read with the transposing LDS read.  One
// swizzle serves both reads of the K tile: chunk c of row r sits at slot
// c ^ f(r), f a bijection of r mod 16 whose bits 2-3 separate any 4
// consecutive rows, so the 16 rows of a quarter-wave row read and the
// 4 rows x 4 chunks of a half-wave transposing read fall in distinct banks.
template <int D>
struct DqDma {
  using T = BT<D>;
  static constexpr int kKeys = 64;                  // keys per iteration
  static constexpr int CPR = D / 8;
  static constexpr int RowB = CPR * 16;             // bytes per row
  static constexpr int kTileB = kKeys * RowB;       // one K or V tile
  static constexpr int kIpw = kTileB / 1024 / kNW;  // 1 KB loads per wave and tile
  static_assert(kIpw >= 1 && kIpw * kNW * 1024 == kTileB, "tile must split over the waves");
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
};

template <int D>
__global__ void __launch_bounds__(kThreads, 1) bwd_dq_kernel(BwdParams p) {
  using T = BT<D>;
  using Q = DqDma<D>;
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
  // this wave's share of the loads of iteration it's K and V tiles
  auto dma = [&](int it) __attribute__((always_inline)) {
    const int k0 = it * Q::kKeys;
    unsigned char* bk = smem + (it & 1) * KTB;
    unsigned char* bv = smem + (2 + (it & 1)) * KTB;
    const bool winT = k0 + Q::kKeys <= p.m;
    const bool memT = k0 >= p.m && k0 + Q::kKeys <= L;
    // window tiles: all table reads first (one LDS wait), then the loads
    uint32_t toff[Q::kIpw];
#pragma unroll
    for (int i = 0; i < Q::kIpw; ++i) {
      const int r = ((wv * Q::kIpw + i) * 64 + lane) / CPR;
      toff[i] = winT ? (uint32_t)tab[k0 + r] * stb : 0u;
    }
#pragma unroll
    for (int i = 0; i < Q::kIpw; ++i) {
      const int ins = wv * Q::kIpw + i;
      const int r = (ins * 64 + lane) / CPR;
      const uint32_t cb = (uint32_t)(((lane % CPR) ^ Q::swz(r)) * 16);
      auto* lk = (__attribute__((address_space(3))) void*)(bk + ins * 1024);
      auto* lv = (__attribute__((address_space(3))) void*)(bv + ins * 1024);
      if (winT) {
        const uint32_t off = toff[i] + cb;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p.k + base), lk, 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p.v + base), lv, 16, off, 0, 0, 0);
      } else if (memT) {
        const uint32_t off = (uint32_t)(k0 - p.m + r) * (D * 2) + cb;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(kmem), lk, 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(vmem), lv, 16, off, 0, 0, 0);
      } else {
        const int key = min(k0 + r, L - 1);   // rows past the end: clamped, masked below
        const char* gk;
        const char* gvp;
        if (key < p.m) {
          const int64_t o = (int64_t)tab[key] * stb + cb;
          gk = reinterpret_cast<const char*>(p.k + base) + o;
          gvp = reinterpret_cast<const char*>(p.v + base) + o;
        } else {
          const int64_t o = (int64_t)(key - p.m) * (D * 2) + cb;
          gk = reinterpret_cast<const char*>(kmem) + o;
          gvp = reinterpret_cast<const char*>(vmem) + o;
        }
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gk, lk, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gvp, lv, 16, 0, 0);
      }
    }
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
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * u + j;
          const int key = it * Q::kKeys + kb * 32 + acc_row(r, hf);
          float xv = s[r] + (key >= p.m ? p.mem_bias_raw : 0.0f);
          xv = key < L ? xv : -INFINITY;
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(xv, c1, -lse2));
          e[j] = pr * (dp[r] - dval);
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
template <int D, bool MEM, int PASS>
__device__ __forceinline__ void dkdv_body(const BwdParams& p, int blk) {
  using T = BT<D>;
  using Q = DqDma<D>;
  constexpr int CPR = Q::CPR, RowB = Q::RowB, TB = Q::kTileB;
  constexpr int kQ = Q::kKeys;                 // queries per iteration
  constexpr int kBufB = 2 * TB + 2 * kQ * 4;   // Q tile, dO tile, lse and Dv
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
  int32_t* tab = reinterpret_cast<int32_t*>(smem + 2 * kBufB);
  if constexpr (!MEM) {
    for (int r = tid; r < p.m; r += kThreads) tab[r] = window_token(p.geo, win, r);
    __syncthreads();
  }

  // this lane's key: K (and V) rows as B operands
  const int key = kbase + wave * 32 + l32;
  const bool kvalid = key < nkeys;
  const int kcl = min(key, nkeys - 1);
  u32x4 kreg[T::QS], vreg[PASS == 1 ? T::QS : 1];
  {
    const uint16_t* ks = MEM ? p.kmem + (int64_t)bh * p.G * D : p.k + base;
    const uint16_t* vs = MEM ? p.vmem + (int64_t)bh * p.G * D : p.v + base;
    const uint32_t koff = MEM ? (uint32_t)kcl * (D * 2) : (uint32_t)tab[kcl] * stb;
    const Rsrc rk = make_rsrc(ks), rv = make_rsrc(vs);
#pragma unroll
    for (int s = 0; s < T::QS; ++s) {
      kreg[s] = buf_load16(rk, koff + hf * D + s * 16, 0);
      if constexpr (PASS == 1) vreg[s] = buf_load16(rv, koff + hf * D + s * 16, 0);
    }
  }
  f32x16 acc[T::DB];
#pragma unroll
  for (int i = 0; i < T::DB; ++i) acc[i] = f32x16{};

  const int nit = (nq + kQ - 1) / kQ;
  auto token_of = [&](int q) __attribute__((always_inline)) {
    return MEM ? qbase + q : tab[q];
  };
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  float lx = INFINITY, dvx = 0.0f;
  // this wave's share of the Q and dO tile loads of iteration it; lse and Dv
  // of the iteration's queries into registers (stored by `put`)
  auto get = [&](int it) __attribute__((always_inline)) {
    unsigned char* b = smem + (it & 1) * kBufB;
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
      lx = ok ? p.lse[idx] * kLog2e : INFINITY;   // a missing query gets P = 0
      dvx = ok ? p.dvec[idx] : 0.0f;
    }
  };
  auto put = [&](int it) __attribute__((always_inline)) {
    if (tid < kQ) {
      float* sl = reinterpret_cast<float*>(smem + (it & 1) * kBufB + 2 * TB);
      sl[(tid / kBlk) * 64 + perm32(tid % kBlk)] = lx;
      sl[(tid / kBlk) * 64 + 32 + perm32(tid % kBlk)] = dvx;
    }
  };
  get(0);
  put(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's tile loads are in LDS
  __syncthreads();
  const float c1 = p.c1;
  const float bias = MEM ? p.mem_bias_raw : 0.0f;
  const int x = Q::swz(l32);
  const int sq = (lane & 15) >> 2;
  const int d0 = 16 * (l32 >> 4) + 4 * (lane & 3);
  for (int it = 0; it < nit; ++it) {
    if (it + 1 < nit) get(it + 1);
    const unsigned char* sqt = smem + (it & 1) * kBufB;   // Q tile
    const unsigned char* sdo = sqt + TB;                  // dO tile
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float* sl = reinterpret_cast<const float*>(sqt + 2 * TB) + kb * 64;
      f32x16 s{};
#pragma unroll
      for (int ss = 0; ss < T::QS; ++ss) {
        const int off = (kb * 32 + l32) * RowB + (((hf * (CPR / 2) + ss) ^ x) * 16);
        s = mfma(*reinterpret_cast<const u32x4*>(sqt + off), kreg[ss], s);
      }
      float pr[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + hf * 16 + r4 * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pr[4 * r4 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * r4 + i] + bias, c1, -l4[i]));
      }
      float w[16];   // pass 0: P; pass 1: dS
      if constexpr (PASS == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i] = pr[i];
      } else {
        f32x16 dp{};
#pragma unroll
        for (int ss = 0; ss < T::QS; ++ss) {
          const int off = (kb * 32 + l32) * RowB + (((hf * (CPR / 2) + ss) ^ x) * 16);
          dp = mfma(*reinterpret_cast<const u32x4*>(sdo + off), vreg[ss], dp);
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(sl + 32 + hf * 16 + r4 * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) w[4 * r4 + i] = pr[4 * r4 + i] * (dp[4 * r4 + i] - d4[i]);
        }
      }
      // pass 0: dV^T += dO^T P; pass 1: dK^T += Q^T dS -- the transposed
      // operand by transposing reads of the row-major tile
      const unsigned char* tt = PASS == 0 ? sdo : sqt;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 pb{pack_bf16x2(w[8 * u], w[8 * u + 1]), pack_bf16x2(w[8 * u + 2], w[8 * u + 3]),
                       pack_bf16x2(w[8 * u + 4], w[8 * u + 5]), pack_bf16x2(w[8 * u + 6], w[8 * u + 7])};
        const int slc = 2 * kb + u;
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          bf16x4 h2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = 16 * slc + 8 * h + 4 * hf + sq;
            const int d = 32 * db + d0;
            h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(
                tt + row * RowB + (((d >> 3) ^ Q::swz(row)) * 16) + (d & 7) * 2));
          }
          const bf16x8 av = {h2[0][0], h2[0][1], h2[0][2], h2[0][3],
                             h2[1][0], h2[1][1], h2[1][2], h2[1][3]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, pb),
                                                           acc[db], 0, 0, 0);
        }
      }
    }
    if (it + 1 < nit) put(it + 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's loads of the next tiles
    __syncthreads();
  }

  if constexpr (MEM) {
    // fp32 partials [bh][qc][key][d]; lane = key, registers = 4 consecutive d
    if (kvalid) {
      const int qc = qbase / p.qchunk;
      float* dst = (PASS == 0 ? p.pv : p.pk) + (((int64_t)bh * p.nqc + qc) * p.G + key) * D;
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
    if (p.G > 0) {
      const int xx = tok % p.geo.Wg;
      const int y = (tok / p.geo.Wg) % p.geo.Hg;
      const int t = tok / (p.geo.Wg * p.geo.Hg);
      const int cell = ((t / p.pt) * p.Gy + y / p.py) * p.Gx + xx / p.px;
      add = (PASS == 0 ? p.gv : p.gk) + ((int64_t)bh * p.G + cell) * D;
    }
    store_rows<D>(acc, PASS == 0 ? 1.0f : p.scale, add, (PASS == 0 ? p.dv : p.dk) + base,
                  (uint32_t)tok * stb, kvalid, hf);
  }
}

// Both passes in one grid: workgroups [0, split) run pass 0 (dV), the rest
// pass 1 (dK); split is a multiple of 8.  One launch lets the second pass
// fill the CUs the first leaves idle at its end.
template <int D, bool MEM>
__global__ void __launch_bounds__(kThreads, 1) bwd_dkdv_kernel(BwdParams p, int split) {
  if ((int)blockIdx.x < split) dkdv_body<D, MEM, 0>(p, blockIdx.x);
  else dkdv_body<D, MEM, 1>(p, blockIdx.x - split);
}

// ---------------------------------------------------------------- memsum
template <int D>
__global__ void __launch_bounds__(256) bwd_memsum_kernel(BwdParams p, float inv_cell) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // over bh, g, d
  const int64_t per = (int64_t)p.G * D;
  if (i >= (int64_t)p.batch_heads * per) return;
  const int64_t bh = i / per, rest = i - bh * per;
  float sk = 0.0f, sv = 0.0f;
  for (int c = 0; c < p.nqc; ++c) {
    const int64_t j = (bh * p.nqc + c) * per + rest;
    sk += p.pk[j];
    sv += p.pv[j];
  }
  p.gk[i] = sk * p.scale * inv_cell;
  p.gv[i] = sv * inv_cell;
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
  const size_t lds = 2 * (2 * (size_t)DqDma<D>::kTileB + 2 * 64 * 4) + (MEM ? 0 : (size_t)p.m * 4);
  if (lds > 160 * 1024) return BASA_ERR_UNSUPPORTED;
  const int64_t units = MEM ? (int64_t)p.batch_heads * ((p.G + kUnit - 1) / kUnit) * p.nqc
                            : (int64_t)p.batch_heads * p.nW * ((p.m + kUnit - 1) / kUnit);
  if (units > INT32_MAX / 4) return BASA_ERR_UNSUPPORTED;
  if (set_lds(&bwd_dkdv_kernel<D, MEM>, lds)) return BASA_ERR_HIP;
  const int64_t per_pass = 8 * ((units + 7) / 8);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, MEM>), dim3((unsigned)(2 * per_pass)), dim3(kThreads), lds,
                     stream, p, (int)per_pass);
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
    hipLaunchKernelGGL((bwd_memsum_kernel<D>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, p, 1.0f / (float)(p.pt * p.py * p.px));
    if (hipGetLastError() != hipSuccess) return BASA_ERR_HIP;
  }
  if ((rc = launch_dkdv<D, false>(p, stream))) return rc;
  {
    const int64_t units = (int64_t)p.batch_heads * p.nW * ((p.m + kUnit - 1) / kUnit);
    const int64_t upx = (units + 7) / 8;
    const size_t lds = 4 * (size_t)DqDma<D>::kTileB + (size_t)p.m * 4;
    if (lds > 160 * 1024) return BASA_ERR_UNSUPPORTED;
    if (set_lds(&bwd_dq_kernel<D>, lds)) return BASA_ERR_HIP;
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)(8 * upx)), dim3(kThreads), lds,
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
