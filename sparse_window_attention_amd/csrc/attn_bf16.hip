// bf16 window / full attention on gfx950 matrix cores.
//
// A work unit is kQT query rows of one window of one (batch, head).  The
// window's keys and the pooled memory keys form one virtual key sequence
// [window keys; memory keys] of length L = m + G, streamed through LDS in
// tiles of kKT keys.  Each wave owns QB blocks of 32 query rows; per tile:
//   S^T = K Q^T        (32x32x16 bf16 MFMA, keys x queries, fp32 accumulate)
//   online softmax     (fp32, base 2; the row max needs one lane swap since a
//                       lane holds 16 keys of one query)
//   O^T += V^T P^T     (32x32x16 bf16 MFMA, P rounded to bf16)
// Computing S transposed puts every query in one lane pair, so the softmax
// reductions stay in registers, and the fp32 scores already sit in the
// operand layout the P V product needs (no shuffles).  Every K or V operand
// read from LDS feeds the QB query blocks of the wave.
//
// The loop is software-pipelined inside each wave: while the exponentials of
// tile t are computed on the vector ALU, the matrix core already runs
// K(t+1) Q^T, and the row max of tile t+1 overlaps the P V product of tile
// t.  K runs one tile ahead of V through two LDS buffers each.
//
// Two kernels share this core.  The unit kernel runs one workgroup per work
// unit and stages tiles through registers (V written transposed).  The
// persistent kernel (used when a unit has at least kPersistentMinTiles tiles
// and its LDS fits) runs one workgroup per CU that walks a list of units of
// one XCD with the same tile loop; it loads K/V tiles straight from global
// memory into LDS (row-major, XOR-swizzled rows) and reads V^T with the
// transposing LDS read.  While a unit runs, the next unit's first three K/V
// tiles are loaded into free tile buffers and its Q rows into a per-wave LDS
// staging area, so the next unit starts from LDS instead of paying a burst
// of HBM loads; the finished unit's output is stored once the next unit's
// first scores are formed, passing through the wave's staging area so that
// every store writes whole rows (non-temporal: the output drains to HBM while
// the kernel runs).
//
// The cyclic shift and the window gather are address arithmetic: a table of
// the window's raster offsets is built in LDS per unit and every Q/K/V/O row
// is addressed through it (BASA forum summary, "The BASA Method": shift,
// partition, attend, shift back -- here without any copy).  Memory keys
// (BASA discussion reply, the four parts of the method: a global memory of
// pooled K/V) are plain rows of the [B,H,G,D] memory tensors.
#include <type_traits>

#include "basa_common.h"
#include "basa_internal.h"

namespace basa {

namespace {

constexpr float kRescaleSlack = 8.0f; // log2 units the stale max may lag
constexpr int kStoreNT = 2;            // cache policy of buffer stores: non-temporal
// Cache policy of the loads of data read once per unit (its Q rows, its
// window's K and V tiles): non-temporal, leaving the caches to the memory
// keys, which every unit of the head reads again.
constexpr int kLoadOnce = 2;
constexpr int kPersistentMinTiles = 4;  // tiles per unit the persistent kernel needs
// Persistent kernel: LDS operand reads this many MFMA steps ahead (score
// product, P V product).
#ifndef BASA_OPERAND_AHEAD
#define BASA_OPERAND_AHEAD 2
#endif
#ifndef BASA_OPERAND_AHEAD_PV
#define BASA_OPERAND_AHEAD_PV BASA_OPERAND_AHEAD
#endif
// Persistent kernel: waves per workgroup and workgroups per CU.
#ifndef BASA_PERSISTENT_WAVES
#define BASA_PERSISTENT_WAVES 8
#endif
#ifndef BASA_PERSISTENT_WGS
#define BASA_PERSISTENT_WGS 1
#endif
// Persistent kernel with direct tile loads: K tile buffers (2 or 3).  With
// three, the K tile of position t+4 is loaded during iteration t and waited
// for only at the end of iteration t+2 (two iterations of load latency
// hidden instead of one); V keeps two buffers.  Three measured 1-3% slower
// than two (the tile loads are not late), so two is the default.
#ifndef BASA_K_DEPTH
#define BASA_K_DEPTH 2
#endif
// Persistent kernel: spread the tiles of window keys among the tiles of
// memory keys (1) or take the key tiles in key order (0).
#ifndef BASA_TILE_INTERLEAVE
#define BASA_TILE_INTERLEAVE 0
#endif
// Persistent kernel: stage the next unit's Q rows in LDS (1) or load them
// into registers at the unit boundary (0).
#ifndef BASA_PERSISTENT_QSTAGE
#define BASA_PERSISTENT_QSTAGE 1
#endif

template <int D, int NW, int QB, int KT>
struct Tiles {
  static constexpr int kKT = KT;                  // keys per tile
  static constexpr int KB = KT / 32;              // 32-key blocks per tile
  static constexpr int kThreads = NW * 64;
  static constexpr int kQPW = 32 * QB;            // query rows per wave
  static constexpr int kQT = NW * kQPW;           // query rows per unit
  static constexpr int KS = D + 8;    // K tile row stride (bf16), 16B aligned, skewed banks
  static constexpr int VS = kKT + 8;  // transposed V tile row stride (bf16)
  static constexpr int kBytes = kKT * KS * 2;
  static constexpr int vBytes = D * VS * 2;
  static constexpr int tileBytes = 2 * kBytes + 2 * vBytes;
  static constexpr int CPR = D / 8;               // 16B chunks per row
  static constexpr int RPP = kThreads / CPR;      // K rows per load pass
  static constexpr int KPASS = kKT / RPP;         // K load passes per tile
  static constexpr int KPT = kKT * D / (kThreads * 8);  // V keys per thread
  static_assert(KPASS >= 1 && KPASS * RPP == kKT, "K tile must split evenly over the threads");
  static_assert(KPT >= 1 && KPT <= 4 && KPT * kThreads * 8 == kKT * D,
                "V tile must split evenly over the threads");
};

template <bool B>
using bool_c = std::integral_constant<bool, B>;

// One work unit: element offset of its (batch, head) slice in Q/O (and, for
// window attention, K/V), the same in K/V for dense attention, its (batch,
// head) index, window and query tile.
struct Unit {
  int64_t base;
  int64_t kvbase;
  int bh;
  int win;
  int qt;
};

__device__ __forceinline__ Unit decode_unit(const AttnParams& p, int unit) {
  Unit u;
  u.qt = unit % p.nQT;
  const int rest = unit / p.nQT;
  u.win = rest % p.nW;
  u.bh = rest / p.nW;
  const int b = u.bh / p.heads, h = u.bh - b * p.heads;
  u.base = (int64_t)b * p.stride_b + (int64_t)h * p.stride_h;
  u.kvbase = (int64_t)b * p.kv_stride_b + (int64_t)h * p.kv_stride_h;
  return u;
}

// Everything one wave keeps for the attention of its query rows, and the
// tile staging of the whole workgroup.
template <int D, bool FULL, int NW, int QB, int KT>
struct Core {
  using TL = Tiles<D, NW, QB, KT>;
  static constexpr int kKT = KT;
  static constexpr int KB = TL::KB;
  static constexpr int QS = D / 16;   // MFMA k-steps over the head dim
  static constexpr int DB = D / 32;   // 32-row blocks of O^T
  using Scores = f32x16[QB][KB];      // S^T of one tile: [query block][32-key block]
  using Probs = u32x4[QB][2 * KB];    // bf16 P^T operands: [query block][16-key slice]

  const AttnParams& p;
  unsigned char* smem;
  int tid, wave, l32, hf;
  int m, L, tmask, nkt;
  uint32_t stb;                       // bytes between tokens
  float c1, bias;
  int kc, kr0, va, vc;                // tile loader geometry
  u32x4 qreg[QB][QS];                 // Q rows (B operand of K Q^T)
  u32x4 kreg[TL::KPASS];              // staged K rows
  u32x4 vreg[TL::KPT];                // staged V rows
  f32x16 acc[QB][DB];                 // O^T accumulators
  float m_used[QB];                   // lagging max (log2 units)
  float l0[QB], l1[QB];               // this lane's row sum halves

  __device__ __forceinline__ Core(const AttnParams& pp, unsigned char* sm) : p(pp), smem(sm) {
    tid = threadIdx.x;
    const int lane = tid & 63;
    wave = tid >> 6;
    l32 = lane & 31;
    hf = lane >> 5;
    m = p.m;
    L = FULL ? p.n_kv : m + p.G;
    stb = (uint32_t)p.stride_tok * 2u;
    c1 = p.c1;
    bias = p.mem_bias_raw;
    kc = tid % TL::CPR;
    kr0 = tid / TL::CPR;
    va = tid % (kKT / TL::KPT);
    vc = tid / (kKT / TL::KPT);
    nkt = (L + kKT - 1) / kKT;
    // first tile whose scores need the mask (memory-key bias or padding)
    tmask = nkt;
    if (bias != 0.0f) tmask = m / kKT;
    if (L % kKT) tmask = min(tmask, nkt - 1);
  }

  // Marks the per-lane indices as redefined here.  Addresses derived from
  // them are then formed after this point instead of being hoisted out of an
  // enclosing loop and held in registers through it.
  __device__ __forceinline__ void redefine_lane_ids() {
    asm volatile("" : "+v"(tid), "+v"(l32), "+v"(hf), "+v"(kc), "+v"(kr0), "+v"(va), "+v"(vc));
    asm volatile("" : "+s"(m), "+s"(L), "+s"(stb), "+s"(c1), "+s"(bias));
  }

  __device__ __forceinline__ uint16_t* sK(int buf) const {
    return reinterpret_cast<uint16_t*>(smem + buf * TL::kBytes);
  }
  __device__ __forceinline__ uint16_t* sV(int buf) const {
    return reinterpret_cast<uint16_t*>(smem + 2 * TL::kBytes + buf * TL::vBytes);
  }
  __device__ __forceinline__ uint32_t* table() const {
    return reinterpret_cast<uint32_t*>(smem + TL::tileBytes);
  }

  // byte offsets of the window's tokens inside the (batch, head) slice
  __device__ __forceinline__ void build_table(uint32_t* t, int win) const {
    for (int r = tid; r < m; r += TL::kThreads) t[r] = (uint32_t)slot_token(p, win, r) * stb;
  }
  // byte offset of slot r of the unit's window (identity map for full attention)
  __device__ __forceinline__ uint32_t tok(const uint32_t* t, int r) const {
    return FULL ? (uint32_t)r * stb : t[r];
  }
  // element offset of the unit's (batch, head) slice of K and V
  __device__ __forceinline__ int64_t kvb(const Unit& u) const { return FULL ? u.kvbase : u.base; }

  // ---- tile loader (global -> registers -> LDS).  Keys past the end are
  // clamped to the last key: those rows load valid data that the score mask
  // removes.  Keys stay below 2^24 and offsets below 2^31 (checked on the
  // host), so 24-bit multiplies form the offsets.
  __device__ __forceinline__ const char* row_ptr(const Unit& u, const uint32_t* t, int key,
                                                  bool isv) const {
    key = min(key, L - 1);
    const char* g = reinterpret_cast<const char*>((isv ? p.v : p.k) + kvb(u));
    if constexpr (FULL) return g + (uint32_t)key * stb;
    const char* gm = reinterpret_cast<const char*>((isv ? p.vmem : p.kmem) + (int64_t)u.bh * p.G * D);
    const bool inwin = key < m;
    const uint32_t off = t[inwin ? key : 0];
    const uint32_t moff = (uint32_t)__mul24(inwin ? 0 : key - m, D * 2);
    return inwin ? g + off : gm + moff;
  }
  // Whole-tile address paths: tiles of window keys read the offset table,
  // tiles of memory keys are plain rows; only tiles straddling the window /
  // memory boundary or the end take the general per-row selects.
  template <int N>
  __device__ __forceinline__ void load_rows(u32x4 (&dst)[N], const Unit& u, const uint32_t* t,
                                            int tile, int r0, int rstep, int chunk,
                                            bool isv) const {
    const int k0 = tile * kKT;
    const uint32_t cb = (uint32_t)chunk * 16u;
    if constexpr (FULL) {
      const Rsrc rs = make_rsrc((isv ? p.v : p.k) + kvb(u));
#pragma unroll
      for (int i = 0; i < N; ++i)
        dst[i] = buf_load16(rs, (uint32_t)min(k0 + r0 + i * rstep, L - 1) * stb + cb, 0);
    } else {
      if (k0 + kKT <= m) {
        const Rsrc rs = make_rsrc((isv ? p.v : p.k) + kvb(u));
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = buf_load16(rs, t[k0 + r0 + i * rstep] + cb, 0);
        return;
      }
      if (k0 >= m && k0 + kKT <= L) {
        const Rsrc rs = make_rsrc((isv ? p.vmem : p.kmem) + (int64_t)u.bh * p.G * D);
        const uint32_t so = (uint32_t)(k0 - m) * (D * 2);
#pragma unroll
        for (int i = 0; i < N; ++i)
          dst[i] = buf_load16(rs, (uint32_t)(r0 + i * rstep) * (D * 2) + cb, so);
        return;
      }
#pragma unroll
      for (int i = 0; i < N; ++i)
        dst[i] = *reinterpret_cast<const u32x4*>(row_ptr(u, t, k0 + r0 + i * rstep, isv) + cb);
    }
  }
  __device__ __forceinline__ void load_k(const Unit& u, const uint32_t* t, int tile) {
    load_rows(kreg, u, t, tile, kr0, TL::RPP, kc, false);
  }
  __device__ __forceinline__ void load_k_to(u32x4 (&dst)[TL::KPASS], const Unit& u,
                                            const uint32_t* t, int tile) const {
    load_rows(dst, u, t, tile, kr0, TL::RPP, kc, false);
  }
  __device__ __forceinline__ void load_v(const Unit& u, const uint32_t* t, int tile) {
    load_rows(vreg, u, t, tile, va * TL::KPT, 1, vc, true);
  }
  __device__ __forceinline__ void store_k_from(const u32x4 (&src)[TL::KPASS], int buf) const {
    uint16_t* dst = sK(buf);
#pragma unroll
    for (int i = 0; i < TL::KPASS; ++i)
      *reinterpret_cast<u32x4*>(dst + (kr0 + i * TL::RPP) * TL::KS + kc * 8) = src[i];
  }
  __device__ __forceinline__ void store_k(int buf) const { store_k_from(kreg, buf); }
  // transpose: for each of the 8 d of this thread's chunk, its KPT keys side by side
  __device__ __forceinline__ void store_v(int buf) const {
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
  }

  // ---- direct global-to-LDS tile path (persistent kernel).  A K or V tile
  // is kKT rows of D bf16, stored row-major without padding by 1 KB
  // buffer-to-LDS loads (64 lanes x 16 bytes each).  The 16-byte chunks of
  // every row are permuted by an XOR with a function of the row, chosen so
  // that the operand reads below spread over all LDS banks: for K, the 16
  // rows read by a quarter wave land in 16 distinct chunk slots; for V, the
  // 4 rows x 4 chunks read by a half wave do.  The chunk a lane fetches from
  // global memory is the one its fixed LDS slot must hold.
  static constexpr int kTileB = kKT * D * 2;    // bytes of one K or V tile
  static constexpr int RPB = 16 / TL::CPR;      // rows per 256 bytes
  static constexpr int kDmaIns = kTileB / 1024; // load instructions per tile
  static constexpr int kDmaIpw = kDmaIns / NW;  // per wave
  static_assert(kDmaIpw >= 1 && kDmaIpw * NW == kDmaIns, "tile must split over the waves");
  __device__ static __forceinline__ int swz_k(int r) { return (r / RPB) & (TL::CPR - 1); }
  __device__ static __forceinline__ int swz_v(int r) { return (4 * (r / RPB)) & (TL::CPR - 4); }

  // Issues this wave's share of the loads of a V tile and a K tile (either
  // may be skipped) into their buffers.  The tile kind is decided once per
  // tile, and the window-offset table reads of both tiles go out before any
  // load, so one wait on LDS covers them.
  __device__ __forceinline__ void dma_pair(bool dv, unsigned char* bv, const Unit& uv,
                                           const uint32_t* tv, int tilev, bool dk,
                                           unsigned char* bk, const Unit& uk, const uint32_t* tk,
                                           int tilek) const {
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    int r[kDmaIpw];
#pragma unroll
    for (int i = 0; i < kDmaIpw; ++i) r[i] = ((wv * kDmaIpw + i) * 64 + lane) / TL::CPR;
    const int kv0 = tilev * kKT, kk0 = tilek * kKT;
    const bool winv = !FULL && kv0 + kKT <= m, wink = !FULL && kk0 + kKT <= m;
    uint32_t ov[kDmaIpw], ok[kDmaIpw];
#pragma unroll
    for (int i = 0; i < kDmaIpw; ++i) {
      ov[i] = (dv && winv) ? tv[kv0 + r[i]] : 0u;
      ok[i] = (dk && wink) ? tk[kk0 + r[i]] : 0u;
    }
    if (dv) dma_issue(bv, uv, tv, kv0, true, r, ov);
    if (dk) dma_issue(bk, uk, tk, kk0, false, r, ok);
  }
  __device__ __forceinline__ void dma_issue(unsigned char* buf, const Unit& u, const uint32_t* t,
                                            int k0, bool isv, const int (&r)[kDmaIpw],
                                            const uint32_t (&off)[kDmaIpw]) const {
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t cb[kDmaIpw];
#pragma unroll
    for (int i = 0; i < kDmaIpw; ++i)
      cb[i] = (uint32_t)(((lane % TL::CPR) ^ (isv ? swz_v(r[i]) : swz_k(r[i]))) * 16);
    auto lds = [&](int i) __attribute__((always_inline)) {
      return (__attribute__((address_space(3))) void*)(buf + (wv * kDmaIpw + i) * 1024);
    };
    if constexpr (FULL) {
      const Rsrc rs = make_rsrc((isv ? p.v : p.k) + kvb(u));
#pragma unroll
      for (int i = 0; i < kDmaIpw; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds(i), 16,
                                                 (uint32_t)min(k0 + r[i], L - 1) * stb + cb[i], 0, 0, 0);
    } else if (k0 + kKT <= m) {
      const Rsrc rs = make_rsrc((isv ? p.v : p.k) + kvb(u));
#pragma unroll
      for (int i = 0; i < kDmaIpw; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds(i), 16, off[i] + cb[i], 0, 0, kLoadOnce);
    } else if (k0 >= m && k0 + kKT <= L) {
      const Rsrc rs = make_rsrc((isv ? p.vmem : p.kmem) + (int64_t)u.bh * p.G * D);
#pragma unroll
      for (int i = 0; i < kDmaIpw; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds(i), 16, (uint32_t)r[i] * (D * 2) + cb[i],
                                                 (uint32_t)(k0 - m) * (D * 2), 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < kDmaIpw; ++i)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(row_ptr(u, t, k0 + r[i], isv) + cb[i]),
            lds(i), 16, 0, 0);
    }
  }
  __device__ __forceinline__ void dma_tile(unsigned char* buf, const Unit& u, const uint32_t* t,
                                           int tile, bool isv) const {
    if (isv) dma_pair(true, buf, u, t, tile, false, buf, u, t, 0);
    else dma_pair(false, buf, u, t, 0, true, buf, u, t, tile);
  }
  // S^T = K Q^T with K from a swizzled tile.  Row kb*32 + l32 has the
  // swizzle x of row l32 (32 rows span whole swizzle periods); chunk
  // hf*CPR/2 + ss sits at slot (hf*CPR/2 + ss) ^ x, so the byte offset is one
  // lane base XOR 16*ss, and kb and the buffer are immediate offsets.
  __device__ __forceinline__ void compute_s_dma(const unsigned char* kt, Scores& s) const {
    const f32x16 zero16 = {};
    constexpr int H = TL::CPR / 2;
    const int x = swz_k(l32);
    const uint32_t kbase = (uint32_t)(l32 * (TL::CPR * 16) + 16 * ((hf * H) ^ (x & H)) + 16 * (x & (H - 1)));
    // operands are read kAhead steps before their products
    constexpr int kAhead = BASA_OPERAND_AHEAD;
    u32x4 a[kAhead + 1][KB];
    auto rd = [&](int ss, int slot) __attribute__((always_inline)) {
      const uint32_t off = kbase ^ (uint32_t)(16 * ss);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        a[slot][kb] = *reinterpret_cast<const u32x4*>(kt + off + kb * 32 * (TL::CPR * 16));
    };
#pragma unroll
    for (int i = 0; i < kAhead && i < QS; ++i) rd(i, i);
#pragma unroll
    for (int ss = 0; ss < QS; ++ss) {
      if (ss + kAhead < QS) rd(ss + kAhead, (ss + kAhead) % (kAhead + 1));
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a[ss % (kAhead + 1)][kb]),
              __builtin_bit_cast(bf16x8, qreg[qb][ss]), ss == 0 ? zero16 : s[qb][kb], 0, 0, 0);
      }
    }
  }
  // O^T += V^T P^T with V^T read from the row-major tile by transposing LDS
  // reads.  One read gives lane i of each 16-lane group element j of the row
  // read by lane 4j + i/4 of its group, column i%4 of that lane's 4 values;
  // the addresses below make lane l receive, for the operand's k index
  // 8*hf + 4*h + j, the key 16*sl + 8*h + 4*hf + j at column d = 32*db + l%32,
  // the key order the P operand takes from the score accumulators.  The
  // swizzle of such a key depends only on j, so each d block has one lane
  // base and (sl, h) are immediate offsets.
  __device__ __forceinline__ void pv_dma(const unsigned char* vt, const Probs& pb) {
    const int lane = tid & 63;
    const int sq = (lane & 15) >> 2;       // row within the 4-row group
    const int d0 = 16 * (l32 >> 4) + 4 * (lane & 3);
    const uint32_t lanev = (uint32_t)((4 * hf + sq) * (TL::CPR * 16) + (d0 & 7) * 2);
    // product i is (d block i % DB, key slice i / DB): consecutive products
    // update different accumulators
    constexpr int NP = DB * 2 * KB;
    auto rd = [&](int i) __attribute__((always_inline)) {
      const int db = i % DB, sl = i / DB;
      const uint32_t vb = lanev + (uint32_t)((((4 * db + (d0 >> 3)) ^ swz_v(sq)) * 16));
      bf16x4 h2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(
            vt + vb + (16 * sl + 8 * h) * (TL::CPR * 16)));
      return bf16x8{h2[0][0], h2[0][1], h2[0][2], h2[0][3], h2[1][0], h2[1][1], h2[1][2], h2[1][3]};
    };
    constexpr int kAhead = BASA_OPERAND_AHEAD_PV;
    bf16x8 av[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead && i < NP; ++i) av[i] = rd(i);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + kAhead < NP) av[(i + kAhead) % (kAhead + 1)] = rd(i + kAhead);
      const int db = i % DB, sl = i / DB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            av[i % (kAhead + 1)], __builtin_bit_cast(bf16x8, pb[qb][sl]), acc[qb][db], 0, 0, 0);
    }
  }

  // ---- query rows of block qb: row wave*kQPW + 32*qb + l32 of the unit
  __device__ __forceinline__ int qrow(const Unit& u, int qb) const {
    return u.qt * TL::kQT + wave * TL::kQPW + 32 * qb + l32;
  }
  // Q rows as B operand: step s, lane half hf holds d = hf*D/2 + 8s .. +7
  __device__ __forceinline__ void load_q(const Unit& u, int qb, uint32_t qoff, bool qvalid) {
    const Rsrc rs = make_rsrc(p.q + u.base);
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      const u32x4 x = buf_load16(rs, qoff + hf * D + s * 16, 0);
      qreg[qb][s] = qvalid ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- softmax pieces
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][i][r] = 0.0f;
      m_used[qb] = -INFINITY;
      l0[qb] = 0.0f;
      l1[qb] = 0.0f;
    }
  }
  __device__ __forceinline__ void compute_s(const uint16_t* kt, Scores& s) const {
    const f32x16 zero16 = {};
    // step-major: the KB independent accumulator chains alternate, so each
    // LDS operand read has a few MFMAs of slack and no MFMA waits on the last
#pragma unroll
    for (int ss = 0; ss < QS; ++ss) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(
            kt + (kb * 32 + l32) * TL::KS + hf * (D / 2) + ss * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qreg[qb][ss]),
              ss == 0 ? zero16 : s[qb][kb], 0, 0, 0);
      }
    }
  }
  // padding keys -> -inf; memory keys get the logit bias (selects, no branches)
  __device__ __forceinline__ void mask_s(Scores& s, int k0) const {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          const float x = s[qb][kb][r] + (key >= m ? bias : 0.0f);
          s[qb][kb][r] = key < L ? x : -INFINITY;
        }
  }
  __device__ __forceinline__ float rowmax(const Scores& s, int qb) const {
    float mx = s[qb][0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  __device__ __forceinline__ void rowmax_all(const Scores& s, float (&mx)[QB]) const {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[qb] = rowmax(s, qb);
  }
  // the first tile's max right after reset(): with the running max at -inf
  // the rescale of update_max would only multiply zeros, so it is skipped
  __device__ __forceinline__ void start_max(const float (&mx)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_used[qb] = mx[qb] * c1;
  }
  // lagging max: rescale O only when the max has grown by more than the slack
  __device__ __forceinline__ void update_max(const float (&mx)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_new = mx[qb] * c1;
      const bool need = m_new > m_used[qb] + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_tgt = need ? m_new : m_used[qb];
        const float alpha = exp2f(m_used[qb] - m_tgt);
        m_used[qb] = m_tgt;
        l0[qb] *= alpha;
        l1[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][i][r] *= alpha;
      }
    }
  }
  // P = exp2(S*c1 + off - m): row sums (two partial sums) and the bf16
  // operands of the P V product.  off is a logit offset (log2 units) shared
  // by every key of the tile.
  __device__ __forceinline__ void make_p(const Scores& s, Probs& pb, float off = 0.0f) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nm = off - m_used[qb];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][8 * u + j], c1, nm));
          const float sum = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
          if (u) l1[qb] += sum;
          else l0[qb] += sum;
          pb[qb][2 * kb + u] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                                     pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
        }
      }
    }
  }
  // O^T += V^T P^T
  __device__ __forceinline__ void pv(const uint16_t* vt, const Probs& pb) {
#pragma unroll
    for (int sl = 0; sl < 2 * KB; ++sl) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(
            vt + (db * 32 + l32) * TL::VS + sl * 16 + hf * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pb[qb][sl]),
              acc[qb][db], 0, 0, 0);
      }
    }
  }
  // normalise and scatter query block qb back to raster order.  A lane
  // holds 4 consecutive d of each 8-d group and its partner lane (32 apart)
  // the other 4; one exchange per group pair gives each lane a whole group,
  // so every store writes 16 bytes and the lane pair 32 contiguous bytes.
  __device__ __forceinline__ void finish(const Unit& u, int qb, uint32_t qoff, bool qvalid) const {
    const float lp = l0[qb] + l1[qb];
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lp), __float_as_uint(lp),
                                                     false, false);
    const float lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const float inv = 1.0f / lsum;
    if (p.lse != nullptr && qvalid && hf == 0) {
      // natural-log log-sum-exp of the scaled, biased logits of this query
      const uint32_t token = qoff / stb;
      p.lse[(int64_t)u.bh * p.n_tok + token] = (m_used[qb] + __builtin_log2f(lsum)) * 0.6931471805599453f;
    }
    const Rsrc rs = make_rsrc(p.out + u.base);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; g += 2) {
        // a: this lane's 4 d of group g; b: of group g+1
        const uint32_t a0 = pack_bf16x2(acc[qb][db][4 * g] * inv, acc[qb][db][4 * g + 1] * inv);
        const uint32_t a1 = pack_bf16x2(acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv);
        const uint32_t b0 =
            pack_bf16x2(acc[qb][db][4 * g + 4] * inv, acc[qb][db][4 * g + 5] * inv);
        const uint32_t b1 =
            pack_bf16x2(acc[qb][db][4 * g + 6] * inv, acc[qb][db][4 * g + 7] * inv);
        // lanes 0-31 end with group g+1 (their own half first), lanes 32-63
        // with group g (the partner's half first)
        const auto x0 = __builtin_amdgcn_permlane32_swap(b0, a0, false, false);
        const auto x1 = __builtin_amdgcn_permlane32_swap(b1, a1, false, false);
        const u32x4 w{x0[0], x1[0], x0[1], x1[1]};
        const int d = db * 32 + 8 * (g + 1 - hf);
        if (qvalid) __builtin_amdgcn_raw_buffer_store_b128(w, rs, qoff + d * 2, 0, 0);
      }
  }
  // The same through this wave's 32-row staging area (stage: row r's 16-byte
  // chunk c at slot c ^ (r % CPR), the Q staging layout): the rows are
  // written there, then read back so that each store instruction writes
  // 64 / CPR whole rows, with the non-temporal policy.  Whole-row stores
  // need no merging in L2, and the output (not read again here) then drains
  // to HBM while the kernel still runs.
  __device__ __forceinline__ void finish_lds(const Unit& u, int qb, uint32_t qoff, bool qvalid,
                                             unsigned char* stage) const {
    const float lp = l0[qb] + l1[qb];
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lp), __float_as_uint(lp),
                                                     false, false);
    const float lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const float inv = 1.0f / lsum;
    if (p.lse != nullptr && qvalid && hf == 0) {
      const uint32_t token = qoff / stb;
      p.lse[(int64_t)u.bh * p.n_tok + token] = (m_used[qb] + __builtin_log2f(lsum)) * 0.6931471805599453f;
    }
    constexpr int CPR = TL::CPR;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; g += 2) {
        const uint32_t a0 = pack_bf16x2(acc[qb][db][4 * g] * inv, acc[qb][db][4 * g + 1] * inv);
        const uint32_t a1 = pack_bf16x2(acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv);
        const uint32_t b0 =
            pack_bf16x2(acc[qb][db][4 * g + 4] * inv, acc[qb][db][4 * g + 5] * inv);
        const uint32_t b1 =
            pack_bf16x2(acc[qb][db][4 * g + 6] * inv, acc[qb][db][4 * g + 7] * inv);
        const auto x0 = __builtin_amdgcn_permlane32_swap(b0, a0, false, false);
        const auto x1 = __builtin_amdgcn_permlane32_swap(b1, a1, false, false);
        const u32x4 w{x0[0], x1[0], x0[1], x1[1]};
        const int ch = db * 4 + g + 1 - hf;   // d = 8 ch .. 8 ch + 7 of row l32
        *reinterpret_cast<u32x4*>(stage + (l32 * CPR + (ch ^ (l32 % CPR))) * 16) = w;
      }
    // a wave's LDS accesses complete in order, so the reads below see the
    // writes; the wave barrier keeps the compiler from moving them across
    __builtin_amdgcn_wave_barrier();
    const Rsrc rs = make_rsrc(p.out + u.base);
    const int lane = tid & 63;
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int r = (64 / CPR) * i + lane / CPR;
      const int ch = (lane % CPR) ^ (r % CPR);
      const u32x4 w = *reinterpret_cast<const u32x4*>(stage + i * 1024 + lane * 16);
      // row r's offset and validity from lane r (rows 0-31 sit in lanes 0-31)
      const uint32_t ro = (uint32_t)__builtin_amdgcn_ds_bpermute(r * 4, (int)qoff);
      const int rv = __builtin_amdgcn_ds_bpermute(r * 4, qvalid ? 1 : 0);
      if (rv) __builtin_amdgcn_raw_buffer_store_b128(w, rs, ro + (uint32_t)ch * 16u, 0, kStoreNT);
    }
  }
};

// One workgroup per work unit.
template <int D, bool FULL, int NW, int QB, int KT>
__global__ void __launch_bounds__(NW * 64, 8 / (NW * QB)) attn_bf16_kernel(AttnParams p) {
  using C = Core<D, FULL, NW, QB, KT>;
  constexpr int kKT = KT;
  using Scores = typename C::Scores;
  using Probs = typename C::Probs;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // XCD-aware: consecutive units run on one XCD's L2
  const int xcd = blockIdx.x & 7;
  const int kidx = blockIdx.x >> 3;
  const int unit = xcd * p.units_per_xcd + kidx;
  if (kidx >= p.units_per_xcd || unit >= p.units) return;

  C c(p, smem);
  const Unit u = decode_unit(p, unit);
  uint32_t* tab = c.table();
  if (!FULL) {
    c.build_table(tab, u.win);
    __syncthreads();
  }
  uint32_t qoff[QB];
  bool qvalid[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = c.qrow(u, qb);
    qvalid[qb] = r < c.m;
    qoff[qb] = qvalid[qb] ? c.tok(tab, r) : 0;
    c.load_q(u, qb, qoff[qb], qvalid[qb]);
  }
  c.reset();
  const int nkt = c.nkt;

  // prologue: K(0), V(0), K(1) loaded together (with Q) and stored; V(1),
  // K(2) then stay in flight
  {
    u32x4 k1[C::TL::KPASS];
    c.load_k(u, tab, 0);
    c.load_v(u, tab, 0);
    c.load_k_to(k1, u, tab, 1);
    c.store_k(0);
    c.store_v(0);
    c.store_k_from(k1, 1);
  }
  __syncthreads();
  c.load_v(u, tab, 1);
  c.load_k(u, tab, 2);
  Scores sA, sB;
  float mx[QB];
  c.compute_s(c.sK(0), sA);
  if (c.tmask == 0) c.mask_s(sA, 0);
  c.rowmax_all(sA, mx);
  c.start_max(mx);
  __syncthreads();  // every wave is done with K(0) before iteration 0 refills its buffer

  // Iteration t: S(t+1) from K buffer (t+1)&1 while P(t) is formed; P(t) V(t)
  // from V buffer t&1 while max S(t+1) is taken; then V(t+1) and K(t+2) go
  // to the buffers that iteration t-1 finished with.
  auto iter = [&](int t, Scores& sc, Scores& sn, auto masked) __attribute__((always_inline)) {
    Probs pb;
    float mxn[QB];
    c.compute_s(c.sK((t + 1) & 1), sn);
    c.make_p(sc, pb);
    c.pv(c.sV(t & 1), pb);
    if constexpr (decltype(masked)::value) c.mask_s(sn, (t + 1) * kKT);
    c.rowmax_all(sn, mxn);
    c.store_v((t + 1) & 1);
    c.store_k(t & 1);
    __syncthreads();
    c.load_v(u, tab, t + 2);
    c.load_k(u, tab, t + 3);
    c.update_max(mxn);
  };
  auto copy = [&](Scores& dst, const Scores& src) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) dst[qb][kb] = src[qb][kb];
  };
  int t = 0;
  const int t1 = min(nkt, c.tmask);  // iterations t < t1 - 1 need no mask on S(t+1)
  for (; t + 2 < t1; t += 2) {
    iter(t, sA, sB, bool_c<false>{});
    iter(t + 1, sB, sA, bool_c<false>{});
  }
  if (t + 1 < t1) {
    iter(t, sA, sB, bool_c<false>{});
    ++t;
    copy(sA, sB);
  }
  for (; t + 2 < nkt; t += 2) {
    iter(t, sA, sB, bool_c<true>{});
    iter(t + 1, sB, sA, bool_c<true>{});
  }
  if (t + 1 < nkt) {
    iter(t, sA, sB, bool_c<true>{});
    ++t;
    copy(sA, sB);
  }
  {
    Probs pb;
    c.make_p(sA, pb);
    c.pv(c.sV(t & 1), pb);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) c.finish(u, qb, qoff[qb], qvalid[qb]);
}


// Barrier that orders LDS accesses only.  Global stores in flight (the output
// of a finished unit) do not hold the workgroup up; loads whose registers feed
// LDS stores are waited for by those stores' own register dependences, and
// direct global-to-LDS loads by an explicit wait_vmem() before the barrier
// that publishes them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Waits until every vector memory operation of this wave has completed
// (vmcnt = 0; expcnt and lgkmcnt left at their maximum).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Waits until at most N of this wave's vector memory operations are
// outstanding (N < 16).  A wave's vector memory operations complete in the
// order they were issued, so all but the N most recent are then done.
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// LDS of the persistent kernel: the tile buffers, two window tables (the
// current unit's and the next one's) and, per wave, a staging area for the
// next unit's Q rows, filled by direct global-to-LDS loads.
template <int D, bool FULL, int NW, int KT, bool DMA>
struct PersistLayout {
  using TL = Tiles<D, NW, 1, KT>;
  // two K and two V tile buffers: padded K and transposed V, or (DMA) four
  // row-major swizzled tiles
  static constexpr int KD = DMA ? BASA_K_DEPTH : 2;   // K tile buffers
  static constexpr int tileBytes = DMA ? (KD + 2) * KT * D * 2 : TL::tileBytes;
  static constexpr int CPR = D / 8;        // 16B chunks per Q row
  static constexpr int RPI = 64 / CPR;     // Q rows per load instruction (64 lanes x 16B)
  static constexpr int QI = 32 / RPI;      // instructions per wave and unit
  static constexpr int kQWave = 32 * D * 2;
  __host__ __device__ static constexpr size_t table_bytes(int m) {
    return FULL ? 0 : ((size_t)m * 4 + 15) / 16 * 16;
  }
  __host__ __device__ static constexpr size_t stage_offset(int m) {
    return tileBytes + 2 * table_bytes(m);
  }
  __host__ __device__ static constexpr size_t bytes(int m) {
    return stage_offset(m) + (BASA_PERSISTENT_QSTAGE ? (size_t)NW * kQWave : 0);
  }
};

// Persistent form of the unit kernel: one workgroup per CU; slot s of XCD x
// runs units x*upx + s + j*S (S workgroups per XCD), j = 0..J-1, with the
// unit kernel's tile loop.  The operands the next unit starts with are loaded
// into registers the current unit no longer needs: its K tile 0 in the slot
// of the current unit's tile nkt, its V tile 0 and K tile 1 in the slots of
// tile nkt+1, and its Q rows once the current unit's last scores are formed.
// The tile count is rounded up to an even number (a padding tile has only
// masked keys), so tile t of every unit uses buffer t & 1.
template <int D, bool FULL, int NW, int KT, bool DMA>
__global__ void __launch_bounds__(NW * 64, BASA_PERSISTENT_WGS) attn_bf16_persistent_kernel(AttnParams p) {
  using C = Core<D, FULL, NW, 1, KT>;
  using TL = typename C::TL;
  using PL = PersistLayout<D, FULL, NW, KT, DMA>;
  constexpr int kKT = KT;
  using Scores = typename C::Scores;
  using Probs = typename C::Probs;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int S = gridDim.x >> 3;
  const int ubeg = xcd * p.units_per_xcd;
  const int uend = min(ubeg + p.units_per_xcd, p.units);
  const int first = ubeg + slot;
  if (first >= uend) return;                  // whole workgroup exits together
  const int J = (uend - first + S - 1) / S;   // units of this workgroup

  C c(p, smem);
  // even tile count; a padding tile holds only keys >= L, which the mask removes
  const int nkt = (c.nkt + 1) & ~1;
  // Per-key masking (the memory bias per key, padding keys to -inf) starts
  // at the tile that straddles the window / memory boundary or holds
  // padding keys.  Tiles of memory keys only before that take the bias as
  // one offset of the tile's row max and exponent instead.
  {
    int tm = nkt;
    if (c.bias != 0.0f && c.m % kKT != 0) tm = c.m / kKT;
    if (c.L % kKT) tm = min(tm, c.nkt - 1);
    c.tmask = min(tm, c.nkt);
  }
  // Order of the key tiles.  Position t of the loop processes key tile
  // kt_of(t).  Before the first masked position (t1), the tiles of window
  // keys (gathered from HBM) are spread evenly among the other tiles (memory
  // keys, served from L2), so that every unit -- and with all compute units
  // walking their units in step, the whole chip -- keeps reading HBM while
  // it works through the memory keys instead of alternating a phase bound by
  // HBM with one bound by the matrix cores.  The softmax does not depend on
  // the order of its keys.  Of the first c positions, ceil(c * nw / t1) hold
  // window tiles (nw of the t1); the division is a multiply by a rounded-up
  // reciprocal, exact while t1 * t1 * (nw + 1) < 2^32 (t1 <= 1024, nw <= 64).
  const int t1 = min(nkt, c.tmask);  // iterations t < t1 - 1 need no mask on S(t+1)
  const int nw = (FULL || !BASA_TILE_INTERLEAVE || t1 > 1024) ? t1 : min(c.m / kKT, t1);
  const uint32_t rcp =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(0xFFFFFFFFu / (uint32_t)max(t1, 1) + 1u));
  auto kt_of = [&](int pos) __attribute__((always_inline)) {
    if (FULL || nw >= t1 || nw == 0 || pos >= t1) return pos;
    const int c0 = (int)__umulhi((uint32_t)(pos * nw + t1 - 1), rcp);
    const int c1n = (int)__umulhi((uint32_t)((pos + 1) * nw + t1 - 1), rcp);
    return __builtin_amdgcn_readfirstlane(c1n > c0 ? c0 : nw + pos - c0);
  };
  // memory-key logit bias of position t taken as one offset (memory-only
  // tiles before the masked ones)
  auto bias_of = [&](int t) __attribute__((always_inline)) {
    if constexpr (FULL) return 0.0f;  // no memory keys
    else return (t < c.tmask && kt_of(t) * kKT >= c.m) ? c.bias : 0.0f;
  };
  // key tiles of positions 0 and 1 (the same for every unit)
  const int kt0 = kt_of(0), kt1 = kt_of(1);
  unsigned char* tables = smem + PL::tileBytes;
  // DMA tile buffers: K buffer b at b * kTileB (b < KD), V buffer b at
  // (KD + b) * kTileB.  The K tiles of all units of this workgroup go through
  // the K buffers in turn: position t of a unit whose position 0 went to
  // buffer kb0 uses buffer (kb0 + t) mod KD, and positions past the unit's
  // last tile are the next unit's first ones (its kb0 is (kb0 + nkt) mod KD).
  // V buffers go by the parity of the position (nkt is even).
  constexpr int KD = PL::KD;
  static_assert(DMA || KD == 2, "registers-staged tiles use two K buffers");
  auto dK = [&](int b) __attribute__((always_inline)) { return smem + b * C::kTileB; };
  auto dV = [&](int b) __attribute__((always_inline)) { return smem + (KD + b) * C::kTileB; };
  int kb0 = 0;
  auto kslot = [&](int pos) __attribute__((always_inline)) {
    if constexpr (KD == 2) return pos & 1;
    else return (kb0 + pos) % KD;
  };
  auto get_v = [&](const Unit& u, const uint32_t* tb, int tile) __attribute__((always_inline)) {
    if constexpr (DMA) c.dma_tile(dV(tile & 1), u, tb, tile, true);
    else c.load_v(u, tb, tile);
  };
  auto get_k = [&](const Unit& u, const uint32_t* tb, int tile) __attribute__((always_inline)) {
    if constexpr (DMA) c.dma_tile(dK(tile & 1), u, tb, tile, false);
    else c.load_k(u, tb, tile);
  };
  auto scores = [&](int b, Scores& sc) __attribute__((always_inline)) {
    if constexpr (DMA) c.compute_s_dma(dK(b), sc);
    else c.compute_s(c.sK(b), sc);
  };
  auto tab_of = [&](int j) __attribute__((always_inline)) {
    return reinterpret_cast<uint32_t*>(tables + (j & 1) * PL::table_bytes(c.m));
  };
  auto unit_at = [&](int j) __attribute__((always_inline)) {
    return decode_unit(p, first + min(j, J - 1) * S);
  };
  // Q rows of unit u; and its output rows, both addressed through its table
  auto load_q_of = [&](const Unit& u, const uint32_t* tb) __attribute__((always_inline)) {
    const int r = c.qrow(u, 0);
    const bool valid = r < c.m;
    c.load_q(u, 0, valid ? c.tok(tb, r) : 0u, valid);
  };
  // This wave's staged Q rows: 16B chunk ch of row r at position ch ^ (r %
  // CPR), so the 32 lanes reading one chunk of 32 rows hit distinct banks.
  const int wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
  unsigned char* qstage = smem + PL::stage_offset(c.m) + wave * PL::kQWave;
  // instruction i of PL::QI: 64 lanes x 16B to qstage + 1024*i + 16*lane
  auto stage_q = [&](const Unit& u, const uint32_t* tb, int i) __attribute__((always_inline)) {
    const int lane = c.tid & 63;
    const int r = PL::RPI * i + lane / PL::CPR;
    const int ch = (lane % PL::CPR) ^ (r % PL::CPR);
    const int row = min(u.qt * TL::kQT + wave * 32 + r, c.m - 1);
    const char* src = reinterpret_cast<const char*>(p.q + u.base) + c.tok(tb, row) + ch * 16;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                      (__attribute__((address_space(3))) void*)(qstage + i * 1024),
                                      16, 0, kLoadOnce);
  };
  auto unstage_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < C::QS; ++s) {
      const int ch = c.hf * (PL::CPR / 2) + s;
      c.qreg[0][s] = *reinterpret_cast<const u32x4*>(
          qstage + (c.l32 * PL::CPR + (ch ^ (c.l32 % PL::CPR))) * 16);
    }
  };
  // the output rows go out through the wave's staging area, free from the
  // read of the next unit's Q rows until the next unit's first staging load
  auto finish_of = [&](const Unit& u, const uint32_t* tb) __attribute__((always_inline)) {
    const int r = c.qrow(u, 0);
    const bool valid = r < c.m;
    if constexpr (BASA_PERSISTENT_QSTAGE) c.finish_lds(u, 0, valid ? c.tok(tb, r) : 0u, valid, qstage);
    else c.finish(u, 0, valid ? c.tok(tb, r) : 0u, valid);
  };

  // ---- unit 0: tables of units 0 and 1; its operands from global memory
  Unit uc = unit_at(0);
  Unit un = unit_at(1);
  if (!FULL) {
    c.build_table(tab_of(0), uc.win);
    if (J > 1) c.build_table(tab_of(1), un.win);
    lds_barrier();
  }
  load_q_of(uc, tab_of(0));
  if constexpr (DMA) {
    c.dma_tile(dK(0), uc, tab_of(0), kt0, false);
    c.dma_tile(dV(0), uc, tab_of(0), kt0, true);
    c.dma_tile(dK(1), uc, tab_of(0), kt1, false);
    if constexpr (KD == 3) c.dma_tile(dK(2), uc, tab_of(0), kt_of(2), false);
    wait_vmem();
  } else {
    u32x4 k1[TL::KPASS];
    c.load_k(uc, tab_of(0), kt0);
    c.load_v(uc, tab_of(0), kt0);
    c.load_k_to(k1, uc, tab_of(0), kt1);
    c.store_k(0);
    c.store_v(0);
    c.store_k_from(k1, 1);
  }
  lds_barrier();  // K tiles 0 .. KD-1 and V tile 0 of unit 0 are in LDS
  Scores sA, sB;
  scores(0, sA);
  auto copy = [&](Scores& dst, const Scores& src) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) dst[0][kb] = src[0][kb];
  };
  const int qstep = nkt - 2;         // staging load i of the next unit's Q goes out in
                                     // iteration i mod qstep (never in the last one)

  // Unit j starts with S(0) in sA, its tile 0 in K buffer 0, tile 1 in K
  // buffer 1 and V tile 0 in V buffer 0.
  for (int j = 0; j < J; ++j) {
    c.redefine_lane_ids();
    const bool has_next = j + 1 < J;
    const uint32_t* tab = tab_of(j);
    const uint32_t* tabn = tab_of(j + 1);
    c.reset();
    {
      float mx[1];
      if (c.tmask == 0) c.mask_s(sA, 0);
      c.rowmax_all(sA, mx);
      mx[0] += bias_of(0);
      c.start_max(mx);
    }
    if constexpr (!DMA) {
      c.load_v(uc, tab, kt1);
      c.load_k(uc, tab, kt_of(2));
    }
    // Every wave is done with K(0) (and with the previous unit's output
    // rows, read through its table) before iteration 0 refills the buffer
    // and the next unit's table overwrites the previous unit's.  Direct
    // loads into LDS go out only after this barrier: until then other waves
    // may still read the buffers (the previous unit's last V tile).
    lds_barrier();
    if constexpr (DMA)
      c.dma_pair(true, dV(1), uc, tab, kt1, true, dK(kslot(KD)), uc, tab, kt_of(KD));
    if (!FULL && j >= 1 && has_next) c.build_table(tab_of(j + 1), un.win);

    // Iteration t: as in the unit kernel; the loads past the unit's last tile
    // bring the next unit's first tiles.
    auto iter = [&](int t, Scores& sc, Scores& sn, auto masked) __attribute__((always_inline)) {
      Probs pb;
      float mxn[1];
      scores(kslot(t + 1), sn);
      c.make_p(sc, pb, bias_of(t) * c.c1);
      if constexpr (DMA) c.pv_dma(dV(t & 1), pb);
      else c.pv(c.sV(t & 1), pb);
      if constexpr (decltype(masked)::value) c.mask_s(sn, (t + 1) * kKT);
      c.rowmax_all(sn, mxn);
      mxn[0] += bias_of(t + 1);
      if constexpr (DMA) {
        // this wave's loads of V(t+1) and K(t+2) (issued in iteration t-1,
        // or before the unit's first iteration); with three K buffers the
        // most recent K tile load (K(t+3), issued last in iteration t-1, if
        // any) may stay in flight
        if constexpr (KD == 3) {
          if (t + 3 < nkt || has_next) wait_vmem_but<C::kDmaIpw>();
          else wait_vmem();
        } else {
          wait_vmem();
        }
      } else {
        c.store_v((t + 1) & 1);
        c.store_k(t & 1);
      }
      lds_barrier();
      const int tv = t + 2, tk = t + 1 + KD;
      const bool do_v = tv < nkt || (has_next && tv == nkt);
      const bool do_k = tk < nkt || (has_next && tk < nkt + KD);
      if constexpr (DMA) {
        // the next unit's Q staging loads go out first, so that the K tile
        // load is this iteration's last (the wait above relies on it)
        if (has_next && t < qstep)
          if constexpr (BASA_PERSISTENT_QSTAGE) {
            for (int i = t; i < PL::QI; i += qstep) stage_q(un, tabn, i);
          }
        const bool cv = tv < nkt, ck = tk < nkt;
        const int jv = cv ? tv : 0, jk = ck ? tk : tk - nkt;
        const Unit u_v = cv ? uc : un;  // by value: the choice stays in registers
        const Unit u_k = ck ? uc : un;
        if (do_v || do_k)
          c.dma_pair(do_v, dV(jv & 1), u_v, cv ? tab : tabn, kt_of(jv), do_k, dK(kslot(tk)), u_k,
                     ck ? tab : tabn, kt_of(jk));
      } else {
        if (do_v) {
          const bool cur = tv < nkt;
          const Unit u = cur ? uc : un;  // by value: the choice stays in registers
          get_v(u, cur ? tab : tabn, cur ? kt_of(tv) : kt0);
        }
        if (do_k) {
          const bool cur = tk < nkt;
          const Unit u = cur ? uc : un;
          get_k(u, cur ? tab : tabn, kt_of(cur ? tk : tk - nkt));
        }
      }
      if constexpr (!DMA) {
        if (has_next && t < qstep)
          if constexpr (BASA_PERSISTENT_QSTAGE) {
            for (int i = t; i < PL::QI; i += qstep) stage_q(un, tabn, i);
          }
      }
      c.update_max(mxn);
    };
    int t = 0;
    for (; t + 2 < t1; t += 2) {
      iter(t, sA, sB, bool_c<false>{});
      iter(t + 1, sB, sA, bool_c<false>{});
    }
    if (t + 1 < t1) {
      iter(t, sA, sB, bool_c<false>{});
      ++t;
      copy(sA, sB);
    }
    for (; t + 2 < nkt; t += 2) {
      iter(t, sA, sB, bool_c<true>{});
      iter(t + 1, sB, sA, bool_c<true>{});
    }
    if (t + 1 < nkt) {
      iter(t, sA, sB, bool_c<true>{});
      ++t;
      copy(sA, sB);
    }
    if (t < c.nkt) {  // the tile padding an odd tile count holds no key
      Probs pb;
      c.make_p(sA, pb, bias_of(t) * c.c1);
      if constexpr (DMA) c.pv_dma(dV(t & 1), pb);
      else c.pv(c.sV(t & 1), pb);
    }
    if (!has_next) {
      finish_of(uc, tab);
      break;
    }
    // The next unit's K tile 0 is in buffer 0 (stored by iteration nkt-2).
    // Its V tile 0 and K tile 1 go to buffers whose last readers (the P V
    // product of tile nkt-2, the scores of tile nkt-1) ran before the last
    // barrier.  Its Q rows come from this wave's staging area (each wave
    // stages and reads only its own rows).  Its first scores are formed
    // before this unit's output stores are issued, so no wait for a load
    // covers those stores.
    // With three K buffers the next unit's K tile 2, issued last, may stay in
    // flight: its first iteration waits for it.
    if constexpr (KD == 3) wait_vmem_but<C::kDmaIpw>();
    else wait_vmem();
    if constexpr (BASA_PERSISTENT_QSTAGE) unstage_q();
    else load_q_of(un, tabn);
    if constexpr (!DMA) {
      c.store_v(0);
      c.store_k(1);
    }
    scores(kslot(nkt), sA);
    finish_of(uc, tab);
    uc = un;
    un = unit_at(j + 2);
    if constexpr (KD == 3) kb0 = (kb0 + nkt) % KD;
  }
}

// Workgroup shape: NW waves of QB query blocks (32 rows each).
#ifndef BASA_ATTN_WAVES
#define BASA_ATTN_WAVES 8
#endif
#ifndef BASA_ATTN_QBLOCKS
#define BASA_ATTN_QBLOCKS 1
#endif
#ifndef BASA_ATTN_KTILE
#define BASA_ATTN_KTILE 64
#endif
// Persistent kernel on/off and its key-tile size.
#ifndef BASA_PERSISTENT
#define BASA_PERSISTENT 1
#endif
#ifndef BASA_PERSISTENT_KTILE
#define BASA_PERSISTENT_KTILE 64
#endif
// K/V tiles of the persistent kernel by direct buffer-to-LDS loads (swizzled,
// V^T read with transposing LDS reads) instead of through registers.
#ifndef BASA_PERSISTENT_DMA
#define BASA_PERSISTENT_DMA 1
#endif
// Per-device record of a kernel's raised LDS limit.
struct DeviceFlags {
  bool set[64] = {};
};

// Raises the kernel's dynamic LDS limit to 160 KB, once per device.
template <typename K>
int set_lds_limit(K kernel, DeviceFlags& done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BASA_ERR_HIP;
  const bool cached = dev >= 0 && dev < 64;
  if (cached && done.set[dev]) return BASA_OK;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
    return BASA_ERR_HIP;
  if (cached) done.set[dev] = true;  // benign race: the call is idempotent
  return BASA_OK;
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cache[dev] = v;  // benign race: every thread stores the same value
  }
  return cache[dev];
}

// Fills in the unit count of a launch with kQT query rows per unit.
inline int set_units(AttnParams& p, int kQT) {
  p.nQT = (p.m + kQT - 1) / kQT;
  const int64_t units = (int64_t)p.batch_heads * p.nW * p.nQT;
  if (units > (int64_t)INT32_MAX / 2) return BASA_ERR_UNSUPPORTED;
  p.units = (int32_t)units;
  p.units_per_xcd = (p.units + 7) / 8;
  return BASA_OK;
}

// Persistent kernel when the units are long enough and its LDS fits; returns
// -1 (nothing launched) otherwise.
template <int D, bool FULL, int NW, int KT>
int launch_persistent(const AttnParams& p0, hipStream_t stream) {
  constexpr bool DMA = BASA_PERSISTENT_DMA != 0;
  using TL = Tiles<D, NW, 1, KT>;
  using SL = PersistLayout<D, FULL, NW, KT, DMA>;
  const int nkt = ((FULL ? p0.n_kv : p0.m + p0.G) + KT - 1) / KT;
  const size_t lds = SL::bytes(p0.m);
  if (nkt < kPersistentMinTiles || lds * BASA_PERSISTENT_WGS > 160 * 1024) return -1;
  AttnParams p = p0;
  if (int e = set_units(p, TL::kQT)) return e;
  static DeviceFlags attr;
  if (set_lds_limit(&attn_bf16_persistent_kernel<D, FULL, NW, KT, DMA>, attr)) return BASA_ERR_HIP;
  const int per_xcd = max(1, min(p.units_per_xcd, BASA_PERSISTENT_WGS * cu_count() / 8));
  hipLaunchKernelGGL((attn_bf16_persistent_kernel<D, FULL, NW, KT, DMA>),
                     dim3((unsigned)(8 * per_xcd)), dim3(TL::kThreads), lds, stream, p);
  return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

template <int D, bool FULL, int NW, int QB, int KT>
int launch_unit(const AttnParams& p0, hipStream_t stream) {
  using TL = Tiles<D, NW, QB, KT>;
  AttnParams p = p0;
  if (int e = set_units(p, TL::kQT)) return e;
  const size_t lds = TL::tileBytes + (FULL ? 0 : (size_t)p.m * 4);
  if (lds > 160 * 1024) return BASA_ERR_UNSUPPORTED;
  static DeviceFlags attr;
  if (set_lds_limit(&attn_bf16_kernel<D, FULL, NW, QB, KT>, attr)) return BASA_ERR_HIP;
  hipLaunchKernelGGL((attn_bf16_kernel<D, FULL, NW, QB, KT>), dim3((unsigned)(8 * p.units_per_xcd)),
                     dim3(TL::kThreads), lds, stream, p);
  return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

template <int D, bool FULL>
int launch_full_or_window(const AttnParams& p, hipStream_t stream) {
  // a head dim of 64 needs 64-key tiles to give every thread of 8 waves work
  constexpr int KT = (D == 64 && BASA_ATTN_KTILE * D < 64 * 64) ? 64 : BASA_ATTN_KTILE;
  constexpr int KTS = (D == 64 && BASA_PERSISTENT_KTILE * D < 64 * 64) ? 64 : BASA_PERSISTENT_KTILE;
#if BASA_PERSISTENT
  const int e = launch_persistent<D, FULL, BASA_PERSISTENT_WAVES, KTS>(p, stream);
  if (e >= 0) return e;
#endif
  return launch_unit<D, FULL, BASA_ATTN_WAVES, BASA_ATTN_QBLOCKS, KT>(p, stream);
}

template <int D>
int launch_d(const AttnParams& p, bool full, hipStream_t stream) {
  return full ? launch_full_or_window<D, true>(p, stream)
              : launch_full_or_window<D, false>(p, stream);
}

}  // namespace

int launch_attn_bf16(const AttnParams& p, bool full, hipStream_t stream) {
  if (p.head_dim == 128) return launch_d<128>(p, full, stream);
  if (p.head_dim == 64) return launch_d<64>(p, full, stream);
  return BASA_ERR_UNSUPPORTED;
}

}  // namespace basa
