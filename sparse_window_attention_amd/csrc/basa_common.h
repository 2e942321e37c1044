// Shared device-side types and helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace basa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Geometry of one call, in the kernels' terms.  Grids are 3D (T = 1 for
// images).  Token offsets are element offsets inside one (batch, head) slice.
struct Geometry {
  int32_t T, Hg, Wg;        // grid
  int32_t wt, wy, wx;       // window
  int32_t st, sy, sx;       // shift, already reduced into [0, window)
  int32_t nwy, nwx;         // windows along y and x
  uint32_t mwx, mwy;        // div_magic multipliers of wx and wy
};

// Multiplier for div_magic: floor((2^32 - 1) / d) + 1, or 0 for d = 1.
__host__ __device__ inline uint32_t magic_of(int32_t d) {
  return d <= 1 ? 0u : (uint32_t)(0xFFFFFFFFull / (uint32_t)d + 1ull);
}

// floor(x / d) as the high half of x * magic_of(d): exact for 0 <= x < 4096
// and 1 <= d <= 4096 (every slot index of a window, every window dimension;
// checked exhaustively on the CPU).
__device__ __forceinline__ int32_t div_magic(int32_t x, uint32_t magic) {
  return magic ? (int32_t)__umulhi((uint32_t)x, magic) : x;
}

// Raster index of slot r of window j under the shifted partition: the grid
// rolled by -shift, cut into windows, window j holds the tokens at
// (j_axis*w_axis + r_axis + s_axis) mod grid_axis.
__device__ __forceinline__ int32_t window_token(const Geometry& g, int32_t j, int32_t r) {
  const int32_t rq = div_magic(r, g.mwx);
  const int32_t rx = r - rq * g.wx;
  const int32_t rt = div_magic(rq, g.mwy);
  const int32_t ry = rq - rt * g.wy;
  const int32_t jx = j % g.nwx;
  const int32_t jq = j / g.nwx;
  const int32_t jy = jq % g.nwy;
  const int32_t jt = jq / g.nwy;
  int32_t t = jt * g.wt + rt + g.st;
  int32_t y = jy * g.wy + ry + g.sy;
  int32_t x = jx * g.wx + rx + g.sx;
  // the shift is below the window, itself no larger than the grid: at most
  // one wrap per axis
  t -= (t >= g.T) ? g.T : 0;
  y -= (y >= g.Hg) ? g.Hg : 0;
  x -= (x >= g.Wg) ? g.Wg : 0;
  return (t * g.Hg + y) * g.Wg + x;
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Slot of row `key` in a transposed tile whose rows are the k index of an
// MFMA fed from an S accumulator (V^T in the forward; K^T, Q^T, dO^T in the
// backward): within each group of 16, the order matches how the
// accumulator registers map onto the k index of the product's operand.
__device__ __forceinline__ int vslot(int key) {
  const int a = key >> 2, i = key & 3;
  return (a >> 2) * 16 + (a & 1) * 8 + ((a >> 1) & 1) * 4 + i;
}

// Raw buffer resource over a (batch, head) slice: wave-uniform base in
// scalar registers, per-lane 32-bit byte offsets (every offset inside a slice
// is below 2^32 bytes, checked on the host).
using Rsrc = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ Rsrc make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xFFFFFFFFu,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace basa
