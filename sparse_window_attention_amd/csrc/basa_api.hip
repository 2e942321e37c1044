// C ABI entry points: argument validation, geometry set-up and dispatch.
// Every check runs before anything is enqueued, so a failing call launches
// nothing and writes no output byte.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "basa_internal.h"

namespace {

thread_local char g_err[320] = "no error";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  snprintf(g_err, sizeof(g_err), "no error");
  return BASA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// NaN or infinity, from the bit pattern (no compiler flag can fold this away)
bool not_finite(float x) {
  uint32_t b;
  memcpy(&b, &x, sizeof b);
  return (b & 0x7f800000u) == 0x7f800000u;
}

struct Grid3 {
  int32_t g[3];
  int64_t n;
};

// Reads an ndim-entry host array into 3 entries (2D: leading 1 / fill).
int read3(int32_t ndim, const int32_t* src, int32_t fill, int32_t out[3], const char* what) {
  if (!src) return fail(BASA_ERR_INVALID_ARG, "%s is NULL", what);
  if (ndim == 2) {
    out[0] = fill;
    out[1] = src[0];
    out[2] = src[1];
  } else {
    out[0] = src[0];
    out[1] = src[1];
    out[2] = src[2];
  }
  return BASA_OK;
}

int check_grid(int32_t ndim, const int32_t* grid, int32_t g[3], int64_t* n) {
  if (ndim != 2 && ndim != 3) return fail(BASA_ERR_INVALID_ARG, "ndim must be 2 or 3 (got %d)", ndim);
  int rc = read3(ndim, grid, 1, g, "grid");
  if (rc) return rc;
  for (int i = 0; i < 3; ++i)
    if (g[i] <= 0) return fail(BASA_ERR_INVALID_ARG, "grid dims must be positive");
  *n = (int64_t)g[0] * g[1] * g[2];
  return BASA_OK;
}

int check_divides(int32_t ndim, const int32_t* part, const int32_t g[3], int32_t out[3],
                  const char* what) {
  int rc = read3(ndim, part, 1, out, what);
  if (rc) return rc;
  for (int i = 0; i < 3; ++i) {
    if (out[i] <= 0) return fail(BASA_ERR_INVALID_ARG, "%s dims must be positive", what);
    if (g[i] % out[i]) return fail(BASA_ERR_INVALID_ARG, "%s does not divide the grid", what);
  }
  return BASA_OK;
}

int check_common(int32_t batch, int32_t heads, int32_t head_dim, int32_t dtype, int32_t layout) {
  if (batch < 0 || heads < 0) return fail(BASA_ERR_INVALID_ARG, "batch and heads must be >= 0");
  if ((int64_t)batch * heads > INT32_MAX / 2) return fail(BASA_ERR_UNSUPPORTED, "batch*heads too large");
  if (dtype != BASA_BF16 && dtype != BASA_F32) return fail(BASA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(BASA_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", head_dim);
  if (layout != BASA_LAYOUT_BHND && layout != BASA_LAYOUT_BNHD)
    return fail(BASA_ERR_INVALID_ARG, "unknown layout %d", layout);
  return BASA_OK;
}

// An empty batch (batch or heads 0) is a call with nothing to do: once the
// scalar arguments are valid it succeeds without reading any pointer, so
// empty tensors (whose data pointers may be NULL) pass through.  Returns -1
// when the batch is not empty, else the status to return.
int empty_call(int32_t batch, int32_t heads, int32_t head_dim, int32_t dtype, int32_t layout) {
  if (batch != 0 && heads != 0) return -1;
  const int rc = check_common(batch, heads, head_dim, dtype, layout);
  return rc ? rc : ok();
}

// Strides (elements) of a B x H x n x D tensor in the given layout.
void strides(int32_t layout, int32_t heads, int64_t n, int32_t D, int64_t* sb, int64_t* sh,
             int64_t* stok) {
  if (layout == BASA_LAYOUT_BHND) {
    *sb = (int64_t)heads * n * D;
    *sh = n * D;
    *stok = D;
  } else {
    *sb = n * heads * D;
    *sh = D;
    *stok = (int64_t)heads * D;
  }
}

float resolve_scale(float scale, int32_t D) { return scale > 0.0f ? scale : 1.0f / sqrtf((float)D); }

// Workspace of basa_window_attn_bwd_noalloc: one array per GPU, from the
// library's first use on that GPU to the end of the process.  Host code never
// passes the array's name to a kernel (on the host it is a stand-in, not a
// device address): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current.
__device__ __align__(256) unsigned char scratch[BASA_BWD_SCRATCH_BYTES];
std::atomic<void*> g_scratch_addr[64];

// Device address of the current device's scratch array.
int scratch_address(void** addr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(BASA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(BASA_ERR_UNSUPPORTED, "device index %d beyond 63", dev);
  void* a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    // two threads may both get here on a device's first call: both store the
    // same address
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || a == nullptr)
      return fail(BASA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s",
                  hipGetErrorString(e));
    g_scratch_addr[dev].store(a, std::memory_order_release);
  }
  *addr = a;
  return BASA_OK;
}

}  // namespace

extern "C" {

int32_t basa_version(void) { return 100; }

const char* basa_status_string(int32_t status) {
  switch (status) {
    case BASA_OK: return "BASA_OK";
    case BASA_ERR_INVALID_ARG: return "BASA_ERR_INVALID_ARG: invalid argument";
    case BASA_ERR_UNSUPPORTED: return "BASA_ERR_UNSUPPORTED: configuration not built";
    case BASA_ERR_HIP: return "BASA_ERR_HIP: HIP runtime error";
    default: return "unknown status";
  }
}

const char* basa_last_error(void) { return g_err; }

int64_t basa_mem_tokens(int32_t ndim, const int32_t* grid, const int32_t* pool) {
  int32_t g[3], pl[3];
  int64_t n;
  if (check_grid(ndim, grid, g, &n)) return -1;
  if (check_divides(ndim, pool, g, pl, "pool")) return -1;
  ok();
  return (int64_t)(g[0] / pl[0]) * (g[1] / pl[1]) * (g[2] / pl[2]);
}

int basa_shift_for_block(int32_t block_idx, int32_t schedule, int32_t ndim,
                         const int32_t* window, int32_t* shift_out) {
  if (ndim != 2 && ndim != 3) return fail(BASA_ERR_INVALID_ARG, "ndim must be 2 or 3 (got %d)", ndim);
  if (!window || !shift_out) return fail(BASA_ERR_INVALID_ARG, "window or shift_out is NULL");
  if (block_idx < 0) return fail(BASA_ERR_INVALID_ARG, "block index must be >= 0");
  for (int i = 0; i < ndim; ++i)
    if (window[i] <= 0) return fail(BASA_ERR_INVALID_ARG, "window dims must be positive");
  int32_t s[3] = {0, 0, 0};
  switch (schedule) {
    case BASA_SCHED_NONE:
      break;
    case BASA_SCHED_ALTERNATE:
      if (block_idx & 1)
        for (int i = 0; i < ndim; ++i) s[i] = window[i] / 2;
      break;
    case BASA_SCHED_FOUR_PHASE: {
      const int phase = block_idx % (1 << ndim);
      for (int i = 0; i < ndim; ++i) s[i] = ((phase >> i) & 1) ? window[i] / 2 : 0;
      break;
    }
    default:
      return fail(BASA_ERR_INVALID_ARG, "unknown schedule %d", schedule);
  }
  for (int i = 0; i < ndim; ++i) shift_out[i] = s[i];
  return ok();
}

int basa_pool_kv(const void* k, const void* v, void* k_mem, void* v_mem, int32_t batch,
                 int32_t heads, int32_t head_dim, int32_t ndim, const int32_t* grid,
                 const int32_t* pool, int32_t dtype, int32_t layout, void* stream) {
  try {
    if (const int e = empty_call(batch, heads, head_dim, dtype, layout); e >= 0) return e;
    if (!k || !v || !k_mem || !v_mem) return fail(BASA_ERR_INVALID_ARG, "k, v, k_mem and v_mem must be non-NULL");
    int rc = check_common(batch, heads, head_dim, dtype, layout);
    if (rc) return rc;
    int32_t g[3], pl[3];
    int64_t n;
    if ((rc = check_grid(ndim, grid, g, &n))) return rc;
    if ((rc = check_divides(ndim, pool, g, pl, "pool"))) return rc;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_mem) || !aligned16(v_mem))
      return fail(BASA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    int64_t sb, sh, stok;
    strides(layout, heads, n, head_dim, &sb, &sh, &stok);
    if (n * stok >= INT32_MAX) return fail(BASA_ERR_UNSUPPORTED, "grid too large for 32-bit token offsets");
    const int64_t G = (int64_t)(g[0] / pl[0]) * (g[1] / pl[1]) * (g[2] / pl[2]);
    const size_t es = dtype == BASA_BF16 ? 2 : 4;
    const size_t in_bytes = (size_t)batch * heads * n * head_dim * es;
    const size_t mem_bytes = (size_t)batch * heads * G * head_dim * es;
    if (overlaps(k_mem, mem_bytes, k, in_bytes) || overlaps(k_mem, mem_bytes, v, in_bytes) ||
        overlaps(v_mem, mem_bytes, k, in_bytes) || overlaps(v_mem, mem_bytes, v, in_bytes) ||
        overlaps(k_mem, mem_bytes, v_mem, mem_bytes))
      return fail(BASA_ERR_INVALID_ARG, "k_mem/v_mem overlap an input or each other");
    basa::PoolParams p{};
    p.k = k; p.v = v; p.kmem = k_mem; p.vmem = v_mem;
    p.stride_b = sb; p.stride_h = sh; p.stride_tok = (int32_t)stok;
    p.heads = heads; p.batch_heads = batch * heads; p.head_dim = head_dim;
    p.T = g[0]; p.Hg = g[1]; p.Wg = g[2];
    p.pt = pl[0]; p.py = pl[1]; p.px = pl[2];
    p.Gt = g[0] / pl[0]; p.Gy = g[1] / pl[1]; p.Gx = g[2] / pl[2];
    p.G = (int32_t)G;
    rc = basa::launch_pool(p, dtype, (hipStream_t)stream);
    if (rc) return fail(rc, "pool launch failed: %s", hipGetErrorString(hipGetLastError()));
    return ok();
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_pool_kv");
  }
}

namespace {

int window_attn_impl(const void* q, const void* k, const void* v, const void* k_mem,
                     const void* v_mem, int64_t n_mem, void* out, float* lse, int32_t batch,
                     int32_t heads, int32_t head_dim, int32_t ndim, const int32_t* grid,
                     const int32_t* window, const int32_t* shift, float scale, float mem_bias,
                     int32_t dtype, int32_t layout, void* stream) {
  {
    if (const int e = empty_call(batch, heads, head_dim, dtype, layout); e >= 0) return e;
    if (!q || !k || !v || !out) return fail(BASA_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
    int rc = check_common(batch, heads, head_dim, dtype, layout);
    if (rc) return rc;
    int32_t g[3], w[3], s[3];
    int64_t n;
    if ((rc = check_grid(ndim, grid, g, &n))) return rc;
    if ((rc = check_divides(ndim, window, g, w, "window"))) return rc;
    if ((rc = read3(ndim, shift, 0, s, "shift"))) return rc;
    if ((k_mem == nullptr) != (v_mem == nullptr))
      return fail(BASA_ERR_INVALID_ARG, "k_mem and v_mem must both be given or both be NULL");
    if (k_mem && (n_mem < 1 || n_mem > (1 << 20)))
      return fail(BASA_ERR_INVALID_ARG, "n_mem must be in [1, 2^20] with memory (got %lld)", (long long)n_mem);
    if (!k_mem && n_mem != 0) return fail(BASA_ERR_INVALID_ARG, "n_mem must be 0 without memory");
    if (not_finite(scale)) return fail(BASA_ERR_INVALID_ARG, "scale must be finite");
    if (not_finite(mem_bias)) return fail(BASA_ERR_INVALID_ARG, "mem_bias must be finite");
    const int64_t m = (int64_t)w[0] * w[1] * w[2];
    if (m > BASA_MAX_WINDOW_TOKENS)
      return fail(BASA_ERR_UNSUPPORTED, "window of %lld tokens exceeds %d", (long long)m, BASA_MAX_WINDOW_TOKENS);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (k_mem && (!aligned16(k_mem) || !aligned16(v_mem))))
      return fail(BASA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    int64_t sb, sh, stok;
    strides(layout, heads, n, head_dim, &sb, &sh, &stok);
    if (n * stok >= INT32_MAX) return fail(BASA_ERR_UNSUPPORTED, "grid too large for 32-bit token offsets");
    const size_t es = dtype == BASA_BF16 ? 2 : 4;
    const size_t tb = (size_t)batch * heads * n * head_dim * es;
    const size_t mb = k_mem ? (size_t)batch * heads * n_mem * head_dim * es : 0;
    if (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb) ||
        overlaps(out, tb, k_mem, mb) || overlaps(out, tb, v_mem, mb))
      return fail(BASA_ERR_INVALID_ARG, "out overlaps an input");
    if (lse) {
      if (dtype != BASA_BF16) return fail(BASA_ERR_UNSUPPORTED, "lse output needs dtype BASA_BF16");
      if ((uintptr_t)lse % 4) return fail(BASA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
      const size_t lb = (size_t)batch * heads * n * 4;
      if (overlaps(lse, lb, q, tb) || overlaps(lse, lb, k, tb) || overlaps(lse, lb, v, tb) ||
          overlaps(lse, lb, out, tb) || overlaps(lse, lb, k_mem, mb) || overlaps(lse, lb, v_mem, mb))
        return fail(BASA_ERR_INVALID_ARG, "lse overlaps an input or out");
    }

    basa::AttnParams p{};
    p.lse = lse;
    p.n_tok = (int32_t)n;
    p.q = (const uint16_t*)q; p.k = (const uint16_t*)k; p.v = (const uint16_t*)v;
    p.kmem = (const uint16_t*)k_mem; p.vmem = (const uint16_t*)v_mem; p.out = (uint16_t*)out;
    p.stride_b = sb; p.stride_h = sh; p.stride_tok = (int32_t)stok;
    p.heads = heads; p.batch_heads = batch * heads; p.head_dim = head_dim;
    p.m = (int32_t)m;
    p.G = k_mem ? (int32_t)n_mem : 0;
    p.nW = (int32_t)(n / m);
    p.scale = resolve_scale(scale, head_dim);
    p.c1 = p.scale * basa::kLog2e;
    p.mem_bias = k_mem ? mem_bias : 0.0f;
    p.mem_bias_raw = p.mem_bias / p.scale;
    basa::Geometry& geo = p.geo;
    geo.T = g[0]; geo.Hg = g[1]; geo.Wg = g[2];
    geo.wt = w[0]; geo.wy = w[1]; geo.wx = w[2];
    // any integer shift, reduced into [0, window)
    geo.st = ((s[0] % w[0]) + w[0]) % w[0];
    geo.sy = ((s[1] % w[1]) + w[1]) % w[1];
    geo.sx = ((s[2] % w[2]) + w[2]) % w[2];
    geo.nwy = g[1] / w[1];
    geo.nwx = g[2] / w[2];
    geo.mwx = basa::magic_of(w[2]);
    geo.mwy = basa::magic_of(w[1]);
    rc = dtype == BASA_BF16 ? basa::launch_attn_bf16(p, false, (hipStream_t)stream)
                            : basa::launch_attn_f32(p, false, (hipStream_t)stream);
    if (rc == BASA_ERR_UNSUPPORTED) return fail(rc, "launch shape not supported");
    if (rc) return fail(rc, "window attention launch failed: %s", hipGetErrorString(hipGetLastError()));
    return ok();
  }
}

}  // namespace

int basa_window_attn(const void* q, const void* k, const void* v, const void* k_mem,
                     const void* v_mem, int64_t n_mem, void* out, int32_t batch, int32_t heads,
                     int32_t head_dim, int32_t ndim, const int32_t* grid, const int32_t* window,
                     const int32_t* shift, float scale, float mem_bias, int32_t dtype,
                     int32_t layout, void* stream) {
  try {
    return window_attn_impl(q, k, v, k_mem, v_mem, n_mem, out, nullptr, batch, heads, head_dim,
                            ndim, grid, window, shift, scale, mem_bias, dtype, layout, stream);
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_window_attn");
  }
}

int basa_window_attn_fwd(const void* q, const void* k, const void* v, const void* k_mem,
                         const void* v_mem, int64_t n_mem, void* out, float* lse, int32_t batch,
                         int32_t heads, int32_t head_dim, int32_t ndim, const int32_t* grid,
                         const int32_t* window, const int32_t* shift, float scale, float mem_bias,
                         int32_t dtype, int32_t layout, void* stream) {
  try {
    if (!lse) return fail(BASA_ERR_INVALID_ARG, "lse must be non-NULL");
    return window_attn_impl(q, k, v, k_mem, v_mem, n_mem, out, lse, batch, heads, head_dim, ndim,
                            grid, window, shift, scale, mem_bias, dtype, layout, stream);
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_window_attn_fwd");
  }
}

namespace {

// Queries per memory-key unit of the backward (a multiple of 32).
constexpr int64_t kBwdQueryChunk = 1024;

struct BwdWorkspace {
  size_t dvec, pk, pv, gk, gv, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

BwdWorkspace bwd_workspace(int64_t bh, int64_t n, int64_t G, int32_t head_dim,
                           int64_t qchunk = kBwdQueryChunk) {
  BwdWorkspace w{};
  const int64_t nqc = (n + qchunk - 1) / qchunk;
  size_t off = 0;
  w.dvec = off; off += align256((size_t)bh * n * 4);
  const size_t part = G ? (size_t)bh * nqc * G * head_dim * 4 : 0;
  const size_t red = G ? (size_t)bh * G * head_dim * 4 : 0;
  w.pk = off; off += align256(part);
  w.pv = off; off += align256(part);
  w.gk = off; off += align256(red);
  w.gv = off; off += align256(red);
  w.total = off;
  return w;
}

}  // namespace

int64_t basa_window_attn_bwd_workspace(int32_t batch, int32_t heads, int32_t head_dim,
                                       int32_t ndim, const int32_t* grid, const int32_t* pool) {
  try {
    if (batch < 1 || heads < 1 || (head_dim != 64 && head_dim != 128)) return -1;
    int32_t g[3];
    int64_t n;
    if (check_grid(ndim, grid, g, &n)) return -1;
    int64_t G = 0;
    if (pool) {
      int32_t pl[3];
      if (check_divides(ndim, pool, g, pl, "pool")) return -1;
      G = (int64_t)(g[0] / pl[0]) * (g[1] / pl[1]) * (g[2] / pl[2]);
    }
    ok();
    return (int64_t)bwd_workspace((int64_t)batch * heads, n, G, head_dim).total;
  } catch (...) {
    return -1;
  }
}

namespace {

// The backward with a caller's workspace, or (use_scratch) with the static
// scratch array, the memory-key query chunk then enlarged until the
// workspace fits it.
int window_attn_bwd_impl(const void* q, const void* k, const void* v, const void* k_mem,
                         const void* v_mem, const void* out, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv, void* workspace, int64_t workspace_bytes,
                         bool use_scratch, int32_t batch, int32_t heads, int32_t head_dim,
                         int32_t ndim, const int32_t* grid, const int32_t* window,
                         const int32_t* shift, const int32_t* pool, float scale, float mem_bias,
                         int32_t dtype, int32_t layout, void* stream) {
  {
    if (const int e = empty_call(batch, heads, head_dim, dtype, layout); e >= 0) return e;
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || (!workspace && !use_scratch))
      return fail(BASA_ERR_INVALID_ARG, "q, k, v, out, dout, lse, dq, dk, dv and workspace must be non-NULL");
    int rc = check_common(batch, heads, head_dim, dtype, layout);
    if (rc) return rc;
    if (dtype != BASA_BF16) return fail(BASA_ERR_UNSUPPORTED, "the backward needs dtype BASA_BF16");
    int32_t g[3], w[3], s[3], pl[3] = {1, 1, 1};
    int64_t n;
    if ((rc = check_grid(ndim, grid, g, &n))) return rc;
    if ((rc = check_divides(ndim, window, g, w, "window"))) return rc;
    if ((rc = read3(ndim, shift, 0, s, "shift"))) return rc;
    if ((pool == nullptr) != (k_mem == nullptr) || (k_mem == nullptr) != (v_mem == nullptr))
      return fail(BASA_ERR_INVALID_ARG, "pool, k_mem and v_mem must all be given or all be NULL");
    int64_t G = 0;
    if (pool) {
      if ((rc = check_divides(ndim, pool, g, pl, "pool"))) return rc;
      G = (int64_t)(g[0] / pl[0]) * (g[1] / pl[1]) * (g[2] / pl[2]);
    }
    if (not_finite(scale)) return fail(BASA_ERR_INVALID_ARG, "scale must be finite");
    if (not_finite(mem_bias)) return fail(BASA_ERR_INVALID_ARG, "mem_bias must be finite");
    const int64_t m = (int64_t)w[0] * w[1] * w[2];
    if (m > BASA_MAX_WINDOW_TOKENS)
      return fail(BASA_ERR_UNSUPPORTED, "window of %lld tokens exceeds %d", (long long)m, BASA_MAX_WINDOW_TOKENS);
    const void* ptrs[] = {q, k, v, out, dout, dq, dk, dv, workspace};
    for (const void* ptr : ptrs)
      if (!aligned16(ptr)) return fail(BASA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    if (k_mem && (!aligned16(k_mem) || !aligned16(v_mem)))
      return fail(BASA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    if ((uintptr_t)lse % 4) return fail(BASA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    int64_t sb, sh, stok;
    strides(layout, heads, n, head_dim, &sb, &sh, &stok);
    if (n * stok >= INT32_MAX) return fail(BASA_ERR_UNSUPPORTED, "grid too large for 32-bit token offsets");
    int64_t qchunk = kBwdQueryChunk;
    BwdWorkspace ws = bwd_workspace((int64_t)batch * heads, n, G, head_dim, qchunk);
    if (use_scratch) {
      // fewer, longer query chunks: fewer memory-key partials to keep
      while (ws.total > (size_t)BASA_BWD_SCRATCH_BYTES && qchunk < n) {
        qchunk *= 2;
        ws = bwd_workspace((int64_t)batch * heads, n, G, head_dim, qchunk);
      }
      if (ws.total > (size_t)BASA_BWD_SCRATCH_BYTES)
        return fail(BASA_ERR_UNSUPPORTED,
                    "the backward needs %lld bytes of workspace, more than the %lld-byte scratch "
                    "array (use basa_window_attn_bwd with a workspace)",
                    (long long)ws.total, (long long)BASA_BWD_SCRATCH_BYTES);
      workspace_bytes = (int64_t)ws.total;
    } else if (workspace_bytes < (int64_t)ws.total) {
      return fail(BASA_ERR_INVALID_ARG, "workspace of %lld bytes is smaller than the %lld needed",
                  (long long)workspace_bytes, (long long)ws.total);
    }
    const size_t tb = (size_t)batch * heads * n * head_dim * 2;
    const size_t mb = (size_t)batch * heads * G * head_dim * 2;
    const size_t lb = (size_t)batch * heads * n * 4;
    const void* ins[] = {q, k, v, out, dout};
    const void* outs[] = {dq, dk, dv};
    for (const void* o : outs) {
      for (const void* i : ins)
        if (overlaps(o, tb, i, tb)) return fail(BASA_ERR_INVALID_ARG, "an output overlaps an input");
      if (overlaps(o, tb, k_mem, mb) || overlaps(o, tb, v_mem, mb) || overlaps(o, tb, lse, lb) ||
          overlaps(o, tb, workspace, ws.total))
        return fail(BASA_ERR_INVALID_ARG, "an output overlaps an input or the workspace");
    }
    if (overlaps(dq, tb, dk, tb) || overlaps(dq, tb, dv, tb) || overlaps(dk, tb, dv, tb))
      return fail(BASA_ERR_INVALID_ARG, "dq, dk and dv overlap");
    for (const void* i : ins)
      if (overlaps(workspace, ws.total, i, tb))
        return fail(BASA_ERR_INVALID_ARG, "the workspace overlaps an input");
    if (overlaps(workspace, ws.total, lse, lb) || overlaps(workspace, ws.total, k_mem, mb) ||
        overlaps(workspace, ws.total, v_mem, mb))
      return fail(BASA_ERR_INVALID_ARG, "the workspace overlaps an input");
    if (use_scratch && (rc = scratch_address(&workspace))) return rc;

    basa::BwdParams p{};
    p.q = (const uint16_t*)q; p.k = (const uint16_t*)k; p.v = (const uint16_t*)v;
    p.kmem = (const uint16_t*)k_mem; p.vmem = (const uint16_t*)v_mem;
    p.out = (const uint16_t*)out; p.dout = (const uint16_t*)dout; p.lse = lse;
    p.dq = (uint16_t*)dq; p.dk = (uint16_t*)dk; p.dv = (uint16_t*)dv;
    char* wsb = (char*)workspace;
    p.dvec = (float*)(wsb + ws.dvec);
    p.pk = (float*)(wsb + ws.pk); p.pv = (float*)(wsb + ws.pv);
    p.gk = (float*)(wsb + ws.gk); p.gv = (float*)(wsb + ws.gv);
    p.stride_b = sb; p.stride_h = sh; p.stride_tok = (int32_t)stok;
    p.heads = heads; p.batch_heads = batch * heads; p.head_dim = head_dim;
    p.n = (int32_t)n; p.m = (int32_t)m; p.G = (int32_t)G; p.nW = (int32_t)(n / m);
    p.qchunk = (int32_t)qchunk;
    p.nqc = (int32_t)((n + qchunk - 1) / qchunk);
    p.scale = resolve_scale(scale, head_dim);
    p.c1 = p.scale * basa::kLog2e;
    p.mem_bias_raw = G ? mem_bias / p.scale : 0.0f;
    basa::Geometry& geo = p.geo;
    geo.T = g[0]; geo.Hg = g[1]; geo.Wg = g[2];
    geo.wt = w[0]; geo.wy = w[1]; geo.wx = w[2];
    geo.st = ((s[0] % w[0]) + w[0]) % w[0];
    geo.sy = ((s[1] % w[1]) + w[1]) % w[1];
    geo.sx = ((s[2] % w[2]) + w[2]) % w[2];
    geo.nwy = g[1] / w[1];
    geo.nwx = g[2] / w[2];
    geo.mwx = basa::magic_of(w[2]);
    geo.mwy = basa::magic_of(w[1]);
    p.pt = pl[0]; p.py = pl[1]; p.px = pl[2];
    p.Gy = g[1] / pl[1]; p.Gx = g[2] / pl[2];
    rc = basa::launch_attn_bwd(p, (hipStream_t)stream);
    if (rc == BASA_ERR_UNSUPPORTED) return fail(rc, "backward launch shape not supported");
    if (rc) return fail(rc, "backward launch failed: %s", hipGetErrorString(hipGetLastError()));
    return ok();
  }
}

}  // namespace

int basa_window_attn_bwd(const void* q, const void* k, const void* v, const void* k_mem,
                         const void* v_mem, const void* out, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv, void* workspace, int64_t workspace_bytes,
                         int32_t batch, int32_t heads, int32_t head_dim, int32_t ndim,
                         const int32_t* grid, const int32_t* window, const int32_t* shift,
                         const int32_t* pool, float scale, float mem_bias, int32_t dtype,
                         int32_t layout, void* stream) {
  try {
    return window_attn_bwd_impl(q, k, v, k_mem, v_mem, out, dout, lse, dq, dk, dv, workspace,
                                workspace_bytes, false, batch, heads, head_dim, ndim, grid, window,
                                shift, pool, scale, mem_bias, dtype, layout, stream);
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_window_attn_bwd");
  }
}

int basa_window_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* k_mem,
                                 const void* v_mem, const void* out, const void* dout,
                                 const float* lse, void* dq, void* dk, void* dv, int32_t batch,
                                 int32_t heads, int32_t head_dim, int32_t ndim,
                                 const int32_t* grid, const int32_t* window,
                                 const int32_t* shift, const int32_t* pool, float scale,
                                 float mem_bias, int32_t dtype, int32_t layout, void* stream) {
  try {
    return window_attn_bwd_impl(q, k, v, k_mem, v_mem, out, dout, lse, dq, dk, dv, nullptr, 0,
                                true, batch, heads, head_dim, ndim, grid, window, shift, pool,
                                scale, mem_bias, dtype, layout, stream);
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_window_attn_bwd_noalloc");
  }
}

int basa_hilbert_order(int32_t side, int32_t* order_out) {
  try {
    if (!order_out) return fail(BASA_ERR_INVALID_ARG, "order_out must be non-NULL");
    if (side < 1 || side > (1 << 15) || (side & (side - 1)))
      return fail(BASA_ERR_INVALID_ARG, "side must be a power of two in [1, 32768] (got %d)", side);
    // Iterative curve index -> (x, y): each level of two bits picks a quadrant
    // and rotates/reflects the coordinates accumulated so far.
    const int64_t n = (int64_t)side * side;
    for (int64_t d = 0; d < n; ++d) {
      int64_t t = d, x = 0, y = 0;
      for (int64_t s = 1; s < side; s *= 2) {
        const int64_t rx = 1 & (t / 2);
        const int64_t ry = 1 & (t ^ rx);
        if (ry == 0) {
          if (rx == 1) {
            x = s - 1 - x;
            y = s - 1 - y;
          }
          const int64_t tmp = x;
          x = y;
          y = tmp;
        }
        x += s * rx;
        y += s * ry;
        t /= 4;
      }
      order_out[d] = (int32_t)(y * side + x);
    }
    return ok();
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_hilbert_order");
  }
}

int basa_gather_kv(const void* k, const void* v, const int32_t* idx, int64_t n_idx, void* k_out,
                   void* v_out, int32_t batch, int32_t heads, int32_t head_dim, int64_t n_tokens,
                   int32_t dtype, int32_t layout, void* stream) {
  try {
    if (const int e = empty_call(batch, heads, head_dim, dtype, layout); e >= 0) return e;
    if (!k || !v || !idx || !k_out || !v_out)
      return fail(BASA_ERR_INVALID_ARG, "k, v, idx, k_out and v_out must be non-NULL");
    int rc = check_common(batch, heads, head_dim, dtype, layout);
    if (rc) return rc;
    if (n_tokens < 1 || n_idx < 1 || n_idx > (1 << 20))
      return fail(BASA_ERR_INVALID_ARG, "n_tokens must be >= 1 and n_idx in [1, 2^20]");
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out) || (uintptr_t)idx % 4)
      return fail(BASA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned (idx 4-byte)");
    int64_t sb, sh, stok;
    strides(layout, heads, n_tokens, head_dim, &sb, &sh, &stok);
    if (n_tokens * stok >= INT32_MAX) return fail(BASA_ERR_UNSUPPORTED, "sequence too long for 32-bit token offsets");
    const size_t es = dtype == BASA_BF16 ? 2 : 4;
    const size_t tb = (size_t)batch * heads * n_tokens * head_dim * es;
    const size_t ob = (size_t)batch * heads * n_idx * head_dim * es;
    if (overlaps(k_out, ob, k, tb) || overlaps(k_out, ob, v, tb) || overlaps(v_out, ob, k, tb) ||
        overlaps(v_out, ob, v, tb) || overlaps(k_out, ob, v_out, ob) ||
        overlaps(k_out, ob, idx, n_idx * 4) || overlaps(v_out, ob, idx, n_idx * 4))
      return fail(BASA_ERR_INVALID_ARG, "an output overlaps an input or the other output");
    basa::GatherParams p{};
    p.k = k; p.v = v; p.idx = idx; p.kout = k_out; p.vout = v_out;
    p.stride_b = sb; p.stride_h = sh; p.stride_tok = (int32_t)stok;
    p.heads = heads; p.batch_heads = batch * heads; p.head_dim = head_dim;
    p.n = (int32_t)n_tokens; p.n_idx = (int32_t)n_idx;
    rc = basa::launch_gather(p, dtype, (hipStream_t)stream);
    if (rc) return fail(rc, "gather launch failed: %s", hipGetErrorString(hipGetLastError()));
    return ok();
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_gather_kv");
  }
}

int basa_curve_attn(const void* q, const void* k, const void* v, const void* k_mem,
                    const void* v_mem, int64_t n_mem, void* out, int32_t batch, int32_t heads,
                    int32_t head_dim, int64_t n_tokens, const int32_t* order, int32_t tile,
                    int64_t slide, float scale, float mem_bias, int32_t dtype, int32_t layout,
                    void* stream) {
  try {
    if (const int e = empty_call(batch, heads, head_dim, dtype, layout); e >= 0) return e;
    if (!q || !k || !v || !out || !order)
      return fail(BASA_ERR_INVALID_ARG, "q, k, v, out and order must be non-NULL");
    int rc = check_common(batch, heads, head_dim, dtype, layout);
    if (rc) return rc;
    if (n_tokens < 1) return fail(BASA_ERR_INVALID_ARG, "n_tokens must be >= 1");
    if (tile < 1 || n_tokens % tile)
      return fail(BASA_ERR_INVALID_ARG, "tile (%d) must be positive and divide n_tokens (%lld)", tile, (long long)n_tokens);
    if (tile > BASA_MAX_WINDOW_TOKENS)
      return fail(BASA_ERR_UNSUPPORTED, "tile of %d tokens exceeds %d", tile, BASA_MAX_WINDOW_TOKENS);
    if ((k_mem == nullptr) != (v_mem == nullptr))
      return fail(BASA_ERR_INVALID_ARG, "k_mem and v_mem must both be given or both be NULL");
    if (k_mem && (n_mem < 1 || n_mem > (1 << 20)))
      return fail(BASA_ERR_INVALID_ARG, "n_mem must be in [1, 2^20] with memory (got %lld)", (long long)n_mem);
    if (!k_mem && n_mem != 0) return fail(BASA_ERR_INVALID_ARG, "n_mem must be 0 without memory");
    if (not_finite(scale)) return fail(BASA_ERR_INVALID_ARG, "scale must be finite");
    if (not_finite(mem_bias)) return fail(BASA_ERR_INVALID_ARG, "mem_bias must be finite");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (k_mem && (!aligned16(k_mem) || !aligned16(v_mem))) || (uintptr_t)order % 4)
      return fail(BASA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned (order 4-byte)");
    int64_t sb, sh, stok;
    strides(layout, heads, n_tokens, head_dim, &sb, &sh, &stok);
    if (n_tokens * stok >= INT32_MAX) return fail(BASA_ERR_UNSUPPORTED, "sequence too long for 32-bit token offsets");
    const size_t es = dtype == BASA_BF16 ? 2 : 4;
    const size_t tb = (size_t)batch * heads * n_tokens * head_dim * es;
    const size_t mb = k_mem ? (size_t)batch * heads * n_mem * head_dim * es : 0;
    if (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb) ||
        overlaps(out, tb, k_mem, mb) || overlaps(out, tb, v_mem, mb) ||
        overlaps(out, tb, order, n_tokens * 4))
      return fail(BASA_ERR_INVALID_ARG, "out overlaps an input");
    basa::AttnParams p{};
    p.q = (const uint16_t*)q; p.k = (const uint16_t*)k; p.v = (const uint16_t*)v;
    p.kmem = (const uint16_t*)k_mem; p.vmem = (const uint16_t*)v_mem; p.out = (uint16_t*)out;
    p.stride_b = sb; p.stride_h = sh; p.stride_tok = (int32_t)stok;
    p.heads = heads; p.batch_heads = batch * heads; p.head_dim = head_dim;
    p.m = tile;
    p.G = k_mem ? (int32_t)n_mem : 0;
    p.nW = (int32_t)(n_tokens / tile);
    p.scale = resolve_scale(scale, head_dim);
    p.c1 = p.scale * basa::kLog2e;
    p.mem_bias = k_mem ? mem_bias : 0.0f;
    p.mem_bias_raw = p.mem_bias / p.scale;
    p.n_tok = (int32_t)n_tokens;
    p.order = order;
    p.slide = (int32_t)(((slide % n_tokens) + n_tokens) % n_tokens);
    // a 1-D grid of nW rows of `tile` tokens; only the window count is read
    basa::Geometry& geo = p.geo;
    geo.T = 1; geo.Hg = p.nW; geo.Wg = tile;
    geo.wt = 1; geo.wy = 1; geo.wx = tile;
    geo.nwy = p.nW; geo.nwx = 1;
    geo.mwx = basa::magic_of(tile);
    geo.mwy = basa::magic_of(1);
    rc = dtype == BASA_BF16 ? basa::launch_attn_bf16(p, false, (hipStream_t)stream)
                            : basa::launch_attn_f32(p, false, (hipStream_t)stream);
    if (rc == BASA_ERR_UNSUPPORTED) return fail(rc, "launch shape not supported");
    if (rc) return fail(rc, "curve attention launch failed: %s", hipGetErrorString(hipGetLastError()));
    return ok();
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_curve_attn");
  }
}

int basa_calib_mfma(float* sink, int32_t blocks, int32_t iters, void* stream) {
  try {
    if (!sink) return fail(BASA_ERR_INVALID_ARG, "sink must be non-NULL");
    if (blocks < 1 || iters < 1) return fail(BASA_ERR_INVALID_ARG, "blocks and iters must be >= 1");
    const int rc = basa::launch_mfma_rate(sink, blocks, iters, (hipStream_t)stream);
    if (rc) return fail(rc, "calibration launch failed: %s", hipGetErrorString(hipGetLastError()));
    return ok();
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_calib_mfma");
  }
}

int basa_dense_attn(const void* q, const void* k, const void* v, void* out, int32_t batch,
                    int32_t heads, int64_t n_q, int64_t n_kv, int32_t head_dim, float scale,
                    int32_t dtype, int32_t layout, void* stream) {
  try {
    if (const int e = empty_call(batch, heads, head_dim, dtype, layout); e >= 0) return e;
    if (!q || !k || !v || !out) return fail(BASA_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
    int rc = check_common(batch, heads, head_dim, dtype, layout);
    if (rc) return rc;
    if (n_q < 1 || n_kv < 1) return fail(BASA_ERR_INVALID_ARG, "n_q and n_kv must be >= 1");
    if (not_finite(scale)) return fail(BASA_ERR_INVALID_ARG, "scale must be finite");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
      return fail(BASA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
    int64_t sb, sh, stok, kb, kh, ktok;
    strides(layout, heads, n_q, head_dim, &sb, &sh, &stok);
    strides(layout, heads, n_kv, head_dim, &kb, &kh, &ktok);
    if (n_q * stok >= INT32_MAX || n_kv * ktok >= INT32_MAX)
      return fail(BASA_ERR_UNSUPPORTED, "sequence too long for 32-bit token offsets");
    const size_t es = dtype == BASA_BF16 ? 2 : 4;
    const size_t qb = (size_t)batch * heads * n_q * head_dim * es;
    const size_t kvb = (size_t)batch * heads * n_kv * head_dim * es;
    if (overlaps(out, qb, q, qb) || overlaps(out, qb, k, kvb) || overlaps(out, qb, v, kvb))
      return fail(BASA_ERR_INVALID_ARG, "out overlaps an input");
    basa::AttnParams p{};
    p.q = (const uint16_t*)q; p.k = (const uint16_t*)k; p.v = (const uint16_t*)v;
    p.kmem = nullptr; p.vmem = nullptr; p.out = (uint16_t*)out;
    p.stride_b = sb; p.stride_h = sh; p.stride_tok = (int32_t)stok;
    p.kv_stride_b = kb; p.kv_stride_h = kh;
    p.heads = heads; p.batch_heads = batch * heads; p.head_dim = head_dim;
    p.m = (int32_t)n_q;
    p.n_kv = (int32_t)n_kv;
    p.G = 0;
    p.nW = 1;
    p.scale = resolve_scale(scale, head_dim);
    p.c1 = p.scale * basa::kLog2e;
    rc = dtype == BASA_BF16 ? basa::launch_attn_bf16(p, true, (hipStream_t)stream)
                            : basa::launch_attn_f32(p, true, (hipStream_t)stream);
    if (rc == BASA_ERR_UNSUPPORTED) return fail(rc, "launch shape not supported");
    if (rc) return fail(rc, "dense attention launch failed: %s", hipGetErrorString(hipGetLastError()));
    return ok();
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_dense_attn");
  }
}

int basa_full_attn(const void* q, const void* k, const void* v, void* out, int32_t batch,
                   int32_t heads, int64_t n_tokens, int32_t head_dim, float scale, int32_t dtype,
                   int32_t layout, void* stream) {
  return basa_dense_attn(q, k, v, out, batch, heads, n_tokens, n_tokens, head_dim, scale, dtype,
                         layout, stream);
}

int basa_center_region(int32_t grid_y, int32_t grid_x, int32_t size_y, int32_t size_x,
                       int32_t* idx_out) {
  try {
    if (!idx_out) return fail(BASA_ERR_INVALID_ARG, "idx_out must be non-NULL");
    if (grid_y < 1 || grid_x < 1 || size_y < 1 || size_x < 1 || size_y > grid_y ||
        size_x > grid_x)
      return fail(BASA_ERR_INVALID_ARG, "need 1 <= size <= grid on both axes");
    if ((int64_t)grid_y * grid_x > INT32_MAX)
      return fail(BASA_ERR_INVALID_ARG, "grid too large for int32 token indices");
    // the block's first row and column leave (grid - size) / 2 tokens before
    // it (rounded down) and the rest after it
    const int32_t y0 = (grid_y - size_y) / 2, x0 = (grid_x - size_x) / 2;
    for (int32_t i = 0; i < size_y; ++i)
      for (int32_t j = 0; j < size_x; ++j) idx_out[i * size_x + j] = (y0 + i) * grid_x + x0 + j;
    return ok();
  } catch (...) {
    return fail(BASA_ERR_HIP, "unexpected exception in basa_center_region");
  }
}

}  // extern "C"
