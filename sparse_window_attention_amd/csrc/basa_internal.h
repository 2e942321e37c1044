// Host/device interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "basa.h"
#include "basa_common.h"

namespace basa {

// Arguments of one attention launch.  Element strides are in elements of the
// call's dtype.  For full attention m = n, nW = 1, G = 0.
struct AttnParams {
  const uint16_t* q;      // bf16 views (reinterpreted for fp32 launches)
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kmem;   // [B, H, G, D]; unused when G = 0
  const uint16_t* vmem;
  uint16_t* out;
  int64_t stride_b;       // between batches
  int64_t stride_h;       // between heads
  int32_t stride_tok;     // between tokens
  int32_t heads;
  int32_t batch_heads;    // B * H
  int32_t head_dim;
  int32_t m;              // tokens per window (queries and window keys)
  int32_t G;              // memory tokens
  int32_t nW;             // windows per (batch, head)
  int32_t nQT;            // query tiles per window (set by the launcher)
  int32_t units;          // B*H*nW*nQT (set by the launcher)
  int32_t units_per_xcd;  // ceil(units / 8) (set by the launcher)
  float c1;               // softmax scale * log2(e)
  float scale;            // softmax scale
  float mem_bias_raw;     // memory logit bias divided by the scale
  float mem_bias;         // memory logit bias (natural log units)
  Geometry geo;
  float* lse;             // optional [B*H, n_tok] fp32 natural-log log-sum-exp of every query
  int32_t n_tok;          // tokens per (batch, head)
  const int32_t* order;   // optional device [n_tok]: a token order whose runs of m
                          // consecutive positions are the windows (replaces geo)
  int32_t slide;          // start of window 0 along `order`, in [0, n_tok)
  // dense attention only: keys (and values) per (batch, head) and the strides
  // of the K/V tensors between batches and heads (the token stride is
  // stride_tok); for window attention the keys are the window's m tokens and
  // the G memory rows, addressed with the strides of Q
  int32_t n_kv;
  int64_t kv_stride_b, kv_stride_h;
};

// Raster token of slot r of window `win`: under the shifted grid partition,
// or, with an explicit token order, position (win*m + slide + r) mod n of
// that order (entries are clamped into [0, n) so any array is memory-safe).
__device__ __forceinline__ int32_t slot_token(const AttnParams& p, int32_t win, int32_t r) {
  if (p.order != nullptr) {
    const int32_t pos = (int32_t)(((int64_t)win * p.m + p.slide + r) % p.n_tok);
    const int32_t t = p.order[pos];
    return t < 0 ? 0 : (t >= p.n_tok ? p.n_tok - 1 : t);
  }
  return window_token(p.geo, win, r);
}

struct PoolParams {
  const void* k;
  const void* v;
  void* kmem;
  void* vmem;
  int64_t stride_b, stride_h;
  int32_t stride_tok;
  int32_t heads, batch_heads, head_dim;
  int32_t T, Hg, Wg;
  int32_t pt, py, px;
  int32_t Gt, Gy, Gx, G;
};

// Arguments of the backward of window attention (bf16).  Element strides as
// in AttnParams; lse, dvec and the workspaces are fp32.
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kmem;   // pooled memory of k, v ([B, H, G, D]); unused when G = 0
  const uint16_t* vmem;
  const uint16_t* out;    // forward output
  const uint16_t* dout;   // gradient of the output
  const float* lse;       // [B*H, n] natural-log log-sum-exp from the forward
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dvec;            // workspace [B*H, n]: row sums of dout * out
  float* pk;              // workspace [B*H, nqc, G, D]: memory-key partial gradients
  float* pv;
  float* gk;              // workspace [B*H, G, D]: memory gradients over the cell size
  float* gv;              //   (gk also carries the softmax scale)
  int64_t stride_b, stride_h;
  int32_t stride_tok;
  int32_t heads, batch_heads, head_dim;
  int32_t n, m, G, nW;
  int32_t qchunk, nqc;    // memory-key units: queries per chunk, chunks per head
  float c1, scale, mem_bias_raw;
  Geometry geo;
  int32_t pt, py, px, Gy, Gx;  // pool cells (G = 0: no memory)
};

int launch_attn_bwd(const BwdParams& p, hipStream_t stream);

int launch_attn_bf16(const AttnParams& p, bool full, hipStream_t stream);
int launch_attn_f32(const AttnParams& p, bool full, hipStream_t stream);
int launch_pool(const PoolParams& p, int dtype, hipStream_t stream);

// Row gather: k_out[bh, i, :] = k[bh, idx[i], :] (same for v), outputs
// [B*H, n_idx, D] contiguous, indices clamped into [0, n).
struct GatherParams {
  const void* k;
  const void* v;
  const int32_t* idx;
  void* kout;
  void* vout;
  int64_t stride_b, stride_h;
  int32_t stride_tok;
  int32_t heads, batch_heads, head_dim, n, n_idx;
};
int launch_gather(const GatherParams& p, int dtype, hipStream_t stream);
// Calibration: the bf16 MFMA loop of calib.hip over `blocks` workgroups.
int launch_mfma_rate(float* sink, int blocks, int iters, hipStream_t stream);

}  // namespace basa
