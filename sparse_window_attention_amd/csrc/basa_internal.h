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
};

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

int launch_attn_bf16(const AttnParams& p, bool full, hipStream_t stream);
int launch_attn_f32(const AttnParams& p, bool full, hipStream_t stream);
int launch_pool(const PoolParams& p, int dtype, hipStream_t stream);

}  // namespace basa
