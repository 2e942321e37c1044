/*
 * basa.h -- C ABI of the shifted-window sparse attention library (gfx950).
 *
 * The library computes BASA-style attention for diffusion transformers:
 * self-attention over the visual token grid of an image (2D) or video (3D)
 * is replaced by dense attention inside non-overlapping local windows, the
 * window partition is cyclically shifted from one DiT block to the next, and
 * each window's keys may be extended by a global memory of mean-pooled K/V
 * tokens under the same softmax.
 *
 * Sources (the web pages this library is written from):
 *   [BASA-1] BASA forum summary, English mirror of "BASA: Backend-Agnostic
 *            Sparse Attention for Fast High-Resolution Diffusion
 *            Transformers" (zhichai.net), sections "Summary", "Overview",
 *            "The BASA Method".
 *   [BASA-2] BASA discussion reply (zhichai.net topic reply), paragraphs on
 *            the method's four parts and on its complexity.
 *   [SFA]    Scale-Free Attention abstract (artificialintelbulletin.com):
 *            mean pooling, token-count correction, one shared softmax.
 *   [HilbertA] "HilbertA: Hilbert Attention for Image Generation with
 *            Diffusion Models", catalogue record (info.umar.mx), abstract:
 *            Hilbert-curve token order, tiles along it, a sliding schedule,
 *            a small shared central region.
 *
 * Conventions shared by every call
 *   - Plain C types only; device buffers are raw device pointers, shape and
 *     geometry arrays are host pointers read during the call only.
 *   - Tensors Q, K, V, O hold B x H x n x D elements with D contiguous and
 *     the n tokens in raster order of the grid, idx = (t*Hg + y)*Wg + x.
 *     layout BASA_LAYOUT_BHND: element (b,h,i,d) at ((b*H + h)*n + i)*D + d.
 *     layout BASA_LAYOUT_BNHD: element (b,h,i,d) at ((b*n + i)*H + h)*D + d.
 *     Memory tensors k_mem, v_mem are always [B, H, G, D] contiguous.
 *   - A 2D grid is given as ndim = 2 with arrays (Hg, Wg); a 3D grid as
 *     ndim = 3 with (T, Hg, Wg).  Window, shift and pool arrays have ndim
 *     entries in the same axis order.
 *   - dtype: BASA_BF16 (inputs and outputs bf16, fp32 accumulation and
 *     softmax) or BASA_F32 (fp32 throughout).  All tensors of one call share
 *     the dtype.
 *   - stream is a hipStream_t passed as void*; NULL means the default stream.
 *     Kernels run on the device current on the calling thread.  The library
 *     enqueues work and returns; it never synchronises the stream.
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     device memory and keeps no data between calls; its process-wide state
 *     is a per-device record of launch attributes already set (the LDS
 *     limit, the compute-unit count) and, for basa_window_attn_bwd_noalloc
 *     only, one static scratch array per GPU (see there).  Calls may run
 *     concurrently on different streams, except basa_window_attn_bwd_noalloc
 *     calls on one GPU.
 *   - Empty batches: batch or heads may be 0.  Such a call has nothing to
 *     do: it returns BASA_OK once head_dim, dtype and layout are valid,
 *     reads no pointer (they may be NULL, as an empty tensor's are) and
 *     launches nothing.
 *   - Errors: every call returns a status.  Arguments are validated before
 *     anything is enqueued; on any error nothing is launched and no output
 *     byte is written.  basa_last_error() gives a sentence naming the
 *     argument at fault (per calling thread).  Faults inside a kernel show
 *     up at the caller's next synchronisation, as for any HIP kernel.
 */
#ifndef BASA_H
#define BASA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  BASA_OK = 0,
  BASA_ERR_INVALID_ARG = 1, /* null pointer, bad dim, non-dividing window/pool,
                               n_mem mismatch, output overlapping an input   */
  BASA_ERR_UNSUPPORTED = 2, /* dtype, head_dim or sizes outside what is built */
  BASA_ERR_HIP = 3          /* the HIP runtime refused the launch            */
};
enum { BASA_F32 = 0, BASA_BF16 = 1 };
enum { BASA_LAYOUT_BHND = 0, BASA_LAYOUT_BNHD = 1 };
enum { BASA_SCHED_NONE = 0, BASA_SCHED_ALTERNATE = 1, BASA_SCHED_FOUR_PHASE = 2 };

/* Largest window (tokens per window) basa_window_attn accepts. */
#define BASA_MAX_WINDOW_TOKENS 4096

/* Bytes of the per-GPU scratch array basa_window_attn_bwd_noalloc uses as its
 * workspace (64 MiB). */
#define BASA_BWD_SCRATCH_BYTES (64ll << 20)

/* Library ABI version (major*100 + minor). */
int32_t basa_version(void);

/* Text for a status code (static storage). */
const char* basa_status_string(int32_t status);

/* Sentence describing the last non-OK status returned on this thread. */
const char* basa_last_error(void);

/*
 * Number of pooled memory tokens G = prod(grid[i] / pool[i]) [BASA-2, the
 * global memory of pooled K/V; SFA, mean pooling].  Returns -1 when ndim is
 * not 2 or 3, a pointer is NULL, a dim is not positive or a pool factor does
 * not divide its grid dim.  Host only.
 */
int64_t basa_mem_tokens(int32_t ndim, const int32_t* grid, const int32_t* pool);

/*
 * Window shift for DiT block block_idx [BASA-1, "The BASA Method": the
 * window partition shifts in a structured way from block to block]:
 *   BASA_SCHED_NONE       zero shift;
 *   BASA_SCHED_ALTERNATE  zero on even blocks, floor(window[i]/2) on odd;
 *   BASA_SCHED_FOUR_PHASE phase = block_idx mod 2^ndim, axis i shifted by
 *                         floor(window[i]/2) when bit i of phase is set
 *                         (2D: (0,0), (w/2,0), (0,w/2), (w/2,w/2)).
 * Writes ndim ints to shift_out (host).  Errors: INVALID_ARG for NULL,
 * ndim not in {2,3}, block_idx < 0, window[i] <= 0, unknown schedule.
 */
int basa_shift_for_block(int32_t block_idx, int32_t schedule, int32_t ndim,
                         const int32_t* window, int32_t* shift_out);

/*
 * Mean-pooled K/V memory [BASA-2, the global memory of pooled K/V; SFA,
 * mean pooling]: k_mem[b,h,g,:] is the mean of k over pool cell g of the
 * unshifted grid (cells in raster order of the pooled grid); the same for v.
 * Accumulates in fp32 and stores in dtype (bf16 rounded to nearest even).
 *   k, v          device, B x H x n x D in `layout`, n = prod(grid)
 *   k_mem, v_mem  device, [B, H, G, D] contiguous, G = basa_mem_tokens()
 *   batch, heads  >= 0 (0: an empty batch);  head_dim in {64, 128}
 *   ndim, grid, pool  host arrays of ndim entries; pool must divide grid
 * Errors: INVALID_ARG (NULL, bad dims, pool not dividing the grid, an output
 * overlapping an input or the other output), UNSUPPORTED (dtype, head_dim).
 */
int basa_pool_kv(const void* k, const void* v, void* k_mem, void* v_mem,
                 int32_t batch, int32_t heads, int32_t head_dim,
                 int32_t ndim, const int32_t* grid, const int32_t* pool,
                 int32_t dtype, int32_t layout, void* stream);

/*
 * Shifted local window attention with optional pooled memory [BASA-1,
 * "Summary" and "The BASA Method"; BASA-2 four-parts paragraph; SFA shared
 * softmax].  For every token i of the grid
 *   out[i] = softmax_j( scale * q[i].k[j] + bias_j ) v[j]
 * over j in the window of i under the shifted partition, followed by the G
 * memory tokens (bias_j = mem_bias for memory keys, 0 otherwise).  Token
 * p = (t,y,x) lies in window ( ((t-st) mod T)/wt, ((y-sy) mod Hg)/wy,
 * ((x-sx) mod Wg)/wx ) (integer division): the grid is cyclically rolled by
 * -shift, cut into windows, attended, and rolled back.  Wrapped tokens are
 * not masked.  No shifted copy is made: the roll is in the addressing.
 *   q, k, v, out  device, B x H x n x D in `layout`; out must not overlap any
 *                 input
 *   k_mem, v_mem  device [B, H, n_mem, D] contiguous, or both NULL with
 *                 n_mem = 0 for no memory.  n_mem is the number of memory
 *                 rows (normally basa_mem_tokens() of the pool that made
 *                 them); any n_mem in [1, 2^20] is accepted
 *   window        divides grid on every axis; prod(window) <=
 *                 BASA_MAX_WINDOW_TOKENS
 *   shift         any integers; reduced modulo the window on each axis (a
 *                 shift equal to the window is no shift)
 *   scale         softmax scale; <= 0 selects 1/sqrt(head_dim)
 *   mem_bias      added to every memory logit before the softmax (natural
 *                 log units); 0 for the plain concatenation, ln(cell size)
 *                 for the token-count corrected reading [SFA]
 *   head_dim      {64, 128}
 * Errors: INVALID_ARG, UNSUPPORTED (dtype, head_dim, window too large).
 */
int basa_window_attn(const void* q, const void* k, const void* v,
                     const void* k_mem, const void* v_mem, int64_t n_mem,
                     void* out,
                     int32_t batch, int32_t heads, int32_t head_dim,
                     int32_t ndim, const int32_t* grid, const int32_t* window,
                     const int32_t* shift, float scale, float mem_bias,
                     int32_t dtype, int32_t layout, void* stream);

/*
 * basa_window_attn that also writes, for every query token, the natural-log
 * log-sum-exp of its scaled and biased logits over [window keys; memory
 * keys] -- the statistic the backward recomputes the softmax from.  The
 * training side of the method (the dense-teacher adaptation the BASA pages
 * describe) needs gradients; this forward feeds basa_window_attn_bwd.
 *   lse   device fp32 [B, H, n] (n = prod(grid), tokens in raster order),
 *         4-byte aligned, not overlapping any other argument
 * Other arguments and errors as basa_window_attn; UNSUPPORTED unless dtype
 * is BASA_BF16.
 */
int basa_window_attn_fwd(const void* q, const void* k, const void* v,
                         const void* k_mem, const void* v_mem, int64_t n_mem,
                         void* out, float* lse,
                         int32_t batch, int32_t heads, int32_t head_dim,
                         int32_t ndim, const int32_t* grid, const int32_t* window,
                         const int32_t* shift, float scale, float mem_bias,
                         int32_t dtype, int32_t layout, void* stream);

/*
 * Bytes of device workspace basa_window_attn_bwd needs for this shape (pool
 * NULL: no memory).  Returns -1 for arguments it rejects.  Host only.
 */
int64_t basa_window_attn_bwd_workspace(int32_t batch, int32_t heads, int32_t head_dim,
                                       int32_t ndim, const int32_t* grid,
                                       const int32_t* pool);

/*
 * Gradients of basa_window_attn with respect to q, k and v [BASA-1, "The
 * BASA Method"; BASA-2 four-parts paragraph; SFA shared softmax], the
 * memory included: k_mem and v_mem must be the mean pool of k and v over
 * `pool` (basa_pool_kv), and their gradient flows back into dk and dv (each
 * token of a cell receives the cell's gradient divided by the cell size).
 * Softmax probabilities are recomputed from lse.
 *   q, k, v          device, B x H x n x D in `layout` (the forward's inputs)
 *   k_mem, v_mem     device [B, H, G, D]: the forward's memory, or NULL with
 *                    pool NULL for attention without memory
 *   out, dout        device, B x H x n x D in `layout`: forward output and
 *                    the gradient of the loss with respect to it
 *   lse              device fp32 [B, H, n] from basa_window_attn_fwd
 *   dq, dk, dv       device, B x H x n x D in `layout`: written entirely
 *   workspace        device, at least basa_window_attn_bwd_workspace()
 *                    bytes, 16-byte aligned; contents are scratch
 *   grid, window, shift, scale, mem_bias as for the forward; pool as for
 *   basa_pool_kv (NULL: no memory)
 * bf16 only; fp32 accumulation; P and dS are rounded to bf16 as MFMA
 * operands.  Errors: INVALID_ARG (NULL, bad dims, non-dividing window or
 * pool, pool/k_mem/v_mem not all given or all NULL, workspace too small,
 * an output overlapping an input, another output or the workspace),
 * UNSUPPORTED (dtype, head_dim, window too large).
 */
int basa_window_attn_bwd(const void* q, const void* k, const void* v,
                         const void* k_mem, const void* v_mem,
                         const void* out, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv,
                         void* workspace, int64_t workspace_bytes,
                         int32_t batch, int32_t heads, int32_t head_dim,
                         int32_t ndim, const int32_t* grid, const int32_t* window,
                         const int32_t* shift, const int32_t* pool,
                         float scale, float mem_bias,
                         int32_t dtype, int32_t layout, void* stream);

/*
 * basa_window_attn_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  Arguments, results and errors as
 * basa_window_attn_bwd.  The call allocates nothing: its workspace is a
 * static device array of BASA_BWD_SCRATCH_BYTES that the library holds on
 * every GPU it runs on, from its first use there to the end of the process.
 * To fit that array the memory-key gradients are summed over query chunks
 * larger than the workspace form uses (1024 queries, doubled as needed), so
 * those sums are grouped differently and dk, dv may differ from
 * basa_window_attn_bwd's in the last bits.  A shape whose workspace does not
 * fit even with one chunk per head returns BASA_ERR_UNSUPPORTED (nothing is
 * launched); at 24 heads of 16384 tokens, D = 128, 256 memory tokens it
 * needs 58 MB.  Every call on one GPU uses that GPU's one array and leaves
 * its contents behind (no part of it needs to start at zero): calls that
 * overlap in time on one GPU (other streams, other threads) race on it and
 * give undefined results; serialise them.
 */
int basa_window_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                                 const void* k_mem, const void* v_mem, const void* out,
                                 const void* dout, const float* lse, void* dq, void* dk,
                                 void* dv, int32_t batch, int32_t heads, int32_t head_dim,
                                 int32_t ndim, const int32_t* grid, const int32_t* window,
                                 const int32_t* shift, const int32_t* pool, float scale,
                                 float mem_bias, int32_t dtype, int32_t layout, void* stream);

/*
 * Token order along a Hilbert curve of a side x side grid [HilbertA,
 * abstract: tokens reordered along Hilbert curves keep 2D neighbourhoods in a
 * contiguous layout]: order_out[d] = y*side + x of curve position d, starting
 * at (0, 0); consecutive positions are grid neighbours and every aligned run
 * of 4^k positions covers a 2^k x 2^k square.  Writes side*side ints (host).
 * Errors: INVALID_ARG for NULL or side not a power of two in [1, 32768].
 */
int basa_hilbert_order(int32_t side, int32_t* order_out);

/*
 * Row gather: k_out[b,h,i,:] = k[b,h,idx[i],:] and the same for v -- the
 * keys of a shared region (HilbertA's small central region every tile also
 * attends to) as the memory operand of basa_curve_attn.
 *   k, v          device, B x H x n_tokens x D in `layout`
 *   idx           device int32 [n_idx] token indices (clamped into range)
 *   k_out, v_out  device [B, H, n_idx, D] contiguous
 * Errors: INVALID_ARG (NULL, sizes, alignment, an output overlapping an
 * input), UNSUPPORTED (dtype, head_dim).
 */
int basa_gather_kv(const void* k, const void* v, const int32_t* idx, int64_t n_idx,
                   void* k_out, void* v_out, int32_t batch, int32_t heads,
                   int32_t head_dim, int64_t n_tokens, int32_t dtype, int32_t layout,
                   void* stream);

/*
 * Attention inside tiles of an explicit token order, with the same kernels
 * and optional memory as basa_window_attn [HilbertA, abstract: contiguous
 * tiles along the curve, a sliding schedule across layers, a shared central
 * region].  Tile j holds the tokens order[(j*tile + slide + r) mod n],
 * r < tile; every query attends to its tile's keys followed by the n_mem
 * memory keys under one softmax.  With the raster order this is window
 * attention over a grid of n/tile rows of `tile` tokens.
 *   order    device int32 [n_tokens]: a permutation of 0..n-1 (entries out
 *            of range are clamped; a non-permutation gives a well-defined
 *            but meaningless result)
 *   tile     divides n_tokens, <= BASA_MAX_WINDOW_TOKENS
 *   slide    any integer, reduced modulo n_tokens
 *   other arguments as basa_window_attn (n_tokens in place of the grid)
 * Errors: INVALID_ARG, UNSUPPORTED as basa_window_attn.
 */
int basa_curve_attn(const void* q, const void* k, const void* v,
                    const void* k_mem, const void* v_mem, int64_t n_mem, void* out,
                    int32_t batch, int32_t heads, int32_t head_dim, int64_t n_tokens,
                    const int32_t* order, int32_t tile, int64_t slide,
                    float scale, float mem_bias, int32_t dtype, int32_t layout,
                    void* stream);

/*
 * Calibration, not part of the method: runs the library's bf16 MFMA loop
 * (four independent chains of 32x32x16 products per wave, no memory
 * traffic) over `blocks` workgroups of 8 waves, `iters` iterations each, so a
 * caller can time the matrix-core rate the chip sustains and use it beside
 * the vendor's dense peak as a roofline denominator.  Work per call:
 * blocks * 8 * iters * 4 * 32768 flops.
 *   sink    device float [blocks], receives one value per workgroup
 *   blocks  >= 1; iters >= 1
 * Errors: INVALID_ARG (NULL sink, sizes), HIP (launch).
 */
int basa_calib_mfma(float* sink, int32_t blocks, int32_t iters, void* stream);

/*
 * Dense full attention out = softmax(scale * q k^T) v over all n_tokens keys
 * per (batch, head) [BASA-2 complexity paragraph: the O(n^2) cost that window
 * attention reduces to O(n*m)].  Built only to measure realised against
 * theoretical speedup.  Arguments as for basa_window_attn; n_tokens >= 1.
 */
int basa_full_attn(const void* q, const void* k, const void* v, void* out,
                   int32_t batch, int32_t heads, int64_t n_tokens,
                   int32_t head_dim, float scale, int32_t dtype, int32_t layout,
                   void* stream);

/*
 * Dense attention with n_q queries and n_kv keys per (batch, head):
 * out = softmax(scale * q k^T) v, with no window, shift or memory.  This is
 * the unmodified dense kernel a stock backend provides [BASA-1, "Overview"
 * and "The BASA Method": the method needs no custom operator and runs on
 * existing dense attention backends once the roll and the window partition
 * are materialised]; the composition baseline calls it over B*nW "batches"
 * of [window keys; memory keys].  basa_full_attn is the case n_q = n_kv.
 *   q, out   device, B x H x n_q x D in `layout`
 *   k, v     device, B x H x n_kv x D in the same layout
 *   n_q, n_kv >= 1; other arguments as basa_full_attn
 * Errors: INVALID_ARG (NULL, sizes, alignment, out overlapping an input),
 * UNSUPPORTED (dtype, head_dim, offsets beyond 32 bits), HIP (launch).
 */
int basa_dense_attn(const void* q, const void* k, const void* v, void* out,
                    int32_t batch, int32_t heads, int64_t n_q, int64_t n_kv,
                    int32_t head_dim, float scale, int32_t dtype, int32_t layout,
                    void* stream);

/*
 * The shared central region of Hilbert-order tiles [HilbertA, abstract: a
 * small central region that every tile also attends to]: raster indices
 * y*grid_x + x of the size_y x size_x block of a grid_y x grid_x grid whose
 * first row and column are (grid - size) / 2 (rounded down), in raster order
 * (host).  The result is the idx argument of basa_gather_kv.
 *   idx_out  host int32 [size_y * size_x], written
 * Errors: INVALID_ARG for NULL, a size outside [1, grid] on either axis, or
 * a grid of more than 2^31 - 1 tokens.
 */
int basa_center_region(int32_t grid_y, int32_t grid_x, int32_t size_y, int32_t size_x,
                       int32_t* idx_out);

#ifdef __cplusplus
}
#endif

#endif /* BASA_H */
