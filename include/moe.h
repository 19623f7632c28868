/*
 * moe.h -- C ABI of the routed sparse-MoE layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (reference page "Agent Field Notes -- full corpus"):
 *   router logits -> float32 softmax with normalized top-k selection
 *     (AFN-001 "Porting Qwen3.8-Flash-Next to Hebrus: evidence before
 *     execution", section "Phase 1: separate math from acceleration");
 *   exact expert IDs in rank order (AFN-021 "Replay decode as prefill ...",
 *     section "The key equivalence -- and where it breaks"), equal scores
 *     resolved toward the lower index while choosing membership (AFN-017
 *     "Top-k chooses the set; time chooses the order", section "Tie handling
 *     belongs to membership");
 *   token rows grouped by expert so every selected expert record is read once
 *     per batch (AFN-019 "Hide SSD misses before the router knows they
 *     exist", sections "Why overlap alone cannot defeat the byte roofline"
 *     and "Hypothesis H5");
 *   SwiGLU experts: gate and up together, down after the intermediate exists,
 *     results in separate slots, weighted sum in route-rank order (AFN-019,
 *     section "Hypothesis H4: ExpertMajor should stream as a wavefront, not a
 *     barrier"); geometry and parameter count per expert (gate [I x H] + up
 *     [I x H] + down [H x I]) from AFN-019 "Why overlap alone cannot defeat
 *     the byte roofline".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory)
 *   owned by the caller; the library never allocates device memory.  Scratch
 *   memory is the caller's workspace of at least moe_workspace_size(shape)
 *   bytes (NULL allowed when that is 0); its contents need no initialisation.
 *   Between calls a workspace carries only the FFN tile plan and the
 *   arrival counters of the single-launch paths, both written by the
 *   library's own kernels (from moe_permute / moe_route_permute to
 *   moe_ffn_gate_up / moe_ffn_down / moe_ffn_down_combine); the library
 *   keeps no other state.
 * - Every call only ENQUEUES work on `stream` (NULL = the null stream) and
 *   returns without synchronizing.  Calls on different streams with disjoint
 *   outputs and workspaces are independent.
 * - Row-major, densely packed layouts; every pointer 16-byte aligned.
 * - Validation is complete before anything is enqueued: a non-MOE_OK return
 *   means no kernel was launched and no output byte was written
 *   (fail-closed, the rule of AFN-001 section "Phase 3: reject before the
 *   GPU exists").  MOE_E_DEVICE reports a HIP error while enqueuing; a fault of
 *   a kernel already enqueued is reported by the HIP runtime at the caller's
 *   next synchronization (a GPU memory fault ends the process), not by a
 *   later call of this library.
 * - Index tensors are int32; weights and logits are float32.
 *
 * Domain (MOE_E_SHAPE / MOE_E_LIMIT otherwise):
 *   0 <= T <= 131072 (T == 0 is a no-op returning MOE_OK),
 *   1 <= top_k <= E <= 1024,
 *   H > 0 with H % 128 == 0, I > 0 with I % 32 == 0, H, I <= 65536,
 *   T * top_k < 2^31, T * max(E, H) < 2^31, and the FFN tile count bound
 *   T*top_k/(16*nb) + min(E, T*top_k) <= 65535 (nb = 1 for T <= 16, float32
 *   or T*top_k <= 12*E; else 2 for T <= 1024; else 8 for bf16 dense weights
 *   in the tiled layout without MOE_F_FUSED_FFN once T*top_k >= 48*E and
 *   I % 128 == 0; else 4).
 * Formats (MOE_E_DTYPE / MOE_E_FORMAT otherwise):
 *   act MOE_DT_F32  with wfmt MOE_WF_DENSE (float32 weights);
 *   act MOE_DT_BF16 with wfmt MOE_WF_DENSE (bf16 weights), MOE_WF_INT4_G32
 *   or MOE_WF_INT2_G32 (the router weight is always in the act type).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_E_NULL = 1,       /* a required pointer is NULL                          */
  MOE_E_SHAPE = 2,      /* a dimension is outside the domain above             */
  MOE_E_DTYPE = 3,      /* unknown activation type                            */
  MOE_E_FORMAT = 4,     /* unknown weight format or unsupported combination    */
  MOE_E_ALIGN = 5,      /* a pointer is not 16-byte aligned                    */
  MOE_E_ALIAS = 6,      /* an output overlaps an input or another output       */
  MOE_E_WORKSPACE = 7,  /* workspace NULL or smaller than moe_workspace_size() */
  MOE_E_LIMIT = 8,      /* index arithmetic would exceed 2^31                  */
  MOE_E_DEVICE = 9,     /* HIP reported an error while enqueuing               */
  MOE_E_FLAGS = 10,     /* unknown bit in moe_shape.flags                      */
  MOE_E_NONFINITE = 11, /* MOE_F_CHECK_FINITE found a NaN or infinity; caller
                           outputs were not written                            */
  MOE_E_MEMORY = 12     /* a source buffer is not memory the device can read
                           (e.g. pageable host memory)                         */
} moe_status;

typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 } moe_dtype;

/* Expert weight storage.  Low-bit formats (AFN-019, "Why overlap alone cannot
 * defeat the byte roofline": low-bit storage) hold signed two's-complement
 * codes q with one IEEE fp16 scale s per 32 consecutive elements along the
 * reduction axis; the weight is q * s.  Codes are packed little-endian along
 * the reduction axis: element k of a row is in byte k/2, low nibble first
 * (int4), or in byte k/4 at bit 2*(k%4) (int2). */
typedef enum { MOE_WF_DENSE = 0, MOE_WF_INT4_G32 = 1, MOE_WF_INT2_G32 = 2 } moe_wformat;

/* moe_shape.flags bits. */
#define MOE_F_TILED_WEIGHTS 0x1u /* expert weights in the tiled layout (moe_tile_experts) */
/* Non-finite rejection with transactional publication ("Agent Field Notes --
 * full corpus", AFN-010 "One bank flip is enough: make the whole inference
 * chunk transactional", section "The publication model": outputs stay
 * private while work is fallible, finite checks and device status must
 * pass, then everything is published at one point).  Honoured by moe_route and moe_layer, ignored by the other entry
 * points: the call computes into the workspace, checks x, the router logits
 * and (moe_layer) the layer output for NaN / infinity on the device, then
 * SYNCHRONIZES the stream.  A non-finite value returns MOE_E_NONFINITE with
 * every caller output untouched; otherwise the results are copied to the
 * caller outputs (enqueued on the stream) and MOE_OK is returned. */
#define MOE_F_CHECK_FINITE 0x2u
/* Fused expert FFN (AFN-019, "Hypothesis H4": gate/up -> down as component
 * waves, no barrier between them; see moe_ffn_fused).  Requires
 * MOE_F_TILED_WEIGHTS (MOE_E_FLAGS otherwise) and T * top_k <= 16384
 * (MOE_E_LIMIT otherwise: the workspace then holds (I/64) float32 partial
 * results per pair and feature).  moe_layer runs the FFN as moe_ffn_fused
 * with one wave of all tiles and adds the partial results in its combine
 * (y is not formed); moe_ffn_fused requires the flag; the other entry
 * points ignore it. */
#define MOE_F_FUSED_FFN 0x4u

typedef struct {
  int32_t T;       /* tokens in the batch                        */
  int32_t H;       /* hidden width                               */
  int32_t E;       /* routed experts                             */
  int32_t I;       /* expert intermediate width                  */
  int32_t top_k;   /* experts selected per token                 */
  int32_t act;     /* moe_dtype of x, W_router, dense W, Y, out   */
  int32_t wfmt;    /* moe_wformat of the expert weights          */
  uint32_t flags;  /* MOE_F_* bits; other bits must be 0        */
} moe_shape;

/* Expert weights, expert-major (one contiguous record per component).
 *   dense: gate, up [E][I][H], down [E][H][I] in the act type.
 *   int4 : gate, up uint8 [E][I][H/2], down uint8 [E][H][I/2];
 *   int2 : gate, up uint8 [E][I][H/4], down uint8 [E][H][I/4];
 *   scales (low-bit only, fp16 bit patterns): gate_scale, up_scale
 *   [E][I][H/32], down_scale [E][H][I/32]; must be NULL for dense. */
typedef struct {
  const void* gate;
  const void* up;
  const void* down;
  const uint16_t* gate_scale;
  const uint16_t* up_scale;
  const uint16_t* down_scale;
} moe_experts;

/* Tiled expert layout (MOE_F_TILED_WEIGHTS).  Same bytes as the row-major
 * layout, reordered so that every 16-row x 32-column MFMA operand fragment is
 * contiguous and a wave's load instruction reads one contiguous block.  For
 * one matrix W[N][K] of one expert (gate/up: N = I, K = H; down: N = H, K = I),
 * with nb < N/16, r < 16, q < 4, j < 8:
 *   bf16: element W[16nb + r][32ks + 8q + j] at element index
 *         ((nb*(K/32) + ks)*64 + 16q + r)*8 + j           (ks < K/32);
 *   int4/int2: the 8 codes c_j = W[16nb + r][128kb + 32s + 8q + j] (j = 0..7,
 *         kb < K/128, s < 4) of lane unit u = (nb*(K/128) + kb)*64 + 16q + r
 *         are stored offset-binary (c + 8 for int4, c + 2 for int2) in the
 *         B bytes at byte offset u*B (B = 16 for int4, 8 for int2), read as
 *         little-endian 32-bit words:
 *         int4: word s holds c_2m at nibble m and c_2m+1 at nibble m+4 (m < 4);
 *         int2: word s/2 holds c_2m at bits 8(s%2) + 2m and c_2m+1 at bits
 *         16 + 8(s%2) + 2m (m < 4);
 *         so that one mask and one OR turn a (c_2m, c_2m+1) pair into two
 *         bf16 values;
 *   scales: scale[16nb + r][4kb + s] at fp16 index ((nb*(K/128) + kb)*16 + r)*4 + s.
 * Requirements: bf16 activations; I % 128 == 0 (MOE_E_SHAPE otherwise). */

/* Per-expert permutation of the P = T*top_k (token, slot) pairs, pair index
 * p = t*top_k + j.  Rows of expert e are rows offsets[e] .. offsets[e+1]-1,
 * in ascending p (hence ascending token).  All arrays int32, device memory:
 *   counts[E], offsets[E+1], sorted_pair[P] (row -> p), pair_row[P]
 *   (p -> row), active[E] (the first *n_active entries are the experts with
 *   counts > 0 in ascending order; the rest are -1), n_active[1]. */
typedef struct {
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_row;
  int32_t* active;
  int32_t* n_active;
} moe_perm;

/* Rewrite row-major expert weights (shape->flags must be 0) into the tiled
 * layout above.  src and dst are disjoint device buffers of the same sizes;
 * the scale pointers are NULL exactly when the format is dense.  One kernel
 * per component, enqueued on `stream`; a one-time conversion done when the
 * weights are loaded. */
int moe_tile_experts(const moe_shape* shape, const moe_experts* src,
                     const moe_experts* dst, hipStream_t stream);

/* Bytes of workspace every entry point below needs for this shape (the
 * maximum over all of them, so one buffer serves every call).  Host-only,
 * pure.  Returns 0 for an invalid shape. */
size_t moe_workspace_size(const moe_shape* shape);

/* Static description of a status code; never NULL. */
const char* moe_status_str(int status);

/* Router (AFN-001, section "Phase 1: separate math from acceleration":
 * float32 router softmax and normalized top-k; AFN-017, section "Tie
 * handling belongs to membership"; AFN-021, section "The key equivalence --
 * and where it breaks": exact IDs in rank order):
 * logits[t][e] = sum_h x[t][h] * w_router[e][h] + bias[e], then the
 * top_k experts of each token by (logit descending, expert index ascending),
 * emitted in rank order, and their weights w[t][j] = exp(l_j - l_0) /
 * sum_i exp(l_i - l_0) over the selected logits (equal to the full float32
 * softmax renormalized over the selection).
 *   x [T][H] act; w_router [E][H] act; router_bias float [E] or NULL;
 *   topk_ids int32 [T][top_k], topk_w float [T][top_k] (outputs);
 *   logits float [T][E] or NULL (optional output, the float32 logits the
 *   selection used).
 * bf16: the exact bf16 products are summed in float32 within each 32-wide
 * chunk of H and the chunk sums in float64, then rounded once to float32.
 * float32: products and sums in float64, rounded once to float32. */
int moe_route(const moe_shape* shape, const void* x, const void* w_router,
              const float* router_bias, int32_t* topk_ids, float* topk_w,
              float* logits, void* workspace, size_t workspace_bytes,
              hipStream_t stream);

/* Stable grouping of the pairs by expert (the permutation described at
 * moe_perm; AFN-019, section "Why overlap alone cannot defeat the byte
 * roofline": token rows grouped by expert, repeated routes read once).  Also writes the grouped-FFN tile plan into the workspace (read
 * by moe_ffn_gate_up and moe_ffn_down).  topk_ids [T][top_k]: every entry in [0, E) and the top_k
 * entries of one token distinct (as moe_route produces); other inputs are
 * memory-safe but give an unspecified permutation. */
int moe_permute(const moe_shape* shape, const int32_t* topk_ids,
                const moe_perm* perm, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/* moe_route followed by moe_permute (same outputs as the two calls, with
 * `perm` receiving the permutation and the workspace the FFN tile plan), in
 * as few launches as the shape allows: for bf16 batches of up to 32 tokens
 * the top-k kernel's last workgroup builds the permutation, so routing and
 * grouping take two kernel launches instead of three (AFN-019, "Why overlap
 * alone cannot defeat the byte roofline": rows grouped by expert, repeated
 * routes deduplicated).  Arguments as moe_route, plus perm (outputs). */
int moe_route_permute(const moe_shape* shape, const void* x, const void* w_router,
                      const float* router_bias, int32_t* topk_ids, float* topk_w, float* logits,
                      const moe_perm* perm, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Grouped SwiGLU experts (AFN-019, section "Why overlap alone cannot defeat
 * the byte roofline": gate [I x H] + up [I x H] + down [H x I] per expert;
 * section "Hypothesis H4": gate and up together, down once the intermediate
 * exists, a separate result slot per (token, expert)).  For every row r of
 * expert e with pair p =
 * sorted_pair[r] and token t = p / top_k:
 *   y[r][n] = sum_i W_down[e][n][i] * silu(g_i) * u_i,
 *   g_i = sum_h W_gate[e][i][h] x[t][h],  u_i = sum_h W_up[e][i][h] x[t][h].
 * Each active expert's weights are streamed from memory once per call for
 * its whole row set when it has at most 16*nb rows, the tile height (nb as
 * in the domain above), otherwise once per tile.  perm: counts, offsets,
 * sorted_pair, active, n_active are read (pair_row is not used).  y [P][H] act (output, rows in permuted order).
 * The SwiGLU intermediate is kept in the act type (bf16 or float32). */
int moe_grouped_ffn(const moe_shape* shape, const void* x,
                    const moe_experts* experts, const moe_perm* perm, void* y,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The two components of moe_grouped_ffn as separate calls, for callers
 * that schedule them separately (AFN-019, "Hypothesis H4": gate and up are
 * used together, down only after the SwiGLU intermediate exists):
 *   moe_ffn_gate_up: h[r][i] = silu(g_i) * u_i for every row r (h [P][I] in
 *     the act type, output; rows in permuted order);
 *   moe_ffn_down:    y[r][n] = sum_i W_down[e][n][i] * h[r][i].
 * Both read the FFN tile plan that moe_permute (or moe_layer) leaves in the
 * workspace for this shape: call moe_permute with the same shape and
 * workspace first and do not write the workspace in between.  perm supplies
 * sorted_pair (gate/up only).  Each call is one kernel launch. */
int moe_ffn_gate_up(const moe_shape* shape, const void* x,
                    const moe_experts* experts, const moe_perm* perm, void* h,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);
int moe_ffn_down(const moe_shape* shape, const void* h,
                 const moe_experts* experts, void* y, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* moe_ffn_down followed by moe_combine: out[t][n] = residual[t][n] +
 * sum_{j ascending} topk_w[t][j] * y_(t,j)[n] with y_(t,j) = W_down[e] h of
 * the pair's row (AFN-019, "Hypothesis H4": separate result slots, the
 * weighted sum in route-rank order).  The expert outputs y stay in the
 * workspace.  With 16-row tiles (the plan's choice while T*top_k <= 12*E or
 * T <= 16) of tiled weights the down kernel writes y in pair order, so the
 * combine reads a token's slots without the pair -> row lookup.  The result
 * equals moe_ffn_down + moe_combine bit for bit.  Reads the tile plan left by moe_permute (or
 * moe_route_permute) for this shape and workspace; perm supplies
 * sorted_pair and pair_row; h [P][I] act as from moe_ffn_gate_up; topk_w
 * [T][top_k]; residual [T][H] act or NULL; out [T][H] act. */
int moe_ffn_down_combine(const moe_shape* shape, const void* h, const moe_experts* experts,
                         const moe_perm* perm, const float* topk_w, const void* residual, void* out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The grouped SwiGLU experts (same y as moe_grouped_ffn, up to float
 * rounding order) as one kernel of component waves (AFN-019, "Hypothesis
 * H4": gate+up first, down as soon as the intermediate exists, waves of 2, 4
 * or all experts, separate result slots).  Work item = (tile, slice of 64
 * intermediate columns): one workgroup computes the SwiGLU intermediate of
 * its tile rows for those 64 columns (bf16, in LDS) and at once its share of
 * the down projection, a float32 partial y_s[row][0..H) for slice s; no
 * workgroup waits for another.  y[r] = bf16(sum over s ascending of
 * y_s[r]).  Items are numbered in waves of `wave_tiles` consecutive tiles of
 * the plan (0: one wave of all tiles), slice-major inside a wave; with
 * T <= 16 each active expert is exactly one tile.  shape->flags must hold
 * MOE_F_TILED_WEIGHTS | MOE_F_FUSED_FFN (MOE_E_FLAGS otherwise);
 * wave_tiles < 0 is MOE_E_SHAPE.  perm as for moe_grouped_ffn.
 * item_clock: NULL, or uint64 [3 * moe_ffn_fused_items(shape)] (output): for
 * item i < n_tiles * (I/64) (i = wave * W * S + slice * nt + tile-in-wave,
 * S = I/64, nt the tiles in that wave), the device wall clock
 * (moe_device_clock_khz) at the item's start, after its gate/up and after its
 * down; entries of items past the last tile are not written. */
int moe_ffn_fused(const moe_shape* shape, const void* x, const moe_experts* experts,
                  const moe_perm* perm, void* y, int32_t wave_tiles, uint64_t* item_clock,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Capacity in items of moe_ffn_fused's item_clock (max tiles * I/64) for a
 * valid shape with MOE_F_FUSED_FFN; 0 otherwise.  Host-only. */
size_t moe_ffn_fused_items(const moe_shape* shape);

/* Rate of the device wall clock of the current device in kHz (ticks per
 * millisecond), for item_clock. */
int moe_device_clock_khz(int32_t* khz);

/* Route-rank-order combine (AFN-019, section "Hypothesis H4": the weighted
 * sum of the separate result slots in a fixed route-rank order):
 * out[t][n] = residual[t][n] +
 * sum_{j=0}^{top_k-1} topk_w[t][j] * y[pair_row[t*top_k+j]][n], accumulated
 * in float32 with j ascending, rounded once to the act type.
 *   y [P][H] act; pair_row [P]; topk_w [T][top_k]; residual [T][H] act or
 *   NULL; out [T][H] act (must not overlap y, residual or topk_w). */
int moe_combine(const moe_shape* shape, const void* y, const int32_t* pair_row,
                const float* topk_w, const void* residual, void* out,
                hipStream_t stream);

/* The whole layer (the passages cited at the four calls; layers in sequence,
 * x_{l+1} = x_l + moe_l(x_l) with residual = x: AFN-019, section "Hypothesis
 * H6"): moe_route -> moe_permute -> moe_grouped_ffn -> moe_combine with the
 * same semantics, enqueued back to back (as moe_route_permute ->
 * moe_ffn_gate_up -> moe_ffn_down_combine).  perm may be
 * NULL (the permutation then lives in the workspace); residual may be NULL;
 * topk_ids/topk_w are outputs.  out must not overlap x or residual. */
int moe_layer(const moe_shape* shape, const void* x, const void* w_router,
              const float* router_bias, const moe_experts* experts,
              const void* residual, void* out, int32_t* topk_ids, float* topk_w,
              const moe_perm* perm, void* workspace, size_t workspace_bytes,
              hipStream_t stream);

/* moe_layer for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same validation, kernels and results as moe_layer, with the workspace
 * taken from a fixed device array inside the library instead of an argument.
 * The call allocates nothing.  Each device holds one such array of
 * MOE_NOALLOC_SCRATCH_BYTES from the first call on it until the process
 * ends; its device address is looked up on that first call, so make the
 * first call on a device outside graph capture.
 *   - A shape whose moe_workspace_size exceeds MOE_NOALLOC_SCRATCH_BYTES is
 *     rejected with MOE_E_WORKSPACE before any HIP call (at H = 2560,
 *     E = 512, I = 640, top-10 that is T > ~800 tokens).
 *   - `stream` must belong to the current device (MOE_E_DEVICE otherwise).
 *   - Every call on one device shares that device's array: calls that may
 *     overlap on one device (different streams, or host threads without
 *     ordering) race and give undefined results.  Calls enqueued on one
 *     stream are ordered and safe.  The array keeps the last call's contents;
 *     the layer needs none of it initialised.
 * Other arguments, outputs and error codes as moe_layer. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_noalloc(const moe_shape* shape, const void* x, const void* w_router,
                      const float* router_bias, const moe_experts* experts,
                      const void* residual, void* out, int32_t* topk_ids, float* topk_w,
                      const moe_perm* perm, hipStream_t stream);

/* Stage the active experts' records into device memory (AFN-019,
 * "Hypothesis H5": a block reads the deduplicated union of its routes;
 * "Why overlap alone cannot defeat the byte roofline": exact bytes first).
 * For a = 0 .. *perm->n_active - 1 and e = perm->active[a], copies the
 * records of expert e selected by `parts` (MOE_STAGE_GATE_UP: gate and up
 * with their scales; MOE_STAGE_DOWN: down with its scale) from `src` to the
 * same expert positions of `dst`; other experts' regions of dst are not
 * written.  Gate and up are needed together and down only after them, so a
 * caller may stage down on a second stream while gate/up runs (the pages'
 * component split).  src and dst have the same layout (row-major, or tiled
 * when shape->flags has MOE_F_TILED_WEIGHTS); dst is device memory.  src may
 * be pinned host memory (hipHostMalloc, torch pin_memory) or device memory:
 * the GPU reads it directly, so the active set never goes to the host.  One
 * kernel launch.  MOE_E_FLAGS if parts is 0 or has an unknown bit;
 * MOE_E_MEMORY if a src buffer is not device-readable or a dst buffer is not
 * device memory. */
#define MOE_STAGE_GATE_UP 0x1u
#define MOE_STAGE_DOWN 0x2u
int moe_stage_experts(const moe_shape* shape, const moe_experts* src, const moe_experts* dst,
                      const moe_perm* perm, uint32_t parts, hipStream_t stream);

/* Route locality of the token sequence t = 0..T-1 of one call (AFN-019,
 * "Hypothesis H7: DFlash block size must follow I/O cost", and its
 * trace-only locality gate).  With S_t the set {topk_ids[t][j]}:
 *   overlap_prev[t] = |S_t intersect S_{t-1}|, overlap_prev[0] = 0;
 *   block_unique[o_B + b] = |S_{bB} union ... union S_{min(T, bB+B) - 1}|
 *     for B = 1..5 and b < ceil(T/B), with o_1 = 0 and
 *     o_{B+1} = o_B + ceil(T/B); moe_route_locality_blocks(T) entries.
 * int32, exact.  topk_ids [T][top_k] rows must hold distinct experts (as
 * moe_route produces); values are only compared.  overlap_prev [T] and
 * block_unique are outputs.  Cost per block value O(B^2 top_k^2) compares.
 * The mean of block_unique over the blocks of size B is U_B; a verifier
 * block of B tokens reads fewer routed bytes per accepted token than top-k
 * decoding iff U_B < top_k * tau(B). */
size_t moe_route_locality_blocks(int32_t T);
int moe_route_locality(const moe_shape* shape, const int32_t* topk_ids, int32_t* overlap_prev,
                       int32_t* block_unique, hipStream_t stream);

/* Measurement helper, not part of the layer: streams `bytes` (a non-zero
 * multiple of 16) from `buf` once with 16-byte loads spread over 2048
 * workgroups, the read-bandwidth ceiling that the layer's kernels are
 * compared with.  `sink` is one uint32 the kernel may write (not a result).
 * buf 16-byte aligned, sink 4-byte aligned and outside buf. */
int moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
