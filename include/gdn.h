/*
 * gdn.h - C ABI of the MI355X (gfx950) Gated DeltaNet decode mixer.
 *
 * The mixer is the part of the GDN layer between the qkv / alpha / beta / z
 * projections and the output projection, in the order the GDN layer's docstring
 * on the "include/strata/core/layer.hpp" page gives and `gdn_layer` on the
 * "src/core/layer.cpp" page runs (its steps 3 to 7):
 *
 *   gdn_conv_silu_norm  depthwise causal conv (d_conv = 4) with a rolling
 *                       conv state, SiLU on all C channels, L2 norm of the q
 *                       and k heads (v untouched), q scaled by 1/sqrt(S)
 *   gdn_decode_step     beta = sigmoid(beta logit), gate = softplus(alpha + dt)
 *                       * ssm_a, then the gated delta rule on each value head's
 *                       S x S fp32 state; T >= 1 tokens per call, state held
 *                       on chip across the tokens of one call
 *   gdn_gated_rmsnorm   y = rms_norm(o) * w * sigmoid(z)   (sigmoid, not SiLU; the
 *                       SiLU gate of an earlier model is a geometry option)
 *
 * States live in a pool of slots carved from caller-provided device memory (the
 * pattern of `gdn_buffers_bytes` / `gdn_buffers_init` / `gdn_buffers_zero_state`
 * on the layer.hpp page); a call works on a batch of B sequences whose states are
 * gathered from the pool by a device array of slot indices.
 *
 * Conventions for every function:
 *   - Pointers are DEVICE pointers unless the comment says host.  `stream` is a
 *     hipStream_t passed as void* (NULL = the null stream of the current device).
 *   - The library never allocates, frees or synchronises device memory and never
 *     throws or exits across this ABI.  Work is only enqueued on `stream`; the
 *     call returns before it runs.  Calls are capturable into HIP graphs (no
 *     memset nodes are recorded; zeroing uses a kernel).
 *   - Outputs are overwritten; state and conv state are updated in place.
 *   - All float data is fp32, row-major, last index fastest, 16-byte aligned.
 *   - Return value: GDN_OK, or a negative GDN_ERR_* code; gdn_last_error() then
 *     names the function and the argument.  Nothing is enqueued on error.
 *   - Errors that only the device can see (a slot index outside the pool, a
 *     token count outside [0, T]) do not fault: the kernel skips that sequence
 *     (slot) or clamps the count, and ORs a GDN_FLAG_* bit into the pool's flag
 *     word (gdn_state_pool_flags), which the caller may read and clear.
 *   - Slots within one call must be unique; duplicates race.  Calls on one pool
 *     are ordered only by the stream they are enqueued on.
 *
 * Geometry supported by the GPU path: s = 128, d_conv = 4, h_k >= 1 and h_v a
 * multiple of h_k (the pages' model is h_k = 16, h_v = 48, C = 10240).  Anything
 * else returns GDN_ERR_UNSUPPORTED.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 7

enum {
    GDN_OK = 0,
    GDN_ERR_ARG = -1,          /* a null, misaligned, negative or inconsistent argument */
    GDN_ERR_UNSUPPORTED = -2,  /* a geometry the GPU kernels are not built for */
    GDN_ERR_HIP = -3           /* the HIP runtime reported an error (message says which) */
};

/* Bits of the pool's device flag word. */
#define GDN_FLAG_BAD_SLOT 0x1u  /* a slot index was < 0 or >= n_slots: that sequence was skipped */
#define GDN_FLAG_BAD_NTOK 0x2u  /* a token count was outside [0, T]: it was clamped */

/* GDN geometry: qk heads, value heads, head size S, conv width.  The value head i
 * reads qk head i / (h_v / h_k).  Channels C = (2*h_k + h_v) * s: q | k | v.
 * Two model options (0 or 1; zero-initialised = the pages' model):
 *   gate_silu            the gated RMSNorm's gate is z * sigmoid(z) (SiLU) instead of
 *                        sigmoid(z): the layer.hpp docstring gives SiLU for an earlier
 *                        model of the family and sigmoid for this one;
 *   scale_after_readout  the extra 1/sqrt(S) multiplies the readout o instead of q
 *                        (step 4 of gdn_layer: the legacy recurrence consumes a
 *                        prescaled q, the pinned CUDA path scales after the readout
 *                        dot); h then carries the unit-norm q.  Same o up to rounding. */
typedef struct gdn_geom {
    int32_t h_k;
    int32_t h_v;
    int32_t s;
    int32_t d_conv;
    int32_t gate_silu;
    int32_t scale_after_readout;
} gdn_geom;

/* Opaque host-side descriptor of a state pool.  It owns no device memory. */
typedef struct gdn_pool gdn_pool;

/* ABI version of the loaded library (GDN_ABI_VERSION it was built with). */
int gdn_abi_version(void);

/* Message of the last failed call on this host thread ("" if none). */
const char* gdn_last_error(void);

/* ---------------------------------------------------------------- state pool
 * Device layout of a pool carved from `dev_base` (256-byte aligned):
 *   [flags: 256 B, one uint32 flag word at offset 0]
 *   [state: n_slots x h_v x s x s fp32]   state[slot][i][r][c]: r = key index,
 *                                          c = value index (o = S^T q reads
 *                                          down the rows)
 *   [conv:  n_slots x C x (d_conv-1) fp32] conv[slot][c][j]: the last d_conv-1
 *                                          RAW qkv inputs of channel c, oldest
 *                                          first
 * Each region starts on a 256-byte boundary.  Per slot at the pages' geometry:
 * 3 MiB of state + 120 KiB of conv history. */

/* Bytes a pool of n_slots needs (0 if the arguments are invalid, n_slots is outside
 * [1, 2^31] or the pool would not fit in the address space).  Host call. */
size_t gdn_state_pool_bytes(const gdn_geom* g, int64_t n_slots);

/* Describe a pool over `dev_base` (>= gdn_state_pool_bytes bytes of device memory
 * on the current device, 256-byte aligned, owned by the caller and outliving the
 * pool).  Contents are NOT initialised: call gdn_state_pool_zero or write the
 * state and conv regions directly.  *out receives a host-allocated descriptor. */
int gdn_state_pool_create(const gdn_geom* g, int64_t n_slots, void* dev_base, size_t bytes,
                          gdn_pool** out);

/* Free the descriptor (not the device memory).  NULL is ignored. */
void gdn_state_pool_destroy(gdn_pool* p);

/* Host-side validation of a slot list before it goes to the device, for callers that
 * want a debug check: the device calls skip and flag an index outside the pool but do
 * not look for repeats, whose state updates would race.  host_slots: HOST int32 [n].
 * GDN_OK when every entry lies in [0, n_slots) and none repeats; otherwise GDN_ERR_ARG,
 * and gdn_last_error() names the first entry out of range or, if none is, the first
 * entry that repeats an earlier one and the position of that earlier one.  n = 0 is
 * valid; n_slots must be positive.  Touches no device and enqueues nothing.  (The
 * pages' layer code turns inputs it cannot handle correctly into an error instead of
 * carrying on with a guess: "src/core/layer.cpp" page, the planes lookup of the
 * quantized forms.) */
int gdn_check_slots(const int32_t* host_slots, int32_t n, int64_t n_slots);

/* Device addresses of the regions above, and the pool's shape (NULL / 0 for p = NULL). */
float* gdn_state_pool_state(const gdn_pool* p);
float* gdn_state_pool_conv(const gdn_pool* p);
uint32_t* gdn_state_pool_flags(const gdn_pool* p);
int64_t gdn_state_pool_slots(const gdn_pool* p);

/* Zero the state and conv history of n slots (device int32 [n]; slots = NULL
 * zeroes every slot and n is ignored), so a fresh sequence starts from zeros
 * as `gdn_buffers_zero_state` does.  Also clears the flag word when slots is NULL. */
int gdn_state_pool_zero(gdn_pool* p, const int32_t* slots, int32_t n, void* stream);

/* ---------------------------------------------------------------- the mixer */

/* Steps 3-4 of gdn_layer for B sequences x T tokens: for every channel c,
 *   u = sum_{j<3} conv_w[c][j] * X[c][j] + conv_w[c][3] * qkv[c],  X rolled with the raw qkv,
 *   h = u * sigmoid(u)                        (all C channels, before the split)
 *   q heads (channels [0, h_k*s)):       h / sqrt(|h|^2 + eps) / sqrt(s)
 *                                        (without the / sqrt(s) when the pool's
 *                                        geometry has scale_after_readout)
 *   k heads (channels [h_k*s, 2*h_k*s)): h / sqrt(|h|^2 + eps)
 *   v (channels [2*h_k*s, C)):           unchanged
 * slots  int32 [B]          pool slot of each sequence (NULL: slot b for sequence b)
 * n_tok  int32 [B]          tokens each sequence takes, in [0, T] (NULL: all T);
 *                           outputs of tokens t >= n_tok[b] are written as 0 and
 *                           the conv history advances by n_tok[b] tokens only
 * qkv    [B][T][C]          raw projections;  conv_w [C][d_conv]
 * h      [B][T][C]          output (may not alias qkv)
 * B >= 0, T >= 1; B = 0 is a no-op. */
int gdn_conv_silu_norm(gdn_pool* p, const int32_t* slots, const int32_t* n_tok, int32_t B,
                       int32_t T, const float* qkv, const float* conv_w, float eps, float* h,
                       void* stream);

/* Steps 5-6 of gdn_layer for B sequences x T tokens, token by token:
 *   beta = sigmoid(beta_logit), g = softplus(alpha + dt[i]) * ssm_a[i]
 *   S <- exp(g) S;  m = S^T k;  S <- S + k (beta (v - m))^T;  o = S^T q
 * for every value head i with q, k of qk head i / (h_v/h_k), taken from h as
 * produced by gdn_conv_silu_norm (q already carries its 1/sqrt(s); with the
 * geometry's scale_after_readout it does not, and o is multiplied by 1/sqrt(s)).
 * slots, n_tok  as above; tokens t >= n_tok[b] leave the state alone and write o = 0
 * h        [B][T][C];  alpha, beta_logit [B][T][h_v];  dt, ssm_a [h_v]
 * o        [B][T][h_v][s]   output
 * The state of each listed slot is read once and written once per call. */
int gdn_decode_step(gdn_pool* p, const int32_t* slots, const int32_t* n_tok, int32_t B, int32_t T,
                    const float* h, const float* alpha, const float* beta_logit, const float* dt,
                    const float* ssm_a, float* o, void* stream);

/* gdn_decode_step with step 7 (the gated RMSNorm below) fused into its epilogue, as
 * the pages' engine fuses its step and output norm (`fused_gdn_step_norm`, step 7 of
 * gdn_layer).  Same arguments as gdn_decode_step plus
 * z       [B][T][h_v*s]   gate input;  norm_w [s];  eps (>= 0)
 * y       [B][T][h_v*s]   output: rms_norm(o) * norm_w * sigmoid(z)  (z * sigmoid(z)
 *                         with the geometry's gate_silu)
 * o       [B][T][h_v][s]  optional: NULL skips writing o (saves its HBM traffic)
 * y and o may not overlap each other, h, z or the pool. */
int gdn_decode_step_norm(gdn_pool* p, const int32_t* slots, const int32_t* n_tok, int32_t B,
                         int32_t T, const float* h, const float* alpha, const float* beta_logit,
                         const float* dt, const float* ssm_a, const float* z, const float* norm_w,
                         float eps, float* o, float* y, void* stream);

/* One decode token of the whole mixer (steps 3-7 of gdn_layer) in a single launch:
 * gdn_conv_silu_norm, then gdn_decode_step_norm, for B sequences x 1 token, with
 * identical results (bit for bit).  One workgroup per (sequence, qk head) owns the
 * conv channels of q, k and the value heads that share them, so h never goes
 * through HBM unless asked for.
 * slots   int32 [B] (NULL: slot b for sequence b)
 * qkv     [B][C];  conv_w [C][d_conv];  alpha, beta_logit [B][h_v];  dt, ssm_a [h_v]
 * z       [B][h_v*s];  norm_w [s];  eps (>= 0, used by both norms)
 * y       [B][h_v*s]   output (NULL allowed when ys is given)
 * h       [B][C]       optional: NULL skips writing the conv/SiLU/L2 output
 * ys      optional: y split for the projection after the mixer, in the layout and with
 *                      the bits of gdn_split_bf16(y, B, h_v*s) (gdn_split_bf16_bytes(B,
 *                      h_v*s) bytes, 16-byte aligned), so that pass is not needed; rows
 *                      past B in its last 32-row tile are left as they are (the product
 *                      only reads them into rows it does not store)
 * The outputs may not overlap each other, qkv, z or the pool.
 * h_v/h_k must be at most 14 (GDN_ERR_UNSUPPORTED otherwise). */
int gdn_decode_fused(gdn_pool* p, const int32_t* slots, int32_t B, const float* qkv,
                     const float* conv_w, const float* alpha, const float* beta_logit,
                     const float* dt, const float* ssm_a, const float* z, const float* norm_w,
                     float eps, float* y, float* h, uint16_t* ys, void* stream);

/* ---------------------------------------------------------------- speculative window
 * The pages' second GDN workload: a verify window runs T drafted tokens from the
 * UNTOUCHED state and conv history (outputs only), and a commit then advances each
 * sequence by the n_keep tokens it accepted (verify.cpp: the GDN branch of the window,
 * and capture_commit's gdn_conv_commit + replay).  Window then commit equals decoding
 * the n_keep tokens directly, bit for bit. */

/* gdn_conv_silu_norm + gdn_decode_step_norm over the window, persisting nothing:
 * h [B][T][C] (keep it for the commit) and y [B][T][h_v*s] are written; the pool is
 * read only.  n_tok as in gdn_decode_step (NULL: all T). */
int gdn_verify_window(gdn_pool* p, const int32_t* slots, const int32_t* n_tok, int32_t B, int32_t T,
                      const float* qkv, const float* conv_w, const float* alpha,
                      const float* beta_logit, const float* dt, const float* ssm_a, const float* z,
                      const float* norm_w, float eps, float* h, float* y, void* stream);

/* Commit the first n_keep[b] tokens of a window (n_keep int32 [B] in [0, T], NULL = T):
 * the conv history advances by those tokens' raw qkv rows, and the recurrence replays
 * them from the window's h, writing the state.  Nothing else is written.  qkv, h,
 * alpha and beta_logit are the window's arrays. */
int gdn_commit(gdn_pool* p, const int32_t* slots, const int32_t* n_keep, int32_t B, int32_t T,
               const float* qkv, const float* h, const float* alpha, const float* beta_logit,
               const float* dt, const float* ssm_a, void* stream);

/* One speculative round: gdn_commit of the previous window (n_keep [B] of its T0
 * tokens, its qkv0, h0, alpha0, beta_logit0) followed by gdn_verify_window of the next
 * (T1 tokens, n_tok, qkv1, alpha1, beta_logit1, z1 -> h1, y1), with the same slots.
 * The results (state, conv history, h1, y1, flags) equal those two calls bit for bit;
 * each state tile is read once instead of twice (two launches: the conv of the
 * window after the history advance, then the replay, the tile store and the window
 * from the committed tile in registers).  Besides the two calls' own checks, h1 and y1
 * may not overlap qkv0, h0, alpha0 or beta_logit0 (GDN_ERR_ARG).  B = 0 is a no-op. */
int gdn_commit_window(gdn_pool* p, const int32_t* slots, int32_t B, const int32_t* n_keep, int32_t T0,
                      const float* qkv0, const float* h0, const float* alpha0, const float* beta_logit0,
                      const int32_t* n_tok, int32_t T1, const float* qkv1, const float* conv_w,
                      const float* alpha1, const float* beta_logit1, const float* dt, const float* ssm_a,
                      const float* z1, const float* norm_w, float eps, float* h1, float* y1, void* stream);

/* Step 7 of gdn_layer: per row of s values,
 *   y = o / sqrt(mean(o^2) + eps) * w * sigmoid(z)      (gate_silu = 0)
 *   y = o / sqrt(mean(o^2) + eps) * w * z * sigmoid(z)  (gate_silu = 1)
 * o, z, y [rows][s] (rows = B*T*h_v); w [s], shared by all rows.  s must be 128.
 * y may alias o. */
int gdn_gated_rmsnorm(const float* o, const float* z, const float* w, float eps, int64_t rows,
                      int32_t s, int32_t gate_silu, float* y, void* stream);

/* ---------------------------------------------------------------- the step before the mixer
 * The alpha / beta projections of step 5 of gdn_layer (bf16 weights; the native
 * path there reads fp32 activations): for every row r of x (one token),
 *   alpha[r][i]      = sum_e w_alpha[i][e] * x[r][e]
 *   beta_logit[r][i] = sum_e w_beta[i][e]  * x[r][e]
 * x [rows][n_embd] fp32 (16-byte aligned, n_embd a multiple of 4);
 * w_alpha, w_beta [h_v][n_embd] bf16 bit patterns (8-byte aligned);
 * alpha, beta_logit [rows][h_v] fp32 outputs, laid out as gdn_decode_step's inputs
 * ([B][T][h_v] when the rows are the B x T tokens).  The sigmoid / softplus that
 * follow them run inside the recurrence kernels.  rows = 0 is a no-op. */
int gdn_ab_project(const float* x, const uint16_t* w_alpha, const uint16_t* w_beta, int64_t rows,
                   int32_t n_embd, int32_t h_v, float* alpha, float* beta_logit, void* stream);

/* ---------------------------------------------------------------- the dense projections
 * qkv = wqkv x and z = attn_gate x before the mixer, out = ssm_out y after it (steps
 * 2, 7 and 8 of gdn_layer), as products with bf16 weights and fp32 activations:
 *   out[r][j] = sum_e w[j][e] * x[r][e]      x [rows][k], w [n][k]
 * Both operands are handed to the matrix cores in a tiled layout of their own:
 *   gdn_pack_bf16   rearranges a weight matrix once (when the weights are loaded);
 *   gdn_split_bf16  writes each fp32 activation as two bf16 values hi = bf16(x),
 *                   lo = bf16(x - hi) (round to nearest even; hi + lo equals x to
 *                   within 2^-16 |x| while lo is a normal number), in the same tiling;
 *                   one split serves every projection of the same activations (qkv
 *                   and z share theirs);
 *   gdn_project_bf16 multiplies them, summing in fp32.
 * The tile is 32 rows x 64 k: rows are padded to a multiple of 32 and k to a
 * multiple of 64 with zeros.  For step s (0..3) of a tile and lane l = i + 32h
 * (i < 32, h < 2), the 8 values of element [32R + i][64C + 32h + 8s + j], j = 0..7,
 * form a 16-byte fragment.  Packed weights: tile (R, C) of R-major order holds the
 * fragments (s, l) at index s*64 + l (4 KiB per tile).  Split activations: tile
 * (R, C) holds the hi fragment (s, l) at index (2s)*64 + l and the lo fragment at
 * (2s + 1)*64 + l (8 KiB per tile).  k must be a positive multiple of 8, at most 2^24. */

/* Bytes of the split activations for [rows][k]: ceil(rows/32)*32 * ceil(k/64)*64 * 4,
 * or -1 for a negative rows or a k that is not a positive multiple of 8. */
int64_t gdn_split_bf16_bytes(int64_t rows, int32_t k);

/* Bytes of the packed weights for [n][k]: ceil(n/32)*32 * ceil(k/64)*64 * 2, or -1. */
int64_t gdn_pack_bf16_bytes(int32_t n, int32_t k);

/* x [rows][k] fp32, 16-byte aligned -> xs (gdn_split_bf16_bytes(rows, k) bytes,
 * 16-byte aligned, not overlapping x).  rows = 0 is a no-op.  Non-finite x gives hi =
 * the value, lo = 0. */
int gdn_split_bf16(const float* x, int64_t rows, int32_t k, uint16_t* xs, void* stream);

/* w [n][k] bf16 bit patterns, 16-byte aligned -> wp (gdn_pack_bf16_bytes(n, k)
 * bytes, 16-byte aligned, not overlapping w).  n >= 1. */
int gdn_pack_bf16(const uint16_t* w, int32_t n, int32_t k, uint16_t* wp, void* stream);

/* Device workspace, in bytes, that gdn_project_bf16 / gdn_project2_bf16 need for a
 * product of rows x k x n (n = n1 + n2 for the two-output form), or -1 for a negative
 * rows or a bad k or n.  It is 0 unless the launch picked for the shape splits a long
 * k range over several workgroups per output tile (at most 64 KiB per 32-row x
 * 128-column share of the output); then the partial sums go through the workspace
 * and a second kernel adds them in a fixed order. */
int64_t gdn_project_workspace_bytes(int64_t rows, int32_t k, int32_t n);

/* xs from gdn_split_bf16 for [rows][k]; wp from gdn_pack_bf16 for [n][k]; out
 * [rows][n] fp32, 4-byte aligned, overlapping neither input.  workspace: device
 * memory of workspace_bytes >= gdn_project_workspace_bytes(rows, k, n) bytes,
 * 16-byte aligned, overlapping no other argument (NULL with 0 when that is 0);
 * its contents are scratch before and after the call, and calls that share one
 * must be ordered (one stream).  A smaller workspace is an argument error.
 * rows = 0 is a no-op.  For one (rows, k, n) the result is the same on every call
 * (a fixed summation order). */
int gdn_project_bf16(const uint16_t* xs, const uint16_t* wp, int64_t rows, int32_t k, int32_t n, float* out,
                     void* workspace, int64_t workspace_bytes, void* stream);

/* Two projections of the same activations in one launch (qkv and z both read the
 * layer input): wp is gdn_pack_bf16 of the (n1 + n2) x k matrix whose first n1 rows
 * are the first weight matrix and whose last n2 rows are the second; columns j < n1
 * of the product go to out1 [rows][n1], the others to out2 [rows][n2] (4-byte
 * aligned, overlapping neither each other nor an input).  n1, n2 >= 1.  The workspace
 * is that of gdn_project_bf16 for n = n1 + n2.  Each output equals gdn_project_bf16
 * of the concatenated weights, column for column. */
int gdn_project2_bf16(const uint16_t* xs, const uint16_t* wp, int64_t rows, int32_t k, int32_t n1, float* out1,
                      int32_t n2, float* out2, void* workspace, int64_t workspace_bytes, void* stream);

/* Up to four projections of the same activations in one launch (qkv, z and the alpha /
 * beta logits all read the layer input, so one launch serves the four): wp is
 * gdn_pack_bf16 of the matrices stacked row-wise, cols[o] >= 1 rows each (host
 * array of n_out entries, 1 <= n_out <= 4); the product's columns go, in that order,
 * to outs[o] [rows][cols[o]] (host array of n_out device pointers, 4-byte aligned,
 * overlapping neither each other nor an input).  The workspace is that of
 * gdn_project_bf16 for n = the sum of cols.  Each output equals, column for column,
 * the matching columns of gdn_project_bf16 of the stacked weights. */
int gdn_project_multi_bf16(const uint16_t* xs, const uint16_t* wp, int64_t rows, int32_t k, int32_t n_out,
                           const int32_t* cols, float* const* outs, void* workspace, int64_t workspace_bytes,
                           void* stream);

/* Bytes of the library's own scratch buffer that gdn_project_bf16_noalloc uses, on
 * each GPU the library runs on. */
#define GDN_PROJECT_SCRATCH_BYTES (4u << 20)

/* gdn_project_bf16 for callers that cannot allocate device memory or hand in a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same operands, result and errors as gdn_project_bf16 (bit for bit the
 * same output for the same shape), except that a launch which splits its k range over
 * workgroups keeps its partial blocks in a scratch buffer of GDN_PROJECT_SCRATCH_BYTES
 * that the library owns, one per GPU, held from the first call on that GPU until the
 * process ends.  A shape whose gdn_project_workspace_bytes exceeds it is GDN_ERR_ARG
 * (at the pages' sizes the out projection, 6144 -> 2560, needs 0.94 MiB at up to 32
 * rows and none above; the qkv and z projections need none).  The call allocates
 * nothing.  Every call on one GPU shares that GPU's buffer: calls ordered on one
 * stream are safe, calls that may run at the same time on one GPU (other streams, no
 * ordering between them) race.  Each launch writes every partial block before reading
 * it, so the buffer's old contents never matter. */
int gdn_project_bf16_noalloc(const uint16_t* xs, const uint16_t* wp, int64_t rows, int32_t k, int32_t n,
                             float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
