/*
 * hvattn.h -- C ABI of libhvattn: the joint video+text attention hot path of a
 * HunyuanVideo-style diffusion transformer, for AMD Instinct MI355X (gfx950).
 *
 * Sources for what is computed (all on the HunyuanVideo notes page
 * "HunyuanVideo 模型结构与数学原理", note.shouss.top, unless stated):
 *   - token grid: section 4 (Causal 3D VAE latent size, 1x2x2 patch count);
 *   - 3D RoPE:    section 5.5 (R_3D = R_t (+) R_h (+) R_w, channel split
 *                 (16, 56, 56)); the technical-report summary page
 *                 (zhao9797.github.io, "hunyuan-video"), Table 2 paragraph,
 *                 gives the same split;
 *   - QK norm:    section 5.4 (per-head RMSNorm of Q and K), section 5.2
 *                 (separate video / text weights in double-stream blocks);
 *   - attention:  section 5.2 (joint softmax attention over [video; text],
 *                 scale 1/sqrt(128)); section 3.1 (at most 256 text tokens);
 *                 section 5.1 (24 heads x 128);
 *   - backward:   the report summary page's Infra section (training:
 *                 fused attention is the bottleneck);
 *   - ring / varlen: section 9.2 (USP: Ring Attention passes K/V blocks, so
 *                 partial results are merged by log-sum-exp); section 9.1
 *                 (the variable-length FlashAttention call: packed segments).
 *
 * Conventions shared by all calls
 *   - Tensors are bfloat16 bit patterns (hv_bf16) in device memory owned by
 *     the caller, laid out [batch][seq][head][channel] with the channel dim
 *     contiguous, head stride 128 elements, token stride layout->stride_l
 *     and batch stride layout->stride_b (both in elements).  The sequence
 *     holds the n_video video tokens first, then the text tokens.
 *   - Device pointers must be 16-byte aligned; strides must be multiples of
 *     8 elements, stride_l >= heads*head_dim, stride_b >= seq_len*stride_l.
 *   - heads must be 24 and head_dim 128, batch <= HV_MAX_BATCH,
 *     seq_len <= HV_MAX_SEQ and stride_l <= HV_MAX_TOKEN_STRIDE
 *     (HV_ERR_UNSUPPORTED otherwise); negative sizes
 *     are HV_ERR_INVALID_ARG.  A call with batch == 0 or seq_len == 0 has
 *     nothing to do and returns HV_OK without launching (so does RoPE with
 *     n_video == 0).
 *   - Every argument is validated on the host before any HIP call; an
 *     invalid call returns a negative status and touches no memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and the call returns without synchronising.  Faults inside a kernel
 *     surface at the caller's next synchronisation.
 *   - The library allocates no memory; calls are thread-safe.  Scratch
 *     memory comes in as workspace arguments (the forward calls' packed V,
 *     the backward's D), except in hv_joint_attention_bwd_noalloc, whose
 *     scratch is a static device array (the only state the library keeps:
 *     that array and its per-device addresses).  Calls that write
 *     overlapping memory on different streams race, as with any kernel.
 *   - No C++ exception crosses this interface.
 */
#ifndef HVATTN_H
#define HVATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HV_HEADS 24
#define HV_HEAD_DIM 128
#define HV_MAX_BATCH 64
#define HV_MAX_SEQ (1 << 24)
#define HV_MAX_TOKEN_STRIDE (1 << 24) /* elements between consecutive tokens */
#define HV_MAX_SEGMENTS 64    /* packed segments per varlen call */
#define HV_MAX_MERGE_PARTS 16 /* partial results per merge call */
/* device scratch of hv_joint_attention_bwd_noalloc: 32 MiB + 256 bytes per GPU */
#define HV_NOALLOC_BWD_SCRATCH_BYTES ((32 << 20) + 256)

typedef uint16_t hv_bf16; /* raw bfloat16 bits */

enum hv_status {
  HV_OK = 0,
  HV_ERR_INVALID_ARG = -1, /* NULL, bad size, range, alignment or overlap */
  HV_ERR_UNSUPPORTED = -2, /* heads != 24, head_dim != 128, batch/seq too large */
  HV_ERR_HIP = -3          /* a HIP launch failed (e.g. no device) */
};

/* Latent and token grid of a clip (notes page, section 4).
 *   t_lat = floor((frames-1)/4) + 1, h_lat = height/8, w_lat = width/8
 *   gt = t_lat, gh = h_lat/2, gw = w_lat/2   (1x2x2 patches)
 *   n_video = gt*gh*gw                        (video tokens) */
typedef struct hv_grid {
  int32_t frames, height, width;
  int32_t t_lat, h_lat, w_lat;
  int32_t gt, gh, gw;
  int32_t reserved; /* 0 */
  int64_t n_video;
} hv_grid;

typedef struct hv_layout {
  int32_t batch;    /* B */
  int32_t seq_len;  /* L = n_video + text capacity */
  int32_t heads;    /* must be HV_HEADS */
  int32_t head_dim; /* must be HV_HEAD_DIM */
  int64_t stride_b; /* elements between batch entries */
  int64_t stride_l; /* elements between consecutive tokens */
} hv_layout;

/* hv_token_grid: fill *out for an F x H x W clip (host only, no GPU use).
 * Notes page section 4 gives the formula for F = 4k+1; section 8 states that
 * sizes must be multiples of 16 and frames 4k+1 to pass the input check.
 * Errors: HV_ERR_INVALID_ARG if out is NULL, any size <= 0, frames != 4k+1,
 * or height/width not multiples of 16.  *out is untouched on error. */
int hv_token_grid(int32_t frames, int32_t height, int32_t width, hv_grid* out);

/* hv_rope3d_apply: rotate the video rows of q and k in place (notes page
 * section 5.5).  For every batch entry b, video token n < grid->n_video with
 * patch coordinates t = n / (gh*gw), h = (n / gw) % gh, w = n % gw, and every
 * head, the channel pair (o + 2j, o + 2j + 1) of axis block
 * (o, d) in {(0,16) for t, (16,56) for h, (72,56) for w} is rotated by
 * angle pos * theta^(-2j/d):  x0' = x0 cos - x1 sin,  x1' = x0 sin + x1 cos.
 * Rotation math is fp32, results are rounded to bf16 (nearest even).
 * Text rows (n >= n_video) and V are never touched.
 *   q, k    device pointers, layout *layout; may not overlap each other
 *   grid    from hv_token_grid; layout->seq_len >= grid->n_video
 *   theta   rotary base, finite and > 0 (10000 in the benchmark workloads)
 * Errors: HV_ERR_INVALID_ARG (NULL, inconsistent grid, theta <= 0,
 * alignment, overlap), HV_ERR_UNSUPPORTED, HV_ERR_HIP. */
int hv_rope3d_apply(hv_bf16* q, hv_bf16* k, const hv_layout* layout,
                    const hv_grid* grid, float theta, void* stream);

/* hv_qk_norm_rope3d_apply: the QK-norm prologue of the attention, in place:
 * per-head RMSNorm of every row of q and k (notes page section 5.4:
 * y = gamma * x / sqrt(mean_j x_j^2 + eps) over the 128 channels of a head),
 * then the rotation of hv_rope3d_apply on the video rows (section 5.5).
 * Video rows (n < grid->n_video) use gamma_q / gamma_k; text rows use
 * gamma_q_text / gamma_k_text (section 5.2: the double-stream blocks keep
 * separate weights per stream); a NULL text weight means the video weight
 * (the shared weights of the single-stream blocks, section 5.3).  All
 * seq_len rows are normalised, padded text rows included.  Math is fp32;
 * each result is rounded to bf16 (nearest even) once, after the rotation.
 *   q, k      device pointers, layout *layout; may not overlap each other
 *   grid      from hv_token_grid; layout->seq_len >= grid->n_video
 *   theta     rotary base, finite and > 0
 *   gamma_*   device pointers to 128 bf16 weights, 16-byte aligned, outside
 *             q and k (they may alias one another)
 *   eps       finite and >= 0 (with eps == 0 an all-zero head gives NaN, as
 *             the formula does)
 * Errors: HV_ERR_INVALID_ARG (NULL q/k/gamma_q/gamma_k, inconsistent grid,
 * theta <= 0, eps < 0 or not finite, alignment, overlap), HV_ERR_UNSUPPORTED,
 * HV_ERR_HIP. */
int hv_qk_norm_rope3d_apply(hv_bf16* q, hv_bf16* k, const hv_layout* layout,
                            const hv_grid* grid, float theta,
                            const hv_bf16* gamma_q, const hv_bf16* gamma_k,
                            const hv_bf16* gamma_q_text, const hv_bf16* gamma_k_text,
                            float eps, void* stream);

/* Workspace of the attention forward calls (hv_joint_attention_fwd,
 * hv_attention_fwd_lse, hv_joint_attention_varlen_fwd).  With a workspace the
 * call first rewrites V, tile by tile, channel-major into it (one pass over V,
 * 2 x |V| bytes of HBM traffic) and the attention then reads every P V operand
 * with a plain 16-byte LDS read; with workspace == NULL it gathers them from V
 * in place with the transposing LDS read.  The workspace also holds a work
 * counter through which the attention's workgroups (one per CU) share the
 * query blocks, so CUs of faster-clocked XCDs take more of them; without it
 * every XCD gets a fixed share.  The NULL path is about 3 % slower at the
 * largest sizes; both give bitwise identical results.  A call
 * needs, over its segments with query rows (a batch entry of the padded
 * forms, a packed clip), sum ceil(keys / 64) * 64 * 24 * 128 * 2 bytes plus
 * 256 bytes (none when no segment has query rows).  A call whose query
 * blocks (24 heads x ceil(rows / 256) per segment) all fit in one round of
 * workgroups (at most one per compute unit) reads V in place even with a
 * workspace: there is nothing to share out, and packing would cost one more
 * launch and pass over V; the results are the same bit for bit.  When even
 * blocks of 128 query rows all fit in one round, those are used (four waves
 * per workgroup instead of eight, each key tile then takes about half the
 * time), again with bitwise the same results.
 * hv_attention_workspace_bytes(n_keys, n_segments) returns an upper bound
 * for n_keys keys in all over n_segments segments:
 *   hv_joint_attention_fwd         n_keys = batch * seq_len, n_segments = batch
 *   hv_attention_fwd_lse           n_keys = batch * kv seq_len, n_segments = batch
 *   hv_joint_attention_varlen_fwd  n_keys = T, n_segments as passed
 * The workspace is device memory, 16-byte aligned, disjoint from every other
 * argument, overwritten by the call and free again when the call's work on
 * its stream has finished.  Calls in flight together need separate
 * workspaces.  Returns 0 for negative arguments. */
int64_t hv_attention_workspace_bytes(int64_t n_keys, int32_t n_segments);

/* hv_joint_attention_fwd: out = softmax(scale * Q K^T) V per (batch, head)
 * over the joint [video; text] sequence (notes page section 5.2).
 * Keys at positions >= n_video + text_valid_len[b] are padding and take no
 * part in the softmax; every one of the seq_len query rows (padded text rows
 * included) attends to the same valid keys.  bf16 inputs, fp32 accumulation
 * and softmax, output rounded to bf16 (nearest even).
 *   q, k, v         device pointers, layout *layout (q, k already rotated)
 *   text_valid_len  HOST array of layout->batch int32 values in
 *                   [0, seq_len - n_video]; NULL means all text is valid
 *   out             device pointer, same layout; must not overlap q, k, v
 *   n_video         video tokens at the head of the sequence, 0..seq_len
 *   softmax_scale   > 0 to override; <= 0 or NaN selects 1/sqrt(128)
 *   workspace, workspace_bytes  packed-V workspace (see above) or NULL, 0;
 *                   too small a workspace is HV_ERR_INVALID_ARG
 * n_video + text_valid_len[b] must be >= 1 for every b.  batch == 0 or
 * seq_len == 0 is an empty call and returns HV_OK without launching.
 * Errors: HV_ERR_INVALID_ARG, HV_ERR_UNSUPPORTED, HV_ERR_HIP. */
int hv_joint_attention_fwd(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
                           const int32_t* text_valid_len, hv_bf16* out,
                           const hv_layout* layout, int64_t n_video,
                           float softmax_scale, void* workspace,
                           int64_t workspace_bytes, void* stream);

/* hv_attention_fwd_lse: attention of query rows against a separate K/V
 * block, with the log-sum-exp of every row, for sequence-parallel (ring)
 * attention: notes page section 9.2 (USP; Ring Attention keeps each rank's
 * query rows and passes K/V blocks around the ring).  Per batch entry b and
 * head h, query row i attends to the first kv_valid_len[b] rows of k, v:
 *   lse[b][h][i] = log sum_j exp(scale * q_i . k_j)       (natural log)
 *   out_i        = sum_j exp(scale * q_i . k_j - lse) v_j
 * Results over disjoint K/V blocks combine exactly with hv_attention_merge.
 * bf16 inputs, fp32 accumulation, out rounded to bf16, lse fp32.
 *   q, out        device pointers, layout *q_layout (out must not overlap
 *                 q, k, v)
 *   k, v          device pointers, layout *kv_layout; batch must equal
 *                 q_layout->batch, seq_len (keys) may differ from q's
 *   kv_valid_len  HOST array [batch] in [1, kv seq_len]; NULL = all keys
 *   lse           device fp32 [batch][24][q seq_len], 4-byte aligned,
 *                 disjoint from the tensors; NULL to skip
 *   softmax_scale, workspace, workspace_bytes  as in hv_joint_attention_fwd
 * Errors: HV_ERR_INVALID_ARG (NULL, batch mismatch, valid length out of
 * range, alignment, overlap, workspace too small), HV_ERR_UNSUPPORTED,
 * HV_ERR_HIP. */
int hv_attention_fwd_lse(const hv_bf16* q, const hv_layout* q_layout,
                         const hv_bf16* k, const hv_bf16* v, const hv_layout* kv_layout,
                         const int32_t* kv_valid_len, hv_bf16* out, float* lse,
                         float softmax_scale, void* workspace, int64_t workspace_bytes,
                         void* stream);

/* hv_attention_merge: combine n_parts attention results computed over
 * disjoint key blocks (e.g. by hv_attention_fwd_lse on each block of a ring)
 * into the result over their union (notes page section 9.2):
 *   lse = log sum_i exp(lse_i),   out = sum_i exp(lse_i - lse) outs[i]
 * per (batch, row, head).  fp32 arithmetic, out rounded to bf16 once.
 *   outs     HOST array of n_parts device pointers, each with *layout
 *   lses     HOST array of n_parts device pointers, fp32 [batch][24][seq_len]
 *   n_parts  1 .. HV_MAX_MERGE_PARTS
 *   out      device pointer, *layout; must not overlap any input
 *   lse_out  device fp32 [batch][24][seq_len] or NULL; must not overlap any
 *            input or out
 * A row whose lse_i are all -inf has no defined result (NaN).
 * Errors: HV_ERR_INVALID_ARG (NULL, n_parts out of range, alignment,
 * overlap), HV_ERR_UNSUPPORTED, HV_ERR_HIP. */
int hv_attention_merge(const hv_bf16* const* outs, const float* const* lses,
                       int32_t n_parts, hv_bf16* out, float* lse_out,
                       const hv_layout* layout, void* stream);

/* hv_joint_attention_varlen_fwd: attention over packed segments, the
 * variable-length form of FlashAttention that the model calls (notes page
 * section 9.1).  q, k, v, out hold T = layout->seq_len packed rows
 * (layout->batch must be 1).  Segment s owns query rows
 * [cu_seqlens_q[s], cu_seqlens_q[s+1]) and key rows
 * [cu_seqlens_k[s], cu_seqlens_k[s+1]); its queries attend to its keys only.
 * Several clips, each [video | valid text], pack back to back; the padded
 * layout of hv_joint_attention_fwd is also expressible with each padded
 * text tail as a segment of its own.  Output rows outside every segment
 * are not written.
 *   cu_seqlens_q/k  HOST arrays [n_segments + 1], non-decreasing, >= 0,
 *                   last entry <= T; a segment with query rows needs >= 1 key
 *   n_segments      1 .. HV_MAX_SEGMENTS
 *   lse             device fp32 [24][T] (natural-log log-sum-exp per row) or
 *                   NULL; rows outside every segment are not written
 *   workspace, workspace_bytes  as in hv_joint_attention_fwd
 * Errors: HV_ERR_INVALID_ARG (NULL, batch != 1, bad offsets, alignment,
 * overlap, workspace too small), HV_ERR_UNSUPPORTED, HV_ERR_HIP. */
int hv_joint_attention_varlen_fwd(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                  int32_t n_segments, hv_bf16* out, float* lse,
                                  const hv_layout* layout, float softmax_scale,
                                  void* workspace, int64_t workspace_bytes, void* stream);

/* hv_joint_attention_bwd: gradients of hv_joint_attention_fwd by the chain
 * rule through the softmax (the training-side attention cost the report
 * summary page names, "FusedAttention" in its Infra section).  Per (batch,
 * head), with P = softmax(scale * Q K^T) over the valid keys:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale * dS K,  dK = scale * dS^T Q.
 * Padded keys (>= n_video + text_valid_len[b]) get dk = dv = 0; every query
 * row contributes.  P is recomputed from lse.  bf16 in and out, fp32
 * accumulation; P and dS are rounded to bf16 as MFMA operands.
 *   q, k, v, out, dout  device pointers, layout *layout; out is the forward's
 *                       output and dout the gradient with respect to it
 *   lse                 device fp32 [batch][24][seq_len]: the natural-log
 *                       log-sum-exp of the forward, as hv_attention_fwd_lse
 *                       writes it for the same q, k, v and valid keys
 *   text_valid_len, n_video, softmax_scale  as in hv_joint_attention_fwd
 *   dq, dk, dv          device pointers, layout *layout; must not overlap any
 *                       input or each other
 *   delta               device workspace of 2 * batch * 24 * seq_len floats
 *                       plus 256 bytes (caller-owned, 4-byte aligned, disjoint
 *                       from all other arguments): it receives
 *                       -rowsum(dO * O), then -lse / softmax_scale, each as
 *                       fp32 [batch][24][seq_len] (the starting accumulators
 *                       of the dP and S products); the last 256 bytes hold
 *                       the work counters through which the two gradient
 *                       kernels' persistent workgroups (one per CU) take their
 *                       blocks.  Its contents need no initialisation; calls
 *                       that share one race.
 * Errors: HV_ERR_INVALID_ARG (NULL, valid length out of range, alignment,
 * overlap), HV_ERR_UNSUPPORTED, HV_ERR_HIP. */
int hv_joint_attention_bwd(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
                           const hv_bf16* out, const hv_bf16* dout, const float* lse,
                           const int32_t* text_valid_len, int64_t n_video,
                           hv_bf16* dq, hv_bf16* dk, hv_bf16* dv, float* delta,
                           const hv_layout* layout, float softmax_scale, void* stream);

/* hv_joint_attention_bwd_noalloc: hv_joint_attention_bwd for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * training or serving loops, harnesses that forbid hipMalloc): the same
 * computation, arguments and results, but the delta workspace lives in a
 * static device array of the library, HV_NOALLOC_BWD_SCRATCH_BYTES on every
 * GPU it runs on (taken when the library's code is loaded onto the GPU and
 * held until the process ends).  The call allocates nothing; its first call
 * on a device looks up that device's copy (hipGetSymbolAddress, with the
 * device current) and keeps the address.
 *   arguments   as hv_joint_attention_bwd, without delta; the current HIP
 *               device must be the one that holds the tensors and runs
 *               `stream`
 *   size limit  2 * batch * 24 * seq_len * 4 + 256 bytes must fit the
 *               scratch, i.e. batch * seq_len <= 174762 (720x1280x129 at
 *               batch 1 is 119056); larger calls return HV_ERR_UNSUPPORTED
 *               without launching
 * Every call on one GPU uses that GPU's one scratch array, which keeps what
 * the last call left there (the kernels rewrite everything they read first):
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and must be ordered by the caller.
 * Errors: as hv_joint_attention_bwd; HV_ERR_UNSUPPORTED also for calls over
 * the size limit or a device index >= 64; HV_ERR_HIP when the scratch
 * address cannot be found. */
int hv_joint_attention_bwd_noalloc(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
                                   const hv_bf16* out, const hv_bf16* dout, const float* lse,
                                   const int32_t* text_valid_len, int64_t n_video,
                                   hv_bf16* dq, hv_bf16* dk, hv_bf16* dv,
                                   const hv_layout* layout, float softmax_scale, void* stream);

/* hv_joint_attention_varlen_bwd: gradients of hv_joint_attention_varlen_fwd
 * (packed segments; notes page section 9.1 for the packed form, the report
 * summary page's Infra section for the training-side cost).  Each segment
 * is an independent attention, so its gradients are those of
 * hv_joint_attention_bwd on that segment with every key valid.  Rows
 * outside every segment are not written in dq; key rows outside every
 * segment are not written in dk, dv; key rows of a segment whose queries
 * are empty get zero dk, dv.
 *   q, k, v, out, dout, dq, dk, dv  T = layout->seq_len packed rows
 *                       (layout->batch must be 1); out is the forward's
 *                       output, dout the gradient with respect to it
 *   lse                 device fp32 [24][T], the forward's log-sum-exp as
 *                       hv_joint_attention_varlen_fwd writes it
 *   cu_seqlens_q/k, n_segments, softmax_scale  as in the forward
 *   delta               device workspace of 2 * 24 * T floats plus 256
 *                       bytes, as in hv_joint_attention_bwd
 * Errors: HV_ERR_INVALID_ARG (NULL, batch != 1, bad offsets, alignment,
 * overlap), HV_ERR_UNSUPPORTED, HV_ERR_HIP. */
int hv_joint_attention_varlen_bwd(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
                                  const hv_bf16* out, const hv_bf16* dout, const float* lse,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                  int32_t n_segments, hv_bf16* dq, hv_bf16* dk, hv_bf16* dv,
                                  float* delta, const hv_layout* layout, float softmax_scale,
                                  void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* hv_status_string(int status);

/* Library ABI version (major*10000 + minor*100 + patch). */
int hv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HVATTN_H */
