/*
 * mmdit.h - C ABI of the packed native-resolution joint-attention core
 * (the attention part of an NR-MMDiT block) for AMD Instinct MI355X (gfx950).
 *
 * What the library computes, per the Mage-Flow pages:
 *   - packing: every sample's text tokens and flattened image-latent grid are
 *     laid back to back in one contiguous batch with per-sample cumulative
 *     offsets, under a fixed token budget, with no padding
 *     (findtube.ai transcript "Mage-Flow: Efficient Native-Resolution Image
 *     Generation and Editing" at [00:03:16] and [00:04:03]; picx.dev summary
 *     "Mage-Flow: An Efficient Native-Resolution Foundation Model for Image
 *     Generation and Editing", section "Native-Resolution MMDiT (NR-MMDiT)");
 *   - modality-specific normalisation before joint attention (same picx.dev
 *     section, first bullet; transcript at [00:00:00]): RMSNorm of Q and K
 *     over each head's d elements, with one gain vector per (Q or K, text or
 *     image);
 *   - per-sample 2D rotary embedding of image tokens from their own (row, col)
 *     (transcript at [00:03:16]; aiany.app entry, "Key Capabilities");
 *   - joint text+image self-attention confined to each sample (variable-length
 *     attention over the cumulative offsets; picx.dev, same section), and its
 *     backward for training;
 *   - around it: packed classifier-free guidance (mmdit_cfg_pack_desc),
 *     editing packs with a frame axis of a 3D RoPE (mmdit_pack_plan_edit) and
 *     the adaptive-LayerNorm modulation with the fused gated residual
 *     (mmdit_adaln_fwd / mmdit_adaln_bwd), each documented at its
 *     declaration.
 *
 * Conventions fixed by this library where the pages are silent:
 *   - token order inside a sample: text tokens, then the latent grid row-major;
 *   - RMSNorm: rho = (mean_k x_k^2 + eps)^(-1/2), y = x * rho * g; then RoPE;
 *   - RoPE: dims [0, d/2) turn by the row index, dims [d/2, d) by the column
 *     index (0-based); inside each half, adjacent pairs (2j, 2j+1) turn by
 *     pos * theta^(-4j/d); text tokens are not rotated;
 *   - editing packs (mmdit_pack_plan_edit) use a third, frame axis: the first
 *     d/8 pairs turn by the frame index (0 for target tokens, 1 for source
 *     tokens), the next 3d/16 pairs by the row and the last 3d/16 by the
 *     column; pair j of a section of n pairs turns by pos * theta^(-j/n),
 *     which for n = d/4 is the 2D rule above;
 *   - softmax scale 1/sqrt(d), no causal mask, natural-log lse.
 *
 * Tensor layout: Q, K, V, O and their gradients are [N][H][d] (token-major,
 * then head, then the d elements contiguous). "stride" arguments give the
 * number of ELEMENTS between consecutive tokens (>= H*d, a multiple of 8, at
 * most MMDIT_MAX_ROW_STRIDE), so
 * Q/K/V may be views into a fused [N][3][H][d] projection output. Output
 * tensors are always dense [N][H][d]. lse and D are [H][N] fp32.
 *
 * Ownership and threading: the caller owns every buffer (host descriptor
 * arrays, the host plan blob, its device copy, tensors, workspace). The
 * library never allocates or frees device memory, and only
 * mmdit_device_faults synchronises: mmdit_attn_fwd / mmdit_attn_bwd only
 * enqueue kernels on the caller's HIP stream and return; buffers must stay
 * alive until the stream passes them.
 * All entry points are reentrant. Errors: every argument is validated on the
 * host before anything is launched; on a non-OK return nothing was enqueued
 * and no output was touched, and mmdit_last_error() (thread-local) says why.
 * The stream of a launching call (NULL = the default stream) must belong to
 * the current device. On the device, every kernel first checks that the blob
 * it was given is the plan's (its header fingerprint); a kernel given another
 * pack's blob writes nothing and records MMDIT_DEVICE_FAULT_STALE_BLOB, which
 * mmdit_device_faults reports after the work has run.
 */
#ifndef MMDIT_H
#define MMDIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MMDIT_ABI_VERSION 5

/* Largest accepted token stride, in elements (2^24). */
#define MMDIT_MAX_ROW_STRIDE (1ll << 24)

typedef enum {
  MMDIT_OK = 0,
  MMDIT_ERR_INVALID_ARG = 1,       /* NULL / negative / misaligned / inconsistent argument */
  MMDIT_ERR_UNSUPPORTED = 2,       /* valid but not built: e.g. head_dim not 64 or 128 */
  MMDIT_ERR_BUFFER_TOO_SMALL = 3,  /* host blob or workspace smaller than required */
  MMDIT_ERR_BUDGET = 4,            /* total tokens exceed the descriptor's token budget */
  MMDIT_ERR_HIP = 5                /* a HIP launch failed; see mmdit_last_error(). Test hook: with
                                      MMDIT_FAULT_INJECT=launch in the environment, mmdit_attn_fwd, mmdit_attn_bwd(_noalloc)
                                      and mmdit_adaln_fwd/bwd return it where they would launch, having launched nothing */
} mmdit_status;

typedef enum { MMDIT_F32 = 0, MMDIT_BF16 = 1 } mmdit_dtype;

/* Description of one pack (host memory, read during mmdit_pack_plan only).
 * Sample i holds text_len[i] text tokens followed by a grid_h[i] x grid_w[i]
 * latent grid (both 0 for a text-only sample); every sample has >= 1 token;
 * the pack holds at most 2^29 tokens. */
typedef struct {
  int32_t num_samples;          /* S >= 1 */
  const int32_t *text_len;      /* [S], >= 0 */
  const int32_t *grid_h;        /* [S], >= 0, < 32768 */
  const int32_t *grid_w;        /* [S], >= 0, < 32768; zero iff grid_h is zero */
  int32_t num_heads;            /* H >= 1 */
  int32_t head_dim;             /* d: 64 or 128 */
  int32_t dtype;                /* mmdit_dtype of Q, K, V, O and gradients */
  float rope_theta;             /* > 0, e.g. 10000 */
  float rms_eps;                /* >= 0, e.g. 1e-6 */
  int64_t token_budget;         /* 0 = none; else total tokens must be <= budget */
} mmdit_pack_desc;

/* Plan: plain data filled by mmdit_pack_plan; valid for every fwd/bwd call on
 * a pack with the same descriptor. The blob (host_blob) it describes must be
 * copied by the caller to device memory (16-byte aligned) once, and that copy
 * passed as plan_blob_dev. Blob sections (offsets in bytes, 256-aligned):
 *   cu_seqlens  int32 [S+1]
 *   tok_meta    int32 [N]   bit 31 = image, bits 30..16 = row, bit 15 = frame,
 *                           bits 14..0 = col
 *   fwd_items   int32 [num_fwd_items][4] = {seg_start, seg_end, tile_start, sample}
 *               one per q_tile-row query tile, longest segment first
 *   bwd_items   int32 [num_bwd_items][4], same for kv_tile-row key tiles
 *   fwd_blocks  int32 [num_fwd_blocks][2] = {item, head} per workgroup of the
 *               query-tile kernels, or {-1, -1} (idle). All tiles of one
 *               (sample, head) form a chunk; chunks are dealt round-robin to
 *               the GPU's 8 XCDs in longest-first order so that each sample's
 *               K/V stay in one XCD's L2 (workgroup b runs on XCD b % 8).
 *   bwd_blocks  int32 [num_bwd_blocks][2], the same for the key-tile kernel
 *   mod_chunks  int32 [num_mod_chunks][4] = {row_start, row_end, 2*sample + stream, 0}:
 *               each (sample, stream) token range (stream 0 = text, 1 = image)
 *               cut into pieces of at most mod_chunk_rows rows, ranges in order
 *   mod_ranges  int32 [2S+1]: chunks of range r are [mod_ranges[r], mod_ranges[r+1])
 *   ds_base     int64 [S+1]: first 1 KiB block of sample s's dS area (all heads) in
 *               the backward's dS store; sample s with L = seg_end - seg_start
 *               tokens has ceil(L/32) * 4 * ceil(L/64) blocks per head
 *   rope        fp32  [rope_rows][d/2][2] = {cos, sin}(pos * omega_p) for
 *               each of the d/2 pairs p (the frequency of its section, see
 *               the RoPE conventions above), computed in double precision and
 *               rounded once. rope_frame_pairs = number of frame pairs (0 for
 *               a generation pack, d/8 for an editing pack). */
typedef struct {
  int32_t num_samples, total_tokens, max_seqlen, num_heads, head_dim, dtype;
  int32_t q_tile, kv_tile, num_fwd_items, num_bwd_items, rope_rows, rope_frame_pairs;
  int32_t num_fwd_blocks, num_bwd_blocks;
  float rope_theta, rms_eps;
  uint64_t blob_bytes;
  uint64_t off_cu_seqlens, off_tok_meta, off_fwd_items, off_bwd_items, off_rope;
  uint64_t off_fwd_blocks, off_bwd_blocks;
  uint64_t fwd_workspace_bytes;  /* needed by mmdit_attn_fwd when q_hat/k_hat are NULL */
  uint64_t bwd_workspace_bytes;  /* needed by mmdit_attn_bwd */
  uint64_t off_mod_chunks, off_mod_ranges;
  int32_t num_mod_chunks;        /* adaLN workgroups; mmdit_adaln_bwd needs a workspace of
                                    num_mod_chunks * 3 * model_dim * 4 bytes */
  int32_t mod_chunk_rows;        /* rows per adaLN chunk (32) */
  uint64_t off_ds_base;
  uint64_t bwd_ds_workspace_bytes; /* workspace of the stored-dS backward (see mmdit_attn_bwd);
                                      equals bwd_workspace_bytes where the plan has no such mode
                                      (fp32 plans, samples over 32,768 tokens) */
  uint64_t fingerprint;          /* hash of every field above; checked on each call */
} mmdit_plan;

/* Build the plan of one pack: the per-sample cumulative offsets (cu_seqlens)
 * of the samples laid back to back without padding, every token's modality
 * and (row, col), the work lists and the RoPE table (picx.dev "Mage-Flow: An
 * Efficient Native-Resolution Foundation Model for Image Generation and
 * Editing", section "Native-Resolution MMDiT (NR-MMDiT)", bullet
 * "Native-resolution packing": variable-length sequences packed into one
 * batch with per-sample cumulative offsets; findtube.ai transcript
 * "Mage-Flow: Efficient Native-Resolution Image Generation and Editing" at
 * [00:03:16] and [00:04:03]: one contiguous batch under a fixed token budget,
 * 2D RoPE per sample from its own grid). host_blob == NULL: size query only
 * (plan is filled, plan->blob_bytes says how much host memory the blob
 * needs). Runs on the host, touches no device. Errors: INVALID_ARG,
 * UNSUPPORTED (head_dim), BUDGET, BUFFER_TOO_SMALL (host_blob_bytes <
 * plan->blob_bytes). */
mmdit_status mmdit_pack_plan(const mmdit_pack_desc *desc, mmdit_plan *plan,
                             void *host_blob, uint64_t host_blob_bytes);

/* Plan of an editing pack (picx.dev "Mage-Flow ...", section
 * "Native-Resolution MMDiT (NR-MMDiT)", the conditioning bullet: source image
 * latents join the target latents in the sequence, told apart by a frame
 * dimension of a 3D RoPE; instruction-based editing timings on the video page
 * at [00:07:49]). Sample i holds text_len[i] text tokens, its grid_h[i] x
 * grid_w[i] target grid (frame 0) and then its src_h[i] x src_w[i] source
 * grid (frame 1), both row-major; src 0 x 0 = a generation sample (frame 0
 * only) in the same pack. Every image token of the pack is rotated with the
 * frame/row/column split. src_h and src_w
 * are [S] host arrays (>= 0, < 32768, both zero or both positive; a source
 * grid needs a target grid). Otherwise as mmdit_pack_plan, whose errors it
 * shares; the plan works with mmdit_attn_fwd / mmdit_attn_bwd unchanged. */
mmdit_status mmdit_pack_plan_edit(const mmdit_pack_desc *desc, const int32_t *src_h,
                                  const int32_t *src_w, mmdit_plan *plan,
                                  void *host_blob, uint64_t host_blob_bytes);

/* Packed classifier-free guidance (picx.dev "Mage-Flow ...", section
 * "Native-Resolution MMDiT (NR-MMDiT)", the packed CFG inference bullet, and
 * its results on native-resolution packing, Table 3; the video page at
 * [00:04:03]): one pack that evaluates the conditional and unconditional
 * branches in a single pass. Writes the descriptor of a pack of 2S samples:
 * the S samples of `cond` (conditional branches) followed, in the same order,
 * by their unconditional twins, which keep the latent grid and carry
 * null_text_len text tokens (0 = an empty prompt) instead of the prompt.
 * The caller provides the three arrays (capacity >= 2S entries each); *out
 * gets them and every other field of *cond (heads, d, dtype, theta, eps,
 * token budget, which the plan then checks against the doubled pack). Token
 * order of the pack: all conditional samples, then all unconditional ones.
 * Host only. Errors: INVALID_ARG (NULL pointers, S < 1, null_text_len < 0,
 * capacity < 2S, or a text-only conditional sample whose twin would be empty
 * because null_text_len is 0); nothing is written on error. */
mmdit_status mmdit_cfg_pack_desc(const mmdit_pack_desc *cond, int32_t null_text_len,
                                 int32_t *text_len, int32_t *grid_h, int32_t *grid_w,
                                 int32_t capacity, mmdit_pack_desc *out);

/* Stage selection for mmdit_fwd_args.stages / mmdit_bwd_args.stages. 0 = all.
 * A later stage alone reads what the earlier ones wrote (e.g. ATTENTION alone
 * reads the caller's q_hat / k_hat). */
#define MMDIT_STAGE_PROLOGUE      1u  /* fwd: RMSNorm + RoPE of Q and K -> q_hat, k_hat */
#define MMDIT_STAGE_ATTENTION     2u  /* fwd: var-len attention -> o, lse */
#define MMDIT_STAGE_BWD_DQ        1u  /* bwd: D = rowsum(dO * O), dQ-hat, inverse RoPE + RMSNorm
                                         backward -> dq, Q gain partials (workspace) */
#define MMDIT_STAGE_BWD_DKDV      2u  /* bwd: dK-hat and dV (reads D), inverse RoPE + RMSNorm
                                         backward -> dk, dv, K gain partials (workspace) */
#define MMDIT_STAGE_BWD_GAINS     4u  /* bwd: fixed-order sum of the gain partials -> dgains */
#define MMDIT_STAGE_BWD_D         8u  /* bwd, stored-dS mode only: D = rowsum(dO * O) */
#define MMDIT_STAGE_BWD_STORE_DS 16u  /* bwd mode flag: the stored-dS backward (see mmdit_attn_bwd);
                                         alone (no stage bit) = all stages of that mode */

typedef struct {
  const void *q, *k, *v;              /* [N][H][d] device, dtype; pre-norm */
  int64_t q_stride, k_stride, v_stride;
  const float *gains;                 /* [4][d] fp32 device: q_text, q_image, k_text, k_image */
  void *o;                            /* [N][H][d] dtype, dense */
  float *lse;                         /* [H][N] fp32 natural-log logsumexp; may be NULL */
  void *q_hat, *k_hat;                /* [N][H][d] dtype, dense; kept for the backward.
                                         Both NULL: use the workspace (inference). */
  float *rstd;                        /* [2][N][H] fp32 (Q then K) or NULL */
  uint32_t stages;                    /* 0 = all */
} mmdit_fwd_args;

/* Forward: q_hat, k_hat = RoPE(RMSNorm_m(q, k) * gain_m) per modality m, then
 * o = per-sample softmax(q_hat k_hat^T / sqrt(d)) v: joint text+image
 * attention confined to each sample of the pack (picx.dev "Mage-Flow ...",
 * section "Native-Resolution MMDiT (NR-MMDiT)": modality-specific
 * normalisation before joint attention, FlashAttention over per-sample
 * cumulative offsets; section "Training Infrastructure": RoPE and
 * normalisation fused into the kernels; transcript at [00:03:16]: 2D RoPE
 * of each image's own grid). workspace may be NULL when q_hat and k_hat
 * are given; else workspace_bytes >= plan->fwd_workspace_bytes. hip_stream is
 * a hipStream_t (NULL = the default stream). Deterministic: the same inputs
 * give bitwise the same outputs. */
mmdit_status mmdit_attn_fwd(const mmdit_plan *plan, const void *plan_blob_dev,
                            const mmdit_fwd_args *args, void *workspace,
                            uint64_t workspace_bytes, void *hip_stream);

typedef struct {
  const void *q, *k, *v;              /* pre-norm inputs of the forward, with strides */
  const void *q_hat, *k_hat, *o;      /* dense [N][H][d], as written by the forward */
  const void *dout;                   /* [N][H][d] dtype, stride dout_stride */
  int64_t q_stride, k_stride, v_stride, dout_stride;
  const float *gains;                 /* [4][d] fp32 */
  const float *lse;                   /* [H][N] fp32 from the forward (required) */
  const float *rstd;                  /* [2][N][H] from the forward, or NULL = recompute */
  void *dq, *dk, *dv;                 /* [N][H][d] dtype, dense: gradients w.r.t. pre-norm q, k, v */
  float *dgains;                      /* [4][d] fp32, overwritten; NULL = skip */
  uint32_t stages;                    /* 0 = all */
} mmdit_bwd_args;

/* Backward of mmdit_attn_fwd for the loss sum(dout * o): the gradients of the
 * pre-norm q, k, v and of the four gain rows, what training through the
 * attention of the pages needs (picx.dev "Mage-Flow ...", sections
 * "Native-Resolution MMDiT (NR-MMDiT)" and "Training Infrastructure";
 * transcript at [00:02:50] and [00:04:20]). workspace_bytes >=
 * plan->bwd_workspace_bytes. Workspace layout (fp32, each part 256-byte
 * aligned): D [H][N] at offset 0, then the Q and K gain-gradient partials;
 * fp32 plans also keep fp32 dQ-hat and dK-hat [N][H][d] after them. A stage
 * subset may run per call, in the order given below for the mode, on the
 * same workspace. Stage D needs o and dout; DQ needs q, dq (and o in the
 * recompute mode); DKDV needs k, dk, dv; both need q_hat, k_hat, v, dout,
 * lse, gains.
 * dQ is formed one of two ways, with equal results up to rounding order:
 *  - recompute (the default): the DQ stage forms D, then S and dP again for
 *    each query tile, and dQ; stages in the order DQ, DKDV, GAINS;
 *  - stored dS, selected only by MMDIT_STAGE_BWD_STORE_DS in stages (bf16
 *    plans with bwd_ds_workspace_bytes > bwd_workspace_bytes; workspace_bytes
 *    >= plan->bwd_ds_workspace_bytes): stage D forms D, the DKDV stage also
 *    writes dS (bf16, 2 bytes per score of every sample and head) to the
 *    workspace past bwd_workspace_bytes (rounded up to 4 KiB), and the DQ
 *    stage multiplies it by K-hat; stages in the order D, DKDV, DQ, GAINS.
 *    Measured 2-3% slower than the recompute mode on the mixed-resolution
 *    pack; the area takes ds_base[S] KiB, about 2 * H * sum(L_i^2) bytes.
 * stages = 0 runs every stage of the recompute mode, stages =
 * MMDIT_STAGE_BWD_STORE_DS every stage of the stored-dS mode. The flag is
 * UNSUPPORTED where the plan has no such mode and BUFFER_TOO_SMALL without
 * the room; stage D is INVALID_ARG without it; and a stored-dS call that
 * asks for both DQ and DKDV must include D (INVALID_ARG otherwise: the dK/dV
 * kernel reads the D that stage D writes).
 * Deterministic: the same inputs and the same workspace size give bitwise
 * the same outputs (no atomics; fixed-order reductions). */
mmdit_status mmdit_attn_bwd(const mmdit_plan *plan, const void *plan_blob_dev,
                            const mmdit_bwd_args *args, void *workspace,
                            uint64_t workspace_bytes, void *hip_stream);

/* Device-side fault flags (see mmdit_device_faults). */
#define MMDIT_DEVICE_FAULT_STALE_BLOB 1u  /* a kernel was given a device blob that is not the plan's */

/* Read and clear the current device's fault word: *flags gets the OR of the
 * MMDIT_DEVICE_FAULT_* flags that the library's kernels on this GPU recorded
 * since the previous call (0 = none). The read is queued on hip_stream (NULL =
 * default; it must belong to the current device) behind the work already
 * queued there, and the call synchronises that stream: the only entry point
 * that does. Errors: INVALID_ARG (flags NULL, stream of another device), HIP. */
mmdit_status mmdit_device_faults(uint32_t *flags, void *hip_stream);

/* Size of the per-GPU device array that mmdit_attn_bwd_noalloc uses as its
 * workspace (64 MiB): packs whose plan->bwd_workspace_bytes exceed it are
 * refused by that entry point. */
#define MMDIT_NOALLOC_WORKSPACE_BYTES (64ull << 20)

/* mmdit_attn_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same backward in its recompute mode, with the workspace taken from a
 * device array that the library owns (one per GPU, held until the process
 * ends) instead of a caller buffer. The caller still passes every input and
 * output, as for mmdit_attn_bwd; stage subsets run as there, and the array
 * keeps what the last call on that GPU left in it (a DKDV-only call reads the
 * D of the DQ call before it). The stream (NULL = default) must belong to the
 * current device. Calls that overlap on one GPU (different streams or
 * threads without ordering) share the array and race. Errors: those of
 * mmdit_attn_bwd; BUFFER_TOO_SMALL when plan->bwd_workspace_bytes >
 * MMDIT_NOALLOC_WORKSPACE_BYTES; UNSUPPORTED with MMDIT_STAGE_BWD_STORE_DS;
 * INVALID_ARG when the stream is on another device; HIP when the array's
 * device address cannot be looked up. Allocates, frees and synchronises
 * nothing. Deterministic, with results bitwise equal to mmdit_attn_bwd's
 * recompute mode. */
mmdit_status mmdit_attn_bwd_noalloc(const mmdit_plan *plan, const void *plan_blob_dev,
                                    const mmdit_bwd_args *args, void *hip_stream);

/* Adaptive LayerNorm modulation with the fused gated residual, the memory-
 * bound chains on either side of the attention core of an NR-MMDiT block
 * (picx.dev "Mage-Flow ...", section "Training Infrastructure": adaptive
 * normalisation and gating fused into kernels; video page at [00:04:20]:
 * normalisation and residual chains fused so that intermediates stay on
 * chip). The pages give no formula; this library computes the DiT-style adaLN
 *   z = x + gate * y                 (only when y is given: the gated residual
 *                                     of the attention's output projection y)
 *   h = (z - mean(z)) * (var(z) + eps)^(-1/2) * (1 + scale) + shift
 * over the model width D of each token (biased variance, eps inside the
 * root), where shift, scale and gate are fp32 tables [S][2][D] holding one row
 * per sample and stream (row 2*sample + stream; stream 0 = text tokens,
 * 1 = image tokens, an editing sample's target and source alike). Token
 * rows x, y, dh, dz: [N][D] of the plan's dtype with a token stride (>= D, a
 * multiple of 4, 16-byte aligned base); z, h, dx, dy: dense [N][D]. The plan
 * is any plan of the pack (its heads, head_dim and RoPE are not used). D is a
 * multiple of 4 in [4, 8192] (else UNSUPPORTED). Same ownership, validation,
 * aliasing and error rules as the attention calls; deterministic. */
typedef struct {
  const void *x;                      /* [N][D] */
  const void *y;                      /* [N][D] or NULL (no residual: z = x, not written) */
  int64_t x_stride, y_stride;
  const float *shift, *scale;         /* [S][2][D] fp32 */
  const float *gate;                  /* [S][2][D] fp32; with y only, else NULL */
  int32_t model_dim;                  /* D */
  float eps;                          /* >= 0, e.g. 1e-6 */
  void *z;                            /* [N][D] out: x + gate * y; with y only, else NULL */
  void *h;                            /* [N][D] out */
  float *stats;                       /* [N][2] out: {mean, rstd} of z per token, or NULL */
} mmdit_adaln_fwd_args;

mmdit_status mmdit_adaln_fwd(const mmdit_plan *plan, const void *plan_blob_dev,
                             const mmdit_adaln_fwd_args *args, void *hip_stream);

/* Backward of mmdit_adaln_fwd for the loss sum(dh * h) + sum(dz * z):
 *   g = dh * (1 + scale), z_hat = (z - mean) * rstd,
 *   dz_total = dz + rstd * (g - mean(g) - z_hat * mean(g * z_hat)),
 *   dx = dz_total, dy = gate * dz_total,
 *   dshift / dscale / dgate = sums over each (sample, stream) of dh,
 *   dh * z_hat and dz_total * y (fixed-order sums; rows with no tokens get 0).
 * workspace_bytes >= plan->num_mod_chunks * 3 * D * 4. */
typedef struct {
  const void *x, *y;                  /* the forward's inputs (y NULL: no residual) */
  int64_t x_stride, y_stride;
  const float *scale, *gate;          /* [S][2][D]; gate with y only */
  int32_t model_dim;
  float eps;
  const float *stats;                 /* [N][2] from the forward, or NULL = recompute */
  const void *dh;                     /* [N][D] gradient of h */
  const void *dz;                     /* [N][D] gradient arriving at z directly, or NULL */
  int64_t dh_stride, dz_stride;
  void *dx, *dy;                      /* [N][D] out; dy with y only */
  float *dshift, *dscale, *dgate;     /* [S][2][D] fp32 out (overwritten); dgate with y only */
} mmdit_adaln_bwd_args;

mmdit_status mmdit_adaln_bwd(const mmdit_plan *plan, const void *plan_blob_dev,
                             const mmdit_adaln_bwd_args *args, void *workspace,
                             uint64_t workspace_bytes, void *hip_stream);

const char *mmdit_status_str(mmdit_status s);
const char *mmdit_last_error(void);   /* detail of this thread's last non-OK return */
int32_t mmdit_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MMDIT_H */
