// Internal declarations shared by the host code and the HIP kernels of the
// packed joint-attention library. Not part of the C ABI (include/mmdit.h).
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "../../include/mmdit.h"

namespace mmdit {

// Rows of one query tile (forward and dQ) / one key tile (dK, dV): the
// work-list granularity. bf16 packs use 256-query tiles (8-wave workgroups);
// fp32 packs use 128-row tiles for both.
constexpr int kFwdTileBf16 = 256;
constexpr int kFwdTileF32 = 128;
constexpr int kBwdTile = 128;
// Limits checked by the plan.
constexpr int kModChunkRows = 32;               // rows per adaLN workgroup (one modulation row)
constexpr int kAdalnMaxDim = 8192;              // largest adaLN model width
constexpr int kMaxGridSide = 32768;             // row and col fit in 15 bits of tok_meta
constexpr int64_t kMaxTokens = 1ll << 29;  // byte offsets of [N] fp32 vectors fit 31 bits
constexpr int64_t kMaxElements = 1ll << 40;     // N*H*d
// Prologue backward: tokens per block and the cap on blocks (= gain partials).
constexpr int kPbwdTokensPerBlock = 64;
constexpr int kPbwdMaxBlocks = 1024;
// XCDs (each with its own L2) of the target GPU; workgroup b runs on XCD b % kXcds.
constexpr int kXcds = 8;
// Stored dS of the bf16 backward: 1 KiB blocks, each 32 keys x 16 queries of
// one (sample, head) in the dK/dV kernel's register order; samples up to
// kDsMaxSeqlen tokens (one sample-head area stays under 4 GiB).
constexpr int kDsBlockBytes = 1024;
constexpr int kDsMaxSeqlen = 32768;
inline int64_t ds_blocks_per_head(int64_t L) { return (L + 31) / 32 * 4 * ((L + 63) / 64); }

constexpr uint32_t kBlobMagic = 0x50444D4Du;    // "MMDP"
constexpr uint64_t kBlobHeaderBytes = 64;

struct BlobHeader {
  uint32_t magic;
  int32_t version;
  int32_t num_samples;
  int32_t total_tokens;
  uint64_t fingerprint;
  uint8_t pad[40];
};
static_assert(sizeof(BlobHeader) == kBlobHeaderBytes, "blob header size");

// Error reporting (thread-local message; see mmdit_last_error).
mmdit_status fail(mmdit_status s, const char *fmt, ...);
void clear_error();

uint64_t plan_fingerprint(const mmdit_plan &p);
// src_h == src_w == nullptr: a generation pack (2D RoPE); both given: an
// editing pack (3D RoPE, source grids after the target grids on frame 1).
mmdit_status build_plan(const mmdit_pack_desc *desc, const int32_t *src_h, const int32_t *src_w,
                        mmdit_plan *plan, void *host_blob, uint64_t host_blob_bytes);
mmdit_status cfg_pack_desc(const mmdit_pack_desc *cond, int32_t null_text_len, int32_t *text_len,
                           int32_t *grid_h, int32_t *grid_w, int32_t capacity, mmdit_pack_desc *out);
uint64_t bwd_partial_blocks(int64_t n_tokens);

// Backward workspace layout (byte offsets, each 256-byte aligned): D [H][N],
// Q gain partials [nq][2][d], K gain partials [nk][2][d], then for fp32 plans
// the dQ-hat and dK-hat accumulators [N][H][d]; `total` bytes in all. The
// stored-dS path (bf16) adds the dS area at `ds` (4 KiB aligned), ds_total
// bytes in all (ds_total = total where the path does not apply).
struct BwdLayout {
  uint64_t delta, nlse, part_q, part_k, dq_acc, dk_acc, total, ds, ds_total;
  int32_t nq, nk;
};
BwdLayout bwd_layout(const mmdit_plan &p);

// The backward behind mmdit_attn_bwd (validation, then launches); also used
// by the entry point that brings its own workspace.
mmdit_status attn_bwd(const mmdit_plan *plan, const void *blob, const mmdit_bwd_args *a, void *ws,
                      uint64_t ws_bytes, void *stream);

// ---------------------------------------------------------------------------
// Kernel launch arguments (device pointers; plain data passed by value).
// ---------------------------------------------------------------------------
// Check of the device blob against the host plan that every kernel makes
// before it reads anything else of the blob or writes anything: the blob
// header's fingerprint must equal the plan's. A kernel that finds otherwise
// ORs MMDIT_DEVICE_FAULT_STALE_BLOB into *status (this device's fault word,
// see mmdit_device_faults) and exits.
struct BlobGuard {
  const uint64_t *blob_fingerprint;  // the fingerprint word of the device blob's header
  uint64_t fingerprint;              // the host plan's
  uint32_t *status;                  // the device's fault word
};

// The current device's fault word, after checking that `stream` (NULL =
// the default stream) belongs to the current device.
mmdit_status device_fault_word(void *stream, uint32_t **word);
mmdit_status injected_launch_fault();  // test hook: MMDIT_FAULT_INJECT=launch

struct PlanDev {
  const int32_t *cu_seqlens;   // [S+1]
  const int32_t *tok_meta;     // [N]
  const int4 *fwd_items;       // [num_fwd_items]
  const int4 *bwd_items;       // [num_bwd_items]
  const int2 *fwd_blocks;      // [num_fwd_blocks] {item, head} or {-1, -1}
  const int2 *bwd_blocks;      // [num_bwd_blocks]
  const float2 *rope;          // [rope_rows][d/2] (cos, sin)
  int32_t num_samples, total_tokens, num_heads, head_dim;
  int32_t num_fwd_items, num_bwd_items, num_fwd_blocks, num_bwd_blocks, rope_rows;
  int32_t rope_frame_pairs;    // pairs [0, fp) turn by frame, then row, then column
  const int4 *mod_chunks;      // [num_mod_chunks] {row_start, row_end, 2*sample + stream, 0}
  const int32_t *mod_ranges;   // [2S+1] first chunk of each (sample, stream) range
  int32_t num_mod_chunks;
  float rms_eps;
  const int64_t *ds_base;      // [S+1] first dS block of each sample (all heads)
  BlobGuard guard;
};

struct PrologueFwdArgs {
  const void *q, *k;
  int64_t q_stride, k_stride;
  const float *gains;
  void *q_hat, *k_hat;
  float *rstd;                 // [2][N][H] or nullptr
};

struct AttnFwdArgs {
  const void *q_hat, *k_hat, *v;
  int64_t v_stride;
  void *o;
  float *lse;                  // [H][N] or nullptr
  float scale_log2;            // log2(e) / sqrt(d)
};

struct BwdPreArgs {
  const void *o, *dout;
  int64_t dout_stride;
  float *delta;                // [H][N]
  float *dq_acc;               // [N][H][d] fp32, zeroed here; nullptr: D only
  const float *lse;            // [H][N] (with nlse)
  float *nlse;                 // [H][N]: -lse * log2(e), or nullptr
};

struct AttnBwdArgs {
  const void *q_hat, *k_hat, *v, *dout, *o;
  int64_t v_stride, dout_stride;
  const float *lse;            // [H][N]
  float *delta;                // [H][N]: written by the dQ pass, read by the dK/dV pass
  float *nlse;                 // [H][N]: -lse * log2(e), written and read like delta (bf16 path)
  float *dq_acc;               // fp32 path: [N][H][d] dQ-hat (scaled by 1/sqrt(d))
  float *dk_acc;               // fp32 path: [N][H][d] dK-hat (scaled by 1/sqrt(d))
  void *dv;                    // [N][H][d] dtype
  float scale_log2;            // log2(e) / sqrt(d)
  float scale;                 // 1 / sqrt(d)
  // bf16 path: the prologue backward runs in the kernels' epilogues.
  const void *q, *k;           // pre-norm inputs
  int64_t q_stride, k_stride;
  const float *gains;          // [4][d]
  const float *rstd;           // [2][N][H] or nullptr = recompute
  void *dq, *dk;               // [N][H][d] dtype, dense
  float *part_q, *part_k;      // [grid blocks][2][d] gain-gradient partials (text, image)
  void *ds;                    // stored-dS area (bf16 path) or nullptr
};

// fp32 path: prologue backward of Q (which = 0) or K (which = 1) from the
// fp32 dX-hat accumulator.
struct PrologueBwdArgs {
  const void *x;
  int64_t x_stride;
  const float *gains;          // [4][d]
  const float *rstd;           // [2][N][H] or nullptr = recompute
  const float *dx_hat;         // [N][H][d] fp32
  void *dx;                    // [N][H][d] dtype, dense
  float *partials;             // [num_blocks][2][d]
  int32_t which;
  int32_t num_blocks;
};

// adaLN modulation (+ fused gated residual). Modulation tables are fp32
// [S][2][D] (row 2*sample + stream).
struct AdalnFwdArgs {
  const void *x, *y;           // [N][D] dtype with strides; y == nullptr: no residual
  int64_t x_stride, y_stride;
  const float *shift, *scale, *gate;
  void *z, *h;                 // dense [N][D] dtype; z only with y
  float2 *stats;               // [N] {mean, rstd} or nullptr
  int32_t dim;
  float eps;
};

struct AdalnBwdArgs {
  const void *x, *y, *dh, *dz; // dz == nullptr: no gradient arriving at z directly
  int64_t x_stride, y_stride, dh_stride, dz_stride;
  const float *scale, *gate;
  const float2 *stats;         // from the forward, or nullptr = recompute
  void *dx, *dy;               // dense [N][D] dtype; dy only with y
  float *partials;             // [num_mod_chunks][3][D]: dshift, dscale, dgate sums
  int32_t dim;
  float eps;
};

// Launchers: enqueue on `stream`, return the launch status.
hipError_t launch_prologue_fwd(int dtype, const PlanDev &p, const PrologueFwdArgs &a,
                               hipStream_t stream);
hipError_t launch_attn_fwd(int dtype, const PlanDev &p, const AttnFwdArgs &a, hipStream_t stream);
hipError_t launch_bwd_pre(int dtype, const PlanDev &p, const BwdPreArgs &a, hipStream_t stream);
// which = kBwdDq: dQ-hat (and D, unless a.ds is set: then dQ-hat from the
// stored dS); which = kBwdDkdv: dK-hat and dV (needs D; writes dS to a.ds
// when set).
constexpr int kBwdDq = 0, kBwdDkdv = 1;
hipError_t launch_attn_bwd(int dtype, const PlanDev &p, const AttnBwdArgs &a, int which,
                           hipStream_t stream);
hipError_t launch_prologue_bwd(int dtype, const PlanDev &p, const PrologueBwdArgs &a,
                               hipStream_t stream);
// dgains[m][e] = fixed-order sums of the gain partials: rows m = 0, 1 from
// part_q[0..nq), rows m = 2, 3 from part_k[0..nk).
hipError_t launch_adaln_fwd(int dtype, const PlanDev &p, const AdalnFwdArgs &a, hipStream_t stream);
hipError_t launch_adaln_bwd(int dtype, const PlanDev &p, const AdalnBwdArgs &a, hipStream_t stream);
// Fixed-order sums of the partials over each range's chunks -> out_k [S][2][D]
// for k = 0 (dshift), 1 (dscale), 2 (dgate, skipped when out2 is nullptr).
hipError_t launch_adaln_reduce(const PlanDev &p, const float *partials, int dim, float *out0,
                               float *out1, float *out2, hipStream_t stream);
hipError_t launch_gain_reduce(const BlobGuard &guard, const float *part_q, int nq, const float *part_k,
                              int nk, int d, float *dgains, hipStream_t stream);

}  // namespace mmdit
