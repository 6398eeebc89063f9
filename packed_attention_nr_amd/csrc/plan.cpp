// Host-side pack plan: cu_seqlens, per-token metadata, longest-first work
// lists and the RoPE table, laid out in one blob for a single H2D copy.
//
// Packing follows the Mage-Flow pages: each sample's text tokens and its
// flattened latent grid are concatenated into one contiguous batch with
// per-sample cumulative offsets, under a fixed token budget (picx.dev summary,
// section "Native-Resolution MMDiT (NR-MMDiT)", bullet "Native-resolution
// packing"; findtube.ai transcript at [00:03:16] and [00:04:03]). Editing
// samples append the source image's latent grid after the target grid, told
// apart by the frame axis of a 3D RoPE (picx.dev, same section, conditioning
// bullet).
// Work lists and their longest-first order are this library's own scheduling
// choice (attention cost of a tile grows with its segment's length).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <vector>

#include "internal.h"

namespace mmdit {

uint64_t plan_fingerprint(const mmdit_plan &p) {
  // FNV-1a over every byte of the plan before the fingerprint field.
  const unsigned char *b = reinterpret_cast<const unsigned char *>(&p);
  size_t n = offsetof(mmdit_plan, fingerprint);
  uint64_t h = 1469598103934665603ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h;
}

static uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

int fwd_tile(int dtype, int d) {
  (void)d;
  return dtype == MMDIT_BF16 ? kFwdTileBf16 : kFwdTileF32;
}
int bwd_tile(int dtype, int d) {
  (void)dtype;
  (void)d;
  return kBwdTile;
}

uint64_t bwd_partial_blocks(int64_t n_tokens) {
  int64_t b = (n_tokens + kPbwdTokensPerBlock - 1) / kPbwdTokensPerBlock;
  return (uint64_t)std::max<int64_t>(1, std::min<int64_t>(b, kPbwdMaxBlocks));
}

BwdLayout bwd_layout(const mmdit_plan &p) {
  BwdLayout w{};
  const bool f32 = p.dtype == MMDIT_F32;
  const uint64_t N = (uint64_t)p.total_tokens, H = (uint64_t)p.num_heads, d = (uint64_t)p.head_dim;
  w.nq = f32 ? (int32_t)bwd_partial_blocks(p.total_tokens) : p.num_fwd_blocks;
  w.nk = f32 ? (int32_t)bwd_partial_blocks(p.total_tokens) : p.num_bwd_blocks;
  uint64_t off = 0;
  w.delta = off;
  off = align_up(off + 4 * H * N, 256);
  w.nlse = off;
  off = align_up(off + 4 * H * N, 256);
  w.part_q = off;
  off = align_up(off + (uint64_t)w.nq * 2 * d * 4, 256);
  w.part_k = off;
  off = align_up(off + (uint64_t)w.nk * 2 * d * 4, 256);
  w.dq_acc = w.dk_acc = off;
  if (f32) {
    off = align_up(off + N * H * d * 4, 256);
    w.dk_acc = off;
    off = align_up(off + N * H * d * 4, 256);
  }
  w.total = off;
  w.ds = align_up(off, 4096);
  w.ds_total = p.bwd_ds_workspace_bytes > off ? p.bwd_ds_workspace_bytes : off;
  return w;
}

// Angles of the RoPE table: pair p of the d/2 pairs belongs to one section
// (frame, row or column, in that order; frame_pairs = 0: row and column
// only) and turns by pos * theta^(-j/n), j its index in the section and n the
// section's size. With two sections of d/4 pairs this is pos * theta^(-4j/d).
static double rope_omega(double theta, int d, int frame_pairs, int p) {
  const int half = d / 2, re = frame_pairs + (half - frame_pairs) / 2;
  int j, n;
  if (p < frame_pairs) {
    j = p, n = frame_pairs;
  } else if (p < re) {
    j = p - frame_pairs, n = re - frame_pairs;
  } else {
    j = p - re, n = half - re;
  }
  return std::pow(theta, -(double)j / (double)n);
}

mmdit_status build_plan(const mmdit_pack_desc *desc, const int32_t *src_h, const int32_t *src_w,
                        mmdit_plan *plan, void *host_blob, uint64_t host_blob_bytes) {
  if (!desc || !plan) return fail(MMDIT_ERR_INVALID_ARG, "desc and plan must not be NULL");
  const bool edit = src_h || src_w;
  if (edit && !(src_h && src_w))
    return fail(MMDIT_ERR_INVALID_ARG, "src_h and src_w must both be given");
  const int S = desc->num_samples;
  if (S < 1) return fail(MMDIT_ERR_INVALID_ARG, "num_samples must be >= 1");
  if (!desc->text_len || !desc->grid_h || !desc->grid_w)
    return fail(MMDIT_ERR_INVALID_ARG, "text_len, grid_h and grid_w must not be NULL");
  if (desc->num_heads < 1) return fail(MMDIT_ERR_INVALID_ARG, "num_heads must be >= 1");
  if (desc->dtype != MMDIT_F32 && desc->dtype != MMDIT_BF16)
    return fail(MMDIT_ERR_INVALID_ARG, "dtype must be MMDIT_F32 or MMDIT_BF16");
  if (desc->head_dim <= 0 || desc->head_dim % 4 != 0)
    return fail(MMDIT_ERR_INVALID_ARG, "head_dim must be a positive multiple of 4");
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return fail(MMDIT_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!(desc->rope_theta > 0.f) || !std::isfinite(desc->rope_theta))
    return fail(MMDIT_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if (!(desc->rms_eps >= 0.f) || !std::isfinite(desc->rms_eps))
    return fail(MMDIT_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (desc->token_budget < 0) return fail(MMDIT_ERR_INVALID_ARG, "token_budget must be >= 0");

  std::vector<int64_t> L(S);
  int64_t N = 0, max_len = 0, max_side = 0;
  for (int i = 0; i < S; ++i) {
    const int32_t t = desc->text_len[i], h = desc->grid_h[i], w = desc->grid_w[i];
    if (t < 0 || h < 0 || w < 0)
      return fail(MMDIT_ERR_INVALID_ARG, "sample %d: negative text_len or grid size", i);
    if ((h == 0) != (w == 0))
      return fail(MMDIT_ERR_INVALID_ARG, "sample %d: grid_h and grid_w must both be 0 or both > 0", i);
    if (h >= kMaxGridSide || w >= kMaxGridSide)
      return fail(MMDIT_ERR_INVALID_ARG, "sample %d: grid side must be < %d", i, kMaxGridSide);
    L[i] = (int64_t)t + (int64_t)h * (int64_t)w;
    if (edit) {
      const int32_t sh = src_h[i], sw = src_w[i];
      if (sh < 0 || sw < 0 || (sh == 0) != (sw == 0))
        return fail(MMDIT_ERR_INVALID_ARG, "sample %d: src_h and src_w must both be 0 or both > 0", i);
      if (sh >= kMaxGridSide || sw >= kMaxGridSide)
        return fail(MMDIT_ERR_INVALID_ARG, "sample %d: grid side must be < %d", i, kMaxGridSide);
      if (sh > 0 && h == 0)
        return fail(MMDIT_ERR_INVALID_ARG, "sample %d: a source grid needs a target grid", i);
      L[i] += (int64_t)sh * (int64_t)sw;
      max_side = std::max<int64_t>(max_side, std::max(sh, sw));
    }
    if (L[i] < 1) return fail(MMDIT_ERR_INVALID_ARG, "sample %d has no tokens", i);
    N += L[i];
    if (N > kMaxTokens) return fail(MMDIT_ERR_INVALID_ARG, "total tokens exceed %lld", (long long)kMaxTokens);
    max_len = std::max(max_len, L[i]);
    max_side = std::max<int64_t>(max_side, std::max(h, w));
  }
  if (desc->token_budget > 0 && N > desc->token_budget)
    return fail(MMDIT_ERR_BUDGET, "pack has %lld tokens, budget is %lld", (long long)N,
                (long long)desc->token_budget);
  const int64_t H = desc->num_heads, d = desc->head_dim;
  if (N * H * d > kMaxElements)
    return fail(MMDIT_ERR_INVALID_ARG, "N*H*d exceeds %lld", (long long)kMaxElements);

  const int qt = fwd_tile(desc->dtype, (int)d), kt = bwd_tile(desc->dtype, (int)d);
  std::vector<int64_t> cu(S + 1, 0);
  for (int i = 0; i < S; ++i) cu[i + 1] = cu[i] + L[i];

  // Longest segment first; ties by sample, then by tile.
  std::vector<int> order(S);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return L[a] > L[b]; });
  auto count_items = [&](int tile) {
    int64_t n = 0;
    for (int i = 0; i < S; ++i) n += (L[i] + tile - 1) / tile;
    return n;
  };
  const int64_t n_fwd = count_items(qt), n_bwd = count_items(kt);
  if ((n_fwd + kXcds) * H > INT32_MAX / 4 || (n_bwd + kXcds) * H > INT32_MAX / 4)
    return fail(MMDIT_ERR_INVALID_ARG, "too many work items");
  // Frame positions are 0 (target) and 1 (source).
  const int rope_rows = (int)std::max<int64_t>(edit ? 2 : 1, max_side);
  const int frame_pairs = edit ? (int)(d / 8) : 0;
  // Workgroup -> (item, head) maps: chunks of all tiles of one (sample, head),
  // dealt round-robin over the XCDs in longest-first order.
  auto block_map = [&](int tile, std::vector<int32_t> &out) {
    std::vector<std::vector<int32_t>> seq(kXcds);
    int64_t item0 = 0, chunk = 0;
    for (int s : order) {
      const int64_t nt = (L[s] + tile - 1) / tile;
      for (int64_t hh = 0; hh < H; ++hh, ++chunk) {
        auto &q = seq[chunk % kXcds];
        for (int64_t t = 0; t < nt; ++t) {
          q.push_back((int32_t)(item0 + t));
          q.push_back((int32_t)hh);
        }
      }
      item0 += nt;
    }
    size_t longest = 0;
    for (auto &q : seq) longest = std::max(longest, q.size() / 2);
    out.assign(2 * longest * kXcds, -1);
    for (int x = 0; x < kXcds; ++x)
      for (size_t pos = 0; pos < seq[x].size() / 2; ++pos) {
        out[2 * (pos * kXcds + x) + 0] = seq[x][2 * pos + 0];
        out[2 * (pos * kXcds + x) + 1] = seq[x][2 * pos + 1];
      }
  };

  std::vector<int32_t> fwd_blocks, bwd_blocks;
  block_map(qt, fwd_blocks);
  block_map(kt, bwd_blocks);

  // Row chunks of the adaLN kernels: each (sample, stream) token range (text
  // [cu, cu + T), image [cu + T, cu + L)) cut into pieces of at most
  // kModChunkRows rows, so that a workgroup's rows share one modulation row
  // and its gradient partials belong to one range.
  std::vector<int32_t> mod_chunks, mod_ranges(2 * S + 1, 0);
  for (int i = 0; i < S; ++i)
    for (int m = 0; m < 2; ++m) {
      const int64_t a = cu[i] + (m ? desc->text_len[i] : 0), b = m ? cu[i + 1] : cu[i] + desc->text_len[i];
      for (int64_t r = a; r < b; r += kModChunkRows) {
        mod_chunks.push_back((int32_t)r);
        mod_chunks.push_back((int32_t)std::min<int64_t>(b, r + kModChunkRows));
        mod_chunks.push_back(2 * i + m);
        mod_chunks.push_back(0);
      }
      mod_ranges[2 * i + m + 1] = (int32_t)(mod_chunks.size() / 4);
    }

  mmdit_plan p;
  std::memset(&p, 0, sizeof(p));
  p.num_samples = S;
  p.total_tokens = (int32_t)N;
  p.max_seqlen = (int32_t)max_len;
  p.num_heads = (int32_t)H;
  p.head_dim = (int32_t)d;
  p.dtype = desc->dtype;
  p.q_tile = qt;
  p.kv_tile = kt;
  p.num_fwd_items = (int32_t)n_fwd;
  p.num_bwd_items = (int32_t)n_bwd;
  p.num_fwd_blocks = (int32_t)(fwd_blocks.size() / 2);
  p.num_bwd_blocks = (int32_t)(bwd_blocks.size() / 2);
  p.num_mod_chunks = (int32_t)(mod_chunks.size() / 4);
  p.mod_chunk_rows = kModChunkRows;
  p.rope_rows = rope_rows;
  p.rope_frame_pairs = frame_pairs;
  p.rope_theta = desc->rope_theta;
  p.rms_eps = desc->rms_eps;
  uint64_t off = align_up(kBlobHeaderBytes, 256);
  p.off_cu_seqlens = off;
  off = align_up(off + 4ull * (S + 1), 256);
  p.off_tok_meta = off;
  off = align_up(off + 4ull * N, 256);
  p.off_fwd_items = off;
  off = align_up(off + 16ull * n_fwd, 256);
  p.off_bwd_items = off;
  off = align_up(off + 16ull * n_bwd, 256);
  p.off_fwd_blocks = off;
  off = align_up(off + 4ull * fwd_blocks.size(), 256);
  p.off_bwd_blocks = off;
  off = align_up(off + 4ull * bwd_blocks.size(), 256);
  p.off_rope = off;
  off = align_up(off + 8ull * rope_rows * (d / 2), 256);
  p.off_mod_chunks = off;
  off = align_up(off + 4ull * mod_chunks.size(), 256);
  p.off_mod_ranges = off;
  off = align_up(off + 4ull * mod_ranges.size(), 256);
  p.off_ds_base = off;
  off = align_up(off + 8ull * (S + 1), 256);
  p.blob_bytes = off;

  const uint64_t elt = desc->dtype == MMDIT_BF16 ? 2 : 4;
  const uint64_t nhd = (uint64_t)N * H * d;
  p.fwd_workspace_bytes = 2 * align_up(nhd * elt, 256);
  p.bwd_workspace_bytes = bwd_layout(p).total;
  // Stored-dS backward: per sample and head ceil(L/32) * 4 * ceil(L/64)
  // blocks of 1 KiB, samples in pack order, heads inside a sample.
  std::vector<int64_t> ds_base(S + 1, 0);
  for (int i = 0; i < S; ++i) ds_base[i + 1] = ds_base[i] + (int64_t)H * ds_blocks_per_head(cu[i + 1] - cu[i]);
  p.bwd_ds_workspace_bytes = p.bwd_workspace_bytes;
  if (desc->dtype == MMDIT_BF16 && max_len <= kDsMaxSeqlen)
    p.bwd_ds_workspace_bytes = bwd_layout(p).ds + (uint64_t)ds_base[S] * kDsBlockBytes;
  p.fingerprint = plan_fingerprint(p);
  *plan = p;

  if (!host_blob) return MMDIT_OK;  // size query
  if (host_blob_bytes < p.blob_bytes)
    return fail(MMDIT_ERR_BUFFER_TOO_SMALL, "host blob needs %llu bytes, got %llu",
                (unsigned long long)p.blob_bytes, (unsigned long long)host_blob_bytes);

  unsigned char *blob = static_cast<unsigned char *>(host_blob);
  std::memset(blob, 0, p.blob_bytes);
  BlobHeader hdr;
  std::memset(&hdr, 0, sizeof(hdr));
  hdr.magic = kBlobMagic;
  hdr.version = MMDIT_ABI_VERSION;
  hdr.num_samples = S;
  hdr.total_tokens = (int32_t)N;
  hdr.fingerprint = p.fingerprint;
  std::memcpy(blob, &hdr, sizeof(hdr));

  int32_t *cu32 = reinterpret_cast<int32_t *>(blob + p.off_cu_seqlens);
  for (int i = 0; i <= S; ++i) cu32[i] = (int32_t)cu[i];

  int32_t *meta = reinterpret_cast<int32_t *>(blob + p.off_tok_meta);
  for (int i = 0; i < S; ++i) {
    const int64_t base = cu[i] + desc->text_len[i];
    for (int64_t t = cu[i]; t < base; ++t) meta[t] = 0;
    const int32_t h = desc->grid_h[i], w = desc->grid_w[i];
    for (int32_t r = 0; r < h; ++r)
      for (int32_t c = 0; c < w; ++c)
        meta[base + (int64_t)r * w + c] = (int32_t)(0x80000000u | ((uint32_t)r << 16) | (uint32_t)c);
    if (!edit) continue;
    // The source grid follows the target grid, on frame 1.
    const int64_t sbase = base + (int64_t)h * w;
    const int32_t sh = src_h[i], sw = src_w[i];
    for (int32_t r = 0; r < sh; ++r)
      for (int32_t c = 0; c < sw; ++c)
        meta[sbase + (int64_t)r * sw + c] =
            (int32_t)(0x80000000u | ((uint32_t)r << 16) | 0x8000u | (uint32_t)c);
  }

  auto fill_items = [&](int32_t *it, int tile) {
    int64_t k = 0;
    for (int s : order)
      for (int64_t t0 = cu[s]; t0 < cu[s + 1]; t0 += tile) {
        it[4 * k + 0] = (int32_t)cu[s];
        it[4 * k + 1] = (int32_t)cu[s + 1];
        it[4 * k + 2] = (int32_t)t0;
        it[4 * k + 3] = s;
        ++k;
      }
  };
  fill_items(reinterpret_cast<int32_t *>(blob + p.off_fwd_items), qt);
  fill_items(reinterpret_cast<int32_t *>(blob + p.off_bwd_items), kt);

  std::memcpy(blob + p.off_fwd_blocks, fwd_blocks.data(), 4 * fwd_blocks.size());
  std::memcpy(blob + p.off_bwd_blocks, bwd_blocks.data(), 4 * bwd_blocks.size());
  std::memcpy(blob + p.off_mod_chunks, mod_chunks.data(), 4 * mod_chunks.size());
  std::memcpy(blob + p.off_mod_ranges, mod_ranges.data(), 4 * mod_ranges.size());
  std::memcpy(blob + p.off_ds_base, ds_base.data(), 8 * ds_base.size());

  // RoPE table [rope_rows][d/2] of {cos, sin}(pos * omega_p), in double,
  // rounded once.
  float *rope = reinterpret_cast<float *>(blob + p.off_rope);
  const int half = (int)(d / 2);
  for (int pr = 0; pr < half; ++pr) {
    const double om = rope_omega((double)desc->rope_theta, (int)d, frame_pairs, pr);
    for (int pos = 0; pos < rope_rows; ++pos) {
      const double a = (double)pos * om;
      rope[2 * ((int64_t)pos * half + pr) + 0] = (float)std::cos(a);
      rope[2 * ((int64_t)pos * half + pr) + 1] = (float)std::sin(a);
    }
  }
  return MMDIT_OK;
}

mmdit_status cfg_pack_desc(const mmdit_pack_desc *cond, int32_t null_text_len, int32_t *text_len,
                           int32_t *grid_h, int32_t *grid_w, int32_t capacity, mmdit_pack_desc *out) {
  if (!cond || !out || !text_len || !grid_h || !grid_w)
    return fail(MMDIT_ERR_INVALID_ARG, "cond, out and the three arrays must not be NULL");
  const int32_t S = cond->num_samples;
  if (S < 1) return fail(MMDIT_ERR_INVALID_ARG, "num_samples must be >= 1");
  if (!cond->text_len || !cond->grid_h || !cond->grid_w)
    return fail(MMDIT_ERR_INVALID_ARG, "cond's text_len, grid_h and grid_w must not be NULL");
  if (null_text_len < 0) return fail(MMDIT_ERR_INVALID_ARG, "null_text_len must be >= 0");
  if (S > INT32_MAX / 2 || capacity < 2 * S)
    return fail(MMDIT_ERR_INVALID_ARG, "capacity %d is below 2 * num_samples (%d)", capacity, S);
  for (int32_t i = 0; i < S; ++i)
    if (null_text_len == 0 && (cond->grid_h[i] == 0 || cond->grid_w[i] == 0))
      return fail(MMDIT_ERR_INVALID_ARG, "sample %d is text-only: its unconditional twin would be empty", i);
  for (int32_t i = 0; i < S; ++i) {
    text_len[i] = cond->text_len[i];
    grid_h[i] = grid_h[S + i] = cond->grid_h[i];
    grid_w[i] = grid_w[S + i] = cond->grid_w[i];
    text_len[S + i] = null_text_len;
  }
  *out = *cond;
  out->num_samples = 2 * S;
  out->text_len = text_len;
  out->grid_h = grid_h;
  out->grid_w = grid_w;
  return MMDIT_OK;
}

}  // namespace mmdit
