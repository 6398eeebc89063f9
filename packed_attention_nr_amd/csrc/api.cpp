// C ABI entry points: host-side validation of every argument, then kernel
// launches on the caller's stream. Nothing is launched unless every check
// passes; no device memory is allocated, freed or synchronised here.
#include <cmath>
#include <cstddef>
#include <cstdio>
#include <string>
#include <vector>

#include "internal.h"

namespace mmdit {

static thread_local std::string g_last_error;

mmdit_status fail(mmdit_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

void clear_error() { g_last_error.clear(); }

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte range [lo, hi) touched by a tensor of n rows with `stride` elements
// between rows and `row` elements per row.
struct Span {
  const char *name;
  uintptr_t lo, hi;
  bool written;
};

static Span span(const char *name, const void *p, int64_t n, int64_t stride, int64_t row, int elt,
                 bool written) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  const uintptr_t bytes = (uintptr_t)(((n - 1) * stride + row) * elt);
  return Span{name, lo, lo + bytes, written};
}

// Every written buffer must be disjoint from every other buffer of the call.
static mmdit_status check_aliasing(const std::vector<Span> &spans) {
  for (size_t i = 0; i < spans.size(); ++i) {
    if (!spans[i].written) continue;
    for (size_t j = 0; j < spans.size(); ++j) {
      if (i == j) continue;
      if (spans[i].lo < spans[j].hi && spans[j].lo < spans[i].hi)
        return fail(MMDIT_ERR_INVALID_ARG, "output %s overlaps %s", spans[i].name, spans[j].name);
    }
  }
  return MMDIT_OK;
}

static mmdit_status check_plan(const mmdit_plan *plan, const void *blob) {
  if (!plan) return fail(MMDIT_ERR_INVALID_ARG, "plan must not be NULL");
  if (plan_fingerprint(*plan) != plan->fingerprint)
    return fail(MMDIT_ERR_INVALID_ARG, "plan fingerprint mismatch: not made by mmdit_pack_plan, or modified");
  if (!blob || !aligned16(blob))
    return fail(MMDIT_ERR_INVALID_ARG, "plan_blob_dev must be a non-NULL 16-byte aligned device pointer");
  return MMDIT_OK;
}

static mmdit_status check_tensor(const char *name, const void *p, int64_t stride, int64_t hd) {
  if (!p) return fail(MMDIT_ERR_INVALID_ARG, "%s must not be NULL", name);
  if (!aligned16(p)) return fail(MMDIT_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  if (stride < hd || stride % 8 != 0 || stride > MMDIT_MAX_ROW_STRIDE)
    return fail(MMDIT_ERR_INVALID_ARG, "%s stride %lld must be >= H*d (%lld), <= %lld and a multiple of 8", name,
                (long long)stride, (long long)hd, (long long)MMDIT_MAX_ROW_STRIDE);
  return MMDIT_OK;
}

static mmdit_status check_ptr(const char *name, const void *p) {
  if (!p) return fail(MMDIT_ERR_INVALID_ARG, "%s must not be NULL", name);
  if (!aligned16(p)) return fail(MMDIT_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return MMDIT_OK;
}

static PlanDev plan_dev(const mmdit_plan &p, const void *blob, uint32_t *fault_word) {
  const char *b = static_cast<const char *>(blob);
  PlanDev d;
  d.guard = BlobGuard{reinterpret_cast<const uint64_t *>(b + offsetof(BlobHeader, fingerprint)), p.fingerprint,
                      fault_word};
  d.cu_seqlens = reinterpret_cast<const int32_t *>(b + p.off_cu_seqlens);
  d.tok_meta = reinterpret_cast<const int32_t *>(b + p.off_tok_meta);
  d.fwd_items = reinterpret_cast<const int4 *>(b + p.off_fwd_items);
  d.bwd_items = reinterpret_cast<const int4 *>(b + p.off_bwd_items);
  d.fwd_blocks = reinterpret_cast<const int2 *>(b + p.off_fwd_blocks);
  d.bwd_blocks = reinterpret_cast<const int2 *>(b + p.off_bwd_blocks);
  d.rope = reinterpret_cast<const float2 *>(b + p.off_rope);
  d.num_samples = p.num_samples;
  d.total_tokens = p.total_tokens;
  d.num_heads = p.num_heads;
  d.head_dim = p.head_dim;
  d.num_fwd_items = p.num_fwd_items;
  d.num_bwd_items = p.num_bwd_items;
  d.num_fwd_blocks = p.num_fwd_blocks;
  d.num_bwd_blocks = p.num_bwd_blocks;
  d.rope_rows = p.rope_rows;
  d.rope_frame_pairs = p.rope_frame_pairs;
  d.mod_chunks = reinterpret_cast<const int4 *>(b + p.off_mod_chunks);
  d.mod_ranges = reinterpret_cast<const int32_t *>(b + p.off_mod_ranges);
  d.num_mod_chunks = p.num_mod_chunks;
  d.rms_eps = p.rms_eps;
  d.ds_base = reinterpret_cast<const int64_t *>(b + p.off_ds_base);
  return d;
}

static uint64_t align256(uint64_t x) { return (x + 255) / 256 * 256; }

static mmdit_status hip_fail(const char *what, hipError_t e) {
  return fail(MMDIT_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
}

static mmdit_status attn_fwd(const mmdit_plan *plan, const void *blob, const mmdit_fwd_args *a,
                             void *ws, uint64_t ws_bytes, void *stream) {
  mmdit_status st = check_plan(plan, blob);
  if (st) return st;
  if (!a) return fail(MMDIT_ERR_INVALID_ARG, "args must not be NULL");
  const uint32_t all = MMDIT_STAGE_PROLOGUE | MMDIT_STAGE_ATTENTION;
  const uint32_t stages = a->stages ? a->stages : all;
  if (stages & ~all) return fail(MMDIT_ERR_INVALID_ARG, "unknown forward stage bits 0x%x", stages);
  const bool pro = stages & MMDIT_STAGE_PROLOGUE, att = stages & MMDIT_STAGE_ATTENTION;
  const int64_t N = plan->total_tokens, H = plan->num_heads, d = plan->head_dim, HD = H * d;
  const int elt = plan->dtype == MMDIT_BF16 ? 2 : 4;

  void *qh = a->q_hat, *kh = a->k_hat;
  if ((qh == nullptr) != (kh == nullptr))
    return fail(MMDIT_ERR_INVALID_ARG, "q_hat and k_hat must both be given or both be NULL");
  std::vector<Span> spans;
  if (!qh) {
    if (!(pro && att))
      return fail(MMDIT_ERR_INVALID_ARG, "running one forward stage alone needs caller-owned q_hat and k_hat");
    if (!ws || !aligned16(ws))
      return fail(MMDIT_ERR_INVALID_ARG, "workspace must be a non-NULL 16-byte aligned device pointer");
    if (ws_bytes < plan->fwd_workspace_bytes)
      return fail(MMDIT_ERR_BUFFER_TOO_SMALL, "forward workspace needs %llu bytes, got %llu",
                  (unsigned long long)plan->fwd_workspace_bytes, (unsigned long long)ws_bytes);
    qh = ws;
    kh = static_cast<char *>(ws) + align256((uint64_t)N * HD * elt);
  } else {
    if ((st = check_ptr("q_hat", qh)) || (st = check_ptr("k_hat", kh))) return st;
  }
  spans.push_back(span("q_hat", qh, N, HD, HD, elt, pro));
  spans.push_back(span("k_hat", kh, N, HD, HD, elt, pro));
  if (pro) {
    if ((st = check_tensor("q", a->q, a->q_stride, HD)) || (st = check_tensor("k", a->k, a->k_stride, HD)) ||
        (st = check_ptr("gains", a->gains)))
      return st;
    spans.push_back(span("q", a->q, N, a->q_stride, HD, elt, false));
    spans.push_back(span("k", a->k, N, a->k_stride, HD, elt, false));
    spans.push_back(span("gains", a->gains, 4, d, d, 4, false));
    if (a->rstd) {
      if ((st = check_ptr("rstd", a->rstd))) return st;
      spans.push_back(span("rstd", a->rstd, 2 * N, H, H, 4, true));
    }
  }
  if (att) {
    if ((st = check_tensor("v", a->v, a->v_stride, HD)) || (st = check_ptr("o", a->o))) return st;
    spans.push_back(span("v", a->v, N, a->v_stride, HD, elt, false));
    spans.push_back(span("o", a->o, N, HD, HD, elt, true));
    if (a->lse) {
      if ((st = check_ptr("lse", a->lse))) return st;
      spans.push_back(span("lse", a->lse, H, N, N, 4, true));
    }
  }
  if ((st = check_aliasing(spans))) return st;
  uint32_t *fault = nullptr;
  if ((st = injected_launch_fault()) || (st = device_fault_word(stream, &fault))) return st;

  const PlanDev pd = plan_dev(*plan, blob, fault);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pro) {
    PrologueFwdArgs pa{a->q, a->k, a->q_stride, a->k_stride, a->gains, qh, kh, a->rstd};
    hipError_t e = launch_prologue_fwd(plan->dtype, pd, pa, s);
    if (e != hipSuccess) return hip_fail("prologue", e);
  }
  if (att) {
    AttnFwdArgs fa{qh, kh, a->v, a->v_stride, a->o, a->lse,
                   (float)(1.4426950408889634 / std::sqrt((double)d))};
    hipError_t e = launch_attn_fwd(plan->dtype, pd, fa, s);
    if (e != hipSuccess) return hip_fail("attention forward", e);
  }
  return MMDIT_OK;
}

mmdit_status attn_bwd(const mmdit_plan *plan, const void *blob, const mmdit_bwd_args *a,
                      void *ws, uint64_t ws_bytes, void *stream) {
  mmdit_status st = check_plan(plan, blob);
  if (st) return st;
  if (!a) return fail(MMDIT_ERR_INVALID_ARG, "args must not be NULL");
  const uint32_t all = MMDIT_STAGE_BWD_DQ | MMDIT_STAGE_BWD_DKDV | MMDIT_STAGE_BWD_GAINS;
  const uint32_t known = all | MMDIT_STAGE_BWD_D | MMDIT_STAGE_BWD_STORE_DS;
  if (a->stages & ~known) return fail(MMDIT_ERR_INVALID_ARG, "unknown backward stage bits 0x%x", a->stages);
  const int64_t N = plan->total_tokens, H = plan->num_heads, d = plan->head_dim, HD = H * d;
  const bool f32 = plan->dtype == MMDIT_F32;
  const int elt = f32 ? 4 : 2;
  if (!ws || !aligned16(ws))
    return fail(MMDIT_ERR_INVALID_ARG, "workspace must be a non-NULL 16-byte aligned device pointer");
  if (ws_bytes < plan->bwd_workspace_bytes)
    return fail(MMDIT_ERR_BUFFER_TOO_SMALL, "backward workspace needs %llu bytes, got %llu",
                (unsigned long long)plan->bwd_workspace_bytes, (unsigned long long)ws_bytes);
  const BwdLayout wl = bwd_layout(*plan);
  const bool has_ds = wl.ds_total > wl.total;  // the plan offers the stored-dS mode
  // The mode comes from the flag alone; no stage bit = every stage of it.
  const bool store_ds = a->stages & MMDIT_STAGE_BWD_STORE_DS;
  uint32_t stages = a->stages & ~MMDIT_STAGE_BWD_STORE_DS;
  if (store_ds && !has_ds)
    return fail(MMDIT_ERR_UNSUPPORTED, "this plan has no stored-dS backward (fp32, or a sample over %d tokens)",
                kDsMaxSeqlen);
  if (store_ds && ws_bytes < wl.ds_total)
    return fail(MMDIT_ERR_BUFFER_TOO_SMALL, "stored-dS backward workspace needs %llu bytes, got %llu",
                (unsigned long long)wl.ds_total, (unsigned long long)ws_bytes);
  if (!stages) stages = all | (store_ds ? MMDIT_STAGE_BWD_D : 0u);
  if ((stages & MMDIT_STAGE_BWD_D) && !store_ds)
    return fail(MMDIT_ERR_INVALID_ARG, "stage D belongs to the stored-dS backward (the DQ stage forms D otherwise)");
  if (store_ds && (stages & MMDIT_STAGE_BWD_DQ) && (stages & MMDIT_STAGE_BWD_DKDV) && !(stages & MMDIT_STAGE_BWD_D))
    return fail(MMDIT_ERR_INVALID_ARG,
                "a stored-dS call with both DQ and DKDV must include stage D (the dK/dV kernel reads its D)");
  const bool sd = stages & MMDIT_STAGE_BWD_D, sdq = stages & MMDIT_STAGE_BWD_DQ,
             skv = stages & MMDIT_STAGE_BWD_DKDV, sgn = stages & MMDIT_STAGE_BWD_GAINS;
  char *w = static_cast<char *>(ws);
  float *delta = reinterpret_cast<float *>(w + wl.delta);
  float *nlse = reinterpret_cast<float *>(w + wl.nlse);
  float *part_q = reinterpret_cast<float *>(w + wl.part_q);
  float *part_k = reinterpret_cast<float *>(w + wl.part_k);
  float *dq_acc = f32 ? reinterpret_cast<float *>(w + wl.dq_acc) : nullptr;
  float *dk_acc = f32 ? reinterpret_cast<float *>(w + wl.dk_acc) : nullptr;

  std::vector<Span> spans;
  spans.push_back(Span{"workspace", reinterpret_cast<uintptr_t>(ws),
                       reinterpret_cast<uintptr_t>(ws) + (store_ds ? wl.ds_total : plan->bwd_workspace_bytes),
                       true});
  if ((sdq && !store_ds) || sd) {
    if ((st = check_ptr("o", a->o))) return st;
    spans.push_back(span("o", a->o, N, HD, HD, elt, false));
  }
  if (sd && !(sdq || skv)) {
    if ((st = check_tensor("dout", a->dout, a->dout_stride, HD))) return st;
    spans.push_back(span("dout", a->dout, N, a->dout_stride, HD, elt, false));
  }
  if (sdq || skv) {
    if ((st = check_ptr("q_hat", a->q_hat)) || (st = check_ptr("k_hat", a->k_hat)) ||
        (st = check_tensor("v", a->v, a->v_stride, HD)) ||
        (st = check_tensor("dout", a->dout, a->dout_stride, HD)) || (st = check_ptr("lse", a->lse)) ||
        (st = check_ptr("gains", a->gains)))
      return st;
    spans.push_back(span("q_hat", a->q_hat, N, HD, HD, elt, false));
    spans.push_back(span("k_hat", a->k_hat, N, HD, HD, elt, false));
    spans.push_back(span("v", a->v, N, a->v_stride, HD, elt, false));
    spans.push_back(span("dout", a->dout, N, a->dout_stride, HD, elt, false));
    spans.push_back(span("lse", a->lse, H, N, N, 4, false));
    spans.push_back(span("gains", a->gains, 4, d, d, 4, false));
    if (a->rstd) {
      if ((st = check_ptr("rstd", a->rstd))) return st;
      spans.push_back(span("rstd", a->rstd, 2 * N, H, H, 4, false));
    }
  }
  if (sdq) {
    if ((st = check_tensor("q", a->q, a->q_stride, HD)) || (st = check_ptr("dq", a->dq))) return st;
    spans.push_back(span("q", a->q, N, a->q_stride, HD, elt, false));
    spans.push_back(span("dq", a->dq, N, HD, HD, elt, true));
  }
  if (skv) {
    if ((st = check_tensor("k", a->k, a->k_stride, HD)) || (st = check_ptr("dk", a->dk)) ||
        (st = check_ptr("dv", a->dv)))
      return st;
    spans.push_back(span("k", a->k, N, a->k_stride, HD, elt, false));
    spans.push_back(span("dk", a->dk, N, HD, HD, elt, true));
    spans.push_back(span("dv", a->dv, N, HD, HD, elt, true));
  }
  if (sgn && a->dgains) {
    if ((st = check_ptr("dgains", a->dgains))) return st;
    spans.push_back(span("dgains", a->dgains, 4, d, d, 4, true));
  }
  if ((st = check_aliasing(spans))) return st;
  uint32_t *fault = nullptr;
  if ((st = injected_launch_fault()) || (st = device_fault_word(stream, &fault))) return st;

  const PlanDev pd = plan_dev(*plan, blob, fault);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale = (float)(1.0 / std::sqrt((double)d));
  AttnBwdArgs ba{a->q_hat, a->k_hat, a->v, a->dout, a->o, a->v_stride, a->dout_stride, a->lse,
                 delta, nlse, dq_acc, dk_acc, a->dv, (float)(1.4426950408889634 / std::sqrt((double)d)),
                 scale, a->q, a->k, a->q_stride, a->k_stride, a->gains, a->rstd, a->dq, a->dk,
                 part_q, part_k, store_ds ? static_cast<void *>(w + wl.ds) : nullptr};
  if (store_ds) {  // D, then dK/dV writing dS, then dQ from dS
    hipError_t e = hipSuccess;
    if (sd) {
      const BwdPreArgs pre{a->o, a->dout, a->dout_stride, delta, nullptr, a->lse, nlse};
      e = launch_bwd_pre(plan->dtype, pd, pre, s);
    }
    if (e == hipSuccess && skv) e = launch_attn_bwd(plan->dtype, pd, ba, kBwdDkdv, s);
    if (e == hipSuccess && sdq) e = launch_attn_bwd(plan->dtype, pd, ba, kBwdDq, s);
    if (e != hipSuccess) return hip_fail("attention backward (stored dS)", e);
  }
  if (sdq && !store_ds) {
    hipError_t e = launch_attn_bwd(plan->dtype, pd, ba, kBwdDq, s);
    if (e == hipSuccess && f32) {
      const PrologueBwdArgs pa{a->q, a->q_stride, a->gains, a->rstd, dq_acc, a->dq, part_q, 0, wl.nq};
      e = launch_prologue_bwd(plan->dtype, pd, pa, s);
    }
    if (e != hipSuccess) return hip_fail("attention backward (dQ)", e);
  }
  if (skv && !store_ds) {
    hipError_t e = launch_attn_bwd(plan->dtype, pd, ba, kBwdDkdv, s);
    if (e == hipSuccess && f32) {
      const PrologueBwdArgs pa{a->k, a->k_stride, a->gains, a->rstd, dk_acc, a->dk, part_k, 1, wl.nk};
      e = launch_prologue_bwd(plan->dtype, pd, pa, s);
    }
    if (e != hipSuccess) return hip_fail("attention backward (dK, dV)", e);
  }
  if (sgn && a->dgains) {
    hipError_t e = launch_gain_reduce(pd.guard, part_q, wl.nq, part_k, wl.nk, (int)d, a->dgains, s);
    if (e != hipSuccess) return hip_fail("gain-gradient reduction", e);
  }
  return MMDIT_OK;
}

// Rows of the adaLN op: D elements per row, `stride` elements between rows.
static mmdit_status check_rows(const char *name, const void *p, int64_t stride, int64_t D) {
  if (!p) return fail(MMDIT_ERR_INVALID_ARG, "%s must not be NULL", name);
  if (!aligned16(p)) return fail(MMDIT_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  if (stride < D || stride % 4 != 0 || stride > MMDIT_MAX_ROW_STRIDE)
    return fail(MMDIT_ERR_INVALID_ARG, "%s stride %lld must be >= model_dim (%lld), <= %lld and a multiple of 4",
                name, (long long)stride, (long long)D, (long long)MMDIT_MAX_ROW_STRIDE);
  return MMDIT_OK;
}

static mmdit_status check_dim_eps(int32_t D, float eps) {
  if (D < 4 || D > kAdalnMaxDim || D % 4 != 0)
    return fail(MMDIT_ERR_UNSUPPORTED, "model_dim %d must be a multiple of 4 in [4, %d]", D, kAdalnMaxDim);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(MMDIT_ERR_INVALID_ARG, "eps must be finite and >= 0");
  return MMDIT_OK;
}

static mmdit_status adaln_fwd(const mmdit_plan *plan, const void *blob, const mmdit_adaln_fwd_args *a,
                              void *stream) {
  mmdit_status st = check_plan(plan, blob);
  if (st) return st;
  if (!a) return fail(MMDIT_ERR_INVALID_ARG, "args must not be NULL");
  if ((st = check_dim_eps(a->model_dim, a->eps))) return st;
  const int64_t N = plan->total_tokens, S = plan->num_samples, D = a->model_dim;
  const int elt = plan->dtype == MMDIT_BF16 ? 2 : 4;
  const bool res = a->y != nullptr;
  std::vector<Span> spans;
  if ((st = check_rows("x", a->x, a->x_stride, D)) || (st = check_ptr("shift", a->shift)) ||
      (st = check_ptr("scale", a->scale)) || (st = check_ptr("h", a->h)))
    return st;
  spans.push_back(span("x", a->x, N, a->x_stride, D, elt, false));
  spans.push_back(span("shift", a->shift, 2 * S, D, D, 4, false));
  spans.push_back(span("scale", a->scale, 2 * S, D, D, 4, false));
  spans.push_back(span("h", a->h, N, D, D, elt, true));
  if (res) {
    if ((st = check_rows("y", a->y, a->y_stride, D)) || (st = check_ptr("gate", a->gate)) ||
        (st = check_ptr("z", a->z)))
      return st;
    spans.push_back(span("y", a->y, N, a->y_stride, D, elt, false));
    spans.push_back(span("gate", a->gate, 2 * S, D, D, 4, false));
    spans.push_back(span("z", a->z, N, D, D, elt, true));
  } else if (a->gate || a->z) {
    return fail(MMDIT_ERR_INVALID_ARG, "gate and z are only taken with y (the gated residual)");
  }
  if (a->stats) {
    if ((st = check_ptr("stats", a->stats))) return st;
    spans.push_back(span("stats", a->stats, N, 2, 2, 4, true));
  }
  if ((st = check_aliasing(spans))) return st;
  uint32_t *fault = nullptr;
  if ((st = injected_launch_fault()) || (st = device_fault_word(stream, &fault))) return st;
  const PlanDev pd = plan_dev(*plan, blob, fault);
  AdalnFwdArgs fa{a->x, a->y, a->x_stride, a->y_stride, a->shift, a->scale, a->gate, a->z, a->h,
                  reinterpret_cast<float2 *>(a->stats), a->model_dim, a->eps};
  hipError_t e = launch_adaln_fwd(plan->dtype, pd, fa, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("adaLN forward", e);
  return MMDIT_OK;
}

static mmdit_status adaln_bwd(const mmdit_plan *plan, const void *blob, const mmdit_adaln_bwd_args *a, void *ws,
                              uint64_t ws_bytes, void *stream) {
  mmdit_status st = check_plan(plan, blob);
  if (st) return st;
  if (!a) return fail(MMDIT_ERR_INVALID_ARG, "args must not be NULL");
  if ((st = check_dim_eps(a->model_dim, a->eps))) return st;
  const int64_t N = plan->total_tokens, S = plan->num_samples, D = a->model_dim;
  const int elt = plan->dtype == MMDIT_BF16 ? 2 : 4;
  const bool res = a->y != nullptr;
  const uint64_t need = (uint64_t)plan->num_mod_chunks * 3 * (uint64_t)D * 4;
  if ((D + 63) / 64 * 2 * S > INT32_MAX)
    return fail(MMDIT_ERR_UNSUPPORTED, "too many samples (%lld) for the modulation-gradient sums", (long long)S);
  if (!ws || !aligned16(ws))
    return fail(MMDIT_ERR_INVALID_ARG, "workspace must be a non-NULL 16-byte aligned device pointer");
  if (ws_bytes < need)
    return fail(MMDIT_ERR_BUFFER_TOO_SMALL, "adaLN backward workspace needs %llu bytes, got %llu",
                (unsigned long long)need, (unsigned long long)ws_bytes);
  std::vector<Span> spans;
  if ((st = check_rows("x", a->x, a->x_stride, D)) || (st = check_rows("dh", a->dh, a->dh_stride, D)) ||
      (st = check_ptr("scale", a->scale)) || (st = check_ptr("dx", a->dx)) ||
      (st = check_ptr("dshift", a->dshift)) || (st = check_ptr("dscale", a->dscale)))
    return st;
  spans.push_back(span("workspace", ws, 1, (int64_t)need, (int64_t)need, 1, true));
  spans.push_back(span("x", a->x, N, a->x_stride, D, elt, false));
  spans.push_back(span("dh", a->dh, N, a->dh_stride, D, elt, false));
  spans.push_back(span("scale", a->scale, 2 * S, D, D, 4, false));
  spans.push_back(span("dx", a->dx, N, D, D, elt, true));
  spans.push_back(span("dshift", a->dshift, 2 * S, D, D, 4, true));
  spans.push_back(span("dscale", a->dscale, 2 * S, D, D, 4, true));
  if (res) {
    if ((st = check_rows("y", a->y, a->y_stride, D)) || (st = check_ptr("gate", a->gate)) ||
        (st = check_ptr("dy", a->dy)) || (st = check_ptr("dgate", a->dgate)))
      return st;
    spans.push_back(span("y", a->y, N, a->y_stride, D, elt, false));
    spans.push_back(span("gate", a->gate, 2 * S, D, D, 4, false));
    spans.push_back(span("dy", a->dy, N, D, D, elt, true));
    spans.push_back(span("dgate", a->dgate, 2 * S, D, D, 4, true));
  } else if (a->gate || a->dy || a->dgate) {
    return fail(MMDIT_ERR_INVALID_ARG, "gate, dy and dgate are only taken with y (the gated residual)");
  }
  if (a->dz) {
    if ((st = check_rows("dz", a->dz, a->dz_stride, D))) return st;
    spans.push_back(span("dz", a->dz, N, a->dz_stride, D, elt, false));
  }
  if (a->stats) {
    if ((st = check_ptr("stats", a->stats))) return st;
    spans.push_back(span("stats", a->stats, N, 2, 2, 4, false));
  }
  if ((st = check_aliasing(spans))) return st;
  uint32_t *fault = nullptr;
  if ((st = injected_launch_fault()) || (st = device_fault_word(stream, &fault))) return st;
  const PlanDev pd = plan_dev(*plan, blob, fault);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *part = static_cast<float *>(ws);
  AdalnBwdArgs ba{a->x, a->y, a->dh, a->dz, a->x_stride, a->y_stride, a->dh_stride, a->dz_stride,
                  a->scale, a->gate, reinterpret_cast<const float2 *>(a->stats), a->dx, a->dy, part,
                  a->model_dim, a->eps};
  hipError_t e = launch_adaln_bwd(plan->dtype, pd, ba, s);
  if (e != hipSuccess) return hip_fail("adaLN backward", e);
  e = launch_adaln_reduce(pd, part, a->model_dim, a->dshift, a->dscale, res ? a->dgate : nullptr, s);
  if (e != hipSuccess) return hip_fail("adaLN modulation-gradient reduction", e);
  return MMDIT_OK;
}

}  // namespace mmdit

extern "C" {

mmdit_status mmdit_pack_plan(const mmdit_pack_desc *desc, mmdit_plan *plan, void *host_blob,
                             uint64_t host_blob_bytes) {
  mmdit::clear_error();
  try {
    return mmdit::build_plan(desc, nullptr, nullptr, plan, host_blob, host_blob_bytes);
  } catch (...) {
    return mmdit::fail(MMDIT_ERR_INVALID_ARG, "pack plan failed (out of host memory?)");
  }
}

mmdit_status mmdit_pack_plan_edit(const mmdit_pack_desc *desc, const int32_t *src_h,
                                  const int32_t *src_w, mmdit_plan *plan, void *host_blob,
                                  uint64_t host_blob_bytes) {
  mmdit::clear_error();
  if (!src_h || !src_w) return mmdit::fail(MMDIT_ERR_INVALID_ARG, "src_h and src_w must not be NULL");
  try {
    return mmdit::build_plan(desc, src_h, src_w, plan, host_blob, host_blob_bytes);
  } catch (...) {
    return mmdit::fail(MMDIT_ERR_INVALID_ARG, "pack plan failed (out of host memory?)");
  }
}

mmdit_status mmdit_cfg_pack_desc(const mmdit_pack_desc *cond, int32_t null_text_len, int32_t *text_len,
                                 int32_t *grid_h, int32_t *grid_w, int32_t capacity, mmdit_pack_desc *out) {
  mmdit::clear_error();
  return mmdit::cfg_pack_desc(cond, null_text_len, text_len, grid_h, grid_w, capacity, out);
}

mmdit_status mmdit_attn_fwd(const mmdit_plan *plan, const void *plan_blob_dev, const mmdit_fwd_args *args,
                            void *workspace, uint64_t workspace_bytes, void *hip_stream) {
  mmdit::clear_error();
  try {
    return mmdit::attn_fwd(plan, plan_blob_dev, args, workspace, workspace_bytes, hip_stream);
  } catch (...) {
    return mmdit::fail(MMDIT_ERR_INVALID_ARG, "forward failed on the host");
  }
}

mmdit_status mmdit_attn_bwd(const mmdit_plan *plan, const void *plan_blob_dev, const mmdit_bwd_args *args,
                            void *workspace, uint64_t workspace_bytes, void *hip_stream) {
  mmdit::clear_error();
  try {
    return mmdit::attn_bwd(plan, plan_blob_dev, args, workspace, workspace_bytes, hip_stream);
  } catch (...) {
    return mmdit::fail(MMDIT_ERR_INVALID_ARG, "backward failed on the host");
  }
}

mmdit_status mmdit_adaln_fwd(const mmdit_plan *plan, const void *plan_blob_dev,
                             const mmdit_adaln_fwd_args *args, void *hip_stream) {
  mmdit::clear_error();
  try {
    return mmdit::adaln_fwd(plan, plan_blob_dev, args, hip_stream);
  } catch (...) {
    return mmdit::fail(MMDIT_ERR_INVALID_ARG, "adaLN forward failed on the host");
  }
}

mmdit_status mmdit_adaln_bwd(const mmdit_plan *plan, const void *plan_blob_dev,
                             const mmdit_adaln_bwd_args *args, void *workspace, uint64_t workspace_bytes,
                             void *hip_stream) {
  mmdit::clear_error();
  try {
    return mmdit::adaln_bwd(plan, plan_blob_dev, args, workspace, workspace_bytes, hip_stream);
  } catch (...) {
    return mmdit::fail(MMDIT_ERR_INVALID_ARG, "adaLN backward failed on the host");
  }
}

const char *mmdit_status_str(mmdit_status s) {
  switch (s) {
    case MMDIT_OK: return "ok";
    case MMDIT_ERR_INVALID_ARG: return "invalid argument";
    case MMDIT_ERR_UNSUPPORTED: return "unsupported";
    case MMDIT_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case MMDIT_ERR_BUDGET: return "token budget exceeded";
    case MMDIT_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *mmdit_last_error(void) { return mmdit::g_last_error.c_str(); }

int32_t mmdit_abi_version(void) { return MMDIT_ABI_VERSION; }

}  // extern "C"
