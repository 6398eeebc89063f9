// Variable-length joint attention in fp32 (forward and backward), for fp32
// packs. Same definition as the bf16 MFMA kernels (per-sample softmax
// attention over the cumulative offsets; picx.dev summary "Mage-Flow: An
// Efficient Native-Resolution Foundation Model ...", section
// "Native-Resolution MMDiT (NR-MMDiT)"), computed on the vector ALU with fp32
// inputs as they are and fp32 accumulation throughout.
//
// Layout: 4 lanes per row (query for the forward and dQ, key for dK/dV), each
// owning d/4 consecutive elements; dot products are reduced over the 4 lanes
// with DPP. 128 rows per workgroup (512 threads); the other operand's rows are
// staged through LDS 32 at a time.
#include "device.h"
#include "internal.h"

namespace mmdit {

namespace f32k {
constexpr int ROWS = 128;        // rows per work item (kFwdTile == kBwdTile)
constexpr int TPR = 4;           // lanes per row
constexpr int NT = ROWS * TPR;   // threads per workgroup
constexpr int ST = 32;           // staged rows per step
constexpr float kLog2e = 1.4426950408889634f;
}  // namespace f32k
static_assert(f32k::ROWS == kFwdTileF32 && f32k::ROWS == kBwdTile, "fp32 kernels use the plan tiles");

template <int D>
__global__ __launch_bounds__(512) void attn_fwd_f32_kernel(PlanDev p, AttnFwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  using namespace f32k;
  constexpr int DC = D / TPR;
  __shared__ float ks[ST][D], vs[ST][D];
  const int H = p.num_heads;
  const int2 wb = p.fwd_blocks[blockIdx.x];
  if (wb.x < 0) return;  // idle slot of the block map (whole workgroup)
  const int4 it = p.fwd_items[wb.x];
  const int h = wb.y;
  const int seg0 = it.x, seg1 = it.y;
  const int qi = it.z + threadIdx.x / TPR;
  const int e0 = (threadIdx.x % TPR) * DC;
  const int qc = min(qi, seg1 - 1);
  const int64_t HD = (int64_t)H * D;
  const float *qh = static_cast<const float *>(a.q_hat);
  const float *kh = static_cast<const float *>(a.k_hat);
  const float *vv = static_cast<const float *>(a.v);
  const float c2 = a.scale_log2;

  float q[DC], o[DC];
#pragma unroll
  for (int e = 0; e < DC; ++e) {
    q[e] = qh[(int64_t)qc * HD + h * D + e0 + e];
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int kb0 = seg0; kb0 < seg1; kb0 += ST) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < ST * D; idx += NT) {
      const int r = idx / D, e = idx % D;
      const int key = min(kb0 + r, seg1 - 1);
      ks[r][e] = kh[(int64_t)key * HD + h * D + e];
      vs[r][e] = vv[(int64_t)key * a.v_stride + h * D + e];
    }
    __syncthreads();
    const int nk = min(ST, seg1 - kb0);
    for (int j = 0; j < nk; ++j) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < DC; ++e) s = fmaf(q[e], ks[j][e0 + e], s);
      s = group_sum<TPR>(s) * c2;
      if (s > m) {
        const float alpha = __builtin_amdgcn_exp2f(m - s);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < DC; ++e) o[e] *= alpha;
        m = s;
      }
      const float pj = __builtin_amdgcn_exp2f(s - m);
      l += pj;
#pragma unroll
      for (int e = 0; e < DC; ++e) o[e] = fmaf(pj, vs[j][e0 + e], o[e]);
    }
  }
  if (qi < seg1) {
    float *dst = static_cast<float *>(a.o) + (int64_t)qi * HD + h * D + e0;
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < DC; ++e) dst[e] = o[e] * inv;
    if (a.lse && e0 == 0) a.lse[(int64_t)h * p.total_tokens + qi] = (m + log2f(l)) * 0.69314718055994531f;
  }
}

// dK-hat and dV: 4 lanes per key, looping over the segment's queries.
template <int D>
__global__ __launch_bounds__(512) void attn_bwd_kv_f32_kernel(PlanDev p, AttnBwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  using namespace f32k;
  constexpr int DC = D / TPR;
  __shared__ float qs[ST][D], gs[ST][D], ls[ST], ds_[ST];
  const int H = p.num_heads;
  const int N = p.total_tokens;
  const int2 wb = p.bwd_blocks[blockIdx.x];
  if (wb.x < 0) return;  // idle slot of the block map (whole workgroup)
  const int4 it = p.bwd_items[wb.x];
  const int h = wb.y;
  const int seg0 = it.x, seg1 = it.y;
  const int ki = it.z + threadIdx.x / TPR;
  const int e0 = (threadIdx.x % TPR) * DC;
  const int kc = min(ki, seg1 - 1);
  const int64_t HD = (int64_t)H * D;
  const float *qh = static_cast<const float *>(a.q_hat);
  const float *kh = static_cast<const float *>(a.k_hat);
  const float *vv = static_cast<const float *>(a.v);
  const float *go = static_cast<const float *>(a.dout);
  const float c2 = a.scale_log2;

  float k[DC], v[DC], dk[DC], dv[DC];
#pragma unroll
  for (int e = 0; e < DC; ++e) {
    k[e] = kh[(int64_t)kc * HD + h * D + e0 + e];
    v[e] = vv[(int64_t)kc * a.v_stride + h * D + e0 + e];
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  for (int qb0 = seg0; qb0 < seg1; qb0 += ST) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < ST * D; idx += NT) {
      const int r = idx / D, e = idx % D;
      const int qq = min(qb0 + r, seg1 - 1);
      qs[r][e] = qh[(int64_t)qq * HD + h * D + e];
      gs[r][e] = go[(int64_t)qq * a.dout_stride + h * D + e];
    }
    for (int r = threadIdx.x; r < ST; r += NT) {
      const int qq = min(qb0 + r, seg1 - 1);
      ls[r] = a.lse[(int64_t)h * N + qq] * kLog2e;
      ds_[r] = a.delta[(int64_t)h * N + qq];
    }
    __syncthreads();
    const int nq = min(ST, seg1 - qb0);
    for (int j = 0; j < nq; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DC; ++e) {
        s = fmaf(qs[j][e0 + e], k[e], s);
        dp = fmaf(gs[j][e0 + e], v[e], dp);
      }
      s = group_sum<TPR>(s);
      dp = group_sum<TPR>(dp);
      const float pj = __builtin_amdgcn_exp2f(s * c2 - ls[j]);
      const float dsj = pj * (dp - ds_[j]);
#pragma unroll
      for (int e = 0; e < DC; ++e) {
        dv[e] = fmaf(pj, gs[j][e0 + e], dv[e]);
        dk[e] = fmaf(dsj, qs[j][e0 + e], dk[e]);
      }
    }
  }
  if (ki < seg1) {
    float *dvp = static_cast<float *>(a.dv) + (int64_t)ki * HD + h * D + e0;
    float *dkp = a.dk_acc + (int64_t)ki * HD + h * D + e0;
#pragma unroll
    for (int e = 0; e < DC; ++e) {
      dvp[e] = dv[e];
      dkp[e] = dk[e] * a.scale;
    }
  }
}

// dQ-hat: 4 lanes per query, looping over the segment's keys.
template <int D>
__global__ __launch_bounds__(512) void attn_bwd_q_f32_kernel(PlanDev p, AttnBwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  using namespace f32k;
  constexpr int DC = D / TPR;
  __shared__ float ks[ST][D], vs[ST][D];
  const int H = p.num_heads;
  const int N = p.total_tokens;
  const int2 wb = p.fwd_blocks[blockIdx.x];
  if (wb.x < 0) return;  // idle slot of the block map (whole workgroup)
  const int4 it = p.fwd_items[wb.x];
  const int h = wb.y;
  const int seg0 = it.x, seg1 = it.y;
  const int qi = it.z + threadIdx.x / TPR;
  const int e0 = (threadIdx.x % TPR) * DC;
  const int qc = min(qi, seg1 - 1);
  const int64_t HD = (int64_t)H * D;
  const float *qh = static_cast<const float *>(a.q_hat);
  const float *kh = static_cast<const float *>(a.k_hat);
  const float *vv = static_cast<const float *>(a.v);
  const float *go = static_cast<const float *>(a.dout);
  const float c2 = a.scale_log2;

  float q[DC], gq[DC], dq[DC];
#pragma unroll
  for (int e = 0; e < DC; ++e) {
    q[e] = qh[(int64_t)qc * HD + h * D + e0 + e];
    gq[e] = go[(int64_t)qc * a.dout_stride + h * D + e0 + e];
    dq[e] = 0.f;
  }
  const float lse2 = a.lse[(int64_t)h * N + qc] * kLog2e;
  const float dlt = a.delta[(int64_t)h * N + qc];
  for (int kb0 = seg0; kb0 < seg1; kb0 += ST) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < ST * D; idx += NT) {
      const int r = idx / D, e = idx % D;
      const int key = min(kb0 + r, seg1 - 1);
      ks[r][e] = kh[(int64_t)key * HD + h * D + e];
      vs[r][e] = vv[(int64_t)key * a.v_stride + h * D + e];
    }
    __syncthreads();
    const int nk = min(ST, seg1 - kb0);
    for (int j = 0; j < nk; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DC; ++e) {
        s = fmaf(q[e], ks[j][e0 + e], s);
        dp = fmaf(gq[e], vs[j][e0 + e], dp);
      }
      s = group_sum<TPR>(s);
      dp = group_sum<TPR>(dp);
      const float pj = __builtin_amdgcn_exp2f(s * c2 - lse2);
      const float dsj = pj * (dp - dlt);
#pragma unroll
      for (int e = 0; e < DC; ++e) dq[e] = fmaf(dsj, ks[j][e0 + e], dq[e]);
    }
  }
  if (qi < seg1) {
    float *dst = a.dq_acc + (int64_t)qi * HD + h * D + e0;
#pragma unroll
    for (int e = 0; e < DC; ++e) dst[e] = dq[e] * a.scale;
  }
}

template <int D>
static hipError_t fwd_f32(const PlanDev &p, const AttnFwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(attn_fwd_f32_kernel<D>, dim3((unsigned)p.num_fwd_blocks), dim3(f32k::NT), 0, s, p, a);
  return hipGetLastError();
}

template <int D>
static hipError_t bwd_f32(const PlanDev &p, const AttnBwdArgs &a, int which, hipStream_t s) {
  if (which == 1) {
    hipLaunchKernelGGL(attn_bwd_kv_f32_kernel<D>, dim3((unsigned)p.num_bwd_blocks), dim3(f32k::NT), 0, s, p, a);
    return hipGetLastError();
  }
  BwdPreArgs pre{a.o, a.dout, a.dout_stride, a.delta, a.dq_acc};
  hipError_t e = launch_bwd_pre(MMDIT_F32, p, pre, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_q_f32_kernel<D>, dim3((unsigned)p.num_fwd_blocks), dim3(f32k::NT), 0, s, p, a);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const PlanDev &p, const AttnFwdArgs &a, hipStream_t stream) {
  if (p.head_dim == 64) return fwd_f32<64>(p, a, stream);
  if (p.head_dim == 128) return fwd_f32<128>(p, a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd_f32(const PlanDev &p, const AttnBwdArgs &a, int which, hipStream_t stream) {
  if (p.head_dim == 64) return bwd_f32<64>(p, a, which, stream);
  if (p.head_dim == 128) return bwd_f32<128>(p, a, which, stream);
  return hipErrorInvalidValue;
}

}  // namespace mmdit
