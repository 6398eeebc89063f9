// Memory-bound kernels of the attention core:
//  * prologue forward: per-modality RMSNorm of Q and K per head, the
//    modality's gain, then the per-sample 2D RoPE of image tokens
//    (picx.dev summary "Mage-Flow: An Efficient Native-Resolution Foundation
//    Model ...", section "Native-Resolution MMDiT (NR-MMDiT)": modality-specific
//    normalisation; findtube.ai transcript at [00:03:16]: per-sample 2D rotary
//    positional embeddings; section "Training Infrastructure": RoPE and
//    normalisation fused into single kernels);
//  * backward preprocess: D = rowsum(dO * O) per (token, head) and clearing
//    of the fp32 dQ-hat accumulator;
//  * prologue backward for the fp32 path (inverse RoPE, RMSNorm backward and
//    per-block gain-gradient partials; the bf16 attention kernels do this in
//    their epilogues), and the fixed-order reduction of the partials.
//
// One (token, head) row of d elements is handled by LPR lanes that each move
// 16 bytes (8 bf16 or 4 fp32); the row's sum of squares is reduced with DPP
// inside the lane group. All math is fp32; bf16 stores round to nearest even.
#include "device.h"
#include "internal.h"

namespace mmdit {

template <typename T>
struct Vec;
template <>
struct Vec<bf16> {
  static constexpr int N = 8;
  __device__ static void load(const bf16 *p, float *x) {
    bf16x8 v = ld_bf16x8(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
  }
  __device__ static void store(bf16 *p, const float *x) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      bf16x2 t = pack2(x[i], x[i + 1]);
      v[i] = t[0];
      v[i + 1] = t[1];
    }
    st16(p, as_u4(v));
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const float *p, float *x) {
    float4 v = *reinterpret_cast<const float4 *>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  __device__ static void store(float *p, const float *x) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

// Rotate the VEC/2 pairs of this lane (elements e0 .. e0+VEC-1 of a row) by
// the token's RoPE angles; sign = -1 applies the inverse rotation.
template <int D, int VEC>
__device__ __forceinline__ void rope_lane(float *x, const float2 *rope, int e0, int fp, int row,
                                          int col, int frame, float sign) {
  const int re = fp + (D / 2 - fp) / 2;
#pragma unroll
  for (int j = 0; j < VEC / 2; ++j) {
    const int pair = e0 / 2 + j;                 // pair index in [0, d/2)
    const int pos = rope_pos(pair, fp, re, row, col, frame);
    const float2 cs = rope[pos * (D / 2) + pair];
    const float c = cs.x, s = sign * cs.y;
    const float a = x[2 * j], b = x[2 * j + 1];
    x[2 * j] = a * c - b * s;
    x[2 * j + 1] = a * s + b * c;
  }
}

// ---------------------------------------------------------------------------
// Prologue forward
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void prologue_fwd_kernel(PlanDev p, PrologueFwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  constexpr int RPB = 256 / LPR;
  const int H = p.num_heads;
  const int64_t rows = (int64_t)p.total_tokens * H;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  if (r >= rows) return;  // whole lane groups exit together
  const int e0 = (threadIdx.x % LPR) * VEC;
  const int t = (int)(r / H), h = (int)(r % H);
  bool img;
  int row, col, frame;
  tok_pos(p.tok_meta[t], img, row, col, frame);

  float xq[VEC], xk[VEC];
  Vec<T>::load(static_cast<const T *>(a.q) + t * a.q_stride + h * D + e0, xq);
  Vec<T>::load(static_cast<const T *>(a.k) + t * a.k_stride + h * D + e0, xk);
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    sq += xq[i] * xq[i];
    sk += xk[i] * xk[i];
  }
  sq = group_sum<LPR>(sq);
  sk = group_sum<LPR>(sk);
  const float rq = rsqrtf(sq * (1.0f / D) + p.rms_eps);
  const float rk = rsqrtf(sk * (1.0f / D) + p.rms_eps);
  const float *gq = a.gains + (img ? 1 : 0) * D + e0;
  const float *gk = a.gains + (img ? 3 : 2) * D + e0;
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    xq[i] = xq[i] * rq * gq[i];
    xk[i] = xk[i] * rk * gk[i];
  }
  if (img) {
    rope_lane<D, VEC>(xq, p.rope, e0, p.rope_frame_pairs, row, col, frame, 1.f);
    rope_lane<D, VEC>(xk, p.rope, e0, p.rope_frame_pairs, row, col, frame, 1.f);
  }
  Vec<T>::store(static_cast<T *>(a.q_hat) + r * D + e0, xq);
  Vec<T>::store(static_cast<T *>(a.k_hat) + r * D + e0, xk);
  if (a.rstd && e0 == 0) {
    a.rstd[r] = rq;
    a.rstd[rows + r] = rk;
  }
}

// ---------------------------------------------------------------------------
// Backward preprocess: D = rowsum(dO * O) and, for the bf16 dK/dV kernel,
// -lse * log2(e) (the value the dQ kernel writes in the other mode, rounded
// the same way); clear the fp32 dQ-hat accumulator when there is one.
// ---------------------------------------------------------------------------
constexpr float kLog2eBwd = 1.4426950408889634f;
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(PlanDev p, BwdPreArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  constexpr int RPB = 256 / LPR;
  const int H = p.num_heads;
  const int N = p.total_tokens;
  const int64_t rows = (int64_t)N * H;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  if (r >= rows) return;
  const int e0 = (threadIdx.x % LPR) * VEC;
  const int t = (int)(r / H), h = (int)(r % H);
  float o[VEC], g[VEC];
  Vec<T>::load(static_cast<const T *>(a.o) + r * D + e0, o);
  Vec<T>::load(static_cast<const T *>(a.dout) + t * a.dout_stride + h * D + e0, g);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VEC; ++i) s += o[i] * g[i];
  s = group_sum<LPR>(s);
  if (e0 == 0) {
    a.delta[(int64_t)h * N + t] = s;
    if (a.nlse) a.nlse[(int64_t)h * N + t] = -(a.lse[(int64_t)h * N + t] * kLog2eBwd);
  }
  if (!a.dq_acc) return;
  float *z = a.dq_acc + r * D + e0;
#pragma unroll
  for (int i = 0; i < VEC; i += 4) *reinterpret_cast<float4 *>(z + i) = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------
// Prologue backward of Q (which = 0) or K (which = 1) from an fp32 dX-hat
// (the fp32 path; the bf16 attention kernels do this in their epilogues).
// Block b handles tokens [c*TPB, (c+1)*TPB) for chunks c = b, b + gridDim.x,
// ...; its gain-gradient sums go to partials[b][2][D] (text, image).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void prologue_bwd_kernel(PlanDev p, PrologueBwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  constexpr int RPB = 256 / LPR;
  constexpr int TPB = kPbwdTokensPerBlock;
  __shared__ float red[RPB][2][D];
  const int H = p.num_heads;
  const int N = p.total_tokens;
  const int64_t rows = (int64_t)N * H;
  const int e0 = (threadIdx.x % LPR) * VEC;
  const int grp = threadIdx.x / LPR;
  float acc[2][VEC];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[m][i] = 0.f;

  for (int64_t c = blockIdx.x; c * TPB < N; c += gridDim.x) {
    const int64_t r_end = min<int64_t>((c + 1) * TPB, N) * H;
    for (int64_t r = c * TPB * H + grp; r < r_end; r += RPB) {
      const int t = (int)(r / H), h = (int)(r % H);
      bool img;
      int row, col, frame;
      tok_pos(p.tok_meta[t], img, row, col, frame);
      const T *xp = static_cast<const T *>(a.x) + t * a.x_stride + h * D + e0;
      const float *dyp = a.dx_hat + r * D + e0;
      float x[VEC], dy[VEC];
      Vec<T>::load(xp, x);
#pragma unroll
      for (int i = 0; i < VEC; i += 4) {
        float4 v = *reinterpret_cast<const float4 *>(dyp + i);
        dy[i] = v.x; dy[i + 1] = v.y; dy[i + 2] = v.z; dy[i + 3] = v.w;
      }
      if (img) rope_lane<D, VEC>(dy, p.rope, e0, p.rope_frame_pairs, row, col, frame, -1.f);
      float rho;
      if (a.rstd) {
        rho = a.rstd[a.which * rows + r];
      } else {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < VEC; ++i) ss += x[i] * x[i];
        ss = group_sum<LPR>(ss);
        rho = rsqrtf(ss * (1.0f / D) + p.rms_eps);
      }
      const float *g = a.gains + (2 * a.which + (img ? 1 : 0)) * D + e0;
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) dot += g[i] * dy[i] * x[i];
      dot = group_sum<LPR>(dot);
      const float c3 = rho * rho * rho * dot * (1.0f / D);
      float dx[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        dx[i] = rho * g[i] * dy[i] - c3 * x[i];
        const float dg = dy[i] * x[i] * rho;
        acc[0][i] += img ? 0.f : dg;
        acc[1][i] += img ? dg : 0.f;
      }
      Vec<T>::store(static_cast<T *>(a.dx) + r * D + e0, dx);
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < VEC; ++i) red[grp][m][e0 + i] = acc[m][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 2 * D; idx += 256) {
    const int m = idx / D, e = idx % D;
    float s = 0.f;
    for (int k = 0; k < RPB; ++k) s += red[k][m][e];
    a.partials[(int64_t)blockIdx.x * 2 * D + idx] = s;
  }
}

// dgains[m][e] for m = 0, 1 is the sum over blocks b < nq of part_q[b][m][e],
// for m = 2, 3 over b < nk of part_k[b][m-2][e]. Workgroup (m, 64-column
// chunk): wave w sums blocks w, w+16, ... in order, then the 16 wave sums are
// added in order -- the same result on every run.
__global__ __launch_bounds__(1024) void gain_reduce_kernel(BlobGuard guard, const float *part_q, int nq,
                                                           const float *part_k, int nk, int d, float *dgains) {
  if (blob_stale(guard)) return;  // the partials came from another pack's blob: write nothing
  __shared__ float red[16][64];
  const int m = blockIdx.x / (d / 64);
  const int e = (blockIdx.x % (d / 64)) * 64 + (threadIdx.x & 63);
  const int w = threadIdx.x >> 6;
  const float *src = m < 2 ? part_q + m * d : part_k + (m - 2) * d;
  const int nb = m < 2 ? nq : nk;
  float s = 0.f;
  int b = w;
  for (; b + 16 * 7 < nb; b += 16 * 8) {  // eight loads in flight, summed in order
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = src[(int64_t)(b + 16 * u) * 2 * d + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += t[u];
  }
  for (; b < nb; b += 16) s += src[(int64_t)b * 2 * d + e];
  red[w][threadIdx.x & 63] = s;
  __syncthreads();
  if (w == 0) {
    float t = 0.f;
    for (int k = 0; k < 16; ++k) t += red[k][threadIdx.x];
    dgains[m * d + e] = t;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T, int D>
static int rows_per_block() {
  return 256 / (D / Vec<T>::N);
}

template <typename T, int D>
static hipError_t prologue_fwd_t(const PlanDev &p, const PrologueFwdArgs &a, hipStream_t s) {
  const int64_t rows = (int64_t)p.total_tokens * p.num_heads;
  const int64_t blocks = (rows + rows_per_block<T, D>() - 1) / rows_per_block<T, D>();
  hipLaunchKernelGGL((prologue_fwd_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, p, a);
  return hipGetLastError();
}
template <typename T, int D>
static hipError_t bwd_pre_t(const PlanDev &p, const BwdPreArgs &a, hipStream_t s) {
  const int64_t rows = (int64_t)p.total_tokens * p.num_heads;
  const int64_t blocks = (rows + rows_per_block<T, D>() - 1) / rows_per_block<T, D>();
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, p, a);
  return hipGetLastError();
}
template <typename T, int D>
static hipError_t prologue_bwd_t(const PlanDev &p, const PrologueBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((prologue_bwd_kernel<T, D>), dim3(a.num_blocks), dim3(256), 0, s, p, a);
  return hipGetLastError();
}

#define MMDIT_DISPATCH(FN, ...)                                         \
  do {                                                                  \
    if (dtype == MMDIT_BF16) {                                          \
      if (p.head_dim == 64) return FN<bf16, 64>(__VA_ARGS__);           \
      if (p.head_dim == 128) return FN<bf16, 128>(__VA_ARGS__);         \
    } else {                                                            \
      if (p.head_dim == 64) return FN<float, 64>(__VA_ARGS__);          \
      if (p.head_dim == 128) return FN<float, 128>(__VA_ARGS__);        \
    }                                                                   \
    return hipErrorInvalidValue;                                        \
  } while (0)

hipError_t launch_prologue_fwd(int dtype, const PlanDev &p, const PrologueFwdArgs &a,
                               hipStream_t stream) {
  MMDIT_DISPATCH(prologue_fwd_t, p, a, stream);
}
hipError_t launch_bwd_pre(int dtype, const PlanDev &p, const BwdPreArgs &a, hipStream_t stream) {
  MMDIT_DISPATCH(bwd_pre_t, p, a, stream);
}
hipError_t launch_prologue_bwd(int dtype, const PlanDev &p, const PrologueBwdArgs &a,
                               hipStream_t stream) {
  MMDIT_DISPATCH(prologue_bwd_t, p, a, stream);
}
hipError_t launch_gain_reduce(const BlobGuard &guard, const float *part_q, int nq, const float *part_k,
                              int nk, int d, float *dgains, hipStream_t stream) {
  if (d % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gain_reduce_kernel, dim3(4 * (d / 64)), dim3(1024), 0, stream, guard, part_q, nq, part_k,
                     nk, d, dgains);
  return hipGetLastError();
}

}  // namespace mmdit
