// Variable-length joint attention, forward, bf16 on gfx950 MFMA.
//
// For each sample i and head h: O = softmax(Q_i K_i^T / sqrt(d)) V_i over the
// sample's own tokens (text and image jointly, no mask inside a sample), and
// lse = ln sum exp(scores). The block-diagonal structure over the per-sample
// cumulative offsets is what the Mage-Flow pages obtain from FlashAttention's
// variable-length kernels (picx.dev summary "Mage-Flow: An Efficient
// Native-Resolution Foundation Model ...", section "Native-Resolution MMDiT
// (NR-MMDiT)"; findtube.ai transcript at [00:03:16]). This kernel is its own
// design for CDNA4, not a port:
//
//  * one workgroup = 4 waves = one 128-query tile of one sample and one head,
//    taken from the plan's longest-first work list;
//  * every wave owns 32 queries and computes the TRANSPOSED scores
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so each lane holds one query's
//    scores: the row max and row sum are in-lane plus one permlane32 swap;
//  * the probabilities P^T stay in registers and feed O^T += V^T P^T directly
//    as the B operand (no LDS round trip); V^T fragments come from LDS with
//    ds_read_b64_tr_b16, in the key order the score accumulator uses;
//  * K/V tiles of 64 keys are double-buffered in LDS; only the last tile of a
//    segment is masked;
//  * online softmax in fp32 in the exp2 domain, with the running reference max
//    only moved when a new score exceeds it by more than 8 (log2 units), so
//    the O^T rescale is rare and the result is unchanged.
#include "device.h"
#include "internal.h"

namespace mmdit {

namespace fwd {
constexpr int BM = 128;            // queries per workgroup (= kFwdTile)
constexpr int BN = 64;             // keys per iteration
// LDS row strides (elements past d), chosen by measured LDS throughput on
// gfx950: K rows are read 16 B per lane down 32 consecutive rows (a 272-byte
// stride is conflict-free), V is read with ds_read_b64_tr_b16 in 4x16 blocks
// (a 320-byte stride is fastest).
constexpr int PAD_K = 8;
constexpr int PAD_V = 32;
constexpr float kRescaleThreshold = 8.0f;
}  // namespace fwd

static_assert(fwd::BM == kFwdTile, "forward tile must match the plan");

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(PlanDev p, AttnFwdArgs a) {
  using namespace fwd;
  constexpr int KS = D / 16;       // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int LDK = D + PAD_K;   // LDS row strides (elements)
  constexpr int LDV = D + PAD_V;
  constexpr int CHUNKS = BN * D / 8 / 256;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) bf16 k_s[2][BN * LDK];
  __shared__ __attribute__((aligned(16))) bf16 v_s[2][BN * LDV];

  const int H = p.num_heads;
  const int item = blockIdx.x / H, h = blockIdx.x % H;
  const int4 it = p.fwd_items[item];
  const int seg0 = it.x, seg1 = it.y, q0 = it.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, g = lane >> 5;
  const int64_t HD = (int64_t)H * D;
  const bf16 *qh = static_cast<const bf16 *>(a.q_hat);
  const bf16 *kh = static_cast<const bf16 *>(a.k_hat);
  const bf16 *vv = static_cast<const bf16 *>(a.v);

  // Q^T as the B operand: lane holds query q0 + 32*wave + lq, d = 16s + 8g + 0..7.
  const int qi = q0 + wave * 32 + lq;
  const int qc = min(qi, seg1 - 1);
  bf16x8 qf[KS];
  {
    const bf16 *src = qh + (int64_t)qc * HD + h * D + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = as_bf16x8(ld16(src + 16 * s));
  }

  // Global -> register staging of one K/V tile. Thread tid moves 16-byte
  // chunk c8 of rows r0 + RSTEP*c; rows are clamped into the segment only in
  // its last tile.
  constexpr int RSTEP = 256 / (D / 8);
  const int r0 = tid / (D / 8), c8 = tid % (D / 8);
  const bf16 *kbase = kh + (int64_t)r0 * HD + h * D + 8 * c8;
  const bf16 *vbase = vv + (int64_t)r0 * a.v_stride + h * D + 8 * c8;
  uint4 kreg[CHUNKS], vreg[CHUNKS];
  auto load_tile = [&](int kb0) {
    if (kb0 + BN <= seg1) {
      const bf16 *kp = kbase + (int64_t)kb0 * HD;
      const bf16 *vp = vbase + (int64_t)kb0 * a.v_stride;
#pragma unroll
      for (int c = 0; c < CHUNKS; ++c) {
        kreg[c] = ld16(kp + (int64_t)(RSTEP * c) * HD);
        vreg[c] = ld16(vp + (int64_t)(RSTEP * c) * a.v_stride);
      }
    } else {
#pragma unroll
      for (int c = 0; c < CHUNKS; ++c) {
        const int key = min(kb0 + r0 + RSTEP * c, seg1 - 1);
        kreg[c] = ld16(kh + (int64_t)key * HD + h * D + 8 * c8);
        vreg[c] = ld16(vv + (int64_t)key * a.v_stride + h * D + 8 * c8);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      st16(&k_s[buf][(r0 + RSTEP * c) * LDK + 8 * c8], kreg[c]);
      st16(&v_s[buf][(r0 + RSTEP * c) * LDV + 8 * c8], vreg[c]);
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
  float m_ref = -INFINITY, l_part = 0.f;
  const float c2 = a.scale_log2;

  const int ntiles = (seg1 - seg0 + BN - 1) / BN;
  load_tile(seg0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const int kb0 = seg0 + j * BN;
    if (j + 1 < ntiles) load_tile(kb0 + BN);
    const bf16 *Ks = k_s[buf];
    const bf16 *Vs = v_s[buf];

    // S^T = K Q^T : two 32-key blocks.
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 kf = as_bf16x8(ld16(&Ks[(kb * 32 + lq) * LDK + 16 * ks + 8 * g]));
        s[kb] = mfma32(kf, qf[ks], s[kb]);
      }
    }
    // Mask keys past the segment end (only the last tile has any).
    if (kb0 + BN > seg1) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb0 + kb * 32 + acc_row(i, g) >= seg1) s[kb][i] = -INFINITY;
    }
    // Online softmax (exp2 domain).
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = half_max(mx) * c2;
    if (__ballot(mx > m_ref + kRescaleThreshold)) {
      const float mn = fmaxf(m_ref, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);
      l_part *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[b][i] *= alpha;
      m_ref = mn;
    }
    bf16x8 pf[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -m_ref));
        s[kb][i] = e;
        l_part += e;
      }
      pf[2 * kb] = acc_to_bf16(s[kb], 0);
      pf[2 * kb + 1] = acc_to_bf16(s[kb], 8);
    }
    // O^T += V^T P^T : 16 keys per MFMA.
#pragma unroll
    for (int t = 0; t < BN / 16; ++t)
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        bf16x8 vf = lds_read_tr(Vs, LDV, t * 16, b * 32, lane);
        o[b] = mfma32(vf, pf[t], o[b]);
      }

    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: normalise, store O (rows inside the segment) and lse.
  const float l = half_sum(l_part);
  const float inv = 1.0f / l;
  if (qi < seg1) {
    bf16 *dst = static_cast<bf16 *>(a.o) + (int64_t)qi * HD + h * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v4;
        bf16x2 t0 = pack2(o[b][4 * r4 + 0] * inv, o[b][4 * r4 + 1] * inv);
        bf16x2 t1 = pack2(o[b][4 * r4 + 2] * inv, o[b][4 * r4 + 3] * inv);
        v4[0] = t0[0]; v4[1] = t0[1]; v4[2] = t1[0]; v4[3] = t1[1];
        *reinterpret_cast<bf16x4 *>(dst + b * 32 + 8 * r4 + 4 * g) = v4;
      }
    if (a.lse && g == 0)
      a.lse[(int64_t)h * p.total_tokens + qi] = (m_ref + __log2f(l)) * 0.69314718055994531f;
  }
}

hipError_t launch_attn_fwd_f32(const PlanDev &p, const AttnFwdArgs &a, hipStream_t stream);

template <int D>
static hipError_t attn_fwd_bf16(const PlanDev &p, const AttnFwdArgs &a, hipStream_t s) {
  const int64_t blocks = (int64_t)p.num_fwd_items * p.num_heads;
  hipLaunchKernelGGL(attn_fwd_bf16_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, s, p, a);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(int dtype, const PlanDev &p, const AttnFwdArgs &a, hipStream_t stream) {
  if (dtype == MMDIT_F32) return launch_attn_fwd_f32(p, a, stream);
  if (p.head_dim == 64) return attn_fwd_bf16<64>(p, a, stream);
  if (p.head_dim == 128) return attn_fwd_bf16<128>(p, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace mmdit
