// Variable-length joint attention, backward, bf16 on gfx950 MFMA.
//
// Gradients of sum(dO * O) for O = softmax(Q K^T / sqrt(d)) V per sample and
// head (the attention of picx.dev "Mage-Flow: An Efficient Native-Resolution
// Foundation Model ...", section "Native-Resolution MMDiT (NR-MMDiT)"; its
// backward is what training through it needs, ibid. "Training
// Infrastructure"). With P recomputed from the forward's lse:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
//
// Design for CDNA4:
//  * one workgroup = 4 waves = one 128-key tile of one sample and one head
//    (plan's longest-first work list); each wave owns 32 keys and keeps its
//    K and V rows in registers as MFMA B operands and its dK, dV accumulators
//    in registers for the whole item;
//  * the loop runs over the sample's queries, 64 at a time, with the Q-hat and
//    dO tiles double-buffered in LDS; S = Q K^T and dP = dO V^T come out with
//    one key per lane, so P and dS feed dV += P^T dO and dK += dS^T Q as A
//    operands straight from registers; the Q/dO operands of those products are
//    read transposed from LDS with ds_read_b64_tr_b16;
//  * dS (bf16) is written to LDS as dS^T and the 64 x d slice of dQ for all
//    128 keys is formed by the 4 waves together, then added to an fp32 dQ
//    accumulator in HBM with atomics (one add per element per key tile);
//  * masking only for keys past the segment end and queries past it in the
//    last query tile.
#include "device.h"
#include "internal.h"

namespace mmdit {

namespace bwd {
constexpr int BN = 128;   // keys per workgroup (= kBwdTile)
constexpr int BMQ = 64;   // queries per iteration
constexpr int PAD = 8;    // LDS row padding (elements)
}  // namespace bwd

static_assert(bwd::BN == kBwdTile, "backward tile must match the plan");

template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_bf16_kernel(PlanDev p, AttnBwdArgs a) {
  using namespace bwd;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int QB = BMQ / 32;
  constexpr int LD = D + PAD;
  constexpr int LDT = BMQ + PAD;
  constexpr int QCH = BMQ * D / 8 / 256;    // 16-byte chunks per thread per Q (or dO) tile
  constexpr int KCH = BN * D / 8 / 256;     // ... per K tile
  constexpr int DQ_BLOCKS = QB * DB / 4;    // dQ output blocks per wave
  __shared__ __attribute__((aligned(16))) bf16 k_s[BN * LD];
  __shared__ __attribute__((aligned(16))) bf16 q_s[2][BMQ * LD];
  __shared__ __attribute__((aligned(16))) bf16 g_s[2][BMQ * LD];
  __shared__ __attribute__((aligned(16))) bf16 dst_s[BN * LDT];
  __shared__ float lse_s[2][BMQ], dlt_s[2][BMQ];

  const int H = p.num_heads;
  const int N = p.total_tokens;
  const int item = blockIdx.x / H, h = blockIdx.x % H;
  const int4 it = p.bwd_items[item];
  const int seg0 = it.x, seg1 = it.y, k0 = it.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, g = lane >> 5;
  const int64_t HD = (int64_t)H * D;
  const bf16 *qh = static_cast<const bf16 *>(a.q_hat);
  const bf16 *kh = static_cast<const bf16 *>(a.k_hat);
  const bf16 *vv = static_cast<const bf16 *>(a.v);
  const bf16 *go = static_cast<const bf16 *>(a.dout);
  constexpr float kLog2e = 1.4426950408889634f;
  const float c2 = a.scale_log2;

  // This lane's key (B operand row of S and dP).
  const int kr = k0 + wave * 32 + lq;
  const bool key_ok = kr < seg1;
  const int kc = min(kr, seg1 - 1);
  bf16x8 kf[KS], vf[KS];
  {
    const bf16 *ks = kh + (int64_t)kc * HD + h * D + 8 * g;
    const bf16 *vs = vv + (int64_t)kc * a.v_stride + h * D + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = as_bf16x8(ld16(ks + 16 * s));
      vf[s] = as_bf16x8(ld16(vs + 16 * s));
    }
  }
  // Whole K tile into LDS for dQ = dS K.
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const int idx = tid + 256 * c;
    const int r = idx / (D / 8), c8 = idx % (D / 8);
    const int key = min(k0 + r, seg1 - 1);
    st16(&k_s[r * LD + 8 * c8], ld16(kh + (int64_t)key * HD + h * D + 8 * c8));
  }

  uint4 qreg[QCH], greg[QCH];
  float lreg = 0.f, dreg = 0.f;
  auto load_q = [&](int qb0) {
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      const int idx = tid + 256 * c;
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      const int qq = min(qb0 + r, seg1 - 1);
      qreg[c] = ld16(qh + (int64_t)qq * HD + h * D + 8 * c8);
      greg[c] = ld16(go + (int64_t)qq * a.dout_stride + h * D + 8 * c8);
    }
    if (tid < BMQ) {
      const int qq = min(qb0 + tid, seg1 - 1);
      lreg = a.lse[(int64_t)h * N + qq] * kLog2e;
      dreg = a.delta[(int64_t)h * N + qq];
    }
  };
  auto store_q = [&](int buf) {
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      const int idx = tid + 256 * c;
      const int r = idx / (D / 8), c8 = idx % (D / 8);
      st16(&q_s[buf][r * LD + 8 * c8], qreg[c]);
      st16(&g_s[buf][r * LD + 8 * c8], greg[c]);
    }
    if (tid < BMQ) {
      lse_s[buf][tid] = lreg;
      dlt_s[buf][tid] = dreg;
    }
  };

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[b][i] = 0.f;
      dv[b][i] = 0.f;
    }

  const int nit = (seg1 - seg0 + BMQ - 1) / BMQ;
  load_q(seg0);
  store_q(0);
  __syncthreads();

  for (int itq = 0; itq < nit; ++itq) {
    const int buf = itq & 1;
    const int qb0 = seg0 + itq * BMQ;
    if (itq + 1 < nit) load_q(qb0 + BMQ);
    const bf16 *Qs = q_s[buf];
    const bf16 *Gs = g_s[buf];

    bf16x8 pa[BMQ / 16], da[BMQ / 16];   // P^T and dS^T as A operands (16 queries each)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 qa = as_bf16x8(ld16(&Qs[(qb * 32 + lq) * LD + 16 * ks + 8 * g]));
        bf16x8 ga = as_bf16x8(ld16(&Gs[(qb * 32 + lq) * LD + 16 * ks + 8 * g]));
        s = mfma32(qa, kf[ks], s);
        dp = mfma32(ga, vf[ks], dp);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ql = qb * 32 + acc_row(i, g);
        const bool ok = key_ok && (qb0 + ql < seg1);
        const float pv = ok ? __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lse_s[buf][ql])) : 0.f;
        s[i] = pv;
        dp[i] = pv * (dp[i] - dlt_s[buf][ql]);
      }
      pa[2 * qb] = acc_to_bf16(s, 0);
      pa[2 * qb + 1] = acc_to_bf16(s, 8);
      da[2 * qb] = acc_to_bf16(dp, 0);
      da[2 * qb + 1] = acc_to_bf16(dp, 8);
      // dS^T rows of this wave's keys, 4 consecutive queries per store.
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v4;
        v4[0] = da[2 * qb + (r4 >> 1)][4 * (r4 & 1) + 0];
        v4[1] = da[2 * qb + (r4 >> 1)][4 * (r4 & 1) + 1];
        v4[2] = da[2 * qb + (r4 >> 1)][4 * (r4 & 1) + 2];
        v4[3] = da[2 * qb + (r4 >> 1)][4 * (r4 & 1) + 3];
        *reinterpret_cast<bf16x4 *>(&dst_s[(wave * 32 + lq) * LDT + qb * 32 + 8 * r4 + 4 * g]) = v4;
      }
    }
    // dV += P^T dO, dK += dS^T Q (queries as the k dimension).
#pragma unroll
    for (int t = 0; t < BMQ / 16; ++t)
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        bf16x8 gb = lds_read_tr(Gs, LD, t * 16, b * 32, lane);
        dv[b] = mfma32(pa[t], gb, dv[b]);
        bf16x8 qbf = lds_read_tr(Qs, LD, t * 16, b * 32, lane);
        dk[b] = mfma32(da[t], qbf, dk[b]);
      }
    __syncthreads();

    // dQ[64 x D] = dS[64 x 128] K[128 x D]: DQ_BLOCKS 32x32 blocks per wave.
#pragma unroll
    for (int ob = 0; ob < DQ_BLOCKS; ++ob) {
      const int blk = wave * DQ_BLOCKS + ob;
      const int qb = blk / DB, b = blk % DB;
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int t = 0; t < BN / 16; ++t) {
        bf16x8 sa = lds_read_tr(dst_s, LDT, t * 16, qb * 32, lane);
        bf16x8 kb = lds_read_tr(k_s, LD, t * 16, b * 32, lane);
        acc = mfma32(sa, kb, acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qg = qb0 + qb * 32 + acc_row(i, g);
        if (qg < seg1)
          unsafeAtomicAdd(a.dq_acc + (int64_t)qg * HD + h * D + b * 32 + lq, acc[i] * a.scale);
      }
    }
    if (itq + 1 < nit) store_q(buf ^ 1);
    __syncthreads();
  }

  // dV (bf16) and dK-hat (fp32, scaled) for the keys inside the segment.
  // Accumulator register i of block b holds key acc_row(i, g), d = 32b + lq.
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = k0 + wave * 32 + acc_row(i, g);
      if (key < seg1) {
        const int64_t off = (int64_t)key * HD + h * D + b * 32 + lq;
        static_cast<bf16 *>(a.dv)[off] = (bf16)dv[b][i];
        a.dk_acc[off] = dk[b][i] * a.scale;
      }
    }
}

hipError_t launch_attn_bwd_f32(const PlanDev &p, const AttnBwdArgs &a, hipStream_t stream);

template <int D>
static hipError_t attn_bwd_bf16(const PlanDev &p, const AttnBwdArgs &a, hipStream_t s) {
  const int64_t blocks = (int64_t)p.num_bwd_items * p.num_heads;
  hipLaunchKernelGGL(attn_bwd_bf16_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, s, p, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(int dtype, const PlanDev &p, const AttnBwdArgs &a, hipStream_t stream) {
  if (dtype == MMDIT_F32) return launch_attn_bwd_f32(p, a, stream);
  if (p.head_dim == 64) return attn_bwd_bf16<64>(p, a, stream);
  if (p.head_dim == 128) return attn_bwd_bf16<128>(p, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace mmdit
