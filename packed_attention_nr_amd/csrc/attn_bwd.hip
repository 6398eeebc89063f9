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
// Two kernels, neither using atomics:
//  * dQ kernel (query-tile items, like the forward): each wave owns 32
//    queries and forms S^T = K Q^T and dP^T = V dO^T with one query per lane,
//    so P^T and dS^T are per-lane and dS^T feeds dQ^T += K^T dS^T as the B
//    operand straight from registers; K^T fragments are read transposed from
//    LDS (ds_read_b64_tr_b16). It also computes and stores D for its queries.
//  * dK/dV kernel (key-tile items): each wave owns 32 keys with K and V rows
//    held in registers, loops over the sample's queries 64 at a time, forms
//    S = Q K^T and dP = dO V^T with one key per lane, and accumulates
//    dV^T += dO^T P and dK^T += Q^T dS with P and dS as B operands from
//    registers and dO^T / Q^T read transposed from LDS.
// dQ is recomputed rather than accumulated across key tiles: device-wide
// fp32 atomics from eight XCDs cost far more than the extra S and dP products.
#include "device.h"
#include "internal.h"

namespace mmdit {

namespace bwd {
constexpr int NWQ = 8;    // waves of a dQ workgroup
constexpr int QT = 32 * NWQ;  // queries per dQ workgroup (= kFwdTileBf16)
constexpr int KT = 128;   // keys per dK/dV workgroup (= kBwdTile)
constexpr int BN = 64;    // keys per dQ iteration
constexpr int BMQ = 64;   // queries per dK/dV iteration
// LDS row strides (elements past d), by measured gfx950 LDS throughput: tiles
// read only 16 B per lane down consecutive rows use a 272-byte stride; tiles
// also read with ds_read_b64_tr_b16 use 304 bytes, fast for both patterns.
constexpr int PAD_ROWS = 8;
constexpr int PAD_BOTH = 24;
constexpr float kLog2e = 1.4426950408889634f;
}  // namespace bwd

static_assert(bwd::QT == kFwdTileBf16 && bwd::KT == kBwdTile, "backward tiles must match the plan");

// ---------------------------------------------------------------------------
// dQ-hat (and D) for one 256-query tile of one sample and head.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * bwd::NWQ, 1) void attn_bwd_dq_kernel(PlanDev p, AttnBwdArgs a) {
  using namespace bwd;
  constexpr int NT = 64 * NWQ;        // threads
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int LDK = D + PAD_BOTH;   // K: row reads and transposed reads
  constexpr int LDV = D + PAD_ROWS;   // V: row reads only
  constexpr int CHUNKS = BN * D / 8 / NT;
  __shared__ __attribute__((aligned(16))) bf16 k_s[2][BN * LDK];
  __shared__ __attribute__((aligned(16))) bf16 v_s[2][BN * LDV];

  const int H = p.num_heads;
  const int N = p.total_tokens;
  const int2 wb = p.fwd_blocks[blockIdx.x];
  if (wb.x < 0) return;  // idle slot of the block map (whole workgroup)
  const int h = wb.y;
  const int4 it = p.fwd_items[wb.x];
  const int seg0 = it.x, seg1 = it.y, q0 = it.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, g = lane >> 5;
  const int64_t HD = (int64_t)H * D;
  const bf16 *qh = static_cast<const bf16 *>(a.q_hat);
  const bf16 *kh = static_cast<const bf16 *>(a.k_hat);
  const bf16 *vv = static_cast<const bf16 *>(a.v);
  const bf16 *go = static_cast<const bf16 *>(a.dout);
  const bf16 *oo = static_cast<const bf16 *>(a.o);
  const float c2 = a.scale_log2;

  // This lane's query: Q-hat and dO rows as B operands (d = 16s + 8g + 0..7).
  const int qi = q0 + wave * 32 + lq;
  const int qc = min(qi, seg1 - 1);
  bf16x8 qf[KS], gf[KS];
  float dlt = 0.f;
  {
    const bf16 *qs = qh + (int64_t)qc * HD + h * D + 8 * g;
    const bf16 *gs = go + (int64_t)qc * a.dout_stride + h * D + 8 * g;
    const bf16 *os = oo + (int64_t)qc * HD + h * D + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = as_bf16x8(ld16(qs + 16 * s));
      gf[s] = as_bf16x8(ld16(gs + 16 * s));
      const bf16x8 of = as_bf16x8(ld16(os + 16 * s));
#pragma unroll
      for (int j = 0; j < 8; ++j) dlt = fmaf((float)gf[s][j], (float)of[j], dlt);
    }
    dlt = half_sum(dlt);
  }
  if (g == 0 && qi < seg1) a.delta[(int64_t)h * N + qi] = dlt;
  const float lse2 = a.lse[(int64_t)h * N + qc] * kLog2e;

  // K/V tile staging: thread tid moves 16-byte chunk c8 of rows r0 + RSTEP*c;
  // rows clamped only in the segment's last tile.
  constexpr int RSTEP = NT / (D / 8);
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

  f32x16 dq[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[b][i] = 0.f;

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
    bf16x8 dsf[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = as_bf16x8(ld16(&Ks[(kb * 32 + lq) * LDK + 16 * ks + 8 * g]));
        const bf16x8 vf = as_bf16x8(ld16(&Vs[(kb * 32 + lq) * LDV + 16 * ks + 8 * g]));
        s = mfma32(kf, qf[ks], s);
        dp = mfma32(vf, gf[ks], dp);
      }
      // Keys past the segment end (last tile only): score -inf, so P = dS = 0.
      if (kb0 + kb * 32 + 32 > seg1) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb0 + kb * 32 + acc_row(i, g) >= seg1) s[i] = -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lse2));
        s[i] = pv * (dp[i] - dlt);
      }
      dsf[2 * kb] = acc_to_bf16(s, 0);
      dsf[2 * kb + 1] = acc_to_bf16(s, 8);
    }
    // dQ^T += K^T dS^T (keys as the k dimension).
#pragma unroll
    for (int t = 0; t < BN / 16; ++t)
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const bf16x8 kt = lds_read_tr(Ks, LDK, t * 16, b * 32, lane);
        dq[b] = mfma32(kt, dsf[t], dq[b]);
      }
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // dQ-hat row of this lane's query: register i of block b is d = 32b + acc_row(i, g).
  if (qi < seg1) {
    float *dst = a.dq_acc + (int64_t)qi * HD + h * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4 *>(dst + b * 32 + 8 * r4 + 4 * g) =
            make_float4(dq[b][4 * r4] * a.scale, dq[b][4 * r4 + 1] * a.scale,
                        dq[b][4 * r4 + 2] * a.scale, dq[b][4 * r4 + 3] * a.scale);
  }
}

// ---------------------------------------------------------------------------
// dK-hat and dV for one 128-key tile of one sample and head.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(PlanDev p, AttnBwdArgs a) {
  using namespace bwd;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int QB = BMQ / 32;
  constexpr int LD = D + PAD_BOTH;    // Q-hat and dO: row reads and transposed reads
  constexpr int QCH = BMQ * D / 8 / 256;
  __shared__ __attribute__((aligned(16))) bf16 q_s[2][BMQ * LD];
  __shared__ __attribute__((aligned(16))) bf16 g_s[2][BMQ * LD];
  __shared__ float lse_s[2][BMQ], dlt_s[2][BMQ];

  const int H = p.num_heads;
  const int N = p.total_tokens;
  const int2 wb = p.bwd_blocks[blockIdx.x];
  if (wb.x < 0) return;  // idle slot of the block map (whole workgroup)
  const int h = wb.y;
  const int4 it = p.bwd_items[wb.x];
  const int seg0 = it.x, seg1 = it.y, k0 = it.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, g = lane >> 5;
  const int64_t HD = (int64_t)H * D;
  const bf16 *qh = static_cast<const bf16 *>(a.q_hat);
  const bf16 *kh = static_cast<const bf16 *>(a.k_hat);
  const bf16 *vv = static_cast<const bf16 *>(a.v);
  const bf16 *go = static_cast<const bf16 *>(a.dout);
  const float c2 = a.scale_log2;

  // This lane's key: K-hat and V rows as B operands.
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

  // Q-hat / dO tile staging: thread tid moves chunk c8 of rows r0 + RSTEP*c;
  // rows clamped into the segment only in its last tile.
  constexpr int RSTEP = 256 / (D / 8);
  const int r0 = tid / (D / 8), c8 = tid % (D / 8);
  const bf16 *qbase = qh + (int64_t)r0 * HD + h * D + 8 * c8;
  const bf16 *gbase = go + (int64_t)r0 * a.dout_stride + h * D + 8 * c8;
  uint4 qreg[QCH], greg[QCH];
  float lreg = 0.f, dreg = 0.f;
  auto load_q = [&](int qb0) {
    if (qb0 + BMQ <= seg1) {
      const bf16 *qp = qbase + (int64_t)qb0 * HD;
      const bf16 *gp = gbase + (int64_t)qb0 * a.dout_stride;
#pragma unroll
      for (int c = 0; c < QCH; ++c) {
        qreg[c] = ld16(qp + (int64_t)(RSTEP * c) * HD);
        greg[c] = ld16(gp + (int64_t)(RSTEP * c) * a.dout_stride);
      }
    } else {
#pragma unroll
      for (int c = 0; c < QCH; ++c) {
        const int qq = min(qb0 + r0 + RSTEP * c, seg1 - 1);
        qreg[c] = ld16(qh + (int64_t)qq * HD + h * D + 8 * c8);
        greg[c] = ld16(go + (int64_t)qq * a.dout_stride + h * D + 8 * c8);
      }
    }
    if (tid < BMQ) {
      const int qq = qb0 + tid;
      const bool ok = qq < seg1;
      const int qcl = min(qq, seg1 - 1);
      // Queries past the segment end get lse = +inf, so their P is exactly 0.
      lreg = ok ? a.lse[(int64_t)h * N + qcl] * kLog2e : INFINITY;
      dreg = a.delta[(int64_t)h * N + qcl];
    }
  };
  auto store_q = [&](int buf) {
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      st16(&q_s[buf][(r0 + RSTEP * c) * LD + 8 * c8], qreg[c]);
      st16(&g_s[buf][(r0 + RSTEP * c) * LD + 8 * c8], greg[c]);
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

    bf16x8 pb[BMQ / 16], db[BMQ / 16];   // P and dS as B operands (16 queries each)
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
        const bf16x8 qa = as_bf16x8(ld16(&Qs[(qb * 32 + lq) * LD + 16 * ks + 8 * g]));
        const bf16x8 ga = as_bf16x8(ld16(&Gs[(qb * 32 + lq) * LD + 16 * ks + 8 * g]));
        s = mfma32(qa, kf[ks], s);
        dp = mfma32(ga, vf[ks], dp);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ql = qb * 32 + acc_row(i, g);
        // Keys past the segment end only feed their own dK/dV rows, which are
        // never stored: no mask needed here.
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lse_s[buf][ql]));
        s[i] = pv;
        dp[i] = pv * (dp[i] - dlt_s[buf][ql]);
      }
      pb[2 * qb] = acc_to_bf16(s, 0);
      pb[2 * qb + 1] = acc_to_bf16(s, 8);
      db[2 * qb] = acc_to_bf16(dp, 0);
      db[2 * qb + 1] = acc_to_bf16(dp, 8);
    }
    // dV^T += dO^T P, dK^T += Q^T dS (queries as the k dimension).
#pragma unroll
    for (int t = 0; t < BMQ / 16; ++t)
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const bf16x8 gt = lds_read_tr(Gs, LD, t * 16, b * 32, lane);
        dv[b] = mfma32(gt, pb[t], dv[b]);
        const bf16x8 qt = lds_read_tr(Qs, LD, t * 16, b * 32, lane);
        dk[b] = mfma32(qt, db[t], dk[b]);
      }
    if (itq + 1 < nit) store_q(buf ^ 1);
    __syncthreads();
  }

  // Rows of this lane's key: register i of block b is d = 32b + acc_row(i, g).
  if (key_ok) {
    const int64_t off = (int64_t)kr * HD + h * D;
    bf16 *dvp = static_cast<bf16 *>(a.dv) + off;
    float *dkp = a.dk_acc + off;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int e = b * 32 + 8 * r4 + 4 * g;
        bf16x4 v4;
        const bf16x2 t0 = pack2(dv[b][4 * r4], dv[b][4 * r4 + 1]);
        const bf16x2 t1 = pack2(dv[b][4 * r4 + 2], dv[b][4 * r4 + 3]);
        v4[0] = t0[0]; v4[1] = t0[1]; v4[2] = t1[0]; v4[3] = t1[1];
        *reinterpret_cast<bf16x4 *>(dvp + e) = v4;
        *reinterpret_cast<float4 *>(dkp + e) =
            make_float4(dk[b][4 * r4] * a.scale, dk[b][4 * r4 + 1] * a.scale,
                        dk[b][4 * r4 + 2] * a.scale, dk[b][4 * r4 + 3] * a.scale);
      }
  }
}

hipError_t launch_attn_bwd_f32(const PlanDev &p, const AttnBwdArgs &a, int which, hipStream_t stream);

template <int D>
static hipError_t bwd_dq(const PlanDev &p, const AttnBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3((unsigned)p.num_fwd_blocks), dim3(64 * bwd::NWQ), 0, s, p, a);
  return hipGetLastError();
}
template <int D>
static hipError_t bwd_dkdv(const PlanDev &p, const AttnBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, dim3((unsigned)p.num_bwd_blocks), dim3(256), 0, s, p, a);
  return hipGetLastError();
}

// which = 0: dQ-hat and D; which = 1: dK-hat and dV (reads D).
hipError_t launch_attn_bwd(int dtype, const PlanDev &p, const AttnBwdArgs &a, int which,
                           hipStream_t stream) {
  if (dtype == MMDIT_F32) return launch_attn_bwd_f32(p, a, which, stream);
  if (p.head_dim == 64) return which == 0 ? bwd_dq<64>(p, a, stream) : bwd_dkdv<64>(p, a, stream);
  if (p.head_dim == 128) return which == 0 ? bwd_dq<128>(p, a, stream) : bwd_dkdv<128>(p, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace mmdit
