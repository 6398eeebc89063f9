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
//  * dK/dV kernel (key-tile items): 128 keys per workgroup, split over two
//    wave roles that share P through LDS (one holds K rows and produces P and
//    dV, the other holds V rows and produces dS and dK); they loop over the
//    sample's queries 64 at a time with one key per lane, forming S = Q K^T
//    and dP = dO V^T and accumulating dV^T += dO^T P and dK^T += Q^T dS with
//    P and dS as B operands from registers and dO^T / Q^T read transposed
//    from a ring of LDS tiles filled by direct global->LDS loads.
// dQ is recomputed rather than accumulated across key tiles: device-wide
// fp32 atomics from eight XCDs cost far more than the extra S and dP products.
#include <type_traits>

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
      qf[s] = ld_bf16x8(qs + 16 * s);
      gf[s] = ld_bf16x8(gs + 16 * s);
      const bf16x8 of = ld_bf16x8(os + 16 * s);
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
        const bf16x8 kf = ld_bf16x8(&Ks[(kb * 32 + lq) * LDK + 16 * ks + 8 * g]);
        const bf16x8 vf = ld_bf16x8(&Vs[(kb * 32 + lq) * LDV + 16 * ks + 8 * g]);
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
//
// Eight waves in two roles, paired per SIMD (wave w and w+4 share keys
// 32*(w%4)..+31 and, by the round-robin wave placement, one SIMD):
//  * P/dV waves hold their 32 K-hat rows as B operands, form S = Q K^T and
//    P = exp2(S*c - lse2) for a 64-query tile, publish P (bf16, in the MFMA
//    accumulator order) through LDS and accumulate dV^T += dO^T P;
//  * dS/dK waves hold their 32 V rows, form dP = dO V^T, read P back, form
//    dS = P * (dP - D) and accumulate dK^T += Q^T dS.
// Each tile takes two phases between workgroup barriers; in each phase one
// role issues matrix instructions while the other does its vector work:
//   phase 1: P/dV waves: softmax(t) -> P(t) to LDS
//            dS/dK waves: dK(t-1), dP(t)
//   phase 2: P/dV waves: dV(t), S(t+1)
//            dS/dK waves: dS(t) (reads P(t)); load tile t+3
// Q-hat / dO tiles, lse and D come by direct global->LDS loads into a
// 4-stage ring; tile t+3 reuses the stage of tile t-1, whose last reader
// (dK(t-1)) ran before the barrier that opens phase 2 of tile t. Each wave
// waits for its own loads of tile t+1 before that barrier, so tile t+1 is
// visible one phase before S(t+1) reads it.
// ---------------------------------------------------------------------------
namespace bwd {
constexpr int KV_NW = 8;   // waves of a dK/dV workgroup
constexpr int KV_NS = 4;   // Q-hat / dO ring stages
}  // namespace bwd

template <int D>
__global__ __launch_bounds__(64 * bwd::KV_NW, 1) void attn_bwd_dkdv_kernel(PlanDev p, AttnBwdArgs a) {
  using namespace bwd;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BMQ * D;
  static_assert(KV_NS == 4 && BMQ == 64 && KT == 32 * KV_NW / 2, "layout below");
  // One LDS object per ring stage, [Q-hat tile | dO tile | lse | D]: distinct
  // objects (at most 8 of them receiving direct loads) let the compiler prove
  // that loads into one stage do not alias reads of another.
  constexpr int STAGE = 2 * TILE + 4 * BMQ;  // bf16 elements
  __shared__ __attribute__((aligned(16))) bf16 st0[STAGE], st1[STAGE], st2[STAGE], st3[STAGE];
  __shared__ __attribute__((aligned(16))) uint4 p_s[4 * (BMQ / 16) * 64];
  auto stg = [&](auto stage) __attribute__((always_inline)) -> bf16 * {
    constexpr int S = decltype(stage)::value;
    if constexpr (S == 0) return st0; else if constexpr (S == 1) return st1;
    else if constexpr (S == 2) return st2; else return st3;
  };
  auto qst = [&](auto stage) __attribute__((always_inline)) -> bf16 * { return stg(stage); };
  auto gst = [&](auto stage) __attribute__((always_inline)) -> bf16 * { return stg(stage) + TILE; };
  auto lst = [&](auto stage) __attribute__((always_inline)) -> float * {
    return reinterpret_cast<float *>(stg(stage) + 2 * TILE);
  };
  auto dst = [&](auto stage) __attribute__((always_inline)) -> float * {
    return reinterpret_cast<float *>(stg(stage) + 2 * TILE) + BMQ;
  };

  const int H = p.num_heads;
  const int N = p.total_tokens;
  const int2 wb = p.bwd_blocks[blockIdx.x];
  if (wb.x < 0) return;  // idle slot of the block map (whole workgroup)
  const int h = wb.y;
  const int4 it = p.bwd_items[wb.x];
  const int seg0 = it.x, seg1 = it.y, k0 = it.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform to the compiler
  const int role = wave >> 2, sub = wave & 3;  // role 0: P/dV, role 1: dS/dK
  const int lq = lane & 31, g = lane >> 5;
  const int64_t HD = (int64_t)H * D;
  const int64_t gstride = a.dout_stride;
  const bf16 *qh = static_cast<const bf16 *>(a.q_hat) + h * D;
  const bf16 *go = static_cast<const bf16 *>(a.dout) + h * D;
  const float *lse_h = a.lse + (int64_t)h * N;
  const float *dlt_h = a.delta + (int64_t)h * N;
  const float c2 = a.scale_log2;

  // This lane's key: its K-hat row (P/dV role) or V row (dS/dK role) as a
  // B operand.
  const int kr = k0 + sub * 32 + lq;
  const bool key_ok = kr < seg1;
  const int kc = min(kr, seg1 - 1);
  bf16x8 kv[KS];
  {
    const bf16 *src = role == 0 ? static_cast<const bf16 *>(a.k_hat) + (int64_t)kc * HD + h * D
                                : static_cast<const bf16 *>(a.v) + (int64_t)kc * a.v_stride + h * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) kv[s] = ld_bf16x8(src + 16 * s + 8 * g);
  }

  const int ntq = (seg1 - seg0 + BMQ - 1) / BMQ;
  TileLoader<D, SWZ_ROWS, BMQ, KV_NW> qload, gload;
  qload.init(wave, lane);
  gload.init(wave, lane);
  constexpr int LQ = TileLoader<D, SWZ_ROWS, BMQ, KV_NW>::LOADS;
  // Tile t -> ring stage; even waves also load lse and odd waves D (the same
  // words from four waves each, so every wave issues the same number of loads
  // per tile). Rows past the segment end are clamped to its last row; their P
  // is zeroed.
  const float *ld_src = (wave & 1) ? dlt_h : lse_h;
  // Every step issues one tile's loads, so the compiler's in-order count of
  // outstanding loads is exact; past the last tile the last tile is loaded
  // again into the stage just freed, which nothing reads afterwards.
  auto issue = [&](auto stage, int t) __attribute__((always_inline)) {
    const int qb0 = seg0 + min(t, ntq - 1) * BMQ;
    qload.issue_clamped(qst(stage), qh, HD, qb0, seg1 - 1);  // branch-free: exact load counts
    gload.issue_clamped(gst(stage), go, gstride, qb0, seg1 - 1);
    g2lds4(ld_src + min(qb0 + lane, seg1 - 1), lst(stage) + (wave & 1) * BMQ);
  };
  constexpr int PER_TILE = 2 * LQ + 1;  // loads per wave per tile

  f32x16 acc[DB];  // dV^T (role 0) or dK^T (role 1): lane = key, rows = d
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
  f32x16 s[2];     // S (role 0) or dP (role 1) of 64 queries x this lane's key
  bf16x8 pb[BMQ / 16];  // P (role 0) or dS (role 1) as B operands, 16 queries each
  uint4 *p_mine = p_s + sub * (BMQ / 16) * 64 + lane;

  // Row products with this lane's key: s[qb] = rows(qb) . kv (Q-hat rows for
  // role 0, dO rows for role 1).
  auto rows_x_key = [&](const bf16 *T) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[qb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ra = ld_bf16x8(&T[swz_off<D, SWZ_ROWS>(qb * 32 + lq, 16 * ks + 8 * g)]);
        s[qb] = mfma32(ra, kv[ks], s[qb]);
      }
    }
  };
  // acc^T += T^T pb (dO^T P for role 0, Q-hat^T dS for role 1).
  auto accumulate = [&](const bf16 *T) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < BMQ / 16; ++u)
#pragma unroll
      for (int b = 0; b < DB; ++b)
        acc[b] = mfma32(lds_read_tr_swz<D, SWZ_ROWS>(T, u * 16, b * 32, lane), pb[u], acc[b]);
  };
  // Role 0: P = exp2(S*c2 - lse*log2e), zero for queries past the segment.
  auto softmax = [&](const float *Ls, int t) __attribute__((always_inline)) {
    const int qb0 = seg0 + t * BMQ;
    const bool tail = qb0 + BMQ > seg1;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&Ls[qb * 32 + 8 * r4 + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * r4 + j;
          float pv = __builtin_amdgcn_exp2f(fmaf(s[qb][i], c2, -l4[j] * kLog2e));
          if (tail && qb0 + qb * 32 + acc_row(i, g) >= seg1) pv = 0.f;
          s[qb][i] = pv;
        }
      }
      pb[2 * qb] = acc_to_bf16(s[qb], 0);
      pb[2 * qb + 1] = acc_to_bf16(s[qb], 8);
    }
#pragma unroll
    for (int u = 0; u < BMQ / 16; ++u) st_bf16x8(p_mine + u * 64, pb[u]);
  };
  // Role 1: dS = P * (dP - D) with P read back from the paired wave.
  auto dscores = [&](const float *Ds) __attribute__((always_inline)) {
    bf16x8 pr[BMQ / 16];
#pragma unroll
    for (int u = 0; u < BMQ / 16; ++u) pr[u] = ld_bf16x8(p_mine + u * 64);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&Ds[qb * 32 + 8 * r4 + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * r4 + j;
          const float pv = (float)pr[2 * qb + i / 8][i % 8];
          s[qb][i] = pv * (s[qb][i] - d4[j]);
        }
      }
      pb[2 * qb] = acc_to_bf16(s[qb], 0);
      pb[2 * qb + 1] = acc_to_bf16(s[qb], 8);
    }
  };

  using S0 = std::integral_constant<int, 0>;
  issue(S0{}, 0);
  issue(std::integral_constant<int, 1>{}, 1);
  issue(std::integral_constant<int, 2>{}, 2);
  wait_vmem_le<2 * PER_TILE>();  // this wave's loads of tile 0
  phase_barrier();  // tile 0 visible

  // Both roles run the same whole number of 4-step groups (every step loads,
  // waits and passes two barriers; work is skipped past the last tile), so the
  // loop has a single exit and barrier counts match across roles.
  if (role == 0) {
    rows_x_key(qst(S0{}));  // S(0)
    auto step = [&](auto stage, int t) __attribute__((always_inline)) {
      constexpr int SG = decltype(stage)::value;
      if (t < ntq) softmax(lst(stage), t);
      wait_vmem_le<PER_TILE>();  // this wave's loads of tile t+1
      phase_barrier();  // P(t) and tile t+1 visible
      issue(std::integral_constant<int, (SG + 3) % KV_NS>{}, t + 3);
      if (t < ntq) {
        accumulate(gst(stage));  // dV(t)
        if (t + 1 < ntq) rows_x_key(qst(std::integral_constant<int, (SG + 1) % KV_NS>{}));  // S(t+1)
      }
      phase_barrier();  // P(t) consumed
    };
    for (int t = 0; t < ntq; t += KV_NS) {
      step(S0{}, t);
      step(std::integral_constant<int, 1>{}, t + 1);
      step(std::integral_constant<int, 2>{}, t + 2);
      step(std::integral_constant<int, 3>{}, t + 3);
    }
  } else {
    auto step = [&](auto stage, int t) __attribute__((always_inline)) {
      constexpr int SG = decltype(stage)::value;
      if (t < ntq) {
        if (t > 0) accumulate(qst(std::integral_constant<int, (SG + 3) % KV_NS>{}));  // dK(t-1)
        rows_x_key(gst(stage));  // dP(t)
      }
      wait_vmem_le<PER_TILE>();  // this wave's loads of tile t+1
      phase_barrier();  // P(t) and tile t+1 visible
      issue(std::integral_constant<int, (SG + 3) % KV_NS>{}, t + 3);
      if (t < ntq) {
        dscores(dst(stage));  // dS(t)
        if (t + 1 == ntq) accumulate(qst(stage));  // last dK
      }
      phase_barrier();  // P(t) consumed
    };
    for (int t = 0; t < ntq; t += KV_NS) {
      step(S0{}, t);
      step(std::integral_constant<int, 1>{}, t + 1);
      step(std::integral_constant<int, 2>{}, t + 2);
      step(std::integral_constant<int, 3>{}, t + 3);
    }
  }

  wait_vmem();  // no load into LDS may outlive the workgroup

  // Rows of this lane's key: register i of block b is d = 32b + acc_row(i, g).
  if (key_ok) {
    const int64_t off = (int64_t)kr * HD + h * D;
    if (role == 0) {
      bf16 *dvp = static_cast<bf16 *>(a.dv) + off;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 v4;
          const bf16x2 t0 = pack2(acc[b][4 * r4], acc[b][4 * r4 + 1]);
          const bf16x2 t1 = pack2(acc[b][4 * r4 + 2], acc[b][4 * r4 + 3]);
          v4[0] = t0[0]; v4[1] = t0[1]; v4[2] = t1[0]; v4[3] = t1[1];
          *reinterpret_cast<bf16x4 *>(dvp + b * 32 + 8 * r4 + 4 * g) = v4;
        }
    } else {
      float *dkp = a.dk_acc + off;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<float4 *>(dkp + b * 32 + 8 * r4 + 4 * g) =
              make_float4(acc[b][4 * r4] * a.scale, acc[b][4 * r4 + 1] * a.scale,
                          acc[b][4 * r4 + 2] * a.scale, acc[b][4 * r4 + 3] * a.scale);
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
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, dim3((unsigned)p.num_bwd_blocks), dim3(64 * bwd::KV_NW), 0, s, p, a);
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
