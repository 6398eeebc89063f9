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
//  * one workgroup = 8 waves = one 256-query tile of one sample and one head,
//    taken from the plan's XCD-aware, longest-first block map; two waves per
//    SIMD;
//  * every wave owns 32 queries and computes the TRANSPOSED scores
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so each lane holds one query's
//    scores: the row max and row sum are in-lane plus one permlane32 swap;
//  * the probabilities P^T stay in registers and feed O^T += V^T P^T directly
//    as the B operand (no LDS round trip); V^T fragments come from LDS with
//    ds_read_b64_tr_b16, in the key order the score accumulator uses;
//  * ping-pong: the waves form two groups (one wave of each per SIMD) that run
//    one barrier phase apart. Phase A is matrix work (PV of the previous tile,
//    then QK^T of the current one), phase B is the softmax (vector ALU) plus
//    issuing the loads of the tile two ahead. While one group is in A the other
//    is in B, so the MFMA pipe of each SIMD stays busy during the softmax;
//  * K/V tiles of 64 keys go global -> LDS directly (global_load_lds_dwordx4,
//    no register staging) into a 4-stage ring of unpadded XOR-swizzled tiles;
//    only the last tile of a segment is masked;
//  * online softmax in fp32 in the exp2 domain against a running reference
//    that moves rarely: each tile's P is formed against the current reference
//    and kept when the lane's sum of P stays within a bound (then no P can
//    overflow the accumulators), so the row maxima are formed only on the
//    first tile and on tiles that pass the bound; the result is the same
//    softmax whichever reference it was formed against.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace mmdit {

namespace fwd {
constexpr int NW = 8;              // waves per workgroup
constexpr int BM = 32 * NW;        // queries per workgroup (= kFwdTileBf16)
constexpr int BN = 64;             // keys per tile
constexpr int NS = 4;              // stages of the K/V ring
constexpr float kRescaleThreshold = 8.0f;
constexpr float kSumLimit = 16384.0f;  // per-lane tile sum of P kept without a rescale
}  // namespace fwd

static_assert(fwd::BM == kFwdTileBf16, "forward tile must match the plan");

template <int D>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_kernel(PlanDev p, AttnFwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  using namespace fwd;
  constexpr int KS = D / 16;       // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int TILE = BN * D;
  // One LDS object per ring stage: distinct objects let the compiler prove
  // that a DMA into one stage does not alias reads of another.
  __shared__ __attribute__((aligned(16))) bf16 k0s[TILE], k1s[TILE], k2s[TILE], k3s[TILE];
  __shared__ __attribute__((aligned(16))) bf16 v0s[TILE], v1s[TILE], v2s[TILE], v3s[TILE];
  static_assert(NS == 4, "ring stages are spelled out");
  auto kst = [&](auto stage) __attribute__((always_inline)) -> bf16 * {
    constexpr int SG = decltype(stage)::value;
    if constexpr (SG == 0) return k0s;
    else if constexpr (SG == 1) return k1s;
    else if constexpr (SG == 2) return k2s;
    else return k3s;
  };
  auto vst = [&](auto stage) __attribute__((always_inline)) -> bf16 * {
    constexpr int SG = decltype(stage)::value;
    if constexpr (SG == 0) return v0s;
    else if constexpr (SG == 1) return v1s;
    else if constexpr (SG == 2) return v2s;
    else return v3s;
  };

  const int2 wb = p.fwd_blocks[blockIdx.x];
  if (wb.x < 0) return;  // idle slot of the block map (whole workgroup)
  const int4 it = p.fwd_items[wb.x];
  const int h = wb.y;
  const int seg0 = it.x, seg1 = it.y, q0 = it.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;       // waves w and w+4 share a SIMD
  const int lq = lane & 31, g = lane >> 5;
  const int64_t HD = (int64_t)p.num_heads * D;
  const bf16 *qh = static_cast<const bf16 *>(a.q_hat);
  const bf16 *kh = static_cast<const bf16 *>(a.k_hat) + h * D;
  const bf16 *vv = static_cast<const bf16 *>(a.v) + h * D;
  const int64_t vs = a.v_stride;

  // Q^T as the B operand: lane holds query q0 + 32*wave + lq, d = 16s + 8g + 0..7.
  // The wave's 32 Q-hat rows arrive whole (direct loads of full rows) in ring
  // stages 2 and 3, which the first two tiles leave free; rows past the
  // segment end arrive as zeros (their scores are formed but never stored).
  static_assert(2 * 32 * D == TILE, "two waves' Q-hat rows fill a stage");
  const int qi = q0 + wave * 32 + lq;
  bf16 *const q_stage = (wave < 2 ? k2s : wave < 4 ? k3s : wave < 6 ? v2s : v3s) + (wave & 1) * 32 * D;
  {
    TileLoader<D, SWZ_ROWS, 32, 1> qload;
    qload.init(0, lane, HD);
    qload.issue(q_stage, qh + h * D, q0 + wave * 32, seg1 - 1);
  }
  bf16x8 qf[KS];  // read from q_stage once tiles 0 and 1 are requested

  const int ntiles = (seg1 - seg0 + BN - 1) / BN;
  // Direct global -> LDS loads of tile t into ring stage t % NS (rows past the
  // segment end clamped to its last row; masked later). Every ring access uses
  // a compile-time stage, so the compiler sees that loads into one stage never
  // alias reads of another and adds no waits for them.
  TileLoader<D, SWZ_ROWS, BN, NW> kload;
  TileLoader<D, SWZ_TRANS, BN, NW> vload;
  kload.init(wave, lane, HD);
  vload.init(wave, lane, vs);
  auto issue = [&](auto stage, int t) __attribute__((always_inline)) {
    if (t >= ntiles) return;
    const int kb0 = seg0 + t * BN;
    kload.issue(kst(stage), kh, kb0, seg1 - 1);
    vload.issue(vst(stage), vv, kb0, seg1 - 1);
  };


  f32x16 o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
  float m_ref = -INFINITY, l_part = 0.f;
  const float c2 = a.scale_log2;
  f32x16 s[BN / 32];
  bf16x8 pf[BN / 16];

  // Phase A pieces (matrix work).
  auto scores = [&](auto stage) __attribute__((always_inline)) {  // s = K Q^T from ring stage
    const bf16 *Ks = kst(stage);
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = ld_bf16x8(&Ks[swz_off<D, SWZ_ROWS>(kb * 32 + lq, 16 * ks + 8 * g)]);
        s[kb] = mfma32(kf, qf[ks], s[kb]);
      }
    }
  };
  auto accumulate = [&](auto stage) __attribute__((always_inline)) {  // O^T += V^T P^T from ring stage
    const bf16 *Vs = vst(stage);
#pragma unroll
    for (int u = 0; u < BN / 16; ++u)
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const bf16x8 vf = lds_read_tr_swz<D, SWZ_TRANS>(Vs, u * 16, b * 32, lane);
        o[b] = mfma32(vf, pf[u], o[b]);
      }
  };
  // Phase B piece (vector ALU): online softmax of tile t's scores -> pf.
  // exp_pack forms P = exp2(S c2 - m_ref) into pf and returns the lane's sum
  // of P; the fp32 scores stay in s.
  auto exp_pack = [&]() __attribute__((always_inline)) -> float {
    float ts = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      f32x16 e;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        e[i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -m_ref));
        ts = (kb == 0 && i == 0) ? e[i] : ts + e[i];
      }
      pf[2 * kb] = acc_to_bf16(e, 0);
      pf[2 * kb + 1] = acc_to_bf16(e, 8);
    }
    return ts;
  };
  auto softmax = [&](int t) __attribute__((always_inline)) {
    const int kb0 = seg0 + t * BN;
    if (kb0 + BN > seg1) {  // keys past the segment end (last tile only)
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb0 + kb * 32 + acc_row(i, g) >= seg1) s[kb][i] = -INFINITY;
    }
    // P is formed against the current reference first. A lane sum of at most
    // kSumLimit bounds each of the lane's P by it, which keeps the fp32
    // accumulators far from overflow, so the reference can stay. Any other
    // sum (larger, infinite or NaN; always on the first tile, where m_ref is
    // -inf) takes the exact online-softmax step: the row maxima, a raised
    // reference when they pass it by kRescaleThreshold, and P formed again.
    // Either way the result is the same softmax; only the reference differs.
    // On the first tile the reference is -inf and the exact step always runs,
    // so P is formed only once there, after the maxima.
    float ts = t == 0 ? INFINITY : exp_pack();
    if (__ballot(!(ts <= kSumLimit))) {
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
      ts = exp_pack();
    }
    l_part += ts;
  };

  // Schedule (every wave passes the same number of barriers; group 1 runs one
  // phase behind group 0):
  //   A_0 = scores(0); then for each tile t: [wait own loads, barrier]
  //   B_t = issue(t+2), softmax(t); [barrier] A_{t+1} = accumulate(t), scores(t+1).
  // Tile t+2 reuses the stage of tile t-2, whose last reader (accumulate(t-2)
  // in A_{t-1}) both groups have passed before either issues in B_t; each wave
  // waits for its own loads at the end of its next A phase, at least one
  // barrier before any wave reads the tile.
  auto step = [&](auto stage, int t) __attribute__((always_inline)) {  // stage = t % NS
    constexpr int SG = decltype(stage)::value;
    wait_vmem();
    phase_barrier();
    issue(std::integral_constant<int, (SG + 2) % NS>{}, t + 2);
    softmax(t);
    phase_barrier();
    // One basic block: past the last tile the scores of a stale stage are
    // formed and never used (in-bounds LDS reads), so the block can be
    // scheduled as one MFMA / LDS-read pipeline.
    accumulate(stage);
    scores(std::integral_constant<int, (SG + 1) % NS>{});
    pipeline_mfma_ds<16 * DB / 4 + KS * BN / 32, BN / 16 * DB, 2, 1, 4>();
  };
  issue(std::integral_constant<int, 0>{}, 0);
  issue(std::integral_constant<int, 1>{}, 1);
  wait_vmem();
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = ld_bf16x8(q_stage + swz_off<D, SWZ_ROWS>(lq, 16 * s + 8 * g));
  lds_barrier();  // tiles 0 and 1 visible; every wave's Q-hat reads done before tile 2 is issued
  if (grp == 1) lds_barrier();
  scores(std::integral_constant<int, 0>{});
  for (int t = 0; t < ntiles; t += NS) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 >= ntiles) break;
    step(std::integral_constant<int, 1>{}, t + 1);
    if (t + 2 >= ntiles) break;
    step(std::integral_constant<int, 2>{}, t + 2);
    if (t + 3 >= ntiles) break;
    step(std::integral_constant<int, 3>{}, t + 3);
  }
  if (grp == 0) lds_barrier();

  // Epilogue: normalise O, store it (rows inside the segment) and lse. The
  // wave's 32 rows go out whole: each lane first writes its O^T columns into
  // an LDS copy of the rows, then the wave stores them 16 lanes to a 256-byte
  // row. The copy uses ring stages (L+2) % 4 and (L+3) % 4 (L = the last
  // tile): no load is issued past the last tile and both groups have passed
  // their last reads of those stages, while group 1's last matrix phase still
  // reads stages L % 4 and (L+1) % 4. Each wave has its own 8 KiB (d = 128).
  const float l = half_sum(l_part);
  const float inv = 1.0f / l;
  {
    const int bi = wave >> 1;                  // stage buffer: K or V of stage (L + 2 + bi / 2) % 4
    const int sg = (ntiles + 1 + (bi >> 1)) & 3;
    bf16 *const buf = (bi & 1) ? (sg == 0 ? v0s : sg == 1 ? v1s : sg == 2 ? v2s : v3s)
                               : (sg == 0 ? k0s : sg == 1 ? k1s : sg == 2 ? k2s : k3s);
    bf16 *const ost = buf + (wave & 1) * 32 * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v4;
        bf16x2 t0 = pack2(o[b][4 * r4 + 0] * inv, o[b][4 * r4 + 1] * inv);
        bf16x2 t1 = pack2(o[b][4 * r4 + 2] * inv, o[b][4 * r4 + 3] * inv);
        v4[0] = t0[0]; v4[1] = t0[1]; v4[2] = t1[0]; v4[3] = t1[1];
        *reinterpret_cast<bf16x4 *>(ost + swz_off<D, SWZ_ROWS>(lq, b * 32 + 8 * r4 + 4 * g)) = v4;
      }
    wait_lds();  // the wave's rows are complete in LDS
    constexpr int CPR = D / 8;     // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;  // rows per instruction
    const int orow = lane / CPR, ochunk = lane % CPR;
    bf16 *const og = static_cast<bf16 *>(a.o) + h * D + 8 * ochunk;
#pragma unroll
    for (int j = 0; j < 32 / RPI; ++j) {
      const int r = RPI * j + orow;
      const int q = q0 + wave * 32 + r;
      const bf16x8 v = ld_bf16x8(ost + swz_off<D, SWZ_ROWS>(r, 8 * ochunk));
      if (q < seg1) st16(og + (int64_t)q * HD, as_u4(v));
    }
  }
  if (a.lse && g == 0 && qi < seg1)
    a.lse[(int64_t)h * p.total_tokens + qi] = (m_ref + __log2f(l)) * 0.69314718055994531f;
}

hipError_t launch_attn_fwd_f32(const PlanDev &p, const AttnFwdArgs &a, hipStream_t stream);

template <int D>
static hipError_t attn_fwd_bf16(const PlanDev &p, const AttnFwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(attn_fwd_bf16_kernel<D>, dim3((unsigned)p.num_fwd_blocks), dim3(64 * fwd::NW), 0, s, p,
                     a);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(int dtype, const PlanDev &p, const AttnFwdArgs &a, hipStream_t stream) {
  if (dtype == MMDIT_F32) return launch_attn_fwd_f32(p, a, stream);
  if (p.head_dim == 64) return attn_fwd_bf16<64>(p, a, stream);
  if (p.head_dim == 128) return attn_fwd_bf16<128>(p, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace mmdit
