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
// Where the caller gives room for it, the dK/dV kernel instead writes dS
// (bf16, in its register order) and a third kernel forms dQ^T = K^T dS^T by
// streaming it, which costs 2 bytes of HBM traffic per score instead of the
// S and dP products (D then comes first, from the backward preprocess).
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace mmdit {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));


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
// Backward of the prologue, fused into the attention kernels' epilogues (the
// per-modality RMSNorm with a learned gain and the 2D RoPE of image tokens,
// picx.dev "Mage-Flow ...", section "Native-Resolution MMDiT (NR-MMDiT)";
// fused as the section "Training Infrastructure" describes). With
// y = rho * g_m * x (rho = 1/sqrt(mean(x^2) + eps)) and x-hat = R(phi) y:
//   dy = R(-phi) dx-hat,   dx = rho g_m dy - rho^3/d (sum_j g_mj dy_j x_j) x,
//   dg_m += rho dy x  (summed over tokens and heads).
// The gradient rows are in the 32x32 accumulator layout: lane (lq, g) holds
// dX-hat / scale of its token at d = 32b + acc_row(i, g) in acc[b][i], the
// other half of the row in lane lq + 32(1-g). The inputs the epilogue needs
// are fetched early (token words and rstd in registers, gains and, where LDS
// allows, the pre-norm rows in LDS) so that it costs at most one round trip
// to memory.
// ---------------------------------------------------------------------------
// Inputs of one lane's row: meta = the token's tok_meta word, rho = its
// rstd (negative: recompute from x), xa(d0) = its pre-norm elements d0..d0+3
// (from LDS or global), g2 = the two gain rows of this input (text, image;
// LDS), fp = the plan's RoPE frame pairs, out = the row's element offset in
// the dense output. Writes dx (bf16) for a valid row and
// leaves in red[m * D + d] (m = 0 text, 1 image) this wave's sums of
// rho*dy*x over its 32 tokens (invalid rows add nothing).
// The pre-norm row's loads are issued before any arithmetic (or by the
// caller, earlier: see RowInputs); the gradient row is transformed in place
// (dX-hat/scale -> dy/scale -> gain terms) and the pre-norm row stays in
// bf16, so the step keeps few registers live and the compiler need not spill.
// B0, NB: the register blocks this wave finishes (d in [32 B0, 32 (B0 + NB))).
// With XCH, another wave finishes the other blocks of the same rows: the two
// exchange their partial row sums through xch (slots self and partner of
// 128 floats; every wave of the workgroup passes the barrier inside), adding
// them in a fixed order (the partial of the wave with first = true first), so
// both get bitwise the same sums.
// With LROWS the outputs go, for every row, to an LDS copy of the wave's 32
// rows (lrows, [32][D], ROWS-swizzled) instead of dx; the caller stores the
// valid rows whole.
// The inputs of NB register blocks of one lane's row that come from memory:
// the pre-norm elements and the {cos, sin} RoPE entries. Lane pairs (d, d+1)
// of register block b are pairs 16b + 4(k/2) + 2g + k%2, k = 0..7: two
// consecutive pairs per k/2, in one RoPE section (section boundaries are
// multiples of 4 pairs), so each k/2 is one 16-byte load; a text row loads
// table row 0 and does not use it. A caller that has registers to spare
// fetches them early (prologue_bwd_fetch), so that their latency overlaps
// other work, and passes them in.
template <int NB>
struct RowInputs {
  bf16x4 x4[NB][4];
  f32x4 cs[NB][4];
};
template <int D, int B0, int NB, typename XA>
__device__ __forceinline__ void prologue_bwd_fetch(RowInputs<NB> &in, int32_t meta, const XA &xa,
                                                   const float2 *rope, int fp, int lane) {
  const int g = lane >> 5;
  bool img;
  int row, col, frame;
  tok_pos(meta, img, row, col, frame);
  const int re = fp + (D / 2 - fp) / 2;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) in.x4[b][r4] = xa(32 * (B0 + b) + 8 * r4 + 4 * g);
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int pair = 16 * (B0 + b) + 4 * k2 + 2 * g;
      const int pos = img ? rope_pos(pair, fp, re, row, col, frame) : 0;
      in.cs[b][k2] = *reinterpret_cast<const f32x4 *>(rope + pos * (D / 2) + pair);
    }
}

// PRE: `pre` holds the row inputs fetched by the caller (prologue_bwd_fetch);
// otherwise they are loaded here (the pre-norm row first, then block by
// block the RoPE entries, which keeps few registers live).
template <int D, int B0, int NB, bool XCH, bool LROWS = false, bool PRE = false, typename XA>
__device__ __forceinline__ void prologue_bwd_rows(f32x16 (&acc)[D / 32], float scale, int32_t meta,
                                                  float rho, bool valid, const XA &xa, const float *g2,
                                                  const float2 *rope, int fp, float eps, bf16 *dx, int64_t out,
                                                  float *red, int lane, float *xch = nullptr, int self = 0,
                                                  int partner = 0, bool first = true, bf16 *lrows = nullptr,
                                                  const RowInputs<NB> &pre = RowInputs<NB>{}) {
  constexpr int DB = D / 32;
  static_assert(B0 >= 0 && NB >= 1 && B0 + NB <= DB, "block range");
  const int lq = lane & 31, g = lane >> 5;
  bool img;
  int row, col, frame;
  tok_pos(meta, img, row, col, frame);
  bf16x4 x4[DB][4];
  if constexpr (PRE) {
#pragma unroll
    for (int b = B0; b < B0 + NB; ++b) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) x4[b][r4] = pre.x4[b - B0][r4];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const f32x4 c4 = pre.cs[b - B0][k >> 1];
        const float c = c4[2 * (k & 1)], sn = c4[2 * (k & 1) + 1];
        const float u = acc[b][2 * k], w = acc[b][2 * k + 1];
        acc[b][2 * k] = img ? u * c + w * sn : u;
        acc[b][2 * k + 1] = img ? w * c - u * sn : w;
      }
    }
  } else {
#pragma unroll
    for (int b = B0; b < B0 + NB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) x4[b][r4] = xa(32 * b + 8 * r4 + 4 * g);
    const int re = fp + (D / 2 - fp) / 2;
#pragma unroll
    for (int b = B0; b < B0 + NB; ++b) {
      if (img) {
        f32x4 cs[4];  // {cos, sin} of two consecutive pairs (see RowInputs)
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          const int pair = 16 * b + 4 * k2 + 2 * g;
          cs[k2] = *reinterpret_cast<const f32x4 *>(rope + rope_pos(pair, fp, re, row, col, frame) * (D / 2) + pair);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float c = cs[k >> 1][2 * (k & 1)], sn = cs[k >> 1][2 * (k & 1) + 1];
          const float u = acc[b][2 * k], w = acc[b][2 * k + 1];
          acc[b][2 * k] = u * c + w * sn;
          acc[b][2 * k + 1] = w * c - u * sn;
        }
      }
    }
  }
  // Two passes over the row: row sums first, then outputs.
  const float *gm = g2 + (img ? D : 0);
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int b = B0; b < B0 + NB; ++b) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 g4 = *reinterpret_cast<const f32x4 *>(gm + 32 * b + 8 * r4 + 4 * g);
      const bf16x4 xb = x4[b][r4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = (float)xb[j];
        ss = fmaf(x, x, ss);
        dot = fmaf(g4[j] * acc[b][4 * r4 + j], x, dot);
      }
    }
  }
  if constexpr (XCH) {
    xch[self * 128 + 2 * lane] = ss;
    xch[self * 128 + 2 * lane + 1] = dot;
    __syncthreads();
    const float ss_p = xch[partner * 128 + 2 * lane], dot_p = xch[partner * 128 + 2 * lane + 1];
    ss = first ? ss + ss_p : ss_p + ss;
    dot = first ? dot + dot_p : dot_p + dot;
  }
  // The row is linear in dX-hat, so its scale goes into rho's factors
  // (rs for the output, rg for the gain terms, zero past the segment end)
  // instead of into every element.
  if (rho < 0.f) rho = rsqrtf(half_sum(ss) * (1.0f / D) + eps);
  dot = half_sum(dot);
  const float c3 = rho * rho * rho * dot * (scale * (1.0f / D));
  const float rs = rho * scale, rg = valid ? rs : 0.f;
#pragma unroll
  for (int b = B0; b < B0 + NB; ++b) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = 32 * b + 8 * r4 + 4 * g;
      const f32x4 g4 = *reinterpret_cast<const f32x4 *>(gm + d0);
      const bf16x4 xb = x4[b][r4];
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * r4 + j;
        const float x = (float)xb[j];
        o[j] = fmaf(rs, g4[j] * acc[b][i], -(c3 * x));
        acc[b][i] = rg * acc[b][i] * x;  // gain-gradient term
      }
      const bf16x2 t0 = pack2(o[0], o[1]), t1 = pack2(o[2], o[3]);
      bf16x4 o4;
      o4[0] = t0[0]; o4[1] = t0[1]; o4[2] = t1[0]; o4[3] = t1[1];
      if constexpr (LROWS)
        *reinterpret_cast<bf16x4 *>(lrows + swz_off<D, SWZ_ROWS>(lq, d0)) = o4;
      else if (valid)
        *reinterpret_cast<bf16x4 *>(dx + out + d0) = o4;
    }
  }
  // Sum the gain terms over the wave's 32 tokens (lanes lq = 0..31 of each
  // half) by a transposing reduction in VALU: at each of four steps the
  // registers pair up (2j, 2j + 1); a lane keeps the one that bit k of its
  // index selects and adds the partner's copy of it, taken by DPP from a
  // lane that differs in bit k and agrees in the bits below (xor 1, xor 2,
  // then rotations by 4 and 8 inside the 16-lane row, which together cover
  // the row). After them register j of lane l holds the row's sum of
  // register 16j + l % 16, and a permlane16 swap adds the other row of the
  // half: lane lq < 16 writes block j's sum for register lq. A wave whose
  // valid tokens are all of one modality reduces once; a mixed wave once
  // per modality.
  const uint64_t has_img = __ballot(valid && img), has_txt = __ballot(valid && !img);
  auto reduce_into = [&](int m, bool select, bool want_img) __attribute__((always_inline)) {
    float v[NB * 16];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) v[16 * b + i] = (!select || img == want_img) ? acc[B0 + b][i] : 0.f;
    auto step = [&](auto ctrl, int bit, int n) __attribute__((always_inline)) {
      const bool hi = (lane & bit) != 0;
#pragma unroll
      for (int j = 0; j < n / 2; ++j) {
        const float x = hi ? v[2 * j + 1] : v[2 * j], y = hi ? v[2 * j] : v[2 * j + 1];
        v[j] = x + dpp<decltype(ctrl)::value>(y);
      }
    };
    step(std::integral_constant<int, 0xB1>{}, 1, NB * 16);   // quad_perm [1,0,3,2]
    step(std::integral_constant<int, 0x4E>{}, 2, NB * 8);    // quad_perm [2,3,0,1]
    step(std::integral_constant<int, 0x124>{}, 4, NB * 4);   // row_ror:4
    step(std::integral_constant<int, 0x128>{}, 8, NB * 2);   // row_ror:8
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float t = row_pair_sum(v[b]);
      if (lq < 16) red[m * D + 32 * (B0 + b) + acc_row(lq, g)] = t;
    }
  };
  auto zero_row = [&](int m) __attribute__((always_inline)) {
    for (int e = 32 * B0 + lane; e < 32 * (B0 + NB); e += 64) red[m * D + e] = 0.f;
  };
  if (has_img && has_txt) {
    reduce_into(0, true, false);
    reduce_into(1, true, true);
  } else if (has_img) {
    reduce_into(1, false, true);
    zero_row(0);
  } else {
    reduce_into(0, false, false);  // text only (or no valid token: all zero)
    zero_row(1);
  }
}

// Store rows r0 .. r0 + n - 1 of an LDS copy of 32 token rows ([32][D],
// ROWS-swizzled; row r is token t0 + r) to dst (token t's row at t * stride),
// 16 lanes to a 256-byte row, rows of tokens >= t_end skipped (one wave).
template <int D>
__device__ __forceinline__ void store_rows(const bf16 *lrows, int r0, int n, int t0, int t_end, bf16 *dst,
                                           int64_t stride, int lane) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  const int orow = lane / CPR, ochunk = lane % CPR;
  for (int j = 0; j < n / RPI; ++j) {
    const int r = r0 + RPI * j + orow;
    const bf16x8 v = ld_bf16x8(lrows + swz_off<D, SWZ_ROWS>(r, 8 * ochunk));
    if (t0 + r < t_end) st16(dst + (int64_t)(t0 + r) * stride + 8 * ochunk, as_u4(v));
  }
}

// Fixed-order sum of nw per-wave gain partials red[w][2][D] into out[2][D]
// (threads 0 .. 2D-1 of the workgroup).
template <int D>
__device__ __forceinline__ void sum_wave_partials(const float *red, int nw, float *out, int tid) {
  if (tid < 2 * D) {
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[w * 2 * D + tid];
    out[tid] = s;
  }
}

// ---------------------------------------------------------------------------
// dQ-hat (and D) for one 256-query tile of one sample and head.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * bwd::NWQ, 1) void attn_bwd_dq_kernel(PlanDev p, AttnBwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  using namespace bwd;
  constexpr int NT = 64 * NWQ;        // threads
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int LDK = D + PAD_BOTH;   // K: row reads and transposed reads
  constexpr int LDV = D + PAD_ROWS;   // V: row reads only
  constexpr int CHUNKS = BN * D / 8 / NT;
  __shared__ __attribute__((aligned(16))) bf16 k_s[2][BN * LDK];
  __shared__ __attribute__((aligned(16))) bf16 v_s[2][BN * LDV];
  __shared__ __attribute__((aligned(16))) bf16 x_s[NWQ * 32 * D];  // pre-norm q rows, for the epilogue
  __shared__ __attribute__((aligned(16))) float g_s[2 * D];         // Q gains: text, image
  __shared__ float red[NWQ * 2 * D];

  const int H = p.num_heads;
  const int N = p.total_tokens;
  const int2 wb = p.fwd_blocks[blockIdx.x];
  float *part = a.part_q + (int64_t)blockIdx.x * 2 * D;
  if (wb.x < 0) {  // idle slot of the block map (whole workgroup): empty partials
    if (threadIdx.x < 2 * D) part[threadIdx.x] = 0.f;
    return;
  }
  const int h = wb.y;
  const int4 it = p.fwd_items[wb.x];
  const int seg0 = it.x, seg1 = it.y, q0 = it.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Start-up: every load is issued before the first wait, and the wave's 32
  // rows of Q-hat, dO and O are read whole (16 lanes per 256-byte row) rather
  // than lane by lane: Q-hat and dO by direct load into LDS (Q-hat where the
  // pre-norm rows go later, dO in the K/V buffers, both free until the first
  // tile is staged), O into registers. Lanes then take their B operands from
  // LDS, and D = rowsum(dO * O) is formed in the row-wide layout and handed to
  // the query's lanes through LDS.
  static_assert(4 * 32 * D <= 2 * BN * LDV && 4 * 32 * D <= 2 * BN * LDK, "dO staging fits the K/V buffers");
  bf16 *q_stage = x_s + wave * 32 * D;
  bf16 *g_stage = (wave < 4 ? &k_s[0][0] : &v_s[0][0]) + (wave & 3) * 32 * D;
  load_tile(seg0);
  {
    TileLoader<D, SWZ_ROWS, 32, 1> qload, gload;
    qload.init(0, lane, HD);
    gload.init(0, lane, a.dout_stride);
    qload.issue(q_stage, qh + h * D, q0 + wave * 32, seg1 - 1);
    gload.issue(g_stage, go + h * D, q0 + wave * 32, seg1 - 1);
  }
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;     // rows per wave-wide instruction
  constexpr int OJ = 32 / RPI;      // instructions for the wave's 32 rows
  const int orow = lane / CPR, ochunk = lane % CPR;
  uint4 oreg[OJ];
#pragma unroll
  for (int j = 0; j < OJ; ++j) {
    const int row = min(q0 + wave * 32 + RPI * j + orow, seg1 - 1);
    oreg[j] = ld16(oo + (int64_t)row * HD + h * D + 8 * ochunk);
  }
  // Epilogue inputs: the Q gains, this query's token word and rstd.
  if (tid < 2 * D) g_s[tid] = a.gains[tid];
  const int32_t meta = p.tok_meta[qc];
  const float rho0 = a.rstd ? a.rstd[(int64_t)qc * H + h] : -1.f;
  const float lse2 = a.lse[(int64_t)h * N + qc] * kLog2e;
  wait_vmem();  // this wave's rows are in LDS and registers
  bf16x8 qf[KS], gf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = ld_bf16x8(q_stage + swz_off<D, SWZ_ROWS>(lq, 16 * s + 8 * g));
    gf[s] = ld_bf16x8(g_stage + swz_off<D, SWZ_ROWS>(lq, 16 * s + 8 * g));
  }
  float *dl = red + wave * 32;  // D of the wave's rows
#pragma unroll
  for (int j = 0; j < OJ; ++j) {
    const int r = RPI * j + orow;
    const bf16x8 gv = ld_bf16x8(g_stage + swz_off<D, SWZ_ROWS>(r, 8 * ochunk));
    const bf16x8 ov = __builtin_bit_cast(bf16x8, oreg[j]);
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) t = fmaf((float)gv[e], (float)ov[e], t);
    t = group_sum<CPR>(t);
    if (ochunk == 0) dl[r] = t;
  }
  wait_lds();  // this wave's reads of its staged rows and its D writes are done
  const float dlt = dl[lq];  // written out with -lse*log2e after the loop
  // The pre-norm q rows for the epilogue, over the wave's Q-hat rows (read
  // above); they land during the main loop.
  {
    TileLoader<D, SWZ_ROWS, 32, 1> xload;
    xload.init(0, lane, a.q_stride);
    xload.issue(q_stage, static_cast<const bf16 *>(a.q) + h * D, q0 + wave * 32, seg1 - 1);
  }

  f32x16 dq[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[b][i] = 0.f;

  const int ntiles = (seg1 - seg0 + BN - 1) / BN;
  __syncthreads();  // every wave is done with its dO rows in the K/V buffers
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
      pipeline_mfma_ds<2 * KS, 0, 0, 1, 4>();
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
    pipeline_mfma_ds<(BN / 16) * DB, (BN / 16) * DB, 2, 0, 4>();
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // D and -lse*log2e for the dK/dV kernel, stored after the loop: a store
  // pending at the loop's start would make the compiler wait for every
  // outstanding memory operation wherever the loop waits for a load.
  if (g == 0 && qi < seg1) {
    a.delta[(int64_t)h * N + qi] = dlt;
    a.nlse[(int64_t)h * N + qi] = -lse2;
  }
  // dQ-hat row of this lane's query -> dq, and the block's Q gain partials.
  wait_vmem();  // the pre-norm rows (a pack of one key tile issues no load after them)
  const bf16 *xt = x_s + wave * 32 * D;
  auto xa = [&](int d0) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x4 *>(xt + swz_off<D, SWZ_ROWS>(lq, d0));
  };
  // The dQ rows go out whole through the wave's dO staging slice (free
  // after the loop).
  prologue_bwd_rows<D, 0, D / 32, false, true>(dq, a.scale, meta, rho0, qi < seg1, xa, g_s, p.rope,
                                               p.rope_frame_pairs, p.rms_eps, nullptr, 0, red + wave * 2 * D, lane,
                                               nullptr, 0, 0, true, g_stage);
  wait_lds();
  store_rows<D>(g_stage, 0, 32, q0 + wave * 32, seg1, static_cast<bf16 *>(a.dq) + h * D, HD, lane);
  __syncthreads();
  sum_wave_partials<D>(red, NWQ, part, tid);
}

// ---------------------------------------------------------------------------
// dQ-hat from the stored dS for one 256-query tile of one sample and head:
// dQ^T += K^T dS^T over the sample's keys, 64 per tile. Each wave owns 32
// queries (two 16-query slices of the stored blocks). Per tile, K-hat (shared
// by the 8 waves) and each wave's own 4 KiB of dS arrive by direct
// global->LDS loads into a 3-stage ring; both MFMA operands are read
// transposed (ds_read_b64_tr_b16): K^T with one d per lane, dS^T with one
// query per lane. A stored 16-byte piece of dS is lane (g, key) of the
// writer: queries acc_row(0..7, g) of its slice, i.e. four consecutive
// queries in each half, so each 8-byte half is one row piece of a
// transposed read. The epilogue is the dQ kernel's.
// ---------------------------------------------------------------------------
namespace bwd {
constexpr int DQS_TK = 64;                             // keys per tile
constexpr int DQS_NS = 3;                              // ring stages
constexpr int DQS_BLK = kDsBlockBytes + 128;           // LDS bytes per stored block
constexpr int DQS_WAVE = 4 * DQS_BLK;                  // a wave's dS of one tile
// Cache policy of the dS stream (written once, read once): non-temporal
// (aux bit 1), which keeps the K/V/Q tiles that other workgroups re-read in
// L2; measured ~3% faster in the dK/dV kernel than the default policy.
constexpr int kDsCachePolicy = 2;
}  // namespace bwd

// dS^T fragment (B operand) of keys 16 t .. 16 t + 15 of the wave's tile
// from its four LDS blocks [key half kb][query slice u] at sw + (2 kb + u) *
// DQS_BLK: lane (G, i) supplies row 4 g + i/4 (and + 8), queries 4 (i % 4)..+3
// of slice u = G % 2, and ends up holding query 16 u + i.
__device__ __forceinline__ bf16x8 ds_frag(const char *sw, int t, int lane) {
  using namespace bwd;
  const int G = lane >> 4, i = lane & 15;
  const int g = G >> 1, u = G & 1;
  const int r = 16 * t + 4 * g + (i >> 2);  // key within the 64-key tile
  const int c4 = i & 3;
  const char *p0 = sw + (2 * (r >> 5) + u) * DQS_BLK + (2 * (r & 31) + (c4 & 1)) * 16 + (c4 >> 1) * 8;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p0 + 2 * 8 * 16));
  bf16x8 out;
  out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
  out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
  return out;
}

template <int D>
__global__ __launch_bounds__(64 * bwd::NWQ, 1) void attn_bwd_dq_ds_kernel(PlanDev p, AttnBwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  using namespace bwd;
  constexpr int DB = D / 32;
  constexpr int TK = DQS_TK;
  using KL = TileLoader<D, SWZ_TRANS, TK, NWQ>;
  constexpr int PER_TILE = KL::LOADS + 4;  // loads per wave per tile
  // One LDS object per ring stage and operand (compile-time stage indices
  // let the compiler see that loads into one stage never alias reads of
  // another).
  __shared__ __attribute__((aligned(16))) bf16 k0s[TK * D], k1s[TK * D], k2s[TK * D];
  __shared__ __attribute__((aligned(16))) char s0s[NWQ * DQS_WAVE], s1s[NWQ * DQS_WAVE], s2s[NWQ * DQS_WAVE];
  __shared__ __attribute__((aligned(16))) float g_s[2 * D];  // Q gains: text, image
  static_assert(NWQ * 2 * D * 4 <= NWQ * DQS_WAVE, "gain partials fit a ring stage");
  auto kst = [&](auto stage) __attribute__((always_inline)) -> bf16 * {
    constexpr int S = decltype(stage)::value;
    if constexpr (S == 0) return k0s; else if constexpr (S == 1) return k1s; else return k2s;
  };
  auto sst = [&](auto stage) __attribute__((always_inline)) -> char * {
    constexpr int S = decltype(stage)::value;
    if constexpr (S == 0) return s0s; else if constexpr (S == 1) return s1s; else return s2s;
  };

  const int H = p.num_heads;
  const int2 wb = p.fwd_blocks[blockIdx.x];
  float *part = a.part_q + (int64_t)blockIdx.x * 2 * D;
  if (wb.x < 0) {  // idle slot of the block map (whole workgroup): empty partials
    if (threadIdx.x < 2 * D) part[threadIdx.x] = 0.f;
    return;
  }
  const int h = wb.y;
  const int4 it = p.fwd_items[wb.x];
  const int seg0 = it.x, seg1 = it.y, q0 = it.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31;
  const int64_t HD = (int64_t)H * D;

  const int qi = q0 + wave * 32 + lq;
  const int qc = min(qi, seg1 - 1);
  if (tid < 2 * D) g_s[tid] = a.gains[tid];
  const int32_t meta = p.tok_meta[qc];
  const float rho0 = a.rstd ? a.rstd[(int64_t)qc * H + h] : -1.f;

  // This sample and head's dS area; blocks past it (keys past the segment
  // end in the last tile) read as zeros, and slices past the last query tile
  // only feed queries past the segment end, whose rows are dropped.
  const int L = seg1 - seg0;
  const int nq16 = 4 * ((L + BMQ - 1) / BMQ);
  const int64_t blocks = (int64_t)((L + 31) / 32) * nq16;
  const rsrc_t ds_rs = make_rsrc(static_cast<const char *>(a.ds) + (p.ds_base[it.w] + h * blocks) * kDsBlockBytes,
                                 (uint32_t)(blocks * kDsBlockBytes));
  const int u0 = (q0 - seg0) / 16 + 2 * wave;  // the wave's first query slice
  KL kload;
  kload.init(wave, lane, HD);
  const bf16 *kh = static_cast<const bf16 *>(a.k_hat) + h * D;
  const int ntiles = (L + TK - 1) / TK;
  // Tile j: K-hat rows seg0 + 64 j .. (rows past the segment end land as
  // zeros) and this wave's blocks (2 j + kb, u0 + u), kb, u in {0, 1}.
  auto issue = [&](auto stage, int j) __attribute__((always_inline)) {
    if (j >= ntiles) return;
    kload.issue(kst(stage), kh, seg0 + j * TK, seg1 - 1);
    char *sw = sst(stage) + wave * DQS_WAVE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t blk = (uint32_t)((2 * j + kb) * nq16 + u0 + u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ds_rs, (__attribute__((address_space(3))) void *)(sw + (2 * kb + u) * DQS_BLK),
                                                 16, blk * kDsBlockBytes + 16u * lane, 0, 0, kDsCachePolicy);
      }
  };

  f32x16 dq[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[b][i] = 0.f;

  // Tile j+2 reuses the stage of tile j-1, which every wave finished reading
  // before the barrier of step j; each wave waits for its own loads of tile
  // j before that barrier.
  auto step = [&](auto stage, int j) __attribute__((always_inline)) {
    constexpr int SG = decltype(stage)::value;
    if (j + 1 < ntiles) wait_vmem_le<PER_TILE>();
    else wait_vmem();
    lds_barrier();
    issue(std::integral_constant<int, (SG + 2) % DQS_NS>{}, j + 2);
    const bf16 *Ks = kst(stage);
    const char *sw = sst(stage) + wave * DQS_WAVE;
    bf16x8 bfr[TK / 16];
#pragma unroll
    for (int t = 0; t < TK / 16; ++t) bfr[t] = ds_frag(sw, t, lane);
#pragma unroll
    for (int t = 0; t < TK / 16; ++t)
#pragma unroll
      for (int b = 0; b < DB; ++b)
        dq[b] = mfma32(lds_read_tr_swz<D, SWZ_TRANS>(Ks, t * 16, b * 32, lane), bfr[t], dq[b]);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TK / 16), 0);  // the dS fragments first
    pipeline_mfma_ds<(TK / 16) * DB, 0, 0, 2, 4>();
  };
  issue(std::integral_constant<int, 0>{}, 0);
  issue(std::integral_constant<int, 1>{}, 1);
  for (int j = 0; j < ntiles; j += DQS_NS) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 >= ntiles) break;
    step(std::integral_constant<int, 1>{}, j + 1);
    if (j + 2 >= ntiles) break;
    step(std::integral_constant<int, 2>{}, j + 2);
  }
  wait_vmem();  // no load into LDS may outlive the workgroup
  __syncthreads();  // the ring is free: stage 0 holds the waves' gain partials

  // dQ-hat row of this lane's query -> dq, and the block's Q gain partials.
  float *red = reinterpret_cast<float *>(s0s);
  const bf16 *xg = static_cast<const bf16 *>(a.q) + (int64_t)qc * a.q_stride + h * D;
  auto xa = [&](int d0) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x4 *>(xg + d0);
  };
  prologue_bwd_rows<D, 0, D / 32, false>(dq, a.scale, meta, rho0, qi < seg1, xa, g_s, p.rope, p.rope_frame_pairs, p.rms_eps,
                       static_cast<bf16 *>(a.dq), ((int64_t)qc * H + h) * D, red + wave * 2 * D, lane);
  __syncthreads();
  sum_wave_partials<D>(red, NWQ, part, tid);
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
// role issues matrix instructions while the other does its vector and
// memory work:
//   phase 1: P/dV waves: load Q-hat, lse of tile t+2; softmax(t) -> P(t) to LDS
//            dS/dK waves: dK(t-1), dP(t)
//   phase 2: P/dV waves: dV(t), S(t+1)
//            dS/dK waves: load dO, D of tile t+3; dS(t) (reads P(t))
// All tile data comes by direct global->LDS loads into a 4-stage ring. Tile
// t+2 (phase 1 of tile t) reuses the stage of tile t-2 and tile t+3 (phase
// 2) that of tile t-1; the last reader of either (dK(t-2), dK(t-1)) ran
// before the barrier that precedes the load. Each wave waits for its own
// loads of tile t+1 before the barrier that opens phase 2 of tile t, so tile
// t+1 is visible one phase before S(t+1) reads it. Loads cost issue cycles,
// so each role issues its half in the phase where it is not feeding the
// matrix cores, and no load in the loop returns into registers (such returns
// compete with the matrix instructions of the other wave on the SIMD). The
// matrix blocks run at raised wave priority, so that the partner wave's
// vector instructions do not delay their MFMA and LDS-read issue.
// ---------------------------------------------------------------------------
namespace bwd {
constexpr int KV_NW = 8;   // waves of a dK/dV workgroup
constexpr int KV_NS = 4;   // Q-hat / dO ring stages
}  // namespace bwd

template <int D, bool DS>
__global__ __launch_bounds__(64 * bwd::KV_NW, 1) void attn_bwd_dkdv_kernel(PlanDev p, AttnBwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  using namespace bwd;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BMQ * D;
  static_assert(KV_NS == 4 && BMQ == 64 && KT == 32 * KV_NW / 2, "layout below");
  // One LDS object per ring stage, [Q-hat tile | dO tile | lse | D]:
  // distinct objects (at most 8 of them receiving direct loads) let the
  // compiler prove that loads into one stage do not alias reads of another.
  constexpr int STAGE = 2 * TILE + 4 * BMQ;  // bf16 elements
  __shared__ __attribute__((aligned(16))) bf16 st0[STAGE], st1[STAGE], st2[STAGE], st3[STAGE];
  __shared__ __attribute__((aligned(16))) uint4 p_s[4 * (BMQ / 16) * 64];
  __shared__ __attribute__((aligned(16))) float g_s[2 * D];  // K gains: text, image
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
  float *part = a.part_k + (int64_t)blockIdx.x * 2 * D;
  if (wb.x < 0) {  // idle slot of the block map (whole workgroup): empty partials
    if (threadIdx.x < 2 * D) part[threadIdx.x] = 0.f;
    return;
  }
  const int h = wb.y;
  const int4 it = p.bwd_items[wb.x];
  const int seg0 = it.x, seg1 = it.y, k0 = it.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform to the compiler
  const int role = wave >> 2, sub = wave & 3;  // role 0: P/dV, role 1: dS/dK
  const int lq = lane & 31, g = lane >> 5;
  // Stored dS (DS): 1 KiB block (kb, u) of this sample and head holds keys
  // 32kb..+31 and queries 16u..+15 (sample-relative), lane (g, key lq) of
  // the writing wave at 16 bytes (2 lq + g) * 16: its eight dS values for
  // queries 16u + acc_row(0..7, g). The descriptor ends with the area, so a
  // wave whose keys all lie past the segment end stores nothing.
  rsrc_t ds_rs = make_rsrc(a.ds, 0u);
  uint32_t ds_off = 0;
  if constexpr (DS) {
    const int L = seg1 - seg0;
    const int nq16 = 4 * ((L + BMQ - 1) / BMQ);
    const int64_t blocks = (int64_t)((L + 31) / 32) * nq16;
    ds_rs = make_rsrc(static_cast<char *>(a.ds) + (p.ds_base[it.w] + h * blocks) * kDsBlockBytes,
                      (uint32_t)(blocks * kDsBlockBytes));
    const int kb = (k0 - seg0) / 32 + sub;
    ds_off = (uint32_t)kb * (uint32_t)nq16 * kDsBlockBytes + 16u * (2 * lq + g);
  }
  const int64_t HD = (int64_t)H * D;
  const int64_t gstride = a.dout_stride;
  const bf16 *qh = static_cast<const bf16 *>(a.q_hat) + h * D;
  const bf16 *go = static_cast<const bf16 *>(a.dout) + h * D;
  const float *nlse_h = a.nlse + (int64_t)h * N;  // -lse * log2(e), from the dQ or D pass
  const float *dlt_h = a.delta + (int64_t)h * N;
  const float c2 = a.scale_log2;

  // This lane's key: its K-hat row (P/dV role) or V row (dS/dK role) as a
  // B operand.
  const int kr = k0 + sub * 32 + lq;
  const bool key_ok = kr < seg1;
  const int kc = min(kr, seg1 - 1);
  bf16x8 kv[KS];
  // Epilogue inputs, fetched now: K gains, this key's token word and rstd.
  if (tid < 2 * D) g_s[tid] = a.gains[2 * D + tid];
  const int32_t meta = p.tok_meta[kc];
  const float rho0 = a.rstd ? a.rstd[((int64_t)N + kc) * H + h] : -1.f;
  {
    const bf16 *src = role == 0 ? static_cast<const bf16 *>(a.k_hat) + (int64_t)kc * HD + h * D
                                : static_cast<const bf16 *>(a.v) + (int64_t)kc * a.v_stride + h * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) kv[s] = ld_bf16x8(src + 16 * s + 8 * g);
  }

  const int ntq = (seg1 - seg0 + BMQ - 1) / BMQ;
  // Q-hat tiles are loaded by the four P/dV waves, dO tiles by the four dS/dK
  // waves (sub = a wave's index within its role).
  TileLoader<D, SWZ_BOTH, BMQ, KV_NW / 2> qload, gload;
  qload.init(sub, lane, HD);
  gload.init(sub, lane, gstride);
  constexpr int LQ = TileLoader<D, SWZ_BOTH, BMQ, KV_NW / 2>::LOADS;
  // Tile t -> ring stage. Every step issues one tile's loads, so the
  // compiler's in-order count of outstanding loads is exact; past the last
  // tile the last tile is loaded again into the stage just freed, which
  // nothing reads afterwards.
  // Queries past the segment end need no mask: their Q-hat and dO rows land
  // as zeros and their -lse*log2e reads as 0 (its descriptor ends at the segment),
  // so S = 0 and P = exp2(0) = 1 there, finite, and both dV^T += dO^T P and
  // dK^T += Q-hat^T dS add zero for them.
  const uint32_t vec_bytes = 4u * (uint32_t)seg1;  // lse / D words up to the segment end
  // With its tile, each role loads one per-query vector into the stage:
  // -lse*log2e (P/dV waves) or D (dS/dK waves), the same 64 words from each
  // of the four.
  const rsrc_t l_rs = make_rsrc(nlse_h, vec_bytes);
  const rsrc_t d_rs = make_rsrc(dlt_h, vec_bytes);
  auto issue_q = [&](auto stage, int t) __attribute__((always_inline)) {
    const int qb0 = seg0 + min(t, ntq - 1) * BMQ;
    qload.issue(qst(stage), qh, qb0, seg1 - 1);  // branch-free: exact load counts
    buf2lds<4>(l_rs, 4u * (uint32_t)(qb0 + lane), lst(stage));
  };
  auto issue_g = [&](auto stage, int t) __attribute__((always_inline)) {
    const int qb0 = seg0 + min(t, ntq - 1) * BMQ;
    gload.issue(gst(stage), go, qb0, seg1 - 1);
    buf2lds<4>(d_rs, 4u * (uint32_t)(qb0 + lane), dst(stage));
  };
  constexpr int PER_TILE = LQ + 1;  // loads per wave per tile
  // A per-query vector of the tile (lse or D) for this lane's accumulator
  // rows: v[4 qb + r4] holds queries qb*32 + 8*r4 + 4*g + 0..3, the rows of
  // registers 4*r4..4*r4+3 of block qb. All eight reads are issued before
  // the first use.
  constexpr int ROW_LOADS = 2 * 4;
  auto read_rows = [&](const float *vec, f32x4 (&v)[ROW_LOADS]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < ROW_LOADS; ++j) v[j] = *reinterpret_cast<const f32x4 *>(&vec[8 * j + 4 * g]);
  };

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
        const bf16x8 ra = ld_bf16x8(&T[swz_off<D, SWZ_BOTH>(qb * 32 + lq, 16 * ks + 8 * g)]);
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
        acc[b] = mfma32(lds_read_tr_swz<D, SWZ_BOTH>(T, u * 16, b * 32, lane), pb[u], acc[b]);
  };
  // Role 0: P = exp2(S*c2 - lse*log2e).
  auto softmax = [&](const float *Ls) __attribute__((always_inline)) {
    f32x4 nl[ROW_LOADS];
    read_rows(Ls, nl);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        s[qb][i] = __builtin_amdgcn_exp2f(fmaf(s[qb][i], c2, nl[4 * qb + (i >> 2)][i & 3]));
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
    f32x4 d4[ROW_LOADS];
    read_rows(Ds, d4);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = (float)pr[2 * qb + i / 8][i % 8];
        s[qb][i] = pv * (s[qb][i] - d4[4 * qb + (i >> 2)][i & 3]);
      }
      pb[2 * qb] = acc_to_bf16(s[qb], 0);
      pb[2 * qb + 1] = acc_to_bf16(s[qb], 8);
    }
  };

  using S0 = std::integral_constant<int, 0>;
  // dK(t-1) runs unconditionally in every step: for t = 0 it multiplies the
  // zeroed Q-hat part of stage 3 (tile 3 arrives there only after step 0) by
  // dS = 0 and adds exactly nothing.
#pragma unroll
  for (int u = 0; u < BMQ / 16; ++u) pb[u] = bf16x8{};
  for (int e = tid * 8; e < TILE; e += 64 * KV_NW * 8) st_bf16x8(st3 + e, bf16x8{});

  // Both roles run one step per query tile (every step loads, waits and
  // passes two barriers) and leave the loop after the same step, so barrier
  // counts match across roles; the loads issued past the last tile are
  // waited for after the loop.
  if (role == 0) {
    issue_q(S0{}, 0);
    issue_q(std::integral_constant<int, 1>{}, 1);
    wait_vmem_le<PER_TILE>();  // this wave's loads of tile 0
    phase_barrier();  // tile 0 and the zeroed stage visible
    rows_x_key(qst(S0{}));  // S(0)
    auto step = [&](auto stage, int t) __attribute__((always_inline)) {
      constexpr int SG = decltype(stage)::value;
      issue_q(std::integral_constant<int, (SG + 2) % KV_NS>{}, t + 2);
      softmax(lst(stage));
      wait_vmem_le<PER_TILE>();  // this wave's loads of tile t+1
      phase_barrier();  // P(t) and tile t+1 visible
      __builtin_amdgcn_s_setprio(3);
      {  // one basic block, scheduled as an MFMA / LDS-read pipeline
        accumulate(gst(stage));  // dV(t)
        // S(t+1); after the last tile the stage holds a repeat of the last
        // tile and the result goes unused
        rows_x_key(qst(std::integral_constant<int, (SG + 1) % KV_NS>{}));
        pipeline_mfma_ds<(BMQ / 16) * DB + 2 * KS, (BMQ / 16) * DB, 2, 1, 4>();
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      phase_barrier();  // P(t) consumed
    };
    for (int t = 0; t < ntq; t += KV_NS) {
      step(S0{}, t);
      if (t + 1 >= ntq) break;
      step(std::integral_constant<int, 1>{}, t + 1);
      if (t + 2 >= ntq) break;
      step(std::integral_constant<int, 2>{}, t + 2);
      if (t + 3 >= ntq) break;
      step(std::integral_constant<int, 3>{}, t + 3);
    }
  } else {
    issue_g(S0{}, 0);
    issue_g(std::integral_constant<int, 1>{}, 1);
    issue_g(std::integral_constant<int, 2>{}, 2);
    wait_vmem_le<2 * PER_TILE>();  // this wave's loads of tile 0
    phase_barrier();  // tile 0 and the zeroed stage visible
    auto step = [&](auto stage, int t) __attribute__((always_inline)) {
      constexpr int SG = decltype(stage)::value;
      __builtin_amdgcn_s_setprio(3);
      {  // one basic block, scheduled as an MFMA / LDS-read pipeline
        accumulate(qst(std::integral_constant<int, (SG + 3) % KV_NS>{}));  // dK(t-1)
        rows_x_key(gst(stage));  // dP(t)
        pipeline_mfma_ds<(BMQ / 16) * DB + 2 * KS, (BMQ / 16) * DB, 2, 1, 4>();
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      // This wave's loads of tile t+1: loads complete in issue order, so at
      // most PER_TILE outstanding operations (tile t+2's loads) leaves none
      // of them. Stores (dS, with DS) may complete out of order with respect
      // to loads, so they are not counted on.
      wait_vmem_le<PER_TILE>();
      phase_barrier();  // P(t) and tile t+1 visible
      if constexpr (DS) {
        dscores(dst(stage));  // dS(t)
#pragma unroll
        for (int u = 0; u < BMQ / 16; ++u)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pb[u]), ds_rs,
                                                 (int)(ds_off + (uint32_t)(4 * t + u) * kDsBlockBytes), 0,
                                                 bwd::kDsCachePolicy);
        issue_g(std::integral_constant<int, (SG + 3) % KV_NS>{}, t + 3);
        if (t + 1 == ntq) accumulate(qst(stage));  // last dK
      } else {
        issue_g(std::integral_constant<int, (SG + 3) % KV_NS>{}, t + 3);
        dscores(dst(stage));  // dS(t)
        if (t + 1 == ntq) accumulate(qst(stage));  // last dK
      }
      phase_barrier();  // P(t) consumed
    };
    for (int t = 0; t < ntq; t += KV_NS) {
      step(S0{}, t);
      if (t + 1 >= ntq) break;
      step(std::integral_constant<int, 1>{}, t + 1);
      if (t + 2 >= ntq) break;
      step(std::integral_constant<int, 2>{}, t + 2);
      if (t + 3 >= ntq) break;
      step(std::integral_constant<int, 3>{}, t + 3);
    }
  }

  wait_vmem();  // no load into LDS may outlive the workgroup
  __syncthreads();  // ... nor reach the ring once it is reused below

  // Epilogue. Rows of this lane's key: register i of block b is d = 32b +
  // acc_row(i, g). The ring and the P buffer are free from here. Each dS/dK wave hands the dK-hat of register blocks DB/2 .. DB-1
  // to its P/dV partner (the same keys) through ring stage 0, and the two
  // finish the prologue backward of the key rows on half of the head
  // dimension each, exchanging partial row sums through ring stage 1; so the
  // P/dV waves, otherwise idle here, take half of the work and each wave
  // needs half the registers. The P buffer holds the gain partials.
  constexpr int HB = DB / 2;
  static_assert(4 * HB * 16 * 64 * 4 <= STAGE * 2 && 8 * 128 * 4 <= STAGE * 2, "hand-over fits a stage");
  float *red = reinterpret_cast<float *>(p_s);
  float *hand = reinterpret_cast<float *>(st0);  // [sub][HB * 16][64 lanes]
  float *xch = reinterpret_cast<float *>(st1);   // [role * 4 + sub][128]
  // dV and dK rows go out whole through LDS copies of each sub-tile's 32
  // key rows: dK in ring stage 2, dV in stage 3 (32 x d each per sub-tile).
  static_assert(4 * 32 * D <= STAGE, "a stage holds four sub-tiles' rows");
  bf16 *const dk_rows = st2 + sub * 32 * D, *const dv_rows = st3 + sub * 32 * D;
  // The pre-norm k elements and RoPE entries of this wave's half of the row
  // are requested first; they arrive while the dV rows and the hand-over
  // pass through LDS (a barrier on LDS operations only, so they stay in
  // flight across it). Each role runs its whole epilogue in one branch, so
  // the fetched values stay in registers; both pass the same barriers.
  const bf16 *xg = static_cast<const bf16 *>(a.k) + (int64_t)kc * a.k_stride + h * D;
  auto xa = [&](int d0) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x4 *>(xg + d0);
  };
  bf16 *dkp = static_cast<bf16 *>(a.dk);
  const int64_t out = ((int64_t)kc * H + h) * D;
  if (role == 1) {
    RowInputs<HB> rin;
    prologue_bwd_fetch<D, 0, HB>(rin, meta, xa, p.rope, p.rope_frame_pairs, lane);
#pragma unroll
    for (int b = HB; b < DB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) hand[((sub * HB + (b - HB)) * 16 + i) * 64 + lane] = acc[b][i];
    lds_barrier();
    prologue_bwd_rows<D, 0, HB, true, true, true>(acc, a.scale, meta, rho0, key_ok, xa, g_s, p.rope,
                                                  p.rope_frame_pairs, p.rms_eps, dkp, out, red + sub * 2 * D, lane,
                                                  xch, 4 + sub, sub, true, dk_rows, rin);
  } else {
    RowInputs<HB> rin;
    prologue_bwd_fetch<D, HB, HB>(rin, meta, xa, p.rope, p.rope_frame_pairs, lane);
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v4;
        const bf16x2 t0 = pack2(acc[b][4 * r4], acc[b][4 * r4 + 1]);
        const bf16x2 t1 = pack2(acc[b][4 * r4 + 2], acc[b][4 * r4 + 3]);
        v4[0] = t0[0]; v4[1] = t0[1]; v4[2] = t1[0]; v4[3] = t1[1];
        *reinterpret_cast<bf16x4 *>(dv_rows + swz_off<D, SWZ_ROWS>(lq, b * 32 + 8 * r4 + 4 * g)) = v4;
      }
    lds_barrier();
#pragma unroll
    for (int b = HB; b < DB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] = hand[((sub * HB + (b - HB)) * 16 + i) * 64 + lane];
    prologue_bwd_rows<D, HB, HB, true, true, true>(acc, a.scale, meta, rho0, key_ok, xa, g_s, p.rope,
                                                   p.rope_frame_pairs, p.rms_eps, dkp, out, red + sub * 2 * D, lane,
                                                   xch, sub, 4 + sub, false, dk_rows, rin);
  }
  __syncthreads();  // both halves of the dK rows, and the dV rows, are in LDS
  store_rows<D>(role ? dk_rows : dv_rows, 0, 32, k0 + sub * 32, seg1, static_cast<bf16 *>(role ? a.dk : a.dv) + h * D,
                HD, lane);
  sum_wave_partials<D>(red, KV_NW / 2, part, tid);
}

hipError_t launch_attn_bwd_f32(const PlanDev &p, const AttnBwdArgs &a, int which, hipStream_t stream);

template <int D>
static hipError_t bwd_dq(const PlanDev &p, const AttnBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3((unsigned)p.num_fwd_blocks), dim3(64 * bwd::NWQ), 0, s, p, a);
  return hipGetLastError();
}
template <int D>
static hipError_t bwd_dkdv(const PlanDev &p, const AttnBwdArgs &a, hipStream_t s) {
  if (a.ds)
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true>), dim3((unsigned)p.num_bwd_blocks), dim3(64 * bwd::KV_NW), 0,
                       s, p, a);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false>), dim3((unsigned)p.num_bwd_blocks), dim3(64 * bwd::KV_NW), 0,
                       s, p, a);
  return hipGetLastError();
}

template <int D>
static hipError_t bwd_dq_ds(const PlanDev &p, const AttnBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(attn_bwd_dq_ds_kernel<D>, dim3((unsigned)p.num_fwd_blocks), dim3(64 * bwd::NWQ), 0, s, p, a);
  return hipGetLastError();
}

// which = kBwdDq: dQ-hat and D (a.ds null) or dQ-hat from the stored dS;
// which = kBwdDkdv: dK-hat and dV (reads D), writing dS when a.ds is set.
hipError_t launch_attn_bwd(int dtype, const PlanDev &p, const AttnBwdArgs &a, int which,
                           hipStream_t stream) {
  if (dtype == MMDIT_F32) return launch_attn_bwd_f32(p, a, which, stream);
  if (which == kBwdDq && a.ds) {
    if (p.head_dim == 64) return bwd_dq_ds<64>(p, a, stream);
    if (p.head_dim == 128) return bwd_dq_ds<128>(p, a, stream);
    return hipErrorInvalidValue;
  }
  if (p.head_dim == 64) return which == 0 ? bwd_dq<64>(p, a, stream) : bwd_dkdv<64>(p, a, stream);
  if (p.head_dim == 128) return which == 0 ? bwd_dq<128>(p, a, stream) : bwd_dkdv<128>(p, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace mmdit
