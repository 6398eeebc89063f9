// Adaptive LayerNorm modulation of the NR-MMDiT block, with the gated
// residual of the attention output fused in front of it:
//   z = x + gate * y        (y: the attention's output projection; optional)
//   h = (z - mean(z)) * rstd(z) * (1 + scale) + shift,  rstd = (var + eps)^(-1/2)
// with (shift, scale, gate) one fp32 row of the model width D per sample and
// per stream (text or image). The pages credit fused adaptive-normalisation
// and gating kernels in the NR-MMDiT (picx.dev summary "Mage-Flow: An
// Efficient Native-Resolution Foundation Model ...", section "Training
// Infrastructure"; findtube.ai transcript at [00:04:20]: normalisation and
// residual chains fused so that intermediates stay on chip); the formula is
// the DiT-style adaLN, which the pages do not print.
//
// Work split: one workgroup (4 waves) per plan chunk of <= 32 rows of one
// (sample, stream) range in the backward, two (one per half) in the forward,
// so a workgroup uses one modulation row.
// Thread t owns the column groups {4g .. 4g+3 : g = t + 256 j}: each load
// instruction of the workgroup covers one contiguous 2 KB (bf16) or 4 KB
// (fp32) stretch of a row. Rows are processed RB at a time; the row sums
// (mean, then the squared deviations, from registers) are reduced with DPP
// inside a wave and over the 4 waves through LDS in a fixed order, so every
// thread holds the same bits. The backward keeps per-thread column sums of
// dshift, dscale and dgate over its chunk and writes one partial row each; a
// second kernel adds each range's partials in chunk order (no atomics: the
// results are deterministic).
#include "device.h"
#include "internal.h"

namespace mmdit {
namespace {

constexpr int kThreads = 256;

// Token rows are moved with raw buffer instructions over the chunk's rows:
// loads past the chunk or past D read 0 and stores there are dropped, so no
// access sits behind a branch. (gfx950 counts loads and stores on one
// counter, so with the previous batch's stores pending the compiler still
// waits for every outstanding access at the top of a batch; the next batch's
// loads overlap the current batch's reductions and stores, and further
// latency is hidden by the other workgroups on the CU.)
constexpr uint32_t kNoAccess = 0x80000000u;  // voffset beyond every chunk resource

// Four consecutive elements: raw loaded form and fp32 values.
template <typename T>
struct Quad;
template <>
struct Quad<bf16> {
  typedef bf16x4 raw;
  __device__ static raw load(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
  }
  __device__ static void cvt(raw v, float (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)v[i];
  }
  __device__ static void store(rsrc_t r, uint32_t off, const float (&x)[4]) {
    const bf16x2 a = pack2(x[0], x[1]), b = pack2(x[2], x[3]);
    const raw v = {a[0], a[1], b[0], b[1]};
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, 0);
  }
};
template <>
struct Quad<float> {
  typedef f32x4 raw;
  __device__ static raw load(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
  }
  __device__ static void cvt(raw v, float (&x)[4]) {
    x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
  }
  __device__ static void store(rsrc_t r, uint32_t off, const float (&x)[4]) {
    const f32x4 v = {x[0], x[1], x[2], x[3]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 0);
  }
};

__device__ __forceinline__ void zero4(float (&x)[4]) { x[0] = x[1] = x[2] = x[3] = 0.f; }

// This thread's column groups of one fp32 modulation row of D values (zeros
// past D, or everywhere for a null row). The loads carry no branch, so the
// rows' loads are all in flight before the first value is used.
template <int G>
__device__ __forceinline__ void load_mod(const float *row, int D, const uint32_t (&moff)[G], float (&x)[G][4]) {
  const rsrc_t r = make_rsrc(row, row ? 4u * (uint32_t)D : 0u);
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const f32x4 v = buf_load_f32x4(r, moff[j]);
    x[j][0] = v[0]; x[j][1] = v[1]; x[j][2] = v[2]; x[j][3] = v[3];
  }
}

// One token tensor seen by a chunk: resource over its rows [r_begin, r_end)
// (row stride `stride` elements, D elements read per row) and the row pitch
// in bytes.
template <typename T>
struct Rows {
  rsrc_t r;
  uint32_t pitch;
  __device__ Rows(const void *base, int64_t stride, int r_begin, int r_end, int D) {
    const T *b = base ? static_cast<const T *>(base) + (int64_t)r_begin * stride : nullptr;
    const uint32_t bytes = base ? (uint32_t)(((int64_t)(r_end - r_begin - 1) * stride + D) * sizeof(T)) : 0u;
    r = make_rsrc(b, bytes);
    pitch = (uint32_t)(stride * sizeof(T));
  }
};

// Sums of v[0 .. NV) over the workgroup; every thread gets the same bits.
// buf: LDS [NV][4]. Consecutive calls must alternate between two buffers.
template <int NV>
__device__ __forceinline__ void block_sums(float (&v)[NV], float *buf, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = group_sum<64>(v[i]);
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < NV; ++i) buf[4 * i + wave] = v[i];
  lds_barrier();
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = (buf[4 * i] + buf[4 * i + 1]) + (buf[4 * i + 2] + buf[4 * i + 3]);
}

// Raw loads of the RB rows starting at chunk-relative row k0 (zeros past the
// chunk; coff[j] = this thread's column byte offset, or kNoAccess).
template <typename T, int G, int RB>
__device__ __forceinline__ void load_rows(typename Quad<T>::raw (&v)[RB][G], const Rows<T> &t, int k0,
                                          const uint32_t (&coff)[G]) {
#pragma unroll
  for (int rr = 0; rr < RB; ++rr)
#pragma unroll
    for (int j = 0; j < G; ++j)
      v[rr][j] = Quad<T>::load(t.r, coff[j] == kNoAccess ? kNoAccess : (uint32_t)(k0 + rr) * t.pitch + coff[j]);
}

// Mean and rstd of RB rows held in registers (two fixed-order passes).
template <int G, int RB>
__device__ __forceinline__ void row_stats(const float (&z)[RB][G][4], const bool (&ok)[G], float inv_d,
                                          float eps, float (&mean)[RB], float (&rstd)[RB], float (*red)[64],
                                          int &nb, int wave, int lane) {
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s += z[rr][j][i];
    mean[rr] = s;
  }
  block_sums<RB>(mean, red[nb++ & 1], wave, lane);
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    mean[rr] *= inv_d;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = ok[j] ? z[rr][j][i] - mean[rr] : 0.f;
        s = fmaf(c, c, s);
      }
    rstd[rr] = s;
  }
  block_sums<RB>(rstd, red[nb++ & 1], wave, lane);
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) rstd[rr] = rsqrtf(rstd[rr] * inv_d + eps);
}

}  // namespace

// Rows are loaded one batch ahead: the loads of batch k+1 are in flight while
// batch k is reduced and stored. Two workgroups share each plan chunk (its
// first and second half): the forward writes no partial sums, so smaller
// pieces only add workgroups in flight.
template <typename T, int G, bool RES>
__global__ __launch_bounds__(kThreads) void adaln_fwd_kernel(PlanDev p, AdalnFwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  constexpr int RB = 2;
  typedef typename Quad<T>::raw raw;
  __shared__ float red[2][64];
  int4 ch = p.mod_chunks[blockIdx.x >> 1];
  {
    const int mid = ch.x + (ch.y - ch.x + 1) / 2;
    if (blockIdx.x & 1) ch.x = mid; else ch.y = mid;
    if (ch.x >= ch.y) return;  // a one-row chunk has no second half
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = a.dim, nrows = ch.y - ch.x;
  const int64_t mrow = (int64_t)ch.z * D;
  const Rows<T> tx(a.x, a.x_stride, ch.x, ch.y, D), ty(a.y, a.y_stride, ch.x, ch.y, D);
  const Rows<T> tz(a.z, D, ch.x, ch.y, D), th(a.h, D, ch.x, ch.y, D);
  const rsrc_t tstat = make_rsrc(a.stats ? a.stats + ch.x : nullptr, a.stats ? 8u * (uint32_t)(ch.y - ch.x) : 0u);
  int col[G];
  bool ok[G];
  uint32_t coff[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    col[j] = 4 * (tid + kThreads * j);
    ok[j] = col[j] < D;
    coff[j] = ok[j] ? (uint32_t)(col[j] * sizeof(T)) : kNoAccess;
  }
  raw nx[RB][G], ny[RB][G];
  load_rows<T, G, RB>(nx, tx, 0, coff);
  if constexpr (RES) load_rows<T, G, RB>(ny, ty, 0, coff);
  float sh[G][4], sc[G][4], gt[G][4];
  {
    uint32_t moff[G];
#pragma unroll
    for (int j = 0; j < G; ++j) moff[j] = ok[j] ? 4u * (uint32_t)col[j] : kNoAccess;
    load_mod<G>(a.shift + mrow, D, moff, sh);
    load_mod<G>(a.scale + mrow, D, moff, sc);
    load_mod<G>(RES ? a.gate + mrow : nullptr, D, moff, gt);
  }
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[j][i] += 1.f;
  const float inv_d = 1.f / (float)D;
  int nb = 0;
  for (int k0 = 0; k0 < nrows; k0 += RB) {
    float z[RB][G][4], mean[RB], rstd[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int j = 0; j < G; ++j) {
        Quad<T>::cvt(nx[rr][j], z[rr][j]);
        if constexpr (RES) {
          float yv[4];
          Quad<T>::cvt(ny[rr][j], yv);
#pragma unroll
          for (int i = 0; i < 4; ++i) z[rr][j][i] = fmaf(gt[j][i], yv[i], z[rr][j][i]);
        }
      }
    load_rows<T, G, RB>(nx, tx, k0 + RB, coff);
    if constexpr (RES) load_rows<T, G, RB>(ny, ty, k0 + RB, coff);
    __builtin_amdgcn_sched_barrier(0);  // issue the next batch's loads here, not after the stores
    row_stats<G, RB>(z, ok, inv_d, a.eps, mean, rstd, red, nb, wave, lane);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const uint32_t o = coff[j] == kNoAccess ? kNoAccess : (uint32_t)(k0 + rr) * th.pitch + coff[j];
        if constexpr (RES) Quad<T>::store(tz.r, o, z[rr][j]);
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = fmaf((z[rr][j][i] - mean[rr]) * rstd[rr], sc[j][i], sh[j][i]);
        Quad<T>::store(th.r, o, hv);
      }
      // thread 0 stores the row's {mean, rstd} (dropped past the chunk, or
      // everywhere when no statistics are wanted)
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 st = {__float_as_uint(mean[rr]), __float_as_uint(rstd[rr])};
      __builtin_amdgcn_raw_buffer_store_b64(st, tstat, tid == 0 ? (int)(8 * (k0 + rr)) : (int)kNoAccess, 0, 0);
    }
  }
}

// Backward, also one row ahead (x, y, dh and dz of row k+1 in flight).
template <typename T, int G, bool RES>
__global__ __launch_bounds__(kThreads) void adaln_bwd_kernel(PlanDev p, AdalnBwdArgs a) {
  if (blob_stale(p.guard)) return;  // another pack's blob: touch nothing
  constexpr int RB = 1;
  typedef typename Quad<T>::raw raw;
  __shared__ float red[2][64];
  const int4 ch = p.mod_chunks[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = a.dim, nrows = ch.y - ch.x;
  const int64_t mrow = (int64_t)ch.z * D;
  const Rows<T> tx(a.x, a.x_stride, ch.x, ch.y, D), ty(a.y, a.y_stride, ch.x, ch.y, D);
  const Rows<T> tg(a.dh, a.dh_stride, ch.x, ch.y, D), te(a.dz, a.dz_stride, ch.x, ch.y, D);
  const Rows<T> tdx(a.dx, D, ch.x, ch.y, D), tdy(a.dy, D, ch.x, ch.y, D);
  const bool has_dz = a.dz != nullptr;
  int col[G];
  bool ok[G];
  uint32_t coff[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    col[j] = 4 * (tid + kThreads * j);
    ok[j] = col[j] < D;
    coff[j] = ok[j] ? (uint32_t)(col[j] * sizeof(T)) : kNoAccess;
  }
  // The chunk's forward statistics, row r in lane r, requested before the
  // first rows: a statistics load inside the loop would be issued behind the
  // next row's loads, and waiting for it would wait for them as well.
  static_assert(kModChunkRows <= 64, "one chunk row per lane");
  float2 st_lane = make_float2(0.f, 0.f);
  if (a.stats && lane < nrows) st_lane = a.stats[ch.x + lane];
  raw nx[RB][G], ny[RB][G], ng[RB][G], ne[RB][G];
  load_rows<T, G, RB>(nx, tx, 0, coff);
  if constexpr (RES) load_rows<T, G, RB>(ny, ty, 0, coff);
  load_rows<T, G, RB>(ng, tg, 0, coff);
  load_rows<T, G, RB>(ne, te, 0, coff);  // all zeros when dz is absent
  float sc[G][4], gt[G][4], ash[G][4], asc[G][4], agt[G][4];
  {
    uint32_t moff[G];
#pragma unroll
    for (int j = 0; j < G; ++j) moff[j] = ok[j] ? 4u * (uint32_t)col[j] : kNoAccess;
    load_mod<G>(a.scale + mrow, D, moff, sc);
    load_mod<G>(RES ? a.gate + mrow : nullptr, D, moff, gt);
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    zero4(ash[j]);
    zero4(asc[j]);
    zero4(agt[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[j][i] += 1.f;
  }
  // Everything above arrives together with the first row; waiting for all of
  // it here lets the loop's waits count the row loads alone.
  wait_vmem();
  const float inv_d = 1.f / (float)D;
  int nb = 0;
  for (int k0 = 0; k0 < nrows; k0 += RB) {
    raw cy[RB][G], ce[RB][G];
    float z[RB][G][4], g[RB][G][4], mean[RB], rstd[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int j = 0; j < G; ++j) {
        Quad<T>::cvt(nx[rr][j], z[rr][j]);
        Quad<T>::cvt(ng[rr][j], g[rr][j]);
        if constexpr (RES) {
          cy[rr][j] = ny[rr][j];
          float yv[4];
          Quad<T>::cvt(ny[rr][j], yv);
#pragma unroll
          for (int i = 0; i < 4; ++i) z[rr][j][i] = fmaf(gt[j][i], yv[i], z[rr][j][i]);
        }
        ce[rr][j] = ne[rr][j];
      }
    load_rows<T, G, RB>(nx, tx, k0 + RB, coff);
    if constexpr (RES) load_rows<T, G, RB>(ny, ty, k0 + RB, coff);
    load_rows<T, G, RB>(ng, tg, k0 + RB, coff);
    load_rows<T, G, RB>(ne, te, k0 + RB, coff);
    __builtin_amdgcn_sched_barrier(0);  // issue the next batch's loads here, not after the stores
    if (a.stats) {
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const int r = min(k0 + rr, nrows - 1);
        mean[rr] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(st_lane.x), r));
        rstd[rr] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(st_lane.y), r));
      }
    } else {
      row_stats<G, RB>(z, ok, inv_d, a.eps, mean, rstd, red, nb, wave, lane);
    }
    // z <- z_hat; column sums of dh and dh * z_hat; g <- dh * (1 + scale);
    // the row sums of g and g * z_hat.
    float s[2 * RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      float sg = 0.f, sgz = 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float zh = ok[j] ? (z[rr][j][i] - mean[rr]) * rstd[rr] : 0.f;
          const float d = g[rr][j][i];
          ash[j][i] += d;
          asc[j][i] = fmaf(d, zh, asc[j][i]);
          const float gg = d * sc[j][i];
          z[rr][j][i] = zh;
          g[rr][j][i] = gg;
          sg += gg;
          sgz = fmaf(gg, zh, sgz);
        }
      s[2 * rr] = sg;
      s[2 * rr + 1] = sgz;
    }
    block_sums<2 * RB>(s, red[nb++ & 1], wave, lane);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const float mg = s[2 * rr] * inv_d, mgz = s[2 * rr + 1] * inv_d;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d[4], e[4];
        Quad<T>::cvt(ce[rr][j], e);
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = rstd[rr] * (g[rr][j][i] - mg - z[rr][j][i] * mgz) + e[i];
        const uint32_t o = coff[j] == kNoAccess ? kNoAccess : (uint32_t)(k0 + rr) * tdx.pitch + coff[j];
        Quad<T>::store(tdx.r, o, d);
        if constexpr (RES) {
          float yv[4], dyv[4];
          Quad<T>::cvt(cy[rr][j], yv);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            agt[j][i] = fmaf(d[i], yv[i], agt[j][i]);
            dyv[i] = gt[j][i] * d[i];
          }
          Quad<T>::store(tdy.r, o, dyv);
        }
      }
    }
  }
  (void)has_dz;
  float *part = a.partials + (int64_t)blockIdx.x * 3 * D;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    if (!ok[j]) continue;
    const f32x4 v0 = {ash[j][0], ash[j][1], ash[j][2], ash[j][3]};
    const f32x4 v1 = {asc[j][0], asc[j][1], asc[j][2], asc[j][3]};
    *reinterpret_cast<f32x4 *>(part + col[j]) = v0;
    *reinterpret_cast<f32x4 *>(part + D + col[j]) = v1;
    if constexpr (RES) {
      const f32x4 v2 = {agt[j][0], agt[j][1], agt[j][2], agt[j][3]};
      *reinterpret_cast<f32x4 *>(part + 2 * D + col[j]) = v2;
    }
  }
}

// Grid: x = (range, 64-column block), y = which sum (0 dshift, 1 dscale,
// 2 dgate). Wave w adds chunks c0 + w, c0 + w + 4, ... of the range for its
// block's 64 columns; the four wave sums are then added in wave order. The
// split depends only on the plan, so the result is the same on every run.
__global__ __launch_bounds__(256) void adaln_reduce_kernel(BlobGuard guard, const int32_t *ranges,
                                                           const float *part, int D, float *o0, float *o1,
                                                           float *o2) {
  if (blob_stale(guard)) return;  // another pack's blob: touch nothing
  __shared__ float red[4][64];
  const int nxb = (D + 63) / 64;
  const int r = blockIdx.x / nxb, k = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = (blockIdx.x % nxb) * 64 + lane;
  const int c0 = ranges[r], c1 = ranges[r + 1];
  float s = 0.f;
  if (c < D) {
    const float *src = part + (int64_t)k * D + c;
    const int64_t step = 3 * (int64_t)D;
    // Up to 32 loads in flight per wave (every chunk of a range of up to 128
    // in one round trip), added in chunk order.
    constexpr int U = 32;
    for (int q = c0 + w; q < c1; q += 4 * U) {
      float t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) t[u] = q + 4 * u < c1 ? src[(int64_t)(q + 4 * u) * step] : 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (q + 4 * u < c1) s += t[u];
    }
  }
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && c < D) {
    float *out = k == 0 ? o0 : (k == 1 ? o1 : o2);
    out[(int64_t)r * D + c] = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
  }
}

namespace {

// Column groups per thread: ceil(D / 1024) rounded up to an instantiated size.
int groups_for(int D) {
  const int g = (D + 4 * kThreads - 1) / (4 * kThreads);
  return g <= 4 ? g : (g <= 6 ? 6 : 8);
}

template <typename T, int G>
hipError_t fwd_g(const PlanDev &p, const AdalnFwdArgs &a, hipStream_t s) {
  const dim3 grid(2u * (unsigned)p.num_mod_chunks);
  if (a.y)
    hipLaunchKernelGGL((adaln_fwd_kernel<T, G, true>), grid, dim3(kThreads), 0, s, p, a);
  else
    hipLaunchKernelGGL((adaln_fwd_kernel<T, G, false>), grid, dim3(kThreads), 0, s, p, a);
  return hipGetLastError();
}

template <typename T, int G>
hipError_t bwd_g(const PlanDev &p, const AdalnBwdArgs &a, hipStream_t s) {
  if (a.y)
    hipLaunchKernelGGL((adaln_bwd_kernel<T, G, true>), dim3(p.num_mod_chunks), dim3(kThreads), 0, s, p, a);
  else
    hipLaunchKernelGGL((adaln_bwd_kernel<T, G, false>), dim3(p.num_mod_chunks), dim3(kThreads), 0, s, p, a);
  return hipGetLastError();
}

template <typename T>
hipError_t fwd_t(const PlanDev &p, const AdalnFwdArgs &a, hipStream_t s) {
  switch (groups_for(a.dim)) {
    case 1: return fwd_g<T, 1>(p, a, s);
    case 2: return fwd_g<T, 2>(p, a, s);
    case 3: return fwd_g<T, 3>(p, a, s);
    case 4: return fwd_g<T, 4>(p, a, s);
    case 6: return fwd_g<T, 6>(p, a, s);
    case 8: return fwd_g<T, 8>(p, a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t bwd_t(const PlanDev &p, const AdalnBwdArgs &a, hipStream_t s) {
  switch (groups_for(a.dim)) {
    case 1: return bwd_g<T, 1>(p, a, s);
    case 2: return bwd_g<T, 2>(p, a, s);
    case 3: return bwd_g<T, 3>(p, a, s);
    case 4: return bwd_g<T, 4>(p, a, s);
    case 6: return bwd_g<T, 6>(p, a, s);
    case 8: return bwd_g<T, 8>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_adaln_fwd(int dtype, const PlanDev &p, const AdalnFwdArgs &a, hipStream_t stream) {
  if (a.dim < 4 || a.dim > kAdalnMaxDim || a.dim % 4) return hipErrorInvalidValue;
  return dtype == MMDIT_BF16 ? fwd_t<bf16>(p, a, stream) : fwd_t<float>(p, a, stream);
}

hipError_t launch_adaln_bwd(int dtype, const PlanDev &p, const AdalnBwdArgs &a, hipStream_t stream) {
  if (a.dim < 4 || a.dim > kAdalnMaxDim || a.dim % 4) return hipErrorInvalidValue;
  return dtype == MMDIT_BF16 ? bwd_t<bf16>(p, a, stream) : bwd_t<float>(p, a, stream);
}

hipError_t launch_adaln_reduce(const PlanDev &p, const float *partials, int dim, float *out0, float *out1,
                               float *out2, hipStream_t stream) {
  const dim3 grid((unsigned)((dim + 63) / 64) * 2u * (unsigned)p.num_samples, out2 ? 3 : 2);
  hipLaunchKernelGGL(adaln_reduce_kernel, grid, dim3(256), 0, stream, p.guard, p.mod_ranges, partials, dim,
                     out0, out1, out2);
  return hipGetLastError();
}

}  // namespace mmdit
