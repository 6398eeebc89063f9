// Device helpers for the gfx950 kernels: vector types, bf16 packing, DPP
// reductions inside a row of 16 lanes, MFMA and LDS transpose-read wrappers.
//
// Lane layouts relied on (checked on gfx950 hardware):
//  * v_mfma_f32_32x32x16_bf16: A lane l holds row l%32 and eight k values
//    selected by (l/32, j); B lane l holds column l%32 with the same k
//    selection; accumulator register i of lane l is element
//    (row 8*(i/4) + 4*(l/32) + i%4, column l%32).
//  * ds_read_b64_tr_b16: in each group of 16 lanes, lane L fetches 4 bf16 at
//    its own address (row L/4 and columns 4*(L%4)..+3 of a 4x16 block) and
//    afterwards lane i holds column i of the block, rows 0..3.
//  * v_permlane32_swap(x, x) returns (x of lane l%32, x of lane l%32 + 32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace mmdit {

// True when the device blob is not the one the host plan describes (its
// header fingerprint differs): thread 0 flags it in the fault word and the
// caller exits before touching anything else. The fingerprint is read first,
// on its own, so no work-list entry of a foreign blob is ever read.
__device__ __forceinline__ bool blob_stale(const BlobGuard &g) {
  const uint64_t f = *g.blob_fingerprint;
  if (__builtin_expect(f == g.fingerprint, 1)) return false;
  if (threadIdx.x == 0) atomicOr(g.status, (uint32_t)MMDIT_DEVICE_FAULT_STALE_BLOB);
  return true;
}

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }

// 16-byte global / LDS accesses, as single vector loads and stores (a HIP
// uint4 struct copy splits into four 4-byte accesses in the IR).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ uint4 ld16(const T *p) {
  return __builtin_bit_cast(uint4, *reinterpret_cast<const u32x4 *>(p));
}
template <typename T>
__device__ __forceinline__ void st16(T *p, uint4 v) {
  *reinterpret_cast<u32x4 *>(p) = __builtin_bit_cast(u32x4, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte load straight into an MFMA operand (no struct round trip, so the
// load stays one vector access).
template <typename T>
__device__ __forceinline__ bf16x8 ld_bf16x8(const T *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void st_bf16x8(void *p, bf16x8 v) { *reinterpret_cast<bf16x8 *>(p) = v; }
__device__ __forceinline__ uint4 as_u4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

// fp32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x2 pack2(float a, float b) {
  bf16x2 r = {(bf16)a, (bf16)b};
  return r;
}

// DPP move inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W lanes (W = 2..64); every lane of a group gets
// the bitwise-same sum (each step adds two values symmetrically).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W >= 2 && W <= 64 && (W & (W - 1)) == 0, "group width");
  x += dpp<0xB1>(x);                      // quad_perm [1,0,3,2]
  if constexpr (W >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (W >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (W >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (W >= 32) x += __shfl_xor(x, 16);
  if constexpr (W >= 64) x += __shfl_xor(x, 32);
  return x;
}

// max/sum of x over lanes l and l^32 (the two halves of the wave).
__device__ __forceinline__ float half_max(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// sum of x over lanes l and l^16 (the two 16-lane rows of each half), in VALU.
__device__ __forceinline__ float row_pair_sum(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposed read of a 16(k) x 32(n) bf16 operand fragment from a row-major
// LDS matrix M[k][n] (row stride `ld` elements): returns, for lane l, the
// values M[k0 + kappa(l/32, j)][n0 + l%32], j = 0..7, where
// kappa(g, j) = 8*(j/4) + 4*g + j%4 -- the k order in which a 32x32
// accumulator holds its rows, so an accumulator converted to bf16 can be the
// other operand of the same product.
__device__ __forceinline__ bf16x8 lds_read_tr(const bf16 *m, int ld, int k0, int n0, int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int g = G >> 1, nh = G & 1;
  const bf16 *p = m + (k0 + 4 * g + (i >> 2)) * ld + n0 + nh * 16 + 4 * (i & 3);
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + 8 * ld));
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// ---------------------------------------------------------------------------
// Unpadded, XOR-swizzled LDS tiles filled by direct global->LDS loads.
// A tile row holds CPR 16-byte chunks; logical chunk c of row r sits at
// physical chunk c ^ swz(r). Swizzles by access pattern: ROWS for tiles read
// 16 bytes per lane down consecutive rows, TRANS for tiles read with
// ds_read_b64_tr_b16 (rows r..r+3 of a 4x16 block land in four different
// 64-byte bank groups), BOTH for tiles read both ways.
// ---------------------------------------------------------------------------
enum Swz { SWZ_ROWS = 0, SWZ_TRANS = 1, SWZ_BOTH = 2 };

// BOTH serves tiles read both ways; for 256-byte rows it was picked by
// measured gfx950 LDS throughput (about 205 B/clk per CU for row reads and
// 275 for transposed reads, against 180 / 205 for ROWS); shorter rows use ROWS.
template <int CPR, int SW>
__device__ __forceinline__ int swz(int r) {
  if constexpr (SW == SWZ_TRANS) return (4 * (r & 3)) & (CPR - 1);
  else if constexpr (SW == SWZ_BOTH && CPR == 16) return 4 * (r & 3) + 2 * ((r >> 2) & 1) + ((r >> 3) & 1);
  else return (((r & 7) << 1) | ((r >> 3) & 1)) & (CPR - 1);
}

// Element offset of (row r, element e) in a swizzled tile of D-element rows.
template <int D, int SW>
__device__ __forceinline__ int swz_off(int r, int e) {
  constexpr int CPR = D / 8;
  return r * D + (((e >> 3) ^ swz<CPR, SW>(r)) << 3) + (e & 7);
}

// Direct global -> LDS copies use the buffer form (MUBUF) of the load: the
// global form is FLAT-encoded, and while a FLAT access to LDS is in flight the
// compiler can only wait for all LDS reads at once (lgkmcnt(0)), which would
// serialise every LDS operand read with the MFMAs that consume it.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferFlags = 0x00020000;  // raw dword-granular buffer (gfx9 family)

// Buffer resource over [base, base + bytes); accesses past the end read 0.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufferFlags);
}

// SIZE-byte global -> LDS copy for every lane of the wave: lane l's bytes at
// rsrc + voffset land at lds_wave_base + SIZE*l (lds_wave_base wave-uniform).
template <int SIZE>
__device__ __forceinline__ void buf2lds(rsrc_t r, uint32_t voffset, void *lds_wave_base) {
  static_assert(SIZE == 4 || SIZE == 16, "dword or dwordx4");
  auto *lds = (__attribute__((address_space(3))) void *)lds_wave_base;
  if constexpr (SIZE == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voffset, 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voffset, 0, 0, 0);
}

// Wait until this wave's outstanding global (and global->LDS) loads are done.
__device__ __forceinline__ void wait_vmem() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wave's vector memory loads are outstanding.
// Loads complete in issue order, so this waits for all but the newest N.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
}

// Wait until this wave's LDS operations (reads returned, writes done) are
// complete; no barrier.
__device__ __forceinline__ void wait_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
}

// Workgroup barrier that waits only for this wave's LDS operations, so global
// (and global->LDS) loads in flight stay in flight across it. Global data a
// wave loaded for others must be covered by its own wait_vmem() before a
// barrier that precedes the readers.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The same barrier as a hard scheduling boundary: the compiler moves no
// instruction across it (keeps the two halves of a ping-pong schedule apart).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Scheduling hint for one basic block holding NM MFMAs whose A operands come
// from LDS: MFMA i (in program order) needs RA DS reads for i < NA and RB
// after. The block is ordered as a pipeline: the reads of the first DIST
// MFMAs, then each MFMA followed by the reads of the MFMA DIST places ahead,
// so LDS latency hides behind DIST MFMAs. Call it at the end of the block.
template <int NA, int RA, int RB>
__device__ constexpr int ds_reads_of(int j, int nm) {
  return j < NA ? RA : (j < nm ? RB : 0);
}
template <int I, int NM, int NA, int RA, int RB, int DIST>
__device__ __forceinline__ void pipeline_steps() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int r = ds_reads_of<NA, RA, RB>(I + DIST, NM);
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // DS reads
    pipeline_steps<I + 1, NM, NA, RA, RB, DIST>();
  }
}
template <int NM, int NA, int RA, int RB, int DIST>
__device__ __forceinline__ void pipeline_mfma_ds() {
  constexpr int pre = [] {
    int n = 0;
    for (int j = 0; j < DIST; ++j) n += ds_reads_of<NA, RA, RB>(j, NM);
    return n;
  }();
  __builtin_amdgcn_sched_group_barrier(0x100, pre, 0);
  pipeline_steps<0, NM, NA, RA, RB, DIST>();
}

// Direct global -> LDS loader of a swizzled D-wide tile of ROWS rows, shared
// by NW waves. Each wave-wide load fills 64/CPR consecutive rows; lane l of
// load u covers tile row r0 + u*RPL (r0 = first row of this lane) and
// physical chunk l % CPR, fetching the logical chunk that the swizzle puts
// there. Per-lane byte offsets (row and chunk parts) are computed once.
template <int D, int SW, int ROWS, int NW>
struct TileLoader {
  static constexpr int CPR = D / 8;
  static constexpr int RPL = 64 / CPR;          // rows per wave-wide load
  static constexpr int LOADS = ROWS / RPL / NW; // loads per wave
  static_assert(ROWS % (RPL * NW) == 0, "tile rows must split evenly over the waves");
  int lds0;               // element offset of this wave's first load (uniform)
  uint32_t off[LOADS];    // byte offset of the lane's row and logical chunk, per load
  uint32_t stride_b;      // bytes between source rows

  // row_stride in elements; ROWS rows of it must span under 4 GiB.
  __device__ __forceinline__ void init(int wave_uniform, int lane, int64_t row_stride) {
    stride_b = (uint32_t)(2 * row_stride);
    const int r0 = wave_uniform * LOADS * RPL + lane / CPR;
    lds0 = wave_uniform * LOADS * RPL * D;
    const int pc = lane % CPR;
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      off[u] = (uint32_t)(r0 + u * RPL) * stride_b + (uint32_t)(16 * (pc ^ swz<CPR, SW>(r0 + u * RPL)));
  }
  // Source rows kb0 + r for r < ROWS; base = element (0, 0) of the source at
  // the wanted head. Rows past last_row are not read and land as zeros: the
  // descriptor ends with the last valid row (a buffer load past a
  // descriptor's size returns zero words).
  __device__ __forceinline__ void issue(bf16 *tile, const bf16 *base, int kb0, int last_row) const {
    const char *b0 = reinterpret_cast<const char *>(base) + (uint64_t)(uint32_t)kb0 * stride_b;
    const int rows = last_row + 1 - kb0;
    const uint32_t bytes = rows <= 0 ? 0u : (uint32_t)((rows < ROWS ? rows : ROWS) - 1) * stride_b + 2 * D;
    const rsrc_t r = make_rsrc(b0, bytes);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) buf2lds<16>(r, off[u], tile + lds0 + u * RPL * D);
  }
};

// Four consecutive fp32 words at byte offset voffset of a buffer, into
// registers; words past the descriptor's size read as zero.
__device__ __forceinline__ f32x4 buf_load_f32x4(rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voffset, 0, 0));
}

// Swizzled counterpart of lds_read_tr (same fragment, same k order).
template <int D, int SW>
__device__ __forceinline__ bf16x8 lds_read_tr_swz(const bf16 *m, int k0, int n0, int lane) {
  const int G = lane >> 4, i = lane & 15;
  const int g = G >> 1, nh = G & 1;
  const int r = k0 + 4 * g + (i >> 2);
  const int e = n0 + nh * 16 + 4 * (i & 3);
  const bf16 *p0 = m + swz_off<D, SW>(r, e);
  const bf16 *p1 = m + swz_off<D, SW>(r + 8, e);
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p1);
  bf16x8 out;
  out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
  out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
  return out;
}

// Row of the 32x32 accumulator held in register i by lanes of half g.
__device__ __forceinline__ constexpr int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// Eight accumulator registers (starting at `base`) packed to bf16: the k
// fragment kappa(g, 0..7) of a 16-wide slice of the accumulator's rows.
__device__ __forceinline__ bf16x8 acc_to_bf16(const f32x16 &c, int base) {
  bf16x8 r;
  bf16x2 t0 = pack2(c[base + 0], c[base + 1]);
  bf16x2 t1 = pack2(c[base + 2], c[base + 3]);
  bf16x2 t2 = pack2(c[base + 4], c[base + 5]);
  bf16x2 t3 = pack2(c[base + 6], c[base + 7]);
  r[0] = t0[0]; r[1] = t0[1]; r[2] = t1[0]; r[3] = t1[1];
  r[4] = t2[0]; r[5] = t2[1]; r[6] = t3[0]; r[7] = t3[1];
  return r;
}

// Decode a tok_meta word: image flag, row, column and frame index.
__device__ __forceinline__ void tok_pos(int32_t meta, bool &img, int &row, int &col, int &frame) {
  img = meta < 0;
  row = (meta >> 16) & 0x7FFF;
  col = meta & 0x7FFF;
  frame = (meta >> 15) & 1;
}

// Position along the RoPE axis of pair p: pairs [0, fp) follow the frame,
// [fp, re) the row and [re, d/2) the column, re = fp + (d/2 - fp) / 2.
__device__ __forceinline__ int rope_pos(int p, int fp, int re, int row, int col, int frame) {
  return p < fp ? frame : (p < re ? row : col);
}

}  // namespace mmdit
