// msa_walk.h -- pieces shared by the query-parallel kernels (forward, dQ).
//
// A work item of the plan is (index head i, queries t0 .. t0+n-1 of one document,
// n <= MSA_FWD_GROUP).  Each query ("unit": its 16 heads share one selection) lists
// up to 16 document-local key blocks.  The plan stores, per item, the union of those
// blocks in ascending order with the bit mask of the units that selected each block;
// the kernels walk that list, loading every block once per item.
//
// Both kernels split a block's work over 4 waves the same way: wave w owns keys
// [32w, 32w + 32) of the score-like tiles (32 x 32 tiles of keys x (2 units x 16
// heads), 32x32x16 MFMAs with the key rows in registers and the units' rows from LDS)
// and head dims [32w, 32w + 32) of the accumulating products (16x16x32 MFMAs, the
// transposed block rows in registers, the per-unit tiles from LDS slots).  The dQ
// kernel's 4 waves (one per SIMD) do both; the forward gives each to a role of its own
// (4 score waves and 4 product waves, two waves per SIMD).
#pragma once
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kWalkThreads = 256;  // 4 waves
constexpr int kWalkWaves = kWalkThreads / 64;

// Per-unit LDS slots ([16 heads][128 keys] bf16, P or dS) with rows padded to 272 B, so
// that the 16-byte B-fragment reads (keys 32 kk + 8 g .., 16 rows) spread over all
// banks.  Slots are 32 B apart beyond their size; the pad must keep every slot 16-byte
// aligned (the fragment reads are 16-byte reads: an 8-byte pad made half of them
// unaligned and the walks about 20 % slower), its size beyond that measured neutral.
constexpr int kSlotRow = 272;
constexpr int kSlotBytes = 16 * kSlotRow;
constexpr int kSlotStride = kSlotBytes + 32;

// Unit rows (a unit's 16 head rows of 256 B) in LDS with rows padded to 272 B: the 16
// lanes reading one 16-byte chunk of 16 rows cover all banks, and a fragment's offset
// within the row is the immediate offset of its read.
constexpr int kUnitRow = 272;

// Per-lane coordinates of the walk.
struct WalkLane {
  int tid, lane, wave, l16, g, l32, hi;
  uint32_t roff[8];  // swizzled byte offset, within a unit row, of the chunk of k-step ks
};

__device__ __forceinline__ void walk_lane(WalkLane &w, int tid) {
  w.tid = tid;
  w.lane = tid & 63;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  w.l16 = w.lane & 15;
  w.g = w.lane >> 4;
  w.l32 = w.lane & 31;
  w.hi = w.lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) w.roff[ks] = (uint32_t)(((2 * ks + w.hi) ^ w.l16) << 4);
}

// Wave-uniform value of v (the compiler cannot see that an LDS load or a function of
// the wave index is the same in every lane; scalar registers avoid divergent control).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The k-th set bit of m.
__device__ __forceinline__ int nth_set_bit(uint32_t m, int k) {
  for (int j = 0; j < k; ++j) m &= m - 1;
  return __builtin_ctz(m);
}

// Next unit of a (uniform, nonzero) unit mask, removed from it.
__device__ __forceinline__ int pop_unit(uint32_t &mr) {
  const int u = __builtin_ctz(mr);
  mr &= mr - 1;
  return u;
}

// The bits of m that belong to the round starting at its r0-th set bit: set bits
// r0 .. r0 + slots - 1 (in ascending order).
__device__ __forceinline__ uint32_t round_bits(uint32_t m, int r0, int slots) {
  for (int k = 0; k < r0; ++k) m &= m - 1;
  uint32_t rest = m;
  for (int k = 0; k < slots && rest; ++k) rest &= rest - 1;
  return m ^ rest;
}

// Bit mask of the units u in [0, 16) whose query (document position p0 + u) lies in
// block b: the units for which b is the diagonal block.
__device__ __forceinline__ uint32_t diag_units(int p0, int b) {
  const int lo = max(0, b * kBlk - p0), hi = min(15, b * kBlk + kBlk - 1 - p0);
  return lo > hi ? 0u : ((2u << hi) - 1u) & ~((1u << lo) - 1u);
}

// s_waitcnt vmcnt(n) (n < 64) with no wait on the other counters.
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)

// Workgroup barrier that publishes LDS data only: waits for this wave's LDS operations
// (lgkmcnt(0)), not for its global loads still in flight, which __syncthreads() would
// also wait for.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Rows [0, nrows) (nrows <= MAXROWS) of 256 B, row r at src + (r / 16) * unit_stride +
// (r % 16) * 256 bytes (16 head rows per unit), into LDS by NT threads.  PADDED: row r
// at dst + 272 r, chunks in order; otherwise row r at dst + 256 r with chunk c stored at
// c ^ (r % 16).  All of a thread's loads are issued before its first store, so the
// copy costs one load latency, not one per row.
template <int NT, int MAXROWS, bool PADDED>
__device__ __forceinline__ void rows_to_lds(char *dst, const char *src, size_t unit_stride, int nrows, int tid) {
  constexpr int kIter = (MAXROWS * 16 + NT - 1) / NT;
  const int q = tid & 15;
  u32x4 v[kIter];
#pragma unroll
  for (int k = 0; k < kIter; ++k) {
    const int r = (tid >> 4) + k * (NT / 16);
    if (r < nrows)
      v[k] = *(const u32x4 *)(src + (size_t)(r >> 4) * unit_stride + (r & 15) * 256 +
                              (PADDED ? q << 4 : (q ^ (r & 15)) << 4));
  }
#pragma unroll
  for (int k = 0; k < kIter; ++k) {
    const int r = (tid >> 4) + k * (NT / 16);
    if (r < nrows) *(u32x4 *)(dst + r * (PADDED ? kUnitRow : 256) + q * 16) = v[k];
  }
}

// A operand of a 32 x 32 tile: key rows 32w + l32 of workspace block gblk (= kv * NB +
// block) of the row-fragment copy X, dims 16 ks + 8 hi .. + 7: one contiguous 1 KB per
// k-step.
__device__ __forceinline__ void load_key_rows(bf16x8 (&k)[8], const uint16_t *__restrict__ X, size_t gblk,
                                              const WalkLane &w) {
  const uint16_t *f = X + gblk * kFragBlock + (w.wave * 8 * 64 + w.lane) * 8;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) k[ks] = *(const bf16x8 *)(f + ks * 512);
}

// Half H (k-steps 4 H .. 4 H + 3) of load_key_rows.
template <int H>
__device__ __forceinline__ void load_key_rows_half(bf16x8 (&k)[8], const uint16_t *__restrict__ X, size_t gblk,
                                                   const WalkLane &w) {
  const uint16_t *f = X + gblk * kFragBlock + (w.wave * 8 * 64 + w.lane) * 8;
#pragma unroll
  for (int ks = 4 * H; ks < 4 * H + 4; ++ks) k[ks] = *(const bf16x8 *)(f + ks * 512);
}

// A operand of the 16x16x32 products from the transposed-fragment copy Xt: lane (dim
// dim0 + l16, g) gets keys 32 kk + 8 g + 0..7 of block gblk (dim0 a multiple of 16).
__device__ __forceinline__ void load_tslice(bf16x8 (&f)[4], const uint16_t *__restrict__ Xt, size_t gblk,
                                            int dim0, const WalkLane &w) {
  const uint16_t *t = Xt + gblk * kFragBlock + ((dim0 >> 4) * 4 * 64 + w.lane) * 8;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) f[kk] = *(const bf16x8 *)(t + kk * 512);
}

// B operand of a 32 x 32 tile for the pair (u0, u1) from unit rows in LDS (rows_to_lds,
// swizzled layout): lane l32 < 16 reads unit u0, the others u1; f[ks] = row[head l16][dims
// 16 ks + 8 hi .. + 7].
__device__ __forceinline__ void load_pair_rows(bf16x8 (&f)[8], const char *s, int u0, int u1,
                                               const WalkLane &w) {
  const char *row = s + (((w.l32 < 16) ? u0 : u1) * 16 + w.l16) * 256;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) f[ks] = *(const bf16x8 *)(row + w.roff[ks]);
}

// load_pair_rows for unit rows in the padded layout (rows_to_lds with PADDED).
__device__ __forceinline__ void load_pair_rows_padded(bf16x8 (&f)[8], const char *s, int u0, int u1,
                                                      const WalkLane &w) {
  const char *row = s + (((w.l32 < 16) ? u0 : u1) * 16 + w.l16) * kUnitRow + 16 * w.hi;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) f[ks] = *(const bf16x8 *)(row + 32 * ks);
}

// 32 x 32 tile t = A B over 128 dims: t[r] = tile[key 32w + 8 (r/4) + 4 hi + r%4][column
// l32], column = (pair half l32 / 16, head l32 % 16).
__device__ __forceinline__ f32x16 tile32(const bf16x8 (&a)[8], const bf16x8 (&b)[8]) {
  f32x16 t;
#pragma unroll
  for (int r = 0; r < 16; ++r) t[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) t = mfma32(a[ks], b[ks], t);
  return t;
}

// Byte offset, within a slot, of the 8 bytes this lane stores for register group j of a
// tile (row l16, keys 32w + 8 j + 4 hi .. + 3): add 16 j.
__device__ __forceinline__ uint32_t slot_store_offset(const WalkLane &w) {
  return (uint32_t)(w.l16 * kSlotRow + (32 * w.wave + 4 * w.hi) * 2);
}

// B operand of the 16x16x32 products from slot s: keys 32 kk + 8 g .. + 7 of row l16.
__device__ __forceinline__ void load_slot(bf16x8 (&f)[4], const char *slots, int s, const WalkLane &w) {
  const char *row = slots + s * kSlotStride + w.l16 * kSlotRow + 16 * w.g;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) f[kk] = *(const bf16x8 *)(row + 64 * kk);
}

}  // namespace msa
