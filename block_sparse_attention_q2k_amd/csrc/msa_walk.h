// msa_walk.h -- pieces shared by the query-parallel kernels (forward, dQ).
//
// A work item of the plan is (index head i, queries t0 .. t0+n-1 of one document,
// n <= MSA_FWD_GROUP).  Each query ("unit": its 16 heads share one selection) lists
// up to 16 document-local key blocks.  The plan stores, per item, the union of those
// blocks in ascending order with the bit mask of the units that selected each block;
// the kernels walk that list, loading every block once per item.
#pragma once
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kWalkThreads = 256;               // 4 waves, one per SIMD
constexpr int kWalkWaves = kWalkThreads / 64;
constexpr int kWalkDims = kD / kWalkWaves;      // head dims owned by one wave (32)
constexpr int kWalkSlots = 16;                  // P / dS slots: active units per round

typedef __attribute__((address_space(1))) void walk_gvoid;
typedef __attribute__((address_space(3))) void walk_lvoid;

// Wave-uniform value of v (the compiler cannot see that an LDS load or a function of
// the wave index is the same in every lane; scalar registers avoid divergent control).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The k-th set bit of m.
__device__ __forceinline__ int nth_set_bit(uint32_t m, int k) {
  for (int j = 0; j < k; ++j) m &= m - 1;
  return __builtin_ctz(m);
}

// The bits of m that belong to the round starting at its r0-th set bit: set bits
// r0 .. r0 + slots - 1 (in ascending order).
__device__ __forceinline__ uint32_t round_bits(uint32_t m, int r0, int slots = kWalkSlots) {
  for (int k = 0; k < r0; ++k) m &= m - 1;
  uint32_t rest = m;
  for (int k = 0; k < slots && rest; ++k) rest &= rest - 1;
  return m ^ rest;
}

// LDS stores that the compiler does not see as LDS accesses.  The compiler makes every
// LDS store wait for all pending global->LDS copies (it cannot tell the buffers
// apart), which would expose the next block's copy at the first P / dS store of a
// step.  These stores only ever target buffers that no copy writes; the code that
// publishes them waits with lds_stores_done() before its barrier.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}
template <int OFF>
__device__ __forceinline__ void lds_store_b64(uint32_t addr, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF) : "memory");
}
__device__ __forceinline__ void lds_store_b32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_add_f32(uint32_t addr, float v) {
  asm volatile("ds_add_f32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
// s_waitcnt lgkmcnt(0): the asm stores above have reached LDS.
__device__ __forceinline__ void lds_stores_done() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that publishes LDS data only: waits for this wave's LDS operations
// (lgkmcnt(0)), not for its global loads or global->LDS copies still in flight, which
// __syncthreads() would also wait for.  The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  lds_stores_done();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(0) in a form the compiler's wait-count tracking understands.
__device__ __forceinline__ void walk_wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Asynchronous copy (global_load_lds_dwordx4) of one 32 KB K or V block -- 128 keys x
// 256 B of KV head kv starting at workspace row row0 -- into `dst` in the swz()
// layout.  Copy k of a wave fills 1 KB of LDS (4 rows); its lane l lands at byte
// 16 l of that KB, i.e. row r = 16 k + tid / 16 at physical chunk tid % 16, which
// holds logical chunk (tid % 16) ^ (r % 16) = (tid % 16) ^ (tid / 16 % 16): one lane
// offset serves every copy.
__device__ __forceinline__ void block_dma(char *dst, const uint16_t *__restrict__ X, size_t row0,
                                          int kv, int tid) {
  static_assert(kWalkThreads == 256, "16 rows per copy");
  constexpr int kCopies = 2048 / kWalkThreads;
  const int wave = tid >> 6;
  const char *src = (const char *)(X + (row0 * kHKV + kv) * kD);
  const uint32_t voff = (uint32_t)(((tid >> 4) * kHKV * kD + (((tid & 15) ^ ((tid >> 4) & 15)) * 8)) * 2);
  __attribute__((address_space(3))) char *base = (__attribute__((address_space(3))) char *)dst + wave * 1024;
#pragma unroll
  for (int k = 0; k < kCopies; ++k)
    __builtin_amdgcn_global_load_lds((const walk_gvoid *)(src + voff + k * 16 * kHKV * kD * 2),
                                     (walk_lvoid *)(base + k * kWalkThreads * 16), 16, 0, 0);
}

// Byte offset (without the 4096 B per 16-key tile) of the A fragment of keys
// 16 mt + l16, dims 32 kk + 8 g .. + 7 in a swz() block: row & 15 = l16, so the
// swizzled chunk (4 kk + g) ^ l16 splits into ((kk ^ l16 / 4) << 2) | (g ^ l16 % 4).
__device__ __forceinline__ uint32_t swz_frag(int kk, int l16, int g) {
  return (uint32_t)(l16 * 256 + ((((kk ^ (l16 >> 2)) << 2) | (g ^ (l16 & 3))) << 4));
}

// P / dS slots: [16 heads][128 keys] bf16 with rows padded to 272 B, so that both the
// 8-byte stores of the score layout (keys 16 mt + 4 g ..) and the 16-byte B-fragment
// reads (keys 32 kk + 8 g ..) spread over all 64 banks with offsets affine in mt, kk.
constexpr int kSlotRow = 272;
constexpr int kSlotBytes = 16 * kSlotRow;

// 16 query-head rows of token t (index head i): lane (head l16, g) gets dims
// 32 kk + 8 g + 0..7, the B operand of a 16x16x32 MFMA with the heads as columns.
__device__ __forceinline__ void load_rows16(bf16x8 (&f)[4], const uint16_t *__restrict__ X, int t,
                                            int i, int l16, int g) {
  const uint16_t *row = X + ((size_t)t * kH + kHPI * i + l16) * kD + 8 * g;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) f[kk] = *(const bf16x8 *)(row + 32 * kk);
}

// A operand slice of a transposed block copy Xt[kv][gb][dim][key]: lane (dim
// dim0 + l16, g) gets keys 32 kk + 8 g + 0..7.
__device__ __forceinline__ void load_tslice(bf16x8 (&f)[4], const uint16_t *__restrict__ Xt,
                                            size_t gblk, int dim0, int l16, int g) {
  const uint16_t *row = Xt + (gblk * kD + dim0 + l16) * kBlk + 8 * g;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) f[kk] = *(const bf16x8 *)(row + 32 * kk);
}

}  // namespace msa
