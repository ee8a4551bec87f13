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

constexpr int kWalkThreads = 256;

// Wave-uniform value of v (the compiler cannot see that an LDS load or a function of
// the wave index is the same in every lane; scalar registers avoid divergent control).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The k-th set bit of m.
__device__ __forceinline__ int nth_set_bit(uint32_t m, int k) {
  for (int j = 0; j < k; ++j) m &= m - 1;
  return __builtin_ctz(m);
}

// 32 KB K or V block (128 keys x 256 B of one KV head) into registers: thread tid
// holds rows tid/16 + 16k, chunk tid%16, k = 0..7.
__device__ __forceinline__ void block_load(u32x4 (&pre)[8], const uint16_t *__restrict__ X,
                                           size_t row0, int kv, int tid) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = (tid >> 4) + 16 * k, c = tid & 15;
    pre[k] = *(const u32x4 *)(X + ((row0 + r) * kHKV + kv) * kD + c * 8);
  }
}
__device__ __forceinline__ void block_store(const u32x4 (&pre)[8], char *dst, int tid) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = (tid >> 4) + 16 * k, c = tid & 15;
    *(u32x4 *)(dst + swz(r, c * 16)) = pre[k];
  }
}

// 16 query-head rows of token t (index head i): lane (head l16, g) gets dims
// 32 kk + 8 g + 0..7, the B operand of a 16x16x32 MFMA with the heads as columns.
__device__ __forceinline__ void load_rows16(bf16x8 (&f)[4], const uint16_t *__restrict__ X, int t,
                                            int i, int l16, int g) {
  const uint16_t *row = X + ((size_t)t * kH + kHPI * i + l16) * kD + 8 * g;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) f[kk] = *(const bf16x8 *)(row + 32 * kk);
}

}  // namespace msa
