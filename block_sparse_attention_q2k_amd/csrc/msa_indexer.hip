// msa_indexer.hip -- the indexer's document-local top-16 block selection (the q2k the
// operator consumes), gfx950.
//
// What is computed (pull-request page "feat(minimax-m3): add SM100 MSA sparse attention
// with custom backward", Design: the indexer selects a document-local q2k; Supported
// scope: 4 index heads, head dim 128, block 128, top-k 16; Testing: truncated top-16).
// The pages leave the scoring rule open; the reading implemented here: for index head i
// and the query at document position p, the score of document-local block b <= p / 128 is
// the largest <IQ[t, i], IK[j, i]> over the keys j of block b with j <= p; the row lists
// the min(16, p / 128 + 1) blocks of highest score (ties to the smaller block id) in
// ascending order, -1 in the unused slots.
//
// Design (gfx950): one workgroup of 4 waves per (index head, 128-query block of a
// document); wave w owns queries 32w .. 32w + 31 of the block, whose index-Q rows it
// holds in registers for the whole walk.  The workgroup walks the causal key blocks
// 0 .. qb of the document in ascending order; each block's 128 index-K rows are staged in
// LDS (rows padded to 272 B: the 16-byte A-fragment reads of 16 rows hit all banks),
// double-buffered, the next block's rows in flight from HBM while the current one is
// scored.  Per block, a wave computes the 128 x 32 score tile as four 32 x 32 tiles
// S^T = K Q^T (32x32x16 MFMAs, fp32 accumulation), masks the keys past each query on
// the diagonal block, and takes each query's maximum over the 128 keys in registers; the
// query's running top-16 (score, block) list, sorted by descending score, also stays in
// registers, and a block enters it only with a strictly larger score than the 16th
// entry, so ties keep the earlier, smaller block id.
#include "msa_walk.h"

namespace msa {

constexpr int kIdxThreads = 256;
constexpr int kIdxRow = 272;  // padded LDS row of one key (256 B of bf16)

// Stages the 128 index-K rows of document-local key block b (rows beyond the document
// end as zeros) for index head i: thread tid moves 16-byte chunks tid, tid + 256, ...
// of the block's 2048; `v` carries them from the global loads to the LDS stores.
__device__ __forceinline__ void idx_load_block(u32x4 (&v)[8], const uint16_t *__restrict__ IK, int c0, int L, int b,
                                               int i, int tid) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = tid + k * kIdxThreads;  // chunk: row c / 16, 16 bytes c % 16
    const int key = b * kBlk + (c >> 4);
    v[k] = u32x4{0u, 0u, 0u, 0u};
    if (key < L) v[k] = *(const u32x4 *)(IK + ((size_t)(c0 + key) * kHI + i) * kD + (c & 15) * 8);
  }
}
__device__ __forceinline__ void idx_store_block(char *sK, const u32x4 (&v)[8], int tid) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = tid + k * kIdxThreads;
    *(u32x4 *)(sK + (c >> 4) * kIdxRow + (c & 15) * 16) = v[k];
  }
}

// Maximum of this lane's query (column l32) over the 128 keys of the staged block:
// four 32 x 32 tiles S^T[key][query] (keys 32 kt .. + 31), each from eight 32x32x16
// MFMAs with the key rows from LDS as A and the query rows q as B.  DIAG: keys past the
// query (key index > query index within the block, both block-relative) are ignored.
template <bool DIAG>
__device__ __forceinline__ float idx_block_max(const char *sK, const bf16x8 (&q)[8], int qrel, const WalkLane &w) {
  float best = -INFINITY;
  const char *rowbase = sK + w.l32 * kIdxRow + 16 * w.hi;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    bf16x8 a[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) a[ks] = *(const bf16x8 *)(rowbase + 32 * kt * kIdxRow + 32 * ks);
    const f32x16 st = tile32(a, q);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * kt + 8 * (r >> 2) + 4 * w.hi + (r & 3);
      const float s = (DIAG && key > qrel) ? -INFINITY : st[r];
      best = fmaxf(best, s);
    }
  }
  return fmaxf(best, __shfl_xor(best, 32));
}

__global__ void __launch_bounds__(kIdxThreads, 2)
idx_select_kernel(const uint16_t *__restrict__ IQ, const uint16_t *__restrict__ IK,
                  const int32_t *__restrict__ cu, const int32_t *__restrict__ cu_ws, int ndocs, int NB, int T,
                  int32_t *__restrict__ q2k) {
  __shared__ __attribute__((aligned(16))) char sK[2][kBlk * kIdxRow];
  const int i = blockIdx.x % kHI;
  const int gb = NB - 1 - (int)(blockIdx.x / kHI);  // the longest walks (late blocks) first
  const int d = upper_index(cu_ws, ndocs, gb * kBlk);
  const int qb = uniform(gb - cu_ws[d] / kBlk);
  const int c0 = cu[d], L = cu[d + 1] - c0;
  WalkLane w;
  walk_lane(w, threadIdx.x);
  const int tid = threadIdx.x;
  const int qrel = 32 * w.wave + w.l32;  // the lane's query within the block
  const int p = qb * kBlk + qrel;        // its document position
  const bool valid = p < L;
  bf16x8 q[8];  // B operand: query row qrel, dims 16 ks + 8 hi .. + 7
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    q[ks] = bf16x8{};
    if (valid) q[ks] = *(const bf16x8 *)(IQ + ((size_t)(c0 + p) * kHI + i) * kD + 16 * ks + 8 * w.hi);
  }
  float v[kTopk];
  int id[kTopk];
#pragma unroll
  for (int k = 0; k < kTopk; ++k) {
    v[k] = -INFINITY;
    id[k] = -1;
  }
  u32x4 stage[8];
  idx_load_block(stage, IK, c0, L, 0, i, tid);
  idx_store_block(sK[0], stage, tid);
  __syncthreads();
  for (int b = 0; b <= qb; ++b) {
    if (b < qb) idx_load_block(stage, IK, c0, L, b + 1, i, tid);
    const float s = b < qb ? idx_block_max<false>(sK[b & 1], q, qrel, w) : idx_block_max<true>(sK[b & 1], q, qrel, w);
    // insertion into the descending list (strictly larger scores only)
    const bool ins = s > v[kTopk - 1];
    if (__ballot(ins) != 0) {
      v[kTopk - 1] = ins ? s : v[kTopk - 1];
      id[kTopk - 1] = ins ? b : id[kTopk - 1];
#pragma unroll
      for (int k = kTopk - 1; k > 0; --k) {
        const bool up = v[k] > v[k - 1];
        const float tv = v[k];
        const int ti = id[k];
        v[k] = up ? v[k - 1] : v[k];
        id[k] = up ? id[k - 1] : id[k];
        v[k - 1] = up ? tv : v[k - 1];
        id[k - 1] = up ? ti : id[k - 1];
      }
    }
    if (b < qb) idx_store_block(sK[(b + 1) & 1], stage, tid);
    __syncthreads();
  }
  // ascending block ids, unused slots (-1) last: odd-even transposition sort
#pragma unroll
  for (int k = 0; k < kTopk; ++k) id[k] = id[k] < 0 ? INT32_MAX : id[k];
#pragma unroll
  for (int r = 0; r < kTopk; ++r) {
#pragma unroll
    for (int k = r & 1; k + 1 < kTopk; k += 2) {
      const int lo = min(id[k], id[k + 1]), hi = max(id[k], id[k + 1]);
      id[k] = lo;
      id[k + 1] = hi;
    }
  }
  if (valid && w.hi == 0) {
    int32_t *row = q2k + ((size_t)i * T + c0 + p) * kTopk;
#pragma unroll
    for (int k = 0; k < kTopk; k += 4)
      *(i32x4 *)(row + k) = i32x4{id[k] == INT32_MAX ? -1 : id[k], id[k + 1] == INT32_MAX ? -1 : id[k + 1],
                                  id[k + 2] == INT32_MAX ? -1 : id[k + 2], id[k + 3] == INT32_MAX ? -1 : id[k + 3]};
  }
}

namespace host {
hipError_t index_select(const void *IQ, const void *IK, const LayoutArgs &L, int32_t *q2k, hipStream_t s) {
  hipLaunchKernelGGL(idx_select_kernel, dim3((unsigned)(kHI * L.NB)), dim3(kIdxThreads), 0, s,
                     (const uint16_t *)IQ, (const uint16_t *)IK, L.cu, L.cu_ws, L.ndocs, L.NB, L.T, q2k);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
