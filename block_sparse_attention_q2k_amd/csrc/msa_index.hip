// msa_index.hip -- HBM-bound steps of the MSA path: K/V workspace alignment, the
// q2k -> k2q CSR inversion, the forward plan, the backward task tables, delta
// preprocessing, pool zeroing and gradient finalization.
//
// Operator reference: "feat(minimax-m3): add SM100 MSA sparse attention with custom
// backward" (Design, Custom kernel) and the msa_backward_sm100 API page (module
// summary, run_backward).
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// ------------------------------------------------------------------ generic fill
__global__ void fill_u32_kernel(uint32_t *__restrict__ p, size_t n, uint32_t v) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  // 16-byte stores for the bulk, words for the tail
  size_t n4 = n / 4;
  u32x4 vv = {v, v, v, v};
  for (size_t k = i; k < n4; k += stride) ((u32x4 *)p)[k] = vv;
  for (size_t k = n4 * 4 + i; k < n; k += stride) p[k] = v;
}

// ------------------------------------------------------------------ K/V alignment
// Both workspace copies of one (block, KV head, tensor) per workgroup: the block's 128
// rows (zero past the document's end) are read once, coalesced, into LDS and written out
// as row fragments and as transposed fragments, each with contiguous 16-byte stores.
__global__ void __launch_bounds__(256)
align_blocks_kernel(const u32x4 *__restrict__ K, const u32x4 *__restrict__ V, const int32_t *__restrict__ cu,
                    const int32_t *__restrict__ cu_ws, int ndocs, int NB, uint16_t *__restrict__ Kw,
                    uint16_t *__restrict__ Vw, uint16_t *__restrict__ Kt, uint16_t *__restrict__ Vt) {
  __shared__ uint32_t tile[128 * 65];  // 128 keys x 128 dims bf16, rows padded to 260 B
  const int gb = blockIdx.x, kv = blockIdx.y, tid = threadIdx.x;
  const u32x4 *X = blockIdx.z ? V : K;
  const int d = upper_index(cu_ws, ndocs - 1, gb * kBlk);
  const int p0 = gb * kBlk - cu_ws[d], len = cu[d + 1] - cu[d], t0 = cu[d];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int id = tid + 256 * k, key = id >> 4, c = id & 15;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (p0 + key < len) v = X[((size_t)(t0 + p0 + key) * kHKV + kv) * 16 + c];
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[key * 65 + 4 * c + q] = v[q];
  }
  __syncthreads();
  const size_t fb = ((size_t)kv * NB + gb) * kFragBlock;
  uint16_t *Yw = (blockIdx.z ? Vw : Kw) + fb, *Yt = (blockIdx.z ? Vt : Kt) + fb;
#pragma unroll
  for (int k = 0; k < 8; ++k) {  // row fragments: chunk j holds key, dims dim .. dim + 7
    const int j = tid + 256 * k;
    const int key = ((j >> 9) << 5) | (j & 31), dim = (((j >> 6) & 7) << 4) | (((j >> 5) & 1) << 3);
    const uint32_t *src = tile + key * 65 + (dim >> 1);
    *(u32x4 *)(Yw + 8 * j) = u32x4{src[0], src[1], src[2], src[3]};
  }
  const uint16_t *t16 = (const uint16_t *)tile;
#pragma unroll
  for (int k = 0; k < 8; ++k) {  // transposed fragments: 8 keys of one dim per chunk
    const int id = tid + 256 * k, dim = id >> 4, c = id & 15;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)t16[(8 * c + 2 * q) * 130 + dim] | ((uint32_t)t16[(8 * c + 2 * q + 1) * 130 + dim] << 16);
    *(u32x4 *)(Yt + frag_t_off(8 * c, dim)) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ------------------------------------------------------------------ q2k membership
// Member blocks of one (index head, query) row: ids in [0, blk_t], first listing only.
// Returns a 16-bit mask of member slots and ORs precondition flags into *flags.
__device__ inline uint32_t member_mask(const int32_t *__restrict__ row, int blk_t, int32_t *ids,
                                       int *flags) {
  const i32x4 *r4 = (const i32x4 *)row;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    i32x4 v = r4[q];
    ids[4 * q + 0] = v[0];
    ids[4 * q + 1] = v[1];
    ids[4 * q + 2] = v[2];
    ids[4 * q + 3] = v[3];
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kTopk; ++j) {
    int b = ids[j];
    bool ok = (b >= 0) && (b <= blk_t);
    if (b != -1 && !ok) *flags |= MSA_Q2K_OUT_OF_RANGE;
    bool dup = false;
#pragma unroll
    for (int jj = 0; jj < j; ++jj) dup |= (ids[jj] == b);
    if (ok && dup) *flags |= MSA_Q2K_DUPLICATE;
    if (ok && !dup) m |= 1u << j;
  }
  return m;
}

// CSR count (pass 0) and fill (pass 1).  Workgroup (chunk, i) handles 256 consecutive
// queries of index head i.  Its rows i * NB + [gb_lo, gb_hi] span at most the blocks of
// the documents it touches; when that span fits in LDS the workgroup first counts per
// row in LDS and issues one global atomic per touched row (the sink and diagonal rows
// are hit by every query of a document), else every slot goes to global memory.
constexpr int kCsrSpan = 4096;
template <int kPass>
__global__ void __launch_bounds__(256)
csr_kernel(const int32_t *__restrict__ q2k, const int32_t *__restrict__ cu,
           const int32_t *__restrict__ cu_ws, int ndocs, int T, int NB,
           int32_t *__restrict__ counter, int32_t *__restrict__ cols, int32_t *__restrict__ status) {
  __shared__ int32_t hist[kCsrSpan];
  __shared__ int32_t base[kPass == 1 ? kCsrSpan : 1];
  const int i = blockIdx.y, tid = threadIdx.x;
  const int t_first = blockIdx.x * 256, t_last = min(T, t_first + 256) - 1;
  const int t = t_first + tid;
  const bool active = t <= t_last;
  int d = 0, pos = 0;
  if (active) {
    d = upper_index(cu, ndocs - 1, t);
    pos = t - cu[d];
  }
  const int d0 = upper_index(cu, ndocs - 1, t_first), d1 = upper_index(cu, ndocs - 1, t_last);
  const int gb_lo = cu_ws[d0] / kBlk;
  const int gb_hi = (cu_ws[d1] + (t_last - cu[d1])) / kBlk;
  const int span = gb_hi - gb_lo + 1;
  const bool local = span <= kCsrSpan;
  int32_t ids[kTopk];
  uint32_t m = 0;
  int flags = 0;
  if (active) m = member_mask(q2k + ((size_t)i * T + t) * kTopk, pos / kBlk, ids, &flags);
  if (kPass == 0 && flags) atomicOr(status, flags);
  const int gb0 = active ? cu_ws[d] / kBlk : 0;
  const int rbase = i * NB;
  if (!local) {
#pragma unroll
    for (int j = 0; j < kTopk; ++j) {
      if (!((m >> j) & 1)) continue;
      const int r = rbase + gb0 + ids[j];
      if (kPass == 0) atomicAdd(&counter[r], 1);
      else cols[atomicAdd(&counter[r], 1)] = t;
    }
    return;
  }
  for (int k = tid; k < span; k += 256) hist[k] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTopk; ++j)
    if ((m >> j) & 1) atomicAdd(&hist[gb0 + ids[j] - gb_lo], 1);
  __syncthreads();
  for (int k = tid; k < span; k += 256) {
    const int c = hist[k];
    if (kPass == 0) {
      if (c) atomicAdd(&counter[rbase + gb_lo + k], c);
    } else {
      base[k] = c ? atomicAdd(&counter[rbase + gb_lo + k], c) : 0;
      hist[k] = 0;
    }
  }
  if (kPass == 0) return;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTopk; ++j) {
    if (!((m >> j) & 1)) continue;
    const int k = gb0 + ids[j] - gb_lo;
    cols[base[k] + atomicAdd(&hist[k], 1)] = t;
  }
}

// Single-workgroup exclusive scan of n counts: out[0..n] (out[n] = total).  If
// `copy` is non-null it receives out[0..n-1] as well.  If `tiles` is set the scanned
// quantity is ceil(in / 8).
__global__ void __launch_bounds__(1024)
scan_kernel(const int32_t *__restrict__ in, int n, int tiles, int32_t *__restrict__ out,
            int32_t *__restrict__ copy) {
  __shared__ int32_t part[1024];
  int tid = threadIdx.x, nt = blockDim.x;
  int per = (n + nt - 1) / nt;
  int lo = min(n, tid * per), hi = min(n, lo + per);
  int s = 0;
  for (int k = lo; k < hi; ++k) s += tiles ? (in[k] + kTileQ - 1) / kTileQ : in[k];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {  // Hillis-Steele inclusive scan
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int k = lo; k < hi; ++k) {
    int v = tiles ? (in[k] + kTileQ - 1) / kTileQ : in[k];  // read before `copy` may alias `in`
    out[k] = run;
    if (copy) copy[k] = run;
    run += v;
  }
  if (tid == nt - 1) out[n] = part[nt - 1];
}

// Row lengths of the CSR from its row pointer.
__global__ void row_len_kernel(const int32_t *__restrict__ row_ptr, int n, int32_t *__restrict__ len) {
  int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < n) len[r] = row_ptr[r + 1] - row_ptr[r];
}

// ------------------------------------------------------------------ forward plan
// plan layout (int32): [0] items, [1] groups per head G, [2] Gmax; items {i, t0, n, doc}
// at [16 + 4p]; walk-list lengths at PlanView::len; walk lists (block, unit mask) at
// PlanView::lists + 2 * kPlanMaxList * p; aux: gstart [ndocs+1], group info {t0,n,d,_}
// x Gmax, cost [4 x Gmax].

// Walk list of one item (one workgroup of 256 threads per item): its queries' member
// blocks in ascending order with the mask of queries selecting each.  The <= 512
// (block, query) keys are bitonic-sorted in LDS; the first key of each block run emits
// (block, OR of the run's query bits).
constexpr int kListThreads = 256;
__global__ void __launch_bounds__(kListThreads)
plan_lists_kernel(const int32_t *__restrict__ q2k, const int32_t *__restrict__ cu, int T,
                  const int32_t *__restrict__ plan, int32_t *__restrict__ len,
                  int32_t *__restrict__ lists) {
  constexpr int kSortN = 512;                     // power of two >= kPlanMaxList
  constexpr int kPer = kSortN / kListThreads;     // keys per thread (2)
  static_assert(kSortN == 2 * kListThreads && kPlanMaxList <= kSortN && kFwdGroup <= 32,
                "one compare pair per thread; unit ids fit 5 bits");
  __shared__ int32_t keys[kSortN];
  __shared__ int32_t wsum[kListThreads / 64 + 1];
  const int p = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (p >= plan[0]) return;
  const i32x4 it = ((const i32x4 *)(plan + kPlanHeaderWords))[p];
  const int i = it[0], t0 = it[1], n = it[2], d = it[3];
  const int p0 = t0 - cu[d];
  constexpr int kNone = 0x7fffffff;
  int start[kPer], mask[kPer], blk[kPer];
  // The item's queries can only select blocks 0 .. nblk - 1.  Up to kSortN of them (64k-token
  // documents): one query-bit mask per block in LDS, OR-ed together; else the sort below.
  const int nblk = (p0 + n - 1) / kBlk + 1;
  if (nblk <= kSortN) {
    for (int b = tid; b < nblk; b += kListThreads) keys[b] = 0;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
      const int e = tid + kListThreads * h, u = e >> 4, j = e & 15;
      if (u < n) {
        const int b = q2k[((size_t)i * T + t0 + u) * kTopk + j];
        if (b >= 0 && b <= (p0 + u) / kBlk) atomicOr(&keys[b], 1 << u);
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
      const int b = tid * kPer + h;  // consecutive blocks per thread keep the list in order
      blk[h] = b;
      mask[h] = b < nblk ? keys[b] : 0;
      start[h] = mask[h] != 0;
    }
  } else {
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
      const int e = tid + kListThreads * h, u = e >> 4, j = e & 15;
      int key = kNone;
      if (u < n) {  // n <= kFwdGroup, so e < kPlanMaxList
        const int b = q2k[((size_t)i * T + t0 + u) * kTopk + j];
        if (b >= 0 && b <= (p0 + u) / kBlk) key = (b << 5) | u;
      }
      keys[e] = key;
    }
    __syncthreads();
    for (int k = 2; k <= kSortN; k <<= 1)
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        {  // kSortN / 2 compare pairs, one per thread
          const int q = tid;
          const int a = (q / jj) * 2 * jj + (q % jj), b = a + jj;
          const int ka = keys[a], kb = keys[b];
          const bool up = (a & k) == 0;
          if ((ka > kb) == up) {
            keys[a] = kb;
            keys[b] = ka;
          }
        }
        __syncthreads();
      }
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
      const int e = tid * kPer + h;  // consecutive keys per thread keep the runs in order
      const int key = keys[e];
      blk[h] = key >> 5;
      start[h] = key != kNone && (e == 0 || (keys[e - 1] >> 5) != blk[h]);
      mask[h] = 0;
      if (start[h])
        for (int f = e; f < kSortN && keys[f] != kNone && (keys[f] >> 5) == blk[h]; ++f)
          mask[h] |= 1 << (keys[f] & 31);
    }
  }
  int mine = 0;
#pragma unroll
  for (int h = 0; h < kPer; ++h) mine += start[h];
  // exclusive prefix of `mine` over the workgroup (thread order = key order)
  int incl = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  int r = base + incl - mine;
  int32_t *out = lists + (size_t)2 * kPlanMaxList * p;
#pragma unroll
  for (int h = 0; h < kPer; ++h)
    if (start[h]) {
      out[2 * r] = blk[h];
      out[2 * r + 1] = mask[h];
      ++r;
    }
  if (tid == kListThreads - 1) len[p] = base + incl;
}

__global__ void __launch_bounds__(1024)
plan_groups_kernel(const int32_t *__restrict__ cu, int ndocs, int Gmax, int32_t *__restrict__ plan,
                   int32_t *__restrict__ gstart) {
  __shared__ int32_t part[1024];
  int tid = threadIdx.x, nt = blockDim.x;
  int per = (ndocs + nt - 1) / nt;
  int lo = min(ndocs, tid * per), hi = min(ndocs, lo + per);
  int s = 0;
  for (int d = lo; d < hi; ++d) s += (cu[d + 1] - cu[d] + kFwdGroup - 1) / kFwdGroup;
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int d = lo; d < hi; ++d) {
    gstart[d] = run;
    run += (cu[d + 1] - cu[d] + kFwdGroup - 1) / kFwdGroup;
  }
  if (tid == nt - 1) {
    int G = part[nt - 1];
    gstart[ndocs] = G;
    plan[0] = kHI * G;
    plan[1] = G;
    plan[2] = Gmax;
  }
}

// Cost (member slots) and {t0, n, doc} of every (index head, query group) of the plan.
__global__ void plan_cost_kernel(const int32_t *__restrict__ q2k, const int32_t *__restrict__ cu,
                                 int ndocs, int T, int Gmax, const int32_t *__restrict__ plan,
                                 const int32_t *__restrict__ gstart, i32x4 *__restrict__ ginfo,
                                 int32_t *__restrict__ cost) {
  // 16 lanes (a quarter wave) per (index head, group), one per query; the group's cost is
  // their sum.  No lane returns early: all 16 take part in the sum.
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int G = plan[1];
  const int team = gid >> 4, u = gid & 15;
  const bool valid = team < kHI * G;
  int c = 0, i = 0, g = 0, d = 0, t0 = 0, n = 0;
  if (valid) {
    i = team / G;
    g = team - i * G;
    d = upper_index(gstart, ndocs - 1, g);
    t0 = cu[d] + (g - gstart[d]) * kFwdGroup;
    n = min(kFwdGroup, cu[d + 1] - t0);
    if (u < n) {
      int32_t ids[kTopk];
      int flags = 0;
      const int t = t0 + u;
      c = __popc(member_mask(q2k + ((size_t)i * T + t) * kTopk, (t - cu[d]) / kBlk, ids, &flags));
    }
  }
  static_assert(kFwdGroup == 16, "one quarter wave per group");
  c += __shfl_xor(c, 8, 16);
  c += __shfl_xor(c, 4, 16);
  c += __shfl_xor(c, 2, 16);
  c += __shfl_xor(c, 1, 16);
  if (valid && u == 0) {
    cost[i * Gmax + g] = c;
    if (i == 0) ginfo[g] = i32x4{t0, n, d, 0};
  }
}

// One workgroup per index head: stable counting sort of its groups by cost,
// descending; item p = rank * 4 + i.  rank = (groups of higher cost) + (earlier groups
// of the same cost); the second term, per chunk of 1024 groups, from a match within
// each wave (one ballot per distinct cost in the wave) and per-wave counts.
__global__ void __launch_bounds__(1024)
plan_sort_kernel(int Gmax, int32_t *__restrict__ plan, const i32x4 *__restrict__ ginfo,
                 const int32_t *__restrict__ cost) {
  constexpr int kMaxCost = kFwdGroup * kTopk;
  constexpr int kWaves = 1024 / 64;
  __shared__ int32_t hist[kMaxCost + 1];
  __shared__ int32_t start[kMaxCost + 1];
  __shared__ int32_t wcount[kWaves][kMaxCost + 1];  // this chunk's count per wave and cost
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = plan[1];
  const int32_t *c = cost + (size_t)i * Gmax;
  for (int k = tid; k <= kMaxCost; k += 1024) hist[k] = 0;
  __syncthreads();
  for (int g = tid; g < G; g += 1024) atomicAdd(&hist[c[g]], 1);
  __syncthreads();
  if (tid == 0) {  // start[v] = number of groups with cost > v
    int run = 0;
    for (int v = kMaxCost; v >= 0; --v) {
      start[v] = run;
      run += hist[v];
    }
  }
  for (int base = 0; base < G; base += 1024) {
    for (int k = tid; k < kWaves * (kMaxCost + 1); k += 1024) (&wcount[0][0])[k] = 0;
    __syncthreads();
    const int g = base + tid;
    const int my = g < G ? c[g] : -1;
    // lanes of this wave holding the same cost (invalid lanes form their own class)
    uint64_t rest = ~0ull, peers = 0;
    while (rest) {
      const int lead = (int)__builtin_ctzll(rest);
      const int v = __builtin_amdgcn_readlane(my, lead);
      const uint64_t same = (uint64_t)__ballot(my == v);
      if (my == v) peers = same;
      rest &= ~same;
    }
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int in_wave = __popcll(peers & below);
    if (my >= 0 && in_wave == 0) wcount[wave][my] = __popcll(peers);
    __syncthreads();
    if (my >= 0) {
      int before = in_wave;
      for (int w = 0; w < wave; ++w) before += wcount[w][my];
      const int rank = start[my] + before;
      const i32x4 gi = ginfo[g];
      ((i32x4 *)(plan + kPlanHeaderWords))[rank * kHI + i] = i32x4{i, gi[0], gi[1], gi[2]};
    }
    __syncthreads();
    // advance the per-cost starts by this chunk's counts
    for (int v = tid; v <= kMaxCost; v += 1024) {
      int n = 0;
      for (int w = 0; w < kWaves; ++w) n += wcount[w][v];
      start[v] += n;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ task tables
// Header, per-head row counts and CTA bounds from the scanned tile offsets.
__global__ void __launch_bounds__(1024)
tasks_header_kernel(const int32_t *__restrict__ tile_off, int NB, int grid, int rmax,
                    int32_t *__restrict__ tasks) {
  int tid = threadIdx.x;
  if (tid == 0) {
    tasks[0] = tile_off[kHI * NB];
    for (int i = 0; i < kHI; ++i) {
      tasks[1 + i] = tile_off[(i + 1) * NB] - tile_off[i * NB];
      tasks[5 + i] = tile_off[i * NB];
    }
    tasks[9] = grid;
    tasks[10] = rmax;
  }
  for (int k = tid; k < kHI * (grid + 1); k += blockDim.x) {
    int i = k / (grid + 1), c = k - i * (grid + 1);
    long long rows = tile_off[(i + 1) * NB] - tile_off[i * NB];
    tasks[kTasksHeaderWords + k] = tile_off[i * NB] + (int)((c * rows) / grid);
  }
}

// One thread per CSR entry e: row of bucket r, slot (e - row_ptr[r]) % 8.  Also the
// stored-dS tile index of the entry: (t * 4 + i) * 16 + j, j = the first q2k slot of
// (i, t) listing the bucket's document-local block.
__global__ void tasks_fill_kernel(const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ cols,
                                  const int32_t *__restrict__ tile_off,
                                  const int32_t *__restrict__ cu, const int32_t *__restrict__ cu_ws,
                                  const int32_t *__restrict__ q2k, int T,
                                  int ndocs, int NB, int cap, i32x4 *__restrict__ meta,
                                  int32_t *__restrict__ qrows, int32_t *__restrict__ qpos,
                                  int32_t *__restrict__ qtile) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  int nrows = kHI * NB;
  if (e >= cap || e >= row_ptr[nrows]) return;
  int r = upper_index(row_ptr, nrows - 1, e);
  while (r + 1 <= nrows - 1 && row_ptr[r + 1] <= e) ++r;  // skip empty rows sharing e
  int rel = e - row_ptr[r];
  int k = rel / kTileQ, s = rel - k * kTileQ;
  int row = tile_off[r] + k;
  int gb = r % NB;
  int d = upper_index(cu_ws, ndocs - 1, gb * kBlk);
  int t = cols[e];
  qrows[(size_t)row * kTileQ + s] = t;
  qpos[(size_t)row * kTileQ + s] = t - cu[d];
  {
    const int i = r / NB, bl = gb - cu_ws[d] / kBlk;
    const i32x4 *sel = (const i32x4 *)(q2k + ((size_t)i * T + t) * kTopk);
    int j = kTopk - 1;  // the CSR entry exists, so some slot lists bl: the first one wins
#pragma unroll
    for (int q = kTopk / 4 - 1; q >= 0; --q) {
      const i32x4 v = sel[q];
#pragma unroll
      for (int e = 3; e >= 0; --e)
        if (v[e] == bl) j = 4 * q + e;
    }
    qtile[(size_t)row * kTileQ + s] = (t * kHI + i) * kTopk + j;
  }
  if (s == 0) {
    int len = row_ptr[r + 1] - row_ptr[r];
    int ntile = (len + kTileQ - 1) / kTileQ;
    int nv = min(kTileQ, len - k * kTileQ);
    int flags = (k == 0 ? 1 : 0) | (k == ntile - 1 ? 2 : 0);
    meta[row] = i32x4{r, nv, flags, k};
    for (int p = nv; p < kTileQ; ++p) {
      qrows[(size_t)row * kTileQ + p] = -1;
      qpos[(size_t)row * kTileQ + p] = -1;
      qtile[(size_t)row * kTileQ + p] = -1;
    }
  }
}

// ------------------------------------------------------------------ delta
// delta[t,h] = sum_c dO*O in fp32.  16 lanes per (t, h) row, 8 elements each.
__global__ void preprocess_kernel(const u32x4 *__restrict__ O, const u32x4 *__restrict__ dO,
                                  size_t rows, float *__restrict__ delta) {
  size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t row = gid >> 4;
  float acc = 0.f;
  if (row < rows) {
    u32x4 a = O[gid], b = dO[gid];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc += bf2f((uint16_t)(a[q] & 0xffff)) * bf2f((uint16_t)(b[q] & 0xffff));
      acc += bf2f((uint16_t)(a[q] >> 16)) * bf2f((uint16_t)(b[q] >> 16));
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 8);
  if (row < rows && (gid & 15) == 0) delta[row] = acc;
}

// ------------------------------------------------------------------ finalize
// The two f16 halves of a 32-bit word, as fp32.
__device__ inline float f16lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ inline float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Part A (dq_chunks threads): dQ pool -> bf16 dQ, 8 elements per thread (f16 head-pair
// pool: 8 dims of both heads of a pair, de-interleaved).
// Part B: dK/dV pools (fp32 workspace rows) -> bf16 compact rows, 8 elements per thread.
__global__ void finalize_kernel(const void *__restrict__ dq_pool, int dq_mode, size_t dq_chunks,
                                const float *__restrict__ dk_pool, const float *__restrict__ dv_pool,
                                const int32_t *__restrict__ cu, const int32_t *__restrict__ cu_ws,
                                int ndocs, int T, u32x4 *__restrict__ dQ, u32x4 *__restrict__ dK,
                                u32x4 *__restrict__ dV) {
  size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < dq_chunks) {
    if (dq_mode == MSA_DQ_ACCUM_F16X2) {
      // chunk gid: head pair hp = gid / 16 % 32 of token gid / 512, dims 8 (gid % 16) ..
      // + 7: 8 words of (even head, odd head) f16 pairs -> 8 bf16 of each head
      const u32x4 *p = (const u32x4 *)dq_pool + 2 * gid;
      const u32x4 a = p[0], b = p[1];
      const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lo[k] = pack_bf16x2(f16lo(w[2 * k]), f16lo(w[2 * k + 1]));
        hi[k] = pack_bf16x2(f16hi(w[2 * k]), f16hi(w[2 * k + 1]));
      }
      const size_t t = gid / (32 * 16), hp = gid / 16 % 32, c = gid % 16;
      u32x4 *row = dQ + (t * kH + 2 * hp) * (kD / 8) + c;
      row[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      row[kD / 8] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    } else if (dq_mode == MSA_DQ_ACCUM_FP32) {
      const f32x4 *p = (const f32x4 *)dq_pool + 2 * gid;
      f32x4 a = p[0], b = p[1];
      dQ[gid] = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                      pack_bf16x2(b[2], b[3])};
    } else {
      dQ[gid] = ((const u32x4 *)dq_pool)[gid];
    }
    return;
  }
  size_t k = gid - dq_chunks;
  if (k >= (size_t)T * kHKV * kD / 8) return;
  int t = (int)(k / (kHKV * kD / 8));
  int c = (int)(k - (size_t)t * (kHKV * kD / 8));
  int d = upper_index(cu, ndocs - 1, t);
  size_t w = (size_t)(cu_ws[d] + t - cu[d]);
  const f32x4 *pk = (const f32x4 *)(dk_pool + w * kHKV * kD) + 2 * c;
  const f32x4 *pv = (const f32x4 *)(dv_pool + w * kHKV * kD) + 2 * c;
  f32x4 a = pk[0], b = pk[1];
  dK[k] = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                pack_bf16x2(b[2], b[3])};
  a = pv[0];
  b = pv[1];
  dV[k] = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                pack_bf16x2(b[2], b[3])};
}

// ================================================================== host launchers
namespace host {

static inline unsigned blocks_for(size_t n, unsigned bs) { return (unsigned)((n + bs - 1) / bs); }

hipError_t fill_u32(void *p, size_t n, uint32_t v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t work = (n + 3) / 4;
  unsigned nb = blocks_for(work, 256);
  if (nb > 8192) nb = 8192;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(nb), dim3(256), 0, s, (uint32_t *)p, n, v);
  return hipGetLastError();
}

hipError_t align_kv(const void *K, const void *V, const LayoutArgs &L, void *Kw, void *Vw,
                    void *Kt, void *Vt, hipStream_t s) {
  hipLaunchKernelGGL(align_blocks_kernel, dim3(L.NB, kHKV, 2), dim3(256), 0, s, (const u32x4 *)K,
                     (const u32x4 *)V, L.cu, L.cu_ws, L.ndocs, L.NB, (uint16_t *)Kw, (uint16_t *)Vw,
                     (uint16_t *)Kt, (uint16_t *)Vt);
  return hipGetLastError();
}

hipError_t build_csr(const int32_t *q2k, const LayoutArgs &L, int32_t *row_ptr, int32_t *cols,
                     int32_t *status, int32_t *counter, hipStream_t s) {
  int nrows = kHI * L.NB;
  hipError_t e = fill_u32(counter, nrows, 0, s);
  if (e != hipSuccess) return e;
  e = fill_u32(status, 1, 0, s);
  if (e != hipSuccess) return e;
  const dim3 g(blocks_for((size_t)L.T, 256), kHI);
  hipLaunchKernelGGL(csr_kernel<0>, g, dim3(256), 0, s, q2k, L.cu, L.cu_ws, L.ndocs, L.T, L.NB,
                     counter, cols, status);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, counter, nrows, 0, row_ptr, counter);
  hipLaunchKernelGGL(csr_kernel<1>, g, dim3(256), 0, s, q2k, L.cu, L.cu_ws, L.ndocs, L.T, L.NB,
                     counter, cols, status);
  return hipGetLastError();
}

size_t plan_gmax(const LayoutArgs &L) { return (size_t)(L.T + kFwdGroup - 1) / kFwdGroup + L.ndocs; }

PlanView plan_view(const LayoutArgs &L, void *plan_v) {
  PlanView v;
  int32_t *plan = (int32_t *)plan_v;
  const size_t gmax = plan_gmax(L), nitems = kHI * gmax;
  v.header = plan;
  v.items = plan + kPlanHeaderWords;
  v.len = v.items + 4 * nitems;
  v.lists = v.len + (nitems + 3) / 4 * 4;
  v.gstart = v.lists + 2 * kPlanMaxList * nitems;
  v.ginfo = v.gstart + ((L.ndocs + 1 + 3) / 4) * 4;
  v.cost = v.ginfo + 4 * gmax;
  v.end = v.cost + kHI * gmax;
  return v;
}

size_t plan_bytes(const LayoutArgs &L) {
  PlanView v = plan_view(L, nullptr);
  return (size_t)(v.end - v.header) * 4;
}

hipError_t build_plan(const LayoutArgs &L, const int32_t *q2k, void *plan_v, hipStream_t s) {
  PlanView v = plan_view(L, plan_v);
  const int gmax = (int)plan_gmax(L);
  hipLaunchKernelGGL(plan_groups_kernel, dim3(1), dim3(1024), 0, s, L.cu, L.ndocs, gmax, v.header,
                     v.gstart);
  hipLaunchKernelGGL(plan_cost_kernel, dim3(blocks_for((size_t)kHI * gmax * 16, 256)), dim3(256), 0, s,
                     q2k, L.cu, L.ndocs, L.T, gmax, v.header, v.gstart, (i32x4 *)v.ginfo, v.cost);
  hipLaunchKernelGGL(plan_sort_kernel, dim3(kHI), dim3(1024), 0, s, gmax, v.header,
                     (const i32x4 *)v.ginfo, v.cost);
  hipLaunchKernelGGL(plan_lists_kernel, dim3(kHI * gmax), dim3(kListThreads), 0, s, q2k, L.cu, L.T,
                     v.header, v.len, v.lists);
  return hipGetLastError();
}

size_t tasks_rmax(const LayoutArgs &L) {
  return (size_t)kHI * L.T * kTopk / kTileQ + (size_t)kHI * L.NB;
}
size_t tasks_meta_offset_words(int grid) {
  size_t w = kTasksHeaderWords + (size_t)kHI * (grid + 1);
  return (w + 63) / 64 * 64;
}
size_t tasks_bytes(const LayoutArgs &L, int grid) {
  size_t rmax = tasks_rmax(L);
  size_t words = tasks_meta_offset_words(grid) + 4 * rmax + 3 * kTileQ * rmax  // meta, qrows, qpos, qtile
                 + 2 * ((size_t)kHI * L.NB + 1) + 64;                        // lengths, tile_off
  return words * 4;
}

TaskView task_view(const LayoutArgs &L, int grid, void *tasks_v) {
  TaskView v;
  int32_t *tasks = (int32_t *)tasks_v;
  size_t rmax = tasks_rmax(L);
  v.header = tasks;
  v.cta = tasks + kTasksHeaderWords;
  v.meta = tasks + tasks_meta_offset_words(grid);
  v.qrows = v.meta + 4 * rmax;
  v.qpos = v.qrows + kTileQ * rmax;
  v.qtile = v.qpos + kTileQ * rmax;
  v.len = v.qtile + kTileQ * rmax;
  v.tile_off = v.len + ((size_t)kHI * L.NB + 1);
  v.rmax = rmax;
  return v;
}

hipError_t build_tasks(const LayoutArgs &L, const int32_t *row_ptr, const int32_t *cols,
                       const int32_t *q2k, int grid, void *tasks_v, hipStream_t s) {
  TaskView v = task_view(L, grid, tasks_v);
  int nrows = kHI * L.NB;
  hipLaunchKernelGGL(row_len_kernel, dim3(blocks_for(nrows, 256)), dim3(256), 0, s, row_ptr, nrows,
                     v.len);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, v.len, nrows, 1, v.tile_off,
                     (int32_t *)nullptr);
  hipLaunchKernelGGL(tasks_header_kernel, dim3(1), dim3(1024), 0, s, v.tile_off, L.NB, grid,
                     (int)v.rmax, v.header);
  size_t cap = (size_t)kHI * L.T * kTopk;
  hipLaunchKernelGGL(tasks_fill_kernel, dim3(blocks_for(cap, 256)), dim3(256), 0, s, row_ptr, cols,
                     v.tile_off, L.cu, L.cu_ws, q2k, L.T, L.ndocs, L.NB, (int)cap, (i32x4 *)v.meta,
                     v.qrows, v.qpos, v.qtile);
  return hipGetLastError();
}

hipError_t preprocess(const void *O, const void *dO, int T, float *delta, hipStream_t s) {
  size_t rows = (size_t)T * kH;
  hipLaunchKernelGGL(preprocess_kernel, dim3(blocks_for(rows * 16, 256)), dim3(256), 0, s,
                     (const u32x4 *)O, (const u32x4 *)dO, rows, delta);
  return hipGetLastError();
}

hipError_t finalize(const void *dq_pool, int mode, const float *dk_pool, const float *dv_pool,
                    const LayoutArgs &L, void *dQ, void *dK, void *dV, hipStream_t s) {
  // no pool: dQ already final; f16 pairs: one chunk per (head pair, 8 dims)
  size_t dq_chunks = dq_pool ? (size_t)L.T * kH * kD / (mode == MSA_DQ_ACCUM_F16X2 ? 16 : 8) : 0;
  size_t kv_chunks = (size_t)L.T * kHKV * kD / 8;
  hipLaunchKernelGGL(finalize_kernel, dim3(blocks_for(dq_chunks + kv_chunks, 256)), dim3(256), 0, s,
                     dq_pool, mode, dq_chunks, dk_pool, dv_pool, L.cu, L.cu_ws, L.ndocs, L.T,
                     (u32x4 *)dQ, (u32x4 *)dK, (u32x4 *)dV);
  return hipGetLastError();
}

}  // namespace host
}  // namespace msa
