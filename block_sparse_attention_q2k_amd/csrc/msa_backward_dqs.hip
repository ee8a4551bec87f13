// msa_backward_dqs.hip -- query-parallel dQ of the MSA prefill backward from stored dS
// tiles (MSA_DQ_STORED), gfx950.
//
// What is computed (msa_backward_sm100 API page, run_backward; the backward of the
// operator in "feat(minimax-m3): add SM100 MSA sparse attention with custom
// backward"): dQ[t,h] = scale sum_j dS_j K_j over the keys j of the blocks q2k[h/16][t]
// selects.  The KV-parallel kernel has already formed every dS value (for its dK / dV
// products) and stored each (query, index head, member slot) tile; this kernel only
// contracts them with K, so nothing of S, P or dP is recomputed.
//
// Design (gfx950): one workgroup of 4 waves per plan item (index head, up to
// MSA_FWD_GROUP queries of one document), walking the item's list of member blocks like
// the forward; two workgroups per CU, so that one computes while the other waits.  Per
// step the tiles of the active queries (at most 8: a block with more active queries
// takes two steps) are copied into LDS slots by the asynchronous global-to-LDS path
// (one 1 KB quarter per wave and tile) while the previous step is computed, and so are
// the block's K^T slices into registers; one wait and barrier per step.  Wave w owns head dims [32w, 32w + 32): dQ^T += K^T dS^T
// with 16x16x32 MFMAs, K^T slices from the transposed-fragment workspace copy, the dS^T
// fragments (keys of one head) read from the [key][head] tiles with the transposing
// LDS read ds_read_b64_tr_b16.  dQ stays in accumulation registers for the whole walk
// and is stored once.
#include "msa_walk.h"

namespace msa {

constexpr int kDqsThreads = kWalkThreads;
constexpr int kDqsSlots = 8;                 // tiles per LDS buffer: at most 8 queries per step
constexpr int kDsTileBytes = kBlk * 16 * 2;  // 16 heads x 128 keys bf16
constexpr int kCachePolicyNT = 2;            // cache-policy operand: nt (streaming)

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// Member slot of document-local block bl in unit u's q2k row (held in LDS, sQ2K[u][j]):
// the first slot listing it (uniform).
__device__ __forceinline__ int dqs_slot(const int32_t *sQ2K, int u, int bl, int lane) {
  const bool hit = (lane < 16) && sQ2K[u * 16 + (lane & 15)] == bl;
  const uint32_t bits = (uint32_t)__ballot(hit) & 0xFFFFu;
  return bits ? __builtin_ctz(bits) : 0;
}

// Asynchronous copy of the tiles of the units in m (block bl) into LDS slot buffer sT
// (slot = rank in m); wave w copies bytes [1024 w, 1024 w + 1024) of each tile.  The
// tiles are read once: non-temporal loads (the K slices stay cached).
__device__ __forceinline__ void dqs_fetch_tiles(const uint16_t *__restrict__ dS, const int32_t *sQ2K, char *sT,
                                                uint32_t m, int bl, int t0, int i, const WalkLane &w) {
  int s = 0;
  while (m) {
    const int u = pop_unit(m);
    const int j = dqs_slot(sQ2K, u, bl, w.lane);
    const uint16_t *src = dS + (((size_t)(t0 + u) * kHI + i) * kTopk + j) * (size_t)(kDsTileBytes / 2) +
                          w.wave * 512 + w.lane * 8;
    __builtin_amdgcn_global_load_lds((const gvoid_t *)src, (lvoid_t *)(sT + s * kDsTileBytes + w.wave * 1024), 16,
                                     0, kCachePolicyNT);
    s = uniform(s + 1);
  }
}

// B operand of the dQ products for slot s of tile buffer sT: lane (l16, g) gets keys
// 32 kk + 8 g + 0..7 of the head at tile position l16, through two transposing reads of
// 4 keys each (16-lane group: lane j16 addresses key base + j16 / 4, positions
// 4 (j16 % 4) .. + 3).
__device__ __forceinline__ void dqs_load_frag(bf16x8 (&f)[4], const char *sT, int s, const WalkLane &w) {
  const lds_char *base = (const lds_char *)(sT + s * kDsTileBytes);
  const int kr = w.l16 >> 2, hc = (w.l16 & 3) * 8;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int k0 = 32 * kk + 8 * w.g + kr;
    f[kk] = cat8(lds_read_tr(base, ds_key_swz(k0) * 32 + hc), lds_read_tr(base, ds_key_swz(k0 + 4) * 32 + hc));
  }
}

// dQ phase of one block: dQ^T[dims 32w.., heads] += K^T dS^T for the units of m, whose
// tiles are in slots 0, 1, ... of sT.  The next slot's fragments are read before the
// current unit's MFMAs are issued.
__device__ __forceinline__ void dqs_accumulate(const bf16x8 (&kt)[2][4], const char *sT, uint32_t m, int nu,
                                               const WalkLane &w, f32x4 (&acc)[kFwdGroup][2]) {
  bf16x8 sf[4];
  dqs_load_frag(sf, sT, 0, w);
  int k = 0;
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if ((m >> u) & 1u) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int md = 0; md < 2; ++md) acc[u][md] = mfma16(kt[md][kk], sf[kk], acc[u][md]);
      k = uniform(k + 1);
      dqs_load_frag(sf, sT, min(k, nu - 1), w);
    }
  }
}

// Walk steps: list entry a (block, query mask) is one step, or two when more than
// kDqsSlots of its queries are active (the first kDqsSlots of them, then the rest).
struct DqsStep {
  int b;
  uint32_t m;
};
__device__ __forceinline__ uint32_t first_units(uint32_t m, int k) {
  uint32_t lo = 0;
  for (int i = 0; i < k && m; ++i) {
    const uint32_t bit = m & (0u - m);
    lo |= bit;
    m ^= bit;
  }
  return lo;
}
__device__ __forceinline__ DqsStep dqs_step(const int32_t *list, int a, int part) {
  const int b = uniform(list[2 * a]);
  const uint32_t m0 = (uint32_t)uniform(list[2 * a + 1]);
  if (__popc(m0) <= kDqsSlots) return DqsStep{b, m0};
  const uint32_t lo = first_units(m0, kDqsSlots);
  return DqsStep{b, part ? m0 ^ lo : lo};
}
__device__ __forceinline__ void dqs_advance(const int32_t *list, int &a, int &part) {
  if (part == 0 && __popc((uint32_t)uniform(list[2 * a + 1])) > kDqsSlots) {
    part = 1;
  } else {
    ++a;
    part = 0;
  }
}

// Waits for every outstanding global access of this wave (loads and asynchronous LDS
// copies), then for the whole workgroup.
__device__ __forceinline__ void dqs_sync() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ void __launch_bounds__(kDqsThreads, 2)
dqs_kernel(const uint16_t *__restrict__ dS, const uint16_t *__restrict__ Kt, const int32_t *__restrict__ q2k,
           int T, const int32_t *__restrict__ cu, const int32_t *__restrict__ cu_ws, int NB,
           const int32_t *__restrict__ plan, const int32_t *__restrict__ plan_len,
           const int32_t *__restrict__ plan_lists, float scale, uint16_t *__restrict__ dQ) {
  __shared__ __attribute__((aligned(16))) char sT[2][kDqsSlots * kDsTileBytes];
  __shared__ int32_t sQ2K[kFwdGroup * kTopk];
  const int p = blockIdx.x;
  if (p >= plan[0]) return;
  const i32x4 item = ((const i32x4 *)(plan + kPlanHeaderWords))[p];
  WalkLane w;
  walk_lane(w, threadIdx.x);
  const int i = uniform(item[0]);
  const int t0 = uniform(item[1]), n = uniform(item[2]), d = uniform(item[3]);
  const int wsrow0 = cu_ws[d];
  const int nact = uniform(plan_len[p]);
  const int32_t *list = plan_lists + (size_t)2 * kPlanMaxList * p;
  // the item's q2k rows (ids no block equals for units past the item's end)
  for (int k = w.tid; k < kFwdGroup * kTopk; k += kDqsThreads) {
    const int u = k / kTopk;
    sQ2K[k] = u < n ? q2k[((size_t)i * T + t0 + u) * kTopk + k % kTopk] : -2;
  }
  __syncthreads();

  f32x4 acc[kFwdGroup][2];
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) acc[u][0] = acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const size_t gblk0 = (size_t)i * NB + (size_t)(wsrow0 / kBlk);
  if (nact > 0) {
    bf16x8 kt0[2][4], kt1[2][4];
    int a = 0, part = 0;
    DqsStep cur = dqs_step(list, 0, 0);
#pragma unroll
    for (int md = 0; md < 2; ++md) load_tslice(kt0[md], Kt, gblk0 + cur.b, 32 * w.wave + 16 * md, w);
    dqs_fetch_tiles(dS, sQ2K, sT[0], cur.m, cur.b, t0, i, w);
    while (true) {
      // ---- step in buffer 0: its tiles and K^T slices arrived; fetch the next step's
      dqs_sync();
      int an = a, pn = part;
      dqs_advance(list, an, pn);
      bool more = an < nact;
      DqsStep nx = cur;
      if (more) {
        nx = dqs_step(list, an, pn);
#pragma unroll
        for (int md = 0; md < 2; ++md) load_tslice(kt1[md], Kt, gblk0 + nx.b, 32 * w.wave + 16 * md, w);
        dqs_fetch_tiles(dS, sQ2K, sT[1], nx.m, nx.b, t0, i, w);
      }
      dqs_accumulate(kt0, sT[0], cur.m, __popc(cur.m), w, acc);
      if (!more) break;
      a = an;
      part = pn;
      cur = nx;
      // ---- step in buffer 1
      dqs_sync();
      dqs_advance(list, an, pn);
      more = an < nact;
      if (more) {
        nx = dqs_step(list, an, pn);
#pragma unroll
        for (int md = 0; md < 2; ++md) load_tslice(kt0[md], Kt, gblk0 + nx.b, 32 * w.wave + 16 * md, w);
        dqs_fetch_tiles(dS, sQ2K, sT[0], nx.m, nx.b, t0, i, w);
      }
      dqs_accumulate(kt1, sT[1], cur.m, __popc(cur.m), w, acc);
      if (!more) break;
      a = an;
      part = pn;
      cur = nx;
    }
  }
  // ---- epilogue: acc[u][md][r] = dQ^T[dim 32w + 16md + 4g + r][head at tile position
  //      l16] / scale (ds_head_pos is its own inverse)
  const int head = kHPI * i + ds_head_pos(w.l16);
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if (u < n) {
      uint16_t *qrow = dQ + ((size_t)(t0 + u) * kH + head) * kD + 32 * w.wave + 4 * w.g;
#pragma unroll
      for (int md = 0; md < 2; ++md) {
        const f32x4 v = acc[u][md] * scale;
        *(u32x2 *)(qrow + 16 * md) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

namespace host {
hipError_t backward_dqs(const void *dS, const void *Kt, const int32_t *q2k, const LayoutArgs &L,
                        const void *plan, float scale, void *dQ, hipStream_t s) {
  PlanView v = plan_view(L, const_cast<void *>(plan));
  const unsigned items = (unsigned)(kHI * plan_gmax(L));
  hipLaunchKernelGGL(dqs_kernel, dim3(items), dim3(kDqsThreads), 0, s, (const uint16_t *)dS,
                     (const uint16_t *)Kt, q2k, L.T, L.cu, L.cu_ws, L.NB, v.header, v.len, v.lists, scale,
                     (uint16_t *)dQ);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
