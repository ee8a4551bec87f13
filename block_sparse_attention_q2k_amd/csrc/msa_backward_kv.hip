// msa_backward_kv.hip -- KV-parallel dK/dV of the MSA prefill backward for gfx950.
//
// What is computed (msa_backward_sm100 API page, module summary): for every task row
// (8 queries x 16 heads = 128 rows that selected one key block of one index head) and
// the block's 128 keys: S = Q K^T, P = exp(scale S - LSE) under the causal mask,
// dP = dO V^T, dS = P (dP - delta), dV += P^T dO, dK += scale dS^T Q.  dK/dV
// accumulate in registers over the consecutive rows of one bucket and are flushed
// with fp32 atomics at the end of the bucket segment.  dQ is produced by a
// query-parallel kernel: from the bf16 dS tiles this kernel stores (STORE_DS,
// msa_backward_dqs.hip) or by recomputation (msa_backward_dq.hip).
//
// Design (gfx950): persistent grid; workgroup c walks, per index head, the task rows
// [cta[i][c], cta[i][c+1]).  Four waves, wave w owns keys [32w, 32w+32): K and V
// slices are MFMA B operands in registers, dK/dV accumulate in registers.  The Q/dO
// rows of the next task row stream into the other half of a double buffer with
// global_load_lds_dwordx4 (asynchronous, no registers) while the current row is
// computed, so each task row costs one barrier.  All products use
// v_mfma_f32_32x32x16_bf16: S and dP with M = 32 rows, N = the wave's 32 keys, so the
// accumulator of P / dS is already the A operand of the dV / dK products (the row
// index is permuted consistently on both operands), whose B operands (dO, Q with rows
// as the contraction index) come through ds_read_b64_tr_b16 from the swizzled tiles.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kKvThreads = 256;
constexpr int kKvTile = 65536;               // Q tile 32 KB + dO tile 32 KB
constexpr int kKvScalBytes = (2 * 128 + 8 + 8) * 4;  // lse2[128], delta[128], qpos[8], dS tile[8]
constexpr int kKvScPos = 256, kKvScTile = 264;      // word offsets of qpos / dS tile indices

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// Swizzle of the Q / dO tiles ([128 rows][256 B]): 16-byte chunk c of row r is stored at
// chunk c ^ f(r), f(r) = ((r & 3) << 2) | ((r >> 2) & 3).  f is a bijection on r % 16,
// so 16 lanes reading one chunk of 16 consecutive rows (A operands) hit 16 chunks; the
// transposing reads (rows 4h + 0..3 of a 16-row step, 4 chunks) hit 16 chunks per 32
// lanes, which is as few bank conflicts as a 512-byte read allows.
__device__ __forceinline__ int kv_f(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ uint32_t swz_kv(int row, int byte_in_row) {
  return (uint32_t)(row * 256 + ((((byte_in_row >> 4) ^ kv_f(row)) << 4) | (byte_in_row & 15)));
}

__device__ inline void kv_atomic_add(float *p, float v) {
  __builtin_amdgcn_global_atomic_fadd_f32((__attribute__((address_space(1))) float *)p, v);
}

// The 8 query ids and positions of a task row (uniform).
struct KvRowIds {
  int t[kTileQ], pos[kTileQ];
};
__device__ __forceinline__ void kv_row_ids(KvRowIds &ids, const int32_t *__restrict__ qrows,
                                           const int32_t *__restrict__ qpos, int row, int nv) {
#pragma unroll
  for (int k = 0; k < kTileQ; ++k) {
    ids.t[k] = qrows[(size_t)row * kTileQ + (k < nv ? k : 0)];  // padding rows reuse a valid row
    ids.pos[k] = k < nv ? qpos[(size_t)row * kTileQ + k] : -1;    // ... and are masked
  }
}
// A task row's ids as one register: lanes 0-7 its query ids, 8-15 their positions, 16-19
// its meta entry {bucket, n_valid, flags, k}.  Loaded a row ahead with one vector load
// (the row's scalar loads would otherwise miss the caches and stall the row's start).
__device__ __forceinline__ int kv_ids_load(const int32_t *__restrict__ qrows, const int32_t *__restrict__ qpos,
                                           const i32x4 *__restrict__ meta, int row, int lane) {
  const int32_t *src = lane < 8    ? qrows + (size_t)row * kTileQ + lane
                       : lane < 16 ? qpos + (size_t)row * kTileQ + (lane - 8)
                                   : (const int32_t *)(meta + row) + ((lane - 16) & 3);
  return lane < 20 ? *src : 0;
}
// Padding queries (k >= nv) take query 0's id and position -1; the selection is made
// once in the vector register, so that every id leaves it by a constant-lane readlane.
__device__ __forceinline__ void kv_ids_unpack(KvRowIds &ids, int v, int nv, int lane) {
  const int v0 = __builtin_amdgcn_readlane(v, 0);
  const bool pad = (lane & 7) >= nv;
  const int u = lane < 8 ? (pad ? v0 : v) : lane < 16 ? (pad ? -1 : v) : v;
#pragma unroll
  for (int k = 0; k < kTileQ; ++k) {
    ids.t[k] = __builtin_amdgcn_readlane(u, k);
    ids.pos[k] = __builtin_amdgcn_readlane(u, 8 + k);
  }
}

// Issue part of the asynchronous gather of one task row into `tile`: queries
// 4 half + J0 .. + 1 of the row (Q and dO).  Chunk p = 256 k + tid of each 32 KB half
// of the tile is row 16 k + hh (query k, head hh = tid / 16), physical chunk tid % 16,
// which holds logical chunk (tid % 16) ^ kv_f(hh) (the swizzle of swz_kv()).
template <int J0>
__device__ __forceinline__ void kv_gather_part(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ dO,
                                               const KvRowIds &ids, int i, char *tile, int tid, int half) {
  const int wave = tid >> 6, hh = tid >> 4, c = (tid & 15) ^ kv_f(hh);
  lds_char *base = (lds_char *)tile + wave * 1024;
#pragma unroll
  for (int j = J0; j < J0 + 2; ++j) {
    const int k = 4 * half + j;
    const int t = half ? ids.t[4 + j] : ids.t[j];
    const size_t src = ((size_t)t * kH + kHPI * i + hh) * kD + c * 8;
    __builtin_amdgcn_global_load_lds((const gvoid *)(Q + src), (lvoid *)(base + k * 4096), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const gvoid *)(dO + src), (lvoid *)(base + 32768 + k * 4096), 16, 0, 0);
  }
}

// Raw per-row scalars for LDS row tid (< 128): LSE, delta and position of query tid/16
// (-1 for a padding query).
__device__ __forceinline__ void kv_scalars(const float *__restrict__ LSE, const float *__restrict__ Delta,
                                           const KvRowIds &ids, int i, int tid, float &lse,
                                           float &del, int &pos) {
  const int q = tid >> 4;
  int t = ids.t[0];
  pos = ids.pos[0];
#pragma unroll
  for (int k = 1; k < kTileQ; ++k)
    if (q == k) {
      t = ids.t[k];
      pos = ids.pos[k];
    }
  const size_t o = (size_t)t * kH + kHPI * i + (tid & 15);
  lse = LSE[o];
  del = Delta[o];
}

__device__ __forceinline__ void kv_store_scalars(float *sc, int tid, float lse, float del, int pos) {
  sc[tid] = lse * kLog2e;
  sc[128 + tid] = del;
  if ((tid & 15) == 0) ((int32_t *)sc)[kKvScPos + (tid >> 4)] = pos;
}

// s_waitcnt vmcnt(0) in a form the compiler's wait-count tracking understands
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

struct KvState {
  f32x16 dkacc[4], dvacc[4];
  bf16x8 kf[8], vf[8];
  int cur_r, kbase, gb;
  int r_row, nv_row;  // bucket and valid-query count of the row about to be computed
  float lse2, del;
  int pos, qt;  // qt: stored-dS tile index of the next row's query tid (tid < 8)
  int idv;      // ids of the next row (kv_ids_load)
};

// One task row: compute from tile `cur` (+ its scalars), prefetch row + 1 into `nxt`.
template <bool STORE_DS>
__device__ __forceinline__ void kv_row(
    KvState &st, int row, int hi, int i, char *cur, float *cur_sc, char *nxt, float *nxt_sc,
    uint16_t *__restrict__ dS, const int32_t *__restrict__ qtile,
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kw, const uint16_t *__restrict__ Vw,
    const uint16_t *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Delta,
    const i32x4 *__restrict__ meta, const int32_t *__restrict__ qrows,
    const int32_t *__restrict__ qpos, const int32_t *__restrict__ cu_ws, int ndocs, int NB,
    float scale, float scale_log2e, float *__restrict__ dk_pool, float *__restrict__ dv_pool,
    int tid) {
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int j16 = lane & 15, G = l32 >> 4;
  const lds_char *lcur = (const lds_char *)cur;
  // this row's meta entry came with the previous row's ids (no scalar load to wait for)
  const int r = st.r_row, nv = st.nv_row;
  // 1. new bucket: this wave's K/V slices (issued before the asynchronous gather so that
  //    waiting for them never waits for the gather)
  if (r != st.cur_r) {
    st.cur_r = r;
    st.gb = r - i * NB;
    const int dd = upper_index(cu_ws, ndocs - 1, st.gb * kBlk);
    st.kbase = st.gb * kBlk - cu_ws[dd];
    // row fragments: lane (key 32 wave + l32, dims 16 ks + 8 h ..), 1 KB per k-step
    const size_t kfr = ((size_t)i * NB + st.gb) * kFragBlock + (wave * 8 * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      st.kf[ks] = *(const bf16x8 *)(Kw + kfr + ks * 512);
      st.vf[ks] = *(const bf16x8 *)(Vw + kfr + ks * 512);
    }
#pragma unroll
    for (int nd = 0; nd < 4; ++nd)
#pragma unroll
      for (int e = 0; e < 16; ++e) st.dkacc[nd][e] = st.dvacc[nd][e] = 0.f;
    wait_vm();  // rare; keeps later waits from covering the asynchronous gather
  }
  // 2. prefetch row + 1: scalars into registers now, Q/dO tiles into `nxt`
  //    (asynchronous) in four parts spread over the compute: issued together right
  //    after the barrier, the gathers of all waves would queue up and stall the waves'
  //    instruction streams until accepted.
  const bool more = row + 1 < hi;
  const int r_next = __builtin_amdgcn_readlane(st.idv, 16);
  const int idv2 = row + 2 < hi ? kv_ids_load(qrows, qpos, meta, row + 2, lane) : 0;
  KvRowIds ids;
  if (more) {
    kv_ids_unpack(ids, st.idv, __builtin_amdgcn_readlane(st.idv, 17), lane);
    if (tid < 128) kv_scalars(LSE, Delta, ids, i, tid, st.lse2, st.del, st.pos);
    if (STORE_DS && tid < kTileQ) st.qt = qtile[(size_t)(row + 1) * kTileQ + tid];
  }
  // 3. compute.  Causal mask of this lane's key against the row's 8 queries, bit q set
  //    when query q sees it (never for padding queries, whose position is -1).
  const int kp = st.kbase + 32 * wave + l32;  // document-local position of this lane's key
  uint32_t vis = 0;
  {
    const i32x4 pa = *(const i32x4 *)((const int32_t *)cur_sc + kKvScPos);
    const i32x4 pb = *(const i32x4 *)((const int32_t *)cur_sc + kKvScPos + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) vis |= (kp <= pa[q] ? 1u : 0u) << q | (kp <= pb[q] ? 16u : 0u) << q;
  }
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    if (more) kv_gather_part<0>(Q, dO, ids, i, nxt, tid, half);
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[m2][e] = pacc[m2][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const uint32_t off = swz_kv(32 * (2 * half + m2) + l32, (16 * ks + 8 * h) * 2);
        sacc[m2] = mfma32(*(const bf16x8 *)(cur + off), st.kf[ks], sacc[m2]);
        pacc[m2] = mfma32(*(const bf16x8 *)(cur + 32768 + off), st.vf[ks], pacc[m2]);
      }
    }
    // order of the block above: the first 8 operand reads, then one MFMA and one read at a
    // time, then the last 8 MFMAs (left to itself the scheduler issues each read right
    // before its MFMA and waits for it)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads
#pragma unroll
    for (int z = 0; z < 24; ++z) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    if (more) kv_gather_part<2>(Q, dO, ids, i, nxt, tid, half);
    // P, dS: register e of sacc[m2] is row 32mt + 8(e/4) + 4h + e%4, query 2mt + e/8
    const uint32_t vh = vis >> (4 * half);
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      const int mt = 2 * half + m2;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r0 = 32 * mt + 8 * q4 + 4 * h;
        const f32x4 l4 = *(const f32x4 *)(cur_sc + r0);
        const f32x4 d4 = *(const f32x4 *)(cur_sc + 128 + r0);
        const bool seen = (vh >> (2 * m2 + (q4 >> 1))) & 1u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pr = seen ? __builtin_amdgcn_exp2f(sacc[m2][4 * q4 + e] * scale_log2e - l4[e]) : 0.f;
          sacc[m2][4 * q4 + e] = pr;
          pacc[m2][4 * q4 + e] = pr * (pacc[m2][4 * q4 + e] - d4[e]);
        }
      }
    }
    const i32x4 tix = STORE_DS ? *(const i32x4 *)((const int32_t *)cur_sc + kKvScTile + 4 * half) : i32x4{};
    // dV += P^T dO, dK += dS^T Q: M = keys, N = dims (4 x 32), K = rows (16 per step)
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int m2 = k2 >> 1, sg = k2 & 1, ks = 4 * half + k2;
      bf16x8 pa, sa;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pa[e] = (__bf16)sacc[m2][8 * sg + e];
        sa[e] = (__bf16)pacc[m2][8 * sg + e];
      }
      if (STORE_DS && 4 * half + k2 < nv) {
        // sa: query 4 half + k2, key 32 w + l32, heads 4 h .. + 3 and 8 + 4 h .. + 3,
        // which are tile positions 8 h .. 8 h + 7.  Streaming (non-temporal) store: the
        // tiles are read once, by the dQ kernel, and should not displace the Q/dO rows
        // the gathers re-read from the caches.
        const size_t tile = (size_t)__builtin_amdgcn_readfirstlane(tix[k2]) * (kBlk * 16);
        __builtin_nontemporal_store(sa, (bf16x8 *)(dS + tile + ds_key_swz(32 * wave + l32) * 16 + 8 * h));
      }
#pragma unroll
      for (int nd = 0; nd < 4; ++nd) {
        // B: lane (dim 32nd + l32, h) holds rows 16ks + 4h + 0..3 and 16ks + 8 + 4h + 0..3
        const int c0 = 32 * nd + 16 * G + 4 * (j16 & 3);
        const int k0 = 16 * ks + 4 * h + (j16 >> 2);
        const bf16x8 db = cat8(lds_read_tr(lcur, 32768 + swz_kv(k0, c0 * 2)),
                               lds_read_tr(lcur, 32768 + swz_kv(k0 + 8, c0 * 2)));
        const bf16x8 qb = cat8(lds_read_tr(lcur, swz_kv(k0, c0 * 2)), lds_read_tr(lcur, swz_kv(k0 + 8, c0 * 2)));
        st.dvacc[nd] = mfma32(pa, db, st.dvacc[nd]);
        st.dkacc[nd] = mfma32(sa, qb, st.dkacc[nd]);
      }
    }
  }
  // 4. end of this bucket's segment in this workgroup: flush dK/dV
  if (!more || r_next != r) {
    // register e of dvacc[nd]: key 32w + 8(e/4) + 4h + e%4, dim 32nd + l32
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = 32 * wave + 8 * (e >> 2) + 4 * h + (e & 3);
      const size_t o = ((size_t)(st.gb * kBlk + key) * kHKV + i) * kD + l32;
#pragma unroll
      for (int nd = 0; nd < 4; ++nd) {
        kv_atomic_add(dk_pool + o + 32 * nd, scale * st.dkacc[nd][e]);
        kv_atomic_add(dv_pool + o + 32 * nd, st.dvacc[nd][e]);
      }
    }
    st.cur_r = -1;
  }
  // 5. scalars of row + 1 -> LDS; wait for its gather; everyone done with `cur`
  if (more && tid < 128) kv_store_scalars(nxt_sc, tid, st.lse2, st.del, st.pos);
  if (STORE_DS && more && tid < kTileQ) ((int32_t *)nxt_sc)[kKvScTile + tid] = st.qt;
  wait_vm();
  st.r_row = r_next;
  st.nv_row = __builtin_amdgcn_readlane(st.idv, 17);
  st.idv = idv2;
  __syncthreads();
}

template <bool STORE_DS>
__global__ void __launch_bounds__(kKvThreads, 1)
bwd_kv_kernel(uint16_t *__restrict__ dS, const int32_t *__restrict__ qtile,
              const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kw,
              const uint16_t *__restrict__ Vw, const uint16_t *__restrict__ dO,
              const float *__restrict__ LSE, const float *__restrict__ Delta,
              const int32_t *__restrict__ cta, const i32x4 *__restrict__ meta,
              const int32_t *__restrict__ qrows, const int32_t *__restrict__ qpos,
              const int32_t *__restrict__ cu_ws, int ndocs, int NB, int grid, float scale,
              float scale_log2e, float *__restrict__ dk_pool, float *__restrict__ dv_pool) {
  // two separate arrays: the compiler can then tell the tile being read from the one
  // being filled by the asynchronous gather and does not wait for the latter
  __shared__ __attribute__((aligned(16))) char tile0[kKvTile];
  __shared__ __attribute__((aligned(16))) char tile1[kKvTile];
  __shared__ __attribute__((aligned(16))) float sc0[kKvScalBytes / 4];
  __shared__ __attribute__((aligned(16))) float sc1[kKvScalBytes / 4];
  const int c = blockIdx.x, tid = threadIdx.x;
  KvState st;
  for (int i = 0; i < kHI; ++i) {
    const int lo = cta[i * (grid + 1) + c], hi = cta[i * (grid + 1) + c + 1];
    if (lo >= hi) continue;
    {  // prologue: row lo into tile 0
      KvRowIds ids;
      const i32x4 m0 = meta[lo];
      st.r_row = m0[0];
      st.nv_row = m0[1];
      kv_row_ids(ids, qrows, qpos, lo, m0[1]);
      st.idv = lo + 1 < hi ? kv_ids_load(qrows, qpos, meta, lo + 1, tid & 63) : 0;
      if (tid < 128) {
        kv_scalars(LSE, Delta, ids, i, tid, st.lse2, st.del, st.pos);
        kv_store_scalars(sc0, tid, st.lse2, st.del, st.pos);
        if (STORE_DS && tid < kTileQ) ((int32_t *)sc0)[kKvScTile + tid] = qtile[(size_t)lo * kTileQ + tid];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        kv_gather_part<0>(Q, dO, ids, i, tile0, tid, half);
        kv_gather_part<2>(Q, dO, ids, i, tile0, tid, half);
      }
      wait_vm();
      __syncthreads();
    }
    st.cur_r = -1;
    for (int row = lo; row < hi; row += 2) {
      kv_row<STORE_DS>(st, row, hi, i, tile0, sc0, tile1, sc1, dS, qtile, Q, Kw, Vw, dO, LSE, Delta, meta,
                       qrows, qpos, cu_ws, ndocs, NB, scale, scale_log2e, dk_pool, dv_pool, tid);
      if (row + 1 < hi)
        kv_row<STORE_DS>(st, row + 1, hi, i, tile1, sc1, tile0, sc0, dS, qtile, Q, Kw, Vw, dO, LSE, Delta,
                         meta, qrows, qpos, cu_ws, ndocs, NB, scale, scale_log2e, dk_pool, dv_pool, tid);
    }
  }
}

namespace host {
hipError_t backward_kv(const void *Q, const void *Kw, const void *Vw, const void *dO,
                       const float *LSE, const float *delta, const void *tasks,
                       const LayoutArgs &L, int grid, float scale, float *dk_pool, float *dv_pool,
                       void *dS, hipStream_t s) {
  TaskView v = task_view(L, grid, const_cast<void *>(tasks));
  auto kern = dS ? bwd_kv_kernel<true> : bwd_kv_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kKvThreads), 0, s, (uint16_t *)dS, v.qtile, (const uint16_t *)Q,
                     (const uint16_t *)Kw, (const uint16_t *)Vw, (const uint16_t *)dO, LSE, delta,
                     v.cta, (const i32x4 *)v.meta, v.qrows, v.qpos, L.cu_ws, L.ndocs, L.NB, grid,
                     scale, scale * kLog2e, dk_pool, dv_pool);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
