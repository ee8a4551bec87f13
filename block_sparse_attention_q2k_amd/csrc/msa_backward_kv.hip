// msa_backward_kv.hip -- KV-parallel dK/dV of the MSA prefill backward for gfx950.
//
// What is computed (msa_backward_sm100 API page, module summary): for every task row
// (8 queries x 16 heads = 128 rows that selected one key block of one index head) and
// the block's 128 keys: S = Q K^T, P = exp(scale S - LSE) under the causal mask,
// dP = dO V^T, dS = P (dP - delta), dV += P^T dO, dK += scale dS^T Q.  dK/dV
// accumulate in registers over the consecutive rows of one bucket and are flushed
// with fp32 atomics at the end of the bucket segment.  This kernel serves the recompute
// mode (MSA_DQ_RECOMPUTE), whose dQ the query-parallel kernel recomputes
// (msa_backward_dq.hip); the stored-dS mode uses msa_backward_kv2.hip.
//
// Design (gfx950): persistent grid; workgroup c walks, per index head, the task rows
// [cta[i][c], cta[i][c+1]).  Four waves, wave w owns keys [32w, 32w+32): K and V
// slices are MFMA B operands in registers, dK/dV accumulate in registers.  The Q/dO
// rows of the next task row are gathered into the other half of an LDS double buffer
// while the current row is computed (through registers: an asynchronous global-to-LDS
// copy in flight would make every LDS wait of the row a full wait), so each task row
// costs one barrier.  All products use v_mfma_f32_32x32x16_bf16: S and dP with M = 32
// rows, N = the wave's 32 keys, so the accumulator of P / dS is already the A operand of
// the dV / dK products (the row index is permuted consistently on both operands), whose
// B operands (dO, Q with rows as the contraction index) come through ds_read_b64_tr_b16
// from the swizzled tiles.  A row is 32 fixed steps of 4 MFMAs (see kv_step): LDS
// operands are read two steps ahead, and each quarter's softmax runs among the next
// quarter's MFMAs; in-kernel cycle counters put the MFMA-only steps within 15-45 % of
// their MFMA time.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kKvThreads = 256;
constexpr int kKvTile = 65536;               // Q tile 32 KB + dO tile 32 KB
constexpr int kKvScalBytes = (2 * 128 + 8) * 4;  // lse2[128], delta[128], qpos[8]
constexpr int kKvScPos = 256;                   // word offset of qpos

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

// The same gather staged through registers, for the rows computed inside the compute
// block: an asynchronous global-to-LDS copy in flight makes the compiler wait for every
// outstanding LDS read (lgkmcnt(0)) wherever an LDS result is used, which would undo the
// block's read-ahead.  Part P (queries 2 P, 2 P + 1): kv_gather_load puts this thread's
// four 16-byte chunks (Q and dO of both queries) in registers; kv_gather_store writes them
// where kv_gather_part would have (the same swizzled layout).
template <int P>
__device__ __forceinline__ void kv_gather_load(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ dO,
                                               const KvRowIds &ids, int i, int tid, u32x4 (&v)[4]) {
  const int hh = tid >> 4, c = (tid & 15) ^ kv_f(hh);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const size_t src = ((size_t)ids.t[2 * P + u] * kH + kHPI * i + hh) * kD + c * 8;
    v[2 * u] = *(const u32x4 *)(Q + src);
    v[2 * u + 1] = *(const u32x4 *)(dO + src);
  }
}
template <int P>
__device__ __forceinline__ void kv_gather_store(char *tile, int tid, const u32x4 (&v)[4]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int k = 2 * P + u;
    *(u32x4 *)(tile + k * 4096 + tid * 16) = v[2 * u];
    *(u32x4 *)(tile + 32768 + k * 4096 + tid * 16) = v[2 * u + 1];
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

// The value of v, opaque to the optimizer: per-lane values derived from it inside the row
// loop are recomputed each row (a few VALU instructions) instead of being hoisted out of
// the loop and kept live across the row's compute block, which spills them to scratch.
__device__ __forceinline__ int kv_opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// s_waitcnt vmcnt(0) in a form the compiler's wait-count tracking understands
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier that waits for this wave's LDS accesses only (lgkmcnt(0)), not for its
// global stores (the dS tiles) still in flight, as __syncthreads() would.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void kv_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- the compute block of one task row
// The row's 128 rows form four quarters (rows 32 q .. 32 q + 31: queries 2 q, 2 q + 1).
// Per quarter: SP(q) = S = Q K^T and dP = dO V^T (M = the quarter's rows, N = this
// wave's 32 keys, 8 k-steps over the head dims; 16 MFMAs); SM(q) = the softmax, P and
// dS (VALU); DK(q) = dV += P^T dO and dK += dS^T Q (M = keys, N = dims 4 x 32, K = the
// quarter's rows in 2 k-steps of 16; 16 MFMAs, B operands through transposing reads).
// The block is 32 steps of 4 MFMAs in the order SP0, SP1 | SM0, DK0, SP2 | SM1, DK1,
// SP3 | SM2, DK2 | SM3, DK3: each step issues the LDS reads of the step after next into
// the third of three operand buffers, so an MFMA never waits for a read issued just before it,
// and a quarter's softmax runs among the MFMAs of the next quarter.  The steps are
// separated by scheduling fences, and inside a step the order is fixed (MFMA, its share
// of reads and VALU work); left to itself the scheduler pairs every read with the MFMA
// that consumes it and waits for it.
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

// An LDS address held in a register the optimizer cannot see through, so that it is
// computed once per row instead of before every read.
__device__ __forceinline__ const lds_char *kv_opaque_lds(const lds_char *p) {
  asm volatile("" : "+v"(p));
  return p;
}

struct KvRowCtx {
  uint32_t vis;  // bit q: query q of the row sees this lane's key
  float c;       // scale * log2(e)
  // this lane's LDS addresses: S/dP operand of k-step ks in quarter 0 of the Q tile (+8192
  // per quarter, +32768 for dO); DK operand rows 4 h + j16 / 4 (+8 for hi) of dims
  // 32 nd .. of k-step 0 (+4096 per k-step, +32768 for dO); LSE of rows 4 h .. (+4 per row,
  // +512 bytes for delta)
  const lds_char *spa[8], *dka[4][2], *sca;
};

__device__ __forceinline__ void kv_row_addresses(KvRowCtx &x, const char *cur, const float *cur_sc, int l32, int h,
                                                 int j16, int G) {
  const lds_char *lc = (const lds_char *)cur;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) x.spa[ks] = kv_opaque_lds(lc + swz_kv(l32, (16 * ks + 8 * h) * 2));
#pragma unroll
  for (int nd = 0; nd < 4; ++nd)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int c0 = 32 * nd + 16 * G + 4 * (j16 & 3);
      x.dka[nd][hi] = kv_opaque_lds(lc + swz_kv(4 * h + (j16 >> 2) + 8 * hi, c0 * 2));
    }
  x.sca = kv_opaque_lds((const lds_char *)cur_sc + 16 * h);
}

struct KvRegs {
  f32x16 s[2], p[2];          // S / dP accumulators of two quarters
  bf16x8 pa[2][2], sa[2][2];  // P / dS as bf16 A operands [quarter set][query of the quarter]
  bf16x8 ob[3][4];            // LDS operands of a step, three steps in flight
  f32x4 sl[3][2];             // LSE (log2) and delta of a softmax chunk, likewise
  u32x4 gq[2][4];             // next row's gather, two parts in flight
};

// Step S: kind and quarter.  SP steps: 0-3 (q 0), 4-7 (q 1), 12-15 (q 2), 20-23 (q 3);
// DK steps: 8-11 (q 0), 16-19 (q 1), 24-27 (q 2), 28-31 (q 3); SM chunks (one per step, 4
// per quarter): steps 4-7 (q 0), 12-15 (q 1), 20-23 (q 2), 24-27 (q 3).
constexpr bool kv_is_sp(int S) { return S < 8 || (S >= 12 && S < 16) || (S >= 20 && S < 24); }
constexpr int kv_quarter(int S) {
  return S < 4 ? 0 : S < 8 ? 1 : S < 12 ? 0 : S < 16 ? 2 : S < 20 ? 1 : S < 24 ? 3 : S < 28 ? 2 : 3;
}
constexpr int kv_sm_quarter(int S) {
  return (S >= 4 && S < 8) ? 0 : (S >= 12 && S < 16) ? 1 : (S >= 20 && S < 24) ? 2 : (S >= 24 && S < 28) ? 3 : -1;
}

// LDS reads of step S into buffer b: its MFMA operands and, if it has a softmax chunk,
// that chunk's LSE / delta.
template <int S>
__device__ __forceinline__ void kv_step_reads(const KvRowCtx &x, KvRegs &g, int b) {
  constexpr int q = kv_quarter(S), j = S & 3;
  if constexpr (kv_is_sp(S)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ks = 2 * j + u;  // rows 32 q + l32 (the swizzle depends on the row mod 16 only)
      g.ob[b][2 * u] = *(const lds_bf16x8 *)(x.spa[ks] + 8192 * q);
      g.ob[b][2 * u + 1] = *(const lds_bf16x8 *)(x.spa[ks] + 8192 * q + 32768);
    }
  } else {
    const int ks = 2 * q + (j >> 1);  // rows 16 ks + 4 h + j16 / 4 (+ 8)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int nd = 2 * (j & 1) + u;
      g.ob[b][2 * u] = cat8(lds_read_tr(x.dka[nd][0], 4096 * ks + 32768), lds_read_tr(x.dka[nd][1], 4096 * ks + 32768));
      g.ob[b][2 * u + 1] = cat8(lds_read_tr(x.dka[nd][0], 4096 * ks), lds_read_tr(x.dka[nd][1], 4096 * ks));
    }
  }
  constexpr int sq = kv_sm_quarter(S);
  if constexpr (sq >= 0) {  // chunk j: accumulator registers 4 j .. 4 j + 3, rows 32 sq + 8 j + 4 h ..
    g.sl[b][0] = *(const lds_f32x4 *)(x.sca + 4 * (32 * sq + 8 * j));
    g.sl[b][1] = *(const lds_f32x4 *)(x.sca + 4 * (32 * sq + 8 * j) + 512);
  }
}

// Softmax chunk j of quarter SQ (registers 4 j .. 4 j + 3 of its S / dP accumulators:
// rows 32 SQ + 8 j + 4 h + 0..3 of query 2 SQ + j / 2).  After chunks 1 and 3 the bf16
// operands of query 2 SQ + j / 2 are complete.
template <int SQ, int J>
__device__ __forceinline__ void kv_sm_chunk(const KvRowCtx &x, KvRegs &g, int b) {
  constexpr int set = SQ & 1, sg = J >> 1;
  const bool seen = (x.vis >> (2 * SQ + sg)) & 1u;
  const f32x4 l = g.sl[b][0], d = g.sl[b][1];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float pr = seen ? __builtin_amdgcn_exp2f(g.s[set][4 * J + e] * x.c - l[e]) : 0.f;
    g.s[set][4 * J + e] = pr;
    g.p[set][4 * J + e] = pr * (g.p[set][4 * J + e] - d[e]);
  }
  if constexpr (J & 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      g.pa[set][sg][e] = (__bf16)g.s[set][8 * sg + e];
      g.sa[set][sg][e] = (__bf16)g.p[set][8 * sg + e];
    }
  }
}

#define KV_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
// Instruction order inside step S: the reads of step S + 2 (0x100) after its first two
// MFMAs; VALU (0x002) after every MFMA.
template <int S>
__device__ __forceinline__ void kv_step_order() {
  constexpr int nds = S + 2 >= 32 ? 0 : (kv_is_sp(S + 2) ? 4 : 8) + (kv_sm_quarter(S + 2) >= 0 ? 2 : 0);
  constexpr int valu = kv_sm_quarter(S) >= 0 ? 10 : 1;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    KV_SGB(0x008, 1);
    constexpr int first = (nds + 1) / 2;
    if (k == 0 && first > 0) KV_SGB(0x100, first);
    if (k == 1 && nds - first > 0) KV_SGB(0x100, nds - first);
    KV_SGB(0x002, valu);
  }
}
#undef KV_SGB

struct KvState {
  f32x16 dkacc[4], dvacc[4];
  bf16x8 kf[8], vf[8];
  int cur_r, kbase, gb;
  int r_row;  // bucket of the row about to be computed
  float lse2, del;
  int pos;
  int idv;      // ids of the next row (kv_ids_load)
};

// Step S of the row: reads of step S + 2 (buffer (S + 2) % 3), the 4 MFMAs of step S
// (operands in buffer S % 3), its softmax chunk, and a quarter of the next row's gather
// in the first step of each DK phase.
template <int S>
__device__ __forceinline__ void kv_step(const KvRowCtx &x, KvRegs &g, KvState &st, const KvRowIds &ids,
                                        const uint16_t *__restrict__ Q, const uint16_t *__restrict__ dO, int i,
                                        char *nxt, int tid) {
  constexpr int b = S % 3, q = kv_quarter(S), j = S & 3, set = q & 1;
  if constexpr (S + 2 < 32) kv_step_reads<S + 2>(x, g, (S + 2) % 3);
  if constexpr (kv_is_sp(S)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ks = 2 * j + u;
      if (j == 0 && u == 0) {
        g.s[set] = mfma32(g.ob[b][0], st.kf[ks], f32x16{});
        g.p[set] = mfma32(g.ob[b][1], st.vf[ks], f32x16{});
      } else {
        g.s[set] = mfma32(g.ob[b][2 * u], st.kf[ks], g.s[set]);
        g.p[set] = mfma32(g.ob[b][2 * u + 1], st.vf[ks], g.p[set]);
      }
    }
  } else {
    constexpr int sg = j >> 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int nd = 2 * (j & 1) + u;
      st.dvacc[nd] = mfma32(g.pa[set][sg], g.ob[b][2 * u], st.dvacc[nd]);
      st.dkacc[nd] = mfma32(g.sa[set][sg], g.ob[b][2 * u + 1], st.dkacc[nd]);
    }
  }
  constexpr int sq = kv_sm_quarter(S);
  if constexpr (sq >= 0) kv_sm_chunk<sq, j>(x, g, b);
  // next row's gather: parts 0, 1 loaded in steps 0, 2 and written to LDS in steps 14, 16;
  // parts 2, 3 loaded in steps 14, 16 and written in steps 28, 30
  if constexpr (S == 14) kv_gather_store<0>(nxt, tid, g.gq[0]);
  if constexpr (S == 16) kv_gather_store<1>(nxt, tid, g.gq[1]);
  if constexpr (S == 28) kv_gather_store<2>(nxt, tid, g.gq[0]);
  if constexpr (S == 30) kv_gather_store<3>(nxt, tid, g.gq[1]);
  if constexpr (S == 0) kv_gather_load<0>(Q, dO, ids, i, tid, g.gq[0]);
  if constexpr (S == 2) kv_gather_load<1>(Q, dO, ids, i, tid, g.gq[1]);
  if constexpr (S == 14) kv_gather_load<2>(Q, dO, ids, i, tid, g.gq[0]);
  if constexpr (S == 16) kv_gather_load<3>(Q, dO, ids, i, tid, g.gq[1]);
  kv_step_order<S>();
  __builtin_amdgcn_sched_barrier(0);
}

template <int S>
__device__ __forceinline__ void kv_steps(const KvRowCtx &x, KvRegs &g, KvState &st, const KvRowIds &ids,
                                         const uint16_t *__restrict__ Q, const uint16_t *__restrict__ dO, int i,
                                         char *nxt, int tid) {
  if constexpr (S < 32) {
    kv_step<S>(x, g, st, ids, Q, dO, i, nxt, tid);
    kv_steps<S + 1>(x, g, st, ids, Q, dO, i, nxt, tid);
  }
}

// One task row: compute from tile `cur` (+ its scalars), prefetch row + 1 into `nxt`.
__device__ __forceinline__ void kv_row(
    KvState &st, int row, int hi, int i, char *cur, float *cur_sc, char *nxt, float *nxt_sc,
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kw, const uint16_t *__restrict__ Vw,
    const uint16_t *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Delta,
    const i32x4 *__restrict__ meta, const int32_t *__restrict__ qrows,
    const int32_t *__restrict__ qpos, const int32_t *__restrict__ cu_ws, int ndocs, int NB,
    float scale, float scale_log2e, float *__restrict__ dk_pool, float *__restrict__ dv_pool, int tid_in) {
  const int tid = kv_opaque(tid_in);
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int j16 = lane & 15, G = l32 >> 4;
  // this row's meta entry came with the previous row's ids (no scalar load to wait for)
  const int r = st.r_row;
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
  // (past the last row st.idv is 0: the gathers below then read token 0's rows into the
  // unused buffer, which keeps the compute block free of branches)
  KvRowIds ids;
  kv_ids_unpack(ids, st.idv, __builtin_amdgcn_readlane(st.idv, 17), lane);
  if (more && tid < 128) kv_scalars(LSE, Delta, ids, i, tid, st.lse2, st.del, st.pos);
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
  KvRowCtx x;
  kv_row_addresses(x, cur, cur_sc, l32, h, j16, G);
  x.vis = vis;
  x.c = scale_log2e;
  KvRegs g;
  kv_step_reads<0>(x, g, 0);
  kv_step_reads<1>(x, g, 1);
  __builtin_amdgcn_sched_barrier(0);
  kv_steps<0>(x, g, st, ids, Q, dO, i, nxt, tid);
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
  // 5. scalars of row + 1 -> LDS; everyone done with `cur` and done writing `nxt`
  if (more && tid < 128) kv_store_scalars(nxt_sc, tid, st.lse2, st.del, st.pos);
  st.r_row = r_next;
  st.idv = idv2;
  kv_lds_barrier();
}

__global__ void __launch_bounds__(kKvThreads, 1)
bwd_kv_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kw,
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
      kv_row_ids(ids, qrows, qpos, lo, m0[1]);
      st.idv = lo + 1 < hi ? kv_ids_load(qrows, qpos, meta, lo + 1, tid & 63) : 0;
      if (tid < 128) {
        kv_scalars(LSE, Delta, ids, i, tid, st.lse2, st.del, st.pos);
        kv_store_scalars(sc0, tid, st.lse2, st.del, st.pos);
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
      kv_row(st, row, hi, i, tile0, sc0, tile1, sc1, Q, Kw, Vw, dO, LSE, Delta, meta, qrows, qpos, cu_ws, ndocs,
             NB, scale, scale_log2e, dk_pool, dv_pool, tid);
      if (row + 1 < hi)
        kv_row(st, row + 1, hi, i, tile1, sc1, tile0, sc0, Q, Kw, Vw, dO, LSE, Delta, meta, qrows, qpos, cu_ws,
               ndocs, NB, scale, scale_log2e, dk_pool, dv_pool, tid);
    }
  }
}

namespace host {
hipError_t backward_kv(const void *Q, const void *Kw, const void *Vw, const void *dO,
                       const float *LSE, const float *delta, const void *tasks,
                       const LayoutArgs &L, int grid, float scale, float *dk_pool, float *dv_pool,
                       hipStream_t s) {
  TaskView v = task_view(L, grid, const_cast<void *>(tasks));
  hipLaunchKernelGGL(bwd_kv_kernel, dim3(grid), dim3(kKvThreads), 0, s, (const uint16_t *)Q,
                     (const uint16_t *)Kw, (const uint16_t *)Vw, (const uint16_t *)dO, LSE, delta,
                     v.cta, (const i32x4 *)v.meta, v.qrows, v.qpos, L.cu_ws, L.ndocs, L.NB, grid,
                     scale, scale * kLog2e, dk_pool, dv_pool);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
