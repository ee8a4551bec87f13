// msa_backward_dq.hip -- query-parallel dQ of the MSA prefill backward by recomputation
// (MSA_DQ_RECOMPUTE), gfx950.
//
// What is computed (msa_backward_sm100 API page, run_backward; the backward of the
// operator in "feat(minimax-m3): add SM100 MSA sparse attention with custom
// backward"): dQ[t,h] = scale sum_j dS_j K_j with dS_j = P_j (dP_j - delta[t,h]),
// P_j = exp(scale <Q[t,h], K_j> - LSE[t,h]) and dP_j = <dO[t,h], V_j>, over the keys j
// of the blocks q2k[h/16][t] selects (document-local, causal).
//
// Design (gfx950): one workgroup of 4 waves per plan item (index head, up to
// MSA_FWD_GROUP queries of one document), walking the item's list of selected blocks
// like the forward.  Because each query's dQ sums over its own selected blocks only,
// walking them with dQ in registers makes every dQ element a plain store -- no pool,
// no atomics.  The item's Q and dO rows, LSE and delta stay in LDS.  Per block:
//   S phase  -- wave w owns keys [32w, 32w + 32): for every pair of active units it
//               recomputes the 32 x 32 tiles S^T = K [Q_u0 | Q_u1]^T (K rows in
//               registers, loaded one step ahead) and dP^T = V [dO_u0 | dO_u1]^T (V
//               rows in registers, loaded at the step's start and first needed after
//               all S tiles of the round), forms P with the saved LSE and
//               dS = P (dP - delta), and stores dS (bf16) to the units' LDS slots;
//   dQ phase -- wave w owns dims [32w, 32w + 32): dQ^T += K^T dS^T for the round's
//               units, K^T from the transposed workspace copy into registers.
#include "msa_walk.h"

namespace msa {

constexpr int kDqThreads = kWalkThreads;
constexpr int kDqSlots = 6;      // dS slots: active units per round (three pairs)

struct DqCtx {
  WalkLane w;
  const uint16_t *Kw, *Vw, *Kt;
  const int32_t *list;
  int nact, i, p0, wsrow0, NB;
  float c;  // scale * log2(e)
  const char *sQ, *sD;
  const float *sLD;  // [unit][head][2] = {LSE log2(e), delta}
  char *sS;
};

// dS = P (dP - delta), P = 2^(c s - LSE log2 e), of a pair's tiles (S in st, dP in dp)
// to the slots s0 + column half; ld = this lane's column {LSE log2 e, delta}.  On the
// diagonal block the causal mask zeroes P.  Without a second unit the second half's
// values land in an unused slot.
__device__ __forceinline__ void dq_pair_ds(const DqCtx &x, const f32x16 &st, const f32x16 &dp, int u0, int u1,
                                           bool diag, float2 ld, int s0, int b) {
  const int half = x.w.l32 >> 4;
  const int qpos = x.p0 + (half ? u1 : u0);
  char *srow = x.sS + (s0 + half) * kSlotStride + slot_store_offset(x.w);
  uint32_t pk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float ds[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * j + e;
      float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], x.c, -ld.x));
      if (diag && b * kBlk + 32 * x.w.wave + 8 * (r >> 2) + 4 * x.w.hi + (r & 3) > qpos) pr = 0.f;
      ds[e] = pr * (dp[r] - ld.y);
    }
    pk[j] = pack_bf16x2(ds[0], ds[1]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) *(u32x2 *)(srow + 16 * j) = u32x2{pk[2 * j], pk[2 * j + 1]};
}

// {LSE log2 e, delta} of this lane's column of the pair (u0, u1).
__device__ __forceinline__ float2 dq_pair_ld(const DqCtx &x, int u0, int u1) {
  return *(const float2 *)(x.sLD + 2 * (((x.w.l32 < 16) ? u0 : u1) * 16 + x.w.l16));
}

__device__ __forceinline__ bool dq_pair_diag(const DqCtx &x, int u0, int u1, int b) {
  return (b == (x.p0 + u0) / kBlk) | (b == (x.p0 + u1) / kBlk);
}

// dQ phase of one round: dQ^T[dims 32w.., heads] += K^T dS^T for the nr units of mr,
// whose dS slots are their ranks in mr.  After a unit's MFMAs are issued, the same
// registers are refilled with the next slot's fragments.
__device__ __forceinline__ void dq_accumulate(const DqCtx &x, const bf16x8 (&kt)[2][4], uint32_t mr, int nr,
                                              f32x4 (&acc)[kFwdGroup][2]) {
  bf16x8 sf[4];
  load_slot(sf, x.sS, 0, x.w);
  int k = 0;
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if ((mr >> u) & 1u) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int md = 0; md < 2; ++md) acc[u][md] = mfma16(kt[md][kk], sf[kk], acc[u][md]);
      k = uniform(k + 1);
      load_slot(sf, x.sS, min(k, nr - 1), x.w);
    }
  }
}

// One round of a step over block b (units mround, nr of them, slots = their ranks):
// dP tiles of the round's pairs (V rows vc, dO from LDS), then S tiles (K rows kr, Q
// from LDS) and dS to the slots, a barrier, and the dQ phase with the K^T slices kt.
// Each pair's LDS operand registers are refilled with the next pair's as soon as its
// MFMAs are issued.  FIRST: the step's first round, which also issues the step's later
// loads at fixed points (K^T of this block after the dP tiles, the next block's V rows
// after the S tiles), so that they are not requested in one burst with the K rows.
template <bool FIRST>
__device__ __forceinline__ void dq_round(const DqCtx &x, uint32_t mround, int nr, int b, int bn,
                                         const bf16x8 (&kr)[8], const bf16x8 (&vc)[8], bf16x8 (&kt)[2][4],
                                         bf16x8 (&vn)[8], f32x4 (&acc)[kFwdGroup][2]) {
  uint32_t ms = mround;
  const int u0 = pop_unit(ms);
  const bool h1 = ms != 0;
  const int u1 = h1 ? pop_unit(ms) : u0;
  const bool h2 = ms != 0;
  const int u2 = h2 ? pop_unit(ms) : u0;
  const bool h3 = ms != 0;
  const int u3 = h3 ? pop_unit(ms) : u2;
  const bool h4 = ms != 0;
  const int u4 = h4 ? pop_unit(ms) : u0;
  const bool h5 = ms != 0;
  const int u5 = h5 ? pop_unit(ms) : u4;
  (void)h1; (void)h3; (void)h5;
  const bool d0 = dq_pair_diag(x, u0, u1, b), d1 = dq_pair_diag(x, u2, u3, b), d2 = dq_pair_diag(x, u4, u5, b);
  // ---- dP tiles (V rows, dO from LDS)
  f32x16 p0t, p1t, p2t;
  bf16x8 f[8];
  load_pair_rows(f, x.sD, u0, u1, x.w);
  p0t = tile32(vc, f);
  if (h2) {
    load_pair_rows(f, x.sD, u2, u3, x.w);
    p1t = tile32(vc, f);
  }
  if (h4) {
    load_pair_rows(f, x.sD, u4, u5, x.w);
    p2t = tile32(vc, f);
  }
  if (FIRST) {
    const size_t gblk = (size_t)x.i * x.NB + (size_t)(x.wsrow0 / kBlk + b);
#pragma unroll
    for (int md = 0; md < 2; ++md) load_tslice(kt[md], x.Kt, gblk, 32 * x.w.wave + 16 * md, x.w);
    WAIT_VMCNT(8);  // this block's K rows (the K^T slices may be in flight)
  }
  // ---- S tiles (K rows, Q from LDS) and dS
  load_pair_rows(f, x.sQ, u0, u1, x.w);
  float2 ld = dq_pair_ld(x, u0, u1);
  {
    const f32x16 st = tile32(kr, f);
    const float2 ldc = ld;
    if (h2) {
      load_pair_rows(f, x.sQ, u2, u3, x.w);
      ld = dq_pair_ld(x, u2, u3);
    }
    dq_pair_ds(x, st, p0t, u0, u1, d0, ldc, 0, b);
  }
  if (h2) {
    const f32x16 st = tile32(kr, f);
    const float2 ldc = ld;
    if (h4) {
      load_pair_rows(f, x.sQ, u4, u5, x.w);
      ld = dq_pair_ld(x, u4, u5);
    }
    dq_pair_ds(x, st, p1t, u2, u3, d1, ldc, 2, b);
  }
  if (h4) {
    const f32x16 st = tile32(kr, f);
    dq_pair_ds(x, st, p2t, u4, u5, d2, ld, 4, b);
  }
  if (FIRST) load_key_rows(vn, x.Vw, (size_t)x.i * x.NB + (size_t)(x.wsrow0 / kBlk + bn), x.w);
  lds_barrier();
  if (FIRST) WAIT_VMCNT(8);  // this block's K^T slices (the next V rows may be in flight)
  // ---- dQ phase
  dq_accumulate(x, kt, mround, nr, acc);
}

// One step over list entry a (block b, units m; the next entry's block bn) with this
// block's V rows in vc (loaded one step ahead); the next block's go to vn.  The K rows
// of the block are loaded at the start of the step and first needed after the dP
// tiles.
__device__ __forceinline__ void dq_step(const DqCtx &x, int b, uint32_t m, int bn, const bf16x8 (&vc)[8],
                                        bf16x8 (&vn)[8], f32x4 (&acc)[kFwdGroup][2]) {
  const int nu = __popc(m);
  bf16x8 kr[8], kt[2][4];
  load_key_rows(kr, x.Kw, (size_t)x.i * x.NB + (size_t)(x.wsrow0 / kBlk + b), x.w);
  WAIT_VMCNT(8);  // this block's V rows (the K rows may be in flight)
  dq_round<true>(x, round_bits(m, 0, kDqSlots), min(kDqSlots, nu), b, bn, kr, vc, kt, vn, acc);
  for (int r0 = kDqSlots; r0 < nu; r0 += kDqSlots) {
    lds_barrier();  // dS slots are rewritten
    dq_round<false>(x, round_bits(m, r0, kDqSlots), min(kDqSlots, nu - r0), b, bn, kr, vc, kt, vn, acc);
  }
  lds_barrier();  // dS slots are rewritten by the next step
}

__global__ void __launch_bounds__(kDqThreads, 1)
dq_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ dO,
          const uint16_t *__restrict__ Kw, const uint16_t *__restrict__ Vw,
          const uint16_t *__restrict__ Kt, const float *__restrict__ LSE,
          const float *__restrict__ Delta, const int32_t *__restrict__ cu,
          const int32_t *__restrict__ cu_ws, int NB, const int32_t *__restrict__ plan,
          const int32_t *__restrict__ plan_len, const int32_t *__restrict__ plan_lists,
          float scale, float scale_log2e, uint16_t *__restrict__ dQ) {
  __shared__ __attribute__((aligned(16))) char sQ[kFwdGroup * 16 * 256];
  __shared__ __attribute__((aligned(16))) char sD[kFwdGroup * 16 * 256];
  __shared__ __attribute__((aligned(16))) char sS[kDqSlots * kSlotStride];
  __shared__ __attribute__((aligned(16))) float sLD[kFwdGroup * 16 * 2];
  const int p = blockIdx.x;
  if (p >= plan[0]) return;
  const i32x4 item = ((const i32x4 *)(plan + kPlanHeaderWords))[p];
  DqCtx x;
  x.Kw = Kw; x.Vw = Vw; x.Kt = Kt;
  x.i = uniform(item[0]);
  const int t0 = uniform(item[1]), n = uniform(item[2]), d = uniform(item[3]);
  walk_lane(x.w, threadIdx.x);
  x.p0 = t0 - cu[d]; x.wsrow0 = cu_ws[d]; x.NB = NB;
  x.nact = uniform(plan_len[p]);
  x.list = plan_lists + (size_t)2 * kPlanMaxList * p;
  x.c = scale_log2e;
  x.sQ = sQ; x.sD = sD; x.sLD = sLD; x.sS = sS;
  const int tid = x.w.tid;

  const size_t row = ((size_t)t0 * kH + kHPI * x.i) * kD;
  rows_to_lds<kDqThreads, kFwdGroup * 16, false>(sQ, (const char *)(Q + row), (size_t)kH * kD * 2, n * 16, tid);
  rows_to_lds<kDqThreads, kFwdGroup * 16, false>(sD, (const char *)(dO + row), (size_t)kH * kD * 2, n * 16, tid);
  for (int k = tid; k < n * 16; k += kDqThreads) {
    const size_t o = (size_t)(t0 + (k >> 4)) * kH + kHPI * x.i + (k & 15);
    sLD[2 * k] = LSE[o] * kLog2e;
    sLD[2 * k + 1] = Delta[o];
  }
  __syncthreads();

  f32x4 acc[kFwdGroup][2];
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) acc[u][0] = acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the walk: list entries are read one step ahead of their use (entries past the
  // end repeat the last block, so that the loads do not depend on the position)
  if (x.nact > 0) {
    bf16x8 v0[8], v1[8];
    int b = uniform(x.list[0]);
    uint32_t m = (uint32_t)uniform(x.list[1]);
    const int e1 = min(1, x.nact - 1);
    int bn = uniform(x.list[2 * e1]);
    uint32_t mn = (uint32_t)uniform(x.list[2 * e1 + 1]);
    load_key_rows(v0, Vw, (size_t)x.i * x.NB + (size_t)(x.wsrow0 / kBlk + b), x.w);
    for (int a = 0; a < x.nact; a += 2) {
      int e2 = min(a + 2, x.nact - 1);
      int b2 = uniform(x.list[2 * e2]);
      uint32_t m2 = (uint32_t)uniform(x.list[2 * e2 + 1]);
      dq_step(x, b, m, bn, v0, v1, acc);
      b = bn; m = mn; bn = b2; mn = m2;
      if (a + 1 >= x.nact) break;
      e2 = min(a + 3, x.nact - 1);
      b2 = uniform(x.list[2 * e2]);
      m2 = (uint32_t)uniform(x.list[2 * e2 + 1]);
      dq_step(x, b, m, bn, v1, v0, acc);
      b = bn; m = mn; bn = b2; mn = m2;
    }
  }
  // ---- epilogue: acc[u][md][r] = dQ^T[dim 32w + 16md + 4g + r][head l16] / scale
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if (u < n) {
      uint16_t *qrow = dQ + ((size_t)(t0 + u) * kH + kHPI * x.i + x.w.l16) * kD + 32 * x.w.wave + 4 * x.w.g;
#pragma unroll
      for (int md = 0; md < 2; ++md) {
        const f32x4 v = acc[u][md] * scale;
        *(u32x2 *)(qrow + 16 * md) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

namespace host {
hipError_t backward_dq(const void *Q, const void *dO, const void *Kw, const void *Vw, const void *Kt,
                       const float *LSE, const float *delta, const int32_t *q2k, const LayoutArgs &L,
                       const void *plan, float scale, void *dQ, hipStream_t s) {
  (void)q2k;  // the walk lists of the plan carry the selection
  PlanView v = plan_view(L, const_cast<void *>(plan));
  const unsigned items = (unsigned)(kHI * plan_gmax(L));
  hipLaunchKernelGGL(dq_kernel, dim3(items), dim3(kDqThreads), 0, s, (const uint16_t *)Q,
                     (const uint16_t *)dO, (const uint16_t *)Kw, (const uint16_t *)Vw,
                     (const uint16_t *)Kt, LSE, delta, L.cu, L.cu_ws, L.NB, v.header, v.len,
                     v.lists, scale, scale * kLog2e, (uint16_t *)dQ);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
