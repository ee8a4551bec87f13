// msa_backward_dq.hip -- query-parallel dQ of the MSA prefill backward for gfx950.
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

// One step over list entry a with the K rows of this step in kc; the next entry's go to
// kn.
__device__ __forceinline__ void dq_step(const DqCtx &x, int a, const bf16x8 (&kc)[8], bf16x8 (&kn)[8],
                                        f32x4 (&acc)[kFwdGroup][2]) {
  const int b = uniform(x.list[2 * a]);
  const uint32_t m = (uint32_t)uniform(x.list[2 * a + 1]);
  const int nu = __popc(m);
  const size_t row0 = (size_t)x.wsrow0 + (size_t)b * kBlk;
  // in the order they are needed: V rows (dP), K^T (dQ phase), next K rows
  bf16x8 vr[8], kt[2][4];
  load_key_rows(vr, x.Vw, row0, x.i, x.w);
  {
    const size_t gblk = (size_t)x.i * x.NB + (size_t)(x.wsrow0 / kBlk + b);
#pragma unroll
    for (int md = 0; md < 2; ++md) load_tslice(kt[md], x.Kt, gblk, 32 * x.w.wave + 16 * md, x.w.l16, x.w.g);
  }
  load_key_rows(kn, x.Kw, (size_t)x.wsrow0 + (size_t)(a + 1 < x.nact ? uniform(x.list[2 * (a + 1)]) : b) * kBlk,
                x.i, x.w);
  for (int r0 = 0; r0 < nu; r0 += kDqSlots) {
    const int nr = min(kDqSlots, nu - r0);
    const uint32_t mround = round_bits(m, r0, kDqSlots);
    if (r0 > 0) lds_barrier();  // dS slots are rewritten
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
    // ---- S tiles of the round's pairs (K rows, Q from LDS); each pair's operand
    // registers are refilled with the next pair's as soon as its MFMAs are issued
    f32x16 s0t, s1t, s2t;
    bf16x8 f[8];
    load_pair_rows(f, x.sQ, u0, u1, x.w);
    s0t = tile32(kc, f);
    if (h2) {
      load_pair_rows(f, x.sQ, u2, u3, x.w);
      s1t = tile32(kc, f);
    }
    if (h4) {
      load_pair_rows(f, x.sQ, u4, u5, x.w);
      s2t = tile32(kc, f);
    }
    // ---- dP tiles (V rows, dO from LDS) and dS
    load_pair_rows(f, x.sD, u0, u1, x.w);
    float2 ld = dq_pair_ld(x, u0, u1);
    {
      const f32x16 dp = tile32(vr, f);
      const float2 ldc = ld;
      if (h2) {
        load_pair_rows(f, x.sD, u2, u3, x.w);
        ld = dq_pair_ld(x, u2, u3);
      }
      dq_pair_ds(x, s0t, dp, u0, u1, d0, ldc, 0, b);
    }
    if (h2) {
      const f32x16 dp = tile32(vr, f);
      const float2 ldc = ld;
      if (h4) {
        load_pair_rows(f, x.sD, u4, u5, x.w);
        ld = dq_pair_ld(x, u4, u5);
      }
      dq_pair_ds(x, s1t, dp, u2, u3, d1, ldc, 2, b);
    }
    if (h4) {
      const f32x16 dp = tile32(vr, f);
      dq_pair_ds(x, s2t, dp, u4, u5, d2, ld, 4, b);
    }
    lds_barrier();
    // ---- dQ phase
    dq_accumulate(x, kt, mround, nr, acc);
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
  bf16x8 k0[8], k1[8];
  if (x.nact > 0) load_key_rows(k0, Kw, (size_t)x.wsrow0 + (size_t)uniform(x.list[0]) * kBlk, x.i, x.w);
  for (int a = 0; a < x.nact; a += 2) {
    dq_step(x, a, k0, k1, acc);
    if (a + 1 < x.nact) dq_step(x, a + 1, k1, k0, acc);
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
