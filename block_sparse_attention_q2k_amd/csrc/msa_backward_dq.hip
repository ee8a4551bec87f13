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
// no atomics.  Per block:
//   S phase  -- the active units are dealt to the waves (slot s to wave s % 4), two at
//               a time so that each K / V fragment read from LDS feeds two units; a
//               wave recomputes S^T = K Q^T and dP^T = V dO^T 32 keys at a time, forms
//               P with the saved LSE and dS = P (dP - delta), and writes dS (bf16) to
//               LDS;
//   dQ phase -- wave w owns dims [32w, 32w + 32): dQ^T += K^T dS^T for the round's
//               units, K^T from the transposed workspace copy.
// K and V of the next block arrive by asynchronous global->LDS copies into the other
// of two buffer pairs while the current block is processed; Q, dO, LSE and delta of
// the next step's first units are fetched one step ahead.  LDS: 4 x 32 KB blocks
// + 8 dS slots of 4 KB = 160 KB, one workgroup per CU.
#include "msa_walk.h"

namespace msa {

constexpr int kDqSlots = 8;  // dS slots: active units per round

struct DqCtx {
  const uint16_t *Q, *dO, *Kw, *Vw, *Kt;
  const float *LSE, *Delta;
  const int32_t *list;
  int nact, i, t0, p0, wsrow0, NB;
  int tid, lane, wave, l16, g;
  float c;  // scale * log2(e)
  char *sS;
};

// Per-unit operands of the S phase: Q and dO rows (B fragments), LSE (base 2) and
// delta of this lane's head.
struct DqUnit {
  bf16x8 q[4], d[4];
  float lse2, del;
};

__device__ __forceinline__ void dq_load_unit(const DqCtx &x, DqUnit &w, int u) {
  const int t = x.t0 + u;
  load_rows16(w.q, x.Q, t, x.i, x.l16, x.g);
  load_rows16(w.d, x.dO, t, x.i, x.l16, x.g);
  const size_t o = (size_t)t * kH + kHPI * x.i + x.l16;
  w.lse2 = x.LSE[o] * kLog2e;
  w.del = x.Delta[o];
}

// Units of slots s0 and s0 + 4 (when present) of mask m.
__device__ __forceinline__ void dq_load_pair(const DqCtx &x, DqUnit (&w)[2], uint32_t m, int s0, int nu) {
  if (s0 < nu) dq_load_unit(x, w[0], nth_set_bit(m, s0));
  if (s0 + 4 < nu) dq_load_unit(x, w[1], nth_set_bit(m, s0 + 4));
}

// dS of keys 32 q4 + 16 t + 4 g + r (t = 0, 1) of one unit into dS slot rel:
// row = head l16, keys contiguous, swz() layout.
__device__ __forceinline__ void dq_ds(const DqCtx &x, const f32x4 (&sc)[2], const f32x4 (&dp)[2],
                                      const DqUnit &w, int u, int rel, int b, int q4) {
  const int qpos = x.p0 + u;
  const bool diag = b == qpos / kBlk;
  const uint32_t srow = lds_addr(x.sS + rel * 4096);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float ds[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = b * kBlk + 32 * q4 + 16 * t + 4 * x.g + r;
      const float pr = (diag && key > qpos) ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][r], x.c, -w.lse2));
      ds[r] = pr * (dp[t][r] - w.del);
    }
    lds_store_b64<0>(srow + swz(x.l16, (32 * q4 + 16 * t + 4 * x.g) * 2),
                     u32x2{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3])});
  }
}

// S phase for one or two units against the K / V blocks in sK / sV.
template <bool TWO>
__device__ __forceinline__ void dq_scores(const DqCtx &x, const char *sK, const char *sV,
                                          const DqUnit (&w)[2], int u0, int rel0, int u1, int rel1,
                                          int b) {
#pragma unroll 1
  for (int q4 = 0; q4 < 4; ++q4) {  // keys 32 q4 .. 32 q4 + 31: tiles 2 q4, 2 q4 + 1
    f32x4 sa[2], sb[2], pa[2], pb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) sa[t] = sb[t] = pa[t] = pb[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t off = swz_frag(kk, x.l16, x.g) + 8192 * q4;
      bf16x8 kf[2], vf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        kf[t] = *(const bf16x8 *)(sK + off + 4096 * t);
        vf[t] = *(const bf16x8 *)(sV + off + 4096 * t);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sa[t] = mfma16(kf[t], w[0].q[kk], sa[t]);
        pa[t] = mfma16(vf[t], w[0].d[kk], pa[t]);
        if (TWO) {
          sb[t] = mfma16(kf[t], w[1].q[kk], sb[t]);
          pb[t] = mfma16(vf[t], w[1].d[kk], pb[t]);
        }
      }
    }
    dq_ds(x, sa, pa, w[0], u0, rel0, b, q4);
    if (TWO) dq_ds(x, sb, pb, w[1], u1, rel1, b, q4);
  }
}

// S phase of the units in slots s0 and s0 + 4 (when present) of the round starting at
// slot r0, with their operands in w.
__device__ __forceinline__ void dq_pair(const DqCtx &x, const char *sK, const char *sV,
                                        const DqUnit (&w)[2], uint32_t m, int r0, int s0, int nr, int b) {
  const int u0 = nth_set_bit(m, r0 + s0);
  if (s0 + 4 < nr)
    dq_scores<true>(x, sK, sV, w, u0, s0, nth_set_bit(m, r0 + s0 + 4), s0 + 4, b);
  else
    dq_scores<false>(x, sK, sV, w, u0, s0, u0, s0, b);
}

// dQ phase of one round: dQ^T[dims 32w.., heads] += K^T dS^T for the units whose bits
// are set in mr, taking dS slots in unit order.
__device__ __forceinline__ void dq_accumulate(const DqCtx &x, const bf16x8 (&kt)[2][4], uint32_t mr,
                                              f32x4 (&acc)[kFwdGroup][2]) {
  const char *srow = x.sS;
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if (mr & 1u) {
      bf16x8 sf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sf[kk] = *(const bf16x8 *)(srow + swz_frag(kk, x.l16, x.g));
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int md = 0; md < 2; ++md) acc[u][md] = mfma16(kt[md][kk], sf[kk], acc[u][md]);
      srow += 4096;
    }
    mr = uniform(mr >> 1);
  }
}

// One step: list entry a, K / V in sKc / sVc; entry a + 1 goes to sKn / sVn.  wn holds
// the operands of this step's slots (wave, wave + 4) and receives the next step's.
__device__ __forceinline__ void dq_step(const DqCtx &x, int a, const char *sKc, const char *sVc,
                                        char *sKn, char *sVn, f32x4 (&acc)[kFwdGroup][2],
                                        DqUnit (&wn)[2]) {
  const int b = uniform(x.list[2 * a]);
  const uint32_t m = (uint32_t)uniform(x.list[2 * a + 1]);
  const int nu = __popc(m);
  const bool more = a + 1 < x.nact;
  const uint32_t m1 = more ? (uint32_t)uniform(x.list[2 * (a + 1) + 1]) : 0u;
  // K^T first: the dQ phase waits for it, but not for the copies issued after it
  const size_t gblk = (size_t)x.i * x.NB + (size_t)(x.wsrow0 / kBlk + b);
  bf16x8 kt[2][4];
#pragma unroll
  for (int md = 0; md < 2; ++md) load_tslice(kt[md], x.Kt, gblk, 32 * x.wave + 16 * md, x.l16, x.g);
  if (more) {
    const size_t row1 = (size_t)x.wsrow0 + (size_t)x.list[2 * (a + 1)] * kBlk;
    block_dma(sKn, x.Kw, row1, x.i, x.tid);
    block_dma(sVn, x.Vw, row1, x.i, x.tid);
  }
  // ---- round 0: the prefetched pair
  const int nr = min(kDqSlots, nu);
  if (x.wave < nr) dq_pair(x, sKc, sVc, wn, m, 0, x.wave, nr, b);
  if (more) dq_load_pair(x, wn, m1, x.wave, __popc(m1));
  lds_barrier();
  dq_accumulate(x, kt, round_bits(m, 0, kDqSlots), acc);
  // ---- further rounds of 8 units (only with more than 8 active units)
  for (int r0 = kDqSlots; r0 < nu; r0 += kDqSlots) {
    const int nr2 = min(kDqSlots, nu - r0);
    lds_barrier();  // dS slots are rewritten
    if (x.wave < nr2) {
      DqUnit wd[2];
      dq_load_pair(x, wd, m, r0 + x.wave, nu);
      dq_pair(x, sKc, sVc, wd, m, r0, x.wave, nr2, b);
    }
    lds_barrier();
    dq_accumulate(x, kt, round_bits(m, r0, kDqSlots), acc);
  }
  walk_wait_vm();  // this wave's copies of the next K / V blocks (and the prefetch)
  lds_stores_done();
  __syncthreads();
}

__global__ void __launch_bounds__(kWalkThreads, 1)
dq_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ dO,
          const uint16_t *__restrict__ Kw, const uint16_t *__restrict__ Vw,
          const uint16_t *__restrict__ Kt, const float *__restrict__ LSE,
          const float *__restrict__ Delta, const int32_t *__restrict__ cu,
          const int32_t *__restrict__ cu_ws, int NB, const int32_t *__restrict__ plan,
          const int32_t *__restrict__ plan_len, const int32_t *__restrict__ plan_lists,
          float scale, float scale_log2e, uint16_t *__restrict__ dQ) {
  __shared__ __attribute__((aligned(16))) char sK0[kBlk * 256];
  __shared__ __attribute__((aligned(16))) char sK1[kBlk * 256];
  __shared__ __attribute__((aligned(16))) char sV0[kBlk * 256];
  __shared__ __attribute__((aligned(16))) char sV1[kBlk * 256];
  __shared__ __attribute__((aligned(16))) char sS[kDqSlots * 4096];
  const int p = blockIdx.x;
  if (p >= plan[0]) return;
  const i32x4 item = ((const i32x4 *)(plan + kPlanHeaderWords))[p];
  DqCtx x;
  x.Q = Q; x.dO = dO; x.Kw = Kw; x.Vw = Vw; x.Kt = Kt; x.LSE = LSE; x.Delta = Delta;
  x.i = uniform(item[0]); x.t0 = uniform(item[1]);
  const int n = uniform(item[2]), d = uniform(item[3]);
  x.tid = threadIdx.x; x.lane = x.tid & 63; x.wave = uniform(x.tid >> 6);
  x.l16 = x.lane & 15; x.g = x.lane >> 4;
  x.p0 = x.t0 - cu[d]; x.wsrow0 = cu_ws[d]; x.NB = NB;
  x.nact = uniform(plan_len[p]);
  x.list = plan_lists + (size_t)2 * kPlanMaxList * p;
  x.c = scale_log2e;
  x.sS = sS;

  f32x4 acc[kFwdGroup][2];
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) acc[u][0] = acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  DqUnit wn[2];
  if (x.nact > 0) {
    const uint32_t m0 = (uint32_t)uniform(x.list[1]);
    dq_load_pair(x, wn, m0, x.wave, __popc(m0));
    const size_t row0 = (size_t)x.wsrow0 + (size_t)x.list[0] * kBlk;
    block_dma(sK0, Kw, row0, x.i, x.tid);
    block_dma(sV0, Vw, row0, x.i, x.tid);
  }
  walk_wait_vm();
  __syncthreads();
  for (int a = 0; a < x.nact; a += 2) {
    dq_step(x, a, sK0, sV0, sK1, sV1, acc, wn);
    if (a + 1 < x.nact) dq_step(x, a + 1, sK1, sV1, sK0, sV0, acc, wn);
  }
  // ---- epilogue: acc[u][md][r] = dQ^T[dim 32w + 16md + 4g + r][head l16] / scale
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if (u < n) {
      uint16_t *qrow = dQ + ((size_t)(x.t0 + u) * kH + kHPI * x.i + x.l16) * kD + 32 * x.wave + 4 * x.g;
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
  hipLaunchKernelGGL(dq_kernel, dim3(items), dim3(kWalkThreads), 0, s, (const uint16_t *)Q,
                     (const uint16_t *)dO, (const uint16_t *)Kw, (const uint16_t *)Vw,
                     (const uint16_t *)Kt, LSE, delta, L.cu, L.cu_ws, L.NB, v.header, v.len,
                     v.lists, scale, scale * kLog2e, (uint16_t *)dQ);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
