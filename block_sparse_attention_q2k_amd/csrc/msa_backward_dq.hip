// msa_backward_dq.hip -- query-parallel dQ of the MSA prefill backward for gfx950.
//
// What is computed (msa_backward_sm100 API page, run_backward; the backward of the
// operator in "feat(minimax-m3): add SM100 MSA sparse attention with custom
// backward"): dQ[t,h] = scale sum_j dS_j K_j with dS_j = P_j (dP_j - delta[t,h]),
// P_j = exp(scale <Q[t,h], K_j> - LSE[t,h]) and dP_j = <dO[t,h], V_j>, over the keys j
// of the blocks q2k[h/16][t] selects (document-local, causal).
//
// Design (gfx950): one workgroup per plan item (index head, up to 8 queries of one
// document), walking the item's list of selected blocks like the forward.  Because
// each query's dQ sums over its own selected blocks only, walking them with dQ in
// registers makes every dQ element a plain store -- no pool, no atomics.  Per block:
//   S phase  -- active units spread over the 4 waves (four at a time); a wave
//               recomputes S^T = K Q^T and dP^T = V dO^T (K, V from LDS), forms P with
//               the saved LSE and dS = P (dP - delta), and writes dS (bf16) to LDS;
//   dQ phase -- wave w owns dims [32w, 32w + 32): dQ^T += K^T dS^T for those units,
//               K^T from the transposed workspace copy.
// Sized for two workgroups per CU (80 KB LDS, <= 256 registers).
#include "msa_walk.h"

namespace msa {

constexpr int kDqSlots = 4;                               // dS slots: active units per round
constexpr int kQsK = 0;                                   // [128 keys][256 B]
constexpr int kQsV = kQsK + 128 * 256;                    // [128 keys][256 B]
constexpr int kQsS = kQsV + 128 * 256;                    // dS [4 slots][16 heads][256 B]
constexpr int kDqLds = kQsS + kDqSlots * 16 * 256;

__global__ void __launch_bounds__(kWalkThreads, 2)
dq_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ dO,
          const uint16_t *__restrict__ Kw, const uint16_t *__restrict__ Vw,
          const uint16_t *__restrict__ Kt, const float *__restrict__ LSE,
          const float *__restrict__ Delta, const int32_t *__restrict__ cu,
          const int32_t *__restrict__ cu_ws, int NB, const int32_t *__restrict__ plan,
          const int32_t *__restrict__ plan_len, const int32_t *__restrict__ plan_lists,
          float scale, float scale_log2e, uint16_t *__restrict__ dQ) {
  __shared__ __attribute__((aligned(16))) char smem[kDqLds];
  const int p = blockIdx.x;
  if (p >= plan[0]) return;
  const i32x4 item = ((const i32x4 *)(plan + kPlanHeaderWords))[p];
  const int i = item[0], t0 = item[1], n = item[2], d = item[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6), l16 = lane & 15, g = lane >> 4;
  const int p0 = t0 - cu[d], wsrow0 = cu_ws[d];
  const int nact = plan_len[p];
  const int32_t *list = plan_lists + (size_t)2 * kPlanMaxList * p;

  f32x4 acc[kFwdGroup][2];
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) acc[u][0] = acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int a = 0; a < nact; ++a) {
    const int b = list[2 * a];
    const uint32_t m = (uint32_t)list[2 * a + 1];
    const size_t gblk = (size_t)i * NB + (size_t)(wsrow0 / kBlk + b);
    {  // this block's K and V into LDS (the previous step ended with a barrier)
      u32x4 pre[8];
      block_load(pre, Kw, (size_t)wsrow0 + (size_t)b * kBlk, i, tid);
      block_store(pre, smem + kQsK, tid);
      block_load(pre, Vw, (size_t)wsrow0 + (size_t)b * kBlk, i, tid);
      block_store(pre, smem + kQsV, tid);
    }
    // K^T slice of this wave (dims 32w + 16md + l16, keys 32kk + 8g + 0..7)
    bf16x8 kt[2][4];
#pragma unroll
    for (int md = 0; md < 2; ++md)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kt[md][kk] = *(const bf16x8 *)(Kt + (gblk * kD + 32 * wave + 16 * md + l16) * kBlk + 32 * kk + 8 * g);
    __syncthreads();
    const int nu = __popc(m);
    for (int c0 = 0; c0 < nu; c0 += kDqSlots) {
      // ---- S phase: unit of slot c0 + wave
      const int s = c0 + wave;
      if (s < nu) {
        const int u = nth_set_bit(m, s);
        const int t = t0 + u, qpos = p0 + u;
        const size_t o = (size_t)t * kH + kHPI * i + l16;  // this lane's head
        const float lse2 = LSE[o] * kLog2e, del = Delta[o];
        bf16x8 qf[4], df[4];
        load_rows16(qf, Q, t, i, l16, g);
        load_rows16(df, dO, t, i, l16, g);
        const bool diag = (b == qpos / kBlk);
        char *srow = smem + kQsS + wave * 4096;
#pragma unroll 1
        for (int h2 = 0; h2 < 2; ++h2) {  // keys 64 h2 .. 64 h2 + 63
          f32x4 sacc[4], pacc[4];
#pragma unroll
          for (int m4 = 0; m4 < 4; ++m4) sacc[m4] = pacc[m4] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            bf16x8 kf[4], vf[4];  // fragments first, then 8 independent MFMAs
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
              const uint32_t off = swz(16 * (4 * h2 + m4) + l16, (32 * kk + 8 * g) * 2);
              kf[m4] = *(const bf16x8 *)(smem + kQsK + off);
              vf[m4] = *(const bf16x8 *)(smem + kQsV + off);
            }
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
              sacc[m4] = mfma16(kf[m4], qf[kk], sacc[m4]);
              pacc[m4] = mfma16(vf[m4], df[kk], pacc[m4]);
            }
          }
          // [m4][r]: key 16 (4 h2 + m4) + 4g + r, head l16
#pragma unroll
          for (int m4 = 0; m4 < 4; ++m4) {
            const int mt = 4 * h2 + m4;
            float ds[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const bool ok = !(diag && (b * kBlk + 16 * mt + 4 * g + r > qpos));
              const float pr = ok ? __builtin_amdgcn_exp2f(sacc[m4][r] * scale_log2e - lse2) : 0.f;
              ds[r] = pr * (pacc[m4][r] - del);
            }
            *(u32x2 *)(srow + swz(l16, (16 * mt + 4 * g) * 2)) =
                u32x2{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3])};
          }
        }
      }
      __syncthreads();
      // ---- dQ phase: dQ^T[dims 32w.., heads] += K^T dS^T for the round's units
#pragma unroll
      for (int u = 0; u < kFwdGroup; ++u) {
        if ((m >> u) & 1) {
          const int su = __popc(m & ((1u << u) - 1)) - c0;
          if (su >= 0 && su < kDqSlots) {
            const char *srow = smem + kQsS + su * 4096;
            bf16x8 sf[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) sf[kk] = *(const bf16x8 *)(srow + swz(l16, (32 * kk + 8 * g) * 2));
#pragma unroll
            for (int md = 0; md < 2; ++md)
#pragma unroll
              for (int kk = 0; kk < 4; ++kk) acc[u][md] = mfma16(kt[md][kk], sf[kk], acc[u][md]);
          }
        }
      }
      __syncthreads();
    }
  }
  // ---- epilogue: acc[u][md][r] = dQ^T[dim 32w + 16md + 4g + r][head l16] / scale
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if (u < n) {
      uint16_t *qrow = dQ + ((size_t)(t0 + u) * kH + kHPI * i + l16) * kD + 32 * wave + 4 * g;
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
