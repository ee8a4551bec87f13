// msa_forward.hip -- query-parallel MSA prefill forward for gfx950.
//
// What is computed ("feat(minimax-m3): add SM100 MSA sparse attention with custom
// backward", Design): for query token t and query head h of index head i = h / 16,
// softmax over the keys of the blocks listed in q2k[i][t] (document-local, causal),
// O[t,h] = sum_j P_j V_j and LSE[t,h] = log sum_j exp(scale <Q[t,h], K_j>).
//
// Design (gfx950): one workgroup per plan item = (index head i, up to 8 consecutive
// queries of one document); a unit is one query with its 16 heads (M = 16 rows that
// share a selection).  The workgroup walks the item's list of selected blocks
// (computed by the plan), so each K block is read once per item, not once per query:
//   S phase  -- the units that selected the block are spread over the 4 waves; a wave
//               computes S^T = K Q^T (16x16x32 bf16 MFMA, K from LDS, Q from global),
//               updates the unit's running max / sum (online softmax in base 2, scale
//               and log2 e folded in) and writes P (bf16) and the rescale factor to LDS;
//   PV phase -- wave w owns head dims [32w, 32w + 32) and updates O^T += V^T P^T for
//               every active unit; its V^T slice comes straight from the transposed
//               workspace copy (keys contiguous), P^T from LDS.
// The next block's K is loaded into registers one step ahead.  Sized for two
// workgroups per CU (< 80 KB LDS, <= 256 registers) so that one workgroup's memory
// waits, barriers and softmax VALU work overlap the other's matrix work.
#include "msa_walk.h"

namespace msa {

constexpr int kFsK = 0;                                   // [128 keys][256 B]
constexpr int kFsP = kFsK + 128 * 256;                    // [8 slots][16 heads][256 B]
constexpr int kFsM = kFsP + kFwdGroup * 16 * 256;         // f32 [8 units][16 heads]
constexpr int kFsL = kFsM + kFwdGroup * 16 * 4;           // f32 [8][16]
constexpr int kFsA = kFsL + kFwdGroup * 16 * 4;           // f32 [8 slots][16 heads]
constexpr int kFwdLds = kFsA + kFwdGroup * 16 * 4;

__global__ void __launch_bounds__(kWalkThreads, 2)
fwd_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kw,
           const uint16_t *__restrict__ Vt, const int32_t *__restrict__ cu,
           const int32_t *__restrict__ cu_ws, int NB, const int32_t *__restrict__ plan,
           const int32_t *__restrict__ plan_len, const int32_t *__restrict__ plan_lists,
           float scale_log2e, uint16_t *__restrict__ O, float *__restrict__ LSE) {
  __shared__ __attribute__((aligned(16))) char smem[kFwdLds];
  const int p = blockIdx.x;
  if (p >= plan[0]) return;
  const i32x4 item = ((const i32x4 *)(plan + kPlanHeaderWords))[p];
  const int i = item[0], t0 = item[1], n = item[2], d = item[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6), l16 = lane & 15, g = lane >> 4;
  const int p0 = t0 - cu[d], wsrow0 = cu_ws[d];
  const int nact = plan_len[p];
  const int32_t *list = plan_lists + (size_t)2 * kPlanMaxList * p;

  float *sM = (float *)(smem + kFsM);
  float *sL = (float *)(smem + kFsL);
  float *sA = (float *)(smem + kFsA);
  for (int k = tid; k < kFwdGroup * 16; k += kWalkThreads) {
    sM[k] = -INFINITY;
    sL[k] = 0.f;
  }
  f32x4 acc[kFwdGroup][2];
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) acc[u][0] = acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 kpre[8];
  if (nact > 0) {
    block_load(kpre, Kw, (size_t)wsrow0 + (size_t)list[0] * kBlk, i, tid);
    block_store(kpre, smem + kFsK, tid);
    if (nact > 1) block_load(kpre, Kw, (size_t)wsrow0 + (size_t)list[2] * kBlk, i, tid);
  }
  __syncthreads();

  for (int a = 0; a < nact; ++a) {
    const int b = list[2 * a];
    const uint32_t m = (uint32_t)list[2 * a + 1];
    const size_t gblk = (size_t)i * NB + (size_t)(wsrow0 / kBlk + b);
    // V^T slice of this wave (dims 32w + 16md + l16, keys 32kk + 8g + 0..7)
    bf16x8 vt[2][4];
#pragma unroll
    for (int md = 0; md < 2; ++md)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        vt[md][kk] = *(const bf16x8 *)(Vt + (gblk * kD + 32 * wave + 16 * md + l16) * kBlk + 32 * kk + 8 * g);
    // ---- S phase: this wave's share of the active units
    const int nu = __popc(m);
    for (int s = wave; s < nu; s += 4) {
      const int u = nth_set_bit(m, s);
      const int qpos = p0 + u;
      bf16x8 qf[4];
      load_rows16(qf, Q, t0 + u, i, l16, g);
      f32x4 sacc[8];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {  // 4 key tiles' fragments first, then 4 MFMAs
          bf16x8 kf[4];
#pragma unroll
          for (int m4 = 0; m4 < 4; ++m4)
            kf[m4] = *(const bf16x8 *)(smem + kFsK + swz(16 * (4 * h2 + m4) + l16, (32 * kk + 8 * g) * 2));
#pragma unroll
          for (int m4 = 0; m4 < 4; ++m4) sacc[4 * h2 + m4] = mfma16(kf[m4], qf[kk], sacc[4 * h2 + m4]);
        }
      // sacc[mt][r] = S^T[key 16mt + 4g + r][head l16]
      const bool diag = (b == qpos / kBlk);
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = sacc[mt][r] * scale_log2e;
          if (diag && (b * kBlk + 16 * mt + 4 * g + r > qpos)) x = -INFINITY;
          sacc[mt][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_old = sM[u * 16 + l16];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.f;
      char *prow = smem + kFsP + s * 4096;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = __builtin_amdgcn_exp2f(sacc[mt][r] - m_new);
          sum += e[r];
        }
        *(u32x2 *)(prow + swz(l16, (16 * mt + 4 * g) * 2)) =
            u32x2{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
      }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);
      if (g == 0) {
        sL[u * 16 + l16] = alpha * sL[u * 16 + l16] + sum;
        sM[u * 16 + l16] = m_new;
        sA[s * 16 + l16] = alpha;
      }
    }
    __syncthreads();
    // next block's K into LDS (every wave is done reading this one); prefetch the one after
    if (a + 1 < nact) {
      block_store(kpre, smem + kFsK, tid);
      if (a + 2 < nact) block_load(kpre, Kw, (size_t)wsrow0 + (size_t)list[2 * (a + 2)] * kBlk, i, tid);
    }
    // ---- PV phase: O^T[dims 32w.., heads] += V^T P^T for every active unit
#pragma unroll
    for (int u = 0; u < kFwdGroup; ++u) {
      if ((m >> u) & 1) {
        const int s = __popc(m & ((1u << u) - 1));
        const float alpha = sA[s * 16 + l16];
        const char *prow = smem + kFsP + s * 4096;
        bf16x8 pf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) pf[kk] = *(const bf16x8 *)(prow + swz(l16, (32 * kk + 8 * g) * 2));
#pragma unroll
        for (int md = 0; md < 2; ++md) {
          acc[u][md] *= alpha;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) acc[u][md] = mfma16(vt[md][kk], pf[kk], acc[u][md]);
        }
      }
    }
    __syncthreads();
  }
  // ---- epilogue: acc[u][md][r] = O^T[dim 32w + 16md + 4g + r][head l16]
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if (u < n) {
      const float l = sL[u * 16 + l16];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t *orow = O + ((size_t)(t0 + u) * kH + kHPI * i + l16) * kD + 32 * wave + 4 * g;
#pragma unroll
      for (int md = 0; md < 2; ++md) {
        const f32x4 v = acc[u][md] * inv;
        *(u32x2 *)(orow + 16 * md) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
  if (tid < n * 16) {
    const int u = tid >> 4, hh = tid & 15;
    const float l = sL[tid], mm = sM[tid];
    LSE[(size_t)(t0 + u) * kH + kHPI * i + hh] = l > 0.f ? (mm + __log2f(l)) * kLn2 : -INFINITY;
  }
}

namespace host {
hipError_t forward(const void *Q, const void *Kw, const void *Vt, const int32_t *q2k,
                   const LayoutArgs &L, const void *plan, float scale, void *O, float *LSE,
                   hipStream_t s) {
  (void)q2k;  // the walk lists of the plan carry the selection
  PlanView v = plan_view(L, const_cast<void *>(plan));
  const unsigned items = (unsigned)(kHI * plan_gmax(L));
  hipLaunchKernelGGL(fwd_kernel, dim3(items), dim3(kWalkThreads), 0, s, (const uint16_t *)Q,
                     (const uint16_t *)Kw, (const uint16_t *)Vt, L.cu, L.cu_ws, L.NB, v.header,
                     v.len, v.lists, scale * kLog2e, (uint16_t *)O, LSE);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
