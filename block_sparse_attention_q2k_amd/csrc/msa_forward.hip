// msa_forward.hip -- query-parallel MSA prefill forward for gfx950.
//
// What is computed ("feat(minimax-m3): add SM100 MSA sparse attention with custom
// backward", Design): for query token t and query head h of index head i = h / 16,
// softmax over the keys of the blocks listed in q2k[i][t] (document-local, causal),
// O[t,h] = sum_j P_j V_j and LSE[t,h] = log sum_j exp(scale <Q[t,h], K_j>).
//
// Design (gfx950): one workgroup per plan item = (index head i, up to 16 consecutive
// queries of one document).  A "unit" is one query of the item with its 16 heads, the
// M=16 rows that share one selection.  The workgroup walks the union of the units'
// selected key blocks in ascending order, so every K/V block is read from HBM/L2 once
// per item instead of once per query.  For each block:
//   S phase  -- the units that selected the block are spread over the 4 waves; a wave
//               computes S^T = K Q^T (16x16x32 bf16 MFMA, K from LDS, Q^T from global),
//               updates the unit's running max/sum (online softmax, base 2 with the
//               scale and log2 e folded in) and writes P (bf16) and the rescale factor
//               to LDS;
//   PV phase -- every wave owns 32 of the 128 head dims and updates O^T += V^T P^T for
//               every active unit (V^T through transposing LDS reads, P^T from LDS),
//               so the PV work is balanced whatever the selection pattern.
// O accumulators stay in registers for the whole item (16 units x 16 heads x 32 dims
// per wave).
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kFwdThreads = 256;
constexpr int kFwdWin = 1024;  // key blocks per union window

// LDS layout (bytes)
constexpr int kFsK = 0;                                   // [128 keys][256 B]
constexpr int kFsV = kFsK + 128 * 256;                    // [128 keys][256 B]
constexpr int kFsP = kFsV + 128 * 256;                    // [16 slots][16 heads][256 B]
constexpr int kFsM = kFsP + kFwdGroup * 16 * 256;         // f32 [16 units][16 heads]
constexpr int kFsL = kFsM + kFwdGroup * 16 * 4;           // f32 [16][16]
constexpr int kFsA = kFsL + kFwdGroup * 16 * 4;           // f32 [16 slots][16 heads]
constexpr int kFsMask = kFsA + kFwdGroup * 16 * 4;        // u32 [kFwdWin]
constexpr int kFsList = kFsMask + kFwdWin * 4;            // i32 [kFwdWin]
constexpr int kFsScan = kFsList + kFwdWin * 4;            // i32 [256]
constexpr int kFwdLds = kFsScan + kFwdThreads * 4;

__device__ inline int nth_set_bit(uint32_t m, int s) {
  for (int k = 0; k < s; ++k) m &= m - 1;
  return __builtin_ctz(m);
}

__global__ void __launch_bounds__(kFwdThreads, 1)
fwd_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kw,
           const uint16_t *__restrict__ Vw, const int32_t *__restrict__ q2k,
           const int32_t *__restrict__ cu, const int32_t *__restrict__ cu_ws, int T,
           const int32_t *__restrict__ plan, float scale_log2e, uint16_t *__restrict__ O,
           float *__restrict__ LSE) {
  __shared__ __attribute__((aligned(16))) char smem[kFwdLds];
  const lds_char *lds = (const lds_char *)smem;
  const int p = blockIdx.x;
  if (p >= plan[0]) return;
  const i32x4 item = ((const i32x4 *)(plan + kPlanHeaderWords))[p];
  const int i = item[0], t0 = item[1], n = item[2], d = item[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int base = cu[d], p0 = t0 - base, wsrow0 = cu_ws[d];
  const int blk_last = (p0 + n - 1) / kBlk;

  float *sM = (float *)(smem + kFsM);
  float *sL = (float *)(smem + kFsL);
  float *sA = (float *)(smem + kFsA);
  uint32_t *sMask = (uint32_t *)(smem + kFsMask);
  int32_t *sList = (int32_t *)(smem + kFsList);
  int32_t *sScan = (int32_t *)(smem + kFsScan);

  for (int k = tid; k < kFwdGroup * 16; k += kFwdThreads) {
    sM[k] = -INFINITY;
    sL[k] = 0.f;
  }
  f32x4 acc[kFwdGroup][2];
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    acc[u][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int wbase = 0; wbase <= blk_last; wbase += kFwdWin) {
    const int wn = min(kFwdWin, blk_last + 1 - wbase);
    for (int k = tid; k < kFwdWin; k += kFwdThreads) sMask[k] = 0;
    __syncthreads();
    {  // thread (unit u, slot j): mark its member block
      const int u = tid >> 4, j = tid & 15;
      if (u < n) {
        const int b = q2k[((size_t)i * T + t0 + u) * kTopk + j];
        const int blk_t = (p0 + u) / kBlk;
        if (b >= 0 && b <= blk_t && b >= wbase && b < wbase + wn) atomicOr(&sMask[b - wbase], 1u << u);
      }
    }
    __syncthreads();
    // compact the non-empty blocks of the window (ascending)
    constexpr int kPer = kFwdWin / kFwdThreads;
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) cnt += (sMask[tid * kPer + k] != 0);
    sScan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kFwdThreads; off <<= 1) {
      int v = tid >= off ? sScan[tid - off] : 0;
      __syncthreads();
      sScan[tid] += v;
      __syncthreads();
    }
    {
      int o = sScan[tid] - cnt;
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        if (sMask[tid * kPer + k] != 0) sList[o++] = tid * kPer + k;
    }
    const int nact = sScan[kFwdThreads - 1];
    __syncthreads();

    for (int a = 0; a < nact; ++a) {
      const int bl = sList[a];
      const int b = wbase + bl;
      const uint32_t m = sMask[bl];
      // ---- K/V block -> LDS
      {
        const size_t row0 = (size_t)(wsrow0 + b * kBlk);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int id = tid + kFwdThreads * k, r = id >> 4, c = id & 15;
          const size_t src = ((row0 + r) * kHKV + i) * kD + c * 8;
          const u32x4 kv = *(const u32x4 *)(Kw + src);
          const u32x4 vv = *(const u32x4 *)(Vw + src);
          *(u32x4 *)(smem + kFsK + swz(r, c * 16)) = kv;
          *(u32x4 *)(smem + kFsV + swz(r, c * 16)) = vv;
        }
      }
      __syncthreads();
      // ---- S phase
      const int nu = __popc(m);
      for (int s = wave; s < nu; s += 4) {
        const int u = nth_set_bit(m, s);
        const int t = t0 + u, qpos = p0 + u;
        const uint16_t *qrow = Q + ((size_t)t * kH + kHPI * i + l16) * kD + 8 * g;
        bf16x8 qf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[kk] = *(const bf16x8 *)(qrow + 32 * kk);
        f32x4 sacc[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 kf = *(const bf16x8 *)(smem + kFsK + swz(16 * mt + l16, (32 * kk + 8 * g) * 2));
            sacc[mt] = mfma16(kf, qf[kk], sacc[mt]);
          }
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
      // ---- PV phase: wave owns dims [32*wave, 32*wave + 32)
      bf16x8 vf[2][4];
#pragma unroll
      for (int md = 0; md < 2; ++md)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int c0 = 32 * wave + 16 * md + 4 * (l16 & 3);
          const int k0 = 32 * kk + 8 * g + (l16 >> 2);
          const bf16x4 lo = lds_read_tr(lds, kFsV + swz(k0, c0 * 2));
          const bf16x4 hi = lds_read_tr(lds, kFsV + swz(k0 + 4, c0 * 2));
          vf[md][kk] = cat8(lo, hi);
        }
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
            for (int kk = 0; kk < 4; ++kk) acc[u][md] = mfma16(vf[md][kk], pf[kk], acc[u][md]);
          }
        }
      }
      __syncthreads();
    }
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
    const int u = tid >> 4, h = tid & 15;
    const float l = sL[tid], mm = sM[tid];
    LSE[(size_t)(t0 + u) * kH + kHPI * i + h] = l > 0.f ? (mm + __log2f(l)) * kLn2 : -INFINITY;
  }
}

namespace host {
hipError_t forward(const void *Q, const void *Kw, const void *Vw, const int32_t *q2k,
                   const LayoutArgs &L, const void *plan, float scale, void *O, float *LSE,
                   hipStream_t s) {
  const unsigned items = (unsigned)(kHI * plan_gmax(L));
  hipLaunchKernelGGL(fwd_kernel, dim3(items), dim3(kFwdThreads), 0, s, (const uint16_t *)Q,
                     (const uint16_t *)Kw, (const uint16_t *)Vw, q2k, L.cu, L.cu_ws, L.T,
                     (const int32_t *)plan, scale * kLog2e, (uint16_t *)O, LSE);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
