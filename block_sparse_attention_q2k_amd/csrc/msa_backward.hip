// msa_backward.hip -- KV-parallel MSA prefill backward for gfx950.
//
// What is computed (msa_backward_sm100 API page, module summary and run_backward):
// for every task row -- 8 queries x 16 heads = 128 rows that selected one key block of
// one index head -- with the block's 128 keys:
//   S = Q K^T, P = exp(scale S - LSE) (causal / padding mask), dP = dO V^T,
//   dS = P (dP - delta), dV += P^T dO, dK += scale dS^T Q, dQ += scale dS K.
// dK/dV accumulate in registers over the consecutive task rows of one bucket and are
// flushed with fp32 atomics at the end of the bucket segment; dQ is added per task
// row with atomics into a pool (fp32, packed bf16 pairs of dims, or packed f16 pairs of
// heads in a head-pair-interleaved pool).
//
// Design (gfx950): a persistent grid; workgroup c walks, for each index head, the task
// rows [cta[i][c], cta[i][c+1]).  Four waves; wave w owns keys [32w, 32w+32) of the
// block: its K and V slices live in registers (MFMA B operands of S and dP) and so do
// its dK/dV accumulators.  Per task row the Q and dO rows are gathered into LDS
// (16-byte-chunk swizzled), S and dP are computed with M = rows so that P and dS come
// out of the accumulators already in the A-operand layout of the dV/dK products (the
// row index is permuted consistently on both operands), and the transposed operands
// (dO, Q for dV/dK; dS and K for dQ) are read with ds_read_b64_tr_b16.  dQ needs the
// sum over all 128 keys, so dS^T goes through LDS and wave w computes dQ for dims
// [32w, 32w+32) with K^T[keys][those dims] held in registers.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr int kBwdThreads = 256;
constexpr int kBsK = 0;                   // [128 keys][256 B]
constexpr int kBsQ = kBsK + 128 * 256;    // [128 rows][256 B]
constexpr int kBsdO = kBsQ + 128 * 256;   // [128 rows][256 B]
constexpr int kBsdS = kBsdO + 128 * 256;  // dS^T [128 keys][128 rows] bf16
constexpr int kBsLse = kBsdS + 128 * 256; // f32 [128] (log2 domain)
constexpr int kBsDel = kBsLse + 512;      // f32 [128]
constexpr int kBsPos = kBsDel + 512;      // i32 [128] query position per row (-1 = empty)
constexpr int kBwdLds = kBsPos + 512;

__device__ inline void atomic_add_f32(float *p, float v) {
  __builtin_amdgcn_global_atomic_fadd_f32((__attribute__((address_space(1))) float *)p, v);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline void atomic_add_bf16x2(uint16_t *p, float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  __builtin_amdgcn_global_atomic_fadd_v2bf16((__attribute__((address_space(1))) bf16x2 *)p, v);
}
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Packed f16 pair add (round to nearest even in the conversion): lo, hi = the two heads of
// a head pair at one dim of the interleaved pool.
__device__ inline void atomic_add_f16x2(uint32_t *p, float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  __builtin_amdgcn_global_atomic_fadd_v2f16((__attribute__((address_space(1))) f16x2 *)p, v);
}

__global__ void __launch_bounds__(kBwdThreads, 1)
bwd_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kw,
           const uint16_t *__restrict__ Vw, const uint16_t *__restrict__ dO,
           const float *__restrict__ LSE, const float *__restrict__ Delta,
           const int32_t *__restrict__ cta, const i32x4 *__restrict__ meta,
           const int32_t *__restrict__ qrows, const int32_t *__restrict__ qpos,
           const int32_t *__restrict__ cu_ws, int ndocs, int NB, int grid, float scale,
           float scale_log2e, int mode, void *__restrict__ dq_pool, float *__restrict__ dk_pool,
           float *__restrict__ dv_pool) {
  __shared__ __attribute__((aligned(16))) char smem[kBwdLds];
  const lds_char *lds = (const lds_char *)smem;
  const int c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  float *sLse = (float *)(smem + kBsLse);
  float *sDel = (float *)(smem + kBsDel);
  int32_t *sPos = (int32_t *)(smem + kBsPos);

  f32x4 dkacc[2][8], dvacc[2][8];
  bf16x8 kf[2][4], vf[2][4];

  for (int i = 0; i < kHI; ++i) {
    const int lo = cta[i * (grid + 1) + c], hi = cta[i * (grid + 1) + c + 1];
    int cur_r = -1, kbase = 0, gb = 0;
    for (int row = lo; row < hi; ++row) {
      const i32x4 mt4 = meta[row];
      const int r = mt4[0], nv = mt4[1];
      if (r != cur_r) {
        cur_r = r;
        gb = r - i * NB;
        const int dd = upper_index(cu_ws, ndocs - 1, gb * kBlk);
        kbase = gb * kBlk - cu_ws[dd];  // document-local position of the block's key 0
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            dkacc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
            dvacc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        // K/V slices of this wave as B operands: lane (key 32w + 16nt + l16, g)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const size_t fb = ((size_t)i * NB + gb) * kFragBlock;
          const int key = 32 * wave + 16 * nt + l16;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            kf[nt][kk] = *(const bf16x8 *)(Kw + fb + frag_row_off(key, 32 * kk + 8 * g));
            vf[nt][kk] = *(const bf16x8 *)(Vw + fb + frag_row_off(key, 32 * kk + 8 * g));
          }
        }
        // whole K block -> LDS (the dQ product reads K^T from it); wait until every wave
        // is done with the previous block
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int id = tid + kBwdThreads * k, rr = id >> 4, cc = id & 15;
          const size_t src = ((size_t)i * NB + gb) * kFragBlock + frag_row_off(rr, cc * 8);
          *(u32x4 *)(smem + kBsK + swz(rr, cc * 16)) = *(const u32x4 *)(Kw + src);
        }
      }
      // ---- gather Q / dO rows of the task row: LDS row rho = 16 q + hh
      const int32_t *tq = qrows + (size_t)row * kTileQ;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int id = tid + kBwdThreads * k, rho = id >> 4, cc = id & 15;
        const int q = rho >> 4, hh = rho & 15;
        u32x4 vq = {0, 0, 0, 0}, vd = {0, 0, 0, 0};
        if (q < nv) {
          const size_t src = ((size_t)tq[q] * kH + kHPI * i + hh) * kD + cc * 8;
          vq = *(const u32x4 *)(Q + src);
          vd = *(const u32x4 *)(dO + src);
        }
        *(u32x4 *)(smem + kBsQ + swz(rho, cc * 16)) = vq;
        *(u32x4 *)(smem + kBsdO + swz(rho, cc * 16)) = vd;
      }
      if (tid < 128) {
        const int q = tid >> 4, hh = tid & 15;
        float lse2 = 0.f, del = 0.f;
        int pos = -1;
        if (q < nv) {
          const size_t o = (size_t)tq[q] * kH + kHPI * i + hh;
          lse2 = LSE[o] * kLog2e;
          del = Delta[o];
          pos = qpos[(size_t)row * kTileQ + q];
        }
        sLse[tid] = lse2;
        sDel[tid] = del;
        sPos[tid] = pos;
      }
      __syncthreads();
      // Two halves of 64 rows: S = Q K^T and dP = dO V^T (M = rows, N = this wave's 32
      // keys), then P, dS, the dV/dK updates and dS^T -> LDS for those rows.
#pragma unroll 1
      for (int half = 0; half < 2; ++half) {
        f32x4 sacc[4][2], pacc[4][2];
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
          const int mt = 4 * half + m4;
          sacc[m4][0] = sacc[m4][1] = pacc[m4][0] = pacc[m4][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const uint32_t off = swz(16 * mt + l16, (32 * kk + 8 * g) * 2);
            const bf16x8 qa = *(const bf16x8 *)(smem + kBsQ + off);
            const bf16x8 da = *(const bf16x8 *)(smem + kBsdO + off);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
              sacc[m4][nt] = mfma16(qa, kf[nt][kk], sacc[m4][nt]);
              pacc[m4][nt] = mfma16(da, vf[nt][kk], pacc[m4][nt]);
            }
          }
        }
        // P and dS (lane: key 32w + 16nt + l16; rows 16mt + 4g + r)
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
          const int mt = 4 * half + m4;
          const f32x4 lse4 = *(const f32x4 *)(sLse + 16 * mt + 4 * g);
          const f32x4 del4 = *(const f32x4 *)(sDel + 16 * mt + 4 * g);
          const i32x4 pos4 = *(const i32x4 *)(sPos + 16 * mt + 4 * g);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const int kp = kbase + 32 * wave + 16 * nt + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float pr = kp <= pos4[r]
                                   ? __builtin_amdgcn_exp2f(sacc[m4][nt][r] * scale_log2e - lse4[r])
                                   : 0.f;
              sacc[m4][nt][r] = pr;
              pacc[m4][nt][r] = pr * (pacc[m4][nt][r] - del4[r]);
            }
          }
        }
        // dV += P^T dO and dK += dS^T Q: M = keys, N = dims (8 tiles), K = rows
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int ks = 2 * half + k2;
          bf16x8 pa[2], sa[2];
#pragma unroll
          for (int mk = 0; mk < 2; ++mk) {
            const f32x4 p0 = sacc[2 * k2][mk], p1 = sacc[2 * k2 + 1][mk];
            const f32x4 s0 = pacc[2 * k2][mk], s1 = pacc[2 * k2 + 1][mk];
            pa[mk] = bf16x8{(__bf16)p0[0], (__bf16)p0[1], (__bf16)p0[2], (__bf16)p0[3],
                            (__bf16)p1[0], (__bf16)p1[1], (__bf16)p1[2], (__bf16)p1[3]};
            sa[mk] = bf16x8{(__bf16)s0[0], (__bf16)s0[1], (__bf16)s0[2], (__bf16)s0[3],
                            (__bf16)s1[0], (__bf16)s1[1], (__bf16)s1[2], (__bf16)s1[3]};
          }
#pragma unroll
          for (int nd = 0; nd < 8; ++nd) {
            // B: lane (dim 16nd + l16, g) holds rows 32ks + 4g + 0..3 and 32ks + 16 + 4g + 0..3
            const int c0 = 16 * nd + 4 * (l16 & 3);
            const int k0 = 32 * ks + 4 * g + (l16 >> 2);
            const bf16x8 db = cat8(lds_read_tr(lds, kBsdO + swz(k0, c0 * 2)),
                                   lds_read_tr(lds, kBsdO + swz(k0 + 16, c0 * 2)));
            const bf16x8 qb = cat8(lds_read_tr(lds, kBsQ + swz(k0, c0 * 2)),
                                   lds_read_tr(lds, kBsQ + swz(k0 + 16, c0 * 2)));
#pragma unroll
            for (int mk = 0; mk < 2; ++mk) {
              dvacc[mk][nd] = mfma16(pa[mk], db, dvacc[mk][nd]);
              dkacc[mk][nd] = mfma16(sa[mk], qb, dkacc[mk][nd]);
            }
          }
        }
        // dS^T -> LDS: lane (key 32w + 16nt + l16) rows 16mt + 4g + 0..3
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const f32x4 v = pacc[m4][nt];
            *(u32x2 *)(smem + kBsdS + swz(32 * wave + 16 * nt + l16, (16 * (4 * half + m4) + 4 * g) * 2)) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
      }
      __syncthreads();
      // ---- dQ = dS K for dims [32w, 32w+32): M = rows (8 tiles), N = 2 x 16 dims, K = keys.
      // A = dS from dS^T in LDS, B = K^T[keys][dims] from the block in LDS (both through
      // transposing reads).
      f32x4 qacc[8][2];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) qacc[mt][0] = qacc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k0 = 32 * kk + 8 * g + (l16 >> 2);
        bf16x8 kt[2];
#pragma unroll
        for (int nd = 0; nd < 2; ++nd) {
          const int c0 = 32 * wave + 16 * nd + 4 * (l16 & 3);
          kt[nd] = cat8(lds_read_tr(lds, kBsK + swz(k0, c0 * 2)), lds_read_tr(lds, kBsK + swz(k0 + 4, c0 * 2)));
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const int c0 = 16 * mt + 4 * (l16 & 3);
          const bf16x8 a = cat8(lds_read_tr(lds, kBsdS + swz(k0, c0 * 2)),
                                lds_read_tr(lds, kBsdS + swz(k0 + 4, c0 * 2)));
          qacc[mt][0] = mfma16(a, kt[0], qacc[mt][0]);
          qacc[mt][1] = mfma16(a, kt[1], qacc[mt][1]);
        }
      }
      // lane: dim 32w + 16nd + l16, rows 16mt + 4g + r = query mt, head 4g + r
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int q = mt;
        if (q < nv) {
          const size_t rowbase = ((size_t)tq[q] * kH + kHPI * i + 4 * g) * kD;
          if (mode == MSA_DQ_ACCUM_FP32) {
            float *pool = (float *)dq_pool + rowbase + 32 * wave + l16;
#pragma unroll
            for (int nd = 0; nd < 2; ++nd)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) atomic_add_f32(pool + rr * kD + 16 * nd, scale * qacc[mt][nd][rr]);
          } else if (mode == MSA_DQ_ACCUM_F16X2) {
            // heads 4g + 2hp and 4g + 2hp + 1 of this lane's dim form head pair
            // 8i + 2g + hp: one packed pair add each, no lane exchange
            uint32_t *pool = (uint32_t *)dq_pool + ((size_t)tq[q] * (kH / 2) + (kHPI / 2) * i + 2 * g) * kD +
                             32 * wave + l16;
#pragma unroll
            for (int nd = 0; nd < 2; ++nd)
#pragma unroll
              for (int hp = 0; hp < 2; ++hp)
                atomic_add_f16x2(pool + hp * kD + 16 * nd, scale * qacc[mt][nd][2 * hp],
                                 scale * qacc[mt][nd][2 * hp + 1]);
          } else {
            // pair lanes (l16 even, odd): even lane adds rows 0,1, odd lane rows 2,3
            uint16_t *pool = (uint16_t *)dq_pool + rowbase + 32 * wave + (l16 & ~1);
            const bool odd = l16 & 1;
#pragma unroll
            for (int nd = 0; nd < 2; ++nd) {
              float o[4];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) o[rr] = __shfl_xor(qacc[mt][nd][rr], 1);
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) {
                const int rr = odd ? 2 + h2 : h2;
                const float mine = scale * qacc[mt][nd][rr], other = scale * o[rr];
                atomic_add_bf16x2(pool + rr * kD + 16 * nd, odd ? other : mine, odd ? mine : other);
              }
            }
          }
        }
      }
      // ---- end of this bucket's segment in this workgroup: flush dK/dV
      const bool seg_end = (row + 1 == hi) || (meta[row + 1][0] != r);
      if (seg_end) {
        // lane (dim 16nd + l16, g): keys 32w + 16mk + 4g + r
#pragma unroll
        for (int mk = 0; mk < 2; ++mk)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const size_t o = ((size_t)(gb * kBlk + 32 * wave + 16 * mk + 4 * g + rr) * kHKV + i) * kD + l16;
#pragma unroll
            for (int nd = 0; nd < 8; ++nd) {
              atomic_add_f32(dk_pool + o + 16 * nd, scale * dkacc[mk][nd][rr]);
              atomic_add_f32(dv_pool + o + 16 * nd, dvacc[mk][nd][rr]);
            }
          }
        cur_r = -1;
      }
    }
  }
}

namespace host {
hipError_t backward_main(const void *Q, const void *Kw, const void *Vw, const void *dO,
                         const float *LSE, const float *delta, const void *tasks,
                         const LayoutArgs &L, int grid, float scale, int mode, void *dq_pool,
                         float *dk_pool, float *dv_pool, hipStream_t s) {
  TaskView v = task_view(L, grid, const_cast<void *>(tasks));
  hipLaunchKernelGGL(bwd_kernel, dim3(grid), dim3(kBwdThreads), 0, s, (const uint16_t *)Q,
                     (const uint16_t *)Kw, (const uint16_t *)Vw, (const uint16_t *)dO, LSE, delta,
                     v.cta, (const i32x4 *)v.meta, v.qrows, v.qpos, L.cu_ws, L.ndocs, L.NB, grid,
                     scale, scale * kLog2e, mode, dq_pool, dk_pool, dv_pool);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
