// msa_forward.hip -- query-parallel MSA prefill forward for gfx950.
//
// What is computed ("feat(minimax-m3): add SM100 MSA sparse attention with custom
// backward", Design): for query token t and query head h of index head i = h / 16,
// softmax over the keys of the blocks listed in q2k[i][t] (document-local, causal),
// O[t,h] = sum_j P_j V_j and LSE[t,h] = log sum_j exp(scale <Q[t,h], K_j>).
//
// Design (gfx950): one workgroup of 4 waves (one per SIMD) per plan item = (index
// head i, up to MSA_FWD_GROUP consecutive queries of one document); a unit is one
// query with its 16 heads (16 rows that share a selection).  The item's Q rows stay in
// LDS for the whole item, and the workgroup walks the item's list of selected blocks,
// so each K / V block is read once per item, not once per query.  Per block:
//   S phase  -- wave w owns keys [32w, 32w + 32) of the block, whose K rows it holds
//               in registers; for every pair of active units it computes the 32 x 32
//               tile S^T = K [Q_u0 | Q_u1]^T (32x32x16 MFMAs, Q from LDS), turns it into
//               P (bf16) and stores P to the units' LDS slots;
//   PV phase -- wave w owns head dims [32w, 32w + 32) and updates O^T += V^T P^T for
//               every active unit (16x16x32 MFMAs); its V^T rows come straight from
//               the transposed workspace copy into registers, P^T from LDS.
// The O accumulators of all units stay in accumulation registers for the whole walk,
// and the K and V^T registers of the next block are loaded one step ahead.
//
// Softmax reference: each row's exponent reference m is the (base-2, scaled) maximum
// of its first block and never moves, so the accumulators are never rescaled and the
// later blocks need no maximum: P = 2^(c s - m), an elementwise step that lets every
// wave work on its own keys.  The reference is taken from wave 0's 32 keys of the
// unit's first block (they always include an unmasked key): any score of the row would
// do, as long as no later score exceeds it by 64 (base 2); then P, l and
// O stay far inside fp32 / bf16 range; a row whose sum l reaches 2^64 (which any such
// score forces) marks its item (LSE of the item's first row, first head = +inf), and a
// second launch of the kernel redoes exactly those items with the exact row maxima,
// found by a first walk over the blocks, as references.
#include "msa_walk.h"

namespace msa {

constexpr int kFwdSlots = 12;                    // P slots: active units per round
constexpr int kFwdSlotStride = kSlotBytes + 32;  // +32 B: paired slots start on other banks

struct FwdCtx {
  const uint16_t *Kw, *Vt;
  const int32_t *list;
  int nact, i, p0, wsrow0, NB;
  int tid, lane, wave, l16, g, l32, hi;
  float c;  // scale * log2(e)
  char *sQ, *sP;
  float *sM, *sLw;  // references; per-wave row sums [wave][unit][head]
  uint32_t qoff[8];  // swizzled byte offset of this lane's Q chunk for k-step ks
};

// Registers of one block: K rows 32w + l32, dims 16 ks + 8 hi .. + 7 (A operand of the
// 32x32x16 S tiles; loaded one step ahead) and V^T rows 32w + 16 md + l16, keys
// 32 kk + 8 g .. + 7 (A operand of the 16x16x32 PV tiles; loaded at the step's start,
// needed only after the S phase).
struct FwdK {
  bf16x8 k[8];
};
struct FwdV {
  bf16x8 v[2][4];
};

__device__ __forceinline__ void fwd_load_k(const FwdCtx &x, FwdK &kb, int b) {
  const uint16_t *krow =
      x.Kw + (((size_t)x.wsrow0 + (size_t)b * kBlk + 32 * x.wave + x.l32) * kHKV + x.i) * kD + 8 * x.hi;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kb.k[ks] = *(const bf16x8 *)(krow + 16 * ks);
}

__device__ __forceinline__ void fwd_load_v(const FwdCtx &x, FwdV &vb, int b) {
  const size_t gblk = (size_t)x.i * x.NB + (size_t)(x.wsrow0 / kBlk + b);
#pragma unroll
  for (int md = 0; md < 2; ++md) load_tslice(vb.v[md], x.Vt, gblk, 32 * x.wave + 16 * md, x.l16, x.g);
}

// Next unit of a (uniform) unit mask, removed from it.
__device__ __forceinline__ int pop_unit(uint32_t &mr) {
  const int u = __builtin_ctz(mr);
  mr &= mr - 1;
  return u;
}

// Q fragments (B operand of the S tile) of the pair (u0, u1): lane l32 < 16 reads unit
// u0, the others u1; q[ks] = Q[u][head l16][dims 16 ks + 8 hi .. + 7].
__device__ __forceinline__ void fwd_load_q(const FwdCtx &x, bf16x8 (&q)[8], int u0, int u1) {
  const char *qrow = x.sQ + (((x.l32 < 16) ? u0 : u1) * 16 + x.l16) * 256;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) q[ks] = *(const bf16x8 *)(qrow + x.qoff[ks]);
}

// S^T tile of the pair (u0, u1) for this wave's keys: st[r] = S^T[key 32w + 8 (r/4) +
// 4 hi + r%4][column l32], column = (half l32 / 16, head l32 % 16); the second half
// belongs to u1 (which may repeat u0 when the pair has one unit).
__device__ __forceinline__ f32x16 fwd_tile(const FwdCtx &x, const FwdK &kb, int u0, int u1) {
  bf16x8 q[8];
  fwd_load_q(x, q, u0, u1);
  f32x16 st;
#pragma unroll
  for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) st = mfma32(kb.k[ks], q[ks], st);
  return st;
}

// Causal mask of the tile when block b is the diagonal block of one of its units.
__device__ __forceinline__ void fwd_tile_mask(const FwdCtx &x, f32x16 &st, int u0, int u1, int b) {
  const int u = (x.l32 < 16) ? u0 : u1;
  const int qpos = x.p0 + u;
  if (b == (x.p0 + u0) / kBlk || b == (x.p0 + u1) / kBlk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = b * kBlk + 32 * x.wave + 8 * (r >> 2) + 4 * x.hi + (r & 3);
      if (key > qpos) st[r] = -INFINITY;
    }
  }
}

// Maximum over this wave's 32 keys of the tile column (all lanes of the column agree).
__device__ __forceinline__ float fwd_tile_max(const f32x16 &st) {
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(st[r], st[r + 1]));
  return fmaxf(mx, __shfl_xor(mx, 32));
}

// P = 2^(c s - m) of the tile to the slots of its units (round slot s0 + column half),
// row sums into this wave's sLw.  `two`: the second half holds a unit.
__device__ __forceinline__ void fwd_tile_p(const FwdCtx &x, const f32x16 &st, int u0, int u1, int s0,
                                           bool two) {
  const int half = x.l32 >> 4;
  const int u = half ? u1 : u0;
  const bool valid = !half || two;
  const float mn = x.sM[u * 16 + x.l16];
  float sum = 0.f;
  char *prow = x.sP + (s0 + half) * kFwdSlotStride + x.l16 * kSlotRow + (32 * x.wave + 4 * x.hi) * 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[4 * j + r], x.c, -mn));
      sum += e[r];
    }
    if (valid) *(u32x2 *)(prow + 16 * j) = u32x2{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
  }
  sum += __shfl_xor(sum, 32);
  if (valid && x.hi == 0) x.sLw[(x.wave * kFwdGroup + u) * 16 + x.l16] += sum;  // own wave only
}

// P^T fragments (B operand of the PV tiles) of P slot k: keys 32 kk + 8 g .., head l16.
__device__ __forceinline__ void fwd_load_p(const FwdCtx &x, bf16x8 (&pf)[4], int k) {
  const char *prow = x.sP + k * kFwdSlotStride + x.l16 * kSlotRow + 16 * x.g;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) pf[kk] = *(const bf16x8 *)(prow + 64 * kk);
}

// PV phase of one round: O^T[dims 32w.., heads] += V^T P^T for the nr units of mr,
// whose P slots are 0 .. nr - 1 in unit order.  The next slot's P fragments are read
// while the current unit's MFMAs run.
__device__ __forceinline__ void fwd_pv(const FwdCtx &x, const FwdV &vb, uint32_t mr, int nr,
                                       f32x4 (&acc)[kFwdGroup][2]) {
  bf16x8 pc[4];
  fwd_load_p(x, pc, 0);
  int k = 0;
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if (mr & 1u) {
      bf16x8 pn[4];
      fwd_load_p(x, pn, min(k + 1, nr - 1));
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int md = 0; md < 2; ++md) acc[u][md] = mfma16(vb.v[md][kk], pc[kk], acc[u][md]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) pc[kk] = pn[kk];
      k = uniform(k + 1);
    }
    mr = uniform(mr >> 1);
  }
}

// References of the units in `units` (a unit's first block): the maximum over wave
// 0's 32 keys of block b, published to all waves through sM.
__device__ __forceinline__ void fwd_references(const FwdCtx &x, const FwdK &blk, uint32_t units,
                                               int b) {
  if (x.wave == 0) {
    const int nf = __popc(units);
    for (int s0 = 0; s0 < nf; s0 += 2) {
      const int u0 = nth_set_bit(units, s0);
      const bool two = s0 + 1 < nf;
      const int u1 = two ? nth_set_bit(units, s0 + 1) : u0;
      f32x16 st = fwd_tile(x, blk, u0, u1);
      fwd_tile_mask(x, st, u0, u1, b);
      const float mx = fwd_tile_max(st) * x.c;
      const int u = (x.l32 < 16) ? u0 : u1;
      if (x.hi == 0 && (x.l32 < 16 || two)) x.sM[u * 16 + x.l16] = mx;
    }
  }
  lds_barrier();
}

// Exact-reference pass: folds the maximum of block b over all keys into sM for every
// unit in `units`.  The per-wave maxima go through sX (the row-sum area, unused in
// this pass); every wave then stores the same folded value.
__device__ __forceinline__ void fwd_fold_max(const FwdCtx &x, const FwdK &blk, uint32_t units, int b) {
  float *sX = x.sLw;
  const int nf = __popc(units);
  for (int s0 = 0; s0 < nf; s0 += 2) {
    const int u0 = nth_set_bit(units, s0);
    const bool two = s0 + 1 < nf;
    const int u1 = two ? nth_set_bit(units, s0 + 1) : u0;
    f32x16 st = fwd_tile(x, blk, u0, u1);
    fwd_tile_mask(x, st, u0, u1, b);
    const float mx = fwd_tile_max(st) * x.c;
    const int u = (x.l32 < 16) ? u0 : u1;
    if (x.hi == 0 && (x.l32 < 16 || two)) sX[(x.wave * kFwdGroup + u) * 16 + x.l16] = mx;
  }
  lds_barrier();
  for (int s0 = 0; s0 < nf; s0 += 2) {
    const int u0 = nth_set_bit(units, s0);
    const bool two = s0 + 1 < nf;
    const int u1 = two ? nth_set_bit(units, s0 + 1) : u0;
    const int u = (x.l32 < 16) ? u0 : u1;
    if (x.hi == 0 && (x.l32 < 16 || two)) {
      float mx = sX[u * 16 + x.l16];
#pragma unroll
      for (int w = 1; w < kWalkWaves; ++w) mx = fmaxf(mx, sX[(w * kFwdGroup + u) * 16 + x.l16]);
      float *pm = x.sM + u * 16 + x.l16;
      *pm = fmaxf(*pm, mx);
    }
  }
}

// S phase for the pair (u0, u1) [and the pair (u2, u3)] at P slots s0, s0 + 1 [s0 + 2,
// s0 + 3]: both tiles' MFMA chains are interleaved.
template <bool QUAD>
__device__ __forceinline__ void fwd_scores(const FwdCtx &x, const FwdK &kb, int u0, int u1, bool two01,
                                           int u2, int u3, bool two23, int s0, int b) {
  bf16x8 qa[8], qb[8];
  fwd_load_q(x, qa, u0, u1);
  if (QUAD) fwd_load_q(x, qb, u2, u3);
  f32x16 sa, sb;
#pragma unroll
  for (int r = 0; r < 16; ++r) sa[r] = sb[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    sa = mfma32(kb.k[ks], qa[ks], sa);
    if (QUAD) sb = mfma32(kb.k[ks], qb[ks], sb);
  }
  fwd_tile_mask(x, sa, u0, u1, b);
  fwd_tile_p(x, sa, u0, u1, s0, two01);
  if (QUAD) {
    fwd_tile_mask(x, sb, u2, u3, b);
    fwd_tile_p(x, sb, u2, u3, s0 + 2, two23);
  }
}

// One step of the walk over list entry a with the K registers in cur; the next entry's
// K registers are loaded into nxt.  seen: units whose reference is set.  MAXPASS only
// folds the block maxima into sM.
template <bool MAXPASS>
__device__ __forceinline__ void fwd_step(const FwdCtx &x, int a, const FwdK &cur, FwdK &nxt,
                                         f32x4 (&acc)[kFwdGroup][2], uint32_t &seen) {
  const int b = uniform(x.list[2 * a]);
  const uint32_t m = (uint32_t)uniform(x.list[2 * a + 1]);
  const int nu = __popc(m);
  FwdV vb;
  if (!MAXPASS) fwd_load_v(x, vb, b);
  // unconditional, so that the wait counts before the S phase do not depend on it (the
  // last step reloads its own block)
  fwd_load_k(x, nxt, a + 1 < x.nact ? uniform(x.list[2 * (a + 1)]) : b);
  if (MAXPASS) {
    fwd_fold_max(x, cur, m, b);
    lds_barrier();  // sX is rewritten by the next step
    return;
  }
  const uint32_t fresh = m & ~seen;
  if (fresh) fwd_references(x, cur, fresh, b);
  seen |= m;
  for (int r0 = 0; r0 < nu; r0 += kFwdSlots) {
    const int nr = min(kFwdSlots, nu - r0);
    const uint32_t mround = round_bits(m, r0, kFwdSlots);
    if (r0 > 0) lds_barrier();  // P slots are rewritten
    // ---- S phase: the round's units in pairs, two pairs at a time; this wave's keys
    uint32_t ms = mround;
    for (int s0 = 0; ms;) {
      const int u0 = pop_unit(ms);
      const bool two01 = ms != 0;
      const int u1 = two01 ? pop_unit(ms) : u0;
      if (ms) {
        const int u2 = pop_unit(ms);
        const bool two23 = ms != 0;
        const int u3 = two23 ? pop_unit(ms) : u2;
        fwd_scores<true>(x, cur, u0, u1, two01, u2, u3, two23, s0, b);
        s0 += 4;
      } else {
        fwd_scores<false>(x, cur, u0, u1, two01, u0, u0, false, s0, b);
        s0 += 2;
      }
    }
    lds_barrier();
    // ---- PV phase
    fwd_pv(x, vb, mround, nr, acc);
  }
  lds_barrier();  // P slots are rewritten by the next step
}

// The whole walk over the item's list.  seen0 = ~0 keeps the references already in
// sM (the exact maxima of the max pass).
template <bool MAXPASS>
__device__ __forceinline__ void fwd_walk(const FwdCtx &x, f32x4 (&acc)[kFwdGroup][2], uint32_t seen0) {
  FwdK k0, k1;
  uint32_t seen = seen0;
  if (x.nact > 0) fwd_load_k(x, k0, uniform(x.list[0]));
  for (int a = 0; a < x.nact; a += 2) {
    fwd_step<MAXPASS>(x, a, k0, k1, acc, seen);
    if (a + 1 < x.nact) fwd_step<MAXPASS>(x, a + 1, k1, k0, acc, seen);
  }
}

// REDO = false: every item, references from each row's first block.  REDO = true:
// only the items the first launch marked, with exact references from a max pass.
template <bool REDO>
__global__ void __launch_bounds__(kWalkThreads, 1)
fwd_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kw,
           const uint16_t *__restrict__ Vt, const int32_t *__restrict__ cu,
           const int32_t *__restrict__ cu_ws, int NB, const int32_t *__restrict__ plan,
           const int32_t *__restrict__ plan_len, const int32_t *__restrict__ plan_lists,
           float scale_log2e, uint16_t *__restrict__ O, float *__restrict__ LSE) {
  __shared__ __attribute__((aligned(16))) char sQ[kFwdGroup * 16 * 256];
  __shared__ __attribute__((aligned(16))) char sP[kFwdSlots * kFwdSlotStride];
  __shared__ float sM[kFwdGroup * 16], sLw[kWalkWaves * kFwdGroup * 16];
  __shared__ int sBad;
  const int p = blockIdx.x;
  if (p >= plan[0]) return;
  const i32x4 item = ((const i32x4 *)(plan + kPlanHeaderWords))[p];
  FwdCtx x;
  x.Kw = Kw; x.Vt = Vt;
  x.i = uniform(item[0]);
  const int t0 = uniform(item[1]), n = uniform(item[2]), d = uniform(item[3]);
  float *mark = LSE + (size_t)t0 * kH + kHPI * x.i;  // first row, first head of the item
  if (REDO && !(*mark == INFINITY)) return;
  x.tid = threadIdx.x; x.lane = x.tid & 63; x.wave = uniform(x.tid >> 6);
  x.l16 = x.lane & 15; x.g = x.lane >> 4; x.l32 = x.lane & 31; x.hi = x.lane >> 5;
  x.p0 = t0 - cu[d]; x.wsrow0 = cu_ws[d]; x.NB = NB;
  x.nact = uniform(plan_len[p]);
  x.list = plan_lists + (size_t)2 * kPlanMaxList * p;
  x.c = scale_log2e;
  x.sQ = sQ; x.sP = sP; x.sM = sM; x.sLw = sLw;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) x.qoff[ks] = (uint32_t)(((2 * ks + x.hi) ^ x.l16) << 4);

  // Q rows of the item (16 rows of 256 B per unit, contiguous in Q) into sQ, swz() layout
  {
    const char *src = (const char *)(Q + ((size_t)t0 * kH + kHPI * x.i) * kD);
    const int q = x.tid & 15;
    for (int r = x.tid >> 4; r < n * 16; r += kWalkThreads / 16)
      *(u32x4 *)(sQ + r * 256 + q * 16) =
          *(const u32x4 *)(src + (size_t)(r >> 4) * kH * kD * 2 + (r & 15) * 256 + ((q ^ (r & 15)) << 4));
  }
  for (int k = x.tid; k < kFwdGroup * 16; k += kWalkThreads) sM[k] = -INFINITY;
  if (x.tid == 0) sBad = 0;
  __syncthreads();
  f32x4 acc[kFwdGroup][2];
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) acc[u][0] = acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (REDO) fwd_walk<true>(x, acc, 0u);  // sM = exact row maxima
  for (int k = x.tid; k < kWalkWaves * kFwdGroup * 16; k += kWalkThreads) sLw[k] = 0.f;
  __syncthreads();
  fwd_walk<false>(x, acc, REDO ? ~0u : 0u);
  __syncthreads();
  // row sums in a fixed order; sLw[0][..] holds the total from here on
  float *sL = sLw;
  for (int k = x.tid; k < kFwdGroup * 16; k += kWalkThreads)
    sL[k] = (sLw[k] + sLw[kFwdGroup * 16 + k]) + (sLw[2 * kFwdGroup * 16 + k] + sLw[3 * kFwdGroup * 16 + k]);
  __syncthreads();
  // ---- epilogue: acc[u][md][r] = O^T[dim 32w + 16md + 4g + r][head l16]
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if (u < n) {
      const float l = sL[u * 16 + x.l16];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t *orow = O + ((size_t)(t0 + u) * kH + kHPI * x.i + x.l16) * kD + 32 * x.wave + 4 * x.g;
#pragma unroll
      for (int md = 0; md < 2; ++md) {
        const f32x4 v = acc[u][md] * inv;
        *(u32x2 *)(orow + 16 * md) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
  if (!REDO) {  // a score 64 (base 2) above its row's reference forces l past 2^64
    for (int k = x.tid; k < n * 16; k += kWalkThreads)
      if (!(sL[k] < 0x1p64f)) sBad = 1;
    __syncthreads();
  }
  const bool bad = !REDO && sBad != 0;
  for (int k = x.tid; k < n * 16; k += kWalkThreads) {
    const int u = k >> 4, hh = k & 15;
    const float l = sL[k], mm = sM[k];
    float lse = l > 0.f ? (mm + __log2f(l)) * kLn2 : -INFINITY;
    if (k == 0 && bad) lse = INFINITY;
    LSE[(size_t)(t0 + u) * kH + kHPI * x.i + hh] = lse;
  }
}

namespace host {
hipError_t forward(const void *Q, const void *Kw, const void *Vt, const int32_t *q2k,
                   const LayoutArgs &L, const void *plan, float scale, void *O, float *LSE,
                   hipStream_t s) {
  (void)q2k;  // the walk lists of the plan carry the selection
  PlanView v = plan_view(L, const_cast<void *>(plan));
  const unsigned items = (unsigned)(kHI * plan_gmax(L));
  hipLaunchKernelGGL(fwd_kernel<false>, dim3(items), dim3(kWalkThreads), 0, s, (const uint16_t *)Q,
                     (const uint16_t *)Kw, (const uint16_t *)Vt, L.cu, L.cu_ws, L.NB, v.header,
                     v.len, v.lists, scale * kLog2e, (uint16_t *)O, LSE);
  hipLaunchKernelGGL(fwd_kernel<true>, dim3(items), dim3(kWalkThreads), 0, s, (const uint16_t *)Q,
                     (const uint16_t *)Kw, (const uint16_t *)Vt, L.cu, L.cu_ws, L.NB, v.header,
                     v.len, v.lists, scale * kLog2e, (uint16_t *)O, LSE);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
