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
//               the transposed workspace copy into registers, P^T from LDS.  The row
//               sums of the same bf16 P values are taken here too (one wave per unit).
// With one wave per SIMD nothing hides an LDS read's latency but the wave's own
// instruction stream, so the LDS operands of the next pair / unit are read before
// the current one's MFMAs are issued.
// The O accumulators of all units stay in accumulation registers for the whole walk;
// the K rows and V^T slices of the next block are loaded during the current step, in
// four groups spread over it.
//
// Softmax reference: each row's exponent reference m is the (base-2, scaled) maximum
// of its first block and never moves, so the accumulators are never rescaled and the
// later blocks need no maximum: P = 2^(c s - m), an elementwise step that lets every
// wave work on its own keys.  The reference is taken from wave 0's 32 keys of the
// unit's first block (they always include an unmasked key): any score of the row would
// do, as long as no later score exceeds it by 64 (base 2); then P, l and O stay far
// inside fp32 / bf16 range.  A row whose sum l reaches 2^64 (which any such score
// forces) marks its item (LSE of the item's first row, first head = +inf), and a
// second launch of the kernel redoes exactly those items with the exact row maxima,
// found by a first walk over the blocks, as references.
#include "msa_walk.h"

namespace msa {

constexpr int kFwdSlots = kFwdGroup;  // P slots: one per unit of the item
static_assert(kFwdGroup <= 32, "unit masks are 32-bit");
static_assert((kFwdSlots & (kFwdSlots - 1)) == 0, "the P slots form a ring indexed modulo their count");

struct FwdCtx {
  WalkLane w;
  const uint16_t *Kw, *Vt;
  const int32_t *list;
  int nact, i, p0, wsrow0, NB;
  float c;  // scale * log2(e)
  const char *sQ;
  char *sP;
  int sbase;  // ring position of the step's first P slot
  float *sM, *sX;  // references [unit][head]; exchange area [wave][unit][head]
  const char *qrow;   // this lane's Q row of unit 0: sQ + l16 * kUnitRow + 16 hi
  const float *mrow;  // this lane's reference of unit 0: sM + l16
  bool lo;            // lane l32 < 16: the first unit of a pair
};

// Workspace block index (KV head, block) of the item's block b.
__device__ __forceinline__ size_t fwd_gblk(const FwdCtx &x, int b) {
  return (size_t)x.i * x.NB + (size_t)(x.wsrow0 / kBlk + b);
}

__device__ __forceinline__ void fwd_load_k(const FwdCtx &x, bf16x8 (&k)[8], int b) {
  load_key_rows(k, x.Kw, fwd_gblk(x, b), x.w);
}

// Half H (dims 64 H .. + 63) of the K rows of block b: k[4 H .. 4 H + 3].
template <int H>
__device__ __forceinline__ void fwd_load_k_half(const FwdCtx &x, bf16x8 (&k)[8], int b) {
  load_key_rows_half<H>(k, x.Kw, fwd_gblk(x, b), x.w);
}

__device__ __forceinline__ void fwd_load_v(const FwdCtx &x, bf16x8 (&v)[2][4], int b) {
#pragma unroll
  for (int md = 0; md < 2; ++md) load_tslice(v[md], x.Vt, fwd_gblk(x, b), 32 * x.w.wave + 16 * md, x.w);
}

// V^T slice md (dims 32 w + 16 md ..) of block b.
template <int MD>
__device__ __forceinline__ void fwd_load_v_half(const FwdCtx &x, bf16x8 (&v)[2][4], int b) {
  load_tslice(v[MD], x.Vt, fwd_gblk(x, b), 32 * x.w.wave + 16 * MD, x.w);
}

// Whether the step's block is the diagonal block of one of the pair's units (uniform;
// dmask = diag_units of the block); decided before the tile's MFMAs so that no branch
// sits between them and the tile's reads.
__device__ __forceinline__ bool fwd_tile_diag(uint32_t dmask, int u0, int u1) {
  return (((dmask >> u0) | (dmask >> u1)) & 1u) != 0;
}

// Causal mask of the tile on a diagonal block.
__device__ __forceinline__ void fwd_tile_mask(const FwdCtx &x, f32x16 &st, int u0, int u1, int b, bool diag) {
  const int qpos = x.p0 + ((x.w.l32 < 16) ? u0 : u1);
  if (diag) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = b * kBlk + 32 * x.w.wave + 8 * (r >> 2) + 4 * x.w.hi + (r & 3);
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

// P = 2^(c s - mn) of the tile, as bf16, to the slots of its units (the step's slot s0 +
// column half, counted on the ring from the step's first slot).  `two`: the second half holds a unit (otherwise its P lands in an unused
// slot); mn: this lane's column reference.  The row sums are taken in the PV phase.
__device__ __forceinline__ void fwd_tile_p(const FwdCtx &x, const f32x16 &st, int s0, float mn) {
  const int half = x.w.l32 >> 4;
  uint32_t pk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    pk[j] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * j], x.c, -mn)),
                        __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * j + 1], x.c, -mn)));
  char *prow = x.sP + ((x.sbase + s0 + half) & (kFwdSlots - 1)) * kSlotStride + slot_store_offset(x.w);
#pragma unroll
  for (int j = 0; j < 4; ++j) *(u32x2 *)(prow + 16 * j) = u32x2{pk[2 * j], pk[2 * j + 1]};
}

// B operand of a pair's tile (load_pair_rows_padded), addressed from the lane's base
// and uniform unit offsets.
__device__ __forceinline__ void fwd_pair_rows(const FwdCtx &x, bf16x8 (&q)[8], int u0, int u1) {
  const int o0 = u0 * (16 * kUnitRow), o1 = u1 * (16 * kUnitRow);
  const char *row = x.qrow + (x.lo ? o0 : o1);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) q[ks] = *(const bf16x8 *)(row + 32 * ks);
}

// This lane's column reference for the pair (u0, u1).
__device__ __forceinline__ float fwd_pair_ref(const FwdCtx &x, int u0, int u1) {
  return x.mrow[x.lo ? 16 * u0 : 16 * u1];
}

// The first pair of unit mask m (u1 = u0 for a lone unit).
__device__ __forceinline__ void fwd_first_pair(uint32_t m, int &u0, int &u1) {
  u0 = __builtin_ctz(m);
  const uint32_t r = m & (m - 1);
  u1 = r ? __builtin_ctz(r) : u0;
}

// S phase of one step (units mr): pairs in unit order at slots 0, 2, 4, ...  q holds the
// first pair's Q rows (read at the end of the previous step).  Once a pair's MFMAs are
// issued (they have read their operands), the same registers are refilled with the
// next pair's Q rows, which then arrive behind the MFMAs and the current pair's
// softmax.  MASKED: the step's block is the diagonal block of some unit; otherwise no
// key needs the causal mask and the pair loop carries no mask code (whose divergent
// select would move every score tile out of the accumulation registers and back).
template <bool MASKED>
__device__ __forceinline__ void fwd_scores(const FwdCtx &x, const bf16x8 (&k)[8], bf16x8 (&q)[8], uint32_t mr,
                                           int b, uint32_t dmask) {
  uint32_t ms = mr;
  int u0 = pop_unit(ms);
  int u1 = ms ? pop_unit(ms) : u0;
  float mn = fwd_pair_ref(x, u0, u1);
  for (int s0 = 0;; s0 += 2) {
    const bool diag = fwd_tile_diag(dmask, u0, u1);
    f32x16 st = tile32(k, q);
    // the next pair (pops kept in scalar registers)
    const uint32_t m0 = (uint32_t)uniform((int)ms);
    const bool more = m0 != 0;
    const int n0 = more ? uniform(__builtin_ctz(m0)) : u0;
    const uint32_t m1 = (uint32_t)uniform((int)(m0 & (m0 - 1)));
    const int n1 = m1 ? uniform(__builtin_ctz(m1)) : n0;
    ms = (uint32_t)uniform((int)(m1 & (m1 - 1)));
    if (more) fwd_pair_rows(x, q, n0, n1);
    const float nmn = fwd_pair_ref(x, n0, n1);
    if (MASKED) fwd_tile_mask(x, st, u0, u1, b, diag);
    fwd_tile_p(x, st, s0, mn);
    if (!more) break;
    u0 = n0;
    u1 = n1;
    mn = nmn;
  }
}

// O^T[dims 32w.., heads] of unit u += V^T P^T with P fragments pf.
__device__ __forceinline__ void fwd_pv_mfma(const bf16x8 (&v)[2][4], const bf16x8 (&pf)[4], f32x4 (&acc)[2]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int md = 0; md < 2; ++md) acc[md] = mfma16(v[md][kk], pf[kk], acc[md]);
}

// Sum of the 32 bf16 P values of a unit's P^T fragments (keys 32 kk + 8 g + 0..7 of the
// lane's head), in fp32: the lane's share of the row sum over this block's keys.
__device__ __forceinline__ float fwd_frag_sum(const bf16x8 (&pf)[4]) {
  float s[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const u32x4 p = __builtin_bit_cast(u32x4, pf[kk]);
    s[kk] = sum_bf16x2(p[3], sum_bf16x2(p[2], sum_bf16x2(p[1], sum_bf16x2(p[0], 0.f))));
  }
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// PV phase of one step: O^T[dims 32w.., heads] += V^T P^T for the nr units of mr,
// whose P slots are their ranks in mr on the ring, and row sums of the same bf16 P
// values the products use: the step's k-th unit is summed by wave k % 4, into ls[u]
// (this lane's keys).  pf holds the first unit's fragments (read by the caller ahead of
// its wait for V); after a unit's MFMAs are issued, the same registers are refilled
// with the next slot's fragments.
__device__ __forceinline__ void fwd_pv(const FwdCtx &x, const bf16x8 (&v)[2][4], uint32_t mr, int nr,
                                       bf16x8 (&pf)[4], f32x4 (&acc)[kFwdGroup][2], float (&ls)[kFwdGroup]) {
  int k = 0;
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if ((mr >> u) & 1u) {
      fwd_pv_mfma(v, pf, acc[u]);
      if ((k & 3) == x.w.wave) ls[u] += fwd_frag_sum(pf);  // the step's k-th unit: wave k % 4
      k = uniform(k + 1);
      load_slot(pf, x.sP, (x.sbase + min(k, nr - 1)) & (kFwdSlots - 1), x.w);
    }
  }
}

// References of the units in `units` (a unit's first block): the maximum over wave
// 0's 32 keys (keys 0..31) of block b, published to all waves through sM.
__device__ __forceinline__ void fwd_references(const FwdCtx &x, const bf16x8 (&k)[8], uint32_t units,
                                               int b) {
  if (x.w.wave == 0) {
    while (units) {
      const int u0 = pop_unit(units);
      const bool two = units != 0;
      const int u1 = two ? pop_unit(units) : u0;
      bf16x8 q[8];
      load_pair_rows_padded(q, x.sQ, u0, u1, x.w);
      const bool diag = fwd_tile_diag(diag_units(x.p0, b), u0, u1);
      f32x16 st = tile32(k, q);
          fwd_tile_mask(x, st, u0, u1, b, diag);
      const float mx = fwd_tile_max(st) * x.c;
      const int u = (x.w.l32 < 16) ? u0 : u1;
      if (x.w.hi == 0 && (x.w.l32 < 16 || two)) x.sM[u * 16 + x.w.l16] = mx;
    }
  }
  lds_barrier();
}

// Exact-reference pass: folds the maximum of block b over all keys into sM for every
// unit in `units`.  The per-wave maxima go through sX; every wave then stores the same
// folded value.
__device__ __forceinline__ void fwd_fold_max(const FwdCtx &x, const bf16x8 (&k)[8], uint32_t units, int b) {
  float *sX = x.sX;
  for (uint32_t us = units; us;) {
    const int u0 = pop_unit(us);
    const bool two = us != 0;
    const int u1 = two ? pop_unit(us) : u0;
    bf16x8 q[8];
    load_pair_rows_padded(q, x.sQ, u0, u1, x.w);
    const bool diag = fwd_tile_diag(diag_units(x.p0, b), u0, u1);
    f32x16 st = tile32(k, q);
      fwd_tile_mask(x, st, u0, u1, b, diag);
    const float mx = fwd_tile_max(st) * x.c;
    const int u = (x.w.l32 < 16) ? u0 : u1;
    if (x.w.hi == 0 && (x.w.l32 < 16 || two)) sX[(x.w.wave * kFwdGroup + u) * 16 + x.w.l16] = mx;
  }
  lds_barrier();
  for (uint32_t us = units; us;) {
    const int u0 = pop_unit(us);
    const bool two = us != 0;
    const int u1 = two ? pop_unit(us) : u0;
    const int u = (x.w.l32 < 16) ? u0 : u1;
    if (x.w.hi == 0 && (x.w.l32 < 16 || two)) {
      float mx = sX[u * 16 + x.w.l16];
#pragma unroll
      for (int w = 1; w < kWalkWaves; ++w) mx = fmaxf(mx, sX[(w * kFwdGroup + u) * 16 + x.w.l16]);
      float *pm = x.sM + u * 16 + x.w.l16;
      *pm = fmaxf(*pm, mx);
    }
  }
}

// The walk's position: list entries a (block b, unit mask m) and a + 1 (block bn; the
// last step's bn is its own block, so that the loads and the wait counts do not depend
// on the position).  The entries are read two steps ahead of their use.
struct FwdPos {
  int b, bn, b2;
  uint32_t m, mn, m2;
};
__device__ __forceinline__ void fwd_pos_init(const FwdCtx &x, FwdPos &q) {
  q.b = uniform(x.list[0]);
  q.m = (uint32_t)uniform(x.list[1]);
  const int a1 = min(1, x.nact - 1);
  q.bn = uniform(x.list[2 * a1]);
  q.mn = (uint32_t)uniform(x.list[2 * a1 + 1]);
}
// Issues the read of entry a + 2 (clamped to the last entry).
__device__ __forceinline__ void fwd_pos_fetch(const FwdCtx &x, FwdPos &q, int a) {
  const int a2 = min(a + 2, x.nact - 1);
  q.b2 = uniform(x.list[2 * a2]);
  q.m2 = (uint32_t)uniform(x.list[2 * a2 + 1]);
}
__device__ __forceinline__ void fwd_pos_advance(FwdPos &q) {
  q.b = q.bn; q.m = q.mn;
  q.bn = q.b2; q.mn = q.m2;
}

// One step of the walk over list entry a (position q) with the K rows and V^T slices of
// its block in kc / vc; the next entry's are loaded into kn / vn.  seen: units whose
// reference is set.  MAXPASS only folds the block maxima into sM.
//
// The P slots form a ring: each step's slots follow the previous step's.  The next
// step's S phase may then start while other waves still read this step's slots in
// their PV phase, unless the two steps' slots (the next step's spare slot of a lone
// unit included) exceed the ring; only then does the step end with a barrier.
template <bool MAXPASS>
__device__ __forceinline__ void fwd_step(FwdCtx &x, int a, FwdPos &q, const bf16x8 (&kc)[8],
                                         const bf16x8 (&vc)[2][4], bf16x8 (&kn)[8], bf16x8 (&vn)[2][4],
                                         bf16x8 (&qf)[8], f32x4 (&acc)[kFwdGroup][2], float (&ls)[kFwdGroup],
                                         uint32_t &seen) {
  const int b = q.b;
  const uint32_t m = q.m;
  const int nu = __popc(m);
  if (MAXPASS) {
    fwd_load_k(x, kn, q.bn);
    fwd_pos_fetch(x, q, a);
    WAIT_VMCNT(8);  // this step's K rows
    fwd_fold_max(x, kc, m, b);
    lds_barrier();  // sX is rewritten by the next step
    fwd_pos_advance(q);
    return;
  }
  // The next block's operands are requested in four groups of four loads spread over
  // the step (the K rows at the start and before the S phase, so that they have a whole
  // step to arrive; the V^T slices before and after the PV phase): issued together right
  // after a barrier, the loads of all waves queue up and stall the waves' instruction
  // streams until they are accepted.
  fwd_load_k_half<0>(x, kn, q.bn);
  fwd_pos_fetch(x, q, a);
  WAIT_VMCNT(12);  // this step's K rows (issued in the previous step)
  const uint32_t dmask = diag_units(x.p0, b);
  const uint32_t fresh = m & ~seen;
  if (fresh) fwd_references(x, kc, fresh, b);
  seen |= m;
  // ---- S phase: the step's units in pairs, this wave's keys (one slot per unit)
  fwd_load_k_half<1>(x, kn, q.bn);
  if (dmask & m)
    fwd_scores<true>(x, kc, qf, m, b, dmask);
  else
    fwd_scores<false>(x, kc, qf, m, b, dmask);
  lds_barrier();
  fwd_load_v_half<0>(x, vn, q.bn);
  bf16x8 pf[4];
  load_slot(pf, x.sP, x.sbase, x.w);
  WAIT_VMCNT(12);  // this step's V^T slices
  // ---- PV phase
  fwd_pv(x, vc, m, nu, pf, acc, ls);
  fwd_load_v_half<1>(x, vn, q.bn);
  {  // the next step's first pair of Q rows
    int n0, n1;
    fwd_first_pair(q.mn, n0, n1);
    fwd_pair_rows(x, qf, n0, n1);
  }
  const int nn = __popc(q.mn);
  if (nu + nn + (nn & 1) > kFwdSlots) lds_barrier();  // the next step's P slots overlap this step's
  x.sbase = (x.sbase + nu) & (kFwdSlots - 1);
  fwd_pos_advance(q);
}

// The whole walk over the item's list.  seen0 = ~0 keeps the references already in
// sM (the exact maxima of the max pass).
template <bool MAXPASS>
__device__ __forceinline__ void fwd_walk(FwdCtx &x, f32x4 (&acc)[kFwdGroup][2], float (&ls)[kFwdGroup],
                                         uint32_t seen0) {
  if (x.nact <= 0) return;
  x.sbase = 0;
  bf16x8 k0[8], k1[8], v0[2][4], v1[2][4], qf[8];
  uint32_t seen = seen0;
  FwdPos q;
  fwd_pos_init(x, q);
  fwd_load_k(x, k0, q.b);
  if (!MAXPASS) {
    fwd_load_v(x, v0, q.b);
    int u0, u1;
    fwd_first_pair(q.m, u0, u1);
    fwd_pair_rows(x, qf, u0, u1);
  }
  for (int a = 0; a < x.nact; a += 2) {
    fwd_step<MAXPASS>(x, a, q, k0, v0, k1, v1, qf, acc, ls, seen);
    if (a + 1 < x.nact) fwd_step<MAXPASS>(x, a + 1, q, k1, v1, k0, v0, qf, acc, ls, seen);
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
  __shared__ __attribute__((aligned(16))) char sQ[kFwdGroup * 16 * kUnitRow];
  __shared__ __attribute__((aligned(16))) char sP[kFwdSlots * kSlotStride];
  __shared__ float sM[kFwdGroup * 16], sX[kWalkWaves * kFwdGroup * 16];
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
  walk_lane(x.w, threadIdx.x);
  x.p0 = t0 - cu[d]; x.wsrow0 = cu_ws[d]; x.NB = NB;
  x.nact = uniform(plan_len[p]);
  x.list = plan_lists + (size_t)2 * kPlanMaxList * p;
  x.c = scale_log2e;
  x.sQ = sQ; x.sP = sP; x.sM = sM; x.sX = sX;
  x.qrow = sQ + x.w.l16 * kUnitRow + 16 * x.w.hi;
  x.mrow = sM + x.w.l16;
  x.lo = x.w.l32 < 16;
  const int tid = x.w.tid;

  // Q rows of the item (16 rows of 256 B per unit) into sQ
  rows_to_lds<kWalkThreads, kFwdGroup * 16, true>(sQ, (const char *)(Q + ((size_t)t0 * kH + kHPI * x.i) * kD),
                                                  (size_t)kH * kD * 2, n * 16, tid);
  for (int k = tid; k < kFwdGroup * 16; k += kWalkThreads) sM[k] = -INFINITY;
  if (tid == 0) sBad = 0;
  __syncthreads();
  f32x4 acc[kFwdGroup][2];
  float ls[kFwdGroup];  // row sums: this lane's keys 8 g .. 8 g + 7 of every 32
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    acc[u][0] = acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    ls[u] = 0.f;
  }
  if (REDO) {
    fwd_walk<true>(x, acc, ls, 0u);  // sM = exact row maxima
    __syncthreads();
  }
  fwd_walk<false>(x, acc, ls, REDO ? ~0u : 0u);
  // row sums: the four 16-lane groups of every wave, then the four waves, add up in a
  // fixed order into sL[unit][head]
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    float l = ls[u] + __shfl_xor(ls[u], 16);
    l += __shfl_xor(l, 32);
    if (x.w.lane < 16) sX[(x.w.wave * kFwdGroup + u) * 16 + x.w.l16] = l;
  }
  __syncthreads();
  float *sL = sX;  // sL[unit][head] = sum over the waves, written over wave 0's part
  float lt = 0.f;
  if (tid < kFwdGroup * 16)
    lt = (sX[tid] + sX[kFwdGroup * 16 + tid]) + (sX[2 * kFwdGroup * 16 + tid] + sX[3 * kFwdGroup * 16 + tid]);
  __syncthreads();
  if (tid < kFwdGroup * 16) sL[tid] = lt;
  __syncthreads();
  // ---- epilogue: acc[u][md][r] = O^T[dim 32w + 16md + 4g + r][head l16]
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if (u < n) {
      const float l = sL[u * 16 + x.w.l16];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t *orow = O + ((size_t)(t0 + u) * kH + kHPI * x.i + x.w.l16) * kD + 32 * x.w.wave + 4 * x.w.g;
#pragma unroll
      for (int md = 0; md < 2; ++md) {
        const f32x4 v = acc[u][md] * inv;
        *(u32x2 *)(orow + 16 * md) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
  if (!REDO) {  // a score 64 (base 2) above its row's reference forces l past 2^64
    for (int k = tid; k < n * 16; k += kWalkThreads)
      if (!(sL[k] < 0x1p64f)) sBad = 1;
    __syncthreads();
  }
  const bool bad = !REDO && sBad != 0;
  for (int k = tid; k < n * 16; k += kWalkThreads) {
    const int u = k >> 4, hh = k & 15;
    const float l = sL[k], mm = sM[k];
    float lse = l > 0.f ? (mm + __log2f(l)) * kLn2 : -INFINITY;
    if (k == 0 && bad) lse = INFINITY;
    LSE[(size_t)(t0 + u) * kH + kHPI * x.i + hh] = lse;
  }
}

namespace host {
hipError_t forward(const void *Q, const void *Kw, const void *Vt, const LayoutArgs &L, const void *plan,
                   float scale, void *O, float *LSE, hipStream_t s) {
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
