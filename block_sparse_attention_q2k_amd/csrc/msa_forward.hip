// msa_forward.hip -- query-parallel MSA prefill forward for gfx950.
//
// What is computed ("feat(minimax-m3): add SM100 MSA sparse attention with custom
// backward", Design): for query token t and query head h of index head i = h / 16,
// softmax over the keys of the blocks listed in q2k[i][t] (document-local, causal),
// O[t,h] = sum_j P_j V_j and LSE[t,h] = log sum_j exp(scale <Q[t,h], K_j>).
//
// Design (gfx950): one workgroup of 8 waves (two per SIMD) per plan item = (index head
// i, up to MSA_FWD_GROUP consecutive queries of one document); a unit is one query with
// its 16 heads (16 rows that share a selection).  The item's Q rows stay in LDS for the
// whole item, and the workgroup walks the item's list of selected blocks, so each K / V
// block is read once per item, not once per query.  The waves have two roles, one wave
// of each role on every SIMD:
//   score waves (0-3) -- wave w owns keys [32w, 32w + 32) of every block, whose K rows
//               it holds in registers; for every pair of the step's units it computes
//               the 32 x 32 tile S^T = K [Q_u0 | Q_u1]^T (32x32x16 MFMAs, Q from LDS),
//               turns it into P (bf16) and stores P to the units' LDS slots;
//   PV waves (4-7) -- wave 4 + w owns head dims [32w, 32w + 32) and updates
//               O^T += V^T P^T for every unit of the step (16x16x32 MFMAs); its V^T rows
//               come straight from the transposed workspace copy into registers, P^T
//               from LDS.  The row sums of the same bf16 P values are taken here too
//               (one wave per unit).
// The roles run one step apart: while the score waves compute the P of step n, the PV
// waves multiply step n - 1's.  Within one wave, matrix products and the softmax's
// vector arithmetic add up in time; across the two waves of a SIMD the score wave's
// vector instructions issue while the PV wave's products occupy the matrix unit.  One
// barrier per step hands the step's slots to the PV waves.  The P slots form a ring
// that holds two consecutive steps: a list entry of more than kFwdSubMax units is
// walked as two steps over the same block (its first half of the units, then the rest).
// With the launch's two waves per SIMD every wave has at most 256 registers, and the
// compiler then keeps the MFMA accumulators (score tiles, O) in ordinary vector
// registers: the softmax reads its scores without accumulator-register copies.
//
// Softmax reference: each row's exponent reference m is the (base-2, scaled) maximum
// of its first block and never moves, so the accumulators are never rescaled and the
// later blocks need no maximum: P = 2^(c s - m), an elementwise step that lets every
// wave work on its own keys.  The reference is taken from score wave 0's 32 keys of the
// unit's first block (they always include an unmasked key): any score of the row would
// do, as long as no later score exceeds it by 64 (base 2); then P, l and O stay far
// inside fp32 / bf16 range.  A row whose sum l reaches 2^64 (which any such score
// forces) marks its item (LSE of the item's first row, first head = +inf), and a
// second launch of the kernel redoes exactly those items with the exact row maxima,
// found by a first walk over the blocks, as references.
#include "msa_walk.h"

namespace msa {

constexpr int kFwdThreads = 512;  // 4 score waves + 4 PV waves
constexpr int kFwdRing = 20;      // P slots (one per unit of a step), used as a ring
constexpr int kFwdSubMax = 10;    // units per step
static_assert(kFwdGroup <= 32, "unit masks are 32-bit");
static_assert(2 * kFwdSubMax <= kFwdRing, "two consecutive steps fit in the ring");
static_assert(kFwdGroup <= 2 * kFwdSubMax, "an entry is split into at most two steps");

// Position s (< 2 kFwdRing) on the ring.
__device__ __forceinline__ int ring_slot(int s) { return s >= kFwdRing ? s - kFwdRing : s; }

struct FwdCtx {
  WalkLane w;  // coordinates within the wave's role (wave 0..3)
  const uint16_t *Kw, *Vt;
  const int32_t *list;
  int nact, i, p0, wsrow0, NB;
  float c;  // scale * log2(e)
  const char *sQ;
  char *sP;
  int sbase;  // ring position of the step's first P slot (score waves)
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

// Causal mask of a tile of key slice kw (keys 32 kw .. of the block) on a diagonal block.
__device__ __forceinline__ void fwd_tile_mask(const FwdCtx &x, f32x16 &st, int u0, int u1, int b, bool diag,
                                              int kw) {
  const int qpos = x.p0 + ((x.w.l32 < 16) ? u0 : u1);
  if (diag) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = b * kBlk + 32 * kw + 8 * (r >> 2) + 4 * x.w.hi + (r & 3);
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
// column half, counted on the ring from the step's first slot); mn: this lane's column
// reference.  `two`: the second column half holds a unit (otherwise those lanes store
// nothing).  The row sums are taken by the PV waves.
__device__ __forceinline__ void fwd_tile_p(const FwdCtx &x, const f32x16 &st, int s0, float mn, bool two) {
  const int half = x.w.l32 >> 4;
  uint32_t pk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    pk[j] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * j], x.c, -mn)),
                        __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * j + 1], x.c, -mn)));
  char *prow = x.sP + ring_slot(x.sbase + s0 + half) * kSlotStride + slot_store_offset(x.w);
  if (x.lo || two) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x2 *)(prow + 16 * j) = u32x2{pk[2 * j], pk[2 * j + 1]};
  }
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

// Score-wave part of one step (units mr): pairs in unit order at slots 0, 2, 4, ...  q
// holds the first pair's Q rows (read at the end of the previous step).  Once a pair's
// MFMAs are issued (they have read their operands), the same registers are refilled
// with the next pair's Q rows, which then arrive behind the MFMAs and the current
// pair's softmax.  MASKED: the step's block is the diagonal block of some unit;
// otherwise no key needs the causal mask and the pair loop carries no mask code.
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
    if (MASKED) fwd_tile_mask(x, st, u0, u1, b, diag, x.w.wave);
    fwd_tile_p(x, st, s0, mn, u1 != u0);
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

// PV-wave part of one step: O^T[dims 32w.., heads] += V^T P^T for the nr units of mr,
// whose P slots are their ranks in mr on the ring from `base`, and row sums of the same
// bf16 P values the products use: the step's k-th unit is summed by PV wave k % 4, into
// ls[u] (this lane's keys).  pf holds the first unit's fragments (read by the caller
// ahead of its wait for V); after a unit's MFMAs are issued, the same registers are
// refilled with the next slot's fragments.
__device__ __forceinline__ void fwd_pv(const FwdCtx &x, const bf16x8 (&v)[2][4], uint32_t mr, int nr, int base,
                                       bf16x8 (&pf)[4], f32x4 (&acc)[kFwdGroup][2], float (&ls)[kFwdGroup]) {
  int k = 0;
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    if ((mr >> u) & 1u) {
      fwd_pv_mfma(v, pf, acc[u]);
      if ((k & 3) == x.w.wave) ls[u] += fwd_frag_sum(pf);  // the step's k-th unit: wave k % 4
      k = uniform(k + 1);
      load_slot(pf, x.sP, ring_slot(base + min(k, nr - 1)), x.w);
    }
  }
}

// Key slice 0 (keys 0..31) of block b as tile operands, in every score wave.
__device__ __forceinline__ void fwd_load_slice0(const FwdCtx &x, bf16x8 (&k)[8], int b) {
  WalkLane w0 = x.w;
  w0.wave = 0;
  load_key_rows(k, x.Kw, fwd_gblk(x, b), w0);
}

// References of the units in `units` (a unit's first block): the maximum over key
// slice 0 (keys 0..31) of block b, whose rows k0 every score wave holds; the unit pairs
// are shared out over the score waves, and the maxima reach all of them through sM
// (the barrier is taken by every wave of the workgroup).
__device__ __forceinline__ void fwd_references(const FwdCtx &x, const bf16x8 (&k0)[8], uint32_t units, int b) {
  int p = 0;
  for (uint32_t us = units; us; ++p) {
    const int u0 = pop_unit(us);
    const bool two = us != 0;
    const int u1 = two ? pop_unit(us) : u0;
    if ((p & (kWalkWaves - 1)) != x.w.wave) continue;
    bf16x8 q[8];
    load_pair_rows_padded(q, x.sQ, u0, u1, x.w);
    const bool diag = fwd_tile_diag(diag_units(x.p0, b), u0, u1);
    f32x16 st = tile32(k0, q);
    fwd_tile_mask(x, st, u0, u1, b, diag, 0);
    const float mx = fwd_tile_max(st) * x.c;
    const int u = (x.w.l32 < 16) ? u0 : u1;
    if (x.w.hi == 0 && (x.w.l32 < 16 || two)) x.sM[u * 16 + x.w.l16] = mx;
  }
  lds_barrier();
}

// Exact-reference pass (score waves): folds the maximum of block b over all keys into
// sM for every unit in `units`.  The per-wave maxima go through sX; every wave then
// stores the same folded value.  Takes one barrier.
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
    fwd_tile_mask(x, st, u0, u1, b, diag, x.w.wave);
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

// The low k set bits of m.
__device__ __forceinline__ uint32_t low_units(uint32_t m, int k) {
  uint32_t rest = m;
  for (int j = 0; j < k; ++j) rest &= rest - 1;
  return m ^ rest;
}

// The walk's position at step n: the unit masks of steps n - 1 (mp), n (m) and n + 1
// (mn) and the blocks of steps n and n + 1; a mask of 0 marks a step past the end,
// whose block is the last entry's (so that the loads do not depend on the position).
// Steps come from the list entries in order, an entry of more than kFwdSubMax units
// as two steps; the entry after the one being split is read ahead.
struct FwdPos {
  int b, bn;
  uint32_t mp, m, mn;
  int be;       // block of the entry the next step comes from
  uint32_t re;  // its units not yet issued as a step
  int af;       // list index of the entry read ahead (bf, mf; mf counts only if fv)
  int bf;
  uint32_t mf;
  bool fv;
};
// Issues the read of entry af (clamped to the last entry) and moves af on.
__device__ __forceinline__ void fwd_pos_fetch(const FwdCtx &x, FwdPos &q) {
  const int a = min(q.af, x.nact - 1);
  q.bf = uniform(x.list[2 * a]);
  q.mf = (uint32_t)uniform(x.list[2 * a + 1]);
  q.fv = q.af < x.nact;
  q.af += 1;
}
// The next step's block and units.
__device__ __forceinline__ void fwd_pos_next(const FwdCtx &x, FwdPos &q, int &b, uint32_t &m) {
  if (q.re == 0) {
    q.be = q.bf;
    q.re = q.fv ? q.mf : 0u;
    fwd_pos_fetch(x, q);
  }
  const int nu = __popc(q.re);
  const uint32_t take = nu > kFwdSubMax ? low_units(q.re, (nu + 1) >> 1) : q.re;
  q.re ^= take;
  b = q.be;
  m = take;
}
__device__ __forceinline__ void fwd_pos_init(const FwdCtx &x, FwdPos &q) {
  q.mp = 0u;
  q.re = 0u;
  q.af = 0;
  fwd_pos_fetch(x, q);
  fwd_pos_next(x, q, q.b, q.m);
  fwd_pos_next(x, q, q.bn, q.mn);
}
__device__ __forceinline__ void fwd_pos_advance(const FwdCtx &x, FwdPos &q) {
  q.mp = q.m;
  q.b = q.bn;
  q.m = q.mn;
  fwd_pos_next(x, q, q.bn, q.mn);
}

// Score waves, one step of the walk (position q) with the K rows of its block in kc;
// the next step's are loaded into kn.  seen: units whose reference is set.  Barriers,
// in order: the references (if the step holds a unit's first block), the step's
// hand-over.
__device__ __forceinline__ void fwd_score_step(FwdCtx &x, FwdPos &q, const bf16x8 (&kc)[8], bf16x8 (&kn)[8],
                                               bf16x8 (&qf)[8], uint32_t &seen, bool first,
                                               const bf16x8 (&ks0)[8]) {
  const int b = q.b;
  const uint32_t m = q.m;
  // The next block's K rows in two groups of four loads, the first at the start of
  // the step and the second after its waits, so that they have a whole step to arrive.
  fwd_load_k_half<0>(x, kn, q.bn);
  WAIT_VMCNT(4);  // this step's K rows (issued in the previous step)
  const uint32_t fresh = m & ~seen;
  if (fresh) {
    if (first) {
      fwd_references(x, ks0, fresh, b);  // key slice 0 of the first block, loaded with its K rows
    } else {
      bf16x8 k0[8];
      fwd_load_slice0(x, k0, b);
      WAIT_VMCNT(0);
      fwd_references(x, k0, fresh, b);
    }
  }
  seen |= m;
  fwd_load_k_half<1>(x, kn, q.bn);
  const uint32_t dmask = diag_units(x.p0, b);
  if (dmask & m)
    fwd_scores<true>(x, kc, qf, m, b, dmask);
  else
    fwd_scores<false>(x, kc, qf, m, b, dmask);
  {  // the next step's first pair of Q rows (unit 0's past the end)
    int n0, n1;
    fwd_first_pair(q.mn ? q.mn : 1u, n0, n1);
    fwd_pair_rows(x, qf, n0, n1);
  }
  lds_barrier();  // hand-over: the step's P to the PV waves
  x.sbase = ring_slot(x.sbase + __popc(m));
  fwd_pos_advance(x, q);
}

// PV waves, step n of the walk: multiplies step n - 1 (V^T slices in vc, slots from
// bprev) while the score waves compute step n, and loads step n's V^T into vn.  Takes
// the same barriers as fwd_score_step; runs one step past the last (its products).
__device__ __forceinline__ void fwd_pv_step(FwdCtx &x, FwdPos &q, const bf16x8 (&vc)[2][4], bf16x8 (&vn)[2][4],
                                            f32x4 (&acc)[kFwdGroup][2], float (&ls)[kFwdGroup], uint32_t &seen,
                                            int &bcur, int &bprev) {
  const bool has = q.mp != 0u, cur = q.m != 0u;
  fwd_load_v_half<0>(x, vn, q.b);
  bf16x8 pf[4];
  if (has) load_slot(pf, x.sP, bprev, x.w);
  WAIT_VMCNT(4);  // step n - 1's V^T slices (issued in the previous step)
  if (cur && (q.m & ~seen)) lds_barrier();  // the score waves' references
  seen |= q.m;
  fwd_load_v_half<1>(x, vn, q.b);
  if (has) fwd_pv(x, vc, q.mp, __popc(q.mp), bprev, pf, acc, ls);
  lds_barrier();  // hand-over: step n - 1's slots released, step n's P published
  bprev = bcur;
  bcur = ring_slot(bcur + __popc(q.m));
  fwd_pos_advance(x, q);
}

// The score waves' walk over the item's list (at least one entry).  seen0 = ~0 keeps
// the references already in sM (the exact maxima of the max pass).
__device__ __forceinline__ void fwd_score_walk(FwdCtx &x, uint32_t seen0) {
  x.sbase = 0;
  bf16x8 k0[8], k1[8], qf[8];
  uint32_t seen = seen0;
  FwdPos q;
  fwd_pos_init(x, q);
  fwd_load_k(x, k0, q.b);
  bf16x8 ks0[8];  // key slice 0 of the first block: its units' references
  fwd_load_slice0(x, ks0, q.b);
  {
    int u0, u1;
    fwd_first_pair(q.m, u0, u1);
    fwd_pair_rows(x, qf, u0, u1);
  }
  bool first = true;
  for (;;) {
    fwd_score_step(x, q, k0, k1, qf, seen, first, ks0);
    first = false;
    if (q.m == 0u) break;
    fwd_score_step(x, q, k1, k0, qf, seen, false, ks0);
    if (q.m == 0u) break;
  }
  lds_barrier();  // the PV waves' last step
}

// The PV waves' walk: one step more than the score waves' (the first only loads V^T).
__device__ __forceinline__ void fwd_pv_walk(FwdCtx &x, f32x4 (&acc)[kFwdGroup][2], float (&ls)[kFwdGroup],
                                            uint32_t seen0) {
  bf16x8 v0[2][4], v1[2][4];
  uint32_t seen = seen0;
  int bcur = 0, bprev = 0;
  FwdPos q;
  fwd_pos_init(x, q);
  for (;;) {
    fwd_pv_step(x, q, v1, v0, acc, ls, seen, bcur, bprev);
    if (q.mp == 0u) break;
    fwd_pv_step(x, q, v0, v1, acc, ls, seen, bcur, bprev);
    if (q.mp == 0u) break;
  }
}

// Exact-reference pass over the same steps: the score waves fold every block's maxima
// into sM (two barriers per step), the PV waves take the same barriers.
__device__ __forceinline__ void fwd_max_walk(FwdCtx &x, bool score) {
  FwdPos q;
  fwd_pos_init(x, q);
  if (!score) {
    while (q.m != 0u) {
      lds_barrier();
      lds_barrier();
      fwd_pos_advance(x, q);
    }
    return;
  }
  bf16x8 k0[8], k1[8];
  fwd_load_k(x, k0, q.b);
  for (;;) {
    fwd_load_k(x, k1, q.bn);
    WAIT_VMCNT(8);  // this step's K rows
    fwd_fold_max(x, k0, q.m, q.b);
    lds_barrier();  // sX is rewritten by the next step
    fwd_pos_advance(x, q);
    if (q.m == 0u) break;
    fwd_load_k(x, k0, q.bn);
    WAIT_VMCNT(8);
    fwd_fold_max(x, k1, q.m, q.b);
    lds_barrier();
    fwd_pos_advance(x, q);
    if (q.m == 0u) break;
  }
}

// The PV waves' part of the item: the walk, their partial row sums (the four 16-lane
// groups of every wave added in a fixed order) into sX[wave][unit][head], and, once the
// score waves have added those into sL, O.  Takes the barriers of the score waves' part.
template <bool REDO>
__device__ __forceinline__ void fwd_pv_role(FwdCtx &x, int t0, int n, const float *sL, uint16_t *__restrict__ O) {
  f32x4 acc[kFwdGroup][2];
  float ls[kFwdGroup];  // row sums: this lane's keys 8 g .. 8 g + 7 of every 32
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    acc[u][0] = acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    ls[u] = 0.f;
  }
  if (x.nact > 0) {
    if (REDO) {
      fwd_max_walk(x, false);
      __syncthreads();
    }
    fwd_pv_walk(x, acc, ls, REDO ? ~0u : 0u);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kFwdGroup; ++u) {
    float l = ls[u] + __shfl_xor(ls[u], 16);
    l += __shfl_xor(l, 32);
    if (x.w.lane < 16) x.sX[(x.w.wave * kFwdGroup + u) * 16 + x.w.l16] = l;
  }
  __syncthreads();
  __syncthreads();  // sL complete
  // acc[u][md][r] = O^T[dim 32w + 16md + 4g + r][head l16]
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
}

// REDO = false: every item, references from each row's first block.  REDO = true:
// only the items the first launch marked, with exact references from a max pass.
template <bool REDO>
__global__ void __launch_bounds__(kFwdThreads, 1)
fwd_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kw,
           const uint16_t *__restrict__ Vt, const int32_t *__restrict__ cu,
           const int32_t *__restrict__ cu_ws, int NB, const int32_t *__restrict__ plan,
           const int32_t *__restrict__ plan_len, const int32_t *__restrict__ plan_lists,
           float scale_log2e, uint16_t *__restrict__ O, float *__restrict__ LSE) {
  __shared__ __attribute__((aligned(16))) char sQ[kFwdGroup * 16 * kUnitRow];
  __shared__ __attribute__((aligned(16))) char sP[kFwdRing * kSlotStride];
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
  const int tid = threadIdx.x;
  const bool score = uniform(tid >> 8) == 0;  // waves 0-3: score waves, 4-7: PV waves
  walk_lane(x.w, tid & 255);
  x.p0 = t0 - cu[d]; x.wsrow0 = cu_ws[d]; x.NB = NB;
  x.nact = uniform(plan_len[p]);
  x.list = plan_lists + (size_t)2 * kPlanMaxList * p;
  x.c = scale_log2e;
  x.sQ = sQ; x.sP = sP; x.sM = sM; x.sX = sX;
  x.qrow = sQ + x.w.l16 * kUnitRow + 16 * x.w.hi;
  x.mrow = sM + x.w.l16;
  x.lo = x.w.l32 < 16;

  // Q rows of the item (16 rows of 256 B per unit) into sQ
  rows_to_lds<kFwdThreads, kFwdGroup * 16, true>(sQ, (const char *)(Q + ((size_t)t0 * kH + kHPI * x.i) * kD),
                                                 (size_t)kH * kD * 2, n * 16, tid);
  for (int k = tid; k < kFwdGroup * 16; k += kFwdThreads) sM[k] = -INFINITY;
  if (tid == 0) sBad = 0;
  __syncthreads();
  float *sL = sX;  // row sums sL[unit][head], written over PV wave 0's part of sX
  if (score) {
    if (x.nact > 0) {
      if (REDO) {
        fwd_max_walk(x, true);  // sM = exact row maxima
        __syncthreads();
      }
      fwd_score_walk(x, REDO ? ~0u : 0u);
    }
    __syncthreads();  // the PV waves' partial row sums
    __syncthreads();
    if (tid < kFwdGroup * 16)  // the four PV waves' parts, added in a fixed order
      sL[tid] = (sX[tid] + sX[kFwdGroup * 16 + tid]) + (sX[2 * kFwdGroup * 16 + tid] + sX[3 * kFwdGroup * 16 + tid]);
    __syncthreads();
  } else {
    fwd_pv_role<REDO>(x, t0, n, sL, O);
  }
  if (!REDO) {  // a score 64 (base 2) above its row's reference forces l past 2^64
    for (int k = tid; k < n * 16; k += kFwdThreads)
      if (!(sL[k] < 0x1p64f)) sBad = 1;
    __syncthreads();
  }
  const bool bad = !REDO && sBad != 0;
  for (int k = tid; k < n * 16; k += kFwdThreads) {
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
  hipLaunchKernelGGL(fwd_kernel<false>, dim3(items), dim3(kFwdThreads), 0, s, (const uint16_t *)Q,
                     (const uint16_t *)Kw, (const uint16_t *)Vt, L.cu, L.cu_ws, L.NB, v.header,
                     v.len, v.lists, scale * kLog2e, (uint16_t *)O, LSE);
  hipLaunchKernelGGL(fwd_kernel<true>, dim3(items), dim3(kFwdThreads), 0, s, (const uint16_t *)Q,
                     (const uint16_t *)Kw, (const uint16_t *)Vt, L.cu, L.cu_ws, L.NB, v.header,
                     v.len, v.lists, scale * kLog2e, (uint16_t *)O, LSE);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
