// msa_backward_kv2.hip -- KV-parallel dK/dV of the MSA prefill backward with stored dS
// tiles (MSA_DQ_STORED), gfx950: score waves and accumulate waves.
//
// What is computed (msa_backward_sm100 API page, module summary; the backward of the
// operator in "feat(minimax-m3): add SM100 MSA sparse attention with custom backward"):
// for every task row (8 queries x 16 heads that selected one key block of one index
// head) and the block's 128 keys: S = Q K^T, P = exp(scale S - LSE) under the causal
// mask, dP = dO V^T, dS = P (dP - delta), dV += P^T dO, dK += scale dS^T Q.  dK / dV
// accumulate in registers over the consecutive rows of one bucket and are flushed with
// fp32 atomics at the end of the bucket segment; every dS value is stored as a bf16
// tile for the query-parallel dQ kernel (msa_backward_dqs.hip).
//
// Design (gfx950): persistent grid of 8-wave workgroups, two waves per SIMD.  A
// workgroup's task rows (over the four index heads) form a sequence of quarters
// (2 queries x 16 heads = 32 rows), one per phase.  Waves w and 4 + w share a SIMD (the
// hardware puts them on one); score wave w owns keys [32w, 32w + 32) of the bucket's
// block, accumulate wave 4 + w dims [32w, 32w + 32):
//   score wave w: in phase n, S and dP of quarter n (32x32x16 MFMAs, M = the quarter's
//     rows from LDS, N = the wave's keys, K / V rows in registers), the softmax (P and
//     dS), the dS tile stores, and P / dS (bf16, as the accumulate wave's A operands)
//     to an LDS exchange slot;
//   accumulate wave 4 + w: in phase n, dV += P^T dO and dK += dS^T Q of quarter n - 1
//     for all 128 keys and dims [32w, 32w + 32) (P / dS of the four score waves from
//     their exchange slots, dO / Q through transposing LDS reads, each read once per
//     k-step for all four key tiles), dK / dV in registers.
// Within one wave, matrix products and vector arithmetic add up in time; across the two
// waves of a SIMD the score wave's softmax issues while the accumulate wave's products
// occupy the matrix unit.  One barrier per phase.  The Q / dO rows of each quarter are
// gathered by the accumulate waves (its LSE and delta by the first of them), kKv2Ahead
// quarters ahead, into a ring of kKv2Slots LDS slots, with asynchronous global-to-LDS
// copies that no register holds; each task row's ids are copied two rows ahead, by the
// second accumulate wave, and completed into a ring of descriptors.  With two waves per
// SIMD the compiler keeps every accumulator in ordinary VGPRs.
#include "msa_walk.h"  // uniform()

namespace msa {

constexpr int kKv2Threads = 512;
constexpr int kKv2Slots = 6;                 // quarter slots (ring)
constexpr int kKv2Ahead = 4;                 // quarters gathered ahead of the score waves
constexpr int kKv2Half = 8192;               // Q rows of a quarter: 32 x 256 B; dO follows
constexpr int kKv2SlotBytes = 2 * kKv2Half + 256;  // + LSE (log2) and delta of the 32 rows
constexpr int kKv2XBytes = 4096;             // P, dS of one wave's keys for one quarter
constexpr int kKv2Desc = 32;                 // words per task-row descriptor
// The copies of quarter n + kKv2Ahead, issued in phase n, go to the slot of quarter n +
// kKv2Ahead - kKv2Slots, which the accumulate waves last read in phase n + kKv2Ahead -
// kKv2Slots + 1 (before phase n); they must land before the score waves read the
// quarter's A operands in phase n + kKv2Ahead - 1.
static_assert(kKv2Ahead - kKv2Slots + 1 < 0 && kKv2Ahead >= 3, "gather ring");

// Descriptor words: 0 index head, 1 bucket, 2 valid queries, 3 the bucket of the
// workgroup's next row (-1 past the last), 4..11 query ids, 12..19 positions, 20..27
// dS tile indices.  Padding queries (past word 2) are stored with query 0's id,
// position -1 (no key visible) and the spare dS tile.
constexpr int kDescI = 0, kDescBucket = 1, kDescNv = 2, kDescNext = 3, kDescT = 4, kDescPos = 12, kDescTile = 20;

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_2;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4_2;

// Swizzle of a quarter's Q / dO rows ([32 rows][256 B]): 16-byte chunk c of row r at
// chunk c ^ f(r), f(r) = ((r & 3) << 2) | ((r >> 2) & 3) (a bijection on r % 16): 16 lanes
// reading one chunk of 16 consecutive rows hit 16 chunks, and the transposing reads of
// 4 rows x 4 chunks per 16-lane group hit 16 chunks per 32 lanes.
__device__ __forceinline__ int kv2_f(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ uint32_t kv2_swz(int row, int byte_in_row) {
  return (uint32_t)(row * 256 + ((((byte_in_row >> 4) ^ kv2_f(row)) << 4) | (byte_in_row & 15)));
}

__device__ __forceinline__ void kv2_atomic_add(float *p, float v) {
  __builtin_amdgcn_global_atomic_fadd_f32((__attribute__((address_space(1))) float *)p, v);
}

// The workgroup's task rows: per index head i, rows [lo_i, lo_i + n_i) (uniform; named
// fields, not arrays, so that a run-time head index never sends them to scratch memory).
struct Kv2Rows {
  int lo0, lo1, lo2, lo3, n0, n1, n2, n3;
  int total;
};
// Index head and task row of the workgroup's g-th row (g < total).
__device__ __forceinline__ void kv2_row(const Kv2Rows &R, int g, int &i, int &row) {
  static_assert(kHI == 4, "four index heads");
  if (g < R.n0) {
    i = 0;
    row = R.lo0 + g;
  } else if ((g -= R.n0) < R.n1) {
    i = 1;
    row = R.lo1 + g;
  } else if ((g -= R.n1) < R.n2) {
    i = 2;
    row = R.lo2 + g;
  } else {
    i = 3;
    row = R.lo3 + g - R.n2;
  }
}

// Descriptor word `lane` (< 32; lanes 32-63 repeat lanes 24-31's sources) of the
// workgroup's row g (clamped to its last row): the address it is loaded from
// (kv2_desc_src; words 0 and 3 not yet final) and the completed word (kv2_desc_fix), so
// that a wave can copy the words ahead and complete them where it uses them.
__device__ __forceinline__ const int32_t *kv2_desc_src(const Kv2Rows &R, int g, const i32x4 *__restrict__ meta,
                                                       const int32_t *__restrict__ qrows,
                                                       const int32_t *__restrict__ qpos,
                                                       const int32_t *__restrict__ qtile, int lane) {
  g = min(g, R.total - 1);
  int i, row;
  kv2_row(R, g, i, row);
  int gn = min(g + 1, R.total - 1), in, rown;
  kv2_row(R, gn, in, rown);
  const int32_t *src = lane < kDescT ? (const int32_t *)(meta + (lane == kDescNext ? rown : row)) + (lane == kDescNv)
                       : lane < kDescPos  ? qrows + (size_t)row * kTileQ + (lane - kDescT)
                       : lane < kDescTile ? qpos + (size_t)row * kTileQ + (lane - kDescPos)
                       : qtile + (size_t)row * kTileQ + ((lane - kDescTile) & 7);
  return src;
}
__device__ __forceinline__ int kv2_desc_fix(int v, const Kv2Rows &R, int g, int lane) {
  g = min(g, R.total - 1);
  int i, row;
  kv2_row(R, g, i, row);
  return lane == kDescI ? i : lane == kDescNext ? (g + 1 < R.total ? v : -1) : v;
}
__device__ __forceinline__ int kv2_desc_load(const Kv2Rows &R, int g, const i32x4 *__restrict__ meta,
                                             const int32_t *__restrict__ qrows, const int32_t *__restrict__ qpos,
                                             const int32_t *__restrict__ qtile, int lane) {
  return kv2_desc_fix(*kv2_desc_src(R, g, meta, qrows, qpos, qtile, lane), R, g, lane);
}

// The padding rule applied to descriptor word v of lane `lane` (every lane of the wave
// holds its word): padding queries take query 0's id, position -1 and the spare tile.
__device__ __forceinline__ int kv2_desc_pad(int v, int lane, int ds_spare) {
  const int nv = __builtin_amdgcn_readlane(v, kDescNv);
  const int t0 = __builtin_amdgcn_readlane(v, kDescT);
  const int k = (lane - kDescT) & 7;
  if (lane >= kDescT && lane < kDescT + 24 && k >= nv)
    v = lane < kDescPos ? t0 : lane < kDescTile ? -1 : ds_spare;
  return v;
}

// Gather of one quarter into its LDS slot by the 256 threads of the accumulate waves
// (at = thread index among them), as asynchronous global-to-LDS copies of 16 bytes per
// lane (lane l of a wave lands at the wave's destination + 16 l): chunks at and at + 256
// of the quarter's Q rows and of its dO rows (chunk ci: row rq = ci / 16 of the quarter,
// query 2 q + rq / 16, head rq % 16; physical chunk ci % 16, which holds logical chunk
// (ci % 16) ^ f(rq)) and, in the first accumulate wave (LEAD), 4 rows of LSE (lanes 0-7)
// or delta (lanes 8-15) (rows 4 m .. 4 m + 3, m = at % 8: query m / 4, heads 4 (m % 4)
// ..).  LSE lands in natural log; kv2_lse_log2 rescales it.  The copies count in the
// issuing wave's vector-memory counter, which the wave waits on before the barrier that
// publishes the slot.
typedef __attribute__((address_space(1))) void kv2_gvoid;
typedef __attribute__((address_space(3))) void kv2_lvoid;
__device__ __forceinline__ void kv2_copy16(const void *src, char *dst) {
  __builtin_amdgcn_global_load_lds((const kv2_gvoid *)src, (kv2_lvoid *)dst, 16, 0, 0);
}
template <bool LEAD>
__device__ __forceinline__ void kv2_gather(char *slot, int i, int t0, int t1, const uint16_t *__restrict__ Q,
                                           const uint16_t *__restrict__ dO, const float *__restrict__ LSE,
                                           const float *__restrict__ Delta, int at) {
  // chunks at and at + 256 share the head (rq % 16) and the chunk, so one lane offset
  // serves both; the row base is wave-uniform
  const int hh = (at >> 4) & 15;
  const unsigned off = (unsigned)(hh * kD + (((at & 15) ^ kv2_f(hh)) << 3)) * 2u;  // bytes
  char *dst = slot + uniform(at & ~63) * 16;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = j ? t1 : t0;  // rows 0..15: query 2 q, 16..31: query 2 q + 1
    const size_t base = ((size_t)t * kH + kHPI * i) * kD;
    kv2_copy16((const char *)(Q + base) + off, dst + 256 * 16 * j);
    kv2_copy16((const char *)(dO + base) + off, dst + kKv2Half + 256 * 16 * j);
  }
  if constexpr (LEAD) {
    if (at < 16) {
      const int m = at & 7;
      const int ts = (m >> 2) ? t1 : t0;
      const float *sb = (at & 8) ? Delta : LSE;
      kv2_copy16(sb + (size_t)ts * kH + kHPI * i + 4 * (m & 3), slot + 2 * kKv2Half);
    }
  }
}

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t kv2_lds_addr(const char *p) { return (uint32_t)(size_t)(const lds_char *)p; }

// LSE of the quarter in slot sl from natural log to log2 (lanes 0-7 of the first
// accumulate wave; its own copies, already waited for).  The compiler orders every LDS
// access of the slot array behind all copies in flight; written as assembly (the read
// waits within its statement), these accesses do not wait for the quarters gathered
// ahead.
__device__ __forceinline__ void kv2_lse_log2(char *sl, int lane) {
  if (lane < 8) {
    const uint32_t a = kv2_lds_addr(sl + 2 * kKv2Half) + 16 * lane;
    f32x4 v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    v = v * kLog2e;
    asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
  }
}

// A task row's descriptor in scalar registers: one LDS read per lane (word lane % 32)
// and constant-lane reads.
struct Kv2Ids {
  int i, bucket, next, t[kTileQ], pos[kTileQ], tix[kTileQ];
};
__device__ __forceinline__ void kv2_ids(Kv2Ids &d, const int *D, int lane) {
  const int v = D[lane & 31];
  d.i = __builtin_amdgcn_readlane(v, kDescI);
  d.bucket = __builtin_amdgcn_readlane(v, kDescBucket);
  d.next = __builtin_amdgcn_readlane(v, kDescNext);
#pragma unroll
  for (int k = 0; k < kTileQ; ++k) {
    d.t[k] = __builtin_amdgcn_readlane(v, kDescT + k);
    d.pos[k] = __builtin_amdgcn_readlane(v, kDescPos + k);
    d.tix[k] = __builtin_amdgcn_readlane(v, kDescTile + k);
  }
}

// Workgroup barrier that waits for this wave's LDS accesses only (not for its global
// stores in flight).
__device__ __forceinline__ void kv2_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- score waves
struct Kv2Score {
  bf16x8 kf[8], vf[8];  // this wave's 32 keys: K / V rows as B operands
  bf16x8 qa[8], oa[8];  // the next quarter's Q / dO rows as A operands (read a phase ahead)
  int bucket;           // bucket of kf / vf (-1: none)
  int kbase;            // document-local position of the block's first key
};

// A operands (Q / dO rows: row l32 of the quarter, dims 16 ks + 8 h ..) of the quarter
// in slot sl.
__device__ __forceinline__ void kv2_score_ops(Kv2Score &s, const char *sl, int lane) {
  const lds_char *lq = (const lds_char *)sl;
  const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const uint32_t off = kv2_swz(l32, (16 * ks + 8 * h) * 2);
    s.qa[ks] = *(const lds_bf16x8_2 *)(lq + off);
    s.oa[ks] = *(const lds_bf16x8_2 *)(lq + kKv2Half + off);
  }
}

// S, dP, softmax, dS tile stores and the exchange of quarter qtr of the row described
// by D, whose rows are in slot sl and whose A operands s holds; then the A operands of
// the next quarter (slot sl_next) are read while the softmax runs.
__device__ __forceinline__ void kv2_score(Kv2Score &s, const Kv2Ids &D, int qtr, const char *sl,
                                          const char *sl_next, char *xs,
                                          uint16_t *__restrict__ dS, const uint16_t *__restrict__ Kw,
                                          const uint16_t *__restrict__ Vw, const int32_t *__restrict__ cu_ws,
                                          int ndocs, int NB, float c, int wave, int lane) {
  const int l32 = lane & 31, h = lane >> 5;
  const int bucket = D.bucket;
  if (bucket != s.bucket) {  // new bucket: this wave's K / V rows
    s.bucket = bucket;
    const int i = D.i;
    const int gb = bucket - i * NB;
    const int dd = upper_index(cu_ws, ndocs - 1, gb * kBlk);
    s.kbase = uniform(gb * kBlk - cu_ws[dd]);
    const size_t kfr = ((size_t)i * NB + gb) * kFragBlock + (wave * 8 * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s.kf[ks] = *(const bf16x8 *)(Kw + kfr + ks * 512);
      s.vf[ks] = *(const bf16x8 *)(Vw + kfr + ks * 512);
    }
    // wait here, on this rare path: the compiler then sees the K / V registers complete on
    // both paths and puts no wait after the join, where it would also wait for the
    // previous phase's dS stores
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }
  const lds_char *lq = (const lds_char *)sl;
  f32x16 sacc, pacc;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    sacc = ks ? mfma32(s.qa[ks], s.kf[ks], sacc) : mfma32(s.qa[ks], s.kf[ks], f32x16{});
    pacc = ks ? mfma32(s.oa[ks], s.vf[ks], pacc) : mfma32(s.oa[ks], s.vf[ks], f32x16{});
  }
  // LSE (log2) and delta of the quarter's rows 8 j + 4 h .. + 3 (chunk j)
  f32x4 lse[4], del[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lse[j] = *(const lds_f32x4_2 *)(lq + 2 * kKv2Half + 4 * (8 * j + 4 * h));
    del[j] = *(const lds_f32x4_2 *)(lq + 2 * kKv2Half + 128 + 4 * (8 * j + 4 * h));
  }
  kv2_score_ops(s, sl_next, lane);
  // register e: row 8 (e / 4) + 4 h + e % 4 of the quarter (query 2 qtr + e / 8), key
  // 32 wave + l32 of the block
  const int kp = s.kbase + 32 * wave + l32;
  bf16x8 pa[2], sa[2];
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const int k = 2 * qtr + sg;
    const int pos = D.pos[k];
    const bool seen = kp <= pos;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * sg + jj;
      const f32x4 l = lse[j], d = del[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pr = seen ? __builtin_amdgcn_exp2f(sacc[4 * j + e] * c - l[e]) : 0.f;
        sacc[4 * j + e] = pr;
        pacc[4 * j + e] = pr * (pacc[4 * j + e] - d[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pa[sg][e] = (__bf16)sacc[8 * sg + e];
      sa[sg][e] = (__bf16)pacc[8 * sg + e];
    }
    // dS tile of query k (padding queries: the spare tile); non-temporal: each tile is
    // read once, by the dQ kernel
    const int tix = D.tix[k];
    const int dsoff = ds_key_swz(32 * wave + l32) * 16 + 8 * h;
    __builtin_nontemporal_store(sa[sg], (bf16x8 *)(dS + (size_t)tix * (kBlk * 16) + dsoff));
  }
  // P / dS to the exchange slot: 16 bytes per lane and operand
  *(bf16x8 *)(xs + (0 * 64 + lane) * 16) = pa[0];
  *(bf16x8 *)(xs + (1 * 64 + lane) * 16) = pa[1];
  *(bf16x8 *)(xs + (2 * 64 + lane) * 16) = sa[0];
  *(bf16x8 *)(xs + (3 * 64 + lane) * 16) = sa[1];
}

// ---- accumulate waves
struct Kv2Acc {
  // all 128 keys x this wave's 32 dims: dk[kt] / dv[kt] hold keys 32 kt .., register e =
  // key 32 kt + 8 (e / 4) + 4 h + e % 4, lane l32 = dim 32 w + l32
  f32x16 dk[4], dv[4];
};

// dV += P^T dO and dK += dS^T Q of the quarter in slot sl, with P / dS of the four score
// waves (key tiles kt) from the exchange slots xs0 + kt kKv2XBytes; then, if the row
// described by D ends its bucket segment and this is its last quarter, the flush of dK /
// dV.  Accumulate wave w owns dims [32 w, 32 w + 32): the B operands (Q / dO with rows as
// the contraction index, through transposing LDS reads) are read once per k-step and
// serve all four key tiles; the A operands are the score waves' bf16 P / dS registers,
// 16-byte reads.
__device__ __forceinline__ void kv2_accumulate(Kv2Acc &a, const Kv2Ids &D, bool last_qtr, const char *sl,
                                               const char *xs0, int NB, float scale, float *__restrict__ dk_pool,
                                               float *__restrict__ dv_pool, int wave, int lane) {
  const int l32 = lane & 31, h = lane >> 5, j16 = lane & 15, G = l32 >> 4;
  // B operands of k-step ks: lane (l32, h) gets dims 32 w + l32 of rows 16 ks + 8 hi +
  // 4 h + 0..3 (hi = 0, 1), matching the row order of the P / dS registers
  // (rows 16 + r: 4096 bytes on; dO: kKv2Half on), read as assembly with the A operands of
  // the first iteration (kv2_lse_log2 gives the reason), waiting within the statement
  bf16x8 ob[2], qb[2];
  bf16x8 pa[2], sa[2];
  {
    static_assert(kKv2Half == 8192, "immediate offsets");
    const int c0 = 32 * wave + 16 * G + 4 * (j16 & 3);
    const uint32_t a0 = kv2_lds_addr(sl) + kv2_swz(4 * h + (j16 >> 2), c0 * 2);
    const uint32_t a1 = kv2_lds_addr(sl) + kv2_swz(4 * h + (j16 >> 2) + 8, c0 * 2);
    const uint32_t ax = kv2_lds_addr(xs0) + 16 * lane;
    u32x2 q00, q01, q10, q11, o00, o01, o10, o11;
    u32x4 p0, s0;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %10\n\t"
        "ds_read_b64_tr_b16 %1, %11\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:4096\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:4096\n\t"
        "ds_read_b64_tr_b16 %4, %10 offset:8192\n\t"
        "ds_read_b64_tr_b16 %5, %11 offset:8192\n\t"
        "ds_read_b64_tr_b16 %6, %10 offset:12288\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:12288\n\t"
        "ds_read_b128 %8, %12\n\t"
        "ds_read_b128 %9, %12 offset:2048\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q00), "=&v"(q01), "=&v"(q10), "=&v"(q11), "=&v"(o00), "=&v"(o01), "=&v"(o10), "=&v"(o11),
          "=&v"(p0), "=&v"(s0)
        : "v"(a0), "v"(a1), "v"(ax)
        : "memory");
    qb[0] = __builtin_bit_cast(bf16x8, u32x4{q00[0], q00[1], q01[0], q01[1]});
    qb[1] = __builtin_bit_cast(bf16x8, u32x4{q10[0], q10[1], q11[0], q11[1]});
    ob[0] = __builtin_bit_cast(bf16x8, u32x4{o00[0], o00[1], o01[0], o01[1]});
    ob[1] = __builtin_bit_cast(bf16x8, u32x4{o10[0], o10[1], o11[0], o11[1]});
    pa[0] = __builtin_bit_cast(bf16x8, p0);
    sa[0] = __builtin_bit_cast(bf16x8, s0);
  }
  // Iteration it = (ks, kt) = (it / 4, it % 4); the A operands of iteration it + 1 are
  // read before the MFMAs of iteration it.
  auto rd = [&](int it, int b) {
    const int ks = it >> 2, kt = it & 3;
    const char *xs = xs0 + kt * kKv2XBytes;
    pa[b] = *(const bf16x8 *)(xs + ((0 + ks) * 64 + lane) * 16);
    sa[b] = *(const bf16x8 *)(xs + ((2 + ks) * 64 + lane) * 16);
  };
  // the products run at raised wave priority, so that the SIMD's matrix unit takes them
  // ahead of the score wave's while both are ready (1-1.5 % faster; the score wave's
  // products first, the other way round, was 8 % slower)
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    if (it + 1 < 8) rd(it + 1, (it + 1) & 1);
    const int ks = it >> 2, kt = it & 3;
    a.dv[kt] = mfma32(pa[it & 1], ob[ks], a.dv[kt]);
    a.dk[kt] = mfma32(sa[it & 1], qb[ks], a.dk[kt]);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  if (last_qtr && D.next != D.bucket) {
    const int i = D.i;
    const int gb = D.bucket - i * NB;
    // a rolled loop (uniform register index): the flush is rare, and unrolled its 128
    // addresses would take registers from the whole walk
#pragma unroll 1
    for (int e = 0; e < 16; e = uniform(e + 1)) {
      const int key = 8 * (e >> 2) + 4 * h + (e & 3);
      const size_t o = ((size_t)(gb * kBlk + key) * kHKV + i) * kD + 32 * wave + l32;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        kv2_atomic_add(dk_pool + o + (size_t)32 * kt * kHKV * kD, scale * a.dk[kt][e]);
        kv2_atomic_add(dv_pool + o + (size_t)32 * kt * kHKV * kD, a.dv[kt][e]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) a.dk[kt][e] = a.dv[kt][e] = 0.f;
  }
}

// One phase n = 4 g + QTR: move the descriptor of row g + 2 (copied in phase 4 g,
// completed and stored in phase 4 g + 3), issue the copies of quarter n + kKv2Ahead, rescale the LSE of
// quarter n + 1, the score waves' quarter n (if n < nq) and the accumulate waves' quarter
// n - 1 (if n >= 1); the accumulate waves then wait for their copies of quarter n + 2
// (issued in phase n - 2), and the barrier.
struct Kv2Ctx {
  char *slots, *xch;
  int *desc, *dstage;
  Kv2Rows R;
  int nq;
  bool score;
  int wave, lane, tid;
};

// ids: the score waves' row g; for the accumulate waves, the row whose quarters they
// gather in this row's phases (g + 1, or the last row) and prev: row g - 1 (its last
// quarter is accumulated in phase 4 g).
// ROLE of an accumulate wave besides its products and gather (a template argument, so
// that no wave's code has a conditional load): 1 moves LSE and delta (the first wave), 2
// the task-row descriptors (the second), 0 nothing more.
template <int QTR, bool SCORE, int ROLE>
__device__ __forceinline__ void kv2_phase(Kv2Ctx &x, int g, const Kv2Ids &ids, const Kv2Ids &prev,
                                          const Kv2Ids &gat, Kv2Score &s,
                                          Kv2Acc &a,
                                          const uint16_t *__restrict__ Q, const uint16_t *__restrict__ dO,
                                          const float *__restrict__ LSE, const float *__restrict__ Delta,
                                          uint16_t *__restrict__ dS, const uint16_t *__restrict__ Kw,
                                          const uint16_t *__restrict__ Vw, const i32x4 *__restrict__ meta,
                                          const int32_t *__restrict__ qrows, const int32_t *__restrict__ qpos,
                                          const int32_t *__restrict__ qtile, const int32_t *__restrict__ cu_ws,
                                          int ndocs, int NB, float c, float scale, float *__restrict__ dk_pool,
                                          float *__restrict__ dv_pool, int ds_spare) {
  const int n = 4 * g + QTR;
  static_assert(kKv2Ahead == 4 && kKv2Slots == 6, "copy schedule");
  if constexpr (!SCORE) {
    if (ROLE == 2 && QTR == 0)  // the words of row g + 2, copied to the staging area
      __builtin_amdgcn_global_load_lds((const kv2_gvoid *)kv2_desc_src(x.R, g + 2, meta, qrows, qpos, qtile, x.lane),
                                       (kv2_lvoid *)x.dstage, 4, 0, 0);
    if (ROLE == 2 && QTR == 3) {
      // the staged words (their copy, issued before phase 4 g's gather, was waited for at
      // the end of phase 4 g + 2) completed into the descriptor ring; read and stored as
      // assembly, which the compiler does not order behind the copies in flight
      int v;
      const uint32_t a = kv2_lds_addr((const char *)x.dstage) + 4 * (x.lane & 31);
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
      v = kv2_desc_pad(kv2_desc_fix(v, x.R, g + 2, x.lane), x.lane, ds_spare);
      if (x.lane < kKv2Desc) {
        const uint32_t d = kv2_lds_addr((const char *)(x.desc + ((g + 2) & 3) * kKv2Desc)) + 4 * x.lane;
        asm volatile("ds_write_b32 %0, %1" ::"v"(d), "v"(v) : "memory");
      }
    }
    // quarter n + kKv2Ahead = quarter QTR of row g + 1 (gat); past the end, a valid
    // quarter (unused)
    const int qa = g + 1 < x.R.total ? QTR : 3;
    kv2_gather<ROLE == 1>(x.slots + ((n + kKv2Ahead) % kKv2Slots) * kKv2SlotBytes, gat.i, gat.t[2 * qa],
                          gat.t[2 * qa + 1], Q, dO, LSE, Delta, x.tid - 256);
    if (ROLE == 1) kv2_lse_log2(x.slots + ((n + 1) % kKv2Slots) * kKv2SlotBytes, x.lane);
  }
  if constexpr (SCORE) {
    if (n < x.nq)
      kv2_score(s, ids, QTR, x.slots + (n % kKv2Slots) * kKv2SlotBytes,
                x.slots + ((n + 1) % kKv2Slots) * kKv2SlotBytes,
                x.xch + ((n & 1) * 4 + x.wave) * kKv2XBytes, dS, Kw, Vw, cu_ws, ndocs, NB, c, x.wave, x.lane);
  } else if (n >= 1 && n - 1 < x.nq) {
    const int m = n - 1;
    kv2_accumulate(a, prev, (m & 3) == 3, x.slots + (m % kKv2Slots) * kKv2SlotBytes,
                   x.xch + (m & 1) * 4 * kKv2XBytes, NB, scale, dk_pool, dv_pool, x.wave, x.lane);
  }
  if constexpr (!SCORE) {
    // this wave's loads issued after the copies of phase n - 2, which complete in order:
    // its copies of phases n - 1 and n (4 each, 5 in the first wave) and, in the second,
    // the descriptor copy issued first in phase 4 g (the dK / dV atomics of a flush, which
    // may complete out of order, only make the wait longer)
    constexpr int kAfter = ROLE == 1 ? 10 : (ROLE == 2 && QTR <= 1) ? 9 : 8;
    WAIT_VMCNT(kAfter);
  }
  kv2_barrier();
}

__global__ void __launch_bounds__(kKv2Threads, 1)
bwd_kv2_kernel(uint16_t *__restrict__ dS, const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kw,
               const uint16_t *__restrict__ Vw, const uint16_t *__restrict__ dO, const float *__restrict__ LSE,
               const float *__restrict__ Delta, const int32_t *__restrict__ cta, const i32x4 *__restrict__ meta,
               const int32_t *__restrict__ qrows, const int32_t *__restrict__ qpos,
               const int32_t *__restrict__ qtile, const int32_t *__restrict__ cu_ws, int ndocs, int NB, int grid,
               float scale, float scale_log2e, float *__restrict__ dk_pool, float *__restrict__ dv_pool,
               int ds_spare) {
  __shared__ __attribute__((aligned(16))) char slots[kKv2Slots * kKv2SlotBytes];
  __shared__ __attribute__((aligned(16))) char xch[2 * 4 * kKv2XBytes];
  __shared__ int desc[4 * kKv2Desc];
  __shared__ int dstage[64];
  const int c = blockIdx.x, tid = threadIdx.x;
  Kv2Ctx x;
  x.slots = slots;
  x.xch = xch;
  x.desc = desc;
  x.dstage = dstage;
  x.tid = tid;
  x.lane = tid & 63;
  x.wave = uniform((tid >> 6) & 3);
  x.score = uniform(tid >> 8) == 0;
  x.R.lo0 = uniform(cta[0 * (grid + 1) + c]);
  x.R.lo1 = uniform(cta[1 * (grid + 1) + c]);
  x.R.lo2 = uniform(cta[2 * (grid + 1) + c]);
  x.R.lo3 = uniform(cta[3 * (grid + 1) + c]);
  x.R.n0 = uniform(cta[0 * (grid + 1) + c + 1]) - x.R.lo0;
  x.R.n1 = uniform(cta[1 * (grid + 1) + c + 1]) - x.R.lo1;
  x.R.n2 = uniform(cta[2 * (grid + 1) + c + 1]) - x.R.lo2;
  x.R.n3 = uniform(cta[3 * (grid + 1) + c + 1]) - x.R.lo3;
  x.R.total = x.R.n0 + x.R.n1 + x.R.n2 + x.R.n3;
  if (x.R.total == 0) return;
  x.nq = 4 * x.R.total;
  // prologue: descriptors of rows 0 and 1, then the quarters of row 0
  if (tid < 64) {  // descriptors of rows 0 (lanes 0-31) and 1 (lanes 32-63)
    const int v = kv2_desc_load(x.R, tid >> 5, meta, qrows, qpos, qtile, tid & 31);
    const bool up = tid >= 32;  // constant lane indices for both rows, then a per-lane choice
    const int nv = up ? __builtin_amdgcn_readlane(v, 32 + kDescNv) : __builtin_amdgcn_readlane(v, kDescNv);
    const int t0 = up ? __builtin_amdgcn_readlane(v, 32 + kDescT) : __builtin_amdgcn_readlane(v, kDescT);
    const int l = tid & 31, k = (l - kDescT) & 7;
    desc[tid] = (l >= kDescT && l < kDescT + 24 && k >= nv) ? (l < kDescPos ? t0 : l < kDescTile ? -1 : ds_spare) : v;
  }
  __syncthreads();
  {
    Kv2Ids d0;
    kv2_ids(d0, desc, x.lane);
    if (!x.score) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        kv2_gather<true>(slots + q * kKv2SlotBytes, d0.i, d0.t[2 * q], d0.t[2 * q + 1], Q, dO, LSE, Delta, tid - 256);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the copies of quarters 0-3
  __syncthreads();
  if (tid >= 256 && tid < 264) kv2_lse_log2(slots, tid - 256);  // quarter 0 (1-3: phases 0-2)
  __syncthreads();
#define KV2_PHASES(SC, LD)                                                                                      \
  for (int g = 0; g < x.R.total; ++g) {                                                                     \
    Kv2Ids ids, prev, gat;                                                                                  \
    kv2_ids(gat, desc + (min(g + 1, x.R.total - 1) & 3) * kKv2Desc, x.lane);                               \
    if (SC)                                                                                                 \
      kv2_ids(ids, desc + (g & 3) * kKv2Desc, x.lane);                                                      \
    else                                                                                                    \
      kv2_ids(prev, desc + ((g + 3) & 3) * kKv2Desc, x.lane);                                               \
    kv2_phase<0, SC, LD>(x, g, ids, prev, gat, s, a, Q, dO, LSE, Delta, dS, Kw, Vw, meta, qrows, qpos, qtile, cu_ws, \
                     ndocs, NB, scale_log2e, scale, dk_pool, dv_pool, ds_spare);                           \
    kv2_phase<1, SC, LD>(x, g, ids, prev, gat, s, a, Q, dO, LSE, Delta, dS, Kw, Vw, meta, qrows, qpos, qtile, cu_ws, \
                     ndocs, NB, scale_log2e, scale, dk_pool, dv_pool, ds_spare);                           \
    kv2_phase<2, SC, LD>(x, g, ids, prev, gat, s, a, Q, dO, LSE, Delta, dS, Kw, Vw, meta, qrows, qpos, qtile, cu_ws, \
                     ndocs, NB, scale_log2e, scale, dk_pool, dv_pool, ds_spare);                           \
    kv2_phase<3, SC, LD>(x, g, ids, prev, gat, s, a, Q, dO, LSE, Delta, dS, Kw, Vw, meta, qrows, qpos, qtile, cu_ws, \
                     ndocs, NB, scale_log2e, scale, dk_pool, dv_pool, ds_spare);                           \
  }
  // each role runs its own loop, so that only its own state is live in it
  if (x.score) {
    Kv2Score s;
    Kv2Acc a;  // unused
    s.bucket = -1;
    s.kbase = 0;
    kv2_score_ops(s, slots, x.lane);  // quarter 0
    KV2_PHASES(true, 0)
  } else {
    Kv2Score s;  // unused
    Kv2Acc a;
#pragma unroll
    for (int nd = 0; nd < 4; ++nd)
#pragma unroll
      for (int e = 0; e < 16; ++e) a.dk[nd][e] = a.dv[nd][e] = 0.f;
    if (x.wave == 0) {
      KV2_PHASES(false, 1)
    } else if (x.wave == 1) {
      KV2_PHASES(false, 2)
    } else {
      KV2_PHASES(false, 0)
    }
    // the last quarter (phase nq)
    const int m = x.nq - 1;
    Kv2Ids last;
    kv2_ids(last, desc + (((m >> 2)) & 3) * kKv2Desc, x.lane);
    kv2_accumulate(a, last, true, slots + (m % kKv2Slots) * kKv2SlotBytes, xch + (m & 1) * 4 * kKv2XBytes, NB,
                   scale, dk_pool, dv_pool, x.wave, x.lane);
    // the copies issued ahead of the end must land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
#undef KV2_PHASES
}

namespace host {
hipError_t backward_kv2(const void *Q, const void *Kw, const void *Vw, const void *dO, const float *LSE,
                        const float *delta, const void *tasks, const LayoutArgs &L, int grid, float scale,
                        float *dk_pool, float *dv_pool, void *dS, hipStream_t s) {
  TaskView v = task_view(L, grid, const_cast<void *>(tasks));
  hipLaunchKernelGGL(bwd_kv2_kernel, dim3(grid), dim3(kKv2Threads), 0, s, (uint16_t *)dS, (const uint16_t *)Q,
                     (const uint16_t *)Kw, (const uint16_t *)Vw, (const uint16_t *)dO, LSE, delta, v.cta,
                     (const i32x4 *)v.meta, v.qrows, v.qpos, v.qtile, L.cu_ws, L.ndocs, L.NB, grid, scale,
                     scale * kLog2e, dk_pool, dv_pool, L.T * kHI * kTopk);
  return hipGetLastError();
}
}  // namespace host
}  // namespace msa
