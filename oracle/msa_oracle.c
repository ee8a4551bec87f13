/*
 * msa_oracle.c -- plain, slow fp64 CPU reference for MiniMax Sparse Attention (MSA)
 * prefill forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header or constant with
 * the HIP library; it is written from the definition of the operator, not from any
 * kernel design.
 *
 * What is computed (MSA PR page, "Design" and "Supported scope"; msa_backward_sm100
 * API page, run_backward):
 *   Documents are packed back to back: document d holds compact tokens
 *   [cu[d], cu[d+1]).  Token t has document-local position pos(t) = t - cu[doc(t)] and
 *   key block blk(t) = pos(t) / BLK.  Query head h belongs to index head
 *   i = h / (H / HI) and reads KV head kv = i / (HI / HKV).  q2k[i][t][*] lists
 *   document-local key-block ids, -1 in unused slots.  The keys that (t, h) attends to:
 *       K(h, t) = { s : doc(s) = doc(t), pos(s) <= pos(t), blk(s) in Sel(i, t) }
 *   with Sel(i, t) the SET of listed ids (causal prefill, document-local selection).
 *   Forward (natural log, softmax scale folded in):
 *       s_j = scale * <Q[t,h], K[j,kv]>,   LSE = log sum_j exp(s_j),
 *       P_j = exp(s_j - LSE),              O[t,h] = sum_j P_j V[j,kv]
 *   Backward, with dO the output gradient:
 *       delta = <dO[t,h], O[t,h]>,  dP_j = <dO[t,h], V[j,kv]>,  dS_j = P_j (dP_j - delta)
 *       dQ[t,h] = scale sum_j dS_j K[j,kv]
 *       dK[j,kv] += scale dS_j Q[t,h],  dV[j,kv] += P_j dO[t,h]
 *   A row whose key set is empty gets O = 0, LSE = -inf and contributes nothing.
 *
 * Every floating-point operation is in double precision.  The shape (H, HKV, HI, D,
 * BLK, TOPK) is a runtime parameter so that tiny shapes can be checked by brute force.
 *
 * Entries of q2k that are -1, outside [0, blk(t)], or repeats of an earlier slot of the
 * same row add no keys: the key set is defined by membership, and a block after blk(t)
 * holds no key with pos(s) <= pos(t).  msa_oracle_validate reports such entries.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int T, H, HKV, HI, D, BLK, TOPK, ndocs;
  const int32_t *cu; /* [ndocs + 1] */
} shape_t;

static int doc_of(const shape_t *s, int t) {
  int lo = 0, hi = s->ndocs - 1; /* largest d with cu[d] <= t */
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (s->cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/* Block id of slot j of (i, t) if it is a member of Sel(i, t) that can contribute
 * keys and is the first listing of that id; -1 otherwise. */
static int slot_block(const shape_t *s, const int32_t *q2k, int i, int t, int j, int blk_t) {
  const int32_t *row = q2k + ((size_t)i * s->T + t) * s->TOPK;
  int b = row[j];
  if (b < 0 || b > blk_t) return -1;
  for (int jj = 0; jj < j; ++jj)
    if (row[jj] == b) return -1;
  return b;
}

static double dot(const double *a, const double *b, int n) {
  double acc = 0.0;
  for (int k = 0; k < n; ++k) acc += a[k] * b[k];
  return acc;
}

/* Gather the key indices of K(h, t) for index head i into keys[]; returns the count. */
static int key_set(const shape_t *s, const int32_t *q2k, int i, int t, int *keys) {
  int d = doc_of(s, t);
  int base = s->cu[d], pos = t - base, blk_t = pos / s->BLK, n = 0;
  for (int j = 0; j < s->TOPK; ++j) {
    int b = slot_block(s, q2k, i, t, j, blk_t);
    if (b < 0) continue;
    for (int k = 0; k < s->BLK; ++k) {
      int kp = b * s->BLK + k;
      if (kp > pos) break;
      keys[n++] = base + kp;
    }
  }
  return n;
}

/* Scores, LSE and probabilities of row (t, h).  sc[] receives P_j on return. */
static double row_softmax(const shape_t *s, const double *Q, const double *K, int t, int h,
                          int kv, const int *keys, int n, double scale, double *sc) {
  if (n == 0) return -INFINITY;
  const double *q = Q + ((size_t)t * s->H + h) * s->D;
  double m = -INFINITY;
  for (int j = 0; j < n; ++j) {
    sc[j] = scale * dot(q, K + ((size_t)keys[j] * s->HKV + kv) * s->D, s->D);
    if (sc[j] > m) m = sc[j];
  }
  double sum = 0.0;
  for (int j = 0; j < n; ++j) sum += exp(sc[j] - m);
  double lse = m + log(sum);
  for (int j = 0; j < n; ++j) sc[j] = exp(sc[j] - lse);
  return lse;
}

static int max_keys(const shape_t *s) { return s->TOPK * s->BLK; }

/* Forward for the rows t with row_mask[t] != 0 (all rows if row_mask is NULL).
 * Q [T,H,D], K/V [T,HKV,D] (compact), O [T,H,D], LSE [T,H]; unselected rows untouched. */
int msa_oracle_forward(int T, int H, int HKV, int HI, int D, int BLK, int TOPK, int ndocs,
                       const int32_t *cu, const double *Q, const double *K, const double *V,
                       const int32_t *q2k, double scale, const uint8_t *row_mask,
                       double *O, double *LSE) {
  shape_t s = {T, H, HKV, HI, D, BLK, TOPK, ndocs, cu};
  if (H % HI || HI % HKV) return 1;
  int heads_per_index = H / HI, index_per_kv = HI / HKV;
#pragma omp parallel
  {
    int *keys = (int *)malloc(sizeof(int) * max_keys(&s));
    double *p = (double *)malloc(sizeof(double) * max_keys(&s));
#pragma omp for schedule(dynamic, 16)
    for (long long ti = 0; ti < (long long)T * HI; ++ti) {
      int t = (int)(ti / HI), i = (int)(ti % HI);
      if (row_mask && !row_mask[t]) continue;
      int n = key_set(&s, q2k, i, t, keys), kv = i / index_per_kv;
      for (int hh = 0; hh < heads_per_index; ++hh) {
        int h = i * heads_per_index + hh;
        double lse = row_softmax(&s, Q, K, t, h, kv, keys, n, scale, p);
        double *o = O + ((size_t)t * H + h) * D;
        for (int c = 0; c < D; ++c) o[c] = 0.0;
        for (int j = 0; j < n; ++j) {
          const double *v = V + ((size_t)keys[j] * HKV + kv) * D;
          for (int c = 0; c < D; ++c) o[c] += p[j] * v[c];
        }
        LSE[(size_t)t * H + h] = lse;
      }
    }
    free(keys);
    free(p);
  }
  return 0;
}

/* delta[t,h] = sum_c dO[t,h,c] * O[t,h,c] for any given O (used on the bf16 forward
 * output that the backward consumes). */
int msa_oracle_delta(int T, int H, int D, const double *O, const double *dO, double *delta) {
#pragma omp parallel for schedule(static)
  for (long long r = 0; r < (long long)T * H; ++r) delta[r] = dot(O + r * D, dO + r * D, D);
  return 0;
}

/* Backward.  dQ rows are produced for t with q_mask[t] != 0; dK/dV rows for the key
 * blocks (kv head, document, block) whose compact tokens have kb_mask[s] != 0 (masks may
 * be NULL = all).  The forward quantities (LSE, O, delta) are recomputed exactly from
 * Q/K/V, so the gradients are those of the exact fp64 forward.  dQ [T,H,D], dK/dV
 * [T,HKV,D]; entries outside the masks are left untouched except that selected dK/dV
 * rows are overwritten. */
int msa_oracle_backward(int T, int H, int HKV, int HI, int D, int BLK, int TOPK, int ndocs,
                        const int32_t *cu, const double *Q, const double *K, const double *V,
                        const double *dO, const int32_t *q2k, double scale,
                        const uint8_t *q_mask, const uint8_t *kb_mask,
                        double *dQ, double *dK, double *dV, double *LSE_out,
                        double *delta_out) {
  shape_t s = {T, H, HKV, HI, D, BLK, TOPK, ndocs, cu};
  if (H % HI || HI % HKV) return 1;
  int hpi = H / HI, ipk = HI / HKV;
  /* Rows whose softmax statistics are needed: dQ rows, and every query that selects a
   * key block with a masked-in key (its (LSE, delta) feed that block's dK/dV). */
  uint8_t *need = (uint8_t *)calloc((size_t)T * HI, 1);
  double *lse = (double *)malloc(sizeof(double) * (size_t)T * H);
  double *dlt = (double *)malloc(sizeof(double) * (size_t)T * H);
  if (!need || !lse || !dlt) { free(need); free(lse); free(dlt); return 2; }
#pragma omp parallel for schedule(dynamic, 64)
  for (long long ti = 0; ti < (long long)T * HI; ++ti) {
    int t = (int)(ti / HI), i = (int)(ti % HI);
    if (!q_mask || q_mask[t]) { need[ti] = 1; continue; }
    int d = doc_of(&s, t), base = cu[d], pos = t - base;
    for (int j = 0; j < TOPK && !need[ti]; ++j) {
      int b = slot_block(&s, q2k, i, t, j, pos / BLK);
      if (b < 0) continue;
      for (int k = 0; k < BLK && b * BLK + k <= pos; ++k)
        if (!kb_mask || kb_mask[base + b * BLK + k]) { need[ti] = 1; break; }
    }
  }
  /* Phase A: per needed row, LSE, exact O, delta; dQ for masked rows. */
#pragma omp parallel
  {
    int *keys = (int *)malloc(sizeof(int) * max_keys(&s));
    double *p = (double *)malloc(sizeof(double) * max_keys(&s));
    double *o = (double *)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 16)
    for (long long ti = 0; ti < (long long)T * HI; ++ti) {
      if (!need[ti]) continue;
      int t = (int)(ti / HI), i = (int)(ti % HI), kv = i / ipk;
      int n = key_set(&s, q2k, i, t, keys);
      for (int hh = 0; hh < hpi; ++hh) {
        int h = i * hpi + hh;
        size_t r = (size_t)t * H + h;
        double l = row_softmax(&s, Q, K, t, h, kv, keys, n, scale, p);
        for (int c = 0; c < D; ++c) o[c] = 0.0;
        for (int j = 0; j < n; ++j) {
          const double *v = V + ((size_t)keys[j] * HKV + kv) * D;
          for (int c = 0; c < D; ++c) o[c] += p[j] * v[c];
        }
        const double *g = dO + r * D;
        double delta = dot(g, o, D);
        lse[r] = l;
        dlt[r] = delta;
        if (q_mask && !q_mask[t]) continue;
        double *dq = dQ + r * D;
        for (int c = 0; c < D; ++c) dq[c] = 0.0;
        for (int j = 0; j < n; ++j) {
          const double *kr = K + ((size_t)keys[j] * HKV + kv) * D;
          const double *vr = V + ((size_t)keys[j] * HKV + kv) * D;
          double ds = p[j] * (dot(g, vr, D) - delta);
          for (int c = 0; c < D; ++c) dq[c] += scale * ds * kr[c];
        }
      }
    }
    free(keys);
    free(p);
    free(o);
  }
  /* Phase B: per (kv head, document, key block), sum over every (t, h) whose key set
   * contains the block's keys.  Each task owns its block's dK/dV rows: no races. */
  int nblk_total = 0;
  int *blk_doc = (int *)malloc(sizeof(int) * (size_t)(T / BLK + ndocs + 1));
  int *blk_id = (int *)malloc(sizeof(int) * (size_t)(T / BLK + ndocs + 1));
  for (int d = 0; d < ndocs; ++d) {
    int L = cu[d + 1] - cu[d];
    for (int b = 0; b * BLK < L; ++b) { blk_doc[nblk_total] = d; blk_id[nblk_total] = b; ++nblk_total; }
  }
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int kv = 0; kv < HKV; ++kv) {
    for (int nb = 0; nb < nblk_total; ++nb) {
      int d = blk_doc[nb], b = blk_id[nb], base = cu[d], L = cu[d + 1] - cu[d];
      int k0 = b * BLK, k1 = (k0 + BLK < L) ? k0 + BLK : L; /* doc-local key range */
      int any = 0;
      for (int kp = k0; kp < k1; ++kp) any |= (!kb_mask || kb_mask[base + kp]);
      if (!any) continue;
      for (int kp = k0; kp < k1; ++kp) {
        if (kb_mask && !kb_mask[base + kp]) continue;
        for (int c = 0; c < D; ++c) {
          dK[((size_t)(base + kp) * HKV + kv) * D + c] = 0.0;
          dV[((size_t)(base + kp) * HKV + kv) * D + c] = 0.0;
        }
      }
      for (int i = kv * ipk; i < (kv + 1) * ipk; ++i) {
        for (int qp = k0; qp < L; ++qp) { /* queries at or after the block start */
          int t = base + qp, blk_t = qp / BLK, member = 0;
          for (int j = 0; j < TOPK; ++j)
            if (slot_block(&s, q2k, i, t, j, blk_t) == b) member = 1;
          if (!member) continue;
          for (int hh = 0; hh < hpi; ++hh) {
            int h = i * hpi + hh;
            size_t r = (size_t)t * H + h;
            const double *q = Q + r * D, *g = dO + r * D;
            for (int kp = k0; kp < k1 && kp <= qp; ++kp) {
              if (kb_mask && !kb_mask[base + kp]) continue;
              size_t kr = ((size_t)(base + kp) * HKV + kv) * D;
              double sc = scale * dot(q, K + kr, D);
              double pj = exp(sc - lse[r]);
              double ds = pj * (dot(g, V + kr, D) - dlt[r]);
              for (int c = 0; c < D; ++c) {
                dK[kr + c] += scale * ds * q[c];
                dV[kr + c] += pj * g[c];
              }
            }
          }
        }
      }
    }
  }
  if (LSE_out) memcpy(LSE_out, lse, sizeof(double) * (size_t)T * H);
  if (delta_out) memcpy(delta_out, dlt, sizeof(double) * (size_t)T * H);
  free(blk_doc);
  free(blk_id);
  free(need);
  free(lse);
  free(dlt);
  return 0;
}

/* Precondition check of q2k (the selection is document-local, causal and duplicate
 * free; -1 marks unused slots).  Returns a bit set: 1 = an id outside [-1, blk(t)],
 * 2 = an id listed twice in one row. */
int msa_oracle_validate(int T, int HI, int BLK, int TOPK, int ndocs, const int32_t *cu,
                        const int32_t *q2k) {
  shape_t s = {T, 0, 0, HI, 0, BLK, TOPK, ndocs, cu};
  int flags = 0;
  for (int i = 0; i < HI; ++i)
    for (int t = 0; t < T; ++t) {
      int blk_t = (t - cu[doc_of(&s, t)]) / BLK;
      const int32_t *row = q2k + ((size_t)i * T + t) * TOPK;
      for (int j = 0; j < TOPK; ++j) {
        if (row[j] == -1) continue;
        if (row[j] < -1 || row[j] > blk_t) flags |= 1;
        else
          for (int jj = 0; jj < j; ++jj)
            if (row[jj] == row[j]) flags |= 2;
      }
    }
  return flags;
}
