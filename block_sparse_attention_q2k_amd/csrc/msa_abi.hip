// msa_abi.hip -- the C ABI of libmsa (declared in include/msa.h): argument checks on
// the host, then kernel launches on the caller's stream.
#include <string.h>

#include <atomic>
#include <mutex>

#include "msa_device.h"
#include "msa_launch.h"

using namespace msa;

// Counters of msa_build_k2q_csr_noalloc (one int32 per CSR row, 4 index heads x the
// largest block count a layout may have, 2 MiB): a device array of the library, so that
// the call allocates nothing.  Each GPU holds its own copy until the process ends; host
// code uses only the per-device address from hipGetSymbolAddress, never this name.
constexpr size_t kNoAllocCsrWords = (size_t)MSA_NUM_INDEX_HEADS * ((size_t)1 << 24) / MSA_BLOCK;
static __device__ __align__(256) int32_t scratch[kNoAllocCsrWords];

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_ptrs(std::initializer_list<const void *> ps) {
  for (const void *p : ps) {
    if (!p) return MSA_ERR_NULL;
    if (!aligned16(p)) return MSA_ERR_ALIGN;
  }
  return MSA_OK;
}

// Host-side consistency of the layout struct (the device arrays are trusted to hold
// what msa_layout_host produced).
int check_layout(const msa_layout *L, LayoutArgs *out) {
  if (!L) return MSA_ERR_NULL;
  if (L->num_docs < 1 || L->num_tokens < 1 || L->num_ws_tokens < L->num_tokens ||
      L->num_ws_tokens % MSA_BLOCK != 0 || L->num_docs > L->num_tokens)
    return MSA_ERR_SHAPE;
  // index arithmetic uses int32 offsets for rows of 64 x 128 elements
  if ((long long)L->num_ws_tokens > (1LL << 24)) return MSA_ERR_SHAPE;
  int rc = check_ptrs({L->cu_seqlens, L->cu_ws});
  if (rc) return rc;
  if (out) {
    out->ndocs = L->num_docs;
    out->T = L->num_tokens;
    out->W = L->num_ws_tokens;
    out->NB = L->num_ws_tokens / MSA_BLOCK;
    out->cu = L->cu_seqlens;
    out->cu_ws = L->cu_ws;
  }
  return MSA_OK;
}

// The kernels are built for gfx950 only.
int check_device() {
  static std::atomic<int> checked[64];  // per device: 0 unknown, 1 ok, 2 bad (any thread)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MSA_ERR_DEVICE;
  const int known = dev < 64 ? checked[dev].load(std::memory_order_relaxed) : 0;
  if (known) return known == 1 ? MSA_OK : MSA_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MSA_ERR_DEVICE;
  int ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) checked[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MSA_OK : MSA_ERR_DEVICE;
}

// The softmax scale: finite and positive.
bool scale_ok(float scale) { return scale > 0.f && scale < __builtin_inff(); }

int launch_rc(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH; }

size_t round16(size_t b) { return (b + 15) / 16 * 16; }

// Stored dS tiles: T x 4 index heads x 16 slots x (16 heads x 128 keys) bf16, plus one
// spare tile that the KV-parallel kernel writes for the padding queries of a task row.
size_t ds_store_bytes(const LayoutArgs &L) {
  return ((size_t)L.T * MSA_NUM_INDEX_HEADS * MSA_TOPK + 1) * 16 * MSA_BLOCK * 2;
}

// Device address of `scratch` per device, looked up once (with that device current) on
// the first msa_build_k2q_csr_noalloc call there.
std::mutex g_scratch_mu;
int32_t *g_scratch_ptr[64] = {};

int noalloc_scratch(int32_t **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MSA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSA_ERR_DEVICE;
    g_scratch_ptr[dev] = (int32_t *)p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

thread_local hipEvent_t t_events[MSA_TIMING_EVENTS] = {};

// Records timing event k on s if the hook is set.
hipError_t mark(int k, hipStream_t s) { return t_events[k] ? hipEventRecord(t_events[k], s) : hipSuccess; }

}  // namespace

extern "C" {

int msa_layout_host(const int32_t *cu_seqlens_host, int32_t num_docs, int32_t *cu_ws_host,
                    int32_t *num_ws_tokens) {
  if (!cu_seqlens_host || !cu_ws_host || !num_ws_tokens) return MSA_ERR_NULL;
  if (num_docs < 1 || cu_seqlens_host[0] != 0) return MSA_ERR_SHAPE;
  long long ws = 0;
  cu_ws_host[0] = 0;
  for (int d = 0; d < num_docs; ++d) {
    long long len = (long long)cu_seqlens_host[d + 1] - cu_seqlens_host[d];
    if (len <= 0) return MSA_ERR_SHAPE;
    ws += (len + MSA_BLOCK - 1) / MSA_BLOCK * MSA_BLOCK;
    if (ws > (1LL << 24)) return MSA_ERR_SHAPE;
    cu_ws_host[d + 1] = (int32_t)ws;
  }
  *num_ws_tokens = (int32_t)ws;
  return MSA_OK;
}

size_t msa_csr_scratch_bytes(const msa_layout *layout) {
  LayoutArgs L;
  if (check_layout(layout, &L)) return 0;
  return round16((size_t)MSA_NUM_INDEX_HEADS * L.NB * 4);
}

size_t msa_csr_cols_capacity(const msa_layout *layout) {
  LayoutArgs L;
  if (check_layout(layout, &L)) return 0;
  return (size_t)MSA_NUM_INDEX_HEADS * L.T * MSA_TOPK;
}

size_t msa_plan_bytes(const msa_layout *layout) {
  LayoutArgs L;
  if (check_layout(layout, &L)) return 0;
  return round16(host::plan_bytes(L));
}

size_t msa_tasks_bytes(const msa_layout *layout, int32_t grid) {
  LayoutArgs L;
  if (check_layout(layout, &L) || grid < 1 || grid > MSA_MAX_GRID) return 0;
  return round16(host::tasks_bytes(L, grid));
}

size_t msa_tasks_meta_offset(int32_t grid) {
  if (grid < 1 || grid > MSA_MAX_GRID) return 0;
  return host::tasks_meta_offset_words(grid);
}

size_t msa_bwd_scratch_bytes(const msa_layout *layout, int dq_accum_mode) {
  LayoutArgs L;
  if (check_layout(layout, &L)) return 0;
  size_t elem;
  switch (dq_accum_mode) {
    case MSA_DQ_ACCUM_FP32: elem = 4; break;
    case MSA_DQ_ACCUM_BF16X2: elem = 2; break;
    case MSA_DQ_ACCUM_F16X2: elem = 2; break;
    case MSA_DQ_RECOMPUTE: elem = 0; break;
    case MSA_DQ_STORED: elem = 0; break;
    default: return 0;
  }
  size_t dq = round16((size_t)L.T * MSA_NUM_Q_HEADS * MSA_HEAD_DIM * elem);
  size_t kv = round16((size_t)L.W * MSA_NUM_KV_HEADS * MSA_HEAD_DIM * 4);
  size_t ds = dq_accum_mode == MSA_DQ_STORED ? ds_store_bytes(L) : 0;
  return dq + 2 * kv + ds;
}

int32_t msa_default_grid(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;
  return cus > MSA_MAX_GRID ? MSA_MAX_GRID : cus;
}

int msa_align_kv(const msa_bf16 *K, const msa_bf16 *V, const msa_layout *layout, msa_bf16 *Kw,
                 msa_bf16 *Vw, msa_bf16 *Kt, msa_bf16 *Vt, void *stream) {
  LayoutArgs L;
  int rc = check_layout(layout, &L);
  if (!rc) rc = check_ptrs({K, V, Kw, Vw, Kt, Vt});
  if (!rc) rc = check_device();
  if (rc) return rc;
  return launch_rc(host::align_kv(K, V, L, Kw, Vw, Kt, Vt, (hipStream_t)stream));
}

int msa_index_select(const msa_bf16 *IQ, const msa_bf16 *IK, const msa_layout *layout, int32_t *q2k,
                     void *stream) {
  LayoutArgs L;
  int rc = check_layout(layout, &L);
  if (!rc) rc = check_ptrs({IQ, IK, q2k});
  if (!rc) rc = check_device();
  if (rc) return rc;
  return launch_rc(host::index_select(IQ, IK, L, q2k, (hipStream_t)stream));
}

int msa_build_k2q_csr(const int32_t *q2k, const msa_layout *layout, int32_t *row_ptr,
                      int32_t *cols, int32_t *status, void *scratch, size_t scratch_bytes,
                      void *stream) {
  LayoutArgs L;
  int rc = check_layout(layout, &L);
  if (!rc) rc = check_ptrs({q2k, row_ptr, cols, status, scratch});
  if (rc) return rc;
  if (scratch_bytes < msa_csr_scratch_bytes(layout)) return MSA_ERR_SCRATCH;
  if ((rc = check_device())) return rc;
  return launch_rc(host::build_csr(q2k, L, row_ptr, cols, status, (int32_t *)scratch,
                                   (hipStream_t)stream));
}

int msa_build_k2q_csr_noalloc(const int32_t *q2k, const msa_layout *layout, int32_t *row_ptr,
                              int32_t *cols, int32_t *status, void *stream) {
  LayoutArgs L;
  int rc = check_layout(layout, &L);
  if (!rc) rc = check_ptrs({q2k, row_ptr, cols, status});
  if (rc) return rc;
  if ((size_t)MSA_NUM_INDEX_HEADS * L.NB > kNoAllocCsrWords) return MSA_ERR_SCRATCH;
  if ((rc = check_device())) return rc;
  int32_t *counters = nullptr;
  if ((rc = noalloc_scratch(&counters))) return rc;
  return launch_rc(host::build_csr(q2k, L, row_ptr, cols, status, counters, (hipStream_t)stream));
}

int msa_plan(const msa_layout *layout, const int32_t *q2k, void *plan, size_t plan_bytes,
             void *stream) {
  LayoutArgs L;
  int rc = check_layout(layout, &L);
  if (!rc) rc = check_ptrs({q2k, plan});
  if (rc) return rc;
  if (plan_bytes < msa_plan_bytes(layout)) return MSA_ERR_SCRATCH;
  if ((rc = check_device())) return rc;
  return launch_rc(host::build_plan(L, q2k, plan, (hipStream_t)stream));
}

int msa_forward(const msa_bf16 *Q, const msa_bf16 *Kw, const msa_bf16 *Vt, const msa_layout *layout,
                const void *plan, float scale, msa_bf16 *O, float *LSE, void *stream) {
  LayoutArgs L;
  int rc = check_layout(layout, &L);
  if (!rc) rc = check_ptrs({Q, Kw, Vt, plan, O, LSE});
  if (rc) return rc;
  if (!scale_ok(scale)) return MSA_ERR_SHAPE;
  if ((rc = check_device())) return rc;
  hipError_t e = mark(0, (hipStream_t)stream);
  if (e == hipSuccess) e = host::forward(Q, Kw, Vt, L, plan, scale, O, LSE, (hipStream_t)stream);
  if (e == hipSuccess) e = mark(1, (hipStream_t)stream);
  return launch_rc(e);
}

int msa_backward_preprocess(const msa_bf16 *O, const msa_bf16 *dO, int32_t num_tokens,
                            float *delta, void *stream) {
  int rc = check_ptrs({O, dO, delta});
  if (rc) return rc;
  if (num_tokens < 1) return MSA_ERR_SHAPE;
  if ((rc = check_device())) return rc;
  return launch_rc(host::preprocess(O, dO, num_tokens, delta, (hipStream_t)stream));
}

int msa_build_tasks(const msa_layout *layout, const int32_t *row_ptr, const int32_t *cols,
                    const int32_t *q2k, int32_t grid, void *tasks, size_t tasks_bytes, void *stream) {
  LayoutArgs L;
  int rc = check_layout(layout, &L);
  if (!rc) rc = check_ptrs({row_ptr, cols, q2k, tasks});
  if (rc) return rc;
  if (grid < 1 || grid > MSA_MAX_GRID) return MSA_ERR_GRID;
  if (tasks_bytes < msa_tasks_bytes(layout, grid)) return MSA_ERR_SCRATCH;
  if ((rc = check_device())) return rc;
  return launch_rc(host::build_tasks(L, row_ptr, cols, q2k, grid, tasks, (hipStream_t)stream));
}

int msa_backward(const msa_bf16 *Q, const msa_bf16 *Kw, const msa_bf16 *Vw, const msa_bf16 *Kt,
                 const msa_bf16 *dO, const float *LSE, const float *delta, const int32_t *q2k,
                 const void *plan, const void *tasks, int32_t grid, const msa_layout *layout,
                 float scale, int dq_accum_mode, msa_bf16 *dQ, msa_bf16 *dK, msa_bf16 *dV,
                 void *scratch, size_t scratch_bytes, void *stream) {
  LayoutArgs L;
  int rc = check_layout(layout, &L);
  if (!rc) rc = check_ptrs({Q, Kw, Vw, Kt, dO, LSE, delta, q2k, plan, tasks, dQ, dK, dV, scratch});
  if (rc) return rc;
  if (grid < 1 || grid > MSA_MAX_GRID) return MSA_ERR_GRID;
  if (dq_accum_mode != MSA_DQ_ACCUM_FP32 && dq_accum_mode != MSA_DQ_ACCUM_BF16X2 &&
      dq_accum_mode != MSA_DQ_RECOMPUTE && dq_accum_mode != MSA_DQ_STORED &&
      dq_accum_mode != MSA_DQ_ACCUM_F16X2)
    return MSA_ERR_MODE;
  if (!scale_ok(scale)) return MSA_ERR_SHAPE;
  if (scratch_bytes < msa_bwd_scratch_bytes(layout, dq_accum_mode)) return MSA_ERR_SCRATCH;
  if ((rc = check_device())) return rc;
  hipStream_t s = (hipStream_t)stream;
  const bool pool = dq_accum_mode == MSA_DQ_ACCUM_FP32 || dq_accum_mode == MSA_DQ_ACCUM_BF16X2 ||
                    dq_accum_mode == MSA_DQ_ACCUM_F16X2;
  const bool stored = dq_accum_mode == MSA_DQ_STORED;
  size_t elem = dq_accum_mode == MSA_DQ_ACCUM_FP32 ? 4 : (pool ? 2 : 0);
  size_t dq_bytes = round16((size_t)L.T * MSA_NUM_Q_HEADS * MSA_HEAD_DIM * elem);
  size_t kv_bytes = round16((size_t)L.W * MSA_NUM_KV_HEADS * MSA_HEAD_DIM * 4);
  // scratch: [dQ pool (pooled modes)] [dK pool] [dV pool] [dS tiles (stored mode)]; only
  // the pools are zeroed (every stored tile is written before it is read)
  char *sc = (char *)scratch;
  float *dk_pool = (float *)(sc + dq_bytes);
  float *dv_pool = (float *)(sc + dq_bytes + kv_bytes);
  void *ds = stored ? (void *)(sc + dq_bytes + 2 * kv_bytes) : nullptr;
  hipError_t e = host::fill_u32(sc, (dq_bytes + 2 * kv_bytes) / 4, 0u, s);
  if (e == hipSuccess) e = mark(2, s);
  if (e == hipSuccess) {
    if (pool)
      e = host::backward_main(Q, Kw, Vw, dO, LSE, delta, tasks, L, grid, scale, dq_accum_mode, sc,
                              dk_pool, dv_pool, s);
    else if (stored)
      e = host::backward_kv2(Q, Kw, Vw, dO, LSE, delta, tasks, L, grid, scale, dk_pool, dv_pool, ds, s);
    else
      e = host::backward_kv(Q, Kw, Vw, dO, LSE, delta, tasks, L, grid, scale, dk_pool, dv_pool, s);
  }
  if (e == hipSuccess) e = mark(3, s);
  if (!pool) {
    if (e == hipSuccess) e = mark(4, s);
    if (e == hipSuccess)
      e = stored ? host::backward_dqs(ds, Kt, q2k, L, plan, scale, dQ, s)
                 : host::backward_dq(Q, dO, Kw, Vw, Kt, LSE, delta, q2k, L, plan, scale, dQ, s);
    if (e == hipSuccess) e = mark(5, s);
  }
  if (e == hipSuccess)
    e = host::finalize(pool ? sc : nullptr, dq_accum_mode, dk_pool, dv_pool, L, dQ, dK, dV, s);
  return launch_rc(e);
}

void msa_set_timing_events(void *const *events) {
  for (int k = 0; k < MSA_TIMING_EVENTS; ++k) t_events[k] = events ? (hipEvent_t)events[k] : nullptr;
}

const char *msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_NULL: return "null pointer";
    case MSA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MSA_ERR_SHAPE: return "inconsistent sizes or layout";
    case MSA_ERR_SCRATCH: return "buffer smaller than its size query";
    case MSA_ERR_MODE: return "unknown dQ accumulation mode";
    case MSA_ERR_GRID: return "grid out of range";
    case MSA_ERR_LAUNCH: return "kernel launch failed";
    case MSA_ERR_DEVICE: return "no gfx950 device current";
    default: return "unknown status";
  }
}

}  // extern "C"
