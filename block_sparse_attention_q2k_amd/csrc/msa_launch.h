// msa_launch.h -- host-side launch interface between the C ABI and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

struct LayoutArgs {
  int ndocs, T, W, NB;
  const int32_t *cu, *cu_ws;
};

struct PlanView {
  int32_t *header, *items, *len, *lists, *gstart, *ginfo, *cost, *end;
};

struct TaskView {
  int32_t *header, *cta, *meta, *qrows, *qpos, *qtile, *len, *tile_off;
  size_t rmax;
};

namespace host {
hipError_t fill_u32(void *p, size_t n, uint32_t v, hipStream_t s);
hipError_t index_select(const void *IQ, const void *IK, const LayoutArgs &L, int32_t *q2k, hipStream_t s);
hipError_t align_kv(const void *K, const void *V, const LayoutArgs &L, void *Kw, void *Vw,
                    void *Kt, void *Vt, hipStream_t s);
hipError_t build_csr(const int32_t *q2k, const LayoutArgs &L, int32_t *row_ptr, int32_t *cols,
                     int32_t *status, int32_t *counter, hipStream_t s);
size_t plan_gmax(const LayoutArgs &L);
size_t plan_bytes(const LayoutArgs &L);
PlanView plan_view(const LayoutArgs &L, void *plan);
hipError_t build_plan(const LayoutArgs &L, const int32_t *q2k, void *plan, hipStream_t s);
size_t tasks_rmax(const LayoutArgs &L);
size_t tasks_meta_offset_words(int grid);
size_t tasks_bytes(const LayoutArgs &L, int grid);
TaskView task_view(const LayoutArgs &L, int grid, void *tasks);
hipError_t build_tasks(const LayoutArgs &L, const int32_t *row_ptr, const int32_t *cols,
                       const int32_t *q2k, int grid, void *tasks, hipStream_t s);
hipError_t preprocess(const void *O, const void *dO, int T, float *delta, hipStream_t s);
hipError_t finalize(const void *dq_pool, int mode, const float *dk_pool, const float *dv_pool,
                    const LayoutArgs &L, void *dQ, void *dK, void *dV, hipStream_t s);
hipError_t forward(const void *Q, const void *Kw, const void *Vt, const LayoutArgs &L, const void *plan, float scale, void *O, float *LSE,
                   hipStream_t s);
hipError_t backward_main(const void *Q, const void *Kw, const void *Vw, const void *dO,
                         const float *LSE, const float *delta, const void *tasks,
                         const LayoutArgs &L, int grid, float scale, int mode, void *dq_pool,
                         float *dk_pool, float *dv_pool, hipStream_t s);
// dK/dV for MSA_DQ_RECOMPUTE (the dQ kernel recomputes S and dP).
hipError_t backward_kv(const void *Q, const void *Kw, const void *Vw, const void *dO,
                       const float *LSE, const float *delta, const void *tasks,
                       const LayoutArgs &L, int grid, float scale, float *dk_pool, float *dv_pool,
                       hipStream_t s);
// The same products for MSA_DQ_STORED (dS stored) with score and accumulate waves.
hipError_t backward_kv2(const void *Q, const void *Kw, const void *Vw, const void *dO, const float *LSE,
                        const float *delta, const void *tasks, const LayoutArgs &L, int grid, float scale,
                        float *dk_pool, float *dv_pool, void *dS, hipStream_t s);
hipError_t backward_dqs(const void *dS, const void *Kt, const int32_t *q2k, const LayoutArgs &L,
                        const void *plan, float scale, void *dQ, hipStream_t s);
hipError_t backward_dq(const void *Q, const void *dO, const void *Kw, const void *Vw, const void *Kt,
                       const float *LSE, const float *delta, const int32_t *q2k, const LayoutArgs &L,
                       const void *plan, float scale, void *dQ, hipStream_t s);
}  // namespace host
}  // namespace msa
