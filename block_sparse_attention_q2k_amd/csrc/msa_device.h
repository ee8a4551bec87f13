// msa_device.h -- device-side helpers shared by the libmsa kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/msa.h"

namespace msa {

constexpr int kH = MSA_NUM_Q_HEADS;         // 64 query heads
constexpr int kHKV = MSA_NUM_KV_HEADS;      // 4 KV heads
constexpr int kHI = MSA_NUM_INDEX_HEADS;    // 4 index heads
constexpr int kD = MSA_HEAD_DIM;            // 128
constexpr int kBlk = MSA_BLOCK;             // 128 keys per block
constexpr int kTopk = MSA_TOPK;             // 16 slots
constexpr int kHPI = kH / kHI;              // 16 query heads per index head
constexpr int kTileQ = MSA_TILE_QUERIES;    // 8 queries per backward task row
constexpr int kFwdGroup = MSA_FWD_GROUP;    // queries per forward work item
constexpr int kTasksHeaderWords = 64;
constexpr int kPlanHeaderWords = 16;
constexpr int kPlanMaxList = kFwdGroup * kTopk;  // walk-list capacity per plan item
constexpr float kLog2e = 1.4426950408889634f;
// Workspace K/V copies are stored per (KV head kv, workspace block gb) as 16384 bf16
// (32 KB) at element offset (kv * NB + gb) * kFragBlock, in the order the MFMA operands
// are loaded, so that every 16-byte-per-lane load of a wave reads 1 KB of contiguous
// memory:
//   row fragments (K, V as 32x32x16 A operands, 4 waves x 32 keys): element (key k,
//     dim d) at ((k/32 * 8 + d/16) * 64 + (d/8 % 2) * 32 + k%32) * 8 + d%8
//   transposed fragments (K^T, V^T as 16x16x32 A operands, 16-dim slices): element
//     (key k, dim d) at ((d/16 * 4 + k/32) * 64 + (k/8 % 4) * 16 + d%16) * 8 + k%8
constexpr int kFragBlock = kBlk * kD;
// Stored dS tiles (MSA_DQ_STORED): the dS values of one (query t, index head i, member
// slot j) -- 16 heads x 128 keys of the block q2k[i][t][j] -- as 2048 bf16 at tile
// (t * 4 + i) * 16 + j, element (key, head) at ds_key_swz(key) * 16 + ds_head_pos(head).
// key' = key ^ (key / 8 % 2) * 4: within every 16 keys the second 8 swap their 4-key
// quarters, which spreads the dQ kernel's transposing LDS reads over all banks.  Head
// positions swap bits 2 and 3 (order 0-3, 8-11, 4-7, 12-15): the 8 heads one lane of
// the KV-parallel kernel holds for a key are then 16 contiguous bytes.
__host__ __device__ inline int ds_key_swz(int key) { return key ^ (((key >> 3) & 1) << 2); }
__host__ __device__ inline int ds_head_pos(int h) { return (h & 3) | ((h & 4) << 1) | ((h & 8) >> 1); }
__host__ __device__ inline int frag_row_off(int k, int d) {
  return (((k >> 5) * 8 + (d >> 4)) * 64 + ((d >> 3) & 1) * 32 + (k & 31)) * 8 + (d & 7);
}
__host__ __device__ inline int frag_t_off(int k, int d) {
  return (((d >> 4) * 4 + (k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (d & 15)) * 8 + (k & 7);
}
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Largest d with a[d] <= x over a sorted array a[0..n] (a[0] <= x assumed).
__device__ inline int upper_index(const int32_t *a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Round-to-nearest-even fp32 -> bf16 (the gfx950 conversion instruction rounds RNE).
__device__ inline uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two values in one v_cvt_pk_bf16_f32 (round to nearest even), lo in bits 0..15.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// Sum of the two bf16 halves of a plus c (v_dot2c_f32_bf16 against (1, 1)).
__device__ inline float sum_bf16x2(uint32_t a, float c) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), one, c, false);
}
__device__ inline float bf2f(uint16_t u) { return __builtin_bit_cast(float, (uint32_t)u << 16); }

// v_mfma_f32_16x16x32_bf16: C[16x16] += A[16x32] * B[32x16].
// Lane l: A row l%16, k = 8*(l/16)+0..7; B column l%16, same k; C column l%16,
// rows 4*(l/16)+0..3.
__device__ inline f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8(l/32)+0..7], B[8(l/32)+0..7][l%32];
// C register r of lane l is C[8(r/4) + 4(l/32) + r%4][l%32].
__device__ inline f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS access helpers.  `lds` is the byte offset inside the kernel's LDS block.
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) char lds_char;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j supplies the address of
// 4 consecutive 16-bit values in[j][0..3]; lane l receives in[4e + l/4][l%4], e=0..3.
// With lane j pointing at X[k0 + j/4][c0 + 4*(j%4)], lane l gets X[k0 + e][c0 + l].
__device__ inline bf16x4 lds_read_tr(const lds_char *base, uint32_t byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(base + byte_off));
}

__device__ inline bf16x8 cat8(const bf16x4 &a, const bf16x4 &b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// 16-byte-chunk swizzle for a [rows][256 B] bf16 tile: chunk c of row r is stored at
// chunk c ^ (r & 15), so 16 lanes reading one chunk of 16 consecutive rows hit 16
// different chunks.
__device__ inline uint32_t swz(int row, int byte_in_row) {
  return (uint32_t)(row * 256 + ((((byte_in_row >> 4) ^ (row & 15)) << 4) | (byte_in_row & 15)));
}

}  // namespace msa
