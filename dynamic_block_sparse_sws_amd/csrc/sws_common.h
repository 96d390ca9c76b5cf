// Internal helpers shared by the HIP kernels of the Sketch&Walk library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sws.h"

namespace sws {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// bf16 <-> fp32.  bf16 is the upper half of an fp32 bit pattern; rounding to
// bf16 is round-to-nearest-even on the discarded 16 bits (NaN kept quiet).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// two floats -> packed bf16 pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Loads of 8 consecutive elements converted to fp32.
__device__ __forceinline__ void load8_f32(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8_f32(const uint16_t* p, float* o) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  o[0] = bf16_bits_to_f32(a.x & 0xffffu); o[1] = bf16_bits_to_f32(a.x >> 16);
  o[2] = bf16_bits_to_f32(a.y & 0xffffu); o[3] = bf16_bits_to_f32(a.y >> 16);
  o[4] = bf16_bits_to_f32(a.z & 0xffffu); o[5] = bf16_bits_to_f32(a.z >> 16);
  o[6] = bf16_bits_to_f32(a.w & 0xffffu); o[7] = bf16_bits_to_f32(a.w >> 16);
}

// Find the sequence holding global block g (linear scan; batches are small).
__device__ __forceinline__ int seq_of_block(const int32_t* cu_blocks, int n_seqs, int g) {
  int s = 0;
  while (s + 1 < n_seqs && cu_blocks[s + 1] <= g) ++s;
  return s;
}

// Dynamic range of the walk state: after every hop, entries smaller in
// magnitude than this fraction of their row's largest magnitude are zero.
// Without a floor the walk over many layers keeps row entries hundreds of
// binary orders of magnitude below the row maximum that grow back layers
// later, so its value would depend on the number format's exponent range;
// 2^-64 keeps every retained value, and its products with the scores, well
// inside the normal fp32 range.
constexpr float kWalkFloor = 0x1p-64f;

// Offset (in elements) of sequence s in the packed walk-state layout.
__device__ __forceinline__ int64_t walk_seq_offset(const int32_t* cu_blocks, int s, int hq) {
  int64_t off = 0;
  for (int t = 0; t < s; ++t) {
    const int64_t bt = cu_blocks[t + 1] - cu_blocks[t];
    off += bt * bt;
  }
  return off * hq;
}

}  // namespace sws

// Internal launchers (defined in the kernel sources, called by sws_api.hip
// after validation).  Each returns the hipError_t of its launches.
namespace sws {
hipError_t launch_sketch(const void* x, int dtype, const int32_t* cu_seqlens,
                         const int32_t* cu_blocks, int n_seqs, int total_blocks, int n_heads,
                         int d, int B, int k, const int8_t* signs, const int32_t* cols,
                         float* sketch_out, int64_t ld_head, float* sum_out, hipStream_t st);
// Appends the new-token rows of one tensor (x0, nh0 heads) and, if nh1 > 0, of
// a second one, in one launch.
hipError_t launch_sketch_append(const void* x0, int nh0, float* rs0, float* c0, const void* x1,
                                int nh1, float* rs1, float* c1, int dtype, const int32_t* pos,
                                int n_seqs, int d, int B, int k, const int8_t* signs,
                                const int32_t* cols, int b_max, hipStream_t st);
hipError_t launch_walk(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                       const int32_t* cu_blocks, int n_seqs, int total_blocks, int max_blocks,
                       int s, const float* R_prev, float* R_out, hipStream_t st);
hipError_t launch_walk_row(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                           int n_seqs, const int32_t* cur_block, int b_max, int s,
                           const float* r_prev, float* r_out, hipStream_t st);
hipError_t launch_walk_variant(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                               const int32_t* cu_blocks, int n_seqs, int total_blocks,
                               int max_blocks, int s, int mode, const float* R_prev,
                               float* R_out, int64_t walk_numel, void* ws, hipStream_t st);
size_t walk_variant_workspace_bytes(int64_t walk_numel);
hipError_t launch_walk_row_variant(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                                   int n_seqs, const int32_t* cur_block, int b_max, int s,
                                   int mode, const float* r_prev, float* r_out, hipStream_t st);
hipError_t launch_select(const float* R, int hq, int hkv, const int32_t* cu_blocks, int n_seqs,
                         int total_blocks, int max_blocks, int rho, int flags, int width,
                         int32_t* idx, int32_t* cnt, hipStream_t st);
hipError_t launch_select_row(const float* r, int hq, int hkv, int n_seqs,
                             const int32_t* cur_block, int b_max, int rho, int flags, int width,
                             int32_t* idx, int32_t* cnt, int32_t* union_idx, int32_t* union_cnt,
                             uint32_t* union_mask, int union_width, hipStream_t st);
hipError_t launch_attn_prefill(const void* q, const void* k, const void* v, int dtype,
                               const int32_t* cu_seqlens, const int32_t* cu_blocks, int n_seqs,
                               int total_blocks, int max_blocks, int hq, int hkv, int d, int B,
                               const int32_t* idx, const int32_t* cnt, int width, float scale,
                               void* out, float* lse, void* ws, hipStream_t st);
hipError_t launch_attn_prefill_f32(const void* q, const void* k, const void* v,
                                   const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                   int n_seqs, int total_blocks, int hq, int hkv, int d, int B,
                                   const int32_t* idx, const int32_t* cnt, int width,
                                   float scale, void* out, float* lse, hipStream_t st);
hipError_t launch_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                              int dtype, bool head_major, const int32_t* ctx_len, int n_seqs,
                              int max_ctx, int hq, int hkv, int d, int B, const int32_t* union_idx,
                              const int32_t* union_cnt, const uint32_t* union_mask,
                              int union_width, float scale, void* out, float* lse, void* ws,
                              hipStream_t st);
hipError_t launch_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                    int kv_dtype, bool head_major, float k_scale, float v_scale,
                                    const int32_t* block_table, int table_width,
                                    int num_pages, const int32_t* ctx_len, int n_seqs, int hq,
                                    int hkv, int d, int B, const int32_t* union_idx,
                                    const int32_t* union_cnt, const uint32_t* union_mask,
                                    int union_width, float scale, void* out, float* lse,
                                    void* ws, hipStream_t st);
size_t decode_workspace_bytes(int n_seqs, int hq, int hkv, int d, int B, int union_width);
}  // namespace sws
