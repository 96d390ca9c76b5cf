// Small-World Sketching (blog page "Scout Before You Attend", section 3.1
// block means and section 3.2 subsampled randomized Hadamard projection).
//
// One workgroup owns one block of one sequence and a slice of up to 2048/d
// heads.  The block's token rows of those heads are contiguous in the
// token-major layout, so the HBM pass is a coalesced stream of 16-byte loads
// (one 8-element vector per thread per token).  Partial sums live in
// registers, are combined through LDS, divided by the block's token count,
// sign-flipped, transformed by an in-LDS Walsh-Hadamard butterfly (log2 d
// stages) and subsampled to the k requested columns, scaled by 1/sqrt(k).
#include "sws_common.h"

namespace sws {
namespace {

constexpr int kThreads = 256;
constexpr int kSliceElems = 2048;  // heads * d handled by one workgroup

// In-LDS unnormalised Walsh-Hadamard transform of nh rows of length D.
template <int D>
__device__ __forceinline__ void fwht_lds(float* f, int nh) {
  const int pairs = nh * (D / 2);
#pragma unroll
  for (int h = 1; h < D; h <<= 1) {
    for (int p = threadIdx.x; p < pairs; p += kThreads) {
      const int row = p / (D / 2);
      const int q = p % (D / 2);
      const int lo = (q / h) * 2 * h + (q % h);
      float* r = f + row * D;
      const float a = r[lo];
      const float b = r[lo + h];
      r[lo] = a + b;
      r[lo + h] = a - b;
    }
    __syncthreads();
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void sketch_kernel(
    const T* __restrict__ x, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int n_seqs, int total_blocks, int n_heads, int hpw,
    int tr_log2, int B, int k, const int8_t* __restrict__ signs,
    const int32_t* __restrict__ cols, float* __restrict__ out, int64_t ld_head,
    float* __restrict__ sum_out, float inv_sqrt_k) {
  __shared__ float red[kSliceElems];
  __shared__ float f[kSliceElems];

  const int g = blockIdx.x;
  const int h0 = blockIdx.y * hpw;
  const int nh = min(hpw, n_heads - h0);
  const int s = seq_of_block(cu_blocks, n_seqs, g);
  const int i = g - cu_blocks[s];
  const int t0 = cu_seqlens[s] + i * B;
  const int c = min(B, cu_seqlens[s + 1] - t0);

  const int tr = 1 << tr_log2;
  const int tid = threadIdx.x;
  const int col = (tid & (tr - 1)) * 8;
  const int tg = tid >> tr_log2;
  const int n_tg = kThreads >> tr_log2;
  const int width = nh * D;

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (col < width) {
    const int64_t stride = (int64_t)n_heads * D;
    const T* p = x + ((int64_t)t0 * n_heads + h0) * D + col;
#pragma unroll 4
    for (int t = tg; t < c; t += n_tg) {
      float v[8];
      load8_f32(p + (int64_t)t * stride, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tg * (tr * 8) + col + e] = acc[e];
  __syncthreads();

  const float inv_c = 1.0f / (float)c;
  for (int e = tid; e < width; e += kThreads) {
    float sum = 0.f;
    for (int q = 0; q < n_tg; ++q) sum += red[q * (tr * 8) + e];
    const int hh = e / D;
    const int r = e % D;
    if (sum_out) sum_out[((int64_t)(h0 + hh) * total_blocks + g) * D + r] = sum;
    f[e] = (sum * inv_c) * (float)signs[r];
  }
  __syncthreads();
  fwht_lds<D>(f, nh);

  for (int e = tid; e < nh * k; e += kThreads) {
    const int hh = e / k;
    const int cc = e % k;
    out[(int64_t)(h0 + hh) * ld_head + (int64_t)g * k + cc] = f[hh * D + cols[cc]] * inv_sqrt_k;
  }
}

// One tensor of new-token rows to append: x [n_seqs][n_heads][D], its running
// block sums and its sketch cache; `slices` workgroups per sequence cover its
// heads, hpw at a time.
template <typename T>
struct AppendSet {
  const T* x;
  float* run_sum;
  float* cache;
  int n_heads, hpw, slices;
};

// Workgroup (s, y) appends the new token of sequence s for one slice of heads
// of set a0 (y < a0.slices) or a1 (the rest), so the query and key rows of a
// decode step can share one launch.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void sketch_append_kernel(
    AppendSet<T> a0, AppendSet<T> a1, const int32_t* __restrict__ pos, int B, int k,
    const int8_t* __restrict__ signs, const int32_t* __restrict__ cols, int b_max,
    float inv_sqrt_k) {
  __shared__ float f[kSliceElems];
  const int s = blockIdx.x;
  const bool second = (int)blockIdx.y >= a0.slices;
  const AppendSet<T> a = second ? a1 : a0;
  const int h0 = (second ? blockIdx.y - a0.slices : blockIdx.y) * a.hpw;
  const int nh = min(a.hpw, a.n_heads - h0);
  const int p = pos[s];
  const int c = p / B;
  const int off = p - c * B;
  const float inv_cnt = 1.0f / (float)(off + 1);
  const int width = nh * D;
  const int col = threadIdx.x * 8;
  if (col < width) {
    const int64_t base = ((int64_t)s * a.n_heads + h0) * D + col;
    float v[8];
    load8_f32(a.x + base, v);
    float* rs = a.run_sum + base;
    // the running sums are loaded whether or not the token opens a block, so
    // the load does not wait for pos (an opening token then drops them)
    const float4 r0 = reinterpret_cast<const float4*>(rs)[0];
    const float4 r1 = reinterpret_cast<const float4*>(rs)[1];
    const float old[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sum = (off == 0) ? v[e] : old[e] + v[e];
      rs[e] = sum;
      const int r = (col + e) % D;
      f[col + e] = (sum * inv_cnt) * (float)signs[r];
    }
  }
  __syncthreads();
  fwht_lds<D>(f, nh);
  for (int e = threadIdx.x; e < nh * k; e += kThreads) {
    const int hh = e / k;
    const int cc = e % k;
    a.cache[(((int64_t)s * a.n_heads + h0 + hh) * b_max + c) * k + cc] =
        f[hh * D + cols[cc]] * inv_sqrt_k;
  }
}

template <typename T, int D>
hipError_t run_sketch(const void* x, const int32_t* cu_seqlens, const int32_t* cu_blocks,
                      int n_seqs, int total_blocks, int n_heads, int B, int k,
                      const int8_t* signs, const int32_t* cols, float* out, int64_t ld_head,
                      float* sum_out, hipStream_t st) {
  const int hpw = min(n_heads, kSliceElems / D);
  int tr = 1, tr_log2 = 0;
  while (tr * 8 < hpw * D) { tr <<= 1; ++tr_log2; }
  dim3 grid(total_blocks, (n_heads + hpw - 1) / hpw);
  hipLaunchKernelGGL((sketch_kernel<T, D>), grid, dim3(kThreads), 0, st,
                     static_cast<const T*>(x), cu_seqlens, cu_blocks, n_seqs, total_blocks,
                     n_heads, hpw, tr_log2, B, k, signs, cols, out, ld_head, sum_out,
                     1.0f / sqrtf((float)k));
  return hipGetLastError();
}

template <typename T, int D>
AppendSet<T> append_set(const void* x, int n_heads, float* run_sum, float* cache) {
  const int hpw = min(n_heads, kSliceElems / D);
  return AppendSet<T>{static_cast<const T*>(x), run_sum, cache, n_heads, hpw,
                      n_heads > 0 ? (n_heads + hpw - 1) / hpw : 0};
}

// Appends set 0 and, when its head count is positive, set 1 in one launch.
template <typename T, int D>
hipError_t run_append(const void* x0, int nh0, float* rs0, float* c0, const void* x1, int nh1,
                      float* rs1, float* c1, const int32_t* pos, int n_seqs, int B, int k,
                      const int8_t* signs, const int32_t* cols, int b_max, hipStream_t st) {
  const AppendSet<T> a0 = append_set<T, D>(x0, nh0, rs0, c0);
  const AppendSet<T> a1 = append_set<T, D>(x1, nh1, rs1, c1);
  dim3 grid(n_seqs, a0.slices + a1.slices);
  hipLaunchKernelGGL((sketch_append_kernel<T, D>), grid, dim3(kThreads), 0, st, a0, a1, pos, B,
                     k, signs, cols, b_max, 1.0f / sqrtf((float)k));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sketch(const void* x, int dtype, const int32_t* cu_seqlens,
                         const int32_t* cu_blocks, int n_seqs, int total_blocks, int n_heads,
                         int d, int B, int k, const int8_t* signs, const int32_t* cols,
                         float* sketch_out, int64_t ld_head, float* sum_out, hipStream_t st) {
  if (total_blocks == 0) return hipSuccess;
  if (dtype == SWS_BF16) {
    if (d == 128)
      return run_sketch<uint16_t, 128>(x, cu_seqlens, cu_blocks, n_seqs, total_blocks, n_heads,
                                       B, k, signs, cols, sketch_out, ld_head, sum_out, st);
    return run_sketch<uint16_t, 64>(x, cu_seqlens, cu_blocks, n_seqs, total_blocks, n_heads, B,
                                    k, signs, cols, sketch_out, ld_head, sum_out, st);
  }
  if (d == 128)
    return run_sketch<float, 128>(x, cu_seqlens, cu_blocks, n_seqs, total_blocks, n_heads, B,
                                  k, signs, cols, sketch_out, ld_head, sum_out, st);
  return run_sketch<float, 64>(x, cu_seqlens, cu_blocks, n_seqs, total_blocks, n_heads, B, k,
                               signs, cols, sketch_out, ld_head, sum_out, st);
}

hipError_t launch_sketch_append(const void* x0, int nh0, float* rs0, float* c0, const void* x1,
                                int nh1, float* rs1, float* c1, int dtype, const int32_t* pos,
                                int n_seqs, int d, int B, int k, const int8_t* signs,
                                const int32_t* cols, int b_max, hipStream_t st) {
  if (n_seqs == 0) return hipSuccess;
#define SWS_APPEND(T, D)                                                                       \
  return run_append<T, D>(x0, nh0, rs0, c0, x1, nh1, rs1, c1, pos, n_seqs, B, k, signs, cols,  \
                          b_max, st)
  if (dtype == SWS_BF16) {
    if (d == 128) SWS_APPEND(uint16_t, 128);
    SWS_APPEND(uint16_t, 64);
  }
  if (d == 128) SWS_APPEND(float, 128);
  SWS_APPEND(float, 64);
#undef SWS_APPEND
}

}  // namespace sws
