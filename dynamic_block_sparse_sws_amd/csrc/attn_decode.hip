// Block-sparse single-token decode attention (blog page "Scout Before You
// Attend", section 5: the same block selection for every decode step; section
// 8.3: decode is bound by reading the KV cache).
//
// Split-KV over the union list of each (sequence, KV head): every workgroup
// takes a chunk of 1024 key tokens (1024/B union blocks) and computes, for all
// query heads of the group that kept each block, the partial softmax state
// (max, sum, weighted V sum).  K rows are read once, as 16-byte vectors, and
// dotted with every kept head's query; V rows are read once and accumulated for
// every kept head.  A second kernel merges the partial states of the chunks
// with the usual log-sum-exp rescaling.
#include "sws_common.h"

namespace sws {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSplitTokens = 1024;
constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 4;

// Sum over the TPL consecutive lanes that share a token row (TPL in {8, 16}),
// with DPP lane permutes: swap neighbours, swap pairs, mirror within 8, mirror
// within 16.
template <int TPL>
__device__ __forceinline__ float token_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  if (TPL == 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  return v;
}

// Eight elements of a K or V row as loaded (bf16: one 16-byte vector, fp32:
// two), converted to fp32 only where they are used.
template <typename T> struct Row8;
template <> struct Row8<uint16_t> {
  uint4 r;
  __device__ __forceinline__ void load(const uint16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float* o) const {
    o[0] = bf16_bits_to_f32(r.x & 0xffffu); o[1] = bf16_bits_to_f32(r.x >> 16);
    o[2] = bf16_bits_to_f32(r.y & 0xffffu); o[3] = bf16_bits_to_f32(r.y >> 16);
    o[4] = bf16_bits_to_f32(r.z & 0xffffu); o[5] = bf16_bits_to_f32(r.z >> 16);
    o[6] = bf16_bits_to_f32(r.w & 0xffffu); o[7] = bf16_bits_to_f32(r.w >> 16);
  }
};
template <> struct Row8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void get(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

// A query head's 8 features of this lane, and its dot product with a K row:
// bf16 pairs through v_dot2_f32_bf16 (exact products, fp32 sums), fp32 with
// plain fused multiply-adds.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <typename T> struct QVec;
template <> struct QVec<uint16_t> {
  uint4 r;
  __device__ __forceinline__ void load(const uint16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { r = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ float dot(const Row8<uint16_t>& k) const {
    float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.r.x),
                                              __builtin_bit_cast(bf16x2_t, r.x), 0.f, false);
    float b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.r.y),
                                              __builtin_bit_cast(bf16x2_t, r.y), 0.f, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.r.z),
                                        __builtin_bit_cast(bf16x2_t, r.z), a, false);
    b = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.r.w),
                                        __builtin_bit_cast(bf16x2_t, r.w), b, false);
    return a + b;
  }
};
template <> struct QVec<float> {
  float v[8];
  __device__ __forceinline__ void load(const float* p) { load8_f32(p, v); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = 0.f;
  }
  __device__ __forceinline__ float dot(const Row8<float>& k) const {
    float kf[8];
    k.get(kf);
    float a = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) a += v[x] * kf[x];
    return a;
  }
};

__device__ __forceinline__ float exp2_or_zero(float x) {
  return x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x);
}

// One split: the workgroup's chunk of the union list is cut into batches of
// TPB tokens (a batch never straddles a block); wave w takes batches w, w + 4,
// ...  Within a batch a lane holds UNR token rows (TPL lanes per row, 8
// features per lane), all K and V loads of the batch are issued before any is
// used, and each row group of the wave keeps its own online-softmax state
// (max, sum, weighted V sum) for up to four query heads at a time.  The row
// groups are merged with cross-lane exchanges, the waves through LDS, and the
// split's state is written for the combine kernel.
template <typename T, int D, int BLK, int GMAX, int UNR>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, int max_ctx, int hq, int hkv,
    const int32_t* __restrict__ uidx, const int32_t* __restrict__ ucnt,
    const uint32_t* __restrict__ umask, int uwidth, int max_splits, float scale_log2,
    float* __restrict__ ws_ml, float* __restrict__ ws_acc) {
  constexpr int BPS = kSplitTokens / BLK;      // blocks per split
  constexpr int TPL = D / 8;                   // lanes per token row
  constexpr int RPW = 64 / TPL;                // token rows per wave-wide load
  constexpr int TPB = RPW * UNR;               // tokens per wave batch
  constexpr int NWV = kDecThreads / 64;
  constexpr int HC = GMAX < 4 ? GMAX : 4;      // query heads per pass
  static_assert(BLK % TPB == 0, "a batch must stay inside one block");
  __shared__ float wm[NWV][HC], wl[NWV][HC];
  __shared__ float wacc[NWV][HC][D];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int seq = blockIdx.z;
  const int G = hq / hkv;
  const int ctx = ctx_len[seq];
  const int nblk = uidx ? ucnt[seq * hkv + g] : (ctx + BLK - 1) / BLK;
  const int e0 = split * BPS;
  if (e0 >= nblk) return;
  const int ntok = (min(nblk, e0 + BPS) - e0) * BLK;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ch = lane % TPL;           // feature chunk (8 features)
  const int slot = lane / TPL;         // row group of the wave
  const int64_t rstride = (int64_t)hkv * D;
  const T* kb = kc + ((int64_t)seq * max_ctx) * rstride + (int64_t)g * D + ch * 8;
  const T* vb = vc + ((int64_t)seq * max_ctx) * rstride + (int64_t)g * D + ch * 8;
  const int32_t* ul = uidx ? uidx + ((int64_t)seq * hkv + g) * uwidth : nullptr;
  const uint32_t* um = umask ? umask + ((int64_t)seq * hkv + g) * uwidth : nullptr;

  for (int h0 = 0; h0 < G; h0 += HC) {
    QVec<T> qv[HC];
    float acc[HC][8], m[HC], l[HC];
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
      if (h0 + hh < G) qv[hh].load(q + ((int64_t)seq * hq + g * G + h0 + hh) * D + ch * 8);
      else qv[hh].zero();
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[hh][x] = 0.f;
      m[hh] = -INFINITY;
      l[hh] = 0.f;
    }
    for (int tb = wave * TPB; tb < ntok; tb += NWV * TPB) {
      const int e = e0 + tb / BLK;
      const int blk = ul ? ul[e] : e;
      const uint32_t mk = um ? um[e] : 0xffffffffu;
      const int r0 = blk * BLK + tb % BLK + slot;      // this lane's first cache row
      Row8<T> kr[UNR], vr[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int64_t r = min(r0 + u * RPW, ctx - 1);  // rows past ctx are masked below
        kr[u].load(kb + r * rstride);
        vr[u].load(vb + r * rstride);
      }
      float sc[UNR][HC];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const bool ok = r0 + u * RPW < ctx;
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
          const float part = token_sum<TPL>(qv[hh].dot(kr[u]));
          sc[u][hh] = (ok && ((mk >> (h0 + hh)) & 1u)) ? part * scale_log2 : -INFINITY;
        }
      }
#pragma unroll
      for (int hh = 0; hh < HC; ++hh) {
        float bm = sc[0][hh];
#pragma unroll
        for (int u = 1; u < UNR; ++u) bm = fmaxf(bm, sc[u][hh]);
        const float mn = fmaxf(m[hh], bm);
        const float alpha = m[hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hh] - mn);
        m[hh] = mn;
        l[hh] *= alpha;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[hh][x] *= alpha;
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float vf[8];
        vr[u].get(vf);
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
          const float p = exp2_or_zero(sc[u][hh] == -INFINITY ? -INFINITY : sc[u][hh] - m[hh]);
          l[hh] += p;
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[hh][x] += p * vf[x];
        }
      }
    }
    // merge the row groups of the wave (lanes TPL, 2 TPL, ... apart)
#pragma unroll
    for (int off = TPL; off < 64; off <<= 1) {
#pragma unroll
      for (int hh = 0; hh < HC; ++hh) {
        const float mo = __shfl_xor(m[hh], off);
        const float lo = __shfl_xor(l[hh], off);
        const float mn = fmaxf(m[hh], mo);
        const float a1 = m[hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hh] - mn);
        const float a2 = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
        l[hh] = l[hh] * a1 + lo * a2;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float ao = __shfl_xor(acc[hh][x], off);
          acc[hh][x] = acc[hh][x] * a1 + ao * a2;
        }
        m[hh] = mn;
      }
    }
    if (slot == 0) {
#pragma unroll
      for (int hh = 0; hh < HC; ++hh) {
#pragma unroll
        for (int x = 0; x < 8; ++x) wacc[wave][hh][ch * 8 + x] = acc[hh][x];
        if (ch == 0) {
          wm[wave][hh] = m[hh];
          wl[wave][hh] = l[hh];
        }
      }
    }
    __syncthreads();
    // merge the waves and write the split state of heads h0 .. h0 + HC - 1
    for (int e = tid; e < HC * D; e += kDecThreads) {
      const int hh = e / D, dd = e % D;
      if (h0 + hh >= G) continue;
      float M = wm[0][hh];
#pragma unroll
      for (int w = 1; w < NWV; ++w) M = fmaxf(M, wm[w][hh]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        const float f = wm[w][hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wm[w][hh] - M);
        L += f * wl[w][hh];
        A += f * wacc[w][hh][dd];
      }
      const int64_t row = ((int64_t)seq * hq + g * G + h0 + hh) * max_splits + split;
      ws_acc[row * D + dd] = A;
      if (dd == 0) {
        ws_ml[row * 2 + 0] = M;
        ws_ml[row * 2 + 1] = L;
      }
    }
    __syncthreads();
  }
}

// Merge of the split states of one (sequence, query head): the weights
// exp2(m_s - max m) go to LDS once, then each thread sums one feature over the
// splits with independent loads.
constexpr int kMaxSplits = 1024;

template <typename T, int D, int BLK>
__global__ __launch_bounds__(D) void decode_combine_kernel(
    const int32_t* __restrict__ ctx_len, int hq, int hkv, const int32_t* __restrict__ uidx,
    const int32_t* __restrict__ ucnt, int max_splits, const float* __restrict__ ws_ml,
    const float* __restrict__ ws_acc, T* __restrict__ out, float* __restrict__ lse) {
  constexpr int BPS = kSplitTokens / BLK;
  constexpr int NW = D / 64;
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[NW];
  __shared__ float s_M, s_L;
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int G = hq / hkv;
  const int g = h / G;
  const int ctx = ctx_len[seq];
  const int nblk = uidx ? ucnt[seq * hkv + g] : (ctx + BLK - 1) / BLK;
  const int ns = (nblk + BPS - 1) / BPS;
  const int64_t row0 = ((int64_t)seq * hq + h) * max_splits;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  float m = -INFINITY;
  for (int si = t; si < ns; si += D) {
    const float v = ws_ml[(row0 + si) * 2];
    wgt[si] = v;
    m = fmaxf(m, v);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (t == 0) {
    float M = red[0];
    for (int w = 1; w < NW; ++w) M = fmaxf(M, red[w]);
    s_M = M;
  }
  __syncthreads();
  const float M = s_M;
  float lsum = 0.f;
  for (int si = t; si < ns; si += D) {
    const float mv = wgt[si];
    const float f = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
    wgt[si] = f;
    lsum += f * ws_ml[(row0 + si) * 2 + 1];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
  __syncthreads();
  if (lane == 0) red[wave] = lsum;
  __syncthreads();
  if (t == 0) {
    float L = 0.f;
    for (int w = 0; w < NW; ++w) L += red[w];
    s_L = L;
  }
  __syncthreads();
  float a = 0.f;
#pragma unroll 8
  for (int si = 0; si < ns; ++si) a += wgt[si] * ws_acc[(row0 + si) * D + t];
  const float L = s_L;
  const float o = a / L;
  T* op = out + ((int64_t)seq * hq + h) * D + t;
  if constexpr (sizeof(T) == 2) *reinterpret_cast<uint16_t*>(op) = (uint16_t)f32_to_bf16_bits(o);
  else *op = o;
  if (lse && t == 0) lse[(int64_t)seq * hq + h] = (M + log2f(L)) * kLn2;
}

template <typename T, int D, int BLK, int GMAX>
hipError_t run_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* ctx_len, int n_seqs, int max_ctx, int hq, int hkv,
                      const int32_t* uidx, const int32_t* ucnt, const uint32_t* umask,
                      int uwidth, float scale, void* out, float* lse, void* ws,
                      hipStream_t st) {
  constexpr int BPS = kSplitTokens / BLK;
  const int max_splits = (uwidth + BPS - 1) / BPS;
  float* ws_ml = static_cast<float*>(ws);
  float* ws_acc = ws_ml + (size_t)n_seqs * hq * max_splits * 2;
  dim3 grid(max_splits, hkv, n_seqs);
  hipLaunchKernelGGL((decode_split_kernel<T, D, BLK, GMAX, kDecUnroll>), grid, dim3(kDecThreads), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(k_cache),
                     static_cast<const T*>(v_cache), ctx_len, max_ctx, hq, hkv, uidx, ucnt,
                     umask, uwidth, max_splits, scale * kLog2e, ws_ml, ws_acc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D, BLK>), dim3(hq, n_seqs), dim3(D), 0, st,
                     ctx_len, hq, hkv, uidx, ucnt, max_splits, ws_ml, ws_acc,
                     static_cast<T*>(out), lse);
  return hipGetLastError();
}

template <typename T, int D, int BLK>
hipError_t pick_g(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* ctx_len, int n_seqs, int max_ctx, int hq, int hkv,
                  const int32_t* uidx, const int32_t* ucnt, const uint32_t* umask, int uwidth,
                  float scale, void* out, float* lse, void* ws, hipStream_t st) {
  const int G = hq / hkv;
  if (G <= 1)
    return run_decode<T, D, BLK, 1>(q, k_cache, v_cache, ctx_len, n_seqs, max_ctx, hq, hkv, uidx,
                                    ucnt, umask, uwidth, scale, out, lse, ws, st);
  if (G <= 4)
    return run_decode<T, D, BLK, 4>(q, k_cache, v_cache, ctx_len, n_seqs, max_ctx, hq, hkv, uidx,
                                    ucnt, umask, uwidth, scale, out, lse, ws, st);
  if (G <= 8)
    return run_decode<T, D, BLK, 8>(q, k_cache, v_cache, ctx_len, n_seqs, max_ctx, hq, hkv, uidx,
                                    ucnt, umask, uwidth, scale, out, lse, ws, st);
  return run_decode<T, D, BLK, 16>(q, k_cache, v_cache, ctx_len, n_seqs, max_ctx, hq, hkv, uidx,
                                   ucnt, umask, uwidth, scale, out, lse, ws, st);
}

}  // namespace

size_t decode_workspace_bytes(int n_seqs, int hq, int hkv, int d, int B, int union_width) {
  (void)hkv;
  const int bps = kSplitTokens / B;
  const size_t max_splits = (size_t)((union_width + bps - 1) / bps);
  return (size_t)n_seqs * hq * max_splits * (size_t)(d + 2) * sizeof(float);
}

hipError_t launch_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                              int dtype, const int32_t* ctx_len, int n_seqs, int max_ctx, int hq,
                              int hkv, int d, int B, const int32_t* union_idx,
                              const int32_t* union_cnt, const uint32_t* union_mask,
                              int union_width, float scale, void* out, float* lse, void* ws,
                              hipStream_t st) {
  if (n_seqs == 0) return hipSuccess;
#define SWS_DEC(T, D, BLK)                                                                     \
  return pick_g<T, D, BLK>(q, k_cache, v_cache, ctx_len, n_seqs, max_ctx, hq, hkv, union_idx, \
                           union_cnt, union_mask, union_width, scale, out, lse, ws, st)
  if (dtype == SWS_BF16) {
    if (d == 128 && B == 64) SWS_DEC(uint16_t, 128, 64);
    if (d == 128 && B == 128) SWS_DEC(uint16_t, 128, 128);
    if (d == 64 && B == 64) SWS_DEC(uint16_t, 64, 64);
    SWS_DEC(uint16_t, 64, 128);
  }
  if (d == 128 && B == 64) SWS_DEC(float, 128, 64);
  if (d == 128 && B == 128) SWS_DEC(float, 128, 128);
  if (d == 64 && B == 64) SWS_DEC(float, 64, 64);
  SWS_DEC(float, 64, 128);
#undef SWS_DEC
}

}  // namespace sws
