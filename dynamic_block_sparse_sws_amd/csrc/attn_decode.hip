// Block-sparse single-token decode attention (blog page "Scout Before You
// Attend", section 5: the same block selection for every decode step; section
// 8.3: decode is bound by reading the KV cache).
//
// Split-KV over the union list of each (sequence, KV head): every workgroup
// takes a chunk of 512 key tokens (512/B union blocks) and computes, for all
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
constexpr int kSplitTokens = 512;
constexpr int kDecThreads = 256;

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

template <typename T, int D, int BLK, int GMAX>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, int max_ctx, int hq, int hkv,
    const int32_t* __restrict__ uidx, const int32_t* __restrict__ ucnt,
    const uint32_t* __restrict__ umask, int uwidth, int max_splits, float scale_log2,
    float* __restrict__ ws_ml, float* __restrict__ ws_acc) {
  constexpr int BPS = kSplitTokens / BLK;      // blocks per split
  constexpr int TPL = D / 8;                   // lanes per token row
  constexpr int SLOTS = kDecThreads / TPL;     // token rows per pass
  constexpr int UNR = 8;                       // token rows in flight per lane
  __shared__ float sc[GMAX][kSplitTokens];
  __shared__ float sm[GMAX], sl[GMAX];
  __shared__ float red[kDecThreads / 64][GMAX][D];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int seq = blockIdx.z;
  const int G = hq / hkv;
  const int ctx = ctx_len[seq];
  const int nblk = uidx ? ucnt[seq * hkv + g] : (ctx + BLK - 1) / BLK;
  const int e0 = split * BPS;
  if (e0 >= nblk) return;
  const int e1 = min(nblk, e0 + BPS);
  const int tid = threadIdx.x;
  const int ch = tid % TPL;            // feature chunk (8 features)
  const int slot = tid / TPL;          // token slot

  float qv[GMAX][8];
#pragma unroll
  for (int hh = 0; hh < GMAX; ++hh) {
    if (hh < G) load8_f32(q + ((int64_t)seq * hq + g * G + hh) * D + ch * 8, qv[hh]);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[hh][e] = 0.f;
  }
  const int64_t rstride = (int64_t)hkv * D;
  const T* kb = kc + ((int64_t)seq * max_ctx) * rstride + (int64_t)g * D + ch * 8;
  const T* vb = vc + ((int64_t)seq * max_ctx) * rstride + (int64_t)g * D + ch * 8;
  const int32_t* ul = uidx ? uidx + ((int64_t)seq * hkv + g) * uwidth : nullptr;
  const uint32_t* um = umask ? umask + ((int64_t)seq * hkv + g) * uwidth : nullptr;
  const uint32_t all = (1u << G) - 1u;
  const int ntok = (e1 - e0) * BLK;

  // Chunk token tt -> cache row; rows past the chunk map to ctx (masked).
  auto token_row = [&](int tt) -> int {
    if (tt >= ntok) return ctx;
    const int e = e0 + tt / BLK;
    const int blk = ul ? ul[e] : e;
    return blk * BLK + (tt % BLK);
  };

  // ---- phase 1: scores of every token of the chunk for every head ----
  // UNR rows are loaded before any is used; rows at or past ctx read row
  // ctx - 1 (in bounds) and are masked.
  for (int base = 0; base < ntok; base += UNR * SLOTS) {
    float kv[UNR][8];
    int tok[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      tok[u] = token_row(base + u * SLOTS + slot);
      load8_f32(kb + (int64_t)min(tok[u], ctx - 1) * rstride, kv[u]);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int tt = base + u * SLOTS + slot;
      const uint32_t mk = (tt < ntok) ? (um ? um[e0 + tt / BLK] : all) : 0u;
#pragma unroll
      for (int hh = 0; hh < GMAX; ++hh) {
        if (hh < G) {
          float part = 0.f;
#pragma unroll
          for (int x = 0; x < 8; ++x) part += qv[hh][x] * kv[u][x];
          part = token_sum<TPL>(part);
          if (ch == 0 && tt < ntok)
            sc[hh][tt] = (tok[u] < ctx && ((mk >> hh) & 1u)) ? part * scale_log2 : -INFINITY;
        }
      }
    }
  }
  __syncthreads();
  // ---- phase 2: per-head max and exponentials ----
  const int wave = tid >> 6, lane = tid & 63;
  for (int hh = wave; hh < G; hh += kDecThreads / 64) {
    float mx = -INFINITY;
    for (int tt = lane; tt < ntok; tt += 64) mx = fmaxf(mx, sc[hh][tt]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float sum = 0.f;
    for (int tt = lane; tt < ntok; tt += 64) {
      const float p = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[hh][tt] - mx);
      sc[hh][tt] = p;
      sum += p;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) { sm[hh] = mx; sl[hh] = sum; }
  }
  __syncthreads();
  // ---- phase 3: weighted V sums (masked rows carry weight 0) ----
  float acc[GMAX][8];
#pragma unroll
  for (int hh = 0; hh < GMAX; ++hh)
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[hh][x] = 0.f;
  for (int base = 0; base < ntok; base += UNR * SLOTS) {
    float vv[UNR][8];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = token_row(base + u * SLOTS + slot);
      load8_f32(vb + (int64_t)min(t, ctx - 1) * rstride, vv[u]);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int tt = base + u * SLOTS + slot;
      if (tt < ntok) {
#pragma unroll
        for (int hh = 0; hh < GMAX; ++hh) {
          if (hh < G) {
            const float p = sc[hh][tt];
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[hh][x] += p * vv[u][x];
          }
        }
      }
    }
  }
  // reduce over the token slots: within a wave (lanes TPL apart), then waves
#pragma unroll
  for (int hh = 0; hh < GMAX; ++hh) {
    if (hh < G) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        float a = acc[hh][x];
#pragma unroll
        for (int off = TPL; off < 64; off <<= 1) a += __shfl_xor(a, off);
        acc[hh][x] = a;
      }
    }
  }
  if (lane < TPL) {
#pragma unroll
    for (int hh = 0; hh < GMAX; ++hh)
      if (hh < G)
#pragma unroll
        for (int x = 0; x < 8; ++x) red[wave][hh][ch * 8 + x] = acc[hh][x];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += kDecThreads) {
    const int hh = e / D, dd = e % D;
    float a = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kDecThreads / 64; ++w2) a += red[w2][hh][dd];
    const int64_t row = ((int64_t)seq * hq + g * G + hh) * max_splits + split;
    ws_acc[row * D + dd] = a;
    if (dd == 0) {
      ws_ml[row * 2 + 0] = sm[hh];
      ws_ml[row * 2 + 1] = sl[hh];
    }
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
  hipLaunchKernelGGL((decode_split_kernel<T, D, BLK, GMAX>), grid, dim3(kDecThreads), 0, st,
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
