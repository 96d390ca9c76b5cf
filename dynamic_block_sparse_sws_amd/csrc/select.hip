// Top-tau key-block selection per query block (blog page "Scout Before You
// Attend", section 4: the tau best blocks from the query block's row of the
// walk state; the diagonal block is always kept).
//
// One wavefront owns one row.  Scores become order-preserving unsigned keys
// (-0 folded onto +0 first), held in registers, 64 candidates per register.
// The tau-th largest key T is found by a most-significant-bit-first search,
// each step counting keys >= candidate with wave ballots.  Then every key > T
// is kept, plus the lowest-index keys equal to T until tau are kept; the
// kept indices are compacted in ascending order with ballot prefix counts, so
// the result is exactly the (score descending, index ascending) top tau.
#include "sws_common.h"

namespace sws {
namespace {

__device__ __forceinline__ uint32_t order_key(float x) {
  const float y = (x == 0.0f) ? 0.0f : x;   // -0 -> +0
  const uint32_t u = __float_as_uint(y);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// Selection flags for row values row[0 .. n) (n candidates), keeping tau of
// them.  key[] holds the keys of candidates e * 64 + lane (0 if absent).
// Returns the threshold and the number of threshold ties to keep.
template <int E>
__device__ __forceinline__ void threshold(const uint32_t (&key)[E], int n, int tau,
                                          uint32_t& T, int& need_eq) {
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e * 64 < n) c += popc64(__ballot(key[e] >= cand));
    }
    if (c >= tau) t = cand;
  }
  int gt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e * 64 < n) gt += popc64(__ballot(key[e] > t));
  }
  T = t;
  need_eq = tau - gt;
}

// flags: SWS_SELECT_DENSE keeps every block <= i; SWS_SELECT_ROW_TAU gives
// row i the budget floor(rho (i + 1) / 100) instead of floor(rho b / 100);
// SWS_SELECT_GROUP scores a row by the fp32 sum, in ascending head order, of
// the rows of the GS query heads of a KV group, and writes the shared list to
// each of them.  blockIdx.y is the query head, or the KV group with
// SWS_SELECT_GROUP.
template <int E>
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ R, int hq,
                                                     const int32_t* __restrict__ cu_blocks,
                                                     int n_seqs, int total_blocks, int rho,
                                                     int flags, int GS, int width,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ cnt) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h0 = blockIdx.y * GS;
  const int seq = blockIdx.z;
  const int b0 = cu_blocks[seq];
  const int b = cu_blocks[seq + 1] - b0;
  if (i >= b) return;
  const int gb = b0 + i;
  const int tau = (flags & SWS_SELECT_ROW_TAU) ? (int)(((int64_t)rho * (i + 1)) / 100)
                                               : (int)(((int64_t)rho * b) / 100);
  if ((flags & SWS_SELECT_DENSE) || i <= tau) {
    for (int hh = 0; hh < GS; ++hh) {
      int32_t* out = idx + ((int64_t)(h0 + hh) * total_blocks + gb) * width;
      for (int m = lane; m <= i; m += 64) out[m] = m;
      if (lane == 0) cnt[(int64_t)(h0 + hh) * total_blocks + gb] = i + 1;
    }
    return;
  }
  const float* row = R + walk_seq_offset(cu_blocks, seq, hq) + ((int64_t)h0 * b + i) * b;
  const int64_t hstride = (int64_t)b * b;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int m = e * 64 + lane;
    float v = 0.f;
    if (m < i) {
      v = row[m];
      for (int hh = 1; hh < GS; ++hh) v += row[hh * hstride + m];
    }
    key[e] = (m < i) ? order_key(v) : 0u;
  }
  uint32_t T;
  int need;
  threshold<E>(key, i, tau, T, need);
  int base = 0, eq_seen = 0;
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e * 64 < i) {
      const int m = e * 64 + lane;
      const bool valid = m < i;
      const bool eq = valid && key[e] == T;
      const uint64_t eqm = __ballot(eq);
      const bool sel = valid && (key[e] > T || (eq && eq_seen + popc64(eqm & lt) < need));
      eq_seen += popc64(eqm);
      const uint64_t sm = __ballot(sel);
      if (sel)
        for (int hh = 0; hh < GS; ++hh)
          idx[((int64_t)(h0 + hh) * total_blocks + gb) * width + base + popc64(sm & lt)] = m;
      base += popc64(sm);
    }
  }
  if (lane == 0) {
    for (int hh = 0; hh < GS; ++hh) {
      idx[((int64_t)(h0 + hh) * total_blocks + gb) * width + tau] = i;
      cnt[(int64_t)(h0 + hh) * total_blocks + gb] = tau + 1;
    }
  }
}

// Decode: the open block c of each sequence; one workgroup per (sequence, KV
// group), one wave per query head of the group; union through an LDS mask.
constexpr int kRowBmax = 4096;

// E: key registers per lane (rows up to 64 * E blocks); NT: 64 * (largest
// group size the instance serves), so small groups get the larger register
// budget and keep every key in registers.
template <int E, int NT>
__global__ __launch_bounds__(NT) void select_row_kernel(
    const float* __restrict__ r, int hq, int hkv, const int32_t* __restrict__ cur_block,
    int b_max, int rho, int flags, int width, int32_t* __restrict__ idx,
    int32_t* __restrict__ cnt, int32_t* __restrict__ union_idx,
    int32_t* __restrict__ union_cnt, uint32_t* __restrict__ union_mask, int union_width) {
  __shared__ uint32_t umask[kRowBmax];
  const int g = blockIdx.x;
  const int seq = blockIdx.y;
  const int G = hq / hkv;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nthreads = blockDim.x;
  const int c = cur_block[seq];
  const int b = c + 1;
  const int tau = (int)(((int64_t)rho * b) / 100);   // = the per-row budget of row c
  const bool dense = (flags & SWS_SELECT_DENSE) != 0;
  const bool group = (flags & SWS_SELECT_GROUP) != 0;
  const uint32_t all = (G >= 32) ? 0xffffffffu : ((1u << G) - 1u);
  for (int m = threadIdx.x; m < b; m += nthreads) umask[m] = (dense || m == c) ? all : 0u;
  __syncthreads();
  if (w < G && !dense) {
    const int h = g * G + w;
    int32_t* out = idx ? idx + ((int64_t)seq * hq + h) * width : nullptr;
    if (c <= tau) {
      for (int m = lane; m < c; m += 64) atomicOr(&umask[m], 1u << w);
      if (out) for (int m = lane; m <= c; m += 64) out[m] = m;
      if (out && lane == 0) cnt[(int64_t)seq * hq + h] = c + 1;
    } else {
      // with SWS_SELECT_GROUP every wave scores the row by the group's fp32
      // sum (heads in ascending order), so all heads keep the same blocks
      const float* row = r + ((int64_t)seq * hq + (group ? g * G : h)) * b_max;
      const int nsum = group ? G : 1;
      uint32_t key[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int m = e * 64 + lane;
        float v = 0.f;
        if (m < c) {
          v = row[m];
          for (int hh = 1; hh < nsum; ++hh) v += row[(int64_t)hh * b_max + m];
        }
        key[e] = (m < c) ? order_key(v) : 0u;
      }
      uint32_t T;
      int need;
      threshold<E>(key, c, tau, T, need);
      int base = 0, eq_seen = 0;
      const uint64_t lt = lanemask_lt();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (e * 64 < c) {
          const int m = e * 64 + lane;
          const bool valid = m < c;
          const bool eq = valid && key[e] == T;
          const uint64_t eqm = __ballot(eq);
          const bool sel = valid && (key[e] > T || (eq && eq_seen + popc64(eqm & lt) < need));
          eq_seen += popc64(eqm);
          const uint64_t sm = __ballot(sel);
          if (sel) {
            atomicOr(&umask[m], 1u << w);
            if (out) out[base + popc64(sm & lt)] = m;
          }
          base += popc64(sm);
        }
      }
      if (out && lane == 0) {
        out[tau] = c;
        cnt[(int64_t)seq * hq + h] = tau + 1;
      }
    }
  } else if (w < G && dense && idx) {
    const int h = g * G + w;
    int32_t* out = idx + ((int64_t)seq * hq + h) * width;
    for (int m = lane; m <= c; m += 64) out[m] = m;
    if (lane == 0) cnt[(int64_t)seq * hq + h] = c + 1;
  }
  __syncthreads();
  if (w == 0) {
    int32_t* uo = union_idx + ((int64_t)seq * hkv + g) * union_width;
    uint32_t* um = union_mask + ((int64_t)seq * hkv + g) * union_width;
    const uint64_t lt = lanemask_lt();
    int base = 0;
    for (int m0 = 0; m0 < b; m0 += 64) {
      const int m = m0 + lane;
      const uint32_t mk = (m < b) ? umask[m] : 0u;
      const uint64_t bm = __ballot(mk != 0u);
      if (mk) {
        const int p = base + popc64(bm & lt);
        uo[p] = m;
        um[p] = mk;
      }
      base += popc64(bm);
    }
    if (lane == 0) union_cnt[(int64_t)seq * hkv + g] = base;
  }
}

}  // namespace

hipError_t launch_select(const float* R, int hq, int hkv, const int32_t* cu_blocks, int n_seqs,
                         int total_blocks, int max_blocks, int rho, int flags, int width,
                         int32_t* idx, int32_t* cnt, hipStream_t st) {
  if (total_blocks == 0 || max_blocks == 0) return hipSuccess;
  const int GS = (flags & SWS_SELECT_GROUP) ? hq / hkv : 1;
  dim3 grid((max_blocks + 3) / 4, hq / GS, n_seqs);
  if (max_blocks <= 256)
    hipLaunchKernelGGL((select_kernel<4>), grid, dim3(256), 0, st, R, hq, cu_blocks, n_seqs,
                       total_blocks, rho, flags, GS, width, idx, cnt);
  else if (max_blocks <= 1024)
    hipLaunchKernelGGL((select_kernel<16>), grid, dim3(256), 0, st, R, hq, cu_blocks, n_seqs,
                       total_blocks, rho, flags, GS, width, idx, cnt);
  else
    hipLaunchKernelGGL((select_kernel<64>), grid, dim3(256), 0, st, R, hq, cu_blocks, n_seqs,
                       total_blocks, rho, flags, GS, width, idx, cnt);
  return hipGetLastError();
}

hipError_t launch_select_row(const float* r, int hq, int hkv, int n_seqs,
                             const int32_t* cur_block, int b_max, int rho, int flags, int width,
                             int32_t* idx, int32_t* cnt, int32_t* union_idx, int32_t* union_cnt,
                             uint32_t* union_mask, int union_width, hipStream_t st) {
  if (n_seqs == 0) return hipSuccess;
  const int G = hq / hkv;
  dim3 grid(hkv, n_seqs);
  dim3 block(64 * G);
#define SWS_SEL_ROW(E, NT)                                                                     \
  hipLaunchKernelGGL((select_row_kernel<E, NT>), grid, block, 0, st, r, hq, hkv, cur_block,   \
                     b_max, rho, flags, width, idx, cnt, union_idx, union_cnt, union_mask,     \
                     union_width)
#define SWS_SEL_ROW_NT(E)           \
  do {                              \
    if (G <= 4) SWS_SEL_ROW(E, 256);  \
    else if (G <= 8) SWS_SEL_ROW(E, 512); \
    else SWS_SEL_ROW(E, 1024);      \
  } while (0)
  if (b_max <= 1024) SWS_SEL_ROW_NT(16);
  else if (b_max <= 2048) SWS_SEL_ROW_NT(32);
  else SWS_SEL_ROW_NT(64);
#undef SWS_SEL_ROW_NT
#undef SWS_SEL_ROW
  return hipGetLastError();
}

}  // namespace sws
