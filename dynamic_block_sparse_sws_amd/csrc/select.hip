// Top-tau key-block selection per query block (blog page "Scout Before You
// Attend", section 4: the tau best blocks from the query block's row of the
// walk state; the diagonal block is always kept).
//
// One wavefront owns one row.  Scores become order-preserving unsigned keys
// (-0 folded onto +0 first), held in registers, 64 candidates per register.
// The tau-th largest key T is found by a radix search over its four bytes
// (a per-wave LDS histogram and a wave scan per byte).  Then every key > T
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

constexpr int kLoadBatch = 16;   // row values loaded per batch (registers in flight)

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// The tau-th largest key T of the candidates key[] (candidate e * 64 + lane,
// n of them, 0 if absent) and the number of keys equal to T to keep, by a
// radix search, one byte at a time from the top:
// each pass histograms the next byte of the keys that match the bytes fixed
// so far into a 256-bin LDS histogram owned by this wave (`hist`), and a
// wave scan over the bins, largest first, finds the byte value where the
// count of larger keys reaches tau.  Wave-local: LDS operations of one wave
// complete in order, so no barrier is needed.
template <int E>
__device__ __forceinline__ void threshold_radix(const uint32_t (&key)[E], int n, int tau,
                                                uint32_t* hist, uint32_t& T, int& need_eq) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0;
  int remaining = tau;                          // keys still to take at or below the prefix
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e * 64 < n) {
        const uint32_t k = key[e];
        const bool match = e * 64 + lane < n && (pass == 0 || (k >> (shift + 8)) == prefix);
        if (match) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
    }
    // lane l holds bins 255 - 4 l .. 252 - 4 l, largest first
    const uint4 h4 = reinterpret_cast<const uint4*>(hist)[63 - lane];
    const int s_l = (int)(h4.x + h4.y + h4.z + h4.w);
    int incl = s_l;
    {
      // inclusive prefix over lanes (row shifts, then row broadcasts)
      int x = incl;
      incl += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false); x = incl;
      incl += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false); x = incl;
      incl += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false); x = incl;
      incl += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false); x = incl;
      incl += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false); x = incl;
      incl += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
    }
    const int excl = incl - s_l;
    // (remaining == 0: nothing more to take, lane 0 and bin 255)
    const uint64_t hit = __ballot(incl >= remaining && (excl < remaining || lane == 0));
    const int L = (int)__builtin_ctzll(hit);    // the lane whose 4 bins hold the answer
    // within that lane: bins in descending order w, z, y, x
    int above = excl, digit = 0;
    {
      const int need = remaining;
      const int bw = (int)h4.w, bz = (int)h4.z, by = (int)h4.y;
      const int base = 255 - 4 * lane;          // bin of h4.w
      if (above + bw >= need) digit = base;
      else if (above + bw + bz >= need) { above += bw; digit = base - 1; }
      else if (above + bw + bz + by >= need) { above += bw + bz; digit = base - 2; }
      else { above += bw + bz + by; digit = base - 3; }
    }
    digit = __builtin_amdgcn_readlane(digit, L);
    above = __builtin_amdgcn_readlane(above, L);
    remaining -= above;
    prefix = (prefix << 8) | (uint32_t)digit;
  }
  T = prefix;
  need_eq = remaining;
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
  __shared__ __attribute__((aligned(16))) uint32_t hist[4][256];
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
  // loads go out (up to) 16 registers at a time, all before any is used
  // (indices past the candidates are clamped to the last one and masked
  // below; i > tau >= 0 here)
  uint32_t key[E];
#pragma unroll
  for (int e0 = 0; e0 < E; e0 += kLoadBatch) {
    constexpr int NB = E < kLoadBatch ? E : kLoadBatch;
    float v[NB];
#pragma unroll
    for (int e = 0; e < NB; ++e) v[e] = row[min((e0 + e) * 64 + lane, i - 1)];
    for (int hh = 1; hh < GS; ++hh) {
#pragma unroll
      for (int e = 0; e < NB; ++e) v[e] += row[hh * hstride + min((e0 + e) * 64 + lane, i - 1)];
    }
#pragma unroll
    for (int e = 0; e < NB; ++e) key[e0 + e] = ((e0 + e) * 64 + lane < i) ? order_key(v[e]) : 0u;
  }
  uint32_t T;
  int need;
  threshold_radix<E>(key, i, tau, hist[threadIdx.x >> 6], T, need);
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
  __shared__ __attribute__((aligned(16))) uint32_t hist[NT / 64][256];
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
      // loads go out 16 registers at a time, all before any is used (indices
      // past the candidates are clamped to the last one and masked below)
      uint32_t key[E];
#pragma unroll
      for (int e0 = 0; e0 < E; e0 += kLoadBatch) {
        float v[kLoadBatch];
#pragma unroll
        for (int e = 0; e < kLoadBatch; ++e) v[e] = row[min((e0 + e) * 64 + lane, c - 1)];
        for (int hh = 1; hh < nsum; ++hh) {
#pragma unroll
          for (int e = 0; e < kLoadBatch; ++e)
            v[e] += row[(int64_t)hh * b_max + min((e0 + e) * 64 + lane, c - 1)];
        }
#pragma unroll
        for (int e = 0; e < kLoadBatch; ++e)
          key[e0 + e] = ((e0 + e) * 64 + lane < c) ? order_key(v[e]) : 0u;
      }
      uint32_t T;
      int need;
      threshold_radix<E>(key, c, tau, hist[w], T, need);
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
  else if (max_blocks <= 2048)
    hipLaunchKernelGGL((select_kernel<32>), grid, dim3(256), 0, st, R, hq, cu_blocks, n_seqs,
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
