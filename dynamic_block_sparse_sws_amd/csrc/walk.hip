// Walk state (blog page "Scout Before You Attend", section 4):
//   R^l = rownorm(R^(l-1) M^s),  M[i][j] = qs_i . ks_j / sqrt(k) for j <= i.
//
// Rows of R are independent, and one hop of a row is the product of a row
// vector with the lower-triangular rank-k matrix M, which factorises into a
// suffix scan:
//   y[m] = ks_m . S_m / sqrt(k),   S_m = sum_{j >= m} x[j] qs_j.
// So a hop costs 2 b k multiply-adds per row instead of b^2, and the walk of
// all b rows costs s b^2 k per head instead of forming M^s.
//
// Prefill: a workgroup owns a chunk of rows of one head and runs all s hops
// on them, streaming the rows through LDS tile by tile from the last column
// down (the scan order), overwriting each tile in place in R_out.  Lanes of a
// row split the k components of S and combine their partial dot products with
// cross-lane shuffles.  Every hop rescales its rows by their largest
// magnitude (positive row scaling commutes with the right-multiplication, so
// only the final division is visible), which keeps s * layers hops in fp32.
//
// Decode: one workgroup per (sequence, query head) walks the single row of
// the open block; the j range is cut into segments, one per lane group, with
// the segment's sketch rows held in registers for all s hops, and the suffix
// carry across segments comes from a wave scan plus an LDS scan of the wave
// totals.
#include "sws_common.h"

namespace sws {
namespace {

template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  // sum over the LPR consecutive lanes of a row (LPR in {2, 4, 8})
  v += __shfl_xor(v, 1);
  if (LPR >= 4) v += __shfl_xor(v, 2);
  if (LPR >= 8) v += __shfl_xor(v, 4);
  return v;
}

// Same sum with DPP lane permutes (no LDS round trip): swap neighbours, swap
// pairs within a quad, then mirror the two quads of an 8-lane half row.
template <int LPR>
__device__ __forceinline__ float group_sum_dpp(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  if (LPR >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  if (LPR >= 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  return v;
}

constexpr int kWalkThreads = 256;
constexpr int kTileJ = 64;

template <int KP>
struct WalkTile {
  static constexpr int LPR = KP / 8;                  // lanes per row
  static constexpr int ROWS = kWalkThreads / LPR;     // rows per workgroup
  static constexpr int XPT = ROWS * kTileJ / kWalkThreads;   // X tile values per thread
  static constexpr int SPT = kTileJ * KP / kWalkThreads;     // sketch values per thread
};

template <int KP>
__global__ __launch_bounds__(kWalkThreads) __attribute__((amdgpu_waves_per_eu(2)))
void walk_kernel(
    const float* __restrict__ q_sk, const float* __restrict__ k_sk, int hq, int hkv, int k,
    const int32_t* __restrict__ cu_blocks, int n_seqs, int total_blocks, int s,
    const float* R_prev, float* R_out, float inv_sqrt_k) {
  using WT = WalkTile<KP>;
  constexpr int LPR = WT::LPR, ROWS = WT::ROWS, XPT = WT::XPT, SPT = WT::SPT;
  __shared__ __attribute__((aligned(16))) float sq[2][kTileJ][KP + 4];
  __shared__ __attribute__((aligned(16))) float sk[2][kTileJ][KP + 4];
  __shared__ float sx[2][ROWS][kTileJ + 1];
  __shared__ float smax[ROWS];

  const int seq = blockIdx.z;
  const int h = blockIdx.y;
  const int b0 = cu_blocks[seq];
  const int b = cu_blocks[seq + 1] - b0;
  const int i0 = blockIdx.x * ROWS;
  if (i0 >= b) return;
  const int64_t roff = walk_seq_offset(cu_blocks, seq, hq) + (int64_t)h * b * b;
  float* Rh = R_out + roff;
  const float* Rp = R_prev ? R_prev + roff : nullptr;
  const int grp = hq / hkv;
  const float* qs = q_sk + ((int64_t)h * total_blocks + b0) * k;
  const float* ks = k_sk + ((int64_t)(h / grp) * total_blocks + b0) * k;

  const int tid = threadIdx.x;
  const int r = tid / LPR;
  const int part = tid % LPR;
  const int jmax = min(b, i0 + ROWS) - 1;
  const int top_tile = (jmax / kTileJ) * kTileJ;

  // prefetch registers for one tile (X values and sketch rows).  Thread tid
  // covers column tid % 64 of rows tid / 64 + (256 / 64) * e of the X tile,
  // and elements tid + 256 * e of the (64 x KP) sketch tiles.
  constexpr int RSTEP = kWalkThreads / kTileJ;
  const int xc = tid % kTileJ;
  const int xr0 = tid / kTileJ;
  float xr[XPT], qr[SPT], kr[SPT];
  auto fetch = [&](int jt, const float* src, bool ident) {
    const int j = jt + xc;
    if (ident) {
#pragma unroll
      for (int e = 0; e < XPT; ++e) xr[e] = (i0 + xr0 + RSTEP * e == j) ? 1.f : 0.f;
    } else if (jt + kTileJ - 1 <= i0 && i0 + ROWS <= b) {
      // tile entirely below the diagonal and inside the matrix: no guards
      const float* p = src + (int64_t)(i0 + xr0) * b + j;
      const int64_t step = (int64_t)RSTEP * b;
#pragma unroll
      for (int e = 0; e < XPT; ++e) xr[e] = p[step * e];
    } else {
#pragma unroll
      for (int e = 0; e < XPT; ++e) {
        const int ii = i0 + xr0 + RSTEP * e;
        xr[e] = (ii < b && j <= ii) ? src[(int64_t)ii * b + j] : 0.f;
      }
    }
    if (k == KP && jt + kTileJ <= b) {
      const float* pq = qs + (int64_t)jt * KP + tid;
      const float* pk = ks + (int64_t)jt * KP + tid;
#pragma unroll
      for (int e = 0; e < SPT; ++e) {
        qr[e] = pq[kWalkThreads * e];
        kr[e] = pk[kWalkThreads * e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < SPT; ++e) {
        const int idx = tid + e * kWalkThreads;
        const int jj = idx / KP, c = idx % KP;
        const bool ok = (jt + jj < b) && (c < k);
        qr[e] = ok ? qs[(int64_t)(jt + jj) * k + c] : 0.f;
        kr[e] = ok ? ks[(int64_t)(jt + jj) * k + c] : 0.f;
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int e = 0; e < XPT; ++e) sx[buf][xr0 + RSTEP * e][xc] = xr[e];
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      const int idx = tid + e * kWalkThreads;
      sq[buf][idx / KP][idx % KP] = qr[e];
      sk[buf][idx / KP][idx % KP] = kr[e];
    }
  };

  // One flat software pipeline over (hop, tile) steps, tiles from the last
  // column down: step st computes tile st while tile st + 1 is fetched.
  const int ntiles = top_tile / kTileJ + 1;
  const int nsteps = s * ntiles;
  float sc = 1.0f;   // rescale of this row's input for the current hop
  float mx = 0.0f;   // largest |y| of this row in the current hop
  float mx_prev = 0.0f;
  float S[8];
  int buf = 0;
  // With a single column tile the next hop re-reads the tile this step writes,
  // so its fetch has to wait for the write-back.
  const bool late = (ntiles == 1);
  auto fetch_step = [&](int st1) {
    const int hop1 = st1 / ntiles;
    const int jt1 = top_tile - (st1 % ntiles) * kTileJ;
    fetch(jt1, hop1 == 0 ? Rp : Rh, hop1 == 0 && Rp == nullptr);
  };
  for (int st = -1; st < nsteps; ++st) {
    // fetch step st + 1 into registers
    if (st + 1 < nsteps && (!late || st < 0)) fetch_step(st + 1);
    if (st >= 0) {
      const int t = st % ntiles;
      const int jt = top_tile - t * kTileJ;
      if (t == 0) {
        // a new hop: reset the scan, rescale by the previous hop's maximum
        if (st > 0) {
          mx_prev = mx;
          sc = (mx > 0.f) ? 1.0f / mx : 1.0f;
        }
        mx = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) S[c] = 0.f;
      }
#pragma unroll 4
      for (int jj = kTileJ - 1; jj >= 0; --jj) {
        const float x = sx[buf][r][jj] * sc;
        const float4 qa = *reinterpret_cast<const float4*>(&sq[buf][jj][part * 8]);
        const float4 qb = *reinterpret_cast<const float4*>(&sq[buf][jj][part * 8 + 4]);
        const float4 ka = *reinterpret_cast<const float4*>(&sk[buf][jj][part * 8]);
        const float4 kb = *reinterpret_cast<const float4*>(&sk[buf][jj][part * 8 + 4]);
        S[0] += x * qa.x; S[1] += x * qa.y; S[2] += x * qa.z; S[3] += x * qa.w;
        S[4] += x * qb.x; S[5] += x * qb.y; S[6] += x * qb.z; S[7] += x * qb.w;
        const float yp = (ka.x * S[0] + ka.y * S[1]) + (ka.z * S[2] + ka.w * S[3]) +
                         ((kb.x * S[4] + kb.y * S[5]) + (kb.z * S[6] + kb.w * S[7]));
        const float y = group_sum_dpp<LPR>(yp) * inv_sqrt_k;
        mx = fmaxf(mx, fabsf(y));
        if (part == 0) sx[buf][r][jj] = y;
      }
      __syncthreads();
      // write the finished tile back (rows are owned by this workgroup)
      for (int e = tid; e < ROWS * kTileJ; e += kWalkThreads) {
        const int rr = e / kTileJ, jj = e % kTileJ;
        const int ii = i0 + rr, j = jt + jj;
        if (ii < b && j <= ii) Rh[(int64_t)ii * b + j] = sx[buf][rr][jj];
      }
      buf ^= 1;
      if (late && st + 1 < nsteps) {
        __syncthreads();
        fetch_step(st + 1);
      }
    }
    if (st + 1 < nsteps) stash(buf);
    __syncthreads();
  }
  (void)mx_prev;
  if (part == 0) smax[r] = mx;
  __syncthreads();
  // final pass: divide by the row maximum, zero the upper triangle
  for (int rr = 0; rr < ROWS; ++rr) {
    const int ii = i0 + rr;
    if (ii >= b) break;
    const float m = smax[rr];
    float* row = Rh + (int64_t)ii * b;
    for (int j = tid; j < b; j += kWalkThreads) {
      float v = 0.f;
      if (j <= ii && m > 0.f) v = row[j] / m;
      row[j] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// decode: one row per (sequence, query head)
// ---------------------------------------------------------------------------
// 512 threads.  Thread t works on component quarter p = t / 128 of the
// sketches (KP / 4 components) and on segment g = t % 128 of the rows j, the
// segments taken in descending j order so that the suffix sum over j becomes
// a prefix scan over the threads of a quarter.  The segment's q and k sketch
// rows stay in registers for all s hops (longer rows stream them from
// memory); each hop is: segment totals, a DPP wave scan plus an LDS scan of
// the quarter's two wave totals, the segment's partial dot products, a sum
// over the four quarters in LDS, and the row maximum.
constexpr int kRowThreads = 512;
constexpr int kRowSeg = 128;        // segments (threads per component quarter)
constexpr int kRowBmax = 4096;      // xs / ypart capacity (largest row)

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts within
// 16-lane rows, then broadcasts of lanes 15 and 31 into the following rows).
__device__ __forceinline__ float wave_prefix_sum(float v) {
  int x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false));  // row_shr:1
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false));  // row_shr:2
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false));  // row_shr:4
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false));  // row_shr:8
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = __builtin_bit_cast(int, v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

template <int KP>
__global__ __launch_bounds__(kRowThreads) void walk_row_kernel(
    const float* __restrict__ q_cache, const float* __restrict__ k_cache, int hq, int hkv,
    int k, const int32_t* __restrict__ cur_block, int b_max, int s, const float* r_prev,
    float* r_out, float inv_sqrt_k) {
  constexpr int CQ = KP / 4;                  // components per quarter
  constexpr int LMAX = 80 / CQ;               // segment rows held in registers
  constexpr int NWAVE = kRowThreads / 64;
  constexpr int WPQ = kRowSeg / 64;           // waves per quarter
  __shared__ float xs[kRowBmax];
  __shared__ float ypart[4][kRowBmax];
  __shared__ float wtot[NWAVE][CQ];
  __shared__ float wmax[NWAVE];

  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int grp = hq / hkv;
  const int c = cur_block[seq];
  const int b = c + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int p = tid / kRowSeg;
  const int g = tid % kRowSeg;
  const int L = (b + kRowSeg - 1) / kRowSeg;
  const bool in_regs = L <= LMAX;
  const int seg = kRowSeg - 1 - g;            // descending j order
  const int j0 = min(b, seg * L);
  const int j1 = min(b, j0 + L);

  const float* qrow = q_cache + ((int64_t)seq * hq + h) * b_max * k;
  const float* krow = k_cache + ((int64_t)seq * hkv + h / grp) * b_max * k;
  const float* rin = r_prev ? r_prev + ((int64_t)seq * hq + h) * b_max : nullptr;
  float* rout = r_out + ((int64_t)seq * hq + h) * b_max;

  float qv[LMAX][CQ], kv[LMAX][CQ];
  if (in_regs && k == KP) {
    // full quarters: the sketch rows go through LDS (the ypart area, unused
    // until the first hop) in chunks of R rows, read with contiguous 16-byte
    // loads across the workgroup; each thread then picks its segment's rows
    constexpr int R = 8192 / KP;               // rows per chunk: q and k fill 64 KB
    constexpr int V4 = KP / 4;                 // float4 per row
    float* stage = &ypart[0][0];
    for (int r0 = 0; r0 < b; r0 += R) {
      const int nr = min(R, b - r0);
      for (int v = tid; v < nr * V4; v += kRowThreads) {
        const int64_t g4 = (int64_t)r0 * V4 + v;
        reinterpret_cast<float4*>(stage)[v] = reinterpret_cast<const float4*>(qrow)[g4];
        reinterpret_cast<float4*>(stage + R * KP)[v] = reinterpret_cast<const float4*>(krow)[g4];
      }
      __syncthreads();
#pragma unroll
      for (int l = 0; l < LMAX; ++l) {
        const int j = j0 + l;
        if (j >= r0 && j < r0 + nr && j < j1) {
          const float* qs = stage + (j - r0) * KP + p * CQ;
          const float* ks = stage + R * KP + (j - r0) * KP + p * CQ;
#pragma unroll
          for (int e = 0; e < CQ; e += 4) {
            const float4 a = *reinterpret_cast<const float4*>(qs + e);
            const float4 bb = *reinterpret_cast<const float4*>(ks + e);
            qv[l][e] = a.x; qv[l][e + 1] = a.y; qv[l][e + 2] = a.z; qv[l][e + 3] = a.w;
            kv[l][e] = bb.x; kv[l][e + 1] = bb.y; kv[l][e + 2] = bb.z; kv[l][e + 3] = bb.w;
          }
        }
      }
      __syncthreads();
    }
  } else {
#pragma unroll
    for (int l = 0; l < LMAX; ++l)
#pragma unroll
      for (int e = 0; e < CQ; ++e) {
        const int j = j0 + l;
        const int cc = p * CQ + e;
        const bool ok = in_regs && j < j1 && cc < k;
        qv[l][e] = ok ? qrow[(int64_t)j * k + cc] : 0.f;
        kv[l][e] = ok ? krow[(int64_t)j * k + cc] : 0.f;
      }
  }
  for (int j = tid; j < b; j += kRowThreads) xs[j] = rin ? rin[j] : (j == c ? 1.0f : 0.0f);
  __syncthreads();

  auto qget = [&](int l, int e) -> float {
    if (in_regs) return qv[l][e];
    const int cc = p * CQ + e;
    return cc < k ? qrow[(int64_t)(j0 + l) * k + cc] : 0.f;
  };
  auto kget = [&](int l, int e) -> float {
    if (in_regs) return kv[l][e];
    const int cc = p * CQ + e;
    return cc < k ? krow[(int64_t)(j0 + l) * k + cc] : 0.f;
  };

  float sc = 1.0f;
  float gmax = 0.0f;
  for (int hop = 0; hop < s; ++hop) {
    float T[CQ];
#pragma unroll
    for (int e = 0; e < CQ; ++e) T[e] = 0.f;
    if (in_regs) {
#pragma unroll
      for (int l = 0; l < LMAX; ++l) {
        if (j0 + l < j1) {
          const float x = xs[j0 + l] * sc;
#pragma unroll
          for (int e = 0; e < CQ; ++e) T[e] += x * qv[l][e];
        }
      }
    } else {
      for (int l = 0; l < j1 - j0; ++l) {
        const float x = xs[j0 + l] * sc;
#pragma unroll
        for (int e = 0; e < CQ; ++e) T[e] += x * qget(l, e);
      }
    }
    // exclusive prefix over the scan order = suffix over the rows above
    float S[CQ];
#pragma unroll
    for (int e = 0; e < CQ; ++e) {
      const float inc = wave_prefix_sum(T[e]);
      S[e] = inc - T[e];
      if (lane == 63) wtot[wave][e] = inc;
    }
    __syncthreads();
    {
      const int w0 = p * WPQ;
#pragma unroll
      for (int e = 0; e < CQ; ++e) {
        float carry = 0.f;
        for (int w2 = w0; w2 < wave; ++w2) carry += wtot[w2][e];
        S[e] += carry;
      }
    }
    if (in_regs) {
#pragma unroll
      for (int l = LMAX - 1; l >= 0; --l) {
        if (j0 + l < j1) {
          const float x = xs[j0 + l] * sc;
          float y = 0.f;
#pragma unroll
          for (int e = 0; e < CQ; ++e) {
            S[e] += x * qv[l][e];
            y += kv[l][e] * S[e];
          }
          ypart[p][j0 + l] = y;
        }
      }
    } else {
      for (int l = j1 - j0 - 1; l >= 0; --l) {
        const float x = xs[j0 + l] * sc;
        float y = 0.f;
#pragma unroll
        for (int e = 0; e < CQ; ++e) {
          S[e] += x * qget(l, e);
          y += kget(l, e) * S[e];
        }
        ypart[p][j0 + l] = y;
      }
    }
    __syncthreads();
    float lmax = 0.f;
    for (int j = tid; j < b; j += kRowThreads) {
      const float y = ((ypart[0][j] + ypart[1][j]) + (ypart[2][j] + ypart[3][j])) * inv_sqrt_k;
      xs[j] = y;
      lmax = fmaxf(lmax, fabsf(y));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off));
    if (lane == 0) wmax[wave] = lmax;
    __syncthreads();
    gmax = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NWAVE; ++w2) gmax = fmaxf(gmax, wmax[w2]);
    sc = (gmax > 0.f) ? 1.0f / gmax : 1.0f;
  }
  for (int j = tid; j < b_max; j += kRowThreads) {
    float v = 0.f;
    if (j < b && gmax > 0.f) v = xs[j] / gmax;
    rout[j] = v;
  }
}

template <int KP>
hipError_t run_walk(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                    const int32_t* cu_blocks, int n_seqs, int total_blocks, int max_blocks, int s,
                    const float* R_prev, float* R_out, hipStream_t st) {
  constexpr int ROWS = kWalkThreads / (KP / 8);
  dim3 grid((max_blocks + ROWS - 1) / ROWS, hq, n_seqs);
  hipLaunchKernelGGL((walk_kernel<KP>), grid, dim3(kWalkThreads), 0, st, q_sk, k_sk, hq, hkv, k,
                     cu_blocks, n_seqs, total_blocks, s, R_prev, R_out, 1.0f / sqrtf((float)k));
  return hipGetLastError();
}

template <int KP>
hipError_t run_walk_row(const float* q_sk, const float* k_sk, int hq, int hkv, int k, int n_seqs,
                        const int32_t* cur_block, int b_max, int s, const float* r_prev,
                        float* r_out, hipStream_t st) {
  dim3 grid(hq, n_seqs);
  hipLaunchKernelGGL((walk_row_kernel<KP>), grid, dim3(kRowThreads), 0, st, q_sk, k_sk, hq, hkv,
                     k, cur_block, b_max, s, r_prev, r_out, 1.0f / sqrtf((float)k));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_walk(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                       const int32_t* cu_blocks, int n_seqs, int total_blocks, int max_blocks,
                       int s, const float* R_prev, float* R_out, hipStream_t st) {
  if (total_blocks == 0 || max_blocks == 0) return hipSuccess;
  if (k <= 16)
    return run_walk<16>(q_sk, k_sk, hq, hkv, k, cu_blocks, n_seqs, total_blocks, max_blocks, s,
                        R_prev, R_out, st);
  if (k <= 32)
    return run_walk<32>(q_sk, k_sk, hq, hkv, k, cu_blocks, n_seqs, total_blocks, max_blocks, s,
                        R_prev, R_out, st);
  return run_walk<64>(q_sk, k_sk, hq, hkv, k, cu_blocks, n_seqs, total_blocks, max_blocks, s,
                      R_prev, R_out, st);
}

hipError_t launch_walk_row(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                           int n_seqs, const int32_t* cur_block, int b_max, int s,
                           const float* r_prev, float* r_out, hipStream_t st) {
  if (n_seqs == 0) return hipSuccess;
  if (k <= 16)
    return run_walk_row<16>(q_sk, k_sk, hq, hkv, k, n_seqs, cur_block, b_max, s, r_prev, r_out,
                            st);
  if (k <= 32)
    return run_walk_row<32>(q_sk, k_sk, hq, hkv, k, n_seqs, cur_block, b_max, s, r_prev, r_out,
                            st);
  return run_walk_row<64>(q_sk, k_sk, hq, hkv, k, n_seqs, cur_block, b_max, s, r_prev, r_out,
                          st);
}

}  // namespace sws
