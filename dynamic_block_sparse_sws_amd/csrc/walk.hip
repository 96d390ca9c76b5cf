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
// on them, streaming the rows tile by tile from the last column down (the
// scan order), overwriting each tile in place in R_out.  For k <= 32 (a
// multiple of 4) the scan within a tile runs as fp32 matrix-core products
// (walk_mfma_kernel); otherwise lanes of a row split the k components of S
// and combine their partial dot products with cross-lane shuffles
// (walk_kernel).  Every hop rescales its rows by their largest magnitude
// (positive row scaling commutes with the right-multiplication, so only the
// final division is visible), which keeps s * layers hops in fp32.
//
// Decode: one workgroup per (sequence, query head) walks the single row of
// the open block; the j range is cut into segments, one per thread of a
// component quarter, with the segment's sketch rows held in registers for all
// s hops, and the suffix carry across segments comes from a wave scan plus
// the wave totals in LDS.
#include "sws_common.h"

#include <type_traits>

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

// Final pass over a workgroup's rows i0 .. i0 + nrows - 1 (those inside the
// sequence): each row divided by its largest magnitude m[r] (an all-zero row
// stays zero), entries below the walk floor and above the diagonal set to
// zero.  The rows are walked as
// one flat range, four accesses per thread at a time, all loads before any
// store, so every thread keeps several loads in flight (row by row, each
// thread's single load per row would expose the memory latency once per row).
template <int NT>
__device__ __forceinline__ void finalize_rows(float* Rh, const float* m, int i0, int nrows,
                                              int b) {
  const int rows = min(nrows, b - i0);
  if (rows <= 0) return;
  const int total = rows * b;                 // <= 64 * 4096
  const float inv_b = 1.0f / (float)b;
  float* base = Rh + (int64_t)i0 * b;
  for (int e0 = threadIdx.x; e0 < total; e0 += 4 * NT) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * NT;
      v[u] = e < total ? base[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * NT;
      if (e < total) {
        // row and column of e (the float quotient is off by at most one)
        int rr = (int)((float)e * inv_b);
        int j = e - rr * b;
        if (j < 0) { --rr; j += b; }
        else if (j >= b) { ++rr; j -= b; }
        const float mm = m[rr];
        const float x = v[u] / mm;
        base[e] = (j <= i0 + rr && mm > 0.f && fabsf(x) >= kWalkFloor) ? x : 0.f;
      }
    }
  }
}

// Workgroup id -> (pair p = sequence * hq + head, row tile I) for the
// prefill walk kernels.  Row tile I costs I + 1 column tiles per hop, so the
// ids are laid out for the usual dispatch order (the first half of the grid
// takes one slot per CU, the second half the next): the first half holds the
// long tiles, longest first, and id + N / 2 gets the complementary short
// tile, so the workgroups sharing a CU add up to about the same work and the
// longest tiles do not share a CU with each other.
__device__ __forceinline__ void walk_tile_of(int id, int P, int n_row_tiles, int& p, int& I) {
  p = id % P;
  const int slot = id / P;
  const int half = (n_row_tiles + 1) / 2;
  I = slot < half ? n_row_tiles - 1 - slot : slot - half;
}


// Ragged batches: every (sequence, head, row tile) tile in descending length,
// longest first across the sequences, the order a greedy schedule over the
// CUs wants when tile lengths differ from sequence to sequence (the mapping
// above pairs long and short tiles of equal-length rows instead).  Level L
// holds the tiles I = L - 1 of the pairs whose sequence has at least L row
// tiles (nt[s] = row tiles of sequence s, in LDS).  Returns false past the
// last tile.
__device__ __forceinline__ bool walk_tile_ragged(int id, int hq, int n_seqs, const int* nt,
                                                 int n_row_tiles, int& p, int& I) {
  int base = 0;
  for (int L = n_row_tiles; L >= 1; --L) {
    int cnt = 0;
    for (int s = 0; s < n_seqs; ++s) cnt += nt[s] >= L;
    if (id < base + cnt * hq) {
      const int k = id - base;
      int want = k / hq, s = 0;
      for (; s < n_seqs; ++s)
        if (nt[s] >= L && want-- == 0) break;
      p = s * hq + k % hq;
      I = L - 1;
      return true;
    }
    base += cnt * hq;
  }
  return false;
}
constexpr int kRaggedMaxSeqs = 64;   // larger batches keep the mapping above

// (sequence x head, row tile) of workgroup `id`: the ragged order for 2 to
// kRaggedMaxSeqs sequences (all threads call it: it fills and syncs an LDS
// table), else walk_tile_of.  False: no tile for this workgroup.
__device__ __forceinline__ bool walk_tile(int id, int hq, int n_seqs,
                                          const int32_t* __restrict__ cu_blocks, int n_row_tiles,
                                          int tile_rows, int* s_nt, int& p, int& I) {
  if (n_seqs > 1 && n_seqs <= kRaggedMaxSeqs) {
    if ((int)threadIdx.x < n_seqs)
      s_nt[threadIdx.x] =
          (cu_blocks[threadIdx.x + 1] - cu_blocks[threadIdx.x] + tile_rows - 1) / tile_rows;
    __syncthreads();
    return walk_tile_ragged(id, hq, n_seqs, s_nt, n_row_tiles, p, I);
  }
  walk_tile_of(id, hq * n_seqs, n_row_tiles, p, I);
  return true;
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
    const int32_t* __restrict__ cu_blocks, int n_seqs, int total_blocks, int n_row_tiles, int s,
    const float* R_prev, float* R_out, float inv_sqrt_k) {
  using WT = WalkTile<KP>;
  constexpr int LPR = WT::LPR, ROWS = WT::ROWS, XPT = WT::XPT, SPT = WT::SPT;
  __shared__ __attribute__((aligned(16))) float sq[2][kTileJ][KP + 4];
  __shared__ __attribute__((aligned(16))) float sk[2][kTileJ][KP + 4];
  __shared__ float sx[2][ROWS][kTileJ + 1];
  __shared__ float smax[ROWS];

  int pid, tile;
  __shared__ int s_nt[kRaggedMaxSeqs];
  if (!walk_tile((int)blockIdx.x, hq, n_seqs, cu_blocks, n_row_tiles, ROWS, s_nt, pid, tile))
    return;
  const int seq = pid / hq;
  const int h = pid % hq;
  const int b0 = cu_blocks[seq];
  const int b = cu_blocks[seq + 1] - b0;
  const int i0 = tile * ROWS;
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
  float thr = 0.0f;  // the walk floor of this row's scaled input (0: none)
  float mx = 0.0f;   // largest |y| of this row in the current hop
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
        // a new hop: reset the scan, rescale by the previous hop's maximum (a
        // power of two, so exactly) and cut its output to the walk floor
        if (st > 0) {
          sc = mx > 0.f ? __builtin_amdgcn_ldexpf(1.0f, min(-__builtin_amdgcn_frexp_expf(mx), 126))
                        : 1.0f;
          thr = (mx * sc) * kWalkFloor;
        }
        mx = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) S[c] = 0.f;
      }
#pragma unroll 4
      for (int jj = kTileJ - 1; jj >= 0; --jj) {
        float x = sx[buf][r][jj] * sc;
        x = fabsf(x) < thr ? 0.f : x;
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
  if (part == 0) smax[r] = mx;
  __syncthreads();
  // final pass: divide by the row maximum, zero the upper triangle
  finalize_rows<kWalkThreads>(Rh, smax, i0, ROWS, b);
}

// ---------------------------------------------------------------------------
// prefill on the matrix cores (fp32 MFMA, k <= 32 and a multiple of 4)
// ---------------------------------------------------------------------------
// The same walk, one workgroup per 64-row tile I of one head, its s hops
// streaming the 64-column tiles J from the diagonal tile down.  Within a
// tile, the suffix scan becomes two products: with M_J the tile's own
// lower-triangular block of M and C the carry (rows i: sum over the later
// tiles of x[i][m] q_m),
//   Y_IJ = X_IJ M_J + C K_J^T,     C += X_IJ Q_J,
// all on v_mfma_f32_32x32x2_f32 (fp32 in, fp32 accumulate).  That is about
// twice the multiply-adds of the scan, on units with twice the vector rate
// and none of its per-column shuffles.  Wave (wi, wj) owns the 32 x 32
// quadrant (rows 32 wi.., columns 32 wj..) of Y; it also forms quadrant
// (wj, wi) of M_J^T and the part of X Q_J over the columns m in 32 wj.. (two
// carry partials, summed when read).  Operand layouts for 32x32x2: lane l
// feeds A[l % 32][l / 32] and B[l / 32][l % 32], and holds D[8 (r / 4) +
// 4 (l / 32) + r % 4][l % 32] in accumulator r; the two k slots of an
// instruction take two contiguous halves of the contraction (slot h, step t:
// index h * n / 2 + t), so every lane reads its operands as contiguous runs.
constexpr int kWmRows = 64;
constexpr int kWmK = 32;

// Workgroup barrier that orders LDS only: __syncthreads also waits for every
// outstanding global load and store, which would expose the next tile's
// prefetch and this tile's write-back at each of a tile's barriers.  Global
// writes that other threads read later are ordered by full barriers placed
// once per hop (see the kernel).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
constexpr int kWmPad = 68;        // LDS row pitch of 64-wide tiles (floats)
constexpr int kWmPadK = 36;       // LDS row pitch of 32-wide tiles

// ONE: every row tile has a single column tile (b <= 64 blocks); that form
// keeps the walk state on chip across hops (see below) and is compiled
// separately, so the multi-tile form's code is not disturbed by it.
template <bool K32, bool ONE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void walk_mfma_kernel(const float* __restrict__ q_sk, const float* __restrict__ k_sk, int hq,
                      int hkv, int k, const int32_t* __restrict__ cu_blocks, int n_seqs,
                      int total_blocks, int n_row_tiles, int s, const float* R_prev,
                      float* R_out, float inv_sqrt_k) {
  __shared__ __attribute__((aligned(16))) float Xs[kWmRows][kWmPad];     // X tile, then Y tile
  __shared__ __attribute__((aligned(16))) float Ms[kWmRows][kWmPad];     // M_J^T [j][m]
  __shared__ __attribute__((aligned(16))) float Qs[kWmRows][kWmPadK];    // Q_J [m][c]
  __shared__ __attribute__((aligned(16))) float QTs[kWmK][kWmPad];       // Q_J^T [c][m]
  __shared__ __attribute__((aligned(16))) float Ks[kWmRows][kWmPadK];    // K_J [j][c]
  __shared__ __attribute__((aligned(16))) float Cs[2][kWmRows][kWmPadK]; // carry partials
  __shared__ float rmax[kWmRows], rsc[kWmRows], rthr[kWmRows];

  __shared__ int s_nt[kRaggedMaxSeqs];
  int pid, I;
  if (!walk_tile((int)blockIdx.x, hq, n_seqs, cu_blocks, n_row_tiles, kWmRows, s_nt, pid, I))
    return;
  const int seq = pid / hq;
  const int h = pid % hq;
  const int b0 = cu_blocks[seq];
  const int b = cu_blocks[seq + 1] - b0;
  const int i0 = I * kWmRows;
  if (i0 >= b) return;
  const int64_t roff = walk_seq_offset(cu_blocks, seq, hq) + (int64_t)h * b * b;
  float* Rh = R_out + roff;
  const float* Rp = R_prev ? R_prev + roff : nullptr;
  const int grp = hq / hkv;
  const float* qs = q_sk + ((int64_t)h * total_blocks + b0) * k;
  const float* ks = k_sk + ((int64_t)(h / grp) * total_blocks + b0) * k;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wi = w >> 1, wj = w & 1;
  const int lc = lane & 31, lh = lane >> 5;
  // staging: thread t loads row t / 4 of a tile, columns 16 (t % 4) .. (X) or
  // 8 (t % 4) .. (sketches)
  const int sr = tid >> 2, sp = tid & 3;

  float4 xv[4], qv[2], kv[2];
  // Tiles strictly below the diagonal tile, with all 64 rows inside the
  // sequence and 16-byte aligned rows, take plain 16-byte loads and stores
  // (thread (sr, sp): 16 consecutive entries of row sr).  The others (the
  // diagonal tile, a sequence's last rows, b not a multiple of 4) are read and
  // written row by row instead (xrow): entry e of wave w's lane l is row
  // 16 w + e, column l, so each access of a wave covers 64 consecutive floats
  // of one row whatever the row's alignment, through clamped, always valid
  // addresses with the out-of-range values replaced.
  const bool plain_rows = i0 + kWmRows <= b && (b & 3) == 0;
  const int row0 = i0 + 16 * __builtin_amdgcn_readfirstlane(w);   // a wave's first row (xrow)
  bool xrow = false;
  bool xin_lds = false;       // the next X is the last Y, left in Xs (ONE)
  auto fetch = [&](int hop, int jt) {
    const int ig = i0 + sr;
    const int jg0 = jt * kWmRows + sp * 16;
    const float* src = hop == 0 ? Rp : Rh;
    xrow = src && !(plain_rows && jt < I);        // uniform
    if (!src) {                                   // the identity (uniform)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) v[x] = (ig < b && jg0 + 4 * e + x == ig) ? 1.f : 0.f;
        xv[e] = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else if (!xrow) {
      const float4* p4 = reinterpret_cast<const float4*>(src + (int64_t)ig * b + jg0);
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[e] = p4[e];
    } else {
      // 32-bit offsets within the head's b x b block (b <= 4096).  A row past
      // the sequence reads the block's last entry (a finite walk value of
      // magnitude <= 1): such rows only ever feed their own output rows, which
      // are zeroed before the write-back, so they need no test here.
      const int jg = jt * kWmRows + lane;
      const int off0 = row0 * b + min(jg, b - 1);
      const int last = b * b - 1;
      float v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float t = src[min(off0 + e * b, last)];
        v[e] = jg <= row0 + e ? t : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[e] = make_float4(v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3]);
    }
    // sketch rows: rows past the sequence (and, for k < 32, components
    // past k) are zero, read from clamped addresses and then replaced
    const int mg = jt * kWmRows + sr;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    if (K32) {
      const int64_t mrow = (int64_t)min(mg, b - 1) * kWmK + sp * 8;
      const float4* pq = reinterpret_cast<const float4*>(qs + mrow);
      const float4* pk = reinterpret_cast<const float4*>(ks + mrow);
      qv[0] = pq[0]; qv[1] = pq[1];
      kv[0] = pk[0]; kv[1] = pk[1];
      if (mg >= b) qv[0] = qv[1] = kv[0] = kv[1] = z;
    } else {
      const int64_t mrow = (int64_t)min(mg, b - 1) * k;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c0 = sp * 8 + 4 * e;
        const int64_t off = mrow + min(c0, k - 4);
        const float4 a = *reinterpret_cast<const float4*>(qs + off);
        const float4 c = *reinterpret_cast<const float4*>(ks + off);
        const bool ok = mg < b && c0 < k;
        qv[e] = ok ? a : z;
        kv[e] = ok ? c : z;
      }
    }
  };
  auto stash = [&]() {
    // the previous hop's output, scaled and cut to the walk floor
    if (ONE && xin_lds) {
      // still in Xs (a single column tile): this thread's 16 entries of row sr
      const float sc = rsc[sr], th = rthr[sr];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float4 v = *reinterpret_cast<const float4*>(&Xs[sr][sp * 16 + 4 * e]);
        v.x *= sc; v.y *= sc; v.z *= sc; v.w *= sc;
        v.x = fabsf(v.x) < th ? 0.f : v.x;
        v.y = fabsf(v.y) < th ? 0.f : v.y;
        v.z = fabsf(v.z) < th ? 0.f : v.z;
        v.w = fabsf(v.w) < th ? 0.f : v.w;
        *reinterpret_cast<float4*>(&Xs[sr][sp * 16 + 4 * e]) = v;
      }
    } else if (xrow) {
      float v[16];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[4 * e] = xv[e].x; v[4 * e + 1] = xv[e].y; v[4 * e + 2] = xv[e].z; v[4 * e + 3] = xv[e].w;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = row0 - i0 + e;              // uniform
        const float x = v[e] * rsc[r];
        Xs[r][lane] = fabsf(x) < rthr[r] ? 0.f : x;
      }
    } else {
      const float sc = rsc[sr], th = rthr[sr];
      auto cut = [&](float x) { x *= sc; return fabsf(x) < th ? 0.f : x; };
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float4 v = xv[e];
        v.x = cut(v.x); v.y = cut(v.y); v.z = cut(v.z); v.w = cut(v.w);
        *reinterpret_cast<float4*>(&Xs[sr][sp * 16 + 4 * e]) = v;
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      *reinterpret_cast<float4*>(&Qs[sr][sp * 8 + 4 * e]) = qv[e];
      *reinterpret_cast<float4*>(&Ks[sr][sp * 8 + 4 * e]) = kv[e];
      QTs[sp * 8 + 4 * e + 0][sr] = qv[e].x;
      QTs[sp * 8 + 4 * e + 1][sr] = qv[e].y;
      QTs[sp * 8 + 4 * e + 2][sr] = qv[e].z;
      QTs[sp * 8 + 4 * e + 3][sr] = qv[e].w;
    }
  };

  if (tid < kWmRows) {
    rmax[tid] = 0.f;
    rsc[tid] = 1.f;
    rthr[tid] = 0.f;
  }
  const int ntiles = I + 1;                 // column tiles I, I - 1, ..., 0
  const int nsteps = s * ntiles;
  fetch(0, I);
  for (int st = 0; st < nsteps; ++st) {
    const int hop = st / ntiles;
    const int jt = I - st % ntiles;
    if (st % ntiles == 0) {
      // a new hop: this hop's row scales from the last one's maxima (a power
      // of two, so the scaling is exact) and the walk floor relative to them,
      // and an empty carry
      __syncthreads();
      if (tid < kWmRows) {
        const float m = rmax[tid];
        const bool rescale = hop > 0 && m > 0.f;
        const float sc =
            rescale ? __builtin_amdgcn_ldexpf(1.0f, min(-__builtin_amdgcn_frexp_expf(m), 126))
                    : 1.f;
        rsc[tid] = sc;
        rthr[tid] = rescale ? (m * sc) * kWalkFloor : 0.f;
        rmax[tid] = 0.f;
      }
      for (int e = tid; e < 2 * kWmRows * kWmPadK; e += 256) (&Cs[0][0][0])[e] = 0.f;
      __syncthreads();
    }
    stash();
    // The next step's tiles are fetched right after this barrier.  On a hop's
    // last tile that fetch reads the next hop's top tile, written back by
    // other threads a whole hop earlier: a full barrier (one per hop) makes
    // those stores visible; the other tiles of the next hop are fetched after
    // the full barriers that open it.  With a single tile the fetch waits for
    // the write-back below instead.
    const bool last = st + 1 == nsteps;
    const bool late = ONE || ntiles == 1;
    if (st % ntiles == ntiles - 1) __syncthreads();
    else lds_barrier();
    if (!last && !late) fetch((st + 1) / ntiles, I - (st + 1) % ntiles);
    floatx16_t acc;
    // ---- M_J^T quadrant (rows j of 32 wj.., columns m of 32 wi..) ----
    // (ONE: M_J is the same at every hop, formed once)
    if (!ONE || st == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int t = 0; t < kWmK / 2; ++t)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[32 * wj + lc][16 * lh + t],
                                                   Qs[32 * wi + lc][16 * lh + t], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = 32 * wj + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int m = 32 * wi + lc;
        Ms[j][m] = j <= m ? acc[r] : 0.f;
      }
      lds_barrier();
    }
    // ---- Y quadrant (rows 32 wi.., columns 32 wj..) and the carry part ----
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll 8
    for (int t = 0; t < kWmRows / 2; ++t)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Xs[32 * wi + lc][32 * lh + t],
                                                 Ms[32 * wj + lc][32 * lh + t], acc, 0, 0, 0);
    // (ONE: no later column tiles, so the carry is zero and unused)
    floatx16_t cp;
#pragma unroll
    for (int r = 0; r < 16; ++r) cp[r] = 0.f;
    if constexpr (!ONE) {
#pragma unroll
      for (int t = 0; t < kWmK / 2; ++t)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(
            Cs[0][32 * wi + lc][16 * lh + t] + Cs[1][32 * wi + lc][16 * lh + t],
            Ks[32 * wj + lc][16 * lh + t], acc, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < kWmRows / 4; ++t)
        cp = __builtin_amdgcn_mfma_f32_32x32x2f32(Xs[32 * wi + lc][32 * wj + 16 * lh + t],
                                                  QTs[lc][32 * wj + 16 * lh + t], cp, 0, 0, 0);
    }
    lds_barrier();
    // carry partial wj of rows 32 wi.. (this wave's own block), Y into Xs
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * wi + 8 * (r >> 2) + 4 * lh + (r & 3);
      if constexpr (!ONE) Cs[wj][i][lc] += cp[r];
      const int j = 32 * wj + lc;
      const bool ok = i0 + i < b && jt * kWmRows + j <= i0 + i;
      Xs[i][j] = ok ? acc[r] * inv_sqrt_k : 0.f;
    }
    lds_barrier();
    // ---- write the tile back, row maxima ----
    // (ONE leaves the hop's output in Xs as the next hop's input, scaled and
    // cut there by the stash, and writes it to memory only after the last
    // hop)
    {
      const int ig = i0 + sr;
      const int jg0 = jt * kWmRows + sp * 16;
      float mx = 0.f;
      float4 v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = *reinterpret_cast<const float4*>(&Xs[sr][sp * 16 + 4 * e]);
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[e].x), fabsf(v[e].y)),
                             fmaxf(fabsf(v[e].z), fabsf(v[e].w))));
      }
      if (ONE && !last) {
        xin_lds = true;
      } else if (plain_rows && jt < I) {          // uniform
        float* dst = Rh + (int64_t)ig * b + jg0;
#pragma unroll
        for (int e = 0; e < 4; ++e) reinterpret_cast<float4*>(dst)[e] = v[e];
      } else {
        // row by row (as xrow reads it back): only entries on or below the
        // diagonal of rows inside the sequence, so never past a row's end
        const int jg = jt * kWmRows + lane;
        const int nr = min(16, b - row0);         // rows of this wave inside the sequence
#pragma unroll 4
        for (int e = 0; e < nr; ++e) {
          if (jg <= row0 + e) Rh[(row0 + e) * b + jg] = Xs[row0 - i0 + e][lane];
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      if (sp == 0) rmax[sr] = fmaxf(rmax[sr], mx);
    }
    if (!ONE && !last && late) {
      __syncthreads();
      fetch((st + 1) / ntiles, I - (st + 1) % ntiles);
    }
    if (last) __syncthreads();        // the final pass reads other threads' stores
    else lds_barrier();
  }
  // final pass: divide by the row maximum, zero the upper triangle
  finalize_rows<256>(Rh, rmax, i0, kWmRows, b);
}

// ---------------------------------------------------------------------------
// decode: one row per (sequence, query head)
// ---------------------------------------------------------------------------
// 1024 threads.  Thread t works on component quarter p = t / 256 of the
// sketches (KP / 4 components) and on segment g = t % 256 of the rows j, the
// segments taken in descending j order so that the suffix sum over j becomes
// a prefix scan over the threads of a quarter.  REG: the segment's q and k
// sketch rows (up to 40 / (KP / 4) of them) stay in registers for all s hops;
// otherwise they are re-read from memory every hop.  The segment's x values
// live in registers too.  A hop:
//   A  x of the segment's rows from the previous hop's four partial products
//      (LDS) and the row's largest |x| (wave maxima to LDS, barrier), then x
//      scaled by the power of two nearest below 1 / max and cut to the walk
//      floor (which needs the maximum before any sum over x);
//   B  T = sum over the segment of x q, a wave scan of T, the wave totals to
//      LDS, barrier;
//   C  S = exclusive scan (+ the totals of the quarter's earlier waves), then
//      the rows' partial products k . S to LDS, barrier.
constexpr int kRowThreads = 1024;
constexpr int kRowSeg = 256;        // segments (threads per component quarter)
constexpr int kRowBmax = 4096;      // ypart capacity (largest row)
// LDS of the row kernel: the hops' partial products (ypart, 64 KB) share it
// with the staging of the sketch rows before the first hop (144 KB: one
// workgroup fills a CU's registers, so it may as well use the CU's LDS, and
// larger chunks mean fewer load round trips).
constexpr int kRowSmemFloats = 36864;
constexpr int kRowLStream = kRowBmax / kRowSeg;   // rows per segment, streaming form

template <int CTRL, int RMASK>
__device__ __forceinline__ float dpp_shifted(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, RMASK, 0xF, false));
}

// The cross-row steps of a wave-wide inclusive scan for N values: lane 15 of
// rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3.  These are
// DPP adds that write only the receiving rows (row_mask), which the compiler
// only forms as a zeroed move plus a masked move plus an add, so they are
// written out here; the s_nop gives the two wait states a DPP read of a VGPR
// needs after a VALU write of it (before the block, between the steps when a
// value's own previous step is too close, and after the block for whatever
// reads the results next).
#define SWS_BC15(i) "v_add_f32_dpp %" #i ", %" #i ", %" #i " row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
#define SWS_BC31(i) "v_add_f32_dpp %" #i ", %" #i ", %" #i " row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
template <int N> struct CrossRows;
template <> struct CrossRows<4> {
  static __device__ __forceinline__ void add(float (&v)[4]) {
    asm volatile("s_nop 1\n\t" SWS_BC15(0) SWS_BC15(1) SWS_BC15(2) SWS_BC15(3)
                 SWS_BC31(0) SWS_BC31(1) SWS_BC31(2) SWS_BC31(3) "s_nop 1"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
  }
};
template <> struct CrossRows<8> {
  static __device__ __forceinline__ void add(float (&v)[8]) {
    asm volatile("s_nop 1\n\t" SWS_BC15(0) SWS_BC15(1) SWS_BC15(2) SWS_BC15(3) SWS_BC15(4)
                 SWS_BC15(5) SWS_BC15(6) SWS_BC15(7) SWS_BC31(0) SWS_BC31(1) SWS_BC31(2)
                 SWS_BC31(3) SWS_BC31(4) SWS_BC31(5) SWS_BC31(6) SWS_BC31(7) "s_nop 1"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                   "+v"(v[6]), "+v"(v[7]));
  }
};
template <> struct CrossRows<16> {
  static __device__ __forceinline__ void add(float (&v)[16]) {
    asm volatile("s_nop 1\n\t" SWS_BC15(0) SWS_BC15(1) SWS_BC15(2) SWS_BC15(3) SWS_BC15(4)
                 SWS_BC15(5) SWS_BC15(6) SWS_BC15(7) SWS_BC15(8) SWS_BC15(9) SWS_BC15(10)
                 SWS_BC15(11) SWS_BC15(12) SWS_BC15(13) SWS_BC15(14) SWS_BC15(15)
                 SWS_BC31(0) SWS_BC31(1) SWS_BC31(2) SWS_BC31(3) SWS_BC31(4) SWS_BC31(5)
                 SWS_BC31(6) SWS_BC31(7) SWS_BC31(8) SWS_BC31(9) SWS_BC31(10) SWS_BC31(11)
                 SWS_BC31(12) SWS_BC31(13) SWS_BC31(14) SWS_BC31(15) "s_nop 1"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                   "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
                   "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15]));
  }
};
#undef SWS_BC15
#undef SWS_BC31

// The same scan for N independent values at once, step by step, so the DPP
// read of one value is separated from its last write by the others.
template <int N>
__device__ __forceinline__ void wave_prefix_sum_n(float (&v)[N]) {
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] += dpp_shifted<0x111, 0xF>(v[e]);   // row_shr:1
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] += dpp_shifted<0x112, 0xF>(v[e]);   // row_shr:2
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] += dpp_shifted<0x114, 0xF>(v[e]);   // row_shr:4
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] += dpp_shifted<0x118, 0xF>(v[e]);   // row_shr:8
  CrossRows<N>::add(v);
}

// Maximum of non-negative values over the wave, valid in lane 63.  Non-negative
// floats order like their bit patterns, so the steps are unsigned maxima
// (absent lanes contribute 0); the cross-row steps are written out as above.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  unsigned u = __builtin_bit_cast(unsigned, v);
  u = max(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0x111, 0xF, 0xF, false));
  u = max(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0x112, 0xF, 0xF, false));
  u = max(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0x114, 0xF, 0xF, false));
  u = max(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0x118, 0xF, 0xF, false));
  asm volatile("s_nop 1\n\t"
               "v_max_u32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
               "s_nop 1\n\t"
               "v_max_u32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
               "s_nop 1"
               : "+v"(u));
  return __builtin_bit_cast(float, u);
}

template <int KP, bool REG>
__global__ __launch_bounds__(kRowThreads) void walk_row_kernel(
    const float* __restrict__ q_cache, const float* __restrict__ k_cache, int hq, int hkv,
    int k, const int32_t* __restrict__ cur_block, int n_seqs, int b_max, int s,
    const float* r_prev, float* r_out, float inv_sqrt_k) {
  constexpr int CQ = KP / 4;                                  // components per quarter
  constexpr int LR = REG ? 40 / CQ : kRowLStream;             // rows per segment (capacity)
  constexpr int NWAVE = kRowThreads / 64;
  constexpr int WPQ = kRowSeg / 64;                           // waves per quarter
  __shared__ __attribute__((aligned(16))) float smem[kRowSmemFloats];
  static_assert(kRowSmemFloats >= 4 * kRowBmax, "ypart fits");
  float (*ypart)[kRowBmax] = reinterpret_cast<float (*)[kRowBmax]>(smem);
  __shared__ float wtot[NWAVE][CQ];
  __shared__ float wmax[NWAVE];

  // Workgroup -> (sequence, head): the query heads of one (sequence, KV head)
  // pair get ids equal modulo 8, so they run on one XCD and read the shared K
  // sketch rows through one L2 (pairs past the last multiple of 8 map plainly).
  const int grp = hq / hkv;
  int pair, hi;
  {
    const int id = blockIdx.x;
    const int np8 = (n_seqs * hkv) / 8 * 8;
    if (id < np8 * grp) {
      pair = id / (8 * grp) * 8 + id % 8;
      hi = id / 8 % grp;
    } else {
      const int t = id - np8 * grp;
      pair = np8 + t / grp;
      hi = t % grp;
    }
  }
  const int seq = pair / hkv;
  const int h = pair % hkv * grp + hi;
  const int c = cur_block[seq];
  const int b = c + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int p = tid / kRowSeg;
  const int g = tid % kRowSeg;
  const int L = (b + kRowSeg - 1) / kRowSeg;                  // <= LR (checked on the host)
  const int seg = kRowSeg - 1 - g;                            // descending j order
  const int j0 = min(b, seg * L);
  const int j1 = min(b, j0 + L);

  const float* qrow = q_cache + ((int64_t)seq * hq + h) * b_max * k;
  const float* krow = k_cache + ((int64_t)seq * hkv + h / grp) * b_max * k;
  const float* rin = r_prev ? r_prev + ((int64_t)seq * hq + h) * b_max : nullptr;
  float* rout = r_out + ((int64_t)seq * hq + h) * b_max;

  // sketch rows of the segment (REG), zero past the segment's end.  They go
  // through LDS (the smem area, ypart's only after the first hop) in chunks of
  // whole segments, read from memory with contiguous 16-byte loads; the
  // 16-byte slots of a staged row are XOR-swizzled by the row index so the
  // threads of consecutive segments (rows L apart) read distinct banks.
  float qv[REG ? LR : 1][CQ], kv[REG ? LR : 1][CQ];
  if (REG) {
    constexpr int V4 = KP / 4;                  // float4 per row
    constexpr int R = kRowSmemFloats / 2 / KP;  // staged rows: q and k fill smem
    float4* stq = reinterpret_cast<float4*>(smem);
    float4* stk = stq + R * V4;
#pragma unroll
    for (int l = 0; l < LR; ++l)
#pragma unroll
      for (int e = 0; e < CQ; ++e) qv[l][e] = kv[l][e] = 0.f;
    const int ns = R / L;                       // whole segments per chunk
    for (int s0 = 0; s0 * L < b; s0 += ns) {
      const int r0 = s0 * L;
      const int nr = min(ns * L, b - r0);
      for (int v = tid; v < nr * V4; v += kRowThreads) {
        const int r = v / V4, cc = v % V4;
        const int64_t src = (int64_t)(r0 + r) * V4 + cc;
        stq[r * V4 + (cc ^ (r & (V4 - 1)))] = reinterpret_cast<const float4*>(qrow)[src];
        stk[r * V4 + (cc ^ (r & (V4 - 1)))] = reinterpret_cast<const float4*>(krow)[src];
      }
      __syncthreads();
      if (seg >= s0 && seg < s0 + ns) {
#pragma unroll
        for (int l = 0; l < LR; ++l) {
          if (l < j1 - j0) {
            const int r = j0 + l - r0;
#pragma unroll
            for (int e = 0; e < CQ; e += 4) {
              const int slot = r * V4 + (((p * CQ + e) / 4) ^ (r & (V4 - 1)));
              const float4 a = stq[slot];
              const float4 bb = stk[slot];
              qv[l][e] = a.x; qv[l][e + 1] = a.y; qv[l][e + 2] = a.z; qv[l][e + 3] = a.w;
              kv[l][e] = bb.x; kv[l][e + 1] = bb.y; kv[l][e + 2] = bb.z; kv[l][e + 3] = bb.w;
            }
          }
        }
      }
      __syncthreads();
    }
  }
  auto qget = [&](int l, int e) -> float {
    if (REG) return qv[REG ? l : 0][e];
    const int cc = p * CQ + e;
    return cc < k ? qrow[(int64_t)(j0 + l) * k + cc] : 0.f;
  };
  auto kget = [&](int l, int e) -> float {
    if (REG) return kv[REG ? l : 0][e];
    const int cc = p * CQ + e;
    return cc < k ? krow[(int64_t)(j0 + l) * k + cc] : 0.f;
  };

  const int nv = j1 - j0;                                     // rows of this segment
  const float* yp = &ypart[0][0] + j0;                        // yp[q * kRowBmax + l]
  float xr[LR];
#pragma unroll
  for (int l = 0; l < LR; ++l) {
    const int j = j0 + l;
    xr[l] = l < nv ? (rin ? rin[j] : (j == c ? 1.0f : 0.0f)) : 0.f;
  }
  for (int hop = 0; hop < s; ++hop) {
    // ---- A: x of the segment's rows and the row's largest |x| ----
    if (hop > 0) {
      // REG: rows past the segment read LDS inside smem and are dropped (no
      // branch); the streaming form's 16 rows would hold too many registers
#pragma unroll
      for (int l = 0; l < LR; ++l) {
        const float y = ((yp[l] + yp[kRowBmax + l]) + (yp[2 * kRowBmax + l] + yp[3 * kRowBmax + l])) *
                        inv_sqrt_k;
        xr[l] = l < nv ? y : 0.f;
      }
    }
    float lmax = 0.f;
#pragma unroll
    for (int l = 0; l < LR; ++l) lmax = fmaxf(lmax, fabsf(xr[l]));
    lmax = wave_max_nonneg(lmax);
    if (lane == 63) wmax[wave] = lmax;
    __syncthreads();
    float gmax = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NWAVE; ++w2) gmax = fmaxf(gmax, wmax[w2]);
    // the hop's scale, a power of two near 1 / gmax (exact; any positive scale
    // leaves the row's direction unchanged), and the previous hop's output
    // cut to the walk floor
    {
      const float sc =
          gmax > 0.f ? __builtin_amdgcn_ldexpf(1.0f, min(-__builtin_amdgcn_frexp_expf(gmax), 126))
                     : 1.0f;
      const float thr = hop > 0 ? (gmax * sc) * kWalkFloor : 0.f;
#pragma unroll
      for (int l = 0; l < LR; ++l) {
        const float x = xr[l] * sc;
        xr[l] = fabsf(x) < thr ? 0.f : x;
      }
    }
    // ---- B: T = sum over the segment of x q, its wave scan and totals ----
    float S[CQ];                                              // T, then its scan
#pragma unroll
    for (int e = 0; e < CQ; ++e) S[e] = 0.f;
#pragma unroll
    for (int l = 0; l < LR; ++l) {
      if (REG || l < nv) {
#pragma unroll
        for (int e = 0; e < CQ; ++e) S[e] += xr[l] * qget(l, e);
      }
    }
    wave_prefix_sum_n<CQ>(S);
    if (lane == 63) {
#pragma unroll
      for (int e = 0; e < CQ; ++e) wtot[wave][e] = S[e];
    }
    // exclusive: the inclusive scan shifted up one lane (wave_shr:1, lane 0
    // gets 0), so T need not stay live through the scan
#pragma unroll
    for (int e = 0; e < CQ; ++e)
      S[e] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, S[e]), 0x138, 0xF, 0xF, true));
    __syncthreads();
    {
      // earlier waves of the quarter (uniform over the wave)
      const int wq = __builtin_amdgcn_readfirstlane(wave - p * WPQ);
#pragma unroll
      for (int w2 = 0; w2 < WPQ - 1; ++w2) {
        if (w2 < wq) {
#pragma unroll
          for (int e = 0; e < CQ; ++e) S[e] += wtot[p * WPQ + w2][e];
        }
      }
    }
    // ---- C: partial products k . S of the segment's rows, last row first ----
    // (REG: the test is l < L, the same for the whole workgroup; rows l in
    // [nv, L) exist only in the truncated or empty segments at the end of the
    // row, hold zero sketches and x, and their products land on rows >= b,
    // below kRowBmax, which no segment reads)
#pragma unroll
    for (int l = LR - 1; l >= 0; --l) {
      if (REG ? l < L : l < nv) {
        const float x = xr[l];
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
  }
  // ---- final row, divided by its largest magnitude ----
  float lmax = 0.f;
#pragma unroll
  for (int l = 0; l < LR; ++l) {
    xr[l] = l < nv ? ((yp[l] + yp[kRowBmax + l]) + (yp[2 * kRowBmax + l] + yp[3 * kRowBmax + l])) *
                         inv_sqrt_k
                   : 0.f;
    lmax = fmaxf(lmax, fabsf(xr[l]));
  }
  lmax = wave_max_nonneg(lmax);
  if (lane == 63) wmax[wave] = lmax;
  __syncthreads();
  float gmax = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < NWAVE; ++w2) gmax = fmaxf(gmax, wmax[w2]);
  if (p == 0) {
#pragma unroll
    for (int l = 0; l < LR; ++l) {
      if (l < nv) {
        const float x = xr[l] / gmax;
        rout[j0 + l] = gmax > 0.f && fabsf(x) >= kWalkFloor ? x : 0.f;
      }
    }
  }
  for (int j = b + tid; j < b_max; j += kRowThreads) rout[j] = 0.f;
}

// ---------------------------------------------------------------------------
// decode, rows of up to 64 * LaneRows<KP> blocks: four waves per row
// ---------------------------------------------------------------------------
// Wave p of the workgroup owns sketch components [p KP/4, (p+1) KP/4) of every
// row j; lane g owns the segment of L = ceil(b / 64) consecutive rows
// j0 = (63 - g) L .. j0 + L - 1 (descending j over the lanes, so the suffix sum
// over j is a prefix scan over the lanes of one wave).  The segment's q and k
// sketch components stay in registers for all s hops.  Each wave therefore
// holds the whole row's x and takes its maximum alone; a hop is
//   B  T = sum over the segment of x q (this wave's components), an in-wave
//      exclusive scan of T over the lanes;
//   C  running down the segment, S += x q and the row's partial product
//      k . S to LDS (one buffer per hop parity), barrier;
//   A  (next hop) x of the segment's rows from the four waves' partials, the
//      row maximum (wave reduction), x scaled by the power of two nearest
//      below 1 / max and cut to the walk floor.
// One barrier per hop: a wave writes the other parity's buffer only after
// every wave has passed the barrier that follows its last read of it.
template <int KP> struct LaneRows;
template <> struct LaneRows<16> { static constexpr int value = 16; };
template <> struct LaneRows<32> { static constexpr int value = 12; };
template <> struct LaneRows<64> { static constexpr int value = 6; };
constexpr int kLaneThreads = 256;

template <int KP>
__global__ __launch_bounds__(kLaneThreads) void walk_row_lane_kernel(
    const float* __restrict__ q_cache, const float* __restrict__ k_cache, int hq, int hkv,
    const int32_t* __restrict__ cur_block, int n_seqs, int b_max, int s,
    const float* r_prev, float* r_out, float inv_sqrt_k) {
  constexpr int CQ = KP / 4;                   // components per wave
  constexpr int LR = LaneRows<KP>::value;      // rows per lane (capacity)
  constexpr int CAP = 64 * LR;                 // rows per partial buffer
  static_assert(CQ % 4 == 0, "whole 16-byte slots per wave");
  __shared__ __attribute__((aligned(16))) float ypart[2][4][CAP];

  // workgroup -> (sequence, head), query heads of one KV head on one XCD
  const int grp = hq / hkv;
  int pair, hi;
  {
    const int id = blockIdx.x;
    const int np8 = (n_seqs * hkv) / 8 * 8;
    if (id < np8 * grp) {
      pair = id / (8 * grp) * 8 + id % 8;
      hi = id / 8 % grp;
    } else {
      const int t = id - np8 * grp;
      pair = np8 + t / grp;
      hi = t % grp;
    }
  }
  const int seq = pair / hkv;
  const int h = pair % hkv * grp + hi;
  const int c = cur_block[seq];
  const int b = c + 1;
  const int lane = threadIdx.x & 63;
  const int p = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = (b + 63) / 64;                 // <= LR (b <= b_max, checked on the host)
  const int j0 = min(b, (63 - lane) * L);
  const int nv = min(b, j0 + L) - j0;          // rows of this lane's segment

  const float* qrow = q_cache + ((int64_t)seq * hq + h) * b_max * KP + p * CQ;
  const float* krow = k_cache + ((int64_t)seq * hkv + h / grp) * b_max * KP + p * CQ;
  const float* rin = r_prev ? r_prev + ((int64_t)seq * hq + h) * b_max : nullptr;
  float* rout = r_out + ((int64_t)seq * hq + h) * b_max;

  // the segment's sketch components (zero past the segment) and its x
  float qv[LR][CQ], kv[LR][CQ], xr[LR];
#pragma unroll
  for (int l = 0; l < LR; ++l) {
    const bool in = l < nv;
    const int j = j0 + l;
#pragma unroll
    for (int e = 0; e < CQ; e += 4) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), bb = a;
      if (in) {
        a = *reinterpret_cast<const float4*>(qrow + (int64_t)j * KP + e);
        bb = *reinterpret_cast<const float4*>(krow + (int64_t)j * KP + e);
      }
      qv[l][e] = a.x; qv[l][e + 1] = a.y; qv[l][e + 2] = a.z; qv[l][e + 3] = a.w;
      kv[l][e] = bb.x; kv[l][e + 1] = bb.y; kv[l][e + 2] = bb.z; kv[l][e + 3] = bb.w;
    }
    xr[l] = in ? (rin ? rin[j] : (j == c ? 1.0f : 0.0f)) : 0.f;
  }

  // x of the segment's rows from the partials of a hop's buffer, and the row's
  // largest |x| (every lane of the wave gets it)
  auto gather = [&](const float (*yp)[CAP]) -> float {
    float lmax = 0.f;
#pragma unroll
    for (int l = 0; l < LR; ++l) {
      if (l < L) {
        const int j = j0 + l;
        const float y = ((yp[0][j] + yp[1][j]) + (yp[2][j] + yp[3][j])) * inv_sqrt_k;
        xr[l] = l < nv ? y : 0.f;
        lmax = fmaxf(lmax, fabsf(xr[l]));
      }
    }
    return __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_max_nonneg(lmax)), 63));
  };

  for (int hop = 0; hop < s; ++hop) {
    // ---- A ----
    float gmax;
    if (hop > 0) {
      gmax = gather(ypart[(hop - 1) & 1]);
    } else {
      float lmax = 0.f;
#pragma unroll
      for (int l = 0; l < LR; ++l) lmax = fmaxf(lmax, fabsf(xr[l]));
      gmax = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_max_nonneg(lmax)), 63));
    }
    {
      const float sc =
          gmax > 0.f ? __builtin_amdgcn_ldexpf(1.0f, min(-__builtin_amdgcn_frexp_expf(gmax), 126))
                     : 1.0f;
      const float thr = hop > 0 ? (gmax * sc) * kWalkFloor : 0.f;
#pragma unroll
      for (int l = 0; l < LR; ++l) {
        const float x = xr[l] * sc;
        xr[l] = fabsf(x) < thr ? 0.f : x;
      }
    }
    // ---- B ----
    float S[CQ];
#pragma unroll
    for (int e = 0; e < CQ; ++e) S[e] = 0.f;
#pragma unroll
    for (int l = 0; l < LR; ++l) {
      if (l < L) {
#pragma unroll
        for (int e = 0; e < CQ; ++e) S[e] += xr[l] * qv[l][e];
      }
    }
    wave_prefix_sum_n<CQ>(S);
    // exclusive: shifted up one lane (wave_shr:1, lane 0 gets 0)
#pragma unroll
    for (int e = 0; e < CQ; ++e)
      S[e] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, S[e]), 0x138, 0xF, 0xF, true));
    // ---- C ----
    // (rows l in [nv, L) exist only in the truncated or empty segments at the
    // end of the row; their x and sketches are zero and their products land on
    // rows >= b, below CAP, which are never read as part of the row)
    float (*yo)[CAP] = ypart[hop & 1];
#pragma unroll
    for (int l = LR - 1; l >= 0; --l) {
      if (l < L) {
        const float x = xr[l];
        float y = 0.f;
#pragma unroll
        for (int e = 0; e < CQ; ++e) {
          S[e] += x * qv[l][e];
          y += kv[l][e] * S[e];
        }
        yo[p][j0 + l] = y;
      }
    }
    __syncthreads();
  }
  // ---- final row, divided by its largest magnitude ----
  const float gmax = gather(ypart[(s - 1) & 1]);
  if (p == 0) {
#pragma unroll
    for (int l = 0; l < LR; ++l) {
      if (l < nv) {
        const float x = xr[l] / gmax;
        rout[j0 + l] = gmax > 0.f && fabsf(x) >= kWalkFloor ? x : 0.f;
      }
    }
  }
  for (int j = b + (int)threadIdx.x; j < b_max; j += kLaneThreads) rout[j] = 0.f;
}

template <int KP>
hipError_t run_walk(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                    const int32_t* cu_blocks, int n_seqs, int total_blocks, int max_blocks, int s,
                    const float* R_prev, float* R_out, hipStream_t st) {
  constexpr int ROWS = kWalkThreads / (KP / 8);
  const int n_row_tiles = (max_blocks + ROWS - 1) / ROWS;
  dim3 grid(n_row_tiles * hq * n_seqs);
  hipLaunchKernelGGL((walk_kernel<KP>), grid, dim3(kWalkThreads), 0, st, q_sk, k_sk, hq, hkv, k,
                     cu_blocks, n_seqs, total_blocks, n_row_tiles, s, R_prev, R_out,
                     1.0f / sqrtf((float)k));
  return hipGetLastError();
}

template <int KP>
hipError_t run_walk_row(const float* q_sk, const float* k_sk, int hq, int hkv, int k, int n_seqs,
                        const int32_t* cur_block, int b_max, int s, const float* r_prev,
                        float* r_out, hipStream_t st) {
  const dim3 grid(hq * n_seqs);
  if (k == KP && b_max <= 64 * LaneRows<KP>::value) {
    hipLaunchKernelGGL((walk_row_lane_kernel<KP>), grid, dim3(kLaneThreads), 0, st, q_sk, k_sk,
                       hq, hkv, cur_block, n_seqs, b_max, s, r_prev, r_out,
                       1.0f / sqrtf((float)k));
    return hipGetLastError();
  }
  // every row has b <= b_max blocks, so ceil(b_max / 256) bounds the segment length
  const int l_max = (b_max + kRowSeg - 1) / kRowSeg;
  if (k == KP && l_max <= 40 / (KP / 4))
    hipLaunchKernelGGL((walk_row_kernel<KP, true>), grid, dim3(kRowThreads), 0, st, q_sk, k_sk,
                       hq, hkv, k, cur_block, n_seqs, b_max, s, r_prev, r_out,
                       1.0f / sqrtf((float)k));
  else
    hipLaunchKernelGGL((walk_row_kernel<KP, false>), grid, dim3(kRowThreads), 0, st, q_sk, k_sk,
                       hq, hkv, k, cur_block, n_seqs, b_max, s, r_prev, r_out,
                       1.0f / sqrtf((float)k));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_walk(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                       const int32_t* cu_blocks, int n_seqs, int total_blocks, int max_blocks,
                       int s, const float* R_prev, float* R_out, hipStream_t st) {
  if (total_blocks == 0 || max_blocks == 0) return hipSuccess;
  if (k <= kWmK && (k & 3) == 0) {
    const int n_row_tiles = (max_blocks + kWmRows - 1) / kWmRows;
    dim3 grid(n_row_tiles * hq * n_seqs);
    auto launch = [&](auto k32, auto one) {
      hipLaunchKernelGGL((walk_mfma_kernel<decltype(k32)::value, decltype(one)::value>), grid,
                         dim3(256), 0, st, q_sk, k_sk, hq, hkv, k, cu_blocks, n_seqs,
                         total_blocks, n_row_tiles, s, R_prev, R_out, 1.0f / sqrtf((float)k));
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (k == kWmK) {
      if (n_row_tiles == 1) launch(T_{}, T_{});
      else launch(T_{}, F_{});
    } else {
      if (n_row_tiles == 1) launch(F_{}, T_{});
      else launch(F_{}, F_{});
    }
    return hipGetLastError();
  }
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
