// Block-sparse prefill attention in plain fp32 (blog page "Scout Before You
// Attend", sections 4-5: attention over the selected key blocks of each query
// block, on the original Q, K, V), for tight-tolerance checks and small fp32
// stacks.  Same lists, clamping and output layout as the bf16 kernel.
#include "sws_common.h"

namespace sws {
namespace {

// ---------------------------------------------------------------------------
// fp32 reference-precision kernel
// ---------------------------------------------------------------------------
// One workgroup per (query head, query block, group of kF32Rows = 8 rows):
// 256 threads, thread t owns row t % 8 and key slice t / 8 (32 slices), and
// takes keys slice and slice + 32 of every staged tile of 64 keys, each
// slice keeping its own online softmax (running maximum, sum, fp32
// accumulator).  The slices of a row are merged at the end through LDS: the
// row maximum over the slices, each slice's sum and accumulator scaled by
// exp(m - max), then summed.  Splitting a block's rows over workgroups and a
// row's keys over threads keeps the short, serial key walk of the plain
// one-thread-per-row form off the critical path when there are few heads
// and blocks (the single-head 1024-token stack has 16 query blocks).  A key
// tile is read once per 8 rows; all threads of a wave that share a slice
// read the same K/V row, so LDS reads are 8-way broadcasts.
constexpr int kF32Rows = 8;
constexpr int kF32Slices = 32;
constexpr int kF32Keys = 64;             // keys per staged tile
constexpr int kF32Threads = kF32Rows * kF32Slices;

template <int D, int BLK>
__global__ __launch_bounds__(kF32Threads) void attn_prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_blocks, int n_seqs,
    int total_blocks, int hq, int hkv, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, int width, float scale, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int P = D + 4;                        // LDS row pitch (16-byte rows, no conflicts)
  constexpr int NRG = BLK / kF32Rows;             // row groups per query block
  constexpr int V4 = kF32Keys * D / 4 / kF32Threads;   // float4 of K (and of V) per thread
  constexpr bool PREFETCH = D <= 64;              // next tile in registers while this one runs
  constexpr int MC = 16;                          // accumulator components merged per round
  static_assert(kF32Slices * kF32Rows * (MC + 1) <= kF32Keys * P, "merge area fits in Ks");
  __shared__ __attribute__((aligned(16))) float Ks[kF32Keys * P];
  __shared__ __attribute__((aligned(16))) float Vs[kF32Keys * P];
  __shared__ float mrow[kF32Slices][kF32Rows], lrow[kF32Slices][kF32Rows];

  const int gb = blockIdx.x / NRG;
  const int rg = blockIdx.x % NRG;
  const int h = blockIdx.y;
  const int G = hq / hkv;
  const int kvh = h / G;
  const int seq = seq_of_block(cu_blocks, n_seqs, gb);
  const int i = gb - cu_blocks[seq];
  const int tok0 = cu_seqlens[seq];
  const int n = cu_seqlens[seq + 1] - tok0;
  const int T = cu_seqlens[n_seqs];
  const int t = threadIdx.x;
  const int r = t % kF32Rows;
  const int g = t / kF32Rows;
  const int row0 = i * BLK + rg * kF32Rows;       // first row of the group
  if (row0 >= n) return;                          // whole group past the sequence (uniform)
  const int qrow = row0 + r;
  const bool active = qrow < n;
  const int last_row = min(row0 + kF32Rows, n) - 1;

  float qv[D], acc[D];
  const float* qp = q + ((int64_t)(tok0 + min(qrow, n - 1)) * hq + h) * D;
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    const float4 x = *reinterpret_cast<const float4*>(qp + e);
    qv[e] = x.x * scale; qv[e + 1] = x.y * scale; qv[e + 2] = x.z * scale; qv[e + 3] = x.w * scale;
  }
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;

  // list entries clamped to [0, i] and the count to [0, min(width, i + 1)]
  const int nb = idx ? min(max(cnt[(int64_t)h * total_blocks + gb], 0), min(width, i + 1))
                     : i + 1;
  const int32_t* lst = idx ? idx + ((int64_t)h * total_blocks + gb) * width : nullptr;
  // tiles: (list entry, 64-key part), skipping parts wholly after the group's last row
  constexpr int PARTS = BLK / kF32Keys;
  auto tile_key0 = [&](int tt) {
    const int nn = tt / PARTS;
    const int j = lst ? min(max(lst[nn], 0), i) : nn;
    return j * BLK + (tt % PARTS) * kF32Keys;
  };
  const int ntiles = nb * PARTS;

  // the K and V float4 of one tile held by this thread: the next tile, loaded
  // while the current one runs (PREFETCH), else loaded right before staging
  float4 kr[V4], vr[V4];
  auto fetch = [&](int key0) {
#pragma unroll
    for (int u = 0; u < V4; ++u) {
      const int e4 = t + u * kF32Threads;         // float4 index within the tile
      const int row = e4 / (D / 4), c4 = e4 % (D / 4);
      const int key = key0 + row;
      const int64_t off = ((int64_t)(tok0 + min(key, n - 1)) * hkv + kvh) * D + c4 * 4;
      const float4 kx = *reinterpret_cast<const float4*>(k + off);
      const float4 vx = *reinterpret_cast<const float4*>(v + off);
      const bool in = key < n;                    // rows past the sequence read as zero
      kr[u] = make_float4(in ? kx.x : 0.f, in ? kx.y : 0.f, in ? kx.z : 0.f, in ? kx.w : 0.f);
      vr[u] = make_float4(in ? vx.x : 0.f, in ? vx.y : 0.f, in ? vx.z : 0.f, in ? vx.w : 0.f);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < V4; ++u) {
      const int e4 = t + u * kF32Threads;
      const int row = e4 / (D / 4), c4 = e4 % (D / 4);
      *reinterpret_cast<float4*>(&Ks[row * P + c4 * 4]) = kr[u];
      *reinterpret_cast<float4*>(&Vs[row * P + c4 * 4]) = vr[u];
    }
  };

  if constexpr (PREFETCH) {
    if (ntiles > 0) fetch(tile_key0(0));
  }
  for (int tt = 0; tt < ntiles; ++tt) {
    const int key0 = tile_key0(tt);
    __syncthreads();                              // the previous tile's readers are done
    if constexpr (!PREFETCH) fetch(key0);
    stash();
    __syncthreads();
    if constexpr (PREFETCH) {
      if (tt + 1 < ntiles) fetch(tile_key0(tt + 1));
    }
    if (key0 > last_row) continue;                // every key of the tile is masked (uniform)
    const int ka = key0 + g, kb = key0 + g + kF32Slices;
    const float* Ka = &Ks[g * P];
    const float* Kb = &Ks[(g + kF32Slices) * P];
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(Ka + e);
      const float4 y = *reinterpret_cast<const float4*>(Kb + e);
      sa = fmaf(qv[e], x.x, sa); sa = fmaf(qv[e + 1], x.y, sa);
      sa = fmaf(qv[e + 2], x.z, sa); sa = fmaf(qv[e + 3], x.w, sa);
      sb = fmaf(qv[e], y.x, sb); sb = fmaf(qv[e + 1], y.y, sb);
      sb = fmaf(qv[e + 2], y.z, sb); sb = fmaf(qv[e + 3], y.w, sb);
    }
    sa = (ka <= qrow && ka < n) ? sa : -INFINITY;
    sb = (kb <= qrow && kb < n) ? sb : -INFINITY;
    const float mn = fmaxf(m, fmaxf(sa, sb));
    if (mn == -INFINITY) continue;                // nothing seen yet by this thread
    const float a = expf(m - mn);                 // m = -inf: 0
    const float pa = expf(sa - mn), pb = expf(sb - mn);
    l = l * a + (pa + pb);
    m = mn;
    const float* Va = &Vs[g * P];
    const float* Vb = &Vs[(g + kF32Slices) * P];
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(Va + e);
      const float4 y = *reinterpret_cast<const float4*>(Vb + e);
      acc[e] = fmaf(pb, y.x, fmaf(pa, x.x, acc[e] * a));
      acc[e + 1] = fmaf(pb, y.y, fmaf(pa, x.y, acc[e + 1] * a));
      acc[e + 2] = fmaf(pb, y.z, fmaf(pa, x.z, acc[e + 2] * a));
      acc[e + 3] = fmaf(pb, y.w, fmaf(pa, x.w, acc[e + 3] * a));
    }
  }

  // ---- merge the slices of each row ----
  mrow[g][r] = m;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll 8
  for (int x = 0; x < kF32Slices; ++x) M = fmaxf(M, mrow[x][r]);
  const float f = m == -INFINITY ? 0.f : expf(m - M);   // a row always sees its own key
  lrow[g][r] = l * f;
  __syncthreads();
  float L = 0.f;
#pragma unroll 8
  for (int x = 0; x < kF32Slices; ++x) L += lrow[x][r];
  const float inv = 1.0f / L;
  float* area = Ks;                               // [slice][row][MC + 1]
  // output component of this thread in a merge round: row r, component t / 8 (t < 128)
  const int oc = t / kF32Rows;
  float* op = out + ((int64_t)(tok0 + qrow) * hq + h) * D;
#pragma unroll
  for (int e0 = 0; e0 < D; e0 += MC) {
    __syncthreads();                              // Ks free (last tile) / previous round read
#pragma unroll
    for (int e = 0; e < MC; ++e) area[(g * kF32Rows + r) * (MC + 1) + e] = acc[e0 + e] * f;
    __syncthreads();
    if (oc < MC) {
      float sum = 0.f;
#pragma unroll 8
      for (int x = 0; x < kF32Slices; ++x) sum += area[(x * kF32Rows + r) * (MC + 1) + oc];
      if (active) op[e0 + oc] = sum * inv;
    }
  }
  if (lse && active && g == 0) lse[(int64_t)h * T + tok0 + qrow] = M + logf(L);
}

template <int D, int BLK>
hipError_t run_f32(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                   const int32_t* cu_blocks, int n_seqs, int total_blocks, int hq, int hkv,
                   const int32_t* idx, const int32_t* cnt, int width, float scale, void* out,
                   float* lse, hipStream_t st) {
  dim3 grid(total_blocks * (BLK / kF32Rows), hq);
  hipLaunchKernelGGL((attn_prefill_f32_kernel<D, BLK>), grid, dim3(kF32Threads), 0, st,
                     static_cast<const float*>(q), static_cast<const float*>(k),
                     static_cast<const float*>(v), cu_seqlens, cu_blocks, n_seqs, total_blocks,
                     hq, hkv, idx, cnt, width, scale, static_cast<float*>(out), lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill_f32(const void* q, const void* k, const void* v,
                                   const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                   int n_seqs, int total_blocks, int hq, int hkv, int d, int B,
                                   const int32_t* idx, const int32_t* cnt, int width,
                                   float scale, void* out, float* lse, hipStream_t st) {
  if (total_blocks == 0) return hipSuccess;
  if (d == 128 && B == 128)
    return run_f32<128, 128>(q, k, v, cu_seqlens, cu_blocks, n_seqs, total_blocks, hq, hkv, idx,
                             cnt, width, scale, out, lse, st);
  if (d == 128 && B == 64)
    return run_f32<128, 64>(q, k, v, cu_seqlens, cu_blocks, n_seqs, total_blocks, hq, hkv, idx,
                            cnt, width, scale, out, lse, st);
  if (d == 64 && B == 128)
    return run_f32<64, 128>(q, k, v, cu_seqlens, cu_blocks, n_seqs, total_blocks, hq, hkv, idx,
                            cnt, width, scale, out, lse, st);
  return run_f32<64, 64>(q, k, v, cu_seqlens, cu_blocks, n_seqs, total_blocks, hq, hkv, idx,
                         cnt, width, scale, out, lse, st);
}

}  // namespace sws
