// Walk variants for two readings the blog page "Scout Before You Attend"
// leaves open in section 4 (the walk update R^l = R^(l-1) (A^l)^s):
//   power    the exponent s read elementwise: R = rownorm(R_prev T),
//            T[i][j] = M[i][j]^s
//   softmax  the scores turned into transition probabilities: row i of T is
//            the softmax of M[i][0..i]; R = rownorm(R_prev T^s)
// with M[i][j] = qs_i . ks_j / sqrt(k) for j <= i.  Neither keeps the rank-k
// structure the default walk exploits, so T is formed explicitly.
//
// Prefill: transition_kernel writes T (one wave per block row, packed like R),
// tri_gemm_kernel multiplies lower-triangular matrices in 64 x 64 fp32 tiles
// staged in LDS (only the tiles J with m-tile <= J <= i-tile contribute), and
// rownorm_kernel divides each row of the last product by its largest
// magnitude into R_out.
//
// Decode: walk_row_variant_kernel, one workgroup per (sequence, query head),
// forms the needed entries of T on the fly from the sketch rows (the softmax
// row normalisers in a first pass) and applies the hops to the row vector.
#include "sws_common.h"

namespace sws {
namespace {

constexpr int kTile = 64;

__device__ __forceinline__ float powi(float x, int s) {
  float r = 1.0f;
  float b = x;
  while (s > 0) {
    if (s & 1) r *= b;
    b *= b;
    s >>= 1;
  }
  return r;
}

// T for one (sequence, head): wave per block row j; entries above the
// diagonal are written 0.
__global__ __launch_bounds__(256) void transition_kernel(
    const float* __restrict__ q_sk, const float* __restrict__ k_sk, int hq, int hkv, int k,
    const int32_t* __restrict__ cu_blocks, int total_blocks, int s, int mode, float inv_sqrt_k,
    float* __restrict__ T) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y;
  const int seq = blockIdx.z;
  const int b0 = cu_blocks[seq];
  const int b = cu_blocks[seq + 1] - b0;
  if (j >= b) return;
  const int g = h / (hq / hkv);
  const float* qrow = q_sk + ((int64_t)h * total_blocks + b0 + j) * k;
  const float* kbase = k_sk + ((int64_t)g * total_blocks + b0) * k;
  float* trow = T + walk_seq_offset(cu_blocks, seq, hq) + ((int64_t)h * b + j) * b;
  float qv[64];
#pragma unroll
  for (int e = 0; e < 64; ++e) qv[e] = e < k ? qrow[e] : 0.f;
  float mx = -INFINITY;
  for (int m = lane; m < b; m += 64) {
    float v = 0.f;
    if (m <= j) {
      const float* kr = kbase + (int64_t)m * k;
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 64; ++e)
        if (e < k) a += qv[e] * kr[e];
      v = a * inv_sqrt_k;
      mx = fmaxf(mx, v);
    }
    trow[m] = (m <= j) ? (mode == SWS_WALK_POWER ? powi(v, s) : v) : 0.f;
  }
  if (mode != SWS_WALK_SOFTMAX) return;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float sum = 0.f;
  for (int m = lane; m <= j; m += 64) {
    const float e = __expf(trow[m] - mx);
    trow[m] = e;
    sum += e;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  const float inv = 1.0f / sum;
  for (int m = lane; m <= j; m += 64) trow[m] *= inv;
}

// Y = X T for one (sequence, head), 64 x 64 output tile (I, Mt) per
// workgroup; X == nullptr is the identity.  Each thread owns a 4 x 4 block of
// the tile.
__global__ __launch_bounds__(256) void tri_gemm_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ T, int hq,
                                                       const int32_t* __restrict__ cu_blocks,
                                                       int tiles_max, float* __restrict__ Y) {
  __shared__ float Xs[kTile][kTile + 4];
  __shared__ __attribute__((aligned(16))) float Ts[kTile][kTile + 4];
  const int I = blockIdx.x / tiles_max;
  const int Mt = blockIdx.x % tiles_max;
  const int h = blockIdx.y;
  const int seq = blockIdx.z;
  const int b0 = cu_blocks[seq];
  const int b = cu_blocks[seq + 1] - b0;
  const int nt = (b + kTile - 1) / kTile;
  if (I >= nt || Mt >= nt) return;
  const int64_t off = walk_seq_offset(cu_blocks, seq, hq) + (int64_t)h * b * b;
  const float* Xh = X ? X + off : nullptr;
  const float* Th = T + off;
  float* Yh = Y + off;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  if (Mt <= I) {
    for (int J = Mt; J <= I; ++J) {
      for (int e = tid; e < kTile * kTile; e += 256) {
        const int r = e / kTile, c = e % kTile;
        const int gi = I * kTile + r, gj = J * kTile + c;
        float xv = 0.f;
        if (gi < b && gj < b) xv = Xh ? Xh[(int64_t)gi * b + gj] : (gi == gj ? 1.0f : 0.f);
        Xs[r][c] = xv;
        const int tj = J * kTile + r, tm = Mt * kTile + c;
        Ts[r][c] = (tj < b && tm < b) ? Th[(int64_t)tj * b + tm] : 0.f;
      }
      __syncthreads();
#pragma unroll 8
      for (int jj = 0; jj < kTile; ++jj) {
        float xa[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) xa[a] = Xs[ty * 4 + a][jj];
        const float4 tv = *reinterpret_cast<const float4*>(&Ts[jj][tx * 4]);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          acc[a][0] += xa[a] * tv.x;
          acc[a][1] += xa[a] * tv.y;
          acc[a][2] += xa[a] * tv.z;
          acc[a][3] += xa[a] * tv.w;
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int gi = I * kTile + ty * 4 + a;
    if (gi >= b) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int gm = Mt * kTile + tx * 4 + c;
      if (gm < b) Yh[(int64_t)gi * b + gm] = acc[a][c];
    }
  }
}

// dst row = src row / max |src row| (an all-zero row stays zero); wave per row
__global__ __launch_bounds__(256) void rownorm_kernel(const float* __restrict__ src, int hq,
                                                      const int32_t* __restrict__ cu_blocks,
                                                      float* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y;
  const int seq = blockIdx.z;
  const int b = cu_blocks[seq + 1] - cu_blocks[seq];
  if (i >= b) return;
  const int64_t off = walk_seq_offset(cu_blocks, seq, hq) + ((int64_t)h * b + i) * b;
  float mx = 0.f;
  for (int m = lane; m < b; m += 64) mx = fmaxf(mx, fabsf(src[off + m]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  for (int m = lane; m < b; m += 64) dst[off + m] = mx > 0.f ? src[off + m] / mx : 0.f;
}

// Decode: row c of the variant walk for one (sequence, query head).
constexpr int kVarRowThreads = 256;
constexpr int kVarRowBmax = 4096;

__global__ __launch_bounds__(kVarRowThreads) void walk_row_variant_kernel(
    const float* __restrict__ q_cache, const float* __restrict__ k_cache, int hq, int hkv, int k,
    const int32_t* __restrict__ cur_block, int b_max, int s, int mode, const float* r_prev,
    float* r_out, float inv_sqrt_k) {
  __shared__ float xs[kVarRowBmax];
  __shared__ float ys[kVarRowBmax];
  __shared__ float rmax[kVarRowBmax];     // softmax: row maximum of M[j][0..j]
  __shared__ float rinv[kVarRowBmax];     // softmax: 1 / row sum
  __shared__ float red[kVarRowThreads / 64];
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int c = cur_block[seq];
  const int b = c + 1;
  const int tid = threadIdx.x;
  const float* qb = q_cache + ((int64_t)seq * hq + h) * b_max * k;
  const float* kb = k_cache + ((int64_t)seq * hkv + h / (hq / hkv)) * b_max * k;
  const float* rin = r_prev ? r_prev + ((int64_t)seq * hq + h) * b_max : nullptr;
  float* rout = r_out + ((int64_t)seq * hq + h) * b_max;
  auto score = [&](int j, int m) -> float {
    const float* qr = qb + (int64_t)j * k;
    const float* kr = kb + (int64_t)m * k;
    float a = 0.f;
    for (int e = 0; e < k; ++e) a += qr[e] * kr[e];
    return a * inv_sqrt_k;
  };
  for (int j = tid; j < b; j += kVarRowThreads) xs[j] = rin ? rin[j] : (j == c ? 1.0f : 0.f);
  if (mode == SWS_WALK_SOFTMAX) {
    for (int j = tid; j < b; j += kVarRowThreads) {
      float mx = -INFINITY;
      for (int m = 0; m <= j; ++m) mx = fmaxf(mx, score(j, m));
      float sum = 0.f;
      for (int m = 0; m <= j; ++m) sum += __expf(score(j, m) - mx);
      rmax[j] = mx;
      rinv[j] = 1.0f / sum;
    }
  }
  __syncthreads();
  const int hops = mode == SWS_WALK_POWER ? 1 : s;
  for (int hop = 0; hop < hops; ++hop) {
    // y[m] = sum_{j = m .. c} x[j] T[j][m]
    for (int m = tid; m < b; m += kVarRowThreads) {
      float y = 0.f;
      for (int j = m; j <= c; ++j) {
        const float x = xs[j];
        if (x == 0.f) continue;
        const float v = score(j, m);
        const float t = mode == SWS_WALK_POWER ? powi(v, s) : __expf(v - rmax[j]) * rinv[j];
        y += x * t;
      }
      ys[m] = y;
    }
    __syncthreads();
    for (int m = tid; m < b; m += kVarRowThreads) xs[m] = ys[m];
    __syncthreads();
  }
  float mx = 0.f;
  for (int m = tid; m < b; m += kVarRowThreads) mx = fmaxf(mx, fabsf(xs[m]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  float g = 0.f;
#pragma unroll
  for (int w = 0; w < kVarRowThreads / 64; ++w) g = fmaxf(g, red[w]);
  for (int m = tid; m < b_max; m += kVarRowThreads) rout[m] = (m < b && g > 0.f) ? xs[m] / g : 0.f;
}

}  // namespace

size_t walk_variant_workspace_bytes(int64_t walk_numel) {
  return (size_t)walk_numel * 3 * sizeof(float);
}

hipError_t launch_walk_variant(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                               const int32_t* cu_blocks, int n_seqs, int total_blocks,
                               int max_blocks, int s, int mode, const float* R_prev,
                               float* R_out, int64_t walk_numel, void* ws, hipStream_t st) {
  if (total_blocks == 0 || max_blocks == 0) return hipSuccess;
  float* T = static_cast<float*>(ws);
  float* Y[2] = {T + walk_numel, T + 2 * walk_numel};
  const float inv_sqrt_k = 1.0f / sqrtf((float)k);
  hipLaunchKernelGGL(transition_kernel, dim3((max_blocks + 3) / 4, hq, n_seqs), dim3(256), 0, st,
                     q_sk, k_sk, hq, hkv, k, cu_blocks, total_blocks, s, mode, inv_sqrt_k, T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tiles = (max_blocks + kTile - 1) / kTile;
  const int hops = mode == SWS_WALK_POWER ? 1 : s;
  const float* X = R_prev;
  for (int hp = 0; hp < hops; ++hp) {
    hipLaunchKernelGGL(tri_gemm_kernel, dim3(tiles * tiles, hq, n_seqs), dim3(256), 0, st, X, T,
                       hq, cu_blocks, tiles, Y[hp & 1]);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    X = Y[hp & 1];
  }
  hipLaunchKernelGGL(rownorm_kernel, dim3((max_blocks + 3) / 4, hq, n_seqs), dim3(256), 0, st, X,
                     hq, cu_blocks, R_out);
  return hipGetLastError();
}

hipError_t launch_walk_row_variant(const float* q_sk, const float* k_sk, int hq, int hkv, int k,
                                   int n_seqs, const int32_t* cur_block, int b_max, int s,
                                   int mode, const float* r_prev, float* r_out, hipStream_t st) {
  if (n_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(walk_row_variant_kernel, dim3(hq, n_seqs), dim3(kVarRowThreads), 0, st,
                     q_sk, k_sk, hq, hkv, k, cur_block, b_max, s, mode, r_prev, r_out,
                     1.0f / sqrtf((float)k));
  return hipGetLastError();
}

}  // namespace sws
