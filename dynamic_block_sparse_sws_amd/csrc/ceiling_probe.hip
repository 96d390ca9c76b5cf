// Ceiling probes for the roofline figures of the attention kernels (gfx950).
//
// A standalone program, not part of libsws.so: each probe is a register- or
// LDS-only loop that measures what one instruction mix can reach on this chip
// (with the clock it runs at, read from GRBM_GUI_ACTIVE when the program runs
// under a counter pass), so that a kernel's fraction of the published peak can
// be split into "what the mix allows" and "what the kernel loses".
//
//   mfma32      v_mfma_f32_32x32x16_bf16, 4 independent accumulators
//   mfma16      v_mfma_f32_16x16x32_bf16, 8 independent accumulators
//   mix<N>      4 x 32x32x16 MFMA plus N independent exp2 per loop trip
//               (the prefill attention step issues 16 MFMA and 16 exp2 per
//               32 x 32 score tile: 4 exp2 per 4 MFMA)
//   lds         ds_read_b128 bandwidth, conflict-free addresses
//   one<M,N>    one wave per SIMD (96 KB of LDS per block keeps one block per
//               CU): M MFMA and N exp2 per trip in the same wave, to see how
//               far one wave overlaps its own MFMA and transcendental work
//   mfma+lds<E> 16 MFMA per trip, each with its A operand read from LDS
//               (ds_read_b128, 1 KB per wave, the prefill step's ratio), plus E
//               exp2 per MFMA: the attention step's mix without its global
//               (L2 -> LDS) traffic
//   + fill      the same plus, per trip, 4 KB per wave copied from a 2 MB
//               (L2-resident) or a 64 MB (MALL-resident) buffer straight into
//               LDS (global_load_lds), the step's tile fill: 16 KB per
//               workgroup of 4 waves and 64 MFMA
//   rand<E>     mfma+lds<E> with random operands: the LDS tile and eight
//               per-lane B fragments (the step's Q fragments) hold hashed
//               bf16 values of random sign and mantissa, so the multipliers
//               toggle as they do on real data (the probes above repeat the
//               same operands, which draws less power)
//   hbm read    a 4 GiB buffer streamed once with 16-byte loads (grid-stride,
//               4 or 8 loads in flight per thread, 2048 or 8192 blocks), an xor
//               of the words kept per thread
//   hbm copy    a 2 GiB buffer copied to another with 16-byte accesses
//
// Every access stays inside the probe's own buffers; the loops have fixed
// trip counts.  Output: one line per probe with the time and the rate.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void operands(bf16x8_t& a, bf16x8_t& b) {
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(threadIdx.x * 1e-3f + e);
    b[e] = (__bf16)(e * 1e-3f);
  }
}

__global__ __launch_bounds__(256) void mfma32_probe(float* out, int iters) {
  bf16x8_t a, b;
  operands(a, b);
  floatx16_t acc[4];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma16_probe(float* out, int iters) {
  bf16x8_t a, b;
  operands(a, b);
  floatx4_t acc[8];
  for (int i = 0; i < 8; ++i)
    for (int r = 0; r < 4; ++r) acc[i][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i)
    for (int r = 0; r < 4; ++r) s += acc[i][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int NEXP>
__global__ __launch_bounds__(256) void mix_probe(float* out, int iters) {
  bf16x8_t a, b;
  operands(a, b);
  floatx16_t acc[4];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float x[16];
  for (int e = 0; e < 16; ++e) x[e] = -(float)(threadIdx.x % 7) * 0.01f - e * 0.001f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < NEXP; ++e) x[e % 16] = __builtin_amdgcn_exp2f(x[e % 16]) - 1.0f;
  }
  float s = 0.f;
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  for (int e = 0; e < 16; ++e) s += x[e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void lds_probe(float* out, int iters) {
  constexpr int N = 8192;                     // 32 KB
  __shared__ __attribute__((aligned(16))) float sm[N];
  for (int i = threadIdx.x; i < N; i += 256) sm[i] = i * 1e-3f;
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int base = (threadIdx.x * 4) & (N - 1);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // consecutive lanes read consecutive 16-byte slots; index < N - 3
      const float4 v =
          *reinterpret_cast<const float4*>(&sm[(base + u * 1024 + (it & 1) * 4) & (N - 4)]);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

template <int NMFMA, int NEXP>
__global__ __launch_bounds__(256) void one_wave_probe(float* out, int iters) {
  __shared__ float pad[24576];                // 96 KB: one block per CU
  pad[threadIdx.x] = 1.f;
  __syncthreads();
  bf16x8_t a, b;
  operands(a, b);
  floatx16_t acc[4];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float x[16];
  for (int e = 0; e < 16; ++e) x[e] = -(float)(threadIdx.x % 7) * 0.01f - e * 0.001f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NMFMA; ++i)
      acc[i % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i % 4], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < NEXP; ++e) x[e % 16] = __builtin_amdgcn_exp2f(x[e % 16]) - 1.0f;
  }
  float s = pad[(threadIdx.x + 1) % 256];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  for (int e = 0; e < 16; ++e) s += x[e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int EXP>
__global__ __launch_bounds__(256) void mfma_lds_probe(float* out, int iters) {
  constexpr int N = 512;                      // 16-byte operand chunks (8 KB)
  __shared__ __attribute__((aligned(16))) bf16x8_t tile[N];
  for (int i = threadIdx.x; i < N; i += 256) {
    bf16x8_t t;
    for (int e = 0; e < 8; ++e) t[e] = (__bf16)(i * 1e-3f + e);
    tile[i] = t;
  }
  __syncthreads();
  bf16x8_t a0, b;
  operands(a0, b);
  floatx16_t acc[4];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float x[16];
  for (int e = 0; e < 16; ++e) x[e] = -(float)(threadIdx.x % 7) * 0.01f - e * 0.001f;
  const int lane = threadIdx.x & 63;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // consecutive lanes, consecutive 16-byte chunks: conflict-free; index < N
      const bf16x8_t a = tile[(lane + i * 64 + (it & 7) * 8) & (N - 1)];
      acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i & 3], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < EXP; ++e) x[(i + e) % 16] = __builtin_amdgcn_exp2f(x[(i + e) % 16]) - 1.0f;
    }
  }
  float s = (float)a0[0];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  for (int e = 0; e < 16; ++e) s += x[e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// A bf16 of random sign and mantissa and magnitude in [0.25, 4) from a
// 32-bit integer hash of i (the "lowbias32" mixer).
__device__ __forceinline__ __bf16 random_bf16(uint32_t i) {
  i ^= i >> 16;
  i *= 0x7feb352du;
  i ^= i >> 15;
  i *= 0x846ca68bu;
  i ^= i >> 16;
  const uint16_t bits = (uint16_t)(((i >> 31) << 15) | ((125u + ((i >> 20) & 3u)) << 7) | (i & 0x7fu));
  return __builtin_bit_cast(__bf16, bits);
}

template <int EXP>
__global__ __launch_bounds__(256) void mfma_rand_probe(float* out, int iters) {
  constexpr int N = 512;                      // 16-byte operand chunks (8 KB)
  __shared__ __attribute__((aligned(16))) bf16x8_t tile[N];
  for (int i = threadIdx.x; i < N; i += 256) {
    bf16x8_t t;
    for (int e = 0; e < 8; ++e) t[e] = random_bf16((blockIdx.x * N + i) * 8 + e);
    tile[i] = t;
  }
  __syncthreads();
  bf16x8_t b[8];
  for (int f = 0; f < 8; ++f)
    for (int e = 0; e < 8; ++e)
      b[f][e] = random_bf16(0x9e3779b9u ^ (((blockIdx.x * 256 + threadIdx.x) * 8 + f) * 8 + e));
  floatx16_t acc[4];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float x[16];
  for (int e = 0; e < 16; ++e) x[e] = -(float)(threadIdx.x % 7) * 0.01f - e * 0.001f;
  const int lane = threadIdx.x & 63;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // consecutive lanes, consecutive 16-byte chunks: conflict-free; index < N
      const bf16x8_t a = tile[(lane + i * 64 + (it & 7) * 8) & (N - 1)];
      acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[i & 7], acc[i & 3], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < EXP; ++e) x[(i + e) % 16] = __builtin_amdgcn_exp2f(x[(i + e) % 16]) - 1.0f;
    }
  }
  float s = 0.f;
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  for (int e = 0; e < 16; ++e) s += x[e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__global__ __launch_bounds__(256) void mfma_lds_fill_probe(float* out, const uint4* src,
                                                           int src16, int iters) {
  constexpr int N = 512;                      // operand chunks (8 KB), read by the MFMAs
  __shared__ __attribute__((aligned(16))) bf16x8_t tile[N];
  __shared__ __attribute__((aligned(16))) char fill[4 * 1024];   // 1 KB per wave, rewritten
  for (int i = threadIdx.x; i < N; i += 256) {
    bf16x8_t t;
    for (int e = 0; e < 8; ++e) t[e] = (__bf16)(i * 1e-3f + e);
    tile[i] = t;
  }
  __syncthreads();
  bf16x8_t a0, b;
  operands(a0, b);
  floatx16_t acc[4];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float x[16];
  for (int e = 0; e < 16; ++e) x[e] = -(float)(threadIdx.x % 7) * 0.01f - e * 0.001f;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // src16 is a power of two; every index below is masked to it
  int pos = ((blockIdx.x * 4 + w) * 256) & (src16 - 1);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ci = (pos + u * 64 + lane) & (src16 - 1);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(src + ci), (lds_void_t*)(fill + w * 1024),
                                       16, 0, 0);
    }
    pos = (pos + 256) & (src16 - 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8_t a = tile[(lane + i * 64 + (it & 7) * 8) & (N - 1)];
      acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i & 3], 0, 0, 0);
      x[i] = __builtin_amdgcn_exp2f(x[i]) - 1.0f;
    }
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  float s = (float)a0[0];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  for (int e = 0; e < 16; ++e) s += x[e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Streams n16 16-byte words: each thread keeps U loads in flight per trip.
template <int U>
__global__ __launch_bounds__(256) void hbm_read_probe(const uint4* __restrict__ src, size_t n16,
                                                      unsigned* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void hbm_copy_probe(const uint4* __restrict__ src, size_t n16,
                                                      uint4* __restrict__ dst) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a; dst[i + stride] = b; dst[i + 2 * stride] = c; dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

#define CHECK(x)                                                                     \
  do {                                                                               \
    const hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                          \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
      std::exit(1);                                                                  \
    }                                                                                \
  } while (0)

}  // namespace

int main() {
  constexpr int kBlocks = 256 * 12;           // 12 blocks of 4 waves per CU
  constexpr int kIters = 20000;
  float* out = nullptr;
  CHECK(hipMalloc(&out, (size_t)kBlocks * 256 * sizeof(float)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  // rate = blocks x 4 waves x iterations x work per wave-iteration / time
  auto run = [&](const char* name, void (*kern)(float*, int), int blocks, double work,
                 const char* unit) {
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, 0, out, 100);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, 0, out, kIters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double rate = blocks * 4.0 * kIters * work / (ms * 1e-3);
    std::printf("%-36s %9.3f ms  %9.1f %-8s %8.1f ns/trip\n", name, ms, rate / 1e12, unit,
                ms * 1e6 / kIters);
  };
  const double f32x32 = 2.0 * 32 * 32 * 16, f16x16 = 2.0 * 16 * 16 * 32;
  run("mfma 32x32x16 bf16, 4 chains", mfma32_probe, kBlocks, 4 * f32x32, "TFLOP/s");
  run("mfma 16x16x32 bf16, 8 chains", mfma16_probe, kBlocks, 8 * f16x16, "TFLOP/s");
  run("mfma 32x32x16 x4 + 0 exp2", mix_probe<0>, kBlocks, 4 * f32x32, "TFLOP/s");
  run("mfma 32x32x16 x4 + 4 exp2", mix_probe<4>, kBlocks, 4 * f32x32, "TFLOP/s");
  run("mfma 32x32x16 x4 + 8 exp2", mix_probe<8>, kBlocks, 4 * f32x32, "TFLOP/s");
  run("mfma 32x32x16 x4 + 16 exp2", mix_probe<16>, kBlocks, 4 * f32x32, "TFLOP/s");
  run("mfma 32x32x16 x4 + 32 exp2", mix_probe<32>, kBlocks, 4 * f32x32, "TFLOP/s");
  run("lds ds_read_b128", lds_probe, kBlocks, 8 * 16.0 * 64, "TB/s");
  run("mfma + lds operand (1 KB per mfma)", mfma_lds_probe<0>, kBlocks, 16 * f32x32, "TFLOP/s");
  run("mfma + lds operand + 1 exp2 per mfma", mfma_lds_probe<1>, kBlocks, 16 * f32x32, "TFLOP/s");
  run("random operands: mfma + lds", mfma_rand_probe<0>, kBlocks, 16 * f32x32, "TFLOP/s");
  run("random operands: + 1 exp2 per mfma", mfma_rand_probe<1>, kBlocks, 16 * f32x32, "TFLOP/s");
  // the same mix plus the tile fill, from a 2 MB buffer (one XCD's L2 holds
  // it) and from a 64 MB one (past the L2s, inside the 256 MB MALL)
  for (const int mb : {2, 64}) {
    const int src16 = (mb << 20) / 16;
    uint4* src = nullptr;
    CHECK(hipMalloc(&src, (size_t)src16 * 16));
    CHECK(hipMemset(src, 0, (size_t)src16 * 16));
    hipLaunchKernelGGL(mfma_lds_fill_probe, dim3(kBlocks), dim3(256), 0, 0, out, src, src16, 100);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(mfma_lds_fill_probe, dim3(kBlocks), dim3(256), 0, 0, out, src, src16,
                       kIters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double flops = kBlocks * 4.0 * kIters * 16 * f32x32;
    const double fill_bytes = kBlocks * 4.0 * kIters * 4096;
    std::printf("mfma + lds + exp2 + fill from %2d MB %9.3f ms  %9.1f %-8s %8.1f TB/s fill\n", mb,
                ms, flops / (ms * 1e-3) / 1e12, "TFLOP/s", fill_bytes / (ms * 1e-3) / 1e12);
    CHECK(hipFree(src));
  }
  run("1 wave/SIMD: 8 mfma", one_wave_probe<8, 0>, 256, 8 * f32x32, "TFLOP/s");
  run("1 wave/SIMD: 16 exp2", one_wave_probe<0, 16>, 256, 0.0, "-");
  run("1 wave/SIMD: 8 mfma + 16 exp2", one_wave_probe<8, 16>, 256, 8 * f32x32, "TFLOP/s");
  run("1 wave/SIMD: 8 mfma + 32 exp2", one_wave_probe<8, 32>, 256, 8 * f32x32, "TFLOP/s");
  run("1 wave/SIMD: 32 exp2", one_wave_probe<0, 32>, 256, 0.0, "-");
  CHECK(hipFree(out));

  // HBM: 4 GiB read once, 2 GiB copied; 8 launches each after one untimed
  const size_t read_bytes = (size_t)4 << 30, copy_bytes = (size_t)2 << 30;
  uint4 *a = nullptr, *b = nullptr;
  unsigned* sink = nullptr;
  constexpr int kStreamBlocks = 256 * 32;   // largest grid of the stream probes
  CHECK(hipMalloc(&a, read_bytes));
  CHECK(hipMalloc(&b, copy_bytes));
  CHECK(hipMalloc(&sink, (size_t)kStreamBlocks * 256 * sizeof(unsigned)));
  CHECK(hipMemset(a, 1, read_bytes));
  CHECK(hipDeviceSynchronize());
  // mode 0: copy; otherwise a read with that many loads in flight per thread
  auto stream = [&](const char* name, int mode, int blocks) {
    const size_t n16 = (mode == 0 ? copy_bytes : read_bytes) / 16;
    auto launch = [&]() {
      if (mode == 0)
        hipLaunchKernelGGL(hbm_copy_probe, dim3(blocks), dim3(256), 0, 0, a, n16, b);
      else if (mode == 4)
        hipLaunchKernelGGL(hbm_read_probe<4>, dim3(blocks), dim3(256), 0, 0, a, n16, sink);
      else
        hipLaunchKernelGGL(hbm_read_probe<8>, dim3(blocks), dim3(256), 0, 0, a, n16, sink);
      CHECK(hipGetLastError());
    };
    launch();
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < 8; ++r) launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double bytes = 8.0 * (mode == 0 ? 2.0 * copy_bytes : (double)read_bytes);
    std::printf("%-36s %9.3f ms  %9.1f %-8s\n", name, ms / 8, bytes / (ms * 1e-3) / 1e9, "GB/s");
  };
  stream("hbm read, 4 in flight, 2048 blocks", 4, 2048);
  stream("hbm read, 4 in flight, 8192 blocks", 4, kStreamBlocks);
  stream("hbm read, 8 in flight, 2048 blocks", 8, 2048);
  stream("hbm read, 8 in flight, 8192 blocks", 8, kStreamBlocks);
  stream("hbm copy, 2 GiB (read + write)", 0, kStreamBlocks);
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  CHECK(hipFree(sink));
  return 0;
}
