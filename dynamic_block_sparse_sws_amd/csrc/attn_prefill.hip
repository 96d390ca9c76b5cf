// Block-sparse prefill attention (blog page "Scout Before You Attend",
// sections 4-5: the real attention runs on the original Q, K, V, but only over
// the key blocks selected for each query block).
//
// bf16 path: one workgroup per (query head, query block of B tokens), B/32
// wavefronts, each owning 32 query rows.  For every selected key block the
// workgroup stages K (row-major) and V (transposed) in LDS, then each wave
// runs a FlashAttention-style step on the matrix cores with
// v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T          (A = K rows from LDS, B = this wave's Q in registers)
//   online softmax       (a lane holds one query column: the row max over the
//                         block is 64 in-register values plus one cross-lane
//                         exchange with the other half-wave)
//   O^T += V^T P^T       (A = V^T from LDS, B = P^T straight from the S^T
//                         accumulators rounded to bf16; V^T's key order in LDS
//                         is permuted to match the accumulator layout, so P
//                         never moves between lanes)
// The causal mask is applied only on the diagonal block (the last entry of
// every list); a partial last block is zero-padded.  Workgroups are ordered
// longest list first, and the query heads of one KV head are mapped to the same
// XCD (workgroup id modulo 8) so their shared K/V blocks meet in one L2.
//
// fp32 path: a plain kernel, one thread per query row, key-by-key online
// softmax with K/V tiles staged in LDS; it exists for tight-tolerance checks.
#include "sws_common.h"

namespace sws {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// V^T tile: D rows (feature) x 128 key slots (256 bytes, no padding); the 16-byte
// chunks of a row are XOR-swizzled by the row so that both the transposed
// 8-byte writes (rows 8 apart) and the 16-byte MFMA operand reads (consecutive
// rows) spread over all banks.
__device__ __forceinline__ int vt_offset(int d, int key) {
  // key -> slot: within every 16 keys, groups of 4 are stored in the order
  // 0, 2, 1, 3 (keys 0-3, 8-11, 4-7, 12-15), matching the MFMA accumulator rows
  const int kg = (key >> 2) & 3;
  const int slot = (key & ~15) | ((((kg & 1) << 1) | (kg >> 1)) << 2) | (key & 3);
  const int chunk = slot >> 3;
  const int swz = (d ^ (d >> 3)) & 15;
  return d * 128 + ((chunk ^ swz) << 3) + (slot & 7);
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(2)))
void attn_prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                              const uint16_t* __restrict__ v,
                              const int32_t* __restrict__ cu_seqlens,
                              const int32_t* __restrict__ cu_blocks, int n_seqs,
                              int total_blocks, int hq, int hkv,
                              const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
                              int width, float scale_log2, uint16_t* __restrict__ out,
                              float* __restrict__ lse) {
  constexpr int NW = BLK / 32;
  constexpr int NT = NW * 64;
  constexpr int KSTR = D + 8;        // K row stride in elements (272 B for D = 128)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BLK * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * 128];

  const int G = hq / hkv;
  const int id = blockIdx.x;
  const int slot = id % hq;
  const int h = (slot % hkv) * G + slot / hkv;
  const int gb = total_blocks - 1 - id / hq;
  const int seq = seq_of_block(cu_blocks, n_seqs, gb);
  const int i = gb - cu_blocks[seq];
  const int tok0 = cu_seqlens[seq];
  const int n = cu_seqlens[seq + 1] - tok0;
  const int T = cu_seqlens[n_seqs];
  const int kvh = h / G;
  const int64_t qstride = (int64_t)hq * D;
  const int64_t kstride = (int64_t)hkv * D;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int qi = w * 32 + l32;          // query row within the block
  const int qrow = i * BLK + qi;        // query row within the sequence

  bf16x8_t qf[D / 16];
  {
    const uint16_t* qp = q + (int64_t)(tok0 + qrow) * qstride + (int64_t)h * D + hl * 8;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (qrow < n) raw = *reinterpret_cast<const u32x4_t*>(qp + dc * 16);
      qf[dc] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  floatx16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int nb = idx ? cnt[(int64_t)h * total_blocks + gb] : i + 1;
  const int32_t* lst = idx ? idx + ((int64_t)h * total_blocks + gb) * width : nullptr;
  const uint16_t* kbase = k + (int64_t)tok0 * kstride + (int64_t)kvh * D;
  const uint16_t* vbase = v + (int64_t)tok0 * kstride + (int64_t)kvh * D;

  for (int nn = 0; nn < nb; ++nn) {
    const int j = lst ? lst[nn] : nn;
    const int key0 = j * BLK;
    __syncthreads();
    // ---- stage K_j (row-major) ----
#pragma unroll
    for (int it = 0; it < (BLK * D / 8) / NT; ++it) {
      const int u = tid + it * NT;
      const int row = u / (D / 8);
      const int ch = u % (D / 8);
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (key0 + row < n) raw = *reinterpret_cast<const u32x4_t*>(kbase + (int64_t)(key0 + row) * kstride + ch * 8);
      *reinterpret_cast<u32x4_t*>(&Ks[row * KSTR + ch * 8]) = raw;
    }
    // ---- stage V_j transposed: 4 keys x 8 features per unit ----
#pragma unroll
    for (int it = 0; it < ((BLK / 4) * (D / 8)) / NT; ++it) {
      const int u = tid + it * NT;
      const int kg = u / (D / 8);
      const int ch = u % (D / 8);
      u32x4_t rr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int key = key0 + kg * 4 + t;
        rr[t] = u32x4_t{0u, 0u, 0u, 0u};
        if (key < n) rr[t] = *reinterpret_cast<const u32x4_t*>(vbase + (int64_t)key * kstride + ch * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2_t pk;
        pk[0] = __builtin_amdgcn_perm(rr[1][wd], rr[0][wd], sel);
        pk[1] = __builtin_amdgcn_perm(rr[3][wd], rr[2][wd], sel);
        *reinterpret_cast<u32x2_t*>(&Vt[vt_offset(ch * 8 + e, kg * 4)]) = pk;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T ----
    floatx16_t st[BLK / 32];
#pragma unroll
    for (int kt = 0; kt < BLK / 32; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kt][r] = 0.f;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&Ks[(kt * 32 + l32) * KSTR + dc * 16 + hl * 8]);
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], st[kt], 0, 0, 0);
      }
    }
    // ---- scale, causal mask on the diagonal block, running max ----
    const bool diag = (j == i);
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < BLK / 32; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        float sv = st[kt][r] * scale_log2;
        if (diag && key > qi) sv = -INFINITY;
        st[kt][r] = sv;
        mx = fmaxf(mx, sv);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    m_run = m_new;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int kc = 0; kc < BLK / 16; ++kc) {
      const int kt = kc >> 1;
      const int r0 = (kc & 1) * 8;
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(st[kt][r0 + e] - m_new);
        l_run += p[e];
      }
      u32x4_t pw;
      pw[0] = pack_bf16x2(p[0], p[1]);
      pw[1] = pack_bf16x2(p[2], p[3]);
      pw[2] = pack_bf16x2(p[4], p[5]);
      pw[3] = pack_bf16x2(p[6], p[7]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int d = dt * 32 + l32;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&Vt[vt_offset(d, kc * 16 + hl * 4)]);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[dt], 0, 0, 0);
      }
    }
  }

  // ---- finalise ----
  l_run += __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_run;
  if (qrow < n) {
    uint16_t* op = out + (int64_t)(tok0 + qrow) * qstride + (int64_t)h * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = dt * 32 + 8 * rg + 4 * hl;
        u32x2_t pk;
        pk[0] = pack_bf16x2(o[dt][rg * 4 + 0] * inv, o[dt][rg * 4 + 1] * inv);
        pk[1] = pack_bf16x2(o[dt][rg * 4 + 2] * inv, o[dt][rg * 4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(op + d0) = pk;
      }
    }
    if (lse && hl == 0) lse[(int64_t)h * T + tok0 + qrow] = (m_run + log2f(l_run)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 reference-precision kernel
// ---------------------------------------------------------------------------
template <int D, int BLK>
__global__ __launch_bounds__(BLK) void attn_prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_blocks, int n_seqs,
    int total_blocks, int hq, int hkv, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, int width, float scale, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int KT = 32;   // keys staged per step
  __shared__ float Ksh[KT][D + 1];
  __shared__ float Vsh[KT][D + 1];
  const int gb = blockIdx.x;
  const int h = blockIdx.y;
  const int G = hq / hkv;
  const int kvh = h / G;
  const int seq = seq_of_block(cu_blocks, n_seqs, gb);
  const int i = gb - cu_blocks[seq];
  const int tok0 = cu_seqlens[seq];
  const int n = cu_seqlens[seq + 1] - tok0;
  const int T = cu_seqlens[n_seqs];
  const int t = threadIdx.x;
  const int qrow = i * BLK + t;
  const bool active = qrow < n;
  float qv[D], acc[D];
  const float* qp = q + ((int64_t)(tok0 + qrow) * hq + h) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = active ? qp[e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int nb = idx ? cnt[(int64_t)h * total_blocks + gb] : i + 1;
  const int32_t* lst = idx ? idx + ((int64_t)h * total_blocks + gb) * width : nullptr;
  for (int nn = 0; nn < nb; ++nn) {
    const int j = lst ? lst[nn] : nn;
    for (int k0 = 0; k0 < BLK; k0 += KT) {
      __syncthreads();
      for (int e = t; e < KT * D; e += BLK) {
        const int row = e / D, c = e % D;
        const int key = j * BLK + k0 + row;
        const int64_t off = ((int64_t)(tok0 + key) * hkv + kvh) * D + c;
        Ksh[row][c] = key < n ? k[off] : 0.f;
        Vsh[row][c] = key < n ? v[off] : 0.f;
      }
      __syncthreads();
      for (int kk = 0; kk < KT; ++kk) {
        const int key = j * BLK + k0 + kk;
        if (key > qrow || key >= n) break;
        float sdot = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) sdot += qv[e] * Ksh[kk][e];
        sdot *= scale;
        if (sdot > m) {
          const float a = expf(m - sdot);
          l *= a;
#pragma unroll
          for (int e = 0; e < D; ++e) acc[e] *= a;
          m = sdot;
        }
        const float p = expf(sdot - m);
        l += p;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] += p * Vsh[kk][e];
      }
    }
  }
  if (active) {
    float* op = out + ((int64_t)(tok0 + qrow) * hq + h) * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < D; ++e) op[e] = acc[e] * inv;
    if (lse) lse[(int64_t)h * T + tok0 + qrow] = m + logf(l);
  }
}

template <int D, int BLK>
hipError_t run_bf16(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                    const int32_t* cu_blocks, int n_seqs, int total_blocks, int hq, int hkv,
                    const int32_t* idx, const int32_t* cnt, int width, float scale, void* out,
                    float* lse, hipStream_t st) {
  dim3 grid((unsigned)total_blocks * hq);
  hipLaunchKernelGGL((attn_prefill_bf16_kernel<D, BLK>), grid, dim3(BLK * 2), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), cu_seqlens, cu_blocks, n_seqs,
                     total_blocks, hq, hkv, idx, cnt, width, scale * kLog2e,
                     static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t run_f32(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                   const int32_t* cu_blocks, int n_seqs, int total_blocks, int hq, int hkv,
                   const int32_t* idx, const int32_t* cnt, int width, float scale, void* out,
                   float* lse, hipStream_t st) {
  dim3 grid(total_blocks, hq);
  hipLaunchKernelGGL((attn_prefill_f32_kernel<D, BLK>), grid, dim3(BLK), 0, st,
                     static_cast<const float*>(q), static_cast<const float*>(k),
                     static_cast<const float*>(v), cu_seqlens, cu_blocks, n_seqs, total_blocks,
                     hq, hkv, idx, cnt, width, scale, static_cast<float*>(out), lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill(const void* q, const void* k, const void* v, int dtype,
                               const int32_t* cu_seqlens, const int32_t* cu_blocks, int n_seqs,
                               int total_blocks, int max_blocks, int hq, int hkv, int d, int B,
                               const int32_t* idx, const int32_t* cnt, int width, float scale,
                               void* out, float* lse, hipStream_t st) {
  (void)max_blocks;
  if (total_blocks == 0) return hipSuccess;
#define SWS_DISPATCH(FN)                                                                      \
  if (d == 128 && B == 128) return FN<128, 128>(q, k, v, cu_seqlens, cu_blocks, n_seqs,     \
                                                total_blocks, hq, hkv, idx, cnt, width,     \
                                                scale, out, lse, st);                       \
  if (d == 128 && B == 64) return FN<128, 64>(q, k, v, cu_seqlens, cu_blocks, n_seqs,       \
                                              total_blocks, hq, hkv, idx, cnt, width, scale, \
                                              out, lse, st);                                \
  if (d == 64 && B == 128) return FN<64, 128>(q, k, v, cu_seqlens, cu_blocks, n_seqs,       \
                                              total_blocks, hq, hkv, idx, cnt, width, scale, \
                                              out, lse, st);                                \
  return FN<64, 64>(q, k, v, cu_seqlens, cu_blocks, n_seqs, total_blocks, hq, hkv, idx, cnt, \
                    width, scale, out, lse, st);
  if (dtype == SWS_BF16) {
    SWS_DISPATCH(run_bf16)
  }
  SWS_DISPATCH(run_f32)
#undef SWS_DISPATCH
}

}  // namespace sws
