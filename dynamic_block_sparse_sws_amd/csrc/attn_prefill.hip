// Block-sparse prefill attention (blog page "Scout Before You Attend",
// sections 4-5: the real attention runs on the original Q, K, V, but only over
// the key blocks selected for each query block).
//
// bf16 path: one workgroup per (query head, query block of B tokens), B/32
// wavefronts, each owning 32 query rows.  A pre-pass writes V transposed per
// block (keys in accumulator-row order) to a workspace.  The selected key
// blocks are walked in steps of 32 keys: the K and V^T tiles of the next step
// stream from memory straight into the other half of a double-buffered,
// XOR-swizzled LDS tile pair while the current step computes (one barrier per
// step).  Each wave runs a FlashAttention-style
// step on the matrix cores with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T          (A = K rows from LDS, B = this wave's Q in registers)
//   online softmax       (Q is pre-scaled by scale * log2(e), so scores are
//                         in log2 units; a lane holds one query column; the
//                         reference max is fixed after a query block's first
//                         step, at 0 when that step's maximum is within +-64,
//                         and only raised if the running sum nears overflow)
//   O^T += V^T P^T       (A = V^T from LDS, B = P^T straight from the S^T
//                         accumulators rounded to bf16; V^T's key order in LDS
//                         is permuted to match the accumulator layout, so P
//                         never moves between lanes)
// The causal mask is applied only on the diagonal block (the last entry of
// every list); a partial last block is zero-padded.  Workgroups are ordered
// longest list first, and the query heads of one KV head are mapped to the same
// XCD (workgroup id modulo 8) so their shared K/V blocks meet in one L2.  For
// B = 128 the register budget is capped so three waves share each SIMD (the
// short 32-key steps keep the score registers small); the extra wave hides
// more of the softmax and load latency behind other waves' MFMAs.
//
// fp32 path: a plain kernel, one thread per query row, key-by-key online
// softmax with K/V tiles staged in LDS; it exists for tight-tolerance checks.
#include "sws_common.h"

#include <type_traits>

namespace sws {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Key order inside every 16 keys of a V^T row: groups of 4 keys stored as
// 0-3, 8-11, 4-7, 12-15, which is the row order of the 32x32 MFMA accumulator
// halves, so a lane's P^T operand (taken straight from its S^T accumulators)
// lines up with 8 contiguous V^T slots.
__device__ __forceinline__ int vt_slot_key(int slot) {
  const int g = (slot >> 2) & 3;
  return (slot & ~15) | ((((g & 1) << 1) | (g >> 1)) << 2) | (slot & 3);
}

// Pre-pass: V [T][hkv][D] -> V^T blocks vt[hkv][total_blocks][D][BLK] (keys in
// slot order, zero past the end of the sequence).
template <int D, int BLK>
__global__ __launch_bounds__(256) void v_transpose_kernel(
    const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int n_seqs, int total_blocks, int hkv,
    uint16_t* __restrict__ vt) {
  __shared__ uint16_t tile[D][BLK + 2];
  const int gb = blockIdx.x;
  const int g = blockIdx.y;
  const int seq = seq_of_block(cu_blocks, n_seqs, gb);
  const int i = gb - cu_blocks[seq];
  const int tok0 = cu_seqlens[seq];
  const int n = cu_seqlens[seq + 1] - tok0;
  const int64_t rstride = (int64_t)hkv * D;
  for (int u = threadIdx.x; u < BLK * (D / 8); u += 256) {
    const int key = u / (D / 8);
    const int ch = u % (D / 8);
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (i * BLK + key < n)
      raw = *reinterpret_cast<const u32x4_t*>(v + (int64_t)(tok0 + i * BLK + key) * rstride + (int64_t)g * D + ch * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[ch * 8 + 2 * e][key] = (uint16_t)(raw[e] & 0xffffu);
      tile[ch * 8 + 2 * e + 1][key] = (uint16_t)(raw[e] >> 16);
    }
  }
  __syncthreads();
  uint16_t* dst = vt + ((int64_t)g * total_blocks + gb) * D * BLK;
  for (int u = threadIdx.x; u < D * (BLK / 8); u += 256) {
    const int d = u / (BLK / 8);
    const int c = u % (BLK / 8);
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[d][vt_slot_key(c * 8 + 2 * e)];
      const uint32_t hi = tile[d][vt_slot_key(c * 8 + 2 * e + 1)];
      w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4_t*>(dst + (int64_t)d * BLK + c * 8) = w;
  }
}

template <int D, int BLK>
struct PrefillTile {
  static constexpr int NW = BLK / 32;               // waves (32 query rows each)
  static constexpr int NT = NW * 64;
  static constexpr int KT = 32;                     // keys per pipeline step
  static constexpr int NSUB = BLK / KT;             // steps per selected block
  static constexpr int KCH = D / 8;                 // 16-byte chunks per K row
  static constexpr int VCH = KT / 8;                // 16-byte chunks per V^T row of a step
  static constexpr int TILE = KT * D * 2;           // bytes of one K (or V^T) step tile
  static constexpr int LOADS = TILE / 16 / NT;      // 16-byte loads per thread per tile
};

// XOR swizzles of the 16-byte chunks of a tile row, chosen so that the 16
// lanes of an MFMA operand read (16 consecutive rows, same logical chunk) hit
// 16 distinct 4-bank groups.
template <int CH>
__device__ __forceinline__ int row_swizzle(int row) {
  if (CH == 16) return row & 15;          // 256-byte rows
  if (CH == 8) return (row >> 1) & 7;     // 128-byte rows: two rows share a bank line
  return (row >> 2) & 3;                  // 64-byte rows
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// max(v, v of the lane 32 away): v_permlane32_swap exchanges the two halves
// of the wave in registers (no LDS round trip); the larger of the swapped pair
// is the answer in either half.
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}

// Softmax reference: after the first step of a query block the reference m
// used for the exponentials stays fixed, and the weights exp2(s - m) are
// formed without the step's column maximum; only when the running sum could
// overflow (it passes 2^100, or is not finite) is the step redone with the
// maximum and a rescale of the output accumulators.  Numerator, denominator
// and log-sum-exp all use the same reference, so the result is unchanged up to
// rounding (fp32 and bf16 keep the same relative precision at any exponent).
// When the first step's maximum lies within +-kZeroRefRange the reference is
// exactly 0: the weights are then exp2(s) with no subtraction (a wave takes
// that form when all its columns have reference 0), and 2^-64 .. 2^64 weights
// plus sums below 2^100 stay far inside the fp32 and bf16 range.
constexpr float kSumLimit = 0x1p100f;
constexpr float kZeroRefRange = 64.f;

// One pipeline step: KT keys of the current block against this wave's 32
// query rows.  ksb / vsb are the step's K and V^T tiles in LDS.
template <int D, int BLK>
__device__ __forceinline__ void attn_step(bool diag, const char* ksb, const char* vsb, int key_base,
                                          const bf16x8_t (&qf)[D / 16],
                                          const int (&k_rd)[D / 16],
                                          const int (&v_rd)[PrefillTile<D, BLK>::KT / 16],
                                          floatx16_t (&o)[D / 32], float& m_run, float& l_run,
                                          int qi, int hl) {
  constexpr int KT = PrefillTile<D, BLK>::KT;
  // ---- S^T = K Q^T ----
  floatx16_t st[KT / 32];
#pragma unroll
  for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st[kt][r] = 0.f;
  static_assert(KT == 32, "one S tile per step");
  {
    bf16x8_t a[D / 16];
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      a[dc] = *reinterpret_cast<const bf16x8_t*>(ksb + k_rd[dc]);
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[dc], qf[dc], st[0], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int dc = 0; dc < D / 16 - 2; ++dc) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
  // ---- causal mask (diagonal block only) ----
  if (diag) {
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key_base + kt * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (key > qi) st[kt][r] = -INFINITY;
      }
  }
  // ---- P = exp2(S * scale - m), bf16; row sum from the same bf16 values ----
  // (the first step of a query block takes the column maximum)
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8_t pb[KT / 16];
  auto exp_step = [&](float& l_acc, auto zero_ref) {
#pragma unroll
    for (int kc = 0; kc < KT / 16; ++kc) {
      const int kt = kc >> 1;
      const int r0 = (kc & 1) * 8;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        bf16x2_t pr;
        if constexpr (decltype(zero_ref)::value) {
          pr[0] = (__bf16)__builtin_amdgcn_exp2f(st[kt][r0 + e]);
          pr[1] = (__bf16)__builtin_amdgcn_exp2f(st[kt][r0 + e + 1]);
        } else {
          pr[0] = (__bf16)__builtin_amdgcn_exp2f(st[kt][r0 + e] - m_run);
          pr[1] = (__bf16)__builtin_amdgcn_exp2f(st[kt][r0 + e + 1] - m_run);
        }
        l_acc = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_acc, false);
        pb[kc][e] = pr[0];
        pb[kc][e + 1] = pr[1];
      }
    }
  };
  auto exp_any = [&](float& l_acc) {
    if (__all(m_run == 0.f)) exp_step(l_acc, std::true_type{});
    else exp_step(l_acc, std::false_type{});
  };
  float l_new = l_run;
  bool redo = m_run == -INFINITY;
  if (!redo) {
    exp_any(l_new);
    redo = __any(!(l_new < kSumLimit));
  }
  if (redo) {
    float mx = st[0][0];
#pragma unroll
    for (int kt = 0; kt < KT / 32; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kt][r]);
    mx = max_halves(mx);
    // a query block's first step takes the reference 0 when its maximum is
    // within +-64 (no subtraction in the later steps' exponentials), else the
    // maximum itself
    const float m_new = m_run == -INFINITY ? (fabsf(mx) <= kZeroRefRange ? 0.f : mx)
                                           : fmaxf(m_run, mx);
    const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    m_run = m_new;
    l_new = l_run;
    exp_any(l_new);
  }
  l_run = l_new;
  // ---- O^T += V^T P^T ----
#pragma unroll
  for (int kc = 0; kc < KT / 16; ++kc) {
    bf16x8_t a[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      a[dt] = *reinterpret_cast<const bf16x8_t*>(vsb + v_rd[kc] + dt * 32 * KT * 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[dt], pb[kc], o[dt], 0, 0, 0);
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(BLK == 128 ? 3 : 2)))
void attn_prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                              const uint16_t* __restrict__ vt,
                              const int32_t* __restrict__ cu_seqlens,
                              const int32_t* __restrict__ cu_blocks, int n_seqs,
                              int total_blocks, int hq, int hkv,
                              const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
                              int width, float scale_log2, uint16_t* __restrict__ out,
                              float* __restrict__ lse) {
  using TL = PrefillTile<D, BLK>;
  constexpr int NT = TL::NT, KT = TL::KT;
  static_assert(TL::NSUB % 2 == 0, "an even number of pipeline steps per block");
  // Two buffers per operand as separate LDS objects, so the compiler can tell
  // that the reads of one buffer do not wait on the direct-to-LDS loads
  // filling the other.
  __shared__ __attribute__((aligned(16))) char Ks0[TL::TILE];
  __shared__ __attribute__((aligned(16))) char Ks1[TL::TILE];
  __shared__ __attribute__((aligned(16))) char Vs0[TL::TILE];
  __shared__ __attribute__((aligned(16))) char Vs1[TL::TILE];

  const int G = hq / hkv;
  const int id = blockIdx.x;
  const int slot = id % hq;
  const int h = (slot % hkv) * G + slot / hkv;
  const int gb = total_blocks - 1 - id / hq;
  const int seq = seq_of_block(cu_blocks, n_seqs, gb);
  const int i = gb - cu_blocks[seq];
  const int blk0 = cu_blocks[seq];
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
  const int qi = w * 32 + l32;
  const int qrow = i * BLK + qi;

  // ---- this wave's Q rows as MFMA B operands ----
  bf16x8_t qf[D / 16];
  {
    const uint16_t* qp = q + (int64_t)(tok0 + qrow) * qstride + (int64_t)h * D + hl * 8;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (qrow < n) raw = *reinterpret_cast<const u32x4_t*>(qp + dc * 16);
      // scaled once by scale * log2(e) (rounded to bf16), so the scores come
      // out of the matrix cores in log2 units
      qf[dc] = __builtin_bit_cast(bf16x8_t, raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[dc][e] = (__bf16)((float)qf[dc][e] * scale_log2);
    }
  }

  // ---- staging geometry: load u of this thread fills tile chunk u * NT + tid ----
  // The tiles go global -> LDS directly (global_load_lds_dwordx4): lane l of
  // wave w writes the 16 bytes at chunk u * NT + 64 w + l, so the XOR swizzle
  // of the LDS layout is applied to the global source column instead.
  int k_roff[TL::LOADS], k_col[TL::LOADS];
  uint32_t v_off[TL::LOADS];
#pragma unroll
  for (int u = 0; u < TL::LOADS; ++u) {
    const int qc = u * NT + tid;
    const int kr = qc / TL::KCH;
    const int kp = qc % TL::KCH;
    k_roff[u] = kr * (int)kstride;
    k_col[u] = (kp ^ row_swizzle<TL::KCH>(kr)) * 8;
    const int vr = qc / TL::VCH;
    const int vp = qc % TL::VCH;
    v_off[u] = (uint32_t)(vr * BLK + (vp ^ row_swizzle<TL::VCH>(vr)) * 8);
  }
  const uint16_t* kbase = k + (int64_t)tok0 * kstride + (int64_t)kvh * D;
  const uint16_t* vtbase = vt + ((int64_t)kvh * total_blocks + blk0) * D * BLK;
  const int wave_chunk = __builtin_amdgcn_readfirstlane(w) * 64 * 16;

  typedef __attribute__((address_space(3))) void lds_void_t;
  typedef __attribute__((address_space(1))) void glb_void_t;
  // Issue the loads of step `sub` of block j into LDS buffer pair (kd, vd).
  // Rows past the end of the sequence (only in the last, partial block, which
  // only its own query block selects, as its diagonal) re-read the last row:
  // the causal mask removes those keys and their V^T is zero.
  auto load_step = [&](int j, int sub, char* kd, char* vd) {
    // offsets from the block's first row: block j holds at least one token,
    // so the clamp row n - 1 - j * BLK is >= 0 and every offset is
    // non-negative (a sub-step of a partial block may start past the end)
    const uint16_t* ks = kbase + (int64_t)j * BLK * kstride;
    const uint16_t* vs = vtbase + (int64_t)j * D * BLK + sub * KT;
    // (the row distance is clamped to the block first: every offset below is
    // under BLK rows anyway, and the product stays in 32 bits at any length)
    const int last_off = min(n - 1 - j * BLK, BLK - 1) * (int)kstride;
    const int sub_off = sub * KT * (int)kstride;
#pragma unroll
    for (int u = 0; u < TL::LOADS; ++u) {
      // 32-bit byte offsets from a uniform base (scalar base + vector offset)
      const uint32_t kb = (uint32_t)(min(sub_off + k_roff[u], last_off) + k_col[u]) * 2u;
      __builtin_amdgcn_global_load_lds((glb_void_t*)(reinterpret_cast<const char*>(ks) + kb),
                                       (lds_void_t*)(kd + u * NT * 16 + wave_chunk), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (glb_void_t*)(reinterpret_cast<const char*>(vs) + v_off[u] * 2u),
          (lds_void_t*)(vd + u * NT * 16 + wave_chunk), 16, 0, 0);
    }
  };
  // A step's tiles are complete for the workgroup once every wave has waited
  // for its own loads and passed the barrier.
  auto step_barrier = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // ---- per-lane LDS read offsets (bytes) of the MFMA A operands ----
  const int ksw = row_swizzle<TL::KCH>(l32);
  const int vsw = row_swizzle<TL::VCH>(l32);
  int k_rd[D / 16], v_rd[KT / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) k_rd[dc] = l32 * (D * 2) + (((2 * dc + hl) ^ ksw) << 4);
#pragma unroll
  for (int kc = 0; kc < KT / 16; ++kc) v_rd[kc] = l32 * (KT * 2) + (((2 * kc + hl) ^ vsw) << 4);

  floatx16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int nb = idx ? cnt[(int64_t)h * total_blocks + gb] : i + 1;
  const int32_t* lst = idx ? idx + ((int64_t)h * total_blocks + gb) * width : nullptr;

  // Step sub of a block uses LDS buffer pair sub % 2; while it computes, the
  // next step (the block's next sub-step, or the first of the next block)
  // streams into the other pair.
  int j = lst ? lst[0] : 0;
  load_step(j, 0, Ks0, Vs0);
  step_barrier();
  for (int nn = 0; nn < nb; ++nn) {
    const bool has_next = nn + 1 < nb;
    const int j_next = has_next ? (lst ? lst[nn + 1] : nn + 1) : j;
#pragma unroll
    for (int sub = 0; sub < TL::NSUB; ++sub) {
      const bool odd = sub & 1;
      const bool last_sub = sub + 1 == TL::NSUB;
      if (!last_sub) load_step(j, sub + 1, odd ? Ks0 : Ks1, odd ? Vs0 : Vs1);
      else if (has_next) load_step(j_next, 0, odd ? Ks0 : Ks1, odd ? Vs0 : Vs1);
      attn_step<D, BLK>(j == i, odd ? Ks1 : Ks0, odd ? Vs1 : Vs0, sub * KT, qf, k_rd, v_rd, o,
                        m_run, l_run, qi, hl);
      step_barrier();
    }
    j = j_next;
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
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        bf16x4_t pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(o[dt][rg * 4 + e] * inv);
        *reinterpret_cast<bf16x4_t*>(op + d0) = pk;
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
                    float* lse, void* ws, hipStream_t st) {
  uint16_t* vt = static_cast<uint16_t*>(ws);
  hipLaunchKernelGGL((v_transpose_kernel<D, BLK>), dim3(total_blocks, hkv), dim3(256), 0, st,
                     static_cast<const uint16_t*>(v), cu_seqlens, cu_blocks, n_seqs,
                     total_blocks, hkv, vt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)total_blocks * hq);
  hipLaunchKernelGGL((attn_prefill_bf16_kernel<D, BLK>), grid, dim3(BLK * 2), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), vt,
                     cu_seqlens, cu_blocks, n_seqs, total_blocks, hq, hkv, idx, cnt, width,
                     scale * kLog2e, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t run_f32(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                   const int32_t* cu_blocks, int n_seqs, int total_blocks, int hq, int hkv,
                   const int32_t* idx, const int32_t* cnt, int width, float scale, void* out,
                   float* lse, void* ws, hipStream_t st) {
  (void)ws;
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
                               void* out, float* lse, void* ws, hipStream_t st) {
  (void)max_blocks;
  if (total_blocks == 0) return hipSuccess;
#define SWS_DISPATCH(FN)                                                                      \
  if (d == 128 && B == 128) return FN<128, 128>(q, k, v, cu_seqlens, cu_blocks, n_seqs,     \
                                                total_blocks, hq, hkv, idx, cnt, width,     \
                                                scale, out, lse, ws, st);                       \
  if (d == 128 && B == 64) return FN<128, 64>(q, k, v, cu_seqlens, cu_blocks, n_seqs,       \
                                              total_blocks, hq, hkv, idx, cnt, width, scale, \
                                              out, lse, ws, st);                            \
  if (d == 64 && B == 128) return FN<64, 128>(q, k, v, cu_seqlens, cu_blocks, n_seqs,       \
                                              total_blocks, hq, hkv, idx, cnt, width, scale, \
                                              out, lse, ws, st);                            \
  return FN<64, 64>(q, k, v, cu_seqlens, cu_blocks, n_seqs, total_blocks, hq, hkv, idx, cnt, \
                    width, scale, out, lse, ws, st);
  if (dtype == SWS_BF16) {
    SWS_DISPATCH(run_bf16)
  }
  SWS_DISPATCH(run_f32)
#undef SWS_DISPATCH
}

}  // namespace sws
