// Block-sparse prefill attention (blog page "Scout Before You Attend",
// sections 4-5: the real attention runs on the original Q, K, V, but only over
// the key blocks selected for each query block).
//
// bf16 path: one workgroup per (query head, query block of B tokens), B/32
// wavefronts, each owning 32 query rows; at B = 64 (groups of two or more
// query heads per KV head) one workgroup per pair of query heads of a group,
// walking the merge of the two heads' lists so a block both selected is
// loaded once.  A pre-pass writes V transposed per
// block (keys in accumulator-row order) to a workspace.  The selected key
// blocks are walked in steps of 32 keys: the K and V^T tiles stream from
// memory straight into XOR-swizzled LDS tiles two steps ahead, through a ring
// of three tile pairs (one barrier per step).
// Each wave runs a FlashAttention-style
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
// B = 128 and for the paired B = 64 form the register budget is capped so
// three waves share each SIMD (the short 32-key steps keep the score registers
// small); the extra wave hides more of the softmax and load latency behind
// other waves' MFMAs.
//
// The fp32 path (plain fp32 arithmetic, for tight-tolerance checks and the
// small fp32 stack) is in attn_prefill_f32.hip.
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

template <int D, int BLK, int HP = 1>
struct PrefillTile {
  static constexpr int NW = BLK / 32 * HP;          // waves (32 query rows each)
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
typedef float float2_t __attribute__((ext_vector_type(2)));

// max(v, v of the lane 32 away): a lane's 16 scores and its partner's are the
// two halves of one query column.  (A lane shuffle, not v_permlane32_swap:
// given the same register as both operands this compiler folds the swap's
// two results into one, which drops the other half.)  Only a query block's
// first step and the rare rescale take it.
__device__ __forceinline__ float max_halves(float v) {
  return fmaxf(v, __shfl_xor(v, 32));
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
                                          int& ref_mode, int qi, int hl) {
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
    // three operand reads in flight ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int dc = 0; dc < D / 16 - 3; ++dc) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
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
  // (the first step of a query block takes the column maximum).  ref_mode is
  // wave-uniform: 0 before the first step, 1 when every column of the wave has
  // reference 0, 2 otherwise.
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  u32x4_t pw[KT / 16];
  auto exp_step = [&](float& l_acc, auto zero_ref) {
#pragma unroll
    for (int kc = 0; kc < KT / 16; ++kc) {
      const int kt = kc >> 1;
      const int r0 = (kc & 1) * 8;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float x0 = st[kt][r0 + e], x1 = st[kt][r0 + e + 1];
        if constexpr (!decltype(zero_ref)::value) {
          x0 -= m_run;
          x1 -= m_run;
        }
        const float2_t ex = {__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1)};
        const bf16x2_t pr = __builtin_convertvector(ex, bf16x2_t);
        l_acc = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_acc, false);
        pw[kc][e >> 1] = __builtin_bit_cast(uint32_t, pr);
      }
    }
  };
  float l_new = l_run;
  bool redo = ref_mode == 0;
  if (!redo) {
    if (ref_mode == 1) exp_step(l_new, std::true_type{});
    else exp_step(l_new, std::false_type{});
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
    const float m_new = ref_mode == 0 ? (fabsf(mx) <= kZeroRefRange ? 0.f : mx)
                                      : fmaxf(m_run, mx);
    const float alpha = ref_mode == 0 ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    m_run = m_new;
    ref_mode = __all(m_run == 0.f) ? 1 : 2;
    l_new = l_run;
    if (ref_mode == 1) exp_step(l_new, std::true_type{});
    else exp_step(l_new, std::false_type{});
  }
  l_run = l_new;
  // ---- O^T += V^T P^T ----
  {
    bf16x8_t a[KT / 16][D / 32];
#pragma unroll
    for (int kc = 0; kc < KT / 16; ++kc)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        a[kc][dt] = *reinterpret_cast<const bf16x8_t*>(vsb + v_rd[kc] + dt * 32 * KT * 2);
#pragma unroll
    for (int kc = 0; kc < KT / 16; ++kc)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a[kc][dt], __builtin_bit_cast(bf16x8_t, pw[kc]), o[dt], 0, 0, 0);
    // three operand reads in flight ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int i = 0; i < 8 - 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
  }
}

template <int D, int BLK, int HP>
__global__ __launch_bounds__(BLK * 2 * HP)
__attribute__((amdgpu_waves_per_eu(BLK == 128 || HP == 2 ? 3 : 2)))
void attn_prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                              const uint16_t* __restrict__ vt,
                              const int32_t* __restrict__ cu_seqlens,
                              const int32_t* __restrict__ cu_blocks, int n_seqs,
                              int total_blocks, int hq, int hkv,
                              const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
                              int width, float scale_log2, uint16_t* __restrict__ out,
                              float* __restrict__ lse) {
  using TL = PrefillTile<D, BLK, HP>;
  constexpr int NT = TL::NT, KT = TL::KT;
  constexpr int WH = BLK / 32;                        // waves per query head
  static_assert(TL::NSUB % 2 == 0, "an even number of pipeline steps per block");
  // Two buffers per operand as separate LDS objects, so the compiler can tell
  // that the reads of one buffer do not wait on the direct-to-LDS loads
  // filling the other.
  __shared__ __attribute__((aligned(16))) char Ks0[TL::TILE];
  __shared__ __attribute__((aligned(16))) char Ks1[TL::TILE];
  __shared__ __attribute__((aligned(16))) char Vs0[TL::TILE];
  __shared__ __attribute__((aligned(16))) char Vs1[TL::TILE];
  // a ring of three buffer pairs: the tiles of step t + 2 load while step t
  // computes
  __shared__ __attribute__((aligned(16))) char Ks2[TL::TILE];
  __shared__ __attribute__((aligned(16))) char Vs2[TL::TILE];

  // Workgroup -> (query head(s), query block).  HP = 2 pairs query heads
  // 2p and 2p + 1 of one KV group (the last pair of an odd group holds one
  // head): the pair walks the merge of its two lists, so a block both heads
  // selected is loaded once for both.
  const int G = hq / hkv;
  const int id = blockIdx.x;
  const int PPG = (G + HP - 1) / HP;                  // head slots per KV group
  const int nslot = hkv * PPG;
  const int slot = id % nslot;
  const int hfirst = (slot % hkv) * G + slot / hkv * HP;
  const int nheads = min(HP, (slot % hkv) * G + G - hfirst);   // 1 or HP
  const int gb = total_blocks - 1 - id / nslot;
  const int seq = seq_of_block(cu_blocks, n_seqs, gb);
  const int i = gb - cu_blocks[seq];
  const int blk0 = cu_blocks[seq];
  const int tok0 = cu_seqlens[seq];
  const int n = cu_seqlens[seq + 1] - tok0;
  const int T = cu_seqlens[n_seqs];
  const int kvh = hfirst / G;
  const int64_t qstride = (int64_t)hq * D;
  const int64_t kstride = (int64_t)hkv * D;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  // this wave's head in the workgroup (a lone head's partner waves idle)
  const int hs = HP == 1 ? 0 : __builtin_amdgcn_readfirstlane(w) / WH;
  const bool head_ok = HP == 1 || hs < nheads;
  const int h = HP == 1 ? hfirst : hfirst + min(hs, nheads - 1);
  const int qi = (HP == 1 ? w : w % WH) * 32 + l32;
  const int qrow = i * BLK + qi;

  // ---- this wave's Q rows as MFMA B operands ----
  bf16x8_t qf[D / 16];
  {
    const uint16_t* qp = q + (int64_t)(tok0 + qrow) * qstride + (int64_t)h * D + hl * 8;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (qrow < n && head_ok) raw = *reinterpret_cast<const u32x4_t*>(qp + dc * 16);
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
  uint32_t k_off[TL::LOADS], v_off[TL::LOADS];
#pragma unroll
  for (int u = 0; u < TL::LOADS; ++u) {
    const int qc = u * NT + tid;
    const int kr = qc / TL::KCH;
    const int kp = qc % TL::KCH;
    k_off[u] = (uint32_t)(kr * (int)kstride + (kp ^ row_swizzle<TL::KCH>(kr)) * 8) * 2u;
    const int vr = qc / TL::VCH;
    const int vp = qc % TL::VCH;
    v_off[u] = (uint32_t)(vr * BLK + (vp ^ row_swizzle<TL::VCH>(vr)) * 8) * 2u;
  }
  const uint16_t* kbase = k + (int64_t)tok0 * kstride + (int64_t)kvh * D;
  const uint16_t* vtbase = vt + ((int64_t)kvh * total_blocks + blk0) * D * BLK;
  const int wave_chunk = __builtin_amdgcn_readfirstlane(w) * 64 * 16;

  typedef __attribute__((address_space(3))) void lds_void_t;
  // Issue the loads of step `sub` of block j into LDS buffer pair (kd, vd),
  // through raw buffer resources (stride 0, the last word selecting 32-bit
  // data as untyped loads require): a scalar base per step plus a 32-bit
  // per-lane offset fixed for the whole kernel, so a step's loads cost no
  // vector address arithmetic.  The K resource covers only the step's rows
  // inside the sequence: rows past its end (only in the last, partial block,
  // which only its own query block selects, as its diagonal) read as zero,
  // and the causal mask removes those keys (their V^T is zero too).  (The
  // offsets are passed as converted values: given the captured array
  // element itself, the host pass of this compiler silently drops the
  // kernel's launch stub.)
  auto load_step = [&](int j, int sub, char* kd, char* vd) {
    const int row0 = j * BLK + sub * KT;
    // (uniform: said explicitly, or the resource is built per lane in a loop)
    const int valid = __builtin_amdgcn_readfirstlane(min(max(n - row0, 0), KT));
    const auto kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kbase + (int64_t)row0 * kstride), (short)0,
        (int)(valid * kstride * 2), 0x00020000);
#pragma unroll
    for (int u = 0; u < TL::LOADS; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void_t*)(kd + u * NT * 16 + wave_chunk), 16,
                                               (int)k_off[u], 0, 0, 0);
    // the step's V^T tile: D rows of KT keys inside the block's D x BLK tile
    const uint16_t* vs = vtbase + (int64_t)j * D * BLK + sub * KT;
    const auto vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vs), (short)0,
                                                      D * BLK * 2, 0x00020000);
#pragma unroll
    for (int u = 0; u < TL::LOADS; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t*)(vd + u * NT * 16 + wave_chunk), 16,
                                               (int)v_off[u], 0, 0, 0);
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
  int ref_mode = 0;

  // List entries are clamped to the causal blocks [0, i] and the count to
  // [0, min(width, i + 1)], so a malformed list gives a wrong answer, never a
  // stray access (a valid list is unchanged by the clamps).
  auto list_len = [&](int hh) {
    return idx ? min(max(cnt[(int64_t)hh * total_blocks + gb], 0), min(width, i + 1)) : i + 1;
  };
  auto list_of = [&](int hh) {
    return idx ? idx + ((int64_t)hh * total_blocks + gb) * width : nullptr;
  };

  // List entries come through the scalar cache: a vector-memory read would
  // wait for every tile load in flight.
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  constexpr int NS = TL::NSUB;
  constexpr int LPS = 2 * TL::LOADS;             // vector-memory loads per step per thread
  // Step t + 1's tiles are complete for the workgroup once every wave has
  // waited for its own loads of them (leaving step t + 2's in flight) and
  // passed the barrier.  (s_waitcnt through the builtin, so the compiler's
  // own wait placement knows which tile loads have completed; the immediate
  // is vmcnt(LPS) with the other counters left open: expcnt 7, lgkmcnt 15.)
  auto wait_next = [&]() {
    static_assert(LPS < 16, "vmcnt in the low bits");
    __builtin_amdgcn_s_waitcnt(0xF70 | LPS);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if constexpr (HP == 1) {
    const int nb = list_len(h);
    const int32_t* lst = list_of(h);
    auto entry = [&](int nn) {
      return lst ? min(max(((const_i32*)lst)[nn], 0), i) : nn;
    };
    const int nsteps = nb * NS;                  // step t: block entry(t / NS), keys (t % NS) KT..
    auto issue = [&](int t, char* kd, char* vd) { load_step(entry(t / NS), t % NS, kd, vd); };
    // Step t computes from buffer pair t % 3 while the tiles of step t + 2
    // stream into pair (t + 2) % 3, the one step t - 1 used.
    // (the last two steps issue the final step's tiles again, into the pair
    // no later step reads, so every step issues the same loads)
    auto step = [&](int t, const char* kc, const char* vc, char* kn, char* vn) {
      issue(min(t + 2, nsteps - 1), kn, vn);
      attn_step<D, BLK>(entry(t / NS) == i, kc, vc, (t % NS) * KT, qf, k_rd, v_rd, o, m_run,
                        l_run, ref_mode, qi, hl);
      wait_next();
    };
    if (nsteps > 0) {
      issue(0, Ks0, Vs0);
      issue(1, Ks1, Vs1);                        // every block has NS >= 2 steps
      wait_next();
    }
    for (int t = 0; t < nsteps; t += 3) {
      step(t, Ks0, Vs0, Ks2, Vs2);
      if (t + 1 < nsteps) step(t + 1, Ks1, Vs1, Ks0, Vs0);
      if (t + 2 < nsteps) step(t + 2, Ks2, Vs2, Ks1, Vs1);
    }
    __builtin_amdgcn_s_waitcnt(0xF70);           // no tile load outlives the loop
  } else {
    // The merge of the heads' ascending lists: each merged block carries a
    // mask of the heads that selected it; a wave computes a step only if its
    // head's bit is set, and every wave takes part in the loads and barriers.
    // Each merged block consumes at least one entry, so the walk ends after
    // at most nbA + nbB blocks whatever the lists hold.
    static_assert(NS == 2, "the paired form takes 64-token blocks: two steps per block");
    const int nbA = list_len(hfirst);
    const int nbB = nheads > 1 ? list_len(hfirst + 1) : 0;
    const int32_t* lA = list_of(hfirst);
    const int32_t* lB = nheads > 1 ? list_of(hfirst + 1) : nullptr;
    constexpr int kEnd = 0x7fffffff;
    int pa = 0, pb = 0;
    // the next merged block (kEnd past the end) and its head mask
    auto next_block = [&](int& jj, int& mm) {
      const int a = pa < nbA ? (lA ? min(max(((const_i32*)lA)[pa], 0), i) : pa) : kEnd;
      const int b = pb < nbB ? (lB ? min(max(((const_i32*)lB)[pb], 0), i) : pb) : kEnd;
      jj = min(a, b);
      mm = (a == jj ? 1 : 0) | (b == jj ? 2 : 0);
      pa += mm & 1;
      pb += mm >> 1;
    };
    const int my_bit = 1 << hs;
    int j, mask, jn, maskn;                      // the current block and the next
    next_block(j, mask);
    next_block(jn, maskn);
    int sub = 0;
    // Step (block j, sub) computes from one buffer pair while the tiles of
    // (jn, sub), two steps ahead, load into the pair the step before used
    // (past the last block the current block's tiles load again, into a pair
    // no later step reads, so every step issues the same loads).
    auto step = [&](const char* kc, const char* vc, char* kn, char* vn) {
      load_step(jn != kEnd ? jn : j, sub, kn, vn);
      if (mask & my_bit)                         // uniform over the wave
        attn_step<D, BLK>(j == i, kc, vc, sub * KT, qf, k_rd, v_rd, o, m_run, l_run, ref_mode,
                          qi, hl);
      wait_next();
      if (sub == 1) {
        j = jn;
        mask = maskn;
        next_block(jn, maskn);
      }
      sub ^= 1;
    };
    if (j != kEnd) {
      load_step(j, 0, Ks0, Vs0);
      load_step(j, 1, Ks1, Vs1);
      wait_next();
      for (;;) {
        step(Ks0, Vs0, Ks2, Vs2);
        if (j == kEnd) break;
        step(Ks1, Vs1, Ks0, Vs0);
        if (j == kEnd) break;
        step(Ks2, Vs2, Ks1, Vs1);
        if (j == kEnd) break;
      }
      __builtin_amdgcn_s_waitcnt(0xF70);         // no tile load outlives the loop
    }
  }

  // ---- finalise ----
  l_run += __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_run;
  if (qrow < n && head_ok) {
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
  // B = 64 with query-head groups of two or more: two query heads per
  // workgroup (their 2 x 2 waves share the tiles of the blocks both
  // selected); otherwise one head per workgroup (B / 32 waves)
  const int G = hq / hkv;
  auto launch = [&](auto hp) {
    constexpr int HP = decltype(hp)::value;
    dim3 grid((unsigned)total_blocks * hkv * ((G + HP - 1) / HP));
    hipLaunchKernelGGL((attn_prefill_bf16_kernel<D, BLK, HP>), grid, dim3(BLK * 2 * HP), 0, st,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), vt,
                       cu_seqlens, cu_blocks, n_seqs, total_blocks, hq, hkv, idx, cnt, width,
                       scale * kLog2e, static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
  };
  if constexpr (BLK == 64) {
    if (G >= 2) return launch(std::integral_constant<int, 2>{});
  }
  return launch(std::integral_constant<int, 1>{});
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
  if (dtype != SWS_BF16)
    return launch_attn_prefill_f32(q, k, v, cu_seqlens, cu_blocks, n_seqs, total_blocks, hq,
                                   hkv, d, B, idx, cnt, width, scale, out, lse, st);
  SWS_DISPATCH(run_bf16)
#undef SWS_DISPATCH
}

}  // namespace sws
