// Block-sparse single-token decode attention (blog page "Scout Before You
// Attend", section 5: the same block selection for every decode step; section
// 8.3: decode is bound by reading the KV cache).
//
// Split-KV over the union lists of all (sequence, KV head) pairs at once: the
// blocks to read across the pairs are numbered and cut into equal ranges, one
// per workgroup; each workgroup computes, for all query heads of the group
// that kept each block, the partial softmax state (max, sum, weighted V sum)
// of every pair its range touches, reading every K and V row once for the
// whole group.  A combine kernel merges the partial states of each pair with
// the usual log-sum-exp rescaling.  bf16 queries (bf16 or fp8 e4m3 caches,
// contiguous or paged) run the matrix-core split kernel; fp32 queries run a
// vector-ALU split kernel (16-byte row loads, dot products per head, DPP
// reductions) kept for tight-tolerance checks.
#include "sws_common.h"

#include <algorithm>
#include <type_traits>

namespace sws {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 4;


// Sum over the TPL consecutive lanes that share a token row (TPL in {8, 16}),
// with DPP lane permutes: swap neighbours, swap pairs, mirror within 8, mirror
// within 16.
template <int TPL>
__device__ __forceinline__ float token_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  if (TPL == 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  return v;
}

// Eight fp32 elements of a K or V row as loaded (two 16-byte vectors).
template <typename T> struct Row8;
template <> struct Row8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void get(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

// A query head's 8 features of this lane, and its dot product with a K row
// (fused multiply-adds).
template <typename T> struct QVec;
template <> struct QVec<float> {
  float v[8];
  __device__ __forceinline__ void load(const float* p) { load8_f32(p, v); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = 0.f;
  }
  __device__ __forceinline__ float dot(const Row8<float>& k) const {
    float kf[8];
    k.get(kf);
    float a = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) a += v[x] * kf[x];
    return a;
  }
};

// A wave-uniform read of a list, mask or page-table entry through the scalar
// cache: a vector load there would make the wave wait for every K / V load
// it has in flight before it can issue the next ones.
template <typename T>
__device__ __forceinline__ T scalar_read(const T* p, int i) {
  typedef __attribute__((address_space(4))) const T const_t;
  return ((const_t*)p)[i];
}

__device__ __forceinline__ float exp2_or_zero(float x) {
  return x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x);
}

// ---------------------------------------------------------------------------
// Work plan.  The blocks to read, over all (sequence, KV head) pairs taken in
// order, are numbered 0 .. W-1 and cut into NWG equal ranges, one per
// workgroup, so every workgroup streams the same number of blocks whatever
// the union sizes are, and there is no tail of half-empty chunks.  A range
// that crosses pair boundaries leaves one partial softmax state ("record")
// per pair it touches.  Every split workgroup derives the plan itself from
// the pairs' block counts (one scan in LDS), so no separate plan launch is
// needed; workgroup 0 also stores it for the combine kernel.  The record of
// workgroup w for pair p is record w + p: ranges are ordered, so a later
// workgroup never touches an earlier pair, the index is unique, and the
// records of one pair are consecutive.
// ---------------------------------------------------------------------------
constexpr int kDecMaxWG = 2048;       // split workgroups at most (sizes the workspace)
constexpr int kDecMaxPairs = 8192;    // sequences x KV heads at most

// floor(x / y) for 0 <= x < 2^53, 0 < y < 2^31, through one fp64 division
// (exact here: a quotient below an integer k is at least 1/y < 2^-31 away
// from it, far more than the rounding error of k * 2^-53).
__device__ __forceinline__ int64_t floor_div(int64_t x, int64_t y) {
  return (int64_t)floor((double)x / (double)y);
}

// first block of workgroup w's range, and the workgroup whose range holds block A
__device__ __forceinline__ int64_t range_lo(int w, int64_t W, int nwg) {
  return floor_div((int64_t)w * W, nwg);
}
__device__ __forceinline__ int wg_of_block(int64_t A, int64_t W, int nwg) {
  return (int)floor_div((A + 1) * nwg - 1, W);
}

// Stored plan: [0] workgroups with work (min(launched, W), so no range is
// empty), then pre[P + 1], the first block of each pair (pre[P] = W).
__device__ __forceinline__ int32_t* plan_nwg(void* ws) { return static_cast<int32_t*>(ws); }
__device__ __forceinline__ int32_t* plan_pre(void* ws) { return static_cast<int32_t*>(ws) + 1; }

// Exclusive prefix sum over the workgroup of one int per thread (wave scans
// with lane shuffles, then the wave totals); also returns the total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = wtot[w];
    base += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();
  return base + inc - v;
}

// The plan in LDS: spre[p] = first block of pair p, spre[P] = W (returned).
// Block counts are the union sizes, or every block of the context (dense).
template <int BLK, int NT>
__device__ __forceinline__ int build_plan(const int32_t* __restrict__ ctx_len,
                                          const int32_t* __restrict__ ucnt, int P, int hkv,
                                          int rows, int uwidth, int32_t* spre, int* wtot) {
  constexpr int LB = 8;                       // loads in flight per thread
  const int t = threadIdx.x;
  for (int p0 = 0; p0 < P; p0 += LB * NT) {
    int v[LB];
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int p = min(p0 + u * NT + t, P - 1);
      // union sizes clamped to the list width, context lengths to the cache
      v[u] = ucnt ? min(max(ucnt[p], 0), uwidth)
                  : (min(max(ctx_len[p / hkv], 1), rows) + BLK - 1) / BLK;
    }
#pragma unroll
    for (int u = 0; u < LB; ++u)
      if (p0 + u * NT + t < P) spre[p0 + u * NT + t] = v[u];
  }
  __syncthreads();
  // thread t scans pairs t * per .. t * per + per - 1
  const int per = (P + NT - 1) / NT;
  int run = 0;
  for (int u = 0; u < per; ++u) {
    const int p = t * per + u;
    if (p < P) run += spre[p];
  }
  int total;
  int acc = block_exclusive_scan<NT>(run, wtot, total);
  for (int u = 0; u < per; ++u) {
    const int p = t * per + u;
    if (p < P) {
      const int c = spre[p];
      spre[p] = acc;
      acc += c;
    }
  }
  if (t == 0) spre[P] = total;
  __syncthreads();
  return total;
}

// Strides (elements) of a KV cache: row t of KV head g of sequence s is at
// s * seq + g * head + t * row.  Token-major caches [n_seqs][max_ctx][hkv][d]
// have (max_ctx hkv d, d, hkv d), head-major ones [n_seqs][hkv][max_ctx][d]
// (hkv max_ctx d, max_ctx d, d).  For pages `seq` is the page stride and rows
// count from the page's first token: [BLK][hkv][d] pages have (BLK hkv d, d,
// hkv d), [hkv][BLK][d] pages (hkv BLK d, BLK d, d).
// `rows` is a sequence's row capacity (max_ctx, or table_width * BLK for
// pages): context lengths are clamped to it, so a length past the cache
// reads inside the sequence's own rows.
struct KvLayout {
  int64_t seq, head, row;
  int rows;
};

// Partial state of blocks [a, b) of pair p's list for every query head of the
// group, written as record `r`.  The range is cut into batches of TPB tokens
// (a batch never straddles a block); wave w takes batches w, w + 4, ...  A
// lane holds UNR token rows of a batch (TPL lanes per row, 8 features per
// lane); all K and V loads of the batch are issued before any is used, and
// each row group of the wave keeps its own online-softmax state (max, sum,
// weighted V sum) for up to four query heads at a time.  Row groups merge
// through lane exchanges, waves through LDS.
// KV addressing: a contiguous cache (table == null), or pages of BLK tokens
// with table[seq][logical block] giving the page; L gives the strides.  TK is the cache element type (the query type
// here); kscale / vscale are per-tensor scales (1 for plain caches).
template <typename T, int D, int BLK, int GMAX, int UNR, typename TK = T>
__device__ __forceinline__ void decode_range(
    const T* __restrict__ q, const TK* __restrict__ kc, const TK* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, KvLayout L, int hq, int hkv,
    const int32_t* __restrict__ uidx, const uint32_t* __restrict__ umask, int uwidth, int p,
    int a, int b, int r, float scale_log2, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, const int32_t* __restrict__ table = nullptr, int table_width = 0,
    int num_pages = 0, float kscale = 1.0f, float vscale = 1.0f) {
  using QV = QVec<T>;
  constexpr int TPL = D / 8;                   // lanes per token row
  constexpr int RPW = 64 / TPL;                // token rows per wave-wide load
  constexpr int TPB = RPW * UNR;               // tokens per wave batch
  constexpr int NWV = kDecThreads / 64;
  constexpr int HC = GMAX < 4 ? GMAX : 4;      // query heads per pass
  static_assert(BLK % TPB == 0, "a batch must stay inside one block");
  __shared__ float wm[NWV][HC], wl[NWV][HC];
  __shared__ float wacc[NWV][HC][D];

  const int seq = p / hkv;
  const int g = p % hkv;
  const int G = hq / hkv;
  const int ctx = min(max(ctx_len[seq], 1), L.rows);   // the new token .. the cache
  const float sl2 = scale_log2 * kscale;
  const int last_blk = (ctx - 1) / BLK;
  const int ntok = (b - a) * BLK;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar list reads
  const int ch = lane % TPL;           // feature chunk (8 features)
  const int slot = lane / TPL;         // row group of the wave
  const int64_t seq_off = table ? 0 : (int64_t)seq * L.seq;
  const TK* kb = kc + seq_off + (int64_t)g * L.head + ch * 8;
  const TK* vb = vc + seq_off + (int64_t)g * L.head + ch * 8;
  const int32_t* trow = table ? table + (int64_t)seq * table_width : nullptr;
  const int32_t* ul = uidx ? uidx + (int64_t)p * uwidth : nullptr;
  const uint32_t* um = umask ? umask + (int64_t)p * uwidth : nullptr;

  for (int h0 = 0; h0 < G; h0 += HC) {
    QV qv[HC];
    float acc[HC][8], m[HC], l[HC];
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
      if (h0 + hh < G) qv[hh].load(q + ((int64_t)seq * hq + g * G + h0 + hh) * D + ch * 8);
      else qv[hh].zero();
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[hh][x] = 0.f;
      m[hh] = -INFINITY;
      l[hh] = 0.f;
    }
    for (int tb = wave * TPB; tb < ntok; tb += NWV * TPB) {
      const int e = a + tb / BLK;
      // list entries are blocks of the context; a stray one is clamped so every
      // access stays inside this sequence's rows
      const int blk = min(max(ul ? scalar_read(ul, e) : e, 0), last_blk);
      const uint32_t mk = um ? scalar_read(um, e) : 0xffffffffu;
      const int r0 = blk * BLK + tb % BLK + slot;      // this lane's first cache row
      // Paged: the batch lies in one logical block, so one page; out-of-range
      // table entries are clamped (the caller's error, never a stray access).
      int64_t pbase = 0;
      if (trow) {
        const int pg = min(max(scalar_read(trow, min(blk, table_width - 1)), 0), num_pages - 1);
        pbase = (int64_t)pg * L.seq - (int64_t)blk * BLK * L.row;
      }
      Row8<TK> kr[UNR], vr[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        // rows past ctx are masked below (the clamped row is in the same block)
        const int64_t row = min(r0 + u * RPW, ctx - 1);
        kr[u].load(kb + pbase + row * L.row);
        vr[u].load(vb + pbase + row * L.row);
      }
      float sc[UNR][HC];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const bool ok = r0 + u * RPW < ctx;
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
          const float part = token_sum<TPL>(qv[hh].dot(kr[u]));
          sc[u][hh] = (ok && ((mk >> (h0 + hh)) & 1u)) ? part * sl2 : -INFINITY;
        }
      }
#pragma unroll
      for (int hh = 0; hh < HC; ++hh) {
        float bm = sc[0][hh];
#pragma unroll
        for (int u = 1; u < UNR; ++u) bm = fmaxf(bm, sc[u][hh]);
        const float mn = fmaxf(m[hh], bm);
        const float alpha = m[hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hh] - mn);
        m[hh] = mn;
        l[hh] *= alpha;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[hh][x] *= alpha;
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float vf[8];
        vr[u].get(vf);
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
          const float pw = exp2_or_zero(sc[u][hh] == -INFINITY ? -INFINITY : sc[u][hh] - m[hh]);
          l[hh] += pw;
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[hh][x] += pw * vf[x];
        }
      }
    }
    // merge the row groups of the wave (lanes TPL, 2 TPL, ... apart)
#pragma unroll
    for (int off = TPL; off < 64; off <<= 1) {
#pragma unroll
      for (int hh = 0; hh < HC; ++hh) {
        const float mo = __shfl_xor(m[hh], off);
        const float lo = __shfl_xor(l[hh], off);
        const float mn = fmaxf(m[hh], mo);
        const float a1 = m[hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hh] - mn);
        const float a2 = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
        l[hh] = l[hh] * a1 + lo * a2;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float ao = __shfl_xor(acc[hh][x], off);
          acc[hh][x] = acc[hh][x] * a1 + ao * a2;
        }
        m[hh] = mn;
      }
    }
    if (slot == 0) {
#pragma unroll
      for (int hh = 0; hh < HC; ++hh) {
#pragma unroll
        for (int x = 0; x < 8; ++x) wacc[wave][hh][ch * 8 + x] = acc[hh][x];
        if (ch == 0) {
          wm[wave][hh] = m[hh];
          wl[wave][hh] = l[hh];
        }
      }
    }
    __syncthreads();
    // merge the waves and write record r for heads h0 .. h0 + HC - 1
    for (int e = tid; e < HC * D; e += kDecThreads) {
      const int hh = e / D, dd = e % D;
      if (h0 + hh >= G) continue;
      float M = wm[0][hh];
#pragma unroll
      for (int w = 1; w < NWV; ++w) M = fmaxf(M, wm[w][hh]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        const float f = wm[w][hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wm[w][hh] - M);
        L += f * wl[w][hh];
        A += f * wacc[w][hh][dd];
      }
      const int64_t row = (int64_t)r * G + h0 + hh;
      ws_acc[row * D + dd] = A * vscale;
      if (dd == 0) {
        ws_ml[row * 2 + 0] = M;
        ws_ml[row * 2 + 1] = L;
      }
    }
    __syncthreads();
  }
}

// Split kernel: workgroup w reads blocks [w W / NWG, (w + 1) W / NWG) of the
// concatenated pair lists, one record per pair the range touches.
template <typename T, int D, int BLK, int GMAX, int UNR, typename TK>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const T* __restrict__ q, const TK* __restrict__ kc, const TK* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, KvLayout L, int n_seqs, int hq, int hkv,
    const int32_t* __restrict__ uidx, const int32_t* __restrict__ ucnt,
    const uint32_t* __restrict__ umask, int uwidth, float scale_log2, int nwg_launched,
    void* ws, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
    const int32_t* __restrict__ table, int table_width, int num_pages, float kscale,
    float vscale) {
  __shared__ int32_t spre[kDecMaxPairs + 1];
  __shared__ int wtot[kDecThreads / 64];
  const int P = n_seqs * hkv;
  const int64_t W = build_plan<BLK, kDecThreads>(ctx_len, uidx ? ucnt : nullptr, P, hkv, L.rows,
                                                 uwidth, spre, wtot);
  // with fewer blocks than workgroups, only the first W get a (one-block) range
  const int nwg = (int)std::min<int64_t>(nwg_launched, std::max<int64_t>(W, 1));
  const int w = blockIdx.x;
  if (w == 0) {
    int32_t* pre = plan_pre(ws);
    for (int p = threadIdx.x; p <= P; p += kDecThreads) pre[p] = spre[p];
    if (threadIdx.x == 0) *plan_nwg(ws) = nwg;
  }
  if (w >= nwg) return;
  const int64_t lo = range_lo(w, W, nwg);
  const int64_t hi = range_lo(w + 1, W, nwg);
  if (lo >= hi) return;
  // first pair: the last pair starting at or before lo (pairs without blocks
  // are skipped below)
  int p = 0;
  {
    int h = P - 1;
    while (p < h) {
      const int m = (p + h + 1) >> 1;
      if (spre[m] <= lo) p = m;
      else h = m - 1;
    }
  }
  for (; p < P; ++p) {
    const int A = spre[p];
    if (A >= hi) break;
    const int Bn = spre[p + 1];
    const int a = (int)(max(lo, (int64_t)A) - A);
    const int b = (int)(min(hi, (int64_t)Bn) - A);
    if (a >= b) continue;
    decode_range<T, D, BLK, GMAX, UNR, TK>(q, kc, vc, ctx_len, L, hq, hkv, uidx, umask,
                                           uwidth, p, a, b, w + p, scale_log2, ws_ml, ws_acc,
                                           table, table_width, num_pages, kscale, vscale);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core form of the split kernel (bf16 queries; bf16 or fp8 e4m3 KV).
// Same plan and records as decode_split_kernel.  A wave takes 32-key steps
// of its workgroup's range (steps w, w + 4, ...) and, per step, with
// v_mfma_f32_16x16x32_bf16 (16 columns = the group's query heads, zero past G):
//   S^T = K Q^T   two 16-key tiles; A = K rows straight from memory (lane l:
//                 key l % 16 of the tile, 8 features of group l / 16 of each
//                 32-feature chunk), B = the queries;
//   V^T           the step's V rows go to the wave's LDS area transposed
//                 (features as rows, keys in the order of the S^T
//                 accumulators, so P needs no lane exchange);
//   softmax       a lane holds 8 scores of one head; the step's max per head
//                 is two lane exchanges;
//   O^T += V^T P^T  one 32-key product per 16-feature tile of O^T.
// The K and V loads of a wave's next step are issued before the current step
// computes, so every wave keeps a step of rows in flight.
// fp8 rows are widened to bf16 (exact) before use; the K scale multiplies the
// scores and the V scale the record.  The waves merge in LDS at the end of
// each pair's range.
// ---------------------------------------------------------------------------
constexpr int kVtStride = 40;            // V^T row: 32 key slots + 8 pad (80 bytes)
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Slot of key k (0..31 within a step) in a V^T row: the B operand of the
// V product takes slots 8 j .. 8 j + 7 from lane group j, which holds the
// scores of keys 4 j .. 4 j + 3 (first tile) and 16 + 4 j .. 16 + 4 j + 3.
__device__ __forceinline__ int vt_slot(int k) {
  return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3);
}

template <typename TK> struct KvFrag;
template <> struct KvFrag<uint16_t> {
  uint4 r;
  __device__ __forceinline__ void load(const uint16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ bf16x8_t bf() const { return __builtin_bit_cast(bf16x8_t, r); }
};
template <> struct KvFrag<uint8_t> {
  uint2 r;
  __device__ __forceinline__ void set(uint32_t lo, uint32_t hi) { r = make_uint2(lo, hi); }
  // one instruction per two codes (fp8 -> bf16 directly, scale 1: exact)
  __device__ __forceinline__ bf16x8_t bf() const {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, 1.0f, true);
    const bf16x8_t f = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return f;
  }
};

template <int D, int BLK, typename TK>
__device__ __forceinline__ void mfma_range(
    const uint16_t* __restrict__ q, const TK* __restrict__ kc, const TK* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, KvLayout L, int hq, int hkv,
    const int32_t* __restrict__ uidx, const uint32_t* __restrict__ umask, int uwidth, int p,
    int a, int b, int r, float scale_log2, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, const int32_t* __restrict__ table, int table_width,
    int num_pages, float kscale, float vscale, __bf16* vt_all, float* mw, float* lw) {
  constexpr int NWV = kDecThreads / 64;
  constexpr int KT = 32;
  constexpr int DC = D / 32;                  // 32-feature chunks (QK operands)
  constexpr int DT = D / 16;                  // 16-feature tiles of O^T
  static_assert(BLK % KT == 0, "a step stays inside one block");
  const int seq = p / hkv;
  const int g = p % hkv;
  const int G = hq / hkv;
  const int ctx = min(max(ctx_len[seq], 1), L.rows);
  const int last_blk = (ctx - 1) / BLK;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar list reads
  const int col = lane & 15, grp = lane >> 4;
  const float sl2 = scale_log2 * kscale;
  __bf16* vt = vt_all + wave * D * kVtStride;
  const int64_t seq_off = table ? 0 : (int64_t)seq * L.seq;
  const TK* kb = kc + seq_off + (int64_t)g * L.head;
  const TK* vb = vc + seq_off + (int64_t)g * L.head;
  const int32_t* trow = table ? table + (int64_t)seq * table_width : nullptr;
  const int32_t* ul = uidx ? uidx + (int64_t)p * uwidth : nullptr;
  const uint32_t* um = umask ? umask + (int64_t)p * uwidth : nullptr;
  // The features lane group grp feeds to the MFMA of 32-feature chunk c (any
  // assignment works if K and Q use the same): bf16 rows take 8 contiguous
  // features per chunk (16 bytes); fp8 rows take 16 contiguous bytes for the
  // chunk pair (2m, 2m + 1), so one 16-byte load serves two chunks and a
  // step needs half the load instructions.
  constexpr bool F8 = sizeof(TK) == 1;
  auto feat = [&](int c) { return F8 ? (c >> 1) * 64 + grp * 16 + (c & 1) * 8 : c * 32 + grp * 8; };

  // the group's queries as B operand columns (heads past G are zero)
  bf16x8_t qf[DC];
  {
    const bool hv = col < G;
    const uint16_t* qp = q + ((int64_t)seq * hq + g * G + min(col, G - 1)) * D;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qp + feat(c));
      qf[c] = __builtin_bit_cast(bf16x8_t, hv ? raw : make_uint4(0u, 0u, 0u, 0u));
    }
  }
  floatx4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int x = 0; x < 4; ++x) o[dt][x] = 0.f;
  float m = -INFINITY, l = 0.f;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  int slot[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) slot[kt] = vt_slot(kt * 16 + col);

  const int nstep = (b - a) * (BLK / KT);
  // loads of step t (rows, block mask and first key), issued one step ahead
  auto issue = [&](int t, KvFrag<TK> (&kf)[2][DC], KvFrag<TK> (&vf)[2][DC], uint32_t& mk,
                   int& key0) {
    const int tt = min(t, nstep - 1);
    const int e = a + tt / (BLK / KT);
    const int blk = min(max(ul ? scalar_read(ul, e) : e, 0), last_blk);
    mk = um ? scalar_read(um, e) : 0xffffffffu;
    key0 = blk * BLK + (tt % (BLK / KT)) * KT;
    int64_t pbase = 0;
    if (trow) {
      const int pg = min(max(scalar_read(trow, min(blk, table_width - 1)), 0), num_pages - 1);
      pbase = (int64_t)pg * L.seq - (int64_t)blk * BLK * L.row;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int64_t row = pbase + (int64_t)min(key0 + kt * 16 + col, ctx - 1) * L.row;
      if constexpr (F8) {
#pragma unroll
        for (int c = 0; c < DC; c += 2) {
          const uint4 ku = *reinterpret_cast<const uint4*>(kb + row + feat(c));
          const uint4 vu = *reinterpret_cast<const uint4*>(vb + row + feat(c));
          kf[kt][c].set(ku.x, ku.y);
          kf[kt][c + 1].set(ku.z, ku.w);
          vf[kt][c].set(vu.x, vu.y);
          vf[kt][c + 1].set(vu.z, vu.w);
        }
      } else {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          kf[kt][c].load(kb + row + feat(c));
          vf[kt][c].load(vb + row + feat(c));
        }
      }
    }
  };
  KvFrag<TK> kn[2][DC], vn[2][DC];
  uint32_t mk_n;
  int key0_n;
  if (wave < nstep) issue(wave, kn, vn, mk_n, key0_n);
  for (int t = wave; t < nstep; t += NWV) {
    KvFrag<TK> kf[2][DC], vf[2][DC];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        kf[kt][c] = kn[kt][c];
        vf[kt][c] = vn[kt][c];
      }
    const uint32_t mk = mk_n;
    const int key0 = key0_n;
    if (t + NWV < nstep) issue(t + NWV, kn, vn, mk_n, key0_n);
    // S^T = K Q^T, two 16-key tiles
    floatx4_t st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int x = 0; x < 4; ++x) st[kt][x] = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c)
        st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt][c].bf(), qf[c], st[kt], 0, 0, 0);
    }
    // V^T of the step into this wave's LDS area
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8_t v = vf[kt][c].bf();
#pragma unroll
        for (int x = 0; x < 8; ++x) vt[(feat(c) + x) * kVtStride + slot[kt]] = v[x];
      }
    // mask (keys past the context, heads that did not keep the block), the
    // step's max per head
    const bool head_ok = col < G && ((mk >> col) & 1u);
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int key = key0 + kt * 16 + grp * 4 + x;
        st[kt][x] = (head_ok && key < ctx) ? st[kt][x] * sl2 : -INFINITY;
        mx = fmaxf(mx, st[kt][x]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    if (__any(m_new > m)) {
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int x = 0; x < 4; ++x) o[dt][x] *= alpha;
      m = m_new;
    }
    bf16x8_t pb;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      bf16x2_t pr;
      const float s0 = st[i >> 2][i & 3], s1 = st[i >> 2][(i & 3) + 1];
      pr[0] = (__bf16)(s0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s0 - m));
      pr[1] = (__bf16)(s1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s1 - m));
      l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
      pb[i] = pr[0];
      pb[i + 1] = pr[1];
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bf16x8_t av =
          *reinterpret_cast<const bf16x8_t*>(vt + (dt * 16 + col) * kVtStride + grp * 8);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, o[dt], 0, 0, 0);
    }
  }
  // ---- merge the waves' states and write record r ----
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();                            // every wave is done with its V^T area
  if (grp == 0) {
    mw[wave * 16 + col] = m;
    lw[wave * 16 + col] = l;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w2 = 0; w2 < NWV; ++w2) M = fmaxf(M, mw[w2 * 16 + col]);
  const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
  // scaled O^T of this wave into LDS (the V^T area): acc[wave][head][feature]
  float* acc = reinterpret_cast<float*>(vt_all);
  if (col < G) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int x = 0; x < 4; ++x) acc[(wave * 16 + col) * D + dt * 16 + grp * 4 + x] = o[dt][x] * f;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kDecThreads) {
    const int h = i / D, d = i % D;
    float s = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NWV; ++w2) s += acc[(w2 * 16 + h) * D + d];
    ws_acc[((int64_t)r * G + h) * D + d] = s * vscale;
    if (d == 0) {
      float Mh = -INFINITY, Lh = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NWV; ++w2) Mh = fmaxf(Mh, mw[w2 * 16 + h]);
#pragma unroll
      for (int w2 = 0; w2 < NWV; ++w2) {
        const float mv = mw[w2 * 16 + h];
        Lh += mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - Mh) * lw[w2 * 16 + h];
      }
      ws_ml[((int64_t)r * G + h) * 2 + 0] = Mh;
      ws_ml[((int64_t)r * G + h) * 2 + 1] = Lh;
    }
  }
  __syncthreads();                            // the LDS areas are reused by the next range
}

template <int D, int BLK, typename TK>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_kernel(
    const uint16_t* __restrict__ q, const TK* __restrict__ kc, const TK* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, KvLayout L, int n_seqs, int hq, int hkv,
    const int32_t* __restrict__ uidx, const int32_t* __restrict__ ucnt,
    const uint32_t* __restrict__ umask, int uwidth, float scale_log2, int nwg_launched,
    void* ws, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
    const int32_t* __restrict__ table, int table_width, int num_pages, float kscale,
    float vscale) {
  constexpr int NWV = kDecThreads / 64;
  __shared__ int32_t spre[kDecMaxPairs + 1];
  __shared__ int wtot[NWV];
  __shared__ __attribute__((aligned(16))) __bf16 vt_all[NWV * D * kVtStride];
  __shared__ float mw[NWV * 16], lw[NWV * 16];
  static_assert(NWV * D * kVtStride * 2 >= NWV * 16 * D * 4, "merge area fits in V^T area");
  const int P = n_seqs * hkv;
  const int64_t W = build_plan<BLK, kDecThreads>(ctx_len, uidx ? ucnt : nullptr, P, hkv, L.rows,
                                                 uwidth, spre, wtot);
  const int nwg = (int)std::min<int64_t>(nwg_launched, std::max<int64_t>(W, 1));
  const int w = blockIdx.x;
  if (w == 0) {
    int32_t* pre = plan_pre(ws);
    for (int p = threadIdx.x; p <= P; p += kDecThreads) pre[p] = spre[p];
    if (threadIdx.x == 0) *plan_nwg(ws) = nwg;
  }
  if (w >= nwg) return;
  const int64_t lo = range_lo(w, W, nwg);
  const int64_t hi = range_lo(w + 1, W, nwg);
  if (lo >= hi) return;
  int p = 0;
  {
    int h = P - 1;
    while (p < h) {
      const int m = (p + h + 1) >> 1;
      if (spre[m] <= lo) p = m;
      else h = m - 1;
    }
  }
  for (; p < P; ++p) {
    const int A = spre[p];
    if (A >= hi) break;
    const int Bn = spre[p + 1];
    const int a = (int)(max(lo, (int64_t)A) - A);
    const int b = (int)(min(hi, (int64_t)Bn) - A);
    if (a >= b) continue;
    mfma_range<D, BLK, TK>(q, kc, vc, ctx_len, L, hq, hkv, uidx, umask, uwidth, p, a, b,
                           w + p, scale_log2, ws_ml, ws_acc, table, table_width, num_pages,
                           kscale, vscale, vt_all, mw, lw);
  }
}

// Merge of the records of one (sequence, query head): the weights
// exp2(m_r - max m) go to LDS once, then each thread sums one feature over the
// records with independent loads.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(
    int n_seqs, int hq, int hkv, const void* ws, const float* __restrict__ ws_ml,
    const float* __restrict__ ws_acc, T* __restrict__ out, float* __restrict__ lse) {
  constexpr int NW = D / 64;
  __shared__ float wgt[kDecMaxWG + 1];
  __shared__ float red[NW];
  __shared__ float s_M, s_L;
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int G = hq / hkv;
  const int hh = h % G;
  const int p = seq * hkv + h / G;
  // this pair's records: those of the workgroups holding its first and last block
  const int32_t* pre = plan_pre(const_cast<void*>(ws));
  const int nwg = *plan_nwg(const_cast<void*>(ws));
  const int64_t W = pre[n_seqs * hkv];
  const int A = pre[p], Bn = pre[p + 1];
  const int r0 = Bn > A ? wg_of_block(A, W, nwg) + p : 0;
  const int ns = Bn > A ? wg_of_block(Bn - 1, W, nwg) + p + 1 - r0 : 0;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  // the first records' partial outputs are loaded now, beside the maxima, so
  // the weighted sum below does not wait for a third round of loads
  constexpr int kPre = 16;
  float av[kPre];
#pragma unroll
  for (int si = 0; si < kPre; ++si)
    av[si] = si < ns ? ws_acc[((int64_t)(r0 + si) * G + hh) * D + t] : 0.f;
  float m = -INFINITY;
  for (int si = t; si < ns; si += D) {
    const float v = ws_ml[((int64_t)(r0 + si) * G + hh) * 2];
    wgt[si] = v;
    m = fmaxf(m, v);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (t == 0) {
    float M = red[0];
    for (int w = 1; w < NW; ++w) M = fmaxf(M, red[w]);
    s_M = M;
  }
  __syncthreads();
  const float M = s_M;
  float lsum = 0.f;
  for (int si = t; si < ns; si += D) {
    const float mv = wgt[si];
    const float f = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
    wgt[si] = f;
    lsum += f * ws_ml[((int64_t)(r0 + si) * G + hh) * 2 + 1];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
  __syncthreads();
  if (lane == 0) red[wave] = lsum;
  __syncthreads();
  if (t == 0) {
    float L = 0.f;
    for (int w = 0; w < NW; ++w) L += red[w];
    s_L = L;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int si = 0; si < kPre; ++si)
    if (si < ns) acc += wgt[si] * av[si];
#pragma unroll 8
  for (int si = kPre; si < ns; ++si)
    acc += wgt[si] * ws_acc[((int64_t)(r0 + si) * G + hh) * D + t];
  const float L = s_L;
  const float o = L > 0.f ? acc / L : 0.f;
  T* op = out + ((int64_t)seq * hq + h) * D + t;
  if constexpr (sizeof(T) == 2) *reinterpret_cast<uint16_t*>(op) = (uint16_t)f32_to_bf16_bits(o);
  else *op = o;
  if (lse && t == 0) lse[(int64_t)seq * hq + h] = (M + log2f(L)) * kLn2;
}

// Workspace: plan (int32: nwg, pre [P + 1]), then the records' (max, sum) and
// weighted V sums, (P + kDecMaxWG) records of G heads.
size_t plan_bytes(int P) {
  return (((size_t)1 + (P + 1)) * sizeof(int32_t) + 255) & ~(size_t)255;
}

// Split workgroups per launch: six per CU (two to three rounds of the split
// kernels' resident workgroups; one or two rounds measure the same).
int split_workgroups() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = std::min(kDecMaxWG, cus * 3 * 2);
  }
  return cached[dev];
}

template <typename T, int D, int BLK, int GMAX, typename TK>
hipError_t run_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* ctx_len, int n_seqs, KvLayout L, int hq, int hkv,
                      const int32_t* uidx, const int32_t* ucnt, const uint32_t* umask,
                      int uwidth, float scale, void* out, float* lse, void* ws,
                      hipStream_t st, const int32_t* table, int table_width, int num_pages,
                      float kscale, float vscale) {
  const int P = n_seqs * hkv;
  const int G = hq / hkv;
  const int nwg = split_workgroups();
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + plan_bytes(P));
  float* ws_acc = ws_ml + (size_t)(P + kDecMaxWG) * G * 2;
  if constexpr (std::is_same<T, uint16_t>::value) {
    hipLaunchKernelGGL((decode_mfma_kernel<D, BLK, TK>), dim3(nwg), dim3(kDecThreads), 0, st,
                       static_cast<const uint16_t*>(q), static_cast<const TK*>(k_cache),
                       static_cast<const TK*>(v_cache), ctx_len, L, n_seqs, hq, hkv, uidx,
                       ucnt, umask, uwidth, scale * kLog2e, nwg, ws, ws_ml, ws_acc, table,
                       table_width, num_pages, kscale, vscale);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<T, D, BLK, GMAX, kDecUnroll, TK>), dim3(nwg),
                       dim3(kDecThreads), 0, st, static_cast<const T*>(q),
                       static_cast<const TK*>(k_cache), static_cast<const TK*>(v_cache), ctx_len,
                       L, n_seqs, hq, hkv, uidx, ucnt, umask, uwidth, scale * kLog2e, nwg,
                       ws, ws_ml, ws_acc, table, table_width, num_pages, kscale, vscale);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(hq, n_seqs), dim3(D), 0, st, n_seqs,
                     hq, hkv, ws, ws_ml, ws_acc, static_cast<T*>(out), lse);
  return hipGetLastError();
}

template <typename T, int D, int BLK, typename TK = T>
hipError_t pick_g(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* ctx_len, int n_seqs, KvLayout L, int hq, int hkv,
                  const int32_t* uidx, const int32_t* ucnt, const uint32_t* umask, int uwidth,
                  float scale, void* out, float* lse, void* ws, hipStream_t st,
                  const int32_t* table = nullptr, int table_width = 0, int num_pages = 0,
                  float kscale = 1.0f, float vscale = 1.0f) {
  const int G = hq / hkv;
#define SWS_RUN(GM)                                                                            \
  return run_decode<T, D, BLK, GM, TK>(q, k_cache, v_cache, ctx_len, n_seqs, L, hq, hkv,        \
                                       uidx, ucnt, umask, uwidth, scale, out, lse, ws, st,     \
                                       table, table_width, num_pages, kscale, vscale)
  if (G <= 1) SWS_RUN(1);
  if (G <= 4) SWS_RUN(4);
  if (G <= 8) SWS_RUN(8);
  SWS_RUN(16);
#undef SWS_RUN
}

}  // namespace

size_t decode_workspace_bytes(int n_seqs, int hq, int hkv, int d, int B, int union_width) {
  (void)B;
  (void)union_width;
  const int P = n_seqs * hkv;
  const size_t G = (size_t)(hq / hkv);
  return plan_bytes(P) + (size_t)(P + kDecMaxWG) * G * (size_t)(d + 2) * sizeof(float);
}

hipError_t launch_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                              int dtype, bool head_major, const int32_t* ctx_len, int n_seqs,
                              int max_ctx, int hq, int hkv, int d, int B, const int32_t* union_idx,
                              const int32_t* union_cnt, const uint32_t* union_mask,
                              int union_width, float scale, void* out, float* lse, void* ws,
                              hipStream_t st) {
  if (n_seqs == 0) return hipSuccess;
  const KvLayout L = head_major
                         ? KvLayout{(int64_t)hkv * max_ctx * d, (int64_t)max_ctx * d, d, max_ctx}
                         : KvLayout{(int64_t)max_ctx * hkv * d, d, (int64_t)hkv * d, max_ctx};
#define SWS_DEC(T, D, BLK)                                                                     \
  return pick_g<T, D, BLK>(q, k_cache, v_cache, ctx_len, n_seqs, L, hq, hkv, union_idx,       \
                           union_cnt, union_mask, union_width, scale, out, lse, ws, st)
  if (dtype == SWS_BF16) {
    if (d == 128 && B == 64) SWS_DEC(uint16_t, 128, 64);
    if (d == 128 && B == 128) SWS_DEC(uint16_t, 128, 128);
    if (d == 64 && B == 64) SWS_DEC(uint16_t, 64, 64);
    SWS_DEC(uint16_t, 64, 128);
  }
  if (d == 128 && B == 64) SWS_DEC(float, 128, 64);
  if (d == 128 && B == 128) SWS_DEC(float, 128, 128);
  if (d == 64 && B == 64) SWS_DEC(float, 64, 64);
  SWS_DEC(float, 64, 128);
#undef SWS_DEC
}

hipError_t launch_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                    int kv_dtype, bool head_major, float k_scale, float v_scale,
                                    const int32_t* block_table, int table_width,
                                    int num_pages, const int32_t* ctx_len, int n_seqs, int hq, int hkv, int d,
                                    int B, const int32_t* union_idx, const int32_t* union_cnt,
                                    const uint32_t* union_mask, int union_width, float scale,
                                    void* out, float* lse, void* ws, hipStream_t st) {
  if (n_seqs == 0) return hipSuccess;
  // a page holds B rows of every KV head: [B][hkv][d] or, head-major, [hkv][B][d]
  const int rows = (int)std::min<int64_t>((int64_t)table_width * B, 0x7fffffff);
  const KvLayout L = head_major ? KvLayout{(int64_t)hkv * B * d, (int64_t)B * d, d, rows}
                                : KvLayout{(int64_t)B * hkv * d, d, (int64_t)hkv * d, rows};
#define SWS_DEC(TK, D, BLK)                                                                    \
  return pick_g<uint16_t, D, BLK, TK>(q, k_pages, v_pages, ctx_len, n_seqs, L, hq, hkv,       \
                                      union_idx, union_cnt, union_mask, union_width, scale,   \
                                      out, lse, ws, st, block_table, table_width, num_pages,  \
                                      k_scale, v_scale)
  if (kv_dtype == SWS_FP8_E4M3) {
    if (d == 128 && B == 64) SWS_DEC(uint8_t, 128, 64);
    if (d == 128 && B == 128) SWS_DEC(uint8_t, 128, 128);
    if (d == 64 && B == 64) SWS_DEC(uint8_t, 64, 64);
    SWS_DEC(uint8_t, 64, 128);
  }
  if (d == 128 && B == 64) SWS_DEC(uint16_t, 128, 64);
  if (d == 128 && B == 128) SWS_DEC(uint16_t, 128, 128);
  if (d == 64 && B == 64) SWS_DEC(uint16_t, 64, 64);
  SWS_DEC(uint16_t, 64, 128);
#undef SWS_DEC
}

}  // namespace sws
