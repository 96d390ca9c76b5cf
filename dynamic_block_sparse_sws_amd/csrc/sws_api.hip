// C ABI of the Sketch&Walk library: host-side argument validation (before any
// HIP call), dispatch to the kernel launchers, error reporting.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "sws_common.h"

namespace {

thread_local std::string g_detail;

sws_status fail(sws_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return code;
}

sws_status ok() {
  g_detail.clear();
  return SWS_OK;
}

sws_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SWS_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// A roctx range around each call of the C ABI, named after the call, so a
// profiler trace (rocprofv3 --marker-trace) shows the host-side validation
// and launches of every call next to its kernels.
struct RocRange {
  explicit RocRange(const char* name) { roctxRangePushA(name); }
  ~RocRange() { roctxRangePop(); }
  RocRange(const RocRange&) = delete;
  RocRange& operator=(const RocRange&) = delete;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(int dt) { return dt == SWS_F32 || dt == SWS_BF16; }

int tau_of(int rho, int b) { return (int)(((int64_t)rho * b) / 100); }

}  // namespace

#define REQUIRE_PTR(p) \
  if (!(p)) return fail(SWS_ERR_NULL, "%s: argument '%s' is NULL", fn, #p)

extern "C" {

int sws_version(void) { return 100; }

const char* sws_status_string(sws_status status) {
  switch (status) {
    case SWS_OK: return "SWS_OK";
    case SWS_ERR_NULL: return "SWS_ERR_NULL";
    case SWS_ERR_SHAPE: return "SWS_ERR_SHAPE";
    case SWS_ERR_UNSUPPORTED: return "SWS_ERR_UNSUPPORTED";
    case SWS_ERR_WORKSPACE: return "SWS_ERR_WORKSPACE";
    case SWS_ERR_LAUNCH: return "SWS_ERR_LAUNCH";
    default: return "SWS_ERR_UNKNOWN";
  }
}

const char* sws_last_error_detail(void) { return g_detail.c_str(); }

sws_status sws_sketch(const void* x, int dtype, const int32_t* cu_seqlens, const int32_t* cu_blocks,
                      int32_t n_seqs, int32_t total_blocks, int32_t n_heads, int32_t d, int32_t B,
                      int32_t k, const int8_t* signs, const int32_t* cols, float* sketch_out,
                      int64_t ld_head, float* sum_out, void* stream) {
  const RocRange roctx_range("sws_sketch");
  const char* fn = "sws_sketch";
  REQUIRE_PTR(x);
  REQUIRE_PTR(cu_seqlens);
  REQUIRE_PTR(cu_blocks);
  REQUIRE_PTR(signs);
  REQUIRE_PTR(cols);
  REQUIRE_PTR(sketch_out);
  if (!dtype_ok(dtype)) return fail(SWS_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (d != 64 && d != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: d=%d not in {64,128}", fn, d);
  if (B != 64 && B != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: B=%d not in {64,128}", fn, B);
  if (k < 1 || k > d || k > 64) return fail(SWS_ERR_UNSUPPORTED, "%s: k=%d outside [1, min(d,64)]", fn, k);
  if (n_seqs < 0 || total_blocks < 0 || n_heads < 1 || (n_seqs == 0 && total_blocks != 0))
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d total_blocks=%d n_heads=%d", fn, n_seqs, total_blocks, n_heads);
  if (ld_head < (int64_t)total_blocks * k)
    return fail(SWS_ERR_SHAPE, "%s: ld_head=%lld < total_blocks*k", fn, (long long)ld_head);
  if (!aligned16(x)) return fail(SWS_ERR_SHAPE, "%s: x is not 16-byte aligned", fn);
  return launched(sws::launch_sketch(x, dtype, cu_seqlens, cu_blocks, n_seqs, total_blocks,
                                     n_heads, d, B, k, signs, cols, sketch_out, ld_head, sum_out,
                                     (hipStream_t)stream),
                  fn);
}

sws_status sws_sketch_append(const void* x_new, int dtype, const int32_t* pos, int32_t n_seqs,
                             int32_t n_heads, int32_t d, int32_t B, int32_t k, const int8_t* signs,
                             const int32_t* cols, float* run_sum, float* sketch_cache, int32_t b_max,
                             void* stream) {
  const RocRange roctx_range("sws_sketch_append");
  const char* fn = "sws_sketch_append";
  REQUIRE_PTR(x_new);
  REQUIRE_PTR(pos);
  REQUIRE_PTR(signs);
  REQUIRE_PTR(cols);
  REQUIRE_PTR(run_sum);
  REQUIRE_PTR(sketch_cache);
  if (!dtype_ok(dtype)) return fail(SWS_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (d != 64 && d != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: d=%d not in {64,128}", fn, d);
  if (B != 64 && B != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: B=%d not in {64,128}", fn, B);
  if (k < 1 || k > d || k > 64) return fail(SWS_ERR_UNSUPPORTED, "%s: k=%d outside [1, min(d,64)]", fn, k);
  if (n_seqs < 0 || n_heads < 1 || b_max < 1)
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d n_heads=%d b_max=%d", fn, n_seqs, n_heads, b_max);
  if (!aligned16(x_new) || !aligned16(run_sum))
    return fail(SWS_ERR_SHAPE, "%s: x_new / run_sum not 16-byte aligned", fn);
  return launched(sws::launch_sketch_append(x_new, n_heads, run_sum, sketch_cache, nullptr, 0,
                                            nullptr, nullptr, dtype, pos, n_seqs, d, B, k, signs,
                                            cols, b_max, (hipStream_t)stream),
                  fn);
}

sws_status sws_sketch_append_qk(const void* q_new, const void* k_new, int dtype, const int32_t* pos,
                                int32_t n_seqs, int32_t hq, int32_t hkv, int32_t d, int32_t B,
                                int32_t k, const int8_t* signs, const int32_t* cols, float* run_sum_q,
                                float* run_sum_k, float* q_cache, float* k_cache, int32_t b_max,
                                void* stream) {
  const RocRange roctx_range("sws_sketch_append_qk");
  const char* fn = "sws_sketch_append_qk";
  REQUIRE_PTR(q_new);
  REQUIRE_PTR(k_new);
  REQUIRE_PTR(pos);
  REQUIRE_PTR(signs);
  REQUIRE_PTR(cols);
  REQUIRE_PTR(run_sum_q);
  REQUIRE_PTR(run_sum_k);
  REQUIRE_PTR(q_cache);
  REQUIRE_PTR(k_cache);
  if (!dtype_ok(dtype)) return fail(SWS_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (d != 64 && d != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: d=%d not in {64,128}", fn, d);
  if (B != 64 && B != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: B=%d not in {64,128}", fn, B);
  if (k < 1 || k > d || k > 64) return fail(SWS_ERR_UNSUPPORTED, "%s: k=%d outside [1, min(d,64)]", fn, k);
  if (n_seqs < 0 || hq < 1 || hkv < 1 || b_max < 1)
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d hq=%d hkv=%d b_max=%d", fn, n_seqs, hq, hkv, b_max);
  if ((int64_t)hq + hkv > 65535)
    return fail(SWS_ERR_SHAPE, "%s: hq + hkv = %lld > 65535", fn, (long long)hq + hkv);
  if (!aligned16(q_new) || !aligned16(k_new) || !aligned16(run_sum_q) || !aligned16(run_sum_k))
    return fail(SWS_ERR_SHAPE, "%s: q_new / k_new / run sums not 16-byte aligned", fn);
  return launched(sws::launch_sketch_append(q_new, hq, run_sum_q, q_cache, k_new, hkv, run_sum_k,
                                            k_cache, dtype, pos, n_seqs, d, B, k, signs, cols,
                                            b_max, (hipStream_t)stream),
                  fn);
}

sws_status sws_walk_update(const float* q_sk, const float* k_sk, int32_t hq, int32_t hkv, int32_t k,
                           const int32_t* cu_blocks, int32_t n_seqs, int32_t total_blocks,
                           int32_t max_blocks, int32_t s, const float* R_prev, float* R_out,
                           void* stream) {
  const RocRange roctx_range("sws_walk_update");
  const char* fn = "sws_walk_update";
  REQUIRE_PTR(q_sk);
  REQUIRE_PTR(k_sk);
  REQUIRE_PTR(cu_blocks);
  REQUIRE_PTR(R_out);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SWS_ERR_SHAPE, "%s: hq=%d hkv=%d (hq must be a multiple of hkv)", fn, hq, hkv);
  if (k < 1 || k > 64) return fail(SWS_ERR_UNSUPPORTED, "%s: k=%d outside [1,64]", fn, k);
  if (n_seqs < 0 || total_blocks < 0 || max_blocks < 0 || max_blocks > total_blocks ||
      (n_seqs == 0 && total_blocks != 0))
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d total_blocks=%d max_blocks=%d", fn, n_seqs, total_blocks, max_blocks);
  if (s < 1) return fail(SWS_ERR_SHAPE, "%s: s=%d must be >= 1", fn, s);
  return launched(sws::launch_walk(q_sk, k_sk, hq, hkv, k, cu_blocks, n_seqs, total_blocks,
                                   max_blocks, s, R_prev, R_out, (hipStream_t)stream),
                  fn);
}

sws_status sws_walk_update_row(const float* q_sk_cache, const float* k_sk_cache, int32_t hq,
                               int32_t hkv, int32_t k, int32_t n_seqs, const int32_t* cur_block,
                               int32_t b_max, int32_t s, const float* r_prev, float* r_out,
                               void* stream) {
  const RocRange roctx_range("sws_walk_update_row");
  const char* fn = "sws_walk_update_row";
  REQUIRE_PTR(q_sk_cache);
  REQUIRE_PTR(k_sk_cache);
  REQUIRE_PTR(cur_block);
  REQUIRE_PTR(r_out);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SWS_ERR_SHAPE, "%s: hq=%d hkv=%d (hq must be a multiple of hkv)", fn, hq, hkv);
  if (k < 1 || k > 64) return fail(SWS_ERR_UNSUPPORTED, "%s: k=%d outside [1,64]", fn, k);
  if (n_seqs < 0 || b_max < 1 || b_max > 4096)
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d b_max=%d (b_max in [1,4096])", fn, n_seqs, b_max);
  if (s < 1) return fail(SWS_ERR_SHAPE, "%s: s=%d must be >= 1", fn, s);
  if (!aligned16(q_sk_cache) || !aligned16(k_sk_cache))
    return fail(SWS_ERR_SHAPE, "%s: q_sk_cache / k_sk_cache must be 16-byte aligned", fn);
  return launched(sws::launch_walk_row(q_sk_cache, k_sk_cache, hq, hkv, k, n_seqs, cur_block,
                                       b_max, s, r_prev, r_out, (hipStream_t)stream),
                  fn);
}

sws_status sws_walk_update_variant(const float* q_sk, const float* k_sk, int32_t hq, int32_t hkv,
                                   int32_t k, const int32_t* cu_blocks, int32_t n_seqs,
                                   int32_t total_blocks, int32_t max_blocks, int32_t s, int32_t mode,
                                   const float* R_prev, float* R_out, int64_t walk_numel, void* ws,
                                   size_t ws_bytes, void* stream) {
  const RocRange roctx_range("sws_walk_update_variant");
  const char* fn = "sws_walk_update_variant";
  if (mode == SWS_WALK_DEFAULT)
    return sws_walk_update(q_sk, k_sk, hq, hkv, k, cu_blocks, n_seqs, total_blocks, max_blocks,
                           s, R_prev, R_out, stream);
  if (mode != SWS_WALK_POWER && mode != SWS_WALK_SOFTMAX)
    return fail(SWS_ERR_UNSUPPORTED, "%s: mode=%d", fn, mode);
  REQUIRE_PTR(q_sk);
  REQUIRE_PTR(k_sk);
  REQUIRE_PTR(cu_blocks);
  REQUIRE_PTR(R_out);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SWS_ERR_SHAPE, "%s: hq=%d hkv=%d (hq must be a multiple of hkv)", fn, hq, hkv);
  if (k < 1 || k > 64) return fail(SWS_ERR_UNSUPPORTED, "%s: k=%d outside [1,64]", fn, k);
  if (n_seqs < 0 || total_blocks < 0 || max_blocks < 0 || max_blocks > total_blocks ||
      (n_seqs == 0 && total_blocks != 0))
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d total_blocks=%d max_blocks=%d", fn, n_seqs, total_blocks, max_blocks);
  if (max_blocks > 4096) return fail(SWS_ERR_UNSUPPORTED, "%s: max_blocks=%d > 4096", fn, max_blocks);
  if (s < 1) return fail(SWS_ERR_SHAPE, "%s: s=%d must be >= 1", fn, s);
  if (walk_numel < (int64_t)hq * max_blocks * max_blocks)
    return fail(SWS_ERR_SHAPE, "%s: walk_numel=%lld smaller than hq * max_blocks^2", fn,
                (long long)walk_numel);
  const size_t need = sws::walk_variant_workspace_bytes(walk_numel);
  if (!ws || ws_bytes < need)
    return fail(SWS_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
  return launched(sws::launch_walk_variant(q_sk, k_sk, hq, hkv, k, cu_blocks, n_seqs,
                                           total_blocks, max_blocks, s, mode, R_prev, R_out,
                                           walk_numel, ws, (hipStream_t)stream),
                  fn);
}

size_t sws_walk_variant_workspace_size(int64_t walk_numel) {
  return walk_numel > 0 ? sws::walk_variant_workspace_bytes(walk_numel) : 0;
}

sws_status sws_walk_update_row_variant(const float* q_sk_cache, const float* k_sk_cache, int32_t hq,
                                       int32_t hkv, int32_t k, int32_t n_seqs,
                                       const int32_t* cur_block, int32_t b_max, int32_t s,
                                       int32_t mode, const float* r_prev, float* r_out, void* stream) {
  const RocRange roctx_range("sws_walk_update_row_variant");
  const char* fn = "sws_walk_update_row_variant";
  if (mode == SWS_WALK_DEFAULT)
    return sws_walk_update_row(q_sk_cache, k_sk_cache, hq, hkv, k, n_seqs, cur_block, b_max, s,
                               r_prev, r_out, stream);
  if (mode != SWS_WALK_POWER && mode != SWS_WALK_SOFTMAX)
    return fail(SWS_ERR_UNSUPPORTED, "%s: mode=%d", fn, mode);
  REQUIRE_PTR(q_sk_cache);
  REQUIRE_PTR(k_sk_cache);
  REQUIRE_PTR(cur_block);
  REQUIRE_PTR(r_out);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SWS_ERR_SHAPE, "%s: hq=%d hkv=%d (hq must be a multiple of hkv)", fn, hq, hkv);
  if (k < 1 || k > 64) return fail(SWS_ERR_UNSUPPORTED, "%s: k=%d outside [1,64]", fn, k);
  if (n_seqs < 0 || b_max < 1 || b_max > 4096)
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d b_max=%d (b_max in [1,4096])", fn, n_seqs, b_max);
  if (s < 1) return fail(SWS_ERR_SHAPE, "%s: s=%d must be >= 1", fn, s);
  return launched(sws::launch_walk_row_variant(q_sk_cache, k_sk_cache, hq, hkv, k, n_seqs,
                                               cur_block, b_max, s, mode, r_prev, r_out,
                                               (hipStream_t)stream),
                  fn);
}

static sws_status select_topk_impl(const char* fn, const float* R, int32_t hq, int32_t hkv,
                                   const int32_t* cu_blocks, int32_t n_seqs, int32_t total_blocks,
                                   int32_t max_blocks, int32_t rho_percent, int32_t flags,
                                   int32_t width, int32_t* idx, int32_t* cnt, void* stream) {
  const bool dense = (flags & SWS_SELECT_DENSE) != 0;
  if (!dense) REQUIRE_PTR(R);
  REQUIRE_PTR(cu_blocks);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(cnt);
  if (flags & ~(SWS_SELECT_DENSE | SWS_SELECT_ROW_TAU | SWS_SELECT_GROUP))
    return fail(SWS_ERR_SHAPE, "%s: unknown flags 0x%x", fn, flags);
  if (hq < 1 || n_seqs < 0 || total_blocks < 0 || max_blocks < 0 || max_blocks > total_blocks ||
      (n_seqs == 0 && total_blocks != 0))
    return fail(SWS_ERR_SHAPE, "%s: hq=%d n_seqs=%d total_blocks=%d max_blocks=%d", fn, hq, n_seqs, total_blocks, max_blocks);
  if (hkv < 1 || hq % hkv != 0)
    return fail(SWS_ERR_SHAPE, "%s: hq=%d hkv=%d (hq must be a multiple of hkv)", fn, hq, hkv);
  if (max_blocks > 4096) return fail(SWS_ERR_UNSUPPORTED, "%s: max_blocks=%d > 4096", fn, max_blocks);
  if (rho_percent < 0 || rho_percent > 100)
    return fail(SWS_ERR_SHAPE, "%s: rho_percent=%d outside [0,100]", fn, rho_percent);
  const int need = dense ? max_blocks : std::min(max_blocks, tau_of(rho_percent, max_blocks) + 1);
  if (width < need || width < 1)
    return fail(SWS_ERR_SHAPE, "%s: width=%d < required %d", fn, width, need);
  return launched(sws::launch_select(R, hq, hkv, cu_blocks, n_seqs, total_blocks, max_blocks,
                                     rho_percent, flags, width, idx, cnt, (hipStream_t)stream),
                  fn);
}

sws_status sws_select_topk(const float* R, int32_t hq, const int32_t* cu_blocks, int32_t n_seqs,
                           int32_t total_blocks, int32_t max_blocks, int32_t rho_percent, int32_t dense,
                           int32_t width, int32_t* idx, int32_t* cnt, void* stream) {
  const RocRange roctx_range("sws_select_topk");
  return select_topk_impl("sws_select_topk", R, hq, hq, cu_blocks, n_seqs, total_blocks,
                          max_blocks, rho_percent, dense ? SWS_SELECT_DENSE : 0, width, idx, cnt,
                          stream);
}

sws_status sws_select_topk_flags(const float* R, int32_t hq, int32_t hkv, const int32_t* cu_blocks,
                                 int32_t n_seqs, int32_t total_blocks, int32_t max_blocks,
                                 int32_t rho_percent, int32_t flags, int32_t width, int32_t* idx,
                                 int32_t* cnt, void* stream) {
  const RocRange roctx_range("sws_select_topk_flags");
  return select_topk_impl("sws_select_topk_flags", R, hq, hkv, cu_blocks, n_seqs, total_blocks,
                          max_blocks, rho_percent, flags, width, idx, cnt, stream);
}

sws_status sws_select_topk_row(const float* r, int32_t hq, int32_t hkv, int32_t n_seqs,
                               const int32_t* cur_block, int32_t b_max, int32_t rho_percent,
                               int32_t flags, int32_t width, int32_t* idx, int32_t* cnt,
                               int32_t* union_idx, int32_t* union_cnt, uint32_t* union_mask,
                               int32_t union_width, void* stream) {
  const RocRange roctx_range("sws_select_topk_row");
  const char* fn = "sws_select_topk_row";
  const bool dense = (flags & SWS_SELECT_DENSE) != 0;
  if (flags & ~(SWS_SELECT_DENSE | SWS_SELECT_ROW_TAU | SWS_SELECT_GROUP))
    return fail(SWS_ERR_SHAPE, "%s: unknown flags 0x%x", fn, flags);
  if (!dense) REQUIRE_PTR(r);
  REQUIRE_PTR(cur_block);
  REQUIRE_PTR(union_idx);
  REQUIRE_PTR(union_cnt);
  REQUIRE_PTR(union_mask);
  if ((idx == nullptr) != (cnt == nullptr))
    return fail(SWS_ERR_NULL, "%s: idx and cnt must both be set or both be NULL", fn);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SWS_ERR_SHAPE, "%s: hq=%d hkv=%d (hq must be a multiple of hkv)", fn, hq, hkv);
  if (hq / hkv > 16) return fail(SWS_ERR_UNSUPPORTED, "%s: hq/hkv=%d > 16", fn, hq / hkv);
  if (n_seqs < 0 || b_max < 1 || b_max > 4096)
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d b_max=%d (b_max in [1,4096])", fn, n_seqs, b_max);
  if (rho_percent < 0 || rho_percent > 100)
    return fail(SWS_ERR_SHAPE, "%s: rho_percent=%d outside [0,100]", fn, rho_percent);
  const int tmax = tau_of(rho_percent, b_max);
  const int need = dense ? b_max : std::min(b_max, tmax + 1);
  const int uneed = dense ? b_max : std::min(b_max, (hq / hkv) * tmax + 1);
  if (idx && width < need) return fail(SWS_ERR_SHAPE, "%s: width=%d < required %d", fn, width, need);
  if (union_width < uneed)
    return fail(SWS_ERR_SHAPE, "%s: union_width=%d < required %d", fn, union_width, uneed);
  return launched(sws::launch_select_row(r, hq, hkv, n_seqs, cur_block, b_max, rho_percent,
                                         flags, width, idx, cnt, union_idx, union_cnt,
                                         union_mask, union_width, (hipStream_t)stream),
                  fn);
}

sws_status sws_sparse_attn_prefill(const void* q, const void* k, const void* v, int dtype,
                                   const int32_t* cu_seqlens, const int32_t* cu_blocks, int32_t n_seqs,
                                   int32_t total_blocks, int32_t max_blocks, int32_t hq, int32_t hkv,
                                   int32_t d, int32_t B, const int32_t* idx, const int32_t* cnt,
                                   int32_t width, float scale, void* out, float* lse, void* ws,
                                   size_t ws_bytes, void* stream) {
  const RocRange roctx_range("sws_sparse_attn_prefill");
  const char* fn = "sws_sparse_attn_prefill";
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(cu_seqlens);
  REQUIRE_PTR(cu_blocks);
  REQUIRE_PTR(out);
  if (idx && !cnt) return fail(SWS_ERR_NULL, "%s: idx given without cnt", fn);
  if (!dtype_ok(dtype)) return fail(SWS_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (d != 64 && d != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: d=%d not in {64,128}", fn, d);
  if (B != 64 && B != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: B=%d not in {64,128}", fn, B);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SWS_ERR_SHAPE, "%s: hq=%d hkv=%d (hq must be a multiple of hkv)", fn, hq, hkv);
  if (n_seqs < 0 || total_blocks < 0 || max_blocks < 0 || max_blocks > total_blocks ||
      (n_seqs == 0 && total_blocks != 0))
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d total_blocks=%d max_blocks=%d", fn, n_seqs, total_blocks, max_blocks);
  if ((int64_t)total_blocks * hq > 0x7fffffffLL)
    return fail(SWS_ERR_SHAPE, "%s: total_blocks*hq too large", fn);
  if (idx && width < 1) return fail(SWS_ERR_SHAPE, "%s: width=%d", fn, width);
  if (!std::isfinite(scale)) return fail(SWS_ERR_SHAPE, "%s: scale is not finite", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(SWS_ERR_SHAPE, "%s: q/k/v/out must be 16-byte aligned", fn);
  const size_t need = sws_prefill_workspace_size(dtype, total_blocks, hkv, d, B);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
    return fail(SWS_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu (or misaligned)", fn,
                ws_bytes, need);
  return launched(sws::launch_attn_prefill(q, k, v, dtype, cu_seqlens, cu_blocks, n_seqs,
                                           total_blocks, max_blocks, hq, hkv, d, B, idx, cnt,
                                           width, scale, out, lse, ws, (hipStream_t)stream),
                  fn);
}

size_t sws_prefill_workspace_size(int dtype, int32_t total_blocks, int32_t hkv, int32_t d,
                                  int32_t B) {
  if (dtype != SWS_BF16 || total_blocks < 0 || hkv < 1 || d < 1 || B < 1) return 0;
  return (size_t)hkv * (size_t)total_blocks * (size_t)d * (size_t)B * 2u;
}

size_t sws_decode_workspace_size(int32_t n_seqs, int32_t hq, int32_t hkv, int32_t d, int32_t B,
                                 int32_t union_width) {
  if (n_seqs < 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || (d != 64 && d != 128) ||
      (B != 64 && B != 128) || union_width < 0)
    return 0;
  return sws::decode_workspace_bytes(n_seqs, hq, hkv, d, B, union_width);
}

}  // extern "C"

namespace {

// Split-KV records of sws_sparse_attn_decode_noalloc: a fixed device array
// (each GPU holds its own copy while the library is loaded), used instead of
// a caller workspace by callers that cannot allocate device memory.  Host
// code must not pass `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory): its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[SWS_DECODE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices] = {};

sws_status scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SWS_ERR_LAUNCH, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SWS_ERR_UNSUPPORTED, "%s: device %d beyond the %d this library tracks", fn, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SWS_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return SWS_OK;
}

// Validation and launch shared by the two contiguous-cache decode calls; with
// use_scratch the split-KV records go to the device array above.
sws_status decode_contiguous(const char* fn, const void* q, const void* k_cache,
                             const void* v_cache, int dtype, const int32_t* ctx_len,
                             int32_t n_seqs, int32_t max_ctx, int32_t hq, int32_t hkv, int32_t d,
                             int32_t B, const int32_t* union_idx, const int32_t* union_cnt,
                             const uint32_t* union_mask, int32_t union_width, float scale,
                             void* out, float* lse, void* ws, size_t ws_bytes, bool use_scratch,
                             void* stream) {
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(ctx_len);
  REQUIRE_PTR(out);
  if (union_idx && (!union_cnt || !union_mask))
    return fail(SWS_ERR_NULL, "%s: union_idx given without union_cnt / union_mask", fn);
  const bool head_major = (dtype & SWS_KV_HEAD_MAJOR) != 0;
  dtype &= ~SWS_KV_HEAD_MAJOR;
  if (!dtype_ok(dtype)) return fail(SWS_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (d != 64 && d != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: d=%d not in {64,128}", fn, d);
  if (B != 64 && B != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: B=%d not in {64,128}", fn, B);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SWS_ERR_SHAPE, "%s: hq=%d hkv=%d (hq must be a multiple of hkv)", fn, hq, hkv);
  if (hq / hkv > 16) return fail(SWS_ERR_UNSUPPORTED, "%s: hq/hkv=%d > 16", fn, hq / hkv);
  if (n_seqs < 0 || max_ctx < 1)
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d max_ctx=%d", fn, n_seqs, max_ctx);
  const int uw = union_idx ? union_width : (max_ctx + B - 1) / B;
  if (union_idx && union_width < 1) return fail(SWS_ERR_SHAPE, "%s: union_width=%d", fn, union_width);
  if ((int64_t)n_seqs * hkv > 8192)
    return fail(SWS_ERR_UNSUPPORTED, "%s: n_seqs * hkv = %lld > 8192", fn,
                (long long)n_seqs * hkv);
  if ((int64_t)n_seqs * hkv * uw > 0x7fffffffLL)
    return fail(SWS_ERR_SHAPE, "%s: n_seqs * hkv * union_width exceeds 2^31", fn);
  if (!std::isfinite(scale)) return fail(SWS_ERR_SHAPE, "%s: scale is not finite", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(SWS_ERR_SHAPE, "%s: q/k_cache/v_cache must be 16-byte aligned", fn);
  const size_t need = sws::decode_workspace_bytes(n_seqs, hq, hkv, d, B, uw);
  if (use_scratch) {
    if (need > (size_t)SWS_DECODE_NOALLOC_SCRATCH_BYTES)
      return fail(SWS_ERR_WORKSPACE,
                  "%s: the call needs %zu bytes of split-KV records, more than the fixed %zu",
                  fn, need, (size_t)SWS_DECODE_NOALLOC_SCRATCH_BYTES);
    if (n_seqs == 0) return ok();
    const sws_status st = scratch_address(fn, &ws);
    if (st != SWS_OK) return st;
  } else if (!ws || ws_bytes < need) {
    return fail(SWS_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
  }
  return launched(sws::launch_attn_decode(q, k_cache, v_cache, dtype, head_major, ctx_len, n_seqs,
                                          max_ctx, hq, hkv, d, B, union_idx, union_cnt,
                                          union_mask, uw, scale, out, lse, ws,
                                          (hipStream_t)stream),
                  fn);
}

}  // namespace

extern "C" {

sws_status sws_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache, int dtype,
                                  const int32_t* ctx_len, int32_t n_seqs, int32_t max_ctx, int32_t hq,
                                  int32_t hkv, int32_t d, int32_t B, const int32_t* union_idx,
                                  const int32_t* union_cnt, const uint32_t* union_mask,
                                  int32_t union_width, float scale, void* out, float* lse, void* ws,
                                  size_t ws_bytes, void* stream) {
  const RocRange roctx_range("sws_sparse_attn_decode");
  return decode_contiguous("sws_sparse_attn_decode", q, k_cache, v_cache, dtype, ctx_len, n_seqs,
                           max_ctx, hq, hkv, d, B, union_idx, union_cnt, union_mask, union_width,
                           scale, out, lse, ws, ws_bytes, false, stream);
}

sws_status sws_sparse_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          int dtype, const int32_t* ctx_len, int32_t n_seqs,
                                          int32_t max_ctx, int32_t hq, int32_t hkv, int32_t d,
                                          int32_t B, const int32_t* union_idx,
                                          const int32_t* union_cnt, const uint32_t* union_mask,
                                          int32_t union_width, float scale, void* out, float* lse,
                                          void* stream) {
  const RocRange roctx_range("sws_sparse_attn_decode_noalloc");
  return decode_contiguous("sws_sparse_attn_decode_noalloc", q, k_cache, v_cache, dtype, ctx_len,
                           n_seqs, max_ctx, hq, hkv, d, B, union_idx, union_cnt, union_mask,
                           union_width, scale, out, lse, nullptr, 0, true, stream);
}

sws_status sws_sparse_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                        int kv_dtype, float k_scale, float v_scale,
                                        const int32_t* block_table, int32_t table_width,
                                        int32_t num_pages, const int32_t* ctx_len, int32_t n_seqs,
                                        int32_t hq, int32_t hkv, int32_t d, int32_t B,
                                        const int32_t* union_idx, const int32_t* union_cnt,
                                        const uint32_t* union_mask, int32_t union_width, float scale,
                                        void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  const RocRange roctx_range("sws_sparse_attn_decode_paged");
  const char* fn = "sws_sparse_attn_decode_paged";
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_pages);
  REQUIRE_PTR(v_pages);
  REQUIRE_PTR(block_table);
  REQUIRE_PTR(ctx_len);
  REQUIRE_PTR(out);
  if (union_idx && (!union_cnt || !union_mask))
    return fail(SWS_ERR_NULL, "%s: union_idx given without union_cnt / union_mask", fn);
  const bool head_major = (kv_dtype & SWS_KV_HEAD_MAJOR) != 0;
  kv_dtype &= ~SWS_KV_HEAD_MAJOR;
  if (kv_dtype != SWS_BF16 && kv_dtype != SWS_FP8_E4M3)
    return fail(SWS_ERR_UNSUPPORTED, "%s: kv_dtype %d", fn, kv_dtype);
  if (d != 64 && d != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: d=%d not in {64,128}", fn, d);
  if (B != 64 && B != 128) return fail(SWS_ERR_UNSUPPORTED, "%s: B=%d not in {64,128}", fn, B);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SWS_ERR_SHAPE, "%s: hq=%d hkv=%d (hq must be a multiple of hkv)", fn, hq, hkv);
  if (hq / hkv > 16) return fail(SWS_ERR_UNSUPPORTED, "%s: hq/hkv=%d > 16", fn, hq / hkv);
  if (n_seqs < 0 || table_width < 1 || num_pages < 1)
    return fail(SWS_ERR_SHAPE, "%s: n_seqs=%d table_width=%d num_pages=%d", fn, n_seqs,
                table_width, num_pages);
  const int uw = union_idx ? union_width : table_width;
  if (union_idx && union_width < 1) return fail(SWS_ERR_SHAPE, "%s: union_width=%d", fn, union_width);
  if ((int64_t)n_seqs * hkv > 8192)
    return fail(SWS_ERR_UNSUPPORTED, "%s: n_seqs * hkv = %lld > 8192", fn,
                (long long)n_seqs * hkv);
  if ((int64_t)n_seqs * hkv * uw > 0x7fffffffLL)
    return fail(SWS_ERR_SHAPE, "%s: n_seqs * hkv * union_width exceeds 2^31", fn);
  if (!std::isfinite(scale)) return fail(SWS_ERR_SHAPE, "%s: scale is not finite", fn);
  if (kv_dtype == SWS_FP8_E4M3 && (!std::isfinite(k_scale) || !std::isfinite(v_scale)))
    return fail(SWS_ERR_SHAPE, "%s: k_scale / v_scale not finite", fn);
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages))
    return fail(SWS_ERR_SHAPE, "%s: q/k_pages/v_pages must be 16-byte aligned", fn);
  const size_t need = sws::decode_workspace_bytes(n_seqs, hq, hkv, d, B, uw);
  if (!ws || ws_bytes < need)
    return fail(SWS_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
  return launched(sws::launch_attn_decode_paged(
                      q, k_pages, v_pages, kv_dtype, head_major, k_scale, v_scale, block_table,
                      table_width,
                      num_pages, ctx_len, n_seqs, hq, hkv, d, B, union_idx, union_cnt,
                      union_mask, uw, scale, out, lse, ws, (hipStream_t)stream),
                  fn);
}

}  // extern "C"
