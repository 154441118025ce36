// C ABI of libcsa: host-side argument checks, then kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/csa.h"
#include "csa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA_OK;
  return fail(CSA_EHIP, "%s: HIP error %d (%s)", what, static_cast<int>(e), hipGetErrorString(e));
}

bool dtype_ok(int32_t dtype) { return dtype == CSA_F32 || dtype == CSA_BF16; }

constexpr int kMaxTopk = 2048;
constexpr int kMaxCandidates = 32768;

}  // namespace

extern "C" {

#ifdef CSA_DEBUG
const char* csa_version(void) { return "csa-gfx950 0.1.0+debug"; }
#else
const char* csa_version(void) { return "csa-gfx950 0.1.0"; }
#endif

const char* csa_last_error(void) { return g_last_error.c_str(); }

// Window sides: non-negative, and small enough that a stream row plus or minus a side
// (and the slot count left + right + 1) stays within int32.
static bool window_fits(int32_t wl, int32_t wr, int32_t Tkv) {
  return wl >= 0 && wr >= 0 && static_cast<long long>(Tkv) + wl + wr + 1 <= 0x7fffffffLL;
}

int csa_build_indices(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t B, int32_t Tq,
                      int32_t Tkv, int32_t global_start, int32_t cmp_ratio, int32_t ori_win_left,
                      int32_t ori_win_right, int32_t* q_seg, int32_t* q_pos, int32_t* win_idx,
                      int32_t* cu_seqlens_cmp, int32_t* cmp_residual, int32_t* q_cmp_lo, int32_t* q_cmp_nvis,
                      int32_t* cmp_group, int32_t Tc_cap, csa_stream_t stream) {
  if (!cu_seqlens_q || !cu_seqlens_kv) return fail(CSA_EINVAL, "csa_build_indices: cu_seqlens_q/kv must not be NULL");
  if (!cu_seqlens_cmp || !cmp_residual)
    return fail(CSA_EINVAL, "csa_build_indices: cu_seqlens_cmp and cmp_residual are required outputs");
  if (B < 1) return fail(CSA_EINVAL, "csa_build_indices: B must be >= 1 (got %d)", B);
  if (Tq < 0 || Tkv < 0 || global_start < 0)
    return fail(CSA_EINVAL, "csa_build_indices: Tq, Tkv and global_start must be >= 0");
  if (static_cast<long long>(global_start) + Tq > Tkv)
    return fail(CSA_EINVAL, "csa_build_indices: global_start + Tq (%lld) exceeds Tkv (%d)",
                static_cast<long long>(global_start) + Tq, Tkv);
  if (cmp_ratio < 1) return fail(CSA_EINVAL, "csa_build_indices: cmp_ratio must be >= 1");
  if (!window_fits(ori_win_left, ori_win_right, Tkv))
    return fail(CSA_EINVAL, "csa_build_indices: window sides must be >= 0 with Tkv + sides < 2^31");
  if (cmp_group && Tc_cap < Tkv / cmp_ratio)
    return fail(CSA_EINVAL, "csa_build_indices: Tc_cap (%d) < Tkv / cmp_ratio (%d)", Tc_cap, Tkv / cmp_ratio);
  return hip_status(csa::launch_build_indices(cu_seqlens_q, cu_seqlens_kv, B, Tq, Tkv, global_start, cmp_ratio,
                                              ori_win_left, ori_win_right, q_seg, q_pos, win_idx, cu_seqlens_cmp,
                                              cmp_residual, q_cmp_lo, q_cmp_nvis, cmp_group, Tc_cap,
                                              static_cast<hipStream_t>(stream)),
                    "csa_build_indices");
}

int csa_compress(const void* x, int32_t Tkv, int32_t d, int32_t dtype, const int32_t* cu_seqlens_kv,
                 const int32_t* cu_seqlens_cmp, int32_t B, int32_t cmp_ratio, void* x_cmp, int32_t Tc_cap,
                 csa_stream_t stream) {
  if (!cu_seqlens_kv || !cu_seqlens_cmp || (!x && Tkv > 0) || (!x_cmp && Tc_cap > 0))
    return fail(CSA_EINVAL, "csa_compress: NULL pointer");
  if (B < 1 || Tkv < 0 || d < 1 || cmp_ratio < 1)
    return fail(CSA_EINVAL, "csa_compress: need B >= 1, Tkv >= 0, d >= 1, cmp_ratio >= 1");
  if (!dtype_ok(dtype)) return fail(CSA_EINVAL, "csa_compress: unknown dtype %d", dtype);
  if (Tc_cap < Tkv / cmp_ratio)
    return fail(CSA_EINVAL, "csa_compress: Tc_cap (%d) < Tkv / cmp_ratio (%d)", Tc_cap, Tkv / cmp_ratio);
  const int vec = dtype == CSA_BF16 ? 8 : 4;
  if (d % vec) return fail(CSA_EUNSUPPORTED, "csa_compress: d (%d) must be a multiple of %d", d, vec);
  return hip_status(csa::launch_compress(x, Tkv, d, dtype, cu_seqlens_kv, cu_seqlens_cmp, B, cmp_ratio, x_cmp,
                                         Tc_cap, static_cast<hipStream_t>(stream)),
                    "csa_compress");
}

int csa_compress_learned(const void* x, int32_t Tkv, int32_t D, int32_t dtype, const void* wkv, const void* wgate,
                         const float* ape, int32_t hd, int32_t overlap, const int32_t* cu_seqlens_kv,
                         const int32_t* cu_seqlens_cmp, int32_t B, int32_t cmp_ratio, void* x_cmp, int32_t Tc_cap,
                         csa_stream_t stream) {
  if (!cu_seqlens_kv || !cu_seqlens_cmp || (Tkv > 0 && (!x || !wkv || !wgate || !ape)) || (!x_cmp && Tc_cap > 0))
    return fail(CSA_EINVAL, "csa_compress_learned: NULL pointer");
  if (B < 1 || Tkv < 0 || D < 1 || hd < 1 || cmp_ratio < 1 || (overlap != 0 && overlap != 1))
    return fail(CSA_EINVAL, "csa_compress_learned: need B >= 1, Tkv >= 0, D >= 1, hd >= 1, cmp_ratio >= 1, "
                "overlap 0 or 1");
  if (!dtype_ok(dtype)) return fail(CSA_EINVAL, "csa_compress_learned: unknown dtype %d", dtype);
  if (Tc_cap < Tkv / cmp_ratio)
    return fail(CSA_EINVAL, "csa_compress_learned: Tc_cap (%d) < Tkv / cmp_ratio (%d)", Tc_cap, Tkv / cmp_ratio);
  if (!csa::learned_shape_supported(D, hd, cmp_ratio, overlap, dtype))
    return fail(CSA_EUNSUPPORTED, "csa_compress_learned: no kernel for D=%d hd=%d cmp_ratio=%d overlap=%d dtype=%d",
                D, hd, cmp_ratio, overlap, dtype);
  if (static_cast<long long>(Tkv) * D * 2 > 0xFFFFFFFFLL)
    return fail(CSA_EUNSUPPORTED, "csa_compress_learned: x of %lld bytes exceeds 4 GiB",
                static_cast<long long>(Tkv) * D * 2);
  return hip_status(csa::launch_compress_learned(x, Tkv, D, wkv, wgate, ape, hd, overlap, cu_seqlens_kv,
                                                 cu_seqlens_cmp, B, x_cmp, Tc_cap, static_cast<hipStream_t>(stream)),
                    "csa_compress_learned");
}

int64_t csa_indexer_topk_workspace_bytes(int32_t Tq, int32_t max_seqlen_kv, int32_t cmp_ratio) {
  if (Tq < 0 || max_seqlen_kv < 0 || cmp_ratio < 1) return -1;
  return static_cast<int64_t>(csa::indexer_workspace_bytes(Tq, max_seqlen_kv / cmp_ratio));
}

int csa_indexer_topk(const void* q_I, const void* w, const void* k_I_cmp, int32_t Tq, int32_t Tc, int32_t H_I,
                     int32_t d_I, int32_t dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                     const int32_t* cu_seqlens_cmp, const int32_t* cmp_residual, int32_t B, int32_t global_start,
                     int32_t cmp_ratio, int32_t max_seqlen_kv, int32_t topk, int32_t* topk_idx, float* topk_score,
                     void* workspace, int64_t workspace_bytes, csa_stream_t stream) {
  if (!cu_seqlens_q || !cu_seqlens_kv || !cu_seqlens_cmp || (Tc > 0 && !k_I_cmp) ||
      (Tq != 0 && (!q_I || !w || !topk_idx)))
    return fail(CSA_EINVAL, "csa_indexer_topk: NULL pointer");
  if (B < 1 || Tq < 0 || Tc < 0 || H_I < 1 || d_I < 1 || topk < 1 || cmp_ratio < 1 || max_seqlen_kv < 0 ||
      global_start < 0)
    return fail(CSA_EINVAL, "csa_indexer_topk: invalid size or parameter");
  if (!dtype_ok(dtype)) return fail(CSA_EINVAL, "csa_indexer_topk: unknown dtype %d", dtype);
  if (topk > kMaxTopk) return fail(CSA_EUNSUPPORTED, "csa_indexer_topk: topk %d > %d", topk, kMaxTopk);
  const int cap = max_seqlen_kv / cmp_ratio;
  if (cap > kMaxCandidates)
    return fail(CSA_EUNSUPPORTED, "csa_indexer_topk: max_seqlen_kv / cmp_ratio = %d candidates > %d", cap,
                kMaxCandidates);
  if (!csa::indexer_shape_supported(H_I, d_I, dtype))
    return fail(CSA_EUNSUPPORTED, "csa_indexer_topk: no kernel for H_I=%d d_I=%d dtype=%d", H_I, d_I, dtype);
  const int64_t need = static_cast<int64_t>(csa::indexer_workspace_bytes(Tq, cap));
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(CSA_EINVAL, "csa_indexer_topk: workspace of %lld bytes < %lld needed",
                workspace ? static_cast<long long>(workspace_bytes) : 0LL, static_cast<long long>(need));
  return hip_status(csa::launch_indexer_topk(q_I, w, k_I_cmp, Tq, Tc, H_I, d_I, dtype, cu_seqlens_q, cu_seqlens_kv,
                                             cu_seqlens_cmp, cmp_residual, B, global_start, cmp_ratio, cap, topk,
                                             topk_idx, topk_score, workspace, static_cast<hipStream_t>(stream)),
                    "csa_indexer_topk");
}

// Index rows: every valid entry a compressed row visible to its query, none repeated
// (synchronises the stream; csa_validate_topk_rows, and every call taking top-k rows in
// a CSA_DEBUG build).
static int rows_check(const char* name, const int32_t* cmp_idx, int32_t topk, int32_t Tq, int32_t Tc,
                      const int32_t* cu_q, const int32_t* cu_kv, const int32_t* cu_cmp, int32_t B,
                      int32_t global_start, int32_t cmp_ratio, csa_stream_t stream) {
  long long q = -1;
  int entry = -1, reason = 0;
  const hipError_t e = csa::check_topk_rows(cmp_idx, topk, Tq, cu_q, cu_kv, cu_cmp, B, global_start, cmp_ratio, Tc,
                                            static_cast<hipStream_t>(stream), &q, &entry, &reason);
  if (e != hipSuccess) return hip_status(e, name);
  if (q < 0) return CSA_OK;
  if (reason == 1)
    return fail(CSA_EINVAL, "%s: query %lld, index entry %d is not a compressed row visible to the query", name, q,
                entry);
  if (reason == 2) return fail(CSA_EINVAL, "%s: query %lld, index entry %d repeats an earlier entry", name, q, entry);
  return fail(CSA_EINVAL, "%s: query %lld sees more compressed rows than the check covers (32768)", name, q);
}

int csa_validate_topk_rows(const int32_t* cmp_idx, int32_t topk, int32_t Tq, int32_t Tc,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, const int32_t* cu_seqlens_cmp,
                           int32_t B, int32_t global_start, int32_t cmp_ratio, csa_stream_t stream) {
  if (!cu_seqlens_q || !cu_seqlens_kv || !cu_seqlens_cmp || (Tq > 0 && !cmp_idx) || topk < 1 || Tq < 0 || Tc < 0 ||
      B < 1 || global_start < 0 || cmp_ratio < 1)
    return fail(CSA_EINVAL, "csa_validate_topk_rows: invalid argument");
  return rows_check("csa_validate_topk_rows", cmp_idx, topk, Tq, Tc, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_cmp, B,
                    global_start, cmp_ratio, stream);
}

int csa_sparse_mla_fwd(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx, int32_t topk,
                       int32_t cmp_idx_kind, int32_t Tq, int32_t Tkv, int32_t Tc, int32_t H, int32_t d,
                       int32_t dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                       const int32_t* cu_seqlens_cmp, const int32_t* cmp_residual, int32_t B, int32_t global_start,
                       int32_t cmp_ratio, int32_t ori_win_left, int32_t ori_win_right, const float* sinks,
                       float softmax_scale, void* out, float* lse, csa_stream_t stream) {
  if (!cu_seqlens_q || !cu_seqlens_kv || !ori_kv || (Tq != 0 && (!q || !out)))
    return fail(CSA_EINVAL, "csa_sparse_mla_fwd: NULL pointer");
  if (cmp_kv && !cu_seqlens_cmp) return fail(CSA_EINVAL, "csa_sparse_mla_fwd: cmp_kv needs cu_seqlens_cmp");
  if (cmp_idx && !cmp_kv) return fail(CSA_EINVAL, "csa_sparse_mla_fwd: cmp_idx given without cmp_kv");
  if (cmp_idx && topk < 1) return fail(CSA_EINVAL, "csa_sparse_mla_fwd: topk must be >= 1 with cmp_idx");
  if (cmp_idx_kind != CSA_IDX_ANY && cmp_idx_kind != CSA_IDX_TOPK)
    return fail(CSA_EINVAL, "csa_sparse_mla_fwd: unknown cmp_idx_kind %d", cmp_idx_kind);
  if (B < 1 || Tq < 0 || Tkv < 0 || Tc < 0 || H < 1 || d < 1 || cmp_ratio < 1 || global_start < 0)
    return fail(CSA_EINVAL, "csa_sparse_mla_fwd: invalid size or parameter");
  if (!window_fits(ori_win_left, ori_win_right, Tkv))
    return fail(CSA_EINVAL, "csa_sparse_mla_fwd: window sides must be >= 0 with Tkv + sides < 2^31");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CSA_EINVAL, "csa_sparse_mla_fwd: softmax_scale (%g) must be positive and finite",
                static_cast<double>(softmax_scale));
  if (static_cast<long long>(global_start) + Tq > Tkv)
    return fail(CSA_EINVAL, "csa_sparse_mla_fwd: global_start + Tq exceeds Tkv");
  if (!dtype_ok(dtype)) return fail(CSA_EINVAL, "csa_sparse_mla_fwd: unknown dtype %d", dtype);
  if (cmp_idx && topk > kMaxTopk) return fail(CSA_EUNSUPPORTED, "csa_sparse_mla_fwd: topk %d > %d", topk, kMaxTopk);
  if (!csa::mla_shape_supported(H, d, dtype))
    return fail(CSA_EUNSUPPORTED, "csa_sparse_mla_fwd: no kernel for H=%d d=%d dtype=%d", H, d, dtype);
#ifdef CSA_DEBUG
  if (cmp_idx && cmp_kv && cmp_idx_kind == CSA_IDX_TOPK) {
    const int st = rows_check("csa_sparse_mla_fwd", cmp_idx, topk, Tq, Tc, cu_seqlens_q, cu_seqlens_kv,
                              cu_seqlens_cmp, B, global_start, cmp_ratio, stream);
    if (st != CSA_OK) return st;
  }
#endif
  return hip_status(csa::launch_sparse_mla(q, ori_kv, cmp_kv, cmp_idx, topk, cmp_idx_kind == CSA_IDX_TOPK, Tq,
                                           cmp_kv ? Tc : 0, H, d, dtype, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_cmp,
                                           cmp_residual, B, global_start, cmp_ratio, ori_win_left, ori_win_right,
                                           sinks, softmax_scale, out, lse, static_cast<hipStream_t>(stream)),
                    "csa_sparse_mla_fwd");
}

// Keys per query the backward may see: the window (no longer than a segment) plus the
// selected rows, or every visible compressed row (at most max_seqlen_kv / cmp_ratio)
// in attend-all mode.
static int bwd_key_cap(int32_t wl, int32_t wr, const void* cmp_kv, const int32_t* cmp_idx, int32_t topk,
                       int32_t max_seqlen_kv, int32_t cmp_ratio) {
  long long W = static_cast<long long>(wl) + wr + 1;
  if (W > max_seqlen_kv) W = max_seqlen_kv > 0 ? max_seqlen_kv : 1;
  long long c = 0;
  if (cmp_kv) c = cmp_idx ? topk : max_seqlen_kv / cmp_ratio;
  return static_cast<int>(W + c > (1LL << 30) ? (1LL << 30) : W + c);
}

// Visible compressed rows per query at most (the selection map of the sparse mode).
static int bwd_nvis_cap(const void* cmp_kv, const int32_t* cmp_idx, int32_t max_seqlen_kv, int32_t cmp_ratio) {
  return (cmp_kv && cmp_idx) ? max_seqlen_kv / cmp_ratio : 0;
}

int64_t csa_sparse_mla_bwd_workspace_bytes(int32_t Tq, int32_t ori_win_left, int32_t ori_win_right,
                                           const void* cmp_kv, const int32_t* cmp_idx, int32_t topk,
                                           int32_t max_seqlen_kv, int32_t cmp_ratio) {
  if (Tq < 0 || !window_fits(ori_win_left, ori_win_right, 0) || cmp_ratio < 1 || max_seqlen_kv < 0) return -1;
  const int cap = bwd_key_cap(ori_win_left, ori_win_right, cmp_kv, cmp_idx, topk, max_seqlen_kv, cmp_ratio);
  return static_cast<int64_t>(csa::mla_bwd_workspace_bytes(Tq, cap, bwd_nvis_cap(cmp_kv, cmp_idx, max_seqlen_kv,
                                                                                 cmp_ratio)));
}

// Partial row-gradient tiles of the deterministic backward (after the common workspace).
static int64_t bwd_partial_bytes(int32_t Tq, int32_t B, int32_t wl, int32_t wr, int32_t Tkv, const void* cmp_kv,
                                 int32_t max_seqlen_kv, int32_t cmp_ratio) {
  return static_cast<int64_t>(csa::mla_bwd_partial_bytes(Tq, B, wl, wr, Tkv, cmp_kv != nullptr, max_seqlen_kv,
                                                         cmp_ratio));
}

int64_t csa_sparse_mla_bwd_deterministic_workspace_bytes(int32_t Tq, int32_t B, int32_t ori_win_left,
                                                         int32_t ori_win_right, const void* cmp_kv,
                                                         const int32_t* cmp_idx, int32_t topk, int32_t max_seqlen_kv,
                                                         int32_t cmp_ratio) {
  const int64_t base = csa_sparse_mla_bwd_workspace_bytes(Tq, ori_win_left, ori_win_right, cmp_kv, cmp_idx, topk,
                                                          max_seqlen_kv, cmp_ratio);
  if (base < 0 || B < 1) return -1;
  return base + bwd_partial_bytes(Tq, B, ori_win_left, ori_win_right, 0x7fffffff, cmp_kv, max_seqlen_kv, cmp_ratio);
}

static int bwd_call(const char* name, bool deterministic, const void* q, const void* ori_kv, const void* cmp_kv,
                    const int32_t* cmp_idx, int32_t topk, int32_t Tq, int32_t Tkv, int32_t Tc, int32_t H, int32_t d,
                    int32_t dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                    const int32_t* cu_seqlens_cmp, int32_t B, int32_t global_start, int32_t cmp_ratio,
                    int32_t ori_win_left, int32_t ori_win_right, int32_t max_seqlen_kv, const float* sinks,
                    float softmax_scale, const void* out, const float* lse, const void* dout, void* dq,
                    float* d_ori_kv, float* d_cmp_kv, float* d_sinks, float* ori_l1, float* cmp_l1,
                    int32_t cmp_slots, void* workspace, int64_t workspace_bytes, csa_stream_t stream) {
  if (!cu_seqlens_q || !cu_seqlens_kv || !ori_kv || !d_ori_kv ||
      (Tq != 0 && (!q || !out || !lse || !dout || !dq || !workspace)))
    return fail(CSA_EINVAL, "%s: NULL pointer", name);
  if (cmp_kv && (!cu_seqlens_cmp || !d_cmp_kv)) return fail(CSA_EINVAL, "%s: cmp_kv needs cu_seqlens_cmp and d_cmp_kv", name);
  if (cmp_idx && !cmp_kv) return fail(CSA_EINVAL, "%s: cmp_idx given without cmp_kv", name);
  if (cmp_idx && topk < 1) return fail(CSA_EINVAL, "%s: topk must be >= 1 with cmp_idx", name);
  if (sinks && !d_sinks) return fail(CSA_EINVAL, "%s: sinks need d_sinks", name);
  if (cmp_l1 && cmp_slots < 1) return fail(CSA_EINVAL, "%s: cmp_l1 needs cmp_slots >= 1", name);
  if (B < 1 || Tq < 0 || Tkv < 0 || Tc < 0 || H < 1 || d < 1 || cmp_ratio < 1 || global_start < 0 ||
      max_seqlen_kv < 0 || cmp_slots < 0)
    return fail(CSA_EINVAL, "%s: invalid size or parameter", name);
  if (!window_fits(ori_win_left, ori_win_right, Tkv))
    return fail(CSA_EINVAL, "%s: window sides must be >= 0 with Tkv + sides < 2^31", name);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CSA_EINVAL, "%s: softmax_scale (%g) must be positive and finite", name,
                static_cast<double>(softmax_scale));
  if (static_cast<long long>(global_start) + Tq > Tkv)
    return fail(CSA_EINVAL, "%s: global_start + Tq exceeds Tkv", name);
  if (!dtype_ok(dtype)) return fail(CSA_EINVAL, "%s: unknown dtype %d", name, dtype);
  if (cmp_idx && topk > kMaxTopk) return fail(CSA_EUNSUPPORTED, "%s: topk %d > %d", name, topk, kMaxTopk);
  if (!csa::mla_bwd_shape_supported(H, d, dtype))
    return fail(CSA_EUNSUPPORTED, "%s: no kernel for H=%d d=%d dtype=%d", name, H, d, dtype);
  const int cap = bwd_key_cap(ori_win_left, ori_win_right, cmp_kv, cmp_idx, topk, max_seqlen_kv, cmp_ratio);
  const int nvis_cap = bwd_nvis_cap(cmp_kv, cmp_idx, max_seqlen_kv, cmp_ratio);
  int64_t need = static_cast<int64_t>(csa::mla_bwd_workspace_bytes(Tq, cap, nvis_cap));
  if (deterministic)
    need += bwd_partial_bytes(Tq, B, ori_win_left, ori_win_right, Tkv, cmp_kv, max_seqlen_kv, cmp_ratio);
  if (workspace_bytes < need)
    return fail(CSA_EINVAL, "%s: workspace of %lld bytes < %lld needed", name,
                static_cast<long long>(workspace_bytes), static_cast<long long>(need));
#ifdef CSA_DEBUG
  if (cmp_idx && cmp_kv) {
    const int st = rows_check(name, cmp_idx, topk, Tq, Tc, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_cmp, B,
                              global_start, cmp_ratio, stream);
    if (st != CSA_OK) return st;
  }
#endif
  return hip_status(csa::launch_sparse_mla_bwd(q, ori_kv, cmp_kv, cmp_idx, topk, Tq, Tkv, cmp_kv ? Tc : 0,
                                               cu_seqlens_q, cu_seqlens_kv, cu_seqlens_cmp, B, global_start,
                                               cmp_ratio, ori_win_left, ori_win_right, max_seqlen_kv, sinks,
                                               softmax_scale, out, lse, dout, dq, d_ori_kv,
                                               cmp_kv ? d_cmp_kv : nullptr, d_sinks, ori_l1, cmp_l1, cmp_slots, cap,
                                               nvis_cap, workspace, deterministic,
                                               static_cast<hipStream_t>(stream)),
                    name);
}

int csa_sparse_mla_bwd(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx, int32_t topk,
                       int32_t Tq, int32_t Tkv, int32_t Tc, int32_t H, int32_t d, int32_t dtype,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, const int32_t* cu_seqlens_cmp,
                       int32_t B, int32_t global_start, int32_t cmp_ratio, int32_t ori_win_left,
                       int32_t ori_win_right, int32_t max_seqlen_kv, const float* sinks, float softmax_scale,
                       const void* out, const float* lse, const void* dout, void* dq, float* d_ori_kv,
                       float* d_cmp_kv, float* d_sinks, float* ori_l1, float* cmp_l1, int32_t cmp_slots,
                       void* workspace, int64_t workspace_bytes, csa_stream_t stream) {
  return bwd_call("csa_sparse_mla_bwd", false, q, ori_kv, cmp_kv, cmp_idx, topk, Tq, Tkv, Tc, H, d, dtype,
                  cu_seqlens_q, cu_seqlens_kv, cu_seqlens_cmp, B, global_start, cmp_ratio, ori_win_left,
                  ori_win_right, max_seqlen_kv, sinks, softmax_scale, out, lse, dout, dq, d_ori_kv, d_cmp_kv, d_sinks,
                  ori_l1, cmp_l1, cmp_slots, workspace, workspace_bytes, stream);
}

int csa_sparse_mla_bwd_deterministic(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx,
                                     int32_t topk, int32_t Tq, int32_t Tkv, int32_t Tc, int32_t H, int32_t d,
                                     int32_t dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                     const int32_t* cu_seqlens_cmp, int32_t B, int32_t global_start,
                                     int32_t cmp_ratio, int32_t ori_win_left, int32_t ori_win_right,
                                     int32_t max_seqlen_kv, const float* sinks, float softmax_scale, const void* out,
                                     const float* lse, const void* dout, void* dq, float* d_ori_kv, float* d_cmp_kv,
                                     float* d_sinks, float* ori_l1, float* cmp_l1, int32_t cmp_slots,
                                     void* workspace, int64_t workspace_bytes, csa_stream_t stream) {
  return bwd_call("csa_sparse_mla_bwd_deterministic", true, q, ori_kv, cmp_kv, cmp_idx, topk, Tq, Tkv, Tc, H, d,
                  dtype, cu_seqlens_q, cu_seqlens_kv, cu_seqlens_cmp, B, global_start, cmp_ratio, ori_win_left,
                  ori_win_right, max_seqlen_kv, sinks, softmax_scale, out, lse, dout, dq, d_ori_kv, d_cmp_kv, d_sinks,
                  ori_l1, cmp_l1, cmp_slots, workspace, workspace_bytes, stream);
}

int64_t csa_indexer_kl_grad_workspace_bytes(int32_t Tq, int32_t topk, int32_t max_seqlen_kv, int32_t cmp_ratio) {
  if (Tq < 0 || topk < 1 || max_seqlen_kv < 0 || cmp_ratio < 1) return -1;
  return static_cast<int64_t>(csa::kl_workspace_bytes(Tq, topk, max_seqlen_kv / cmp_ratio));
}

int csa_indexer_kl_grad(const void* q_I, const void* w, const void* k_I_cmp, const int32_t* cmp_idx,
                        const float* attn_l1, int32_t topk, int32_t Tq, int32_t Tc, int32_t H_I, int32_t d_I,
                        int32_t dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                        const int32_t* cu_seqlens_cmp, int32_t B, int32_t global_start, int32_t cmp_ratio,
                        int32_t max_seqlen_kv, float loss_scale, void* d_q_I, float* d_w, float* d_k_I_cmp,
                        float* loss, void* workspace, int64_t workspace_bytes, csa_stream_t stream) {
  if (!cu_seqlens_q || !cu_seqlens_kv || !cu_seqlens_cmp || (Tc > 0 && (!k_I_cmp || !d_k_I_cmp)) ||
      (Tq != 0 && (!q_I || !w || !cmp_idx || !attn_l1 || !d_q_I || !d_w || !workspace)))
    return fail(CSA_EINVAL, "csa_indexer_kl_grad: NULL pointer");
  if (B < 1 || Tq < 0 || Tc < 0 || H_I < 1 || d_I < 1 || topk < 1 || cmp_ratio < 1 || global_start < 0 ||
      max_seqlen_kv < 0)
    return fail(CSA_EINVAL, "csa_indexer_kl_grad: invalid size or parameter");
  if (!dtype_ok(dtype)) return fail(CSA_EINVAL, "csa_indexer_kl_grad: unknown dtype %d", dtype);
  if (topk > kMaxTopk) return fail(CSA_EUNSUPPORTED, "csa_indexer_kl_grad: topk %d > %d", topk, kMaxTopk);
  if (!csa::kl_shape_supported(H_I, d_I, dtype))
    return fail(CSA_EUNSUPPORTED, "csa_indexer_kl_grad: no kernel for H_I=%d d_I=%d dtype=%d", H_I, d_I, dtype);
  const int nvis_cap = max_seqlen_kv / cmp_ratio;
  const int64_t need = static_cast<int64_t>(csa::kl_workspace_bytes(Tq, topk, nvis_cap));
  if (workspace_bytes < need)
    return fail(CSA_EINVAL, "csa_indexer_kl_grad: workspace of %lld bytes < %lld needed",
                static_cast<long long>(workspace_bytes), static_cast<long long>(need));
#ifdef CSA_DEBUG
  if (const int st = rows_check("csa_indexer_kl_grad", cmp_idx, topk, Tq, Tc, cu_seqlens_q, cu_seqlens_kv,
                                cu_seqlens_cmp, B, global_start, cmp_ratio, stream);
      st != CSA_OK)
    return st;
#endif
  return hip_status(csa::launch_indexer_kl_grad(q_I, w, k_I_cmp, cmp_idx, attn_l1, topk, Tq, Tc, cu_seqlens_q,
                                                cu_seqlens_kv, cu_seqlens_cmp, B, global_start, cmp_ratio,
                                                max_seqlen_kv, loss_scale, d_q_I, d_w, d_k_I_cmp, loss, nvis_cap,
                                                workspace, static_cast<hipStream_t>(stream)),
                    "csa_indexer_kl_grad");
}

int csa_indexer_kl_grad_noalloc(const void* q_I, const void* w, const void* k_I_cmp, const int32_t* cmp_idx,
                                const float* attn_l1, int32_t topk, int32_t Tq, int32_t Tc, int32_t H_I, int32_t d_I,
                                int32_t dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                const int32_t* cu_seqlens_cmp, int32_t B, int32_t global_start, int32_t cmp_ratio,
                                int32_t max_seqlen_kv, float loss_scale, void* d_q_I, float* d_w, float* d_k_I_cmp,
                                float* loss, csa_stream_t stream) {
  if (!cu_seqlens_q || !cu_seqlens_kv || !cu_seqlens_cmp || (Tc > 0 && (!k_I_cmp || !d_k_I_cmp)) ||
      (Tq != 0 && (!q_I || !w || !cmp_idx || !attn_l1 || !d_q_I || !d_w)))
    return fail(CSA_EINVAL, "csa_indexer_kl_grad_noalloc: NULL pointer");
  if (B < 1 || Tq < 0 || Tc < 0 || H_I < 1 || d_I < 1 || topk < 1 || cmp_ratio < 1 || global_start < 0 ||
      max_seqlen_kv < 0)
    return fail(CSA_EINVAL, "csa_indexer_kl_grad_noalloc: invalid size or parameter");
  if (!dtype_ok(dtype)) return fail(CSA_EINVAL, "csa_indexer_kl_grad_noalloc: unknown dtype %d", dtype);
  if (topk > kMaxTopk)
    return fail(CSA_EUNSUPPORTED, "csa_indexer_kl_grad_noalloc: topk %d > %d", topk, kMaxTopk);
  if (!csa::kl_shape_supported(H_I, d_I, dtype))
    return fail(CSA_EUNSUPPORTED, "csa_indexer_kl_grad_noalloc: no kernel for H_I=%d d_I=%d dtype=%d", H_I, d_I,
                dtype);
  const int nvis_cap = max_seqlen_kv / cmp_ratio;
  const size_t need = csa::kl_workspace_bytes(Tq, topk, nvis_cap);
  if (need > csa::kKlScratchBytes)
    return fail(CSA_EINVAL, "csa_indexer_kl_grad_noalloc: the call needs %zu bytes of scratch, more than the %zu "
                "the library holds (Tq * (4 topk + 2 floor(max_seqlen_kv / cmp_ratio)) must stay within it)",
                need, csa::kKlScratchBytes);
#ifdef CSA_DEBUG
  if (const int st = rows_check("csa_indexer_kl_grad_noalloc", cmp_idx, topk, Tq, Tc, cu_seqlens_q, cu_seqlens_kv,
                                cu_seqlens_cmp, B, global_start, cmp_ratio, stream);
      st != CSA_OK)
    return st;
#endif
  void* ws = nullptr;
  if (const int st = hip_status(csa::kl_scratch(&ws), "csa_indexer_kl_grad_noalloc"); st != CSA_OK) return st;
  return hip_status(csa::launch_indexer_kl_grad(q_I, w, k_I_cmp, cmp_idx, attn_l1, topk, Tq, Tc, cu_seqlens_q,
                                                cu_seqlens_kv, cu_seqlens_cmp, B, global_start, cmp_ratio,
                                                max_seqlen_kv, loss_scale, d_q_I, d_w, d_k_I_cmp, loss, nvis_cap, ws,
                                                static_cast<hipStream_t>(stream)),
                    "csa_indexer_kl_grad_noalloc");
}

int csa_validate_layout(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t B, int32_t Tq,
                        int32_t Tkv, int32_t global_start, int32_t max_seqlen_kv, int32_t cmp_ratio,
                        const int32_t* cu_seqlens_cmp, const int32_t* cmp_residual, csa_stream_t stream) {
  if (!cu_seqlens_q || !cu_seqlens_kv || B < 1 || Tq < 0 || Tkv < 0 || global_start < 0 || cmp_ratio < 0)
    return fail(CSA_EINVAL, "csa_validate_layout: invalid argument");
  std::vector<int32_t> cq(B + 1), ck(B + 1), cc(B + 1), rs(B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool want_cmp = cmp_ratio >= 1 && cu_seqlens_cmp, want_res = cmp_ratio >= 1 && cmp_residual;
  hipError_t e = hipMemcpyAsync(cq.data(), cu_seqlens_q, sizeof(int32_t) * (B + 1), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(ck.data(), cu_seqlens_kv, sizeof(int32_t) * (B + 1), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && want_cmp)
    e = hipMemcpyAsync(cc.data(), cu_seqlens_cmp, sizeof(int32_t) * (B + 1), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && want_res)
    e = hipMemcpyAsync(rs.data(), cmp_residual, sizeof(int32_t) * B, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "csa_validate_layout");
  if (ck[0] != 0) return fail(CSA_EINVAL, "csa_validate_layout: cu_seqlens_kv[0] = %d, expected 0", ck[0]);
  for (int b = 0; b < B; ++b) {
    if (ck[b + 1] < ck[b]) return fail(CSA_EINVAL, "csa_validate_layout: cu_seqlens_kv decreases at %d", b + 1);
    if (max_seqlen_kv >= 0 && ck[b + 1] - ck[b] > max_seqlen_kv)
      return fail(CSA_EINVAL, "csa_validate_layout: segment %d has %d rows > max_seqlen_kv %d", b,
                  ck[b + 1] - ck[b], max_seqlen_kv);
  }
  if (ck[B] != Tkv) return fail(CSA_EINVAL, "csa_validate_layout: cu_seqlens_kv[B] = %d != Tkv = %d", ck[B], Tkv);
  for (int b = 0; b <= B; ++b) {
    long long want = static_cast<long long>(ck[b]) - global_start;
    want = want < 0 ? 0 : (want > Tq ? Tq : want);
    if (cq[b] != want)
      return fail(CSA_EINVAL, "csa_validate_layout: cu_seqlens_q[%d] = %d, expected %lld", b, cq[b], want);
  }
  long long acc = 0;
  for (int b = 0; b < B; ++b) {
    const int len = ck[b + 1] - ck[b];
    if (want_cmp) {
      if (cc[b] != acc)
        return fail(CSA_EINVAL, "csa_validate_layout: cu_seqlens_cmp[%d] = %d, expected %lld", b, cc[b], acc);
      acc += len / cmp_ratio;
      if (b + 1 == B && cc[B] != acc)
        return fail(CSA_EINVAL, "csa_validate_layout: cu_seqlens_cmp[%d] = %d, expected %lld", B, cc[B], acc);
    }
    if (want_res && rs[b] != len % cmp_ratio)
      return fail(CSA_EINVAL, "csa_validate_layout: cmp_residual[%d] = %d, expected %d (segment length %d mod %d)",
                  b, rs[b], len % cmp_ratio, len, cmp_ratio);
  }
  return CSA_OK;
}

}  // extern "C"
