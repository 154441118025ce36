/*
 * csa.h - C ABI of the MI355X (gfx950) library for the forward pass of
 * DeepSeek-V4 Compressed Sparse Attention (CSA) on a THD-packed token stream.
 *
 * Pages cited (by title and section):
 *   [MI] "PR #2038 完整报告: Enable THD packed-sequence training for
 *        DeepSeek-V4-Flash, with context parallelism" - 功能与动机, 实现拆解,
 *        关键源码片段 (thd_utils.py, deepseek_v4.py, compressor.py), 风险与影响.
 *   [HP] "【RFC】DeepSeek-V4 CSA/HCA 自定义算子接入与对外接口对标 torch_extension" -
 *        背景, 1. npu_lightning_indexer, 2. npu_sparse_flash_mla,
 *        缺失入参的用途分析（对照实验）.
 *   [MS] "MindSpeed-LLM pull 4842" - 主要改动.
 *   [ML] "feat(deepseek_v4): faithful THD context-parallel path for DS4 CSA
 *        (bounded activation memory)" - Design, Environment note.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller, contiguous,
 *   row-major.  The library allocates nothing and keeps no state between calls
 *   (besides two device arrays it holds per GPU: the workspace of
 *   csa_indexer_kl_grad_noalloc and the 8-byte result of csa_validate_topk_rows).
 * - Every call enqueues its kernels on `stream` (a hipStream_t; NULL = the null
 *   stream) and returns without synchronising.  Outputs are valid once the
 *   stream reaches that point.
 * - Host integers size the grids, so no call copies anything device -> host (the
 *   two csa_validate_* checks excepted: they are synchronous).
 * - Debug build: the library built with CSA_DEBUG defined (libcsa_debug.so, from
 *   `build.py --debug`; csa_version() ends in "+debug") runs csa_validate_topk_rows
 *   on the index rows of csa_sparse_mla_bwd(_deterministic), csa_indexer_kl_grad(_noalloc)
 *   and csa_sparse_mla_fwd with CSA_IDX_TOPK before launching, synchronising the
 *   stream, and fails those calls with CSA_EINVAL naming the first bad query.
 * - THD layout: `cu_seqlens_kv` [B+1] int32 holds stream-absolute segment
 *   bounds (the prefix of the stream whose KV is resident; a context-parallel
 *   rank passes the global segmentation truncated at its KV prefix end).
 *   `cu_seqlens_q` [B+1] int32 counts this call's local query rows per segment.
 *   Local query row i is stream row t = global_start + i ([MI] 关键源码片段,
 *   ThdLayout.from_packed_seq_params); it must lie inside its segment:
 *   cu_seqlens_q[b] == clamp(cu_seqlens_kv[b] - global_start, 0, Tq) for all b.
 *   `csa_validate_layout` checks this synchronously; the other calls assume it.
 * - Compressed rows: segment b owns floor(len_b / r) rows, numbered stream-
 *   absolutely from cu_seqlens_cmp[b] ([MI] compressor._forward_thd).  Buffers
 *   of compressed rows are sized Tc_cap >= floor(Tkv / r) >= the true count
 *   cu_seqlens_cmp[B]; rows at or past the true count are never written.
 * - dtype: CSA_BF16 (bfloat16 storage, fp32 accumulation) or CSA_F32.
 *   `sinks`, `lse` and `topk_score` are always float32; indices are int32.
 * - A tensor argument whose governing size is zero (e.g. q when Tq == 0) may be NULL.
 * - Return value: CSA_OK or an error code.  All argument checks run on the host
 *   before any launch, so a failed call enqueues nothing and writes nothing.
 *   csa_last_error() returns the calling thread's last error message.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* csa_stream_t; /* hipStream_t */

enum {
  CSA_OK = 0,
  CSA_EINVAL = 1,        /* a pointer, size or parameter is invalid */
  CSA_EUNSUPPORTED = 2,  /* a shape combination no kernel is built for */
  CSA_EHIP = 4           /* the HIP runtime reported an error (message has its text) */
};

enum { CSA_F32 = 0, CSA_BF16 = 1 };

/* Library version string, e.g. "csa-gfx950 0.1.0". */
const char* csa_version(void);

/* Message of the calling thread's last failed call ("" if none). */
const char* csa_last_error(void);

/*
 * csa_build_indices - segment layout of a THD pack (integer, bit-exact).
 *
 * Defined by [MI] 功能与动机 (windows clamp to the query's own segment start,
 * positions restart per segment, compressor groups respect segment bounds) and
 * [MI] 关键源码片段 thd_utils.get_window_topk_idxs_thd / compressed_cu_seqlens.
 *
 * Outputs, per segment b:
 *   cu_seqlens_cmp [B+1]  prefix sums of floor(len_b / r)               (required)
 *   cmp_residual   [B]    len_b mod r, the tail that forms no row ([HP] 背景 1) (required)
 * per local query row i (t = global_start + i, segment b, p = t - s_b):
 *   q_seg      [Tq]      b
 *   q_pos      [Tq]      p (rotary position, restarts per segment)
 *   win_idx    [Tq, W]   W = ori_win_left + ori_win_right + 1 slots; slot k holds
 *                        lo + k while lo + k <= hi, else -1, where
 *                        lo = max(s_b, t - ori_win_left), hi = min(e_b - 1, t + ori_win_right)
 *   q_cmp_lo   [Tq]      cu_seqlens_cmp[b]
 *   q_cmp_nvis [Tq]      floor((p + 1) / r): causally complete compressed rows
 * per compressed row c < cu_seqlens_cmp[B]:
 *   cmp_group  [Tc_cap]  segment-local group id c - cu_seqlens_cmp[b]
 * Every per-query / per-row output pointer may be NULL (not written).
 * Errors: EINVAL for NULL cu_seqlens_*, B < 1, Tq < 0, Tkv < 0, global_start < 0,
 * global_start + Tq > Tkv, cmp_ratio < 1, a window side < 0 (or Tkv plus both
 * sides >= 2^31), Tc_cap < Tkv / r,
 * or a NULL required output.
 */
int csa_build_indices(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t B,
                      int32_t Tq, int32_t Tkv, int32_t global_start, int32_t cmp_ratio,
                      int32_t ori_win_left, int32_t ori_win_right,
                      int32_t* q_seg, int32_t* q_pos, int32_t* win_idx,
                      int32_t* cu_seqlens_cmp, int32_t* cmp_residual,
                      int32_t* q_cmp_lo, int32_t* q_cmp_nvis, int32_t* cmp_group,
                      int32_t Tc_cap, csa_stream_t stream);

/*
 * csa_compress - segment-local mean pooling of cmp_ratio consecutive rows.
 *
 * x [Tkv, d] -> x_cmp [Tc_cap, d]; compressed row c of segment b (group
 * j = c - cu_seqlens_cmp[b]) is the mean of stream rows s_b + j*r + [0, r)
 * ([MI] compressor._forward_thd group gather; the learned pooling tail is not
 * printed there, the mean is this library's operator).  The sum is formed in
 * float64 in ascending row order and rounded once to the storage dtype (nearest,
 * ties to even).  Tail rows are never read.  `cu_seqlens_cmp` is the device array
 * written by csa_build_indices.  Used for the latent KV (d = 512) and the
 * indexer keys (d = 128).
 * Errors: EINVAL for NULL pointers, B < 1, Tkv < 0, d < 1, cmp_ratio < 1,
 * Tc_cap < Tkv / r, unknown dtype; EUNSUPPORTED when d is not a multiple of
 * 16 bytes' worth of elements (8 for bf16, 4 for f32).
 */
int csa_compress(const void* x, int32_t Tkv, int32_t d, int32_t dtype,
                 const int32_t* cu_seqlens_kv, const int32_t* cu_seqlens_cmp, int32_t B,
                 int32_t cmp_ratio, void* x_cmp, int32_t Tc_cap, csa_stream_t stream);

/*
 * csa_compress_learned - the learned gated, overlapping compressor ([MI] 关键源码片段
 * compressor.py: _forward_thd and _overlap_transform_thd), in place of mean pooling.
 *
 * For compressed row c (segment b, group j = c - cu_seqlens_cmp[b], stream rows
 * t_m = s_b + j*r + m, m < r):
 *   kv[m]    = x[t_m] wkv^T,  score[m] = x[t_m] wgate^T + ape[m]   (C channels each)
 *   overlap = 1 (C = 2 hd): 2r positions of hd channels, positions m < r taking the
 *     previous group's channels [0, hd) (its kv, its score), positions r + m the
 *     group's own channels [hd, 2 hd); a segment's first group has no previous group
 *     (kv 0, score -inf at those positions).  overlap = 0 (C = hd): the r positions.
 *   x_cmp[c, ch] = sum over positions of softmax(score[., ch]) kv[., ch]
 * The page prints the position table as ape.view(1, ratio, 1, -1) without its use;
 * it is read as an addition to the scores.  The page also elides the pooling tail;
 * it is read as the per-channel softmax over the positions and the weighted sum.
 * Products are bf16 x bf16 summed in float32 (MFMA), the softmax is float32 and
 * x_cmp is rounded once to bf16.  Tail rows are never read.
 *   x [Tkv, D], wkv and wgate [C, D] (call dtype), ape [cmp_ratio, C] float32,
 *   x_cmp [Tc_cap, hd] (call dtype; rows >= cu_seqlens_cmp[B] untouched).
 * Errors: EINVAL for NULL pointers, B < 1, Tkv < 0, D < 1, hd < 1, cmp_ratio < 1,
 * overlap other than 0 / 1, Tc_cap < Tkv / r, unknown dtype; EUNSUPPORTED unless
 * dtype is bf16, cmp_ratio = 4, D is a multiple of 64, hd a multiple of 64 (overlap)
 * or 128 (no overlap), and x spans less than 4 GiB.
 */
int csa_compress_learned(const void* x, int32_t Tkv, int32_t D, int32_t dtype, const void* wkv, const void* wgate,
                         const float* ape, int32_t hd, int32_t overlap, const int32_t* cu_seqlens_kv,
                         const int32_t* cu_seqlens_cmp, int32_t B, int32_t cmp_ratio, void* x_cmp, int32_t Tc_cap,
                         csa_stream_t stream);

/*
 * csa_indexer_topk - lightning indexer scores and per-query top-k within the
 * query's own segment ([HP] 1. npu_lightning_indexer; [MI] 功能与动机 item 4).
 *
 * For local query i in segment b at position p, the candidates are compressed
 * rows c in [cu_seqlens_cmp[b], cu_seqlens_cmp[b] + floor((p+1)/r)), scored
 *     score(i, c) = sum_h w[i, h] * max(0, <q_I[i, h, :], k_I_cmp[c, :]>)
 * with float32 accumulation.  If there are at most `topk` candidates all are
 * kept; otherwise the `topk` highest scores are kept, exact ties going to the
 * lower row (-0.0 ranks equal to +0.0).  topk_idx[i, :] lists the kept rows in
 * ascending order (stream-absolute compressed-row ids, as on [MI] 评论区精华
 * item 1), then -1.  topk_score (optional, may be NULL) holds each kept row's
 * score aligned with topk_idx, -inf in empty slots.
 *   q_I [Tq, H_I, d_I], w [Tq, H_I] (call dtype), k_I_cmp [Tc, d_I] (call dtype,
 *   from csa_compress), topk_idx [Tq, topk] int32, topk_score [Tq, topk] float32.
 * Tc is the number of rows k_I_cmp holds: candidates at or past
 * min(Tc, cu_seqlens_cmp[B]) are never read (they do not exist).
 * cmp_residual (optional, [B] int32 device, may be NULL): the per-segment tail
 * count len_b mod r that the operator schema carries as cmp_residual_k ([HP] 1.,
 * item 9; 背景 1: it fixes the valid compressed range).  Here cu_seqlens_kv already
 * fixes that range, so the value must equal len_b mod r (what csa_build_indices
 * writes); a query whose segment disagrees gets an all -1 row (and NaN scores), so
 * a stale residual shows in the output instead of passing silently.
 * workspace: device memory of at least csa_indexer_topk_workspace_bytes(Tq,
 * max_seqlen_kv, cmp_ratio) = Tq * floor(max_seqlen_kv / r) * 4 bytes, owned by the caller:
 * the order-preserving keys of the scores, written by a scoring pass and read by the
 * selection (no memory is allocated; nothing in it needs clearing).
 * `max_seqlen_kv` must bound every segment length; it sizes the workspace rows (and,
 * for the small shapes, the on-chip key storage): floor(max_seqlen_kv / r) candidates
 * per query.  Segments longer than it give unspecified (but in-bounds) results.
 * Errors: EINVAL for NULL required pointers, B < 1, Tq < 0, Tc < 0, H_I < 1, d_I < 1,
 * topk < 1, cmp_ratio < 1, max_seqlen_kv < 0, a missing or short workspace; EUNSUPPORTED
 * for floor(max_seqlen_kv / r) > 32768 candidates, topk > 2048, or a shape other
 * than (H_I, d_I) = (64, 128) bf16 or H_I * d_I <= 8192 with d_I % 8 == 0.
 */
int64_t csa_indexer_topk_workspace_bytes(int32_t Tq, int32_t max_seqlen_kv, int32_t cmp_ratio);
int csa_indexer_topk(const void* q_I, const void* w, const void* k_I_cmp,
                     int32_t Tq, int32_t Tc, int32_t H_I, int32_t d_I, int32_t dtype,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                     const int32_t* cu_seqlens_cmp, const int32_t* cmp_residual, int32_t B,
                     int32_t global_start, int32_t cmp_ratio, int32_t max_seqlen_kv, int32_t topk,
                     int32_t* topk_idx, float* topk_score, void* workspace, int64_t workspace_bytes,
                     csa_stream_t stream);

/* How the rows of a cmp_idx argument were formed (csa_sparse_mla_fwd). */
enum {
  CSA_IDX_ANY = 0,  /* any entries, any order: entries outside [0, Tc) are skipped */
  CSA_IDX_TOPK = 1  /* csa_indexer_topk's output for this layout and topk (see below) */
};

/*
 * csa_sparse_mla_fwd - sparse MLA forward over one shared latent KV
 * ([HP] 背景 item 2 and 2. npu_sparse_flash_mla; DS4 geometry d = d_v = 512,
 * [ML] Environment note).
 *
 * For local query i (stream row t, segment b) and head h the keys are
 *   window rows   ori_kv[lo .. hi], lo = max(s_b, t - ori_win_left),
 *                 hi = min(e_b - 1, t + ori_win_right)   (band parameters, not an
 *                 index list: [HP] 对照实验 shows ori_sparse_indices is ignored)
 *   compressed    cmp_kv[c] for every valid c in cmp_idx[i, 0:topk]  (sparse), or
 *                 every causally complete row of the segment when cmp_idx is NULL
 *                 (compressor-only layers, [MS] 主要改动 LayerCompressMode), or
 *                 none when cmp_kv is NULL (no compression).
 * Keys are also values (K = V).  One joint softmax spans both branches and the
 * sink: logits z = softmax_scale * <q[i,h], key>, the sink logit sinks[h] (not
 * scaled) adds exp(sinks[h]) to the denominator with a zero value.  Online
 * softmax in float32; MFMA products of bf16 inputs with float32 accumulation.
 *   q [Tq, H, d], ori_kv [Tkv, d], cmp_kv [Tc, d] (call dtype),
 *   cmp_idx [Tq, topk] int32, sinks [H] float32 (NULL = no sink),
 *   out [Tq, H, d] (call dtype), lse [Tq, H] float32 (NULL = not written):
 *   natural log of the full denominator in the scaled-logit domain.
 * Tc is the number of rows cmp_kv holds; rows at or past min(Tc, cu_seqlens_cmp[B])
 * are never read.
 * cmp_idx_kind says how the cmp_idx rows were formed:
 *   CSA_IDX_ANY   valid entries are those in [0, min(Tc, cu_seqlens_cmp[B])), in any
 *                 order; the others are skipped.
 *   CSA_IDX_TOPK  the rows are csa_indexer_topk's output for the same layout, Tc
 *                 and topk.  The top-k of at most topk candidates is all of them
 *                 ([HP] 1.), so for a query with at most topk visible compressed
 *                 rows the row lists exactly those rows and the call does not read
 *                 it; otherwise the row holds exactly topk rows, used as given
 *                 (each entry clamped into the buffer).  Rows that are not such
 *                 output give unspecified results; every read stays in bounds.
 * cmp_residual (optional, [B] int32 device, may be NULL): the per-segment tail
 * count len_b mod r of the operator schema (cmp_residual_kv, [HP] 2.; required
 * there when cmp_ratio != 1).  cu_seqlens_kv fixes the same quantity here, so the
 * value must equal len_b mod r; a query whose segment disagrees gets NaN in out
 * and lse, so a stale residual shows in the output instead of passing silently
 * (the page's control experiment finds the operator's output depends on it).
 * Errors: EINVAL for NULL q/ori_kv/out/cu_seqlens*, cmp_idx without cmp_kv,
 * topk < 1 with cmp_idx, an unknown cmp_idx_kind, B < 1, Tq < 0, Tc < 0, a window
 * side < 0 (or Tkv plus both sides >= 2^31), cmp_ratio < 1,
 * global_start + Tq > Tkv, softmax_scale not positive and finite; EUNSUPPORTED for
 * shapes other than (H, d) = (64, 512)
 * bf16 or H * d <= 8192 with d % 8 == 0, or topk > 2048.
 */
int csa_sparse_mla_fwd(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx,
                       int32_t topk, int32_t cmp_idx_kind, int32_t Tq, int32_t Tkv, int32_t Tc, int32_t H,
                       int32_t d, int32_t dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                       const int32_t* cu_seqlens_cmp, const int32_t* cmp_residual, int32_t B,
                       int32_t global_start, int32_t cmp_ratio, int32_t ori_win_left, int32_t ori_win_right,
                       const float* sinks, float softmax_scale, void* out, float* lse,
                       csa_stream_t stream);

/*
 * csa_sparse_mla_bwd - gradients of csa_sparse_mla_fwd ([HP] 4.
 * npu_sparse_flash_mla_grad: the operator's backward returns d_query, d_ori_kv,
 * d_cmp_kv, d_sinks and the window / compressed "softmax_l1_norm").
 *
 * Same key sets, softmax and sink as the forward, K = V.  With the forward's out and
 * lse and the output gradient dout, for each query i and head h:
 *   P[h,k] = exp(scale <q,kv_k> - lse),  dP[h,k] = <dout, kv_k>,  D = <dout, out>,
 *   dS = P (dP - D),  dq = scale sum_k dS kv_k,
 *   d_kv[row of k] += sum_h (scale dS q + P dout)   (window rows into d_ori_kv,
 *                                                    compressed rows into d_cmp_kv),
 *   d_sinks[h] = -sum_i exp(sinks[h] - lse) D.
 * ori_l1[i, k] (window slot k = stream row lo + k, the csa_build_indices win_idx
 * order) and cmp_l1[i, j] (the j-th attended compressed row: the j-th valid entry of
 * the cmp_idx row, or visible row q_cmp_lo + j in attend-all mode) hold P averaged
 * over the heads; unused slots are 0.  P and scale * dS enter the MFMA products as
 * bf16, all accumulation is float32.
 *   q, out, dout, dq [Tq, H, d] (call dtype), lse [Tq, H] float32 (the forward's),
 *   d_ori_kv [Tkv, d] and d_cmp_kv [Tc, d] float32 (overwritten; Tc = rows of
 *   cmp_kv), d_sinks [H] float32 (overwritten when sinks is given),
 *   ori_l1 [Tq, W] float32, cmp_l1 [Tq, cmp_slots] float32 (optional, overwritten),
 *   W = ori_win_left + ori_win_right + 1.
 * Precondition of the sparse mode: the valid entries of a cmp_idx row are distinct
 * rows visible to the query ([q_cmp_lo, q_cmp_lo + q_cmp_nvis)), as csa_indexer_topk
 * emits them; the row gradients of other entries are not formed.
 * max_seqlen_kv bounds the longest segment (it sizes the attend-all key list, the
 * selection map and the row-gradient work items).  workspace: device memory of at
 * least csa_sparse_mla_bwd_workspace_bytes() bytes (scale*dS and P of every
 * (query, key) pair as 256-byte rows, key rows, sink terms, the selection map),
 * owned by the caller; no memory is allocated.  d_ori_kv and d_cmp_kv take float
 * atomics from the work items that share a key tile, so their last bits vary from
 * run to run (csa_sparse_mla_bwd_deterministic below does not); dq, d_sinks and the
 * l1 outputs are deterministic.
 * Errors: as csa_sparse_mla_fwd, plus EINVAL for a missing out/lse/dout/dq/
 * workspace/d_ori_kv, cmp_kv without d_cmp_kv, sinks without d_sinks, cmp_l1 with
 * cmp_slots < 1, or a workspace smaller than required; EUNSUPPORTED for any shape
 * other than (H, d) = (64, 512) bf16.
 */
int64_t csa_sparse_mla_bwd_workspace_bytes(int32_t Tq, int32_t ori_win_left, int32_t ori_win_right,
                                           const void* cmp_kv, const int32_t* cmp_idx, int32_t topk,
                                           int32_t max_seqlen_kv, int32_t cmp_ratio);
int csa_sparse_mla_bwd(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx, int32_t topk,
                       int32_t Tq, int32_t Tkv, int32_t Tc, int32_t H, int32_t d, int32_t dtype,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, const int32_t* cu_seqlens_cmp,
                       int32_t B, int32_t global_start, int32_t cmp_ratio, int32_t ori_win_left,
                       int32_t ori_win_right, int32_t max_seqlen_kv, const float* sinks, float softmax_scale,
                       const void* out, const float* lse, const void* dout, void* dq, float* d_ori_kv,
                       float* d_cmp_kv, float* d_sinks, float* ori_l1, float* cmp_l1, int32_t cmp_slots,
                       void* workspace, int64_t workspace_bytes, csa_stream_t stream);

/*
 * csa_sparse_mla_bwd_deterministic - csa_sparse_mla_bwd with bit-reproducible row
 * gradients (the gradients of [HP] 4. npu_sparse_flash_mla_grad; the page's GPU
 * verification of the unfused path reports bit-identical reruns).
 *
 * Same arguments, results and errors as csa_sparse_mla_bwd.  Each row-gradient work
 * item (a key tile of up to 256 rows, 256 latent dims, swept by a chunk of up to 128
 * queries) writes its float32 tile to its own slot of the workspace instead of adding
 * it with atomics, and one more kernel sums, for every row of d_ori_kv and d_cmp_kv,
 * the tiles that hold it in ascending query-chunk order and stores the row.  Every
 * output is then identical from run to run; d_ori_kv / d_cmp_kv equal
 * csa_sparse_mla_bwd's up to float32 summation order.  workspace: at least
 * csa_sparse_mla_bwd_deterministic_workspace_bytes() bytes: csa_sparse_mla_bwd's
 * workspace plus the tiles, (ceil(Tq / 128) + B) chunks x 2 (n_w + n_c) items x 256 KiB
 * with n_w = min(127 + ori_win_left + ori_win_right, max_seqlen_kv - 1) / 256 + 1 and
 * n_c = ceil(floor(max_seqlen_kv / cmp_ratio) / 256) (0 without cmp_kv); -1 for
 * invalid sizes (B < 1 among them).
 */
int64_t csa_sparse_mla_bwd_deterministic_workspace_bytes(int32_t Tq, int32_t B, int32_t ori_win_left,
                                                         int32_t ori_win_right, const void* cmp_kv,
                                                         const int32_t* cmp_idx, int32_t topk,
                                                         int32_t max_seqlen_kv, int32_t cmp_ratio);
int csa_sparse_mla_bwd_deterministic(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx,
                                     int32_t topk, int32_t Tq, int32_t Tkv, int32_t Tc, int32_t H, int32_t d,
                                     int32_t dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                     const int32_t* cu_seqlens_cmp, int32_t B, int32_t global_start,
                                     int32_t cmp_ratio, int32_t ori_win_left, int32_t ori_win_right,
                                     int32_t max_seqlen_kv, const float* sinks, float softmax_scale, const void* out,
                                     const float* lse, const void* dout, void* dq, float* d_ori_kv, float* d_cmp_kv,
                                     float* d_sinks, float* ori_l1, float* cmp_l1, int32_t cmp_slots,
                                     void* workspace, int64_t workspace_bytes, csa_stream_t stream);

/*
 * csa_indexer_kl_grad - the lightning indexer's KL loss against the main attention and
 * its gradients ([HP] 3. npu_sparse_lightning_indexer_kl_loss_grad: inputs q, k, w,
 * the sparse indices and attn_softmax_l1_norm; [HP] 4.: that tensor is the main
 * attention's target distribution, i.e. the cmp_l1 output of csa_sparse_mla_bwd).
 *
 * For local query i with selected compressed rows c_j (the valid entries of
 * cmp_idx[i], in order) and targets p_j = attn_l1[i, j]:
 *   p^ = p / sum_j p_j,  u_hj = <q_I[i,h], k_I_cmp[c_j]>,  I_j = sum_h w[i,h] relu(u_hj),
 *   loss[i] = KL(p^ || softmax(I)),  G_j = loss_scale * (softmax_j(I) - p^_j),
 *   d_w[i,h] = sum_j G_j relu(u_hj),   d_q_I[i,h] = sum_j G_j w[i,h] [u_hj > 0] k_I_cmp[c_j],
 *   d_k_I_cmp[c_j] += sum_h G_j w[i,h] [u_hj > 0] q_I[i,h].
 * loss_scale carries the upstream gradient and the mean over the global token count
 * ([MS] 主要改动: in TND the loss divides by the global token count).  A query with
 * nothing selected or zero target mass contributes nothing (loss 0).  Scores are
 * float32 MFMA sums of the bf16 inputs; M = G w [u > 0] enters the d_q / d_k
 * products as bf16.
 *   q_I [Tq, H_I, d_I], w [Tq, H_I], k_I_cmp [Tc, d_I] (call dtype), cmp_idx [Tq, topk]
 *   int32 whose valid entries are distinct rows visible to the query (what
 *   csa_indexer_topk emits), attn_l1 [Tq, topk] float32 (slot j = the j-th valid
 *   entry), d_q_I [Tq, H_I, d_I] (call dtype), d_w [Tq, H_I] float32, d_k_I_cmp
 *   [Tc, d_I] float32 (overwritten), loss [Tq] float32 (NULL = not written: the
 *   unscaled KL of each query).
 * workspace: at least csa_indexer_kl_grad_workspace_bytes() bytes (the G of every
 * selected slot and a map of the visible rows), owned by the caller.  d_k_I_cmp takes
 * float atomics from the query chunks that share a row tile, so its last bits vary
 * between runs; the other outputs are deterministic.
 * Errors: EINVAL for NULL pointers, topk < 1, B < 1, Tq < 0, Tc < 0, cmp_ratio < 1,
 * global_start < 0, max_seqlen_kv < 0 or a workspace smaller than required;
 * EUNSUPPORTED for topk > 2048 or any shape other than (H_I, d_I) = (64, 128) bf16.
 */
int64_t csa_indexer_kl_grad_workspace_bytes(int32_t Tq, int32_t topk, int32_t max_seqlen_kv, int32_t cmp_ratio);
int csa_indexer_kl_grad(const void* q_I, const void* w, const void* k_I_cmp, const int32_t* cmp_idx,
                        const float* attn_l1, int32_t topk, int32_t Tq, int32_t Tc, int32_t H_I, int32_t d_I,
                        int32_t dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                        const int32_t* cu_seqlens_cmp, int32_t B, int32_t global_start, int32_t cmp_ratio,
                        int32_t max_seqlen_kv, float loss_scale, void* d_q_I, float* d_w, float* d_k_I_cmp,
                        float* loss, void* workspace, int64_t workspace_bytes, csa_stream_t stream);

/*
 * csa_indexer_kl_grad_noalloc - csa_indexer_kl_grad without a caller workspace and
 * without any device allocation, for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results and errors as csa_indexer_kl_grad, minus workspace and
 * workspace_bytes.  The workspace is a device array the library holds: 64 MiB
 * (CSA_KL_NOALLOC_SCRATCH_BYTES) on every GPU the call runs on, from the first call
 * on that GPU until the process ends.  A call needing more,
 * Tq * (4 topk + 2 floor(max_seqlen_kv / cmp_ratio)) bytes > 64 MiB, fails with
 * CSA_EINVAL before any launch.  All calls on one GPU share that array: calls that
 * overlap on one GPU (e.g. on two streams) race and give undefined results.
 */
#define CSA_KL_NOALLOC_SCRATCH_BYTES (64ll << 20)
int csa_indexer_kl_grad_noalloc(const void* q_I, const void* w, const void* k_I_cmp, const int32_t* cmp_idx,
                                const float* attn_l1, int32_t topk, int32_t Tq, int32_t Tc, int32_t H_I, int32_t d_I,
                                int32_t dtype, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                const int32_t* cu_seqlens_cmp, int32_t B, int32_t global_start, int32_t cmp_ratio,
                                int32_t max_seqlen_kv, float loss_scale, void* d_q_I, float* d_w, float* d_k_I_cmp,
                                float* loss, csa_stream_t stream);

/*
 * csa_validate_layout - synchronous debug check of a THD layout held in device
 * memory: cu_seqlens_kv starts at 0, is non-decreasing and ends at Tkv;
 * cu_seqlens_q equals clamp(cu_seqlens_kv - global_start, 0, Tq); and the longest
 * segment is at most max_seqlen_kv (pass -1 to skip that check).  With cmp_ratio
 * >= 1 it also checks the compressed layout a caller holds: cu_seqlens_cmp (if not
 * NULL) must be the prefix sums of floor(len_b / cmp_ratio) and cmp_residual (if
 * not NULL) must equal len_b mod cmp_ratio ([HP] 背景 1: the residual is the original
 * length mod cmp_ratio); pass cmp_ratio = 0 to skip both.  Copies the arrays to
 * the host (blocks on `stream`).  Returns CSA_OK or CSA_EINVAL with a message naming
 * the first violated condition.
 */
int csa_validate_layout(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t B,
                        int32_t Tq, int32_t Tkv, int32_t global_start, int32_t max_seqlen_kv,
                        int32_t cmp_ratio, const int32_t* cu_seqlens_cmp, const int32_t* cmp_residual,
                        csa_stream_t stream);

/*
 * csa_validate_topk_rows - synchronous check of the index rows the sparse-MLA
 * backward and the indexer KL gradient assume, and csa_sparse_mla_fwd's
 * CSA_IDX_TOPK kind declares ([HP] 1. npu_lightning_indexer: the top-k of each
 * query's visible candidates): every valid entry (>= 0) of cmp_idx[i, :] is a
 * compressed row visible to query i, i.e. in [cu_seqlens_cmp[b], cu_seqlens_cmp[b]
 * + min(floor((p + 1) / cmp_ratio), len_b / cmp_ratio, Tc - cu_seqlens_cmp[b])) for
 * its segment b and position p, and no entry repeats another of the same row.  One
 * GPU workgroup per query (an LDS bitmap of the visible rows); blocks on `stream`.
 * Returns CSA_OK, or CSA_EINVAL naming the first bad query and entry; CSA_EINVAL also
 * for invalid arguments and for a query with more than 32768 visible rows (not checked).
 * The first violation is gathered in an 8-byte device word the library holds per GPU:
 * checks that overlap on one GPU (two streams, or two host threads; also the debug
 * build's checks inside other calls) race on it and may report each other's result.
 */
int csa_validate_topk_rows(const int32_t* cmp_idx, int32_t topk, int32_t Tq, int32_t Tc,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, const int32_t* cu_seqlens_cmp,
                           int32_t B, int32_t global_start, int32_t cmp_ratio, csa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
