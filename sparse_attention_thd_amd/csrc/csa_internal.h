// Internal launcher declarations of libcsa (host side; argument checks happen in csa_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

// Let kernel `k` take `bytes` of dynamic LDS (beyond the default limit); the launchers
// return this call's error instead of launching when it fails.
inline hipError_t allow_dynamic_lds(const void* k, size_t bytes) {
  return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

hipError_t launch_build_indices(const int32_t* cu_q, const int32_t* cu_kv, int B, int Tq, int Tkv,
                                int global_start, int r, int wl, int wr, int32_t* q_seg, int32_t* q_pos,
                                int32_t* win_idx, int32_t* cu_cmp, int32_t* residual, int32_t* q_cmp_lo,
                                int32_t* q_cmp_nvis, int32_t* cmp_group, int Tc_cap, hipStream_t s);

hipError_t launch_compress(const void* x, int Tkv, int d, int dtype, const int32_t* cu_kv,
                           const int32_t* cu_cmp, int B, int r, void* x_cmp, int Tc_cap, hipStream_t s);

// Caller workspace of the indexer: one row of `cap` uint32 score keys per query.
size_t indexer_workspace_bytes(int Tq, int cap);
hipError_t launch_indexer_topk(const void* q_I, const void* w, const void* k_cmp, int Tq, int Tc, int H_I, int d_I,
                               int dtype, const int32_t* cu_q, const int32_t* cu_kv, const int32_t* cu_cmp,
                               const int32_t* residual, int B, int global_start, int r, int cap, int topk,
                               int32_t* idx, float* score, void* workspace, hipStream_t s);

// `topk_rows`: cmp_idx holds csa_indexer_topk's rows for this layout (CSA_IDX_TOPK).
hipError_t launch_sparse_mla(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx,
                             int topk, bool topk_rows, int Tq, int Tc, int H, int d, int dtype, const int32_t* cu_q,
                             const int32_t* cu_kv, const int32_t* cu_cmp, const int32_t* residual, int B,
                             int global_start, int r, int wl, int wr, const float* sinks, float scale, void* out,
                             float* lse, hipStream_t s);

hipError_t launch_sparse_mla_bwd(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx,
                                 int topk, int Tq, int Tkv, int Tc, const int32_t* cu_q, const int32_t* cu_kv,
                                 const int32_t* cu_cmp, int B, int global_start, int r, int wl, int wr,
                                 int max_seqlen_kv, const float* sinks, float scale, const void* out,
                                 const float* lse, const void* dout, void* dq, float* d_ori, float* d_cmp,
                                 float* d_sinks, float* ori_l1, float* cmp_l1, int cmp_slots, int key_cap,
                                 int nvis_cap, void* workspace, bool deterministic, hipStream_t s);

hipError_t launch_indexer_kl_grad(const void* q_I, const void* w, const void* k_cmp, const int32_t* cmp_idx,
                                  const float* attn_l1, int topk, int Tq, int Tc, const int32_t* cu_q,
                                  const int32_t* cu_kv, const int32_t* cu_cmp, int B, int global_start, int r,
                                  int max_seqlen_kv, float loss_scale, void* d_q, float* d_w, float* d_k, float* loss,
                                  int nvis_cap, void* workspace, hipStream_t s);
bool kl_shape_supported(int H_I, int d_I, int dtype);
size_t kl_workspace_bytes(int Tq, int topk, int nvis_cap);
// Library-held workspace of csa_indexer_kl_grad_noalloc: its device address on the
// current device (looked up once per device).
constexpr size_t kKlScratchBytes = size_t(64) << 20;
hipError_t kl_scratch(void** ptr);

hipError_t launch_compress_learned(const void* x, int Tkv, int D, const void* wkv, const void* wgate,
                                   const float* ape, int hd, int overlap, const int32_t* cu_kv,
                                   const int32_t* cu_cmp, int B, void* out, int Tc_cap, hipStream_t s);
bool learned_shape_supported(int D, int hd, int cmp_ratio, int overlap, int dtype);

// First violation of the index-row precondition (visible, not repeated): bad_query -1 if none;
// reason 1 not visible, 2 repeated, 3 too many visible rows to check.  Synchronises s.
hipError_t check_topk_rows(const int32_t* rows, int topk, int Tq, const int32_t* cu_q, const int32_t* cu_kv,
                           const int32_t* cu_cmp, int B, int global_start, int r, int Tc, hipStream_t s,
                           long long* bad_query, int* bad_entry, int* reason);

bool indexer_shape_supported(int H_I, int d_I, int dtype);
bool mla_shape_supported(int H, int d, int dtype);
bool mla_bwd_shape_supported(int H, int d, int dtype);
size_t mla_bwd_workspace_bytes(int Tq, int key_cap, int nvis_cap);
// Partial row-gradient tiles of the deterministic backward (an upper bound from the sizes).
size_t mla_bwd_partial_bytes(int Tq, int B, int wl, int wr, int Tkv, bool has_cmp, int max_seqlen_kv, int r);

}  // namespace csa
