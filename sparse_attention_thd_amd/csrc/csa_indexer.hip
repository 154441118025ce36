// Lightning indexer + per-query top-k over the query's own segment.
//
// One workgroup (4 wavefronts) per query.  Queries with no more candidates than
// top-k only write the ascending candidate list.  Otherwise every candidate is
// scored into LDS as an order-preserving uint32 key, a 4-pass 8-bit radix select
// finds the k-th largest key, and an ordered block scan emits the kept rows in
// ascending order (exact ties go to the lower row).
//
// Scoring paths:
//   * (H_I, d_I) = (64, 128) bf16: v_mfma_f32_16x16x32_bf16 with the query's 64
//     heads as M (register-resident A operand), 16 candidates as N (B operand
//     loaded straight from global/L2), ReLU and head weighting on the fp32 C
//     fragments, then a 4-lane-group reduction.
//   * small shapes (H_I * d_I <= 8192, either dtype): scalar fp32 per candidate.
#include "csa_common.h"
#include "csa_internal.h"

namespace csa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

struct SelectShared {
  uint32_t hist[256];
  uint32_t wsum[kWaves];
  uint32_t digit;
  uint32_t kk;
};

// Exclusive count of `f` over the block in thread order; `total` gets the block count.
__device__ __forceinline__ uint32_t block_count_excl(bool f, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(f);
  const uint32_t in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(m);
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    const uint32_t v = wsum[k];
    off += (k < wave) ? v : 0u;
    tot += v;
  }
  __syncthreads();
  total = tot;
  return off + in_wave;
}

// Inclusive sum over the block in thread order.
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) add += (k < wave) ? wsum[k] : 0u;
  __syncthreads();
  return v + add;
}

// Select the `topk` largest of keys[0:nv] (nv > topk) and write them ascending.
__device__ void select_and_emit(const uint32_t* keys, int nv, int topk, int lo, int32_t* __restrict__ out_idx,
                                float* __restrict__ out_sc, SelectShared& sh) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0, kk = static_cast<uint32_t>(topk);
  for (int shift = 24; shift >= 0; shift -= 8) {
    sh.hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < nv; j += kThreads) {
      const uint32_t key = keys[j];
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t c = sh.hist[255 - tid];  // digits in descending order
    const uint32_t incl = block_scan_incl(c, sh.wsum);
    const uint32_t excl = incl - c;
    if (excl < kk && incl >= kk) {
      sh.digit = static_cast<uint32_t>(255 - tid);
      sh.kk = kk - excl;
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    pmask |= 0xffu << shift;
    kk = sh.kk;
    __syncthreads();
  }
  const uint32_t T = prefix;  // the topk-th largest key; kk of its copies are kept
  uint32_t base_sel = 0, base_tie = 0;
  for (int j0 = 0; j0 < nv; j0 += kThreads) {
    const int j = j0 + tid;
    const uint32_t key = (j < nv) ? keys[j] : 0u;
    const bool gt = (j < nv) && key > T;
    const bool eq = (j < nv) && key == T;
    uint32_t eq_total, take_total;
    const uint32_t eq_rank = block_count_excl(eq, sh.wsum, eq_total);
    const bool take = gt || (eq && base_tie + eq_rank < kk);
    const uint32_t pos = base_sel + block_count_excl(take, sh.wsum, take_total);
    if (take && pos < static_cast<uint32_t>(topk)) {
      out_idx[pos] = lo + j;
      if (out_sc) out_sc[pos] = order_key_to_float(key);
    }
    base_sel += take_total;
    base_tie += eq_total;
  }
  for (int k = static_cast<int>(base_sel) + tid; k < topk; k += kThreads) {
    out_idx[k] = -1;
    if (out_sc) out_sc[k] = -__builtin_huge_valf();
  }
}

__device__ __forceinline__ float load_elem(const float* p, long long k) { return p[k]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, long long k) { return bf16_bits_to_f32(p[k]); }

// Scalar scoring for small shapes: q_I row and weights staged in LDS as fp32.
template <typename T>
__device__ void score_generic(const T* __restrict__ q_I, const T* __restrict__ w, const T* __restrict__ k_cmp,
                              int i, int H_I, int d_I, int lo, int nv, uint32_t* keys, float* qs) {
  const int tid = threadIdx.x;
  const int hd = H_I * d_I;
  float* ws = qs + hd;
  for (int e = tid; e < hd; e += kThreads) qs[e] = load_elem(q_I, static_cast<long long>(i) * hd + e);
  for (int h = tid; h < H_I; h += kThreads) ws[h] = load_elem(w, static_cast<long long>(i) * H_I + h);
  __syncthreads();
  for (int j = tid; j < nv; j += kThreads) {
    const long long kr = static_cast<long long>(lo + j) * d_I;
    float s = 0.f;
    for (int h = 0; h < H_I; ++h) {
      float dot = 0.f;
      for (int e = 0; e < d_I; ++e) dot += qs[h * d_I + e] * load_elem(k_cmp, kr + e);
      s += ws[h] * fmaxf(dot, 0.f);
    }
    keys[j] = float_order_key(s);
  }
}

// MFMA scoring, 64 indexer heads x 128 dims, bf16.
__device__ void score_mfma_64x128(const uint16_t* __restrict__ q_I, const uint16_t* __restrict__ w,
                                  const uint16_t* __restrict__ k_cmp, int i, int lo, int nv, uint32_t* keys) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  // A operand: q_I[i, 16*mb + n, 32*ks + 8*g + 0..7]
  bf16x8 qa[4][4];
  const uint16_t* qrow = q_I + static_cast<long long>(i) * 64 * 128;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qa[mb][ks] = *reinterpret_cast<const bf16x8*>(qrow + (16 * mb + n) * 128 + 32 * ks + 8 * g);
  // head weights for the C rows this lane holds: heads 16*mb + 4*g + j
  float wv[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) wv[mb][j] = bf16_bits_to_f32(w[static_cast<long long>(i) * 64 + 16 * mb + 4 * g + j]);
  const int nblk = (nv + 15) >> 4;
  for (int jb = wave; jb < nblk; jb += kWaves) {
    const int c = 16 * jb + n;  // candidate of this lane's B column
    bf16x8 kb[4];
    if (c < nv) {
      const uint16_t* krow = k_cmp + static_cast<long long>(lo + c) * 128;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[ks] = *reinterpret_cast<const bf16x8*>(krow + 32 * ks + 8 * g);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[ks] = bf16x8{};
    }
    float s = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mb][ks], kb[ks], acc, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) s += wv[mb][j] * fmaxf(acc[j], 0.f);
    }
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    if (g == 0 && c < nv) keys[c] = float_order_key(s);
  }
}

// MFMA scoring of two queries of one segment (same candidate rows) in one pass: every
// 16-candidate block of keys is loaded once and multiplied by both queries' q (128
// register rows), which halves the key bytes per MFMA of the vector-memory path.
__device__ void score_mfma_64x128_pair(const uint16_t* __restrict__ q_I, const uint16_t* __restrict__ w,
                                       const uint16_t* __restrict__ k_cmp, int i0, int lo, int nv0, int nv1,
                                       uint32_t* keys0, uint32_t* keys1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  bf16x8 qa[2][4][4];
  float wv[2][4][4];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint16_t* qrow = q_I + static_cast<long long>(i0 + e) * 64 * 128;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qa[e][mb][ks] = *reinterpret_cast<const bf16x8*>(qrow + (16 * mb + n) * 128 + 32 * ks + 8 * g);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wv[e][mb][j] = bf16_bits_to_f32(w[static_cast<long long>(i0 + e) * 64 + 16 * mb + 4 * g + j]);
  }
  const int nvm = max(nv0, nv1);
  const int nblk = (nvm + 15) >> 4;
  for (int jb = wave; jb < nblk; jb += kWaves) {
    const int c = 16 * jb + n;
    bf16x8 kb[4];
    if (c < nvm) {
      const uint16_t* krow = k_cmp + static_cast<long long>(lo + c) * 128;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[ks] = *reinterpret_cast<const bf16x8*>(krow + 32 * ks + 8 * g);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[ks] = bf16x8{};
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float sc = 0.f;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[e][mb][ks], kb[ks], acc, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) sc += wv[e][mb][j] * fmaxf(acc[j], 0.f);
      }
      sc += __shfl_xor(sc, 16, 64);
      sc += __shfl_xor(sc, 32, 64);
      if (g == 0 && c < (e ? nv1 : nv0)) (e ? keys1 : keys0)[c] = float_order_key(sc);
    }
  }
}

// Candidate range of local query i: rows [lo, lo + nv) of its segment b that are
// causally complete, exist in the k_cmp buffer (Tc rows) and fit the score storage.
// With a caller-held residual that disagrees with the segment length, nv = -1 (the
// query's row is then written as all -1).
__device__ __forceinline__ void candidate_range(int i, const int32_t* __restrict__ cu_q,
                                                const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp,
                                                const int32_t* __restrict__ residual, int B, int global_start, int r,
                                                int cap, int Tc, int& lo, int& nv) {
  const int b = segment_of(cu_q, B, i);
  const int s = cu_kv[b];
  const int p = global_start + i - s;
  lo = cu_cmp[b];
  int v = (p + 1) / r;
  v = min(v, cu_cmp[b + 1] - lo);
  v = min(v, Tc - lo);
  nv = max(0, min(v, cap));
  if (residual != nullptr && residual[b] != (cu_kv[b + 1] - s) % r) nv = -1;
}

// The row of a query whose segment's residual disagrees: no selection, NaN scores.
__device__ __forceinline__ void write_poisoned_row(int32_t* __restrict__ out_idx, float* __restrict__ out_sc,
                                                   int topk) {
  for (int k = threadIdx.x; k < topk; k += kThreads) {
    out_idx[k] = -1;
    if (out_sc) out_sc[k] = __builtin_nanf("");
  }
}

// (H_I, d_I) = (64, 128) bf16, two queries per workgroup: queries 2 x and 2 x + 1.
// A query with no more candidates than top-k only writes its ascending list.  Two
// selecting queries of one segment are scored in one pass (above); otherwise each is
// scored alone.  The selections then run one after the other.
__global__ __launch_bounds__(kThreads) void indexer_topk_pair_kernel(
    const uint16_t* __restrict__ q_I, const uint16_t* __restrict__ w, const uint16_t* __restrict__ k_cmp,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp,
    const int32_t* __restrict__ residual, int B, int global_start, int r, int cap, int Tc, int topk, int Tq,
    int32_t* __restrict__ idx, float* __restrict__ score) {
  extern __shared__ uint32_t dyn[];  // two key arrays of cap entries
  __shared__ SelectShared sh;
  const int i0 = 2 * static_cast<int>(blockIdx.x);
  const int tid = threadIdx.x;
  const int nq = min(2, Tq - i0);
  int lo[2] = {0, 0}, nv[2] = {0, 0};
  bool heavy[2] = {false, false};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    if (e >= nq) break;
    const int i = i0 + e;
    candidate_range(i, cu_q, cu_kv, cu_cmp, residual, B, global_start, r, cap, Tc, lo[e], nv[e]);
    if (nv[e] < 0) {
      write_poisoned_row(idx + static_cast<long long>(i) * topk, score ? score + static_cast<long long>(i) * topk : nullptr,
                         topk);
      nv[e] = 0;
      continue;
    }
    heavy[e] = !(nv[e] <= topk && score == nullptr);
    if (!heavy[e]) {
      int32_t* out_idx = idx + static_cast<long long>(i) * topk;
      for (int k = tid; k < topk; k += kThreads) out_idx[k] = (k < nv[e]) ? lo[e] + k : -1;
    }
  }
  if (!heavy[0] && !heavy[1]) return;
  uint32_t* keys[2] = {dyn, dyn + cap};
  if (heavy[0] && heavy[1] && lo[0] == lo[1]) {
    score_mfma_64x128_pair(q_I, w, k_cmp, i0, lo[0], nv[0], nv[1], keys[0], keys[1]);
  } else {
#pragma unroll
    for (int e = 0; e < 2; ++e)
      if (heavy[e]) score_mfma_64x128(q_I, w, k_cmp, i0 + e, lo[e], nv[e], keys[e]);
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    if (!heavy[e]) continue;
    const int i = i0 + e;
    int32_t* out_idx = idx + static_cast<long long>(i) * topk;
    float* out_sc = score ? score + static_cast<long long>(i) * topk : nullptr;
    if (nv[e] <= topk) {
      for (int k = tid; k < topk; k += kThreads) {
        out_idx[k] = (k < nv[e]) ? lo[e] + k : -1;
        out_sc[k] = (k < nv[e]) ? order_key_to_float(keys[e][k]) : -__builtin_huge_valf();
      }
    } else {
      select_and_emit(keys[e], nv[e], topk, lo[e], out_idx, out_sc, sh);
    }
    __syncthreads();  // the selection state is reused by the second query
  }
}

template <int PATH, typename T>
__global__ __launch_bounds__(kThreads) void indexer_topk_kernel(const T* __restrict__ q_I, const T* __restrict__ w,
                                                                const T* __restrict__ k_cmp, int H_I, int d_I,
                                                                const int32_t* __restrict__ cu_q,
                                                                const int32_t* __restrict__ cu_kv,
                                                                const int32_t* __restrict__ cu_cmp,
                                                                const int32_t* __restrict__ residual, int B,
                                                                int global_start, int r, int cap, int Tc, int topk,
                                                                int32_t* __restrict__ idx, float* __restrict__ score) {
  extern __shared__ uint32_t dyn[];
  __shared__ SelectShared sh;
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  int lo, nv;
  candidate_range(i, cu_q, cu_kv, cu_cmp, residual, B, global_start, r, cap, Tc, lo, nv);
  int32_t* out_idx = idx + static_cast<long long>(i) * topk;
  float* out_sc = score ? score + static_cast<long long>(i) * topk : nullptr;
  if (nv < 0) {
    write_poisoned_row(out_idx, out_sc, topk);
    return;
  }
  if (nv <= topk && out_sc == nullptr) {
    for (int k = tid; k < topk; k += kThreads) out_idx[k] = (k < nv) ? lo + k : -1;
    return;
  }
  uint32_t* keys = dyn;
  if constexpr (PATH == 1) {
    score_mfma_64x128(q_I, w, k_cmp, i, lo, nv, keys);
  } else {
    score_generic<T>(q_I, w, k_cmp, i, H_I, d_I, lo, nv, keys, reinterpret_cast<float*>(dyn + cap));
  }
  __syncthreads();
  if (nv <= topk) {
    for (int k = tid; k < topk; k += kThreads) {
      out_idx[k] = (k < nv) ? lo + k : -1;
      out_sc[k] = (k < nv) ? order_key_to_float(keys[k]) : -__builtin_huge_valf();
    }
    return;
  }
  select_and_emit(keys, nv, topk, lo, out_idx, out_sc, sh);
}

}  // namespace

bool indexer_shape_supported(int H_I, int d_I, int dtype) {
  if (dtype == 1 && H_I == 64 && d_I == 128) return true;
  return H_I * d_I <= 8192 && d_I % 8 == 0;
}

hipError_t launch_indexer_topk(const void* q_I, const void* w, const void* k_cmp, int Tq, int Tc, int H_I, int d_I,
                               int dtype, const int32_t* cu_q, const int32_t* cu_kv, const int32_t* cu_cmp,
                               const int32_t* residual, int B, int global_start, int r, int cap, int topk,
                               int32_t* idx, float* score, hipStream_t s) {
  if (Tq <= 0) return hipSuccess;
  const bool mfma = (dtype == 1 && H_I == 64 && d_I == 128);
  size_t lds = static_cast<size_t>(cap) * 4;
  if (!mfma) lds += static_cast<size_t>(H_I) * d_I * 4 + static_cast<size_t>(H_I) * 4;
  const dim3 grid(Tq), block(kThreads);
  // Two queries per workgroup for long candidate lists, where halving the key bytes per
  // MFMA pays for the lower occupancy and the back-to-back selections (measured: the
  // 22999-token CP share 2.63 -> 2.31 ms; with lists of about 1000 candidates, as in the
  // 16k pack, one query per workgroup is faster), and only while the two key arrays
  // leave room for two workgroups per CU.
  const bool pair = cap >= 2048 && 2 * static_cast<size_t>(cap) * 4 <= 64 * 1024;
  if (mfma && !pair) {
    auto k = indexer_topk_kernel<1, uint16_t>;
    if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess)
      return e;
    hipLaunchKernelGGL(k, grid, block, lds, s, static_cast<const uint16_t*>(q_I), static_cast<const uint16_t*>(w),
                       static_cast<const uint16_t*>(k_cmp), H_I, d_I, cu_q, cu_kv, cu_cmp, residual, B, global_start, r,
                       cap, Tc, topk, idx, score);
  } else if (mfma) {
    auto k = indexer_topk_pair_kernel;
    const size_t lds2 = 2 * static_cast<size_t>(cap) * 4;
    if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(k), lds2); e != hipSuccess)
      return e;
    hipLaunchKernelGGL(k, dim3((Tq + 1) / 2), block, lds2, s, static_cast<const uint16_t*>(q_I),
                       static_cast<const uint16_t*>(w), static_cast<const uint16_t*>(k_cmp), cu_q, cu_kv, cu_cmp, residual, B,
                       global_start, r, cap, Tc, topk, Tq, idx, score);
  } else if (dtype == 1) {
    auto k = indexer_topk_kernel<0, uint16_t>;
    if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess)
      return e;
    hipLaunchKernelGGL(k, grid, block, lds, s, static_cast<const uint16_t*>(q_I), static_cast<const uint16_t*>(w),
                       static_cast<const uint16_t*>(k_cmp), H_I, d_I, cu_q, cu_kv, cu_cmp, residual, B, global_start, r,
                       cap, Tc, topk, idx, score);
  } else {
    auto k = indexer_topk_kernel<0, float>;
    if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess)
      return e;
    hipLaunchKernelGGL(k, grid, block, lds, s, static_cast<const float*>(q_I), static_cast<const float*>(w),
                       static_cast<const float*>(k_cmp), H_I, d_I, cu_q, cu_kv, cu_cmp, residual, B, global_start, r, cap,
                       Tc, topk, idx, score);
  }
  return hipGetLastError();
}

}  // namespace csa
