// Segment layout of a THD pack: compressed prefix sums, per-query tables and
// segment-clamped window indices.  Integer work, bound by launch latency and a
// few MiB of coalesced int32 writes.
#include "csa_common.h"
#include "csa_internal.h"

namespace csa {
namespace {

constexpr int kThreads = 256;

// One workgroup: cu_cmp[b+1] = cu_cmp[b] + floor(len_b / r) and residual[b] = len_b mod r,
// scanned 256 segments at a time.
__global__ __launch_bounds__(kThreads) void segment_scan_kernel(const int32_t* __restrict__ cu_kv, int B, int r,
                                                               int32_t* __restrict__ cu_cmp,
                                                               int32_t* __restrict__ residual) {
  __shared__ int wave_sum[kThreads / 64];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { cu_cmp[0] = 0; carry_s = 0; }
  __syncthreads();
  for (int base = 0; base < B; base += kThreads) {
    const int b = base + tid;
    int n = 0;
    if (b < B) {
      const int len = cu_kv[b + 1] - cu_kv[b];
      n = len / r;
      residual[b] = len - n * r;
    }
    // inclusive wave scan
    int v = n;
    for (int off = 1; off < 64; off <<= 1) {
      int u = __shfl_up(v, off, 64);
      if (lane >= off) v += u;
    }
    if (lane == 63) wave_sum[wave] = v;
    __syncthreads();
    int before = carry_s;
    for (int k = 0; k < wave; ++k) before += wave_sum[k];
    if (b < B) cu_cmp[b + 1] = before + v;
    __syncthreads();
    if (tid == kThreads - 1) carry_s = before + v;
    __syncthreads();
  }
}

constexpr int kWinQueries = 16;  // queries per workgroup of the window-slot job (4 per wavefront)

// Segment of row x (largest b < B with cu[b] <= x, cu[0] <= x) for a whole wavefront:
// one coalesced load per 64 entries and a ballot count, result wave-uniform.
__device__ __forceinline__ int segment_of_wave(const int32_t* __restrict__ cu, int B, int x) {
  const int lane = threadIdx.x & 63;
  int count = 0;
  for (int base = 0; base < B; base += 64) count += __popcll(__ballot(base + lane < B && cu[base + lane] <= x));
  return __builtin_amdgcn_readfirstlane(count - 1);
}

// One 1-D grid, three jobs by block range: [0, n0) per-query tables (one thread per
// query); [n0, n0 + n1) window slots (one wavefront per query: the slots of a query are
// one contiguous row, written 64 at a time); [n0 + n1, ...) compressed group ids.
__global__ __launch_bounds__(kThreads) void layout_kernel(const int32_t* __restrict__ cu_q,
                                                          const int32_t* __restrict__ cu_kv,
                                                          const int32_t* __restrict__ cu_cmp, int B, int Tq,
                                                          int global_start, int r, int wl, int wr,
                                                          int32_t* __restrict__ q_seg, int32_t* __restrict__ q_pos,
                                                          int32_t* __restrict__ win_idx,
                                                          int32_t* __restrict__ q_cmp_lo,
                                                          int32_t* __restrict__ q_cmp_nvis,
                                                          int32_t* __restrict__ cmp_group, int Tc_cap, int n0,
                                                          int n1) {
  const int bx = static_cast<int>(blockIdx.x);
  const int W = wl + wr + 1;
  if (bx < n0) {
    const int i = bx * kThreads + static_cast<int>(threadIdx.x);
    if (i >= Tq) return;
    const int b = segment_of(cu_q, B, i);
    const int t = global_start + i;
    const int p = t - cu_kv[b];
    if (q_seg) q_seg[i] = b;
    if (q_pos) q_pos[i] = p;
    if (q_cmp_lo) q_cmp_lo[i] = cu_cmp[b];
    if (q_cmp_nvis) q_cmp_nvis[i] = (p + 1) / r;
  } else if (bx < n0 + n1) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
#pragma unroll
    for (int j = 0; j < kWinQueries / (kThreads / 64); ++j) {
      const int i = (bx - n0) * kWinQueries + wave * (kWinQueries / (kThreads / 64)) + j;
      if (i >= Tq) break;
      const int b = segment_of_wave(cu_q, B, i);
      const int t = global_start + i;
      const int lo = max(cu_kv[b], t - wl);
      const int hi = min(cu_kv[b + 1] - 1, t + wr);
      int32_t* row = win_idx + static_cast<long long>(i) * W;
      for (int k = lane; k < W; k += 64) row[k] = (lo + k <= hi) ? lo + k : -1;
    }
  } else {
    const int c = (bx - n0 - n1) * kThreads + static_cast<int>(threadIdx.x);
    if (c >= Tc_cap) return;
    if (c >= cu_cmp[B]) return;  // rows past the true count stay untouched
    const int b = segment_of(cu_cmp, B, c);
    cmp_group[c] = c - cu_cmp[b];
  }
}

}  // namespace

hipError_t launch_build_indices(const int32_t* cu_q, const int32_t* cu_kv, int B, int Tq, int Tkv,
                                int global_start, int r, int wl, int wr, int32_t* q_seg, int32_t* q_pos,
                                int32_t* win_idx, int32_t* cu_cmp, int32_t* residual, int32_t* q_cmp_lo,
                                int32_t* q_cmp_nvis, int32_t* cmp_group, int Tc_cap, hipStream_t s) {
  (void)Tkv;
  hipLaunchKernelGGL(segment_scan_kernel, dim3(1), dim3(kThreads), 0, s, cu_kv, B, r, cu_cmp, residual);
  const bool tables = q_seg || q_pos || q_cmp_lo || q_cmp_nvis;
  const long long n0 = tables ? (static_cast<long long>(Tq) + kThreads - 1) / kThreads : 0;
  const long long n1 = win_idx ? (static_cast<long long>(Tq) + kWinQueries - 1) / kWinQueries : 0;
  const long long n2 = cmp_group ? (static_cast<long long>(Tc_cap) + kThreads - 1) / kThreads : 0;
  const long long nb = n0 + n1 + n2;
  if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (nb > 0)
    hipLaunchKernelGGL(layout_kernel, dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0, s, cu_q, cu_kv, cu_cmp, B,
                       Tq, global_start, r, wl, wr, q_seg, q_pos, win_idx, q_cmp_lo, q_cmp_nvis, cmp_group,
                       n2 ? Tc_cap : 0, static_cast<int>(n0), static_cast<int>(n1));
  return hipGetLastError();
}

}  // namespace csa
