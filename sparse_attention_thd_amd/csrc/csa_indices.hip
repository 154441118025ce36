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

// blockIdx.y == 0: per-query tables; 1: window slots (one thread per slot); 2: compressed group ids.
__global__ __launch_bounds__(kThreads) void layout_kernel(const int32_t* __restrict__ cu_q,
                                                          const int32_t* __restrict__ cu_kv,
                                                          const int32_t* __restrict__ cu_cmp, int B, int Tq,
                                                          int global_start, int r, int wl, int wr,
                                                          int32_t* __restrict__ q_seg, int32_t* __restrict__ q_pos,
                                                          int32_t* __restrict__ win_idx,
                                                          int32_t* __restrict__ q_cmp_lo,
                                                          int32_t* __restrict__ q_cmp_nvis,
                                                          int32_t* __restrict__ cmp_group, int Tc_cap) {
  const long long e = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  const int W = wl + wr + 1;
  if (blockIdx.y == 0) {
    if (e >= Tq || !(q_seg || q_pos || q_cmp_lo || q_cmp_nvis)) return;
    const int i = static_cast<int>(e);
    const int b = segment_of(cu_q, B, i);
    const int t = global_start + i;
    const int p = t - cu_kv[b];
    if (q_seg) q_seg[i] = b;
    if (q_pos) q_pos[i] = p;
    if (q_cmp_lo) q_cmp_lo[i] = cu_cmp[b];
    if (q_cmp_nvis) q_cmp_nvis[i] = (p + 1) / r;
  } else if (blockIdx.y == 1) {
    if (win_idx == nullptr || e >= static_cast<long long>(Tq) * W) return;
    const int i = static_cast<int>(e / W);
    const int k = static_cast<int>(e - static_cast<long long>(i) * W);
    const int b = segment_of(cu_q, B, i);
    const int t = global_start + i;
    const int lo = max(cu_kv[b], t - wl);
    const int hi = min(cu_kv[b + 1] - 1, t + wr);
    win_idx[e] = (lo + k <= hi) ? lo + k : -1;
  } else {
    if (cmp_group == nullptr || e >= Tc_cap) return;
    const int c = static_cast<int>(e);
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
  const long long W = static_cast<long long>(wl) + wr + 1;
  const long long n0 = (q_seg || q_pos || q_cmp_lo || q_cmp_nvis) ? Tq : 0;
  const long long n1 = win_idx ? Tq * W : 0;
  const long long n2 = cmp_group ? Tc_cap : 0;
  const long long nmax = n0 > n1 ? (n0 > n2 ? n0 : n2) : (n1 > n2 ? n1 : n2);
  if (nmax > 0) {
    const unsigned gx = static_cast<unsigned>((nmax + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(layout_kernel, dim3(gx, 3), dim3(kThreads), 0, s, cu_q, cu_kv, cu_cmp, B, Tq,
                       global_start, r, wl, wr, n0 ? q_seg : nullptr, n0 ? q_pos : nullptr,
                       n1 ? win_idx : nullptr, n0 ? q_cmp_lo : nullptr, n0 ? q_cmp_nvis : nullptr,
                       n2 ? cmp_group : nullptr, n2 ? Tc_cap : 0);
  }
  return hipGetLastError();
}

}  // namespace csa
