// Precondition check of index rows: every valid entry (>= 0) of a query's row must be a
// compressed row visible to that query (in [q_cmp_lo, q_cmp_lo + q_cmp_nvis), bounded by
// the Tc rows that exist), and no entry may repeat.  That is what csa_indexer_topk emits
// and what the sparse-MLA backward and the indexer KL gradient assume (page "【RFC】
// DeepSeek-V4 CSA/HCA ...", 1. npu_lightning_indexer: the top-k of the visible candidates).
#include <mutex>

#include "csa_common.h"
#include "csa_internal.h"

namespace csa {
namespace {

constexpr int kCheckThreads = 256;
constexpr int kMaxVisible = 32768;  // visible compressed rows per query the bitmap covers

// First violation over all queries: (query << 32) | (reason << 24) | entry, minimised.
// reason 1: outside the query's visible rows, 2: repeated, 3: more visible rows than
// the bitmap covers (the row is then not checked).
static __device__ __align__(16) unsigned long long g_first_bad;

__global__ void check_init_kernel(unsigned long long* first_bad) { *first_bad = ~0ull; }

__global__ __launch_bounds__(kCheckThreads) void check_rows_kernel(
    const int32_t* __restrict__ rows, int topk, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv,
    const int32_t* __restrict__ cu_cmp, int B, int global_start, int r, int Tc, unsigned long long* first_bad) {
  __shared__ uint32_t seen[kMaxVisible / 32];
  const int i = static_cast<int>(blockIdx.x);
  const int tid = threadIdx.x;
  const int b = segment_of(cu_q, B, i);
  const int s = cu_kv[b];
  const int lo = cu_cmp[b];
  const int p = global_start + i - s;
  const int nv = max(0, min(min((p + 1) / r, cu_cmp[b + 1] - lo), Tc - lo));
  const unsigned long long qkey = static_cast<unsigned long long>(i) << 32;
  if (nv > kMaxVisible) {
    if (tid == 0) atomicMin(first_bad, qkey | (3ull << 24));
    return;
  }
  for (int k = tid; k < (nv + 31) / 32; k += kCheckThreads) seen[k] = 0u;
  __syncthreads();
  const int32_t* row = rows + static_cast<long long>(i) * topk;
  for (int j = tid; j < topk; j += kCheckThreads) {
    const int c = row[j];
    if (c < 0) continue;  // a hole
    if (c < lo || c >= lo + nv) {
      atomicMin(first_bad, qkey | (1ull << 24) | static_cast<unsigned long long>(j));
      continue;
    }
    const int bit = c - lo;
    const uint32_t old = atomicOr(&seen[bit >> 5], 1u << (bit & 31));
    if (old & (1u << (bit & 31))) atomicMin(first_bad, qkey | (2ull << 24) | static_cast<unsigned long long>(j));
  }
}

std::once_flag g_once[64];
void* g_addr[64];
hipError_t g_err[64];

}  // namespace

hipError_t check_topk_rows(const int32_t* rows, int topk, int Tq, const int32_t* cu_q, const int32_t* cu_kv,
                           const int32_t* cu_cmp, int B, int global_start, int r, int Tc, hipStream_t s,
                           long long* bad_query, int* bad_entry, int* reason) {
  *bad_query = -1;
  *bad_entry = -1;
  *reason = 0;
  if (Tq <= 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  // the result slot's device address, looked up once per device with that device current
  std::call_once(g_once[dev], [&] { g_err[dev] = hipGetSymbolAddress(&g_addr[dev], HIP_SYMBOL(g_first_bad)); });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  auto* slot = static_cast<unsigned long long*>(g_addr[dev]);
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(1), 0, s, slot);
  hipLaunchKernelGGL(check_rows_kernel, dim3(static_cast<unsigned>(Tq)), dim3(kCheckThreads), 0, s, rows, topk, cu_q,
                     cu_kv, cu_cmp, B, global_start, r, Tc, slot);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  unsigned long long v = 0;
  if ((e = hipMemcpyAsync(&v, slot, sizeof(v), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  if (v != ~0ull) {
    *bad_query = static_cast<long long>(v >> 32);
    *reason = static_cast<int>((v >> 24) & 0xff);
    *bad_entry = static_cast<int>(v & 0xffffff);
  }
  return hipSuccess;
}

}  // namespace csa
