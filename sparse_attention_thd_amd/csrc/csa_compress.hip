// Segment-local mean pooling of cmp_ratio consecutive rows (HBM streaming).
// One wavefront per compressed row; each lane owns 16-byte chunks of the row and
// sums the r source rows in float64 in ascending order, then rounds once.
#include "csa_common.h"
#include "csa_internal.h"

namespace csa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;

template <typename T>
struct Chunk;
template <>
struct Chunk<uint16_t> {  // bf16: 8 elements per 16 bytes
  static constexpr int N = 8;
  __device__ static void add(double* acc, const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] += static_cast<double>(__uint_as_float(w[k] << 16));
      acc[2 * k + 1] += static_cast<double>(__uint_as_float(w[k] & 0xffff0000u));
    }
  }
  // The mean is the correctly rounded float64 quotient sum / r, then one rounding to
  // the storage type (a product with 1 / r would round twice for r not a power of two).
  __device__ static uint4 finish(const double* acc, double r) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = f64_to_bf16_bits(acc[2 * k] / r);
      const uint32_t hi = f64_to_bf16_bits(acc[2 * k + 1] / r);
      w[k] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Chunk<float> {  // f32: 4 elements per 16 bytes
  static constexpr int N = 4;
  __device__ static void add(double* acc, const uint4& v) {
    acc[0] += static_cast<double>(__uint_as_float(v.x));
    acc[1] += static_cast<double>(__uint_as_float(v.y));
    acc[2] += static_cast<double>(__uint_as_float(v.z));
    acc[3] += static_cast<double>(__uint_as_float(v.w));
  }
  __device__ static uint4 finish(const double* acc, double r) {
    return make_uint4(__float_as_uint(static_cast<float>(acc[0] / r)),
                      __float_as_uint(static_cast<float>(acc[1] / r)),
                      __float_as_uint(static_cast<float>(acc[2] / r)),
                      __float_as_uint(static_cast<float>(acc[3] / r)));
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void compress_kernel(const T* __restrict__ x, int d,
                                                            const int32_t* __restrict__ cu_kv,
                                                            const int32_t* __restrict__ cu_cmp, int B, int r,
                                                            T* __restrict__ x_cmp, int Tc_cap) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (c >= Tc_cap || c >= cu_cmp[B]) return;
  const int b = segment_of(cu_cmp, B, c);
  const long long first = static_cast<long long>(cu_kv[b]) + static_cast<long long>(c - cu_cmp[b]) * r;
  const int nchunk = d / Chunk<T>::N;
  const double rd = static_cast<double>(r);
  for (int ch = lane; ch < nchunk; ch += 64) {
    double acc[Chunk<T>::N];
#pragma unroll
    for (int k = 0; k < Chunk<T>::N; ++k) acc[k] = 0.0;
    const uint4* src = reinterpret_cast<const uint4*>(x + first * d) + ch;
    const long long stride = nchunk;  // uint4 per row
    int m = 0;
    for (; m + 4 <= r; m += 4) {
      const uint4 v0 = src[(m + 0) * stride];
      const uint4 v1 = src[(m + 1) * stride];
      const uint4 v2 = src[(m + 2) * stride];
      const uint4 v3 = src[(m + 3) * stride];
      Chunk<T>::add(acc, v0);
      Chunk<T>::add(acc, v1);
      Chunk<T>::add(acc, v2);
      Chunk<T>::add(acc, v3);
    }
    for (; m < r; ++m) Chunk<T>::add(acc, src[m * stride]);
    reinterpret_cast<uint4*>(x_cmp + static_cast<long long>(c) * d)[ch] = Chunk<T>::finish(acc, rd);
  }
}

}  // namespace

hipError_t launch_compress(const void* x, int Tkv, int d, int dtype, const int32_t* cu_kv,
                           const int32_t* cu_cmp, int B, int r, void* x_cmp, int Tc_cap, hipStream_t s) {
  (void)Tkv;
  if (Tc_cap <= 0) return hipSuccess;
  const dim3 grid((Tc_cap + kRowsPerBlock - 1) / kRowsPerBlock);
  if (dtype == 1) {
    hipLaunchKernelGGL(compress_kernel<uint16_t>, grid, dim3(kThreads), 0, s, static_cast<const uint16_t*>(x), d,
                       cu_kv, cu_cmp, B, r, static_cast<uint16_t*>(x_cmp), Tc_cap);
  } else {
    hipLaunchKernelGGL(compress_kernel<float>, grid, dim3(kThreads), 0, s, static_cast<const float*>(x), d, cu_kv,
                       cu_cmp, B, r, static_cast<float*>(x_cmp), Tc_cap);
  }
  return hipGetLastError();
}

}  // namespace csa
