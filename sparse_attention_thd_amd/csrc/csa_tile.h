// MFMA tile machinery shared by the sparse-MLA forward and backward kernels of libcsa:
// one workgroup of four wavefronts per query, keys streamed through LDS in padded
// 32-row tiles with global_load_lds_dwordx4, bf16 fragments for
// v_mfma_f32_16x16x32_bf16 (not part of the ABI).
#pragma once

#include "csa_common.h"

namespace csa {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kMaxTopk = 2048;

struct QueryKeys {
  int nwin;      // window rows lo .. lo + nwin - 1
  int lo;
  int ncmp;      // compressed rows
  int cmp_base;  // first visible row (attend-all mode)
};

// Workgroup barrier that only orders LDS traffic: it waits for this wavefront's
// LDS operations but, unlike __syncthreads(), leaves global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt == 0
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Exclusive count of `f` over the block in thread order (block-uniform call).
__device__ __forceinline__ uint32_t count_excl(bool f, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(f);
  const uint32_t in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(m);
  lds_barrier();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    const uint32_t v = wsum[k];
    off += (k < wave) ? v : 0u;
    tot += v;
  }
  lds_barrier();
  total = tot;
  return off + in_wave;
}

// Compact the valid entries of a cmp_idx row (in their given order) into crow;
// `vals` holds this thread's entries j = threadIdx.x + kThreads * c.  Returns the count.
template <int NC>
__device__ int compact_rows(const int (&vals)[NC], int topk, int Tc, int32_t* crow, uint32_t* wsum) {
  uint32_t base = 0;
#pragma unroll
  for (int ch = 0; ch < NC; ++ch) {
    if (ch * kThreads >= topk) break;
    const int c = vals[ch];
    const bool ok = c >= 0 && c < Tc;  // entries outside the compressed rows are dropped
    uint32_t tot;
    const uint32_t pos = base + count_excl(ok, wsum, tot);
    if (ok) crow[pos] = c;
    base += tot;
  }
  lds_barrier();
  return static_cast<int>(base);
}

// ----------------------------------------------------------------------------- tiles

constexpr int kNT = 32;                      // keys per tile
constexpr int kRowBytes = 1024;              // one latent row: 512 bf16
constexpr int kRowStride = kRowBytes + 16;   // padded tile row, see kpi()
constexpr int kTileBytes = kNT * kRowStride; // 32.5 KiB, two buffers in flight

// Tile rows are padded to 1040 bytes, so row r starts 4 banks (of 64 x 4 bytes) after
// row r - 1, and every fragment read is a per-lane base plus an immediate offset.
// The 16 K rows of an S^T MFMA are taken in the order kpi(0..15) = 0, 2, .., 14, 1,
// 3, .., 15 (accumulator row k holds key kpi(k)).  Then a b64 K read (16 rows x 16
// bytes per half-wavefront) and a transpose V read (rows kpi(0..7) or kpi(8..15),
// 32 bytes each, per half-wavefront) both touch each bank once.
__device__ __forceinline__ int kpi(int k) { return ((k & 7) << 1) | (k >> 3); }

// Output staging (1 KiB rows): 16-byte chunk q of row `row` lives at chunk q ^ swz(row).
__device__ __forceinline__ int swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define CSA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// One 1 KiB row (64 lanes x 16 bytes) from global memory straight into LDS at byte
// offset `lds_off` (wave-uniform).  Issued as inline asm so the compiler does not
// treat the in-flight copy as a pending LDS write (it would drain the vector memory
// counter before every LDS read); the caller waits on it with s_waitcnt vmcnt.
__device__ __forceinline__ void row_to_lds(const void* row_base, uint32_t lane_off, uint32_t lds_off) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_off), "v"(lane_off), "s"(row_base)
      : "memory", "m0");
}

// Staged 256-byte rows (16 chunks of 16 B, e.g. 128 bf16 indexer keys): chunk c of row r
// lives at chunk c ^ (r % 16), so 16 consecutive rows read at one logical chunk hit 16
// distinct bank groups.
__device__ __forceinline__ int kchunk(int r, int c) { return c ^ (r & 15); }

// 16 bytes per lane from a per-lane global address into LDS at M0 = lds_off + 16 lane
// (one global_load_lds_dwordx4: 1 KiB, four 256-byte rows when lanes 16 k .. 16 k + 15
// fill row k).  Inline asm, waited on with s_waitcnt vmcnt, as row_to_lds.
__device__ __forceinline__ void gather16_to_lds(const void* src, uint32_t lds_off) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(lds_off), "v"(src)
      : "memory", "m0");
}

// Workgroup barrier without the full memory-counter drain that __syncthreads()
// implies, so the next tile's global->LDS loads stay in flight across it.  The
// empty asm keeps the compiler from moving LDS accesses across the barrier; the
// caller waits for exactly the loads it needs with s_waitcnt.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// max / sum over the four lanes l, l^16, l^32, l^48 that hold one head's keys
__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// K fragment as two 8-byte LDS reads (lo: k-slots 0..3, hi: 4..7 of the lane group).
// volatile keeps the pair from being fused into one ds_read2 (16 bytes per lane),
// which is as slow as ds_read_b128.
__device__ __forceinline__ bf16x8 kfrag(const unsigned char* tb, int off_lo, int off_hi) {
  typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
  typedef const volatile __attribute__((address_space(3))) unsigned long long lds_u64;
  const unsigned long long lo = *(lds_u64*)(tb + off_lo);
  const unsigned long long hi = *(lds_u64*)(tb + off_hi);
  return __builtin_bit_cast(bf16x8, u64x2{lo, hi});
}

__device__ __forceinline__ bf16x4 ds_read_tr(const unsigned char* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                         (__attribute__((address_space(3))) s16x4*)(p)));
}

}  // namespace csa
