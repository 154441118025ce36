// Learned gated compressor (the alternative to mean pooling), r = 4, bf16 operands.
//
// Per compressed row c (segment b, group j, stream rows t = s_b + 4 j + m):
//   kv = x wkv^T, score = x wgate^T (float32 sums of bf16 products), score += ape[m]
//   overlap (C = 2 hd): positions 0..3 = previous group's channels [0, hd),
//                       positions 4..7 = own channels [hd, 2 hd); a segment's first
//                       group has no previous group (kv 0, score -inf there)
//   out[c, ch] = sum over positions of softmax(score[., ch]) kv[., ch]
//
// One GEMM tile per workgroup: 256 stream rows (64 groups) x 256 projection columns,
// K = the hidden size in steps of 64 staged through LDS with global_load_lds_dwordx4.
// Four wavefronts, each a 128 x 128 quarter as 4 x 4 v_mfma_f32_32x32x16_bf16
// accumulators.  The tile's columns are weight rows chosen so that one accumulator
// column holds, for one channel, every projection the pooling needs:
//   overlap:    column blocks [wkv ch, wkv hd + ch, wgate ch, wgate hd + ch] (32 ch)
//   no overlap: column blocks [wkv ch, wgate ch, wkv ch + 32, wgate ch + 32]
// An accumulator lane holds rows 8 q + 4 (lane / 32) + m, m < 4: whole groups, so
// the pooling runs in registers; the previous group sits in the other lane half
// (permlane32 swap) or, for a wavefront's first group, in the wavefront above it
// (LDS).  With overlap a tile starts one group early and emits 63 groups.
#include "csa_common.h"
#include "csa_internal.h"
#include "csa_tile.h"

namespace csa {
namespace {

constexpr int kLrRows = 256;                    // stream rows per tile (64 groups of 4)
constexpr int kLrGroups = kLrRows / 4;
constexpr int kLrK = 64;                        // hidden dims per K step (128-byte rows)
constexpr int kLrStageA = kLrRows * kLrK * 2;   // 32 KiB
constexpr int kLrStage = 2 * kLrStageA;         // A rows then B columns
constexpr int kLrXchg = 2 * 2 * 4 * 32 * 4;     // [wn][kv, score][m][32 ch] float

// 16-byte chunk c of 128-byte LDS row R lives at chunk c ^ lsw(R): any 16 consecutive
// rows read at one logical chunk touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ int lsw(int R) { return (R >> 1) & 7; }

__device__ __forceinline__ float other_half(float v, int h) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(h ? r[0] : r[1]);
}

template <bool OVERLAP>
__global__ __launch_bounds__(kThreads) void learned_compress_kernel(
    const uint16_t* __restrict__ x, int D, const uint16_t* __restrict__ wkv, const uint16_t* __restrict__ wgate,
    const float* __restrict__ ape, int hd, const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp,
    int B, int Tc_cap, int n_mt, int n_nt, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kLrStage + kLrXchg];
  __shared__ int32_t s_base[kLrGroups];
  __shared__ int32_t s_first[kLrGroups];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;

  // ---- work item: consecutive items on one XCD (workgroup x runs on XCD x % 8)
  const int total = n_mt * n_nt;
  const int per = (total + 7) / 8;
  const int item = (static_cast<int>(blockIdx.x) & 7) * per + (static_cast<int>(blockIdx.x) >> 3);
  if (item >= total) return;
  const int mt = item / n_nt, nt = item % n_nt;
  const int Tc = min(cu_cmp[B], Tc_cap);
  const int G0 = OVERLAP ? mt * (kLrGroups - 1) - 1 : mt * kLrGroups;
  if (G0 + (OVERLAP ? 1 : 0) >= Tc) return;

  if (tid < kLrGroups) {
    const int c = G0 + tid;
    int base = 0, first = 0;
    if (c >= 0 && c < Tc) {
      const int b = segment_of(cu_cmp, B, c);
      const int j = c - cu_cmp[b];
      base = cu_kv[b] + 4 * j;
      first = j == 0;
    }
    s_base[tid] = base;  // groups outside [0, Tc) read rows 0..3 and are not written
    s_first[tid] = first;
  }
  __syncthreads();

  // ---- per-lane load offsets: wavefront w fills LDS rows 64 w + 8 v + lane / 8
  // (v < 8) of the A rows and of the B columns, chunk lane % 8
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(CSA_LDS(lds)));
  const int chs = OVERLAP ? nt * 64 + 32 * wn : nt * 128 + 64 * wn;  // this wavefront's first channel
  uint32_t aoff[8], boff[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int R = 64 * wave + 8 * v + (lane >> 3);
    const int src = (lane & 7) ^ lsw(R);
    aoff[v] = static_cast<uint32_t>(s_base[R >> 2] + (R & 3)) * static_cast<uint32_t>(2 * D) +
              static_cast<uint32_t>(src * 16);
    // B column R: wavefront pair (R / 128), block (R / 32) % 4, channel offset R % 32
    const int nb = (R >> 5) & 3, i = R & 31;
    const int cwn = R >> 7;
    int wrow;
    if (OVERLAP) wrow = nt * 64 + 32 * cwn + i + ((nb & 1) ? hd : 0);
    else wrow = nt * 128 + 64 * cwn + i + ((nb >> 1) ? 32 : 0);
    boff[v] = static_cast<uint32_t>(wrow * D * 2 + src * 16);
  }
  // B column blocks of this wavefront's loads: (64 w + 8 v) / 32 % 4 = 2 (w % 2) + v / 4
  auto stage = [&](int ks, int bf) {
    const unsigned char* xa = reinterpret_cast<const unsigned char*>(x) + ks * kLrK * 2;
    const uint32_t la = lds0 + static_cast<uint32_t>(bf * kLrStage);
#pragma unroll
    for (int v = 0; v < 8; ++v) row_to_lds(xa, aoff[v], la + static_cast<uint32_t>((8 * wave + v) * 1024));
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int nb = 2 * (wave & 1) + (v >> 2);
      const bool gate = OVERLAP ? (nb >= 2) : (nb & 1);
      const unsigned char* wb = reinterpret_cast<const unsigned char*>(gate ? wgate : wkv) + ks * kLrK * 2;
      row_to_lds(wb, boff[v], la + static_cast<uint32_t>(kLrStageA + (8 * wave + v) * 1024));
    }
  };

  // fragment offsets: row (or column) 32 blk + lane % 32 of the quarter, k-chunk 2 s + h
  uint32_t foff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) foff[s] = static_cast<uint32_t>((lane & 31) * 128 + (((2 * s + h) ^ lsw(lane & 31)) * 16));

  f32x16 acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.f;

  const int nk = D / kLrK;
  stage(0, 0);
  for (int ks = 0; ks < nk; ++ks) {
    const int bf = ks & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's rows of step ks landed
    tile_barrier();                      // ... and everyone's; buffer bf ^ 1 is free
    if (ks + 1 < nk) stage(ks + 1, bf ^ 1);
    const unsigned char* A = lds + bf * kLrStage + wm * 128 * 128;
    const unsigned char* Bm = lds + bf * kLrStage + kLrStageA + wn * 128 * 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = *reinterpret_cast<const bf16x8*>(A + q * 32 * 128 + foff[s]);
        b[q] = *reinterpret_cast<const bf16x8*>(Bm + q * 32 * 128 + foff[s]);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
    }
  }

  // ---- pooling epilogue.  Lane (h, l % 32): channel(s) chs + l % 32 (+ 32), groups
  // gi = 32 wm + 8 mb + 2 q + h, positions m = 0..3 in acc[mb][.][4 q + m].
  const int cl = lane & 31;
  if (OVERLAP) {
    const int ch = chs + cl;
    const int C = 2 * hd;
    float ape_lo[4], ape_hi[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      ape_lo[m] = ape[m * C + ch];
      ape_hi[m] = ape[m * C + hd + ch];
    }
    // the wavefront's first group takes its previous group from the wavefront above
    float* xch = reinterpret_cast<float*>(lds + 2 * kLrStage);  // not touched by the K loop
    if (wm == 0 && h == 1) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        xch[((wn * 2 + 0) * 4 + m) * 32 + cl] = acc[3][0][12 + m];
        xch[((wn * 2 + 1) * 4 + m) * 32 + cl] = acc[3][2][12 + m];
      }
    }
    __syncthreads();
    float up_kv[4], up_sc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      up_kv[m] = xch[((wn * 2 + 0) * 4 + m) * 32 + cl];
      up_sc[m] = xch[((wn * 2 + 1) * 4 + m) * 32 + cl];
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gi = 32 * wm + 8 * mb + 2 * q + h;
        float pkv[4], psc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // previous group: h = 1 -> (mb, q) of lane - 32; h = 0 -> (mb, q - 1) of lane + 32
          const float o_same_kv = other_half(acc[mb][0][4 * q + m], h);
          const float o_same_sc = other_half(acc[mb][2][4 * q + m], h);
          float o_prev_kv, o_prev_sc;
          if (q > 0) {
            o_prev_kv = other_half(acc[mb][0][4 * q - 4 + m], h);
            o_prev_sc = other_half(acc[mb][2][4 * q - 4 + m], h);
          } else if (mb > 0) {
            o_prev_kv = other_half(acc[mb - 1][0][12 + m], h);
            o_prev_sc = other_half(acc[mb - 1][2][12 + m], h);
          } else {
            o_prev_kv = up_kv[m];
            o_prev_sc = up_sc[m];
          }
          pkv[m] = h ? o_same_kv : o_prev_kv;
          psc[m] = (h ? o_same_sc : o_prev_sc) + ape_lo[m];
        }
        const int c = G0 + gi;
        if (gi == 0 || c >= Tc) continue;  // the tile's leading group only feeds the next one
        const bool first = s_first[gi] != 0;
        float sc[8], kvv[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          sc[m] = first ? -__builtin_huge_valf() : psc[m];
          kvv[m] = first ? 0.f : pkv[m];
          sc[4 + m] = acc[mb][3][4 * q + m] + ape_hi[m];
          kvv[4 + m] = acc[mb][1][4 * q + m];
        }
        float mx = sc[4];
#pragma unroll
        for (int k = 0; k < 8; ++k) mx = fmaxf(mx, sc[k]);
        float den = 0.f, num = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float e = __expf(sc[k] - mx);
          den += e;
          num += e * kvv[k];
        }
        out[static_cast<long long>(c) * hd + ch] = f32_to_bf16_bits(num / den);
      }
    }
  } else {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int ch = chs + 32 * half + cl;
      float ap[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) ap[m] = ape[m * hd + ch];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = G0 + 32 * wm + 8 * mb + 2 * q + h;
          if (c >= Tc) continue;
          float sc[4], mx = -__builtin_huge_valf();
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            sc[m] = acc[mb][2 * half + 1][4 * q + m] + ap[m];
            mx = fmaxf(mx, sc[m]);
          }
          float den = 0.f, num = 0.f;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float e = __expf(sc[m] - mx);
            den += e;
            num += e * acc[mb][2 * half][4 * q + m];
          }
          out[static_cast<long long>(c) * hd + ch] = f32_to_bf16_bits(num / den);
        }
      }
    }
  }
}

}  // namespace

bool learned_shape_supported(int D, int hd, int cmp_ratio, int overlap, int dtype) {
  return dtype == 1 && cmp_ratio == 4 && D >= kLrK && D % kLrK == 0 && hd > 0 && hd % (overlap ? 64 : 128) == 0;
}

hipError_t launch_compress_learned(const void* x, int Tkv, int D, const void* wkv, const void* wgate,
                                   const float* ape, int hd, int overlap, const int32_t* cu_kv,
                                   const int32_t* cu_cmp, int B, void* out, int Tc_cap, hipStream_t s) {
  if (Tc_cap <= 0 || Tkv <= 0) return hipSuccess;  // nothing to launch
  const int per_tile = overlap ? kLrGroups - 1 : kLrGroups;
  const int n_mt = (Tc_cap + per_tile - 1) / per_tile;
  const int n_nt = hd / (overlap ? 64 : 128);
  const long long total = static_cast<long long>(n_mt) * n_nt;
  const long long grid = (total + 7) / 8 * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const auto* x16 = static_cast<const uint16_t*>(x);
  const auto* wk = static_cast<const uint16_t*>(wkv);
  const auto* wg = static_cast<const uint16_t*>(wgate);
  auto* o16 = static_cast<uint16_t*>(out);
  if (overlap)
    hipLaunchKernelGGL(learned_compress_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, x16,
                       D, wk, wg, ape, hd, cu_kv, cu_cmp, B, Tc_cap, n_mt, n_nt, o16);
  else
    hipLaunchKernelGGL(learned_compress_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, x16,
                       D, wk, wg, ape, hd, cu_kv, cu_cmp, B, Tc_cap, n_mt, n_nt, o16);
  return hipGetLastError();
}

}  // namespace csa
