// Learned gated compressor (the alternative to mean pooling), r = 4, bf16 operands.
//
// Per compressed row c (segment b, group j, stream rows t = s_b + 4 j + m):
//   kv = x wkv^T, score = x wgate^T (float32 sums of bf16 products), score += ape[m]
//   overlap (C = 2 hd): positions 0..3 = previous group's channels [0, hd),
//                       positions 4..7 = own channels [hd, 2 hd); a segment's first
//                       group has no previous group (kv 0, score -inf there)
//   out[c, ch] = sum over positions of softmax(score[., ch]) kv[., ch]
//
// One GEMM tile per workgroup: 64 groups (256 stream rows) x 256 projection columns,
// K = the hidden size in steps of 64 staged through LDS with global_load_lds_dwordx4,
// two stages (one in flight).  Four wavefronts, each a 128 x 128 quarter as 4 x 4
// v_mfma_f32_32x32x16_bf16 accumulators.  When that leaves CUs idle (fewer than 512
// tiles) a half-height tile is used: 32 groups, 2 x 4 accumulators per wavefront, 32
// dims per stage in three stages, two workgroups per CU.  The tile's columns are weight rows chosen so
// that one accumulator column holds, for one channel, every projection the pooling
// needs:
//   overlap:    column blocks [wkv ch, wkv hd + ch, wgate ch, wgate hd + ch] (32 ch)
//   no overlap: column blocks [wkv ch, wgate ch, wkv ch + 32, wgate ch + 32]
// and the first-half blocks (wkv ch, wgate ch) multiply the rows one group earlier
// than the second-half blocks: the A stage holds the 4 rows before the tile too.  An
// accumulator lane holds rows 8 q + 4 (lane / 32) + m, m < 4, i.e. whole groups, so
// every lane finds its group's own second half and its previous group's first half in
// its own registers, and the pooling runs there.
#include "csa_common.h"
#include "csa_internal.h"
#include "csa_tile.h"

namespace csa {
namespace {

// Tile shape: MT stream rows (MT / 4 groups) x 256 projection columns, KS hidden dims
// per LDS stage, NST stages.  Measured on the 16k pack at hidden size 4096: 64 dims per
// stage with two stages beats 32 dims with three or four (fewer barriers per MFMA).
template <int MT, int KS, int NST>
struct LrCfg {
  static constexpr int kMT = MT;
  static constexpr int kMinBlocks = MT == 128 ? 2 : 1;          // workgroups per CU the registers must allow
  static constexpr int kGroups = MT / 4;                        // groups per tile
  static constexpr int kMB = MT / 64;                           // 32-row blocks per wavefront
  static constexpr int kK = KS;
  static constexpr int kStages = NST;
  static constexpr int kRB = KS * 2;                            // LDS row bytes
  static constexpr int kRPI = 1024 / kRB;                       // rows per load instruction (1 KiB)
  static constexpr int kAinst = (MT + 4 + kRPI - 1) / kRPI;     // A: 4 leading rows + MT
  static constexpr int kArows = kAinst * kRPI;
  static constexpr int kBinst = 256 / kRPI;
  static constexpr int kStageA = kArows * kRB;
  static constexpr int kStageB = 256 * kRB;
  static constexpr int kStage = kStageA + kStageB;
  static constexpr int kAper = (kAinst - 1) / 4;                // A instructions per wavefront (+1 for wavefront 0)
  static constexpr int kBper = kBinst / 4;
  static constexpr int kPerStage = kAper + kBper;               // loads per stage (wavefront 0: one more)
  static_assert(kAinst == 4 * kAper + 1 && kBinst == 4 * kBper, "load split");
  static_assert(NST * kStage <= 160 * 1024 - 1024, "LDS");
  static_assert(kArows / 4 <= kThreads, "table fill");
  // 16-byte chunk c of LDS row L lives at chunk c ^ lsw(L): any 16 consecutive rows
  // read at one logical chunk touch 16 distinct 16-byte bank groups (of 256 bytes).
  __device__ static int lsw(int L) { return (L / (256 / kRB)) & (kRB / 16 - 1); }
};
using LrBig = LrCfg<256, 64, 2>;    // 64 groups per tile
using LrSmall = LrCfg<128, 32, 3>;  // 32 groups per tile: twice the tiles, two workgroups per CU

// s_waitcnt vmcnt(V) (expcnt and lgkmcnt not waited on)
template <int V>
__device__ __forceinline__ void wait_vm() {
  static_assert(V >= 0 && V < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | 0x0F70);
}

// wait until at most `later` stages' loads (n per stage) are outstanding
template <int N>
__device__ __forceinline__ void wait_stages(int later) {
  if (later >= 3) wait_vm<3 * N>();
  else if (later == 2) wait_vm<2 * N>();
  else if (later == 1) wait_vm<N>();
  else wait_vm<0>();
}

template <bool OVERLAP, class Cfg>
__global__ __launch_bounds__(kThreads, Cfg::kMinBlocks) void learned_compress_kernel(
    const uint16_t* __restrict__ x, int D, const uint16_t* __restrict__ wkv, const uint16_t* __restrict__ wgate,
    const float* __restrict__ ape, int hd, const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp,
    int B, int Tc_cap, int n_mt, int n_nt, uint16_t* __restrict__ out) {
  constexpr int kLrGroups = Cfg::kGroups, kLrK = Cfg::kK, kLrStages = Cfg::kStages, kLrRB = Cfg::kRB;
  constexpr int kLrRPI = Cfg::kRPI, kLrAinst = Cfg::kAinst, kLrArows = Cfg::kArows, kLrStageA = Cfg::kStageA;
  constexpr int kLrStage = Cfg::kStage, kLrAper = Cfg::kAper, kLrBper = Cfg::kBper, kLrPerStage = Cfg::kPerStage;
  constexpr int MB = Cfg::kMB, HALF = Cfg::kMT / 2;  // 32-row blocks and rows per wavefront
  auto lsw = [](int L) { return Cfg::lsw(L); };
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kLrStages * kLrStage];
  __shared__ int32_t s_base[kLrArows / 4];  // entry e: group G0 - 1 + e
  __shared__ int32_t s_first[kLrArows / 4];

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
  const int G0 = mt * kLrGroups;
  if (G0 >= Tc) return;

  if (tid < kLrArows / 4) {
    const int c = G0 - 1 + tid;
    int base = 0, first = 0;
    if (c >= 0 && c < Tc) {
      const int b = segment_of(cu_cmp, B, c);
      const int j = c - cu_cmp[b];
      base = cu_kv[b] + 4 * j;
      first = j == 0;
    }
    s_base[tid] = base;  // groups outside [0, Tc) read rows 0..3; their results are unused
    s_first[tid] = first;
  }
  __syncthreads();

  // ---- per-lane load offsets.  One load instruction fills kLrRPI LDS rows: lane l ->
  // row kLrRPI u + l / (64 / kLrRPI), 16-byte chunk l % (64 / kLrRPI).  A: instructions
  // u = wave + 4 v and, for wavefront 0, the last one as well; B: u = wave + 4 v.
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(CSA_LDS(lds)));
  const int chs = OVERLAP ? nt * 64 + 32 * wn : nt * 128 + 64 * wn;  // this wavefront's first channel
  const bool extra = wave == 0;  // wavefront 0 also loads the last A instruction
  constexpr int CPR = kLrRB / 16;  // chunks per row
  uint32_t aoff[kLrAper + 1], boff[kLrBper];
#pragma unroll
  for (int v = 0; v <= kLrAper; ++v) {
    const int u = (v < kLrAper) ? wave + 4 * v : kLrAinst - 1;
    const int L = kLrRPI * u + lane / CPR;
    const int src = (lane % CPR) ^ lsw(L);
    aoff[v] = static_cast<uint32_t>(s_base[L >> 2] + (L & 3)) * static_cast<uint32_t>(2 * D) +
              static_cast<uint32_t>(src * 16);
  }
#pragma unroll
  for (int v = 0; v < kLrBper; ++v) {
    const int u = wave + 4 * v;
    const int Rb = kLrRPI * u + lane / CPR;  // tile column
    const int src = (lane % CPR) ^ lsw(Rb);
    const int nb = (Rb >> 5) & 3, i = Rb & 31, cwn = Rb >> 7;
    int wrow;
    if (OVERLAP) wrow = nt * 64 + 32 * cwn + i + ((nb & 1) ? hd : 0);
    else wrow = nt * 128 + 64 * cwn + i + ((nb >> 1) ? 32 : 0);
    boff[v] = static_cast<uint32_t>(wrow * D * 2 + src * 16);
  }
  auto stage = [&](int ks, int bf) {
    const unsigned char* xa = reinterpret_cast<const unsigned char*>(x) + ks * kLrK * 2;
    const uint32_t la = lds0 + static_cast<uint32_t>(bf * kLrStage);
#pragma unroll
    for (int v = 0; v < kLrAper; ++v)
      row_to_lds(xa, aoff[v], la + static_cast<uint32_t>((wave + 4 * v) * 1024));
    if (extra) row_to_lds(xa, aoff[kLrAper], la + static_cast<uint32_t>((kLrAinst - 1) * 1024));
#pragma unroll
    for (int v = 0; v < kLrBper; ++v) {
      const int u = wave + 4 * v;
      const int nb = ((kLrRPI * u) >> 5) & 3;  // column block of rows kLrRPI u ..
      const bool gate = OVERLAP ? (nb >= 2) : (nb & 1);
      const unsigned char* wb = reinterpret_cast<const unsigned char*>(gate ? wgate : wkv) + ks * kLrK * 2;
      row_to_lds(wb, boff[v], la + static_cast<uint32_t>(kLrStageA + u * 1024));
    }
  };

  // fragment offsets: row 32 blk + lane % 32 (+ 4 for the group-aligned A rows), chunk 2 s + h
  constexpr int NS = kLrK / 16;  // MFMA k-steps per stage
  uint32_t fo_lo[NS], fo_hi[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int r0 = lane & 31, r1 = r0 + 4;
    fo_lo[s] = static_cast<uint32_t>(r0 * kLrRB + (((2 * s + h) ^ lsw(r0)) * 16));
    fo_hi[s] = static_cast<uint32_t>(r1 * kLrRB + (((2 * s + h) ^ lsw(r1)) * 16));
  }

  f32x16 acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.f;

  const int nk = D / kLrK;
#pragma unroll
  for (int st = 0; st < kLrStages - 1; ++st)
    if (st < nk) stage(st, st);
  for (int ks = 0; ks < nk; ++ks) {
    // this wavefront's rows of stage ks have landed once only the later stages' loads
    // remain (kLrPerStage + 1 instructions per stage for wavefront 0)
    const int later = min(nk - 1 - ks, kLrStages - 2);
    if (extra) wait_stages<kLrPerStage + 1>(later);
    else wait_stages<kLrPerStage>(later);
    tile_barrier();  // everyone's rows landed; the buffer of stage ks - 1 is free
    if (ks + kLrStages - 1 < nk) stage(ks + kLrStages - 1, (ks + kLrStages - 1) % kLrStages);
    const unsigned char* A = lds + (ks % kLrStages) * kLrStage + wm * HALF * kLrRB;
    const unsigned char* Bm = lds + (ks % kLrStages) * kLrStage + kLrStageA + wn * 128 * kLrRB;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 alo[MB], ahi[MB], b[4];
#pragma unroll
      for (int q = 0; q < MB; ++q) {
        ahi[q] = *reinterpret_cast<const bf16x8*>(A + q * 32 * kLrRB + fo_hi[s]);
        if (OVERLAP) alo[q] = *reinterpret_cast<const bf16x8*>(A + q * 32 * kLrRB + fo_lo[s]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = *reinterpret_cast<const bf16x8*>(Bm + q * 32 * kLrRB + fo_lo[s]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const bf16x8 a = (OVERLAP && (nb == 0 || nb == 2)) ? alo[mb] : ahi[mb];
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[nb], acc[mb][nb], 0, 0, 0);
        }
    }
  }

  // ---- pooling epilogue.  Lane (h, l % 32): channel(s) chs + l % 32 (+ 32), groups
  // gi = (MT / 8) wm + 8 mb + 2 q + h, positions m = 0..3 in acc[mb][.][4 q + m]; with overlap
  // blocks 0 and 2 hold the previous group's rows.
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
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gi = (HALF / 4) * wm + 8 * mb + 2 * q + h;
        const int c = G0 + gi;
        if (c >= Tc) continue;
        const bool first = s_first[gi + 1] != 0;
        float sc[8], kvv[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          sc[m] = first ? -__builtin_huge_valf() : acc[mb][2][4 * q + m] + ape_lo[m];
          kvv[m] = first ? 0.f : acc[mb][0][4 * q + m];
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
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = G0 + (HALF / 4) * wm + 8 * mb + 2 * q + h;
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
  return dtype == 1 && cmp_ratio == 4 && D >= 64 && D % 64 == 0 && hd > 0 && hd % (overlap ? 64 : 128) == 0;
}

template <class Cfg>
static hipError_t launch_learned_cfg(const uint16_t* x, int D, const uint16_t* wk, const uint16_t* wg, const float* ape, int hd,
                              int overlap, const int32_t* cu_kv, const int32_t* cu_cmp, int B, uint16_t* out,
                              int Tc_cap, hipStream_t s) {
  const int n_mt = (Tc_cap + Cfg::kGroups - 1) / Cfg::kGroups;
  const int n_nt = hd / (overlap ? 64 : 128);
  const long long total = static_cast<long long>(n_mt) * n_nt;
  const long long grid = (total + 7) / 8 * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (overlap)
    hipLaunchKernelGGL((learned_compress_kernel<true, Cfg>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s,
                       x, D, wk, wg, ape, hd, cu_kv, cu_cmp, B, Tc_cap, n_mt, n_nt, out);
  else
    hipLaunchKernelGGL((learned_compress_kernel<false, Cfg>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s,
                       x, D, wk, wg, ape, hd, cu_kv, cu_cmp, B, Tc_cap, n_mt, n_nt, out);
  return hipGetLastError();
}

hipError_t launch_compress_learned(const void* x, int Tkv, int D, const void* wkv, const void* wgate,
                                   const float* ape, int hd, int overlap, const int32_t* cu_kv,
                                   const int32_t* cu_cmp, int B, void* out, int Tc_cap, hipStream_t s) {
  if (Tc_cap <= 0 || Tkv <= 0) return hipSuccess;  // nothing to launch
  const auto* x16 = static_cast<const uint16_t*>(x);
  const auto* wk = static_cast<const uint16_t*>(wkv);
  const auto* wg = static_cast<const uint16_t*>(wgate);
  auto* o16 = static_cast<uint16_t*>(out);
  // the large tile unless it leaves CUs idle: 256 CUs take one large tile each
  const long long big_tiles =
      static_cast<long long>((Tc_cap + LrBig::kGroups - 1) / LrBig::kGroups) * (hd / (overlap ? 64 : 128));
  if (big_tiles >= 2 * 256)
    return launch_learned_cfg<LrBig>(x16, D, wk, wg, ape, hd, overlap, cu_kv, cu_cmp, B, o16, Tc_cap, s);
  return launch_learned_cfg<LrSmall>(x16, D, wk, wg, ape, hd, overlap, cu_kv, cu_cmp, B, o16, Tc_cap, s);
}

}  // namespace csa
