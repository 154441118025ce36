// Lightning indexer + per-query top-k over the query's own segment.
//
// Queries with no more candidates than top-k only write the ascending candidate list.
// Otherwise every candidate gets an order-preserving uint32 key of its score, a 4-pass
// 8-bit radix select finds the k-th largest key, and an ordered scan emits the kept rows
// in ascending order (exact ties go to the lower row).
//
// (H_I, d_I) = (64, 128) bf16: indexer_score_kernel, a workgroup of 8 wavefronts per 8
// consecutive queries.  The queries of one segment share that segment's compressed keys,
// staged through LDS in chunks of 64 rows (16 KiB, global_load_lds, XOR-swizzled 16-byte
// chunks, three buffers) once for all of them.  Wavefront w scores query w:
// v_mfma_f32_16x16x32_bf16 with the 64 indexer heads as M (q_I in registers), 16
// candidates as N (conflict-free 16-byte LDS reads), ReLU and head weights on the fp32 C
// fragments, a 4-lane-group sum; the keys go to the caller's workspace (one row of
// floor(max_seqlen_kv / r) per query).  indexer_select_kernel then gives each query one
// wavefront that selects from its keys with no workgroup barrier (wave_select_emit), the
// keys held in registers when every list fits 6144 of them.
// Small shapes (H_I * d_I <= 8192, either dtype): indexer_topk_kernel scores with scalar
// fp32 straight into LDS and selects with the whole workgroup.
#include "csa_common.h"
#include "csa_internal.h"
#include "csa_tile.h"

namespace csa {
namespace {

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

// Candidate range of local query i: rows [lo, lo + nv) of its segment b that are
// causally complete, exist in the k_cmp buffer (Tc rows) and fit the score storage.
// With a caller-held residual that disagrees with the segment length, nv = -1 (the
// query's row is then written as all -1).
__device__ __forceinline__ int candidate_range(int i, const int32_t* __restrict__ cu_q,
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
  return b;
}

// The row of a query whose segment's residual disagrees: no selection, NaN scores.
__device__ __forceinline__ void write_poisoned_row(int32_t* __restrict__ out_idx, float* __restrict__ out_sc,
                                                   int topk) {
  for (int k = threadIdx.x; k < topk; k += kThreads) {
    out_idx[k] = -1;
    if (out_sc) out_sc[k] = __builtin_nanf("");
  }
}

// The scoring kernel's template parameters: CH candidates per LDS chunk (rows of 256 B,
// CH / 16 MFMA blocks) and NW queries (wavefronts) per workgroup, each wavefront staging
// CH / (4 NW) rows-of-4 (1 KiB global_load_lds) per chunk.  Launched as CH = 64, NW = 8.
constexpr int kStages = 3;                 // chunk buffers: loads run two chunks ahead
constexpr int kRun = 4;                    // consecutive tiles per XCD run

constexpr int kList = 768;  // per-wavefront LDS list of the keys in the threshold bin

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64)));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64)));
  return v;
}

// 256 LDS bins of one wavefront: the bin d that holds the kk-th largest entry (counting
// from the top bin down) and the count of entries in the bins above it.  Lane l reads
// bins 255 - 4 l .. 252 - 4 l, so lane order is descending bin order.
__device__ __forceinline__ void wave_hist_find(const uint32_t* hist, uint32_t kk, uint32_t& digit, uint32_t& above) {
  const int lane = threadIdx.x & 63;
  uint32_t c[4], loc = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    c[t] = hist[255 - 4 * lane - t];
    loc += c[t];
  }
  uint32_t incl = loc;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(incl, off, 64);
    if (lane >= off) incl += u;
  }
  const uint32_t excl = incl - loc;
  const bool here = excl < kk && incl >= kk;
  int dsel = 0;
  uint32_t ab = excl;
  if (here) {
    uint32_t run = excl;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (run + c[t] >= kk) {
        dsel = 255 - 4 * lane - t;
        ab = run;
        break;
      }
      run += c[t];
    }
  }
  const int src = __ffsll(static_cast<long long>(__ballot(here))) - 1;
  digit = static_cast<uint32_t>(__shfl(dsel, src, 64));
  above = static_cast<uint32_t>(__shfl(static_cast<int>(ab), src, 64));
}

__device__ __forceinline__ void wave_hist_zero(uint32_t* hist) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < 4; ++t) hist[64 * t + lane] = 0u;
}

// Bin of a key on the linear scale between fmin and fmax (scale = 256 / (fmax - fmin),
// finite): the subtraction, the product and the truncation are each monotone, so the bin
// never decreases with the key.
__device__ __forceinline__ uint32_t linear_bin(uint32_t key, float fmin, float scale) {
  const float x = (order_key_to_float(key) - fmin) * scale;
  return static_cast<uint32_t>(min(max(static_cast<int>(x), 0), 255));
}

// Radix select over bits top..0 of the keys that have the given prefix in the bits above
// top: the kk-th largest such key.  FROM_LIST: the m keys in list (LDS); otherwise the nv
// keys in global memory that fall in linear bin `bsel` (bsel < 0: every key).
template <bool FROM_LIST>
__device__ uint32_t wave_radix_kth(const uint32_t* __restrict__ keys, int nv, const uint32_t* list, int m, int top,
                                   uint32_t prefix, uint32_t& kk, int bsel, float fmin, float scale, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t pmask = (top >= 31) ? 0u : ~((2u << top) - 1u);
  prefix &= pmask;
  while (top >= 0) {
    const int w = min(8, top + 1);
    const int shift = top - w + 1;
    const uint32_t dmask = (1u << w) - 1u;
    wave_hist_zero(hist);
    const int n = FROM_LIST ? m : nv;
    for (int j = lane; j < n; j += 64) {
      const uint32_t k = FROM_LIST ? list[j] : keys[j];
      bool in = (k & pmask) == prefix;
      if (!FROM_LIST && bsel >= 0) in = in && linear_bin(k, fmin, scale) == static_cast<uint32_t>(bsel);
      if (in) atomicAdd(&hist[(k >> shift) & dmask], 1u);
    }
    uint32_t d, ab;
    wave_hist_find(hist, kk, d, ab);
    prefix |= d << shift;
    pmask |= dmask << shift;
    kk -= ab;
    top -= w;
  }
  return prefix;
}

// Keys of one query, slot t of lane l = key 64 t + l: KPL > 0 holds the nv <= 64 KPL keys
// in registers (loaded once); KPL == 0 streams them from the workspace row on every pass.
template <int KPL>
struct WaveKeys {
  uint32_t kr[KPL > 0 ? KPL : 1];
  const uint32_t* __restrict__ keys;
  int nv;
  __device__ __forceinline__ int slots() const { return KPL > 0 ? KPL : (nv + 63) / 64; }
  // key of slot t (0 past nv); only slots with 64 t < nv are asked for
  __device__ __forceinline__ uint32_t at(int t, int lane) const {
    const int j = 64 * t + lane;
    if constexpr (KPL > 0) {
      return kr[t];
    } else {
      return (j < nv) ? keys[j] : 0u;
    }
  }
};

// Select the topk largest of one query's nv > topk keys and write them ascending, exact
// ties to the lower row, with this wavefront alone (no workgroup barrier):
//   1. min and max key;
//   2. a 256-bin histogram linear in the score between them (scores cluster in a few
//      binades, so bins of the raw key bits would collide on every LDS atomic): the bin of
//      the topk-th largest key and the count above it;
//   3. the keys of that bin go to an LDS list (when they fit), and a radix select from
//      their first differing bit finds the threshold key T exactly;
//   4. an ordered ballot scan emits every key above T and the first kk copies of T.
// KPL > 0: the keys sit in registers for every pass; KPL == 0: each pass streams them.
template <int KPL>
__device__ __forceinline__ void wave_select_emit(const WaveKeys<KPL>& K, int topk, int lo, int32_t* __restrict__ out_idx,
                                 float* __restrict__ out_sc, uint32_t* hist, uint32_t* list) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  const int nv = K.nv, ns = K.slots();
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int t = 0; t < (KPL > 0 ? KPL : ns); ++t) {
    if (64 * t >= nv) break;
    if (64 * t + lane < nv) {
      const uint32_t k = K.at(t, lane);
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  uint32_t kk = static_cast<uint32_t>(topk);
  uint32_t T;
  if (kmin == kmax) {
    T = kmin;
  } else {
    const float fmin = order_key_to_float(kmin);
    const float range = order_key_to_float(kmax) - fmin;
    if (range > 0.f && range < __builtin_huge_valf()) {  // false for NaN keys and overflow
      const float scale = 256.f / range;
      wave_hist_zero(hist);
#pragma unroll
  for (int t = 0; t < (KPL > 0 ? KPL : ns); ++t) {
        if (64 * t >= nv) break;
        if (64 * t + lane < nv) atomicAdd(&hist[linear_bin(K.at(t, lane), fmin, scale)], 1u);
      }
      uint32_t bsel, ab;
      wave_hist_find(hist, kk, bsel, ab);
      kk -= ab;
      const int m = __builtin_amdgcn_readfirstlane(static_cast<int>(hist[bsel]));
      if (m <= kList) {
        // compact the bin's keys (any order) and narrow the radix to their differing bits
        uint32_t base = 0, bmin = 0xffffffffu, bmax = 0u;
#pragma unroll
  for (int t = 0; t < (KPL > 0 ? KPL : ns); ++t) {
          if (64 * t >= nv) break;
          const uint32_t k = K.at(t, lane);
          const bool in = 64 * t + lane < nv && linear_bin(k, fmin, scale) == bsel;
          const uint64_t mk = __ballot(in);
          const uint32_t at = base + static_cast<uint32_t>(__popcll(mk & below));
          if (in && at < static_cast<uint32_t>(kList)) {  // at < m <= kList: the same bins as counted
            list[at] = k;
            bmin = min(bmin, k);
            bmax = max(bmax, k);
          }
          base += static_cast<uint32_t>(__popcll(mk));
        }
        bmin = wave_min_u32(bmin);
        bmax = wave_max_u32(bmax);
        if (bmin == bmax) {
          T = bmin;
        } else {
          const int top = 31 - __builtin_clz(bmin ^ bmax);
          T = wave_radix_kth<true>(K.keys, nv, list, m, top, bmin, kk, -1, 0.f, 0.f, hist);
        }
      } else {
        T = wave_radix_kth<false>(K.keys, nv, list, 0, 31, 0u, kk, static_cast<int>(bsel), fmin, scale, hist);
      }
    } else {
      const int top = 31 - __builtin_clz(kmin ^ kmax);
      T = wave_radix_kth<false>(K.keys, nv, list, 0, top, kmin, kk, -1, 0.f, 0.f, hist);
    }
  }
  // T is the topk-th largest key; kk of its copies are kept
  uint32_t base_sel = 0, base_tie = 0;
#pragma unroll
  for (int t = 0; t < (KPL > 0 ? KPL : ns); ++t) {
    if (64 * t >= nv) break;
    const int j = 64 * t + lane;
    const uint32_t key = K.at(t, lane);
    const bool gt = j < nv && key > T;
    const bool eq = j < nv && key == T;
    const uint64_t me = __ballot(eq);
    const bool take = gt || (eq && base_tie + static_cast<uint32_t>(__popcll(me & below)) < kk);
    const uint64_t mt = __ballot(take);
    const uint32_t pos = base_sel + static_cast<uint32_t>(__popcll(mt & below));
    if (take && pos < static_cast<uint32_t>(topk)) {
      out_idx[pos] = lo + j;
      if (out_sc) out_sc[pos] = order_key_to_float(key);
    }
    base_sel += static_cast<uint32_t>(__popcll(mt));
    base_tie += static_cast<uint32_t>(__popcll(me));
  }
  for (int k = static_cast<int>(base_sel) + lane; k < topk; k += 64) {
    out_idx[k] = -1;
    if (out_sc) out_sc[k] = -__builtin_huge_valf();
  }
}

// One wavefront per query (4 per workgroup): the row of every query: poisoned, the
// ascending list (with scores from the keys when asked), or the top-k of the keys the
// scoring kernel wrote (KPL > 0: every candidate list fits 64 KPL keys in registers).
// The 96-slot instance (lists of more than 4096 candidates) is held to 168 registers for
// three wavefronts per SIMD (no spill): the 32k CP share's indexer call 1.71-1.73 ->
// 1.61-1.63 ms; the smaller instances measured no change either way.
template <int KPL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(KPL >= 96 ? 3 : 1))) void indexer_select_kernel(
    int Tq, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp,
    const int32_t* __restrict__ residual, int B, int global_start, int r, int cap, int Tc, int topk,
    const uint32_t* __restrict__ keys, int32_t* __restrict__ idx, float* __restrict__ score) {
  __shared__ uint32_t hist[kWaves][256];
  __shared__ uint32_t list[kWaves][kList];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int i = static_cast<int>(blockIdx.x) * kWaves + wave;
  if (i >= Tq) return;
  int lo, nv;
  candidate_range(i, cu_q, cu_kv, cu_cmp, residual, B, global_start, r, cap, Tc, lo, nv);
  lo = __builtin_amdgcn_readfirstlane(lo);
  nv = __builtin_amdgcn_readfirstlane(nv);
  int32_t* out_idx = idx + static_cast<long long>(i) * topk;
  float* out_sc = score ? score + static_cast<long long>(i) * topk : nullptr;
  const uint32_t* my_keys = keys + static_cast<long long>(i) * cap;
  if (nv < 0) {
    for (int k = lane; k < topk; k += 64) {
      out_idx[k] = -1;
      if (out_sc) out_sc[k] = __builtin_nanf("");
    }
    return;
  }
  if (nv <= topk) {
    for (int k = lane; k < topk; k += 64) {
      out_idx[k] = (k < nv) ? lo + k : -1;
      if (out_sc) out_sc[k] = (k < nv) ? order_key_to_float(my_keys[k]) : -__builtin_huge_valf();
    }
    return;
  }
  WaveKeys<KPL> K;
  K.keys = my_keys;
  K.nv = nv;
  if constexpr (KPL > 0) {
#pragma unroll
    for (int t = 0; t < KPL; ++t) K.kr[t] = (64 * t + lane < nv) ? my_keys[64 * t + lane] : 0u;
  }
  wave_select_emit<KPL>(K, topk, lo, out_idx, out_sc, hist[wave], list[wave]);
}

// ---- pieces of indexer_score_kernel (plain functions: a by-reference lambda closure
// would escape through the barriers' memory clobbers and put its captures in scratch)

// Stage chunk c of a group's key rows into LDS buffer at lds_buf: wavefront w of NW stages
// rows CH / NW * w onward (CH / (4 NW) 1 KiB instructions of 4 rows); rows past the
// group's nvmax candidates re-read its first row.
template <int CH, int NW>
__device__ __forceinline__ void score_stage(const uint16_t* __restrict__ k_cmp, int glo, int nvmax, int c,
                                            uint32_t lds_buf, int wave, int lane) {
#pragma unroll
  for (int v = 0; v < CH / (4 * NW); ++v) {
    const int rr = (CH / NW) * wave + 4 * v + (lane >> 4);
    int cand = CH * c + rr;
    cand = (cand < nvmax) ? cand : 0;
    const uint16_t* src = k_cmp + static_cast<long long>(glo + cand) * 128 + kchunk(rr, lane & 15) * 8;
    gather16_to_lds(src, lds_buf + static_cast<uint32_t>(((CH / NW) * wave + 4 * v) * 256));
  }
}

// B operand of block jb (candidates 16 jb + n of the staged chunk), K slots 32 ks + 8 g ..
__device__ __forceinline__ void score_read_kf(const unsigned char* kb, int jb, int n, int g, bf16x8 (&dst)[4]) {
  const int row = 16 * jb + n;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) dst[ks] = *reinterpret_cast<const bf16x8*>(kb + row * 256 + kchunk(row, 4 * ks + g) * 16);
}

// S[16 mb + 4 g + j, n] for the 64 heads and the block's 16 candidates
__device__ __forceinline__ void score_block_mfma(const bf16x8 (&qa)[4][4], const bf16x8 (&kv)[4], f32x4 (&a)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      a[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mb][ks], kv[ks], ks ? a[mb] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                       0);
}

// Order key of sum_h w_h * max(S_h, 0) for candidate n (every lane group gets it).  The
// ReLU is an integer max on the bits (negative floats, -0 included, are negative
// integers): one op, the same values as fmaxf(x, 0).
__device__ __forceinline__ uint32_t score_block_key(const float (&wv)[4][4], const f32x4 (&a)[4]) {
  float sc = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) sc = fmaf(wv[mb][j], __int_as_float(max(__float_as_int(a[mb][j]), 0)), sc);
  return float_order_key(quad_sum(sc));
}

// Lane (n, g) writes the keys of candidates base + 64 q + 16 g + n (blocks 4 q + g, which
// this lane kept in mine[q]): one 256-byte store per four blocks.
template <int NQ>
__device__ __forceinline__ void score_store_keys(const uint32_t (&mine)[NQ], uint32_t* __restrict__ my_keys, int base,
                                                 int nv, int n, int g) {
#pragma unroll
  for (int qd = 0; qd < NQ; ++qd) {
    const int cand = base + 64 * qd + 16 * g + n;
    if (cand < nv) my_keys[cand] = mine[qd];
  }
}

// One pipeline step is one scheduling region: the next block's LDS reads first, then each
// MFMA followed by a few VALU ops of the previous block's epilogue.
__device__ __forceinline__ void score_interleave() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS reads
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Keys of the candidates of up to 8 consecutive local queries [8 t, 8 t + 8) (tile t), one
// per wavefront: every query with more candidates than topk (or any candidate, when scores
// are returned) gets the key of each candidate c < nv in keys[i * cap + c]; the queries of
// one segment share each staged chunk of key rows.  Tiles run on XCDs in runs of kRun, so
// a run's queries (the same segment, mostly) also share the key rows in one L2.
template <int CH, int NW>
__global__ __launch_bounds__(64 * NW) void indexer_score_kernel(
    const uint16_t* __restrict__ q_I, const uint16_t* __restrict__ w, const uint16_t* __restrict__ k_cmp, int Tq,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp,
    const int32_t* __restrict__ residual, int B, int global_start, int r, int cap, int Tc, int topk, int score_all,
    int ntile, uint32_t* __restrict__ keys) {
  __shared__ __attribute__((aligned(1024))) unsigned char kst[kStages][CH * 256];
  __shared__ int wseg[NW], wlo[NW], wnv[NW];
  static_assert(CH % (4 * NW) == 0 && CH / (4 * NW) < 16, "chunk loads per wavefront: whole, and within vmcnt's low field");
  constexpr int NB = CH / 16;
  const int xcd = static_cast<int>(blockIdx.x) & 7, kk = static_cast<int>(blockIdx.x) >> 3;
  const int tile = ((kk / kRun) * 8 + xcd) * kRun + (kk % kRun);
  if (tile >= ntile) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int i = NW * tile + wave;
  if (lane == 0) {
    int seg = -1, lo = 0, nv = 0;
    if (i < Tq) {
      const int b = candidate_range(i, cu_q, cu_kv, cu_cmp, residual, B, global_start, r, cap, Tc, lo, nv);
      if (nv > topk || (score_all && nv > 0)) seg = b;
    }
    wseg[wave] = seg;
    wlo[wave] = lo;
    wnv[wave] = nv;
  }
  __syncthreads();
  const bool heavy = wseg[wave] >= 0;
  const int my_nv = __builtin_amdgcn_readfirstlane(wnv[wave]);
  uint32_t* my_keys = keys + static_cast<long long>(i) * cap;
  const uint32_t kbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(CSA_LDS(kst)));

  // ---- phase 1: scores
  {
    // A operand: q_I[i, 16 mb + n, 32 ks + 8 g + 0..7]; head weights of the C rows this lane
    // holds (heads 16 mb + 4 g + j)
    bf16x8 qa[4][4];
    float wv[4][4];
    if (heavy) {
      const uint16_t* qrow = q_I + static_cast<long long>(i) * 64 * 128;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qa[mb][ks] = *reinterpret_cast<const bf16x8*>(qrow + (16 * mb + n) * 128 + 32 * ks + 8 * g);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wv[mb][j] = bf16_bits_to_f32(w[static_cast<long long>(i) * 64 + 16 * mb + 4 * g + j]);
    }
    // q_I and w are in registers before any chunk load is counted against vmcnt
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    // The heavy queries of one segment form a group that shares every staged chunk; a
    // tile straddling a segment boundary runs its groups one after the other.
    int done = 0;
    while (true) {
      int gseg = -1, glo = 0, nvmax = 0, mask = 0;
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        const int sk = wseg[k];
        if (sk < 0 || ((done >> k) & 1)) continue;
        if (gseg < 0) {
          gseg = sk;
          glo = wlo[k];
        }
        if (sk == gseg) {
          mask |= 1 << k;
          nvmax = max(nvmax, wnv[k]);
        }
      }
      if (gseg < 0) break;
      done |= mask;
      const bool mine = (mask >> wave) & 1;
      const int nch = (nvmax + CH - 1) / CH;
      score_stage<CH, NW>(k_cmp, glo, nvmax, 0, kbase, wave, lane);
      if (nch > 1) score_stage<CH, NW>(k_cmp, glo, nvmax, 1, kbase + CH * 256, wave, lane);
      // Software pipeline over 16-candidate blocks: block (c, jb) issues its 16 MFMAs into
      // acc0 / acc1 (alternately) while the VALU epilogue (ReLU, head weights, lane-group sum) of the
      // previous block runs on the other buffer, so the matrix core and the VALU overlap
      // within one wavefront; the K fragments are read one block ahead.  A live chunk
      // computes every block (the queries of one group differ by at most a few
      // candidates, so only the last chunk's tail is wasted) to keep each step one basic
      // block; only keys of candidates below nv are stored.
      f32x4 acc0[4], acc1[4];
      bf16x8 kf0[4], kf1[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc1[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // keys of blocks 4 q + g: every lane group holds every block's key after the lane-group
      // sum, and lane group g keeps those of blocks 4 q + g (a conditional move per block
      // with a constant block index; a select over an indexed array would live in scratch)
      uint32_t pm[NB / 4], cm[NB / 4];  // the previous chunk's (its last block once reduced), this chunk's
#pragma unroll
      for (int qd = 0; qd < NB / 4; ++qd) pm[qd] = cm[qd] = 0u;
      for (int c = 0; c < nch; ++c) {
        const int bf = c % kStages;
        // chunk c has landed: the only younger vector-memory loads are chunk c + 1's
        // (loads retire in order; key stores in between do not matter)
        if (c + 1 < nch) {
          __builtin_amdgcn_s_waitcnt(0x0F70 | (CH / (4 * NW)));  // vmcnt(CH / (4 NW))
        } else {
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        }
        // every wavefront's rows of chunk c are visible; every wavefront is done with
        // chunk c - 1, whose buffer chunk c + 2 refills
        tile_barrier();
        if (c + 2 < nch) score_stage<CH, NW>(k_cmp, glo, nvmax, c + 2, kbase + ((c + 2) % kStages) * CH * 256, wave, lane);
        if (mine && my_nv > CH * c) {
          const unsigned char* kb = kst[bf];
          score_read_kf(kb, 0, n, g, kf0);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int jb = 0; jb < NB; ++jb) {
            if (jb + 1 < NB) score_read_kf(kb, jb + 1, n, g, ((jb + 1) & 1) ? kf1 : kf0);
            score_block_mfma(qa, (jb & 1) ? kf1 : kf0, (jb & 1) ? acc1 : acc0);
            if (jb == 0) {
              const uint32_t kx = score_block_key(wv, acc1);  // block (c - 1, NB - 1); unused when c == 0
              pm[NB / 4 - 1] = (g == 3) ? kx : pm[NB / 4 - 1];
            } else {
              const uint32_t kx = score_block_key(wv, ((jb - 1) & 1) ? acc1 : acc0);
              cm[(jb - 1) / 4] = (g == (jb - 1) % 4) ? kx : cm[(jb - 1) / 4];
            }
            score_interleave();
          }
          if (c > 0) score_store_keys(pm, my_keys, CH * (c - 1), my_nv, n, g);
#pragma unroll
          for (int qd = 0; qd < NB / 4; ++qd) pm[qd] = cm[qd];
        }
      }
      if (mine && my_nv > 0) {
        const uint32_t kx = score_block_key(wv, acc1);
        pm[NB / 4 - 1] = (g == 3) ? kx : pm[NB / 4 - 1];
        score_store_keys(pm, my_keys, CH * ((my_nv - 1) / CH), my_nv, n, g);
      }
      __syncthreads();  // every wavefront is done with the buffers before the next group stages
    }
  }

}

// Small shapes: score with scalar fp32 into LDS, then select with the whole workgroup.
template <typename T>
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
  score_generic<T>(q_I, w, k_cmp, i, H_I, d_I, lo, nv, keys, reinterpret_cast<float*>(dyn + cap));
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

size_t indexer_workspace_bytes(int Tq, int cap) { return static_cast<size_t>(Tq) * static_cast<size_t>(cap) * 4; }

hipError_t launch_indexer_topk(const void* q_I, const void* w, const void* k_cmp, int Tq, int Tc, int H_I, int d_I,
                               int dtype, const int32_t* cu_q, const int32_t* cu_kv, const int32_t* cu_cmp,
                               const int32_t* residual, int B, int global_start, int r, int cap, int topk,
                               int32_t* idx, float* score, void* workspace, hipStream_t s) {
  if (Tq <= 0) return hipSuccess;
  const bool mfma = (dtype == 1 && H_I == 64 && d_I == 128);
  size_t lds = static_cast<size_t>(cap) * 4;
  const dim3 grid(Tq), block(kThreads);
  if (mfma) {
    uint32_t* keys = static_cast<uint32_t*>(workspace);
    auto launch_score = [&](auto kern, int nw) {
      const int ntile = (Tq + nw - 1) / nw;
      const int runs = (ntile + 8 * kRun - 1) / (8 * kRun);
      hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(runs * 8 * kRun)), dim3(64 * nw), 0, s,
                         static_cast<const uint16_t*>(q_I), static_cast<const uint16_t*>(w),
                         static_cast<const uint16_t*>(k_cmp), Tq, cu_q, cu_kv, cu_cmp, residual, B, global_start, r,
                         cap, Tc, topk, score != nullptr ? 1 : 0, ntile, keys);
    };
    // 64-row chunks and 8 queries per workgroup for every list length.  Measured: 128-row
    // chunks on long lists are 2% slower on the 32k CP share (1.72 against 1.69 ms) and
    // equal elsewhere; 4 queries per workgroup (two workgroups per CU) are 6% faster where
    // few queries need scores (pack16k: 0.083 against 0.088 ms) but 2-6% slower where many
    // do (4k pack, CP share), and which case holds is only known on the device.
    launch_score(indexer_score_kernel<64, 8>, 8);
    // keys in registers up to 6144 candidates per query (one read of the workspace row),
    // streamed from the row on every pass beyond that
    const dim3 sgrid((Tq + kWaves - 1) / kWaves);
#define CSA_SELECT(KPL)                                                                                     \
  hipLaunchKernelGGL(indexer_select_kernel<KPL>, sgrid, block, 0, s, Tq, cu_q, cu_kv, cu_cmp, residual, B, \
                     global_start, r, cap, Tc, topk, keys, idx, score)
    if (cap <= 64 * 16) {
      CSA_SELECT(16);
    } else if (cap <= 64 * 32) {
      CSA_SELECT(32);
    } else if (cap <= 64 * 64) {
      CSA_SELECT(64);
    } else if (cap <= 64 * 96) {
      CSA_SELECT(96);
    } else {
      CSA_SELECT(0);
    }
#undef CSA_SELECT
    return hipGetLastError();
  }
  lds += static_cast<size_t>(H_I) * d_I * 4 + static_cast<size_t>(H_I) * 4;
  if (dtype == 1) {
    auto k = indexer_topk_kernel<uint16_t>;
    if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess) return e;
    hipLaunchKernelGGL(k, grid, block, lds, s, static_cast<const uint16_t*>(q_I), static_cast<const uint16_t*>(w),
                       static_cast<const uint16_t*>(k_cmp), H_I, d_I, cu_q, cu_kv, cu_cmp, residual, B, global_start,
                       r, cap, Tc, topk, idx, score);
  } else {
    auto k = indexer_topk_kernel<float>;
    if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess) return e;
    hipLaunchKernelGGL(k, grid, block, lds, s, static_cast<const float*>(q_I), static_cast<const float*>(w),
                       static_cast<const float*>(k_cmp), H_I, d_I, cu_q, cu_kv, cu_cmp, residual, B, global_start, r,
                       cap, Tc, topk, idx, score);
  }
  return hipGetLastError();
}

}  // namespace csa
