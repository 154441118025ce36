// Sparse MLA backward, (H, d) = (64, 512) bf16: the exact gradients of the forward's
// joint softmax over window rows, compressed rows and a per-head sink, with K = V.
//
//   P = exp(scale q.kv - lse),  dP = dout.kv,  D = dout.out,  dS = P (dP - D)
//   dq = scale sum_k dS kv,   dkv[k] += sum_h (scale dS q + P dout),   dsink = -sum p_sink D
//
// Four kernels on the caller's stream, all one workgroup (4 wavefronts x 16 heads, or
// x 128 latent dims) per query, sharing the forward's tile machinery:
//   prep  S^T and dP^T tile by tile from one K fragment each (K = V), P and
//         scale * dS as bf16 MFMA fragments into the workspace, the key row of every
//         tile slot, the head-averaged probabilities and the per-query sink terms;
//   dq    O^T-style accumulation dq^T += K^T (scale dS)^T from the same tiles;
//   dkv   (dims x keys) = Q^T (scale dS)^T + dout^T P^T per tile, added to the float32
//         row gradients with float atomics (a row is shared by many queries);
//   sinks one reduction per head over the per-query sink terms.
#include "csa_common.h"
#include "csa_internal.h"
#include "csa_tile.h"

namespace csa {
namespace {

constexpr int kFragBytes = kWaves * 64 * 16;  // one 16-byte fragment per lane of 4 wavefronts
constexpr int kTileWs = 2 * kFragBytes;       // P and scale * dS fragments of one tile

struct BwdWorkspace {
  unsigned char* frags;  // [Tq][ntc][2][kFragBytes]
  int32_t* rows;         // [Tq][ntc][32] key row codes: window row r >= 0, compressed row c -> -1 - c
  int32_t* nkeys;        // [Tq]
  float* sink_terms;     // [Tq][64]
};

__host__ __device__ inline size_t ws_bytes(long long Tq, int ntc) {
  return static_cast<size_t>(Tq) * (static_cast<size_t>(ntc) * (kTileWs + 32 * 4) + 4 + 64 * 4);
}

__host__ __device__ inline BwdWorkspace ws_layout(void* base, long long Tq, int ntc) {
  BwdWorkspace w;
  unsigned char* p = static_cast<unsigned char*>(base);
  w.frags = p;
  p += static_cast<size_t>(Tq) * ntc * kTileWs;
  w.rows = reinterpret_cast<int32_t*>(p);
  p += static_cast<size_t>(Tq) * ntc * 32 * 4;
  w.nkeys = reinterpret_cast<int32_t*>(p);
  p += static_cast<size_t>(Tq) * 4;
  w.sink_terms = reinterpret_cast<float*>(p);
  return w;
}

// Key ranges of query i (segment search by ballot; compressed count only in
// attend-all mode, the selection mode fills it in from the compaction).
__device__ QueryKeys bwd_ranges(int i, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv,
                                const int32_t* __restrict__ cu_cmp, int B, int global_start, int r, int wl, int wr,
                                bool attend_all, int Tc) {
  const int lane = threadIdx.x & 63;
  int count = 0;
  for (int base = 0; base < B; base += 64) count += __popcll(__ballot(base + lane < B && cu_q[base + lane] <= i));
  const int b = __builtin_amdgcn_readfirstlane(count - 1);
  const int t = global_start + i;
  const int s = cu_kv[b], e = cu_kv[b + 1];
  QueryKeys k;
  k.lo = max(s, t - wl);
  k.nwin = min(e - 1, t + wr) - k.lo + 1;
  k.cmp_base = (cu_cmp != nullptr) ? cu_cmp[b] : 0;
  k.ncmp = attend_all ? max(0, min((t - s + 1) / r, min(cu_cmp[b + 1], Tc) - k.cmp_base)) : 0;
  return k;
}

// Zero-fill (a kernel, so the sequence stays capturable in a HIP graph).
__global__ void zero_f32_kernel(float* __restrict__ p, long long n) {
  for (long long k = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; k < n;
       k += static_cast<long long>(gridDim.x) * blockDim.x)
    p[k] = 0.f;
}

// Q-style B operand of S^T = K . X^T (X = q or dout): k-slot 8g + j of MFMA step ks
// stands for latent dim 32*ks + 4*g + j (j < 4) or 32*ks + 16 + 4*g + (j - 4), the
// permutation the K fragments use.
__device__ __forceinline__ void load_qstyle(const uint16_t* __restrict__ row, bf16x8 (&f)[16]) {
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const uint2 lo = *reinterpret_cast<const uint2*>(row + 32 * ks);
    const uint2 hi = *reinterpret_cast<const uint2*>(row + 32 * ks + 16);
    f[ks] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
}

// ----------------------------------------------------------------------------- prep

template <int NC>  // cmp_idx row chunks of kThreads entries
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_bwd_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ori_kv, const uint16_t* __restrict__ cmp_kv,
    const int32_t* __restrict__ cmp_idx, int topk, int Tq, int Tc, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp, int B, int global_start, int r, int wl,
    int wr, const float* __restrict__ sinks, float scale, const uint16_t* __restrict__ out,
    const float* __restrict__ lse, const uint16_t* __restrict__ dout, void* ws_base, int ntc,
    float* __restrict__ ori_l1, int W, float* __restrict__ cmp_l1, int cmp_slots) {
  __shared__ __attribute__((aligned(1024))) unsigned char kt[2 * kTileBytes];
  __shared__ int32_t crow[kMaxTopk];
  __shared__ uint32_t wsum[kWaves];
  __shared__ float l1s[2][kWaves][kNT];  // per-wavefront head sums, added in a fixed order

  const int i = static_cast<int>(blockIdx.x);
  if (i >= Tq) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int head = 16 * wave + n;
  const bool sparse = cmp_kv != nullptr && cmp_idx != nullptr;
  const BwdWorkspace ws = ws_layout(ws_base, Tq, ntc);
  const float scale_log2 = scale * kLog2e;

  int vals[NC];
  if (sparse) {
    const int32_t* row = cmp_idx + static_cast<long long>(i) * topk;
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
      const int j = ch * kThreads + tid;
      vals[ch] = (j < topk) ? row[j] : -1;
    }
  }
  const long long qoff = (static_cast<long long>(i) * 64 + head) * 512 + 4 * g;
  bf16x8 qf[16], df[16];
  load_qstyle(q + qoff, qf);
  load_qstyle(dout + qoff, df);
  // D = dout . out for this lane's head: each lane sums its 128 dims, then the quad
  float dsum = 0.f;
  {
    bf16x8 of[16];
    load_qstyle(out + qoff, of);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum += static_cast<float>(df[ks][j]) * static_cast<float>(of[ks][j]);
  }
  const float Dh = quad_sum(dsum);
  const float lse2 = lse[static_cast<long long>(i) * 64 + head] * kLog2e;

  // compressed rows past the caller's Tc are never read (nor their gradients written)
  QueryKeys qk = bwd_ranges(i, cu_q, cu_kv, cu_cmp, B, global_start, r, wl, wr, cmp_kv != nullptr && !sparse, Tc);
  if (sparse) qk.ncmp = compact_rows(vals, topk, min(cu_cmp[B], Tc), crow, wsum);
  // the workspace holds at most ntc tiles per query
  const int nkeys = min(qk.nwin + qk.ncmp, ntc * kNT);
  const int ntiles = (nkeys + kNT - 1) / kNT;
  if (tid == 0) ws.nkeys[i] = nkeys;
  if (sinks != nullptr && g == 0)
    ws.sink_terms[static_cast<long long>(i) * 64 + head] = -exp2f(sinks[head] * kLog2e - lse2) * Dh;
  const bool want_l1 = ori_l1 != nullptr || cmp_l1 != nullptr;

  const uint32_t kt_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(CSA_LDS(kt)));
  const uint32_t lane16 = static_cast<uint32_t>(lane) << 4;
  auto key_code = [&](int kidx) {
    if (kidx < qk.nwin) return qk.lo + kidx;
    const int c = (cmp_idx != nullptr) ? crow[kidx - qk.nwin] : qk.cmp_base + (kidx - qk.nwin);
    return -1 - c;
  };
  auto issue = [&](int t, int bf) {
    const int p = lane & 7;
    int kidx = t * kNT + 4 * p + wave;
    kidx = (kidx < nkeys) ? kidx : 0;
    const int code = key_code(kidx);
    const uint16_t* src = (code >= 0) ? ori_kv + static_cast<long long>(code) * 512
                                      : cmp_kv + static_cast<long long>(-1 - code) * 512;
    const unsigned long long a = reinterpret_cast<unsigned long long>(src);
    const uint32_t a_lo = static_cast<uint32_t>(a), a_hi = static_cast<uint32_t>(a >> 32);
#pragma unroll
    for (int pass = 0; pass < kNT / kWaves; ++pass) {
      const int rr = pass * kWaves + wave;
      const unsigned long long base = (static_cast<unsigned long long>(__builtin_amdgcn_readlane(a_hi, pass)) << 32) |
                                      static_cast<uint32_t>(__builtin_amdgcn_readlane(a_lo, pass));
      row_to_lds(reinterpret_cast<const void*>(base), lane16,
                 kt_base + static_cast<uint32_t>(bf * kTileBytes + rr * kRowStride));
    }
  };
  // key rows of every tile slot, for the dq and dkv passes (slots past nkeys: code of key 0)
  for (int k = tid; k < ntiles * kNT; k += kThreads)
    ws.rows[static_cast<long long>(i) * ntc * kNT + k] = key_code(k < nkeys ? k : 0);
  if (ntiles > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const int offq = kpi(n) * kRowStride + 8 * g;
  auto flush_l1 = [&](int t) {  // head-averaged probabilities of tile t
    if (tid < kNT) {
      const int kidx = t * kNT + tid;
      const float (&part)[kWaves][kNT] = l1s[t & 1];
      const float v = ((part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid])) * (1.f / 64.f);
      if (kidx < nkeys) {
        if (kidx < qk.nwin) {
          if (ori_l1 != nullptr && kidx < W) ori_l1[static_cast<long long>(i) * W + kidx] = v;
        } else if (cmp_l1 != nullptr && kidx - qk.nwin < cmp_slots) {
          cmp_l1[static_cast<long long>(i) * cmp_slots + kidx - qk.nwin] = v;
        }
      }
    }
  };

  for (int t = 0; t < ntiles; ++t) {
    const int bf = t & 1;
    // this wavefront's rows of tile t have landed and its LDS adds of tile t - 1 are done
    __builtin_amdgcn_s_waitcnt(0x0070);
    tile_barrier();  // all rows landed; buffer bf ^ 1 is free; l1s[bf ^ 1] is complete
    if (t + 1 < ntiles) issue(t + 1, bf ^ 1);
    if (want_l1 && t > 0) flush_l1(t - 1);
    const unsigned char* tb = kt + bf * kTileBytes;

    // ---- S^T = K . Q^T and dP^T = K . dout^T from the same K fragments (K = V)
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, p0 = s0, p1 = s0;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8 a0 = kfrag(tb, offq + 64 * ks, offq + 64 * ks + 32);
      const bf16x8 a1 = kfrag(tb + 16 * kRowStride, offq + 64 * ks, offq + 64 * ks + 32);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, df[ks], p0, 0, 0, 0);
      p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, df[ks], p1, 0, 0, 0);
    }

    // ---- P and scale * dS for keys kpi(4g+j) (j < 4) and 16 + kpi(4g+j-4); masked keys 0
    bf16x8 pf, sf;
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kk = (j < 4) ? kpi(4 * g + j) : 16 + kpi(4 * g + j - 4);
      const float sv = (j < 4) ? s0[j] : s1[j - 4];
      const float dp = (j < 4) ? p0[j] : p1[j - 4];
      const float p = (t * kNT + kk < nkeys) ? exp2f(sv * scale_log2 - lse2) : 0.f;
      pv[j] = p;
      pf[j] = static_cast<__bf16>(p);
      sf[j] = static_cast<__bf16>(scale * p * (dp - Dh));
    }
    {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      unsigned char* fb = ws.frags + (static_cast<long long>(i) * ntc + t) * kTileWs + wave * 1024 + lane * 16;
      *reinterpret_cast<u32x4*>(fb) = __builtin_bit_cast(u32x4, pf);
      *reinterpret_cast<u32x4*>(fb + kFragBytes) = __builtin_bit_cast(u32x4, sf);
    }
    if (want_l1) {
      // sum over the 16 heads of this wavefront (lanes n of one lane group); the
      // four wavefront sums meet in LDS
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = pv[j];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        v += __shfl_xor(v, 8, 64);
        if (n == 0) {
          const int kk = (j < 4) ? kpi(4 * g + j) : 16 + kpi(4 * g + j - 4);
          l1s[bf][wave][kk] = v;
        }
      }
    }
  }
  if (want_l1 && ntiles > 0) {
    lds_barrier();
    flush_l1(ntiles - 1);
  }
}

// ----------------------------------------------------------------------------- dq

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_bwd_dq_kernel(
    const uint16_t* __restrict__ ori_kv, const uint16_t* __restrict__ cmp_kv, int Tq, const void* ws_base, int ntc,
    uint16_t* __restrict__ dq) {
  __shared__ __attribute__((aligned(1024))) unsigned char kt[2 * kTileBytes];
  const int i = static_cast<int>(blockIdx.x);
  if (i >= Tq) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const BwdWorkspace ws = ws_layout(const_cast<void*>(ws_base), Tq, ntc);
  const int nkeys = __builtin_amdgcn_readfirstlane(ws.nkeys[i]);
  const int ntiles = (nkeys + kNT - 1) / kNT;
  const int32_t* rows = ws.rows + static_cast<long long>(i) * ntc * kNT;
  const uint32_t kt_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(CSA_LDS(kt)));
  const uint32_t lane16 = static_cast<uint32_t>(lane) << 4;
  auto issue = [&](int t, int bf) {
    const int code = rows[t * kNT + 4 * (lane & 7) + wave];
    const uint16_t* src = (code >= 0) ? ori_kv + static_cast<long long>(code) * 512
                                      : cmp_kv + static_cast<long long>(-1 - code) * 512;
    const unsigned long long a = reinterpret_cast<unsigned long long>(src);
    const uint32_t a_lo = static_cast<uint32_t>(a), a_hi = static_cast<uint32_t>(a >> 32);
#pragma unroll
    for (int pass = 0; pass < kNT / kWaves; ++pass) {
      const int rr = pass * kWaves + wave;
      const unsigned long long base = (static_cast<unsigned long long>(__builtin_amdgcn_readlane(a_hi, pass)) << 32) |
                                      static_cast<uint32_t>(__builtin_amdgcn_readlane(a_lo, pass));
      row_to_lds(reinterpret_cast<const void*>(base), lane16,
                 kt_base + static_cast<uint32_t>(bf * kTileBytes + rr * kRowStride));
    }
  };
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  auto frag = [&](int t) {  // scale * dS^T fragment of tile t for this lane
    const unsigned char* fb =
        ws.frags + (static_cast<long long>(i) * ntc + t) * kTileWs + kFragBytes + wave * 1024 + lane * 16;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(fb));
  };
  if (ntiles > 0) issue(0, 0);
  bf16x8 sf = (ntiles > 0) ? frag(0) : bf16x8{};
  __builtin_amdgcn_s_waitcnt(0x0F70);
  f32x4 o[32];
#pragma unroll
  for (int mb = 0; mb < 32; ++mb) o[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int offv = kpi(4 * g + (n >> 2)) * kRowStride + 8 * (n & 3);
  for (int t = 0; t < ntiles; ++t) {
    const int bf = t & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    tile_barrier();
    bf16x8 sf_next = sf;
    if (t + 1 < ntiles) {
      issue(t + 1, bf ^ 1);
      sf_next = frag(t + 1);
    }
    const unsigned char* tb = kt + bf * kTileBytes;
    bf16x4 vlo[4], vhi[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      vlo[mb] = ds_read_tr(tb + offv + 32 * mb);
      vhi[mb] = ds_read_tr(tb + offv + 32 * mb + 16 * kRowStride);
    }
#pragma unroll
    for (int mb = 0; mb < 32; ++mb) {
      const int sl = mb % 4;
      const bf16x8 a = {vlo[sl][0], vlo[sl][1], vlo[sl][2], vlo[sl][3],
                        vhi[sl][0], vhi[sl][1], vhi[sl][2], vhi[sl][3]};
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, sf, o[mb], 0, 0, 0);
      if (mb + 4 < 32) {
        vlo[sl] = ds_read_tr(tb + offv + 32 * (mb + 4));
        vhi[sl] = ds_read_tr(tb + offv + 32 * (mb + 4) + 16 * kRowStride);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sf = sf_next;
  }
  // dq^T column (head 16w + n), dims 16 mb + 4 g + j; rows of 8 bytes per lane
  uint16_t* qrow = dq + (static_cast<long long>(i) * 64 + 16 * wave + n) * 512 + 4 * g;
#pragma unroll
  for (int mb = 0; mb < 32; ++mb) {
    const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16_bits(o[mb][0])) |
                        (static_cast<uint32_t>(f32_to_bf16_bits(o[mb][1])) << 16);
    const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16_bits(o[mb][2])) |
                        (static_cast<uint32_t>(f32_to_bf16_bits(o[mb][3])) << 16);
    *reinterpret_cast<uint2*>(qrow + 16 * mb) = make_uint2(w0, w1);
  }
}

// ----------------------------------------------------------------------------- dkv

// Per query, per tile: C[keys x dims] = (scale dS)[keys x heads] . q[heads x dims]
// + P[keys x heads] . dout[heads x dims], wavefront w owning dims [128w, 128w+128).
// MFMA k-slots run over heads: k-slot 8g + j of a 32-head half hh stands for head
// 32 hh + 4 g + j (j < 4) or 32 hh + 16 + 4 g + (j - 4).  The q / dout B operands come
// from transpose reads of the query's rows staged once in LDS; the dS / P A operands
// from the tile's fragments regrouped through LDS as [key][head].
constexpr int kQStride = 1040;  // staged q / dout rows (64 heads), padded like the tiles
constexpr int kKH = 64 * 2 + 16; // staged [key][head] bf16 row, padded

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, int Tq, const void* ws_base, int ntc,
    float* __restrict__ d_ori, float* __restrict__ d_cmp) {
  __shared__ __attribute__((aligned(1024))) unsigned char qs[64 * kQStride];
  __shared__ __attribute__((aligned(16))) unsigned char kh[2][kNT * kKH];  // [P, scale dS][key][head]
  const int i = static_cast<int>(blockIdx.x);
  if (i >= Tq) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const BwdWorkspace ws = ws_layout(const_cast<void*>(ws_base), Tq, ntc);
  const int nkeys = __builtin_amdgcn_readfirstlane(ws.nkeys[i]);
  const int ntiles = (nkeys + kNT - 1) / kNT;
  if (ntiles == 0) return;
  const int32_t* rows = ws.rows + static_cast<long long>(i) * ntc * kNT;

  // B operands, constant per query: for dim block db (dims 128w + 16db ..) and head
  // half hh, lane (n, g) holds X[heads of k-slots 8g..8g+7][dim 128w + 16db + n].
  bf16x8 qb[8][2], db_[8][2];
  auto stage_rows = [&](const uint16_t* __restrict__ src) {
    // 64 head rows of 1 KiB: thread tid copies 16-byte chunks
    for (int k = tid; k < 64 * 64; k += kThreads) {
      const int h = k >> 6, c = k & 63;
      *reinterpret_cast<uint4*>(qs + h * kQStride + c * 16) =
          *reinterpret_cast<const uint4*>(src + (static_cast<long long>(i) * 64 + h) * 512 + c * 8);
    }
  };
  auto read_b = [&](bf16x8 (&b)[8][2]) {
    const int rlo = 4 * g + (n >> 2);
    const int coff = 2 * (128 * wave) + 8 * (n & 3);
#pragma unroll
    for (int d8 = 0; d8 < 8; ++d8)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const unsigned char* p = qs + (32 * hh + rlo) * kQStride + coff + 32 * d8;
        const bf16x4 lo = ds_read_tr(p);
        const bf16x4 hi = ds_read_tr(p + 16 * kQStride);
        b[d8][hh] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
  };
  stage_rows(q);
  __syncthreads();
  read_b(qb);
  __syncthreads();
  stage_rows(dout);
  __syncthreads();
  read_b(db_);

  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  for (int t = 0; t < ntiles; ++t) {
    // regroup the tile's P and scale * dS fragments as [key][head]: wavefront w takes the
    // fragments of head block w (lane (n, g): head 16w + n, keys kpi(4g+j), 16 + kpi(4g+j))
    __syncthreads();  // previous tile's reads of kh are done
    {
      const unsigned char* fb = ws.frags + (static_cast<long long>(i) * ntc + t) * kTileWs + wave * 1024 + lane * 16;
      const bf16x8 pf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(fb));
      const bf16x8 sf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(fb + kFragBytes));
      const int h = 16 * wave + n;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = (j < 4) ? kpi(4 * g + j) : 16 + kpi(4 * g + j - 4);
        *reinterpret_cast<__bf16*>(kh[0] + kk * kKH + 2 * h) = pf[j];
        *reinterpret_cast<__bf16*>(kh[1] + kk * kKH + 2 * h) = sf[j];
      }
    }
    __syncthreads();
    int code[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) code[kb][j] = rows[t * kNT + 16 * kb + 4 * g + j];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // A operands: key 16 kb + n, heads of the k-slot order, two 8-byte reads each
      bf16x8 ap[2], as[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int o_lo = (16 * kb + n) * kKH + 2 * (32 * hh + 4 * g);
        const int o_hi = o_lo + 2 * 16;
        ap[hh] = kfrag(kh[0], o_lo, o_hi);
        as[hh] = kfrag(kh[1], o_lo, o_hi);
      }
#pragma unroll
      for (int d8 = 0; d8 < 8; ++d8) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as[hh], qb[d8][hh], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap[hh], db_[d8][hh], c, 0, 0, 0);
        }
        // C layout: lane (n, g) holds keys 16 kb + 4 g + j, dim 128w + 16 d8 + n
        const int dim = 128 * wave + 16 * d8 + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (t * kNT + 16 * kb + 4 * g + j >= nkeys) continue;
          const int cd = code[kb][j];
          float* dst = (cd >= 0) ? d_ori + static_cast<long long>(cd) * 512 + dim
                                 : d_cmp + static_cast<long long>(-1 - cd) * 512 + dim;
          atomicAdd(dst, c[j]);
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------- sinks

__global__ __launch_bounds__(kThreads) void mla_bwd_sink_kernel(const void* ws_base, int Tq, int ntc,
                                                                float* __restrict__ d_sinks) {
  __shared__ float part[kThreads];
  const BwdWorkspace ws = ws_layout(const_cast<void*>(ws_base), Tq, ntc);
  const int h = static_cast<int>(blockIdx.x);
  float s = 0.f;
  for (int k = threadIdx.x; k < Tq; k += kThreads) s += ws.sink_terms[static_cast<long long>(k) * 64 + h];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (static_cast<int>(threadIdx.x) < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) d_sinks[h] = part[0];
}

void zero(float* p, long long n, hipStream_t s) {
  if (p == nullptr || n <= 0) return;
  const unsigned blocks = static_cast<unsigned>(min(4096LL, (n + 255) / 256));
  hipLaunchKernelGGL(zero_f32_kernel, dim3(blocks), dim3(256), 0, s, p, n);
}

}  // namespace

bool mla_bwd_shape_supported(int H, int d, int dtype) { return dtype == 1 && H == 64 && d == 512; }

int mla_bwd_tiles_cap(int key_cap) { return (key_cap + kNT - 1) / kNT; }

size_t mla_bwd_workspace_bytes(int Tq, int key_cap) {
  return ws_bytes(Tq, mla_bwd_tiles_cap(key_cap));
}

hipError_t launch_sparse_mla_bwd(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx,
                                 int topk, int Tq, int Tkv, int Tc, const int32_t* cu_q, const int32_t* cu_kv,
                                 const int32_t* cu_cmp, int B, int global_start, int r, int wl, int wr,
                                 const float* sinks, float scale, const void* out, const float* lse,
                                 const void* dout, void* dq, float* d_ori, float* d_cmp, float* d_sinks,
                                 float* ori_l1, float* cmp_l1, int cmp_slots, int key_cap, void* workspace,
                                 hipStream_t s) {
  const int W = wl + wr + 1;
  zero(d_ori, static_cast<long long>(Tkv) * 512, s);
  zero(d_cmp, static_cast<long long>(Tc) * 512, s);
  zero(ori_l1, static_cast<long long>(Tq) * W, s);
  zero(cmp_l1, static_cast<long long>(Tq) * cmp_slots, s);
  if (d_sinks != nullptr && (Tq == 0 || sinks == nullptr)) zero(d_sinks, 64, s);
  if (Tq <= 0) return hipGetLastError();
  if (cmp_idx == nullptr) topk = 0;
  const int ntc = mla_bwd_tiles_cap(key_cap);
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* kv16 = static_cast<const uint16_t*>(ori_kv);
  const auto* c16 = static_cast<const uint16_t*>(cmp_kv);
  auto prep = (topk <= 2 * kThreads) ? mla_bwd_prep_kernel<2> : mla_bwd_prep_kernel<kMaxTopk / kThreads>;
  hipLaunchKernelGGL(prep, dim3(Tq), dim3(kThreads), 0, s, q16, kv16, c16, cmp_idx, topk, Tq, Tc, cu_q, cu_kv, cu_cmp,
                     B, global_start, r, wl, wr, sinks, scale, static_cast<const uint16_t*>(out), lse,
                     static_cast<const uint16_t*>(dout), workspace, ntc, ori_l1, W, cmp_l1, cmp_slots);
  hipLaunchKernelGGL(mla_bwd_dq_kernel, dim3(Tq), dim3(kThreads), 0, s, kv16, c16, Tq,
                     static_cast<const void*>(workspace), ntc, static_cast<uint16_t*>(dq));
  hipLaunchKernelGGL(mla_bwd_dkv_kernel, dim3(Tq), dim3(kThreads), 0, s, q16, static_cast<const uint16_t*>(dout),
                     Tq, static_cast<const void*>(workspace), ntc, d_ori, d_cmp);
  if (d_sinks != nullptr && sinks != nullptr)
    hipLaunchKernelGGL(mla_bwd_sink_kernel, dim3(64), dim3(kThreads), 0, s, static_cast<const void*>(workspace), Tq,
                       ntc, d_sinks);
  return hipGetLastError();
}

}  // namespace csa
