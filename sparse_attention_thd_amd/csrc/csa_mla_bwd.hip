// Sparse MLA backward, (H, d) = (64, 512) bf16: the exact gradients of the forward's
// joint softmax over window rows, compressed rows and a per-head sink, with K = V.
//
//   P = exp(scale q.kv - lse),  dP = dout.kv,  D = dout.out,  dS = P (dP - D)
//   dq = scale sum_k dS kv,   dkv[k] += sum_h (scale dS q + P dout),   dsink = -sum p_sink D
//
// Kernels on the caller's stream:
//   prep  query-major (one workgroup of 4 wavefronts x 16 heads per query): S and dP
//         tile by tile from one kv fragment each (K = V) against the query's q and dout
//         held in registers; writes scale * dS and P of every (query, key) pair as a
//         256-byte slot row (64 heads each, bf16), the key row of every slot, the
//         head-averaged probabilities and the per-query sink terms;
//   dq    query-major: dq^T += kv^T (scale dS)^T per tile, kv and the dS rows staged in
//         LDS;
//   dkv   key-major: a workgroup owns 128 keys (window rows or compressed rows of one
//         segment) x 256 latent dims and sweeps up to 128 queries, accumulating
//         C[keys x dims] += [scale dS | P][keys x (head, term)] . [q ; dout] in
//         registers (32x32x16 MFMAs), then adds C to the float32 row gradients.  Only
//         the query chunks of one key tile meet in the atomics, so the row gradients
//         take a few float atomics per element instead of one per (query, key) pair;
//   sinks one reduction per head over the per-query sink terms.
#include "csa_common.h"
#include "csa_internal.h"
#include "csa_tile.h"

namespace csa {
namespace {

constexpr int kSlotBytes = 256;  // scale * dS (bytes 0..127) then P (128..255), 64 heads bf16 each
constexpr int kDsStride = 144;   // staged dS row of the dq pass (128 bytes + pad)
// row-gradient (dkv) pass
constexpr int kGK = 256;                // keys per tile
constexpr int kQCH = 128;               // queries per chunk
constexpr int kDkvThreads = 512;        // 8 wavefronts
constexpr int kYRow = 512;              // staged q or dout row: 256 dims
constexpr int kYChunk = 64 * kYRow;     // one term's 64 head rows of one query
constexpr int kAChunk = kGK * 128;      // one term's 64 heads of the tile's keys
constexpr int kStage = kYChunk + kAChunk;  // one (query, term) stage: 64 KiB

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct BwdWorkspace {
  unsigned char* slots;  // [Tq][nslot][kSlotBytes]
  float* sink_terms;     // [Tq][64]
  int32_t* nkeys;        // [Tq]
  int16_t* cmap;         // [Tq][nvis_cap] compacted index of each visible compressed row, -1 if not selected
  unsigned char* zero;   // one slot row of zeros (the A rows of keys a query does not attend)
};

__host__ __device__ inline size_t ws_bytes(long long Tq, int nslot, int nvis_cap) {
  const size_t head = static_cast<size_t>(Tq) *
                      (static_cast<size_t>(nslot) * kSlotBytes + 64 * 4 + 4 + static_cast<size_t>(nvis_cap) * 2);
  return (head + 15) / 16 * 16 + kSlotBytes;  // + one zero slot row
}

__host__ __device__ inline BwdWorkspace ws_layout(void* base, long long Tq, int nslot, int nvis_cap) {
  BwdWorkspace w;
  unsigned char* p = static_cast<unsigned char*>(base);
  w.slots = p;
  p += static_cast<size_t>(Tq) * nslot * kSlotBytes;
  w.sink_terms = reinterpret_cast<float*>(p);
  p += static_cast<size_t>(Tq) * 64 * 4;
  w.nkeys = reinterpret_cast<int32_t*>(p);
  p += static_cast<size_t>(Tq) * 4;
  w.cmap = reinterpret_cast<int16_t*>(p);
  w.zero = static_cast<unsigned char*>(base) + ws_bytes(Tq, nslot, nvis_cap) - kSlotBytes;
  return w;
}

struct BwdKeys {
  int b, s, e;   // segment and its stream rows [s, e)
  int lo, nwin;  // window rows lo .. lo + nwin - 1
  int cmp_base;  // first compressed row of the segment
  int nvis;      // causally complete compressed rows of the segment (below Tc)
  int ncmp;      // attended compressed rows
};

// Key ranges of local query i (segment search by ballot).  Window sides are clamped
// to Tkv by the launcher, so t + wr cannot overflow.
__device__ BwdKeys bwd_ranges(int i, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv,
                              const int32_t* __restrict__ cu_cmp, int B, int global_start, int r, int wl, int wr,
                              bool attend_all, int Tc) {
  const int lane = threadIdx.x & 63;
  int count = 0;
  for (int base = 0; base < B; base += 64) count += __popcll(__ballot(base + lane < B && cu_q[base + lane] <= i));
  BwdKeys k;
  k.b = __builtin_amdgcn_readfirstlane(count - 1);
  const int t = global_start + i;
  k.s = cu_kv[k.b];
  k.e = cu_kv[k.b + 1];
  k.lo = max(k.s, t - wl);
  k.nwin = min(k.e - 1, t + wr) - k.lo + 1;
  k.cmp_base = 0;
  k.nvis = 0;
  if (cu_cmp != nullptr) {
    k.cmp_base = cu_cmp[k.b];
    k.nvis = max(0, min((t - k.s + 1) / r, min(cu_cmp[k.b + 1], Tc) - k.cmp_base));
  }
  k.ncmp = attend_all ? k.nvis : 0;
  return k;
}

// Zero-fill (a kernel, so the sequence stays capturable in a HIP graph).
__global__ void zero_f32_kernel(float* __restrict__ p, long long n) {
  for (long long k = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; k < n;
       k += static_cast<long long>(gridDim.x) * blockDim.x)
    p[k] = 0.f;
}

// dout fragments of one head row in the kv fragments' k-slot order (k-slot 8 g + j of MFMA
// step ks is latent dim 32 ks + 4 g + j for j < 4, 32 ks + 16 + 4 g + (j - 4) for j >= 4),
// and D = dout . out of that row.  Split into four-dim groups G0..G7, block ks holds the
// slots (G_g, G_g+4) of lane group g.  Lane group g loads the 16-byte chunk
// ((g & 1) << 1) | (g >> 1) of every block (whole 64-byte runs of the row per instruction;
// 8-byte pieces measured 8% slower per query), so groups 0..3 hold (G0 G1), (G4 G5),
// (G2 G3), (G6 G7); one permlane16_swap of the second pair of groups 0, 2 with the first
// pair of groups 1, 3 leaves (G0 G4), (G1 G5), (G2 G6), (G3 G7).  D is summed from the
// loaded pieces (each lane 128 dims, then the lane quad).
__device__ __forceinline__ float load_dout_frags(const uint16_t* __restrict__ drow, const uint16_t* __restrict__ orow,
                                                 bf16x8 (&f)[16]) {
  const int g = (threadIdx.x & 63) >> 4;
  const int c = ((g & 1) << 1) | (g >> 1);
  const u32x4* dp = reinterpret_cast<const u32x4*>(drow) + c;
  const u32x4* op = reinterpret_cast<const u32x4*>(orow) + c;
  u32x4 dv[16], ov[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    dv[ks] = dp[4 * ks];
    ov[ks] = op[4 * ks];
  }
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = dv[ks][e], y = ov[ks][e];
      dsum += __uint_as_float(x << 16) * __uint_as_float(y << 16);
      dsum += __uint_as_float(x & 0xffff0000u) * __uint_as_float(y & 0xffff0000u);
    }
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const auto a = __builtin_amdgcn_permlane16_swap(dv[ks][0], dv[ks][2], false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(dv[ks][1], dv[ks][3], false, false);
    f[ks] = __builtin_bit_cast(bf16x8, u32x4{a[0], b[0], a[1], b[1]});
  }
  return quad_sum(dsum);
}

// ----------------------------------------------------------------------------- prep + dq

constexpr int kPrepThreads = 512;  // wavefronts 0-3: S and dP; 4-7: the dq product

// One workgroup per query, 8 wavefronts sharing the query's kv tiles in LDS.  Wavefront w
// (w < 4) forms S and dP for heads 16 w .. 16 w + 15 from q and dout held in registers,
// writes scale * dS and P of every (query, key) pair as a 256-byte slot row, the
// tile's dS rows to LDS and the head-averaged probabilities; wavefront 4 + w multiplies
// those dS rows into dq for the same heads one tile later.  Each SIMD thus runs one
// wavefront of each kind.
template <int NC>  // cmp_idx row chunks of kThreads entries
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_bwd_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ori_kv, const uint16_t* __restrict__ cmp_kv,
    const int32_t* __restrict__ cmp_idx, int topk, int Tq, int Tc, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp, int B, int global_start, int r, int wl,
    int wr, const float* __restrict__ sinks, float scale, const uint16_t* __restrict__ out,
    const float* __restrict__ lse, const uint16_t* __restrict__ dout, void* ws_base, int nslot, int nvis_cap,
    float* __restrict__ ori_l1, int W, float* __restrict__ cmp_l1, int cmp_slots, uint16_t* __restrict__ dq) {
  // three kv tiles in flight: tile t is multiplied into S and dP while tile t - 1 finishes
  // its dq product and tile t + 1 loads
  __shared__ __attribute__((aligned(1024))) unsigned char kt[3 * kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char dsb[2][kNT * kDsStride];  // scale dS [key][head]
  __shared__ int32_t crow[kMaxTopk];
  __shared__ uint32_t wsum[2 * kWaves];
  __shared__ float l1s[2][kWaves][kNT];  // per-wavefront head sums, added in a fixed order

  // Workgroups are dealt round-robin to the 8 XCDs; each XCD takes runs of 8
  // consecutive queries, which share window and compressed rows in its L2.
  const int kx = static_cast<int>(blockIdx.x >> 3);
  const int i = ((kx >> 3) * 8 + static_cast<int>(blockIdx.x & 7u)) * 8 + (kx & 7);
  if (i >= Tq) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool s_wave = wave8 < kWaves;
  const int wave = wave8 & (kWaves - 1);  // head block of this wavefront
  const int n = lane & 15, g = lane >> 4;
  const int head = 16 * wave + n;
  const bool sparse = cmp_kv != nullptr && cmp_idx != nullptr;
  const BwdWorkspace ws = ws_layout(ws_base, Tq, nslot, nvis_cap);
  const float scale_log2 = scale * kLog2e;

  int vals[NC];
#pragma unroll
  for (int ch = 0; ch < NC; ++ch) vals[ch] = -1;
  if (sparse && s_wave) {
    const int32_t* row = cmp_idx + static_cast<long long>(i) * topk;
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
      const int j = ch * kThreads + tid;
      vals[ch] = (j < topk) ? row[j] : -1;
    }
  }

  BwdKeys qk = bwd_ranges(i, cu_q, cu_kv, cu_cmp, B, global_start, r, wl, wr, cmp_kv != nullptr && !sparse, Tc);
  // compressed rows past the caller's Tc are never read (nor their gradients written);
  // every wavefront takes part in the compaction's barriers, the dq ones with no entries
  if (sparse) qk.ncmp = compact_rows(vals, topk, min(cu_cmp[B], Tc), crow, wsum);
  const int nkeys = min(qk.nwin + qk.ncmp, nslot);  // the workspace holds nslot keys per query
  const int ntiles = (nkeys + kNT - 1) / kNT;
  if (tid == 0) ws.nkeys[i] = nkeys;
  if (i == 0 && tid < kSlotBytes / 16) reinterpret_cast<u32x4*>(ws.zero)[tid] = u32x4{0u, 0u, 0u, 0u};
  // Map of the visible compressed rows for the key-major dkv pass (sparse mode): the
  // compacted index of each selected row, -1 elsewhere.
  if (sparse && nvis_cap > 0) {
    int16_t* m = ws.cmap + static_cast<long long>(i) * nvis_cap;
    const int nv = min(qk.nvis, nvis_cap);
    for (int v = tid; v < nv; v += kPrepThreads) m[v] = -1;
    __syncthreads();  // the -1 fill lands before the entries below
    for (int j = tid; j < qk.ncmp; j += kPrepThreads) {
      const int v = crow[j] - qk.cmp_base;
      if (v >= 0 && v < nv && qk.nwin + j < nslot) m[v] = static_cast<int16_t>(j);
    }
  }
  const bool want_l1 = ori_l1 != nullptr || cmp_l1 != nullptr;

  const uint32_t kt_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(CSA_LDS(kt)));
  const uint32_t lane16 = static_cast<uint32_t>(lane) << 4;
  auto key_code = [&](int kidx) {
    if (kidx < qk.nwin) return qk.lo + kidx;
    const int c = (cmp_idx != nullptr) ? crow[kidx - qk.nwin] : qk.cmp_base + (kidx - qk.nwin);
    return -1 - c;
  };
  // tile t into kv buffer bf: wavefront w8 loads rows 8 pass + w8 (pass < 4)
  auto issue = [&](int t, int bf) {
    int kidx = t * kNT + 8 * (lane & 3) + wave8;
    kidx = (kidx < nkeys) ? kidx : 0;
    const int code = key_code(kidx);
    const uint16_t* src = (code >= 0) ? ori_kv + static_cast<long long>(code) * 512
                                      : cmp_kv + static_cast<long long>(-1 - code) * 512;
    const unsigned long long a = reinterpret_cast<unsigned long long>(src);
    const uint32_t a_lo = static_cast<uint32_t>(a), a_hi = static_cast<uint32_t>(a >> 32);
#pragma unroll
    for (int pass = 0; pass < kNT / 8; ++pass) {
      const int rr = 8 * pass + wave8;
      const unsigned long long base = (static_cast<unsigned long long>(__builtin_amdgcn_readlane(a_hi, pass)) << 32) |
                                      static_cast<uint32_t>(__builtin_amdgcn_readlane(a_lo, pass));
      row_to_lds(reinterpret_cast<const void*>(base), lane16,
                 kt_base + static_cast<uint32_t>(bf * kTileBytes + rr * kRowStride));
    }
  };
  // The query's 64 q rows (64 KiB, contiguous) arrive as whole 1 KiB rows in kv buffers
  // 1 and 2 (idle until the loop's first barrier), one global_load_lds_dwordx4 per row
  // (wavefront w8: rows 8 w8 .. 8 w8 + 7), issued before tile 0 so that vmcnt(4) covers
  // them; the S wavefronts read their fragments from there.
  {
    const uint16_t* qsrc = q + (static_cast<long long>(i) * 64 + 8 * wave8) * 512;
#pragma unroll
    for (int hh = 0; hh < 8; ++hh)
      row_to_lds(qsrc + hh * 512, lane16, kt_base + static_cast<uint32_t>(kTileBytes + (8 * wave8 + hh) * kRowStride));
  }
  if (ntiles > 0) issue(0, 0);
  if (ntiles > 0) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4): only tile 0 may be in flight
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  tile_barrier();  // every wavefront's q rows have landed

  if (s_wave) {
    const long long hrow = (static_cast<long long>(i) * 64 + head) * 512;
    bf16x8 qf[16], df[16];
    {
      const unsigned char* qb = kt + kTileBytes + head * kRowStride + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[ks] = kfrag(qb, 64 * ks, 64 * ks + 32);
    }
    const float Dh = load_dout_frags(dout + hrow, out + hrow, df);  // D = dout . out of head 16 wave + n
    const float lse2_h = lse[static_cast<long long>(i) * 64 + head] * kLog2e;
    if (sinks != nullptr && g == 0)
      ws.sink_terms[static_cast<long long>(i) * 64 + head] = -exp2f(sinks[head] * kLog2e - lse2_h) * Dh;
    // The S tiles (heads x keys) give lane (n, g) the heads 16 wave + 4 g + j.
    float lse2[4], Dq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lse2[j] = __shfl(lse2_h, 4 * g + j, 64);
      Dq[j] = __shfl(Dh, 4 * g + j, 64);
    }
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
    unsigned char* slot_base = ws.slots + static_cast<long long>(i) * nslot * kSlotBytes + 2 * (16 * wave + 4 * g);

    for (int t = 0; t < ntiles; ++t) {
      const int bf = t & 1;
      // This wavefront's rows of tile t have landed and its LDS writes of tile t - 1 are
      // done.  Vector memory operations retire in issue order and the last four issued
      // are the slot-row stores of tile t - 1 (after the loads of tile t), so those may
      // stay in flight: vmcnt(4), lgkmcnt(0).
      __builtin_amdgcn_s_waitcnt(0x0074);
      tile_barrier();  // all rows landed; kv buffer (t + 1) % 3 and dS buffer bf are free
      if (t + 1 < ntiles) issue(t + 1, (t + 1) % 3);
      if (want_l1 && t > 0) flush_l1(t - 1);
      const unsigned char* tb = kt + (t % 3) * kTileBytes;

      // ---- S = Q . K^T and dP = dout . K^T (heads x keys) from the same K fragments (K = V)
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, p0 = s0, p1 = s0;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const bf16x8 a0 = kfrag(tb, offq + 64 * ks, offq + 64 * ks + 32);
        const bf16x8 a1 = kfrag(tb + 16 * kRowStride, offq + 64 * ks, offq + 64 * ks + 32);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], a0, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], a1, s1, 0, 0, 0);
        p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(df[ks], a0, p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(df[ks], a1, p1, 0, 0, 0);
      }

      // ---- lane (n, g): keys kpi(n) and 16 + kpi(n) of the tile, heads 16 wave + 4 g + j
      const int k0 = kpi(n), k1 = 16 + kpi(n);
      const bool v0 = t * kNT + k0 < nkeys, v1 = t * kNT + k1 < nkeys;
      bf16x4 P0, P1, S0, S1;
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // v_exp_f32 directly: exponents are <= 0 here, and results below 2^-126 (flushed
        // to zero) are far under the bf16 rounding of P
        const float pa = v0 ? __builtin_amdgcn_exp2f(__builtin_fmaf(s0[j], scale_log2, -lse2[j])) : 0.f;
        const float pb = v1 ? __builtin_amdgcn_exp2f(__builtin_fmaf(s1[j], scale_log2, -lse2[j])) : 0.f;
        P0[j] = static_cast<__bf16>(pa);
        P1[j] = static_cast<__bf16>(pb);
        S0[j] = static_cast<__bf16>(scale * pa * (p0[j] - Dq[j]));
        S1[j] = static_cast<__bf16>(scale * pb * (p1[j] - Dq[j]));
        l0 += pa;
        l1 += pb;
      }
      unsigned char* row0 = slot_base + static_cast<long long>(t * kNT + k0) * kSlotBytes;
      unsigned char* row1 = slot_base + static_cast<long long>(t * kNT + k1) * kSlotBytes;
      *reinterpret_cast<uint2*>(row0) = __builtin_bit_cast(uint2, S0);
      *reinterpret_cast<uint2*>(row0 + 128) = __builtin_bit_cast(uint2, P0);
      *reinterpret_cast<uint2*>(row1) = __builtin_bit_cast(uint2, S1);
      *reinterpret_cast<uint2*>(row1 + 128) = __builtin_bit_cast(uint2, P1);
      *reinterpret_cast<uint2*>(dsb[bf] + k0 * kDsStride + 2 * (16 * wave + 4 * g)) = __builtin_bit_cast(uint2, S0);
      *reinterpret_cast<uint2*>(dsb[bf] + k1 * kDsStride + 2 * (16 * wave + 4 * g)) = __builtin_bit_cast(uint2, S1);
      if (want_l1) {
        // sum over the 16 heads of this wavefront (4 per lane, then the lane quad); the
        // four wavefront sums meet in LDS
        l0 = quad_sum(l0);
        l1 = quad_sum(l1);
        if (g == 0) {
          l1s[bf][wave][k0] = l0;
          l1s[bf][wave][k1] = l1;
        }
      }
    }
    if (ntiles > 0) {
      lds_barrier();  // pairs with the dq wavefronts' last barrier
      if (want_l1) flush_l1(ntiles - 1);
      lds_barrier();  // pairs with the dq wavefronts' staging barrier
    }
  } else {
    // dq^T (dims x heads) += kv^T . (scale dS)^T per tile, split by latent dims: wavefront
    // 4 + w accumulates dims [128 w, 128 w + 128) of all 64 heads, so each kv element is
    // read from LDS once per workgroup.  The A operand comes from transpose reads of the kv
    // tile (lane (n, g): dim 128 w + 16 mb + n, keys kpi(4 g + j) and 16 + kpi(4 g + j)),
    // the B operands from transpose reads of the tile's dS rows (source lane m of lane
    // group g points at key kpi(4 g + m / 4), heads 16 hb + 4 (m % 4) ..).
    f32x4 o[32];  // o[8 hb + mb]: heads 16 hb + n, dims 128 w + 16 mb + 4 g + j
#pragma unroll
    for (int k = 0; k < 32; ++k) o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int offv = kpi(4 * g + (n >> 2)) * kRowStride + 8 * (n & 3) + 256 * wave;
    const int dso = kpi(4 * g + (n >> 2)) * kDsStride + 8 * (n & 3);
    auto dq_tile = [&](int t) {
      const unsigned char* tb = kt + (t % 3) * kTileBytes;
      const unsigned char* dsr = dsb[t & 1];
      bf16x8 sf[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const bf16x4 slo = ds_read_tr(dsr + dso + 32 * hb);
        const bf16x4 shi = ds_read_tr(dsr + dso + 32 * hb + 16 * kDsStride);
        sf[hb] = bf16x8{slo[0], slo[1], slo[2], slo[3], shi[0], shi[1], shi[2], shi[3]};
      }
      bf16x4 vlo[2], vhi[2];
      vlo[0] = ds_read_tr(tb + offv);
      vhi[0] = ds_read_tr(tb + offv + 16 * kRowStride);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const int sl = mb & 1;
        if (mb + 1 < 8) {
          vlo[sl ^ 1] = ds_read_tr(tb + offv + 32 * (mb + 1));
          vhi[sl ^ 1] = ds_read_tr(tb + offv + 32 * (mb + 1) + 16 * kRowStride);
        }
        const bf16x8 av = {vlo[sl][0], vlo[sl][1], vlo[sl][2], vlo[sl][3],
                           vhi[sl][0], vhi[sl][1], vhi[sl][2], vhi[sl][3]};
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          o[8 * hb + mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, sf[hb], o[8 * hb + mb], 0, 0, 0);
      }
    };
    for (int t = 0; t < ntiles; ++t) {
      __builtin_amdgcn_s_waitcnt(0x0070);
      tile_barrier();  // tile t landed; the dS rows of tile t - 1 are complete
      if (t + 1 < ntiles) issue(t + 1, (t + 1) % 3);
      if (t > 0) dq_tile(t - 1);
    }
    if (ntiles > 0) {
      lds_barrier();  // the dS rows of the last tile
      dq_tile(ntiles - 1);
    }
    // The rows leave whole: every dq wavefront writes its dims of all 64 head rows
    // (padded, conflict-free 8-byte writes) into two kv buffers nobody reads any more (not
    // the last tile's; no load is in flight), rows 0..31 in buffer ntiles % 3 and 32..63
    // in the next; after a barrier each stores 16 whole rows, one 1 KiB row per
    // instruction.  With no tile at all the q rows may still sit in buffers 1 and 2, so
    // that case stores its (zero) rows directly.
    auto pack = [&](int k) {
      const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16_bits(o[k][0])) |
                          (static_cast<uint32_t>(f32_to_bf16_bits(o[k][1])) << 16);
      const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16_bits(o[k][2])) |
                          (static_cast<uint32_t>(f32_to_bf16_bits(o[k][3])) << 16);
      return make_uint2(w0, w1);
    };
    if (ntiles == 0) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        uint16_t* qrow = dq + (static_cast<long long>(i) * 64 + 16 * hb + n) * 512 + 128 * wave + 4 * g;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<uint2*>(qrow + 16 * mb) = pack(8 * hb + mb);
      }
    } else {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        unsigned char* sb = kt + ((ntiles + (hb >> 1)) % 3) * kTileBytes + (16 * (hb & 1) + n) * kRowStride +
                            256 * wave + 8 * g;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<uint2*>(sb + 32 * mb) = pack(8 * hb + mb);
      }
      lds_barrier();  // every dq wavefront's dims are staged (pairs with the S wavefronts' last barrier)
      const unsigned char* st = kt + ((ntiles + (wave >> 1)) % 3) * kTileBytes + (16 * (wave & 1)) * kRowStride;
      uint16_t* obase = dq + (static_cast<long long>(i) * 64 + 16 * wave) * 512 + 8 * lane;
#pragma unroll
      for (int hh = 0; hh < 16; ++hh)
        *reinterpret_cast<uint4*>(obase + hh * 512) = *reinterpret_cast<const uint4*>(st + hh * kRowStride + 16 * lane);
    }
  }
}

// ----------------------------------------------------------------------------- dkv

// Work items.  The queries of a segment are cut into chunks of 128; a chunk's group
// holds the window tiles (256 latent rows from the first row its queries see) and the
// compressed tiles (256 rows) visible to its last query, each in two dims halves.  All
// items of a group stream the same q / dout rows, so a group takes consecutive
// workgroup slots on one XCD.
struct ChunkGroup {
  int T0, T1;  // stream rows of the chunk's first and last query
  int k_lo;    // first window row of the chunk
  int k_hi;    // last window row of the chunk
  int n_w;     // window tiles k_lo + 256 j
  int n_c;     // compressed tiles 0 .. n_c - 1
};

__device__ __forceinline__ ChunkGroup chunk_group(int b, int c, const int32_t* __restrict__ cu_q,
                                                  const int32_t* __restrict__ cu_kv,
                                                  const int32_t* __restrict__ cu_cmp, int global_start, int r,
                                                  int wl, int wr, int Tc) {
  ChunkGroup gr;
  const int s = cu_kv[b], e = cu_kv[b + 1];
  const int qa = cu_q[b], qb = cu_q[b + 1];
  gr.T0 = global_start + qa + kQCH * c;
  gr.T1 = global_start + min(qb, qa + kQCH * (c + 1)) - 1;
  gr.k_lo = max(s, gr.T0 - wl);
  gr.k_hi = min(e - 1, gr.T1 + wr);
  gr.n_w = (gr.k_lo <= gr.k_hi) ? (gr.k_hi - gr.k_lo) / kGK + 1 : 0;
  gr.n_c = 0;
  if (cu_cmp != nullptr) {
    const int Lc = max(0, min(cu_cmp[b + 1], Tc) - cu_cmp[b]);
    const int nvis = min((gr.T1 - s + 1) / r, Lc);
    gr.n_c = (nvis + kGK - 1) / kGK;
  }
  return gr;
}

__device__ __forceinline__ int seg_chunks(int b, const int32_t* __restrict__ cu_q,
                                          const int32_t* __restrict__ cu_kv) {
  const int Lq = cu_q[b + 1] - cu_q[b];
  return (Lq > 0 && cu_kv[b + 1] > cu_kv[b]) ? (Lq + kQCH - 1) / kQCH : 0;
}

__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(x, o, 64);
    if (lane >= o) x += v;
  }
  return x;
}

// Staged q / dout rows (64 heads x 256 dims): 16-byte chunk c of row r lives at chunk
// c ^ (4 (r % 4)), so that the transpose reads of a half-wavefront (4 rows x 4 chunks)
// touch every bank once.
__device__ __forceinline__ int ychunk(int row, int c) { return c ^ (4 * (row & 3)); }
// Staged A rows (tile keys x 64 heads of one term, 128 bytes): chunk c of key row r at
// chunk c ^ ((r / 2) % 8), so that 16 lanes reading 16 bytes of 16 consecutive keys touch
// every bank once.
__device__ __forceinline__ int achunk(int row, int c) { return c ^ ((row >> 1) & 7); }

// 16 bytes per lane from a per-lane address into LDS at M0 + 16 lane (wave-uniform base).
__device__ __forceinline__ void gather_to_lds(const void* src, uint32_t lds_off) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(lds_off), "v"(src)
      : "memory", "m0");
}

// C[tile keys x 256 dims] += sum over the item's queries i and (term, head) k of
// A[key, k] Y[k, dim]: A = scale dS (term 0) or P (term 1) of pair (i, key) from its slot
// row, Y = q or dout of query i.  Each (query, term) is one 64 KiB stage in LDS: the 64
// head rows of Y and the 256 keys' A rows, both loaded with global_load_lds.  Wavefront
// (a, b) owns key blocks a and a + 4 (32 keys each) and dims 128 b .. of the half.
__global__ __launch_bounds__(kDkvThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, int Tq, const void* ws_base, int nslot,
    int nvis_cap, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv,
    const int32_t* __restrict__ cu_cmp, int B, int global_start, int r, int wl, int wr, int Tc, int sparse,
    float* __restrict__ d_ori, float* __restrict__ d_cmp, float* __restrict__ part, int items_per_chunk) {
  __shared__ __attribute__((aligned(1024))) unsigned char stg[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wa = wave & 3, wb = wave >> 2;

  // ---- the work item.  The hardware deals workgroups to the 8 XCDs round robin
  // (workgroup x to XCD x % 8, in order), so group g goes to XCD g % 8 and takes
  // consecutive workgroup slots there: two per item (the dims halves).
  const int x = static_cast<int>(blockIdx.x);
  const int xcd = x & 7, slot = x >> 3;
  int seg = -1, chunk = 0, local = 0, off = 0, g_base = 0, gchunk = 0;
  for (int b = 0; b < B && seg < 0; ++b) {
    const int nch = seg_chunks(b, cu_q, cu_kv);
    for (int cbase = 0; cbase < nch && seg < 0; cbase += 64) {
      const int c = cbase + lane;
      int v = 0;
      if (c < nch && ((g_base + c) & 7) == xcd) {
        const ChunkGroup gr = chunk_group(b, c, cu_q, cu_kv, cu_cmp, global_start, r, wl, wr, Tc);
        v = 2 * (gr.n_w + gr.n_c);
      }
      const int incl = wave_incl_scan(v) + off;
      const unsigned long long hit = __ballot(v > 0 && incl - v <= slot && slot < incl);
      if (hit != 0ull) {
        const int src = __builtin_ctzll(hit);
        seg = b;
        chunk = cbase + src;
        gchunk = g_base + chunk;
        local = slot - __shfl(incl - v, src, 64);
      }
      off = __shfl(incl, 63, 64);
    }
    g_base += nch;
  }
  seg = __builtin_amdgcn_readfirstlane(seg);
  if (seg < 0) return;
  chunk = __builtin_amdgcn_readfirstlane(chunk);
  gchunk = __builtin_amdgcn_readfirstlane(gchunk);
  local = __builtin_amdgcn_readfirstlane(local);
  // deterministic mode: this item's tile goes to its own slot of the partial buffer
  float* tile = (part != nullptr)
                    ? part + (static_cast<long long>(gchunk) * items_per_chunk + local) * (static_cast<long long>(kGK) * 256)
                    : nullptr;
  const ChunkGroup gr = chunk_group(seg, chunk, cu_q, cu_kv, cu_cmp, global_start, r, wl, wr, Tc);
  const int half = local & 1, u = local >> 1;
  const int s = cu_kv[seg], e = cu_kv[seg + 1];
  const bool win = u < gr.n_w;
  int key0, key_end, i0, i1, cb = 0, nvis_seg = 0;
  if (win) {
    key0 = gr.k_lo + kGK * u;
    key_end = min(key0 + kGK, gr.k_hi + 1);
    i0 = max(gr.T0, key0 - wr) - global_start;
    i1 = min(gr.T1, key_end - 1 + wl) - global_start + 1;
  } else {
    cb = cu_cmp[seg];
    nvis_seg = min(cu_cmp[seg + 1], Tc) - cb;
    key0 = cb + kGK * (u - gr.n_w);
    key_end = min(key0 + kGK, cb + nvis_seg);
    // the first query that sees row key0 sits at segment position (key0 - cb + 1) r - 1
    const long long first = static_cast<long long>(s) + static_cast<long long>(key0 - cb + 1) * r - 1;
    i0 = static_cast<int>(max(static_cast<long long>(gr.T0), first)) - global_start;
    i1 = gr.T1 - global_start + 1;
  }
  if (i0 >= i1) {
    if (tile != nullptr) {  // no query meets these keys: the slot holds zeros
      for (int k = tid; k < (key_end - key0) * 64; k += kDkvThreads)
        reinterpret_cast<float4*>(tile)[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }

  const BwdWorkspace ws = ws_layout(const_cast<void*>(ws_base), Tq, nslot, nvis_cap);
  const uint32_t sb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(CSA_LDS(stg)));

  // ---- per-query key window: rows [lo, lo + nwin) of the segment; nk keys in the workspace
  struct QInfo {
    int lo, hi, nwin, vis, nk;
  };
  auto qinfo = [&](int i) {
    QInfo w;
    const int t = global_start + i;
    w.lo = max(s, t - wl);
    w.hi = min(e - 1, t + wr);
    w.nwin = w.hi - w.lo + 1;
    w.vis = win ? 0 : min((t - s + 1) / r, nvis_seg);
    w.nk = ws.nkeys[i];
    return w;
  };
  // this lane's 4 tile keys in the A staging: key rows 32 wave + 8 v + lane / 8
  auto key_of = [&](int v) { return 32 * wave + 8 * v + (lane >> 3); };
  // selection-map entries of this lane's 4 keys for query i (sparse compressed items)
  auto load_map = [&](int i, int (&mp)[4]) {
#pragma unroll
    for (int v = 0; v < 4; ++v) mp[v] = -1;
    if (!win && sparse) {
      const int t = global_start + i;
      const int vis = min(min((t - s + 1) / r, nvis_seg), nvis_cap);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int vv = key0 + key_of(v) - cb;
        if (vv < vis) mp[v] = ws.cmap[static_cast<long long>(i) * nvis_cap + vv];
      }
    }
  };
  // slot row base of this lane's 4 keys for query i (the zero row where i does not attend)
  auto slot_rows = [&](int i, const QInfo& w, const int (&mp)[4], const unsigned char* (&rowp)[4]) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int key = key0 + key_of(v);
      int sl = -1;
      if (key < key_end) {
        if (win) {
          if (key >= w.lo && key <= w.hi) sl = key - w.lo;
        } else if (key - cb < w.vis) {
          const int j = sparse ? mp[v] : key - cb;
          sl = (j >= 0) ? w.nwin + j : -1;
        }
        if (sl >= w.nk) sl = -1;
      }
      rowp[v] = (sl >= 0) ? ws.slots + (static_cast<long long>(i) * nslot + sl) * kSlotBytes : ws.zero;
    }
  };
  // one (query, term) stage into buffer bf: Y rows (4 instructions per wavefront, 2 rows of
  // 512 bytes each) then A rows (4 instructions, 8 keys of 128 bytes each)
  auto stage = [&](int i, int term, const unsigned char* const (&rowp)[4], int bf) {
    const uint16_t* ysrc = (term ? dout : q) + static_cast<long long>(i) * 64 * 512;
    const uint32_t base = sb + static_cast<uint32_t>(bf * kStage);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int uu = 4 * wave + v;
      const int row = 2 * uu + (lane >> 5);
      const uint32_t yoff = static_cast<uint32_t>(row * 1024 + half * 512 + ychunk(row, lane & 31) * 16);
      row_to_lds(ysrc, yoff, base + static_cast<uint32_t>(uu * 1024));
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int kk = key_of(v);
      gather_to_lds(rowp[v] + term * 128 + achunk(kk, lane & 7) * 16,
                    base + static_cast<uint32_t>(kYChunk + (8 * wave + 2 * v) * 512));
    }
  };
  // Wait: the A instruction of (wave, v) covers keys 8 (4 wave + v) .. + 7, i.e. 1 KiB at
  // kYChunk + (4 wave + v) * 1024 = kYChunk + (8 wave + 2 v) * 512.  key_of(v) matches.

  // transpose-read bases of Y (B operand) per dim block db: source lane m of lane group G
  // reads head row 8 (G / 2) + m / 4 (+ 16 st, + 4 for the second read), dims
  // 128 wb + 32 db + 16 (G % 2) + 4 (m % 4)
  const int G = lane >> 4, m = lane & 15;
  int boff[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int row = 8 * (G >> 1) + (m >> 2);
    const int c = 16 * wb + 4 * db + 2 * (G & 1) + ((m & 3) >> 1);
    boff[db] = row * kYRow + ychunk(row, c) * 16 + (m & 1) * 8;
  }
  // A reads (16 bytes: key 32 blk + l % 32, heads 16 st + 8 (l / 32) ..) per K step st;
  // the chunk swizzle of these keys does not depend on the block
  int aoff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int kk = lane & 31;
    aoff[st] = kYChunk + (32 * wa + kk) * 128 + achunk(kk, 2 * st + (lane >> 5)) * 16;
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[kb][db][j] = 0.f;
  bool used[2] = {false, false};

  // ---- pipeline: stage n + 1 is issued while stage n is multiplied
  int mp[4];
  const unsigned char* rowp[4];
  load_map(i0, mp);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  QInfo cur = qinfo(i0);
  slot_rows(i0, cur, mp, rowp);
  stage(i0, 0, rowp, 0);
  if (i0 + 1 < i1) load_map(i0 + 1, mp);
  for (int i = i0; i < i1; ++i) {
    // blocks of this wavefront with attended keys for query i
    bool act[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k_first = key0 + 32 * (wa + 4 * kb);
      const int k_last = min(k_first + 31, key_end - 1);
      act[kb] = win ? (max(k_first, cur.lo) <= min(k_last, cur.hi)) : (k_first < min(cb + cur.vis, key_end));
      used[kb] |= act[kb];
    }
#pragma unroll
    for (int term = 0; term < 2; ++term) {
      const int n = 2 * (i - i0) + term;
      const int bf = n & 1;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // stage n (and the map entries of query i + 1) landed
      tile_barrier();                      // every wavefront's part landed; buffer bf ^ 1 is free
      QInfo nxt = cur;
      if (term == 0) {
        stage(i, 1, rowp, bf ^ 1);
      } else if (i + 1 < i1) {
        nxt = qinfo(i + 1);
        slot_rows(i + 1, nxt, mp, rowp);
        stage(i + 1, 0, rowp, bf ^ 1);
        if (i + 2 < i1) load_map(i + 2, mp);
      }
      if (act[0] || act[1]) {
        const unsigned char* y = stg + bf * kStage;
        auto read_b = [&](int st, bf16x8 (&bfr)[4]) {
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf16x4 lo = ds_read_tr(y + boff[db] + st * 16 * kYRow);
            const bf16x4 hi = ds_read_tr(y + boff[db] + st * 16 * kYRow + 4 * kYRow);
            bfr[db] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        };
        bf16x8 bcur[4], bnxt[4];
        read_b(0, bcur);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          if (st + 1 < 4) read_b(st + 1, bnxt);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (!act[kb]) continue;
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(y + aoff[st] + kb * 4 * 32 * 128);
#pragma unroll
            for (int db = 0; db < 4; ++db)
              acc[kb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bcur[db], acc[kb][db], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < 4; ++db) bcur[db] = bnxt[db];
        }
      }
      if (term == 1) cur = nxt;
    }
  }

  // ---- C (32x32 blocks: lane l holds column l % 32, rows 8 (j / 4) + 4 (l / 32) + j % 4)
  if (tile != nullptr) {
    // deterministic mode: plain stores of the whole tile (rows below key_end), zeros included
    const int tcol = 128 * wb + (lane & 31);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kr = 32 * (wa + 4 * kb) + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
        if (key0 + kr >= key_end) continue;
#pragma unroll
        for (int db = 0; db < 4; ++db) tile[kr * 256 + tcol + 32 * db] = acc[kb][db][j];
      }
    }
    return;
  }
  float* dst = win ? d_ori : d_cmp;
  const int col = half * 256 + 128 * wb + (lane & 31);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (!used[kb]) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = key0 + 32 * (wa + 4 * kb) + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
      if (key >= key_end) continue;
#pragma unroll
      for (int db = 0; db < 4; ++db) atomicAdd(dst + static_cast<long long>(key) * 512 + col + 32 * db, acc[kb][db][j]);
    }
  }
}

// ----------------------------------------------------------------------------- deterministic row gradients

// One workgroup of 128 threads per gradient row (window rows 0 .. Tkv - 1, then
// compressed rows 0 .. Tc - 1); thread l sums dims 4 l .. 4 l + 3 over the work items
// whose key tile holds the row, in ascending query-chunk order (the same items the
// atomic mode adds, in a fixed order), and stores the row.
__global__ __launch_bounds__(128) void mla_bwd_dkv_reduce_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp, int B,
    int Tkv, int Tc, int global_start, int r, int wl, int wr, const float* __restrict__ part, int items_per_chunk,
    float* __restrict__ d_ori, float* __restrict__ d_cmp) {
  const int row = static_cast<int>(blockIdx.x);
  const int tid = threadIdx.x;
  const bool win = row < Tkv;
  const int key = win ? row : row - Tkv;
  // segment of the row: cu_kv for latent rows, cu_cmp (bounded by Tc) for compressed rows
  const int32_t* cu = win ? cu_kv : cu_cmp;
  int lo = 0, hi = B - 1;  // largest b with cu[b] <= key
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= key) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  const bool inside = key < cu[b + 1];
  if (inside) {
    int g_base = 0;
    for (int bb = 0; bb < b; ++bb) g_base += seg_chunks(bb, cu_q, cu_kv);
    const int qa = cu_q[b], qb = cu_q[b + 1], s = cu_kv[b];
    const int nch = seg_chunks(b, cu_q, cu_kv);
    int c_lo = 0, c_hi = -1;
    if (nch > 0) {
      if (win) {
        // queries t with t - wl <= key <= t + wr
        const int i_lo = max(qa, key - wr - global_start), i_hi = min(qb - 1, key + wl - global_start);
        if (i_lo <= i_hi) {
          c_lo = (i_lo - qa) / kQCH;
          c_hi = (i_hi - qa) / kQCH;
        }
      } else {
        // compressed row jl of the segment is visible from segment position (jl + 1) r - 1
        const int jl = key - cu_cmp[b];
        const long long i_first = static_cast<long long>(s) + static_cast<long long>(jl + 1) * r - 1 - global_start;
        if (i_first <= qb - 1) {
          c_lo = static_cast<int>((max(i_first, static_cast<long long>(qa)) - qa) / kQCH);
          c_hi = nch - 1;
        }
      }
    }
    const int dim = 4 * tid;
    const int half = dim >> 8;
    for (int c = c_lo; c <= c_hi; ++c) {
      const ChunkGroup gr = chunk_group(b, c, cu_q, cu_kv, cu_cmp, global_start, r, wl, wr, Tc);
      int u, key0;
      if (win) {
        if (key < gr.k_lo || key > gr.k_hi) continue;
        u = (key - gr.k_lo) / kGK;
        key0 = gr.k_lo + kGK * u;
      } else {
        const int jl = key - cu_cmp[b];
        if (jl / kGK >= gr.n_c) continue;
        u = gr.n_w + jl / kGK;
        key0 = cu_cmp[b] + kGK * (jl / kGK);
      }
      const float* t = part + (static_cast<long long>(g_base + c) * items_per_chunk + 2 * u + half) *
                                  (static_cast<long long>(kGK) * 256);
      const float4 v = *reinterpret_cast<const float4*>(t + (key - key0) * 256 + (dim & 255));
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
    }
  }
  float* dst = win ? d_ori : d_cmp;
  reinterpret_cast<float4*>(dst + static_cast<long long>(key) * 512)[tid] = sum;
}

// ----------------------------------------------------------------------------- sinks

__global__ __launch_bounds__(kThreads) void mla_bwd_sink_kernel(const void* ws_base, int Tq, int nslot, int nvis_cap,
                                                                float* __restrict__ d_sinks) {
  __shared__ float part[kThreads];
  const BwdWorkspace ws = ws_layout(const_cast<void*>(ws_base), Tq, nslot, nvis_cap);
  const int h = static_cast<int>(blockIdx.x);
  float acc = 0.f;
  for (int k = threadIdx.x; k < Tq; k += kThreads) acc += ws.sink_terms[static_cast<long long>(k) * 64 + h];
  part[threadIdx.x] = acc;
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

int slots_per_query(int key_cap) { return (key_cap + kNT - 1) / kNT * kNT; }

}  // namespace

bool mla_bwd_shape_supported(int H, int d, int dtype) { return dtype == 1 && H == 64 && d == 512; }

size_t mla_bwd_workspace_bytes(int Tq, int key_cap, int nvis_cap) {
  return ws_bytes(Tq, slots_per_query(key_cap), nvis_cap);
}

size_t mla_bwd_partial_bytes(int Tq, int B, int wl, int wr, int Tkv, bool has_cmp, int max_seqlen_kv, int r) {
  const long long wl_c = min(wl, Tkv), wr_c = min(wr, Tkv);
  const long long seg_max = max(1, max_seqlen_kv);
  const long long groups = (static_cast<long long>(Tq) + kQCH - 1) / kQCH + B;
  const long long n_w = min(static_cast<long long>(kQCH) - 1 + wl_c + wr_c, seg_max - 1) / kGK + 1;
  const long long n_c = has_cmp ? (seg_max / r + kGK - 1) / kGK : 0;
  return static_cast<size_t>(groups * 2 * (n_w + n_c)) * kGK * 256 * sizeof(float);
}

hipError_t launch_sparse_mla_bwd(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx,
                                 int topk, int Tq, int Tkv, int Tc, const int32_t* cu_q, const int32_t* cu_kv,
                                 const int32_t* cu_cmp, int B, int global_start, int r, int wl, int wr,
                                 int max_seqlen_kv, const float* sinks, float scale, const void* out,
                                 const float* lse, const void* dout, void* dq, float* d_ori, float* d_cmp,
                                 float* d_sinks, float* ori_l1, float* cmp_l1, int cmp_slots, int key_cap,
                                 int nvis_cap, void* workspace, bool deterministic, hipStream_t s) {
  const int W = wl + wr + 1;
  if (!deterministic) {  // the deterministic reduce writes every row itself
    zero(d_ori, static_cast<long long>(Tkv) * 512, s);
    zero(d_cmp, static_cast<long long>(Tc) * 512, s);
  }
  zero(ori_l1, static_cast<long long>(Tq) * W, s);
  zero(cmp_l1, static_cast<long long>(Tq) * cmp_slots, s);
  if (d_sinks != nullptr && (Tq == 0 || sinks == nullptr)) zero(d_sinks, 64, s);
  if (Tq <= 0) return hipGetLastError();
  if (cmp_idx == nullptr) topk = 0;
  // window sides past the stream length change nothing and keep t +- w in range
  const int wl_c = min(wl, Tkv), wr_c = min(wr, Tkv);
  const int nslot = slots_per_query(key_cap);
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* kv16 = static_cast<const uint16_t*>(ori_kv);
  const auto* c16 = static_cast<const uint16_t*>(cmp_kv);
  const auto* d16 = static_cast<const uint16_t*>(dout);
  auto prep = (topk <= 2 * kThreads) ? mla_bwd_prep_kernel<2> : mla_bwd_prep_kernel<kMaxTopk / kThreads>;
  const unsigned prep_grid = static_cast<unsigned>((Tq + 63) / 64) * 64u;  // whole runs of 8 queries x 8 XCDs
  hipLaunchKernelGGL(prep, dim3(prep_grid), dim3(kPrepThreads), 0, s, q16, kv16, c16, cmp_idx, topk, Tq, Tc, cu_q, cu_kv,
                     cu_cmp, B, global_start, r, wl_c, wr_c, sinks, scale, static_cast<const uint16_t*>(out), lse, d16,
                     workspace, nslot, nvis_cap, ori_l1, W, cmp_l1, cmp_slots, static_cast<uint16_t*>(dq));
  // dkv: an upper bound of the workgroup slots per XCD (the exact count needs cu_seqlens
  // on the host): groups <= Tq / 128 + B, each with at most n_w + n_c items x 2 halves
  const long long seg_max = max(1, max_seqlen_kv);
  const long long groups = (static_cast<long long>(Tq) + kQCH - 1) / kQCH + B;
  const long long n_w = min(static_cast<long long>(kQCH) - 1 + wl_c + wr_c, seg_max - 1) / kGK + 1;
  const long long n_c = (cmp_kv != nullptr) ? (seg_max / r + kGK - 1) / kGK : 0;
  const long long items = (groups + 7) / 8 * 2 * (n_w + n_c) * 8;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int per_chunk = static_cast<int>(2 * (n_w + n_c));
  float* part = deterministic ? reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                                         ws_bytes(Tq, nslot, nvis_cap))
                              : nullptr;
  hipLaunchKernelGGL(mla_bwd_dkv_kernel, dim3(static_cast<unsigned>(items)), dim3(kDkvThreads), 0, s, q16, d16, Tq,
                     static_cast<const void*>(workspace), nslot, nvis_cap, cu_q, cu_kv,
                     cmp_kv != nullptr ? cu_cmp : nullptr, B, global_start, r, wl_c, wr_c, Tc,
                     cmp_idx != nullptr ? 1 : 0, d_ori, d_cmp, part, per_chunk);
  if (deterministic && Tkv + Tc > 0)
    hipLaunchKernelGGL(mla_bwd_dkv_reduce_kernel, dim3(static_cast<unsigned>(Tkv + Tc)), dim3(128), 0, s, cu_q, cu_kv,
                       cmp_kv != nullptr ? cu_cmp : nullptr, B, Tkv, Tc, global_start, r, wl_c, wr_c, part, per_chunk,
                       d_ori, d_cmp);
  if (d_sinks != nullptr && sinks != nullptr)
    hipLaunchKernelGGL(mla_bwd_sink_kernel, dim3(64), dim3(kThreads), 0, s, static_cast<const void*>(workspace), Tq,
                       nslot, nvis_cap, d_sinks);
  return hipGetLastError();
}

}  // namespace csa
