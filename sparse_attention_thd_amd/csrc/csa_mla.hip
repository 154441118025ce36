// Sparse MLA forward: window branch + compressed branch + per-head sink over one
// shared latent KV (keys are values), fp32 online softmax.
//
// MFMA path, (H, d) = (64, 512) bf16: one workgroup of 4 wavefronts per query.  Keys
// stream through LDS in tiles of 32 rows (window rows first, then the compacted
// compressed rows).  Per tile, wavefront w
//   forms S^T[32 keys x 16 heads] = K[32 x 512] . Q^T[512 x 16] for heads [16w, 16w+16)
//     (A = K from LDS, B = Q in VGPRs) and runs their online softmax in registers (each
//     lane owns one head column); the accumulator layout of S^T is directly the P^T
//     MFMA operand, which goes to LDS as plain 16-byte fragments with the heads'
//     rescale factors;
//   then, after a barrier, accumulates O^T[128 dims x 64 heads] += V^T[128 x 32] . P^T[32 x 64]
//     for latent dims [128w, 128w+128) (A = V^T from LDS, B = the four P^T fragments).
// Splitting the PV product by dims means each V element is read from LDS once per
// workgroup instead of once per head block.
//
// Generic path (H * d <= 8192, either dtype): scalar fp32, one key at a time.
#include "csa_common.h"
#include "csa_internal.h"
#include "csa_tile.h"

namespace csa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// row_to_lds for a row that one workgroup reads once (the query's q rows): the load
// carries the non-temporal hint, so the streamed rows are the first to leave the caches
// and the key rows that neighbouring queries share stay resident.  Measured with the
// non-temporal output stores below: 0.998 against 1.014 ms on the 16k pack (six
// same-box A/B pairs).  In the backward the same hints measured slower (its row
// gradients re-read q and dout), so it keeps the plain forms.
__device__ __forceinline__ void row_to_lds_once(const void* row_base, uint32_t lane_off, uint32_t lds_off) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt"
      :
      : "s"(lds_off), "v"(lane_off), "s"(row_base)
      : "memory", "m0");
}

// Largest b in [0, B) with cu[b] <= x (cu non-decreasing, cu[0] <= x), found with
// one wide load per 64 entries and a ballot instead of a chain of dependent loads.
// The result is wave-uniform, so the loads that depend on it are scalar.
__device__ __forceinline__ int segment_of_wave(const int32_t* __restrict__ cu, int B, int x) {
  const int lane = threadIdx.x & 63;
  int count = 0;
  for (int base = 0; base < B; base += 64) {
    const int k = base + lane;
    const bool le = (k < B) && cu[k] <= x;
    count += __popcll(__ballot(le));
  }
  return __builtin_amdgcn_readfirstlane(count - 1);
}

// Resolve the query's window and compressed key ranges.  Compressed rows are bounded by
// the segment and by the Tc rows the cmp_kv buffer holds.  `bad` is set when a
// caller-held residual disagrees with the segment length.
__device__ QueryKeys query_ranges(int i, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv,
                                  const int32_t* __restrict__ cu_cmp, const int32_t* __restrict__ residual, int B,
                                  int global_start, int r, int wl, int wr, int Tc, bool has_cmp, bool attend_all,
                                  bool& bad) {
  QueryKeys k;
  const int b = segment_of_wave(cu_q, B, i);
  const int t = global_start + i;
  const int s = cu_kv[b], e = cu_kv[b + 1];
  k.lo = max(s, t - wl);
  const int hi = min(e - 1, t + wr);
  k.nwin = hi - k.lo + 1;
  k.ncmp = 0;
  k.cmp_base = (cu_cmp != nullptr) ? cu_cmp[b] : 0;
  if (has_cmp && attend_all) {
    const int nv = (t - s + 1) / r;
    k.ncmp = max(0, min(min(nv, cu_cmp[b + 1] - k.cmp_base), Tc - k.cmp_base));
  }
  bad = residual != nullptr && residual[b] != (e - s) % r;
  return k;
}

// Generic-path helper: ranges plus compaction, loading the cmp_idx row itself.
__device__ QueryKeys query_keys(int i, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv,
                                const int32_t* __restrict__ cu_cmp, const int32_t* __restrict__ residual, int B,
                                int global_start, int r, int wl, int wr, int Tc, bool has_cmp,
                                const int32_t* __restrict__ cmp_idx, int topk, int32_t* crow, uint32_t* wsum,
                                bool& bad) {
  QueryKeys k = query_ranges(i, cu_q, cu_kv, cu_cmp, residual, B, global_start, r, wl, wr, Tc, has_cmp,
                             cmp_idx == nullptr, bad);
  if (!has_cmp || cmp_idx == nullptr) return k;
  const int32_t* row = cmp_idx + static_cast<long long>(i) * topk;
  int vals[kMaxTopk / kThreads];
#pragma unroll
  for (int ch = 0; ch < kMaxTopk / kThreads; ++ch) {
    const int j = ch * kThreads + static_cast<int>(threadIdx.x);
    vals[ch] = (j < topk) ? row[j] : -1;
  }
  k.ncmp = compact_rows(vals, topk, min(cu_cmp[B], Tc), crow, wsum);
  return k;
}

// ----------------------------------------------------------------------------- MFMA path

constexpr int kQD = 2;                       // K-fragment prefetch distance (MFMA pairs)
constexpr int kVD = 4;                       // V^T-fragment prefetch distance (MFMAs)

template <int NC>  // cmp_idx row chunks of kThreads entries: ceil(topk / 256)
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_fwd_h64_d512_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ori_kv, const uint16_t* __restrict__ cmp_kv,
    const int32_t* __restrict__ cmp_idx, int topk, int topk_rows, int Tq, int Tc, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp, const int32_t* __restrict__ residual, int B,
    int global_start, int r, int wl, int wr, const float* __restrict__ sinks, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) unsigned char kt[2 * kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char pfr[kWaves * 64 * 16];  // P^T fragments of the tile
  __shared__ float alpha_h[64];  // per-head rescale factor of the tile (1 when not rescaled)
  __shared__ int resc[kWaves];   // whether head block w rescaled in this tile
  __shared__ int32_t crow[kMaxTopk];
  __shared__ uint32_t wsum[kWaves];

  // Blocks are dispatched round-robin over the 8 XCDs.  Each XCD takes runs of 8
  // consecutive queries (which share window rows and compressed rows in its L2),
  // and runs alternate between XCDs so long, expensive segments spread evenly.
  const int kx = static_cast<int>(blockIdx.x >> 3);
  const int i = ((kx >> 3) * 8 + static_cast<int>(blockIdx.x & 7u)) * 8 + (kx & 7);
  if (i >= Tq) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int head = 16 * wave + n;
  const bool has_idx = cmp_kv != nullptr && cmp_idx != nullptr;

  // Prologue loads are issued cheapest-first and all stay in flight together; each
  // later use waits only for the loads it needs (the counter retires them in order).
  // With B < 64 every lane b <= B also fetches cu_kv[b] and cu_cmp[b], so the segment's
  // bounds come from a register broadcast instead of a second dependent load.
  const bool small_b = B < 64;
  const int cu0 = (lane < B) ? cu_q[lane] : 0x7fffffff;  // first 64 segment starts
  const int kv0 = (small_b && lane <= B) ? cu_kv[lane] : 0;
  const int cm0 = (small_b && lane <= B && cu_cmp != nullptr) ? cu_cmp[lane] : 0;
  // An arbitrary index row is needed whatever the query's visible count: fetch it now.
  const int32_t* idx_row = has_idx ? cmp_idx + static_cast<long long>(i) * topk : nullptr;
  int vals[NC];
  if (has_idx && !topk_rows) {
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) vals[ch] = idx_row[min(ch * kThreads + tid, topk - 1)];
  }
  // The query's 64 q rows (64 KiB, contiguous) are staged through the idle tile buffers
  // as whole 1 KiB rows, one global_load_lds_dwordx4 per row (wave w: heads 16w ..
  // 16w + 15, padded rows), and read back as fragments once they have landed.
  const uint32_t kt_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(CSA_LDS(kt)));
  const uint32_t lane16 = static_cast<uint32_t>(lane) << 4;
  {
    const uint16_t* qsrc = q + (static_cast<long long>(i) * 64 + 16 * wave) * 512;
#pragma unroll
    for (int hh = 0; hh < 16; ++hh)
      row_to_lds_once(qsrc + hh * 512, lane16, kt_base + static_cast<uint32_t>((16 * wave + hh) * kRowStride));
  }
  // segment of query row i: count segment starts <= i (one ballot per 64 segments)
  int count = __popcll(__ballot(cu0 <= i));
  for (int base = 64; base < B; base += 64) count += __popcll(__ballot(base + lane < B && cu_q[base + lane] <= i));
  const int b = __builtin_amdgcn_readfirstlane(count - 1);
  QueryKeys qk;
  int cmp_end = 0, cmp_total = 0;  // cu_cmp[b + 1], cu_cmp[B]
  const int t_abs = global_start + i;
  int seg_s, seg_e;
  {
    if (small_b) {
      seg_s = __builtin_amdgcn_readlane(kv0, b);
      seg_e = __builtin_amdgcn_readlane(kv0, b + 1);
      qk.cmp_base = __builtin_amdgcn_readlane(cm0, b);
      cmp_end = __builtin_amdgcn_readlane(cm0, b + 1);
      cmp_total = __builtin_amdgcn_readlane(cm0, B);
    } else {
      seg_s = cu_kv[b];
      seg_e = cu_kv[b + 1];
      if (cu_cmp != nullptr) {
        qk.cmp_base = cu_cmp[b];
        cmp_end = cu_cmp[b + 1];
        cmp_total = cu_cmp[B];
      } else {
        qk.cmp_base = 0;
      }
    }
    qk.lo = max(seg_s, t_abs - wl);
    qk.nwin = min(seg_e - 1, t_abs + wr) - qk.lo + 1;
    qk.ncmp = 0;
  }
  // Compressed rows that exist: the segment's, inside the Tc rows of the buffer.
  const int nvis = (cmp_kv != nullptr)
                       ? max(0, min(min((t_abs - seg_s + 1) / r, cmp_end - qk.cmp_base), Tc - qk.cmp_base))
                       : 0;
  // Contiguous compressed rows [cmp_base, cmp_base + nvis): attend-all layers, and top-k
  // rows of a query with at most topk visible rows (its top-k is all of them); none
  // without compression.
  const bool direct = cmp_kv == nullptr || cmp_idx == nullptr || (topk_rows && nvis <= topk);
  if (direct) qk.ncmp = nvis;
  // A caller-held residual that disagrees with the segment length poisons the output.
  const bool bad = residual != nullptr && residual[b] != (seg_e - seg_s) % r;
  // Every address of a direct query's tiles is wave-uniform (rows lo + k of the window,
  // then cmp_base + k): formed in scalar registers, no lane lookup.
  auto issue_direct_tile = [&](int t, int bf, int nkeys_) {
#pragma unroll
    for (int pass = 0; pass < kNT / kWaves; ++pass) {
      int kidx = t * kNT + pass * kWaves + wave;
      kidx = (kidx < nkeys_) ? kidx : 0;
      const uint16_t* src = (kidx < qk.nwin) ? ori_kv + static_cast<long long>(qk.lo + kidx) * 512
                                             : cmp_kv + static_cast<long long>(qk.cmp_base + kidx - qk.nwin) * 512;
      row_to_lds(src, lane16, kt_base + static_cast<uint32_t>(bf * kTileBytes + (pass * kWaves + wave) * kRowStride));
    }
  };
  if (has_idx && !direct) {
    if (topk_rows) {
      // a selecting query: exactly topk rows, ascending, used as given (clamped into the buffer)
      const int hi_row = max(0, min(cmp_total, Tc) - 1);
#pragma unroll
      for (int ch = 0; ch < NC; ++ch) {
        const int j = ch * kThreads + tid;
        if (j < topk) crow[j] = min(max(idx_row[j], 0), hi_row);
      }
      qk.ncmp = topk;
    } else {
#pragma unroll
      for (int ch = 0; ch < NC; ++ch) vals[ch] = (ch * kThreads + tid < topk) ? vals[ch] : -1;
      qk.ncmp = compact_rows(vals, topk, min(cmp_total, Tc), crow, wsum);
    }
  }
  const int nkeys = qk.nwin + qk.ncmp;
  const int ntiles = (nkeys + kNT - 1) / kNT;

  // Stage tile t (32 rows) into buffer bf: wave w issues rows w, w+4, ..., one 1 KiB
  // row per global_load_lds_dwordx4.  Lane p < 8 first resolves the source address
  // of row 4p + w (one LDS lookup for all of them); each load then takes it as a
  // scalar base, and lane l fetches the 16-byte chunk that lands at chunk l of the
  // row.  Rows past the key list re-read a valid row; their
  // probabilities are exactly zero.
  auto issue = [&](int t, int bf) {
    if (direct || (t + 1) * kNT <= qk.nwin) {
      issue_direct_tile(t, bf, nkeys);
      return;
    }
    const int p = lane & 7;
    int kidx = t * kNT + 4 * p + wave;
    kidx = (kidx < nkeys) ? kidx : 0;
    const uint16_t* src;
    if (kidx < qk.nwin) {
      src = ori_kv + static_cast<long long>(qk.lo + kidx) * 512;
    } else {
      src = cmp_kv + static_cast<long long>(crow[kidx - qk.nwin]) * 512;
    }
    const unsigned long long a = reinterpret_cast<unsigned long long>(src);
    const uint32_t a_lo = static_cast<uint32_t>(a), a_hi = static_cast<uint32_t>(a >> 32);
#pragma unroll
    for (int pass = 0; pass < kNT / kWaves; ++pass) {
      const int rr = pass * kWaves + wave;
      const unsigned long long base =
          (static_cast<unsigned long long>(__builtin_amdgcn_readlane(a_hi, pass)) << 32) |
          static_cast<uint32_t>(__builtin_amdgcn_readlane(a_lo, pass));
      row_to_lds(reinterpret_cast<const void*>(base), lane16,
                 kt_base + static_cast<uint32_t>(bf * kTileBytes + rr * kRowStride));
    }
  };
  // Running max in log2 units; the sink is the initial state (value 0, weight 1 counted
  // once).  Read before the wait below, so that no load of the compiler's own is still
  // outstanding once the tile loads start (a compiler-placed wait for it inside the
  // first tile would also drain the second tile's loads).
  float m_run = -__builtin_huge_valf();
  float l_run = 0.f;
  if (sinks != nullptr) {
    m_run = sinks[head] * kLog2e;
    l_run = (g == 0) ? 1.f : 0.f;
  }
  // q rows landed everywhere -> B operand of S^T = K . Q^T.  Within MFMA step ks, k-slot
  // 8g + j of lane group g stands for latent dim 32*ks + 4*g + j (j < 4) or 32*ks + 16 +
  // 4*g + (j - 4): the same permutation the K fragments use, so each half is one
  // conflict-free 8-byte LDS read (rows 1040 bytes apart fall 4 banks apart).  This
  // barrier also publishes crow where a selecting query wrote its index row straight
  // into it (no barrier of its own) before any wavefront gathers tile 0 through it.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  tile_barrier();
  bf16x8 qf[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
    qf[ks] = kfrag(kt, head * kRowStride + 64 * ks + 8 * g, head * kRowStride + 64 * ks + 8 * g + 32);
  lds_barrier();  // every wavefront has its q fragments: the tile buffers are free
  // Both buffers are free, so tiles 0 and 1 are issued together: tile 1's gathers then
  // run under tile 0's instead of starting once tile 0 has landed (0.956 against
  // 0.980 ms on the 16k pack, three same-box A/B pairs).  Later tiles are issued one
  // ahead, into the buffer the previous tile freed.
  if (ntiles > 0) issue(0, 0);
  if (ntiles > 1) issue(1, 1);
  f32x4 o[32];
#pragma unroll
  for (int mb = 0; mb < 32; ++mb) o[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane LDS byte offsets inside a tile: K reads of row kpi(n) at dims 32ks + 4g
  // (+16); transpose V reads of row kpi(4g + n/4) at dims 16mb + 4(n%4)
  const int offq = kpi(n) * kRowStride + 8 * g;
  const int offv = kpi(4 * g + (n >> 2)) * kRowStride + 8 * (n & 3);

  for (int t = 0; t < ntiles; ++t) {
    const int bf = t & 1;
    // This wavefront's rows of tile t have landed: every load but the 8 most recent
    // (tile 1's, each wavefront issues 8 per tile) before tile 0, every load after that
    // (loads retire in order).
    static_assert(kNT / kWaves == 8, "the wait before tile 0 leaves tile 1's 8 loads per wavefront in flight");
    if (t == 0 && ntiles > 1) {
      __builtin_amdgcn_s_waitcnt(0x0F78);
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    // The barrier publishes every wavefront's rows of tile t, and it also means all
    // of them are done reading buffer bf ^ 1 (tile t - 1), which the next loads refill.
    tile_barrier();
    if (t > 0 && t + 1 < ntiles) issue(t + 1, bf ^ 1);
    const unsigned char* tb = kt + bf * kTileBytes;

    // ---- S^T = K . Q^T for keys [0,16) and [16,32) of the tile; K fragments are
    // staged kQD steps ahead and the order is pinned with scheduling fences.
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    {
      bf16x8 a0[kQD], a1[kQD];
#pragma unroll
      for (int ks = 0; ks < kQD; ++ks) {
        a0[ks] = kfrag(tb, offq + 64 * ks, offq + 64 * ks + 32);
        a1[ks] = kfrag(tb + 16 * kRowStride, offq + 64 * ks, offq + 64 * ks + 32);
      }
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const int sl = ks % kQD;
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[sl], qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[sl], qf[ks], s1, 0, 0, 0);
        if (ks + kQD < 16) {
          const int kn = ks + kQD;
          a0[sl] = kfrag(tb, offq + 64 * kn, offq + 64 * kn + 32);
          a1[sl] = kfrag(tb + 16 * kRowStride, offq + 64 * kn, offq + 64 * kn + 32);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- online softmax; this lane holds keys kpi(4g+j) and 16+kpi(4g+j) of head `head`.
    // Only the last tile can reach past the key list; its missing keys get -inf.  The
    // scale is positive (checked by the caller), so the tile maximum is taken on the raw
    // scores and scaled once, and each exponent is one fma.
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    if ((t + 1) * kNT > nkeys) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k0 = t * kNT + kpi(4 * g + j);
        sv[j] = (k0 < nkeys) ? sv[j] : -__builtin_huge_valf();
        sv[4 + j] = (k0 + 16 < nkeys) ? sv[4 + j] : -__builtin_huge_valf();
      }
    }
    float smax = fmaxf(sv[0], sv[4]);
#pragma unroll
    for (int j = 1; j < 4; ++j) smax = fmaxf(smax, fmaxf(sv[j], sv[4 + j]));
    const float tmax = quad_max(smax) * scale_log2;
    // Lazy rescale: keep a stale maximum while the tile stays within 2^8 of it.
    const bool rescale = __any(tmax > m_run + 8.f);
    float alpha = 1.f;
    if (rescale) {
      const float m_new = fmaxf(m_run, tmax);
      alpha = exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
    }
    bf16x8 pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[j], scale_log2, -m_run));
      l_run += p;
      pb[j] = static_cast<__bf16>(p);
    }
    // publish this head block's P^T fragment and rescale factors to the workgroup
    *reinterpret_cast<bf16x8*>(pfr + (wave * 64 + lane) * 16) = pb;
    if (g == 0) alpha_h[head] = alpha;
    if (lane == 0) resc[wave] = rescale ? 1 : 0;
    lds_barrier();  // every head block's P^T and factors are visible (tile t + 1 stays in flight)

    // ---- O^T[dims 128 wave + 16 db .. , heads 16 hb + n] += V^T . P^T.  k-slot 8g+j <->
    // key kpi(4g+j) (j < 4) or 16+kpi(4g+j-4), in both operands.
    if (resc[0] | resc[1] | resc[2] | resc[3]) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const float a = alpha_h[16 * hb + n];
#pragma unroll
        for (int db = 0; db < 8; ++db) o[8 * hb + db] *= a;
      }
    }
    {
      bf16x8 pf[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) pf[hb] = *reinterpret_cast<const bf16x8*>(pfr + (hb * 64 + lane) * 16);
      bf16x4 vlo[2], vhi[2];
      const unsigned char* pv0 = tb + offv + 32 * (8 * wave);
      vlo[0] = ds_read_tr(pv0);
      vhi[0] = ds_read_tr(pv0 + 16 * kRowStride);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int sl = db & 1;
        if (db + 1 < 8) {
          vlo[sl ^ 1] = ds_read_tr(pv0 + 32 * (db + 1));
          vhi[sl ^ 1] = ds_read_tr(pv0 + 32 * (db + 1) + 16 * kRowStride);
        }
        const bf16x8 a = {vlo[sl][0], vlo[sl][1], vlo[sl][2], vlo[sl][3],
                          vhi[sl][0], vhi[sl][1], vhi[sl][2], vhi[sl][3]};
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          o[8 * hb + db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[hb], o[8 * hb + db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  const float l_tot = quad_sum(l_run);
  float* inv_h = alpha_h;  // reused: 1 / l of every head
  tile_barrier();          // every wavefront is done with the factors of the last tile
  if (g == 0) inv_h[head] = bad ? __builtin_nanf("") : 1.f / l_tot;
  lds_barrier();           // all reads of the last tile are done; inv_h is visible
  // Stage the output through the (now idle) tile buffers so it leaves as one contiguous
  // 1 KiB head row per store instruction.  This wavefront holds dims [128 wave, +128) of
  // every head: head row h, 16-byte chunk c lives at chunk c ^ swz(h).
  // Lane-derived offsets are recomputed from an opaque copy of the lane id so the
  // compiler does not hoist them above the tile loop (where they would spill).
  int el;
  asm volatile("v_mov_b32 %0, %1" : "=v"(el) : "v"(lane));
  const int en = el & 15, eg = el >> 4;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int h = 16 * hb + en;
    const float inv = inv_h[h];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const f32x4 v = o[8 * hb + db];
      const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16_bits(v[0] * inv)) |
                          (static_cast<uint32_t>(f32_to_bf16_bits(v[1] * inv)) << 16);
      const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16_bits(v[2] * inv)) |
                          (static_cast<uint32_t>(f32_to_bf16_bits(v[3] * inv)) << 16);
      // dims 128 wave + 16 db + 4 eg .. + 3: chunk 16 wave + 2 db + eg / 2, half eg % 2
      const int chunk = (16 * wave + 2 * db + (eg >> 1)) ^ swz(h);
      *reinterpret_cast<uint2*>(kt + h * kRowBytes + chunk * 16 + (eg & 1) * 8) = make_uint2(w0, w1);
    }
  }
  lds_barrier();  // every head row is complete
  // The output rows are written once and not read again by this launch: non-temporal stores.
  uint16_t* obase = out + (static_cast<long long>(i) * 64 + 16 * wave) * 512;
#pragma unroll
  for (int hh = 0; hh < 16; ++hh) {
    const int h = 16 * wave + hh;
    const u32x4 v = *reinterpret_cast<const u32x4*>(kt + h * kRowBytes + ((el ^ swz(h)) << 4));
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + hh * 512 + el * 8));
  }
  if (lse != nullptr && g == 0)
    lse[static_cast<long long>(i) * 64 + head] = bad ? __builtin_nanf("") : m_run * kLn2 + logf(l_tot);
}

// ----------------------------------------------------------------------------- generic path

__device__ __forceinline__ float ld(const float* p, long long k) { return p[k]; }
__device__ __forceinline__ float ld(const uint16_t* p, long long k) { return bf16_bits_to_f32(p[k]); }
__device__ __forceinline__ void st(float* p, long long k, float v) { p[k] = v; }
__device__ __forceinline__ void st(uint16_t* p, long long k, float v) { p[k] = f32_to_bf16_bits(v); }

constexpr int kGenMaxHD = 8192;
constexpr int kGenPerThread = kGenMaxHD / kThreads;

template <typename T>
__global__ __launch_bounds__(kThreads) void mla_fwd_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ ori_kv, const T* __restrict__ cmp_kv,
    const int32_t* __restrict__ cmp_idx, int topk, int Tc, int H, int d, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp, const int32_t* __restrict__ residual, int B,
    int global_start, int r, int wl, int wr, const float* __restrict__ sinks, float scale, T* __restrict__ out,
    float* __restrict__ lse) {
  extern __shared__ float gdyn[];
  __shared__ int32_t crow[kMaxTopk];
  __shared__ uint32_t wsum[kWaves];
  float* qs = gdyn;               // [H*d]
  float* krow = qs + H * d;       // [d]
  float* m = krow + d;            // [H]
  float* l = m + H;               // [H]
  float* al = l + H;              // [H]
  float* pv = al + H;             // [H]
  const int i = blockIdx.x, tid = threadIdx.x;
  bool bad;
  const QueryKeys qk = query_keys(i, cu_q, cu_kv, cu_cmp, residual, B, global_start, r, wl, wr, Tc, cmp_kv != nullptr,
                                  cmp_idx, topk, crow, wsum, bad);
  const int hd = H * d;
  for (int e = tid; e < hd; e += kThreads) qs[e] = ld(q, static_cast<long long>(i) * hd + e);
  for (int h = tid; h < H; h += kThreads) {
    m[h] = sinks ? sinks[h] : -__builtin_huge_valf();
    l[h] = sinks ? 1.f : 0.f;
  }
  float acc[kGenPerThread];
#pragma unroll
  for (int u = 0; u < kGenPerThread; ++u) acc[u] = 0.f;
  __syncthreads();
  const int nkeys = qk.nwin + qk.ncmp;
  for (int kidx = 0; kidx < nkeys; ++kidx) {
    const T* src;
    if (kidx < qk.nwin) {
      src = ori_kv + static_cast<long long>(qk.lo + kidx) * d;
    } else {
      const int c = (cmp_idx != nullptr) ? crow[kidx - qk.nwin] : qk.cmp_base + (kidx - qk.nwin);
      src = cmp_kv + static_cast<long long>(c) * d;
    }
    for (int e = tid; e < d; e += kThreads) krow[e] = ld(src, e);
    __syncthreads();
    for (int h = tid; h < H; h += kThreads) {
      float dot = 0.f;
      for (int e = 0; e < d; ++e) dot += qs[h * d + e] * krow[e];
      const float z = dot * scale;
      const float mn = fmaxf(m[h], z);
      const float a = expf(m[h] - mn);
      const float p = expf(z - mn);
      l[h] = l[h] * a + p;
      m[h] = mn;
      al[h] = a;
      pv[h] = p;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kGenPerThread; ++u) {
      const int e = tid + u * kThreads;
      if (e < hd) {
        const int h = e / d;
        acc[u] = acc[u] * al[h] + pv[h] * krow[e - h * d];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < kGenPerThread; ++u) {
    const int e = tid + u * kThreads;
    if (e < hd) st(out, static_cast<long long>(i) * hd + e, bad ? __builtin_nanf("") : acc[u] / l[e / d]);
  }
  if (lse != nullptr)
    for (int h = tid; h < H; h += kThreads)
      lse[static_cast<long long>(i) * H + h] = bad ? __builtin_nanf("") : m[h] + logf(l[h]);
}

}  // namespace

bool mla_shape_supported(int H, int d, int dtype) {
  if (dtype == 1 && H == 64 && d == 512) return true;
  return H * d <= kGenMaxHD && d % 8 == 0;
}

hipError_t launch_sparse_mla(const void* q, const void* ori_kv, const void* cmp_kv, const int32_t* cmp_idx,
                             int topk, bool topk_rows, int Tq, int Tc, int H, int d, int dtype, const int32_t* cu_q,
                             const int32_t* cu_kv, const int32_t* cu_cmp, const int32_t* residual, int B,
                             int global_start, int r, int wl, int wr, const float* sinks, float scale, void* out,
                             float* lse, hipStream_t s) {
  if (Tq <= 0) return hipSuccess;
  if (cmp_idx == nullptr) topk = 0;
  if (dtype == 1 && H == 64 && d == 512) {
    const unsigned grid = static_cast<unsigned>((Tq + 63) / 64) * 64u;  // whole runs of 8 queries x 8 XCDs
    auto kern = (topk <= 2 * kThreads) ? mla_fwd_h64_d512_kernel<2> : mla_fwd_h64_d512_kernel<kMaxTopk / kThreads>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, s, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(ori_kv), static_cast<const uint16_t*>(cmp_kv), cmp_idx, topk,
                       topk_rows ? 1 : 0, Tq, Tc, cu_q, cu_kv, cu_cmp, residual, B, global_start, r, wl, wr, sinks,
                       scale * kLog2e, static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
  }
  const size_t lds = (static_cast<size_t>(H) * d + d + 4 * static_cast<size_t>(H)) * sizeof(float);
  if (dtype == 1) {
    auto k = mla_fwd_generic_kernel<uint16_t>;
    if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess)
      return e;
    hipLaunchKernelGGL(k, dim3(Tq), dim3(kThreads), lds, s, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(ori_kv), static_cast<const uint16_t*>(cmp_kv), cmp_idx, topk, Tc,
                       H, d, cu_q, cu_kv, cu_cmp, residual, B, global_start, r, wl, wr, sinks, scale,
                       static_cast<uint16_t*>(out), lse);
  } else {
    auto k = mla_fwd_generic_kernel<float>;
    if (const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(k), lds); e != hipSuccess)
      return e;
    hipLaunchKernelGGL(k, dim3(Tq), dim3(kThreads), lds, s, static_cast<const float*>(q),
                       static_cast<const float*>(ori_kv), static_cast<const float*>(cmp_kv), cmp_idx, topk, Tc, H, d,
                       cu_q, cu_kv, cu_cmp, residual, B, global_start, r, wl, wr, sinks, scale,
                       static_cast<float*>(out), lse);
  }
  return hipGetLastError();
}

}  // namespace csa
