// Lightning-indexer KL loss against the main attention and its gradients,
// (H_I, d_I) = (64, 128) bf16.  For query i with selected compressed rows c_j (the
// valid entries of its top-k row) and targets p_j (the main attention's
// head-averaged probabilities at those slots):
//   p^ = p / sum p,  I_j = sum_h w_h relu(u_hj),  u_hj = <q_I[i,h], k[c_j]>
//   loss_i = KL(p^ || softmax(I)),  G_j = loss_scale * (softmax_j(I) - p^_j)
//   d_w[i,h] = sum_j G_j relu(u_hj),  d_q[i,h] = sum_j G_j w_h [u_hj > 0] k[c_j]
//   d_k[c_j] += sum_h G_j w_h [u_hj > 0] q_I[i,h]
//
// Two kernels:
//   kl_query  one workgroup (4 wavefronts x 16 heads) per query.  The selected rows
//             stream through LDS 32 at a time; u^T = K . q^T with
//             v_mfma_f32_16x16x32_bf16 (K rows from LDS, q in registers).  Pass 1
//             forms I (the head sum crosses wavefronts through LDS), the softmax
//             and G; pass 2 recomputes u and accumulates d_w and d_q^T = K^T . M^T
//             (K^T by transpose reads, M^T = G w [u > 0] straight from the u^T
//             accumulators).  G and a map of the visible rows go to the workspace.
//   kl_dk     key-major d_k: a workgroup holds 128 compressed rows of one segment in
//             registers and sweeps a chunk of 128 queries, forming u = q . K^T and
//             d_k^T += q^T . M per query (q staged in LDS), then adds its tile to the
//             float32 gradient once.
#include <mutex>

#include "csa_common.h"
#include "csa_internal.h"
#include "csa_tile.h"

namespace csa {
namespace {

constexpr int kKlRows = 32;      // selected rows per step of the query kernel
constexpr int kKlTile = 128;     // compressed rows per d_k tile
constexpr int kKlChunk = 128;    // queries per d_k chunk


struct KlWorkspace {
  float* G;       // [Tq][topk] loss-scaled gradient of each selected slot's score
  int16_t* cmap;  // [Tq][nvis_cap] slot of each visible compressed row, -1 if not selected
};

__host__ __device__ inline size_t kl_ws_bytes(long long Tq, int topk, int nvis_cap) {
  return static_cast<size_t>(Tq) * (static_cast<size_t>(topk) * 4 + static_cast<size_t>(nvis_cap) * 2);
}

__host__ __device__ inline KlWorkspace kl_ws_layout(void* base, long long Tq, int topk) {
  KlWorkspace w;
  w.G = static_cast<float*>(base);
  w.cmap = reinterpret_cast<int16_t*>(static_cast<unsigned char*>(base) + static_cast<size_t>(Tq) * topk * 4);
  return w;
}

// Sum / max over the 256 threads (block-uniform call); red holds kWaves floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ----------------------------------------------------------------------------- per query

// s_waitcnt vmcnt(2 * later): at most `later` later steps' gathers (two per
// wavefront each) still in flight
__device__ __forceinline__ void wait_gathers(int later) {
  if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0F74);
  else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F72);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Registers held to five wavefronts per SIMD, so the top-k <= 512 instance (27 KiB of LDS,
// six workgroups' worth per CU) runs five workgroups per CU instead of four: 96 registers
// per lane, four of them spilled, 0.76 against 0.77-0.78 ms on the 16k pack (six, with 21
// spilled, 0.89 ms).  The larger instance stays at two workgroups per CU (57 KiB of LDS).
template <int NC, int KB>  // cmp_idx row chunks of kThreads entries; K stage buffers
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5))) void kl_query_kernel(
    const uint16_t* __restrict__ q_I, const uint16_t* __restrict__ w, const uint16_t* __restrict__ k_cmp,
    const int32_t* __restrict__ cmp_idx, const float* __restrict__ attn_l1, int topk, int Tq, int Tc,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp, int B,
    int global_start, int r, float loss_scale, uint16_t* __restrict__ d_q, float* __restrict__ d_w,
    float* __restrict__ loss, void* ws_base, int nvis_cap) {
  static_assert(KB >= 2 && KB <= 3, "stage buffers");
  constexpr int kCap = NC * kThreads;  // largest selection this instance handles
  __shared__ __attribute__((aligned(1024))) unsigned char kst[KB][kKlRows * 256];
  __shared__ int32_t crow[kCap];
  __shared__ float sI[kWaves][kCap];  // per-wavefront partial scores; row 0 then holds G
  __shared__ uint32_t wsum[kWaves];
  __shared__ float red[kWaves];

  const int i = static_cast<int>(blockIdx.x);
  if (i >= Tq) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int head = 16 * wave + n;
  const KlWorkspace ws = kl_ws_layout(ws_base, Tq, topk);

  int vals[NC];
  const int32_t* row = cmp_idx + static_cast<long long>(i) * topk;
#pragma unroll
  for (int ch = 0; ch < NC; ++ch) {
    const int j = ch * kThreads + tid;
    vals[ch] = (j < topk) ? row[j] : -1;
  }
  // q^T as the B operand of u^T = K . q^T: q_I[i, head, 32 ks + 8 g .. + 7]
  bf16x8 qb[4];
  const uint16_t* qrow = q_I + (static_cast<long long>(i) * 64 + head) * 128 + 8 * g;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  const float wh = bf16_bits_to_f32(w[static_cast<long long>(i) * 64 + head]);
  // pass 1 takes u = q . K^T (heads 16 w + 4 g + j of row n in lane (n, g)): their weights
  float wq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wq[j] = bf16_bits_to_f32(w[static_cast<long long>(i) * 64 + 16 * wave + 4 * g + j]);

  // segment and visible compressed range
  int count = 0;
  for (int base = 0; base < B; base += 64) count += __popcll(__ballot(base + lane < B && cu_q[base + lane] <= i));
  const int b = __builtin_amdgcn_readfirstlane(count - 1);
  const int t = global_start + i;
  const int s = cu_kv[b];
  const int cmp_lo = cu_cmp[b];
  const int nvis = max(0, min((t - s + 1) / r, min(cu_cmp[b + 1], Tc) - cmp_lo));
  const int n_sel = compact_rows(vals, topk, min(cu_cmp[B], Tc), crow, wsum);

  // selection map of the visible rows for the key-major d_k pass
  if (nvis_cap > 0) {
    int16_t* m = ws.cmap + static_cast<long long>(i) * nvis_cap;
    const int nv = min(nvis, nvis_cap);
    for (int v = tid; v < nv; v += kThreads) m[v] = -1;
    __syncthreads();  // the -1 fill lands before the entries below
    for (int j = tid; j < n_sel; j += kThreads) {
      const int v = crow[j] - cmp_lo;
      if (v >= 0 && v < nv) m[v] = static_cast<int16_t>(j);
    }
  }

  const int nsteps = (n_sel + kKlRows - 1) / kKlRows;
  const uint32_t kbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(CSA_LDS(kst)));
  // step sb into buffer bf: wavefront w loads stage rows 8 w .. 8 w + 7 (two 1 KiB
  // instructions of 4 rows); rows past the selection re-read the first selected row
  auto stage = [&](int sb, int bf) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int rr = 8 * wave + 4 * v + (lane >> 4);
      int j = sb * kKlRows + rr;
      j = (j < n_sel) ? j : 0;
      const uint16_t* src = k_cmp + static_cast<long long>(crow[j]) * 128 + kchunk(rr, lane & 15) * 8;
      gather16_to_lds(src, kbase + static_cast<uint32_t>(bf * kKlRows * 256 + (8 * wave + 4 * v) * 256));
    }
  };
  // u^T[16 rows x 16 heads] of row block cb: lane (n, g) gets rows 16 cb + 4 g + j of head `head`
  auto scores = [&](const unsigned char* kb, int cb, f32x4& acc) {
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const int rr = 16 * cb + n;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + rr * 256 + kchunk(rr, 4 * ks + g) * 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], acc, 0, 0, 0);
    }
  };

  // ---- pass 1: scores.  KB - 1 steps of gathers in flight; the bare barrier keeps
  // the later steps' gathers outstanding across it.
#pragma unroll
  for (int d = 0; d < KB - 1; ++d)
    if (d < nsteps) stage(d, d);
  for (int sb = 0; sb < nsteps; ++sb) {
    const int bf = sb % KB;
    wait_gathers(min(nsteps - 1 - sb, KB - 2));
    tile_barrier();  // step sb landed everywhere; the buffer of step sb - 1 is free
    if (sb + KB - 1 < nsteps) stage(sb + KB - 1, (sb + KB - 1) % KB);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      // u[16 heads x 16 rows] = q . K^T: the same fragments as u^T with the operands
      // swapped; the head sum is then four in-lane terms and one 4-lane reduction
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int rr = 16 * cb + n;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kst[bf] + rr * 256 + kchunk(rr, 4 * ks + g) * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[ks], kf, acc, 0, 0, 0);
      }
      float v = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) v += wq[j] * fmaxf(acc[j], 0.f);
      v = quad_sum(v);
      if (g == 0) sI[wave][sb * kKlRows + rr] = v;
    }
  }
  __syncthreads();

  // ---- softmax over the selected rows, normalised targets, G, loss
  float mx = -__builtin_huge_valf(), psum = 0.f;
  for (int j = tid; j < n_sel; j += kThreads) {
    const float I = (sI[0][j] + sI[1][j]) + (sI[2][j] + sI[3][j]);
    sI[0][j] = I;
    mx = fmaxf(mx, I);
    psum += attn_l1[static_cast<long long>(i) * topk + j];
  }
  mx = block_max(mx, red);
  psum = block_sum(psum, red);
  float esum = 0.f;
  for (int j = tid; j < n_sel; j += kThreads) esum += __expf(sI[0][j] - mx);
  esum = block_sum(esum, red);
  const bool live = n_sel > 0 && psum > 0.f;
  const float lse = mx + __logf(esum);
  float kl = 0.f;
  for (int j = tid; j < n_sel; j += kThreads) {
    const float ls = sI[0][j] - lse;                    // log softmax
    const float ph = live ? attn_l1[static_cast<long long>(i) * topk + j] / psum : 0.f;
    if (ph > 0.f) kl += ph * (__logf(ph) - ls);
    const float G = live ? loss_scale * (__expf(ls) - ph) : 0.f;
    sI[0][j] = G;
    ws.G[static_cast<long long>(i) * topk + j] = G;
  }
  kl = block_sum(kl, red);  // its barriers also publish G
  if (loss != nullptr && tid == 0) loss[i] = live ? kl : 0.f;

  // ---- pass 2: d_w and d_q^T = K^T . M^T, M^T[row, head] = G_row w_head [u > 0]
  f32x4 dq[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) dq[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dw = 0.f;
  // K^T transpose reads: source lane m of lane group g points at stage row 4 g + m / 4
  // (+ 16 for the second row block), dims 16 db + 4 (m % 4)
  const int trow = 4 * g + (n >> 2);
#pragma unroll
  for (int d = 0; d < KB - 1; ++d)
    if (live && d < nsteps) stage(d, d);
  for (int sb = 0; live && sb < nsteps; ++sb) {
    const int bf = sb % KB;
    wait_gathers(min(nsteps - 1 - sb, KB - 2));
    tile_barrier();
    if (sb + KB - 1 < nsteps) stage(sb + KB - 1, (sb + KB - 1) % KB);
    bf16x8 mfrag;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      f32x4 acc;
      scores(kst[bf], cb, acc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float G = sI[0][sb * kKlRows + 16 * cb + 4 * g + j];  // 0 past the selection? see below
        const bool in = sb * kKlRows + 16 * cb + 4 * g + j < n_sel;
        const float Gv = in ? G : 0.f;
        dw += Gv * fmaxf(acc[j], 0.f);
        mfrag[4 * cb + j] = static_cast<__bf16>(acc[j] > 0.f ? Gv * wh : 0.f);
      }
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int c0 = 2 * db + ((n & 3) >> 1);  // 16-byte chunk of dims 16 db + 4 (n % 4)
      const unsigned char* p0 = kst[bf] + trow * 256 + kchunk(trow, c0) * 16 + (n & 1) * 8;
      const unsigned char* p1 = kst[bf] + (trow + 16) * 256 + kchunk(trow + 16, c0) * 16 + (n & 1) * 8;
      const bf16x4 lo = ds_read_tr(p0);
      const bf16x4 hi = ds_read_tr(p1);
      const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      dq[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, mfrag, dq[db], 0, 0, 0);
    }
  }
  // d_w[head]: the lane quad holds disjoint rows
  dw = quad_sum(dw);
  if (g == 0) d_w[static_cast<long long>(i) * 64 + head] = dw;
  // d_q rows leave as whole rows: staged in the (now idle) K stage buffers as 64 rows of
  // 256 bytes, 16-byte chunk c of row h at chunk c ^ (h & 15) (conflict-free writes),
  // then stored 1 KiB per instruction.  A wavefront's rows are its own heads, so after
  // the barrier that frees the buffers it reads back only what it wrote itself.  The
  // stores are non-temporal (nothing in this call reads d_q back, and the lines then
  // leave the caches before the key rows the next queries gather): 0.734 against
  // 0.753 ms for the whole call on the 16k pack (six same-box A/B pairs); the same hint
  // on the q_I loads measured slower (the d_k kernel re-reads q_I).
  lds_barrier();
  unsigned char* st = &kst[0][0];
#pragma unroll
  for (int db = 0; db < 8; ++db) {  // dims 16 db + 4 g + j of head `head`
    const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16_bits(dq[db][0])) |
                        (static_cast<uint32_t>(f32_to_bf16_bits(dq[db][1])) << 16);
    const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16_bits(dq[db][2])) |
                        (static_cast<uint32_t>(f32_to_bf16_bits(dq[db][3])) << 16);
    const int c = 2 * db + (g >> 1);
    *reinterpret_cast<uint2*>(st + head * 256 + ((c ^ (head & 15)) << 4) + (g & 1) * 8) = make_uint2(w0, w1);
  }
  uint16_t* obase = d_q + (static_cast<long long>(i) * 64 + 16 * wave) * 128;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 4 * k + (lane >> 4), c = lane & 15;  // row 16 wave + r, chunk c
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = *reinterpret_cast<const u32x4*>(st + (16 * wave + r) * 256 + ((c ^ r) << 4));
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + r * 128 + c * 8));
  }
}

// ----------------------------------------------------------------------------- d_k

// Work items: the local queries of a segment in chunks of 128; a chunk's group holds
// the compressed tiles (128 rows) visible to its last query.  Group g goes to XCD g % 8
// (the hardware deals workgroup x to XCD x % 8, in order) and takes consecutive
// workgroup slots there, so the chunk's q rows are shared in one L2.
struct KlGroup {
  int T0, T1, n_t;
};

__device__ __forceinline__ KlGroup kl_group(int b, int c, const int32_t* __restrict__ cu_q,
                                            const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ cu_cmp,
                                            int global_start, int r, int Tc) {
  KlGroup gr;
  const int s = cu_kv[b];
  const int qa = cu_q[b], qb = cu_q[b + 1];
  gr.T0 = global_start + qa + kKlChunk * c;
  gr.T1 = global_start + min(qb, qa + kKlChunk * (c + 1)) - 1;
  const int Lc = max(0, min(cu_cmp[b + 1], Tc) - cu_cmp[b]);
  const int nvis = max(0, min((gr.T1 - s + 1) / r, Lc));
  gr.n_t = (nvis + kKlTile - 1) / kKlTile;
  return gr;
}

__device__ __forceinline__ int kl_chunks(int b, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv) {
  const int Lq = cu_q[b + 1] - cu_q[b];
  return (Lq > 0 && cu_kv[b + 1] > cu_kv[b]) ? (Lq + kKlChunk - 1) / kKlChunk : 0;
}

__device__ __forceinline__ int kl_wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(x, o, 64);
    if (lane >= o) x += v;
  }
  return x;
}

// One tile of 128 compressed rows x a chunk of queries.  Wavefront w holds rows
// 32 w .. 32 w + 31 of the tile (two 16-row blocks) as the B operand of
// u[heads x rows] = q . K^T; per query the 64 q rows are staged in LDS and
//   d_k^T[128 dims x rows] += q^T[dims x heads] . M[heads x rows],  M = G w [u > 0],
// with M taken straight from the u accumulators (k-slot 8 g + j of head step hs is head
// 32 hs + 4 g + j for j < 4, 32 hs + 16 + 4 g + (j - 4) otherwise) and q^T by
// transpose reads in the same head order.
__global__ __launch_bounds__(kThreads) void kl_dk_kernel(
    const uint16_t* __restrict__ q_I, const uint16_t* __restrict__ w, const uint16_t* __restrict__ k_cmp, int topk,
    int Tq, int Tc, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_kv,
    const int32_t* __restrict__ cu_cmp, int B, int global_start, int r, const void* ws_base, int nvis_cap,
    float* __restrict__ d_k) {
  __shared__ __attribute__((aligned(1024))) unsigned char qs[2][64 * 256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;

  // ---- work item
  const int x = static_cast<int>(blockIdx.x);
  const int xcd = x & 7, slot = x >> 3;
  int seg = -1, chunk = 0, local = 0, off = 0, g_base = 0;
  for (int b = 0; b < B && seg < 0; ++b) {
    const int nch = kl_chunks(b, cu_q, cu_kv);
    for (int cbase = 0; cbase < nch && seg < 0; cbase += 64) {
      const int c = cbase + lane;
      int v = 0;
      if (c < nch && ((g_base + c) & 7) == xcd) v = kl_group(b, c, cu_q, cu_kv, cu_cmp, global_start, r, Tc).n_t;
      const int incl = kl_wave_incl_scan(v) + off;
      const unsigned long long hit = __ballot(v > 0 && incl - v <= slot && slot < incl);
      if (hit != 0ull) {
        const int src = __builtin_ctzll(hit);
        seg = b;
        chunk = cbase + src;
        local = slot - __shfl(incl - v, src, 64);
      }
      off = __shfl(incl, 63, 64);
    }
    g_base += nch;
  }
  seg = __builtin_amdgcn_readfirstlane(seg);
  if (seg < 0) return;
  chunk = __builtin_amdgcn_readfirstlane(chunk);
  local = __builtin_amdgcn_readfirstlane(local);
  const KlGroup gr = kl_group(seg, chunk, cu_q, cu_kv, cu_cmp, global_start, r, Tc);
  const int s = cu_kv[seg];
  const int cb0 = cu_cmp[seg];
  const int Lc = min(cu_cmp[seg + 1], Tc) - cb0;
  const int c0 = cb0 + kKlTile * local;
  const int c_end = min(c0 + kKlTile, cb0 + Lc);
  // the first query that sees row c0 sits at segment position (c0 - cb0 + 1) r - 1
  const long long first = static_cast<long long>(s) + static_cast<long long>(c0 - cb0 + 1) * r - 1;
  const int i0 = static_cast<int>(max(static_cast<long long>(gr.T0), first)) - global_start;
  const int i1 = gr.T1 - global_start + 1;
  if (i0 >= i1) return;
  const KlWorkspace ws = kl_ws_layout(const_cast<void*>(ws_base), Tq, topk);

  // B operand rows of this wavefront: K[c0 + 32 wave + 16 cb + n, 32 ks + 8 g ..]
  bf16x8 kreg[2][4];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = c0 + 32 * wave + 16 * cb + n;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kreg[cb][ks] = (c < c_end) ? *reinterpret_cast<const bf16x8*>(k_cmp + static_cast<long long>(c) * 128 + 32 * ks + 8 * g)
                                 : bf16x8{};
  }

  const uint32_t qbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(CSA_LDS(qs)));
  // q rows of query i into buffer bf: 16 instructions of 4 rows (1 KiB), 4 per wavefront
  auto stage = [&](int i, int bf) {
    const uint16_t* src = q_I + static_cast<long long>(i) * 64 * 128;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int u = 4 * wave + v;
      const int row = 4 * u + (lane >> 4);
      const uint32_t loff = static_cast<uint32_t>(row * 256 + kchunk(row, lane & 15) * 16);
      row_to_lds(src, loff, qbase + static_cast<uint32_t>(bf * 64 * 256 + u * 1024));
    }
  };
  // G of this lane's rows (one per row block) for query i, from the selection map
  auto load_slots = [&](int i, int (&sl)[2]) {
    const int t = global_start + i;
    const int vis = min(min((t - s + 1) / r, Lc), nvis_cap);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int v = c0 + 32 * wave + 16 * cb + n - cb0;
      sl[cb] = (v < vis && c0 + 32 * wave + 16 * cb + n < c_end) ? ws.cmap[static_cast<long long>(i) * nvis_cap + v]
                                                                  : -1;
    }
  };
  auto load_G = [&](int i, const int (&sl)[2], float (&G)[2]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) G[cb] = (sl[cb] >= 0) ? ws.G[static_cast<long long>(i) * topk + sl[cb]] : 0.f;
  };
  // head weights of the u rows this lane holds: heads 16 mb + 4 g + j
  auto load_w = [&](int i, float (&wv)[4][4]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const uint2 v = *reinterpret_cast<const uint2*>(w + static_cast<long long>(i) * 64 + 16 * mb + 4 * g);
      wv[mb][0] = __uint_as_float(v.x << 16);
      wv[mb][1] = __uint_as_float(v.x & 0xffff0000u);
      wv[mb][2] = __uint_as_float(v.y << 16);
      wv[mb][3] = __uint_as_float(v.y & 0xffff0000u);
    }
  };

  f32x4 acc[8][2];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[db][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  int sl[2];
  float G[2], Gn[2];
  float wv[4][4], wn[4][4];
  load_slots(i0, sl);
  load_G(i0, sl, G);
  load_w(i0, wv);
  stage(i0, 0);
  for (int i = i0; i < i1; ++i) {
    const int bf = (i - i0) & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();  // q rows of query i landed; buffer bf ^ 1 is free
    if (i + 1 < i1) {
      stage(i + 1, bf ^ 1);
      load_slots(i + 1, sl);
      load_w(i + 1, wn);
    }
    const unsigned char* qb = qs[bf];
    if (__any(G[0] != 0.f || G[1] != 0.f)) {  // wave-uniform: the MFMAs and transpose reads need every lane
      // u[heads x rows] and M = G w [u > 0] as bf16 B fragments per head step
      bf16x8 mf[2][2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int row = 16 * mb + n;
        bf16x8 a[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          a[ks] = *reinterpret_cast<const bf16x8*>(qb + row * 256 + kchunk(row, 4 * ks + g) * 16);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], kreg[cb][ks], u, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            mf[cb][mb >> 1][4 * (mb & 1) + j] = static_cast<__bf16>(u[j] > 0.f ? G[cb] * wv[mb][j] : 0.f);
        }
      }
      // d_k^T += q^T . M: A = q^T for dims 16 db + n, heads of step hs (two transpose reads)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const int r0 = 32 * hs + 4 * g + (n >> 2), r1 = r0 + 16;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const int c = 2 * db + ((n & 3) >> 1);
          const bf16x4 lo = ds_read_tr(qb + r0 * 256 + kchunk(r0, c) * 16 + (n & 1) * 8);
          const bf16x4 hi = ds_read_tr(qb + r1 * 256 + kchunk(r1, c) * 16 + (n & 1) * 8);
          const bf16x8 aq = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            acc[db][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, mf[cb][hs], acc[db][cb], 0, 0, 0);
        }
      }
    }
    if (i + 1 < i1) {
      load_G(i + 1, sl, Gn);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) G[cb] = Gn[cb];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[mb][j] = wn[mb][j];
    }
  }
  // d_k^T column = row c0 + 32 wave + 16 cb + n, dims 16 db + 4 g + j
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = c0 + 32 * wave + 16 * cb + n;
    if (c >= c_end) continue;
    float* dst = d_k + static_cast<long long>(c) * 128 + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) atomicAdd(dst + 16 * db + j, acc[db][cb][j]);
  }
}

__global__ void kl_zero_kernel(float* __restrict__ p, long long n) {
  for (long long k = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; k < n;
       k += static_cast<long long>(gridDim.x) * blockDim.x)
    p[k] = 0.f;
}

}  // namespace

bool kl_shape_supported(int H_I, int d_I, int dtype) { return dtype == 1 && H_I == 64 && d_I == 128; }

size_t kl_workspace_bytes(int Tq, int topk, int nvis_cap) { return kl_ws_bytes(Tq, topk, nvis_cap); }

// ---------------------------------------------------------------- library-held scratch

// The workspace of the allocation-free entry point: a file-scope device array that
// every GPU the library runs on holds from the first use until the process ends.  The
// query kernel writes every slot the d_k kernel reads, so no clearing is needed.  All
// calls on one GPU share it: calls that overlap on one GPU (on different streams)
// race.  In host code the array's name is a host-side stand-in, never a device
// address: kernels get the pointer hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kKlScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t kl_scratch(void** ptr) {
  int dev = 0;
  if (const hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = (g_scratch_err[dev] == hipSuccess) ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_indexer_kl_grad(const void* q_I, const void* w, const void* k_cmp, const int32_t* cmp_idx,
                                  const float* attn_l1, int topk, int Tq, int Tc, const int32_t* cu_q,
                                  const int32_t* cu_kv, const int32_t* cu_cmp, int B, int global_start, int r,
                                  int max_seqlen_kv, float loss_scale, void* d_q, float* d_w, float* d_k, float* loss,
                                  int nvis_cap, void* workspace, hipStream_t s) {
  if (d_k != nullptr && Tc > 0) {
    const long long nk = static_cast<long long>(Tc) * 128;
    hipLaunchKernelGGL(kl_zero_kernel, dim3(static_cast<unsigned>(min(4096LL, (nk + 255) / 256))), dim3(256), 0, s,
                       d_k, nk);
  }
  if (Tq <= 0) return hipGetLastError();
  const auto* q16 = static_cast<const uint16_t*>(q_I);
  const auto* w16 = static_cast<const uint16_t*>(w);
  const auto* k16 = static_cast<const uint16_t*>(k_cmp);
  // two K stage buffers (a third measured slower)
  auto kq = (topk <= 2 * kThreads) ? kl_query_kernel<2, 2> : kl_query_kernel<kMaxTopk / kThreads, 2>;
  hipLaunchKernelGGL(kq, dim3(Tq), dim3(kThreads), 0, s, q16, w16, k16, cmp_idx, attn_l1, topk, Tq, Tc, cu_q, cu_kv,
                     cu_cmp, B, global_start, r, loss_scale, static_cast<uint16_t*>(d_q), d_w, loss, workspace,
                     nvis_cap);
  // d_k: an upper bound of the workgroup slots per XCD (groups <= Tq / 128 + B, each with
  // at most ceil(max_seqlen_kv / r / 128) tiles)
  const long long groups = (static_cast<long long>(Tq) + kKlChunk - 1) / kKlChunk + B;
  const long long n_t = (static_cast<long long>(max(1, max_seqlen_kv)) / r + kKlTile - 1) / kKlTile;
  const long long grid = (groups + 7) / 8 * n_t * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (grid > 0)
    hipLaunchKernelGGL(kl_dk_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, q16, w16, k16, topk, Tq,
                       Tc, cu_q, cu_kv, cu_cmp, B, global_start, r, static_cast<const void*>(workspace), nvis_cap, d_k);
  return hipGetLastError();
}

}  // namespace csa
