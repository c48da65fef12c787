// Stage 3: varlen GQA verify attention over a paged KV cache, with the window's K/V
// appended to the cache.
//
// Sources: "DFlash 到 DSpark in SGLang：解码提速 4.3×，以及 DeepSeek-V4 支持"
// (yichizhang.dev, AI-Infra-Visualized), section "Ragged verify under full CUDA graphs",
// and section 3 of the devpress.csdn.net DSpark-in-SGLang article: each packed verify
// token attends only to its own request's KV, delimited by cu_seqlens.
//
// bf16 path (D in {64, 128}, page_size a power of two >= 32, B <= 1024): attn_sk_kernel
//   * Work: a segment is one (request b, kv head g); it is cut into tiles of 32 keys.
//     Every K/V byte of a segment is read once for ALL window rows and ALL Hq/Hkv query
//     heads of the group: the (window row, head-in-group) pairs are the N side of the
//     MFMA tiles (NB blocks of 16 columns, NB chosen per segment from its window).
//   * Balance: persistent grid, one workgroup per CU slot; all segments form one weighted
//     sequence (each segment = its tiles + a fixed start cost of kSegCost tile units) and
//     workgroup p owns the contiguous share [W p / P, W (p+1) / P) (stream-K over bytes AND
//     per-segment overhead; with W < P, unit p alone).  A segment that lies inside one
//     share is finished by that workgroup; a segment cut by share boundaries leaves at most
//     one partial per workgroup side and attn_merge_kernel combines them.  No workgroup
//     ever waits for another.  At a segment's end the 4 waves park (m, l, o) in LDS slices
//     and combine them after one barrier.
//   * Inside a workgroup the 4 waves take the segment's tiles round-robin, one wave per
//     SIMD.  Each wave alternates two register buffers, so the next tile (16 KB at
//     D = 128) is in flight while it computes the current one (NB = 4 keeps one buffer: its
//     accumulators take the registers).  Page numbers are scalar loads from the block
//     table; operand addresses are a uniform SGPR base per tile plus lane-constant 32-bit
//     offsets (global loads, no 64-bit lane arithmetic).
//   * Scores are computed transposed, S^T = K Q^T, with mfma_f32_16x16x32_bf16 (K rows are
//     the A operand, 16-byte loads from the (page, head) block, a contiguous
//     [page_size, D] tile in this cache layout).  Row m of 16-key block mb holds key
//     8(m/4) + 4mb + m%4, so each lane's accumulator holds 8 CONSECUTIVE keys for one
//     query column; those probabilities are then directly the B operand of
//     O^T = V^T P^T, and the V^T operand is one 16-byte load per lane from the transposed
//     per-page V tile [D, page_size].  No LDS round trip on the streaming path.
//   * Online softmax in the log2 domain with lazy rescaling: the running max only moves
//     (and the accumulators are only rescaled) when a tile's max exceeds it by more than
//     2^8, so most tiles cost no rescale.  P is narrowed to bf16 with v_cvt_pk_bf16_f32.
//   * The 1-2 tiles of a segment that reach past the cached context take the window keys
//     from k_new / v_new (packed rows) and apply the causal mask.  The window K/V is
//     appended to the cache (positions L .. L+w-1) by attn_merge_kernel, after every read.
//   * The V cache is transposed in column blocks of 32 slots ([D][32] per block), so each
//     tile's V^T operand is one contiguous 8 KB block, like its K rows: every load
//     instruction fetches full cache lines.
// Any other dtype / shape uses attn_generic_kernel (one workgroup per query column, one
// key per thread, online softmax), which is also the float32 path.
#include "rva_common.h"

#include <algorithm>
#include <mutex>

namespace rva {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kTile = 32;     // keys per tile
constexpr int kMaxB = 1024;   // requests the persistent path takes
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.f;  // lazy-rescale threshold, log2 units
// Fixed cost of starting a segment (Q load, pipeline fill, merge, stores), in tile units:
// shares are balanced over tiles + kSegCost per segment.
constexpr int kSegCost = 16;

struct ReqInfo {
  int L, r0, w, ok;
};

// Validates request b's metadata; raises device-status bits when `report`.
__device__ __forceinline__ ReqInfo req_info(const AttnArgs& a, int b, bool report) {
  ReqInfo r;
  r.L = a.context_lens[b];
  r.r0 = a.cu[b];
  r.w = a.cu[b + 1] - r.r0;
  r.ok = 1;
  if (r.w < 1 || r.w > a.max_window) {
    if (report) flag(a.status, RVA_DEV_BAD_WINDOW);
    r.ok = 0;
  } else if (r.L < 0 || r.L + r.w > a.max_pages * a.page_size) {
    if (report) flag(a.status, RVA_DEV_BAD_CONTEXT);
    r.ok = 0;
  } else if (r.r0 < 0 || r.r0 + r.w > a.max_rows) {
    if (report) flag(a.status, RVA_DEV_BAD_ROWS);
    r.ok = 0;
  }
  return r;
}

__device__ __forceinline__ short8 load16(const uint16_t* p) { return *reinterpret_cast<const short8*>(p); }

// Global-address-space views: loads through them become global_load (not flat) with a
// uniform 64-bit base in SGPRs and a 32-bit per-lane offset.
typedef const __attribute__((address_space(1))) uint16_t* gptr16;
__device__ __forceinline__ gptr16 as_global(const void* p) {
  return reinterpret_cast<gptr16>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ short8 gload16(gptr16 base, uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(1))) short8*>(base + off);
}

// V cache: transposed in column blocks of vblk(P) slots, element (page, g, slot, d) at
// ((page * Hkv + g) * P + (slot / VB) * VB) * D + d * VB + slot % VB.
__host__ __device__ __forceinline__ int vblk(int P) { return P % 32 == 0 ? 32 : P; }
__device__ __forceinline__ size_t v_index(int pg, int g, int Hkv, int P, int D, int slot, int d) {
  const int VB = vblk(P);
  return (size_t(pg) * Hkv + g) * P * D + size_t(slot / VB) * VB * D + size_t(d) * VB + slot % VB;
}

__device__ __forceinline__ int page_of(const AttnArgs& a, int b, int p, bool& bad) {
  const int pg = a.block_table[size_t(b) * a.max_pages + p / a.page_size];
  if (pg < 0 || pg >= a.num_pages) {
    bad = true;
    return -1;
  }
  return pg;
}

// ------------------------------------------------------------------ work split
struct ReqTable {
  int nt[kMaxB];       // tiles per segment of request b (0 if the request is invalid)
  int pre[kMaxB + 1];  // exclusive prefix of Hkv * span(b), span = nt + kSegCost (0 if nt = 0):
                       // first work unit of request b in the weighted sequence
  int L[kMaxB];
  int r0[kMaxB];
  int w[kMaxB];
};

// Work units of one segment: its tiles plus the fixed start cost (none if it has no tiles).
__device__ __forceinline__ int seg_span(int nt) { return nt > 0 ? nt + kSegCost : 0; }

// Every workgroup (of both kernels) builds the same table from the same device data.
__device__ __forceinline__ void build_table(const AttnArgs& a, ReqTable& t, bool report) {
  __shared__ int part[kThreads];
  const int tid = threadIdx.x, B = a.B;
  for (int b = tid; b < B; b += kThreads) {
    const ReqInfo ri = req_info(a, b, report);
    t.L[b] = ri.L;
    t.r0[b] = ri.r0;
    t.w[b] = ri.w;
    t.nt[b] = ri.ok ? (ri.L + ri.w + kTile - 1) / kTile : 0;
  }
  __syncthreads();
  const int per = (B + kThreads - 1) / kThreads;
  const int b0 = tid * per;
  int run = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < B) run += seg_span(t.nt[b0 + i]) * a.Hkv;
  part[tid] = run;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int acc = tid > 0 ? part[tid - 1] : 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < B) {
      t.pre[b0 + i] = acc;
      acc += seg_span(t.nt[b0 + i]) * a.Hkv;
    }
  if (tid == kThreads - 1) t.pre[B] = part[kThreads - 1];
  __syncthreads();
}

// Workgroup p's share of the T weighted units is [share_lo(p), share_lo(p + 1)); share_owner
// is the workgroup whose share holds unit x.  With at least as many units as workgroups the
// shares are the even split floor(T p / P), none of them empty.  With fewer (a small batch
// of short contexts), workgroup p < T takes unit p alone and the others take nothing: an
// even split would leave empty shares between non-empty ones, and the merge of a cut
// segment reads one partial from every workgroup from its first to its last share.
__device__ __forceinline__ int share_lo(int T, int P, int p) {
  return T >= P ? int((long long)T * p / P) : min(p, T);
}
__device__ __forceinline__ int share_owner(int T, int P, int x) {
  return T >= P ? int(((long long)(x + 1) * P - 1) / T) : x;
}

// Largest b with pre[b] <= x (skips requests without tiles).
__device__ __forceinline__ int find_req(const ReqTable& t, int B, int x) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.pre[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------------ tile math
template <int D, int NB, bool MASK>
__device__ __forceinline__ void tile_compute(const short8 (&kop)[2][D / 32], const short8 (&vop)[D / 16],
                                             const short8 (&qop)[NB][D / 32], f32x4 (&oacc)[D / 16][NB],
                                             float (&m)[NB], float (&l)[NB], float sl2, int key0,
                                             const int (&limit)[NB], int lq) {
  constexpr int DS = D / 32, DB = D / 16;
  f32x4 s[2][NB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < DS; ++k)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[mb][k]),
                                                      __builtin_bit_cast(bf16x8, qop[nb][k]), acc, 0, 0, 0);
      s[mb][nb] = acc;
    }
  // this lane: column lc, keys key0 + 8 lq + 4 mb + t
  float sc[NB][8];
  bool need = false;
  float mt[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float v = s[mb][nb][t] * sl2;
        if (MASK && key0 + 8 * lq + 4 * mb + t > limit[nb]) v = -INFINITY;
        sc[nb][mb * 4 + t] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mt[nb] = mx;
    need |= mx > m[nb] + kRescale;
  }
  if (__ballot(need)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float mn = fmaxf(m[nb], mt[nb]);
      if (mn != m[nb]) {
        const float alpha = (m[nb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[nb] - mn);
        l[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db][nb] *= alpha;
        m[nb] = mn;
      }
    }
  }
  short8 pop[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float ps = 0.f;
    uint32_t packed[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // two probabilities per v_cvt_pk_bf16_f32
      f32x2 p2;
      p2[0] = __builtin_amdgcn_exp2f(sc[nb][2 * i] - m[nb]);
      p2[1] = __builtin_amdgcn_exp2f(sc[nb][2 * i + 1] - m[nb]);
      if (MASK && m[nb] == -INFINITY) p2 = f32x2{0.f, 0.f};
      ps += p2[0] + p2[1];
      packed[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p2, bf16x2));
    }
    l[nb] += ps;
    pop[nb] = __builtin_bit_cast(short8, packed);
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      oacc[db][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop[db]),
                                                             __builtin_bit_cast(bf16x8, pop[nb]), oacc[db][nb], 0, 0, 0);
}

// Key held by A-operand row m of 16-key block mb (see the file comment).
__device__ __forceinline__ int row_key(int m, int mb) { return 8 * (m >> 2) + 4 * mb + (m & 3); }

// Lane-constant element offsets of the fast-path operands inside one (page, head) block.
template <int D>
struct LaneOffsets {
  uint32_t k[2];  // + 32 k per MFMA k-step (immediate offsets)
  uint32_t v;     // + 512 db per 16-row block of the tile's [D][32] V^T block
};

// One 32-key tile: K rows [32][D] and the V^T block [D][32], each 8 KB contiguous (D = 128).
template <int D>
__device__ __forceinline__ void load_fast(gptr16 kbase, gptr16 vbase, const LaneOffsets<D>& lo,
                                          short8 (&kop)[2][D / 32], short8 (&vop)[D / 16]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int k = 0; k < D / 32; ++k) kop[mb][k] = gload16(kbase, lo.k[mb] + k * 32);
#pragma unroll
  for (int db = 0; db < D / 16; ++db) vop[db] = gload16(vbase, lo.v + uint32_t(db * 16 * 32));
}

// Tile that reaches past the cached context.  The tile lies inside one page, so one page
// lookup serves its cached keys (p < L); window keys (L <= p < Lw) come from the packed
// k_new / v_new rows; keys past the window (masked later) read the window's first row so
// that every lane issues a load from a valid, finite address.  Addresses are selected,
// not branched on, so all loads are in flight together.
template <int D>
__device__ __forceinline__ void load_tail(const AttnArgs& a, int b, int g, int L, int r0, int Lw, int key0, int lc,
                                          int lq, short8 (&kop)[2][D / 32], short8 (&vop)[D / 16], bool& bad) {
  const int Hkv = a.Hkv, P = a.page_size;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const uint16_t* kn = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(a.v_new);
  int pg = 0;
  if (key0 < L) {
    pg = a.block_table[size_t(b) * a.max_pages + key0 / P];
    if (pg < 0 || pg >= a.num_pages) {
      bad = true;
      pg = 0;
    }
  }
  const int slot0 = key0 % P;
  const uint16_t* kpage = kc + ((size_t(pg) * Hkv + g) * P + slot0) * D;  // key key0 + i at kpage + i*D
  const uint16_t* vtile = vc + ((size_t(pg) * Hkv + g) * P + slot0) * D;  // (d, key0 + i) at vtile + d*32 + i
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int i = row_key(lc, mb), p = key0 + i;
    const uint16_t* krow = p < L ? kpage + size_t(i) * D
                                 : kn + (size_t(r0 + (p < Lw ? p - L : 0)) * Hkv + g) * D;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) kop[mb][k] = load16(krow + k * 32 + 8 * lq);
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const int d = db * 16 + lc;
    short8 v;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = 8 * lq + t, p = key0 + i;
      const uint16_t* src = p < L ? vtile + size_t(d) * 32 + i
                                  : vn + (size_t(r0 + (p < Lw ? p - L : 0)) * Hkv + g) * D + d;
      v[t] = short(*src);
    }
    vop[db] = v;
  }
}

template <int D, int NBMAX>
struct SkShared {
  ReqTable tab;
  float m[kWaves][NBMAX * 16];
  float l[kWaves][NBMAX * 16];
  float M[NBMAX * 16];
  float Ls[NBMAX * 16];
  // per-wave partial outputs for the segment-end merge (4 slices; 2 when NBMAX = 4, the
  // other two waves add into them)
  float o[NBMAX <= 2 ? 4 : 2][NBMAX * 16][D + 4];
};

// One segment's share: tiles [t0, t0 + n) of (b, g); `full`: the whole segment (final
// output), otherwise a partial into workspace slot `slot_index`.
template <int D, int NB, int NBMAX>
__device__ __forceinline__ void run_segment(const AttnArgs& a, SkShared<D, NBMAX>& sh, int b, int g, int t0, int n, bool full,
                            int slot_index) {
  constexpr int DS = D / 32, DB = D / 16;
  // The thread index passes through an empty asm so that the lane-constant addresses below
  // are recomputed per segment instead of being hoisted to the kernel entry, where they
  // would stay live (for every instantiation) across the whole kernel.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid / kWave, lane = tid % kWave;
  const int lc = lane % 16, lq = lane / 16;
  const int L = sh.tab.L[b], r0 = sh.tab.r0[b], w = sh.tab.w[b], Lw = L + w;
  const int Hkv = a.Hkv, P = a.page_size, G = a.Hq / a.Hkv, nq = w * G;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const float sl2 = a.scale * kLog2e;
  bool bad = false;

  short8 qop[NB][DS];
  int limit[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = nb * 16 + lc;
    const bool valid = col < nq;
    limit[nb] = valid ? L + col / G : Lw - 1;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (size_t(r0 + (valid ? col / G : 0)) * a.Hq + g * G + (valid ? col % G : 0)) * D;
#pragma unroll
    for (int k = 0; k < DS; ++k) qop[nb][k] = valid ? load16(qrow + k * 32 + 8 * lq) : short8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  f32x4 oacc[DB][NB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[NB], l[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = -INFINITY;
    l[nb] = 0.f;
  }

  // ---- fully cached tiles of this share: [t0, tf); this wave takes every 4th one
  const int tf = min(t0 + n, L / kTile);
  const int nfast = max(0, tf - t0);
  const int nk = nfast > wave ? (nfast - wave + kWaves - 1) / kWaves : 0;
  const int lp = a.log2_page;
  const size_t page_elems = size_t(Hkv) * P * D;  // one physical page of K (or V), all heads
  const gptr16 kseg = as_global(kc) + size_t(g) * P * D;
  const gptr16 vseg = as_global(vc) + size_t(g) * D * P;
  LaneOffsets<D> lo;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) lo.k[mb] = uint32_t(row_key(lc, mb) * D + 8 * lq);
  lo.v = uint32_t(lc * 32 + 8 * lq);
  // block-table row through the scalar cache: page lookups are s_load (lgkmcnt), so they
  // never make a vector-memory wait drain the tile loads in flight
  const __attribute__((address_space(4))) int* btrow =
      reinterpret_cast<const __attribute__((address_space(4))) int*>(
          reinterpret_cast<uintptr_t>(a.block_table + size_t(b) * a.max_pages));
  const int num_pages = a.num_pages;
  auto page_k = [&](int k) -> int {  // physical page of this wave's k-th cached tile (clamped)
    const int kk = min(k, nk - 1);
    int pg = btrow[((t0 + wave + kWaves * kk) * kTile) >> lp];
    if (pg < 0 || pg >= num_pages) {
      bad = true;
      pg = 0;
    }
    return pg;
  };
  // Register double buffer: tile k+1 is in flight while tile k is computed (kStages = 2);
  // NB = 4 reloads one buffer (kStages = 1: its accumulators take the registers).  A third
  // buffer spills at D = 128, and a two-stage LDS ring filled by LDS DMA (two tiles in flight
  // without the registers) measured no faster on HBM data.  kC / vC hold the tail tile.
  // Loads are issued unconditionally (past the end they repeat the last tile), so every
  // path has the same number of loads outstanding and each wait is exact.
  constexpr int kStages = NB >= 4 ? 1 : 2;
  short8 kA[2][DS], vA[DB], kB[2][DS], vB[DB], kC[2][DS], vC[DB];
  int pg_next = 0;
  auto issue = [&](int k, short8 (&kb)[2][DS], short8 (&vb)[DB]) {
    const int pg = pg_next;
    pg_next = page_k(k + 1);
    const int slot0 = ((t0 + wave + kWaves * min(k, nk - 1)) * kTile) & (P - 1);
    load_fast<D>(kseg + size_t(pg) * page_elems + size_t(slot0) * D, vseg + size_t(pg) * page_elems + size_t(slot0) * D,
                 lo, kb, vb);
  };
  auto key_k = [&](int k) { return (t0 + wave + kWaves * k) * kTile; };
  // A tile that reaches past the cached context (at most one per wave) is loaded first, into
  // buffer C, so its loads overlap the first cached tile's loads; it is computed before the
  // loop starts.  Both branches leave the same loads in flight.
  const int jt = nfast + ((wave - nfast) % kWaves + kWaves) % kWaves;
  // NB = 4 keeps too many accumulators for a third buffer: its tail goes after the loop
  constexpr bool kTailFirst = NB <= 2;
  const bool has_tail = kTailFirst && jt < n;
  auto tail_compute = [&]() {
    tile_compute<D, NB, true>(kC, vC, qop, oacc, m, l, sl2, (t0 + jt) * kTile, limit, lq);
  };
  if (nk == 0) {
    if (kTailFirst && jt < n) {
      load_tail<D>(a, b, g, L, r0, Lw, (t0 + jt) * kTile, lc, lq, kC, vC, bad);
      tail_compute();
    }
  } else {
    pg_next = page_k(0);
    if (has_tail) {
      load_tail<D>(a, b, g, L, r0, Lw, (t0 + jt) * kTile, lc, lq, kC, vC, bad);
      issue(0, kA, vA);
      tail_compute();
    } else {
      issue(0, kA, vA);
    }
    if constexpr (kStages == 2) {
      for (int k = 0; k < nk; k += 2) {
        issue(k + 1, kB, vB);
        tile_compute<D, NB, false>(kA, vA, qop, oacc, m, l, sl2, key_k(k), limit, lq);
        if (k + 1 >= nk) break;
        issue(k + 2, kA, vA);
        tile_compute<D, NB, false>(kB, vB, qop, oacc, m, l, sl2, key_k(k + 1), limit, lq);
      }
    } else {
      for (int k = 0; k < nk; ++k) {
        if (k > 0) issue(k, kA, vA);
        tile_compute<D, NB, false>(kA, vA, qop, oacc, m, l, sl2, key_k(k), limit, lq);
      }
    }
  }
  if (!kTailFirst && jt < n) {
    load_tail<D>(a, b, g, L, r0, Lw, (t0 + jt) * kTile, lc, lq, kA, vA, bad);
    tile_compute<D, NB, true>(kA, vA, qop, oacc, m, l, sl2, (t0 + jt) * kTile, limit, lq);
  }
  if (bad) flag(a.status, RVA_DEV_BAD_PAGE);

  // ---- merge the 4 waves
  constexpr int S = NBMAX <= 2 ? 4 : 2;
  constexpr int ROWS = NBMAX * 16;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float sum = l[nb];
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    if (lq == 0) {
      sh.m[wave][nb * 16 + lc] = m[nb];
      sh.l[wave][nb * 16 + lc] = sum;
    }
  }
  if constexpr (S == kWaves) {
    // one slice per wave: each wave parks its unscaled (m, l, o) and a single barrier
    // separates that from the combine, which weighs slice v by 2^(m_v - M) per column
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int t = 0; t < 4; ++t) sh.o[wave][nb * 16 + lc][db * 16 + 4 * lq + t] = oacc[db][nb][t];
    __syncthreads();
  } else {
    // two slices: waves 2, 3 add into waves 0, 1's, so every wave first rescales to the
    // common maximum (the combine below then finds weights of 1 for every slice)
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = nb * 16 + lc;
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sh.m[v][col]);
      const float e = (m[nb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[nb] - M);
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db][nb] *= e;
      if (wave == 0 && lq == 0) {
        float Ls = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v)
          if (sh.m[v][col] != -INFINITY) Ls += sh.l[v][col] * __builtin_amdgcn_exp2f(sh.m[v][col] - M);
        sh.M[col] = M;
        sh.Ls[col] = Ls;
      }
    }
    if (wave < S) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int t = 0; t < 4; ++t) sh.o[wave][nb * 16 + lc][db * 16 + 4 * lq + t] = oacc[db][nb][t];
    }
    __syncthreads();
    if (wave >= S) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int t = 0; t < 4; ++t) sh.o[wave - S][nb * 16 + lc][db * 16 + 4 * lq + t] += oacc[db][nb][t];
    }
    __syncthreads();
  }
  for (int it = tid; it < nq * (D / 8); it += kThreads) {  // 8 consecutive d per thread
    const int col = it / (D / 8), d0 = (it % (D / 8)) * 8;
    float wgt[S];
    float M, Ls;
    if constexpr (S == kWaves) {
      M = -INFINITY;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sh.m[v][col]);
      Ls = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float mv = sh.m[v][col];
        wgt[v] = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - M);
        Ls += sh.l[v][col] * wgt[v];
      }
    } else {
      M = sh.M[col];
      Ls = sh.Ls[col];
#pragma unroll
      for (int v = 0; v < S; ++v) wgt[v] = 1.f;
    }
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = 0.f;
#pragma unroll
    for (int sl = 0; sl < S; ++sl)
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] += wgt[sl] * sh.o[sl][col][d0 + u];
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    if (full) {
      uint32_t pk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pk[u] = uint32_t(f32_to_bf16(v[2 * u] * inv)) | (uint32_t(f32_to_bf16(v[2 * u + 1] * inv)) << 16);
      uint16_t* o = static_cast<uint16_t*>(a.out) + (size_t(r0 + col / G) * a.Hq + g * G + col % G) * D + d0;
      *reinterpret_cast<uint4*>(o) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else {
      float* ws_o = static_cast<float*>(a.ws) + (size_t(slot_index) * ROWS + col) * D + d0;
      reinterpret_cast<float4*>(ws_o)[0] = make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      reinterpret_cast<float4*>(ws_o)[1] = make_float4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
      if (d0 == 0) {
        float* ws_lse = static_cast<float*>(a.ws) + size_t(gridDim.x) * 2 * ROWS * D;
        ws_lse[size_t(slot_index) * ROWS + col] = Ls > 0.f ? M + __log2f(Ls) : -INFINITY;
      }
    }
  }
  __syncthreads();  // LDS merge buffers are reused by the next segment
}

// Appends request b's window K/V for kv head g at cache positions L .. L+w-1 (after the main
// kernel, which took those keys from k_new / v_new).  A pass moves kThreads 4-element K
// pieces (consecutive threads: consecutive pieces of one key row, a contiguous cache row) and
// 4 kThreads V elements (consecutive threads: consecutive slots of one d, contiguous in the
// transposed column blocks).  A pass's loads are unconditional (indices clamped into the
// window; the stores check them), so they all go out before its first store: a window of up
// to 8 rows at D = 128 is one pass, one round trip.
struct AppendPass {
  uint2 kval;
  int kpg;
  int vpg[4];
  uint16_t vval[4];
};

template <int D>
__device__ __forceinline__ void append_load(const AttnArgs& a, int b, int g, int L, int r0, int w, int base,
                                            AppendPass& ap) {
  const int Hkv = a.Hkv, P = a.page_size, n = w * D, tid = threadIdx.x;
  const int* bt = a.block_table + size_t(b) * a.max_pages;
  const int ik = min(base / 4 + tid, n / 4 - 1);
  const int kj = ik / (D / 4), kd = (ik % (D / 4)) * 4;
  ap.kpg = bt[(L + kj) / P];
  ap.kval = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.k_new) + (size_t(r0 + kj) * Hkv + g) * D + kd);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int iv = min(base + e * kThreads + tid, n - 1);
    const int vj = iv % w, vd = iv / w;
    ap.vpg[e] = bt[(L + vj) / P];
    ap.vval[e] = static_cast<const uint16_t*>(a.v_new)[(size_t(r0 + vj) * Hkv + g) * D + vd];
  }
}

template <int D>
__device__ __forceinline__ void append_store(const AttnArgs& a, int g, int L, int w, int base, const AppendPass& ap) {
  const int Hkv = a.Hkv, P = a.page_size, n = w * D, tid = threadIdx.x;
  uint16_t* kcw = static_cast<uint16_t*>(a.k_cache);
  uint16_t* vcw = static_cast<uint16_t*>(a.v_cache);
  const int ik = base / 4 + tid;
  if (ik < n / 4) {
    if (ap.kpg < 0 || ap.kpg >= a.num_pages) {
      flag(a.status, RVA_DEV_BAD_PAGE);
    } else {
      const int kj = ik / (D / 4), kd = (ik % (D / 4)) * 4, p = L + kj;
      *reinterpret_cast<uint2*>(kcw + ((size_t(ap.kpg) * Hkv + g) * P + p % P) * D + kd) = ap.kval;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int iv = base + e * kThreads + tid;
    if (iv >= n || ap.vpg[e] < 0 || ap.vpg[e] >= a.num_pages) continue;  // a bad page is reported above
    const int p = L + iv % w;
    vcw[v_index(ap.vpg[e], g, Hkv, P, D, p % P, iv / w)] = ap.vval[e];
  }
}

// Per-segment record for the merge kernel: the shares holding its tiles and the partial slot
// of the first one (written every launch by the workgroup that holds the segment's tile 0).
struct SegMeta {
  int pa, pb, first_slot, pad;
};
__host__ __device__ inline size_t seg_meta_offset(int P, int nbmax, int D) {
  return size_t(P) * 2 * size_t(nbmax * 16) * (D + 1) * sizeof(float);
}

template <int D, int NBMAX>
__global__ __launch_bounds__(kThreads, 1) void attn_sk_kernel(AttnArgs a) {
  __shared__ SkShared<D, NBMAX> sh;
  build_table(a, sh.tab, blockIdx.x == 0);
  const int B = a.B, P = gridDim.x, W = sh.tab.pre[B];
  if (W == 0) return;
  const int x0 = share_lo(W, P, blockIdx.x), x1 = share_lo(W, P, blockIdx.x + 1);
  const int G = a.Hq / a.Hkv;
  for (int x = x0; x < x1;) {
    const int b = find_req(sh.tab, B, x);
    const int nt = sh.tab.nt[b], span = seg_span(nt);
    const int rel = x - sh.tab.pre[b];
    const int g = rel / span;
    const int seg_w0 = sh.tab.pre[b] + g * span, seg_w1 = seg_w0 + span;
    const int t0 = max(0, rel - g * span - kSegCost);
    const int t_end = max(0, min(x1, seg_w1) - seg_w0 - kSegCost);
    if (t_end > t0) {
      const int n = t_end - t0;
      const bool full = (t0 == 0 && t_end == nt);
      const int slot = blockIdx.x * 2 + (x0 < seg_w0 ? 1 : 0);
      const int cols = sh.tab.w[b] * G;
      if (NBMAX == 1 || cols <= 16) run_segment<D, 1, NBMAX>(a, sh, b, g, t0, n, full, slot);
      else if (NBMAX == 2 || cols <= 32) run_segment<D, (NBMAX >= 2 ? 2 : 1), NBMAX>(a, sh, b, g, t0, n, full, slot);
      else run_segment<D, NBMAX, NBMAX>(a, sh, b, g, t0, n, full, slot);
      if (t0 == 0 && threadIdx.x == 0) {
        SegMeta m;
        m.pa = blockIdx.x;
        m.pb = share_owner(W, P, seg_w1 - 1);
        m.first_slot = slot;
        m.pad = 0;
        reinterpret_cast<SegMeta*>(static_cast<char*>(a.ws) + seg_meta_offset(P, NBMAX, D))[b * a.Hkv + g] = m;
      }
    }
    x = min(x1, seg_w1);
  }
}

// Appends each segment's window K/V to the cache, combines the partials of segments cut by
// share boundaries, and zero-fills output rows [M, tier).  Blocks [0, B*Hkv) handle one
// segment each (its record from the main kernel says whether it was cut), the rest
// zero-fill.  Every load of a thread is independent of
// its others (partials are read four at a time), so a merge costs about one memory round
// trip after the record.
template <int D, int NBMAX>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(AttnArgs a, int P, int merge_blocks, int pad_blocks) {
  constexpr int ROWS = NBMAX * 16;
  const int tid = threadIdx.x;
  if (int(blockIdx.x) >= merge_blocks) {
    const int M = max(a.total_tier[0], 0);
    const int tier = min(a.total_tier[1], a.max_rows);
    const size_t row_elems = size_t(a.Hq) * D;
    for (int r = M + int(blockIdx.x) - merge_blocks; r < tier; r += pad_blocks) {
      uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + size_t(r) * row_elems);
      for (size_t k = tid; k < row_elems / 8; k += kThreads) o[k] = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  const int b = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  const SegMeta meta =
      reinterpret_cast<const SegMeta*>(static_cast<const char*>(a.ws) + seg_meta_offset(P, NBMAX, D))[blockIdx.x];
  const ReqInfo ri = req_info(a, b, false);
  if (!ri.ok) return;  // no tiles: the main kernel wrote no record for it
  const int pa = meta.pa, pb = meta.pb, first_slot = meta.first_slot;  // then p * 2 for p > pa
  const bool cut = pa != pb && pb - pa < 4;  // cut segments reach at most 3 shares in practice
  const int G = a.Hq / a.Hkv, nq = ri.w * G;
  const float* ws_o = static_cast<const float*>(a.ws);
  const float* ws_lse = ws_o + size_t(P) * 2 * ROWS * D;
  // Every load is issued before any store, so the whole merge costs about one round trip:
  // the first pass of the window K/V append (positions L .. L+w-1) goes first, so that its
  // stores wait for it alone (the wait counter drains in order)...
  AppendPass ap;
  append_load<D>(a, b, g, ri.L, ri.r0, ri.w, 0, ap);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // ...then the partials of a cut segment (kItems output items of 4 d per thread, up to 4
  // shares).  Those loads are unconditional too (column and share clamped into the segment;
  // the masks are applied after the compiler barrier), so that the append's stores wait for
  // an exact count of later loads.  Each branch has its own copy of the append's stores.
  auto append_rest = [&]() {
    append_store<D>(a, g, ri.L, ri.w, 0, ap);
    for (int base = 4 * kThreads; base < ri.w * D; base += 4 * kThreads) {  // windows of more than 8 rows
      append_load<D>(a, b, g, ri.L, ri.r0, ri.w, base, ap);
      append_store<D>(a, g, ri.L, ri.w, base, ap);
    }
  };
  if (cut) {
    constexpr int kItems = (ROWS * D / 4 + kThreads - 1) / kThreads;
    float lse[kItems][4];
    float4 po[kItems][4];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int it = tid + i * kThreads;
      const int col = min(it / (D / 4), nq - 1), c4 = it % (D / 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = min(pa + u, pb);
        const size_t sl = p == pa ? first_slot : size_t(p) * 2;
        lse[i][u] = ws_lse[sl * ROWS + col];
        po[i][u] = reinterpret_cast<const float4*>(ws_o + (sl * ROWS + col) * D)[c4];
      }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    append_rest();
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int it = tid + i * kThreads;
      if (it >= nq * (D / 4)) break;
      const int col = it / (D / 4), c4 = it % (D / 4);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (pa + u > pb) lse[i][u] = -INFINITY;  // past the segment's last share
      float M = -INFINITY;
#pragma unroll
      for (int u = 0; u < 4; ++u) M = fmaxf(M, lse[i][u]);
      float sum = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      if (M != -INFINITY) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float e = lse[i][u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lse[i][u] - M);
          sum += e;
          acc.x += e * po[i][u].x; acc.y += e * po[i][u].y; acc.z += e * po[i][u].z; acc.w += e * po[i][u].w;
        }
      }
      const float inv = sum > 0.f ? 1.f / sum : 0.f;
      uint16_t* out = static_cast<uint16_t*>(a.out) + (size_t(ri.r0 + col / G) * a.Hq + g * G + col % G) * D + c4 * 4;
      const uint32_t lo16 = f32_to_bf16(acc.x * inv) | (uint32_t(f32_to_bf16(acc.y * inv)) << 16);
      const uint32_t hi16 = f32_to_bf16(acc.z * inv) | (uint32_t(f32_to_bf16(acc.w * inv)) << 16);
      *reinterpret_cast<uint2*>(out) = make_uint2(lo16, hi16);
    }
    return;
  }
  append_rest();
  if (pa == pb) return;  // finished inside one share
  // a segment spread over more than 4 shares: the general loop, 4 shares at a time
  for (int it = tid; it < nq * (D / 4); it += kThreads) {
    const int col = it / (D / 4), c4 = it % (D / 4);
    float M = -INFINITY, sum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = pa; p0 <= pb; p0 += 4) {
      float l4[4];
      float4 o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = min(p0 + u, pb);
        const size_t sl = p == pa ? first_slot : size_t(p) * 2;
        l4[u] = p0 + u <= pb ? ws_lse[sl * ROWS + col] : -INFINITY;
        o[u] = reinterpret_cast<const float4*>(ws_o + (sl * ROWS + col) * D)[c4];
      }
      float m4 = M;
#pragma unroll
      for (int u = 0; u < 4; ++u) m4 = fmaxf(m4, l4[u]);
      if (m4 != -INFINITY) {
        const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - m4);
        sum *= r;
        acc.x *= r; acc.y *= r; acc.z *= r; acc.w *= r;
        M = m4;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float e = l4[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(l4[u] - M);
          sum += e;
          acc.x += e * o[u].x; acc.y += e * o[u].y; acc.z += e * o[u].z; acc.w += e * o[u].w;
        }
      }
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    uint16_t* out = static_cast<uint16_t*>(a.out) + (size_t(ri.r0 + col / G) * a.Hq + g * G + col % G) * D + c4 * 4;
    const uint32_t lo16 = f32_to_bf16(acc.x * inv) | (uint32_t(f32_to_bf16(acc.y * inv)) << 16);
    const uint32_t hi16 = f32_to_bf16(acc.z * inv) | (uint32_t(f32_to_bf16(acc.w * inv)) << 16);
    *reinterpret_cast<uint2*>(out) = make_uint2(lo16, hi16);
  }
}

// Generic path: any element type and page size.  One workgroup at a time per (request b,
// query column n = i*G + head offset, kv head g), so a request's columns run side by side
// instead of in turn (the grid is capped; workgroups then take several pairs).  The 256 threads split the keys 0 .. L+i of the column: each owns
// one key per pass (its K row in 16-byte loads, its V column from the transposed tile)
// and keeps a running max, sum and D-wide accumulator; the threads are merged at the end
// through DPP row sums and LDS.  Workgroup ids are dealt so that each XCD gets a
// contiguous run of (request, column) pairs: the columns of one request then read its
// K/V through one L2.  The workgroup of column i*G also appends window row i to the
// caches (no workgroup reads cache positions L and above).
// One key's D elements in registers, as loaded (bf16 stays packed two to a register and
// is widened where it is used).
template <typename T, int D>
struct RowRegs;
template <int D>
struct RowRegs<float, D> {
  float x[D];
  __device__ __forceinline__ void load_row(const float* r) {
#pragma unroll
    for (int j = 0; j < D / 4; ++j) {
      const float4 v = reinterpret_cast<const float4*>(r)[j];
      x[4 * j] = v.x, x[4 * j + 1] = v.y, x[4 * j + 2] = v.z, x[4 * j + 3] = v.w;
    }
  }
  __device__ __forceinline__ void load_strided(const float* r, int stride) {
#pragma unroll
    for (int d = 0; d < D; ++d) x[d] = r[size_t(d) * stride];
  }
  __device__ __forceinline__ float at(int d) const { return x[d]; }
};
template <int D>
struct RowRegs<uint16_t, D> {
  uint32_t x[D / 2];
  __device__ __forceinline__ void load_row(const uint16_t* r) {
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
      const uint4 v = reinterpret_cast<const uint4*>(r)[j];
      x[4 * j] = v.x, x[4 * j + 1] = v.y, x[4 * j + 2] = v.z, x[4 * j + 3] = v.w;
    }
  }
  __device__ __forceinline__ void load_strided(const uint16_t* r, int stride) {
#pragma unroll
    for (int j = 0; j < D / 2; ++j)
      x[j] = uint32_t(r[size_t(2 * j) * stride]) | (uint32_t(r[size_t(2 * j + 1) * stride]) << 16);
  }
  __device__ __forceinline__ float at(int d) const {
    return __uint_as_float(d % 2 ? x[d / 2] & 0xffff0000u : x[d / 2] << 16);
  }
};

// Sum over each row of 16 lanes, in the row's last lane (every lane must be active).
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_move<kDppRowShr + 1, 0xf>(0.f, x);
  x += dpp_move<kDppRowShr + 2, 0xf>(0.f, x);
  x += dpp_move<kDppRowShr + 4, 0xf>(0.f, x);
  x += dpp_move<kDppRowShr + 8, 0xf>(0.f, x);
  return x;
}

// Zero-fills output rows [M, tier): workgroup x of nx takes rows M + x, M + x + nx, ...
template <typename T, int D>
__device__ __forceinline__ void pad_rows(const AttnArgs& a, int x, int nx) {
  const int M = max(a.total_tier[0], 0);
  const int tier = min(a.total_tier[1], a.max_rows);
  const size_t row_elems = size_t(a.Hq) * D;
  for (int r = M + x; r < tier; r += nx) {
    T* o = static_cast<T*>(a.out) + size_t(r) * row_elems;
    for (size_t k = threadIdx.x; k < row_elems; k += 256) Elem<T>::store(o, k, 0.f);
  }
}

// One (request, query column) pair lid = b * NQ + n of kv head g; every return is taken by
// the whole workgroup except the append's bad-page exit.
template <typename T, int D>
__device__ void generic_column(const AttnArgs& a, int lid, int NQ, int g) {
  constexpr int kRows = kWaves * 4;  // rows of 16 lanes in the workgroup
  __shared__ float sq[D];
  __shared__ float red[kRows][D + 1];
  __shared__ float red_l[kRows];
  __shared__ float red_m[kWaves];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int b = lid / NQ, n = lid % NQ;
  if (b >= a.B) return;
  const ReqInfo ri = req_info(a, b, n == 0 && g == 0 && tid == 0);
  if (!ri.ok) return;
  const int G = a.Hq / a.Hkv, Hkv = a.Hkv, P = a.page_size;
  if (n >= ri.w * G) return;
  const int L = ri.L, r0 = ri.r0, i = n / G, h = g * G + n % G;
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  const T* kn = static_cast<const T*>(a.k_new);
  const T* vn = static_cast<const T*>(a.v_new);
  const T* qrow = static_cast<const T*>(a.q) + (size_t(r0 + i) * a.Hq + h) * D;
  for (int d = tid; d < D; d += 256) sq[d] = Elem<T>::load(qrow, d) * a.scale;
  __syncthreads();

  bool bad_page = false;
  float m = -INFINITY, l = 0.f, acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  const int nk = L + i + 1;
  const int* bt = a.block_table + size_t(b) * a.max_pages;
  int pg_cur = tid < L ? bt[tid / P] : 0;
  for (int p = tid; p < nk; p += 256) {
    const T* krow;
    const T* vbase;
    int vstride;
    const int pg = pg_cur;
    pg_cur = p + 256 < L ? bt[(p + 256) / P] : 0;  // the next pass's page, in flight now
    if (p < L) {
      if (pg < 0 || pg >= a.num_pages) {
        bad_page = true;
        continue;
      }
      krow = kc + ((size_t(pg) * Hkv + g) * P + p % P) * D;
      vbase = vc + v_index(pg, g, Hkv, P, D, p % P, 0);
      vstride = vblk(P);
    } else {
      krow = kn + (size_t(r0 + p - L) * Hkv + g) * D;
      vbase = vn + (size_t(r0 + p - L) * Hkv + g) * D;
      vstride = 1;
    }
    RowRegs<T, D> kr, vv;
    kr.load_row(krow);
    vv.load_strided(vbase, vstride);
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < D; ++d) s4[d % 4] = fmaf(sq[d], kr.at(d), s4[d % 4]);
    const float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    const float mn = fmaxf(m, s);
    const float c = __expf(m - mn);
    const float e = __expf(s - mn);
    l = fmaf(l, c, e);
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(acc[d], c, e * vv.at(d));
    m = mn;
  }
  if (bad_page) flag(a.status, RVA_DEV_BAD_PAGE);

  // merge: workgroup max, then every thread's share rescaled to it and summed
  const float mw = wave_max(m);
  if (lane == 0) red_m[wave] = mw;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  const float f = (m == -INFINITY) ? 0.f : __expf(m - M);
  const bool row_last = lane % 16 == 15;
  const int row = wave * 4 + lane / 16;
  const float lr = row_sum(l * f);
  if (row_last) red_l[row] = lr;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const float v = row_sum(acc[d] * f);
    if (row_last) red[row][d] = v;
  }
  __syncthreads();
  if (tid < D) {
    float o = 0.f, Ls = 0.f;
#pragma unroll
    for (int r = 0; r < kRows; ++r) o += red[r][tid], Ls += red_l[r];
    Elem<T>::store(static_cast<T*>(a.out), (size_t(r0 + i) * a.Hq + h) * D + tid, o / Ls);
  }

  // append window row i (position L + i) to both caches
  if (n % G == 0 && tid < D) {
    const int p = L + i;
    bool badp = false;
    const int pg = page_of(a, b, p, badp);
    if (pg < 0) {
      flag(a.status, RVA_DEV_BAD_PAGE);
      return;
    }
    const size_t src = (size_t(r0 + i) * Hkv + g) * D + tid;
    static_cast<T*>(a.k_cache)[((size_t(pg) * Hkv + g) * P + p % P) * D + tid] = kn[src];
    static_cast<T*>(a.v_cache)[v_index(pg, g, Hkv, P, D, p % P, tid)] = vn[src];
  }
}

// Grid (nx, Hkv + 1): nx a multiple of 8; workgroup x takes the (request, column) slots
// x, x + nx, ... of 8 * per_xcd, each mapped XCD-major (slot s -> pair (s % 8) * per_xcd
// + s / 8), so each XCD gets contiguous runs of pairs.  Row Hkv zero-fills the pad rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnArgs a, int NQ, int per_xcd) {
  if (int(blockIdx.y) == a.Hkv) {
    pad_rows<T, D>(a, blockIdx.x, gridDim.x);
    return;
  }
  const int slots = 8 * per_xcd;
  for (int x = blockIdx.x; x < slots; x += gridDim.x) {
    generic_column<T, D>(a, (x % 8) * per_xcd + x / 8, NQ, blockIdx.y);
    __syncthreads();  // the next pair rewrites the LDS
  }
}

int nbmax_for(int max_window, int G) {
  const int r = max_window * G;
  return r <= 16 ? 1 : r <= 32 ? 2 : 4;
}

bool use_sk(int kv_dtype, int D, int page_size, int max_window, int G, int B) {
  return kv_dtype == RVA_BF16 && (D == 64 || D == 128) && page_size >= kTile &&
         (page_size & (page_size - 1)) == 0 && max_window * G <= 64 && B <= kMaxB;
}

// Persistent grid: CUs x resident workgroups per CU of the current device (cached).
template <int D, int NBMAX>
int sk_grid() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  if (!cache[dev]) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, attn_sk_kernel<D, NBMAX>, kThreads, 0) != hipSuccess)
      per = 0;
    cache[dev] = (cus > 0 ? cus : 256) * (per > 0 ? per : 1);
  }
  return cache[dev];
}

int sk_grid_for(int D, int nbmax) {
  if (D == 128) return nbmax == 1 ? sk_grid<128, 1>() : nbmax == 2 ? sk_grid<128, 2>() : sk_grid<128, 4>();
  return nbmax == 1 ? sk_grid<64, 1>() : nbmax == 2 ? sk_grid<64, 2>() : sk_grid<64, 4>();
}

template <int D, int NBMAX>
hipError_t launch_sk(const AttnArgs& a, hipStream_t stream) {
  const int P = sk_grid<D, NBMAX>();
  hipLaunchKernelGGL((attn_sk_kernel<D, NBMAX>), dim3(P), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int merge = a.B * a.Hkv, pad = 32;
  hipLaunchKernelGGL((attn_merge_kernel<D, NBMAX>), dim3(merge + pad), dim3(kThreads), 0, stream, a, P, merge, pad);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_generic(const AttnArgs& a, hipStream_t stream) {
  // (request, column) pairs padded to a multiple of the 8 XCDs, dealt XCD-major; one more
  // row of workgroups for the pad rows
  const int NQ = a.max_window * (a.Hq / a.Hkv);
  const int per_xcd = int((int64_t(a.B) * NQ + 7) / 8);
  const int nx = 8 * std::min(per_xcd, 2048);  // at most 16384 workgroups per row; they loop
  hipLaunchKernelGGL((attn_generic_kernel<T, D>), dim3(nx, a.Hkv + 1), dim3(256), 0, stream, a, NQ, per_xcd);
  return hipGetLastError();
}

// Library-owned scratch of rva_verify_attention_noalloc: the stream-K partials and the
// merge records live here instead of in a caller workspace.  Zero-initialised at load, held
// by every device the library runs on until the process ends; every noalloc call on one
// device shares it (calls that overlap on one device race).  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in): the device address comes
// from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(24) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

}  // namespace

hipError_t attention_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

size_t attention_workspace_bytes(int B, int max_window, int Hq, int Hkv, int D, int page_size,
                                 int max_pages, int kv_dtype) {
  const int G = Hq / Hkv;
  (void)max_pages;
  if (!use_sk(kv_dtype, D, page_size, max_window, G, B)) return 0;
  const int nbmax = nbmax_for(max_window, G);
  const size_t P = sk_grid_for(D, nbmax);
  return seg_meta_offset(int(P), nbmax, D) + size_t(B) * Hkv * sizeof(SegMeta);
}

hipError_t launch_attention(const AttnArgs& a, int kv_dtype, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (use_sk(kv_dtype, a.D, a.page_size, a.max_window, G, a.B)) {
    const int nbmax = nbmax_for(a.max_window, G);
    if (a.D == 128) {
      if (nbmax == 1) return launch_sk<128, 1>(a, stream);
      if (nbmax == 2) return launch_sk<128, 2>(a, stream);
      return launch_sk<128, 4>(a, stream);
    }
    if (nbmax == 1) return launch_sk<64, 1>(a, stream);
    if (nbmax == 2) return launch_sk<64, 2>(a, stream);
    return launch_sk<64, 4>(a, stream);
  }
  if (kv_dtype == RVA_BF16)
    return a.D == 128 ? launch_generic<uint16_t, 128>(a, stream) : launch_generic<uint16_t, 64>(a, stream);
  return a.D == 128 ? launch_generic<float, 128>(a, stream) : launch_generic<float, 64>(a, stream);
}

}  // namespace rva
