// Stage 3: varlen GQA verify attention over a paged KV cache, with the window's K/V
// appended to the cache.
//
// Sources: "DFlash 到 DSpark in SGLang：解码提速 4.3×，以及 DeepSeek-V4 支持"
// (yichizhang.dev, AI-Infra-Visualized), section "Ragged verify under full CUDA graphs",
// and section 3 of the devpress.csdn.net DSpark-in-SGLang article: each packed verify
// token attends only to its own request's KV, delimited by cu_seqlens.
//
// Design (bf16, D in {64, 128}, page_size % 32 == 0):
//   * Work item = (request b, kv head g, chunk of kChunk keys); grid (chunks, Hkv, B),
//     chunks beyond a request's length exit at once.  Every K/V byte of the request is
//     read exactly once for ALL window rows and ALL Hq/Hkv query heads of the group: the
//     (window row, head-in-group) pairs form the N side of the MFMA tiles (NB blocks of 16).
//   * Each of the 4 waves streams kKeysPerWave keys in tiles of 32 keys.  Scores are
//     computed transposed, S^T = K Q^T, with mfma_f32_16x16x32_bf16: K rows are the A
//     operand, loaded as 16-byte vectors straight from the (page, head) block, which is a
//     contiguous [page_size, D] tile in this layout.  The accumulator lane layout leaves
//     each lane with 4 keys x 1 query column per 16-key block; with the contraction index
//     of the PV product permuted to match (slot 8q+t <-> key 4q+t, slot 8q+4+t <-> key
//     16+4q+t), the probabilities P^T are ALREADY the B operand of O^T = V^T P^T: no LDS
//     round trip.  V is stored transposed per page ([D, page_size]), so the A operand V^T
//     is two 8-byte loads per lane.
//   * Online softmax in the log2 domain per query column; the 4 waves of a workgroup are
//     merged through LDS in a fixed order (deterministic), then either the final output
//     (one chunk) or a normalised partial + log-sum-exp goes out; a small combine kernel
//     merges the chunks and zero-fills the pad rows [M, tier).
//   * The tile that reaches past the cached context takes the window keys from k_new /
//     v_new (packed rows) and applies the causal mask; the last chunk's workgroup writes
//     the window K/V into the cache (positions L .. L+w-1), which no other work item of
//     this launch reads.
// Any other dtype / page size uses attn_generic_kernel (one wave per query column, one key
// per lane, online softmax), which is also the float32 path.
#include "rva_common.h"

namespace rva {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef short short4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttnWaves = 4;
constexpr int kAttnThreads = kAttnWaves * kWave;
constexpr int kKeysPerWave = 256;
constexpr int kChunk = kAttnWaves * kKeysPerWave;  // keys per workgroup
constexpr int kTile = 32;
constexpr float kLog2e = 1.4426950408889634f;

struct ReqInfo {
  int L, r0, w, ok;
};

// Validates request b's metadata; raises device-status bits once per request.
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

__device__ __forceinline__ short8 load16(const uint16_t* p) {
  return *reinterpret_cast<const short8*>(p);
}
__device__ __forceinline__ short4 load8(const uint16_t* p) {
  return *reinterpret_cast<const short4*>(p);
}

__device__ __forceinline__ int page_of(const AttnArgs& a, int b, int p, bool& bad) {
  const int pg = a.block_table[size_t(b) * a.max_pages + p / a.page_size];
  if (pg < 0 || pg >= a.num_pages) {
    bad = true;
    return -1;
  }
  return pg;
}

template <int D, int NB>
__global__ __launch_bounds__(kAttnThreads) void attn_mfma_kernel(AttnArgs a, int max_splits) {
  constexpr int DS = D / 32;  // k-steps of the score MFMA
  constexpr int DB = D / 16;  // 16-row blocks of O^T
  constexpr int ROWS = NB * 16;
  __shared__ float sm_m[kAttnWaves][ROWS];
  __shared__ float sm_l[kAttnWaves][ROWS];
  __shared__ float sm_M[ROWS];
  __shared__ float sm_L[ROWS];
  __shared__ float sm_o[ROWS][D + 4];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int lc = lane % 16, lq = lane / 16;
  const ReqInfo ri = req_info(a, b, split == 0 && g == 0 && tid == 0);
  if (!ri.ok) return;
  const int L = ri.L, r0 = ri.r0, w = ri.w, Lw = L + w;
  const int nsplit = (Lw + kChunk - 1) / kChunk;
  if (split >= nsplit) return;
  const int G = a.Hq / a.Hkv;
  const int nq = w * G;
  const int Hkv = a.Hkv, P = a.page_size;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const uint16_t* kn = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(a.v_new);
  const float sl2 = a.scale * kLog2e;
  bool bad_page = false;

  // Q^T as the B operand: lane holds column n = nb*16 + lc, d = s*32 + 8*lq .. +7
  short8 qop[NB][DS];
  int limit[NB];  // last visible key position for column n
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + lc;
    const bool valid = n < nq;
    limit[nb] = valid ? L + n / G : Lw - 1;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (size_t(r0 + (valid ? n / G : 0)) * a.Hq + g * G + (valid ? n % G : 0)) * D;
#pragma unroll
    for (int s = 0; s < DS; ++s) qop[nb][s] = valid ? load16(qrow + s * 32 + 8 * lq) : short8{0, 0, 0, 0, 0, 0, 0, 0};
  }

  f32x4 oacc[DB][NB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
  }

  const int kb = split * kChunk + wave * kKeysPerWave;
  const int ke = min(kb + kKeysPerWave, Lw);
  for (int t0 = kb; t0 < ke; t0 += kTile) {
    short8 kop[2][DS];
    short8 vop[DB];
    const bool fast = t0 + kTile <= L;
    if (fast) {
      const int pg = page_of(a, b, t0, bad_page);
      if (pg < 0) break;
      const int slot0 = t0 % P;
      const uint16_t* kbase = kc + ((size_t(pg) * Hkv + g) * P + slot0) * D;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int s = 0; s < DS; ++s) kop[mb][s] = load16(kbase + size_t(mb * 16 + lc) * D + s * 32 + 8 * lq);
      const uint16_t* vbase = vc + (size_t(pg) * Hkv + g) * D * P + slot0 + 4 * lq;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = vbase + size_t(db * 16 + lc) * P;
        const short4 lo = load8(vrow), hi = load8(vrow + 16);
        vop[db] = short8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int p = t0 + mb * 16 + lc;
        const uint16_t* krow = nullptr;
        if (p < L) {
          const int pg = page_of(a, b, p, bad_page);
          if (pg >= 0) krow = kc + ((size_t(pg) * Hkv + g) * P + p % P) * D;
        } else if (p < Lw) {
          krow = kn + (size_t(r0 + p - L) * Hkv + g) * D;
        }
#pragma unroll
        for (int s = 0; s < DS; ++s)
          kop[mb][s] = krow ? load16(krow + s * 32 + 8 * lq) : short8{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 16 + lc;
        short8 v;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int p = t0 + h * 16 + 4 * lq + t;
            short x = 0;
            if (p < L) {
              const int pg = page_of(a, b, p, bad_page);
              if (pg >= 0) x = short(vc[((size_t(pg) * Hkv + g) * D + d) * P + p % P]);
            } else if (p < Lw) {
              x = short(vn[(size_t(r0 + p - L) * Hkv + g) * D + d]);
            }
            v[h * 4 + t] = x;
          }
        vop[db] = v;
      }
    }

    // scores S^T[key][col] for the 32 keys of the tile
    f32x4 sacc[2][NB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DS; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[mb][s]),
                                                        __builtin_bit_cast(bf16x8, qop[nb][s]), acc, 0, 0, 0);
        sacc[mb][nb] = acc;
      }

    short8 pop[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float sc[2][4];
      float mt = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int p = t0 + mb * 16 + 4 * lq + t;
          const float v = (p <= limit[nb]) ? sacc[mb][nb][t] * sl2 : -INFINITY;
          sc[mb][t] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mnew = fmaxf(m_run[nb], mt);
      const bool none = mnew == -INFINITY;
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - mnew);
      float psum = 0.f;
      short8 pv;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float pf = none ? 0.f : __builtin_amdgcn_exp2f(sc[mb][t] - mnew);
          const uint16_t pb = f32_to_bf16(pf);
          psum += bf16_to_f32(pb);
          pv[mb * 4 + t] = short(pb);
        }
      l_run[nb] = l_run[nb] * alpha + psum;
      m_run[nb] = mnew;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db][nb] *= alpha;
      pop[nb] = pv;
    }

#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        oacc[db][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop[db]),
                                                               __builtin_bit_cast(bf16x8, pop[nb]),
                                                               oacc[db][nb], 0, 0, 0);
  }
  if (bad_page) flag(a.status, RVA_DEV_BAD_PAGE);

  // ---- merge the 4 waves (fixed order) ----
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l = l_run[nb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    l_run[nb] = l;
    if (lq == 0) {
      sm_m[wave][nb * 16 + lc] = m_run[nb];
      sm_l[wave][nb * 16 + lc] = l;
    }
  }
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + lc;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kAttnWaves; ++v) M = fmaxf(M, sm_m[v][n]);
    float Lsum = 0.f;
#pragma unroll
    for (int v = 0; v < kAttnWaves; ++v)
      if (sm_m[v][n] != -INFINITY) Lsum += sm_l[v][n] * __builtin_amdgcn_exp2f(sm_m[v][n] - M);
    const float e = (m_run[nb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[nb] - M);
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db][nb] *= e;
    if (wave == 0 && lq == 0) {
      sm_M[n] = M;
      sm_L[n] = Lsum;
    }
  }
  for (int v = 0; v < kAttnWaves; ++v) {
    if (wave == v) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            float& dst = sm_o[nb * 16 + lc][db * 16 + 4 * lq + t];
            dst = (v == 0) ? oacc[db][nb][t] : dst + oacc[db][nb][t];
          }
    }
    __syncthreads();
  }

  // ---- write: final output (single chunk) or normalised partial + lse ----
  const size_t bg = size_t(b) * Hkv + g;
  float* ws_o = static_cast<float*>(a.ws);
  float* ws_lse = ws_o + size_t(a.B) * Hkv * max_splits * ROWS * D;
  for (int idx = tid; idx < nq * D; idx += kAttnThreads) {
    const int n = idx / D, d = idx % D;
    const float Ls = sm_L[n];
    const float val = Ls > 0.f ? sm_o[n][d] / Ls : 0.f;
    if (nsplit == 1) {
      uint16_t* o = static_cast<uint16_t*>(a.out);
      o[(size_t(r0 + n / G) * a.Hq + g * G + n % G) * D + d] = f32_to_bf16(val);
    } else {
      ws_o[((bg * max_splits + split) * ROWS + n) * D + d] = val;
      if (d == 0) ws_lse[(bg * max_splits + split) * ROWS + n] = Ls > 0.f ? sm_M[n] + __log2f(Ls) : -INFINITY;
    }
  }

  // ---- append the window K/V (positions L .. L+w-1) from the last chunk ----
  if (split == nsplit - 1) {
    uint16_t* kcw = static_cast<uint16_t*>(a.k_cache);
    uint16_t* vcw = static_cast<uint16_t*>(a.v_cache);
    for (int idx = tid; idx < w * D; idx += kAttnThreads) {
      const int j = idx / D, d = idx % D;
      const int p = L + j;
      bool badp = false;
      const int pg = page_of(a, b, p, badp);
      if (pg < 0) {
        flag(a.status, RVA_DEV_BAD_PAGE);
        continue;
      }
      const size_t src = (size_t(r0 + j) * Hkv + g) * D + d;
      kcw[((size_t(pg) * Hkv + g) * P + p % P) * D + d] = kn[src];
      vcw[((size_t(pg) * Hkv + g) * D + d) * P + p % P] = vn[src];
    }
  }
}

// Merges the per-chunk partials of every (request, kv head) with more than one chunk, and
// zero-fills output rows [M, tier).  Blocks [0, B*Hkv) merge, the rest zero-fill.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, int max_splits, int rows_cap,
                                                           int merge_blocks, int pad_blocks) {
  __shared__ float sm_M[64];
  __shared__ float sm_inv[64];
  const int tid = threadIdx.x;
  if (int(blockIdx.x) >= merge_blocks) {
    const int M = max(a.total_tier[0], 0);
    const int tier = min(a.total_tier[1], a.max_rows);
    const size_t row_elems = size_t(a.Hq) * D;
    for (int r = M + int(blockIdx.x) - merge_blocks; r < tier; r += pad_blocks) {
      T* o = static_cast<T*>(a.out) + size_t(r) * row_elems;
      for (size_t k = tid; k < row_elems; k += 256) Elem<T>::store(o, k, 0.f);
    }
    return;
  }
  if (rows_cap == 0) return;  // single-pass kernels wrote every output
  const int b = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  const ReqInfo ri = req_info(a, b, false);
  if (!ri.ok) return;
  const int Lw = ri.L + ri.w;
  const int nsplit = (Lw + kChunk - 1) / kChunk;
  if (nsplit <= 1) return;
  const int G = a.Hq / a.Hkv, nq = ri.w * G;
  const size_t bg = size_t(b) * a.Hkv + g;
  const float* ws_o = static_cast<const float*>(a.ws);
  const float* ws_lse = ws_o + size_t(a.B) * a.Hkv * max_splits * rows_cap * D;
  for (int n = tid; n < nq; n += 256) {
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws_lse[(bg * max_splits + s) * rows_cap + n]);
    float sum = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float l = ws_lse[(bg * max_splits + s) * rows_cap + n];
      if (l != -INFINITY) sum += __builtin_amdgcn_exp2f(l - M);
    }
    sm_M[n] = M;
    sm_inv[n] = sum > 0.f ? 1.f / sum : 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < nq * D; idx += 256) {
    const int n = idx / D, d = idx % D;
    const float M = sm_M[n];
    float acc = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float l = ws_lse[(bg * max_splits + s) * rows_cap + n];
      if (l != -INFINITY) acc += __builtin_amdgcn_exp2f(l - M) * ws_o[((bg * max_splits + s) * rows_cap + n) * D + d];
    }
    T* o = static_cast<T*>(a.out);
    Elem<T>::store(o, (size_t(ri.r0 + n / G) * a.Hq + g * G + n % G) * D + d, acc * sm_inv[n]);
  }
}

// Generic path: any element type and page size.  One workgroup per (request, kv head);
// each wave takes query columns in turn; each lane owns one key at a time and keeps a
// running max, sum and D-wide accumulator; the lanes are merged at the end.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnArgs a) {
  __shared__ float sm_q[4][D];
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const ReqInfo ri = req_info(a, b, g == 0 && tid == 0);
  if (!ri.ok) return;
  const int L = ri.L, r0 = ri.r0, w = ri.w, Lw = L + w;
  const int G = a.Hq / a.Hkv, nq = w * G, Hkv = a.Hkv, P = a.page_size;
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  const T* kn = static_cast<const T*>(a.k_new);
  const T* vn = static_cast<const T*>(a.v_new);
  bool bad_page = false;
  for (int n0 = 0; n0 < nq; n0 += 4) {  // same trip count in every wave
    const int n = n0 + wave;
    const bool active = n < nq;
    const int i = active ? n / G : 0, h = g * G + (active ? n % G : 0);
    const T* qrow = static_cast<const T*>(a.q) + (size_t(r0 + i) * a.Hq + h) * D;
    if (active)
      for (int d = lane; d < D; d += kWave) sm_q[wave][d] = Elem<T>::load(qrow, d) * a.scale;
    __syncthreads();
    if (active) {
      float m = -INFINITY, l = 0.f;
      float acc[D];
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = 0.f;
      for (int p = lane; p <= L + i; p += kWave) {
        const T* krow;
        const T* vbase;
        size_t vstride;
        if (p < L) {
          const int pg = page_of(a, b, p, bad_page);
          if (pg < 0) continue;
          krow = kc + ((size_t(pg) * Hkv + g) * P + p % P) * D;
          vbase = vc + (size_t(pg) * Hkv + g) * D * P + p % P;
          vstride = P;
        } else {
          krow = kn + (size_t(r0 + p - L) * Hkv + g) * D;
          vbase = vn + (size_t(r0 + p - L) * Hkv + g) * D;
          vstride = 1;
        }
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) s += sm_q[wave][d] * Elem<T>::load(krow, d);
        const float mn = fmaxf(m, s);
        const float c = __expf(m - mn);
        const float e = __expf(s - mn);
        l = l * c + e;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = acc[d] * c + e * Elem<T>::load(vbase, size_t(d) * vstride);
        m = mn;
      }
      const float M = wave_max(m);
      const float f = (m == -INFINITY) ? 0.f : __expf(m - M);
      const float Ls = wave_sum(l * f);
      T* orow = static_cast<T*>(a.out) + (size_t(r0 + i) * a.Hq + h) * D;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const float v = wave_sum(acc[d] * f);
        if (lane == 0) Elem<T>::store(orow, d, v / Ls);
      }
    }
    __syncthreads();
  }
  if (bad_page) flag(a.status, RVA_DEV_BAD_PAGE);
  __syncthreads();
  // append the window K/V (all of this head's work is done; no wave reads the cache again)
  T* kcw = static_cast<T*>(a.k_cache);
  T* vcw = static_cast<T*>(a.v_cache);
  for (int idx = tid; idx < w * D; idx += 256) {
    const int j = idx / D, d = idx % D;
    const int p = L + j;
    bool badp = false;
    const int pg = page_of(a, b, p, badp);
    if (pg < 0) {
      flag(a.status, RVA_DEV_BAD_PAGE);
      continue;
    }
    const size_t src = (size_t(r0 + j) * Hkv + g) * D + d;
    kcw[((size_t(pg) * Hkv + g) * P + p % P) * D + d] = kn[src];
    vcw[((size_t(pg) * Hkv + g) * D + d) * P + p % P] = vn[src];
  }
}

int rows_for(int max_window, int G) {
  const int r = max_window * G;
  return r <= 16 ? 16 : r <= 32 ? 32 : 64;
}

bool use_mfma(int kv_dtype, int D, int page_size, int max_window, int G) {
  return kv_dtype == RVA_BF16 && (D == 64 || D == 128) && page_size % kTile == 0 &&
         max_window * G <= 64;
}

int max_splits_for(int page_size, int max_pages) {
  const long long cap = (long long)page_size * max_pages;
  return int((cap + kChunk - 1) / kChunk);
}

template <int D, int NB>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t stream) {
  const int ms = max_splits_for(a.page_size, a.max_pages);
  hipLaunchKernelGGL((attn_mfma_kernel<D, NB>), dim3(ms, a.Hkv, a.B), dim3(kAttnThreads), 0, stream, a, ms);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int merge = a.B * a.Hkv, pad = 32;
  hipLaunchKernelGGL((attn_combine_kernel<uint16_t, D>), dim3(merge + pad), dim3(256), 0, stream, a, ms,
                     NB * 16, merge, pad);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_generic(const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_generic_kernel<T, D>), dim3(a.Hkv, a.B), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int pad = 32;
  hipLaunchKernelGGL((attn_combine_kernel<T, D>), dim3(pad), dim3(256), 0, stream, a, 1, 0, 0, pad);
  return hipGetLastError();
}

}  // namespace

size_t attention_workspace_bytes(int B, int max_window, int Hq, int Hkv, int D, int page_size,
                                 int max_pages, int kv_dtype) {
  const int G = Hq / Hkv;
  if (!use_mfma(kv_dtype, D, page_size, max_window, G)) return 0;
  const size_t rows = rows_for(max_window, G);
  const size_t ms = max_splits_for(page_size, max_pages);
  return size_t(B) * Hkv * ms * rows * (D + 1) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& a, int kv_dtype, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (use_mfma(kv_dtype, a.D, a.page_size, a.max_window, G)) {
    const int rows = rows_for(a.max_window, G);
    if (a.D == 128) {
      if (rows == 16) return launch_mfma<128, 1>(a, stream);
      if (rows == 32) return launch_mfma<128, 2>(a, stream);
      return launch_mfma<128, 4>(a, stream);
    }
    if (rows == 16) return launch_mfma<64, 1>(a, stream);
    if (rows == 32) return launch_mfma<64, 2>(a, stream);
    return launch_mfma<64, 4>(a, stream);
  }
  if (kv_dtype == RVA_BF16)
    return a.D == 128 ? launch_generic<uint16_t, 128>(a, stream) : launch_generic<uint16_t, 64>(a, stream);
  return a.D == 128 ? launch_generic<float, 128>(a, stream) : launch_generic<float, 64>(a, stream);
}

}  // namespace rva
