// Stages 4 and 5: full-vocabulary speculative-sampling acceptance, the residual / bonus
// draw, the commit, and the TV-distance confidence labels.
//
// Sources: "DSpark：投机解码与生产级 Serving 学习笔记" (sorenprojections.com) section 02
// (the acceptance rule keeps the target distribution; acceptance is prefix-only) and
// section 07 (label c* = 1 - 0.5 ||p_d - p_t||_1); "DFlash 到 DSpark in SGLang" section
// "Background" (each verify forward also yields one target token).
//
// Rows are cut into segments of kSeg vocabulary entries (32 KB of bf16).  Four kernels:
//   stats_kernel    grid (segment, row): exact max m_s and sum of exp(x - m_s) of every
//                   active row (float32 exp2, float32 runs of 8, float64 accumulation).  The
//                   one full HBM pass over the logits.
//   decide_kernel   one workgroup per request: row normalisers (max M, sum S) of the
//                   request's rows from the segment stats, p_t(x) and p_d(x) at the drafted
//                   tokens in float64, accept bits, first rejection, which rows the draw uses.
//   pair_kernel_*   grid (segment, slot).  Draw slots (one per request, dispatched first):
//                   float64 sums over the draw rows (target row n, and draft row n for a
//                   residual draw) of e_t = exp(x_t - M_t), e_d = exp(x_d - M_d), and of the
//                   unnormalised residual max(0, e_t - rho' e_d) with the draft entries it
//                   keeps, at rho' = S_t / S_d from the float32-accurate stats; per segment
//                   and per 512-entry sub-segment.  Pair slots: the segment's share of the
//                   overlap sum min(p_t, p_d) = 1 - TV of every other draft pair, as
//                   2^min(l_t, l_d) with l = (x - M) log2 e - log2 S (one float32
//                   exponential per entry pair, float64 sum).
//   pick_kernel     one workgroup per request: labels = the summed overlaps; the exact ratio
//                   rho = S_t / S_d from the float64 sums corrects each residual mass to
//                   first order, A(rho) = A(rho') - (rho - rho') D (exact up to the entries
//                   whose sign differs between rho' and rho, a second-order term); u * Q
//                   locates the segment, then the sub-segment, whose 512 entries are
//                   rescanned with exact weights max(0, e_t - rho e_d) and a block-wide
//                   prefix sum; then the commit (accept_len, committed, context_lens).
// The draw returns an index that has to agree with a float64 definition, so everything the
// draw reads is float64: exp is 2^y by range reduction, a 256-entry table of 2^(j/256) and a
// degree-4 Taylor polynomial of 2^f on |f| <= 1/512 (about 1.5 ulp); the table itself and the
// few other float64 exponentials use a degree-13 polynomial on |f| <= 1/2.
#include <type_traits>

#include "exp2_f64.h"
#include "rva_common.h"

namespace rva {
namespace {

constexpr int kSeg = 16384;
constexpr int kThreads = 256;          // stats pass
constexpr int kPer = kSeg / kThreads;  // entries per thread per segment in the stats pass
constexpr int kWideThreads = 512;      // float64 passes (draw sums, pair pass)
constexpr int kWidePer = kSeg / kWideThreads;
constexpr int kSubLen = 512;                // sub-segment: what one wave covers per group
constexpr int kSub = kSeg / kSubLen;         // sub-segments per segment
constexpr int kPickThreads = kSubLen;        // the pick rescans one sub-segment, an entry a thread
static_assert(kSubLen == 8 * kWave, "a wave's group of 8 entries per lane is one sub-segment");
static_assert(kSub <= kWave, "the pick holds one sub-segment per lane");
constexpr float kLog2e = 1.44269504088896341f;

// e^(x - m) in float32 (x = -inf gives 0; m must be finite)
__device__ __forceinline__ float exp_shift(float x, float m) {
  return __builtin_amdgcn_exp2f((x - m) * kLog2e);
}

// Per-request decision record written by decide_kernel.
struct Decision {
  int n;         // accepted drafts; -1: request skipped (invalid window)
  int id_t;      // row id of the draw's target row
  int id_d;      // row id of the residual draw's draft row, -1 for the bonus draw
  int pad;
  float Mt, Md;  // maxima of those rows
  double rho32;  // S_t / S_d from the float32-accurate segment stats
};

// Float64 per-segment sums of a draw slot: S_t, S_d, A(rho'), D (see the header); per
// sub-segment: S_t, A(rho'), D.
constexpr int kDrawSums = 4;
constexpr int kSubSums = 3;

struct WsLayout {
  int nseg, n_ids;
  size_t off_m, off_s, off_nm, off_tv, off_dec, off_r1, off_sub, total;
};

__host__ __device__ inline WsLayout ws_layout(int B, int gamma, int V, int max_rows) {
  WsLayout w;
  w.nseg = (V + kSeg - 1) / kSeg;
  const int G1 = gamma - 1;
  w.n_ids = max_rows + B * G1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  w.off_m = take(sizeof(float) * size_t(w.n_ids) * w.nseg);
  w.off_s = take(sizeof(double) * size_t(w.n_ids) * w.nseg);
  w.off_nm = take(sizeof(float2) * size_t(w.n_ids));
  w.off_tv = take(sizeof(double) * size_t(B) * G1 * w.nseg);
  w.off_dec = take(sizeof(Decision) * size_t(B));
  w.off_r1 = take(sizeof(double) * size_t(B) * w.nseg * kDrawSums);
  w.off_sub = take(sizeof(double) * size_t(B) * w.nseg * kSub * kSubSums);
  w.total = off;
  return w;
}

// Row ids: target row r (packed row index) is id r; draft row (b, k) is id max_rows + b*G1 + k.
struct Ctx {
  AcceptArgs a;
  Exp2Poly P;
  WsLayout L;
  float* st_m;    // [n_ids][nseg] segment maxima
  double* st_s;   // [n_ids][nseg] segment sums of exp(x - m_s)
  float2* nm;     // [n_ids] (row max, 1 / row sum) of the rows decide_kernel covered
  double* tv;     // [B*G1][nseg] segment shares of the overlap sum min(p_t, p_d) = 1 - TV
  Decision* dec;  // [B]
  double* r1;     // [B][nseg][kDrawSums] float64 sums of the draw slots
  double* sub;    // [B][nseg][kSub][kSubSums] the same per sub-segment
};

// Request b's packed rows [cu[b], cu[b] + w) lie inside [0, max_rows) and w in [1, gamma].
// Both offsets are loaded before either is tested (no short-circuit: one round trip).
__device__ __forceinline__ bool req_ok(const Ctx& c, int b) {
  const int r0 = c.a.cu[b], r1 = c.a.cu[b + 1];
  return (r0 >= 0) & (r1 - r0 >= 1) & (r1 - r0 <= c.a.gamma) & (r1 <= c.a.max_rows);
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(const Ctx& c, int id) {
  if (id < c.a.max_rows) return static_cast<const T*>(c.a.target) + size_t(id) * c.a.V;
  return static_cast<const T*>(c.a.draft) + size_t(id - c.a.max_rows) * c.a.V;
}

// A thread's share (kSeg / NT entries) of one segment, kept as loaded: bf16 as packed pairs
// (half the registers of float32), float32 as is.  Entry q = 8 g + j of thread t is
// segment entry g * 8 NT + 8 t + j, so for each group g a wave covers 512 consecutive
// entries (sub-segment 8 g NT / 512 + wave).  Entries past the row end read as -inf.
template <typename T, int NT>
struct SegData;

template <int NT>
struct SegData<uint16_t, NT> {
  static constexpr int P = kSeg / NT;
  uint32_t w[P / 2];
  __device__ __forceinline__ float operator[](int q) const {
    return (q & 1) ? __uint_as_float(w[q >> 1] & 0xffff0000u) : __uint_as_float(w[q >> 1] << 16);
  }
  __device__ __forceinline__ void load(const uint16_t* row, int V, int seg) {
    constexpr uint32_t kNegInf2 = 0xff80ff80u;  // two bf16 -inf
    const int base = seg * kSeg + int(threadIdx.x) * 8;
    if (V % 8 == 0) {
#pragma unroll
      for (int g = 0; g < P / 8; ++g) {
        const int v = base + g * 8 * NT;
        if (v < V) {
          const uint4 u = *reinterpret_cast<const uint4*>(row + v);
          w[4 * g] = u.x;
          w[4 * g + 1] = u.y;
          w[4 * g + 2] = u.z;
          w[4 * g + 3] = u.w;
        } else {
          w[4 * g] = w[4 * g + 1] = w[4 * g + 2] = w[4 * g + 3] = kNegInf2;
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < P / 8; ++g)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int v = base + g * 8 * NT + 2 * k;
          const uint32_t lo = v < V ? row[v] : 0xff80u;
          const uint32_t hi = v + 1 < V ? row[v + 1] : 0xff80u;
          w[4 * g + k] = lo | (hi << 16);
        }
    }
  }
};

template <int NT>
struct SegData<float, NT> {
  static constexpr int P = kSeg / NT;
  float f[P];
  __device__ __forceinline__ float operator[](int q) const { return f[q]; }
  __device__ __forceinline__ void load(const float* row, int V, int seg) {
    const int base = seg * kSeg + int(threadIdx.x) * 8;
    if (V % 4 == 0) {
#pragma unroll
      for (int g = 0; g < P / 8; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int v = base + g * 8 * NT + 4 * h;
          float4 u = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
          if (v < V) u = *reinterpret_cast<const float4*>(row + v);
          f[8 * g + 4 * h] = u.x;
          f[8 * g + 4 * h + 1] = u.y;
          f[8 * g + 4 * h + 2] = u.z;
          f[8 * g + 4 * h + 3] = u.w;
        }
    } else {
#pragma unroll
      for (int g = 0; g < P / 8; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int v = base + g * 8 * NT + j;
          f[8 * g + j] = v < V ? row[v] : -INFINITY;
        }
    }
  }
};

template <int NT>
__device__ __forceinline__ float block_max(float v, float* sm) {
  v = wave_max(v);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __syncthreads();
  if (lane == 0) sm[wave] = v;
  __syncthreads();
  float r = sm[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, sm[i]);
  return r;
}

// float64 sum in a fixed order (wave butterfly, then the wave totals in order); every thread
// receives the same value.
template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, double* sm) {
  v = wave_sum_f64(v);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __syncthreads();
  if (lane == 0) sm[wave] = v;
  __syncthreads();
  double r = sm[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r += sm[i];
  return r;
}

// Draw-row totals S_t, S_d over all segments: one wave, lanes over segments, butterfly sum
// (every lane gets the same value).
__device__ __forceinline__ void draw_totals(const Ctx& c, int b, double& St, double& Sd) {
  const int lane = threadIdx.x % kWave;
  double st = 0.0, sd = 0.0;
  for (int s = lane; s < c.L.nseg; s += kWave) {
    const double* r = c.r1 + (size_t(b) * c.L.nseg + s) * kDrawSums;
    st += r[0];
    sd += r[1];
  }
  St = wave_sum_f64(st);
  Sd = wave_sum_f64(sd);
}

// Draw mass of segment s: the residual A(rho) (first-order corrected, clamped at 0) or the
// target mass S_t of the segment (bonus draw and the all-zero-residual fallback).
__device__ __forceinline__ double seg_mass(const Ctx& c, int b, int s, bool residual, double drho) {
  const double* r = c.r1 + (size_t(b) * c.L.nseg + s) * kDrawSums;
  if (!residual) return r[0];
  const double m = r[2] - drho * r[3];
  return m > 0.0 ? m : 0.0;
}

// Draw mass of sub-segment u of segment s (same rule as seg_mass).
__device__ __forceinline__ double sub_mass(const Ctx& c, int b, int s, int u, bool residual,
                                           double drho) {
  const double* r = c.sub + ((size_t(b) * c.L.nseg + s) * kSub + u) * kSubSums;
  if (!residual) return r[0];
  const double m = r[1] - drho * r[2];
  return m > 0.0 ? m : 0.0;
}

// ------------------------------------------------------------------ stats
__device__ __forceinline__ bool id_active(const Ctx& c, int id) {
  if (id < c.a.max_rows) return id < c.a.cu[c.a.B];
  const int j = id - c.a.max_rows, G1 = c.a.gamma - 1;
  const int b = j / G1, k = j % G1;
  return req_ok(c, b) && k < c.a.cu[b + 1] - c.a.cu[b] - 1;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void stats_kernel(Ctx c) {
  __shared__ float smf[kThreads / kWave];
  __shared__ double smd[kThreads / kWave];
  const int seg = blockIdx.x, id = blockIdx.y;
  if (!id_active(c, id)) return;
  SegData<T, kThreads> x;
  x.load(row_ptr<T>(c, id), c.a.V, seg);
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i) m = fmaxf(m, x[i]);
  m = block_max<kThreads>(m, smf);
  const float ms = m == -INFINITY ? 0.f : m;  // fully masked segment: every term is 0
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kPer; i += 8) {
    float run = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) run += exp_shift(x[i + j], ms);
    s += double(run);
  }
  s = block_sum_f64<kThreads>(s, smd);
  if (threadIdx.x == 0) {
    c.st_m[size_t(id) * c.L.nseg + seg] = m;
    c.st_s[size_t(id) * c.L.nseg + seg] = s;
  }
}

// ------------------------------------------------------------------ decide
constexpr int kDecideThreads = 512;

// Row rr of request b in decide order: target rows 0..w-1, then draft rows 0..w-2.
__device__ __forceinline__ int decide_row_id(const Ctx& c, int b, int r0, int w, int rr) {
  return rr < w ? r0 + rr : c.a.max_rows + b * (c.a.gamma - 1) + (rr - w);
}

template <typename T, bool commit>
__global__ __launch_bounds__(kDecideThreads) void decide_kernel(Ctx c) {
  __shared__ float sM[2 * 64];
  __shared__ double sS[2 * 64];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int G1 = c.a.gamma - 1;
  // wave 0, lane k: the drafted token and its uniform are loaded before the window is known
  // (they do not depend on it), so that only the logit loads wait for cu_seqlens.  Every
  // lane of every wave loads (lanes past G1 repeat the last draft; wave 0's are used): a
  // load into a register that other lanes set on another path would be waited for where
  // the paths join, and the compiler cannot tell that a wave test is uniform.
  int x = 0;
  float u = 0.f;
  if (commit) {
    const int k = min(lane, G1 - 1);
    x = c.a.tokens[size_t(b) * G1 + k];
    u = c.a.u_acc[size_t(b) * G1 + k];
  }
  if (!req_ok(c, b)) {
    if (tid == 0) {
      flag(c.a.status, RVA_DEV_BAD_WINDOW);
      if (commit) c.dec[b].n = -1;
    }
    return;
  }
  const int r0 = c.a.cu[b];
  const int w = c.a.cu[b + 1] - r0;
  // row normalisers: one wave per row, lanes over segments.  A wave's first row (every row
  // when nseg <= 64) has its segment maxima and sums requested at once, before the drafted
  // tokens' logits, so that waiting for them does not also wait for those (the wait counter
  // drains in order).
  const int nrows = 2 * w - 1;
  const int nseg = c.L.nseg;
  float m0 = -INFINITY;
  double s0 = 0.0;
  if (wave < nrows && lane < nseg) {
    const int id = decide_row_id(c, b, r0, w, wave);
    m0 = c.st_m[size_t(id) * nseg + lane];
    s0 = c.st_s[size_t(id) * nseg + lane];
  }
  // lane k < w-1 of wave 0: the drafted token's logits, kept raw until the decision (every
  // lane loads, from a clamped draft: see above)
  T lt_raw = T(0), ld_raw = T(0);
  if (commit) {
    const int k = min(lane, max(w - 2, 0));
    const bool bad = x < 0 || x >= c.a.V;
    if (bad && wave == 0 && lane < w - 1) flag(c.a.status, RVA_DEV_BAD_TOKEN);
    x = x < 0 ? 0 : (x >= c.a.V ? c.a.V - 1 : x);
    lt_raw = row_ptr<T>(c, r0 + k)[x];
    ld_raw = row_ptr<T>(c, c.a.max_rows + b * G1 + k)[x];
  }
  for (int rr = wave; rr < nrows; rr += kDecideThreads / kWave) {
    const int id = decide_row_id(c, b, r0, w, rr);
    const float* rm = c.st_m + size_t(id) * nseg;
    const double* rs = c.st_s + size_t(id) * nseg;
    const bool first = rr == wave;
    float m = first ? m0 : -INFINITY;
    for (int s = lane + (first ? kWave : 0); s < nseg; s += kWave) m = fmaxf(m, rm[s]);
    m = wave_max(m);
    double acc = (first && lane < nseg) ? s0 * exp_shift_f64(c.P, m0, m) : 0.0;
    for (int s = lane + (first ? kWave : 0); s < nseg; s += kWave) acc += rs[s] * exp_shift_f64(c.P, rm[s], m);
    acc = wave_sum_f64(acc);
    if (lane == 0) {
      sM[rr] = m;
      sS[rr] = acc;
      c.nm[id] = make_float2(m, float(1.0 / acc));
    }
  }
  if (!commit) return;
  __syncthreads();
  if (wave != 0) return;
  const float qnan = __int_as_float(0x7fc00000);
  bool reject = false;
  if (lane < G1) {
    const size_t o = size_t(b) * G1 + lane;
    if (lane < w - 1) {
      const float lt = Elem<T>::load(&lt_raw, 0), ld = Elem<T>::load(&ld_raw, 0);
      const double pt = exp_shift_f64(c.P, lt, sM[lane]) / sS[lane];
      const double pd = exp_shift_f64(c.P, ld, sM[w + lane]) / sS[w + lane];
      if (c.a.pt_at) c.a.pt_at[o] = float(pt);
      if (c.a.pd_at) c.a.pd_at[o] = float(pd);
      const double r = pd == 0.0 ? INFINITY : pt / pd;
      reject = !(double(u) < (r < 1.0 ? r : 1.0));
    } else {
      if (c.a.pt_at) c.a.pt_at[o] = qnan;
      if (c.a.pd_at) c.a.pd_at[o] = qnan;
    }
  }
  // first rejected draft (G1 <= 63: one lane per draft)
  const unsigned long long rej = __ballot(reject);
  const int n_full = rej ? __ffsll(rej) - 1 : w - 1;
  // cap-accept: the whole block was verified, but only drafts inside the window (cap - 1 of
  // them) may be committed; a rejection inside the window draws its residual, otherwise the
  // bonus comes from the window's last target row -- what compact mode does for that window
  int cap = w;
  if (c.a.cap) {
    cap = c.a.cap[b];
    if (cap < 1 || cap > w) {
      if (lane == 0) flag(c.a.status, RVA_DEV_BAD_WINDOW);
      cap = cap < 1 ? 1 : w;
    }
  }
  const bool residual = n_full < cap - 1;
  const int n = residual ? n_full : cap - 1;
  if (lane == 0) {
    Decision d;
    d.n = n;
    d.id_t = r0 + n;
    d.id_d = residual ? c.a.max_rows + b * G1 + n : -1;
    d.pad = 0;
    d.Mt = sM[n];
    d.Md = residual ? sM[w + n] : 0.f;
    d.rho32 = residual ? sS[n] / sS[w + n] : 0.0;
    c.dec[b] = d;
    if (c.a.accept_len_full) c.a.accept_len_full[b] = n_full;
  }
}

// ------------------------------------------------------------------ pair pass
// Wave butterfly then wave totals in order, for N sums at once; thread 0 gets the results.
template <int N>
__device__ __forceinline__ void block_sums_f64(double (&v)[N], double (*sm)[N]) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = wave_sum_f64(v[q]);
  if (lane == 0)
#pragma unroll
    for (int q = 0; q < N; ++q) sm[wave][q] = v[q];
  __syncthreads();
  if (threadIdx.x == 0)
#pragma unroll
    for (int q = 0; q < N; ++q) {
      double r = sm[0][q];
      for (int i = 1; i < kWideThreads / kWave; ++i) r += sm[i][q];
      v[q] = r;
    }
}

// blockIdx.y < draw_slots: the draw slot of request blockIdx.y (float64-heavy, dispatched
// first); above: draft pair (blockIdx.y - draw_slots) = b*G1 + k for the labels (when per_pair).
template <typename T>
__device__ __forceinline__ void pair_body(const Ctx& c, int draw_slots, int per_pair) {
  __shared__ double sm[kWideThreads / kWave][kDrawSums + 1];
  __shared__ double smd[kWideThreads / kWave];
  const int seg = blockIdx.x;
  const int G1 = c.a.gamma - 1;
  const int y = blockIdx.y;
  if (y < draw_slots) {
    const int b = y;
    const Decision d = c.dec[b];
    if (d.n < 0) return;
    const bool residual = d.id_d >= 0;
    const bool lab = per_pair && residual;  // this pair's overlap share is taken here too
    SegData<T, kWideThreads> xt, xd;
    xt.load(row_ptr<T>(c, d.id_t), c.a.V, seg);
    double v[kDrawSums + 1] = {0.0, 0.0, 0.0, 0.0, 0.0};
    double it = 0.0, id = 0.0;
    if (residual) xd.load(row_ptr<T>(c, d.id_d), c.a.V, seg);
    __shared__ double tab[256];
    fill_exp2_tab(c.P, tab);  // overlaps the row loads
    if (lab) {
      it = double(c.nm[d.id_t].y);
      id = double(c.nm[d.id_d].y);
    }
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    double* subp = c.sub + (size_t(b) * c.L.nseg + seg) * kSub * kSubSums;
#pragma unroll
    for (int g = 0; g < kWidePer / 8; ++g) {
      double gs[kSubSums] = {0.0, 0.0, 0.0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double et = exp_shift_tab(c.P, tab, xt[8 * g + j], d.Mt);
        gs[0] += et;
        if (residual) {
          const double ed = exp_shift_tab(c.P, tab, xd[8 * g + j], d.Md);
          v[1] += ed;
          const double r = et - d.rho32 * ed;
          if (r > 0.0) {
            gs[1] += r;
            gs[2] += ed;
          }
          v[4] += fmin(et * it, ed * id);  // overlap min(p_t, p_d)
        }
      }
      v[0] += gs[0];
      v[2] += gs[1];
      v[3] += gs[2];
#pragma unroll
      for (int q = 0; q < kSubSums; ++q) gs[q] = wave_sum_f64(gs[q]);
      if (lane == 0)
#pragma unroll
        for (int q = 0; q < kSubSums; ++q) subp[(g * (kWideThreads / kWave) + wave) * kSubSums + q] = gs[q];
    }
    block_sums_f64<kDrawSums + 1>(v, sm);
    if (threadIdx.x == 0) {
      double* r = c.r1 + (size_t(b) * c.L.nseg + seg) * kDrawSums;
#pragma unroll
      for (int q = 0; q < kDrawSums; ++q) r[q] = v[q];
      if (lab) c.tv[(size_t(b) * G1 + d.n) * c.L.nseg + seg] = v[4];
    }
    return;
  }
  const int j = y - draw_slots;
  const int b = j / G1, k = j % G1;
  // the window and the decision record go out together (the record does not depend on
  // the window), so the row loads wait for one round trip, not two
  const int r0 = c.a.cu[b], r1 = c.a.cu[b + 1];
  Decision d;
  d.id_d = -1;
  d.n = -1;
  if (draw_slots > 0) d = c.dec[b];
  if (!((r0 >= 0) & (r1 - r0 >= 1) & (r1 - r0 <= c.a.gamma) & (r1 <= c.a.max_rows))) return;  // req_ok
  if (k >= r1 - r0 - 1) return;
  if (d.id_d >= 0 && d.n == k) return;  // done by the draw slot
  const int id_t = r0 + k;
  const int id_d = c.a.max_rows + b * G1 + k;
  SegData<T, kWideThreads> xt, xd;
  xt.load(row_ptr<T>(c, id_t), c.a.V, seg);
  xd.load(row_ptr<T>(c, id_d), c.a.V, seg);
  const float2 nt = c.nm[id_t], nd = c.nm[id_d];
  // min(p_t, p_d) = 2^min(lt, ld) with l = (x - M) log2 e - log2 S = x log2 e + c,
  // c = -(M log2 e + log2 S): one FMA per entry and one exponential per entry pair (the label
  // is the segment sums of these overlaps).  Forming l from x log2 e instead of (x - M) log2 e
  // moves it by a few float32 ulp of |x log2 e| (< 30 for logits of magnitude < 20), a
  // relative change of about 1e-6 in each term.
  const float ct = -fmaf(nt.x, kLog2e, -__log2f(nt.y));  // nm.y = 1 / S
  const float cd = -fmaf(nd.x, kLog2e, -__log2f(nd.y));
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kWidePer; i += 8) {
    float run = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float lt = fmaf(xt[i + u], kLog2e, ct);
      const float ld = fmaf(xd[i + u], kLog2e, cd);
      run += __builtin_amdgcn_exp2f(fminf(lt, ld));
    }
    acc += double(run);
  }
  acc = block_sum_f64<kWideThreads>(acc, smd);
  if (threadIdx.x == 0) c.tv[(size_t(b) * G1 + k) * c.L.nseg + seg] = acc;
}

// bfloat16 rows: 8 waves per SIMD (64 VGPRs), four workgroups per CU, so that one computing
// still leaves three streaming (the draw slots' float64 path spills a few registers to
// scratch).  float32 rows hold twice the registers and keep the default.
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void pair_kernel_bf16(
    Ctx c, int draw_slots, int per_pair) {
  pair_body<uint16_t>(c, draw_slots, per_pair);
}
__global__ __launch_bounds__(kWideThreads) void pair_kernel_f32(Ctx c, int draw_slots, int per_pair) {
  pair_body<float>(c, draw_slots, per_pair);
}

// ------------------------------------------------------------------ pick + commit + labels
// One wave: the first of n items (masses mass(i) >= 0, in index order) at which the running
// sum, started at `start`, passes t; `found` = that item and `base` = the running sum before
// it.  If rounding leaves t unpassed, the last item with mass (or item 0).
template <typename F>
__device__ __forceinline__ void locate(double t, double start, int n, F mass, int& found,
                                       double& base) {
  const int lane = threadIdx.x % kWave;
  int last = 0;
  double base_last = start, carry = start;
  found = -1;
  base = start;
  for (int i0 = 0; i0 < n && found < 0; i0 += kWave) {
    const int i = i0 + lane;
    const double m = i < n ? mass(i) : 0.0;
    const double inc = wave_inclusive(m, 0.0, [](double x, double y) { return x + y; }) + carry;
    const double exc = inc - m;
    const unsigned long long hit = __ballot(m > 0.0 && inc > t);
    const unsigned long long pos = __ballot(m > 0.0);
    if (pos) {
      const int l = 63 - __clzll(pos);
      last = i0 + l;
      base_last = readlane_f64(exc, l);
    }
    if (hit) {
      const int l = __ffsll(hit) - 1;
      found = i0 + l;
      base = readlane_f64(exc, l);
    }
    carry = lane63(inc);
  }
  if (found < 0) {
    found = last;
    base = base_last;
  }
}

template <typename T, bool commit>
__global__ __launch_bounds__(kPickThreads) void pick_kernel(Ctx c) {
  __shared__ double s_t, s_base, s_rho;
  __shared__ int s_pos, s_residual;
  __shared__ double s_wave[kPickThreads / kWave];
  __shared__ int s_y, s_last;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int G1 = c.a.gamma - 1;
  const int nseg = c.L.nseg;
  // Every load that depends on no other goes out first, before the window check and the
  // label stores (which may alias them as far as the compiler knows): the decision record,
  // the drafted tokens, the context length and lane s's draw sums of segment s (when a wave
  // covers every segment).
  const bool lanes_cover = nseg <= kWave;
  Decision d;
  double r1v[kDrawSums] = {0.0, 0.0, 0.0, 0.0};
  int tok = -1, ctx0 = 0;  // thread i < gamma: drafted token i; thread 0: the context length
  if (commit) {
    d = c.dec[b];
    if (tid < G1) tok = c.a.tokens[size_t(b) * G1 + tid];
    if (tid == 0) ctx0 = c.a.context_lens[b];
    if (wave == 0 && lanes_cover && lane < nseg) {
      const double* r = c.r1 + (size_t(b) * nseg + lane) * kDrawSums;
#pragma unroll
      for (int q = 0; q < kDrawSums; ++q) r1v[q] = r[q];
    }
  }
  if (!req_ok(c, b)) return;
  const int w = c.a.cu[b + 1] - c.a.cu[b];
  if (c.a.labels) {  // one wave per draft (wave 0 is left to the draw when there is one):
                     // lanes sum the segment shares of the overlap
    const int first = commit ? 1 : 0, stride = kPickThreads / kWave - first;
    for (int k = wave - first; k >= 0 && k < G1; k += stride) {
      const size_t o = size_t(b) * G1 + k;
      double ov = 0.0;
      if (k < w - 1)
        for (int s = lane; s < nseg; s += kWave) ov += c.tv[o * nseg + s];
      ov = wave_sum_f64(ov);
      // c* = 1 - TV = sum_v min(p_d, p_t)
      if (lane == 0) c.a.labels[o] = k < w - 1 ? float(ov) : __int_as_float(0x7fc00000);
    }
  }
  if (!commit) return;
  if (d.n < 0) return;
  // the 2^(j/256) table of the rescan is filled by waves 1.. while wave 0 locates the
  // sub-segment; the barrier after the search publishes both
  static_assert(kPickThreads - kWave >= 256, "waves 1.. fill the 256-entry table");
  __shared__ double tab[256];
  if (tid >= kWave && tid - kWave < 256) tab[tid - kWave] = exp2_f64(c.P, double(tid - kWave) / 256.0);
  if (wave == 0 && lanes_cover) {
    // the general path below with every per-segment value held by its lane: the same sums
    // in the same order, without re-reading the draw sums for each step
    const double St = wave_sum_f64(r1v[0]), Sd = wave_sum_f64(r1v[1]);
    bool residual = d.id_d >= 0;
    const double rho = residual ? St / Sd : 0.0;
    const double drho = rho - d.rho32;
    auto lane_mass = [&](bool res) {
      if (lane >= nseg) return 0.0;
      if (!res) return r1v[0];
      const double m = r1v[2] - drho * r1v[3];
      return m > 0.0 ? m : 0.0;
    };
    double mass = lane_mass(residual);
    double Q = wave_sum_f64(mass);
    if (residual && !(Q > 0.0)) {  // residual identically zero: draw from p_t instead
      residual = false;
      Q = St;
      mass = lane_mass(false);
    }
    const double t = double(c.a.u_res[b]) * Q;
    int seg = -1;
    double base = 0.0;
    locate(t, 0.0, nseg, [&](int) { return mass; }, seg, base);
    // lane u: sub-segment u of the chosen segment (kSub <= kWave)
    double sm = 0.0;
    if (lane < kSub) sm = sub_mass(c, b, seg, lane, residual, drho);
    int sub = -1;
    double base2 = base;
    locate(t, base, kSub, [&](int) { return sm; }, sub, base2);
    if (lane == 0) {
      s_t = t;
      s_base = base2;
      s_pos = seg * kSeg + sub * kSubLen;
      s_residual = residual;
      s_rho = rho;
      s_y = 0x7fffffff;
      s_last = -1;
    }
  } else if (wave == 0) {
    double St, Sd;
    draw_totals(c, b, St, Sd);
    bool residual = d.id_d >= 0;
    const double rho = residual ? St / Sd : 0.0;
    const double drho = rho - d.rho32;
    double q = 0.0;
    for (int s = lane; s < nseg; s += kWave) q += seg_mass(c, b, s, residual, drho);
    double Q = wave_sum_f64(q);
    if (residual && !(Q > 0.0)) {  // residual identically zero: draw from p_t instead
      residual = false;
      Q = St;
    }
    const double t = double(c.a.u_res[b]) * Q;
    // first segment whose running mass passes t, then the first sub-segment inside it
    int seg = -1;
    double base = 0.0;
    locate(t, 0.0, nseg, [&](int s) { return seg_mass(c, b, s, residual, drho); }, seg, base);
    int sub = -1;
    double base2 = base;
    locate(t, base, kSub, [&](int u) { return sub_mass(c, b, seg, u, residual, drho); }, sub, base2);
    if (lane == 0) {
      s_t = t;
      s_base = base2;
      s_pos = seg * kSeg + sub * kSubLen;
      s_residual = residual;
      s_rho = rho;
      s_y = 0x7fffffff;
      s_last = -1;
    }
  }
  __syncthreads();
  const bool residual = s_residual;
  const int v = s_pos + tid;
  // both rows' entries requested together (the draft row's from the target row for a bonus
  // draw, and past V from the last entry), then weighed
  const int vc = min(v, c.a.V - 1);
  const T xt = row_ptr<T>(c, d.id_t)[vc];
  const T xd = row_ptr<T>(c, residual ? d.id_d : d.id_t)[vc];
  asm volatile("" ::: "memory");  // keeps both loads here, ahead of the branches that use them
  double wgt = 0.0;
  if (v < c.a.V) {
    wgt = exp_shift_tab(c.P, tab, Elem<T>::load(&xt, 0), d.Mt);
    if (residual) {
      wgt -= s_rho * exp_shift_tab(c.P, tab, Elem<T>::load(&xd, 0), d.Md);
      wgt = wgt > 0.0 ? wgt : 0.0;
    }
  }
  // inclusive prefix in index order: wave scan (DPP), then the wave totals
  const double inc = wave_inclusive(wgt, 0.0, [](double x, double y) { return x + y; });
  if (lane == kWave - 1) s_wave[wave] = inc;
  __syncthreads();
  double cum = s_base;
  for (int i = 0; i < wave; ++i) cum += s_wave[i];
  cum += inc;
  // the first entry past u * Q and the last positive entry: found per wave by ballot (entry
  // v = s_pos + tid is in lane order), then one LDS atomic per wave -- one atomic per lane
  // on a single address serialises the whole workgroup
  const unsigned long long hit = __ballot(wgt > 0.0 && cum > s_t), pos = __ballot(wgt > 0.0);
  if (lane == 0) {
    if (hit) atomicMin(&s_y, v + __ffsll(hit) - 1);
    if (pos) atomicMax(&s_last, v + 63 - __clzll(pos));
  }
  __syncthreads();
  // the commit, one thread per block position (rounding that left u * Q past this
  // sub-segment's end takes its last positive entry)
  const int y = s_y != 0x7fffffff ? s_y : (s_last >= 0 ? s_last : s_pos);
  const int n = d.n;
  if (tid < c.a.gamma) c.a.committed[size_t(b) * c.a.gamma + tid] = tid < n ? tok : (tid == n ? y : -1);
  if (tid == 0) {
    c.a.accept_len[b] = n;
    c.a.context_lens[b] = ctx0 + n + 1;
  }
}

template <typename T>
hipError_t launch_typed(const Ctx& c, bool commit, hipStream_t stream) {
  const AcceptArgs& a = c.a;
  const int nseg = c.L.nseg, G1 = a.gamma - 1;
  const bool with_labels = a.labels != nullptr;
  hipLaunchKernelGGL(stats_kernel<T>, dim3(nseg, c.L.n_ids), dim3(kThreads), 0, stream, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (commit)
    hipLaunchKernelGGL((decide_kernel<T, true>), dim3(a.B), dim3(kDecideThreads), 0, stream, c);
  else
    hipLaunchKernelGGL((decide_kernel<T, false>), dim3(a.B), dim3(kDecideThreads), 0, stream, c);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int draw_slots = commit ? a.B : 0;
  const int slots = draw_slots + (with_labels ? a.B * G1 : 0);
  if (slots > 0) {
    if constexpr (std::is_same<T, uint16_t>::value)
      hipLaunchKernelGGL(pair_kernel_bf16, dim3(nseg, slots), dim3(kWideThreads), 0, stream, c,
                         draw_slots, int(with_labels));
    else
      hipLaunchKernelGGL(pair_kernel_f32, dim3(nseg, slots), dim3(kWideThreads), 0, stream, c,
                         draw_slots, int(with_labels));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (commit)
    hipLaunchKernelGGL((pick_kernel<T, true>), dim3(a.B), dim3(kPickThreads), 0, stream, c);
  else
    hipLaunchKernelGGL((pick_kernel<T, false>), dim3(a.B), dim3(kPickThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace

size_t accept_workspace_bytes(int B, int gamma, int V, int max_rows) {
  return ws_layout(B, gamma, V, max_rows).total;
}

hipError_t launch_accept(const AcceptArgs& a, int logit_dtype, bool commit, hipStream_t stream) {
  Ctx c;
  c.a = a;
  c.P = kExp2Taylor;
  c.L = ws_layout(a.B, a.gamma, a.V, a.max_rows);
  char* base = static_cast<char*>(a.ws);
  c.st_m = reinterpret_cast<float*>(base + c.L.off_m);
  c.st_s = reinterpret_cast<double*>(base + c.L.off_s);
  c.nm = reinterpret_cast<float2*>(base + c.L.off_nm);
  c.tv = reinterpret_cast<double*>(base + c.L.off_tv);
  c.dec = reinterpret_cast<Decision*>(base + c.L.off_dec);
  c.r1 = reinterpret_cast<double*>(base + c.L.off_r1);
  c.sub = reinterpret_cast<double*>(base + c.L.off_sub);
  return logit_dtype == RVA_BF16 ? launch_typed<uint16_t>(c, commit, stream)
                                 : launch_typed<float>(c, commit, stream);
}

}  // namespace rva
