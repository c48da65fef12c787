// Stages 4 and 5: full-vocabulary speculative-sampling acceptance, the residual / bonus
// draw, the commit, and the TV-distance confidence labels.
//
// Sources: "DSpark：投机解码与生产级 Serving 学习笔记" (sorenprojections.com) section 02
// (the acceptance rule keeps the target distribution; acceptance is prefix-only) and
// section 07 (label c* = 1 - 0.5 ||p_d - p_t||_1); "DFlash 到 DSpark in SGLang" section
// "Background" (each verify forward also yields one target token).
//
// Rows are split into segments of kSeg vocabulary entries; every kernel below is a grid
// over (segment, row or request) so that hundreds of rows spread over all CUs.
//   stats_kernel   per (row, segment): exact max, and sum of exp(x - max) (float32 exp,
//                  float64 accumulation).  One HBM pass over every active row.
//   tv_kernel      per (draft pair, segment): row normalisers from the segment stats,
//                  then sum over the segment of max(0, p_t - p_d) in float64 (= the
//                  segment's share of the TV distance).  Only launched when labels are
//                  requested.
//   decide_kernel  one wave per request, one lane per draft: p_t(x), p_d(x) with a float64
//                  exp at the drafted token, accept bits, first rejection by ballot;
//                  labels = 1 - sum of the TV shares; records which row pair to draw from.
//   draw_sum_kernel / draw_q_kernel / draw_pick_kernel: the residual or bonus draw in
//                  float64 throughout (exp and sums), because its result is an index that
//                  must match a float64 definition bit for bit: first the two float64
//                  normalisers, then per-segment masses of the draw weights, then one
//                  workgroup per request locates the segment holding u * S and scans it.
//                  The pick kernel also commits (accept_len, committed, context_lens).
#include "rva_common.h"

namespace rva {
namespace {

constexpr int kSeg = 8192;
constexpr int kThreads = 256;
constexpr int kPer = kSeg / kThreads;  // elements per thread per segment

struct WsLayout {
  int nseg, n_ids;
  size_t off_m, off_s, off_tv, off_dec, off_r1, off_r2, total;
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
  w.off_tv = take(sizeof(double) * size_t(B) * G1 * w.nseg);
  w.off_dec = take(sizeof(int) * size_t(B) * 4);
  w.off_r1 = take(sizeof(double) * size_t(B) * w.nseg * 2);
  w.off_r2 = take(sizeof(double) * size_t(B) * w.nseg);
  w.total = off;
  return w;
}

struct Ctx {
  AcceptArgs a;
  WsLayout L;
  float* st_m;
  double* st_s;
  double* tv;
  int* dec;
  double* r1;
  double* r2;
};

__device__ __forceinline__ int window_of(const Ctx& c, int b) {
  const int w = c.a.cu[b + 1] - c.a.cu[b];
  return w < 1 ? 1 : (w > c.a.gamma ? c.a.gamma : w);
}

// Request b's packed rows [cu[b], cu[b] + w) lie inside [0, max_rows) and w in [1, gamma].
__device__ __forceinline__ bool req_ok(const Ctx& c, int b) {
  const int r0 = c.a.cu[b], r1 = c.a.cu[b + 1];
  return r0 >= 0 && r1 - r0 >= 1 && r1 - r0 <= c.a.gamma && r1 <= c.a.max_rows;
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(const Ctx& c, int id) {
  if (id < c.a.max_rows) return static_cast<const T*>(c.a.target) + size_t(id) * c.a.V;
  return static_cast<const T*>(c.a.draft) + size_t(id - c.a.max_rows) * c.a.V;
}

// Loads this thread's kPer elements of segment `seg` (as float; -inf past the row end).
template <typename T>
__device__ __forceinline__ void load_seg(const T* row, int V, int seg, float (&x)[kPer]) {
  const int base = seg * kSeg;
  if constexpr (sizeof(T) == 2) {
    if (V % 8 == 0) {
#pragma unroll
      for (int i = 0; i < kPer / 8; ++i) {
        const int v = base + (i * kThreads + int(threadIdx.x)) * 8;
        if (v < V) {
          const uint4 u = *reinterpret_cast<const uint4*>(row + v);
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[i * 8 + 2 * j] = __uint_as_float(w[j] << 16);
            x[i * 8 + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[i * 8 + j] = -INFINITY;
        }
      }
      return;
    }
  } else {
    if (V % 4 == 0) {
#pragma unroll
      for (int i = 0; i < kPer / 4; ++i) {
        const int v = base + (i * kThreads + int(threadIdx.x)) * 4;
        if (v < V) {
          const float4 u = *reinterpret_cast<const float4*>(row + v);
          x[i * 4] = u.x;
          x[i * 4 + 1] = u.y;
          x[i * 4 + 2] = u.z;
          x[i * 4 + 3] = u.w;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) x[i * 4 + j] = -INFINITY;
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int v = base + i * kThreads + int(threadIdx.x);
    x[i] = v < V ? Elem<T>::load(row, v) : -INFINITY;
  }
}

__device__ float block_max(float v, float* sm) {
  v = wave_max(v);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __syncthreads();
  if (lane == 0) sm[wave] = v;
  __syncthreads();
  float r = sm[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) r = fmaxf(r, sm[i]);
  return r;
}

// float64 sum in a fixed order (wave tree, then the 4 wave totals in order).
__device__ double block_sum_f64(double v, double* sm) {
  v = wave_sum_f64(v);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __syncthreads();
  if (lane == 0) sm[wave] = v;
  __syncthreads();
  double r = sm[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) r += sm[i];
  return r;
}

// Row normaliser from the segment stats: exact max, and S = sum_s s_s * exp(m_s - max).
__device__ __forceinline__ void row_norm(const Ctx& c, int id, float& M, double& S) {
  const int nseg = c.L.nseg;
  float m = -INFINITY;
  for (int s = 0; s < nseg; ++s) m = fmaxf(m, c.st_m[size_t(id) * nseg + s]);
  double acc = 0.0;
  for (int s = 0; s < nseg; ++s) {
    const float ms = c.st_m[size_t(id) * nseg + s];
    if (ms != -INFINITY) acc += c.st_s[size_t(id) * nseg + s] * exp(double(ms) - double(m));
  }
  M = m;
  S = acc;
}

__device__ __forceinline__ bool id_active(const Ctx& c, int id, int M_rows) {
  if (id < c.a.max_rows) return id < M_rows;
  const int j = id - c.a.max_rows, G1 = c.a.gamma - 1;
  const int b = j / G1, k = j % G1;
  return req_ok(c, b) && k < window_of(c, b) - 1;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void stats_kernel(Ctx c) {
  __shared__ float smf[kThreads / kWave];
  __shared__ double smd[kThreads / kWave];
  const int seg = blockIdx.x, id = blockIdx.y;
  const int M_rows = c.a.cu[c.a.B];
  if (!id_active(c, id, M_rows)) return;
  float x[kPer];
  load_seg<T>(row_ptr<T>(c, id), c.a.V, seg, x);
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i) m = fmaxf(m, x[i]);
  m = block_max(m, smf);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (x[i] != -INFINITY) s += double(expf(x[i] - m));
  s = block_sum_f64(s, smd);
  if (threadIdx.x == 0) {
    c.st_m[size_t(id) * c.L.nseg + seg] = m;
    c.st_s[size_t(id) * c.L.nseg + seg] = s;
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void tv_kernel(Ctx c) {
  __shared__ double smd[kThreads / kWave];
  __shared__ float sM[2];
  __shared__ double sInv[2];
  const int seg = blockIdx.x, j = blockIdx.y;
  const int G1 = c.a.gamma - 1;
  const int b = j / G1, kk = j % G1;
  if (!req_ok(c, b) || kk >= window_of(c, b) - 1) return;
  const int id_t = c.a.cu[b] + kk;
  const int id_d = c.a.max_rows + j;
  if (threadIdx.x < 2) {
    float M;
    double S;
    row_norm(c, threadIdx.x == 0 ? id_t : id_d, M, S);
    sM[threadIdx.x] = M;
    sInv[threadIdx.x] = 1.0 / S;
  }
  __syncthreads();
  float xt[kPer], xd[kPer];
  load_seg<T>(row_ptr<T>(c, id_t), c.a.V, seg, xt);
  load_seg<T>(row_ptr<T>(c, id_d), c.a.V, seg, xd);
  const float Mt = sM[0], Md = sM[1];
  const double it = sInv[0], id = sInv[1];
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (xt[i] == -INFINITY && xd[i] == -INFINITY) continue;
    const double pt = double(expf(xt[i] - Mt)) * it;
    const double pd = double(expf(xd[i] - Md)) * id;
    acc += pt > pd ? pt - pd : 0.0;
  }
  acc = block_sum_f64(acc, smd);
  if (threadIdx.x == 0) c.tv[size_t(j) * c.L.nseg + seg] = acc;
}

// One wave per request.  commit == false: labels only.
template <typename T>
__global__ __launch_bounds__(kThreads) void decide_kernel(Ctx c, int with_labels, int commit) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int b = blockIdx.x * (kThreads / kWave) + wave;
  if (b >= c.a.B) return;
  const int G1 = c.a.gamma - 1;
  if (!req_ok(c, b)) {
    if (lane == 0) {
      flag(c.a.status, RVA_DEV_BAD_WINDOW);
      if (commit) c.dec[size_t(b) * 4 + 1] = -1;  // nothing to draw or commit
    }
    return;
  }
  const int w = window_of(c, b);
  const float qnan = __int_as_float(0x7fc00000);
  bool reject = false;
  for (int kk = lane; kk < G1; kk += kWave) {
    const size_t o = size_t(b) * G1 + kk;
    if (kk >= w - 1) {
      if (c.a.labels) c.a.labels[o] = qnan;
      if (commit && c.a.pt_at) c.a.pt_at[o] = qnan;
      if (commit && c.a.pd_at) c.a.pd_at[o] = qnan;
      continue;
    }
    if (with_labels && c.a.labels) {
      double tv = 0.0;
      for (int s = 0; s < c.L.nseg; ++s) tv += c.tv[o * c.L.nseg + s];
      c.a.labels[o] = float(1.0 - tv);
    }
    if (!commit) continue;
    const int id_t = c.a.cu[b] + kk, id_d = c.a.max_rows + int(o);
    float Mt, Md;
    double St, Sd;
    row_norm(c, id_t, Mt, St);
    row_norm(c, id_d, Md, Sd);
    int x = c.a.tokens[o];
    if (x < 0 || x >= c.a.V) {
      flag(c.a.status, RVA_DEV_BAD_TOKEN);
      x = x < 0 ? 0 : c.a.V - 1;
    }
    const double lt = Elem<T>::load(row_ptr<T>(c, id_t), x);
    const double ld = Elem<T>::load(row_ptr<T>(c, id_d), x);
    const double pt = exp(lt - double(Mt)) / St;
    const double pd = exp(ld - double(Md)) / Sd;
    if (c.a.pt_at) c.a.pt_at[o] = float(pt);
    if (c.a.pd_at) c.a.pd_at[o] = float(pd);
    const double r = pd == 0.0 ? INFINITY : pt / pd;
    const double u = double(c.a.u_acc[o]);
    if (!(u < (r < 1.0 ? r : 1.0))) reject = true;
  }
  if (!commit) return;
  // first rejected draft (lanes cover kk = lane; G1 <= 63 so one pass suffices)
  const unsigned long long rej = __ballot(reject);
  const int n = rej ? __ffsll(rej) - 1 : w - 1;
  if (lane == 0) {
    int* d = c.dec + size_t(b) * 4;
    d[0] = n;
    d[1] = c.a.cu[b] + n;                                   // target row of the draw
    d[2] = n < w - 1 ? c.a.max_rows + b * G1 + n : -1;      // draft row (residual) or -1 (bonus)
  }
}

// float64 normaliser pieces of the draw rows, per segment.
template <typename T>
__global__ __launch_bounds__(kThreads) void draw_sum_kernel(Ctx c) {
  __shared__ double smd[kThreads / kWave];
  __shared__ float sM[2];
  const int seg = blockIdx.x, b = blockIdx.y;
  const int* d = c.dec + size_t(b) * 4;
  const int id_t = d[1], id_d = d[2];
  if (id_t < 0) return;
  if (threadIdx.x < 2) {
    const int id = threadIdx.x == 0 ? id_t : id_d;
    float m = -INFINITY;
    if (id >= 0)
      for (int s = 0; s < c.L.nseg; ++s) m = fmaxf(m, c.st_m[size_t(id) * c.L.nseg + s]);
    sM[threadIdx.x] = m;
  }
  __syncthreads();
  float x[kPer];
  load_seg<T>(row_ptr<T>(c, id_t), c.a.V, seg, x);
  double st = 0.0;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (x[i] != -INFINITY) st += exp(double(x[i]) - double(sM[0]));
  st = block_sum_f64(st, smd);
  double sd = 0.0;
  if (id_d >= 0) {
    load_seg<T>(row_ptr<T>(c, id_d), c.a.V, seg, x);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (x[i] != -INFINITY) sd += exp(double(x[i]) - double(sM[1]));
    sd = block_sum_f64(sd, smd);
  }
  if (threadIdx.x == 0) {
    c.r1[(size_t(b) * c.L.nseg + seg) * 2] = st;
    c.r1[(size_t(b) * c.L.nseg + seg) * 2 + 1] = sd;
  }
}

struct DrawRow {
  float Mt, Md;
  double St, Sd;
  int id_t, id_d;
};

__device__ __forceinline__ DrawRow draw_row(const Ctx& c, int b) {
  DrawRow r;
  const int* d = c.dec + size_t(b) * 4;
  r.id_t = d[1];
  r.id_d = d[2];
  r.Mt = -INFINITY;
  r.Md = -INFINITY;
  r.St = 0.0;
  r.Sd = 0.0;
  for (int s = 0; s < c.L.nseg; ++s) {  // same order everywhere: identical values
    r.Mt = fmaxf(r.Mt, c.st_m[size_t(r.id_t) * c.L.nseg + s]);
    r.St += c.r1[(size_t(b) * c.L.nseg + s) * 2];
    if (r.id_d >= 0) {
      r.Md = fmaxf(r.Md, c.st_m[size_t(r.id_d) * c.L.nseg + s]);
      r.Sd += c.r1[(size_t(b) * c.L.nseg + s) * 2 + 1];
    }
  }
  return r;
}

// Draw weight of one vocabulary entry: residual max(0, p_t - p_d), or the unnormalised
// target weight for the bonus draw (and for the all-zero-residual fallback).
__device__ __forceinline__ double draw_weight(const DrawRow& r, bool residual, float xt, float xd) {
  if (xt == -INFINITY) return 0.0;
  const double et = exp(double(xt) - double(r.Mt));
  if (!residual) return et;
  const double q = et / r.St - exp(double(xd) - double(r.Md)) / r.Sd;
  return q > 0.0 ? q : 0.0;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void draw_q_kernel(Ctx c) {
  __shared__ double smd[kThreads / kWave];
  __shared__ DrawRow sr;
  const int seg = blockIdx.x, b = blockIdx.y;
  if (c.dec[size_t(b) * 4 + 1] < 0) return;
  if (threadIdx.x == 0) sr = draw_row(c, b);
  __syncthreads();
  const DrawRow r = sr;
  if (r.id_d < 0) {  // bonus: the weights are exp(x - M); their segment mass is already known
    if (threadIdx.x == 0) c.r2[size_t(b) * c.L.nseg + seg] = c.r1[(size_t(b) * c.L.nseg + seg) * 2];
    return;
  }
  float xt[kPer], xd[kPer];
  load_seg<T>(row_ptr<T>(c, r.id_t), c.a.V, seg, xt);
  load_seg<T>(row_ptr<T>(c, r.id_d), c.a.V, seg, xd);
  double q = 0.0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) q += draw_weight(r, true, xt[i], xd[i]);
  q = block_sum_f64(q, smd);
  if (threadIdx.x == 0) c.r2[size_t(b) * c.L.nseg + seg] = q;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void draw_pick_kernel(Ctx c) {
  __shared__ DrawRow sr;
  __shared__ double s_t, s_base;
  __shared__ int s_seg, s_residual;
  __shared__ double run_tot[kThreads];
  __shared__ int s_y;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int nseg = c.L.nseg;
  if (c.dec[size_t(b) * 4 + 1] < 0) return;
  if (tid == 0) {
    sr = draw_row(c, b);
    bool residual = sr.id_d >= 0;
    double Q = 0.0;
    for (int s = 0; s < nseg; ++s) Q += residual ? c.r2[size_t(b) * nseg + s] : c.r1[(size_t(b) * nseg + s) * 2];
    if (residual && !(Q > 0.0)) {  // residual identically zero: draw from p_t instead
      residual = false;
      Q = 0.0;
      for (int s = 0; s < nseg; ++s) Q += c.r1[(size_t(b) * nseg + s) * 2];
    }
    const double t = double(c.a.u_res[b]) * Q;
    double cum = 0.0;
    int seg = -1, last_pos = 0;
    double base = 0.0, base_last = 0.0;
    for (int s = 0; s < nseg; ++s) {
      const double qs = residual ? c.r2[size_t(b) * nseg + s] : c.r1[(size_t(b) * nseg + s) * 2];
      if (qs > 0.0) {
        last_pos = s;
        base_last = cum;
      }
      if (seg < 0 && cum + qs > t) {
        seg = s;
        base = cum;
      }
      cum += qs;
    }
    if (seg < 0) {  // u*Q reached the end by rounding: take the last segment with mass
      seg = last_pos;
      base = base_last;
    }
    s_t = t;
    s_base = base;
    s_seg = seg;
    s_residual = residual;
    s_y = 0x7fffffff;
  }
  __syncthreads();
  const DrawRow r = sr;
  const int seg = s_seg;
  const bool residual = s_residual;
  // each thread owns kPer consecutive indices of the segment (index order for the scan)
  const int v0 = seg * kSeg + tid * kPer;
  double wgt[kPer];
  const T* rowt = row_ptr<T>(c, r.id_t);
  const T* rowd = residual ? row_ptr<T>(c, r.id_d) : nullptr;
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int v = v0 + i;
    double q = 0.0;
    if (v < c.a.V) q = draw_weight(r, residual, Elem<T>::load(rowt, v), residual ? Elem<T>::load(rowd, v) : 0.f);
    wgt[i] = q;
    tot += q;
  }
  run_tot[tid] = tot;
  __syncthreads();
  if (tid == 0) {  // sequential scan of the 256 run totals (index order)
    double acc = s_base;
    for (int i = 0; i < kThreads; ++i) {
      const double t = run_tot[i];
      run_tot[i] = acc;
      acc += t;
    }
  }
  __syncthreads();
  double cum = run_tot[tid];
  const double t = s_t;
  int found = 0x7fffffff;
  int last_pos = -1;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (wgt[i] > 0.0) last_pos = v0 + i;
    cum += wgt[i];
    if (found == 0x7fffffff && cum > t && wgt[i] > 0.0) found = v0 + i;
  }
  atomicMin(&s_y, found);
  __syncthreads();
  if (s_y == 0x7fffffff) {  // rounding left u*S past this segment's end: last positive entry
    __shared__ int s_last;
    if (tid == 0) s_last = -1;
    __syncthreads();
    atomicMax(&s_last, last_pos);
    __syncthreads();
    if (tid == 0) s_y = s_last < 0 ? seg * kSeg : s_last;
    __syncthreads();
  }
  if (tid == 0) {
    const int y = s_y;
    const int n = c.dec[size_t(b) * 4];
    const int G1 = c.a.gamma - 1;
    int32_t* com = c.a.committed + size_t(b) * c.a.gamma;
    for (int i = 0; i < c.a.gamma; ++i) com[i] = i < n ? c.a.tokens[size_t(b) * G1 + i] : (i == n ? y : -1);
    c.a.accept_len[b] = n;
    c.a.context_lens[b] += n + 1;
  }
}

template <typename T>
hipError_t launch_typed(const Ctx& c, bool commit, hipStream_t stream) {
  const AcceptArgs& a = c.a;
  const int nseg = c.L.nseg, G1 = a.gamma - 1;
  hipLaunchKernelGGL(stats_kernel<T>, dim3(nseg, c.L.n_ids), dim3(kThreads), 0, stream, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool with_labels = a.labels != nullptr;
  if (with_labels) {
    hipLaunchKernelGGL(tv_kernel<T>, dim3(nseg, a.B * G1), dim3(kThreads), 0, stream, c);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int wpb = kThreads / kWave;
  hipLaunchKernelGGL(decide_kernel<T>, dim3((a.B + wpb - 1) / wpb), dim3(kThreads), 0, stream, c,
                     int(with_labels), int(commit));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!commit) return hipSuccess;
  hipLaunchKernelGGL(draw_sum_kernel<T>, dim3(nseg, a.B), dim3(kThreads), 0, stream, c);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(draw_q_kernel<T>, dim3(nseg, a.B), dim3(kThreads), 0, stream, c);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(draw_pick_kernel<T>, dim3(a.B), dim3(kThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace

size_t accept_workspace_bytes(int B, int gamma, int V, int max_rows) {
  return ws_layout(B, gamma, V, max_rows).total;
}

hipError_t launch_accept(const AcceptArgs& a, int logit_dtype, bool commit, hipStream_t stream) {
  Ctx c;
  c.a = a;
  c.L = ws_layout(a.B, a.gamma, a.V, a.max_rows);
  char* base = static_cast<char*>(a.ws);
  c.st_m = reinterpret_cast<float*>(base + c.L.off_m);
  c.st_s = reinterpret_cast<double*>(base + c.L.off_s);
  c.tv = reinterpret_cast<double*>(base + c.L.off_tv);
  c.dec = reinterpret_cast<int*>(base + c.L.off_dec);
  c.r1 = reinterpret_cast<double*>(base + c.L.off_r1);
  c.r2 = reinterpret_cast<double*>(base + c.L.off_r2);
  return logit_dtype == RVA_BF16 ? launch_typed<uint16_t>(c, commit, stream)
                                 : launch_typed<float>(c, commit, stream);
}

}  // namespace rva
