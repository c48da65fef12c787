// Calibration of the confidence head: Sequential Temperature Scaling (STS) fit and the
// expected calibration error (ECE) of the predicted prefix survival, from acceptance traces.
//
// Sources: "DSpark：投机解码与生产级 Serving 学习笔记" (sorenprojections.com), section
// "07 · Confidence Head" (a temperature per draft position calibrates the prefix survival
// to the measured acceptance rate); the devpress.csdn.net article on DSpark in SGLang,
// section "5. 可观测性：理解修剪下的真实性能" (per-request confidence and ECE for analysis;
// only full-block runs observe positions past the window).
//
// Trace sample i: head logits z[i, 0 .. G1-1], accepted drafts n_i, observed positions o_i.
// Position k (0-based) is observed iff k < o_i and its outcome is E = [n_i > k].  With
// temperatures T the predicted survival is a[i, k] = exp(sum_{j <= k} log sigmoid(z[i, j] /
// T_j)) in float64.
//
// STS fit, position by position (earlier temperatures fixed): T_k minimises the Bernoulli
// negative log-likelihood of the observed outcomes of position k over [T_lo, T_hi].  The
// minimum is located by iterated grid refinement in u = ln T: 64 log-spaced temperatures,
// the best one's two neighbouring cells become the next round's bracket, six rounds (final
// spacing about 1e-8 in u).  Every round is two launches: a data-parallel pass over (sample
// chunk, pair of temperatures) whose workgroups write partial sums, and a one-wave
// selection that sums the partials in chunk order, so the result is reproducible run to
// run and the bracket stays on the device (no host round trip).
//
// ECE: the observed (a, E) pairs are binned by a into n_bins equal bins of [0, 1]
// (bin = min(floor(a n_bins), n_bins - 1)); per workgroup the bins live in LDS, partial bins
// are reduced in a fixed order by one final workgroup.
#include <algorithm>
#include <cmath>

#include "rva_common.h"

namespace rva {
namespace {

constexpr int kCalThreads = 256;
constexpr int kGrid = 64;     // temperatures per refinement round
constexpr int kRounds = 6;
constexpr int kGroup = 2;     // temperatures per workgroup (grid.y = kGrid / kGroup)
constexpr int kMaxChunks = 512;
constexpr int kMaxEceChunks = 256;

struct StsState {
  double u_lo, du, T, pad;  // bracket of the current round; the last fitted temperature
};

__device__ __forceinline__ double log_sigmoid(double x) { return fmin(x, 0.0) - log1p(exp(-fabs(x))); }

// log(1 - exp(y)) for y <= 0
__device__ __forceinline__ double log1mexp(double y) {
  return y > -0.69314718055994530942 ? log(-expm1(y)) : log1p(-exp(y));
}

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < kCalThreads / kWave; ++w) s += red[w];
  return s;
}

// Workspace: two running log-survival buffers (position k's prefix lives in L[k & 1]), the
// per-workgroup partial sums of one round, and the round state.
struct StsLayout {
  size_t off_L0, off_L1, off_part, off_state, total;
  int chunks;
};

StsLayout sts_layout(int N) {
  StsLayout l;
  l.chunks = std::min(kMaxChunks, (N + kCalThreads - 1) / kCalThreads);
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  l.off_L0 = 0;
  l.off_L1 = up(size_t(N) * sizeof(double));
  l.off_part = l.off_L1 + up(size_t(N) * sizeof(double));
  l.off_state = l.off_part + up(size_t(kMaxChunks) * (kGrid + 1) * sizeof(double));
  l.total = l.off_state + 256;
  return l;
}

__global__ __launch_bounds__(kCalThreads) void sts_init_kernel(StsArgs a, StsLayout l) {
  double* L = reinterpret_cast<double*>(static_cast<char*>(a.ws) + l.off_L0);
  for (int i = blockIdx.x * kCalThreads + threadIdx.x; i < a.N; i += gridDim.x * kCalThreads) L[i] = 0.0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    StsState* st = reinterpret_cast<StsState*>(static_cast<char*>(a.ws) + l.off_state);
    const double lo = log(double(a.T_lo)), hi = log(double(a.T_hi));
    st->u_lo = lo;
    st->du = (hi - lo) / (kGrid - 1);
    st->T = 1.0;
  }
}

// One refinement round of position k.  Workgroup (x, y) sums the negative log-likelihood of
// its chunk x of samples at the round's temperatures 2y, 2y+1 (and, for y = 0, counts the
// observed samples).  In round 0 of a position k > 0 each thread first extends its samples'
// log survival by position k-1 at the temperature just fitted (workgroups y = 0 store it for
// the later rounds, in the other buffer, so no workgroup reads a value another one is
// rewriting).  sts_select_kernel then picks the round's best temperature.
__global__ __launch_bounds__(kCalThreads) void sts_round_kernel(StsArgs a, StsLayout l, int k, int round) {
  __shared__ double s_T[kGroup];
  __shared__ double red[kCalThreads / kWave];
  char* ws = static_cast<char*>(a.ws);
  const StsState st = *reinterpret_cast<const StsState*>(ws + l.off_state);
  double* Lcur = reinterpret_cast<double*>(ws + ((k & 1) ? l.off_L1 : l.off_L0));
  const double* Lprev = reinterpret_cast<const double*>(ws + ((k & 1) ? l.off_L0 : l.off_L1));
  double* part = reinterpret_cast<double*>(ws + l.off_part);
  const int tid = threadIdx.x, g0 = blockIdx.y * kGroup;
  if (tid < kGroup) s_T[tid] = exp(st.u_lo + (g0 + tid) * st.du);
  __syncthreads();
  const bool extend = round == 0 && k > 0;
  double acc[kGroup];
#pragma unroll
  for (int p = 0; p < kGroup; ++p) acc[p] = 0.0;
  double cnt = 0.0;
  for (int i = blockIdx.x * kCalThreads + tid; i < a.N; i += gridDim.x * kCalThreads) {
    const int o = a.observed_len ? a.observed_len[i] : a.G1;
    if (k >= o) continue;  // unobserved here, and so at every later position
    double Lp;
    if (extend) {
      Lp = Lprev[i] + log_sigmoid(double(a.z[size_t(i) * a.G1 + k - 1]) / st.T);
      if (blockIdx.y == 0) Lcur[i] = Lp;
    } else {
      Lp = k == 0 ? 0.0 : Lcur[i];
    }
    const double z = a.z[size_t(i) * a.G1 + k];
    const bool E = a.accept_len[i] > k;
    cnt += 1.0;
#pragma unroll
    for (int p = 0; p < kGroup; ++p) {
      const double la = Lp + log_sigmoid(z / s_T[p]);
      acc[p] += E ? -la : -log1mexp(la);
    }
  }
  double* my = part + size_t(blockIdx.x) * (kGrid + 1);
#pragma unroll
  for (int p = 0; p < kGroup; ++p) {
    const double sp = block_sum_f64(acc[p], red);
    if (tid == 0) my[g0 + p] = sp;
  }
  const double c = block_sum_f64(cnt, red);
  if (tid == 0 && blockIdx.y == 0) my[kGrid] = c;
}

// The selection after a round (one wave, thread p = temperature p of the round): sums the
// partials in chunk order (the loads of 16 chunks at a time are independent, so they are in
// flight together), picks the best temperature (first on a tie), and narrows the bracket
// or, after the last round, publishes T_k.  A launch of its own: the kernel boundary makes
// every partial visible, where a device-scope fence in each round workgroup and a
// last-to-finish counter cost more than the round's arithmetic.
__global__ __launch_bounds__(kGrid) void sts_select_kernel(StsArgs a, StsLayout l, int k, int last, int chunks) {
  const char* ws = static_cast<const char*>(a.ws);
  StsState* stp = reinterpret_cast<StsState*>(static_cast<char*>(a.ws) + l.off_state);
  const StsState st = *stp;
  const double* part = reinterpret_cast<const double*>(ws + l.off_part);
  const int p = threadIdx.x;
  double f = 0.0, n_obs = 0.0;
#pragma unroll 16
  for (int ch = 0; ch < chunks; ++ch) {
    f += part[size_t(ch) * (kGrid + 1) + p];
    n_obs += part[size_t(ch) * (kGrid + 1) + kGrid];
  }
  double bf = f;
  int bp = p;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double of = __shfl_xor(bf, o);
    const int op = __shfl_xor(bp, o);
    if (of < bf || (of == bf && op < bp)) {
      bf = of;
      bp = op;
    }
  }
  if (p != 0) return;
  StsState nx = st;
  const double lo0 = log(double(a.T_lo)), hi0 = log(double(a.T_hi));
  if (n_obs == 0.0 || last) {
    const double T = n_obs == 0.0 ? 1.0 : exp(st.u_lo + bp * st.du);
    a.T_out[k] = float(T);
    if (a.nll_out) a.nll_out[k] = n_obs == 0.0 ? 0.0 : bf;
    nx.T = T;
    nx.u_lo = lo0;  // the next position starts from the whole bracket
    nx.du = (hi0 - lo0) / (kGrid - 1);
  } else {
    const int lo = bp > 0 ? bp - 1 : 0, hi = bp < kGrid - 1 ? bp + 1 : kGrid - 1;
    nx.u_lo = st.u_lo + lo * st.du;
    nx.du = (hi - lo) * st.du / (kGrid - 1);
  }
  *stp = nx;
}

// ---------------------------------------------------------------- ECE
struct EceLayout {
  size_t off_cnt, off_se, off_sa, total;
  int chunks, bins;  // bins = G1 * n_bins entries per chunk
};

EceLayout ece_layout(int N, int G1, int n_bins) {
  EceLayout l;
  l.chunks = std::min(kMaxEceChunks, (N + kCalThreads - 1) / kCalThreads);
  l.bins = G1 * n_bins;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t n = size_t(l.chunks) * l.bins;
  l.off_cnt = 0;
  l.off_se = up(n * sizeof(int));
  l.off_sa = l.off_se + up(n * sizeof(int));
  l.total = l.off_sa + up(n * sizeof(double));
  return l;
}

__global__ __launch_bounds__(kCalThreads) void ece_bins_kernel(EceArgs a, EceLayout l) {
  extern __shared__ double lds[];
  double* sa = lds;
  int* cnt = reinterpret_cast<int*>(sa + l.bins);
  int* se = cnt + l.bins;
  const int tid = threadIdx.x, G1 = a.G1, nb = a.n_bins;
  for (int e = tid; e < l.bins; e += kCalThreads) {
    sa[e] = 0.0;
    cnt[e] = 0;
    se[e] = 0;
  }
  __syncthreads();
  for (int i = blockIdx.x * kCalThreads + tid; i < a.N; i += gridDim.x * kCalThreads) {
    const int o = a.observed_len ? min(a.observed_len[i], G1) : G1;
    const int n = a.accept_len[i];
    double Lsum = 0.0;
    for (int k = 0; k < o; ++k) {
      const double T = a.T ? double(a.T[k]) : 1.0;
      Lsum += log_sigmoid(double(a.z[size_t(i) * G1 + k]) / T);
      const double av = exp(Lsum);
      // av is in [0, 1]; a NaN logit gives a NaN av, which lands in bin 0 (and a NaN ECE)
      const int b = av >= 0.0 ? min(int(av * nb), nb - 1) : 0;
      const int e = k * nb + b;
      atomicAdd(&cnt[e], 1);
      if (n > k) atomicAdd(&se[e], 1);
      atomicAdd(&sa[e], av);
    }
  }
  __syncthreads();
  const size_t base = size_t(blockIdx.x) * l.bins;
  char* ws = static_cast<char*>(a.ws);
  for (int e = tid; e < l.bins; e += kCalThreads) {
    reinterpret_cast<int*>(ws + l.off_cnt)[base + e] = cnt[e];
    reinterpret_cast<int*>(ws + l.off_se)[base + e] = se[e];
    reinterpret_cast<double*>(ws + l.off_sa)[base + e] = sa[e];
  }
}

__global__ __launch_bounds__(kCalThreads) void ece_final_kernel(EceArgs a, EceLayout l) {
  extern __shared__ double lds[];
  double* sa = lds;
  int* cnt = reinterpret_cast<int*>(sa + l.bins);
  int* se = cnt + l.bins;
  __shared__ double p_sa[64];
  __shared__ int p_cnt[64], p_se[64];
  const int tid = threadIdx.x, G1 = a.G1, nb = a.n_bins;
  const char* ws = static_cast<const char*>(a.ws);
  for (int e = tid; e < l.bins; e += kCalThreads) {
    int c = 0, s = 0;
    double x = 0.0;
    for (int ch = 0; ch < l.chunks; ++ch) {
      const size_t q = size_t(ch) * l.bins + e;
      c += reinterpret_cast<const int*>(ws + l.off_cnt)[q];
      s += reinterpret_cast<const int*>(ws + l.off_se)[q];
      x += reinterpret_cast<const double*>(ws + l.off_sa)[q];
    }
    cnt[e] = c;
    se[e] = s;
    sa[e] = x;
    if (a.bin_counts) a.bin_counts[e] = c;
  }
  __syncthreads();
  auto ece_of = [](const int* c, const int* s, const double* x, int n, int step) {
    long long tot = 0;
    for (int b = 0; b < n; ++b) tot += c[b * step];
    if (tot == 0) return 0.0;
    double r = 0.0;
    for (int b = 0; b < n; ++b) {
      const int cb = c[b * step];
      if (cb == 0) continue;
      r += double(cb) / double(tot) * fabs(x[b * step] / cb - double(s[b * step]) / cb);
    }
    return r;
  };
  if (tid < G1) a.ece_out[1 + tid] = ece_of(cnt + tid * nb, se + tid * nb, sa + tid * nb, nb, 1);
  if (tid < nb) {
    int c = 0, s = 0;
    double x = 0.0;
    for (int k = 0; k < G1; ++k) {
      c += cnt[k * nb + tid];
      s += se[k * nb + tid];
      x += sa[k * nb + tid];
    }
    p_cnt[tid] = c;
    p_se[tid] = s;
    p_sa[tid] = x;
  }
  __syncthreads();
  if (tid == 0) a.ece_out[0] = ece_of(p_cnt, p_se, p_sa, nb, 1);
}

}  // namespace

size_t sts_workspace_bytes(int N) { return sts_layout(N).total; }

hipError_t launch_sts_fit(const StsArgs& a, hipStream_t stream) {
  const StsLayout l = sts_layout(a.N);
  hipLaunchKernelGGL(sts_init_kernel, dim3(l.chunks), dim3(kCalThreads), 0, stream, a, l);
  for (int k = 0; k < a.G1; ++k)
    for (int r = 0; r < kRounds; ++r) {
      hipLaunchKernelGGL(sts_round_kernel, dim3(l.chunks, kGrid / kGroup), dim3(kCalThreads), 0, stream, a,
                         l, k, r);
      hipLaunchKernelGGL(sts_select_kernel, dim3(1), dim3(kGrid), 0, stream, a, l, k, int(r == kRounds - 1),
                         l.chunks);
    }
  return hipGetLastError();
}

size_t ece_workspace_bytes(int N, int G1, int n_bins) { return ece_layout(N, G1, n_bins).total; }

hipError_t launch_ece(const EceArgs& a, hipStream_t stream) {
  const EceLayout l = ece_layout(a.N, a.G1, a.n_bins);
  const size_t lds = size_t(l.bins) * (sizeof(double) + 2 * sizeof(int));
  hipLaunchKernelGGL(ece_bins_kernel, dim3(l.chunks), dim3(kCalThreads), lds, stream, a, l);
  hipLaunchKernelGGL(ece_final_kernel, dim3(1), dim3(kCalThreads), lds, stream, a, l);
  return hipGetLastError();
}

}  // namespace rva
