// Stage 1: confidence head + temperature scaling, prefix survival, window argmax.
//
// Sources: "DSpark：投机解码与生产级 Serving 学习笔记" (sorenprojections.com) sections
// 07 (confidence head, survival product, Sequential Temperature Scaling) and 08 (the
// throughput-maximising prefix scheduler); the devpress.csdn.net DSpark-in-SGLang article,
// section 4 (additive step cost T(bs, K) = bias + alpha(bs) + theta(bs + K)).
//
// Two kernels:
//   conf_head_kernel  one wave per (request, draft position): float64 dot product of the
//                     hidden state with the head weights, + bias, / T_k, logistic in
//                     float64, rounded to float32.  Skipped when the caller supplies c.
//   schedule_kernel   ONE workgroup (256 to 1024 threads, by batch size) for the whole batch:
//                     (1) one lane per request forms the survival product left to right
//                         in float32 (bit-identical to a sequential definition);
//                     (2) 64-bit keys (inverted survival bits, candidate index) order
//                         "survival desc, request asc, position asc" in one comparison;
//                         each request's keys are already in order, so the rank order is
//                         a merge of B sorted runs (log2 B rounds, a binary search per key);
//                     (3) a workgroup scan in float64 gives S_K for every K;
//                     (4) a workgroup argmax of (B + S_K) / T(B, K), smallest K on ties;
//                     (5) LDS counters turn the first K* ranks into per-request windows.
#include "rva_common.h"

namespace rva {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kMaxCand = 4096;

template <typename T>
__global__ __launch_bounds__(256) void conf_head_kernel(const T* __restrict__ hidden, int rows,
                                                        int G, int H,
                                                        const float* __restrict__ w, float b0,
                                                        const float* __restrict__ sts_T,
                                                        float* __restrict__ conf_out,
                                                        int32_t* status) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const T* h = hidden + size_t(row) * H;
  double acc = 0.0;
  for (int i = lane; i < H; i += kWave) acc += double(Elem<T>::load(h, i)) * double(w[i]);
  acc = wave_sum_f64(acc);
  if (lane == 0) {
    double z = acc + double(b0);
    if (sts_T) z = z / double(sts_T[row % G]);
    const float c = float(1.0 / (1.0 + exp(-z)));
    if (!(c >= 0.f && c <= 1.f)) flag(status, RVA_DEV_BAD_CONF);
    conf_out[row] = c;
  }
}

template <int NT>
__device__ __forceinline__ double block_exclusive_scan_f64(double v, double* lds_waves,
                                                           double* total) {
  // Inclusive scan inside the wave, then across the NT / 64 wave totals.
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  double x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) lds_waves[wave] = x;
  __syncthreads();
  if (wave == 0) {
    double t = lane < NT / kWave ? lds_waves[lane] : 0.0;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(t, o);
      if (lane >= o) t += y;
    }
    if (lane < NT / kWave) lds_waves[lane] = t;  // inclusive wave prefix
  }
  __syncthreads();
  const double wave_off = wave > 0 ? lds_waves[wave - 1] : 0.0;
  *total = lds_waves[NT / kWave - 1];
  return wave_off + x - v;
}

// Rank order of the candidates by merging sorted runs.  Each request's keys are already in
// ascending order along its draft positions (survival never grows along a prefix, and the
// candidate index breaks ties), so the B runs of G keys are merged pairwise, log2(B) rounds:
// a key finds its place in the partner run by binary search (keys are unique), and lands at
// pair start + its index in its own run + the partner keys below it.  One barrier a round.
// `buf` holds two arrays of kMaxCand keys; returns the one that ends up sorted.  With invalid
// confidences (a run not in order) the positions may collide; both arrays start with the keys,
// so every slot still holds some candidate's key.
template <int E, int NT>
__device__ __forceinline__ const uint64_t* merge_runs(const uint64_t (&x)[E], uint64_t* buf, int N, int G) {
  const int tid = threadIdx.x;
  uint64_t* cur = buf;
  uint64_t* nxt = buf + kMaxCand;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    if (i < N) cur[i] = nxt[i] = x[e];
  }
  __syncthreads();
  for (int len = G; len < N; len <<= 1) {
    if constexpr (E > 1) {
      // merge path: thread c writes kChunk consecutive outputs of one pair of runs, starting
      // where a binary search along its diagonal puts it, then merges sequentially; far
      // fewer scattered LDS probes than a search per key
      constexpr int kChunk = 4;
      const int per_pair = (2 * len + kChunk - 1) / kChunk;
      const int pairs = (N + 2 * len - 1) / (2 * len);
      for (int c = tid; c < pairs * per_pair; c += NT) {
        const int p = c / per_pair, a0 = p * 2 * len, b0 = a0 + len;
        const int lenA = min(len, N - a0), lenB = max(0, min(len, N - b0));
        const int d0 = (c % per_pair) * kChunk, d1 = min(d0 + kChunk, lenA + lenB);
        if (d0 >= d1) continue;
        int lo = max(0, d0 - lenB), hi = min(d0, lenA);
        while (lo < hi) {  // smallest i whose A[i] is not among the first d0 outputs
          const int mid = (lo + hi) >> 1;
          if (cur[a0 + mid] < cur[b0 + d0 - mid - 1]) lo = mid + 1; else hi = mid;
        }
        int i = lo, j = d0 - lo;
        for (int d = d0; d < d1; ++d) {
          const bool takeA = j >= lenB || (i < lenA && cur[a0 + i] < cur[b0 + j]);
          nxt[a0 + d] = takeA ? cur[a0 + i++] : cur[b0 + j++];
        }
      }
    } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = tid * E + e;
      if (i >= N) continue;
      const uint64_t k = cur[i];
      const int q = i / len, start = q * len;
      const int ps = (q ^ 1) * len, pe = min(ps + len, N);
      int pos = i;
      if (ps < N) {
        int lo = ps, hi = pe;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (cur[mid] < k) lo = mid + 1; else hi = mid;
        }
        pos = (q & ~1) * len + (i - start) + (lo - ps);
      }
      nxt[pos] = k;
    }
    }
    __syncthreads();
    uint64_t* t = cur;
    cur = nxt;
    nxt = t;
  }
  return cur;
}

// E keys per thread, NT threads (small batches take fewer waves: each merge round's
// searches and barrier then involve fewer of them).
template <int E, int NT>
__global__ __launch_bounds__(NT) void schedule_kernel(
    int B, int G, int mode, const float* __restrict__ conf, float* __restrict__ conf_out,
    float* __restrict__ surv_out, float bias, const float* __restrict__ alpha,
    const float* __restrict__ theta, int32_t* __restrict__ windows, int32_t* __restrict__ K_out,
    double* __restrict__ ratio_out, int32_t* status) {
  __shared__ uint64_t keybuf[2 * kMaxCand];
  __shared__ float sa[kMaxCand];
  __shared__ int cnt[kMaxCand];
  __shared__ double wave_tot[NT / kWave];
  __shared__ double red_ratio[NT / kWave];
  __shared__ int red_K[NT / kWave];

  const int tid = threadIdx.x;
  const int N = B * G;

  // the cost table entries this thread needs later (rank r = tid*E + e uses theta[B + r + 1])
  // are loaded now, so their round trip overlaps the survival products and the sort
  float th[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int r = tid * E + e;
    th[e] = r < N ? theta[B + r + 1] : 0.f;
  }
  const float alpha_B = alpha[B], theta_0 = theta[B];
  const float theta_N = theta[B + N];
  // (1) survival: the confidences are staged in LDS by one coalesced load, then one lane per
  // request forms the float32 products left to right
  for (int i = tid; i < N; i += NT) {
    const float c = conf[i];
    if (!(c >= 0.f && c <= 1.f)) flag(status, RVA_DEV_BAD_CONF);
    if (conf_out) conf_out[i] = c;
    sa[i] = c;
  }
  __syncthreads();
  for (int b = tid; b < B; b += NT) {
    float a = 1.f;
    for (int j = 0; j < G; ++j) {
      a = (j == 0) ? sa[b * G + j] : __fmul_rn(a, sa[b * G + j]);
      sa[b * G + j] = a;
    }
    cnt[b] = 0;
  }
  __syncthreads();
  // (2) sort keys (inverted survival bits, candidate index): ascending key order is
  // "survival desc, request asc, position asc"
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    x[e] = ~0ull;
    if (i < N) {
      const float a = sa[i];
      surv_out[i] = a;
      const uint32_t bits = (a == 0.f) ? 0u : __float_as_uint(a);
      x[e] = (uint64_t(~bits) << 32) | uint32_t(i);
    }
  }
  const uint64_t* keys = merge_runs<E, NT>(x, keybuf, N, G);

  // (3) S_K: each thread owns a contiguous run of ranks
  constexpr int per = E;
  const int r0 = tid * per;
  double run = 0.0;
  for (int i = 0; i < per; ++i) {
    const int r = r0 + i;
    if (r < N) run += double(__uint_as_float(~uint32_t(keys[r] >> 32)));
  }
  double total;
  double prefix = block_exclusive_scan_f64<NT>(run, wave_tot, &total);

  // (4) ratio (B + S_K) / T(B, K); K = r + 1 for rank r, K = 0 handled by thread 0
  const double ba = double(bias) + double(alpha_B);
  double best = -INFINITY;
  int bestK = 0x7fffffff;
  if (tid == 0) {
    const double T0 = ba + double(theta_0);
    if (!(T0 > 0.0)) flag(status, RVA_DEV_BAD_COST);
    best = T0 > 0.0 ? double(B) / T0 : -INFINITY;
    bestK = 0;
  }
  double S = prefix;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int r = r0 + i;
    if (r < N) {
      S += double(__uint_as_float(~uint32_t(keys[r] >> 32)));
      const double T = ba + double(th[i]);
      if (!(T > 0.0)) flag(status, RVA_DEV_BAD_COST);
      const double ratio = T > 0.0 ? (double(B) + S) / T : -INFINITY;
      if (ratio > best) {
        best = ratio;
        bestK = r + 1;
      }
    }
  }
  // workgroup argmax: larger ratio wins, smaller K on equal ratio
  const int lane = tid % kWave, wave = tid / kWave;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double ob = __shfl_xor(best, o);
    const int ok = __shfl_xor(bestK, o);
    if (ob > best || (ob == best && ok < bestK)) {
      best = ob;
      bestK = ok;
    }
  }
  if (lane == 0) {
    red_ratio[wave] = best;
    red_K[wave] = bestK;
  }
  __syncthreads();
  if (wave == 0) {
    best = lane < NT / kWave ? red_ratio[lane] : -INFINITY;
    bestK = lane < NT / kWave ? red_K[lane] : 0x7fffffff;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int ok = __shfl_xor(bestK, o);
      if (ob > best || (ob == best && ok < bestK)) {
        best = ob;
        bestK = ok;
      }
    }
    if (lane == 0) {
      red_ratio[0] = best;
      red_K[0] = bestK;
    }
  }
  __syncthreads();
  int Kstar = red_K[0];
  double ratio = red_ratio[0];
  if (mode == RVA_MODE_STATIC) {
    Kstar = N;
    const double T = ba + double(theta_N);
    ratio = T > 0.0 ? (double(B) + total) / T : -INFINITY;
  }

  // (5) windows from the first K* ranks
  for (int i = 0; i < per; ++i) {
    const int r = r0 + i;
    if (r < Kstar && r < N) atomicAdd(&cnt[min(int(uint32_t(keys[r]) / uint32_t(G)), B - 1)], 1);
  }
  __syncthreads();
  for (int b = tid; b < B; b += NT) windows[b] = 1 + cnt[b];
  if (tid == 0) {
    *K_out = Kstar;
    *ratio_out = ratio;
  }
}

}  // namespace

hipError_t launch_schedule(int B, int gamma, int mode, const void* hidden, int hidden_dtype,
                           int H, const float* head_w, float head_b, const float* conf_in,
                           const float* sts_T, float bias, const float* alpha,
                           const float* theta, float* conf_out, float* surv_out,
                           int32_t* windows, int32_t* K_out, double* ratio_out,
                           int32_t* status, hipStream_t stream) {
  const int G = gamma - 1;
  const int rows = B * G;
  const float* conf = conf_in;
  if (!conf_in) {
    const dim3 grid((rows + 3) / 4), block(256);
    if (hidden_dtype == RVA_BF16)
      hipLaunchKernelGGL(conf_head_kernel<uint16_t>, grid, block, 0, stream,
                         static_cast<const uint16_t*>(hidden), rows, G, H, head_w, head_b, sts_T,
                         conf_out, status);
    else
      hipLaunchKernelGGL(conf_head_kernel<float>, grid, block, 0, stream,
                         static_cast<const float*>(hidden), rows, G, H, head_w, head_b, sts_T,
                         conf_out, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    conf = conf_out;
  }
  // conf_in is echoed into conf_out by the schedule kernel itself
  float* echo = conf_in ? conf_out : nullptr;
  int Npad = 2;
  while (Npad < rows) Npad <<= 1;
  if (Npad <= 256)
    hipLaunchKernelGGL((schedule_kernel<1, 256>), dim3(1), dim3(256), 0, stream, B, G, mode,
                       conf, echo, surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
  else if (Npad <= 512)
    hipLaunchKernelGGL((schedule_kernel<1, 512>), dim3(1), dim3(512), 0, stream, B, G, mode,
                       conf, echo, surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
  else if (Npad <= kSchedThreads)
    hipLaunchKernelGGL((schedule_kernel<1, kSchedThreads>), dim3(1), dim3(kSchedThreads), 0, stream, B, G,
                       mode, conf, echo, surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
  else if (Npad <= 2 * kSchedThreads)
    hipLaunchKernelGGL((schedule_kernel<2, kSchedThreads>), dim3(1), dim3(kSchedThreads), 0, stream, B, G,
                       mode, conf, echo, surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
  else
    hipLaunchKernelGGL((schedule_kernel<4, kSchedThreads>), dim3(1), dim3(kSchedThreads), 0, stream, B, G,
                       mode, conf, echo, surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
  return hipGetLastError();
}

}  // namespace rva
