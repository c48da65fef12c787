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
//   schedule_kernel   ONE workgroup of 1024 threads for the whole batch:
//                     (1) one lane per request forms the survival product left to right
//                         in float32 (bit-identical to a sequential definition);
//                     (2) a bitonic sort in LDS of 64-bit keys (inverted survival bits,
//                         candidate index) gives the rank order "survival desc, request
//                         asc, position asc" in one comparison;
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

__device__ __forceinline__ double block_exclusive_scan_f64(double v, double* lds_waves,
                                                           double* total) {
  // Inclusive scan inside the wave, then across the 16 wave totals.
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
    double t = lane < kSchedThreads / kWave ? lds_waves[lane] : 0.0;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(t, o);
      if (lane >= o) t += y;
    }
    if (lane < kSchedThreads / kWave) lds_waves[lane] = t;  // inclusive wave prefix
  }
  __syncthreads();
  const double wave_off = wave > 0 ? lds_waves[wave - 1] : 0.0;
  *total = lds_waves[kSchedThreads / kWave - 1];
  return wave_off + x - v;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(
    int B, int G, int mode, const float* __restrict__ conf, float* __restrict__ surv_out,
    float bias, const float* __restrict__ alpha, const float* __restrict__ theta,
    int32_t* __restrict__ windows, int32_t* __restrict__ K_out, double* __restrict__ ratio_out,
    int32_t* status) {
  __shared__ uint64_t keys[kMaxCand];
  __shared__ int cnt[kMaxCand];
  __shared__ double wave_tot[kSchedThreads / kWave];
  __shared__ double red_ratio[kSchedThreads / kWave];
  __shared__ int red_K[kSchedThreads / kWave];
  __shared__ int bad;

  const int tid = threadIdx.x;
  const int N = B * G;
  int Npad = 2;
  while (Npad < N) Npad <<= 1;
  if (tid == 0) bad = 0;

  // (1) survival, one lane per request, float32 products in order
  for (int b = tid; b < B; b += kSchedThreads) {
    float a = 1.f;
    for (int j = 0; j < G; ++j) {
      const float c = conf[b * G + j];
      if (!(c >= 0.f && c <= 1.f)) flag(status, RVA_DEV_BAD_CONF);
      a = (j == 0) ? c : __fmul_rn(a, c);
      surv_out[b * G + j] = a;
      const uint32_t bits = (a == 0.f) ? 0u : __float_as_uint(a);
      keys[b * G + j] = (uint64_t(~bits) << 32) | uint32_t(b * G + j);
    }
    cnt[b] = 0;
  }
  for (int i = N + tid; i < Npad; i += kSchedThreads) keys[i] = ~0ull;
  __syncthreads();

  // (2) bitonic sort, ascending key == (survival desc, index asc)
  for (int k = 2; k <= Npad; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < Npad; i += kSchedThreads) {
        const int p = i ^ j;
        if (p > i) {
          const uint64_t x = keys[i], y = keys[p];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            keys[i] = y;
            keys[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }

  // (3) S_K: each thread owns a contiguous run of ranks
  const int per = (Npad + kSchedThreads - 1) / kSchedThreads;
  const int r0 = tid * per;
  double run = 0.0;
  for (int i = 0; i < per; ++i) {
    const int r = r0 + i;
    if (r < N) run += double(__uint_as_float(~uint32_t(keys[r] >> 32)));
  }
  double total;
  double prefix = block_exclusive_scan_f64(run, wave_tot, &total);

  // (4) ratio (B + S_K) / T(B, K); K = r + 1 for rank r, K = 0 handled by thread 0
  const double ba = double(bias) + double(alpha[B]);
  double best = -INFINITY;
  int bestK = 0x7fffffff;
  if (tid == 0) {
    const double T0 = ba + double(theta[B]);
    if (!(T0 > 0.0)) flag(status, RVA_DEV_BAD_COST);
    best = T0 > 0.0 ? double(B) / T0 : -INFINITY;
    bestK = 0;
  }
  double S = prefix;
  for (int i = 0; i < per; ++i) {
    const int r = r0 + i;
    if (r < N) {
      S += double(__uint_as_float(~uint32_t(keys[r] >> 32)));
      const double T = ba + double(theta[B + r + 1]);
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
    best = lane < kSchedThreads / kWave ? red_ratio[lane] : -INFINITY;
    bestK = lane < kSchedThreads / kWave ? red_K[lane] : 0x7fffffff;
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
    const double T = ba + double(theta[B + N]);
    ratio = T > 0.0 ? (double(B) + total) / T : -INFINITY;
  }

  // (5) windows from the first K* ranks
  for (int i = 0; i < per; ++i) {
    const int r = r0 + i;
    if (r < Kstar && r < N) atomicAdd(&cnt[int(uint32_t(keys[r]) / uint32_t(G))], 1);
  }
  __syncthreads();
  for (int b = tid; b < B; b += kSchedThreads) windows[b] = 1 + cnt[b];
  if (tid == 0) {
    *K_out = Kstar;
    *ratio_out = ratio;
  }
  (void)bad;
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
  } else {
    hipError_t e = hipMemcpyAsync(conf_out, conf_in, sizeof(float) * rows,
                                  hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, B, G, mode, conf,
                     surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
  return hipGetLastError();
}

}  // namespace rva
