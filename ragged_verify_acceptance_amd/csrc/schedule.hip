// Stage 1: confidence head + temperature scaling, prefix survival, window argmax.
//
// Sources: "DSpark：投机解码与生产级 Serving 学习笔记" (sorenprojections.com) sections
// 07 (confidence head, survival product, Sequential Temperature Scaling) and 08 (the
// throughput-maximising prefix scheduler); the devpress.csdn.net DSpark-in-SGLang article,
// section 4 (additive step cost T(bs, K) = bias + alpha(bs) + theta(bs + K)).
//
// Kernels:
//   conf_head_kernel  one wave per (request, draft position): float64 dot product of the
//                     hidden state with the head weights, + bias, / T_k, logistic in
//                     float64, rounded to float32.  Skipped when the caller supplies c.
//   rank_kernel       batches of more than 1024 candidates only: the rank order of (2)
//                     below, one workgroup per request, each key ranked by binary searches
//                     in the other requests' runs (the ordering work of one workgroup
//                     would bound the whole pass on one compute unit).
//   schedule_kernel   ONE workgroup (256 to 1024 threads, by batch size) for the whole batch:
//                     (1) one lane per request forms the survival product left to right
//                         in float32 (bit-identical to a sequential definition);
//                     (2) keys (inverted survival bits, candidate index) order "survival
//                         desc, request asc, position asc"; each request's keys are already
//                         in order, so the rank order is a merge of B sorted runs (log2 B
//                         rounds, a binary search per key), or, after rank_kernel, the
//                         keys are stored at their ranks;
//                     (3) a workgroup scan in float64 gives S_K for every K;
//                     (4) a workgroup argmax of (B + S_K) / T(B, K), smallest K on ties;
//                     (5) LDS counters turn the first K* ranks into per-request windows.
#include "pack_block.h"
#include "rva_common.h"

namespace rva {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kRankThreads = 1024;
constexpr int kMaxCand = 4096;

template <typename T, bool VEC>
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
  if constexpr (VEC) {
    // 16-byte pieces of the row and of w (H a multiple of the piece, both 16-byte aligned),
    // kPieces per lane at a time from clamped indices, so that they are all in flight
    // together (one round trip up to kPieces * 64 pieces); pieces past the row add nothing
    constexpr int E = 16 / sizeof(T);
    constexpr int kPieces = 8;
    const int n = H / E;
    for (int j0 = 0; j0 < n; j0 += kPieces * kWave) {
      uint4 hv[kPieces];
      float4 wq[kPieces][E / 4];
#pragma unroll
      for (int k = 0; k < kPieces; ++k) {
        const int j = min(j0 + k * kWave + lane, n - 1);
        hv[k] = reinterpret_cast<const uint4*>(h)[j];
#pragma unroll
        for (int q = 0; q < E / 4; ++q) wq[k][q] = reinterpret_cast<const float4*>(w + size_t(j) * E)[q];
      }
      asm volatile("" ::: "memory");  // every piece is requested before the first is used
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kPieces; ++k) {
        float x[E];
        if constexpr (sizeof(T) == 2) {
          const uint32_t u[4] = {hv[k].x, hv[k].y, hv[k].z, hv[k].w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            x[2 * t] = __uint_as_float(u[t] << 16);
            x[2 * t + 1] = __uint_as_float(u[t] & 0xffff0000u);
          }
        } else {
          x[0] = __uint_as_float(hv[k].x), x[1] = __uint_as_float(hv[k].y);
          x[2] = __uint_as_float(hv[k].z), x[3] = __uint_as_float(hv[k].w);
        }
        double part = 0.0;
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          part += double(x[4 * q]) * double(wq[k][q].x);
          part += double(x[4 * q + 1]) * double(wq[k][q].y);
          part += double(x[4 * q + 2]) * double(wq[k][q].z);
          part += double(x[4 * q + 3]) * double(wq[k][q].w);
        }
        if (j0 + k * kWave + lane < n) acc += part;
      }
    }
  } else {
    for (int i = lane; i < H; i += kWave) acc += double(Elem<T>::load(h, i)) * double(w[i]);
  }
  acc = wave_sum_f64(acc);
  if (lane == 0) {
    double z = acc + double(b0);
    if (sts_T) z = z / double(sts_T[row % G]);
    const float c = float(1.0 / (1.0 + exp(-z)));
    if (!(c >= 0.f && c <= 1.f)) flag(status, RVA_DEV_BAD_CONF);
    conf_out[row] = c;
  }
}

// Inclusive float64 prefix sum over the wave's lanes (DPP); lane 63 ends with the total.
__device__ __forceinline__ double wave_inclusive_sum_f64(double x) {
  return wave_inclusive(x, 0.0, [](double p, double q) { return p + q; });
}

// One step of the argmax prefix: the moved (ratio, K) replaces this lane's when its ratio is
// larger, or equal with a smaller K.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(double& best, int& bestK) {
  const double o = dpp_move<CTRL, ROW_MASK>(double(-INFINITY), best);
  const int ok = dpp_move<CTRL, ROW_MASK>(int(0x7fffffff), bestK);
  if (o > best || (o == best && ok < bestK)) {
    best = o;
    bestK = ok;
  }
}

// Wave argmax in the same pattern; lane 63 ends with the wave's best (ratio, K).
__device__ __forceinline__ void wave_argmax(double& best, int& bestK) {
  argmax_step<kDppRowShr + 1, 0xf>(best, bestK);
  argmax_step<kDppRowShr + 2, 0xf>(best, bestK);
  argmax_step<kDppRowShr + 4, 0xf>(best, bestK);
  argmax_step<kDppRowShr + 8, 0xf>(best, bestK);
  argmax_step<kDppBcast15, 0xa>(best, bestK);
  argmax_step<kDppBcast31, 0xc>(best, bestK);
}

// Exclusive float64 prefix sum over the workgroup (one barrier): a DPP scan inside each wave,
// then every thread adds the totals of the waves before its own, in wave order, from LDS.
// *total: the sum of all wave totals (same order for every thread).
template <int NT>
__device__ __forceinline__ double block_exclusive_scan_f64(double v, double* lds_waves,
                                                           double* total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const double x = wave_inclusive_sum_f64(v);
  if (lane == kWave - 1) lds_waves[wave] = x;
  __syncthreads();
  double off = 0.0, tot = 0.0;
#pragma unroll
  for (int k = 0; k < NT / kWave; ++k) {
    if (k == wave) off = tot;
    tot += lds_waves[k];
  }
  *total = tot;
  return off + x - v;
}

// Sort key of a survival: its bits inverted (+0 for -0), so that ascending keys are
// descending survivals.
__device__ __forceinline__ uint32_t sort_key(float a) { return ~((a == 0.f) ? 0u : __float_as_uint(a)); }

// Rank order of the candidates by merging sorted runs.  A candidate's key is (h, i): h the
// inverted bits of its survival, i its index; ascending keys are "survival desc, request asc,
// position asc".  Each request's keys are already in order along its draft positions
// (survival never grows along a prefix), so the B runs of G keys are merged pairwise,
// log2(B) rounds, one barrier each.  In every round a run holds a contiguous range of
// requests, so all of a left run's indices are below its right partner's: comparing h alone,
// with ties going to the left run, gives the order of the full keys, and the searches read
// 4-byte words.  One key a thread (N <= NT): a binary search in the partner run, then the
// key lands at pair start + its index in its own run + the partner keys before it.  Returns
// the set holding the sorted h and i arrays (`buf` holds two sets).
// With invalid confidences (a run not in order) per-key positions may collide; both sets
// start with the keys, so every slot still holds some candidate.
template <int CAP>
struct MergeBuf {
  alignas(16) uint32_t h[2][CAP];
  uint32_t i[2][CAP];
};

template <int CAP>
__device__ __forceinline__ int merge_runs(uint32_t xh, uint32_t xi, MergeBuf<CAP>& buf, int N, int G) {
  const int tid = threadIdx.x;
  int c = 0;  // current set
  if (tid < N) {
    buf.h[0][tid] = buf.h[1][tid] = xh;
    buf.i[0][tid] = buf.i[1][tid] = xi;
  }
  __syncthreads();
  for (int len = G; len < N; len <<= 1) {
    const uint32_t* ch = buf.h[c];
    const uint32_t* ci = buf.i[c];
    uint32_t* nh = buf.h[c ^ 1];
    uint32_t* ni = buf.i[c ^ 1];
    const int i = tid;
    if (i < N) {
      const uint32_t kh = ch[i], ki = ci[i];
      const int q = i / len, start = q * len;
      const int ps = (q ^ 1) * len, pe = min(ps + len, N);
      int pos = i;
      if (ps < N) {
        const bool right = q & 1;  // partner keys with the same h come first
        int lo = ps, hi = pe;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          const uint32_t v = ch[mid];
          if (v < kh || (right && v == kh)) lo = mid + 1; else hi = mid;
        }
        pos = (q & ~1) * len + (i - start) + (lo - ps);
      }
      nh[pos] = kh;
      ni[pos] = ki;
    }
    __syncthreads();
    c ^= 1;
  }
  return c;
}

// LDS of one scheduling pass over up to CAP candidates.
template <int NT, int CAP>
struct SchedShared {
  MergeBuf<CAP> mb;
  float sa[CAP];
  int cnt[CAP];  // per request: drafts in the window, then the window itself
  double wave_tot[NT / kWave];
  double red_ratio[NT / kWave];
  int red_K[NT / kWave];
};

// The whole scheduling pass by one workgroup over N = B G candidates, E a thread (NT threads;
// small batches take fewer waves, so each merge round's searches and barrier involve fewer of
// them).  kRanked = false (N <= NT, E = 1): the rank order comes from merge_runs.  kRanked =
// true: rank_kernel ran first and left every candidate's rank in surv_out (as bits), and has
// validated and echoed the confidences; the keys are stored at their ranks and surv_out is
// overwritten with the survivals.  On return sh.cnt[b] holds request b's window.  `publish`:
// this workgroup writes the outputs (conf echo, survival, windows, K*, ratio) and raises the
// status bits.
// The pass's global loads, issued first by schedule_loads() (a caller may issue its own
// loads behind them before schedule_block() waits for these: the wait counter drains in
// order).  Every load reads a clamped index unconditionally, so that no branch makes the
// compiler wait for it where the branch joins.
template <int E>
struct SchedLoads {
  uint32_t rk[E];  // ranks from rank_kernel (ranked path)
  float th[E];     // theta[B + r + 1] for this thread's ranks r = tid*E + e
  float cv[E];     // confidences tid + e NT
  float alpha_B, theta_0, theta_N;
};

template <int E, int NT, bool kRanked>
__device__ __forceinline__ SchedLoads<E> schedule_loads(int B, int G, const float* __restrict__ conf,
                                                        const float* __restrict__ surv_out,
                                                        const float* __restrict__ alpha,
                                                        const float* __restrict__ theta) {
  SchedLoads<E> ld;
  const int tid = threadIdx.x, N = B * G;
  // ranks: this thread's own candidates, read before it writes their survivals
#pragma unroll
  for (int e = 0; e < E; ++e) ld.rk[e] = kRanked ? __float_as_uint(surv_out[min(tid * E + e, N - 1)]) : 0u;
  // the cost table entries of this thread's ranks: their round trip overlaps the survival
  // products and the sort
#pragma unroll
  for (int e = 0; e < E; ++e) ld.th[e] = theta[B + min(tid * E + e, N - 1) + 1];
  ld.alpha_B = alpha[B];
  ld.theta_0 = theta[B];
  ld.theta_N = theta[B + N];
#pragma unroll
  for (int e = 0; e < E; ++e) ld.cv[e] = conf[min(tid + e * NT, N - 1)];
  return ld;
}

template <int E, int NT, int CAP, bool kRanked>
__device__ __forceinline__ void schedule_block(SchedShared<NT, CAP>& sh, int B, int G, int mode,
                                               const SchedLoads<E>& ld, float* __restrict__ conf_out,
                                               float* __restrict__ surv_out, float bias,
                                               int32_t* __restrict__ windows, int32_t* __restrict__ K_out,
                                               double* __restrict__ ratio_out, int32_t* status, bool publish) {
  float* sa = sh.sa;
  int* cnt = sh.cnt;
  double* wave_tot = sh.wave_tot;
  double* red_ratio = sh.red_ratio;
  int* red_K = sh.red_K;
  const int tid = threadIdx.x;
  const int N = B * G;
  static_assert(kRanked || E == 1, "the merge takes one key a thread");

  const uint32_t* rk = ld.rk;
  const float* th = ld.th;
  const float alpha_B = ld.alpha_B, theta_0 = ld.theta_0, theta_N = ld.theta_N;
  // (1) survival: the confidences are staged in LDS by one coalesced load, then one lane per
  // request forms the float32 products left to right
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid + e * NT;  // < E NT <= CAP: slots past N are written but never read
    const float c = ld.cv[e];
    sa[i] = c;  // unconditional, so the load is not sunk into the branch below
    if (i < N) {
      if (!kRanked && publish && !(c >= 0.f && c <= 1.f)) flag(status, RVA_DEV_BAD_CONF);
      if (!kRanked && publish && conf_out) conf_out[i] = c;
    }
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
  int set = 0;
  if constexpr (kRanked) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = tid * E + e;
      if (i < N) {
        const float a = sa[i];
        if (publish) surv_out[i] = a;
        const uint32_t r = rk[e];
        if (r < uint32_t(N)) {  // a permutation of [0, N) for valid confidences
          sh.mb.h[0][r] = sort_key(a);
          sh.mb.i[0][r] = uint32_t(i);
        }
      }
    }
    __syncthreads();
  } else {
    const int i = tid;
    uint32_t xh = ~0u;
    if (i < N) {
      const float a = sa[i];
      if (publish) surv_out[i] = a;
      xh = sort_key(a);
    }
    set = merge_runs<CAP>(xh, uint32_t(i), sh.mb, N, G);
  }
  const uint32_t* key_h = sh.mb.h[set];
  const uint32_t* key_i = sh.mb.i[set];

  // (3) S_K: each thread owns a contiguous run of ranks, read as 16-byte words when it can
  constexpr int per = E;
  const int r0 = tid * per;
  uint32_t kh[per];
  if (per % 4 == 0 && r0 + per <= N) {
#pragma unroll
    for (int i = 0; i < per; i += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(&key_h[r0 + i]);
      kh[i] = q.x;
      kh[i + 1] = q.y;
      kh[i + 2] = q.z;
      kh[i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < per; ++i) kh[i] = r0 + i < N ? key_h[r0 + i] : ~0u;
  }
  double run = 0.0;
#pragma unroll
  for (int i = 0; i < per; ++i)
    if (r0 + i < N) run += double(__uint_as_float(~kh[i]));
  double total;
  double prefix = block_exclusive_scan_f64<NT>(run, wave_tot, &total);

  // (4) ratio (B + S_K) / T(B, K); K = r + 1 for rank r, K = 0 handled by thread 0
  const double ba = double(bias) + double(alpha_B);
  double best = -INFINITY;
  int bestK = 0x7fffffff;
  if (tid == 0) {
    const double T0 = ba + double(theta_0);
    if (publish && !(T0 > 0.0)) flag(status, RVA_DEV_BAD_COST);
    best = T0 > 0.0 ? double(B) / T0 : -INFINITY;
    bestK = 0;
  }
  double S = prefix;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int r = r0 + i;
    if (r < N) {
      S += double(__uint_as_float(~kh[i]));
      const double T = ba + double(th[i]);
      if (publish && !(T > 0.0)) flag(status, RVA_DEV_BAD_COST);
      const double ratio = T > 0.0 ? (double(B) + S) / T : -INFINITY;
      if (ratio > best) {
        best = ratio;
        bestK = r + 1;
      }
    }
  }
  // workgroup argmax: larger ratio wins, smaller K on equal ratio.  DPP inside each wave,
  // then every thread folds the per-wave bests itself, in wave order (one barrier)
  const int lane = tid % kWave, wave = tid / kWave;
  wave_argmax(best, bestK);
  if (lane == kWave - 1) {
    red_ratio[wave] = best;
    red_K[wave] = bestK;
  }
  __syncthreads();
  best = -INFINITY;
  bestK = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < NT / kWave; ++k) {
    const double o = red_ratio[k];
    const int ok = red_K[k];
    if (o > best || (o == best && ok < bestK)) {
      best = o;
      bestK = ok;
    }
  }
  int Kstar = bestK;
  double ratio = best;
  if (mode == RVA_MODE_STATIC) {
    Kstar = N;
    const double T = ba + double(theta_N);
    ratio = T > 0.0 ? (double(B) + total) / T : -INFINITY;
  }

  // (5) windows from the first K* ranks
  for (int i = 0; i < per; ++i) {
    const int r = r0 + i;
    if (r < Kstar && r < N) atomicAdd(&cnt[min(int(key_i[r] / uint32_t(G)), B - 1)], 1);
  }
  __syncthreads();
  for (int b = tid; b < B; b += NT) {
    const int w = 1 + cnt[b];
    cnt[b] = w;
    if (publish) windows[b] = w;
  }
  if (publish && tid == 0) {
    *K_out = Kstar;
    *ratio_out = ratio;
  }
  __syncthreads();
}

template <int E, int NT, bool kRanked>
__global__ __launch_bounds__(NT) void schedule_kernel(
    int B, int G, int mode, const float* __restrict__ conf, float* __restrict__ conf_out,
    float* __restrict__ surv_out, float bias, const float* __restrict__ alpha,
    const float* __restrict__ theta, int32_t* __restrict__ windows, int32_t* __restrict__ K_out,
    double* __restrict__ ratio_out, int32_t* status) {
  __shared__ SchedShared<NT, kMaxCand> sh;
  const SchedLoads<E> ld = schedule_loads<E, NT, kRanked>(B, G, conf, surv_out, alpha, theta);
  schedule_block<E, NT, kMaxCand, kRanked>(sh, B, G, mode, ld, conf_out, surv_out, bias, windows, K_out,
                                           ratio_out, status, true);
}

// Ranks for batches of more than one workgroup's threads, spread over B workgroups (one per
// request) so that the ordering work runs on many compute units instead of one.  Every
// workgroup forms all N survivals in LDS (the float32 products of the single-workgroup pass)
// and turns them into sort keys.  Key j of this workgroup's request b then has rank
//   j + sum over requests b' != b of (keys of b' that come before it),
// each count a binary search in the run of b' (a run is in ascending key order; on equal
// survival the lower request comes first).  Ranks go to surv_out as bits; schedule_kernel
// <E, NT, true> stores the keys at their ranks and overwrites surv_out with the survivals.
// Request b's workgroup also validates and echoes request b's confidences.
template <int NT>
__global__ __launch_bounds__(NT) void rank_kernel(int B, int G, const float* __restrict__ conf,
                                                  float* __restrict__ conf_out, float* __restrict__ surv_out,
                                                  int32_t* status) {
  __shared__ uint32_t key[kMaxCand];
  __shared__ int acc[64];  // G <= 63
  const int tid = threadIdx.x, b = blockIdx.x, N = B * G;
  if (tid < G) {
    acc[tid] = 0;
    const float c = conf[b * G + tid];
    if (!(c >= 0.f && c <= 1.f)) flag(status, RVA_DEV_BAD_CONF);
    if (conf_out) conf_out[b * G + tid] = c;
  }
  for (int i = tid; i < N; i += NT) key[i] = __float_as_uint(conf[i]);
  __syncthreads();
  for (int r = tid; r < B; r += NT) {
    float a = 1.f;
    for (int j = 0; j < G; ++j) {
      const float c = __uint_as_float(key[r * G + j]);
      a = (j == 0) ? c : __fmul_rn(a, c);
      key[r * G + j] = sort_key(a);
    }
  }
  __syncthreads();
  // thread (group g, position j) counts against the runs g, g + P, ... (P groups of G
  // threads), four runs at a time so that their searches overlap
  const int P = NT / G, j = tid % G, g = tid / G;
  if (g < P) {
    const uint32_t x = key[b * G + j];
    int top = 1;  // largest power of two <= G
    while (2 * top <= G) top *= 2;
    int count = 0;
    for (int r0 = g; r0 < B; r0 += 4 * P) {
      int lo[4], base[4];
      bool before[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rr = r0 + u * P;
        lo[u] = 0;
        base[u] = min(rr, B - 1) * G;
        before[u] = rr < b;
      }
      // lo = keys of the run before x: a search over powers of two, reads clamped into the run
      for (int step = top; step > 0; step >>= 1) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = lo[u] + step;
          const uint32_t v = key[base[u] + min(q, G) - 1];
          if (q <= G && (v < x || (before[u] && v == x))) lo[u] = q;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rr = r0 + u * P;
        if (rr < B && rr != b) count += lo[u];
      }
    }
    atomicAdd(&acc[j], count);
  }
  __syncthreads();
  if (tid < G) surv_out[b * G + tid] = __uint_as_float(uint32_t(tid + acc[tid]));
}

// Stages 1 and 2 in one launch for batches of at most NT candidates: every workgroup runs
// the (deterministic) scheduling pass itself, so all of them hold the same windows without
// exchanging anything; workgroup 0 publishes the schedule, and each workgroup then packs its
// own kRowsPerBlock(NT) destination rows.
template <int NT, bool kPre>
__global__ __launch_bounds__(NT) void schedule_pack_kernel(
    int B, int G, int mode, const float* __restrict__ conf, float* __restrict__ conf_out,
    float* __restrict__ surv_out, float bias, const float* __restrict__ alpha,
    const float* __restrict__ theta, int32_t* __restrict__ windows, int32_t* __restrict__ K_out,
    double* __restrict__ ratio_out, const int32_t* __restrict__ context_lens, TierTable tiers,
    const uint8_t* __restrict__ src, size_t row_bytes, uint8_t* __restrict__ dst, int max_rows,
    int32_t* __restrict__ cu_out, int32_t* __restrict__ row_req, int32_t* __restrict__ row_pos,
    int32_t* __restrict__ total_tier, int32_t* status) {
  __shared__ SchedShared<NT, NT> sh;
  __shared__ PackShared<NT, NT> psh;
  __shared__ int ctx[NT];
  const int tid = threadIdx.x, gamma = G + 1;
  const bool first = blockIdx.x == 0;
  // The context lengths (row positions) and this block's kPackRows SOURCE rows are
  // requested during the scheduling pass, right behind its own loads (which it then waits
  // for alone) and land while it runs.  Source rows are request-major, row s = b gamma + i
  // (the grid covers max_rows >= B gamma of them): once the windows are known, row s goes to
  // destination row cu[b] + i when i < w_b.  Rows of up to 2 NT x 16 bytes, 16-byte aligned;
  // others are copied destination-first after the pass (pack_block); the host picks kPre
  // (pre_ok below).  The loads read clamped rows and pieces unconditionally (the stores
  // check them), in straight-line code, so that the pass's waits count them exactly.
  const int n16 = int(row_bytes / 16);
  constexpr bool pre = kPre;
  const SchedLoads<1> ld = schedule_loads<1, NT, false>(B, G, conf, surv_out, alpha, theta);
  __builtin_amdgcn_sched_barrier(0);
  const int ctx_v = context_lens[min(tid, B - 1)];
  uint4 v[kPackRows][2];
#pragma unroll
  for (int rr = 0; rr < kPackRows; ++rr)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int srow = min(int(blockIdx.x) * kPackRows + rr, B * gamma - 1), k = min(h * NT + tid, max(n16 - 1, 0));
      v[rr][h] = kPre ? reinterpret_cast<const uint4*>(src + size_t(srow) * row_bytes)[k] : make_uint4(0, 0, 0, 0);
    }
  schedule_block<1, NT, NT, false>(sh, B, G, mode, ld, conf_out, surv_out, bias, windows, K_out, ratio_out, status,
                                   first);
  if (tid < B) ctx[tid] = ctx_v;  // published by pack_block's barrier
  pack_block<NT, NT, kPackRows>(psh, B, gamma, sh.cnt, false, ctx, tiers, pre ? nullptr : src, row_bytes,
                                pre ? nullptr : dst, max_rows, cu_out, row_req, row_pos, total_tier, status,
                                blockIdx.x, first);
  if (!pre) return;
  const int M = psh.s_M, tier = psh.s_tier;
#pragma unroll
  for (int rr = 0; rr < kPackRows; ++rr) {
    const int srow = blockIdx.x * kPackRows + rr;
    const int b = srow / gamma, i = srow % gamma;
    if (srow < B * gamma && i < psh.cu[b + 1] - psh.cu[b]) {
      uint4* d = reinterpret_cast<uint4*>(dst + size_t(psh.cu[b] + i) * row_bytes);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (h * NT + tid < n16) d[h * NT + tid] = v[rr][h];
    }
    // this block's destination rows in [M, tier) are pad rows: zero
    const int r = blockIdx.x * kPackRows + rr;
    if (r >= M && r < tier && r < max_rows) {
      uint4* d = reinterpret_cast<uint4*>(dst + size_t(r) * row_bytes);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (h * NT + tid < n16) d[h * NT + tid] = make_uint4(0, 0, 0, 0);
    }
  }
}

}  // namespace

namespace {

// Stage 1's confidences: the head kernel's output when hidden states are given, else the
// caller's; `echo` is where the schedule kernel copies caller confidences (nullptr when the
// head wrote conf_out itself).
hipError_t confidences(int B, int G, const void* hidden, int hidden_dtype, int H, const float* head_w,
                       float head_b, const float* conf_in, const float* sts_T, float* conf_out,
                       int32_t* status, hipStream_t stream, const float** conf, float** echo) {
  const int rows = B * G;
  *conf = conf_in;
  *echo = conf_in ? conf_out : nullptr;
  if (conf_in) return hipSuccess;
  const dim3 grid((rows + 3) / 4), block(256);
  const bool aligned16 = (reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(head_w)) % 16 == 0;
  if (hidden_dtype == RVA_BF16) {
    const uint16_t* hp = static_cast<const uint16_t*>(hidden);
    if (aligned16 && H % 8 == 0)
      hipLaunchKernelGGL((conf_head_kernel<uint16_t, true>), grid, block, 0, stream, hp, rows, G, H, head_w, head_b,
                         sts_T, conf_out, status);
    else
      hipLaunchKernelGGL((conf_head_kernel<uint16_t, false>), grid, block, 0, stream, hp, rows, G, H, head_w, head_b,
                         sts_T, conf_out, status);
  } else {
    const float* hp = static_cast<const float*>(hidden);
    if (aligned16 && H % 4 == 0)
      hipLaunchKernelGGL((conf_head_kernel<float, true>), grid, block, 0, stream, hp, rows, G, H, head_w, head_b,
                         sts_T, conf_out, status);
    else
      hipLaunchKernelGGL((conf_head_kernel<float, false>), grid, block, 0, stream, hp, rows, G, H, head_w, head_b,
                         sts_T, conf_out, status);
  }
  *conf = conf_out;
  return hipGetLastError();
}

int pad_pow2(int n) {
  int p = 2;
  while (p < n) p <<= 1;
  return p;
}

}  // namespace

hipError_t launch_schedule(int B, int gamma, int mode, const void* hidden, int hidden_dtype,
                           int H, const float* head_w, float head_b, const float* conf_in,
                           const float* sts_T, float bias, const float* alpha,
                           const float* theta, float* conf_out, float* surv_out,
                           int32_t* windows, int32_t* K_out, double* ratio_out,
                           int32_t* status, hipStream_t stream) {
  const int G = gamma - 1;
  const float* conf = nullptr;
  float* echo = nullptr;
  hipError_t e = confidences(B, G, hidden, hidden_dtype, H, head_w, head_b, conf_in, sts_T, conf_out, status,
                             stream, &conf, &echo);
  if (e != hipSuccess) return e;
  const int Npad = pad_pow2(B * G);
  if (Npad <= 256)
    hipLaunchKernelGGL((schedule_kernel<1, 256, false>), dim3(1), dim3(256), 0, stream, B, G, mode,
                       conf, echo, surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
  else if (Npad <= 512)
    hipLaunchKernelGGL((schedule_kernel<1, 512, false>), dim3(1), dim3(512), 0, stream, B, G, mode,
                       conf, echo, surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
  else if (Npad <= kSchedThreads)
    hipLaunchKernelGGL((schedule_kernel<1, kSchedThreads, false>), dim3(1), dim3(kSchedThreads), 0, stream, B,
                       G, mode, conf, echo, surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
  else {
    // ranks on B workgroups, then the scan / argmax / windows on one
    hipLaunchKernelGGL((rank_kernel<kRankThreads>), dim3(B), dim3(kRankThreads), 0, stream, B, G, conf, echo,
                       surv_out, status);
    if (Npad <= 2 * kSchedThreads)
      hipLaunchKernelGGL((schedule_kernel<2, kSchedThreads, true>), dim3(1), dim3(kSchedThreads), 0, stream, B,
                         G, mode, conf, echo, surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
    else
      hipLaunchKernelGGL((schedule_kernel<4, kSchedThreads, true>), dim3(1), dim3(kSchedThreads), 0, stream, B,
                         G, mode, conf, echo, surv_out, bias, alpha, theta, windows, K_out, ratio_out, status);
  }
  return hipGetLastError();
}

hipError_t launch_schedule_pack(int B, int gamma, int mode, const void* hidden, int hidden_dtype, int H,
                                const float* head_w, float head_b, const float* conf_in, const float* sts_T,
                                float bias, const float* alpha, const float* theta, float* conf_out,
                                float* surv_out, int32_t* windows, int32_t* K_out, double* ratio_out,
                                const int32_t* context_lens, const TierTable& tiers, const void* src,
                                size_t row_bytes, void* dst, int max_rows, int32_t* cu, int32_t* row_req,
                                int32_t* row_pos, int32_t* total_tier, int32_t* status, hipStream_t stream) {
  const int G = gamma - 1;
  const int Npad = pad_pow2(B * G);
  if (Npad > kSchedThreads) {  // more candidates than one workgroup's threads: two launches
    hipError_t e = launch_schedule(B, gamma, mode, hidden, hidden_dtype, H, head_w, head_b, conf_in, sts_T, bias,
                                   alpha, theta, conf_out, surv_out, windows, K_out, ratio_out, status, stream);
    if (e != hipSuccess) return e;
    return launch_pack(B, gamma, windows, context_lens, tiers, src, row_bytes, dst, max_rows, cu, row_req,
                       row_pos, total_tier, status, stream);
  }
  const float* conf = nullptr;
  float* echo = nullptr;
  hipError_t e = confidences(B, G, hidden, hidden_dtype, H, head_w, head_b, conf_in, sts_T, conf_out, status,
                             stream, &conf, &echo);
  if (e != hipSuccess) return e;
  const dim3 grid((max_rows + kPackRows - 1) / kPackRows);
  const uint8_t* s8 = static_cast<const uint8_t*>(src);
  uint8_t* d8 = static_cast<uint8_t*>(dst);
  const int NT = Npad <= 256 ? 256 : (Npad <= 512 ? 512 : kSchedThreads);
  // source rows prefetched during the scheduling pass: 16-byte pieces, at most 2 NT a row
  const bool pre = s8 && row_bytes % 16 == 0 && row_bytes / 16 <= size_t(2 * NT) &&
                   ((reinterpret_cast<uintptr_t>(s8) | reinterpret_cast<uintptr_t>(d8)) % 16 == 0);
#define RVA_SP_LAUNCH(NTV, PRE)                                                                                \
  hipLaunchKernelGGL((schedule_pack_kernel<NTV, PRE>), grid, dim3(NTV), 0, stream, B, G, mode, conf, echo,      \
                     surv_out, bias, alpha, theta, windows, K_out, ratio_out, context_lens, tiers, s8, row_bytes, \
                     d8, max_rows, cu, row_req, row_pos, total_tier, status)
  if (NT == 256) {
    if (pre) RVA_SP_LAUNCH(256, true); else RVA_SP_LAUNCH(256, false);
  } else if (NT == 512) {
    if (pre) RVA_SP_LAUNCH(512, true); else RVA_SP_LAUNCH(512, false);
  } else {
    if (pre) RVA_SP_LAUNCH(kSchedThreads, true); else RVA_SP_LAUNCH(kSchedThreads, false);
  }
#undef RVA_SP_LAUNCH
  return hipGetLastError();
}

}  // namespace rva
