// Markov sequential head of the block drafter: per draft position, the base logits of the
// parallel backbone plus a previous-token bias from rank-r factors, then one draw; the
// positions run in order because each bias needs the token drawn before it.
//
// Source: "DSpark：投机解码与生产级 Serving 学习笔记" (sorenprojections.com), section
// "05 · Core Innovation A", 5.1-5.3: the backbone emits U_1 .. U_gamma in one pass; the
// sequential head adds B(x_{k-1}, v) = (W1 W2)[x_{k-1}, v] of rank r = 256 (an embedding
// lookup and a projection per step); section "09 · End-to-End Cycle": the light module
// samples the positions one after another.
//
// Weights are int8 with float32 scales, both factors stored as [V, r] rows (q1[x] is the
// embedding of the previous token, q2[v] the projection row of token v), so the dot
// product is exact in int32 and the logit U_k(v) + (s1[x] s2[v]) dot is formed in float64
// with explicitly rounded operations (no contraction) and stored in the dtype of U.  The
// draw uses the stored logits (the draft distribution the acceptance step sees).
//
// Per position, two launches:
//  * markov_logits_kernel: one workgroup per 128-token vocabulary tile.  Its four waves
//    hold the tile's q2 rows in registers as the MFMA's A operand and run
//    v_mfma_i32_16x16x32_i8 against the B operand, q1[x_b] of 64 requests at a time
//    gathered into LDS.  Both operands walk r in one permuted order (an integer sum does
//    not care about the order), chosen so that the four lanes of a q2 row load 64
//    contiguous bytes per instruction.  The A rows of a wave's column blocks interleave
//    their tokens so that each lane ends with 8 consecutive tokens of one request: the
//    epilogue reads U (requested before the MFMA) and writes the logits 16 bytes at a
//    time straight from the accumulators, and each request's tile max and float64 mass
//    below it are merged over lanes and waves for the draw.
//  * markov_sample_kernel: one workgroup per request combines the tile statistics into
//    the row's maximum and total mass, finds the tile where the cumulative mass passes
//    u * S (block scan of per-thread tile runs), and rescans that tile with one wave.
#include <cmath>

#include "exp2_f64.h"
#include "rva_common.h"

namespace rva {
namespace {

constexpr int kMkThreads = 256;
constexpr int kCB = 2;               // 16-token column blocks per wave
constexpr int kTileV = 4 * kCB * 16;  // vocabulary entries per workgroup (4 waves)
constexpr int kLaneTok = kTileV / kWave;  // tokens per lane in the draw's tile rescan
constexpr int kReqGroup = 64;        // requests per MFMA pass (4 row blocks of 16)
constexpr int kSampleThreads = 256;

typedef int v4i __attribute__((ext_vector_type(4)));

struct MkLayout {
  size_t off_max, off_sum, off_e, off_s1, total;
  int ntiles;
};

MkLayout mk_layout(int B, int V) {
  MkLayout l;
  l.ntiles = (V + kTileV - 1) / kTileV;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  l.off_max = 0;
  l.off_sum = up(size_t(B) * l.ntiles * sizeof(float));
  l.off_e = l.off_sum + up(size_t(B) * l.ntiles * sizeof(double));  // q1 row of x_b, [B][256]
  l.off_s1 = l.off_e + up(size_t(B) * 256);                          // s1[x_b], [B]
  l.total = l.off_s1 + up(size_t(B) * sizeof(float));
  return l;
}

template <typename T> struct Out;
template <> struct Out<uint16_t> {
  __device__ static float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ static float round(double x) { return bf16_to_f32(f32_to_bf16(float(x))); }
  __device__ static void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};
template <> struct Out<float> {
  __device__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ static float round(double x) { return float(x); }
  __device__ static void store(float* p, size_t i, float v) { p[i] = v; }
};

__device__ __forceinline__ int prev_token(const MarkovArgs& a, int b, int k) {
  int x = k == 0 ? a.anchor[b] : a.tokens[size_t(b) * a.G1 + k - 1];
  if (x < 0 || x >= a.V) {
    flag(a.status, RVA_DEV_BAD_TOKEN);
    x = 0;
  }
  return x;
}

// VEC: V is a multiple of 8 and U / out are 16-byte aligned, so a lane's 4 tokens are one
// aligned vector access; its loads are then issued unconditionally from clamped addresses
// (no branch between issue and use, so the compiler keeps them in flight together).
// The rows the next logits pass multiplies by: q1[x] and s1[x] of request b's previous
// token, copied to the workspace by one wave (R bytes), so the pass itself loads them
// without a dependent lookup.
template <int R>
__device__ __forceinline__ void stage_row(const MarkovArgs& a, const MkLayout& l, int b, int x, int lane) {
  int8_t* e = static_cast<int8_t*>(a.ws) + l.off_e + size_t(b) * R;
  if (lane < R / 16) *reinterpret_cast<uint4*>(e + lane * 16) = *reinterpret_cast<const uint4*>(a.w1 + size_t(x) * R + lane * 16);
  if (lane == 0) reinterpret_cast<float*>(static_cast<char*>(a.ws) + l.off_s1)[b] = a.s1[x];
}

// Stages the anchors' rows for the first position: one wave per request.
template <int R>
__global__ __launch_bounds__(256) void markov_stage_kernel(MarkovArgs a, MkLayout l) {
  const int b = blockIdx.x * 4 + threadIdx.x / kWave;
  if (b >= a.B) return;
  stage_row<R>(a, l, b, prev_token(a, b, 0), threadIdx.x % kWave);
}

template <typename T, int R, bool VEC>
__global__ __launch_bounds__(kMkThreads, VEC ? 4 : 1) void markov_logits_kernel(MarkovArgs a, MkLayout l, int k,
                                                                                  Exp2Poly P) {
  constexpr int kSteps = R / 32;       // MFMA k-steps (8 bytes per lane each)
  constexpr int kEPitch = R + 8;       // LDS row pitch of the gathered embeddings (8-aligned)
  constexpr int kW = kMkThreads / kWave;
  __shared__ __align__(16) int8_t sE[kReqGroup * kEPitch];
  __shared__ float sS1[kReqGroup];
  __shared__ double tab[256];
  __shared__ float wmax[kW][kReqGroup];
  __shared__ double wsum[kW][kReqGroup];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = lane / 16, c16 = lane % 16;
  const int v0 = blockIdx.x * kTileV;
  if (tid < 256) tab[tid] = exp2_f64(P, double(tid) / 256.0);  // read after the barriers below

  // The staged q1[x_b] rows (16 bytes per piece) and scales of a request group; rows past
  // the batch repeat its last row (their results are never used).  The first group's are
  // requested before anything else: their stores then wait for them alone (the wait
  // counter drains in order), not for the q2 and U loads behind them.
  const int8_t* estage = static_cast<const int8_t*>(a.ws) + l.off_e;
  const float* s1stage = reinterpret_cast<const float*>(static_cast<const char*>(a.ws) + l.off_s1);
  constexpr int kEIt = kReqGroup * (R / 16) / kMkThreads;  // 16-byte pieces per thread
  static_assert(kEIt * kMkThreads == kReqGroup * (R / 16), "whole pieces per thread");
  uint4 ev[kEIt];
  float s1v;
  auto stage_load = [&](int b0, int nb) {
#pragma unroll
    for (int j = 0; j < kEIt; ++j) {
      const int it = tid + j * kMkThreads, rl = it / (R / 16), c = it % (R / 16);
      ev[j] = *reinterpret_cast<const uint4*>(estage + size_t(b0 + min(rl, nb - 1)) * R + c * 16);
    }
    s1v = s1stage[b0 + min(tid % kReqGroup, nb - 1)];
  };
  auto stage_store = [&]() {
#pragma unroll
    for (int j = 0; j < kEIt; ++j) {
      const int it = tid + j * kMkThreads, rl = it / (R / 16), c = it % (R / 16);
      uint2* dst = reinterpret_cast<uint2*>(sE + rl * kEPitch + c * 16);
      dst[0] = make_uint2(ev[j].x, ev[j].y);
      dst[1] = make_uint2(ev[j].z, ev[j].w);
    }
    if (tid < kReqGroup) sS1[tid] = s1v;
  };
  stage_load(0, min(kReqGroup, a.B));
  const int vw = v0 + kCB * 16 * wave;
  // the scales of this lane's 4 kCB consecutive tokens (4 per column block)
  const int vl = vw + 4 * kCB * g;  // this lane's first token
  float s2v[kCB][4];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int vb = vl + 4 * cb;
    if constexpr (VEC) {
      const float4 w = *reinterpret_cast<const float4*>(a.s2 + min(vb, a.V - 4));
      s2v[cb][0] = w.x; s2v[cb][1] = w.y; s2v[cb][2] = w.z; s2v[cb][3] = w.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) s2v[cb][i] = a.s2[min(vb + i, a.V - 1)];
    }
  }
  // keep the compiler from moving these loads behind the q2 loads (or the s1 load into the
  // store's branch): the stores, and the scales' conversions, would then wait for q2 too
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // this wave's kCB 16-token column blocks of q2 as the MFMA's A operand.  Row rho of block
  // cb is token vw + 4 kCB (rho / 4) + 4 cb + rho % 4 (vw: the wave's first token), so the
  // result rows 4g..4g+3 of every block are the kCB*4 consecutive tokens vw + 4 kCB g + ...
  // of one lane.  k order: step s takes bytes 64 (s / 2) + 16 g + 8 (s % 2) of r (every byte
  // once; the B operand below walks the same order), so lanes g = 0..3 of a row load 64
  // contiguous bytes per instruction.
  long afrag[kCB][kSteps];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int v = min(vw + 4 * kCB * (c16 / 4) + 4 * cb + c16 % 4, a.V - 1);
    const int8_t* row = a.w2 + size_t(v) * R + g * 16;
#pragma unroll
    for (int s = 0; s < kSteps; s += 2) {
      const uint4 w = *reinterpret_cast<const uint4*>(row + (s / 2) * 64);
      afrag[cb][s] = (long(w.y) << 32) | long(uint32_t(w.x));
      afrag[cb][s + 1] = (long(w.w) << 32) | long(uint32_t(w.z));
    }
  }

  const T* U = static_cast<const T*>(a.base);
  T* O = static_cast<T*>(a.out);
  float* tmax = reinterpret_cast<float*>(static_cast<char*>(a.ws) + l.off_max);
  double* tsum = reinterpret_cast<double*>(static_cast<char*>(a.ws) + l.off_sum);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  stage_store();
  // output element of (row block rb, column block cb, i): request rb*16 + c16, token
  // vl + 4 cb + i (the MFMA result layout: lane column c16, rows 4g + i)
  for (int b0 = 0; b0 < a.B; b0 += kReqGroup) {
    const int nb = min(kReqGroup, a.B - b0);
    if (b0 > 0) {
      __syncthreads();  // the previous group's LDS is no longer read
      stage_load(b0, nb);
      stage_store();
    }
    // the epilogue's base logits, requested before the MFMA and kept in their storage
    // format (bf16 pairs stay packed: half the registers)
    constexpr int kU = sizeof(T) == 2 ? 2 : 4;
    static_assert(kCB % 2 == 0, "bf16 tokens are loaded and stored 8 at a time");
    uint32_t uv[4][kCB][kU];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const int rl = rb * 16 + c16, vb = vl + 4 * cb;
        if constexpr (VEC) {
          // rows past the batch and tokens past V read a valid place; their values are unused
          // (V is a multiple of 8 and vl of 8, so a run of 8 is all in or all out)
          const size_t base = (size_t(b0 + min(rl, nb - 1)) * a.G1 + k) * a.V + min(vb, a.V - 4);
          if constexpr (sizeof(T) == 2) {
            if (cb % 2 == 0) {  // 8 tokens: this block's 4 and the next one's
              const size_t b8 = (size_t(b0 + min(rl, nb - 1)) * a.G1 + k) * a.V + min(vb, a.V - 8);
              const uint4 w = *reinterpret_cast<const uint4*>(U + b8);
              uv[rb][cb][0] = w.x;
              uv[rb][cb][1] = w.y;
              uv[rb][cb + 1][0] = w.z;
              uv[rb][cb + 1][1] = w.w;
            }
          } else {
            const uint4 w = *reinterpret_cast<const uint4*>(U + base);
            uv[rb][cb][0] = w.x; uv[rb][cb][1] = w.y; uv[rb][cb][2] = w.z; uv[rb][cb][3] = w.w;
          }
        } else {
          const size_t base = (size_t(b0 + rl) * a.G1 + k) * a.V;
          float x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = (rl < nb && vb + i < a.V) ? Out<T>::load(U, base + vb + i) : 0.f;
          if constexpr (sizeof(T) == 2) {
            uv[rb][cb][0] = uint32_t(f32_to_bf16(x[0])) | (uint32_t(f32_to_bf16(x[1])) << 16);
            uv[rb][cb][1] = uint32_t(f32_to_bf16(x[2])) | (uint32_t(f32_to_bf16(x[3])) << 16);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) uv[rb][cb][i] = __float_as_uint(x[i]);
          }
        }
      }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int rl = rb * 16 + c16;
      v4i acc[kCB];
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) acc[cb] = v4i{0, 0, 0, 0};
      const int8_t* erow = sE + rl * kEPitch + g * 16;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const long bv = *reinterpret_cast<const long*>(erow + (s / 2) * 64 + (s % 2) * 8);
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          acc[cb] = __builtin_amdgcn_mfma_i32_16x16x32_i8(afrag[cb][s], bv, acc[cb], 0, 0, 0);
      }
      // logits of request rl at this lane's 8 tokens, and their (max, mass) summary
      const double s1 = double(sS1[rl]);
      const size_t base = (size_t(b0 + rl) * a.G1 + k) * a.V;
      float lv[kCB][4];
      float m = -INFINITY;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const int vb = vl + 4 * cb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = vb + i;
          lv[cb][i] = -INFINITY;
          if (rl < nb && v < a.V) {
            const double t = s1 * double(s2v[cb][i]);  // exact: a product of two float32
            const float uf = sizeof(T) == 2 ? bf16_to_f32(uint16_t(i & 1 ? uv[rb][cb][i >> 1] >> 16
                                                                            : uv[rb][cb][i >> 1] & 0xffff))
                                            : __uint_as_float(uv[rb][cb][i % kU]);
            const double lg = __dadd_rn(double(uf), __dmul_rn(t, double(acc[cb][i])));
            lv[cb][i] = Out<T>::round(lg);
            m = fmaxf(m, lv[cb][i]);
          }
        }
        if (rl < nb) {
          if (VEC && vb < a.V) {
            if constexpr (sizeof(T) == 2) {
              if (cb % 2 == 1)  // 8 tokens: the previous block's 4 and this one's
                *reinterpret_cast<uint4*>(O + base + vb - 4) =
                    make_uint4(f32_to_bf16(lv[cb - 1][0]) | (uint32_t(f32_to_bf16(lv[cb - 1][1])) << 16),
                               f32_to_bf16(lv[cb - 1][2]) | (uint32_t(f32_to_bf16(lv[cb - 1][3])) << 16),
                               f32_to_bf16(lv[cb][0]) | (uint32_t(f32_to_bf16(lv[cb][1])) << 16),
                               f32_to_bf16(lv[cb][2]) | (uint32_t(f32_to_bf16(lv[cb][3])) << 16));
            } else {
              *reinterpret_cast<float4*>(O + base + vb) = make_float4(lv[cb][0], lv[cb][1], lv[cb][2], lv[cb][3]);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (vb + i < a.V) Out<T>::store(O, base + vb + i, lv[cb][i]);
          }
        }
      }
      // the wave's 32 tokens of this request sit in the 4 lanes c16, c16+16, +32, +48
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      double sum = 0.0;
      if (m != -INFINITY) {
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (lv[cb][i] != -INFINITY) sum += exp2_tab(P, tab, (double(lv[cb][i]) - double(m)) * kLog2eF64);
      }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      if (g == 0) {
        wmax[wave][rl] = m;
        wsum[wave][rl] = sum;
      }
    }
    __syncthreads();
    // tile summary per request: the four waves' (max, mass) merged in wave order
    if (tid < nb) {
      float M = wmax[0][tid];
      for (int w = 1; w < kW; ++w) M = fmaxf(M, wmax[w][tid]);
      double S = 0.0;
      for (int w = 0; w < kW; ++w)
        if (wmax[w][tid] != -INFINITY) S += wsum[w][tid] * exp2_tab(P, tab, (double(wmax[w][tid]) - double(M)) * kLog2eF64);
      tmax[size_t(b0 + tid) * l.ntiles + blockIdx.x] = M;
      tsum[size_t(b0 + tid) * l.ntiles + blockIdx.x] = S;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kSampleThreads) void markov_sample_kernel(MarkovArgs a, MkLayout l, int k,
                                                                       Exp2Poly P) {
  __shared__ double tab[256];
  __shared__ double sc[kSampleThreads / kWave];
  __shared__ float smax[kSampleThreads / kWave];
  __shared__ int s_tile;
  __shared__ double s_before, s_S;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  tab[tid] = exp2_f64(P, double(tid) / 256.0);  // read after the barriers below
  auto ex = [&](float x, float m) { return exp2_tab(P, tab, (double(x) - double(m)) * kLog2eF64); };
  const float* tmax = reinterpret_cast<const float*>(static_cast<const char*>(a.ws) + l.off_max) + size_t(b) * l.ntiles;
  const double* tsum = reinterpret_cast<const double*>(static_cast<const char*>(a.ws) + l.off_sum) + size_t(b) * l.ntiles;
  const int nt = l.ntiles, per = (nt + kSampleThreads - 1) / kSampleThreads;
  const int t0 = min(tid * per, nt), t1 = min(t0 + per, nt);
  // Loads that depend on nothing else go out first: the draw's uniform and this thread's run
  // of tile statistics, held in registers when the run is at most kRun tiles (V up to
  // kRun x 256 x 128 tokens; longer runs take the loops below).
  const float uu = a.u[size_t(b) * a.G1 + k];
  constexpr int kRun = 8;
  const bool regs = per <= kRun;
  float tm[kRun];
  double ts[kRun];
  if (regs) {
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      const int t = min(t0 + i, nt - 1);
      tm[i] = tmax[t];
      ts[i] = tsum[t];
    }
  }
  asm volatile("" ::: "memory");  // keep the uniform's load here, ahead of its use
  __builtin_amdgcn_sched_barrier(0);
  // row maximum
  float m = -INFINITY;
  if (regs) {
#pragma unroll
    for (int i = 0; i < kRun; ++i)
      if (t0 + i < t1) m = fmaxf(m, tm[i]);
  } else {
    for (int t = t0; t < t1; ++t) m = fmaxf(m, tmax[t]);
  }
  m = wave_max(m);
  if (lane == 0) smax[wave] = m;
  __syncthreads();
  float M = smax[0];
  for (int w = 1; w < kSampleThreads / kWave; ++w) M = fmaxf(M, smax[w]);
  // this thread's run of tile masses, then a scan over threads (tile order).  Thread i
  // owns [off + excl_i, off + inc_i); the next thread's lower end is the same value moved
  // one lane up, so the runs tile [0, S) without gaps or overlaps.
  double part = 0.0;
  if (regs) {
#pragma unroll
    for (int i = 0; i < kRun; ++i)
      if (t0 + i < t1) part += ts[i] * ex(tm[i], M);
  } else {
    for (int t = t0; t < t1; ++t) part += tsum[t] * ex(tmax[t], M);
  }
  const double inc = wave_inclusive(part, 0.0, [](double x, double y) { return x + y; });
  const double excl = dpp_move<kDppWaveShr1, 0xf>(0.0, inc);
  if (lane == kWave - 1) sc[wave] = inc;
  __syncthreads();
  double off = 0.0;
  for (int w = 0; w < wave; ++w) off += sc[w];
  double S = 0.0;
  for (int w = 0; w < kSampleThreads / kWave; ++w) S += sc[w];
  const double before = off + excl, upper = off + inc;
  const double target = double(uu) * S;
  if (tid == 0) {
    s_tile = nt - 1;  // rounding can leave u * S at or past the last edge: the last tile
    s_before = -1.0;
    s_S = S;
  }
  __syncthreads();
  if (t1 > t0 && before <= target && target < upper) {
    double c = before;
    int t = t0;
    if (regs) {
#pragma unroll
      for (int i = 0; i < kRun; ++i) {
        if (t0 + i >= t1 - 1) break;
        const double mt = ts[i] * ex(tm[i], M);
        if (target < c + mt) break;
        c += mt;
        ++t;
      }
    } else {
      for (; t < t1 - 1; ++t) {
        const double mt = tsum[t] * ex(tmax[t], M);
        if (target < c + mt) break;
        c += mt;
      }
    }
    s_tile = t;
    s_before = c;
  }
  __syncthreads();
  if (wave != 0) return;
  // rescan the tile: lane j takes its kLaneTok consecutive tokens
  const int t = s_tile;
  const T* O = static_cast<const T*>(a.out);
  const size_t base = (size_t(b) * a.G1 + k) * a.V;
  const int v = t * kTileV + kLaneTok * lane;
  double e[kLaneTok];
  double own = 0.0;
#pragma unroll
  for (int i = 0; i < kLaneTok; ++i) {
    e[i] = v + i < a.V ? ex(Out<T>::load(O, base + v + i), M) : 0.0;
    own += e[i];
  }
  double c0;
  if (s_before >= 0.0) {
    c0 = s_before;
  } else {
    // the last tile after a rounding overshoot: its start is S minus its own mass
    c0 = S - tsum[t] * ex(tmax[t], M);
  }
  const double pinc = wave_inclusive(own, 0.0, [](double x, double y) { return x + y; });
  // cumulative mass through each of this lane's tokens, in token order
  double cum = c0 + (pinc - own);
  int cand = a.V;                                 // smallest token whose cumulative passes
#pragma unroll
  for (int i = 0; i < kLaneTok; ++i) {
    cum += e[i];
    if (cand == a.V && v + i < a.V && cum > target) cand = v + i;
  }
  cand = lane63(wave_inclusive(cand, int(a.V), [](int x, int y) { return min(x, y); }));
  bool in_tile = true;
  if (cand == a.V) {
    // nothing in the tile passes: past the last edge (u * S >= S after rounding) the inverse
    // CDF clamps to the last token; otherwise the tile's recomputed mass fell short of its
    // summary by a rounding step, and its last token is the edge within that rounding
    cand = s_before >= 0.0 ? min(a.V - 1, t * kTileV + kTileV - 1) : a.V - 1;
    in_tile = cand >= t * kTileV && cand < t * kTileV + kTileV;
  }
  if (lane == 0) a.tokens[size_t(b) * a.G1 + k] = cand;
  if (a.p_at) {
    // p(token) from the rescan's own weight of it (the same expression), when it has one
    const int rel = cand - t * kTileV;
    if (in_tile && lane == rel / kLaneTok) {
      double et = e[0];
#pragma unroll
      for (int i = 1; i < kLaneTok; ++i)
        if (rel % kLaneTok == i) et = e[i];
      a.p_at[size_t(b) * a.G1 + k] = float(et / s_S);
    } else if (!in_tile && lane == 0) {
      a.p_at[size_t(b) * a.G1 + k] = float(ex(Out<T>::load(O, base + cand), M) / s_S);
    }
  }
  if (k + 1 < a.G1) {
    if (a.r == 256) stage_row<256>(a, l, b, cand, lane);
    else if (a.r == 128) stage_row<128>(a, l, b, cand, lane);
    else stage_row<64>(a, l, b, cand, lane);
  }
}

template <typename T, int R>
hipError_t launch_markov_typed(const MarkovArgs& a, hipStream_t stream) {
  const MkLayout l = mk_layout(a.B, a.V);
  hipLaunchKernelGGL(markov_stage_kernel<R>, dim3((a.B + 3) / 4), dim3(256), 0, stream, a, l);
  for (int k = 0; k < a.G1; ++k) {
    if (a.vec_ok)
      hipLaunchKernelGGL((markov_logits_kernel<T, R, true>), dim3(l.ntiles), dim3(kMkThreads), 0, stream, a,
                         l, k, kExp2Taylor);
    else
      hipLaunchKernelGGL((markov_logits_kernel<T, R, false>), dim3(l.ntiles), dim3(kMkThreads), 0, stream, a,
                         l, k, kExp2Taylor);
    hipLaunchKernelGGL((markov_sample_kernel<T>), dim3(a.B), dim3(kSampleThreads), 0, stream, a, l, k,
                       kExp2Taylor);
  }
  return hipGetLastError();
}

}  // namespace

size_t markov_workspace_bytes(int B, int V) { return mk_layout(B, V).total; }

hipError_t launch_markov(const MarkovArgs& a, int dtype, hipStream_t stream) {
  if (dtype == RVA_BF16) {
    if (a.r == 256) return launch_markov_typed<uint16_t, 256>(a, stream);
    if (a.r == 128) return launch_markov_typed<uint16_t, 128>(a, stream);
    return launch_markov_typed<uint16_t, 64>(a, stream);
  }
  if (a.r == 256) return launch_markov_typed<float, 256>(a, stream);
  if (a.r == 128) return launch_markov_typed<float, 128>(a, stream);
  return launch_markov_typed<float, 64>(a, stream);
}

}  // namespace rva
