// Stages 4 and 5 in one pass over the logits: full-vocabulary speculative-sampling acceptance,
// the residual / bonus draw, the commit, and the TV-distance confidence labels.
//
// Sources: "DSpark：投机解码与生产级 Serving 学习笔记" (sorenprojections.com) section 02
// (the acceptance rule keeps the target distribution; acceptance is prefix-only) and
// section 07 (label c* = 1 - 0.5 ||p_d - p_t||_1); "DFlash 到 DSpark in SGLang" section
// "Background" (each verify forward also yields one target token).
//
// Work split.  An ITEM is one packed target row r < M (M = cu[B]): for a row that is not the
// last of its request's window it is the PAIR (target row r, draft row of the same position),
// otherwise the target row alone (the bonus row).  A row is cut into segments of 32 KB
// (16384 bf16 / 8192 float32 entries) and a UNIT is one segment of an item: one workgroup of
// 512 threads holds it in registers (4 x 16 B per thread and row) from its HBM read to the
// end, so every logit is read from HBM once.
//
// The segments of one item form a TEAM.  After reading its unit, a workgroup posts the
// segment statistics (max and float64 sum of exp(x - max), per row) and waits for the rest of
// its team; every member then combines the same posted values in the same order, so all
// of them hold identical row normalisers and take identical decisions.  Then, from the
// registers:
//   * the accept test of the pair's drafted token, u < min(1, p_t(x) / p_d(x)), in float64;
//   * the segment's share of the label, sum min(p_t, p_d) = 1 - TV;
//   * for the units that may carry the draw -- a pair whose own test rejects (it is the draw
//     row when every earlier draft was accepted), or the bonus row of the window -- the
//     float64 segment sums of the draw: S_t, S_d (exact normalisers), the unnormalised
//     residual A(rho') = sum max(0, e_t - rho' e_d) and the draft mass D it keeps, at
//     rho' = S_t / S_d of the float32-accurate normalisers (e = exp(x - max)).
// The last workgroup of a request to finish (per-request counter) decides: accept length
// from the posted test results, the residual or bonus draw, the segment holding u * Q (the
// residual masses corrected to the exact rho to first order, A(rho) = A(rho') - (rho - rho')
// D, exact but for entries whose sign differs between rho' and rho), then one exact float64
// rescan of that segment (a re-read of 32 or 64 KB) and the commit; it also sums the label
// shares.
//
// Exchange.  Every posted value is a 64-bit word (tag << 32 | payload), written and read with
// relaxed agent-scope atomics, so a word is valid exactly when it carries this call's tag:
// no counters guard the data, no fences, nothing to reset.  The tag is epoch + 1, the epoch
// word of the workspace advanced by the last workgroup of the call (counters per 64
// workgroups, then per call); the workspace must be zero before its first use with a shape.
// Waits only ever point at units that are read before the waiter's own (same team, earlier
// dispatch): posts never wait.  A wait gives up after 20 ms (RVA_DEV_TIMEOUT), so a kernel
// always ends.
//
// Dispatch order.  Workgroups i, i+8, i+16, ... run on one XCD; an item's units take
// consecutive places in one XCD's order (item k -> XCD k mod 8), so a team is dispatched
// together and its exchange stays local.
//
// The draw returns an index that has to agree with a float64 definition, so everything it
// reads is float64: exp is 2^y by range reduction, a 256-entry table of 2^(j/256) and a
// degree-4 Taylor polynomial of 2^f on |f| <= 1/512 (about 1.5 ulp); the table itself and the
// few other float64 exponentials use a degree-13 polynomial on |f| <= 1/2.
#include <type_traits>

#include "exp2_f64.h"
#include "rva_common.h"

namespace rva {
namespace {

constexpr int kNT = 512;                    // threads per workgroup
constexpr int kWaves = kNT / kWave;
constexpr int kVec = 4;                     // 16-byte vectors per thread and row
constexpr int kSegBytes = kNT * kVec * 16;  // one row's part of a unit: 32 KB
constexpr int kLanes = 8;                   // workgroups i, i + 8, ... share an XCD
constexpr int kChunk = 8 * kLanes;          // workgroups per completion counter
constexpr int kStatWords = 6;               // m_t, S_t (hi, lo), m_d, S_d (hi, lo)
constexpr int kDrawWords = 10;              // S_t, S_d, A, D, rho' in float64 (hi, lo)
constexpr float kLog2e = 1.44269504088896341f;
constexpr unsigned long long kWaitTicks = 2000000ull;  // 20 ms at the 100 MHz constant clock

__device__ __forceinline__ float exp_shift(float x, float m) {
  return __builtin_amdgcn_exp2f((x - m) * kLog2e);
}

// ------------------------------------------------------------------ tagged words
__device__ __forceinline__ void put(uint64_t* p, uint32_t tag, uint32_t v) {
  __hip_atomic_store(p, (uint64_t(tag) << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_f64(uint64_t* p, uint32_t tag, double d) {
  put(p, tag, uint32_t(__double2hiint(d)));
  put(p + 1, tag, uint32_t(__double2loint(d)));
}
__device__ __forceinline__ uint64_t get(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float payload_f32(uint64_t w) { return __uint_as_float(uint32_t(w)); }
__device__ __forceinline__ double payload_f64(uint64_t hi, uint64_t lo) {
  return __hiloint2double(int(uint32_t(hi)), int(uint32_t(lo)));
}

// values that are the same in every lane (read back from LDS) live in scalar registers
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return uint32_t(__builtin_amdgcn_readfirstlane(int(v))); }
__device__ __forceinline__ float uni(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }
__device__ __forceinline__ double uni(double v) {
  return __hiloint2double(__builtin_amdgcn_readfirstlane(__double2hiint(v)),
                          __builtin_amdgcn_readfirstlane(__double2loint(v)));
}

// ------------------------------------------------------------------ workspace
struct Control {
  uint32_t epoch;   // tags of the current call are epoch + 1
  uint32_t done;    // completed counter chunks of the current call
  uint32_t giveup;  // set when a wait timed out: later waits return at once
};

struct WsLayout {
  int nseg, n_chunks;
  size_t off_ctl, off_req, off_chunk, off_stat, off_bit, off_share, off_draw, total;
};

__host__ __device__ inline int seg_len_entries(int elem_bytes) { return kSegBytes / elem_bytes; }

__host__ __device__ inline WsLayout ws_layout(int B, int gamma, int V, int max_rows, int elem_bytes) {
  (void)gamma;
  WsLayout w;
  const int len = seg_len_entries(elem_bytes);
  w.nseg = (V + len - 1) / len;
  const long long grid = (long long)kLanes * w.nseg * ((max_rows + kLanes - 1) / kLanes);
  w.n_chunks = int((grid + kChunk - 1) / kChunk);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  w.off_ctl = take(sizeof(Control));
  w.off_req = take(sizeof(uint32_t) * size_t(B));
  w.off_chunk = take(sizeof(uint32_t) * size_t(w.n_chunks));
  w.off_stat = take(sizeof(uint64_t) * size_t(max_rows) * w.nseg * kStatWords);
  w.off_bit = take(sizeof(uint64_t) * size_t(max_rows));
  w.off_share = take(sizeof(uint64_t) * size_t(max_rows) * w.nseg);
  w.off_draw = take(sizeof(uint64_t) * size_t(max_rows) * w.nseg * kDrawWords);
  w.total = off;
  return w;
}

struct Ctx {
  AcceptArgs a;
  Exp2Poly P;
  WsLayout L;
  Control* ctl;
  uint32_t* req_cnt;   // [B] workgroups of the request that have finished
  uint32_t* chunk;     // [n_chunks] workgroups of the chunk that have finished
  uint64_t* stat;      // [max_rows][nseg][kStatWords]
  uint64_t* bit;       // [max_rows]: the pair's accept test (1 = rejected)
  uint64_t* share;     // [max_rows][nseg]: label share (float32 payload)
  uint64_t* draw;      // [max_rows][nseg][kDrawWords]
  int commit;          // 0: labels only
};

// ------------------------------------------------------------------ a thread's share of a unit
template <typename T>
struct Seg {
  static constexpr int kEpv = 16 / int(sizeof(T));    // entries per vector: 8 bf16, 4 float32
  static constexpr int kLen = kSegBytes / int(sizeof(T));
  static constexpr int kPer = kVec * kEpv;            // entries per thread
  uint4 v[kVec];

  __device__ __forceinline__ static uint32_t comp(const uint4& q, int k) {
    return k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w;
  }
  // entry e (< kEpv) of vector i; the thread's vector i holds segment entries
  // (i * kNT + threadIdx.x) * kEpv + e
  __device__ __forceinline__ float at(int i, int e) const {
    if constexpr (std::is_same<T, uint16_t>::value) {
      const uint32_t w = comp(v[i], e >> 1);
      return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    } else {
      return __uint_as_float(comp(v[i], e));
    }
  }
  __device__ __forceinline__ static int index(int seg, int i, int e) {
    return seg * kLen + (i * kNT + int(threadIdx.x)) * kEpv + e;
  }
  // entries past the row end read as -inf
  __device__ __forceinline__ void load(const T* row, int V, int seg, bool vec_ok) {
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      const int base = index(seg, i, 0);
      if (vec_ok && base + kEpv <= V) {
        v[i] = *reinterpret_cast<const uint4*>(row + base);
      } else {
        uint32_t w[4];
        if constexpr (std::is_same<T, uint16_t>::value) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t lo = base + 2 * k < V ? row[base + 2 * k] : 0xff80u;
            const uint32_t hi = base + 2 * k + 1 < V ? row[base + 2 * k + 1] : 0xff80u;
            w[k] = lo | (hi << 16);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) w[k] = base + k < V ? __float_as_uint(row[base + k]) : 0xff800000u;
        }
        v[i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
  // keeps the widened values from being held across phases (they are one instruction each)
  __device__ __forceinline__ void touch() {
#pragma unroll
    for (int i = 0; i < kVec; ++i) touch(i);
  }
  __device__ __forceinline__ void touch(int i) {
    asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
  }
};

// ------------------------------------------------------------------ block reductions
struct Shared {
  float f[kWaves];
  double d[kWaves][5];
  double tab[256];
  // item description and decisions, broadcast by wave 0
  int M, b, r0, w, cap, item_ok, last;
  float Mt, Md;
  double St, Sd;
  float it, id;  // 1 / S in float32 (labels)
  int reject;
  // pick
  double t, base, rho;
  int seg, residual, n, n_full, y, ylast;
};

__device__ __forceinline__ float block_max(float v, Shared& sh) {
  v = wave_max(v);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __syncthreads();
  if (lane == 0) sh.f[wave] = v;
  __syncthreads();
  float r = sh.f[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, sh.f[i]);
  return r;
}

// float64 sums of N values in a fixed order (wave butterfly, then the wave totals in order);
// every thread gets the results
template <int N>
__device__ __forceinline__ void block_sums(double (&v)[N], Shared& sh) {
  static_assert(N <= 5, "");
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = wave_sum_f64(v[q]);
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int q = 0; q < N; ++q) sh.d[wave][q] = v[q];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < N; ++q) {
    double r = sh.d[0][q];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r += sh.d[i][q];
    v[q] = r;
  }
}

// max and float64 sum of exp(x - max) of a thread-distributed segment (float32 exponentials
// in runs of 8, float64 accumulation)
template <typename T>
__device__ __forceinline__ void seg_stats(Seg<T>& s, Shared& sh, float& m, double& S) {
  float mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
#pragma unroll
    for (int e = 0; e < Seg<T>::kEpv; ++e) mt = fmaxf(mt, s.at(i, e));
    s.touch(i);
  }
  m = block_max(mt, sh);
  const float ms = m == -INFINITY ? 0.f : m;  // fully masked segment: every term is 0
  double acc = 0.0;
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
#pragma unroll
    for (int e = 0; e < Seg<T>::kEpv; ++e) {
      run += exp_shift(s.at(i, e), ms);
      if (((i * Seg<T>::kEpv + e) & 7) == 7) {
        acc += double(run);
        run = 0.f;
      }
    }
    s.touch(i);
  }
  double v[1] = {acc};
  block_sums<1>(v, sh);
  S = v[0];
}

// ------------------------------------------------------------------ waiting for words
// Each lane with `mine` waits until its word carries the tag; one wave calls this (wave-uniform
// loop, no barrier inside).  Gives up after kWaitTicks (sets giveup and RVA_DEV_TIMEOUT).
__device__ __forceinline__ uint64_t wait_word(Control* ctl, int32_t* status, uint32_t tag,
                                              const uint64_t* p, bool mine) {
  uint64_t w = mine ? get(p) : 0;
  if (__all(!mine || uint32_t(w >> 32) == tag)) return w;
  const unsigned long long t0 = wall_clock64();
  while (__any(mine && uint32_t(w >> 32) != tag)) {
    if (__hip_atomic_load(&ctl->giveup, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
    if (wall_clock64() - t0 > kWaitTicks) {
      if ((threadIdx.x % kWave) == 0) {
        atomicOr(&ctl->giveup, 1u);
        flag(status, RVA_DEV_TIMEOUT);
      }
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    if (mine && uint32_t(w >> 32) != tag) w = get(p);
  }
  return w;
}

// Row normalisers of an item from its team's posted statistics (wave 0; every lane gets them).
// The order of combination is fixed, so every caller obtains the same bits.
__device__ __forceinline__ void team_normalisers(Control* ctl, int32_t* status, const Exp2Poly& P,
                                                 const uint64_t* stat, int nseg, uint32_t tag,
                                                 int item, bool pair, float& Mt, double& St,
                                                 float& Md, double& Sd) {
  const int lane = threadIdx.x % kWave;
  const uint64_t* base = stat + size_t(item) * nseg * kStatWords;
  const int nw = pair ? kStatWords : 3;
  // wait until every word is there (lanes over words, 64 at a time)
  for (int k0 = 0; k0 < nseg * kStatWords; k0 += kWave) {
    const int k = k0 + lane;
    const bool mine = k < nseg * kStatWords && (k % kStatWords) < nw;
    wait_word(ctl, status, tag, base + k, mine);
  }
  float mt = -INFINITY, md = -INFINITY;
  for (int s = lane; s < nseg; s += kWave) {
    mt = fmaxf(mt, payload_f32(get(base + s * kStatWords)));
    if (pair) md = fmaxf(md, payload_f32(get(base + s * kStatWords + 3)));
  }
  Mt = wave_max(mt);
  Md = wave_max(md);
  double at = 0.0, ad = 0.0;
  for (int s = lane; s < nseg; s += kWave) {
    const uint64_t* q = base + s * kStatWords;
    at += payload_f64(get(q + 1), get(q + 2)) * exp_shift_f64(P, payload_f32(get(q)), Mt);
    if (pair) ad += payload_f64(get(q + 4), get(q + 5)) * exp_shift_f64(P, payload_f32(get(q + 3)), Md);
  }
  St = wave_sum_f64(at);
  Sd = wave_sum_f64(ad);
}

// wave-parallel search of the request holding packed row r: the largest b with cu[b] <= r
// (cu non-decreasing); every lane gets it
__device__ __forceinline__ int find_request(const int32_t* cu, int B, int r) {
  const int lane = threadIdx.x % kWave;
  int lo = 0, n = B;
  while (n > 1) {
    const int step = (n - 1 + kWave - 1) / kWave;
    const int k = lo + 1 + lane * step;
    const bool le = k < lo + n && cu[k] <= r;
    const int cnt = __popcll(__ballot(le));
    if (cnt == 0) {
      n = 1;
    } else {
      const int nlo = lo + 1 + (cnt - 1) * step;
      n = min(step, lo + n - nlo);
      lo = nlo;
    }
  }
  return lo;
}

// One wave: the first of n items (masses >= 0, in index order) at which the running sum,
// started at `start`, passes t; `base` = the running sum before it.  If rounding leaves t
// unpassed, the last item with mass (or item 0).
template <typename F>
__device__ __forceinline__ void locate(double t, double start, int n, F mass, int& found, double& base) {
  const int lane = threadIdx.x % kWave;
  int last = 0;
  double base_last = start, carry = start;
  found = -1;
  base = start;
  for (int i0 = 0; i0 < n && found < 0; i0 += kWave) {
    const int i = i0 + lane;
    const double m = i < n ? mass(i) : 0.0;
    double inc = m;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double x = __shfl_up(inc, o);
      if (lane >= o) inc += x;
    }
    inc += carry;
    const double exc = inc - m;
    const unsigned long long hit = __ballot(m > 0.0 && inc > t);
    const unsigned long long pos = __ballot(m > 0.0);
    if (pos) {
      const int l = 63 - __clzll(pos);
      last = i0 + l;
      base_last = __shfl(exc, l);
    }
    if (hit) {
      const int l = __ffsll(hit) - 1;
      found = i0 + l;
      base = __shfl(exc, l);
    }
    carry = __shfl(inc, kWave - 1);
  }
  if (found < 0) {
    found = last;
    base = base_last;
  }
}

// ------------------------------------------------------------------ the pick (last arriver)
// What the pick needs, staged in LDS by the workgroup that runs it (the pick is a separate,
// not inlined function, so that its registers do not weigh on the streaming path).
struct PickCtx {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* u_res;
  int32_t* committed;
  int32_t* accept_len;
  int32_t* context_lens;
  int32_t* accept_len_full;
  float* pt_at;
  float* pd_at;
  float* labels;
  int32_t* status;
  const uint64_t* stat;
  const uint64_t* bit;
  const uint64_t* share;
  const uint64_t* draw;
  Control* ctl;
  int V, gamma, nseg, commit;
  uint32_t tag;
  int b, r0, w, cap;
};
__constant__ Exp2Poly kPickPoly = kExp2Taylor;

// Decision, draw and commit of request pc.b, and its labels; the whole workgroup.
template <typename T>
__device__ __attribute__((noinline)) void pick(const PickCtx& pc, Shared& sh) {
  Seg<T> xt, xd;
  const PickCtx& a = pc;
  const Exp2Poly& P = kPickPoly;
  const uint32_t tag = pc.tag;
  const int b = pc.b, r0 = pc.r0, w = pc.w, cap = pc.cap;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int G1 = a.gamma - 1, nseg = pc.nseg;
  const float qnan = __int_as_float(0x7fc00000);
  // labels: wave k sums the shares of draft k (fixed order: lanes over segments, butterfly)
  if (a.labels) {
    for (int k = wave; k < G1; k += kWaves) {
      double ov = 0.0;
      if (k < w - 1) {
        const uint64_t* q = pc.share + size_t(r0 + k) * nseg;
        for (int s0 = 0; s0 < nseg; s0 += kWave) {
          const int s = s0 + lane;
          const uint64_t wd = wait_word(pc.ctl, pc.status, tag, q + s, s < nseg);
          if (s < nseg) ov += double(payload_f32(wd));
        }
        ov = wave_sum_f64(ov);
      }
      if (lane == 0) a.labels[size_t(b) * G1 + k] = k < w - 1 ? float(ov) : qnan;
    }
  }
  if (!pc.commit) return;
  if (tid >= w - 1 && tid < G1) {  // positions past the window
    if (a.pt_at) a.pt_at[size_t(b) * G1 + tid] = qnan;
    if (a.pd_at) a.pd_at[size_t(b) * G1 + tid] = qnan;
  }
  // decision: the first rejected draft (test results posted by the pairs' teams)
  if (wave == 0) {
    const bool mine = lane < w - 1;
    const uint64_t wd = wait_word(pc.ctl, pc.status, tag, pc.bit + r0 + lane, mine);
    const unsigned long long rej = __ballot(mine && (uint32_t(wd) & 1u));
    const int n_full = rej ? __ffsll(rej) - 1 : w - 1;
    const bool residual = n_full < cap - 1;
    const int n = residual ? n_full : cap - 1;
    // the draw's segment sums (lanes over segments)
    const int item = r0 + n;
    const uint64_t* dq = pc.draw + size_t(item) * nseg * kDrawWords;
    for (int k0 = 0; k0 < nseg * kDrawWords; k0 += kWave) {
      const int k = k0 + lane;
      wait_word(pc.ctl, pc.status, tag, dq + k, k < nseg * kDrawWords && (residual || (k % kDrawWords) < 2));
    }
    auto dval = [&](int s, int q) { return payload_f64(get(dq + s * kDrawWords + 2 * q), get(dq + s * kDrawWords + 2 * q + 1)); };
    double st = 0.0, sd = 0.0;
    for (int s = lane; s < nseg; s += kWave) {
      st += dval(s, 0);
      if (residual) sd += dval(s, 1);
    }
    st = wave_sum_f64(st);
    sd = wave_sum_f64(sd);
    const double rho = residual ? st / sd : 0.0;
    const double drho = residual ? rho - dval(0, 4) : 0.0;
    bool res = residual;
    auto mass = [&](int s) {
      if (!res) return dval(s, 0);
      const double m = dval(s, 2) - drho * dval(s, 3);
      return m > 0.0 ? m : 0.0;
    };
    double q = 0.0;
    for (int s = lane; s < nseg; s += kWave) q += mass(s);
    double Q = wave_sum_f64(q);
    if (res && !(Q > 0.0)) {  // residual identically zero: draw from p_t of that row instead
      res = false;
      Q = st;
    }
    const double t = double(a.u_res[b]) * Q;
    int seg = 0;
    double base = 0.0;
    locate(t, 0.0, nseg, mass, seg, base);
    if (lane == 0) {
      sh.n = n;
      sh.n_full = n_full;
      sh.residual = res;
      sh.rho = rho;
      sh.t = t;
      sh.base = base;
      sh.seg = seg;
      sh.y = 0x7fffffff;
      sh.ylast = -1;
      sh.Mt = 0.f;
      sh.Md = 0.f;
    }
  }
  __syncthreads();
  const int n = sh.n, seg = sh.seg;
  const bool res = sh.residual;
  const int item = r0 + n;
  // the maxima the candidate units used for e_t, e_d: the item's team normalisers
  if (wave == 0) {
    float Mt, Md;
    double St, Sd;
    team_normalisers(pc.ctl, pc.status, P, pc.stat, nseg, tag, item, res, Mt, St, Md, Sd);
    if (lane == 0) {
      sh.Mt = Mt;
      sh.Md = Md;
    }
  }
  fill_exp2_tab(P, sh.tab);  // ends with a barrier: sh.Mt / sh.Md visible
  const T* trow = static_cast<const T*>(a.target) + size_t(item) * a.V;
  const T* drow = static_cast<const T*>(a.draft) + size_t(b * G1 + n) * a.V;
  const bool vec_ok = a.V % Seg<T>::kEpv == 0;
  xt.load(trow, a.V, seg, vec_ok);
  if (res) xd.load(drow, a.V, seg, vec_ok);
  const float Mt = sh.Mt, Md = sh.Md;
  const double rho = sh.rho;
  // exact weights in index order: vector group i covers entries [i kNT kEpv, (i+1) kNT kEpv)
  // of the segment with thread t holding kEpv consecutive ones
  double running = sh.base;
  // the weights are formed twice (thread sum, then the running sum), so that none is held
  auto weight = [&](int i, int e) {
    double x = exp_shift_tab(P, sh.tab, xt.at(i, e), Mt);
    if (res) {
      x -= rho * exp_shift_tab(P, sh.tab, xd.at(i, e), Md);
      x = x > 0.0 ? x : 0.0;
    }
    return x;
  };
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    double tsum = 0.0;
#pragma unroll
    for (int e = 0; e < Seg<T>::kEpv; ++e) tsum += weight(i, e);
    // inclusive prefix of the thread sums over the workgroup
    double inc = tsum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    __syncthreads();
    if (lane == kWave - 1) sh.d[wave][0] = inc;
    __syncthreads();
    double before = running;
    for (int k = 0; k < wave; ++k) before += sh.d[k][0];
    double total = 0.0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) total += sh.d[k][0];
    double cum = before + (inc - tsum);  // running sum before this thread's entries
    int hit = 0x7fffffff, lastpos = -1;
#pragma unroll
    for (int e = 0; e < Seg<T>::kEpv; ++e) {
      const double wv = weight(i, e);
      cum += wv;
      const int v = Seg<T>::index(seg, i, e);
      if (wv > 0.0) {
        lastpos = v;
        if (hit == 0x7fffffff && cum > sh.t) hit = v;
      }
    }
    // the first hit in index order (thread order within the group), the last positive entry
    const unsigned long long hb = __ballot(hit != 0x7fffffff), pb = __ballot(lastpos >= 0);
    if (hb && lane == __ffsll(hb) - 1) atomicMin(&sh.y, hit);
    if (pb && lane == 63 - __clzll(pb)) atomicMax(&sh.ylast, lastpos);
    running += total;
  }
  __syncthreads();
  const int y = sh.y != 0x7fffffff ? sh.y : (sh.ylast >= 0 ? sh.ylast : seg * Seg<T>::kLen);
  if (tid < a.gamma) {
    const int tok = tid < n ? a.tokens[size_t(b) * G1 + tid] : 0;
    a.committed[size_t(b) * a.gamma + tid] = tid < n ? tok : (tid == n ? y : -1);
  }
  if (tid == 0) {
    a.accept_len[b] = n;
    a.context_lens[b] = a.context_lens[b] + n + 1;
    if (a.accept_len_full) a.accept_len_full[b] = sh.n_full;
  }
}

// ------------------------------------------------------------------ the kernel
// Units of lane x (workgroups x, x + 8, ...): items x, x + 8, x + 16, ..., nseg units each.
__device__ __forceinline__ int lane_units(int x, int M, int nseg) {
  return x < M ? ((M - x + kLanes - 1) / kLanes) * nseg : 0;
}

template <typename T>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(6, 6))) void accept_kernel(Ctx c) {
  __shared__ Shared sh;
  const AcceptArgs& a = c.a;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int nseg = c.L.nseg, G1 = a.gamma - 1;
  const int bid = blockIdx.x, x = bid % kLanes, q = bid / kLanes;
  const int item = (q / nseg) * kLanes + x, seg = q % nseg;
  if (item >= a.max_rows) return;  // grid padding (never counted)
  const uint32_t epoch = uni(__hip_atomic_load(&c.ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const uint32_t tag = epoch + 1u == 0u ? 1u : epoch + 1u;

  // ---- which request, which position (wave 0)
  if (wave == 0) {
    const int M = a.cu[a.B];
    int b = 0, r0 = 0, w = 0, cap = 0, ok = 0;
    if (item < M) {
      b = find_request(a.cu, a.B, item);
      r0 = a.cu[b];
      w = a.cu[b + 1] - r0;
      ok = r0 >= 0 && w >= 1 && w <= a.gamma && r0 + w <= a.max_rows && item >= r0 && item < r0 + w;
      cap = w;
      if (ok && c.commit && a.cap) {
        cap = a.cap[b];
        if (cap < 1 || cap > w) {
          if (lane == 0 && seg == 0 && item == r0) flag(a.status, RVA_DEV_BAD_WINDOW);
          cap = cap < 1 ? 1 : w;
        }
      }
      if (!ok && lane == 0 && seg == 0) flag(a.status, RVA_DEV_BAD_WINDOW);
    }
    if (lane == 0) {
      sh.M = M;
      sh.b = b;
      sh.r0 = r0;
      sh.w = w;
      sh.cap = cap;
      sh.item_ok = ok;
    }
  }
  __syncthreads();
  const int M = min(max(uni(sh.M), 0), a.max_rows);
  if (item >= M) return;  // no such row this call (not counted: the chunk targets follow M)
  const int b = uni(sh.b), r0 = uni(sh.r0), w = uni(sh.w), cap = uni(sh.cap);
  const bool ok = uni(sh.item_ok) != 0;
  const int j = item - r0;
  const bool pair = ok && j < w - 1;
  Seg<T> xt, xd;
  if (ok) {
    const bool vec_ok = a.V % Seg<T>::kEpv == 0;
    const T* trow = static_cast<const T*>(a.target) + size_t(item) * a.V;
    const T* drow = static_cast<const T*>(a.draft) + size_t(b * G1 + j) * a.V;
    xt.load(trow, a.V, seg, vec_ok);
    if (pair) xd.load(drow, a.V, seg, vec_ok);
    // the drafted token, its uniform and its two logits (wave 0, lane 0)
    float lt = 0.f, ld = 0.f, u = 0.f;
    if (pair && c.commit && wave == 0 && lane == 0) {
      int xtok = a.tokens[size_t(b) * G1 + j];
      u = a.u_acc[size_t(b) * G1 + j];
      if (xtok < 0 || xtok >= a.V) {
        if (seg == 0) flag(a.status, RVA_DEV_BAD_TOKEN);
        xtok = xtok < 0 ? 0 : a.V - 1;
      }
      lt = Elem<T>::load(trow, xtok);
      ld = Elem<T>::load(drow, xtok);
    }
    // ---- segment statistics, posted for the team
    float mt, md = -INFINITY;
    double St, Sd = 0.0;
    seg_stats(xt, sh, mt, St);
    if (pair) seg_stats(xd, sh, md, Sd);
    uint64_t* sw = c.stat + (size_t(item) * nseg + seg) * kStatWords;
    if (tid == 0) {
      put(sw, tag, __float_as_uint(mt));
      put_f64(sw + 1, tag, St);
      if (pair) {
        put(sw + 3, tag, __float_as_uint(md));
        put_f64(sw + 4, tag, Sd);
      }
    }
    // ---- the team's normalisers, the accept test (wave 0)
    if (wave == 0) {
      float Mt, Md;
      double St_, Sd_;
      team_normalisers(c.ctl, a.status, c.P, c.stat, nseg, tag, item, pair, Mt, St_, Md, Sd_);
      int reject = 0;
      if (pair && c.commit && lane == 0) {
        const double pt = exp_shift_f64(c.P, lt, Mt) / St_;
        const double pd = exp_shift_f64(c.P, ld, Md) / Sd_;
        const double r = pd == 0.0 ? INFINITY : pt / pd;
        reject = !(double(u) < (r < 1.0 ? r : 1.0));
        if (seg == 0) {
          if (a.pt_at) a.pt_at[size_t(b) * G1 + j] = float(pt);
          if (a.pd_at) a.pd_at[size_t(b) * G1 + j] = float(pd);
          put(c.bit + item, tag, uint32_t(reject));
        }
      }
      if (lane == 0) {
        sh.Mt = Mt;
        sh.Md = Md;
        sh.St = St_;
        sh.Sd = Sd_;
        sh.it = float(1.0 / St_);
        sh.id = pair ? float(1.0 / Sd_) : 0.f;
        sh.reject = reject;
      }
    }
    __syncthreads();
    // ---- the label share: sum min(p_t, p_d) over the segment = 2^min(l_t, l_d), with
    // l = x log2 e + c, c = -(M log2 e + log2 S): one FMA per entry, one exponential per
    // entry pair (forming l from x log2 e instead of (x - M) log2 e moves it by a few float32
    // ulp of |x log2 e|, about 1e-6 relative per term)
    if (pair && a.labels) {
      const float ct = uni(-fmaf(sh.Mt, kLog2e, -__log2f(sh.it)));
      const float cd = uni(-fmaf(sh.Md, kLog2e, -__log2f(sh.id)));
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        float run = 0.f;
#pragma unroll
        for (int e = 0; e < Seg<T>::kEpv; ++e)
          run += __builtin_amdgcn_exp2f(fminf(fmaf(xt.at(i, e), kLog2e, ct), fmaf(xd.at(i, e), kLog2e, cd)));
        acc += double(run);
        xt.touch(i);
        xd.touch(i);
      }
      double v[1] = {acc};
      block_sums<1>(v, sh);
      if (tid == 0) put(c.share + size_t(item) * nseg + seg, tag, __float_as_uint(float(v[0])));
    }
    // ---- the draw's segment sums, for the units that may carry it
    const bool residual_cand = c.commit && pair && j < cap - 1 && uni(sh.reject);
    const bool bonus_cand = c.commit && j == cap - 1;
    if (residual_cand || bonus_cand) {
      fill_exp2_tab(c.P, sh.tab);
      const float Mt = uni(sh.Mt), Md = uni(sh.Md);
      const double rho1 = residual_cand ? uni(sh.St) / uni(sh.Sd) : 0.0;
      double v[4] = {0.0, 0.0, 0.0, 0.0};  // S_t, S_d, A(rho'), D
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        xt.touch(i);
        xd.touch(i);
#pragma unroll
        for (int e = 0; e < Seg<T>::kEpv; ++e) {
          const double et = exp_shift_tab(c.P, sh.tab, xt.at(i, e), Mt);
          v[0] += et;
          if (residual_cand) {
            const double ed = exp_shift_tab(c.P, sh.tab, xd.at(i, e), Md);
            v[1] += ed;
            const double r = et - rho1 * ed;
            if (r > 0.0) {
              v[2] += r;
              v[3] += ed;
            }
          }
        }
      }
      block_sums<4>(v, sh);
      uint64_t* dw = c.draw + (size_t(item) * nseg + seg) * kDrawWords;
      if (tid < 5) {
        const double val = tid == 4 ? rho1 : v[tid];
        if (tid < 1 || residual_cand) put_f64(dw + 2 * tid, tag, val);
      }
    }
    // ---- the request's last workgroup decides, draws and commits
    if (tid == 0) {
      const uint32_t target = uint32_t(w) * uint32_t(nseg);
      const uint32_t old = atomicAdd(&c.req_cnt[b], 1u);
      sh.last = old + 1u == target;
      if (sh.last) atomicExch(&c.req_cnt[b], 0u);
    }
    __syncthreads();
    if (sh.last) {
      __shared__ PickCtx pc;
      if (tid == 0) {
        pc.target = a.target;
        pc.draft = a.draft;
        pc.tokens = a.tokens;
        pc.u_res = a.u_res;
        pc.committed = a.committed;
        pc.accept_len = a.accept_len;
        pc.context_lens = a.context_lens;
        pc.accept_len_full = a.accept_len_full;
        pc.pt_at = a.pt_at;
        pc.pd_at = a.pd_at;
        pc.labels = a.labels;
        pc.status = a.status;
        pc.stat = c.stat;
        pc.bit = c.bit;
        pc.share = c.share;
        pc.draw = c.draw;
        pc.ctl = c.ctl;
        pc.V = a.V;
        pc.gamma = a.gamma;
        pc.nseg = nseg;
        pc.commit = c.commit;
        pc.tag = tag;
        pc.b = b;
        pc.r0 = r0;
        pc.w = w;
        pc.cap = cap;
      }
      __syncthreads();
      pick<T>(pc, sh);
    }
  }
  // ---- completion: the last workgroup of the call advances the epoch
  if (tid == 0) {
    const int k = bid / kChunk;
    int in_chunk = 0;
#pragma unroll
    for (int xx = 0; xx < kLanes; ++xx) in_chunk += min(max(lane_units(xx, M, nseg) - k * (kChunk / kLanes), 0), kChunk / kLanes);
    const int chunks = (lane_units(0, M, nseg) + kChunk / kLanes - 1) / (kChunk / kLanes);
    if (atomicAdd(&c.chunk[k], 1u) + 1u == uint32_t(in_chunk)) {
      atomicExch(&c.chunk[k], 0u);
      if (atomicAdd(&c.ctl->done, 1u) + 1u == uint32_t(chunks)) {
        atomicExch(&c.ctl->done, 0u);
        atomicExch(&c.ctl->giveup, 0u);
        atomicExch(&c.ctl->epoch, tag);
      }
    }
  }
}

}  // namespace

// sized for float32 rows (twice the segments of bf16), so one size serves both dtypes
size_t accept_workspace_bytes(int B, int gamma, int V, int max_rows) {
  const size_t a = ws_layout(B, gamma, V, max_rows, 2).total;
  const size_t b = ws_layout(B, gamma, V, max_rows, 4).total;
  return a > b ? a : b;
}

hipError_t launch_accept(const AcceptArgs& a, int logit_dtype, bool commit, hipStream_t stream) {
  Ctx c;
  c.a = a;
  c.P = kExp2Taylor;
  const int eb = logit_dtype == RVA_BF16 ? 2 : 4;
  c.L = ws_layout(a.B, a.gamma, a.V, a.max_rows, eb);
  c.commit = commit ? 1 : 0;
  char* base = static_cast<char*>(a.ws);
  c.ctl = reinterpret_cast<Control*>(base + c.L.off_ctl);
  c.req_cnt = reinterpret_cast<uint32_t*>(base + c.L.off_req);
  c.chunk = reinterpret_cast<uint32_t*>(base + c.L.off_chunk);
  c.stat = reinterpret_cast<uint64_t*>(base + c.L.off_stat);
  c.bit = reinterpret_cast<uint64_t*>(base + c.L.off_bit);
  c.share = reinterpret_cast<uint64_t*>(base + c.L.off_share);
  c.draw = reinterpret_cast<uint64_t*>(base + c.L.off_draw);
  const long long grid = (long long)kLanes * c.L.nseg * ((a.max_rows + kLanes - 1) / kLanes);
  if (logit_dtype == RVA_BF16)
    hipLaunchKernelGGL(accept_kernel<uint16_t>, dim3(unsigned(grid)), dim3(kNT), 0, stream, c);
  else
    hipLaunchKernelGGL(accept_kernel<float>, dim3(unsigned(grid)), dim3(kNT), 0, stream, c);
  return hipGetLastError();
}

}  // namespace rva
