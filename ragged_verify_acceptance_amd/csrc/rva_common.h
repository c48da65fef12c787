// Shared device helpers and launcher declarations of librva (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <type_traits>

#include "../../include/rva.h"

namespace rva {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 <-> f32
// bf16 is carried as its 16 raw bits; widening is exact (shift into the high half).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even narrowing (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ---------------------------------------------------------------- wave reductions
// By DPP, without an LDS round trip: row_shr:n moves each lane's value n lanes up inside
// its row of 16; row_bcast:15 hands the last lane of rows 0 and 2 to rows 1 and 3, and
// row_bcast:31 hands lane 31 to rows 2 and 3 (GFX9 controls).  Lanes with no source, and
// rows outside ROW_MASK, get `id`.  Every lane of the wave must be active: a disabled lane
// still serves its stale register as a source.
constexpr int kDppRowShr = 0x110, kDppBcast15 = 0x142, kDppBcast31 = 0x143;
constexpr int kDppWaveShr1 = 0x138;  // the whole wave up by one lane (lane 0 gets id)

template <int CTRL, int ROW_MASK, typename T>
__device__ __forceinline__ T dpp_move(T id, T x) {
  if constexpr (sizeof(T) == 8) {
    const int lo = __builtin_amdgcn_update_dpp(__double2loint(id), __double2loint(x), CTRL, ROW_MASK, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(__double2hiint(id), __double2hiint(x), CTRL, ROW_MASK, 0xf, false);
    return __hiloint2double(hi, lo);
  } else if constexpr (std::is_same_v<T, float>) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
  } else {
    return __builtin_amdgcn_update_dpp(id, x, CTRL, ROW_MASK, 0xf, false);
  }
}

// Inclusive prefix of `op` (associative, identity id) over the wave's lanes: log steps
// inside each row, then the two row broadcasts.  Lane 63 ends with the whole wave.
template <typename T, typename Op>
__device__ __forceinline__ T wave_inclusive(T x, T id, Op op) {
  x = op(x, dpp_move<kDppRowShr + 1, 0xf>(id, x));
  x = op(x, dpp_move<kDppRowShr + 2, 0xf>(id, x));
  x = op(x, dpp_move<kDppRowShr + 4, 0xf>(id, x));
  x = op(x, dpp_move<kDppRowShr + 8, 0xf>(id, x));
  x = op(x, dpp_move<kDppBcast15, 0xa>(id, x));
  x = op(x, dpp_move<kDppBcast31, 0xc>(id, x));
  return x;
}

// Lane l's value (l the same in every lane), in every lane.
__device__ __forceinline__ double readlane_f64(double x, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), l),
                          __builtin_amdgcn_readlane(__double2loint(x), l));
}

// Lane 63's value, the same in every lane.
__device__ __forceinline__ int lane63(int x) { return __builtin_amdgcn_readlane(x, 63); }
__device__ __forceinline__ float lane63(float x) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63)); }
__device__ __forceinline__ double lane63(double x) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), 63),
                          __builtin_amdgcn_readlane(__double2loint(x), 63));
}

// Whole-wave results, the same value in every lane (one summation order for all of them).
__device__ __forceinline__ float wave_max(float v) {
  return lane63(wave_inclusive(v, -INFINITY, [](float a, float b) { return fmaxf(a, b); }));
}
__device__ __forceinline__ float wave_sum(float v) {
  return lane63(wave_inclusive(v, 0.f, [](float a, float b) { return a + b; }));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  return lane63(wave_inclusive(v, 0.0, [](double a, double b) { return a + b; }));
}

__device__ __forceinline__ void flag(int32_t* status, int bits) {
  if (status) atomicOr(status, bits);
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are validated by the caller.

struct TierTable {
  int n;
  int t[512];
};

hipError_t launch_schedule(int B, int gamma, int mode, const void* hidden, int hidden_dtype,
                           int H, const float* head_w, float head_b, const float* conf_in,
                           const float* sts_T, float bias, const float* alpha,
                           const float* theta, float* conf_out, float* surv_out,
                           int32_t* windows, int32_t* K_out, double* ratio_out,
                           int32_t* status, hipStream_t stream);

hipError_t launch_pack(int B, int gamma, const int32_t* windows, const int32_t* context_lens,
                       const TierTable& tiers, const void* src, size_t row_bytes, void* dst,
                       int max_rows, int32_t* cu, int32_t* row_req, int32_t* row_pos,
                       int32_t* total_tier, int32_t* status, hipStream_t stream);

hipError_t launch_schedule_pack(int B, int gamma, int mode, const void* hidden, int hidden_dtype, int H,
                                const float* head_w, float head_b, const float* conf_in, const float* sts_T,
                                float bias, const float* alpha, const float* theta, float* conf_out,
                                float* surv_out, int32_t* windows, int32_t* K_out, double* ratio_out,
                                const int32_t* context_lens, const TierTable& tiers, const void* src,
                                size_t row_bytes, void* dst, int max_rows, int32_t* cu, int32_t* row_req,
                                int32_t* row_pos, int32_t* total_tier, int32_t* status, hipStream_t stream);

struct AttnArgs {
  int B, max_window, max_rows, Hq, Hkv, D, page_size, num_pages, max_pages;
  int log2_page;  // log2(page_size) when it is a power of two, else -1
  const void* q;
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  const int32_t* cu;
  const int32_t* total_tier;
  float scale;
  void* out;
  int32_t* status;
  void* ws;
};
size_t attention_workspace_bytes(int B, int max_window, int Hq, int Hkv, int D, int page_size,
                                 int max_pages, int kv_dtype);
hipError_t launch_attention(const AttnArgs& a, int kv_dtype, hipStream_t stream);
// Device address and size of the library-owned attention scratch on the current device
// (looked up once per device with hipGetSymbolAddress).
hipError_t attention_scratch(void** ptr, size_t* bytes);

struct AcceptArgs {
  int B, gamma, V, max_rows;
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* u_acc;
  const float* u_res;
  const int32_t* cu;
  int32_t* accept_len;
  int32_t* committed;
  int32_t* context_lens;
  float* pt_at;
  float* pd_at;
  float* labels;
  int32_t* status;
  void* ws;
  const int32_t* cap;        // cap-accept mode: commit cap (window) per request, else NULL
  int32_t* accept_len_full;  // cap-accept mode: accepted drafts over the whole block
};
size_t accept_workspace_bytes(int B, int gamma, int V, int max_rows);
hipError_t launch_accept(const AcceptArgs& a, int logit_dtype, bool commit, hipStream_t stream);

struct StsArgs {
  int N, G1;
  const float* z;
  const int32_t* accept_len;
  const int32_t* observed_len;
  float T_lo, T_hi;
  float* T_out;
  double* nll_out;
  void* ws;
};
size_t sts_workspace_bytes(int N);
hipError_t launch_sts_fit(const StsArgs& a, hipStream_t stream);

struct EceArgs {
  int N, G1, n_bins;
  const float* z;
  const int32_t* accept_len;
  const int32_t* observed_len;
  const float* T;
  double* ece_out;
  int32_t* bin_counts;
  void* ws;
};
size_t ece_workspace_bytes(int N, int G1, int n_bins);
hipError_t launch_ece(const EceArgs& a, hipStream_t stream);

struct MarkovArgs {
  int B, G1, V, r;
  const void* base;        // [B, G1, V] base logits
  const int32_t* anchor;   // [B]
  const float* u;          // [B, G1]
  const int8_t* w1;        // [V, r]
  const float* s1;         // [V]
  const int8_t* w2;        // [V, r]
  const float* s2;         // [V]
  void* out;               // [B, G1, V] logits (dtype of base)
  int32_t* tokens;         // [B, G1]
  float* p_at;             // [B, G1] or NULL
  int32_t* status;
  void* ws;
  bool vec_ok;             // V a multiple of 8 and base / out / s2 16-byte aligned
};
size_t markov_workspace_bytes(int B, int V);
hipError_t launch_markov(const MarkovArgs& a, int dtype, hipStream_t stream);

}  // namespace rva
