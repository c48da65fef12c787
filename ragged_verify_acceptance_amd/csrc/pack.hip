// Stage 2: ragged packing of the scheduled verify rows and tier rounding.
//
// Source: "DFlash 到 DSpark in SGLang：解码提速 4.3×，以及 DeepSeek-V4 支持"
// (yichizhang.dev, AI-Infra-Visualized), section "Ragged verify under full CUDA graphs":
// the scheduled tokens of all requests sit back to back in one [total_tokens, hidden]
// buffer with cu_seqlens offsets, and the total is rounded up to the nearest captured
// tier so that a smaller graph is replayed when the budget shrinks.
//
// One launch, destination-row oriented: every workgroup rebuilds cu_seqlens for the whole
// batch in LDS (a 256-lane scan of at most a few thousand ints, cheaper than a second
// launch), picks the tier, and then handles kRowsPerBlock destination rows: a binary
// search in LDS finds the owning request, the row is copied with 16-byte vector accesses
// when alignment allows, rows [M, tier) are zero-filled.  Workgroup 0 publishes
// cu_seqlens and {M, tier}.
#include "rva_common.h"

namespace rva {
namespace {

constexpr int kPackThreads = 256;
constexpr int kRowsPerBlock = 4;
constexpr int kMaxPackB = 4096;

__global__ __launch_bounds__(kPackThreads) void pack_kernel(
    int B, int gamma, const int32_t* __restrict__ windows,
    const int32_t* __restrict__ context_lens, TierTable tiers, const uint8_t* __restrict__ src,
    size_t row_bytes, uint8_t* __restrict__ dst, int max_rows, int32_t* __restrict__ cu_out,
    int32_t* __restrict__ row_req, int32_t* __restrict__ row_pos,
    int32_t* __restrict__ total_tier, int32_t* status) {
  __shared__ int cu[kMaxPackB + 1];
  __shared__ int part[kPackThreads / kWave];
  __shared__ int s_M, s_tier;
  const int tid = threadIdx.x;

  // per-thread run of consecutive requests, then a scan over the 256 run totals
  const int per = (B + kPackThreads - 1) / kPackThreads;
  const int b0 = tid * per;
  int run = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < B) {
      int w = windows[b];
      if (w < 1 || w > gamma) {
        if (blockIdx.x == 0) flag(status, RVA_DEV_BAD_WINDOW);
        w = w < 1 ? 1 : gamma;
      }
      run += w;
      cu[b + 1] = w;  // temporarily the window
    }
  }
  // inclusive scan of the run totals: inside each wave by shuffles, then the wave totals
  const int lane = tid % kWave, wave = tid / kWave;
  int inc = run;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(inc, o);
    if (lane >= o) inc += v;
  }
  if (lane == kWave - 1) part[wave] = inc;
  __syncthreads();
  int wave_off = 0;
  for (int w = 0; w < wave; ++w) wave_off += part[w];
  int total = 0;
  for (int w = 0; w < kPackThreads / kWave; ++w) total += part[w];
  int acc = wave_off + inc - run;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < B) {
      acc += cu[b + 1];
      cu[b + 1] = acc;
    }
  }
  // tier = the first (ascending) tier >= M = tiers.t[#tiers below M]; the count is taken by
  // all threads at once (the table sits in the kernel arguments, and a sequential search
  // would chain its loads)
  static_assert(sizeof(tiers.t) / sizeof(tiers.t[0]) == 2 * kPackThreads, "two tiers a thread");
  const int M_all = total;
  const int n_below = __syncthreads_count(tid < tiers.n && tiers.t[tid] < M_all) +
                      __syncthreads_count(tid + kPackThreads < tiers.n &&
                                          tiers.t[tid + kPackThreads] < M_all);
  if (tid == 0) {
    cu[0] = 0;
    s_M = M_all;
    s_tier = tiers.t[n_below < tiers.n ? n_below : tiers.n - 1];
  }
  __syncthreads();
  const int M = s_M, tier = s_tier;
  if (blockIdx.x == 0) {
    for (int b = tid; b <= B; b += kPackThreads) cu_out[b] = cu[b];
    if (tid == 0) {
      total_tier[0] = M;
      total_tier[1] = tier;
    }
  }

  // largest b with cu[b] <= r (rows r < M)
  auto owner = [&](int r) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  // row metadata: one thread per row of this block, so the context_lens loads overlap
  if (tid < kRowsPerBlock) {
    const int r = blockIdx.x * kRowsPerBlock + tid;
    if (r < max_rows) {
      const int b = r < M ? owner(r) : -1;
      row_req[r] = b;
      row_pos[r] = b >= 0 ? context_lens[b] + (r - cu[b]) : -1;
    }
  }
  if (!src) return;
  const bool vec16 = (row_bytes % 16 == 0) && ((reinterpret_cast<uintptr_t>(src) |
                                                reinterpret_cast<uintptr_t>(dst)) % 16 == 0);
  // source row of each of this block's rows (nullptr: a pad row, zero-filled)
  const uint8_t* srow[kRowsPerBlock];
  int nrows = 0;
#pragma unroll
  for (int rr = 0; rr < kRowsPerBlock; ++rr) {
    const int r = blockIdx.x * kRowsPerBlock + rr;
    srow[rr] = nullptr;
    if (r < max_rows && r < tier) {
      nrows = rr + 1;
      const int b = r < M ? owner(r) : -1;
      if (b >= 0) srow[rr] = src + (size_t(b) * gamma + (r - cu[b])) * row_bytes;
    }
  }
  uint8_t* drow0 = dst + size_t(blockIdx.x) * kRowsPerBlock * row_bytes;
  if (vec16) {
    // rows of up to 8 KB: a pass loads 2 vectors of every row before storing any, so the
    // block's copy costs about one round trip per pass
    const size_t n = row_bytes / 16;
    for (size_t k0 = 0; k0 < n; k0 += 2 * kPackThreads) {
      uint4 v[kRowsPerBlock][2];
#pragma unroll
      for (int rr = 0; rr < kRowsPerBlock; ++rr)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const size_t k = k0 + h * kPackThreads + tid;
          v[rr][h] = (rr < nrows && srow[rr] && k < n) ? reinterpret_cast<const uint4*>(srow[rr])[k]
                                                      : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
      for (int rr = 0; rr < kRowsPerBlock; ++rr)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const size_t k = k0 + h * kPackThreads + tid;
          if (rr < nrows && k < n) reinterpret_cast<uint4*>(drow0 + size_t(rr) * row_bytes)[k] = v[rr][h];
        }
    }
  } else {
    for (int rr = 0; rr < nrows; ++rr) {
      uint8_t* d = drow0 + size_t(rr) * row_bytes;
      const uint8_t* s = srow[rr];
      for (size_t k = tid; k < row_bytes; k += kPackThreads) d[k] = s ? s[k] : uint8_t(0);
    }
  }
}

}  // namespace

hipError_t launch_pack(int B, int gamma, const int32_t* windows, const int32_t* context_lens,
                       const TierTable& tiers, const void* src, size_t row_bytes, void* dst,
                       int max_rows, int32_t* cu, int32_t* row_req, int32_t* row_pos,
                       int32_t* total_tier, int32_t* status, hipStream_t stream) {
  const int blocks = (max_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(kPackThreads), 0, stream, B, gamma, windows,
                     context_lens, tiers, static_cast<const uint8_t*>(src), row_bytes,
                     static_cast<uint8_t*>(dst), max_rows, cu, row_req, row_pos, total_tier,
                     status);
  return hipGetLastError();
}

}  // namespace rva
