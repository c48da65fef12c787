// Stage 2 body shared by pack_kernel (pack.hip) and the one-launch schedule + pack kernel
// (schedule.hip): ragged packing of the scheduled verify rows and tier rounding.
//
// Source: "DFlash 到 DSpark in SGLang：解码提速 4.3×，以及 DeepSeek-V4 支持"
// (yichizhang.dev, AI-Infra-Visualized), section "Ragged verify under full CUDA graphs":
// the scheduled tokens of all requests sit back to back in one [total_tokens, hidden]
// buffer with cu_seqlens offsets, and the total is rounded up to the nearest captured
// tier so that a smaller graph is replayed when the budget shrinks.
//
// Destination-row oriented: every workgroup rebuilds cu_seqlens for the whole batch in LDS
// (one wave's scan of at most a few thousand ints, cheaper than a second launch), picks the
// tier, and then handles ROWS destination rows: a binary search in LDS finds the owning
// request, the row is copied with 16-byte vector accesses when alignment allows, rows
// [M, tier) are zero-filled.  Long rows are cut into `nparts` column parts, one workgroup
// each (part 0 also writes the row metadata).  The publishing workgroup writes cu_seqlens
// and {M, tier}.
#pragma once

#include "rva_common.h"

namespace rva {

constexpr int kPackRows = 4;  // destination rows per workgroup

template <int NT, int BCAP>
struct PackShared {
  int cu[BCAP + 1];
  int s_M, s_tier;
};

// `windows` and `context_lens` may point to global memory or to LDS; `check`: validate the
// windows (clamped into [1, gamma], RVA_DEV_BAD_WINDOW raised by the publishing workgroup).
// Requires B <= BCAP.
template <int NT, int BCAP, int ROWS>
__device__ __forceinline__ void pack_block(PackShared<NT, BCAP>& sh, int B, int gamma, const int32_t* windows,
                                           bool check, const int32_t* context_lens,
                                           const TierTable& tiers, const uint8_t* __restrict__ src,
                                           size_t row_bytes, uint8_t* __restrict__ dst, int max_rows,
                                           int32_t* __restrict__ cu_out, int32_t* __restrict__ row_req,
                                           int32_t* __restrict__ row_pos, int32_t* __restrict__ total_tier,
                                           int32_t* status, int block, bool publish, int part = 0,
                                           int nparts = 1) {
  int* cu = sh.cu;
  const int tid = threadIdx.x;

  // offsets by wave 0 alone (one barrier for the whole step): lane l sums the windows of
  // requests [l per, (l + 1) per), a wave scan of the 64 sums gives its start, then it writes
  // its requests' cu_seqlens.  tier = the first (ascending) tier >= M = tiers.t[#tiers
  // below M], counted by ballots over the table (it sits in the kernel arguments)
  if (tid < kWave) {
    const int lane = tid;
    const int per = (B + kWave - 1) / kWave;
    const int b0 = lane * per;
    int run = 0;
    for (int i = 0; i < per; ++i) {
      const int b = b0 + i;
      if (b < B) {
        int w = windows[b];
        if (check && (w < 1 || w > gamma)) {
          if (publish) flag(status, RVA_DEV_BAD_WINDOW);
          w = w < 1 ? 1 : gamma;
        }
        run += w;
        cu[b + 1] = w;  // temporarily the window
      }
    }
    int inc = run;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(inc, o);
      if (lane >= o) inc += v;
    }
    const int M_all = __shfl(inc, kWave - 1);
    int acc = inc - run;
    for (int i = 0; i < per; ++i) {
      const int b = b0 + i;
      if (b < B) {
        acc += cu[b + 1];
        cu[b + 1] = acc;
      }
    }
    constexpr int kTierSlots = sizeof(tiers.t) / sizeof(tiers.t[0]);
    int n_below = 0;
    for (int t0 = 0; t0 < tiers.n; t0 += kWave)
      n_below += __popcll(__ballot(t0 + lane < tiers.n && tiers.t[t0 + lane] < M_all));
    static_assert(kTierSlots % kWave == 0, "tier table in whole waves");
    if (lane == 0) {
      cu[0] = 0;
      sh.s_M = M_all;
      sh.s_tier = tiers.t[n_below < tiers.n ? n_below : tiers.n - 1];
    }
  }
  __syncthreads();
  const int M = sh.s_M, tier = sh.s_tier;
  if (publish) {
    for (int b = tid; b <= B; b += NT) cu_out[b] = cu[b];
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
  if (part == 0 && tid < ROWS) {
    const int r = block * ROWS + tid;
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
  const uint8_t* srow[ROWS];
  int nrows = 0;
#pragma unroll
  for (int rr = 0; rr < ROWS; ++rr) {
    const int r = block * ROWS + rr;
    srow[rr] = nullptr;
    if (r < max_rows && r < tier) {
      nrows = rr + 1;
      const int b = r < M ? owner(r) : -1;
      if (b >= 0) srow[rr] = src + (size_t(b) * gamma + (r - cu[b])) * row_bytes;
    }
  }
  uint8_t* drow0 = dst + size_t(block) * ROWS * row_bytes;
  // this workgroup's part of every row: bytes [c_lo, c_hi), a multiple of 16 bytes apart
  const size_t chunk = ((row_bytes + nparts - 1) / nparts + 15) / 16 * 16;
  const size_t c_lo = min(row_bytes, size_t(part) * chunk), c_hi = min(row_bytes, c_lo + chunk);
  if (vec16) {
    // a pass loads 2 vectors of every row before storing any, so the block's copy costs
    // about one round trip per pass (one pass for parts of up to 2 NT x 16 bytes)
    const size_t n = c_hi / 16;
    for (size_t k0 = c_lo / 16; k0 < n; k0 += 2 * NT) {
      uint4 v[ROWS][2];
#pragma unroll
      for (int rr = 0; rr < ROWS; ++rr)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const size_t k = k0 + h * NT + tid;
          v[rr][h] = (rr < nrows && srow[rr] && k < n) ? reinterpret_cast<const uint4*>(srow[rr])[k]
                                                      : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
      for (int rr = 0; rr < ROWS; ++rr)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const size_t k = k0 + h * NT + tid;
          if (rr < nrows && k < n) reinterpret_cast<uint4*>(drow0 + size_t(rr) * row_bytes)[k] = v[rr][h];
        }
    }
  } else {
    for (int rr = 0; rr < nrows; ++rr) {
      uint8_t* d = drow0 + size_t(rr) * row_bytes;
      const uint8_t* s = srow[rr];
      for (size_t k = c_lo + tid; k < c_hi; k += NT) d[k] = s ? s[k] : uint8_t(0);
    }
  }
}

}  // namespace rva
