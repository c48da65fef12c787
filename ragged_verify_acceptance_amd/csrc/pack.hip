// Stage 2: ragged packing of the scheduled verify rows and tier rounding (the body is in
// pack_block.h, shared with the one-launch schedule + pack kernel in schedule.hip).
//
// Source: "DFlash 到 DSpark in SGLang：解码提速 4.3×，以及 DeepSeek-V4 支持"
// (yichizhang.dev, AI-Infra-Visualized), section "Ragged verify under full CUDA graphs".
#include <algorithm>

#include "pack_block.h"

namespace rva {
namespace {

constexpr int kPackThreads = 256;
constexpr int kMaxPackB = 4096;

__global__ __launch_bounds__(kPackThreads) void pack_kernel(
    int B, int gamma, const int32_t* __restrict__ windows,
    const int32_t* __restrict__ context_lens, TierTable tiers, const uint8_t* __restrict__ src,
    size_t row_bytes, uint8_t* __restrict__ dst, int max_rows, int32_t* __restrict__ cu_out,
    int32_t* __restrict__ row_req, int32_t* __restrict__ row_pos,
    int32_t* __restrict__ total_tier, int32_t* status) {
  __shared__ PackShared<kPackThreads, kMaxPackB> sh;
  pack_block<kPackThreads, kMaxPackB, kPackRows>(sh, B, gamma, windows, true, context_lens, tiers, src, row_bytes,
                                                 dst, max_rows, cu_out, row_req, row_pos, total_tier, status,
                                                 blockIdx.x, blockIdx.x == 0 && blockIdx.y == 0, blockIdx.y,
                                                 gridDim.y);
}

}  // namespace

hipError_t launch_pack(int B, int gamma, const int32_t* windows, const int32_t* context_lens,
                       const TierTable& tiers, const void* src, size_t row_bytes, void* dst,
                       int max_rows, int32_t* cu, int32_t* row_req, int32_t* row_pos,
                       int32_t* total_tier, int32_t* status, hipStream_t stream) {
  const int blocks = (max_rows + kPackRows - 1) / kPackRows;
  // rows longer than 16 KB are cut into column parts of about 16 KB, one workgroup each, so
  // that a batch of long rows (e.g. vocabulary-wide logits) spreads over the whole chip
  const int parts = src ? int(std::min<size_t>(256, (row_bytes + 16383) / 16384)) : 1;
  hipLaunchKernelGGL(pack_kernel, dim3(blocks, parts), dim3(kPackThreads), 0, stream, B, gamma, windows,
                     context_lens, tiers, static_cast<const uint8_t*>(src), row_bytes,
                     static_cast<uint8_t*>(dst), max_rows, cu, row_req, row_pos, total_tier,
                     status);
  return hipGetLastError();
}

}  // namespace rva
