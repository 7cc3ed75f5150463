// MFMA retention kernels (bf16 inputs): placeholder until the tiles land.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

bool mfma_supported(int, int) { return false; }

hipError_t launch_mfma_parallel(const RetArgs &, hipStream_t) { return hipErrorNotSupported; }

ChunkPlan chunk_plan(int, int, int, int, int, int) { return ChunkPlan{1, 1, 0}; }

hipError_t launch_mfma_chunkwise(const RetArgs &, const ChunkPlan &, void *, const float *, float *,
                                 hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace ret
