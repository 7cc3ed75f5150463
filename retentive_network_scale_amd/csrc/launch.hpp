// Kernel launchers behind the C ABI.  Each returns the launch status; arguments
// have already been validated by the entry points.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace ret {

// vector (FMA) kernels
hipError_t launch_vec_parallel(const RetArgs &a, hipStream_t st);
hipError_t launch_vec_chunkwise(const RetArgs &a, float *state_ws, const float *state_in,
                                hipStream_t st);
hipError_t launch_vec_step(const RetArgs &a, float *state, const int *pos, hipStream_t st);

// MFMA kernels (bf16 inputs, supported (dk, dv) pairs only)
bool mfma_supported(int dk, int dv);
// Parallel form: chunk >= L, no state.
hipError_t launch_mfma_parallel(const RetArgs &a, hipStream_t st);
// Chunkwise form.  Workspace layout and size come from chunk_plan().
struct ChunkPlan {
  int seg_chunks;     // chunks per segment (one block per segment)
  int nseg;           // segments per (b, h)
  size_t ws_bytes;    // segment-state workspace
};
ChunkPlan chunk_plan(int B, int H, int L, int dk, int dv, int chunk);
hipError_t launch_mfma_chunkwise(const RetArgs &a, const ChunkPlan &plan, void *ws,
                                 const float *state_in, float *state_out, hipStream_t st);

// bf16 GEMM: C[M][N] = A[M][K] . W^T with W stored [N][K]; see gemm.hip for epilogues.
struct GemmEpilogue {
  int kind;              // 0: plain bf16 row-major store; 1: head-major scatter; 2: swish
  void *out;
  long long ld_out;      // row stride of out (kind 0, 2)
  int L, H, dh;          // kind 1: row r = (b, l), column c = (h, j) -> out[((b*H+h)*L+l)*dh+j]
};
hipError_t launch_gemm_bf16(const uint16_t *A, const uint16_t *W, int M, int N, int K,
                            const GemmEpilogue &ep, hipStream_t st);

}  // namespace ret
