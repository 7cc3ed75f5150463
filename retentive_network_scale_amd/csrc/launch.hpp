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
// Backward passes (backward.hip): rotate and/or reverse the token order of a
// [rows, L, d] tensor; un-rotate (and reverse) an fp32 gradient into out.
hipError_t launch_bwd_prep(const void *x, void *dst_fwd, void *dst_rev, long long rows, int L, int d, bool rot,
                           long long pos0, bool bf16, const RetArgs &th, hipStream_t st);
// dst_a = R x_a and dst_b = R x_b (forward order, rotation on) in one pass.
hipError_t launch_bwd_prep2(const void *xa, void *dst_a, const void *xb, void *dst_b, long long rows, int L, int d,
                            long long pos0, bool bf16, const RetArgs &th, hipStream_t st);
hipError_t launch_bwd_final(const float *src, void *out, long long rows, int L, int d, bool rev, bool rot,
                            long long pos0, bool out_bf16, const RetArgs &th, hipStream_t st);
// pos[b] += 1 for b < B (device positions of decode steps)
hipError_t launch_advance_pos(int *pos, int B, hipStream_t st);

// MFMA kernels (bf16 inputs, supported (dk, dv) pairs only)
bool mfma_supported(int dk, int dv);
// Parallel form: chunk >= L, no state.
hipError_t launch_mfma_parallel(const RetArgs &a, hipStream_t st);
// Chunkwise form.  Workspace layout and size come from chunk_plan().
struct ChunkPlan {
  int seg_chunks;     // chunks per segment
  int nseg;           // segments per (b, h)
  size_t seg_bytes;   // fp32 segment states [B*H][nseg][dk][dv]
  size_t sinT_bytes;  // bf16 incoming segment states, transposed [B*H][nseg][dv][dk]
  size_t ws_bytes;    // total
  bool in_regs;       // design A (segment-output kernel); else design B (query-block kernel per chunk)
};
ChunkPlan chunk_plan(int B, int H, int L, int dk, int dv, int chunk);
// Whether chunkwise retention of these dimensions runs design A, the only one
// that reads reversed inputs (RetArgs::in_rev).
bool chunk_state_in_regs(int B, int H, int L, int dk, int dv, int chunk);
// fork: a small first-blocks launch may run on a second stream of the library's
// own (created on first use); false keeps every launch on st.
hipError_t launch_mfma_chunkwise(const RetArgs &a, const ChunkPlan &plan, void *ws,
                                 const float *state_in, float *state_out, hipStream_t st, bool fork = true);
// Design A's segment-output pass alone (plan.in_regs), on the states entering
// each segment already in ws; with a.state_t they are read transposed, as left
// by launch_mfma_chunkwise on the same sequence with dk and dv swapped (the
// backward's dk and dv sums carry transposed states).
hipError_t launch_mfma_chunkwise_out(const RetArgs &a, const ChunkPlan &plan, void *ws, hipStream_t st);
// Longest chunk whose keys design A's segment-output pass keeps resident in LDS
// for query/key width dk.
int resident_chunk_max(int dk);

// Plain bf16 GEMM through hipBLASLt (blaslt.hip): C[t][n] = sum_k X[t][k] W[n][k]
// (+ R[t][n] when R is given, same layout as C) for t < T, n < N, row-major with
// row stride ldc.  hipErrorNotSupported when hipBLASLt has no algorithm for the
// shape within ws_bytes of workspace.
// out_f32: C is fp32 (no residual then).
hipError_t blaslt_gemm_nt(const uint16_t *X, const uint16_t *W, void *C, int T, int N, int K, int ldc, void *ws,
                          size_t ws_bytes, hipStream_t st, const uint16_t *R = nullptr, bool out_f32 = false);

// Row-wise bf16 passes of the residual block (block.hip): LayerNorm without
// affine (y may alias x) and exact gelu in place.
hipError_t launch_layernorm_bf16(const uint16_t *x, uint16_t *y, long long rows, int d, float eps, hipStream_t st);
hipError_t launch_gelu_bf16(uint16_t *x, long long n, hipStream_t st);

}  // namespace ret
