// Device helpers and launch arguments shared by the retention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "retention.h"

namespace ret {

constexpr int kMaxHeads = RETENTION_MAX_HEADS;
constexpr int kMaxPairs = RETENTION_MAX_DK / 2;

// Everything a retention kernel needs, passed by value (gamma and theta travel in
// the kernel arguments, so a captured launch records their values).
// Strides are in elements.  q and k share one layout.
struct RetArgs {
  const void *q, *k, *v;
  void *o;
  const uint16_t *gate;  // optional multiplier applied after GroupNorm (gated layer); bf16, or
                         // fp32 on the vector kernels when the inputs are fp32
  int gate_swish;        // the multiplier is swish(gate) = gate / (1 + exp(-gate)) instead of gate
  // Output transforms of the MFMA epilogue (used by the backward): out_rev stores
  // row n at L-1-n; out_rot multiplies output pair i of a row whose source token
  // sits at position p by exp(-i p theta_i) (theta from this struct, p = pos0 +
  // the row's index after any reversal).
  int out_rev, out_rot;
  // Input reversal (segment-state and segment-output kernels, no rotation): the
  // kernels' token n is row L-1-n of q, k and v
  int in_rev;
  // Segment-output pass run on its own (launch_mfma_chunkwise_out): the states
  // entering the segments were written as [dv][dk] by a call with dk and dv swapped
  int state_t;
  long long q_sb, q_sh, q_sn;
  long long v_sb, v_sh, v_sn;
  long long o_sb, o_sh, o_sn;
  long long g_sb, g_sh, g_sn;
  long long pos0;
  int B, H, L, dk, dv, chunk;
  int in_bf16, out_bf16, use_theta, use_gn;
  float gn_eps;
  float gamma[kMaxHeads];
  float theta[kMaxPairs];
};

// ------------------------------------------------------------------ numerics
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __attribute__((ext_vector_type(2))) float ret_f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 ret_bf16x2;

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even, NaN kept:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(ret_f32x2{lo, hi}, ret_bf16x2));
}

__device__ __forceinline__ uint16_t f2bf(float f) { return (uint16_t)(pack_bf2(f, 0.0f) & 0xffffu); }

__device__ __forceinline__ float load_elem(const void *p, long long i, int is_bf16) {
  return is_bf16 ? bf2f(((const uint16_t *)p)[i]) : ((const float *)p)[i];
}

__device__ __forceinline__ void store_elem(void *p, long long i, float x, int is_bf16) {
  if (is_bf16)
    ((uint16_t *)p)[i] = f2bf(x);
  else
    ((float *)p)[i] = x;
}

// cos and sin of the rotation angle p * theta.  The angle is formed and reduced
// in fp64 (p up to 2^31, angles far beyond fp32's exact range); the reduced
// angle, in revolutions within [-1/2, 1/2], goes to fp32 sin/cos.
// PRECISE selects the libm sincospi (a few ulp) over the hardware sin/cos.
template <bool PRECISE>
__device__ __forceinline__ void rot_cs(long long p, float theta, float &c, float &s) {
  double r = (double)p * (double)theta * 0.15915494309189535;  // revolutions
  r -= rint(r);
  float rf = (float)r;
  if constexpr (PRECISE) {
    sincospif(2.0f * rf, &s, &c);
  } else {
    s = __builtin_amdgcn_sinf(rf);  // sin(2*pi*x)
    c = __builtin_amdgcn_cosf(rf);
  }
}

// gamma^d for an integer distance d >= 0 (0^0 = 1).
__device__ __forceinline__ float decay_pow(float g, float lg2, int d) {
  if (d == 0) return 1.0f;
  if (g == 0.0f) return 0.0f;
  return exp2f((float)d * lg2);
}

__device__ __forceinline__ float safe_log2(float g) { return g > 0.0f ? log2f(g) : -INFINITY; }

// Gate multiplier from a gate value: swish(x) = x / (1 + e^-x) when `swish`
// (the gated layer's swish(X W_G)), else x itself.
__device__ __forceinline__ float gate_value(float x, int swish) {
  return swish ? x / (1.0f + __expf(-x)) : x;
}

// ------------------------------------------------------------------ reductions
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Sum over a block of NT threads (NT a multiple of 64); red has NT/64 floats.
// Every thread gets the result.  Contains barriers: call from all threads.
template <int NT>
__device__ __forceinline__ float block_sum(float x, float *red) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = x;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += red[i];
  return t;
}

}  // namespace ret
