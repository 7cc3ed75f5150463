// Row-wise passes of the pre-LN residual block around the gated layer ("Retentive
// Network" paper summary, block equations: Y = MSR(LN(X)) + X, X' = FFN(LN(Y)) + Y,
// FFN(X) = gelu(X W_1) W_2).  The residual adds ride in the GEMMs (beta = 1);
// these kernels are the LayerNorm and the gelu.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

// One workgroup of 256 threads per row of d bf16 values (d % 8 == 0): mean and
// biased variance in fp32, then (x - mean) / sqrt(var + eps); no affine.
__global__ __launch_bounds__(256) void layernorm_bf16_kernel(const uint16_t *x, uint16_t *y, int d, float eps) {
  __shared__ float red[4];
  const long long row = blockIdx.x;
  const uint16_t *xr = x + row * d;
  constexpr int MAXV = 4;  // up to 4 chunks of 8 per thread: d <= 8192
  float v[MAXV][8];
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXV; ++c) {
    const int j = 8 * (threadIdx.x + 256 * c);
    if (j < d) {
      const uint4 raw = *(const uint4 *)(xr + j);
      const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[c][2 * e] = __uint_as_float(wv[e] << 16);
        v[c][2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[c][e];
    }
  }
  const float mean = block_sum<256>(s, red) / (float)d;
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXV; ++c)
    if (8 * (threadIdx.x + 256 * c) < d)
#pragma unroll
      for (int e = 0; e < 8; ++e) q += (v[c][e] - mean) * (v[c][e] - mean);
  const float inv = rsqrtf(block_sum<256>(q, red) / (float)d + eps);
#pragma unroll
  for (int c = 0; c < MAXV; ++c) {
    const int j = 8 * (threadIdx.x + 256 * c);
    if (j < d) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[c][e] - mean) * inv;
      *(uint4 *)(y + row * d + j) =
          make_uint4(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]), pack_bf2(o[4], o[5]), pack_bf2(o[6], o[7]));
    }
  }
}

// x <- x * Phi(x) = x (1 + erf(x / sqrt 2)) / 2, 8 bf16 values per thread (n % 8 == 0).
__global__ void gelu_bf16_kernel(uint16_t *x, long long n8) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  uint4 raw = *(const uint4 *)(x + 8 * i);
  uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float a = __uint_as_float(wv[e] << 16), b = __uint_as_float(wv[e] & 0xffff0000u);
    a = 0.5f * a * (1.0f + erff(a * 0.70710678118654752f));
    b = 0.5f * b * (1.0f + erff(b * 0.70710678118654752f));
    wv[e] = pack_bf2(a, b);
  }
  *(uint4 *)(x + 8 * i) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
}

hipError_t launch_layernorm_bf16(const uint16_t *x, uint16_t *y, long long rows, int d, float eps, hipStream_t st) {
  hipLaunchKernelGGL(layernorm_bf16_kernel, dim3((unsigned)rows), dim3(256), 0, st, x, y, d, eps);
  return hipGetLastError();
}

hipError_t launch_gelu_bf16(uint16_t *x, long long n, hipStream_t st) {
  const long long n8 = n / 8;
  hipLaunchKernelGGL(gelu_bf16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, x, n8);
  return hipGetLastError();
}

}  // namespace ret
