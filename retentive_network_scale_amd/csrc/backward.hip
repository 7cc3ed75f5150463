// Elementwise passes of the chunkwise backward (gradients of retention with
// respect to q, k and v; "Retentive Network" paper summary, Sec. 2.1, scalar-gamma
// form).  With a_nm = gamma^(n-m) for n >= m and rotated rows q~, k~:
//   dq~_n = sum_{m<=n} a_nm (dO_n . v_m) k~_m     retention(q=dO, k=V, v=K~)
//   dk~_m = sum_{n>=m} a_nm (dO_n . v_m) q~_n     the same on the reversed sequence:
//                                                 retention(q=V', k=dO', v=Q~')
//   dv_m  = sum_{n>=m} a_nm (q~_n . k~_m) dO_n    retention(q=K~', k=Q~', v=dO')
// (' = token order reversed: n' = L-1-n turns "n >= m" into "n' <= m'" with the
// same distance), then dq = R^T dq~ and dk = R^T dk~.  The three retentions run on
// the forward kernels without rotation; these kernels prepare their inputs and
// finish their outputs.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

// One thread per 8 consecutive elements (4 pairs) of a token row of a
// [B*H, L, d] tensor (d % 8 == 0); rows = B*H*L, token row r is position
// n = r % L of its sequence.  dst_fwd[n] = R_n x_n and dst_rev[L-1-n] = R_n x_n
// (R = identity unless rot; the angle is reduced in fp64 and the sine and cosine
// taken in hardware, as the forward kernels do).
template <typename E>
__global__ void bwd_prep_kernel(const E *x, E *dst_fwd, E *dst_rev, long long rows, int L, int d, int rot,
                                long long pos0, RetArgs th) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int c8s = d / 8;
  if (i >= rows * c8s) return;
  const long long row = i / c8s;
  const int c8 = (int)(i % c8s);
  const int n = (int)(row % L);
  const long long off = row * d + 8 * c8;
  float v[8];
  if constexpr (sizeof(E) == 2) {
    const uint4 raw = *(const uint4 *)(x + off);
    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(wv[e] << 16);
      v[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
    }
  } else {
    const float4 lo = *(const float4 *)(x + off), hi = *(const float4 *)(x + off + 4);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  }
  if (rot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float c, sn;
      rot_cs<false>(pos0 + n, th.theta[4 * c8 + j], c, sn);
      const float re = v[2 * j], im = v[2 * j + 1];
      v[2 * j] = re * c - im * sn;
      v[2 * j + 1] = re * sn + im * c;
    }
  }
  E *dsts[2] = {dst_fwd ? dst_fwd + off : nullptr,
                dst_rev ? dst_rev + (row - n + (L - 1 - n)) * d + 8 * c8 : nullptr};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (!dsts[t]) continue;
    if constexpr (sizeof(E) == 2) {
      *(uint4 *)dsts[t] = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                                     pack_bf2(v[6], v[7]));
    } else {
      *(float4 *)dsts[t] = make_float4(v[0], v[1], v[2], v[3]);
      *(float4 *)(dsts[t] + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

// Two tensors of the same shape rotated at the same positions in one pass
// (the backward's K~ and Q~ in forward order): one thread per 8 consecutive
// elements of both, one angle reduction and one sine/cosine per pair serving
// both.  dst_a[r] = R_n a[r], dst_b[r] = R_n b[r].
template <typename E>
__device__ __forceinline__ void load8(const E *p, float (&v)[8]) {
  if constexpr (sizeof(E) == 2) {
    const uint4 raw = *(const uint4 *)p;
    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(wv[e] << 16);
      v[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
    }
  } else {
    const float4 lo = *(const float4 *)p, hi = *(const float4 *)(p + 4);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  }
}

template <typename E>
__device__ __forceinline__ void store8(E *p, const float (&v)[8]) {
  if constexpr (sizeof(E) == 2) {
    *(uint4 *)p = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
  } else {
    *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4 *)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <typename E>
__global__ void bwd_prep2_kernel(const E *xa, E *dst_a, const E *xb, E *dst_b, long long rows, int L, int d,
                                 long long pos0, RetArgs th) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int c8s = d / 8;
  if (i >= rows * c8s) return;
  const long long row = i / c8s;
  const int c8 = (int)(i % c8s);
  const int n = (int)(row % L);
  const long long off = row * d + 8 * c8;
  float va[8], vb[8];
  load8(xa + off, va);
  load8(xb + off, vb);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float c, sn;
    rot_cs<false>(pos0 + n, th.theta[4 * c8 + j], c, sn);
    float re = va[2 * j], im = va[2 * j + 1];
    va[2 * j] = re * c - im * sn;
    va[2 * j + 1] = re * sn + im * c;
    re = vb[2 * j];
    im = vb[2 * j + 1];
    vb[2 * j] = re * c - im * sn;
    vb[2 * j + 1] = re * sn + im * c;
  }
  store8(dst_a + off, va);
  store8(dst_b + off, vb);
}

// out[n] = R_n^T src[rev ? L-1-n : n] (R = identity unless rot); src fp32.
__global__ void bwd_final_kernel(const float *src, void *out, long long rows, int L, int d, int rev, int rot,
                                 long long pos0, int out_bf16, RetArgs th) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int pairs = d / 2;
  if (i >= rows * pairs) return;
  const long long row = i / pairs;
  const int pr = (int)(i % pairs);
  const int n = (int)(row % L);
  const long long sr = rev ? row - n + (L - 1 - n) : row;
  float re = src[sr * d + 2 * pr], im = src[sr * d + 2 * pr + 1];
  if (rot) {
    float c, s;
    rot_cs<true>(pos0 + n, th.theta[pr], c, s);
    const float r2 = re * c + im * s, i2 = -re * s + im * c;
    re = r2;
    im = i2;
  }
  store_elem(out, row * d + 2 * pr, re, out_bf16);
  store_elem(out, row * d + 2 * pr + 1, im, out_bf16);
}

hipError_t launch_bwd_prep(const void *x, void *dst_fwd, void *dst_rev, long long rows, int L, int d, bool rot,
                           long long pos0, bool bf16, const RetArgs &th, hipStream_t st) {
  const long long n = rows * (d / 8);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(bwd_prep_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)x, (uint16_t *)dst_fwd,
                       (uint16_t *)dst_rev, rows, L, d, (int)rot, pos0, th);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<float>, grid, dim3(256), 0, st, (const float *)x, (float *)dst_fwd,
                       (float *)dst_rev, rows, L, d, (int)rot, pos0, th);
  return hipGetLastError();
}

hipError_t launch_bwd_prep2(const void *xa, void *dst_a, const void *xb, void *dst_b, long long rows, int L, int d,
                            long long pos0, bool bf16, const RetArgs &th, hipStream_t st) {
  const long long n = rows * (d / 8);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(bwd_prep2_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)xa, (uint16_t *)dst_a,
                       (const uint16_t *)xb, (uint16_t *)dst_b, rows, L, d, pos0, th);
  else
    hipLaunchKernelGGL(bwd_prep2_kernel<float>, grid, dim3(256), 0, st, (const float *)xa, (float *)dst_a,
                       (const float *)xb, (float *)dst_b, rows, L, d, pos0, th);
  return hipGetLastError();
}

hipError_t launch_bwd_final(const float *src, void *out, long long rows, int L, int d, bool rev, bool rot,
                            long long pos0, bool out_bf16, const RetArgs &th, hipStream_t st) {
  const long long n = rows * (d / 2);
  hipLaunchKernelGGL(bwd_final_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, out, rows, L, d,
                     (int)rev, (int)rot, pos0, (int)out_bf16, th);
  return hipGetLastError();
}

}  // namespace ret
