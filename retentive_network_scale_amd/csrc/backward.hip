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

// One thread per element pair (2i, 2i+1) of a token row of a [B*H, L, d] tensor;
// rows = B*H*L, and token row r is position n = r % L of its sequence.
// dst_fwd[n] = R_n x_n and dst_rev[L-1-n] = R_n x_n (R = identity unless rot).
__global__ void bwd_prep_kernel(const void *x, void *dst_fwd, void *dst_rev, long long rows, int L, int d, int rot,
                                long long pos0, int is_bf16, RetArgs th) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int pairs = d / 2;
  if (i >= rows * pairs) return;
  const long long row = i / pairs;
  const int pr = (int)(i % pairs);
  const int n = (int)(row % L);
  const long long off = row * d + 2 * pr;
  float re = load_elem(x, off, is_bf16), im = load_elem(x, off + 1, is_bf16);
  if (rot) {
    float c, s;
    rot_cs<true>(pos0 + n, th.theta[pr], c, s);
    const float r2 = re * c - im * s, i2 = re * s + im * c;
    re = r2;
    im = i2;
  }
  if (dst_fwd) {
    store_elem(dst_fwd, off, re, is_bf16);
    store_elem(dst_fwd, off + 1, im, is_bf16);
  }
  if (dst_rev) {
    const long long roff = (row - n + (L - 1 - n)) * d + 2 * pr;
    store_elem(dst_rev, roff, re, is_bf16);
    store_elem(dst_rev, roff + 1, im, is_bf16);
  }
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
  const long long n = rows * (d / 2);
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, dst_fwd, dst_rev,
                     rows, L, d, (int)rot, pos0, (int)bf16, th);
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
