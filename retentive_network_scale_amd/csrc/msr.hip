// Gated multi-scale retention layer ("Retentive Network" paper summary, Sec. 2.2
// "Gated Multi-Scale Retention"):
//   gamma = 1 - 2^(-5 - arange(h))  (passed in by the caller)
//   head_i = Retention(X, gamma_i);  Y = GroupNorm_h(Concat(heads));
//   MSR(X) = (swish(X W_G) (.) Y) W_O
// Launch sequence on the caller's stream:
//   1. one GEMM for [W_Q | W_K | W_V | W_G]: Q, K, V scattered head-major
//      [B,H,L,d] (bf16), swish(X W_G) token-major [B*L, H*dv] (bf16);
//   2. chunkwise retention (MFMA kernels) with the per-(token, head) GroupNorm
//      and the gate applied in the epilogue -> Z bf16 token-major [B*L, H*dv];
//   3. GEMM Z . W_O -> y [B*L, d_model] bf16.
#include <string.h>

#include <cmath>

#include "common.hpp"
#include "launch.hpp"
#include "retention.h"

using namespace ret;

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct MsrLayout {
  size_t q, k, v, gate, z, cw, total;
};

MsrLayout msr_layout(int B, int L, int H, int dk, int dv, int chunk) {
  MsrLayout m;
  const size_t T = (size_t)B * L;
  size_t off = 0;
  m.q = off;
  off += align256(T * H * dk * 2);
  m.k = off;
  off += align256(T * H * dk * 2);
  m.v = off;
  off += align256(T * H * dv * 2);
  m.gate = off;
  off += align256(T * H * dv * 2);
  m.z = off;
  off += align256(T * H * dv * 2);
  m.cw = off;
  off += align256(chunk_plan(B, H, L, dk, dv, chunk).ws_bytes);
  m.total = off;
  return m;
}

}  // namespace

// Defined in abi.hip: records the message returned by retention_last_error().
ret_status_t retention_fail_(ret_status_t s, const char *msg);

extern "C" {

size_t msr_layer_fwd_workspace_bytes(int B, int L, int d_model, int H, int dk, int dv, int chunk) {
  if (B <= 0 || L <= 0 || d_model <= 0 || H <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return 0;
  if (!mfma_supported(dk, dv)) return 0;
  return msr_layout(B, L, H, dk, dv, chunk).total;
}

ret_status_t msr_layer_fwd(const void *x, const void *w_q, const void *w_k, const void *w_v, const void *w_g,
                           const void *w_o, void *y, int B, int L, int d_model, int H, int dk, int dv, int chunk,
                           const float *gamma, const float *theta, long long pos0, float gn_eps, void *workspace,
                           size_t workspace_bytes, void *hip_stream) {
  if (B <= 0 || H <= 0 || L < 0 || d_model <= 0 || dk <= 0 || dv <= 0 || chunk <= 0)
    return retention_fail_(RET_ERR_INVALID_ARG, "sizes must be positive");
  if (!gamma) return retention_fail_(RET_ERR_INVALID_ARG, "gamma is NULL");
  if (H > RETENTION_MAX_HEADS) return retention_fail_(RET_ERR_UNSUPPORTED, "too many heads");
  for (int h = 0; h < H; ++h)
    if (!(gamma[h] >= 0.0f && gamma[h] <= 1.0f)) return retention_fail_(RET_ERR_INVALID_ARG, "gamma outside [0,1]");
  if (theta) {
    if (dk % 2) return retention_fail_(RET_ERR_INVALID_ARG, "rotation needs an even dk");
    for (int i = 0; i < dk / 2; ++i)
      if (!std::isfinite(theta[i])) return retention_fail_(RET_ERR_INVALID_ARG, "theta not finite");
  }
  if (!(gn_eps >= 0.0f) || !std::isfinite(gn_eps))
    return retention_fail_(RET_ERR_INVALID_ARG, "gn_eps must be finite and >= 0 (the layer always normalises)");
  if (pos0 < 0 || pos0 > (1LL << 52) - (long long)L) return retention_fail_(RET_ERR_INVALID_ARG, "pos0 out of range");
  if (!mfma_supported(dk, dv))
    return retention_fail_(RET_ERR_UNSUPPORTED, "(dk, dv) has no MFMA kernel");
  if (d_model % 128 || (H * dk) % 128 || (H * dv) % 128)
    return retention_fail_(RET_ERR_UNSUPPORTED, "d_model, H*dk and H*dv must be multiples of 128");
  if (L == 0) return retention_fail_(RET_OK, "");
  if (!x || !w_q || !w_k || !w_v || !w_g || !w_o || !y) return retention_fail_(RET_ERR_INVALID_ARG, "NULL pointer");
  const void *ptrs[] = {x, w_q, w_k, w_v, w_g, w_o, y, workspace};
  for (const void *p : ptrs)
    if ((uintptr_t)p & 15u) return retention_fail_(RET_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const MsrLayout m = msr_layout(B, L, H, dk, dv, chunk);
  if (!workspace || workspace_bytes < m.total) return retention_fail_(RET_ERR_WORKSPACE, "workspace too small");
  const size_t T = (size_t)B * L;
  {
    const uintptr_t y0 = (uintptr_t)y, y1 = y0 + T * d_model * 2;
    const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + m.total, x0 = (uintptr_t)x, x1 = x0 + T * d_model * 2;
    if ((y0 < w1 && w0 < y1) || (y0 < x1 && x0 < y1))
      return retention_fail_(RET_ERR_INVALID_ARG, "y overlaps x or the workspace");
  }
  hipStream_t st = (hipStream_t)hip_stream;
  char *ws = (char *)workspace;
  uint16_t *qh = (uint16_t *)(ws + m.q), *kh = (uint16_t *)(ws + m.k), *vh = (uint16_t *)(ws + m.v);
  uint16_t *gs = (uint16_t *)(ws + m.gate), *z = (uint16_t *)(ws + m.z);

  // 1. projections
  GemmArgs g1;
  memset(&g1, 0, sizeof(g1));
  g1.A = (const uint16_t *)x;
  g1.M = (int)T;
  g1.K = d_model;
  g1.nseg = 4;
  g1.seg[0] = GemmSeg{(const uint16_t *)w_q, H * dk, GEMM_HEADS, qh, 0, L, H, dk};
  g1.seg[1] = GemmSeg{(const uint16_t *)w_k, H * dk, GEMM_HEADS, kh, 0, L, H, dk};
  g1.seg[2] = GemmSeg{(const uint16_t *)w_v, H * dv, GEMM_HEADS, vh, 0, L, H, dv};
  g1.seg[3] = GemmSeg{(const uint16_t *)w_g, H * dv, GEMM_SWISH, gs, (long long)H * dv, L, H, dv};
  hipError_t e = launch_gemm_bf16(g1, st);
  if (e != hipSuccess) return retention_fail_(RET_ERR_HIP, hipGetErrorString(e));

  // 2.+3. chunkwise retention with GroupNorm and the gate in the epilogue -> Z
  RetArgs a;
  memset(&a, 0, sizeof(a));
  a.q = qh;
  a.k = kh;
  a.v = vh;
  a.o = z;
  a.gate = gs;
  a.q_sn = dk;
  a.q_sh = (long long)L * dk;
  a.q_sb = (long long)H * L * dk;
  a.v_sn = dv;
  a.v_sh = (long long)L * dv;
  a.v_sb = (long long)H * L * dv;
  a.o_sn = (long long)H * dv;
  a.o_sh = dv;
  a.o_sb = (long long)L * H * dv;
  a.g_sn = a.o_sn;
  a.g_sh = a.o_sh;
  a.g_sb = a.o_sb;
  a.pos0 = pos0;
  a.B = B;
  a.H = H;
  a.L = L;
  a.dk = dk;
  a.dv = dv;
  a.chunk = chunk;
  a.in_bf16 = 1;
  a.out_bf16 = 1;
  a.use_theta = theta != nullptr;
  a.use_gn = 1;
  a.gn_eps = gn_eps;
  for (int h = 0; h < H; ++h) a.gamma[h] = gamma[h];
  if (theta)
    for (int i = 0; i < dk / 2; ++i) a.theta[i] = theta[i];
  const ChunkPlan plan = chunk_plan(B, H, L, dk, dv, chunk);
  e = launch_mfma_chunkwise(a, plan, ws + m.cw, nullptr, nullptr, st);
  if (e != hipSuccess) return retention_fail_(RET_ERR_HIP, hipGetErrorString(e));

  // 4. output projection
  GemmArgs g2;
  memset(&g2, 0, sizeof(g2));
  g2.A = z;
  g2.M = (int)T;
  g2.K = H * dv;
  g2.nseg = 1;
  g2.seg[0] = GemmSeg{(const uint16_t *)w_o, d_model, GEMM_PLAIN, y, (long long)d_model, L, H, dv};
  e = launch_gemm_bf16(g2, st);
  if (e != hipSuccess) return retention_fail_(RET_ERR_HIP, hipGetErrorString(e));
  return retention_fail_(RET_OK, "");
}

}  // extern "C"
