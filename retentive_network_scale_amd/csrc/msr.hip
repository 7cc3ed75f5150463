// Gated multi-scale retention layer ("Retentive Network" paper summary, Sec. 2.2
// "Gated Multi-Scale Retention"):
//   gamma = 1 - 2^(-5 - arange(h))  (passed in by the caller)
//   head_i = Retention(X, gamma_i);  Y = GroupNorm_h(Concat(heads));
//   MSR(X) = (swish(X W_G) (.) Y) W_O
// Launch sequence on the caller's stream:
//   1. four plain GEMMs X W_Q, X W_K, X W_V, X W_G into one token-major bf16
//      buffer P[B*L][2 H dk + 2 H dv] (hipBLASLt);
//   2. chunkwise retention (MFMA kernels) reading Q, K, V and the gate straight
//      from P through strides, with the per-(token, head) GroupNorm and the swish
//      gate applied in the epilogue -> Z bf16 token-major [B*L, H*dv];
//   3. GEMM Z . W_O -> y [B*L, d_model] bf16 (as in 1).
#include <string.h>

#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "launch.hpp"
#include "retention.h"

using namespace ret;

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr size_t BLAS_WS = 32u << 20;  // hipBLASLt workspace

struct MsrLayout {
  size_t proj, z, cw, blas, total;
};

MsrLayout msr_layout(int B, int L, int H, int dk, int dv, int chunk) {
  MsrLayout m;
  const size_t T = (size_t)B * L;
  size_t off = 0;
  m.proj = off;
  off += align256(T * (2 * (size_t)H * dk + 2 * (size_t)H * dv) * 2);
  m.z = off;
  off += align256(T * H * dv * 2);
  m.cw = off;
  off += align256(chunk_plan(B, H, L, dk, dv, chunk).ws_bytes);
  m.blas = off;
  off += BLAS_WS;
  m.total = off;
  return m;
}

// C[t][n] = sum_k X[t][k] W[n][k] (+ R[t][n]) (row stride ldc; bf16, or fp32 when
// out_f32) through hipBLASLt; hipErrorNotSupported when hipBLASLt offers no
// algorithm for the shape.
hipError_t plain_gemm(const uint16_t *X, const uint16_t *W, void *C, int T, int N, int K, int ldc, void *blas_ws,
                      hipStream_t st, const uint16_t *R = nullptr, bool out_f32 = false) {
  return blaslt_gemm_nt(X, W, C, T, N, K, ldc, blas_ws, BLAS_WS, st, R, out_f32);
}

// P[T][NP] = X [W_Q|W_K|W_V|W_G]^T (fp32 for a decode step, else bf16), plain
// hipBLASLt GEMMs.  When the
// four weights sit back to back in memory (one [2 H dk + 2 H dv][K] matrix, rows
// in that order) this is a single GEMM over all NP columns; otherwise one GEMM
// per weight.
hipError_t projections(bool step, const uint16_t *X, const void *w_q, const void *w_k, const void *w_v,
                       const void *w_g, void *P, int T, int K, int H, int dk, int dv, void *blas_ws,
                       hipStream_t st) {
  const size_t esz = step ? 4 : 2;
  const long long NP = 2LL * H * dk + 2LL * H * dv;
  const size_t qk_bytes = (size_t)H * dk * K * 2, vg_bytes = (size_t)H * dv * K * 2;
  const char *q = (const char *)w_q;
  if ((const char *)w_k == q + qk_bytes && (const char *)w_v == q + 2 * qk_bytes &&
      (const char *)w_g == q + 2 * qk_bytes + vg_bytes)
    return plain_gemm(X, (const uint16_t *)w_q, P, T, (int)NP, K, (int)NP, blas_ws, st, nullptr, step);
  const struct {
    const void *w;
    long long col;
    int n;
  } proj_w[4] = {{w_q, 0, H * dk}, {w_k, (long long)H * dk, H * dk}, {w_v, 2LL * H * dk, H * dv},
                 {w_g, 2LL * H * dk + (long long)H * dv, H * dv}};
  for (const auto &pw : proj_w) {
    hipError_t e = plain_gemm(X, (const uint16_t *)pw.w, (char *)P + pw.col * esz, T, pw.n, K, (int)NP, blas_ws,
                              st, nullptr, step);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// Defined in abi.hip: records the message returned by retention_last_error().
ret_status_t retention_fail_(ret_status_t s, const char *msg);

// Status of a failed launch sequence: a GEMM shape for which hipBLASLt offers no
// algorithm is UNSUPPORTED (nothing of the call was enqueued after it), anything
// else a HIP error.
static ret_status_t launch_fail(hipError_t e) {
  if (e == hipErrorNotSupported)
    return retention_fail_(RET_ERR_UNSUPPORTED, "hipBLASLt offers no algorithm for one of the GEMM shapes");
  return retention_fail_(RET_ERR_HIP, hipGetErrorString(e));
}

// The layer on validated arguments: y = MSR(x) (+ residual, same layout as y).
static ret_status_t msr_forward(const void *x, const void *w_q, const void *w_k, const void *w_v, const void *w_g,
                         const void *w_o, void *y, const uint16_t *residual, int B, int L, int d_model, int H, int dk,
                         int dv, int chunk, const float *gamma, const float *theta, long long pos0, float gn_eps,
                         char *ws, const MsrLayout &m, hipStream_t st) {
  const size_t T = (size_t)B * L;
  uint16_t *proj = (uint16_t *)(ws + m.proj), *z = (uint16_t *)(ws + m.z);
  const long long NP = 2LL * H * dk + 2LL * H * dv;  // row length of P
  const long long cq = 0, ck = (long long)H * dk, cv = 2LL * H * dk, cg = cv + (long long)H * dv;

  // 1. projections into P
  {
    hipError_t e = projections(false, (const uint16_t *)x, w_q, w_k, w_v, w_g, proj, (int)T, d_model, H, dk, dv,
                               ws + m.blas, st);
    if (e != hipSuccess) return launch_fail(e);
  }

  // 2. chunkwise retention with GroupNorm and the swish gate in the epilogue -> Z
  RetArgs a;
  memset(&a, 0, sizeof(a));
  a.q = proj + cq;
  a.k = proj + ck;
  a.v = proj + cv;
  a.o = z;
  a.gate = proj + cg;
  a.gate_swish = 1;
  a.q_sn = NP;
  a.q_sh = dk;
  a.q_sb = (long long)L * NP;
  a.v_sn = NP;
  a.v_sh = dv;
  a.v_sb = (long long)L * NP;
  a.g_sn = NP;
  a.g_sh = dv;
  a.g_sb = (long long)L * NP;
  a.o_sn = (long long)H * dv;
  a.o_sh = dv;
  a.o_sb = (long long)L * H * dv;
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
  hipError_t e = launch_mfma_chunkwise(a, plan, ws + m.cw, nullptr, nullptr, st);
  if (e != hipSuccess) return launch_fail(e);

  // 3. output projection
  e = plain_gemm(z, (const uint16_t *)w_o, (uint16_t *)y, (int)T, d_model, H * dv, d_model, ws + m.blas, st, residual);
  if (e != hipSuccess) return launch_fail(e);
  return retention_fail_(RET_OK, "");
}


extern "C" {

size_t msr_layer_fwd_workspace_bytes(int B, int L, int d_model, int H, int dk, int dv, int chunk) {
  if (B <= 0 || L <= 0 || d_model <= 0 || H <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return 0;
  if (!mfma_supported(dk, dv) || (long long)B * H * L > RETENTION_MAX_TOKEN_HEADS) return 0;
  chunk = std::min(chunk, L);
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
  if (pos0 < 0 || pos0 > RETENTION_POS_LIMIT - (long long)L)
    return retention_fail_(RET_ERR_INVALID_ARG, "pos0 outside [0, 2^31 - L]");
  if ((long long)B * H * L > RETENTION_MAX_TOKEN_HEADS) return retention_fail_(RET_ERR_UNSUPPORTED, "B*H*L too large");
  chunk = std::min(chunk, std::max(L, 1));
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
  return msr_forward(x, w_q, w_k, w_v, w_g, w_o, y, nullptr, B, L, d_model, H, dk, dv, chunk, gamma, theta, pos0,
                     gn_eps, (char *)workspace, m, (hipStream_t)hip_stream);
}

size_t msr_layer_step_workspace_bytes(int B, int d_model, int H, int dk, int dv) {
  if (B <= 0 || d_model <= 0 || H <= 0 || dk <= 0 || dv <= 0) return 0;
  const size_t NP = 2 * (size_t)H * dk + 2 * (size_t)H * dv;
  return align256((size_t)B * NP * 4) + align256((size_t)B * H * dv * 2) + BLAS_WS;
}

// One decode step of the gated layer for B sequences (one token each):
//   P = x [W_Q|W_K|W_V|W_G]^T (plain GEMMs, fp32 out), the recurrent retention step of every
//   (sequence, head) at its position pos[b] on the caller's fp32 state, GroupNorm,
//   the swish gate, then y = Z W_O^T; pos[b] += 1 on the device when advance_pos.
ret_status_t msr_layer_step(const void *x, const void *w_q, const void *w_k, const void *w_v, const void *w_g,
                            const void *w_o, void *y, float *state, int *pos, int advance_pos, int B, int d_model,
                            int H, int dk, int dv, const float *gamma, const float *theta, float gn_eps,
                            void *workspace, size_t workspace_bytes, void *hip_stream) {
  if (B <= 0 || H <= 0 || d_model <= 0 || dk <= 0 || dv <= 0)
    return retention_fail_(RET_ERR_INVALID_ARG, "sizes must be positive");
  if (!gamma) return retention_fail_(RET_ERR_INVALID_ARG, "gamma is NULL");
  if (H > RETENTION_MAX_HEADS || dk > RETENTION_MAX_DK || dv > RETENTION_MAX_DV)
    return retention_fail_(RET_ERR_UNSUPPORTED, "too many heads or head size too large");
  for (int h = 0; h < H; ++h)
    if (!(gamma[h] >= 0.0f && gamma[h] <= 1.0f)) return retention_fail_(RET_ERR_INVALID_ARG, "gamma outside [0,1]");
  if (theta) {
    if (dk % 2) return retention_fail_(RET_ERR_INVALID_ARG, "rotation needs an even dk");
    for (int i = 0; i < dk / 2; ++i)
      if (!std::isfinite(theta[i])) return retention_fail_(RET_ERR_INVALID_ARG, "theta not finite");
  }
  if (!(gn_eps >= 0.0f) || !std::isfinite(gn_eps))
    return retention_fail_(RET_ERR_INVALID_ARG, "gn_eps must be finite and >= 0 (the layer always normalises)");
  if (d_model % 128 || (H * dk) % 128 || (H * dv) % 128 || dk % 8 || dv % 8)
    return retention_fail_(RET_ERR_UNSUPPORTED, "d_model, H*dk and H*dv must be multiples of 128, dk and dv of 8");
  if (dv / 4 > 256) return retention_fail_(RET_ERR_UNSUPPORTED, "dv too large for the step kernel");
  if (!x || !w_q || !w_k || !w_v || !w_g || !w_o || !y || !state || !pos)
    return retention_fail_(RET_ERR_INVALID_ARG, "NULL pointer");
  const void *ptrs[] = {x, w_q, w_k, w_v, w_g, w_o, y, state, workspace};
  for (const void *p : ptrs)
    if ((uintptr_t)p & 15u) return retention_fail_(RET_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t need = msr_layer_step_workspace_bytes(B, d_model, H, dk, dv);
  if (!workspace || workspace_bytes < need) return retention_fail_(RET_ERR_WORKSPACE, "workspace too small");
  {
    const uintptr_t y0 = (uintptr_t)y, y1 = y0 + (size_t)B * d_model * 2;
    const uintptr_t s0 = (uintptr_t)state, s1 = s0 + (size_t)B * H * dk * dv * 4;
    const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + need, x0 = (uintptr_t)x, x1 = x0 + (size_t)B * d_model * 2;
    if ((y0 < w1 && w0 < y1) || (y0 < x1 && x0 < y1) || (y0 < s1 && s0 < y1) || (s0 < w1 && w0 < s1) ||
        (s0 < x1 && x0 < s1))
      return retention_fail_(RET_ERR_INVALID_ARG, "y, state, x and the workspace must not overlap");
  }
  hipStream_t st = (hipStream_t)hip_stream;
  char *ws = (char *)workspace;
  const long long NP = 2LL * H * dk + 2LL * H * dv;
  // the step's projections stay fp32: a (token, head) row whose retention output
  // nearly cancels is divided by its small deviation in GroupNorm, which would
  // magnify the bf16 rounding of q and k
  float *proj = (float *)ws;
  uint16_t *z = (uint16_t *)(ws + align256((size_t)B * NP * 4));
  void *blas = ws + align256((size_t)B * NP * 4) + align256((size_t)B * H * dv * 2);
  const long long cq = 0, ck = (long long)H * dk, cv = 2LL * H * dk, cg = cv + (long long)H * dv;

  // 1. projections of this step's tokens into P[B][NP]
  {
    hipError_t e =
        projections(true, (const uint16_t *)x, w_q, w_k, w_v, w_g, proj, B, d_model, H, dk, dv, blas, st);
    if (e != hipSuccess) return launch_fail(e);
  }

  // 2. retention step with GroupNorm and the swish gate -> Z[B][H*dv]
  RetArgs a;
  memset(&a, 0, sizeof(a));
  a.q = proj + cq;
  a.k = proj + ck;
  a.v = proj + cv;
  a.o = z;
  a.gate = (const uint16_t *)(proj + cg);
  a.gate_swish = 1;
  a.q_sb = NP;
  a.q_sh = dk;
  a.q_sn = dk;
  a.v_sb = NP;
  a.v_sh = dv;
  a.v_sn = dv;
  a.g_sb = NP;
  a.g_sh = dv;
  a.g_sn = dv;
  a.o_sb = (long long)H * dv;
  a.o_sh = dv;
  a.o_sn = dv;
  a.B = B;
  a.H = H;
  a.L = 1;
  a.dk = dk;
  a.dv = dv;
  a.chunk = 1;
  a.in_bf16 = 0;
  a.out_bf16 = 1;
  a.use_theta = theta != nullptr;
  a.use_gn = 1;
  a.gn_eps = gn_eps;
  for (int h = 0; h < H; ++h) a.gamma[h] = gamma[h];
  if (theta)
    for (int i = 0; i < dk / 2; ++i) a.theta[i] = theta[i];
  hipError_t e = launch_vec_step(a, state, pos, st);
  if (e != hipSuccess) return launch_fail(e);

  // 3. output projection, 4. positions
  e = plain_gemm(z, (const uint16_t *)w_o, y, B, d_model, H * dv, d_model, blas, st);
  if (e != hipSuccess) return launch_fail(e);
  if (advance_pos) {
    e = launch_advance_pos(pos, B, st);
    if (e != hipSuccess) return launch_fail(e);
  }
  return retention_fail_(RET_OK, "");
}

size_t retnet_block_fwd_workspace_bytes(int B, int L, int d_model, int H, int dk, int dv, int d_ffn, int chunk) {
  if (B <= 0 || L <= 0 || d_model <= 0 || H <= 0 || dk <= 0 || dv <= 0 || d_ffn <= 0 || chunk <= 0) return 0;
  if (!mfma_supported(dk, dv) || (long long)B * H * L > RETENTION_MAX_TOKEN_HEADS) return 0;
  chunk = std::min(chunk, L);
  const size_t T = (size_t)B * L;
  return 2 * align256(T * d_model * 2) + align256(T * d_ffn * 2) + msr_layout(B, L, H, dk, dv, chunk).total;
}

// The pre-LN residual block around the gated layer:
//   Y = MSR(LN(X)) + X,   out = gelu(LN(Y) W_1^T) W_2^T + Y
// (LayerNorm without affine; both residual adds run inside the output GEMMs).
ret_status_t retnet_block_fwd(const void *x, const void *w_q, const void *w_k, const void *w_v, const void *w_g,
                              const void *w_o, const void *w_1, const void *w_2, void *out, int B, int L, int d_model,
                              int H, int dk, int dv, int d_ffn, int chunk, const float *gamma, const float *theta,
                              long long pos0, float gn_eps, float ln_eps, void *workspace, size_t workspace_bytes,
                              void *hip_stream) {
  if (B <= 0 || H <= 0 || L < 0 || d_model <= 0 || dk <= 0 || dv <= 0 || d_ffn <= 0 || chunk <= 0)
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
  if (!(gn_eps >= 0.0f) || !std::isfinite(gn_eps) || !(ln_eps >= 0.0f) || !std::isfinite(ln_eps))
    return retention_fail_(RET_ERR_INVALID_ARG, "gn_eps and ln_eps must be finite and >= 0");
  if (pos0 < 0 || pos0 > RETENTION_POS_LIMIT - (long long)L)
    return retention_fail_(RET_ERR_INVALID_ARG, "pos0 outside [0, 2^31 - L]");
  if ((long long)B * H * L > RETENTION_MAX_TOKEN_HEADS) return retention_fail_(RET_ERR_UNSUPPORTED, "B*H*L too large");
  chunk = std::min(chunk, std::max(L, 1));
  if (!mfma_supported(dk, dv)) return retention_fail_(RET_ERR_UNSUPPORTED, "(dk, dv) has no MFMA kernel");
  if (d_model % 128 || (H * dk) % 128 || (H * dv) % 128 || d_ffn % 128 || d_model > 8192)
    return retention_fail_(RET_ERR_UNSUPPORTED,
                           "d_model, H*dk, H*dv and d_ffn must be multiples of 128, and d_model <= 8192");
  if (L == 0) return retention_fail_(RET_OK, "");
  if (!x || !w_q || !w_k || !w_v || !w_g || !w_o || !w_1 || !w_2 || !out)
    return retention_fail_(RET_ERR_INVALID_ARG, "NULL pointer");
  const void *ptrs[] = {x, w_q, w_k, w_v, w_g, w_o, w_1, w_2, out, workspace};
  for (const void *p : ptrs)
    if ((uintptr_t)p & 15u) return retention_fail_(RET_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t need = retnet_block_fwd_workspace_bytes(B, L, d_model, H, dk, dv, d_ffn, chunk);
  if (!workspace || workspace_bytes < need) return retention_fail_(RET_ERR_WORKSPACE, "workspace too small");
  const size_t T = (size_t)B * L;
  {
    const uintptr_t o0 = (uintptr_t)out, o1 = o0 + T * d_model * 2;
    const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + need, x0 = (uintptr_t)x, x1 = x0 + T * d_model * 2;
    if ((o0 < w1 && w0 < o1) || (o0 < x1 && x0 < o1))
      return retention_fail_(RET_ERR_INVALID_ARG, "out overlaps x or the workspace");
  }
  hipStream_t st = (hipStream_t)hip_stream;
  char *ws = (char *)workspace;
  uint16_t *h = (uint16_t *)ws, *yb = (uint16_t *)(ws + align256(T * d_model * 2));
  uint16_t *u = (uint16_t *)(ws + 2 * align256(T * d_model * 2));
  char *mws = ws + 2 * align256(T * d_model * 2) + align256(T * d_ffn * 2);
  hipError_t e = launch_layernorm_bf16((const uint16_t *)x, h, (long long)T, d_model, ln_eps, st);
  if (e != hipSuccess) return launch_fail(e);
  ret_status_t s = msr_forward(h, w_q, w_k, w_v, w_g, w_o, yb, (const uint16_t *)x, B, L, d_model, H, dk, dv, chunk,
                               gamma, theta, pos0, gn_eps, mws, msr_layout(B, L, H, dk, dv, chunk), st);
  if (s != RET_OK) return s;
  void *blas = mws + msr_layout(B, L, H, dk, dv, chunk).blas;
  if ((e = launch_layernorm_bf16(yb, h, (long long)T, d_model, ln_eps, st)) != hipSuccess ||
      (e = plain_gemm(h, (const uint16_t *)w_1, u, (int)T, d_ffn, d_model, d_ffn, blas, st)) != hipSuccess ||
      (e = launch_gelu_bf16(u, (long long)T * d_ffn, st)) != hipSuccess ||
      (e = plain_gemm(u, (const uint16_t *)w_2, (uint16_t *)out, (int)T, d_model, d_ffn, d_model, blas, st, yb)) !=
          hipSuccess)
    return launch_fail(e);
  return retention_fail_(RET_OK, "");
}

}  // extern "C"
