// C ABI entry points: host-side validation, workspace sizing and dispatch.
// Declarations, argument meanings and error behaviour: include/retention.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "retention.h"

using namespace ret;

namespace {

thread_local char g_err[512] = "";

ret_status_t fail(ret_status_t s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

ret_status_t ok() {
  g_err[0] = '\0';
  return RET_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t esize(ret_dtype_t t) { return t == RET_BF16 ? 2 : 4; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Checks shared by the three retention entry points.
ret_status_t check_common(int B, int H, int L, int dk, int dv, const float *gamma,
                          const float *theta, long long pos0, float gn_eps, ret_dtype_t in_dtype,
                          ret_dtype_t out_dtype) {
  if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0 || L < 0)
    return fail(RET_ERR_INVALID_ARG, "sizes must be positive (B=%d H=%d L=%d dk=%d dv=%d)", B, H, L,
                dk, dv);
  if ((in_dtype != RET_F32 && in_dtype != RET_BF16) || (out_dtype != RET_F32 && out_dtype != RET_BF16))
    return fail(RET_ERR_INVALID_ARG, "unknown dtype");
  if (!gamma) return fail(RET_ERR_INVALID_ARG, "gamma is NULL");
  if (H > RETENTION_MAX_HEADS) return fail(RET_ERR_UNSUPPORTED, "H=%d above %d", H, RETENTION_MAX_HEADS);
  if (dk > RETENTION_MAX_DK || dv > RETENTION_MAX_DV)
    return fail(RET_ERR_UNSUPPORTED, "dk=%d/dv=%d above %d/%d", dk, dv, RETENTION_MAX_DK, RETENTION_MAX_DV);
  for (int h = 0; h < H; ++h)
    if (!(gamma[h] >= 0.0f && gamma[h] <= 1.0f))
      return fail(RET_ERR_INVALID_ARG, "gamma[%d]=%g outside [0,1]", h, (double)gamma[h]);
  if (theta) {
    if (dk % 2) return fail(RET_ERR_INVALID_ARG, "rotation needs an even dk (dk=%d)", dk);
    for (int i = 0; i < dk / 2; ++i)
      if (!isfinite(theta[i])) return fail(RET_ERR_INVALID_ARG, "theta[%d] not finite", i);
  }
  if (isnan(gn_eps) || (gn_eps >= 0.0f && !isfinite(gn_eps)))
    return fail(RET_ERR_INVALID_ARG, "gn_eps must be finite (or negative for no GroupNorm)");
  if ((long long)B * H * L > RETENTION_MAX_TOKEN_HEADS)
    return fail(RET_ERR_UNSUPPORTED, "B*H*L=%lld above %lld", (long long)B * H * L, RETENTION_MAX_TOKEN_HEADS);
  if (pos0 < 0 || pos0 > RETENTION_POS_LIMIT - (long long)L)
    return fail(RET_ERR_INVALID_ARG, "pos0=%lld outside [0, 2^31 - L]", pos0);
  return RET_OK;
}

RetArgs make_args(const void *q, const void *k, const void *v, void *o, int B, int H, int L, int dk,
                  int dv, int chunk, const float *gamma, const float *theta, long long pos0,
                  float gn_eps, ret_dtype_t in_dtype, ret_dtype_t out_dtype) {
  RetArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.gate = nullptr;
  a.q_sn = dk;
  a.q_sh = (long long)L * dk;
  a.q_sb = (long long)H * L * dk;
  a.v_sn = dv;
  a.v_sh = (long long)L * dv;
  a.v_sb = (long long)H * L * dv;
  a.o_sn = a.v_sn;
  a.o_sh = a.v_sh;
  a.o_sb = a.v_sb;
  a.pos0 = pos0;
  a.B = B;
  a.H = H;
  a.L = L;
  a.dk = dk;
  a.dv = dv;
  a.chunk = chunk;
  a.in_bf16 = in_dtype == RET_BF16;
  a.out_bf16 = out_dtype == RET_BF16;
  a.use_theta = theta != nullptr;
  a.use_gn = gn_eps >= 0.0f;
  a.gn_eps = a.use_gn ? gn_eps : 0.0f;
  for (int h = 0; h < H; ++h) a.gamma[h] = gamma[h];
  if (theta)
    for (int i = 0; i < dk / 2; ++i) a.theta[i] = theta[i];
  return a;
}

__global__ void copy_or_zero_kernel(float *dst, const float *src, long long n) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (long long)gridDim.x * blockDim.x) dst[i] = src ? src[i] : 0.0f;
}

hipError_t copy_or_zero(float *dst, const float *src, long long n, hipStream_t st) {
  if (dst == src || n == 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dst, src, n);
  return hipGetLastError();
}

ret_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(RET_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
}

bool use_mfma(int dk, int dv, ret_dtype_t in_dtype) {
  return in_dtype == RET_BF16 && mfma_supported(dk, dv);
}

size_t vec_chunk_ws(int B, int H, int dk, int dv) { return (size_t)B * H * dk * dv * sizeof(float); }

size_t chunk_ws_bytes(int B, int H, int L, int dk, int dv, int chunk, ret_dtype_t in_dtype) {
  return use_mfma(dk, dv, in_dtype) ? chunk_plan(B, H, L, dk, dv, chunk).ws_bytes : vec_chunk_ws(B, H, dk, dv);
}

// Backward workspace: rotated / reversed copies of the inputs (input dtype), the
// three fp32 retention outputs and one chunkwise workspace shared by the three
// retention calls (they run one after the other on the stream).
// Chunks the backward's inner retentions walk their segments in: divisors of the
// caller's chunk, so the segment boundaries (multiples of the caller's chunk)
// stay where the caller's chunk puts them.  narrow: the dv sum, queries and keys
// dk wide; wide: the dk~ and dq~ sums, queries and keys dv wide, at most the
// longest chunk whose keys stay resident in LDS.  wide divides narrow.  A chunk
// only blocks the computation (the sums are the same up to rounding); 64-token
// chunks cost the least here: the intra-chunk work shrinks with the chunk, the
// state work does not grow.
constexpr int BWD_NARROW_CHUNK = 64, BWD_WIDE_CHUNK = 64;
struct BwdChunks {
  int narrow, wide;
};
BwdChunks bwd_chunks(int dv, int chunk) {
  auto part = [chunk](int t) { return chunk > t && chunk % t == 0 ? t : chunk; };
  BwdChunks c;
  c.narrow = part(BWD_NARROW_CHUNK);
  c.wide = part(std::min(BWD_WIDE_CHUNK, resident_chunk_max(dv)));
  if (c.narrow % c.wide) c.wide = c.narrow;
  return c;
}

struct BwdPlan {
  size_t kr, krev, qrev, vrev, dorev, dq, dk, dv, cws, cws_bytes, total;
};

BwdPlan bwd_plan(int B, int H, int L, int dk, int dv, int chunk, ret_dtype_t in_dtype) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t e = esize(in_dtype), R = (size_t)B * H * L;
  BwdPlan p;
  size_t off = 0;
  p.kr = off;
  off += al(R * dk * e);
  p.krev = off;
  off += al(R * dk * e);
  p.qrev = off;
  off += al(R * dk * e);
  p.vrev = off;
  off += al(R * dv * e);
  p.dorev = off;
  off += al(R * dv * e);
  p.dq = off;
  off += al(R * dk * 4);
  p.dk = off;
  off += al(R * dk * 4);
  p.dv = off;
  off += al(R * dv * 4);
  p.cws = off;
  p.cws_bytes = std::max(chunk_ws_bytes(B, H, L, dv, dk, chunk, in_dtype), chunk_ws_bytes(B, H, L, dk, dv, chunk, in_dtype));
  const BwdChunks bc = bwd_chunks(dv, chunk);
  p.cws_bytes = std::max({p.cws_bytes, chunk_ws_bytes(B, H, L, dk, dv, bc.narrow, in_dtype),
                          chunk_ws_bytes(B, H, L, dv, dk, bc.wide, in_dtype)});
  off += al(p.cws_bytes);
  p.total = off;
  return p;
}

// One chunkwise retention of the backward (no input rotation, no GroupNorm),
// writing the gradient `out` directly: on the MFMA kernels the epilogue applies
// the inverse rotation (out_rot) and the token reversal (out_rev); on the vector
// path the result goes through fp32 scratch and a separate pass.
// in_rev (MFMA path, states kept in registers): the retention reads q, k and v
// in reversed token order itself, so no reversed copies are needed.
hipError_t bwd_retention(const void *q, const void *k, const void *v, void *out, float *scratch, int B, int H, int L,
                         int dqk, int dvv, int chunk, const float *gamma, const float *theta, long long pos0,
                         bool out_rot, bool out_rev, ret_dtype_t in_dtype, ret_dtype_t out_dtype, void *cws,
                         hipStream_t st, bool in_rev = false) {
  if (use_mfma(dqk, dvv, in_dtype)) {
    RetArgs a = make_args(q, k, v, out, B, H, L, dqk, dvv, chunk, gamma, nullptr, pos0, -1.0f, in_dtype, out_dtype);
    a.in_rev = in_rev;
    a.out_rev = out_rev;
    a.out_rot = out_rot && theta;
    if (a.out_rot)
      for (int i = 0; i < dvv / 2; ++i) a.theta[i] = theta[i];
    return launch_mfma_chunkwise(a, chunk_plan(B, H, L, dqk, dvv, chunk), cws, nullptr, nullptr, st);
  }
  RetArgs a = make_args(q, k, v, scratch, B, H, L, dqk, dvv, chunk, gamma, nullptr, 0, -1.0f, in_dtype, RET_F32);
  hipError_t e = launch_vec_chunkwise(a, (float *)cws, nullptr, st);
  if (e != hipSuccess) return e;
  RetArgs th = make_args(q, k, v, out, B, H, L, dvv, dvv, chunk, gamma, theta, pos0, -1.0f, in_dtype, out_dtype);
  return launch_bwd_final(scratch, out, (long long)B * H * L, L, dvv, out_rev, out_rot && theta, pos0,
                          out_dtype == RET_BF16, th, st);
}

}  // namespace

// Records the per-thread message of retention_last_error() for the other
// translation units (the layer); RET_OK clears it.
ret_status_t retention_fail_(ret_status_t s, const char *msg) {
  if (s == RET_OK) return ok();
  return fail(s, "%s", msg);
}

extern "C" {

int retention_abi_version(void) { return RETENTION_ABI_VERSION; }

const char *retention_status_string(int s) {
  switch (s) {
    case RET_OK: return "ok";
    case RET_ERR_INVALID_ARG: return "invalid argument";
    case RET_ERR_UNSUPPORTED: return "unsupported";
    case RET_ERR_WORKSPACE: return "workspace too small";
    case RET_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char *retention_last_error(void) { return g_err; }

ret_status_t retention_parallel(const void *q, const void *k, const void *v, void *o, int B, int H,
                                int L, int dk, int dv, const float *gamma, const float *theta,
                                long long pos0, float gn_eps, ret_dtype_t in_dtype,
                                ret_dtype_t out_dtype, void *hip_stream) {
  ret_status_t s = check_common(B, H, L, dk, dv, gamma, theta, pos0, gn_eps, in_dtype, out_dtype);
  if (s != RET_OK) return s;
  if (L == 0) return ok();
  if (!q || !k || !v || !o) return fail(RET_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(RET_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const size_t nqk = (size_t)B * H * L * dk * esize(in_dtype), nv = (size_t)B * H * L * dv * esize(in_dtype);
  const size_t no = (size_t)B * H * L * dv * esize(out_dtype);
  if (overlap(o, no, q, nqk) || overlap(o, no, k, nqk) || overlap(o, no, v, nv))
    return fail(RET_ERR_INVALID_ARG, "o overlaps an input");
  RetArgs a = make_args(q, k, v, o, B, H, L, dk, dv, L, gamma, theta, pos0, gn_eps, in_dtype, out_dtype);
  hipStream_t st = (hipStream_t)hip_stream;
  if (use_mfma(dk, dv, in_dtype)) return hip_status(launch_mfma_parallel(a, st));
  return hip_status(launch_vec_parallel(a, st));
}

size_t retention_chunkwise_workspace_bytes(int B, int H, int L, int dk, int dv, int chunk,
                                           ret_dtype_t in_dtype) {
  if (B <= 0 || H <= 0 || L <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return 0;
  if ((long long)B * H * L > RETENTION_MAX_TOKEN_HEADS) return 0;
  chunk = std::min(chunk, L);
  if (use_mfma(dk, dv, in_dtype)) return chunk_plan(B, H, L, dk, dv, chunk).ws_bytes;
  return vec_chunk_ws(B, H, dk, dv);
}

}  // extern "C"

namespace {

// The chunkwise call on a given workspace.  fork: whether a small launch may use
// the library's second stream (the allocation-free entry point keeps every launch
// on the caller's stream).
ret_status_t chunkwise_impl(const void *q, const void *k, const void *v, void *o, int B, int H, int L, int dk, int dv,
                            int chunk, const float *gamma, const float *theta, long long pos0, const float *state_in,
                            float *state_out, float gn_eps, ret_dtype_t in_dtype, ret_dtype_t out_dtype,
                            void *workspace, size_t workspace_bytes, void *hip_stream, bool fork) {
  ret_status_t s = check_common(B, H, L, dk, dv, gamma, theta, pos0, gn_eps, in_dtype, out_dtype);
  if (s != RET_OK) return s;
  if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk=%d must be positive", chunk);
  chunk = std::min(chunk, std::max(L, 1));
  if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out)))
    return fail(RET_ERR_INVALID_ARG, "state pointers must be 16-byte aligned");
  const size_t ns = (size_t)B * H * dk * dv * sizeof(float);
  hipStream_t st = (hipStream_t)hip_stream;
  if (L == 0) {  // nothing to compute: the state passes through unchanged
    if (state_out && state_in && state_in != state_out && overlap(state_out, ns, state_in, ns))
      return fail(RET_ERR_INVALID_ARG, "state_out partially overlaps state_in");
    if (state_out) return hip_status(copy_or_zero(state_out, state_in, (long long)ns / 4, st));
    return ok();
  }
  if (!q || !k || !v || !o) return fail(RET_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(RET_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const size_t nqk = (size_t)B * H * L * dk * esize(in_dtype), nv = (size_t)B * H * L * dv * esize(in_dtype);
  const size_t no = (size_t)B * H * L * dv * esize(out_dtype);
  if (overlap(o, no, q, nqk) || overlap(o, no, k, nqk) || overlap(o, no, v, nv))
    return fail(RET_ERR_INVALID_ARG, "o overlaps an input");
  if (state_out &&
      (overlap(state_out, ns, q, nqk) || overlap(state_out, ns, k, nqk) || overlap(state_out, ns, v, nv) ||
       overlap(state_out, ns, o, no) || (state_in && state_in != state_out && overlap(state_out, ns, state_in, ns))))
    return fail(RET_ERR_INVALID_ARG, "state_out overlaps another tensor (only exact aliasing of state_in is allowed)");
  RetArgs a = make_args(q, k, v, o, B, H, L, dk, dv, chunk, gamma, theta, pos0, gn_eps, in_dtype, out_dtype);
  if (use_mfma(dk, dv, in_dtype)) {
    ChunkPlan plan = chunk_plan(B, H, L, dk, dv, chunk);
    if (plan.ws_bytes && (!workspace || workspace_bytes < plan.ws_bytes))
      return fail(RET_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws_bytes, workspace_bytes);
    if (workspace && !aligned16(workspace)) return fail(RET_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    return hip_status(launch_mfma_chunkwise(a, plan, workspace, state_in, state_out, st, fork));
  }
  // vector path: the running state lives in state_out when given, else in the workspace
  float *S = state_out;
  if (!S) {
    const size_t need = vec_chunk_ws(B, H, dk, dv);
    if (!workspace || workspace_bytes < need)
      return fail(RET_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (!aligned16(workspace)) return fail(RET_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    S = (float *)workspace;
  }
  return hip_status(launch_vec_chunkwise(a, S, state_in, st));
}

// Scratch of the allocation-free chunkwise entry point: a file-scope device
// array, one copy per GPU, held until the process ends.  Host code never uses
// its name as an address (in host code it is only a stand-in for the symbol):
// the device address comes from hipGetSymbolAddress, once per device with that
// device current, and is kept per device.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)RETENTION_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;

// This device's address of `scratch` (nullptr and the error on failure).
void *scratch_ptr(hipError_t *err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) return it->second;
  void *ptr = nullptr;
  *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || !ptr) {
    if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
    return nullptr;
  }
  g_scratch_ptr.emplace(dev, ptr);
  return ptr;
}

}  // namespace

extern "C" {

ret_status_t retention_chunkwise(const void *q, const void *k, const void *v, void *o, int B, int H,
                                 int L, int dk, int dv, int chunk, const float *gamma,
                                 const float *theta, long long pos0, const float *state_in,
                                 float *state_out, float gn_eps, ret_dtype_t in_dtype,
                                 ret_dtype_t out_dtype, void *workspace, size_t workspace_bytes,
                                 void *hip_stream) {
  return chunkwise_impl(q, k, v, o, B, H, L, dk, dv, chunk, gamma, theta, pos0, state_in, state_out, gn_eps, in_dtype,
                        out_dtype, workspace, workspace_bytes, hip_stream, true);
}

ret_status_t retention_chunkwise_noalloc(const void *q, const void *k, const void *v, void *o, int B, int H, int L,
                                         int dk, int dv, int chunk, const float *gamma, const float *theta,
                                         long long pos0, const float *state_in, float *state_out, float gn_eps,
                                         ret_dtype_t in_dtype, ret_dtype_t out_dtype, void *hip_stream) {
  ret_status_t s = check_common(B, H, L, dk, dv, gamma, theta, pos0, gn_eps, in_dtype, out_dtype);
  if (s != RET_OK) return s;
  if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk=%d must be positive", chunk);
  const size_t need = L > 0 ? retention_chunkwise_workspace_bytes(B, H, L, dk, dv, chunk, in_dtype) : 0;
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(RET_ERR_UNSUPPORTED, "needs %zu bytes of scratch, the allocation-free entry point has %zu", need,
                NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if (need) {
    hipError_t e = hipSuccess;
    ws = scratch_ptr(&e);
    if (!ws) return fail(RET_ERR_HIP, "HIP error: %s (address of the scratch array)", hipGetErrorString(e));
  }
  return chunkwise_impl(q, k, v, o, B, H, L, dk, dv, chunk, gamma, theta, pos0, state_in, state_out, gn_eps, in_dtype,
                        out_dtype, ws, need, hip_stream, false);
}

size_t retention_chunkwise_bwd_workspace_bytes(int B, int H, int L, int dk, int dv, int chunk, ret_dtype_t in_dtype) {
  if (B <= 0 || H <= 0 || L <= 0 || dk <= 0 || dv <= 0 || chunk <= 0) return 0;
  if ((long long)B * H * L > RETENTION_MAX_TOKEN_HEADS) return 0;
  chunk = std::min(chunk, L);
  return bwd_plan(B, H, L, dk, dv, chunk, in_dtype).total;
}

// The backward; fwd_ws (optional) is the workspace of the forward call whose
// segment states the dq~ sum reads instead of computing its own.
static ret_status_t chunkwise_bwd(const void *q, const void *k, const void *v, const void *d_o, void *dq,
                                  void *dk_out, void *dv_out, int B, int H, int L, int dk, int dv, int chunk,
                                  const float *gamma, const float *theta, long long pos0, ret_dtype_t in_dtype,
                                  ret_dtype_t out_dtype, const void *fwd_ws, size_t fwd_ws_bytes, void *workspace,
                                  size_t workspace_bytes, void *hip_stream) {
  ret_status_t s = check_common(B, H, L, dk, dv, gamma, theta, pos0, -1.0f, in_dtype, out_dtype);
  if (s != RET_OK) return s;
  if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk=%d must be positive", chunk);
  chunk = std::min(chunk, std::max(L, 1));
  if (dk % 8 || dv % 8) return fail(RET_ERR_UNSUPPORTED, "the backward needs dk and dv multiples of 8");
  if (dv > RETENTION_MAX_DK)  // dv is the query/key width of two of the inner retentions
    return fail(RET_ERR_UNSUPPORTED, "the backward needs dv <= %d", RETENTION_MAX_DK);
  if (L == 0) return ok();
  if (!q || !k || !v || !d_o || !dq || !dk_out || !dv_out) return fail(RET_ERR_INVALID_ARG, "NULL tensor pointer");
  const void *ptrs[] = {q, k, v, d_o, dq, dk_out, dv_out, workspace, fwd_ws};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return fail(RET_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const BwdPlan p = bwd_plan(B, H, L, dk, dv, chunk, in_dtype);
  // the forward's segment states: fp32 [B*H][nseg][dk][dv] at the start of its workspace
  const ChunkPlan fwd_plan = chunk_plan(B, H, L, dk, dv, chunk);
  if (fwd_ws && fwd_ws_bytes < fwd_plan.seg_bytes)
    return fail(RET_ERR_WORKSPACE, "forward workspace of %zu bytes needed, %zu given", fwd_plan.seg_bytes,
                fwd_ws_bytes);
  if (!workspace || workspace_bytes < p.total)
    return fail(RET_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", p.total, workspace_bytes);
  // the backward's own passes write their workspace before the dq sum reads the forward's states
  if (fwd_ws && overlap(fwd_ws, fwd_plan.seg_bytes, workspace, p.total))
    return fail(RET_ERR_INVALID_ARG, "the forward workspace overlaps the backward's workspace");
  const size_t R = (size_t)B * H * L;
  const size_t nqk = R * dk * esize(in_dtype), nv = R * dv * esize(in_dtype);
  const size_t oqk = R * dk * esize(out_dtype), ov = R * dv * esize(out_dtype);
  const struct {
    const void *p;
    size_t n;
  } ins[] = {{q, nqk}, {k, nqk}, {v, nv}, {d_o, nv}, {workspace, p.total}, {fwd_ws, fwd_ws ? fwd_plan.seg_bytes : 0}},
    outs[] = {{dq, oqk}, {dk_out, oqk}, {dv_out, ov}};
  for (const auto &o : outs) {
    for (const auto &i : ins)
      if (overlap(o.p, o.n, i.p, i.n)) return fail(RET_ERR_INVALID_ARG, "a gradient overlaps an input or the workspace");
    for (const auto &o2 : outs)
      if (o.p != o2.p && overlap(o.p, o.n, o2.p, o2.n)) return fail(RET_ERR_INVALID_ARG, "gradients overlap");
  }
  hipStream_t st = (hipStream_t)hip_stream;
  char *ws = (char *)workspace;
  RetArgs th = make_args(q, k, v, dq, B, H, L, dk, dv, chunk, gamma, theta, pos0, -1.0f, in_dtype, out_dtype);
  const bool rot = theta != nullptr, bf = in_dtype == RET_BF16;
  const long long rows = (long long)B * H * L;  // token rows of every tensor
  hipError_t e;
  float *dqr = (float *)(ws + p.dq), *dkr = (float *)(ws + p.dk), *dvr = (float *)(ws + p.dv);
  void *cws = ws + p.cws;
  if (use_mfma(dk, dv, in_dtype) && use_mfma(dv, dk, in_dtype) && chunk_state_in_regs(B, H, L, dk, dv, chunk) &&
      chunk_state_in_regs(B, H, L, dv, dk, chunk)) {
    // the MFMA kernels read the reversed sequences themselves: only the rotated
    // keys and queries are prepared (forward order; the p.kr and p.qrev slots).
    // The dv sum's state, sum over later tokens of q~^T dO, is the transpose of
    // the dk~ sum's, sum of dO^T q~ (same segments, same decay): the dv sum runs
    // first, and the dk~ sum's output pass reads the states it left in the
    // workspace, transposed, instead of a state pass and a scan of its own.
    // Without rotation the sums read k and q themselves.
    const void *kr = rot ? (const void *)(ws + p.kr) : k, *qr = rot ? (const void *)(ws + p.qrev) : q;
    e = rot ? launch_bwd_prep2(k, ws + p.kr, q, ws + p.qrev, rows, L, dk, pos0, bf, th, st) : hipSuccess;
    const BwdChunks bc = bwd_chunks(dv, chunk);
    const int cw = bc.wide;
    if (e != hipSuccess ||
        (e = bwd_retention(kr, qr, d_o, dv_out, dvr, B, H, L, dk, dv, bc.narrow, gamma, nullptr, pos0, false, true,
                           in_dtype, out_dtype, cws, st, true)) != hipSuccess)
      return hip_status(e);
    {
      // the dv sum's segments, walked in chunks of cw
      ChunkPlan pl = chunk_plan(B, H, L, dk, dv, bc.narrow);
      pl.seg_chunks *= bc.narrow / cw;
      RetArgs a = make_args(v, d_o, qr, dk_out, B, H, L, dv, dk, cw, gamma, nullptr, pos0, -1.0f, in_dtype,
                            out_dtype);
      a.in_rev = 1;
      a.out_rev = 1;
      a.out_rot = rot;
      if (rot)
        for (int i = 0; i < dk / 2; ++i) a.theta[i] = theta[i];
      a.state_t = 1;
      if ((e = launch_mfma_chunkwise_out(a, pl, cws, st)) != hipSuccess) return hip_status(e);
    }
    if (fwd_ws && fwd_plan.in_regs && chunk % cw == 0) {
      // The dq~ sum's states, sums over earlier tokens of v^T k~, are the
      // transposes of the forward's k~^T v over the same segments with the same
      // decay: its output pass reads the states entering each segment from the
      // forward call's workspace, transposed, with no state pass or scan.
      ChunkPlan pl = fwd_plan;
      pl.seg_chunks *= chunk / cw;
      RetArgs a = make_args(d_o, v, kr, dq, B, H, L, dv, dk, cw, gamma, nullptr, pos0, -1.0f, in_dtype, out_dtype);
      a.out_rot = rot;
      if (rot)
        for (int i = 0; i < dk / 2; ++i) a.theta[i] = theta[i];
      a.state_t = 1;
      if ((e = launch_mfma_chunkwise_out(a, pl, const_cast<void *>(fwd_ws), st)) != hipSuccess)
        return hip_status(e);
      return ok();
    }
    if ((e = bwd_retention(d_o, v, kr, dq, dqr, B, H, L, dv, dk, cw, gamma, theta, pos0, true, false, in_dtype,
                           out_dtype, cws, st)) != hipSuccess)
      return hip_status(e);
    return ok();
  }
  // rotated keys (forward and reversed), rotated queries (reversed), reversed V and dO
  if ((e = launch_bwd_prep(k, ws + p.kr, ws + p.krev, rows, L, dk, rot, pos0, bf, th, st)) != hipSuccess ||
      (e = launch_bwd_prep(q, nullptr, ws + p.qrev, rows, L, dk, rot, pos0, bf, th, st)) != hipSuccess ||
      (e = launch_bwd_prep(v, nullptr, ws + p.vrev, rows, L, dv, false, 0, bf, th, st)) != hipSuccess ||
      (e = launch_bwd_prep(d_o, nullptr, ws + p.dorev, rows, L, dv, false, 0, bf, th, st)) != hipSuccess)
    return hip_status(e);
  if ((e = bwd_retention(d_o, v, ws + p.kr, dq, dqr, B, H, L, dv, dk, chunk, gamma, theta, pos0, true, false,
                         in_dtype, out_dtype, cws, st)) != hipSuccess ||
      (e = bwd_retention(ws + p.vrev, ws + p.dorev, ws + p.qrev, dk_out, dkr, B, H, L, dv, dk, chunk, gamma, theta,
                         pos0, true, true, in_dtype, out_dtype, cws, st)) != hipSuccess ||
      (e = bwd_retention(ws + p.krev, ws + p.qrev, ws + p.dorev, dv_out, dvr, B, H, L, dk, dv, chunk, gamma, nullptr,
                         pos0, false, true, in_dtype, out_dtype, cws, st)) != hipSuccess)
    return hip_status(e);
  return ok();
}

ret_status_t retention_chunkwise_bwd(const void *q, const void *k, const void *v, const void *d_o, void *dq,
                                     void *dk_out, void *dv_out, int B, int H, int L, int dk, int dv, int chunk,
                                     const float *gamma, const float *theta, long long pos0, ret_dtype_t in_dtype,
                                     ret_dtype_t out_dtype, void *workspace, size_t workspace_bytes,
                                     void *hip_stream) {
  return chunkwise_bwd(q, k, v, d_o, dq, dk_out, dv_out, B, H, L, dk, dv, chunk, gamma, theta, pos0, in_dtype,
                       out_dtype, nullptr, 0, workspace, workspace_bytes, hip_stream);
}

ret_status_t retention_chunkwise_bwd_saved(const void *q, const void *k, const void *v, const void *d_o, void *dq,
                                           void *dk_out, void *dv_out, int B, int H, int L, int dk, int dv,
                                           int chunk, const float *gamma, const float *theta, long long pos0,
                                           ret_dtype_t in_dtype, ret_dtype_t out_dtype, const void *fwd_workspace,
                                           size_t fwd_workspace_bytes, void *workspace, size_t workspace_bytes,
                                           void *hip_stream) {
  if (!fwd_workspace) return fail(RET_ERR_INVALID_ARG, "NULL forward workspace");
  return chunkwise_bwd(q, k, v, d_o, dq, dk_out, dv_out, B, H, L, dk, dv, chunk, gamma, theta, pos0, in_dtype,
                       out_dtype, fwd_workspace, fwd_workspace_bytes, workspace, workspace_bytes, hip_stream);
}

ret_status_t retention_recurrent_step(const void *q, const void *k, const void *v, float *state,
                                      void *o, int B, int H, int dk, int dv, const float *gamma,
                                      const float *theta, const int *pos, float gn_eps,
                                      ret_dtype_t in_dtype, ret_dtype_t out_dtype, void *hip_stream) {
  ret_status_t s = check_common(B, H, 1, dk, dv, gamma, theta, 0, gn_eps, in_dtype, out_dtype);
  if (s != RET_OK) return s;
  if (!q || !k || !v || !o || !state) return fail(RET_ERR_INVALID_ARG, "NULL tensor pointer");
  if (theta && !pos) return fail(RET_ERR_INVALID_ARG, "pos is NULL but rotation is on");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state))
    return fail(RET_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!(dv % 4 == 0 ? dv / 4 <= 256 : dv <= 256))
    return fail(RET_ERR_UNSUPPORTED, "dv=%d: the step kernel needs dv %% 4 == 0 or dv <= 256", dv);
  const size_t ns = (size_t)B * H * dk * dv * sizeof(float);
  const size_t nqk = (size_t)B * H * dk * esize(in_dtype), nv = (size_t)B * H * dv * esize(in_dtype);
  const size_t no = (size_t)B * H * dv * esize(out_dtype);
  if (overlap(o, no, q, nqk) || overlap(o, no, k, nqk) || overlap(o, no, v, nv) || overlap(o, no, state, ns) ||
      overlap(state, ns, q, nqk) || overlap(state, ns, k, nqk) || overlap(state, ns, v, nv))
    return fail(RET_ERR_INVALID_ARG, "state or o overlaps another tensor");
  RetArgs a = make_args(q, k, v, o, B, H, 1, dk, dv, 1, gamma, theta, 0, gn_eps, in_dtype, out_dtype);
  a.q_sn = a.q_sh = dk;
  a.q_sb = (long long)H * dk;
  a.v_sn = a.v_sh = a.o_sn = a.o_sh = dv;
  a.v_sb = a.o_sb = (long long)H * dv;
  return hip_status(launch_vec_step(a, state, pos, (hipStream_t)hip_stream));
}

}  // extern "C"
