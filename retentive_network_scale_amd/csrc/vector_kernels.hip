// Vector-ALU (fp32 FMA) retention kernels: the general path for fp32 inputs and
// for head sizes without an MFMA kernel, and the recurrent decode step, which is
// bound by streaming the fp32 state and has no dense contraction.
//
// Pages: "Retentive Network" paper summary (blog.csdn.net), Sec. 2.1
// "Retention" (parallel, recurrent and chunkwise representations) and Sec. 2.2
// (per-head GroupNorm); "RetNet dual-mode hands-on manual", Sec. 3.2 and 4.2
// (explicit recurrent state, custom operator for its update).
#include "common.hpp"
#include "launch.hpp"

namespace ret {

constexpr int VT = 256;      // threads per block
constexpr int SCORE_T = 1024; // scores staged in LDS per pass
constexpr int MAXC = RETENTION_MAX_DV / VT;  // output columns per thread

// Rotate row x (dk values at element offset `off`) at position p into LDS dst.
__device__ __forceinline__ void rotate_into(const RetArgs &a, const void *x, long long off,
                                            long long p, float *dst) {
  const int t = threadIdx.x;
  if (a.use_theta) {
    for (int i = t; i < a.dk / 2; i += VT) {
      float c, s;
      rot_cs<true>(p, a.theta[i], c, s);
      float re = load_elem(x, off + 2 * i, a.in_bf16), im = load_elem(x, off + 2 * i + 1, a.in_bf16);
      dst[2 * i] = re * c - im * s;
      dst[2 * i + 1] = re * s + im * c;
    }
  } else {
    for (int i = t; i < a.dk; i += VT) dst[i] = load_elem(x, off + i, a.in_bf16);
  }
}

// Score of query row qrot (in LDS) against key row m, with the key rotated on the fly.
__device__ __forceinline__ float score_vs_key(const RetArgs &a, const float *qrot, long long koff,
                                              long long p) {
  float s = 0.0f;
  if (a.use_theta) {
    for (int i = 0; i < a.dk / 2; ++i) {
      float c, sn;
      rot_cs<true>(p, a.theta[i], c, sn);
      float re = load_elem(a.k, koff + 2 * i, a.in_bf16), im = load_elem(a.k, koff + 2 * i + 1, a.in_bf16);
      s += qrot[2 * i] * (re * c - im * sn) + qrot[2 * i + 1] * (re * sn + im * c);
    }
  } else {
    for (int i = 0; i < a.dk; ++i) s += qrot[i] * load_elem(a.k, koff + i, a.in_bf16);
  }
  return s;
}

// GroupNorm over the dv columns spread as acc[c] <-> column threadIdx.x + c*VT, then
// the gate (when given; at element offset goff + column, bf16 or fp32 as the
// inputs), then store.
__device__ __forceinline__ void gn_store(const RetArgs &a, float *acc, long long ooff, float *red,
                                         long long goff = 0) {
  const int t = threadIdx.x;
  if (a.use_gn) {
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (t + c * VT < a.dv) s += acc[c];
    const float mean = block_sum<VT>(s, red) / (float)a.dv;
    float q = 0.0f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (t + c * VT < a.dv) q += (acc[c] - mean) * (acc[c] - mean);
    const float var = block_sum<VT>(q, red) / (float)a.dv;
    const float inv = 1.0f / sqrtf(var + a.gn_eps);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) acc[c] = (acc[c] - mean) * inv;
  }
  if (a.gate)
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (t + c * VT < a.dv) {
        const long long gi = goff + t + c * VT;
        acc[c] *= gate_value(a.in_bf16 ? bf2f(a.gate[gi]) : ((const float *)a.gate)[gi], a.gate_swish);
      }
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
    if (t + c * VT < a.dv) store_elem(a.o, ooff + t + c * VT, acc[c], a.out_bf16);
}

// Intra part shared by the parallel and chunkwise forms: acc += sum over keys
// m in [m_lo, n] of gamma^(n-m) (q_n . k_m) v_m.
__device__ __forceinline__ void accumulate_keys(const RetArgs &a, int b, int h, int n, int m_lo,
                                                const float *qrot, float *w, float *acc) {
  const int t = threadIdx.x;
  const float g = a.gamma[h], lg = safe_log2(g);
  const long long kbase = (long long)b * a.q_sb + (long long)h * a.q_sh;
  const long long vbase = (long long)b * a.v_sb + (long long)h * a.v_sh;
  for (int m0 = m_lo; m0 <= n; m0 += SCORE_T) {
    const int cnt = min(SCORE_T, n + 1 - m0);
    for (int i = t; i < cnt; i += VT) {
      const int m = m0 + i;
      w[i] = decay_pow(g, lg, n - m) * score_vs_key(a, qrot, kbase + (long long)m * a.q_sn, a.pos0 + m);
    }
    __syncthreads();
    for (int i = 0; i < cnt; ++i) {
      const float wi = w[i];
      const long long vo = vbase + (long long)(m0 + i) * a.v_sn;
#pragma unroll
      for (int c = 0; c < MAXC; ++c)
        if (t + c * VT < a.dv) acc[c] += wi * load_elem(a.v, vo + t + c * VT, a.in_bf16);
    }
    __syncthreads();
  }
}

// Parallel form: grid (B*H, row blocks); each block walks its rows in order.
__global__ __launch_bounds__(VT) void vec_parallel_kernel(RetArgs a, int rows_per_block) {
  __shared__ float qrot[RETENTION_MAX_DK];
  __shared__ float w[SCORE_T];
  __shared__ float red[VT / 64];
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int n_lo = blockIdx.y * rows_per_block, n_hi = min(a.L, n_lo + rows_per_block);
  for (int n = n_lo; n < n_hi; ++n) {
    float acc[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) acc[c] = 0.0f;
    __syncthreads();
    rotate_into(a, a.q, (long long)b * a.q_sb + (long long)h * a.q_sh + (long long)n * a.q_sn,
                a.pos0 + n, qrot);
    __syncthreads();
    accumulate_keys(a, b, h, n, 0, qrot, w, acc);
    gn_store(a, acc, (long long)b * a.o_sb + (long long)h * a.o_sh + (long long)n * a.o_sn, red);
  }
}

// Chunkwise form, one block per (b, h) walking the chunks in order.  The state
// S (dk x dv fp32) lives in `state` (workspace, or state_out when given).
__global__ __launch_bounds__(VT) void vec_chunkwise_kernel(RetArgs a, float *state_all,
                                                           const float *state_in) {
  __shared__ float qrot[RETENTION_MAX_DK];
  __shared__ float w[SCORE_T];
  __shared__ float red[VT / 64];
  constexpr int TB = 16;  // tokens per state-update pass
  __shared__ float krot[TB * RETENTION_MAX_DK];
  const int t = threadIdx.x;
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const float g = a.gamma[h], lg = safe_log2(g);
  float *S = state_all + (long long)bh * a.dk * a.dv;
  const long long SZ = (long long)a.dk * a.dv;
  for (long long e = t; e < SZ; e += VT) S[e] = state_in ? state_in[(long long)bh * SZ + e] : 0.0f;
  __threadfence_block();
  __syncthreads();
  const long long qbase = (long long)b * a.q_sb + (long long)h * a.q_sh;
  const long long vbase = (long long)b * a.v_sb + (long long)h * a.v_sh;
  for (int c0 = 0; c0 < a.L; c0 += a.chunk) {
    const int Cc = min(a.chunk, a.L - c0);
    for (int j = 0; j < Cc; ++j) {
      const int n = c0 + j;
      __syncthreads();
      rotate_into(a, a.q, qbase + (long long)n * a.q_sn, a.pos0 + n, qrot);
      __syncthreads();
      float acc[MAXC];
      const float xi = decay_pow(g, lg, j + 1);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int col = t + c * VT;
        float x = 0.0f;
        if (col < a.dv)
          for (int i = 0; i < a.dk; ++i) x += qrot[i] * S[(long long)i * a.dv + col];
        acc[c] = xi * x;
      }
      accumulate_keys(a, b, h, n, c0, qrot, w, acc);
      gn_store(a, acc, (long long)b * a.o_sb + (long long)h * a.o_sh + (long long)n * a.o_sn, red);
    }
    // S <- gamma^Cc S + sum_i gamma^(Cc-1-i) k_i^T v_i
    __syncthreads();
    const float gc = decay_pow(g, lg, Cc);
    for (long long e = t; e < SZ; e += VT) S[e] *= gc;
    for (int t0 = 0; t0 < Cc; t0 += TB) {
      const int nt = min(TB, Cc - t0);
      __syncthreads();
      for (int r = 0; r < nt; ++r)
        rotate_into(a, a.k, qbase + (long long)(c0 + t0 + r) * a.q_sn, a.pos0 + c0 + t0 + r,
                    krot + r * a.dk);
      __syncthreads();
      for (int r = t; r < nt * a.dk; r += VT) krot[r] *= decay_pow(g, lg, Cc - 1 - (t0 + r / a.dk));
      __syncthreads();
      for (long long e = t; e < SZ; e += VT) {
        const int i = (int)(e / a.dv), col = (int)(e % a.dv);
        float x = S[e];
        for (int r = 0; r < nt; ++r)
          x += krot[r * a.dk + i] * load_elem(a.v, vbase + (long long)(c0 + t0 + r) * a.v_sn + col, a.in_bf16);
        S[e] = x;
      }
    }
    __threadfence_block();
    __syncthreads();
  }
}

// Rows r, r + nrg, ... of one thread's VEC state columns in chunks of U rows
// (all U loads issued before the first update): s <- g s + k_r v, o += q_r s.
// Advances r past the last whole chunk.
template <int U, int VEC>
__device__ __forceinline__ void step_rows(float *S, int &r, int nrg, int dk, int dv, const float *qk, float g,
                                          const float (&vv)[VEC], float (&oo)[VEC]) {
  for (; r + (U - 1) * nrg < dk; r += U * nrg) {
    float s[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float *src = S + (long long)(r + u * nrg) * dv;
      if constexpr (VEC == 4) {
        const float4 x = *(const float4 *)src;
        s[u][0] = x.x;
        s[u][1] = x.y;
        s[u][2] = x.z;
        s[u][3] = x.w;
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[u][e] = src[e];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float kr = qk[RETENTION_MAX_DK + r + u * nrg], qr = qk[r + u * nrg];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        s[u][e] = g * s[u][e] + kr * vv[e];
        oo[e] += qr * s[u][e];
      }
      float *dst = S + (long long)(r + u * nrg) * dv;
      if constexpr (VEC == 4) {
        *(float4 *)dst = make_float4(s[u][0], s[u][1], s[u][2], s[u][3]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) dst[e] = s[u][e];
      }
    }
  }
}

// One recurrent step per (b, h).  Threads tile the state as (row group, column
// group of VEC); every thread streams dk / row_groups rows of its columns:
//   s <- gamma s + k_r v ;  o += q_r s.
// The state is read and written exactly once, with VEC*4-byte accesses.
template <int VEC>
__global__ __launch_bounds__(VT) void vec_step_kernel(RetArgs a, float *state, const int *pos) {
  // The rotated q and k are read only in the state loop and the partial
  // outputs written only after it (past a barrier): one buffer holds both, so
  // eight workgroups fit a CU's LDS and a step's workgroups all run at once.
  static_assert(2 * RETENTION_MAX_DK <= RETENTION_MAX_DV * 4, "q, k fit the partial-output buffer");
  __shared__ float qk_opart[RETENTION_MAX_DV * 4];
  float *const qk = qk_opart, *const opart = qk_opart;
  __shared__ float red[VT / 64];
  const int t = threadIdx.x;
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int ncg = a.dv / VEC;               // column groups
  const int nrg = VT / ncg;                 // row groups (ncg <= VT is checked on the host)
  const int cg = t % ncg, rg = t / ncg;
  const bool active = rg < nrg && t < nrg * ncg;
  const float g = a.gamma[h];
  const long long qo = (long long)b * a.q_sb + (long long)h * a.q_sh;
  const long long vo = (long long)b * a.v_sb + (long long)h * a.v_sh;
  // rotated q and k into LDS (fp32)
  if (a.use_theta) {
    const long long p = pos[b];
    for (int i = t; i < a.dk / 2; i += VT) {
      float c, s;
      rot_cs<true>(p, a.theta[i], c, s);
      float qr = load_elem(a.q, qo + 2 * i, a.in_bf16), qi = load_elem(a.q, qo + 2 * i + 1, a.in_bf16);
      float kr = load_elem(a.k, qo + 2 * i, a.in_bf16), ki = load_elem(a.k, qo + 2 * i + 1, a.in_bf16);
      qk[2 * i] = qr * c - qi * s;
      qk[2 * i + 1] = qr * s + qi * c;
      qk[RETENTION_MAX_DK + 2 * i] = kr * c - ki * s;
      qk[RETENTION_MAX_DK + 2 * i + 1] = kr * s + ki * c;
    }
  } else {
    for (int i = t; i < a.dk; i += VT) {
      qk[i] = load_elem(a.q, qo + i, a.in_bf16);
      qk[RETENTION_MAX_DK + i] = load_elem(a.k, qo + i, a.in_bf16);
    }
  }
  __syncthreads();
  float vv[VEC], oo[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    vv[e] = active ? load_elem(a.v, vo + cg * VEC + e, a.in_bf16) : 0.0f;
    oo[e] = 0.0f;
  }
  if (active) {
    float *S = state + (long long)bh * a.dk * a.dv + cg * VEC;
    // rows r, r + nrg, ...: chunks of 16 rows (all of them in flight), then 8,
    // then one at a time.  At 16 the registers allow three waves per SIMD,
    // which streams faster than more waves with fewer loads each.
    int r = rg;
    step_rows<16, VEC>(S, r, nrg, a.dk, a.dv, qk, g, vv, oo);
    step_rows<8, VEC>(S, r, nrg, a.dk, a.dv, qk, g, vv, oo);
    step_rows<1, VEC>(S, r, nrg, a.dk, a.dv, qk, g, vv, oo);
  }
  // reduce the row groups' partial outputs through LDS, up to 4 groups per pass
  for (int base = 0; base < nrg; base += 4) {
    const int ng = min(4, nrg - base);
    __syncthreads();
    if (active && rg >= base && rg < base + ng)
#pragma unroll
      for (int e = 0; e < VEC; ++e) opart[(rg - base) * a.dv + cg * VEC + e] = oo[e];
    __syncthreads();
    if (active && rg == 0)
      for (int j = (base == 0 ? 1 : 0); j < ng; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) oo[e] += opart[j * a.dv + cg * VEC + e];
  }
  __syncthreads();
  if (active && rg == 0)
#pragma unroll
    for (int e = 0; e < VEC; ++e) opart[cg * VEC + e] = oo[e];
  __syncthreads();
  // GroupNorm + store; thread t handles columns t, t+VT, ...
  float acc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) acc[c] = (t + c * VT < a.dv) ? opart[t + c * VT] : 0.0f;
  gn_store(a, acc, (long long)b * a.o_sb + (long long)h * a.o_sh, red, (long long)b * a.g_sb + (long long)h * a.g_sh);
}

// Advances each sequence's position by one after a decode step (positions on the
// device, so a captured step replays without host updates).
__global__ void advance_pos_kernel(int *pos, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) pos[b] += 1;
}

// ------------------------------------------------------------------ launchers
hipError_t launch_vec_parallel(const RetArgs &a, hipStream_t st) {
  const int rpb = 8;
  dim3 grid(a.B * a.H, (a.L + rpb - 1) / rpb);
  hipLaunchKernelGGL(vec_parallel_kernel, grid, dim3(VT), 0, st, a, rpb);
  return hipGetLastError();
}

hipError_t launch_vec_chunkwise(const RetArgs &a, float *state_ws, const float *state_in,
                                hipStream_t st) {
  hipLaunchKernelGGL(vec_chunkwise_kernel, dim3(a.B * a.H), dim3(VT), 0, st, a, state_ws, state_in);
  return hipGetLastError();
}

hipError_t launch_advance_pos(int *pos, int B, hipStream_t st) {
  hipLaunchKernelGGL(advance_pos_kernel, dim3((B + 255) / 256), dim3(256), 0, st, pos, B);
  return hipGetLastError();
}

hipError_t launch_vec_step(const RetArgs &a, float *state, const int *pos, hipStream_t st) {
  // the host checks dv % 4 == 0 with dv / 4 <= VT, or dv <= VT
  if (a.dv % 4 == 0)
    hipLaunchKernelGGL(vec_step_kernel<4>, dim3(a.B * a.H), dim3(VT), 0, st, a, state, pos);
  else
    hipLaunchKernelGGL(vec_step_kernel<1>, dim3(a.B * a.H), dim3(VT), 0, st, a, state, pos);
  return hipGetLastError();
}

}  // namespace ret
