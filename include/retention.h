/*
 * retention.h -- C ABI of the MI355X (gfx950) multi-scale retention library.
 *
 * What is computed (pages cited by title and section):
 *   "Retentive Network: A Successor to Transformer for Large Language Models",
 *   paper summary on blog.csdn.net:
 *     Sec. 2.1 "Retention": scalar-gamma retention
 *         o_n = sum_{m<=n} gamma^(n-m) (Q_n e^{i n theta}) (K_m e^{i m theta})^dagger v_m
 *       and its three representations -- (1) parallel (Q K^T (.) D) V with
 *       D_nm = gamma^(n-m) for n >= m else 0; (2) recurrent
 *       S_n = gamma S_{n-1} + K_n^T V_n, o_n = Q_n S_n; (3) chunkwise recurrent
 *       (parallel inside a chunk, recurrent across chunks).
 *     Sec. 2.2 "Gated Multi-Scale Retention": per-head gamma, per-head
 *       GroupNorm, MSR(X) = (swish(X W_G) (.) Y) W_O.
 *   "RetNet dual-mode hands-on manual" (lanjinlin.com.cn), Sec. 1 (decay
 *     matrix), Sec. 3.2 (explicit per-sequence state for recurrent inference),
 *     Sec. 4.1 (mode switch with states passed in and out).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates or frees tensor memory and keeps no pointer
 *     after a call returns.  Tensors are dense row-major in the shapes given,
 *     16-byte aligned.
 *   - Positions are 0-based.  Token n of a call is at absolute position
 *     p = pos0 + n.
 *   - Rotation (xPOS phase): coordinates (2i, 2i+1) of a q or k row form the
 *     complex number x_{2i} + i x_{2i+1}, multiplied by exp(i p theta_i).  The
 *     score of query n and key m is the real dot product of the rotated rows,
 *     i.e. Re[q_rot conj(k_rot)].  theta == NULL means no rotation; otherwise
 *     theta is a HOST array of dk/2 fp32 frequencies and dk must be even.
 *   - gamma is a HOST array of H fp32 decay constants in [0, 1].  gamma and
 *     theta are copied into kernel arguments at launch.
 *   - No 1/sqrt(dk) scaling is applied: scale Q or K beforehand if wanted.
 *   - gn_eps < 0: no normalisation.  gn_eps >= 0: every output row of dv
 *     values (one token, one head) is replaced by (o - mean) / sqrt(var + eps),
 *     biased variance, no affine parameters.
 *   - Accumulation is fp32.  The recurrent state is fp32 [B,H,dk,dv] and holds
 *     sum_m gamma^(n-m) k_rot_m^T v_m with keys rotated at their absolute
 *     positions.
 *   - All calls are asynchronous on hip_stream (NULL = default stream); none
 *     synchronises the device.
 *
 * Errors: every argument is checked on the host before anything is enqueued.
 * On any error nothing is enqueued and outputs are untouched.  The library
 * never aborts, throws or prints.  retention_last_error() gives a message for
 * the calling thread's last failure.  Asynchronous device faults surface at
 * the caller's next synchronisation.
 */
#ifndef RETENTION_H_
#define RETENTION_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RETENTION_ABI_VERSION 1

typedef enum {
  RET_OK = 0,
  RET_ERR_INVALID_ARG = 1, /* null pointer, bad size, gamma outside [0,1], bad eps, misaligned ... */
  RET_ERR_UNSUPPORTED = 2, /* legal arguments this build does not handle (see each call) */
  RET_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_bytes query */
  RET_ERR_HIP = 4          /* a HIP launch error (hipGetLastError) */
} ret_status_t;

typedef enum { RET_F32 = 0, RET_BF16 = 1 } ret_dtype_t;

/* Library limits (UNSUPPORTED beyond them). */
#define RETENTION_MAX_HEADS 128
#define RETENTION_MAX_DK 512
#define RETENTION_MAX_DV 1024
#define RETENTION_MAX_TOKEN_HEADS (1LL << 28) /* B * H * L of one call */
/* Positions: every absolute position is a non-negative int32, pos0 + L <=
 * RETENTION_POS_LIMIT (INVALID_ARG beyond), as for the decode step's int32 pos. */
#define RETENTION_POS_LIMIT (1LL << 31)

int retention_abi_version(void);
const char *retention_status_string(int status);
/* Message describing the calling thread's most recent failed call ("" if none). */
const char *retention_last_error(void);

/*
 * Parallel representation (Sec. 2.1 (1)): O = (Q_rot K_rot^T (.) D) V per (b, h),
 * D_nm = gamma_h^(n-m) for n >= m, else 0; then the optional GroupNorm.
 *   q, k : [B,H,L,dk] in_dtype          v : [B,H,L,dv] in_dtype
 *   o    : [B,H,L,dv] out_dtype (must not alias an input)
 * bf16 inputs with (dk, dv) in {(64,128),(128,128),(128,256),(256,256),
 * (256,512)} use the MFMA kernels; every other case uses the vector (FMA) kernels.
 * With rotation on the MFMA path the keys are rotated once per call into
 * B*H*L*dk bf16 of scratch taken stream-ordered from the device's default memory
 * pool (hipMallocAsync / hipFreeAsync on hip_stream; the pool is told once to
 * keep freed memory); RET_ERR_HIP if that allocation fails.
 * L == 0 is a no-op.
 */
ret_status_t retention_parallel(const void *q, const void *k, const void *v, void *o, int B,
                                int H, int L, int dk, int dv, const float *gamma,
                                const float *theta, long long pos0, float gn_eps,
                                ret_dtype_t in_dtype, ret_dtype_t out_dtype, void *hip_stream);

/*
 * Chunkwise recurrent representation (Sec. 2.1 (3)): tokens are split into
 * chunks of `chunk` (the last may be shorter).  Inside a chunk the parallel
 * form is used; the state entering chunk c, S_c, adds gamma^(j+1) q_rot S_c to
 * token j of the chunk, and S_{c+1} = gamma^Cc S_c + sum_i gamma^(Cc-1-i) k_rot_i^T v_i.
 *   q, k, v, o : as retention_parallel
 *   state_in   : [B,H,dk,dv] fp32 state before token 0, or NULL for zeros
 *   state_out  : [B,H,dk,dv] fp32 state after token L-1, or NULL; may alias state_in
 *   workspace  : device scratch of at least retention_chunkwise_workspace_bytes()
 *                bytes (NULL allowed when that is 0); its contents on entry do
 *                not matter.  Calls sharing a workspace must not overlap.
 * A chunk longer than L is taken as L (one chunk: the parallel form), here and
 * in every call and workspace query that takes a chunk size.
 */
size_t retention_chunkwise_workspace_bytes(int B, int H, int L, int dk, int dv, int chunk,
                                           ret_dtype_t in_dtype);
ret_status_t retention_chunkwise(const void *q, const void *k, const void *v, void *o, int B,
                                 int H, int L, int dk, int dv, int chunk, const float *gamma,
                                 const float *theta, long long pos0, const float *state_in,
                                 float *state_out, float gn_eps, ret_dtype_t in_dtype,
                                 ret_dtype_t out_dtype, void *workspace, size_t workspace_bytes,
                                 void *hip_stream);

/*
 * retention_chunkwise without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same computation, arguments (less the workspace) and
 * errors as retention_chunkwise; the call allocates nothing.  Its scratch is a
 * device array inside the library, RETENTION_NOALLOC_SCRATCH_BYTES on each GPU
 * it runs on, held until the process ends.  UNSUPPORTED when
 * retention_chunkwise_workspace_bytes() of the same arguments exceeds that size
 * (B1 H8 L32768 dk128 dv256 chunk 256 needs 32 MiB).  Every call on a GPU uses
 * that GPU's one array and it keeps the last call's contents (nothing in it needs
 * clearing): calls that overlap on one GPU -- other streams, other host threads
 * -- race, so the caller serialises them.  Every launch stays on hip_stream.
 */
#define RETENTION_NOALLOC_SCRATCH_BYTES (64u << 20)
ret_status_t retention_chunkwise_noalloc(const void *q, const void *k, const void *v, void *o, int B,
                                         int H, int L, int dk, int dv, int chunk,
                                         const float *gamma, const float *theta, long long pos0,
                                         const float *state_in, float *state_out, float gn_eps,
                                         ret_dtype_t in_dtype, ret_dtype_t out_dtype,
                                         void *hip_stream);

/*
 * One recurrent step (Sec. 2.1 (2); the custom operator for the state update
 * of "RetNet dual-mode hands-on manual" Sec. 4.2):
 *   S <- gamma_h S + k_rot^T v   (rank-1 update of the dk x dv state)
 *   o <- q_rot S                 (then the optional GroupNorm)
 *   q, k  : [B,H,dk] in_dtype     v : [B,H,dv] in_dtype
 *   state : [B,H,dk,dv] fp32, read then overwritten in place
 *   o     : [B,H,dv] out_dtype
 *   pos   : DEVICE int32 [B], absolute position of this token for each
 *           sequence (used only for rotation; ignored when theta == NULL, and
 *           may then be NULL).  The caller advances it.
 */
ret_status_t retention_recurrent_step(const void *q, const void *k, const void *v, float *state,
                                      void *o, int B, int H, int dk, int dv, const float *gamma,
                                      const float *theta, const int *pos, float gn_eps,
                                      ret_dtype_t in_dtype, ret_dtype_t out_dtype,
                                      void *hip_stream);

/*
 * Gradients of chunkwise retention (Sec. 2.1, no GroupNorm) with respect to q, k
 * and v, for training ("RetNet dual-mode hands-on manual", Sec. 2.2: chunkwise
 * mode for long-sequence training).  With a_nm = gamma^(n-m) for n >= m and the
 * rotated rows q~, k~ of the forward call:
 *   dv_m = sum_{n>=m} a_nm (q~_n . k~_m) dO_n
 *   dq_n = R_n^T sum_{m<=n} a_nm (dO_n . v_m) k~_m
 *   dk_m = R_m^T sum_{n>=m} a_nm (dO_n . v_m) q~_n
 * (R_n: the rotation at position pos0 + n).  The initial state is zero.
 * Each sum is itself a retention and runs on the chunkwise kernels (the two
 * anti-causal sums on the token-reversed sequence), in segments whose bounds are
 * multiples of the given chunk; on the MFMA kernels a chunk that is a multiple of
 * 64 is walked in 64-token pieces inside them (a chunk only blocks the sums: the
 * gradients are the same up to rounding).
 *   q, k : [B,H,L,dk]   v, d_o : [B,H,L,dv]   (in_dtype)
 *   dq, dk_out : [B,H,L,dk]   dv_out : [B,H,L,dv]   (out_dtype)
 * UNSUPPORTED unless dk and dv are multiples of 8 and dv <= RETENTION_MAX_DK.  Gradients must not
 * overlap the inputs, the workspace or each other.
 */
size_t retention_chunkwise_bwd_workspace_bytes(int B, int H, int L, int dk, int dv, int chunk,
                                               ret_dtype_t in_dtype);
ret_status_t retention_chunkwise_bwd(const void *q, const void *k, const void *v, const void *d_o,
                                     void *dq, void *dk_out, void *dv_out, int B, int H, int L,
                                     int dk, int dv, int chunk, const float *gamma,
                                     const float *theta, long long pos0, ret_dtype_t in_dtype,
                                     ret_dtype_t out_dtype, void *workspace, size_t workspace_bytes,
                                     void *hip_stream);

/*
 * The same gradients, reusing the segment states of the forward call
 * (retention_chunkwise, "Retentive Network" paper summary, Sec. 2.1 (3): the state
 * carried across chunks).  The dq sum carries sum_{m<=n} gamma^(n-m) v_m^T k~_m,
 * the transpose of the forward's state sum_{m<=n} gamma^(n-m) k~_m^T v_m, so with
 * the forward's states it needs no state pass of its own: a training step keeps
 * the forward's workspace (as it keeps activations) and hands it over here.
 *   fwd_workspace : the workspace of a retention_chunkwise call with the same q, k,
 *                   v (bf16), B, H, L, dk, dv, chunk, gamma, theta and pos0 and no
 *                   state_in, unchanged since (its first part holds the fp32 states
 *                   entering each segment, written by that call); read only.
 *                   Its content is not checked: other contents give other dq.
 *   fwd_workspace_bytes : its size (at least the forward's segment states).
 * Where the states are not usable (inputs on the vector path, or a forward plan
 * whose segments do not take the states in registers) the dq sum computes its own,
 * as retention_chunkwise_bwd does.  INVALID_ARG for a NULL or unaligned
 * fwd_workspace or one that overlaps a gradient or the backward's workspace;
 * WORKSPACE if it is too small.
 */
ret_status_t retention_chunkwise_bwd_saved(const void *q, const void *k, const void *v,
                                           const void *d_o, void *dq, void *dk_out, void *dv_out,
                                           int B, int H, int L, int dk, int dv, int chunk,
                                           const float *gamma, const float *theta, long long pos0,
                                           ret_dtype_t in_dtype, ret_dtype_t out_dtype,
                                           const void *fwd_workspace, size_t fwd_workspace_bytes,
                                           void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Gated multi-scale retention layer (Sec. 2.2), bf16 in and out:
 *   Q = X W_Q, K = X W_K, V = X W_V (head h = column block h of width dk / dv)
 *   head_h = chunkwise retention of (Q_h, K_h, V_h) with gamma_h, theta, pos0
 *   Y = GroupNorm per (token, head) with gn_eps (>= 0)
 *   out = (swish(X W_G) (.) Y) W_O,   swish(x) = x / (1 + exp(-x))
 * Weights are stored transposed ([out, in], one output column per row):
 *   x   : [B,L,d_model] bf16         y   : [B,L,d_model] bf16
 *   w_q, w_k : [H*dk, d_model] bf16   w_v, w_g : [H*dv, d_model] bf16
 *   w_o : [d_model, H*dv] bf16
 * UNSUPPORTED unless d_model, H*dk and H*dv are multiples of 128 and (dk, dv) is
 * one of the MFMA pairs listed under retention_parallel.
 * The four projections and W_O are plain GEMMs run through hipBLASLt; a shape
 * for which hipBLASLt offers no algorithm returns UNSUPPORTED.  When w_q,
 * w_k, w_v and w_g are stored back to back in that order (one fused
 * [2 H dk + 2 H dv, d_model] matrix), the projections run as one GEMM.  The first
 * call on a device creates that device's hipBLASLt handle, kept until the
 * process ends.  The workspace (size from msr_layer_fwd_workspace_bytes) holds
 * the projections [B*L][2 H dk + 2 H dv], the gated normalised heads
 * [B*L][H*dv], the chunkwise workspace and 32 MiB for hipBLASLt.
 */
size_t msr_layer_fwd_workspace_bytes(int B, int L, int d_model, int H, int dk, int dv,
                                     int chunk);
ret_status_t msr_layer_fwd(const void *x, const void *w_q, const void *w_k, const void *w_v,
                           const void *w_g, const void *w_o, void *y, int B, int L, int d_model,
                           int H, int dk, int dv, int chunk, const float *gamma,
                           const float *theta, long long pos0, float gn_eps, void *workspace,
                           size_t workspace_bytes, void *hip_stream);

/*
 * One decode step of the gated multi-scale retention layer (Sec. 2.2 with the
 * recurrent representation, Sec. 2.1 (2); "RetNet dual-mode hands-on manual",
 * Sec. 3.2 and 4.2: explicit per-sequence state, one token per step, replayed
 * as a captured graph).  Every sequence b advances by one token x[b]:
 *   q, k, v, g = x W_Q^T, x W_K^T, x W_V^T, x W_G^T   (per head: column blocks)
 *   per head: S <- gamma_h S + k_rot^T v,  o = q_rot S   (rotation at pos[b])
 *   y = (swish(g) (.) GroupNorm(o)) W_O^T
 * so that steps over tokens 0..t-1 from a zero state reproduce msr_layer_fwd's
 * outputs for those tokens (pos0 = 0).
 *   x : [B, d_model] bf16      y : [B, d_model] bf16      weights as msr_layer_fwd
 *   state : [B, H, dk, dv] fp32, DEVICE, read then overwritten in place
 *   pos : DEVICE int32 [B], the position of this step's token per sequence; when
 *         advance_pos != 0 the call adds 1 to every entry on the device after the
 *         step, so a captured call can be replayed without host updates
 * UNSUPPORTED unless d_model, H*dk and H*dv are multiples of 128, dk and dv are
 * multiples of 8 and dv <= 1024.  y, state, x and the workspace must not overlap.
 * The projections run through hipBLASLt as in msr_layer_fwd but are kept in
 * fp32 (a (token, head) row whose retention output nearly cancels is divided by
 * its small deviation in GroupNorm, which would magnify a bf16 rounding of q and
 * k); W_O takes the bf16 gated heads.
 */
size_t msr_layer_step_workspace_bytes(int B, int d_model, int H, int dk, int dv);
ret_status_t msr_layer_step(const void *x, const void *w_q, const void *w_k, const void *w_v,
                            const void *w_g, const void *w_o, void *y, float *state, int *pos,
                            int advance_pos, int B, int d_model, int H, int dk, int dv,
                            const float *gamma, const float *theta, float gn_eps, void *workspace,
                            size_t workspace_bytes, void *hip_stream);

/*
 * The pre-LN residual block around the gated layer (paper summary, the block
 * equations; FFN(X) = gelu(X W_1) W_2), bf16 in and out:
 *   Y = MSR(LN(X)) + X,   out = FFN(LN(Y)) + Y
 * LN: per token over d_model, (x - mean) / sqrt(var + ln_eps), biased variance,
 * no affine; gelu(x) = x Phi(x) (the exact form).  MSR as msr_layer_fwd.
 *   w_1 : [d_ffn, d_model] bf16   w_2 : [d_model, d_ffn] bf16   (stored [out, in])
 * UNSUPPORTED unless d_model, H*dk, H*dv and d_ffn are multiples of 128,
 * d_model <= 8192 and (dk, dv) is an MFMA pair.  out must not overlap x or the
 * workspace.  GEMMs run through hipBLASLt as in msr_layer_fwd.
 */
size_t retnet_block_fwd_workspace_bytes(int B, int L, int d_model, int H, int dk, int dv, int d_ffn,
                                        int chunk);
ret_status_t retnet_block_fwd(const void *x, const void *w_q, const void *w_k, const void *w_v,
                              const void *w_g, const void *w_o, const void *w_1, const void *w_2,
                              void *out, int B, int L, int d_model, int H, int dk, int dv, int d_ffn,
                              int chunk, const float *gamma, const float *theta, long long pos0,
                              float gn_eps, float ln_eps, void *workspace, size_t workspace_bytes,
                              void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* RETENTION_H_ */
