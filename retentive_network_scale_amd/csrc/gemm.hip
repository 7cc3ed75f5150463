// bf16 MFMA GEMM for the projections of the gated multi-scale retention layer
// ("Retentive Network" paper summary, Sec. 2.2: Q = X W_Q, K = X W_K, V = X W_V,
// the gate X W_G and the output projection (.) W_O).
//
//   C[M][N] = A[M][K] . W[N][K]^T     (A row-major, W stored [out][in]: both K-contiguous)
//
// One launch may cover several weight matrices side by side in N ("segments"),
// each with its own epilogue:
//   PLAIN  : C as bf16, row-major with leading dimension ld
//   HEADS  : row r = (b, l), column c = (h, j)  ->  out[((b*H + h)*L + l)*dh + j]
//   SWISH  : swish(C) = C / (1 + exp(-C)) as bf16, row-major
//
// Tiles: 128 x 128 per workgroup (4 waves, each 64 x 64 = 4 x 4 MFMA blocks of
// v_mfma_f32_16x16x32_bf16), K in steps of 64 staged through LDS, the next
// step's global loads held in registers while the current one is multiplied.
// The epilogue stages the fp32 tile through LDS so that stores are 16-byte
// and row-contiguous.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

typedef __attribute__((ext_vector_type(8))) __bf16 g_bf16x8;
typedef __attribute__((ext_vector_type(4))) float g_f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t g_u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t g_u32x2;

constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int GT = 256;
constexpr int GLD = GBK + 8;          // LDS row length (bf16) of the A / W tiles
constexpr int GCLD = GBN + 4;         // LDS row length (fp32) of the output tile

__device__ __forceinline__ g_f32x4 g_mfma(g_u32x4 a, g_u32x4 b, g_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(g_bf16x8, a),
                                                 __builtin_bit_cast(g_bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ g_u32x4 g_ld_op(const uint16_t *row, int k0, int g) {
  g_u32x2 lo = *(const g_u32x2 *)(row + k0 + 4 * g);
  g_u32x2 hi = *(const g_u32x2 *)(row + k0 + 16 + 4 * g);
  return g_u32x4{lo.x, lo.y, hi.x, hi.y};
}

__global__ __launch_bounds__(GT) void gemm_bf16_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * GBM * GLD > GBM * GCLD * 2
                                                         ? 2 * 2 * GBM * GLD
                                                         : GBM * GCLD * 2];
  uint16_t *As = smem;                       // [2][GBM][GLD]
  uint16_t *Ws = smem + 2 * GBM * GLD;       // [2][GBN][GLD]
  float *Cs = (float *)smem;                 // [GBM][GCLD] after the K loop

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wm = w >> 1, wn = w & 1;
  // XCD-aware order: each XCD takes a contiguous range of tiles (row-block major)
  const int per = (p.ntiles + 7) / 8;
  const int t = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= p.ntiles) return;
  const int nN = p.n_total / GBN;
  const int mt = t / nN, nt = t % nN;
  const int m0 = mt * GBM;
  int n0 = nt * GBN, sg = 0;
  while (sg + 1 < p.nseg && n0 >= p.seg[sg].n) {
    n0 -= p.seg[sg].n;
    ++sg;
  }
  const GemmSeg S = p.seg[sg];
  const uint16_t *A = p.A;
  const uint16_t *W = S.w;

  // global -> register tile loader: 128 rows x 64 cols bf16 = 1024 chunks of 16 B per operand
  uint4 ra[4], rw[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + GT * i, r = c >> 3, c8 = c & 7;
      const int gm = m0 + r;
      ra[i] = gm < p.M ? *(const uint4 *)(A + (long long)gm * p.K + k0 + 8 * c8) : make_uint4(0, 0, 0, 0);
      rw[i] = *(const uint4 *)(W + (long long)(n0 + r) * p.K + k0 + 8 * c8);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + GT * i, r = c >> 3, c8 = c & 7;
      *(uint4 *)(As + (buf * GBM + r) * GLD + 8 * c8) = ra[i];
      *(uint4 *)(Ws + (buf * GBN + r) * GLD + 8 * c8) = rw[i];
    }
  };

  g_f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = g_f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / GBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * GBK);
#pragma unroll
    for (int ks = 0; ks < GBK / 32; ++ks) {
      g_u32x4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = g_ld_op(As + (cur * GBM + wm * 64 + 16 * i + l16) * GLD, 32 * ks, g);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = g_ld_op(Ws + (cur * GBN + wn * 64 + 16 * j + l16) * GLD, 32 * ks, g);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = g_mfma(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // epilogue: acc -> LDS (fp32), then row-contiguous 16-byte stores
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) Cs[(wm * 64 + 16 * i + 4 * g + e) * GCLD + wn * 64 + 16 * j + l16] = acc[i][j][e];
  __syncthreads();
#pragma unroll
  for (int it = 0; it < (GBM * GBN / 8) / GT; ++it) {
    const int c = tid + GT * it, r = c / (GBN / 8), c8 = c % (GBN / 8);
    const int gm = m0 + r;
    if (gm >= p.M) continue;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = Cs[r * GCLD + 8 * c8 + e];
    if (S.kind == GEMM_SWISH)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = x[e] / (1.0f + __expf(-x[e]));
    uint4 o;
    o.x = pack_bf2(x[0], x[1]);
    o.y = pack_bf2(x[2], x[3]);
    o.z = pack_bf2(x[4], x[5]);
    o.w = pack_bf2(x[6], x[7]);
    const int gn = n0 + 8 * c8;
    long long off;
    if (S.kind == GEMM_HEADS) {
      const int b = gm / S.L, l = gm % S.L, h = gn / S.dh, j = gn % S.dh;
      off = (((long long)b * S.H + h) * S.L + l) * S.dh + j;
    } else {
      off = (long long)gm * S.ld + gn;
    }
    *(uint4 *)((uint16_t *)S.out + off) = o;
  }
}

hipError_t launch_gemm_bf16(const GemmArgs &args, hipStream_t st) {
  GemmArgs p = args;
  p.n_total = 0;
  for (int s = 0; s < p.nseg; ++s) p.n_total += p.seg[s].n;
  p.ntiles = ((p.M + GBM - 1) / GBM) * (p.n_total / GBN);
  const unsigned grid = (unsigned)(((p.ntiles + 7) / 8) * 8);
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3(grid), dim3(GT), 0, st, p);
  return hipGetLastError();
}

}  // namespace ret
