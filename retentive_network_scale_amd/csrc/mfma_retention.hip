// bf16 MFMA retention kernels for gfx950 (parallel and chunkwise forms).
//
// Pages: "Retentive Network" paper summary (blog.csdn.net), Sec. 2.1
// "Retention": parallel form (Q K^T (.) D) V with D_nm = gamma^(n-m) for n >= m,
// recurrent form S_n = gamma S_{n-1} + K_n^T V_n, and the chunkwise form
// (parallel inside a chunk, state carried across chunks); Sec. 2.2 (per-head
// GroupNorm).  "RetNet dual-mode hands-on manual", Sec. 2.2 (chunked training
// with the hidden state carried from chunk to chunk).
//
// Chunkwise identity used (from the recurrence by induction; chunk c covers
// tokens c0..c0+Cc-1 and S_c is the state entering it):
//   o_{c0+j} = gamma^(j+1) q_{c0+j} S_c + sum_{i<=j} gamma^(j-i) (q_{c0+j}.k_{c0+i}) v_{c0+i}
//   S_{c+1}  = gamma^Cc S_c + sum_i gamma^(Cc-1-i) k_{c0+i}^T v_{c0+i}
// and, for a segment of whole chunks holding tokens s0..s1-1,
//   S(s1) = gamma^(s1-s0) S(s0) + sum_t gamma^(s1-1-t) k_t^T v_t.
//
// Work layout.  One workgroup = 8 waves (512 threads).  The output is built
// transposed, O^T[dv][query], so that:
//   * the decayed scores S^T = K Q^T come out of the MFMA in the lane layout
//     of the B operand of O^T += V^T P^T (no register shuffles),
//   * the fp32 state S[dk][dv], kept in MFMA accumulators, is already in the
//     lane layout of the A operand of the cross term O^T += S^T Q^T.
// Every wave owns RW = DVW/8 rows of O^T (dv) and the matching columns of the
// state.  Scores of a 64x64 block are split over the 8 waves (16 queries x 32
// keys each) and shared through LDS in bf16.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l, g = l/16: A holds A[l%16][K-set],
// B holds B[K-set][l%16], D holds D[4g+i][l%16].  The K-set of lane group g in
// the k-step is {4g..4g+3, 16+4g..16+4g+3}; any K permutation shared by A and
// B gives the same product, and this one maps a pair of D blocks straight
// onto an operand.
//
// Chunkwise runs as three launches (the cross-chunk carry over segments):
//   1. seg_state: per (b, h, segment, dv slice) the segment's own state
//      sum_t gamma^(s1-1-t) k_t^T v_t  (zero incoming state) -> workspace;
//   2. seg_scan : per state element, S_in(s+1) = gamma^len(s) S_in(s) + dS(s),
//      written back in place (exclusive) plus the final state;
//   3. seg_out  : per segment, the chunk loop above, starting from S_in.
#include "common.hpp"
#include "launch.hpp"

namespace ret {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int NT = 512;   // threads per workgroup
constexpr int BT = 64;    // query / key block (tokens)
constexpr int LDT = BT + 8;  // row length (bf16) of token-minor LDS tiles

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Operand for lane group g from a bf16 row in LDS: elements [k0+4g, +4) and [k0+16+4g, +4).
__device__ __forceinline__ u32x4 ld_op(const uint16_t *row, int k0, int g) {
  u32x2 lo = *(const u32x2 *)(row + k0 + 4 * g);
  u32x2 hi = *(const u32x2 *)(row + k0 + 16 + 4 * g);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
  return u32x2{pack_bf2(a, b), pack_bf2(c, d)};
}

// gamma^d for integer d >= 0, d == 0 -> 1 (so gamma = 0 gives the identity).
__device__ __forceinline__ float dpow(float lg2, int d) {
  return d == 0 ? 1.0f : exp2f((float)d * lg2);
}

template <int DK, int DVW>
struct Tile {
  static constexpr int RW = DVW / 8;   // O^T rows / state columns per wave
  static constexpr int RB = RW / 16;   // 16-row blocks per wave
  static constexpr int KS = DK / 32;   // k-steps over dk
  static constexpr int DKB = DK / 16;  // 16-row blocks of dk
  static constexpr int LDQ = DK + 8;   // row length (bf16) of token-major LDS tiles
  static_assert(RW % 16 == 0 && DK % 32 == 0, "tile shape");
};

// Stage a 64-token block of a [tokens][D] bf16 tensor into LDS.
//   rows (if ROWS): dst[r][0..D)   (token-major, row length D+8)
//   trans (if TRANS): dstT[d][0..64) (token-minor, row length LDT), scaled per token by zeta
// Tokens at or beyond `valid` are zero.  Rotation (ROT) by the xPOS phase at
// absolute position pos_base + r uses the fp32 theta table in LDS.
template <int D, bool ROWS, bool TRANS, bool ROT, bool LO = false>
__device__ __forceinline__ void stage(const uint16_t *src, long long stride, int valid,
                                      long long pos_base, const float *theta_s, uint16_t *dst,
                                      uint16_t *dstT, const float *zeta, uint16_t *dstLo = nullptr) {
  constexpr int C8 = D / 8;
  for (int idx = threadIdx.x; idx < 16 * C8; idx += NT) {
    const int c8 = idx % C8, kq = idx / C8;
    float x[4][8];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * kq + rr;
      if (r < valid) {
        const uint4 u = *(const uint4 *)(src + (long long)r * stride + 8 * c8);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[rr][2 * e] = __uint_as_float(w[e] << 16);
          x[rr][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
        if constexpr (ROT) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            float c, s;
            rot_cs<false>(pos_base + r, theta_s[4 * c8 + p], c, s);
            const float re = x[rr][2 * p], im = x[rr][2 * p + 1];
            x[rr][2 * p] = re * c - im * s;
            x[rr][2 * p + 1] = re * s + im * c;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[rr][e] = 0.0f;
      }
    }
    if constexpr (ROWS) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        uint4 o;
        o.x = pack_bf2(x[rr][0], x[rr][1]);
        o.y = pack_bf2(x[rr][2], x[rr][3]);
        o.z = pack_bf2(x[rr][4], x[rr][5]);
        o.w = pack_bf2(x[rr][6], x[rr][7]);
        *(uint4 *)(dst + (4 * kq + rr) * (D + 8) + 8 * c8) = o;
        if constexpr (LO) {
          // x - bf16(x), rounded to bf16: hi + lo carries ~16 significant bits
          const uint32_t hw[4] = {o.x, o.y, o.z, o.w};
          uint4 lo;
          uint32_t lw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            lw[e] = pack_bf2(x[rr][2 * e] - __uint_as_float(hw[e] << 16),
                             x[rr][2 * e + 1] - __uint_as_float(hw[e] & 0xffff0000u));
          lo.x = lw[0]; lo.y = lw[1]; lo.z = lw[2]; lo.w = lw[3];
          *(uint4 *)(dstLo + (4 * kq + rr) * (D + 8) + 8 * c8) = lo;
        }
      }
    }
    if constexpr (TRANS) {
      float z[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) z[rr] = zeta ? zeta[4 * kq + rr] : 1.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *(u32x2 *)(dstT + (8 * c8 + e) * LDT + 4 * kq) =
            pack4(x[0][e] * z[0], x[1][e] * z[1], x[2][e] * z[2], x[3][e] * z[3]);
    }
  }
}

struct TaskGeom {
  int nseg, seg_chunks, nsplit, nqb, ntasks;
};

// XCD-aware task order: workgroup ids are dealt round-robin to the 8 XCDs, so
// give each XCD a contiguous range of tasks (neighbouring tasks share K/V in
// that XCD's L2).  The grid is ntasks rounded up to a multiple of 8; ids that
// map past the last task exit.
__device__ __forceinline__ int xcd_task(int bid, int ntasks) {
  const int per = (ntasks + 7) / 8;
  const int t = (bid % 8) * per + bid / 8;
  return t < ntasks ? t : -1;
}

static inline unsigned xcd_grid(int ntasks) { return (unsigned)(((ntasks + 7) / 8) * 8); }

// ---------------------------------------------------------------- main tile kernel
// PAR: parallel form, one task = (b, h, 64-query block).  Otherwise chunkwise
// output pass, one task = (b, h, segment, dv slice), state from `seg_state`.
// SPLIT: scores from hi + lo bf16 parts of the rotated q and k (three MFMAs per
// k-step), accurate to ~2^-16 instead of the ~2^-8 of one bf16 rounding of the
// rotated values.  Used when GroupNorm follows: rows whose variance is near eps
// magnify absolute score errors by ~1/sqrt(eps).
template <int DK, int DVW, bool PAR, bool SPLIT>
__global__ __launch_bounds__(NT) void tile_kernel(RetArgs a, TaskGeom geo, const float *seg_state) {
  using T = Tile<DK, DVW>;
  constexpr int LDQ = T::LDQ, RW = T::RW, RB = T::RB, KS = T::KS, DKB = T::DKB;
  // Chunkwise: Qs (rotated query block, bf16) is read only before the key loop and
  // Kt only inside it, so they share storage.  Parallel: the query block is staged
  // through Ks / KsL, which are free until the key loop starts.
  constexpr int QK_SZ = PAR ? 8 : (BT * LDQ > DK * LDT ? BT * LDQ : DK * LDT);
  __shared__ __attribute__((aligned(16))) uint16_t QKs[QK_SZ];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BT * LDQ];
  __shared__ __attribute__((aligned(16))) uint16_t KsL[SPLIT ? BT * LDQ : 8];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DVW * LDT];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[BT * LDT];
  uint16_t *const Qs = PAR ? Ks : QKs;
  uint16_t *const Kt = QKs;
  __shared__ float theta_s[DK / 2];
  __shared__ float zeta_s[BT];
  __shared__ float red[8][BT];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int task = xcd_task(blockIdx.x, geo.ntasks);
  if (task < 0) return;

  int bh, split = 0, seg = 0, qb_only = 0;
  if constexpr (PAR) {
    bh = task / geo.nqb;
    qb_only = geo.nqb - 1 - task % geo.nqb;  // longest blocks first
  } else {
    split = task % geo.nsplit;
    seg = (task / geo.nsplit) % geo.nseg;
    bh = task / (geo.nsplit * geo.nseg);
  }
  const int b = bh / a.H, h = bh % a.H;
  const float lg = safe_log2(a.gamma[h]);
  const uint16_t *q = (const uint16_t *)a.q + (long long)b * a.q_sb + (long long)h * a.q_sh;
  const uint16_t *k = (const uint16_t *)a.k + (long long)b * a.q_sb + (long long)h * a.q_sh;
  const uint16_t *v = (const uint16_t *)a.v + (long long)b * a.v_sb + (long long)h * a.v_sh + split * DVW;
  const long long obase = (long long)b * a.o_sb + (long long)h * a.o_sh + split * DVW;
  if (a.use_theta)
    for (int i = tid; i < DK / 2; i += NT) theta_s[i] = a.theta[i];

  // fp32 state S[dk][w*RW + dv'] in D layout: st[dkb][rb][i] = S[16dkb+4g+i][w*RW+16rb+l16]
  f32x4 st[PAR ? 1 : DKB][PAR ? 1 : RB];
  int t_lo, t_hi;  // token range of the task
  if constexpr (PAR) {
    t_lo = 0;
    t_hi = a.L;
  } else {
    const int c_lo = seg * geo.seg_chunks;
    t_lo = c_lo * a.chunk;
    t_hi = min(a.L, (c_lo + geo.seg_chunks) * a.chunk);
    const float *S_in = seg_state + ((long long)bh * geo.nseg + seg) * DK * a.dv + split * DVW;
#pragma unroll
    for (int dkb = 0; dkb < DKB; ++dkb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          st[dkb][rb][i] = S_in[(long long)(16 * dkb + 4 * g + i) * a.dv + w * RW + 16 * rb + l16];
  }
  __syncthreads();

  const int qblk = w & 3, kh = w >> 2;  // score split: 16 queries x 32 keys per wave
  for (int c0 = t_lo; c0 < t_hi; c0 += (PAR ? a.L : a.chunk)) {
    const int Cc = PAR ? a.L : min(a.chunk, a.L - c0);
    const bool carry = !PAR && (c0 + Cc < t_hi);  // state needed after this chunk
    const int nqb_c = (Cc + BT - 1) / BT;
    for (int qb = (PAR ? qb_only : 0); qb < (PAR ? qb_only + 1 : nqb_c); ++qb) {
      const int q0 = c0 + qb * BT;  // first query of the block
      __syncthreads();
      if (a.use_theta)
        stage<DK, true, false, true, SPLIT>(q + (long long)q0 * a.q_sn, a.q_sn, min(BT, c0 + Cc - q0),
                                            a.pos0 + q0, theta_s, Qs, nullptr, nullptr, KsL);
      else
        stage<DK, true, false, false, SPLIT>(q + (long long)q0 * a.q_sn, a.q_sn, min(BT, c0 + Cc - q0), 0,
                                             theta_s, Qs, nullptr, nullptr, KsL);
      __syncthreads();
      // this wave's query operand for the scores (hi, and lo when SPLIT)
      u32x4 qreg[KS], qlo[SPLIT ? KS : 1];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qreg[ks] = ld_op(Qs + (16 * qblk + l16) * LDQ, 32 * ks, g);
        if constexpr (SPLIT) qlo[ks] = ld_op(KsL + (16 * qblk + l16) * LDQ, 32 * ks, g);
      }
      // O^T accumulators: ot[rb][qb4][i] = O^T[w*RW+16rb+4g+i][16qb4+l16]
      f32x4 ot[RB][4];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int qb4 = 0; qb4 < 4; ++qb4) ot[rb][qb4] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      // The state still holds S_c here: the chunk's key blocks are folded into it
      // only while the last query block of the chunk runs (it visits them all).
      const bool last_qb = qb == nqb_c - 1;
      if constexpr (!PAR) {
        // cross term gamma^(j+1) q S_c; A operand = S_c^T in bf16, straight from the
        // accumulators: D blocks (2ks, rb) and (2ks+1, rb) are the two halves of k-step ks
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 as[RB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const f32x4 lo = st[2 * ks][rb], hi = st[2 * ks + 1][rb];
            as[rb] = u32x4{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(hi[0], hi[1]),
                           pack_bf2(hi[2], hi[3])};
          }
#pragma unroll
          for (int qb4 = 0; qb4 < 4; ++qb4) {
            const u32x4 bq = ld_op(Qs + (16 * qb4 + l16) * LDQ, 32 * ks, g);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) ot[rb][qb4] = mfma(as[rb], bq, ot[rb][qb4]);
          }
        }
#pragma unroll
        for (int qb4 = 0; qb4 < 4; ++qb4) {
          const float xi = dpow(lg, q0 - c0 + 16 * qb4 + l16 + 1);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) ot[rb][qb4] *= xi;
        }
        if (carry && last_qb) {
          const float gc = dpow(lg, Cc);
#pragma unroll
          for (int dkb = 0; dkb < DKB; ++dkb)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) st[dkb][rb] *= gc;
        }
      }
      for (int kb = 0; kb <= qb; ++kb) {
        const int k0 = c0 + kb * BT;
        const int kvalid = min(BT, c0 + Cc - k0);
        const bool upd = carry && last_qb;
        __syncthreads();
        if (upd)
          for (int r = tid; r < BT; r += NT) zeta_s[r] = r < kvalid ? dpow(lg, Cc - 1 - (k0 - c0 + r)) : 0.0f;
        __syncthreads();
        const uint16_t *kp = k + (long long)k0 * a.q_sn;
        if (a.use_theta) {
          if (upd)
            stage<DK, true, true, true, SPLIT>(kp, a.q_sn, kvalid, a.pos0 + k0, theta_s, Ks, Kt, zeta_s, KsL);
          else
            stage<DK, true, false, true, SPLIT>(kp, a.q_sn, kvalid, a.pos0 + k0, theta_s, Ks, nullptr, nullptr,
                                                KsL);
        } else {
          if (upd)
            stage<DK, true, true, false, SPLIT>(kp, a.q_sn, kvalid, 0, theta_s, Ks, Kt, zeta_s, KsL);
          else
            stage<DK, true, false, false, SPLIT>(kp, a.q_sn, kvalid, 0, theta_s, Ks, nullptr, nullptr, KsL);
        }
        stage<DVW, false, true, false>(v + (long long)k0 * a.v_sn, a.v_sn, kvalid, 0, theta_s, nullptr, Vt,
                                       nullptr);
        __syncthreads();
        // scores S^T[key][query] for keys 32kh..+32, queries 16qblk..+16; decay, mask, -> Ps
#pragma unroll
        for (int kb16 = 0; kb16 < 2; ++kb16) {
          f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const u32x4 ak = ld_op(Ks + (32 * kh + 16 * kb16 + l16) * LDQ, 32 * ks, g);
            s = mfma(ak, qreg[ks], s);
            if constexpr (SPLIT) {
              s = mfma(ld_op(KsL + (32 * kh + 16 * kb16 + l16) * LDQ, 32 * ks, g), qreg[ks], s);
              s = mfma(ak, qlo[ks], s);
            }
          }
          const int n = q0 + 16 * qblk + l16;
          const int m0 = k0 + 32 * kh + 16 * kb16 + 4 * g;
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d = n - (m0 + i);
            p[i] = d >= 0 ? s[i] * dpow(lg, d) : 0.0f;
          }
          *(u32x2 *)(Ps + (16 * qblk + l16) * LDT + 32 * kh + 16 * kb16 + 4 * g) = pack4(p[0], p[1], p[2], p[3]);
        }
        __syncthreads();
        // O^T += V^T P^T
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4 av[RB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) av[rb] = ld_op(Vt + (w * RW + 16 * rb + l16) * LDT, 32 * ks, g);
#pragma unroll
          for (int qb4 = 0; qb4 < 4; ++qb4) {
            const u32x4 bp = ld_op(Ps + (16 * qb4 + l16) * LDT, 32 * ks, g);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) ot[rb][qb4] = mfma(av[rb], bp, ot[rb][qb4]);
          }
        }
        if constexpr (!PAR) {
          if (upd) {
            // S += (zeta K)^T V over this key block
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              u32x4 bv[RB];
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) bv[rb] = ld_op(Vt + (w * RW + 16 * rb + l16) * LDT, 32 * ks, g);
#pragma unroll
              for (int dkb = 0; dkb < DKB; ++dkb) {
                const u32x4 ak = ld_op(Kt + (16 * dkb + l16) * LDT, 32 * ks, g);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) st[dkb][rb] = mfma(ak, bv[rb], st[dkb][rb]);
              }
            }
          }
        }
      }
      // ---- epilogue: optional GroupNorm over dv (only when this block holds all of dv), store
      const int nvalid = min(BT, c0 + Cc - q0);
      if (a.use_gn && DVW == a.dv) {
        float mean[4], inv[4];
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
          float part[4];
#pragma unroll
          for (int qb4 = 0; qb4 < 4; ++qb4) {
            float sacc = 0.0f;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float x = ot[rb][qb4][i];
                sacc += pass == 0 ? x : (x - mean[qb4]) * (x - mean[qb4]);
              }
            sacc += __shfl_xor(sacc, 16, 64);
            sacc += __shfl_xor(sacc, 32, 64);
            part[qb4] = sacc;
          }
          __syncthreads();
          if (g == 0)
#pragma unroll
            for (int qb4 = 0; qb4 < 4; ++qb4) red[w][16 * qb4 + l16] = part[qb4];
          __syncthreads();
#pragma unroll
          for (int qb4 = 0; qb4 < 4; ++qb4) {
            float tot = 0.0f;
#pragma unroll
            for (int ww = 0; ww < 8; ++ww) tot += red[ww][16 * qb4 + l16];
            tot /= (float)a.dv;
            if (pass == 0)
              mean[qb4] = tot;
            else
              inv[qb4] = 1.0f / sqrtf(tot + a.gn_eps);
          }
        }
#pragma unroll
        for (int qb4 = 0; qb4 < 4; ++qb4)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) ot[rb][qb4] = (ot[rb][qb4] - mean[qb4]) * inv[qb4];
      }
#pragma unroll
      for (int qb4 = 0; qb4 < 4; ++qb4) {
        const int r = 16 * qb4 + l16;
        if (r < nvalid) {
          const long long ro = obase + (long long)(q0 + r) * a.o_sn;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int col = w * RW + 16 * rb + 4 * g;
            const f32x4 x = ot[rb][qb4];
            if (a.out_bf16)
              *(u32x2 *)((uint16_t *)a.o + ro + col) = pack4(x[0], x[1], x[2], x[3]);
            else
              *(float4 *)((float *)a.o + ro + col) = make_float4(x[0], x[1], x[2], x[3]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- pass 1: segment states
template <int DK, int DVW>
__global__ __launch_bounds__(NT) void seg_state_kernel(RetArgs a, TaskGeom geo, float *seg_state) {
  using T = Tile<DK, DVW>;
  constexpr int RW = T::RW, RB = T::RB, DKB = T::DKB;
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DVW * LDT];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[DK * LDT];
  __shared__ float theta_s[DK / 2];
  __shared__ float zeta_s[BT];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int task = xcd_task(blockIdx.x, geo.ntasks);
  if (task < 0) return;
  const int split = task % geo.nsplit;
  const int seg = (task / geo.nsplit) % geo.nseg;
  const int bh = task / (geo.nsplit * geo.nseg);
  const int b = bh / a.H, h = bh % a.H;
  const float lg = safe_log2(a.gamma[h]);
  const uint16_t *k = (const uint16_t *)a.k + (long long)b * a.q_sb + (long long)h * a.q_sh;
  const uint16_t *v = (const uint16_t *)a.v + (long long)b * a.v_sb + (long long)h * a.v_sh + split * DVW;
  if (a.use_theta)
    for (int i = tid; i < DK / 2; i += NT) theta_s[i] = a.theta[i];
  const int t_lo = seg * geo.seg_chunks * a.chunk;
  const int t_hi = min(a.L, (seg + 1) * geo.seg_chunks * a.chunk);
  f32x4 st[DKB][RB];
#pragma unroll
  for (int dkb = 0; dkb < DKB; ++dkb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) st[dkb][rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = t_lo; k0 < t_hi; k0 += BT) {
    const int kvalid = min(BT, t_hi - k0);
    __syncthreads();
    for (int r = tid; r < BT; r += NT) zeta_s[r] = r < kvalid ? dpow(lg, t_hi - 1 - (k0 + r)) : 0.0f;
    __syncthreads();
    if (a.use_theta)
      stage<DK, false, true, true>(k + (long long)k0 * a.q_sn, a.q_sn, kvalid, a.pos0 + k0, theta_s, nullptr,
                                   Kt, zeta_s);
    else
      stage<DK, false, true, false>(k + (long long)k0 * a.q_sn, a.q_sn, kvalid, 0, theta_s, nullptr, Kt,
                                    zeta_s);
    stage<DVW, false, true, false>(v + (long long)k0 * a.v_sn, a.v_sn, kvalid, 0, theta_s, nullptr, Vt,
                                   nullptr);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 bv[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) bv[rb] = ld_op(Vt + (w * RW + 16 * rb + l16) * LDT, 32 * ks, g);
#pragma unroll
      for (int dkb = 0; dkb < DKB; ++dkb) {
        const u32x4 ak = ld_op(Kt + (16 * dkb + l16) * LDT, 32 * ks, g);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) st[dkb][rb] = mfma(ak, bv[rb], st[dkb][rb]);
      }
    }
  }
  float *dst = seg_state + ((long long)bh * geo.nseg + seg) * DK * a.dv + split * DVW;
#pragma unroll
  for (int dkb = 0; dkb < DKB; ++dkb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[(long long)(16 * dkb + 4 * g + i) * a.dv + w * RW + 16 * rb + l16] = st[dkb][rb][i];
}

// ---------------------------------------------------------------- pass 2: scan over segments
// In place: ws[bh][s] holds the segment's own state on entry and the state
// entering segment s on exit.  Also writes the state after the last token.
__global__ __launch_bounds__(256) void seg_scan_kernel(RetArgs a, TaskGeom geo, float *ws, const float *state_in,
                                                       float *state_out) {
  const long long SZ = (long long)a.dk * a.dv;
  const long long n4 = SZ / 4;
  const int bh = blockIdx.y;
  const float lg = safe_log2(a.gamma[bh % a.H]);
  const int seg_len = geo.seg_chunks * a.chunk;
  const float g_full = dpow(lg, seg_len);
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += (long long)gridDim.x * blockDim.x) {
    float4 run = state_in ? ((const float4 *)(state_in + (long long)bh * SZ))[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 *base = (float4 *)(ws + (long long)bh * geo.nseg * SZ);
    int s = 0;
    constexpr int U = 4;
    for (; s + U <= geo.nseg; s += U) {
      float4 d[U];
#pragma unroll
      for (int u = 0; u < U; ++u) d[u] = base[(long long)(s + u) * n4 + e];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        base[(long long)(s + u) * n4 + e] = run;
        const int len = min(a.L, (s + u + 1) * seg_len) - (s + u) * seg_len;
        const float gm = len == seg_len ? g_full : dpow(lg, len);
        run.x = gm * run.x + d[u].x;
        run.y = gm * run.y + d[u].y;
        run.z = gm * run.z + d[u].z;
        run.w = gm * run.w + d[u].w;
      }
    }
    for (; s < geo.nseg; ++s) {
      const float4 d = base[(long long)s * n4 + e];
      base[(long long)s * n4 + e] = run;
      const int len = min(a.L, (s + 1) * seg_len) - s * seg_len;
      const float gm = dpow(lg, len);
      run.x = gm * run.x + d.x;
      run.y = gm * run.y + d.y;
      run.z = gm * run.z + d.z;
      run.w = gm * run.w + d.w;
    }
    if (state_out) ((float4 *)(state_out + (long long)bh * SZ))[e] = run;
  }
}

// GroupNorm of output rows in place, for chunkwise launches whose dv is split
// over several workgroups.  One block per (b, h, token) row.
__global__ __launch_bounds__(256) void gn_rows_kernel(RetArgs a) {
  __shared__ float red[4];
  const long long row = blockIdx.x;
  const int n = (int)(row % a.L);
  const int bh = (int)(row / a.L);
  const long long off = (long long)(bh / a.H) * a.o_sb + (long long)(bh % a.H) * a.o_sh + (long long)n * a.o_sn;
  float x[RETENTION_MAX_DV / 256];
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < RETENTION_MAX_DV / 256; ++c) {
    const int j = threadIdx.x + 256 * c;
    x[c] = j < a.dv ? load_elem(a.o, off + j, a.out_bf16) : 0.0f;
    s += x[c];
  }
  const float mean = block_sum<256>(s, red) / (float)a.dv;
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < RETENTION_MAX_DV / 256; ++c) {
    const int j = threadIdx.x + 256 * c;
    if (j < a.dv) q += (x[c] - mean) * (x[c] - mean);
  }
  const float inv = 1.0f / sqrtf(block_sum<256>(q, red) / (float)a.dv + a.gn_eps);
#pragma unroll
  for (int c = 0; c < RETENTION_MAX_DV / 256; ++c) {
    const int j = threadIdx.x + 256 * c;
    if (j < a.dv) store_elem(a.o, off + j, (x[c] - mean) * inv, a.out_bf16);
  }
}

// ---------------------------------------------------------------- dispatch
bool mfma_supported(int dk, int dv) {
  return (dk == 64 && dv == 128) || (dk == 128 && dv == 128) ||
         (dk == 128 && dv == 256) || (dk == 256 && dv == 256) || (dk == 256 && dv == 512);
}

// dv columns per workgroup in the chunkwise kernels: the fp32 state slice
// DK x DVW lives in the accumulators of 8 waves (<= 64 registers each).
static int chunk_dvw(int dk, int dv) {
  int dvw = dv;
  while ((long long)dk * dvw > 128 * 256) dvw /= 2;
  return dvw;
}

ChunkPlan chunk_plan(int B, int H, int L, int dk, int dv, int chunk) {
  ChunkPlan p;
  const int nsplit = dv / chunk_dvw(dk, dv);
  const int nchunks = (L + chunk - 1) / chunk;
  const int units = B * H * nsplit;
  const int target = 256;  // one workgroup per CU
  int nseg = (target + units - 1) / units;
  if (nseg > nchunks) nseg = nchunks;
  if (nseg < 1) nseg = 1;
  p.seg_chunks = (nchunks + nseg - 1) / nseg;
  p.nseg = (nchunks + p.seg_chunks - 1) / p.seg_chunks;
  p.ws_bytes = (size_t)B * H * p.nseg * dk * dv * sizeof(float);
  return p;
}

template <int DK, int DV>
static hipError_t run_parallel(const RetArgs &a, hipStream_t st) {
  TaskGeom geo{1, 1, 1, (a.L + BT - 1) / BT, 0};
  geo.ntasks = a.B * a.H * geo.nqb;
  if (a.use_gn)
    hipLaunchKernelGGL((tile_kernel<DK, DV, true, true>), dim3(xcd_grid(geo.ntasks)), dim3(NT), 0, st, a, geo,
                       nullptr);
  else
    hipLaunchKernelGGL((tile_kernel<DK, DV, true, false>), dim3(xcd_grid(geo.ntasks)), dim3(NT), 0, st, a, geo,
                       nullptr);
  return hipGetLastError();
}

template <int DK, int DVW>
static hipError_t run_chunkwise(const RetArgs &a, const ChunkPlan &p, float *ws, const float *state_in,
                                float *state_out, hipStream_t st) {
  TaskGeom geo{p.nseg, p.seg_chunks, a.dv / DVW, 1, 0};
  geo.ntasks = a.B * a.H * geo.nseg * geo.nsplit;
  const unsigned nblk = xcd_grid(geo.ntasks);
  hipLaunchKernelGGL((seg_state_kernel<DK, DVW>), dim3(nblk), dim3(NT), 0, st, a, geo, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n4 = (long long)a.dk * a.dv / 4;
  const int gx = (int)((n4 + 255) / 256);
  hipLaunchKernelGGL(seg_scan_kernel, dim3(gx, a.B * a.H), dim3(256), 0, st, a, geo, ws, state_in, state_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  RetArgs a2 = a;
  const bool split_gn = a.use_gn && DVW != a.dv;
  if (split_gn) a2.use_gn = 0;
  if (a.use_gn)
    hipLaunchKernelGGL((tile_kernel<DK, DVW, false, true>), dim3(nblk), dim3(NT), 0, st, a2, geo, ws);
  else
    hipLaunchKernelGGL((tile_kernel<DK, DVW, false, false>), dim3(nblk), dim3(NT), 0, st, a2, geo, ws);
  e = hipGetLastError();
  if (e != hipSuccess || !split_gn) return e;
  hipLaunchKernelGGL(gn_rows_kernel, dim3((unsigned)((long long)a.B * a.H * a.L)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_mfma_parallel(const RetArgs &a, hipStream_t st) {
  if (a.dk == 64 && a.dv == 128) return run_parallel<64, 128>(a, st);
  if (a.dk == 128 && a.dv == 128) return run_parallel<128, 128>(a, st);
  if (a.dk == 128 && a.dv == 256) return run_parallel<128, 256>(a, st);
  if (a.dk == 256 && a.dv == 256) return run_parallel<256, 256>(a, st);
  if (a.dk == 256 && a.dv == 512) return run_parallel<256, 512>(a, st);
  return hipErrorNotSupported;
}

hipError_t launch_mfma_chunkwise(const RetArgs &a, const ChunkPlan &p, void *ws, const float *state_in,
                                 float *state_out, hipStream_t st) {
  float *w = (float *)ws;
  if (a.dk == 64 && a.dv == 128) return run_chunkwise<64, 128>(a, p, w, state_in, state_out, st);
  if (a.dk == 128 && a.dv == 128) return run_chunkwise<128, 128>(a, p, w, state_in, state_out, st);
  if (a.dk == 128 && a.dv == 256) return run_chunkwise<128, 256>(a, p, w, state_in, state_out, st);
  if (a.dk == 256 && a.dv == 256) return run_chunkwise<256, 128>(a, p, w, state_in, state_out, st);
  if (a.dk == 256 && a.dv == 512) return run_chunkwise<256, 128>(a, p, w, state_in, state_out, st);
  return hipErrorNotSupported;
}

}  // namespace ret
