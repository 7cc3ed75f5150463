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
//   * a chunk state stored as bf16 S^T[dv][dk] is directly the A operand of
//     the cross term O^T += S^T Q^T.
// Every wave owns RW = DV/8 rows of O^T (dv).  Scores of a 64x64 block are
// split over the 8 waves (16 queries x 32 keys each) and shared through LDS.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l, g = l/16: A holds A[l%16][K-set],
// B holds B[K-set][l%16], D holds D[4g+i][l%16].  The K-set of lane group g in
// the k-step is {4g..4g+3, 16+4g..16+4g+3}; any K permutation shared by A and
// B gives the same product, and this one maps a pair of D blocks straight
// onto an operand.
//
// Chunkwise runs as three launches (the cross-chunk carry over segments of
// whole chunks):
//   1. seg_state: per (b, h, segment, dv slice) the segment's own state
//      sum_t gamma^(s1-1-t) k_t^T v_t  (zero incoming state) -> workspace;
//   2. seg_scan : per state element, S_in(s+1) = gamma^len(s) S_in(s) + dS(s),
//      written back in place (exclusive) plus the final state;
//   3. seg_out  : per segment, the chunk loop, starting from S_in, with the
//      fp32 state in MFMA accumulators (it is then also the A operand of the
//      cross term, converted to bf16).
// The parallel form is the query-block kernel: one task per (b, h, 64-query
// block), key blocks up to the diagonal, no state.
#include <map>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace ret {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int NT = 512;   // threads per workgroup
constexpr int BT = 64;    // query / key block (tokens)
// LDS row lengths (bf16).  MFMA operands are read as 8-byte pieces from 16
// consecutive rows; a row stride of 34 dwords (mod 32: 2) puts those 16 reads
// on 32 distinct banks.  Rows are therefore only 8-byte aligned and every LDS
// access is at most 8 bytes wide.
constexpr int LDT = BT + 4;  // token-minor tiles (Ps, transposed keys): 136 bytes

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

// The same operand from a row-major tile T[k][m] (rows = the K index, pitch ldr
// elements): lane group g needs T[k0+4g+j][m0+l16] and T[k0+16+4g+j][m0+l16],
// j < 4.  ds_read_b64_tr_b16 returns to lane r of a 16-lane group element j of
// the 8-byte piece addressed by lane 4j + r/4; so lane p points at row
// k0 + 4g + p/4, columns m0 + 4(p%4) .. +3 (8-byte aligned).  Conflict-free
// when the pitch in dwords is 8 mod 32.
typedef short tr_v4s __attribute__((ext_vector_type(4)));
// Row pitch (elements) of a row-major tile of D columns for ld_op_tr: the
// smallest length >= D whose dword count is 8 mod 32.
__host__ __device__ constexpr int tr_pitch(int D) { return 2 * (((D / 2 - 8 + 31) / 32) * 32 + 8); }
__device__ __forceinline__ u32x4 ld_op_tr(const uint16_t *T, int ldr, int k0, int m0, int g, int l16) {
  const uint16_t *p0 = T + (k0 + 4 * g + (l16 >> 2)) * ldr + m0 + 4 * (l16 & 3);
  const tr_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr_v4s *)p0);
  const tr_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr_v4s *)(p0 + 16 * ldr));
  const u32x2 l = __builtin_bit_cast(u32x2, lo), h = __builtin_bit_cast(u32x2, hi);
  return u32x4{l.x, l.y, h.x, h.y};
}

__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
  return u32x2{pack_bf2(a, b), pack_bf2(c, d)};
}

// gamma^d for integer d >= 0, d == 0 -> 1 (so gamma = 0 gives the identity).
// Raw v_exp_f32: results below the fp32 normal range flush to 0, far below any
// term they would be added to.
__device__ __forceinline__ float dpow(float lg2, int d) {
  return d == 0 ? 1.0f : __builtin_amdgcn_exp2f((float)d * lg2);
}

// Rotation tables of a kernel: theta_s[i] = theta_i and step_s[i] = (cos theta_i,
// sin theta_i) (libm, to an ulp).  A thread rotating consecutive tokens p0,
// p0+1, ... of pair i takes the angle of the first from its fp64-reduced
// revolutions, frac(p0 theta_i / 2pi), and the hardware v_cos/v_sin, then steps
// to each next token by a complex multiplication with step_s[i]: a few fp32
// roundings per token, far below the bf16 rounding of the result, and one
// hardware sine/cosine pair per run of tokens instead of one per token.
__device__ __forceinline__ float base_rev(long long p0, float theta) {
  double r = (double)p0 * (double)theta * 0.15915494309189535;
  return (float)(r - rint(r));
}

__device__ __forceinline__ void fill_rot_tables(const RetArgs &a, float *theta_s, float2 *step_s, int npairs) {
  for (int i = threadIdx.x; i < npairs; i += blockDim.x) {
    theta_s[i] = a.theta[i];
    step_s[i] = make_float2(cosf(a.theta[i]), sinf(a.theta[i]));
  }
}

// Decay table of one head in LDS: dt[x + 64] = gamma^x for 0 <= x < 128 and 0
// for -64 <= x < 0, so a lookup also applies the causal mask.  For a query block
// starting at q0 and a key block at k0 = q0 - 64*delta, the distance of query
// q0+n' and key k0+m' is 64*delta + d' with d' = n' - m' in [-63, 63]:
//   delta == 0: gamma^d' or 0 (masked) = dt[d' + 64]
//   delta >= 1: gamma^(64(delta-1)) * gamma^(d'+64), and d' + 64 is in [1, 127]
constexpr int DT_SZ = 192;
__device__ __forceinline__ void fill_decay_table(float *dt, float lg, int nthreads) {
  for (int i = threadIdx.x; i < DT_SZ; i += nthreads) dt[i] = i < 64 ? 0.0f : dpow(lg, i - 64);
}

template <int DK, int DVW>
struct Tile {
  static constexpr int RW = DVW / 8;   // O^T rows / state columns per wave
  static constexpr int RB = RW / 16;   // 16-row blocks per wave
  static constexpr int KS = DK / 32;   // k-steps over dk
  static constexpr int DKB = DK / 16;  // 16-row blocks of dk
  static constexpr int LDQ = DK + 4;   // token-major tiles (Qs, Ks): 2*DK + 8 bytes
  static_assert(RW % 16 == 0 && DK % 32 == 0, "tile shape");
};

// Moving a 64-token tile of a [tokens][D] bf16 tensor from HBM to LDS, in two
// steps so that the global loads of the next tile overlap the MFMA work on the
// current one: fetch() issues 16-byte loads into registers, commit() converts
// them (rotation, per-token scale) and writes LDS.
//
// Thread mapping: work item = (token group tg, 16-byte column chunk c8), tg
// fastest across lanes; a thread holds TPT consecutive tokens of one chunk.
// The transposed (token-minor) LDS write of a column then covers TPT tokens in
// one 4/8/16-byte store, and consecutive lanes write consecutive addresses of
// the same LDS row: no bank conflicts.  Each global row segment read by a wave
// is 64 bytes or more and fully used.
template <int D>
struct TileIO {
  static constexpr int C8 = D / 8;
  static constexpr int TPT = (C8 / 8 < 2) ? 2 : C8 / 8;  // tokens per thread
  static constexpr int NG = BT / TPT;                     // token groups
  static constexpr int ITEMS = NG * C8;
  static constexpr int NI = (ITEMS + NT - 1) / NT;
  static constexpr int CG = 4;  // consecutive lanes on consecutive chunks of a row: 64-byte global segments
  static_assert(TPT == 2 || TPT == 4 || TPT == 8, "tokens per thread");
  static_assert(C8 % CG == 0, "column chunks");
  uint4 raw[NI][TPT];

  __device__ __forceinline__ static void item(int idx, int &tg, int &c8) {
    const int lo = idx % CG, rest = idx / CG;
    tg = rest % NG;
    c8 = (rest / NG) * CG + lo;
  }

  // Buffer loads through a resource whose range ends after row valid-1: rows at
  // or past `valid` read as zero (hardware range check), with no branches and
  // 32-bit offsets.  Rows are `stride` elements apart.  rev: tile row t is row
  // valid-1-t of src (rows past `valid` then have negative offsets, which the
  // range check also rejects).
  __device__ __forceinline__ void fetch(const uint16_t *src, long long stride, int valid, bool rev = false) {
    const int nbytes = valid > 0 ? (int)((long long)valid * stride * 2) : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, nbytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = threadIdx.x + NT * i;
      int tg, c8;
      item(idx, tg, c8);
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
        const int row = rev ? valid - 1 - (TPT * tg + r) : TPT * tg + r;
        const int off = (row * (int)stride + 8 * c8) * 2;
        if (ITEMS % NT == 0 || idx < ITEMS) {
          const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
          raw[i][r] = make_uint4(x.x, x.y, x.z, x.w);
        } else {
          raw[i][r] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
  }

  // Reload a tile already in LDS, token-major rows of pitch ldr (8-byte aligned).
  __device__ __forceinline__ void load_lds(const uint16_t *src, int ldr) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = threadIdx.x + NT * i;
      int tg, c8;
      item(idx, tg, c8);
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
        if (ITEMS % NT == 0 || idx < ITEMS) {
          const uint16_t *sr = src + (TPT * tg + r) * ldr + 8 * c8;
          const u32x2 lo = *(const u32x2 *)sr, hi = *(const u32x2 *)(sr + 4);
          raw[i][r] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
      }
    }
  }

  // Two tiles of the same tokens (q and k of one block), rotated with shared
  // sines and cosines, written as rows: dA / dB[t * ldr + col].
  __device__ __forceinline__ static void commit_rows2(const TileIO &A, const TileIO &B, bool rot, long long p0,
                                                      const float *theta_s, const float2 *step_s, uint16_t *dA,
                                                      uint16_t *dB, int ldr) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = threadIdx.x + NT * i;
      if (idx >= ITEMS) continue;
      int tg, c8;
      item(idx, tg, c8);
      float xa[TPT][8], xb[TPT][8];
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
        const uint32_t wa[4] = {A.raw[i][r].x, A.raw[i][r].y, A.raw[i][r].z, A.raw[i][r].w};
        const uint32_t wb[4] = {B.raw[i][r].x, B.raw[i][r].y, B.raw[i][r].z, B.raw[i][r].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xa[r][2 * e] = __uint_as_float(wa[e] << 16);
          xa[r][2 * e + 1] = __uint_as_float(wa[e] & 0xffff0000u);
          xb[r][2 * e] = __uint_as_float(wb[e] << 16);
          xb[r][2 * e + 1] = __uint_as_float(wb[e] & 0xffff0000u);
        }
      }
      if (rot) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int pi = 4 * c8 + pp;
          const float A0 = base_rev(p0 + TPT * tg, theta_s[pi]);
          const float2 stp = step_s[pi];
          float c = __builtin_amdgcn_cosf(A0), sn = __builtin_amdgcn_sinf(A0);
#pragma unroll
          for (int r = 0; r < TPT; ++r) {
            if (r > 0) {
              const float c2 = c * stp.x - sn * stp.y;
              sn = sn * stp.x + c * stp.y;
              c = c2;
            }
            float re = xa[r][2 * pp], im = xa[r][2 * pp + 1];
            xa[r][2 * pp] = re * c - im * sn;
            xa[r][2 * pp + 1] = re * sn + im * c;
            re = xb[r][2 * pp];
            im = xb[r][2 * pp + 1];
            xb[r][2 * pp] = re * c - im * sn;
            xb[r][2 * pp + 1] = re * sn + im * c;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
        uint16_t *ra = dA + (TPT * tg + r) * ldr + 8 * c8, *rb = dB + (TPT * tg + r) * ldr + 8 * c8;
        *(u32x2 *)ra = u32x2{pack_bf2(xa[r][0], xa[r][1]), pack_bf2(xa[r][2], xa[r][3])};
        *(u32x2 *)(ra + 4) = u32x2{pack_bf2(xa[r][4], xa[r][5]), pack_bf2(xa[r][6], xa[r][7])};
        *(u32x2 *)rb = u32x2{pack_bf2(xb[r][0], xb[r][1]), pack_bf2(xb[r][2], xb[r][3])};
        *(u32x2 *)(rb + 4) = u32x2{pack_bf2(xb[r][4], xb[r][5]), pack_bf2(xb[r][6], xb[r][7])};
      }
    }
  }

  // rows:  dst[t * ldr + col]            (token-major, bf16; lo part to dstLo when LO)
  // trans: dstT[col * LDT + t] * zeta_t  (token-minor), zeta_t = gamma^(zoff - t) when `zeta`;
  //        with ZR instead dstT[t * ldz + col] * zeta_t (token-major, 16-byte stores, ldz % 8 == 0)
  // Rotation (rot): token t of the tile sits at absolute position p0 + t.
  template <bool ROWS, bool TRANS, bool LO, bool ZR = false>
  __device__ __forceinline__ void commit(bool rot, long long p0, const float *theta_s, const float2 *step_s,
                                         uint16_t *dst, int ldr, uint16_t *dstLo, uint16_t *dstT, bool zeta,
                                         float zlg, int zoff, int ldz = 0) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = threadIdx.x + NT * i;
      if (idx >= ITEMS) continue;
      int tg, c8;
      item(idx, tg, c8);
      float x[TPT][8];
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
        const uint32_t wv[4] = {raw[i][r].x, raw[i][r].y, raw[i][r].z, raw[i][r].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[r][2 * e] = __uint_as_float(wv[e] << 16);
          x[r][2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
        }
      }
      if (rot) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int pi = 4 * c8 + pp;
          const float A = base_rev(p0 + TPT * tg, theta_s[pi]);
          const float2 stp = step_s[pi];
          float c = __builtin_amdgcn_cosf(A), sn = __builtin_amdgcn_sinf(A);
#pragma unroll
          for (int r = 0; r < TPT; ++r) {
            if (r > 0) {
              const float c2 = c * stp.x - sn * stp.y;
              sn = sn * stp.x + c * stp.y;
              c = c2;
            }
            const float re = x[r][2 * pp], im = x[r][2 * pp + 1];
            x[r][2 * pp] = re * c - im * sn;
            x[r][2 * pp + 1] = re * sn + im * c;
          }
        }
      }
      if constexpr (ROWS) {
#pragma unroll
        for (int r = 0; r < TPT; ++r) {
          uint4 o;
          o.x = pack_bf2(x[r][0], x[r][1]);
          o.y = pack_bf2(x[r][2], x[r][3]);
          o.z = pack_bf2(x[r][4], x[r][5]);
          o.w = pack_bf2(x[r][6], x[r][7]);
          uint16_t *dr = dst + (TPT * tg + r) * ldr + 8 * c8;
          *(u32x2 *)dr = u32x2{o.x, o.y};
          *(u32x2 *)(dr + 4) = u32x2{o.z, o.w};
          if constexpr (LO) {
            // x - bf16(x), rounded to bf16: hi + lo carries ~16 significant bits
            const uint32_t hw[4] = {o.x, o.y, o.z, o.w};
            uint32_t lw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              lw[e] = pack_bf2(x[r][2 * e] - __uint_as_float(hw[e] << 16),
                               x[r][2 * e + 1] - __uint_as_float(hw[e] & 0xffff0000u));
            uint16_t *dl = dstLo + (TPT * tg + r) * ldr + 8 * c8;
            *(u32x2 *)dl = u32x2{lw[0], lw[1]};
            *(u32x2 *)(dl + 4) = u32x2{lw[2], lw[3]};
          }
        }
      }
      if constexpr (TRANS) {
        float z[TPT];
#pragma unroll
        for (int r = 0; r < TPT; ++r) {
          const int d = zoff - (TPT * tg + r);  // d < 0: a zero-filled token past the chunk
          z[r] = zeta ? (d >= 0 ? dpow(zlg, d) : 0.0f) : 1.0f;
        }
        if constexpr (ZR) {
#pragma unroll
          for (int r = 0; r < TPT; ++r)
            *(u32x4 *)(dstT + (TPT * tg + r) * ldz + 8 * c8) =
                u32x4{pack_bf2(x[r][0] * z[r], x[r][1] * z[r]), pack_bf2(x[r][2] * z[r], x[r][3] * z[r]),
                      pack_bf2(x[r][4] * z[r], x[r][5] * z[r]), pack_bf2(x[r][6] * z[r], x[r][7] * z[r])};
          continue;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint16_t *row = dstT + (8 * c8 + e) * LDT + TPT * tg;
          if constexpr (TPT == 2) {
            *(uint32_t *)row = pack_bf2(x[0][e] * z[0], x[1][e] * z[1]);
          } else if constexpr (TPT == 4) {
            *(u32x2 *)row = pack4(x[0][e] * z[0], x[1][e] * z[1], x[2][e] * z[2], x[3][e] * z[3]);
          } else {
            *(u32x2 *)row = pack4(x[0][e] * z[0], x[1][e] * z[1], x[2][e] * z[2], x[3][e] * z[3]);
            *(u32x2 *)(row + 4) = pack4(x[4][e] * z[4], x[5][e] * z[5], x[6][e] * z[6], x[7][e] * z[7]);
          }
        }
      }
    }
  }
};

// Row-major staging of a 64-token tile of a [tokens][D] bf16 tensor: work item =
// (token t, 16-byte column chunk c8) with c8 fastest across lanes, so a wave
// reads whole rows from memory and writes whole rows to LDS (16-byte stores, no
// bank conflicts).  MFMA operands are then read with ld_op (along the row) or
// ld_op_tr (across rows).
template <int D>
struct RowIO {
  static constexpr int C8 = D / 8;
  static constexpr int ITEMS = BT * C8;
  static constexpr int NI = ITEMS / NT;
  static_assert(ITEMS % NT == 0, "whole items per thread");
  uint4 raw[NI];

  // as TileIO::fetch, rev included
  __device__ __forceinline__ void fetch(const uint16_t *src, long long stride, int valid, bool rev = false) {
    const int nbytes = valid > 0 ? (int)((long long)valid * stride * 2) : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, nbytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = threadIdx.x + NT * i, t = idx / C8, c8 = idx % C8;
      const int row = rev ? valid - 1 - t : t;
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, (row * (int)stride + 8 * c8) * 2, 0, 0);
      raw[i] = make_uint4(x.x, x.y, x.z, x.w);
    }
  }

  // dst[t * ldr + col] = raw, optionally rotated (token t at position p0 + t) and
  // scaled by zeta_t = gamma^(zoff - t) (0 for t > zoff: a zero-filled row).
  template <bool ROT, bool ZETA>
  __device__ __forceinline__ void commit(uint16_t *dst, int ldr, long long p0, const float *theta_s, float zlg,
                                         int zoff) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = threadIdx.x + NT * i, t = idx / C8, c8 = idx % C8;
      uint4 o = raw[i];
      if (ROT || ZETA) {
        const uint32_t wv[4] = {o.x, o.y, o.z, o.w};
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(wv[e] << 16);
          x[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
        }
        if constexpr (ROT) {
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const float rv = base_rev(p0 + t, theta_s[4 * c8 + pp]);
            const float sn = __builtin_amdgcn_sinf(rv), c = __builtin_amdgcn_cosf(rv);
            const float re = x[2 * pp], im = x[2 * pp + 1];
            x[2 * pp] = re * c - im * sn;
            x[2 * pp + 1] = re * sn + im * c;
          }
        }
        if constexpr (ZETA) {
          const int d = zoff - t;
          const float z = d >= 0 ? dpow(zlg, d) : 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= z;
        }
        o = make_uint4(pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7]));
      }
      *(uint4 *)(dst + t * ldr + 8 * c8) = o;
    }
  }
};

// First row of the tile [k0, k0 + valid) of a sequence in memory.  With in_rev
// the kernel's token n is row L-1-n of the tensor, so the tile is rows
// [L - k0 - valid, L - k0), fetched bottom-up (fetch(..., rev = true)).
__device__ __forceinline__ const uint16_t *tile_src(const uint16_t *seq, long long k0, int valid, long long sn,
                                                    const RetArgs &a) {
  return seq + (a.in_rev ? (long long)a.L - k0 - valid : k0) * sn;
}

struct TaskGeom {
  int nseg, seg_chunks, nsplit, nqb, ntasks;
  int nchunks;  // chunks per (b, h)
  // query-block kernel task selection: 0 every query block; 1 only the first
  // query block of each sequence (one task per (b, h)); 2 all but those
  int sel = 0;
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

// Epilogue of a 64-query block held as O^T accumulators: optional GroupNorm over
// all DV values of each (token, head) row (every wave holds RW of them), optional
// bf16 gate multiply, store (bf16 or fp32) with the output strides of `a`.
// Column order of a wave's O^T rows.  With PAIR (two 16-row blocks per wave), row
// m of block rb holds dv offset 8*(m/4) + 4*rb + m%4 of the wave's 32 columns, so
// the D-layout accumulators of a lane -- rows 4g..4g+3 of both blocks -- are 8
// consecutive columns: one 16-byte store per query row.  The same order is
// applied wherever a dv index enters an MFMA operand (V^T rows, state columns).
template <bool PAIR>
__device__ __forceinline__ int dv_of(int rb, int m) {
  return PAIR ? 8 * (m >> 2) + 4 * rb + (m & 3) : 16 * rb + m;
}

// out_rot of the epilogue: pairs (x[2j], x[2j+1]) of output columns pair0 + j
// multiplied by exp(-i p theta) (the transpose of the rotation at position p).
template <int N>
__device__ __forceinline__ void unrotate_pairs(const RetArgs &a, float *x, long long p, int pair0) {
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    float c, sn;
    rot_cs<false>(p, a.theta[pair0 + j], c, sn);
    const float re = x[2 * j], im = x[2 * j + 1];
    x[2 * j] = re * c + im * sn;
    x[2 * j + 1] = im * c - re * sn;
  }
}

// Per-(query, head) GroupNorm over the DV columns held by the 8 waves (rows of
// O^T in the accumulators), in place.  Contains barriers: call from all threads.
template <int RB, int DV>
__device__ __forceinline__ void epilogue_groupnorm(const RetArgs &a, f32x4 (&ot)[RB][4], float (*red)[BT], int w,
                                                   int g, int l16) {
  {
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
        tot /= (float)DV;
        if (pass == 0)
          mean[qb4] = tot;
        else
          inv[qb4] = __builtin_amdgcn_rsqf(tot + a.gn_eps);
      }
    }
#pragma unroll
    for (int qb4 = 0; qb4 < 4; ++qb4)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) ot[rb][qb4] = (ot[rb][qb4] - mean[qb4]) * inv[qb4];
  }
}

// Output of a 64-query block (bf16): the accumulators (after GroupNorm) go to
// LDS as rows of O in the Os buffer (pitch DV + 8), then every store writes whole
// 16-byte pieces of rows, coalesced across lanes; the gate, the inverse rotation
// and the row reversal are applied in that row-wise pass.  stage_out writes the
// block to Os (which must be free); store_staged, after a barrier, does the row
// pass.  epilogue_staged is the two with the barriers around them.
// Staging addresses: row pitch DV + 8 (SW false), or DV with the 16-byte chunks
// of row r stored at chunk index c ^ (r & 7) (SW: the block fills a 64 x DV
// buffer exactly; 8-byte stores of 16 rows then meet at most two per bank).
template <int DV, bool SW>
__device__ __forceinline__ int stage_idx(int row, int col) {
  return SW ? row * DV + (((col >> 3) ^ (row & 7)) << 3) + (col & 7) : row * (DV + 8) + col;
}

template <int RB, int RW, int DV, bool PAIR, bool SW = false>
__device__ __forceinline__ void stage_out(const f32x4 (&ot)[RB][4], uint16_t *Os, int w, int g, int l16) {
  constexpr int DVP = DV + 8;
  static_assert(!(PAIR && SW), "paired order is staged unswizzled");
#pragma unroll
  for (int qb4 = 0; qb4 < 4; ++qb4) {
    const int row = 16 * qb4 + l16;
    if constexpr (PAIR) {
      *(u32x4 *)(Os + row * DVP + w * RW + 8 * g) =
          u32x4{pack_bf2(ot[0][qb4][0], ot[0][qb4][1]), pack_bf2(ot[0][qb4][2], ot[0][qb4][3]),
                pack_bf2(ot[1][qb4][0], ot[1][qb4][1]), pack_bf2(ot[1][qb4][2], ot[1][qb4][3])};
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        *(u32x2 *)(Os + stage_idx<DV, SW>(row, w * RW + 16 * rb + 4 * g)) =
            pack4(ot[rb][qb4][0], ot[rb][qb4][1], ot[rb][qb4][2], ot[rb][qb4][3]);
    }
  }
}

template <int DV, bool SW = false>
__device__ __forceinline__ void store_staged(const RetArgs &a, const uint16_t *Os, int b, int h, int q0, int nvalid,
                                             long long obase) {
  constexpr int C8 = DV / 8, NPT = BT * C8 / NT;  // 16-byte pieces per thread
  static_assert(BT * C8 % NT == 0, "whole pieces per thread");
  const int tid = threadIdx.x;
  // Stores go through a buffer resource covering the block's valid rows only
  // (rows at or past nvalid fall outside it and are dropped by the hardware), so
  // the pass has no branches.  With out_rev, row r goes to n = L-1-(q0+r): the
  // resource starts at the lowest such n and offsets count down from it.
  const long long nbase = a.out_rev ? (long long)a.L - q0 - nvalid : q0;
  const int range = (int)((long long)nvalid * a.o_sn * 2);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)((uint16_t *)a.o + obase + nbase * a.o_sn), (short)0, range,
                                        0x00020000);
  // the gate's pieces first, all in flight together (rows past nvalid read the
  // last valid row; their results are dropped)
  u32x4 gt[NPT];
  if (a.gate) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int c = tid + NT * i, row = min(c / C8, max(nvalid - 1, 0)), col = 8 * (c % C8);
      gt[i] = *(const u32x4 *)(a.gate + (long long)b * a.g_sb + (long long)h * a.g_sh + (long long)(q0 + row) * a.g_sn +
                               col);
    }
  }
  u32x4 o[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int c = tid + NT * i;
    o[i] = *(const u32x4 *)(Os + stage_idx<DV, SW>(c / C8, 8 * (c % C8)));
  }
  if (a.gate || a.out_rot) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int c = tid + NT * i, row = c / C8, col = 8 * (c % C8);
      const uint32_t ow[4] = {o[i].x, o[i].y, o[i].z, o[i].w};
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(ow[e] << 16);
        x[2 * e + 1] = __uint_as_float(ow[e] & 0xffff0000u);
      }
      if (a.gate) {
        const u32x4 gg = gt[i];
        const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] *= gate_value(__uint_as_float(gw[e] << 16), a.gate_swish);
          x[2 * e + 1] *= gate_value(__uint_as_float(gw[e] & 0xffff0000u), a.gate_swish);
        }
      }
      if (a.out_rot) unrotate_pairs<8>(a, x, a.pos0 + (a.out_rev ? a.L - 1 - (q0 + row) : q0 + row), col / 2);
      o[i] = u32x4{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])};
    }
  }
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int c = tid + NT * i, row = c / C8, col = 8 * (c % C8);
    const long long n = a.out_rev ? (long long)nvalid - 1 - row : row;  // row index inside the resource
    // rows past nvalid: offset at the end of the range -> every dword dropped
    const int off = row < nvalid ? (int)((n * a.o_sn + col) * 2) : range;
    __builtin_amdgcn_raw_buffer_store_b128(o[i], rs, off, 0, 2 /* slc: streaming */);
  }
}

template <int RB, int RW, int DV, bool PAIR>
__device__ __forceinline__ void epilogue_staged(const RetArgs &a, f32x4 (&ot)[RB][4], uint16_t *Os, int b, int h,
                                                int q0, int nvalid, long long obase, int w, int g, int l16) {
  __syncthreads();
  stage_out<RB, RW, DV, PAIR>(ot, Os, w, g, l16);
  __syncthreads();
  store_staged<DV>(a, Os, b, h, q0, nvalid, obase);
}

template <int RB, int RW, int DV, bool PAIR = false>
__device__ __forceinline__ void epilogue_store(const RetArgs &a, f32x4 (&ot)[RB][4], float (*red)[BT], int b, int h,
                                               int q0, int nvalid, long long obase, int w, int g, int l16) {
  static_assert(!PAIR || RB == 2, "paired column order needs two row blocks");
  if (a.use_gn) epilogue_groupnorm<RB, DV>(a, ot, red, w, g, l16);
  if constexpr (PAIR) {
#pragma unroll
    for (int qb4 = 0; qb4 < 4; ++qb4) {
      const int r = 16 * qb4 + l16;
      if (r < nvalid) {
        const int n = a.out_rev ? a.L - 1 - (q0 + r) : q0 + r;
        const long long ro = obase + (long long)n * a.o_sn;
        const int col = w * RW + 8 * g;
        float x[8] = {ot[0][qb4][0], ot[0][qb4][1], ot[0][qb4][2], ot[0][qb4][3],
                      ot[1][qb4][0], ot[1][qb4][1], ot[1][qb4][2], ot[1][qb4][3]};
        if (a.out_rot) unrotate_pairs<8>(a, x, a.pos0 + n, col / 2);
        if (a.gate) {
          const long long go = (long long)b * a.g_sb + (long long)h * a.g_sh + (long long)(q0 + r) * a.g_sn + col;
          const u32x4 gg = *(const u32x4 *)(a.gate + go);
          const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] *= gate_value(__uint_as_float(gw[e] << 16), a.gate_swish);
            x[2 * e + 1] *= gate_value(__uint_as_float(gw[e] & 0xffff0000u), a.gate_swish);
          }
        }
        if (a.out_bf16) {
          // streaming store: the output is not read again by this call
          __builtin_nontemporal_store(
              u32x4{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])},
              (u32x4 *)((uint16_t *)a.o + ro + col));
        } else {
          float *dst = (float *)a.o + ro + col;
          *(float4 *)dst = make_float4(x[0], x[1], x[2], x[3]);
          *(float4 *)(dst + 4) = make_float4(x[4], x[5], x[6], x[7]);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int qb4 = 0; qb4 < 4; ++qb4) {
    const int r = 16 * qb4 + l16;
    if (r < nvalid) {
      const int n = a.out_rev ? a.L - 1 - (q0 + r) : q0 + r;
      const long long ro = obase + (long long)n * a.o_sn;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int col = w * RW + 16 * rb + 4 * g;
        f32x4 x = ot[rb][qb4];
        if (a.out_rot) {
          float xr[4] = {x[0], x[1], x[2], x[3]};
          unrotate_pairs<4>(a, xr, a.pos0 + n, col / 2);
          x = f32x4{xr[0], xr[1], xr[2], xr[3]};
        }
        if (a.gate) {
          const long long go = (long long)b * a.g_sb + (long long)h * a.g_sh + (long long)(q0 + r) * a.g_sn + col;
          const u32x2 gg = *(const u32x2 *)(a.gate + go);
          x[0] *= gate_value(__uint_as_float(gg.x << 16), a.gate_swish);
          x[1] *= gate_value(__uint_as_float(gg.x & 0xffff0000u), a.gate_swish);
          x[2] *= gate_value(__uint_as_float(gg.y << 16), a.gate_swish);
          x[3] *= gate_value(__uint_as_float(gg.y & 0xffff0000u), a.gate_swish);
        }
        if (a.out_bf16)
          *(u32x2 *)((uint16_t *)a.o + ro + col) = pack4(x[0], x[1], x[2], x[3]);
        else
          *(float4 *)((float *)a.o + ro + col) = make_float4(x[0], x[1], x[2], x[3]);
      }
    }
  }
}

// ---------------------------------------------------------------- V tiles by LDS-DMA
// A V tile (64 token rows of DV bf16) stored unpadded, the 16-byte chunks of
// row r at chunk index c ^ vswz(r), which makes the transposed operand reads
// (ld_op_trs) conflict-free.  It is filled by LDS-DMA loads (buffer_load ...
// lds): wave instruction J of the tile writes LDS bytes [1024 J, 1024 J + 1024),
// lane l the 16 bytes at 1024 J + 16 l, fetched from whichever global chunk
// belongs there.  Rows at or past `valid` read as zero (range-checked resource).
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 3); }

template <int DV>
__device__ __forceinline__ void v_dma(uint16_t *Vb, const uint16_t *src, long long v_sn, int valid) {
  constexpr int RBYTES = DV * 2, NJ = BT * RBYTES / 1024 / (NT / 64);  // instructions per wave
  static_assert(BT * RBYTES % (1024 * (NT / 64)) == 0, "whole instructions per wave");
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int nbytes = valid > 0 ? (int)((long long)valid * v_sn * 2) : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, nbytes, 0x00020000);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int J = w * NJ + j, off = J * 1024 + 16 * l;
    const int row = off / RBYTES, c = ((off % RBYTES) >> 4) ^ vswz(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(Vb + J * 512), 16,
                                             (int)(row * v_sn * 2) + 16 * c, 0, 0, 0);
  }
}

// ld_op_tr on a V tile in that layout: rows k0 + 4g + p/4 (+16), columns
// m0 + 4(p%4) (m0 % 16 == 0), i.e. chunk m0/8 + (p%4)/2, half p%2.
template <int DV>
__device__ __forceinline__ u32x4 ld_op_trs(const uint16_t *Vb, int k0, int m0, int g, int l16) {
  const int row = k0 + 4 * g + (l16 >> 2);
  const int c = (m0 >> 3) + ((l16 & 3) >> 1);
  const uint16_t *p0 = Vb + row * DV + ((c ^ vswz(row)) << 3) + 4 * (l16 & 1);
  const tr_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr_v4s *)p0);
  const tr_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr_v4s *)(p0 + 16 * DV));
  const u32x2 l = __builtin_bit_cast(u32x2, lo), h = __builtin_bit_cast(u32x2, hi);
  return u32x4{l.x, l.y, h.x, h.y};
}

// Rotated key tiles by LDS-DMA: 64 token rows of DK bf16, unpadded, the 16-byte
// chunk c of row r stored at chunk c ^ (r & 7).  The score operand of lane
// (g, l16) is 8 consecutive elements (chunk 4ks + g) of row r0 + l16: each run
// of 8 lanes then reads 8 different chunk slots of rows with equal bank
// offsets, i.e. all 32 banks once (DK*2 is a multiple of 128 bytes).  Wave
// instruction J writes LDS bytes [1024 J, 1024 J + 1024), lane l 16 of them;
// rows at or past `valid` read as zero.
template <int DK>
__device__ __forceinline__ void k_dma(uint16_t *Ks, const uint16_t *src, long long sn, int valid) {
  constexpr int RBYTES = DK * 2, NJ = BT * RBYTES / 1024 / (NT / 64);  // instructions per wave
  static_assert(BT * RBYTES % (1024 * (NT / 64)) == 0 && DK >= 64, "whole instructions per wave, 8 chunks a row");
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int nbytes = valid > 0 ? (int)((long long)valid * sn * 2) : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, nbytes, 0x00020000);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int J = w * NJ + j, off = J * 1024 + 16 * l;
    const int row = off / RBYTES, c = ((off % RBYTES) >> 4) ^ (row & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(Ks + J * 512), 16,
                                             (int)(row * sn * 2) + 16 * c, 0, 0, 0);
  }
}

// Elements [8c, 8c + 8) of row r of a key tile in that layout.
template <int DK>
__device__ __forceinline__ u32x4 ld_k8(const uint16_t *Ks, int r, int c) {
  return *(const u32x4 *)(Ks + r * DK + 8 * (c ^ (r & 7)));
}

// The rotated keys of a call, once, for the query-block kernels:
// kt[((b H + h) L + n) DK + j] = bf16 of k[b, h, n, :] with pair i = (2i, 2i+1)
// turned by the angle (pos0 + n) theta_i ("Retentive Network" paper summary,
// Sec. 2.1: the e^(i n theta) factor of Q and K).  One thread per 8 elements;
// each token's angle is reduced in fp64 from its own position.
template <int DK>
__global__ __launch_bounds__(256) void rotate_keys_kernel(RetArgs a, uint16_t *kt) {
  constexpr int C8 = DK / 8;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = idx / C8;  // (b H + h) L + n
  if (row >= (long long)a.B * a.H * a.L) return;
  const int c8 = (int)(idx % C8), n = (int)(row % a.L);
  const long long bh = row / a.L;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const uint16_t *src = (const uint16_t *)a.k + (long long)b * a.q_sb + (long long)h * a.q_sh + (long long)n * a.q_sn;
  // streamed: the input keys are not read again by this call, and caching them
  // would evict what the retention kernel reads next
  const u32x4 x = __builtin_nontemporal_load((const u32x4 *)(src + 8 * c8));
  const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float re = __uint_as_float(wv[e] << 16), im = __uint_as_float(wv[e] & 0xffff0000u);
    const float A = base_rev(a.pos0 + n, a.theta[4 * c8 + e]);
    const float c = __builtin_amdgcn_cosf(A), sn = __builtin_amdgcn_sinf(A);
    o[e] = pack_bf2(re * c - im * sn, re * sn + im * c);
  }
  *(u32x4 *)(kt + row * DK + 8 * c8) = u32x4{o[0], o[1], o[2], o[3]};
}

// Waits for this wave's outstanding vector-memory operations, LDS-DMA loads
// included (s_waitcnt vmcnt(0)).  A DMA-filled tile is read by other waves, so
// every wave calls this before the barrier that publishes the tile.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier that publishes LDS stores only: waits for this wave's LDS
// operations (lgkmcnt(0)) but not for outstanding global loads or LDS-DMA, which
// stay in flight across it (__syncthreads would wait for those too).  The
// signal fences keep the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- query-block kernel
constexpr int LPT_G = 4;  // (bh, chunk) units per longest-first task group

// One task = (b, h, chunk c, 64-query block qb).  PAR: the parallel form (one
// chunk spanning the sequence, no cross term).  Otherwise the chunkwise output
// with the state entering chunk c, S_c, stored bf16 as S_c^T[dv][dk] in SinT
// (every chunk is a segment of its own on this path).
// SPLIT: scores from hi + lo bf16 parts of the rotated q and k (three MFMAs per
// k-step), accurate to ~2^-16 instead of the ~2^-8 of one bf16 rounding of the
// rotated values.  Used when GroupNorm follows: rows whose variance is near eps
// magnify absolute score errors by ~1/sqrt(eps).
// The global loads of the next key block are issued right after the current
// one is committed to LDS, so they are in flight during the MFMA work.
// KPRE (plain scores only): the keys arrive rotated -- from kt ([B*H][L][DK],
// rotate_keys_kernel), or straight from k when there is no rotation (kt null) --
// and go to LDS by DMA, no register pass: the next block's DMA is issued once
// the scores are done with the current one and lands during the P.V products.
template <int DK, int DV, bool PAR, bool SPLIT, bool KPRE = false>
__global__ __launch_bounds__(NT) void qblock_kernel(RetArgs a, TaskGeom geo, const uint16_t *SinT,
                                                    const uint16_t *kt = nullptr) {
  static_assert(!(KPRE && SPLIT), "pre-rotated keys carry no lo part");
  using T = Tile<DK, DV>;
  constexpr int LDQ = T::LDQ, RW = T::RW, RB = T::RB, KS = T::KS;
  // The query block is staged through Ks / KsL (free until the key loop starts).
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BT * LDQ];
  __shared__ __attribute__((aligned(16))) uint16_t KsL[SPLIT ? BT * LDQ : 8];
  __shared__ __attribute__((aligned(16))) uint16_t Vb[BT * DV];  // V tile (LDS-DMA, swizzled)
  __shared__ __attribute__((aligned(16))) uint16_t Ps[BT * LDT];
  __shared__ float theta_s[DK / 2];
  __shared__ float2 step_s[DK / 2];
  __shared__ float red[8][BT];
  __shared__ float dt[DT_SZ];
  // With keys by DMA the query tile is staged in the V tile's space where it
  // fits, so that the first key block can load from the start.
  constexpr bool QV = KPRE && DV >= DK + 4;
  uint16_t *const Qs = QV ? Vb : Ks;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int task = xcd_task(blockIdx.x, geo.ntasks);
  if (task < 0) return;
  // Task order, longest first: the (bh, chunk) units go in groups of LPT_G, and
  // inside a group the query blocks run from the last (the most key blocks to
  // visit) to the first, across the group's units.  Each XCD takes a contiguous
  // range of tasks (xcd_task), so it starts on the long tasks of its groups and
  // fills its tail with short ones.  (Units one after another, longest first
  // within each: parallel workload 383 -> 353 us, MSR layer 1245 -> 1207 us; the
  // four units in flight re-read more K and V past the L2, which costs less.)
  int qb = 0, c = 0, bh = task;  // sel 1: one task per (b, h), its first query block
  if (geo.sel != 1) {
    const int nunits = geo.ntasks / geo.nqb, grp = task / (geo.nqb * LPT_G);
    const int gsz = min(LPT_G, nunits - grp * LPT_G), r = task - grp * geo.nqb * LPT_G;
    const int unit = grp * LPT_G + r % gsz;
    qb = geo.nqb - 1 - r / gsz;
    c = unit % geo.nchunks;
    bh = unit / geo.nchunks;
  }
  if (geo.sel == 2 && qb == 0 && c == 0) return;
  const int cstep = PAR ? a.L : a.chunk;
  const int c0 = c * cstep, Cc = min(cstep, a.L - c0);
  const int q0 = c0 + qb * BT;
  if (q0 >= c0 + Cc) return;  // short last chunk: fewer query blocks
  const int b = bh / a.H, h = bh % a.H;
  const float lg = safe_log2(a.gamma[h]);
  const bool rot = a.use_theta;
  const uint16_t *q = (const uint16_t *)a.q + (long long)b * a.q_sb + (long long)h * a.q_sh;
  const uint16_t *k = (const uint16_t *)a.k + (long long)b * a.q_sb + (long long)h * a.q_sh;
  const uint16_t *v = (const uint16_t *)a.v + (long long)b * a.v_sb + (long long)h * a.v_sh;
  const long long obase = (long long)b * a.o_sb + (long long)h * a.o_sh;
  if (rot) fill_rot_tables(a, theta_s, step_s, DK / 2);
  fill_decay_table(dt, lg, NT);

  // key rows of this (b, h): the rotated copy, else the input
  const uint16_t *ksrc = kt ? kt + (long long)bh * a.L * DK : k;
  const long long ksn = kt ? DK : a.q_sn;
  TileIO<DK> qio, kio;
  if constexpr (QV) k_dma<DK>(Ks, ksrc + (long long)c0 * ksn, ksn, min(BT, Cc));
  qio.fetch(q + (long long)q0 * a.q_sn, a.q_sn, min(BT, c0 + Cc - q0));
  // The cross term's A operands (rows S_c^T[w*RW + 16rb + l16][dk] of the state
  // entering the chunk; inside each 32-wide k-step lane group g takes k = 8g ..
  // 8g+7 for both operands, so every load is 16 contiguous bytes): all of them
  // are issued here, behind the query tile, so their latency overlaps the
  // prologue instead of stalling every k-step of the cross term.
  u32x4 sa[PAR ? 1 : KS][RB];
  if constexpr (!PAR) {
    const uint16_t *s_t = SinT + ((long long)bh * geo.nchunks + c) * DK * DV + (long long)(w * RW + l16) * DK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sa[ks][rb] = *(const u32x4 *)(s_t + 16 * rb * DK + 32 * ks);
  }
  if constexpr (!KPRE) kio.fetch(k + (long long)c0 * a.q_sn, a.q_sn, min(BT, Cc));
  __syncthreads();
  qio.template commit<true, false, SPLIT>(rot, a.pos0 + q0, theta_s, step_s, Qs, LDQ, KsL, nullptr, false, 0.f, 0);
  __syncthreads();
  // score split of the 64 x 64 block over the 8 waves: QW 16-query blocks x KW
  // 16-key blocks per wave.  Plain scores: 32 queries x 16 keys, each key
  // operand read from LDS feeding two MFMAs.  hi+lo scores hold twice the query
  // operands, so there 16 queries x 32 keys.
  constexpr int QW = SPLIT ? 1 : 2, KW = 2 / QW;
  const int qp = w % (4 / QW), kq = w / (4 / QW);
  const int qrow0 = 16 * QW * qp, krow0 = 16 * KW * kq;
  // O^T accumulators: ot[rb][qb4][i] = O^T[w*RW+16rb+4g+i][16qb4+l16]
  f32x4 ot[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int qb4 = 0; qb4 < 4; ++qb4) ot[rb][qb4] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (!PAR) {
    // cross term gamma^(j+1) q S_c, A operands prefetched above
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int qb4 = 0; qb4 < 4; ++qb4) {
        const uint16_t *qr = Qs + (16 * qb4 + l16) * LDQ + 32 * ks + 8 * g;
        const u32x2 lo = *(const u32x2 *)qr, hi = *(const u32x2 *)(qr + 4);
        const u32x4 bq = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) ot[rb][qb4] = mfma(sa[ks][rb], bq, ot[rb][qb4]);
      }
    }
#pragma unroll
    for (int qb4 = 0; qb4 < 4; ++qb4) {
      const float xi = dpow(lg, q0 - c0 + 16 * qb4 + l16 + 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) ot[rb][qb4] *= xi;
    }
  }
  // the query operands of the scores (read after the cross term: fewer live registers there)
  u32x4 qreg[QW][KS], qlo[QW][SPLIT ? KS : 1];
#pragma unroll
  for (int qq = 0; qq < QW; ++qq)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (KPRE) {  // k-step elements 8g..8g+7, as ld_k8 gives the keys
        const uint16_t *qr = Qs + (qrow0 + 16 * qq + l16) * LDQ + 32 * ks + 8 * g;
        const u32x2 lo = *(const u32x2 *)qr, hi = *(const u32x2 *)(qr + 4);
        qreg[qq][ks] = u32x4{lo.x, lo.y, hi.x, hi.y};
      } else {
        qreg[qq][ks] = ld_op(Qs + (qrow0 + 16 * qq + l16) * LDQ, 32 * ks, g);
      }
      if constexpr (SPLIT) qlo[qq][ks] = ld_op(KsL + (qrow0 + 16 * qq + l16) * LDQ, 32 * ks, g);
    }
  if constexpr (KPRE && !QV) {  // the query tile (Qs = Ks) is read: the first key block
    __syncthreads();
    k_dma<DK>(Ks, ksrc + (long long)c0 * ksn, ksn, min(BT, Cc));
  }
  for (int kb = 0; kb <= qb; ++kb) {
    const int k0 = c0 + kb * BT;
    const int delta = qb - kb;
    const float gdel = delta ? dpow(lg, 64 * (delta - 1)) : 1.0f;
    if constexpr (KPRE) {
      wait_vmem();  // this wave's part of the key tile; the barrier publishes all of it
      __syncthreads();
      v_dma<DV>(Vb, v + (long long)k0 * a.v_sn, a.v_sn, min(BT, c0 + Cc - k0));
    } else {
      __syncthreads();
      // this visit's V tile streams into LDS during the key commit and the scores
      v_dma<DV>(Vb, v + (long long)k0 * a.v_sn, a.v_sn, min(BT, c0 + Cc - k0));
      kio.template commit<true, false, SPLIT>(rot, a.pos0 + k0, theta_s, step_s, Ks, LDQ, KsL, nullptr, false, 0.f,
                                              0);
      lds_barrier();  // the keys; the V tile stays in flight
    }
    // scores S^T[key][query] for the wave's keys and queries; decay, mask, -> Ps
#pragma unroll
    for (int kb = 0; kb < KW; ++kb) {
      f32x4 sc[QW];
#pragma unroll
      for (int qq = 0; qq < QW; ++qq) sc[qq] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 ak = KPRE ? ld_k8<DK>(Ks, krow0 + 16 * kb + l16, 4 * ks + g)
                              : ld_op(Ks + (krow0 + 16 * kb + l16) * LDQ, 32 * ks, g);
        u32x4 akl;
        if constexpr (SPLIT) akl = ld_op(KsL + (krow0 + 16 * kb + l16) * LDQ, 32 * ks, g);
#pragma unroll
        for (int qq = 0; qq < QW; ++qq) {
          sc[qq] = mfma(ak, qreg[qq][ks], sc[qq]);
          if constexpr (SPLIT) {
            sc[qq] = mfma(akl, qreg[qq][ks], sc[qq]);
            sc[qq] = mfma(ak, qlo[qq][ks], sc[qq]);
          }
        }
      }
      // decay and causal mask from the table (delta = qb - kb blocks apart)
#pragma unroll
      for (int qq = 0; qq < QW; ++qq) {
        const int qr = qrow0 + 16 * qq + l16, kc = krow0 + 16 * kb + 4 * g;
        const int dp = qr - kc + (delta ? 128 : 64);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = sc[qq][i] * (gdel * dt[dp - i]);
        *(u32x2 *)(Ps + qr * LDT + kc) = pack4(p[0], p[1], p[2], p[3]);
      }
    }
    wait_vmem();  // this wave's part of the V tile has landed; the barrier publishes all of it
    __syncthreads();
    if (kb < qb) {  // the next visit's keys, in flight during the P.V products
      const int n0 = k0 + BT;
      if constexpr (KPRE)
        k_dma<DK>(Ks, ksrc + (long long)n0 * ksn, ksn, min(BT, c0 + Cc - n0));
      else
        kio.fetch(k + (long long)n0 * a.q_sn, a.q_sn, min(BT, c0 + Cc - n0));
    }
    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 av[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) av[rb] = ld_op_trs<DV>(Vb, 32 * ks, w * RW + 16 * rb, g, l16);
#pragma unroll
      for (int qb4 = 0; qb4 < 4; ++qb4) {
        const u32x4 bp = ld_op(Ps + (16 * qb4 + l16) * LDT, 32 * ks, g);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) ot[rb][qb4] = mfma(av[rb], bp, ot[rb][qb4]);
      }
    }
  }
  if (a.out_bf16) {  // staged (swizzled) through the V tile's LDS, free after the last visit
    if (a.use_gn) epilogue_groupnorm<RB, DV>(a, ot, red, w, g, l16);
    __syncthreads();
    stage_out<RB, RW, DV, false, true>(ot, Vb, w, g, l16);
    __syncthreads();
    store_staged<DV, true>(a, Vb, b, h, q0, min(BT, c0 + Cc - q0), obase);
  } else {
    epilogue_store<RB, RW, DV>(a, ot, red, b, h, q0, min(BT, c0 + Cc - q0), obase, w, g, l16);
  }
}

// ---------------------------------------------------------------- segment output kernel
// Chunkwise output when the fp32 state of one (b, h), DK x DV, fits in the
// accumulators of the 8 waves (DK*DV <= 128*256).  One task = (b, h, segment):
// the state S_in(segment) is loaded once, then for every chunk of the segment
// and every 64-query block qb of the chunk: the cross term gamma^(j+1) q S_c
// (A operand = S_c^T in bf16, straight from the accumulators: D blocks (2ks, rb)
// and (2ks+1, rb) are the two halves of k-step ks), then the key blocks
// kb = 0..qb.  The chunk's key blocks are folded into the state only while the
// last query block runs (it visits them all), so the cross terms of the
// earlier blocks see S_c.  Global loads of the next visit are in flight
// during the current one.
// RES (chunks of at most kres_of(DK) key blocks, no hi/lo split): the chunk's rotated
// keys stay in LDS, so each key block is fetched and rotated once, at its
// diagonal visit; the update's zeta-scaled transposed copy of an earlier block
// is rebuilt from LDS.
constexpr int KRES = 4;  // resident key blocks: chunks up to 256 tokens
// Resident key blocks that fit beside the other tiles in LDS: four for DK <= 128,
// two (chunks up to 128 tokens) for DK = 256.
constexpr int kres_of(int DK) { return DK <= 128 ? KRES : 2; }
template <int DK, int DV, bool SPLIT, bool RES>
__global__ __launch_bounds__(NT) void seg_out_kernel(RetArgs a, TaskGeom geo, const float *seg_state) {
  using T = Tile<DK, DV>;
  constexpr int LDQ = T::LDQ, RW = T::RW, RB = T::RB, KS = T::KS, DKB = T::DKB;
  constexpr bool PAIR = false;
  // V tiles and the zeta-scaled keys of the update are kept token-major and read
  // across rows (ld_op_tr)
  constexpr int LDV = tr_pitch(DV), LDZ = tr_pitch(DK);
  static_assert(!(RES && SPLIT), "resident keys carry no lo part");
  // Qs (rotated query block, bf16) is read only before the key loop and Kz
  // (zeta-scaled keys of the update) only inside it: shared storage.
  constexpr int QK_SZ = BT * LDQ > BT * LDZ ? BT * LDQ : BT * LDZ;
  __shared__ __attribute__((aligned(16))) uint16_t QKs[QK_SZ];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[(RES ? kres_of(DK) : 1) * BT * LDQ];
  __shared__ __attribute__((aligned(16))) uint16_t KsL[SPLIT ? BT * LDQ : 8];
  __shared__ __attribute__((aligned(16))) uint16_t Vr[BT * LDV];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[BT * LDT];
  uint16_t *const Qs = QKs;
  uint16_t *const Kz = QKs;
  __shared__ float theta_s[DK / 2];
  __shared__ float2 step_s[DK / 2];
  __shared__ float red[8][BT];
  __shared__ float dt[DT_SZ];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int task = xcd_task(blockIdx.x, geo.ntasks);
  if (task < 0) return;
  const int seg = task % geo.nseg;
  const int bh = task / geo.nseg;
  const int b = bh / a.H, h = bh % a.H;
  const float lg = safe_log2(a.gamma[h]);
  const bool rot = a.use_theta;
  const uint16_t *q = (const uint16_t *)a.q + (long long)b * a.q_sb + (long long)h * a.q_sh;
  const uint16_t *k = (const uint16_t *)a.k + (long long)b * a.q_sb + (long long)h * a.q_sh;
  const uint16_t *v = (const uint16_t *)a.v + (long long)b * a.v_sb + (long long)h * a.v_sh;
  const long long obase = (long long)b * a.o_sb + (long long)h * a.o_sh;
  if (rot) fill_rot_tables(a, theta_s, step_s, DK / 2);
  fill_decay_table(dt, lg, NT);

  // fp32 state in D layout: st[dkb][rb][i] = S[16dkb+4g+i][w*RW+16rb+l16]
  f32x4 st[DKB][RB];
  const int c_lo = seg * geo.seg_chunks;
  const int t_lo = c_lo * a.chunk;
  const int t_hi = min(a.L, (c_lo + geo.seg_chunks) * a.chunk);
  {
    const float *S_in = seg_state + ((long long)bh * geo.nseg + seg) * DK * DV;
    if (a.state_t) {  // stored [DV][DK]: a lane's four rows are 16 contiguous bytes
#pragma unroll
      for (int dkb = 0; dkb < DKB; ++dkb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float4 x = *(const float4 *)(S_in + (long long)(w * RW + dv_of<PAIR>(rb, l16)) * DK + 16 * dkb + 4 * g);
          st[dkb][rb] = f32x4{x.x, x.y, x.z, x.w};
        }
    } else {
#pragma unroll
      for (int dkb = 0; dkb < DKB; ++dkb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            st[dkb][rb][i] = S_in[(long long)(16 * dkb + 4 * g + i) * DV + w * RW + dv_of<PAIR>(rb, l16)];
    }
  }
  TileIO<DK> qio, kio;
  RowIO<DV> vio;
  {
    const int Cc = min(a.chunk, a.L - t_lo);
    qio.fetch(tile_src(q, t_lo, min(BT, Cc), a.q_sn, a), a.q_sn, min(BT, Cc), a.in_rev);
    kio.fetch(tile_src(k, t_lo, min(BT, Cc), a.q_sn, a), a.q_sn, min(BT, Cc), a.in_rev);
    vio.fetch(tile_src(v, t_lo, min(BT, Cc), a.v_sn, a), a.v_sn, min(BT, Cc), a.in_rev);
  }

  const int qblk = w & 3, kh = w >> 2;  // score split: 16 queries x 32 keys per wave
  f32x4 ot[RB][4];
  int out_q0 = -1, out_rows = 0;  // the block whose accumulators ot still holds
  for (int c0 = t_lo; c0 < t_hi; c0 += a.chunk) {
    const int Cc = min(a.chunk, a.L - c0);
    const bool carry = c0 + Cc < t_hi;  // state needed after this chunk
    const int nqb_c = (Cc + BT - 1) / BT;
    for (int qb = 0; qb < nqb_c; ++qb) {
      const int q0 = c0 + qb * BT;
      const bool last_qb = qb == nqb_c - 1;
      // ---- block boundary: the previous block's output and this block's query
      // (and, with resident keys, key) tiles share one pair of barriers
      if (out_q0 >= 0 && !a.out_bf16) epilogue_store<RB, RW, DV, PAIR>(a, ot, red, b, h, out_q0, out_rows, obase, w, g, l16);
      if (out_q0 >= 0 && a.out_bf16 && a.use_gn) epilogue_groupnorm<RB, DV>(a, ot, red, w, g, l16);
      __syncthreads();  // readers of Vr, Qs/Kz, Ps and the resident slot qb are done
      if (out_q0 >= 0 && a.out_bf16) {
        static_assert(BT * (DV + 8) <= BT * LDV, "output staging fits in Vr");
        stage_out<RB, RW, DV, PAIR>(ot, Vr, w, g, l16);
      }
      if constexpr (RES)  // q and k of the same tokens: one set of sines and cosines
        TileIO<DK>::commit_rows2(qio, kio, rot, a.pos0 + q0, theta_s, step_s, Qs, Ks + qb * BT * LDQ, LDQ);
      else
        qio.template commit<true, false, SPLIT>(rot, a.pos0 + q0, theta_s, step_s, Qs, LDQ, KsL, nullptr, false, 0.f,
                                                0);
      __syncthreads();
      // unconditional (no rows when there is nothing staged), so that the stores
      // and the cross-term MFMAs below share one basic block
      store_staged<DV>(a, Vr, b, h, max(out_q0, 0), out_q0 >= 0 && a.out_bf16 ? out_rows : 0, obase);
      u32x4 qreg[KS], qlo[SPLIT ? KS : 1];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qreg[ks] = ld_op(Qs + (16 * qblk + l16) * LDQ, 32 * ks, g);
        if constexpr (SPLIT) qlo[ks] = ld_op(KsL + (16 * qblk + l16) * LDQ, 32 * ks, g);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int qb4 = 0; qb4 < 4; ++qb4) ot[rb][qb4] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 as[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const f32x4 lo = st[2 * ks][rb], hi = st[2 * ks + 1][rb];
          as[rb] = u32x4{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(hi[0], hi[1]), pack_bf2(hi[2], hi[3])};
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
      // key blocks qb-1, qb-2, ..., 0, then the diagonal block qb: a block's last
      // visit and the next block's first visit (inside a chunk) take the same
      // key block, whose tiles are then still in registers and not fetched
      // again (the sums do not depend on the order)
      for (int vi = 0; vi <= qb; ++vi) {
        const int kb = vi < qb ? qb - 1 - vi : qb;
        const bool last_visit = vi == qb;
        const int k0 = c0 + kb * BT;
        const bool upd = carry && last_qb;
        const int delta = qb - kb;
        const float gdel = delta ? dpow(lg, 64 * (delta - 1)) : 1.0f;
        uint16_t *const Kb = RES ? Ks + kb * BT * LDQ : Ks;
        __syncthreads();
        if constexpr (RES) {
          if (upd) {  // zeta-scaled copy of the resident block for the update
            TileIO<DK> kres;
            kres.load_lds(Kb, LDQ);
            kres.template commit<false, true, false, true>(false, 0, theta_s, step_s, nullptr, LDQ, nullptr, Kz, true,
                                                           lg, Cc - 1 - (k0 - c0), LDZ);
          }
        } else {
          if (upd)
            kio.template commit<true, true, SPLIT, true>(rot, a.pos0 + k0, theta_s, step_s, Kb, LDQ, KsL, Kz, true,
                                                         lg, Cc - 1 - (k0 - c0), LDZ);
          else
            kio.template commit<true, false, SPLIT>(rot, a.pos0 + k0, theta_s, step_s, Kb, LDQ, KsL, nullptr, false,
                                                    0.f, 0);
        }
        vio.template commit<false, false>(Vr, LDV, 0, theta_s, 0.0f, 0);
        // the scores read only the key block, which with resident keys was written
        // at its block boundary: no barrier between these stores and the scores
        if constexpr (!RES) __syncthreads();
        // next visit: next key block of this query block, else the first key block
        // of the next query block (of this chunk, or query block 0 of the next
        // chunk).  Its loads are issued in two parts -- K before the scores, V
        // before PV -- so the memory system absorbs them while the MFMAs run.
        int nk0 = c0 + (vi + 1 < qb ? qb - 2 - vi : qb) * BT, nend = c0 + Cc;
        if (last_visit && last_qb) {  // key block 0 of the next chunk
          nk0 = c0 + Cc;
          nend = min(a.L, nk0 + a.chunk);
        }
        const bool has_next = nk0 < t_hi;
        const bool same_tile = last_visit && !last_qb;  // its raw tiles are still in registers
        if constexpr (!RES)
          if (has_next && !same_tile)
            kio.fetch(tile_src(k, nk0, min(BT, nend - nk0), a.q_sn, a), a.q_sn, min(BT, nend - nk0), a.in_rev);
        // at the last visit: the next block's query tile (and resident key
        // tile), committed at the next block boundary.  Issued this late so the
        // registers are free during the earlier visits.
        if (last_visit) {
          const int nq0 = last_qb ? c0 + Cc : q0 + BT;
          if (nq0 < t_hi) {
            qio.fetch(tile_src(q, nq0, min(BT, nend - nq0), a.q_sn, a), a.q_sn, min(BT, nend - nq0), a.in_rev);
            if constexpr (RES)
              kio.fetch(tile_src(k, nq0, min(BT, nend - nq0), a.q_sn, a), a.q_sn, min(BT, nend - nq0), a.in_rev);
          }
        }
#pragma unroll
        for (int kb16 = 0; kb16 < 2; ++kb16) {
          f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const u32x4 ak = ld_op(Kb + (32 * kh + 16 * kb16 + l16) * LDQ, 32 * ks, g);
            sc = mfma(ak, qreg[ks], sc);
            if constexpr (SPLIT) {
              sc = mfma(ld_op(KsL + (32 * kh + 16 * kb16 + l16) * LDQ, 32 * ks, g), qreg[ks], sc);
              sc = mfma(ak, qlo[ks], sc);
            }
          }
          const int dp = (16 * qblk + l16) - (32 * kh + 16 * kb16 + 4 * g) + (delta ? 128 : 64);
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = sc[i] * (gdel * dt[dp - i]);
          *(u32x2 *)(Ps + (16 * qblk + l16) * LDT + 32 * kh + 16 * kb16 + 4 * g) = pack4(p[0], p[1], p[2], p[3]);
        }
        if (has_next && !same_tile)
          vio.fetch(tile_src(v, nk0, min(BT, nend - nk0), a.v_sn, a), a.v_sn, min(BT, nend - nk0), a.in_rev);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4 av[RB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) av[rb] = ld_op_tr(Vr, LDV, 32 * ks, w * RW + 16 * rb, g, l16);
#pragma unroll
          for (int qb4 = 0; qb4 < 4; ++qb4) {
            const u32x4 bp = ld_op(Ps + (16 * qb4 + l16) * LDT, 32 * ks, g);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) ot[rb][qb4] = mfma(av[rb], bp, ot[rb][qb4]);
          }
          if (upd) {
            // S += (zeta K)^T V over this key block
#pragma unroll
            for (int dkb = 0; dkb < DKB; ++dkb) {
              const u32x4 ak = ld_op_tr(Kz, LDZ, 32 * ks, 16 * dkb, g, l16);
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) st[dkb][rb] = mfma(ak, av[rb], st[dkb][rb]);
            }
          }
        }
      }
      out_q0 = q0;
      out_rows = min(BT, c0 + Cc - q0);
    }
  }
  // the last block's output
  if (out_q0 < 0) return;
  if (!a.out_bf16) {
    epilogue_store<RB, RW, DV, PAIR>(a, ot, red, b, h, out_q0, out_rows, obase, w, g, l16);
  } else {
    if (a.use_gn) epilogue_groupnorm<RB, DV>(a, ot, red, w, g, l16);
    epilogue_staged<RB, RW, DV, PAIR>(a, ot, Vr, b, h, out_q0, out_rows, obase, w, g, l16);
  }
}

// ---------------------------------------------------------------- pass 1: segment states
// Walks the segment chunk by chunk from a zero state:
//   S <- gamma^Cc S + sum_i gamma^(Cc-1-i) k_i^T v_i     (per chunk)
// 64 tokens at a time, double-buffered in LDS, with the global loads of the
// next two blocks in flight (two register sets, used alternately).  At the end
// it stores the segment's own state (fp32, [dk][dv]) in seg_state.

// Position of a 64-token block: its first token, and its chunk's start and length.
struct BlockPos {
  int k0, c0, Cc;
  __device__ __forceinline__ void advance(int L, int chunk) {
    k0 += BT;
    if (k0 >= c0 + Cc) {
      c0 += Cc;
      k0 = c0;
      Cc = min(chunk, L - c0);
    }
  }
  __device__ __forceinline__ int valid() const { return min(BT, c0 + Cc - k0); }
};

template <int DK, int DVW>
__global__ __launch_bounds__(NT) void seg_state_kernel(RetArgs a, TaskGeom geo, float *seg_state) {
  using T = Tile<DK, DVW>;
  constexpr int RW = T::RW, RB = T::RB, DKB = T::DKB;
  constexpr int LDK = tr_pitch(DK), LDV = tr_pitch(DVW);
  // row-major (token-major) tiles, read across rows by ld_op_tr
  __shared__ __attribute__((aligned(16))) uint16_t Vr[2][BT * LDV];
  __shared__ __attribute__((aligned(16))) uint16_t Kr[2][BT * LDK];
  __shared__ float theta_s[DK / 2];
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
  __syncthreads();
  const int c_lo = seg * geo.seg_chunks;
  const int c_hi = min(geo.nchunks, c_lo + geo.seg_chunks);
  const int t_lo = c_lo * a.chunk, t_hi = min(a.L, c_hi * a.chunk);
  f32x4 st[DKB][RB];
#pragma unroll
  for (int dkb = 0; dkb < DKB; ++dkb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) st[dkb][rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // NSET register sets of global loads in flight (block i uses set i % NSET; deeper
  // sets measured no faster); two LDS buffers
  constexpr int NSET = 2;
  RowIO<DK> kio[NSET];
  RowIO<DVW> vio[NSET];
  // pf: the next block to fetch; a block past the segment fetches no rows
  BlockPos cur{t_lo, t_lo, min(a.chunk, a.L - t_lo)}, pf = cur;
#pragma unroll
  for (int s = 0; s < NSET; ++s) {
    const int nv = pf.k0 < t_hi ? pf.valid() : 0;
    kio[s].fetch(tile_src(k, pf.k0, nv, a.q_sn, a), a.q_sn, nv, a.in_rev);
    vio[s].fetch(tile_src(v, pf.k0, nv, a.v_sn, a), a.v_sn, nv, a.in_rev);
    pf.advance(a.L, a.chunk);
  }
  int buf = 0;
  // NSET blocks per iteration, one per register set
  for (bool more = true; more;) {
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
      if (cur.k0 >= t_hi) {
        more = false;
        break;
      }
      if (cur.k0 == cur.c0 && cur.c0 > t_lo) {
        // a new chunk of the segment: decay the state over it
        const float gc = dpow(lg, cur.Cc);
#pragma unroll
        for (int dkb = 0; dkb < DKB; ++dkb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) st[dkb][rb] *= gc;
      }
      // buffer `buf` was last read two blocks ago; the barrier of the previous
      // block ordered those reads before this write
      const int zoff = cur.c0 + cur.Cc - 1 - cur.k0;
      if (a.use_theta)
        kio[s].template commit<true, true>(Kr[buf], LDK, a.pos0 + cur.k0, theta_s, lg, zoff);
      else
        kio[s].template commit<false, true>(Kr[buf], LDK, 0, theta_s, lg, zoff);
      vio[s].template commit<false, false>(Vr[buf], LDV, 0, theta_s, 0.0f, 0);
      __syncthreads();
      {  // this register set now takes the block NSET ahead
        const int nv = pf.k0 < t_hi ? pf.valid() : 0;
        kio[s].fetch(tile_src(k, pf.k0, nv, a.q_sn, a), a.q_sn, nv, a.in_rev);
        vio[s].fetch(tile_src(v, pf.k0, nv, a.v_sn, a), a.v_sn, nv, a.in_rev);
        pf.advance(a.L, a.chunk);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 bv[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) bv[rb] = ld_op_tr(Vr[buf], LDV, 32 * ks, w * RW + 16 * rb, g, l16);
#pragma unroll
        for (int dkb = 0; dkb < DKB; ++dkb) {
          const u32x4 ak = ld_op_tr(Kr[buf], LDK, 32 * ks, 16 * dkb, g, l16);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) st[dkb][rb] = mfma(ak, bv[rb], st[dkb][rb]);
        }
      }
      buf ^= 1;
      cur.advance(a.L, a.chunk);
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
// The state entering each segment of a (b, h) follows the linear recurrence
//   S(s + 1) = g_s S(s) + A_s,   g_s = gamma^len(s),   S(0) = the incoming state,
// with A_s the segment's own state from pass 1 ("Retentive Network" paper
// summary, Sec. 2.1 (3): the state carried from chunk to chunk, taken over
// whole segments).  Each step is an affine map x -> g x + A, and maps compose
// associatively: (g1, A1) then (g2, A2) is (g2 g1, g2 A1 + A2).  So the scan runs
// across the lanes of a wave: every state element (column) is held by NL
// lanes, lane j composing the maps of its R consecutive segments R j ..
// R j + R - 1 in registers; log2(NL) steps of cross-lane moves (DPP row
// shifts, no LDS traffic) compose the lanes' maps (inclusive scan), and the map
// of lanes 0 .. j-1 applied to the incoming state is the state entering lane
// j's first segment, from which the lane walks its segments again.
//
// seg_scan_kernel (state kept in registers by the output kernel): in place,
// ws[bh][s] holds the segment's own state on entry and the state entering
// segment s on exit, plus the state after the last segment in state_out.
// Lane (j, cg) of a wave takes the U consecutive elements of column group cg
// for segments R j .. R j + R - 1, loaded and stored as float4 runs straight
// from and to memory (the NL lanes of a group read U * 4 * (64 / NL) contiguous
// bytes of NL * R rows); all the scan's data stay in registers.  NSP: segments
// rounded up to a power of two.

// x from lane (lane - D) of the same 16-lane row (DPP row_shr:D); lanes
// whose source lies outside the row keep their own value.
template <int D>
__device__ __forceinline__ float lane_shr(float x) {
  static_assert(D >= 1 && D <= 15, "row shift");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                                               0x110 + D, 0xF, 0xF, false));
}

// Lanes per state element for NSP segments: few lanes keep the per-element
// overhead of the cross-lane steps low (four lanes of eight segments at 32).
__host__ __device__ constexpr int scan_lanes(int nsp) { return nsp <= 4 ? nsp : (nsp <= 32 ? 4 : (nsp <= 128 ? nsp / 8 : 16)); }

template <int NSP>
__global__ __launch_bounds__(256) void seg_scan_kernel(RetArgs a, TaskGeom geo, float *ws, const float *state_in,
                                                       float *state_out) {
  // lanes per column: a power of two within one 16-lane DPP row, R <= 16 segments each
  constexpr int NL = scan_lanes(NSP);
  constexpr int R = NSP / NL;
  constexpr int U = R <= 8 ? 8 : 4;       // consecutive elements per lane
  constexpr int CB = 4 * (64 / NL) * U;   // elements per block
  static_assert(NL <= 16 && U % 4 == 0, "lane layout");
  const long long E = (long long)a.dk * a.dv;
  const int bh = blockIdx.y, nseg = geo.nseg;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane % NL, cg = lane / NL;
  const long long e0 = (long long)blockIdx.x * CB + ((long long)w * (64 / NL) + cg) * U;  // the lane's first element
  const bool live = e0 < E;  // E is a multiple of U
  float *base = ws + (long long)bh * nseg * E + e0;
  // the incoming state first, then the segments in order, all in flight together
  float sv[U];
#pragma unroll
  for (int q = 0; q < U / 4; ++q) {
    const float4 x = (live && state_in) ? *(const float4 *)(state_in + (long long)bh * E + e0 + 4 * q)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
    sv[4 * q] = x.x;
    sv[4 * q + 1] = x.y;
    sv[4 * q + 2] = x.z;
    sv[4 * q + 3] = x.w;
  }
  float A[R][U];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int sg = j * R + r;
#pragma unroll
    for (int q = 0; q < U / 4; ++q) {
      const float4 x = (live && sg < nseg) ? *(const float4 *)(base + (long long)sg * E + 4 * q)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
      A[r][4 * q] = x.x;
      A[r][4 * q + 1] = x.y;
      A[r][4 * q + 2] = x.z;
      A[r][4 * q + 3] = x.w;
    }
  }
  const float lg = safe_log2(a.gamma[bh % a.H]);
  const int seg_len = geo.seg_chunks * a.chunk;
  float gs[R];  // g of the lane's segments; padding segments are the identity map
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int sg = j * R + r;
    gs[r] = sg < nseg ? dpow(lg, min(a.L, (sg + 1) * seg_len) - sg * seg_len) : 1.0f;
  }
  // the lane's segments composed, per element: state after = G * state before + X
  float X[U], G = 1.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) X[u] = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int u = 0; u < U; ++u) X[u] = gs[r] * X[u] + A[r][u];
    G *= gs[r];
  }
  // inclusive composition over lanes 0 .. j of the group (G is the same for
  // every element of a lane)
#define RET_SCAN_STEP(D)                                   \
  if constexpr (NL > D) {                                  \
    const float Gp = lane_shr<D>(G);                       \
    float Xp[U];                                           \
    _Pragma("unroll") for (int u = 0; u < U; ++u) Xp[u] = lane_shr<D>(X[u]); \
    if (j >= D) {                                          \
      _Pragma("unroll") for (int u = 0; u < U; ++u) X[u] = G * Xp[u] + X[u]; \
      G *= Gp;                                             \
    }                                                      \
  }
  RET_SCAN_STEP(1)
  RET_SCAN_STEP(2)
  RET_SCAN_STEP(4)
  RET_SCAN_STEP(8)
#undef RET_SCAN_STEP
  // the state entering segment R j: lanes 0 .. j-1 applied to the incoming state
  float run[U];
  {
    const float Ge = lane_shr<1>(G);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float Xe = lane_shr<1>(X[u]);
      run[u] = (NL > 1 && j > 0) ? Ge * sv[u] + Xe : sv[u];
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int sg = j * R + r;
#pragma unroll
    for (int q = 0; q < U / 4; ++q)
      if (live && sg < nseg)
        *(float4 *)(base + (long long)sg * E + 4 * q) =
            make_float4(run[4 * q], run[4 * q + 1], run[4 * q + 2], run[4 * q + 3]);
#pragma unroll
    for (int u = 0; u < U; ++u) run[u] = gs[r] * run[u] + A[r][u];
  }
  if (j == NL - 1 && live && state_out)
#pragma unroll
    for (int q = 0; q < U / 4; ++q)
      *(float4 *)(state_out + (long long)bh * E + e0 + 4 * q) =
          make_float4(run[4 * q], run[4 * q + 1], run[4 * q + 2], run[4 * q + 3]);
}

// seg_scan_seq_kernel: the same scan with one thread per four state elements
// walking all segments in order (loads of SB segments in flight, each prefix
// stored as soon as it is known).  It does the least arithmetic and streams
// best, so it is taken whenever the (b, h) x element columns alone give a
// thread to every lane of the GPU (about one 256-thread block per CU); with
// fewer heads the wavefront-level scan above spreads each column's segments
// over several lanes instead.
__global__ __launch_bounds__(256) void seg_scan_seq_kernel(RetArgs a, TaskGeom geo, float *ws, const float *state_in,
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
    constexpr int SB = 4;  // segments whose loads are in flight together
    for (int s0 = 0; s0 < geo.nseg; s0 += SB) {
      float4 d[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j)
        if (s0 + j < geo.nseg) d[j] = base[(long long)(s0 + j) * n4 + e];
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const int s = s0 + j;
        if (s >= geo.nseg) break;
        base[(long long)s * n4 + e] = run;
        const int len = min(a.L, (s + 1) * seg_len) - s * seg_len;
        const float gm = len == seg_len ? g_full : dpow(lg, len);
        run.x = gm * run.x + d[j].x;
        run.y = gm * run.y + d[j].y;
        run.z = gm * run.z + d[j].z;
        run.w = gm * run.w + d[j].w;
      }
    }
    if (state_out) ((float4 *)(state_out + (long long)bh * SZ))[e] = run;
  }
}


template <int NSP>
static void launch_seg_scan(const RetArgs &a, const TaskGeom &geo, float *ws, const float *state_in, float *state_out,
                            hipStream_t st) {
  constexpr int NL = scan_lanes(NSP), R = NSP / NL, U = R <= 8 ? 8 : 4;
  constexpr int CB = 4 * (64 / NL) * U;
  const long long E = (long long)a.dk * a.dv;
  hipLaunchKernelGGL(seg_scan_kernel<NSP>, dim3((unsigned)((E + CB - 1) / CB), a.B * a.H), dim3(256), 0, st, a, geo,
                     ws, state_in, state_out);
}

// Segments per (b, h) are at most 256 (the segment target below).
static hipError_t run_seg_scan(const RetArgs &a, const TaskGeom &geo, float *ws, const float *state_in,
                               float *state_out, hipStream_t st) {
  const int n = geo.nseg;
  const long long n4 = (long long)a.dk * a.dv / 4, seq_blocks = (n4 + 255) / 256 * a.B * a.H;
  if (seq_blocks >= 256 || n <= 1) {  // a block of the sequential scan for every CU
    hipLaunchKernelGGL(seg_scan_seq_kernel, dim3((unsigned)((n4 + 255) / 256), a.B * a.H), dim3(256), 0, st, a, geo,
                       ws, state_in, state_out);
    return hipGetLastError();
  }
  if (n <= 1) launch_seg_scan<1>(a, geo, ws, state_in, state_out, st);
  else if (n <= 2) launch_seg_scan<2>(a, geo, ws, state_in, state_out, st);
  else if (n <= 4) launch_seg_scan<4>(a, geo, ws, state_in, state_out, st);
  else if (n <= 8) launch_seg_scan<8>(a, geo, ws, state_in, state_out, st);
  else if (n <= 16) launch_seg_scan<16>(a, geo, ws, state_in, state_out, st);
  else if (n <= 32) launch_seg_scan<32>(a, geo, ws, state_in, state_out, st);
  else if (n <= 64) launch_seg_scan<64>(a, geo, ws, state_in, state_out, st);
  else if (n <= 128) launch_seg_scan<128>(a, geo, ws, state_in, state_out, st);
  else if (n <= 256) launch_seg_scan<256>(a, geo, ws, state_in, state_out, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// seg_scan_t_kernel (states handed to the query-block kernel): the state
// entering segment s goes to sinT[bh][s] as bf16 S^T[dv][dk] only.  One block
// per 64 x 64 tile of (dk, dv): each thread scans four float4s of the tile
// (coalesced loads of ws[bh][s]); the transposition goes through LDS so that
// every store writes 16 contiguous bytes of a dv row.
__global__ __launch_bounds__(256) void seg_scan_t_kernel(RetArgs a, TaskGeom geo, const float *ws, uint16_t *sinT,
                                                         const float *state_in, float *state_out) {
  constexpr int TP = 64 + 8;  // LDS pitch (bf16) of the transposed tile
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * TP];
  const long long SZ = (long long)a.dk * a.dv;
  const int bh = blockIdx.y;
  const int ntc = a.dv / 64;  // tiles along dv
  const int r0 = 64 * (blockIdx.x / ntc), c0 = 64 * (blockIdx.x % ntc);
  const int t = threadIdx.x, tr = t / 16, tc = 4 * (t % 16);  // rows tr + 16j, columns tc..tc+3
  const float lg = safe_log2(a.gamma[bh % a.H]);
  const int seg_len = geo.seg_chunks * a.chunk;
  const float g_full = dpow(lg, seg_len);
  float4 run[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    run[j] = state_in ? *(const float4 *)(state_in + bh * SZ + (long long)(r0 + tr + 16 * j) * a.dv + c0 + tc)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
  const float *base = ws + (long long)bh * geo.nseg * SZ;
  uint16_t *tb = sinT + (long long)bh * geo.nseg * SZ;
  float4 d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) d[j] = *(const float4 *)(base + (long long)(r0 + tr + 16 * j) * a.dv + c0 + tc);
  for (int s = 0; s < geo.nseg; ++s) {
    // tile[col][row] = bf16(run): thread's column tc+i, rows tr+16j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = tr + 16 * j;
      tile[(tc + 0) * TP + row] = f2bf(run[j].x);
      tile[(tc + 1) * TP + row] = f2bf(run[j].y);
      tile[(tc + 2) * TP + row] = f2bf(run[j].z);
      tile[(tc + 3) * TP + row] = f2bf(run[j].w);
    }
    const int len = min(a.L, (s + 1) * seg_len) - s * seg_len;
    const float gm = len == seg_len ? g_full : dpow(lg, len);
    float4 dn[4];
    if (s + 1 < geo.nseg)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dn[j] = *(const float4 *)(base + (long long)(s + 1) * SZ + (long long)(r0 + tr + 16 * j) * a.dv + c0 + tc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      run[j].x = gm * run[j].x + d[j].x;
      run[j].y = gm * run[j].y + d[j].y;
      run[j].z = gm * run[j].z + d[j].z;
      run[j].w = gm * run[j].w + d[j].w;
      d[j] = dn[j];
    }
    __syncthreads();
    // 64 dv rows x 64 dk (128 bytes): two 16-byte pieces per thread
    uint16_t *dst = tb + (long long)s * SZ;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pc = t + 256 * i, col = pc / 8, piece = pc % 8;
      const uint16_t *src = tile + col * TP + 8 * piece;
      const u32x2 lo = *(const u32x2 *)src, hi = *(const u32x2 *)(src + 4);
      *(u32x4 *)(dst + (long long)(c0 + col) * a.dk + r0 + 8 * piece) = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
    __syncthreads();
  }
  if (state_out)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(float4 *)(state_out + bh * SZ + (long long)(r0 + tr + 16 * j) * a.dv + c0 + tc) = run[j];
}

// ---------------------------------------------------------------- dispatch
bool mfma_supported(int dk, int dv) {
  return (dk == 64 && dv == 128) || (dk == 128 && dv == 128) || (dk == 128 && dv == 256) ||
         (dk == 256 && dv == 128) || (dk == 256 && dv == 256) || (dk == 256 && dv == 512);
}

// dv columns per workgroup in the segment-state pass: the fp32 state slice
// DK x DVW lives in the accumulators of 8 waves (<= 64 registers each).
// States of up to 128 x 256 fp32 stay in the output kernel's accumulators (eight
// waves, 64 registers each) through a segment.  Larger ones go to the
// query-block kernel; their segment-state pass holds up to 256 x 256 (128
// registers per lane) and splits d_v beyond that (each split re-reads K).
constexpr long long IN_REGS_MAX = 128 * 256, SPLIT_STATE_MAX = 256 * 256;
static bool state_in_regs(int dk, int dv) { return (long long)dk * dv <= IN_REGS_MAX; }
static int state_dvw(int dk, int dv) {
  if (state_in_regs(dk, dv)) return dv;
  int dvw = dv;
  while ((long long)dk * dvw > SPLIT_STATE_MAX) dvw /= 2;
  return dvw;
}

// Segments the segment-state pass aims for: about one workgroup per CU.
constexpr int SEG_TARGET = 256;

// Design A (the segment-output kernel, the state in its accumulators through a
// segment) when the state fits and either the chunk has at most KRES key
// blocks (its rotated keys stay in LDS) or there are chunks enough for a
// segment per CU; otherwise design B (the query-block kernel per chunk and
// 64-query block, with the bf16 state entering every chunk), whose tasks fill
// the GPU where design A's few long segments cannot (at L = 32768, 8 heads:
// chunk 2048 639 us against 1136 us; chunks 512 and 1024 stay faster in A).
// Only design A reads reversed inputs (RetArgs::in_rev).
bool chunk_state_in_regs(int B, int H, int L, int dk, int dv, int chunk) {
  if (!state_in_regs(dk, dv)) return false;
  if (chunk <= KRES * BT) return true;
  return (long long)B * H * ((L + chunk - 1) / chunk) >= SEG_TARGET;
}

ChunkPlan chunk_plan(int B, int H, int L, int dk, int dv, int chunk) {
  ChunkPlan p;
  const int nsplit = dv / state_dvw(dk, dv);
  const int nchunks = (L + chunk - 1) / chunk;
  const int units = B * H * nsplit;
  // design A: segments of several chunks; design B: every chunk a segment of its own
  const bool in_regs = chunk_state_in_regs(B, H, L, dk, dv, chunk);
  p.in_regs = in_regs;
  int nseg = in_regs ? (SEG_TARGET + units - 1) / units : nchunks;
  if (nseg > nchunks) nseg = nchunks;
  if (nseg < 1) nseg = 1;
  p.seg_chunks = (nchunks + nseg - 1) / nseg;
  p.nseg = (nchunks + p.seg_chunks - 1) / p.seg_chunks;
  const size_t SZ = (size_t)dk * dv;
  p.seg_bytes = (size_t)B * H * p.nseg * SZ * sizeof(float);
  p.sinT_bytes = in_regs ? 0 : (size_t)B * H * p.nseg * SZ * 2;
  p.ws_bytes = p.seg_bytes + p.sinT_bytes;
  return p;
}

// A second stream per device (default priority) on which a small launch can run
// beside the main one: fork from and join back to the caller's stream with
// events.  The events are shared, so the fork/launch/join sequence is done under
// a mutex; graph capture follows the fork into the side stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};

static SideStream *side_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  static std::mutex mu;
  static std::map<int, SideStream *> per_dev;
  std::lock_guard<std::mutex> lock(mu);
  auto it = per_dev.find(dev);
  if (it != per_dev.end()) return it->second;
  SideStream *ss = new SideStream;
  if (hipStreamCreateWithFlags(&ss->s, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&ss->join, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    delete ss;  // (handles that were created are kept by the runtime until exit)
    ss = nullptr;
  }
  per_dev[dev] = ss;
  return ss;
}

// Scores from hi + lo bf16 parts of the rotated q and k for every block: when
// rotation is on and some head decays fast (gamma < 0.75), its rows sum fewer
// than about (1 + gamma) / (1 - gamma) < 7 effective terms, so the rounding of
// the rotated values to bf16 (relative 2^-9 per element, which cancels only
// in exact arithmetic) would not average out (at gamma = 0 every row is one
// score times one value row).  Unrotated bf16 operands multiply exactly.
static bool split_all_blocks(const RetArgs &a) {
  if (!a.use_theta) return false;
  for (int h = 0; h < a.H; ++h)
    if (a.gamma[h] < 0.75f) return true;
  return false;
}

// Stream-ordered scratch for the parallel form's rotated keys (that call takes
// no workspace).  The device's default memory pool is told once to keep what is
// freed (release threshold raised), so repeated calls reuse the same memory
// instead of mapping it again.
static hipError_t scratch_alloc(void **p, size_t bytes, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    static std::mutex mu;
    static std::map<int, bool> kept;
    std::lock_guard<std::mutex> lock(mu);
    if (!kept[dev]) {
      hipMemPool_t pool;
      if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
        uint64_t thr = UINT64_MAX;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
      }
      (void)hipGetLastError();
      kept[dev] = true;
    }
  }
  return hipMallocAsync(p, bytes, st);
}

// The parallel form's plain-score launches take their keys by DMA, rotated once
// into stream-ordered scratch first; the chunkwise query-block launches (short
// tasks of at most chunk/64 visits, measured slower that way) rotate each key
// block as they stage it.
template <int DK, int DV>
static hipError_t run_qblocks(const RetArgs &a, TaskGeom geo, bool par, const uint16_t *sinT, hipStream_t st,
                              bool fork) {
  geo.nqb = par ? (a.L + BT - 1) / BT : (a.chunk + BT - 1) / BT;
  geo.nchunks = par ? 1 : (a.L + a.chunk - 1) / a.chunk;
  geo.ntasks = a.B * a.H * geo.nchunks * geo.nqb;
  const dim3 grid(xcd_grid(geo.ntasks));
  if (split_all_blocks(a)) {
    if (par)
      hipLaunchKernelGGL((qblock_kernel<DK, DV, true, true>), grid, dim3(NT), 0, st, a, geo, sinT, nullptr);
    else
      hipLaunchKernelGGL((qblock_kernel<DK, DV, false, true>), grid, dim3(NT), 0, st, a, geo, sinT, nullptr);
    return hipGetLastError();
  }
  if (a.in_rev) return hipErrorNotSupported;  // reversed inputs: the segment kernels only
  uint16_t *kt = nullptr;
  if (par && a.use_theta) {
    const long long nth = (long long)a.B * a.H * a.L * (DK / 8);
    const hipError_t e = scratch_alloc((void **)&kt, (size_t)nth * 16, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(rotate_keys_kernel<DK>, dim3((unsigned)((nth + 255) / 256)), dim3(256), 0, st, a, kt);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.use_gn && a.use_theta) {
    // Under GroupNorm a row whose output variance is near eps is divided by
    // about sqrt(eps), which magnifies the rounding of the rotated q and k to
    // bf16: the first query block of a sequence (the rows that sum the fewest
    // terms) takes hi+lo scores, the others plain bf16 ones.  Without rotation
    // the bf16 operands are the inputs themselves and their products are exact.
    TaskGeom g1 = geo, g2 = geo;
    g1.sel = 1;
    g1.ntasks = a.B * a.H;
    g2.sel = 2;
    const dim3 grid1(xcd_grid(g1.ntasks));
    // chunkwise: the first blocks (one small launch) run on the side stream,
    // beside the rest (measured no faster for the parallel form, whose first
    // blocks take a single short visit)
    SideStream *ss = (par || !fork) ? nullptr : side_stream();
    std::unique_lock<std::mutex> lock;
    hipStream_t st1 = st;
    if (ss) {
      lock = std::unique_lock<std::mutex>(ss->mu);
      if (hipEventRecord(ss->fork, st) == hipSuccess && hipStreamWaitEvent(ss->s, ss->fork, 0) == hipSuccess)
        st1 = ss->s;
      else
        (void)hipGetLastError();
    }
    if (par) {
      hipLaunchKernelGGL((qblock_kernel<DK, DV, true, true>), grid1, dim3(NT), 0, st1, a, g1, sinT, nullptr);
      hipLaunchKernelGGL((qblock_kernel<DK, DV, true, false, true>), grid, dim3(NT), 0, st, a, g2, sinT, kt);
    } else {
      hipLaunchKernelGGL((qblock_kernel<DK, DV, false, true>), grid1, dim3(NT), 0, st1, a, g1, sinT, nullptr);
      hipLaunchKernelGGL((qblock_kernel<DK, DV, false, false>), grid, dim3(NT), 0, st, a, g2, sinT, nullptr);
    }
    e = hipGetLastError();
    if (st1 != st) {
      const hipError_t ej = hipEventRecord(ss->join, st1) == hipSuccess ? hipStreamWaitEvent(st, ss->join, 0)
                                                                         : hipGetLastError();
      if (e == hipSuccess) e = ej;
    }
  } else if (e == hipSuccess) {
    if (par)
      hipLaunchKernelGGL((qblock_kernel<DK, DV, true, false, true>), grid, dim3(NT), 0, st, a, geo, sinT, kt);
    else
      hipLaunchKernelGGL((qblock_kernel<DK, DV, false, false>), grid, dim3(NT), 0, st, a, geo, sinT, nullptr);
    e = hipGetLastError();
  }
  if (kt) {
    const hipError_t ef = hipFreeAsync(kt, st);
    if (e == hipSuccess) e = ef;
  }
  return e;
}

// The segment-output pass of design A: hi+lo scores when GroupNorm follows
// rotation (or a head decays fast), resident keys when they fit, else plain.
template <int DK, int DV>
static hipError_t launch_seg_out(const RetArgs &a, TaskGeom geo, const float *seg, hipStream_t st) {
  geo.ntasks = a.B * a.H * geo.nseg;
  const dim3 grid(xcd_grid(geo.ntasks));
  if ((a.use_gn && a.use_theta) || split_all_blocks(a))
    hipLaunchKernelGGL((seg_out_kernel<DK, DV, true, false>), grid, dim3(NT), 0, st, a, geo, seg);
  else if (a.chunk <= kres_of(DK) * BT)  // the chunk's keys fit in LDS
    hipLaunchKernelGGL((seg_out_kernel<DK, DV, false, true>), grid, dim3(NT), 0, st, a, geo, seg);
  else
    hipLaunchKernelGGL((seg_out_kernel<DK, DV, false, false>), grid, dim3(NT), 0, st, a, geo, seg);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t run_chunkwise(const RetArgs &a, const ChunkPlan &p, char *ws, const float *state_in,
                                float *state_out, hipStream_t st, bool fork) {
  constexpr bool FITS = (long long)DK * DV <= IN_REGS_MAX;  // design A possible
  constexpr int DVW1 = FITS ? DV : (DK * DV > SPLIT_STATE_MAX ? (int)(SPLIT_STATE_MAX / DK) : DV);
  const bool in_regs = FITS && p.in_regs;
  if (a.in_rev && !in_regs) return hipErrorNotSupported;  // reversed inputs: design A only
  float *seg = (float *)ws;
  uint16_t *sinT = in_regs ? nullptr : (uint16_t *)(ws + p.seg_bytes);
  TaskGeom geo{p.nseg, p.seg_chunks, DV / DVW1, 1, 0, (a.L + a.chunk - 1) / a.chunk};
  geo.ntasks = a.B * a.H * geo.nseg * geo.nsplit;
  hipLaunchKernelGGL((seg_state_kernel<DK, DVW1>), dim3(xcd_grid(geo.ntasks)), dim3(NT), 0, st, a, geo, seg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (in_regs) {
    e = run_seg_scan(a, geo, seg, state_in, state_out, st);
    if (e != hipSuccess) return e;
  } else {
    static_assert(DK % 64 == 0 && DV % 64 == 0, "64 x 64 scan tiles");
    hipLaunchKernelGGL(seg_scan_t_kernel, dim3((DK / 64) * (DV / 64), a.B * a.H), dim3(256), 0, st, a, geo, seg, sinT,
                       state_in, state_out);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (FITS) {
    if (!in_regs) return run_qblocks<DK, DV>(a, geo, false, sinT, st, fork);
    return launch_seg_out<DK, DV>(a, geo, seg, st);
  } else {
    return run_qblocks<DK, DV>(a, geo, false, sinT, st, fork);
  }
}

// Design A's output pass alone, on the states entering each segment already in
// ws (RetArgs::state_t: written transposed by a call with dk and dv swapped).
template <int DK, int DV>
static hipError_t run_chunkwise_out(const RetArgs &a, const ChunkPlan &p, char *ws, hipStream_t st) {
  if constexpr ((long long)DK * DV <= IN_REGS_MAX) {
    if (!p.in_regs) return hipErrorNotSupported;
    TaskGeom geo{p.nseg, p.seg_chunks, 1, 1, 0, (a.L + a.chunk - 1) / a.chunk};
    return launch_seg_out<DK, DV>(a, geo, (float *)ws, st);
  } else {
    return hipErrorNotSupported;
  }
}

hipError_t launch_mfma_parallel(const RetArgs &a, hipStream_t st) {
  TaskGeom geo{1, 1, 1, 1, 0, 1};
  if (a.dk == 64 && a.dv == 128) return run_qblocks<64, 128>(a, geo, true, nullptr, st, false);
  if (a.dk == 128 && a.dv == 128) return run_qblocks<128, 128>(a, geo, true, nullptr, st, false);
  if (a.dk == 128 && a.dv == 256) return run_qblocks<128, 256>(a, geo, true, nullptr, st, false);
  if (a.dk == 256 && a.dv == 128) return run_qblocks<256, 128>(a, geo, true, nullptr, st, false);
  if (a.dk == 256 && a.dv == 256) return run_qblocks<256, 256>(a, geo, true, nullptr, st, false);
  if (a.dk == 256 && a.dv == 512) return run_qblocks<256, 512>(a, geo, true, nullptr, st, false);
  return hipErrorNotSupported;
}

int resident_chunk_max(int dk) { return kres_of(dk) * BT; }

hipError_t launch_mfma_chunkwise_out(const RetArgs &a, const ChunkPlan &p, void *ws, hipStream_t st) {
  char *w = (char *)ws;
  if (a.dk == 64 && a.dv == 128) return run_chunkwise_out<64, 128>(a, p, w, st);
  if (a.dk == 128 && a.dv == 128) return run_chunkwise_out<128, 128>(a, p, w, st);
  if (a.dk == 128 && a.dv == 256) return run_chunkwise_out<128, 256>(a, p, w, st);
  if (a.dk == 256 && a.dv == 128) return run_chunkwise_out<256, 128>(a, p, w, st);
  return hipErrorNotSupported;
}

hipError_t launch_mfma_chunkwise(const RetArgs &a, const ChunkPlan &p, void *ws, const float *state_in,
                                 float *state_out, hipStream_t st, bool fork) {
  char *w = (char *)ws;
  if (a.dk == 64 && a.dv == 128) return run_chunkwise<64, 128>(a, p, w, state_in, state_out, st, fork);
  if (a.dk == 128 && a.dv == 128) return run_chunkwise<128, 128>(a, p, w, state_in, state_out, st, fork);
  if (a.dk == 128 && a.dv == 256) return run_chunkwise<128, 256>(a, p, w, state_in, state_out, st, fork);
  if (a.dk == 256 && a.dv == 128) return run_chunkwise<256, 128>(a, p, w, state_in, state_out, st, fork);
  if (a.dk == 256 && a.dv == 256) return run_chunkwise<256, 256>(a, p, w, state_in, state_out, st, fork);
  if (a.dk == 256 && a.dv == 512) return run_chunkwise<256, 512>(a, p, w, state_in, state_out, st, fork);
  return hipErrorNotSupported;
}

}  // namespace ret
