// Skinny path of the Muon step: matrices whose short side m is at most 32
// (e.g. the 74 fused [24, 10240] parameters of the HyperParallel RFC, item 3).
//
// The m x m Gram matrix is tiny and the long side n is long, so the work is
// memory-bound.  X (m x n in the Newton-Schulz orientation, rows padded to 32)
// is cut into chunks of L columns, one workgroup per chunk.  sk_first fuses
// momentum, the Nesterov direction U, the Frobenius-norm partials and the
// split-K Gram partial U_c U_c^T of each chunk (bf16 MFMA, fp32 accumulation)
// and stores U, unnormalised, in MFMA-ready 32-column x 8-row tiles.  Two
// forms of Newton-Schulz follow.
//
// Gram space (default).  Every step left-multiplies X by a polynomial of the
// Gram matrix, X_{k+1} = B_k X_k with B_k = a I + b A_k + c A_k^2 (the
// HyperParallel-FSDP Eq. (1) step), so with A_0 = X_0 X_0^T
//   A_{k+1} = B_k A_k B_k,   X_K = (B_{K-1} ... B_0) X_0,
// exactly in exact arithmetic (the Gram Newton-Schulz of the DMuon-2 paper,
// Appendix C.3: iterate on the Gram matrix, multiply back into X once).  All
// B_k are polynomials in A_0, so they commute and stay symmetric.
//   sk_gram_ns  one workgroup per matrix: A_0 = (sum of the chunk partials,
//               in chunk order, fp64) / (||U||_F + eps)^2, then the K steps
//               on 16x16x4 MFMA (fp32 on the bf16 paths, fp64 on the check
//               path), Q = B_{K-1} ... B_0 / (||U||_F + eps) written as the
//               per-lane operand fragments of the apply kernel: a bf16 hi +
//               lo pair (the product keeps about 16 bits of Q), or fp32.
//   sk_apply    one wave per 64 columns: O = Q U on 32x32 MFMA, then the
//               decoupled decay and the update of W (or O written out).  A
//               wide W gets O^T = U^T Q (Q is symmetric; the MFMA operands
//               swapped) through a wave-private LDS buffer, so W is read and
//               written as 16-byte row segments; for a tall W, whose rows are
//               the columns of U, O = Q U leaves each lane a run of 4
//               consecutive elements of one W row.
// Three launches and two passes over U, whatever K is.
//
// Step by step.  The iteration in the pages' order, K rounds of
//   sk_bprime   one workgroup per matrix: A = X X^T from the chunk partials,
//               A A on fp32 MFMA, B' = a I + b A + c A A as fragments;
//   sk_iter     one workgroup per chunk: stage the chunk in LDS, X' = B' X on
//               MFMA in place, store X' and its Gram partial for the next
//               step; the last step applies the update instead.
//
// X stays in the L2 / Infinity Cache between launches.  Every reduction has a
// fixed order, so results are bitwise reproducible.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace muon {
namespace {

constexpr int SK_THREADS = 256;
constexpr int SK_WAVES = SK_THREADS / WAVE;
constexpr int SK_MP = 32;  // rows padded to one 32x32 MFMA block

// MODE 0: X stored bf16 (bf16 operands).  MODE 1: X stored fp32, fp32 Gram
// operands, bf16 hi+lo operands for B' X.  MODE 2: fp32 everywhere.
template <int MODE> struct SkCfg;
template <> struct SkCfg<0> { typedef bf16_t XS; static constexpr int L = MUON_SK_CHUNK_BF16, LDX = L + 8; };
template <> struct SkCfg<1> { typedef float XS; static constexpr int L = MUON_SK_CHUNK_F32, LDX = L + 4; };
template <> struct SkCfg<2> { typedef float XS; static constexpr int L = MUON_SK_CHUNK_F32, LDX = L + 4; };

template <int MODE> struct SkLds {
  static constexpr int TILE = SK_MP * SkCfg<MODE>::LDX * (int)sizeof(typename SkCfg<MODE>::XS);
  static constexpr int RED = SK_WAVES * SK_MP * (SK_MP + 1) * 4;   // Gram partial reduction buffer
  static constexpr int BYTES = TILE > RED ? TILE : RED;
};
static_assert(MUON_SK_CHUNK_BF16 % 64 == 0 && MUON_SK_CHUNK_F32 % 64 == 0, "chunk must be a multiple of 64");

__device__ __forceinline__ void tri_rc(int idx, int& r, int& s) {
  int rr = (int)((sqrtf(8.0f * idx + 1.0f) - 1.0f) * 0.5f);
  while (rr * (rr + 1) / 2 > idx) --rr;
  while ((rr + 1) * (rr + 2) / 2 <= idx) ++rr;
  r = rr;
  s = idx - rr * (rr + 1) / 2;
}

// Element (row r, column j) of a stored [M,N] matrix in the Newton-Schulz
// orientation (m x n): row-major if not transposed, else the transpose.
__device__ __forceinline__ int64_t stored_index(bool transposed, int r, int64_t j, int m, int64_t n) {
  return transposed ? j * m + r : (int64_t)r * n + j;
}

// 16-byte vectors of the staged chunk.
template <int MODE> struct Vec {
  typedef typename SkCfg<MODE>::XS XS;
  static constexpr int EPV = 16 / (int)sizeof(XS);
  static constexpr int PER_ROW = SkCfg<MODE>::L / EPV;
};

// Gram partial of the staged chunk: out[idx(r,s)] = sum_k X[r][k] X[s][k] over
// the L staged columns, lower triangle packed (idx = r(r+1)/2 + s).  Wave w
// takes columns [w L/4, (w+1) L/4); the four wave sums are added in order.
// The tile holds mr rows (mr >= m, rows >= m zero); rows >= mr read as zero.
template <int MODE>
__device__ void gram_partial(unsigned char* lds_raw, float* __restrict__ out, int T, int mr) {
  typedef SkCfg<MODE> C;
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = threadIdx.x / WAVE;
  const bool live = (lane & 31) < mr;
  const int row = live ? (lane & 31) : 0;
  f32x16 acc = {};
  constexpr int KW = C::L / SK_WAVES;
  if constexpr (MODE == 0) {
    const bf16_t* lx = reinterpret_cast<const bf16_t*>(lds_raw);
    const int koff = (lane >> 5) * 8;
#pragma unroll 4
    for (int k0 = w * KW; k0 < (w + 1) * KW; k0 += 16) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(lx + row * C::LDX + k0 + koff);
      if (!live) v = bf16x8{};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, v, acc, 0, 0, 0);
    }
  } else {
    const float* lx = reinterpret_cast<const float*>(lds_raw);
    const int koff = lane >> 5;
#pragma unroll 8
    for (int k0 = w * KW; k0 < (w + 1) * KW; k0 += 2) {
      const float v = live ? lx[row * C::LDX + k0 + koff] : 0.f;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(v, v, acc, 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done reading the staged chunk
  float* red = reinterpret_cast<float*>(lds_raw);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    red[(w * SK_MP + mfma32_row(lane, r)) * (SK_MP + 1) + mfma32_col(lane)] = acc[r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < T; idx += SK_THREADS) {
    int r, s;
    tri_rc(idx, r, s);
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < SK_WAVES; ++q) v += red[(q * SK_MP + r) * (SK_MP + 1) + s];
    out[idx] = v;
  }
}

// Sum of a per-thread value over the workgroup, fixed order.
__device__ float block_sum(float v, float* wsum) {
  v = wave_sum(v);
  if ((threadIdx.x & (WAVE - 1)) == 0) wsum[threadIdx.x / WAVE] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < SK_WAVES; ++q) s += wsum[q];
  return s;
}

// Staged chunk <-> workspace, 16-byte vectors; rows >= m of the LDS tile zeroed.
template <int MODE>
__device__ void chunk_load(const typename SkCfg<MODE>::XS* __restrict__ src, unsigned char* lds_raw, int m,
                           int64_t ldx) {
  typedef SkCfg<MODE> C;
  typedef Vec<MODE> V;
  typename C::XS* lx = reinterpret_cast<typename C::XS*>(lds_raw);
  constexpr int N = SK_MP * V::PER_ROW / SK_THREADS;
  uint4 d[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int v = threadIdx.x + SK_THREADS * i;
    const int r = v / V::PER_ROW, cv = (v % V::PER_ROW) * V::EPV;
    d[i] = make_uint4(0, 0, 0, 0);
    if (r < m) d[i] = *reinterpret_cast<const uint4*>(src + r * ldx + cv);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int v = threadIdx.x + SK_THREADS * i;
    const int r = v / V::PER_ROW, cv = (v % V::PER_ROW) * V::EPV;
    *reinterpret_cast<uint4*>(lx + r * C::LDX + cv) = d[i];
  }
}

template <int MODE>
__device__ void chunk_store(typename SkCfg<MODE>::XS* __restrict__ dst, const unsigned char* lds_raw, int m,
                            int64_t ldx) {
  typedef SkCfg<MODE> C;
  typedef Vec<MODE> V;
  const typename C::XS* lx = reinterpret_cast<const typename C::XS*>(lds_raw);
  for (int v = threadIdx.x; v < m * V::PER_ROW; v += SK_THREADS) {
    const int r = v / V::PER_ROW, cv = (v % V::PER_ROW) * V::EPV;
    *reinterpret_cast<uint4*>(dst + r * ldx + cv) = *reinterpret_cast<const uint4*>(lx + r * C::LDX + cv);
  }
}

// Gram path: U in MFMA-ready tiles.  For matrix b, 32-column block jb and
// 8-row group g, a 256-element tile holds X[8 g + t][32 jb + c] at c * 8 + t;
// tiles are ordered (b, jb, g), NB = ceil(n / 32) blocks, G = ceil(m / 8)
// groups.  Rows >= m and columns >= n hold zeros.  A lane's MFMA operand (8
// rows of one column) is one contiguous 16- or 32-byte run, and the 64 lanes
// of a wave read 1 or 2 KB in one piece.
__device__ __forceinline__ int64_t xg_tile(int64_t b, int64_t jb, int g, int64_t NB, int G) {
  return ((b * NB + jb) * G + g) * 256;
}

// Staged chunk (columns [32 jb0, 32 jb0 + L)) -> tiles.
template <int MODE>
__device__ void chunk_store_xg(typename SkCfg<MODE>::XS* __restrict__ xg, const unsigned char* lds_raw, int64_t b,
                               int64_t jb0, int64_t NB, int G) {
  typedef SkCfg<MODE> C;
  typedef typename C::XS XS;
  const XS* lx = reinterpret_cast<const XS*>(lds_raw);
  constexpr int NBC = C::L / 32;
  const int nb = (int)(NB - jb0 < NBC ? NB - jb0 : NBC);
  for (int v = threadIdx.x; v < nb * G * 32; v += SK_THREADS) {
    const int c = v & 31, g = (v >> 5) % G, jl = (v >> 5) / G;
    const XS* src = lx + (8 * g) * C::LDX + jl * 32 + c;
    XS* dst = xg + xg_tile(b, jb0 + jl, g, NB, G) + c * 8;
    if constexpr (sizeof(XS) == 2) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = (uint32_t)src[(2 * q) * C::LDX] | ((uint32_t)src[(2 * q + 1) * C::LDX] << 16);
      *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      f32x4 lo, hi;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lo[q] = src[q * C::LDX];
        hi[q] = src[(q + 4) * C::LDX];
      }
      *reinterpret_cast<f32x4*>(dst) = lo;
      *reinterpret_cast<f32x4*>(dst + 4) = hi;
    }
  }
}

// B' fragments of one lane, as written by sk_bprime and read by sk_iter:
// 64 bytes per lane, 4 KB per matrix.
//   bf16 modes: hi[kb][t], lo[kb][t] = B'[lane%32][kb*16 + (lane/32)*8 + t]  (kb < 2, t < 8)
//   fp32 mode:  f[kb] = B'[lane%32][kb*2 + lane/32]                          (kb < 16)
struct BFrag {
  uint4 q[4];
};

// X' = B' X for the staged chunk, in place in LDS.  Wave w handles 32-column
// blocks w, w+4, ...
template <int MODE>
__device__ void apply_bx(unsigned char* lds_raw, const BFrag& fr) {
  typedef SkCfg<MODE> C;
  typedef typename C::XS XS;
  XS* lx = reinterpret_cast<XS*>(lds_raw);
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = threadIdx.x / WAVE;
  const int row = lane & 31, hi8 = (lane >> 5) * 8;
  constexpr int NB = C::L / 32;
  if constexpr (MODE == 2) {
    float bf[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf[4 * i] = __uint_as_float(fr.q[i].x);
      bf[4 * i + 1] = __uint_as_float(fr.q[i].y);
      bf[4 * i + 2] = __uint_as_float(fr.q[i].z);
      bf[4 * i + 3] = __uint_as_float(fr.q[i].w);
    }
    for (int jb = w; jb < NB; jb += SK_WAVES) {
      const int col = jb * 32 + row;
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < 16; ++kb) {
        const float xv = lx[(kb * 2 + (lane >> 5)) * C::LDX + col];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(bf[kb], xv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) lx[mfma32_row(lane, r) * C::LDX + col] = acc[r];
    }
  } else {
    const bf16x8 bh[2] = {__builtin_bit_cast(bf16x8, fr.q[0]), __builtin_bit_cast(bf16x8, fr.q[1])};
    const bf16x8 bl[2] = {__builtin_bit_cast(bf16x8, fr.q[2]), __builtin_bit_cast(bf16x8, fr.q[3])};
    for (int jb = w; jb < NB; jb += SK_WAVES) {
      const int col = jb * 32 + row;
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if constexpr (MODE == 0) {
          bf16x8 xv;
#pragma unroll
          for (int t = 0; t < 8; ++t) xv[t] = __builtin_bit_cast(__bf16, lx[(kb * 16 + hi8 + t) * C::LDX + col]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[kb], xv, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl[kb], xv, acc, 0, 0, 0);
        } else {
          bf16x8 xh, xl;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float v = lx[(kb * 16 + hi8 + t) * C::LDX + col];
            const bf16_t h = f2bf(v);
            xh[t] = __builtin_bit_cast(__bf16, h);
            xl[t] = __builtin_bit_cast(__bf16, f2bf(v - bf2f(h)));
          }
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[kb], xh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[kb], xl, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl[kb], xh, acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (MODE == 0) lx[mfma32_row(lane, r) * C::LDX + col] = f2bf(acc[r]);
        else lx[mfma32_row(lane, r) * C::LDX + col] = acc[r];
      }
    }
  }
}

// Fragments of a 32x32 fp32 matrix Q (zero outside m x m) in the BFrag layout,
// one lane each; called by the 64 lanes of one wave.  HALVES (fp32 only): the
// K slot (kb, lane/32) is column 16 (lane/32) + kb instead of 2 kb + lane/32,
// so that a lane's 16 slots are 16 consecutive rows of X.
template <int MODE, bool HALVES = false>
__device__ __forceinline__ BFrag make_frag(const float (*Q)[SK_MP + 1], int lane) {
  const int row = lane & 31;
  BFrag f;
  if constexpr (MODE == 2) {
    float v[16];
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) v[kb] = Q[row][HALVES ? 16 * (lane >> 5) + kb : 2 * kb + (lane >> 5)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.q[i] = make_uint4(__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]), __float_as_uint(v[4 * i + 2]),
                          __float_as_uint(v[4 * i + 3]));
  } else {
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t h2 = 0, l2 = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float v = Q[row][kb * 16 + (lane >> 5) * 8 + 2 * p + e];
          const bf16_t h = f2bf(v);
          const bf16_t l = f2bf(v - bf2f(h));
          h2 |= (uint32_t)h << (16 * e);
          l2 |= (uint32_t)l << (16 * e);
        }
        hw[kb * 4 + p] = h2;
        lw[kb * 4 + p] = l2;
      }
    }
    f.q[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    f.q[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
    f.q[2] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    f.q[3] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
  }
  return f;
}
template <int MODE, bool HALVES = false>
__device__ void write_frag(const float (*Q)[SK_MP + 1], BFrag* __restrict__ out, int lane) {
  out[lane] = make_frag<MODE, HALVES>(Q, lane);
}

// ---------------------------------------------------------------------------
// B' of one Newton-Schulz step, one workgroup per matrix.
//   first: A and B' are scaled by inv^2 and inv, inv = 1/(||U||_F + eps)
//          from the norm partials (the first step works on U = X0 / inv).
// ---------------------------------------------------------------------------
template <int MODE>
__global__ void __launch_bounds__(SK_THREADS)
sk_bprime(const float* __restrict__ gp, const float* __restrict__ sp, int first, float eps, int m, int S, int T,
          float ca, float cb, float cc, BFrag* __restrict__ bfrag) {
  __shared__ float As[SK_MP][SK_MP + 1];
  __shared__ float Bp[SK_MP][SK_MP + 1];
  __shared__ float inv_s;
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (WAVE - 1);
  for (int e = t; e < SK_MP * (SK_MP + 1); e += SK_THREADS) (&As[0][0])[e] = 0.f;
  if (t < WAVE) {
    // inv from the norm partials: lane-strided sums, then a fixed butterfly
    float inv = 1.f;
    if (first) {
      float v = 0.f;
      for (int q = lane; q < S; q += WAVE) v += sp[b * S + q];
      v = wave_sum(v);
      const float den = sqrtf(v) + eps;
      inv = den > 0.f ? 1.f / den : 0.f;
    }
    if (lane == 0) inv_s = inv;
  }
  __syncthreads();
  const float inv = inv_s;
  const float scaleA = inv * inv;
  const float* g = gp + b * S * (int64_t)T;
  for (int idx = t; idx < T; idx += SK_THREADS) {
    // all chunk partials of one entry: 16 loads in flight, added in chunk order
    float v = 0.f;
    for (int q0 = 0; q0 < S; q0 += 16) {
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (q0 + i < S) ? g[(int64_t)(q0 + i) * T + idx] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) v += x[i];
    }
    int r, s;
    tri_rc(idx, r, s);
    v *= scaleA;
    As[r][s] = v;
    As[s][r] = v;
  }
  __syncthreads();
  if (t < WAVE) {
    // A A on fp32 MFMA: A operand A[lane%32][2kb + lane/32], B operand A[2kb + lane/32][lane%32]
    f32x16 acc = {};
#pragma unroll
    for (int kb = 0; kb < 16; ++kb)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[lane & 31][2 * kb + (lane >> 5)],
                                                 As[2 * kb + (lane >> 5)][lane & 31], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = mfma32_row(lane, r), j = mfma32_col(lane);
      const float v = (i < m && j < m) ? cb * As[i][j] + cc * acc[r] + (i == j ? ca : 0.f) : 0.f;
      Bp[i][j] = v * inv;
    }
  }
  __syncthreads();
  if (t < WAVE) write_frag<MODE>(Bp, bfrag + b * WAVE, lane);
}

// ---------------------------------------------------------------------------
// Newton-Schulz in Gram space, one workgroup per matrix (four waves).  The
// 32x32 products run on 16x16x4 MFMA in fp32 (bf16 modes: the recurrence's
// rounding stays near 1e-6 of O, far below what bf16 operands cost) or in
// fp64 (fp32 check path).
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int GSD = SK_MP + 1;                 // LDS row stride of the 32x32 matrices
constexpr int GS_MAT = SK_MP * GSD;            // elements per matrix
constexpr int GS_STAGE = 6144;                 // floats of partials staged per round
static_assert(GS_STAGE % SK_THREADS == 0, "whole rounds of loads");
static_assert(SK_MP * (SK_MP + 1) / 2 <= 3 * SK_THREADS, "each thread owns at most three Gram entries");

// Per-step coefficients (a_k, b_k, c_k), k < 64, passed by value.
struct Coeffs {
  float c[3 * 64];
};

// 16x16x4 MFMA per scalar type.  Lane l supplies X[l%16][k + l/16] and
// Y[k + l/16][l%16]; the result's register r is column l%16 and row row(r, l)
// (the two types place rows differently).
template <typename R> struct Mf;
template <> struct Mf<double> {
  typedef f64x4 V;
  static __device__ __forceinline__ V mma(double a, double b, V c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int row(int r, int lane) { return 4 * r + (lane >> 4); }
};
template <> struct Mf<float> {
  typedef f32x4 V;
  static __device__ __forceinline__ V mma(float a, float b, V c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int row(int r, int lane) { return 4 * (lane >> 4) + r; }
};

// Block (bi, bj), 16x16, of X Y for 32x32 X, Y in LDS; only k < KM
// contributes (rows and columns >= m are zero padding).
template <typename R, int KM>
__device__ __forceinline__ typename Mf<R>::V mul_blk(const R* X, const R* Y, int bi, int bj, int lane) {
  typename Mf<R>::V acc = {};
  const int i = 16 * bi + (lane & 15), j = 16 * bj + (lane & 15), g = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 < KM; k0 += 4) acc = Mf<R>::mma(X[i * GSD + k0 + g], Y[(k0 + g) * GSD + j], acc);
  return acc;
}
template <typename R>
__device__ __forceinline__ void put_blk(R* Z, const typename Mf<R>::V& v, int bi, int bj, int lane) {
#pragma unroll
  for (int r = 0; r < 4; ++r) Z[(16 * bi + Mf<R>::row(r, lane)) * GSD + 16 * bj + (lane & 15)] = v[r];
}

// The K steps on A (= A_0 in, overwritten) and P (= I in P0; the result,
// B_{K-1} ... B_0, is returned: P0 or P1, which alternate so that a step's
// new P needs no barrier against the reads of the old one); wave w owns
// output block (w / 2, w % 2) of every product, three barriers per step.
// Padded rows and columns of A stay zero and never reach the m x m corner of P.
template <typename R, int KM>
__device__ R* gram_steps(R* A, R* Bm, R* P0, R* P1, R* Tm, int steps, const Coeffs& cf) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = threadIdx.x / WAVE, bi = w >> 1, bj = w & 1;
  const bool active = w < 4;   // waves beyond the fourth only take the barriers
  R* P = P0;
  R* Pn = P1;
  for (int k = 0; k < steps; ++k) {
    const R ca = cf.c[3 * k], cb = cf.c[3 * k + 1], cc = cf.c[3 * k + 2];
    if (active) {
      const typename Mf<R>::V a2 = mul_blk<R, KM>(A, A, bi, bj, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * bi + Mf<R>::row(r, lane), j = 16 * bj + (lane & 15);
        Bm[i * GSD + j] = (i == j ? ca : R(0)) + cb * A[i * GSD + j] + cc * a2[r];
      }
    }
    __syncthreads();
    const bool more = k + 1 < steps;
    if (active) {
      put_blk<R>(Pn, mul_blk<R, KM>(Bm, P, bi, bj, lane), bi, bj, lane);                // B_k P
      if (more) put_blk<R>(Tm, mul_blk<R, KM>(A, Bm, bi, bj, lane), bi, bj, lane);      // A_k B_k
    }
    __syncthreads();
    R* t = P; P = Pn; Pn = t;
    if (more) {
      if (active) put_blk<R>(A, mul_blk<R, KM>(Tm, Bm, bi, bj, lane), bi, bj, lane);   // A_{k+1} = B_k A_k B_k
      __syncthreads();
    }
  }
  return P;
}

// LDS of gram_q: A | B | P0 | P1 | Tm, the partials stage aliasing B, P0,
// P1 and Tm (and beyond).
template <int MODE>
struct GramLds {
  typedef typename std::conditional<MODE == 2, double, float>::type R;
  static constexpr int MATB = GS_MAT * (int)sizeof(R);
  static constexpr int RAW = 5 * MATB > MATB + 4 * GS_STAGE ? 5 * MATB : MATB + 4 * GS_STAGE;
};

// Q = B_{K-1} ... B_0 / (||U||_F + eps) of matrix b into Qf (zero outside
// m x m) by a workgroup of NT threads: all of them load the partials, the
// first SK_THREADS do the rest, every thread takes the barriers.  raw is
// GramLds<MODE>::RAW bytes of LDS, free again when this returns (it ends with
// a barrier).  mid() runs in every thread once the partials are summed (the
// loads of the workgroup's other work may start there without delaying the
// partials).
struct NoMid {
  __device__ void operator()() const {}
};
template <int MODE, int NT = SK_THREADS, typename MID = NoMid>
__device__ void gram_q(const float* __restrict__ gp, const float* __restrict__ sp, float eps, int m, int S, int T,
                       int steps, const Coeffs& cf, int64_t b, unsigned char* raw, float (*Qf)[SK_MP + 1],
                       double* inv_s, MID mid = MID{}) {
  typedef typename GramLds<MODE>::R R;
  R* A = reinterpret_cast<R*>(raw);
  R* Bm = A + GS_MAT;
  R* P = A + 2 * GS_MAT;
  R* P1 = A + 3 * GS_MAT;
  R* Tm = A + 4 * GS_MAT;
  float* stage = reinterpret_cast<float*>(raw + GramLds<MODE>::MATB);

  const int t = threadIdx.x;
  const int lane = t & (WAVE - 1);
  const bool worker = t < SK_THREADS;
  if (worker)
    for (int e = t; e < GS_MAT; e += SK_THREADS) A[e] = R(0);

  // A_0 entries: thread t owns packed entries t, t + 256, t + 512 and adds the
  // chunk partials in chunk order (fp64); the partials pass through LDS in
  // rounds of up to GS_STAGE floats, all loads of a round in flight at once.
  double acc[3] = {0., 0., 0.};
  const float* g = gp + b * (int64_t)S * T;
  const int qb = GS_STAGE / T;
  static_assert(GS_STAGE % NT == 0 && NT % SK_THREADS == 0, "whole rounds of loads");
  constexpr int PER = GS_STAGE / NT;
  for (int q0 = 0; q0 < S; q0 += qb) {
    const int nq = S - q0 < qb ? S - q0 : qb;
    const int tot = nq * T;
    const float* src = g + (int64_t)q0 * T;
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int f = t + NT * i;
      v[i] = f < tot ? src[f] : 0.f;
    }
    if (q0 == 0 && t < WAVE) {
      // 1 / (||U||_F + eps) from the chunk norm partials, fp64 (its loads
      // overlap the first round of Gram partials)
      double sv = 0.;
      for (int q = lane; q < S; q += WAVE) sv += (double)sp[b * S + q];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) sv += __shfl_xor(sv, o, WAVE);
      const double den = sqrt(sv) + (double)eps;
      if (lane == 0) *inv_s = den > 0. ? 1. / den : 0.;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int f = t + NT * i;
      if (f < tot) stage[f] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int e = t + SK_THREADS * u;
      if (worker && e < T)
        for (int q = 0; q < nq; ++q) acc[u] += (double)stage[q * T + e];
    }
    __syncthreads();
  }
  mid();
  const double inv = *inv_s;
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int e = t + SK_THREADS * u;
    if (worker && e < T) {
      int r, s;
      tri_rc(e, r, s);
      const R v = (R)(acc[u] * inv * inv);
      A[r * GSD + s] = v;
      A[s * GSD + r] = v;
    }
  }
  if (worker)
    for (int e = t; e < GS_MAT; e += SK_THREADS) P[e] = (e / GSD == e % GSD) ? R(1) : R(0);
  __syncthreads();

  switch ((m + 7) >> 3) {
    case 1: P = gram_steps<R, 8>(A, Bm, P, P1, Tm, steps, cf); break;
    case 2: P = gram_steps<R, 16>(A, Bm, P, P1, Tm, steps, cf); break;
    case 3: P = gram_steps<R, 24>(A, Bm, P, P1, Tm, steps, cf); break;
    default: P = gram_steps<R, 32>(A, Bm, P, P1, Tm, steps, cf); break;
  }

  // Q = P / (||U||_F + eps): the result applies to the stored, unnormalised U
  if (worker)
    for (int e = t; e < SK_MP * SK_MP; e += SK_THREADS) {
      const int i = e / SK_MP, j = e % SK_MP;
      Qf[i][j] = (i < m && j < m) ? (float)(inv * (double)P[i * GSD + j]) : 0.f;
    }
  __syncthreads();
}

template <int MODE>
__global__ void __launch_bounds__(SK_THREADS)
sk_gram_ns(const float* __restrict__ gp, const float* __restrict__ sp, float eps, int m, int S, int T, int steps,
           Coeffs cf, BFrag* __restrict__ bfrag) {
  __shared__ __attribute__((aligned(16))) unsigned char raw[GramLds<MODE>::RAW];
  __shared__ float Qf[SK_MP][SK_MP + 1];
  __shared__ double inv_s;
  const int64_t b = blockIdx.x;
  gram_q<MODE>(gp, sp, eps, m, S, T, steps, cf, b, raw, Qf, &inv_s);
  if (threadIdx.x < WAVE) write_frag<MODE, true>(Qf, bfrag + b * WAVE, threadIdx.x);
}

// ---------------------------------------------------------------------------
// First kernel: momentum + Nesterov direction (or a given U), ||U||^2 partial,
// U into the workspace, and the Gram partial of U.
//   mode 0: M' = mu M + G (in place), U = G + mu M' (or M' without Nesterov)
//   mode 1: U read from u_in
// vec: stored rows are X rows and n % 8 == 0 (16-byte vectors along rows).
// XG: U goes out as MFMA-ready tiles (Gram path), else row-major [m, ldx].
// ---------------------------------------------------------------------------
template <int MODE, typename GT, bool XG, bool ROWS>
__global__ void __launch_bounds__(SK_THREADS)
sk_first(int mode, const GT* __restrict__ grad, float* __restrict__ mom, const float* __restrict__ u_in,
         typename SkCfg<MODE>::XS* __restrict__ xws, float* __restrict__ gp_out, float* __restrict__ sp,
         int m, int64_t n, int64_t ldx, int S, int T, int transposed, int vec, float mu, int nesterov,
         int64_t NB, int G, MatTabs tabs) {
  typedef SkCfg<MODE> C;
  typedef typename C::XS XS;
  // dynamic LDS: max(mr rows of the tile, the Gram reduction buffer) bytes
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  __shared__ float wsum[SK_WAVES];
  XS* lx = reinterpret_cast<XS*>(lds_raw);
  const int mr = (m + 7) & ~7;

  const int64_t blk = blockIdx.x;
  const int64_t b = blk / S;
  const int c = (int)(blk % S);
  const int64_t j0 = (int64_t)c * C::L;
  const int64_t mat = b * (int64_t)m * n;
  grad = batch_view(grad, tabs.grad, b, (int64_t)m * n);
  mom = batch_view(mom, tabs.mom, b, (int64_t)m * n);
  float ss = 0.f;

  // zero the padding rows of the tile
  for (int e = threadIdx.x; e < (mr - m) * C::LDX; e += SK_THREADS) lx[m * C::LDX + e] = (XS)0;

  if (vec) {
    // 8 consecutive columns of one row per item
    constexpr int PR = C::L / 8;
    const int items = m * PR;
    // U of item v into the tile and the norm partial
    auto finish = [&](int v, const float* u) __attribute__((always_inline)) {
      const int r = v / PR, jl = (v % PR) * 8;
#pragma unroll
      for (int q = 0; q < 8; ++q) ss += u[q] * u[q];
      if constexpr (MODE == 0) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = (uint32_t)f2bf(u[2 * q]) | ((uint32_t)f2bf(u[2 * q + 1]) << 16);
        *reinterpret_cast<u32x4*>(lx + r * C::LDX + jl) = w;
      } else {
        *reinterpret_cast<f32x4*>(lx + r * C::LDX + jl) = f32x4{u[0], u[1], u[2], u[3]};
        *reinterpret_cast<f32x4*>(lx + r * C::LDX + jl + 4) = f32x4{u[4], u[5], u[6], u[7]};
      }
    };
    if (mode == 0) {
      // momentum: a thread's next item is loaded before the current item's
      // momentum is stored (the stores could alias the loads, so the compiler
      // would otherwise wait out one memory latency per item)
      Raw8<GT> gc, gn;
      f32x4 mc0 = {}, mc1 = {}, mn0 = {}, mn1 = {};
      auto load_item = [&](int v, Raw8<GT>& gr, f32x4& m0, f32x4& m1) __attribute__((always_inline)) {
        if (v >= items) return;
        const int r = v / PR, jl = (v % PR) * 8;
        const int64_t j = j0 + jl;
        if (j >= n) return;   // n % 8 == 0: the 8 columns are all in range or all out
        const int64_t si = mat + (int64_t)r * n + j;
        if constexpr (ROWS) gr.load(row_of<const GT>(tabs.grad_rows, b, m, r) + j);
        else gr.load(grad + si);
        m0 = *reinterpret_cast<const f32x4*>(mom + si);
        m1 = *reinterpret_cast<const f32x4*>(mom + si + 4);
      };
      load_item(threadIdx.x, gc, mc0, mc1);
      for (int v = threadIdx.x; v < items; v += SK_THREADS) {
        load_item(v + SK_THREADS, gn, mn0, mn1);
        const int r = v / PR, jl = (v % PR) * 8;
        const int64_t j = j0 + jl;
        float u[8];
        if (j < n) {
          const int64_t si = mat + (int64_t)r * n + j;
          float g[8];
          gc.to_f32(g);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float a0 = mu * mc0[q] + g[q];
            const float a1 = mu * mc1[q] + g[q + 4];
            mc0[q] = a0;
            mc1[q] = a1;
            u[q] = nesterov ? g[q] + mu * a0 : a0;
            u[q + 4] = nesterov ? g[q + 4] + mu * a1 : a1;
          }
          *reinterpret_cast<f32x4*>(mom + si) = mc0;
          *reinterpret_cast<f32x4*>(mom + si + 4) = mc1;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) u[q] = 0.f;
        }
        finish(v, u);
        gc = gn;
        mc0 = mn0;
        mc1 = mn1;
      }
    } else {
      for (int v = threadIdx.x; v < items; v += SK_THREADS) {
        const int r = v / PR, jl = (v % PR) * 8;
        const int64_t j = j0 + jl;
        float u[8];
        if (j < n) {
          const int64_t si = mat + (int64_t)r * n + j;
          const f32x4 u0 = *reinterpret_cast<const f32x4*>(u_in + si);
          const f32x4 u1 = *reinterpret_cast<const f32x4*>(u_in + si + 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) { u[q] = u0[q]; u[q + 4] = u1[q]; }
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) u[q] = 0.f;
        }
        finish(v, u);
      }
    }
  } else {
    // element by element, walking the stored layout of the chunk
    for (int e = threadIdx.x; e < m * C::L; e += SK_THREADS) {
      int r, jl;
      if (transposed) { jl = e / m; r = e % m; }
      else { r = e / C::L; jl = e % C::L; }
      const int64_t j = j0 + jl;
      float u = 0.f;
      if (j < n) {
        const int64_t si = mat + stored_index(transposed, r, j, m, n);
        if (mode == 0) {
          float g;
          if constexpr (ROWS)
            g = ld_as_f32(row_of<const GT>(tabs.grad_rows, b, transposed ? n : m, transposed ? j : r),
                          transposed ? r : j);
          else
            g = ld_as_f32(grad, si);
          const float mn = mu * mom[si] + g;
          mom[si] = mn;
          u = nesterov ? g + mu * mn : mn;
        } else {
          u = u_in[si];
        }
      }
      ss += u * u;
      if constexpr (MODE == 0) lx[r * C::LDX + jl] = f2bf(u);
      else lx[r * C::LDX + jl] = u;
    }
  }
  const float tot = block_sum(ss, wsum);   // includes a barrier: the tile is complete
  if (threadIdx.x == 0) sp[blk] = tot;
  if constexpr (XG) chunk_store_xg<MODE>(xws, lds_raw, b, j0 / 32, NB, G);
  else chunk_store<MODE>(xws + b * m * ldx + j0, lds_raw, m, ldx);
  gram_partial<MODE>(lds_raw, gp_out + blk * T, T, mr);
}

// ---------------------------------------------------------------------------
// One Newton-Schulz step on a chunk: X' = B' X.  LAST: apply the update (or
// write O) instead of storing X' and its Gram partial.
// ---------------------------------------------------------------------------
template <int MODE, typename PT, bool LAST, bool ROWS>
__global__ void __launch_bounds__(SK_THREADS)
sk_iter(typename SkCfg<MODE>::XS* __restrict__ xws, const BFrag* __restrict__ bfrag, float* __restrict__ gp_out,
        int m, int64_t n, int64_t ldx, int S, int T, int transposed, int vec,
        PT* __restrict__ param, float* __restrict__ ns_out, float lr, float wd, float s_scale,
        const float* __restrict__ lrwd, MatTabs tabs) {
  typedef SkCfg<MODE> C;
  if constexpr (LAST) update_scalars(lrwd, lr, wd);
  typedef typename C::XS XS;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[SkLds<MODE>::BYTES];
  XS* lx = reinterpret_cast<XS*>(lds_raw);

  const int64_t blk = blockIdx.x;
  const int64_t b = blk / S;
  const int c = (int)(blk % S);
  const int64_t j0 = (int64_t)c * C::L;
  const int t = threadIdx.x;
  const int64_t mat = b * (int64_t)m * n;
  if constexpr (LAST) {
    param = batch_view(param, tabs.param, b, (int64_t)m * n);
    ns_out = batch_view(ns_out, tabs.ns, b, (int64_t)m * n);
  }
  const bool has_w = ROWS || param != nullptr;
  // W's stored element (row sr, column sc), rows of ncols elements
  [[maybe_unused]] auto w_at = [&](int64_t sr, int64_t sc, int64_t ncols) -> PT* {
    if constexpr (ROWS) return row_of<PT>(tabs.param_rows, b, transposed ? n : m, sr) + sc;
    else return param + mat + sr * ncols + sc;
  };
  constexpr int PR8 = C::L / 8;                      // 8-column items per row
  constexpr int NI = SK_MP * PR8 / SK_THREADS;       // items per thread (upper bound)

  const BFrag fr = bfrag[b * WAVE + (t & (WAVE - 1))];

  // last step, bf16 W: start reading W now, it is needed only at the end
  uint4 wpre[LAST && sizeof(PT) == 2 ? NI : 1];
  if constexpr (LAST && sizeof(PT) == 2) {
    if (vec && has_w) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int v = t + SK_THREADS * i;
        const int r = v / PR8, jl = (v % PR8) * 8;
        if (r < m && j0 + jl < n) wpre[i] = *reinterpret_cast<const uint4*>(w_at(r, j0 + jl, n));
      }
    }
  }

  chunk_load<MODE>(xws + b * m * ldx + j0, lds_raw, m, ldx);
  __syncthreads();
  apply_bx<MODE>(lds_raw, fr);
  __syncthreads();

  if constexpr (!LAST) {
    chunk_store<MODE>(xws + b * m * ldx + j0, lds_raw, m, ldx);
    gram_partial<MODE>(lds_raw, gp_out + blk * T, T, SK_MP);
  } else {
    if (vec) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int v = t + SK_THREADS * i;
        const int r = v / PR8, jl = (v % PR8) * 8;
        const int64_t j = j0 + jl;
        if (r >= m || j >= n) continue;
        const int64_t si = mat + (int64_t)r * n + j;
        float o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if constexpr (MODE == 0) o[q] = bf2f(lx[r * C::LDX + jl + q]);
          else o[q] = lx[r * C::LDX + jl + q];
        }
        if (ns_out) {
          *reinterpret_cast<f32x4*>(ns_out + si) = f32x4{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<f32x4*>(ns_out + si + 4) = f32x4{o[4], o[5], o[6], o[7]};
        }
        if (has_w) {
          PT* wp = w_at(r, j, n);
          if constexpr (sizeof(PT) == 2) {
            const uint4 wv = wpre[i];
            uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float w0 = __uint_as_float(w4[q] << 16);
              const float w1 = __uint_as_float(w4[q] & 0xffff0000u);
              const uint32_t n0 = f2bf(apply_update(w0, o[2 * q], lr, wd, s_scale));
              const uint32_t n1 = f2bf(apply_update(w1, o[2 * q + 1], lr, wd, s_scale));
              w4[q] = n0 | (n1 << 16);
            }
            *reinterpret_cast<uint4*>(wp) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
          } else {
            f32x4 w0 = *reinterpret_cast<const f32x4*>(wp);
            f32x4 w1 = *reinterpret_cast<const f32x4*>(wp + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              w0[q] = apply_update(w0[q], o[q], lr, wd, s_scale);
              w1[q] = apply_update(w1[q], o[q + 4], lr, wd, s_scale);
            }
            *reinterpret_cast<f32x4*>(wp) = w0;
            *reinterpret_cast<f32x4*>(wp + 4) = w1;
          }
        }
      }
    } else {
      for (int e = t; e < m * C::L; e += SK_THREADS) {
        int r, jl;
        if (transposed) { jl = e / m; r = e % m; }
        else { r = e / C::L; jl = e % C::L; }
        const int64_t j = j0 + jl;
        if (j >= n) continue;
        float o;
        if constexpr (MODE == 0) o = bf2f(lx[r * C::LDX + jl]);
        else o = lx[r * C::LDX + jl];
        const int64_t si = mat + stored_index(transposed, r, j, m, n);
        if (ns_out) ns_out[si] = o;
        if (has_w) {
          PT* wp = transposed ? w_at(j, r, m) : w_at(r, j, n);
          st_from_f32(wp, 0, apply_update(ld_as_f32(wp, 0), o, lr, wd, s_scale));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Gram path, last kernel: O = Q U and the update, one wave per 64 columns (two
// 32-column blocks) of one matrix, no workgroup barriers.  The U operand comes
// straight from the tiles, Q from the fragments.
//   Row-major W (!TRANS): O^T = U^T Q^T (the same registers, operands
//   swapped); the accumulators go to a wave-private LDS buffer as 16-byte
//   quads (4 consecutive columns of one row), and W is read, updated and
//   written as 128-byte row segments, 16 bytes per lane.
//     vec: n % 8 == 0 (aligned 8-element runs inside the matrix).
//   Stored-transposed W (TRANS): O = Q U straight from the accumulators, 4
//   consecutive rows of one column per quad.
//     vec: m % 4 == 0 (aligned 4-element runs).
// ---------------------------------------------------------------------------
template <typename PT> struct Quad;
template <> struct Quad<bf16_t> {
  typedef uint2 V;
  static __device__ __forceinline__ float get(const V& v, int i) {
    const uint32_t w = i < 2 ? v.x : v.y;
    return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
  static __device__ __forceinline__ V make(const float* f) {
    return make_uint2((uint32_t)f2bf(f[0]) | ((uint32_t)f2bf(f[1]) << 16),
                      (uint32_t)f2bf(f[2]) | ((uint32_t)f2bf(f[3]) << 16));
  }
};
template <> struct Quad<float> {
  typedef f32x4 V;
  static __device__ __forceinline__ float get(const V& v, int i) { return v[i]; }
  static __device__ __forceinline__ V make(const float* f) { return f32x4{f[0], f[1], f[2], f[3]}; }
};

constexpr int AP_LD = 68;   // LDS row stride (floats) of a wave's 32 x 64 O block

// 8 consecutive elements of PT <-> floats.
template <typename PT> struct Oct;
template <> struct Oct<bf16_t> {
  typedef u32x4 V;
  static __device__ __forceinline__ float get(const V& v, int i) {
    const uint32_t w = v[i >> 1];
    return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
  static __device__ __forceinline__ void put(bf16_t* p, const float* f) {
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = (uint32_t)f2bf(f[2 * q]) | ((uint32_t)f2bf(f[2 * q + 1]) << 16);
    *reinterpret_cast<u32x4*>(p) = v;
  }
  // W is device memory: a global load (a pointer from a row table would
  // otherwise make it a flat load, which also holds the LDS counter that the
  // next barrier waits on)
  static __device__ __forceinline__ V load(const bf16_t* p) {
    return *(const __attribute__((address_space(1))) u32x4*)(p);
  }
};
template <> struct Oct<float> {
  struct V { f32x4 a, b; };
  static __device__ __forceinline__ float get(const V& v, int i) { return i < 4 ? v.a[i] : v.b[i - 4]; }
  static __device__ __forceinline__ void put(float* p, const float* f) {
    *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
  }
  static __device__ __forceinline__ V load(const float* p) {
    typedef const __attribute__((address_space(1))) f32x4* G;
    return V{*(G)(p), *(G)(p + 4)};
  }
};

// O block of one 32-column block: acc = U^T Q^T (!TRANS) or Q U (TRANS).
template <int MODE, bool TRANS>
__device__ __forceinline__ f32x16 apply_block(const uint32_t (*xr)[MODE == 0 ? 4 : 8], const BFrag& fr) {
  f32x16 acc = {};
  if constexpr (MODE == 2) {
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const uint4 qw = fr.q[kk >> 2];
      const uint32_t qb = (kk & 3) == 0 ? qw.x : (kk & 3) == 1 ? qw.y : (kk & 3) == 2 ? qw.z : qw.w;
      const float qv = __uint_as_float(qb);
      const float xv = __uint_as_float(xr[kk >> 3][kk & 7]);
      if constexpr (!TRANS) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xv, qv, acc, 0, 0, 0);
      else acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv, xv, acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 qh = __builtin_bit_cast(bf16x8, fr.q[kb]);
      const bf16x8 ql = __builtin_bit_cast(bf16x8, fr.q[2 + kb]);
      if constexpr (MODE == 0) {
        const bf16x8 xv = __builtin_bit_cast(bf16x8, u32x4{xr[kb][0], xr[kb][1], xr[kb][2], xr[kb][3]});
        if constexpr (!TRANS) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xv, qh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xv, ql, acc, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh, xv, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ql, xv, acc, 0, 0, 0);
        }
      } else {
        bf16x8 xh, xl;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float v = __uint_as_float(xr[kb][t]);
          const bf16_t hb = f2bf(v);
          xh[t] = __builtin_bit_cast(__bf16, hb);
          xl[t] = __builtin_bit_cast(__bf16, f2bf(v - bf2f(hb)));
        }
        if constexpr (!TRANS) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, qh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, qh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, ql, acc, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh, xh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh, xl, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ql, xh, acc, 0, 0, 0);
        }
      }
    }
  }
  return acc;
}

template <int MODE, typename PT, bool TRANS, bool ROWS>
__global__ void __launch_bounds__(SK_THREADS)
sk_apply(const typename SkCfg<MODE>::XS* __restrict__ xg, const BFrag* __restrict__ qfrag, int m, int64_t n,
         int64_t NB, int G, int64_t upm, int64_t units, int vec, PT* __restrict__ param, float* __restrict__ ns_out,
         float lr, float wd, float s_scale, const float* __restrict__ lrwd, MatTabs tabs) {
  update_scalars(lrwd, lr, wd);
  typedef typename SkCfg<MODE>::XS XS;
  constexpr int XW = MODE == 0 ? 4 : 8;     // 32-bit words of U per lane per K block
  const int lane = threadIdx.x & (WAVE - 1);
  // wave index as a scalar: the matrix index and the pointers taken from the
  // tables stay in scalar registers and the null tests stay uniform branches
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int h = lane >> 5, c = lane & 31;
  const int64_t unit = (int64_t)blockIdx.x * SK_WAVES + w;
  if (unit >= units) return;   // whole waves only; the kernel has no workgroup barriers
  const int64_t b = unit / upm;
  const int64_t jb0 = (unit % upm) * 2;
  const int64_t mat = b * (int64_t)m * n;
  param = batch_view(param, tabs.param, b, (int64_t)m * n);
  ns_out = batch_view(ns_out, tabs.ns, b, (int64_t)m * n);
  const bool has_w = ROWS || param != nullptr;
  // W's stored element (row sr, column sc): stored rows are U rows (n long),
  // or U columns (m long) when W is tall
  auto w_at = [&](int64_t sr, int64_t sc) -> PT* {
    if constexpr (ROWS) return row_of<PT>(tabs.param_rows, b, TRANS ? n : m, sr) + sc;
    else return param + mat + sr * (TRANS ? (int64_t)m : n) + sc;
  };

  // U operands of both blocks: bf16 modes K block kb = rows of group 2 kb + h,
  // fp32 mode rows 16 h .. 16 h + 15 (groups 2 h, 2 h + 1)
  uint32_t xr[2][2][XW];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int64_t jb = jb0 + jj;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int g = MODE == 2 ? 2 * h + kb : 2 * kb + h;
      if (jb < NB && g < G) {
        const XS* src = xg + xg_tile(b, jb, g, NB, G) + c * 8;
        const u32x4 v0 = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int q = 0; q < 4; ++q) xr[jj][kb][q] = v0[q];
        if constexpr (XW == 8) {
          const u32x4 v1 = *reinterpret_cast<const u32x4*>(src + 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) xr[jj][kb][4 + q] = v1[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < XW; ++q) xr[jj][kb][q] = 0u;
      }
    }
  }

  if constexpr (!TRANS) {
    // dynamic LDS: SK_WAVES x mr x AP_LD floats, one O buffer per wave
    extern __shared__ __attribute__((aligned(16))) float ob_raw[];
    const int mr = 8 * G;
    typedef Oct<PT> OV;
    // W rows 8 i + lane / 8, columns 64 jb0 / 2 + 8 (lane % 8) .. + 7
    const int rr = lane >> 3, cc = (lane & 7) * 8;
    const int64_t col0 = 32 * jb0 + cc;
    typename OV::V wv[4];
    if (has_w && vec) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * i + rr;
        if (i < G && row < m && col0 < n) wv[i] = OV::load(w_at(row, col0));
      }
    }
    const BFrag fr = qfrag[b * WAVE + lane];
    float* o = ob_raw + w * mr * AP_LD;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const f32x16 acc = apply_block<MODE, false>(xr[jj], fr);
      // lane holds O row c, columns 32 jj + 8 qd + 4 h + 0..3
      if (c < mr) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<f32x4*>(o + c * AP_LD + 32 * jj + 8 * qd + 4 * h) =
              f32x4{acc[4 * qd], acc[4 * qd + 1], acc[4 * qd + 2], acc[4 * qd + 3]};
      }
    }
    wave_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * i + rr;
      if (i >= G || row >= m) continue;
      float ov[8], nw[8];
      const f32x4 o0 = *reinterpret_cast<const f32x4*>(o + row * AP_LD + cc);
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(o + row * AP_LD + cc + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) { ov[q] = o0[q]; ov[q + 4] = o1[q]; }
      if (vec) {
        if (col0 >= n) continue;
        const int64_t idx = mat + (int64_t)row * n + col0;
        if (ns_out) Oct<float>::put(ns_out + idx, ov);
        if (has_w) {
#pragma unroll
          for (int q = 0; q < 8; ++q) nw[q] = apply_update(OV::get(wv[i], q), ov[q], lr, wd, s_scale);
          OV::put(w_at(row, col0), nw);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (col0 + q >= n) break;
          const int64_t idx = mat + (int64_t)row * n + col0 + q;
          if (ns_out) ns_out[idx] = ov[q];
          if (has_w) {
            PT* wp = w_at(row, col0 + q);
            st_from_f32(wp, 0, apply_update(ld_as_f32(wp, 0), ov[q], lr, wd, s_scale));
          }
        }
      }
    }
  } else {
    typedef Quad<PT> QV;
    // W at the accumulator positions: quad qd of block jj holds rows
    // 8 qd + 4 h + 0..3 of column 32 jb + c
    typename QV::V wq[2][4];
    if (has_w && vec) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int64_t col = 32 * (jb0 + jj) + c;
          const int d = 8 * qd + 4 * h;
          if (col < n && d < m) wq[jj][qd] = *reinterpret_cast<const typename QV::V*>(w_at(col, d));
        }
    }
    const BFrag fr = qfrag[b * WAVE + lane];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int64_t col = 32 * (jb0 + jj) + c;
      if (jb0 + jj >= NB) break;
      const f32x16 acc = apply_block<MODE, true>(xr[jj], fr);
      if (col >= n) continue;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d = 8 * qd + 4 * h;
        float ov[4], nw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = acc[4 * qd + i];
        if (vec) {
          if (d >= m) continue;
          const int64_t idx = mat + col * m + d;
          if (ns_out) *reinterpret_cast<f32x4*>(ns_out + idx) = f32x4{ov[0], ov[1], ov[2], ov[3]};
          if (has_w) {
#pragma unroll
            for (int i = 0; i < 4; ++i) nw[i] = apply_update(QV::get(wq[jj][qd], i), ov[i], lr, wd, s_scale);
            *reinterpret_cast<typename QV::V*>(w_at(col, d)) = QV::make(nw);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (d + i >= m) break;
            const int64_t idx = mat + col * m + d + i;
            if (ns_out) ns_out[idx] = ov[i];
            if (has_w) {
              PT* wp = w_at(col, d + i);
              st_from_f32(wp, 0, apply_update(ld_as_f32(wp, 0), ov[i], lr, wd, s_scale));
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Gram-space Newton-Schulz and the apply in one launch.  R workgroups of NW
// waves per matrix, one per CU: the first four waves of each form Q from the
// chunk partials exactly as sk_gram_ns does (the R copies are bitwise equal;
// one workgroup per CU keeps their dependent MFMA chains from sharing a SIMD
// with another copy's), then every wave applies it to its share of the
// matrix's 64-column units exactly as sk_apply does, in both orientations of
// W: wave w of workgroup r takes units r * NW + w + i * R * NW, so the R
// workgroups sweep the matrix front to back together.  The waves that do not
// form Q load their first unit (U and a wide W) once the partials are summed,
// while the iteration runs (loaded before the partials, they delayed the
// partials Q needs first).  For a
// row-major W the O buffers alias gram_q's LDS, which is free once Q is in Qf.
// All waves take part in gram_q's barriers; after it there are none.
//   NW = 16: bf16 operands (the 16-wave register budget, 128 per lane, holds
//            them), batches too large for R >= 8 workgroups per matrix;
//   NW = 8:  fp32 operands (bf16_x32 and the check path need the 256-register
//            budget of two waves per SIMD), and small batches, whose R already
//            fills the CUs: fewer waves per workgroup wait at fewer barriers.
// ---------------------------------------------------------------------------
template <int MODE, typename PT, bool ROWS, int NW, bool TRANS>
__global__ void __launch_bounds__(NW * WAVE)
sk_ns_apply(const float* __restrict__ gp, const float* __restrict__ sp, float eps, int S, int T, int steps, Coeffs cf,
            const typename SkCfg<MODE>::XS* __restrict__ xg, int m, int64_t n, int64_t NB, int G, int64_t upm, int R,
            int vec, PT* __restrict__ param, float* __restrict__ ns_out, float lr, float wd, float s_scale,
            const float* __restrict__ lrwd, MatTabs tabs) {
  typedef typename SkCfg<MODE>::XS XS;
  constexpr int XW = MODE == 0 ? 4 : 8;     // 32-bit words of U per lane per K block
  constexpr int OBUF = TRANS ? 0 : NW * SK_MP * AP_LD * 4;
  constexpr int RAW = GramLds<MODE>::RAW > OBUF ? GramLds<MODE>::RAW : OBUF;
  __shared__ __attribute__((aligned(16))) unsigned char raw[RAW];
  __shared__ float Qf[SK_MP][SK_MP + 1];
  __shared__ double inv_s;

  update_scalars(lrwd, lr, wd);
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int h = lane >> 5, c = lane & 31;
  const int64_t b = blockIdx.x / R;
  const int64_t r = blockIdx.x % R;
  const int64_t stride = (int64_t)R * NW;
  const int64_t mat = b * (int64_t)m * n;
  param = batch_view(param, tabs.param, b, (int64_t)m * n);
  ns_out = batch_view(ns_out, tabs.ns, b, (int64_t)m * n);
  const bool has_w = ROWS || param != nullptr;
  // W's stored element (row sr, column sc): stored rows are U rows (n long),
  // or U columns (m long) when W is tall
  auto w_at = [&](int64_t sr, int64_t sc) -> PT* {
    if constexpr (ROWS) return row_of<PT>(tabs.param_rows, b, TRANS ? n : m, sr) + sc;
    else return param + mat + sr * (TRANS ? (int64_t)m : n) + sc;
  };

  // U operands of both 32-column blocks of unit u (bf16 modes: K block kb =
  // rows of group 2 kb + h; fp32 mode: rows 16 h .. 16 h + 15)
  auto load_u = [&](int64_t u, uint32_t (&xd)[2][2][XW]) __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int64_t jb = 2 * u + jj;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int g = MODE == 2 ? 2 * h + kb : 2 * kb + h;
        if (jb < NB && g < G) {
          const XS* src = xg + xg_tile(b, jb, g, NB, G) + c * 8;
          const u32x4 v0 = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
          for (int q = 0; q < 4; ++q) xd[jj][kb][q] = v0[q];
          if constexpr (XW == 8) {
            const u32x4 v1 = *reinterpret_cast<const u32x4*>(src + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) xd[jj][kb][4 + q] = v1[q];
          }
        } else {
#pragma unroll
          for (int q = 0; q < XW; ++q) xd[jj][kb][q] = 0u;
        }
      }
    }
  };

  uint32_t xr[2][2][XW];
  if constexpr (!TRANS) {
    typedef Oct<PT> OV;
    // W rows 8 i + lane / 8, columns 64 u + 8 (lane % 8) .. + 7 of unit u
    const int rr = lane >> 3, cc = (lane & 7) * 8;
    const int mr = 8 * G;
    typename OV::V wv[4];
    auto load_w = [&](int64_t u) __attribute__((always_inline)) {
      const int64_t col0 = 64 * u + cc;
      if (has_w && vec) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 8 * i + rr;
          if (i < G && row < m && col0 < n) wv[i] = OV::load(w_at(row, col0));
        }
      }
    };
    // The waves that do not form Q load their first unit (U and W) while the
    // first four run the Newton-Schulz iteration, once the partials are in.
    const int64_t u0 = r * NW + w;
    const bool pre = w * WAVE >= SK_THREADS && u0 < upm;
    gram_q<MODE, NW * WAVE>(gp, sp, eps, m, S, T, steps, cf, b, raw, Qf, &inv_s, [&]() {
      if (pre) {
        load_u(u0, xr);
        load_w(u0);
      }
    });
    const BFrag fr = make_frag<MODE, true>(Qf, lane);
    float* o = reinterpret_cast<float*>(raw) + w * mr * AP_LD;
    for (int64_t u = u0; u < upm; u += stride) {
      if (!pre || u != u0) {
        load_u(u, xr);
        load_w(u);
      }
      const int64_t col0 = 64 * u + cc;
      wave_sync();   // this wave's reads of the previous unit's O are done
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const f32x16 acc = apply_block<MODE, false>(xr[jj], fr);
        // lane holds O row c, columns 32 jj + 8 qd + 4 h + 0..3
        if (c < mr) {
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            *reinterpret_cast<f32x4*>(o + c * AP_LD + 32 * jj + 8 * qd + 4 * h) =
                f32x4{acc[4 * qd], acc[4 * qd + 1], acc[4 * qd + 2], acc[4 * qd + 3]};
        }
      }
      wave_sync();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * i + rr;
        if (i >= G || row >= m) continue;
        float ov[8], nw[8];
        const f32x4 o0 = *reinterpret_cast<const f32x4*>(o + row * AP_LD + cc);
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(o + row * AP_LD + cc + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) { ov[q] = o0[q]; ov[q + 4] = o1[q]; }
        if (vec) {
          if (col0 >= n) continue;
          const int64_t idx = mat + (int64_t)row * n + col0;
          if (ns_out) Oct<float>::put(ns_out + idx, ov);
          if (has_w) {
#pragma unroll
            for (int q = 0; q < 8; ++q) nw[q] = apply_update(OV::get(wv[i], q), ov[q], lr, wd, s_scale);
            OV::put(w_at(row, col0), nw);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (col0 + q >= n) break;
            const int64_t idx = mat + (int64_t)row * n + col0 + q;
            if (ns_out) ns_out[idx] = ov[q];
            if (has_w) {
              PT* wp = w_at(row, col0 + q);
              st_from_f32(wp, 0, apply_update(ld_as_f32(wp, 0), ov[q], lr, wd, s_scale));
            }
          }
        }
      }
    }
  } else {
    gram_q<MODE, NW * WAVE>(gp, sp, eps, m, S, T, steps, cf, b, raw, Qf, &inv_s);
    const BFrag fr = make_frag<MODE, true>(Qf, lane);
    // stored-transposed W: O = Q U straight from the accumulators; quad qd of
    // block jj holds rows 8 qd + 4 h + 0..3 of column 32 jb + c (as sk_apply)
    typedef Quad<PT> QV;
    typename QV::V wq[2][4];
    for (int64_t u = r * NW + w; u < upm; u += stride) {
      const int64_t jb0 = 2 * u;
      load_u(u, xr);
      if (has_w && vec) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int64_t col = 32 * (jb0 + jj) + c;
            const int d = 8 * qd + 4 * h;
            if (col < n && d < m) wq[jj][qd] = *reinterpret_cast<const typename QV::V*>(w_at(col, d));
          }
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int64_t col = 32 * (jb0 + jj) + c;
        if (jb0 + jj >= NB) break;
        const f32x16 acc = apply_block<MODE, true>(xr[jj], fr);
        if (col >= n) continue;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int d = 8 * qd + 4 * h;
          float ov[4], nw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = acc[4 * qd + i];
          if (vec) {
            if (d >= m) continue;
            const int64_t idx = mat + col * m + d;
            if (ns_out) *reinterpret_cast<f32x4*>(ns_out + idx) = f32x4{ov[0], ov[1], ov[2], ov[3]};
            if (has_w) {
#pragma unroll
              for (int i = 0; i < 4; ++i) nw[i] = apply_update(QV::get(wq[jj][qd], i), ov[i], lr, wd, s_scale);
              *reinterpret_cast<typename QV::V*>(w_at(col, d)) = QV::make(nw);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (d + i >= m) break;
              const int64_t idx = mat + col * m + d + i;
              if (ns_out) ns_out[idx] = ov[i];
              if (has_w) {
                PT* wp = w_at(col, d + i);
                st_from_f32(wp, 0, apply_update(ld_as_f32(wp, 0), ov[i], lr, wd, s_scale));
              }
            }
          }
        }
      }
    }
  }
}

template <int MODE, typename GT>
hipError_t launch_first(const StepArgs& a, const WsLayout& L, int mode, int vec) {
  typedef typename SkCfg<MODE>::XS XS;
  const BatchShape& sh = a.shape;
  dim3 grid((unsigned)(sh.count * L.S)), block(SK_THREADS);
  const char* name = mode == 0 ? "sk_momentum_norm_gram" : "sk_norm_gram";
  const int64_t NB = (sh.n + 31) / 32;
  const int G = (int)((sh.m + 7) / 8);
  const size_t tile = (size_t)(8 * G) * SkCfg<MODE>::LDX * sizeof(XS);
  const size_t red = (size_t)SK_WAVES * SK_MP * (SK_MP + 1) * 4;
  const size_t shm = tile > red ? tile : red;
  // XG: U as MFMA tiles (Gram path); ROWS: the gradient comes through a row table
  auto go = [&](auto xg, auto rows) {
    MUON_LAUNCH_SHM(name, (sk_first<MODE, GT, decltype(xg)::value, decltype(rows)::value>), grid, block, shm,
                    a.stream, mode, (const GT*)a.grad, a.mom, a.u_in, (XS*)(a.ws + L.x), (float*)(a.ws + L.gp0),
                    (float*)(a.ws + L.sp), (int)sh.m, sh.n, L.ldx, (int)L.S, (int)L.T, (int)sh.transposed, vec, a.mu,
                    a.nesterov, NB, G, a.tabs);
  };
  const bool rows = a.tabs.grad_rows != nullptr;
  if (L.path == PATH_SKINNY_GRAM || L.path == PATH_SKINNY_FUSED) {
    if (rows) go(std::true_type{}, std::true_type{});
    else go(std::true_type{}, std::false_type{});
  } else {
    if (rows) go(std::false_type{}, std::true_type{});
    else go(std::false_type{}, std::false_type{});
  }
  return hipGetLastError();
}

template <int MODE, typename PT>
hipError_t launch_iters(const StepArgs& a, const WsLayout& L, int vec) {
  typedef typename SkCfg<MODE>::XS XS;
  const BatchShape& sh = a.shape;
  dim3 grid((unsigned)(sh.count * L.S)), block(SK_THREADS);
  float* gp[2] = {(float*)(a.ws + L.gp0), (float*)(a.ws + L.gp1)};
  BFrag* bfrag = (BFrag*)(a.ws + L.bfrag);
  PT* param = a.phase == PH_FULL ? (PT*)a.param : nullptr;
  for (int k = 0; k < a.steps; ++k) {
    const float ca = a.coeffs[3 * k], cb = a.coeffs[3 * k + 1], cc = a.coeffs[3 * k + 2];
    // step k reads the Gram partials in gp[k & 1] and writes its own into gp[(k + 1) & 1]
    MUON_LAUNCH("sk_bprime", (sk_bprime<MODE>), dim3((unsigned)sh.count), block, a.stream, gp[k & 1],
                (const float*)(a.ws + L.sp), (int)(k == 0), a.eps, (int)sh.m, (int)L.S, (int)L.T, ca, cb, cc,
                bfrag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (k < a.steps - 1)
      MUON_LAUNCH("sk_ns_step", (sk_iter<MODE, PT, false, false>), grid, block, a.stream, (XS*)(a.ws + L.x),
                  (const BFrag*)bfrag, gp[(k + 1) & 1], (int)sh.m, sh.n, L.ldx, (int)L.S, (int)L.T,
                  (int)sh.transposed, vec, param, a.ns_out, a.lr, a.wd, a.s, a.lrwd, a.tabs);
    else if (a.tabs.param_rows)
      MUON_LAUNCH("sk_apply_update", (sk_iter<MODE, PT, true, true>), grid, block, a.stream, (XS*)(a.ws + L.x),
                  (const BFrag*)bfrag, gp[(k + 1) & 1], (int)sh.m, sh.n, L.ldx, (int)L.S, (int)L.T,
                  (int)sh.transposed, vec, param, a.ns_out, a.lr, a.wd, a.s, a.lrwd, a.tabs);
    else
      MUON_LAUNCH("sk_apply_update", (sk_iter<MODE, PT, true, false>), grid, block, a.stream, (XS*)(a.ws + L.x),
                  (const BFrag*)bfrag, gp[(k + 1) & 1], (int)sh.m, sh.n, L.ldx, (int)L.S, (int)L.T,
                  (int)sh.transposed, vec, param, a.ns_out, a.lr, a.wd, a.s, a.lrwd, a.tabs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Workgroups per matrix of sk_ns_apply: one per CU over the whole batch (a
// second resident workgroup would run its copy of the Gram iteration on the
// same SIMDs), but no more than give every wave a unit.
template <int MODE, typename PT, bool ROWS, int NW, bool TRANS>
int64_t fused_groups(int64_t count, int64_t upm) {
  static std::atomic<int> per_dev[kMaxDevices];   // CUs of the device
  const int slots = per_device_cached(per_dev, [](int dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    return cus;
  });
  int64_t R = slots / count;
  const int64_t most = (upm + NW - 1) / NW;
  if (R > most) R = most;
  return R < 1 ? 1 : R;
}

// Waves per workgroup of sk_ns_apply: 8 for fp32 operands, and for batches of
// at most 32 matrices (R >= 8 workgroups per matrix fill the CUs);
// 16 otherwise.
inline int fused_waves(int mode, int64_t count) { return (mode != 0 || count <= 32) ? 8 : 16; }

template <int MODE, typename PT>
hipError_t launch_fused(const StepArgs& a, const WsLayout& L, const Coeffs& cf) {
  typedef typename SkCfg<MODE>::XS XS;
  const BatchShape& sh = a.shape;
  PT* param = a.phase == PH_FULL ? (PT*)a.param : nullptr;
  const int64_t NB = (sh.n + 31) / 32;
  const int G = (int)((sh.m + 7) / 8);
  const int64_t upm = (NB + 1) / 2;                    // 64-column units per matrix
  const char* name = (param || a.tabs.param || a.tabs.param_rows) ? "sk_ns_apply_update" : "sk_ns_apply";
  // ROWS: W through a row table; NW waves per workgroup; TRANS: W stored as U^T
  auto go = [&](auto rows, auto nw, auto trans) {
    constexpr bool RW = decltype(rows)::value;
    constexpr int NW = decltype(nw)::value;
    constexpr bool TR = decltype(trans)::value;
    const int vec = TR ? (sh.m % 4 == 0 ? 1 : 0) : (sh.n % 8 == 0 ? 1 : 0);
    const int64_t R = fused_groups<MODE, PT, RW, NW, TR>(sh.count, upm);
    if (sh.count * R > 0x7fffffffll) return hipErrorInvalidValue;
    MUON_LAUNCH(name, (sk_ns_apply<MODE, PT, RW, NW, TR>), dim3((unsigned)(sh.count * R)), dim3(NW * WAVE), a.stream,
                (const float*)(a.ws + L.gp0), (const float*)(a.ws + L.sp), a.eps, (int)L.S, (int)L.T, a.steps, cf,
                (const XS*)(a.ws + L.x), (int)sh.m, sh.n, NB, G, upm, (int)R, vec, param, a.ns_out, a.lr, a.wd,
                a.s, a.lrwd, a.tabs);
    return hipGetLastError();
  };
  auto by_trans = [&](auto rows, auto nw) {
    return sh.transposed ? go(rows, nw, std::true_type{}) : go(rows, nw, std::false_type{});
  };
  auto by_waves = [&](auto rows) {
    if constexpr (MODE == 0)
      if (fused_waves(MODE, sh.count) == 16) return by_trans(rows, std::integral_constant<int, 16>{});
    return by_trans(rows, std::integral_constant<int, 8>{});
  };
  return a.tabs.param_rows ? by_waves(std::true_type{}) : by_waves(std::false_type{});
}

template <int MODE, typename PT>
hipError_t launch_gram(const StepArgs& a, const WsLayout& L, int vec) {
  typedef typename SkCfg<MODE>::XS XS;
  const BatchShape& sh = a.shape;
  if (a.steps < 0 || a.steps > 64 || (int)a.coeffs.size() < 3 * a.steps) return hipErrorInvalidValue;
  Coeffs cf = {};
  for (int i = 0; i < 3 * a.steps; ++i) cf.c[i] = a.coeffs[i];
  if (L.path == PATH_SKINNY_FUSED) return launch_fused<MODE, PT>(a, L, cf);
  BFrag* bfrag = (BFrag*)(a.ws + L.bfrag);
  MUON_LAUNCH("sk_gram_ns", (sk_gram_ns<MODE>), dim3((unsigned)sh.count), dim3(SK_THREADS), a.stream,
              (const float*)(a.ws + L.gp0), (const float*)(a.ws + L.sp), a.eps, (int)sh.m, (int)L.S, (int)L.T,
              a.steps, cf, bfrag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PT* param = a.phase == PH_FULL ? (PT*)a.param : nullptr;
  const int64_t NB = (sh.n + 31) / 32;
  const int G = (int)((sh.m + 7) / 8);
  const int64_t upm = (NB + 1) / 2;                    // 64-column units per matrix
  const int64_t units = sh.count * upm;
  const dim3 grid((unsigned)((units + SK_WAVES - 1) / SK_WAVES));
  const char* name = (param || a.tabs.param || a.tabs.param_rows) ? "sk_apply_update" : "sk_apply";
  // ROWS: W comes through a row table
  auto go = [&](auto trans, auto rows) {
    constexpr bool TR = decltype(trans)::value;
    const int vec = TR ? (sh.m % 4 == 0 ? 1 : 0) : (sh.n % 8 == 0 ? 1 : 0);
    const size_t shm = TR ? 0 : (size_t)SK_WAVES * (8 * G) * AP_LD * 4;
    MUON_LAUNCH_SHM(name, (sk_apply<MODE, PT, TR, decltype(rows)::value>), grid, dim3(SK_THREADS), shm, a.stream,
                    (const XS*)(a.ws + L.x), (const BFrag*)bfrag, (int)sh.m, sh.n, NB, G, upm, units, vec, param,
                    a.ns_out, a.lr, a.wd, a.s, a.lrwd, a.tabs);
  };
  const bool rows = a.tabs.param_rows != nullptr;
  if (!sh.transposed) {
    if (rows) go(std::false_type{}, std::true_type{});
    else go(std::false_type{}, std::false_type{});
  } else {
    if (rows) go(std::true_type{}, std::true_type{});
    else go(std::true_type{}, std::false_type{});
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t run_mode(const StepArgs& a, const WsLayout& L) {
  // the workspace carve-up and the kernels must agree on the chunk width
  if (L.S * SkCfg<MODE>::L != L.ldx || L.ldx < a.shape.n) return hipErrorInvalidValue;
  if (L.T != a.shape.m * (a.shape.m + 1) / 2 || a.shape.m > SK_MP) return hipErrorInvalidValue;
  const int mode = a.phase == PH_FULL ? 0 : 1;
  // 16-byte vectors along stored rows need rows = X rows and 8 | n
  const int vec = (!a.shape.transposed && a.shape.n % 8 == 0) ? 1 : 0;
  hipError_t e = a.grad_dtype == DT_BF16 ? launch_first<MODE, bf16_t>(a, L, mode, vec)
                                         : launch_first<MODE, float>(a, L, mode, vec);
  if (e != hipSuccess) return e;
  const bool pbf = (a.phase == PH_FULL && a.param_dtype == DT_BF16);
  if (L.path == PATH_SKINNY_GRAM || L.path == PATH_SKINNY_FUSED)
    return pbf ? launch_gram<MODE, bf16_t>(a, L, vec) : launch_gram<MODE, float>(a, L, vec);
  return pbf ? launch_iters<MODE, bf16_t>(a, L, vec) : launch_iters<MODE, float>(a, L, vec);
}

}  // namespace

hipError_t run_skinny(const StepArgs& a, const WsLayout& L) {
  switch (a.prec) {
    case PREC_BF16: return run_mode<0>(a, L);
    case PREC_BF16_X32: return run_mode<1>(a, L);
    default: return run_mode<2>(a, L);
  }
}

}  // namespace muon
