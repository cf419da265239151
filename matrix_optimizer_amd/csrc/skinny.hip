// Skinny path of the Muon step: matrices whose short side m is at most 32
// (e.g. the 74 fused [24, 10240] parameters of the HyperParallel RFC, item 3).
//
// The m x m Gram matrix is tiny and the long side n is long, so the work is
// memory-bound.  Each workgroup owns a chunk of L columns of X (m x n in the
// Newton-Schulz orientation) and one Newton-Schulz step is one kernel:
//
//   1. sum the split-K Gram partials of the previous step in a fixed order
//      -> A = X X^T (fp32, m x m), identical in every workgroup of a matrix;
//   2. B = b A + c A A in fp32 (the polynomial of HyperParallel-FSDP Eq. (1));
//   3. X' = a X + B X on the chunk, fp32 arithmetic, written back in place;
//   4. the chunk's Gram partial X'_c X'_c^T on MFMA (bf16 operands, or fp32
//      operands on the check path) for the next step; the last step instead
//      applies decay and update to W.
//
// The first kernel fuses momentum, the Nesterov direction, the Frobenius-norm
// partials and the Gram partial of U, so a whole K-step update is K+1 launches
// and X never leaves the L2 / Infinity Cache between steps.  All reductions
// are fixed-order: results are bitwise reproducible run to run.
#include "common.h"
#include "internal.h"

namespace muon {
namespace {

constexpr int SK_THREADS = 256;
constexpr int SK_WAVES = SK_THREADS / WAVE;
constexpr int SK_MP = 32;  // rows padded to one 32x32 MFMA block

template <bool F32OP> struct SkCfg;
template <> struct SkCfg<false> {  // bf16 Gram operands
  static constexpr int L = 1024, CPT = L / SK_THREADS, LDX = L + 8;
  typedef bf16_t Op;
};
template <> struct SkCfg<true> {   // fp32 Gram operands (check path)
  static constexpr int L = 512, CPT = L / SK_THREADS, LDX = L + 4;
  typedef float Op;
};

constexpr int kLdsXBytes = SK_MP * (1024 + 8) * 2;  // == SK_MP * (512 + 4) * 4
static_assert(kLdsXBytes == SK_MP * (512 + 4) * 4, "LDS staging sizes differ");
static_assert(SK_WAVES * SK_MP * (SK_MP + 1) * 4 <= kLdsXBytes, "reduction buffer must fit");

__device__ __forceinline__ void tri_rc(int idx, int& r, int& s) {
  int rr = (int)((sqrtf(8.0f * idx + 1.0f) - 1.0f) * 0.5f);
  while (rr * (rr + 1) / 2 > idx) --rr;
  while ((rr + 1) * (rr + 2) / 2 <= idx) ++rr;
  r = rr;
  s = idx - rr * (rr + 1) / 2;
}

// Gram partial of the staged chunk: out[idx(r,s)] = sum_k X[r][k] X[s][k] over
// the L staged columns, lower triangle packed (idx = r(r+1)/2 + s).  Wave w
// takes columns [w L/4, (w+1) L/4); the four wave sums are added in order.
template <bool F32OP>
__device__ void gram_partial(unsigned char* lds_raw, float* __restrict__ out, int T) {
  typedef SkCfg<F32OP> C;
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = threadIdx.x / WAVE;
  f32x16 acc = {};
  if constexpr (!F32OP) {
    const bf16_t* lx = reinterpret_cast<const bf16_t*>(lds_raw);
    const int row = lane & 31;
    const int koff = (lane >> 5) * 8;
#pragma unroll 4
    for (int k0 = w * (C::L / SK_WAVES); k0 < (w + 1) * (C::L / SK_WAVES); k0 += 16) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(lx + row * C::LDX + k0 + koff);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, v, acc, 0, 0, 0);
    }
  } else {
    const float* lx = reinterpret_cast<const float*>(lds_raw);
    const int row = lane & 31;
    const int koff = lane >> 5;
#pragma unroll 8
    for (int k0 = w * (C::L / SK_WAVES); k0 < (w + 1) * (C::L / SK_WAVES); k0 += 2) {
      float v = lx[row * C::LDX + k0 + koff];
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

// Element (row r, column j) of a stored [M,N] matrix seen in the Newton-Schulz
// orientation (m x n): row-major if not transposed, else the transpose.
__device__ __forceinline__ int64_t stored_index(bool transposed, int r, int64_t j, int m, int64_t n) {
  return transposed ? j * m + r : (int64_t)r * n + j;
}

// ---------------------------------------------------------------------------
// First kernel: momentum + Nesterov direction (or a given U), ||U||^2 partial,
// U into the workspace, and the Gram partial of U.
//   mode 0: M' = mu M + G (in place), U = G + mu M' (or M' without Nesterov)
//   mode 1: U read from u_in
// ---------------------------------------------------------------------------
template <bool F32OP, typename XS, typename GT>
__global__ void __launch_bounds__(SK_THREADS)
sk_first(int mode, const GT* __restrict__ grad, float* __restrict__ mom, const float* __restrict__ u_in,
         XS* __restrict__ xws, float* __restrict__ gp_out, float* __restrict__ sp,
         int m, int64_t n, int64_t ldx, int S, int T, int transposed, float mu, int nesterov) {
  typedef SkCfg<F32OP> C;
  typedef typename C::Op Op;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[kLdsXBytes];
  __shared__ float wsum[SK_WAVES];
  Op* lx = reinterpret_cast<Op*>(lds_raw);

  const int64_t blk = blockIdx.x;
  const int64_t b = blk / S;
  const int c = (int)(blk % S);
  const int t = threadIdx.x;
  const int64_t mat = b * (int64_t)m * n;
  float ss = 0.f;

  for (int r = 0; r < SK_MP; ++r) {
#pragma unroll
    for (int q = 0; q < C::CPT; ++q) {
      const int jl = t * C::CPT + q;
      const int64_t j = (int64_t)c * C::L + jl;
      float u = 0.f;
      if (r < m && j < n) {
        const int64_t si = mat + stored_index(transposed, r, j, m, n);
        if (mode == 0) {
          const float g = ld_as_f32(grad, si);
          const float mn = mu * mom[si] + g;
          mom[si] = mn;
          u = nesterov ? g + mu * mn : mn;
        } else {
          u = u_in[si];
        }
      }
      float us = 0.f;
      if (r < m) {
        us = round_to<XS>(u);
        st_from_f32(xws, (b * m + r) * ldx + j, u);
      }
      ss += u * u;
      if constexpr (F32OP) lx[r * C::LDX + jl] = us;
      else lx[r * C::LDX + jl] = f2bf(us);
    }
  }
  ss = wave_sum(ss);
  if ((t & (WAVE - 1)) == 0) wsum[t / WAVE] = ss;
  __syncthreads();
  if (t == 0) {
    float v = 0.f;
    for (int q = 0; q < SK_WAVES; ++q) v += wsum[q];
    sp[blk] = v;
  }
  gram_partial<F32OP>(lds_raw, gp_out + blk * T, T);
}

// ---------------------------------------------------------------------------
// One Newton-Schulz step on a chunk.  LAST: apply the update (or write O).
// ---------------------------------------------------------------------------
template <int MAXM, bool F32OP, typename XS, typename PT, bool LAST>
__global__ void __launch_bounds__(SK_THREADS)
sk_iter(XS* __restrict__ xws, const float* __restrict__ gp_in, float* __restrict__ gp_out,
        const float* __restrict__ sp, int first, float eps,
        int m, int64_t n, int64_t ldx, int S, int T, int transposed,
        float ca, float cb, float cc,
        PT* __restrict__ param, float* __restrict__ ns_out, float lr, float wd, float s_scale) {
  typedef SkCfg<F32OP> C;
  typedef typename C::Op Op;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[kLdsXBytes];
  __shared__ float As[SK_MP][SK_MP + 1];
  __shared__ float Bs[SK_MP][SK_MP + 1];
  __shared__ float inv_s;
  Op* lx = reinterpret_cast<Op*>(lds_raw);

  const int64_t blk = blockIdx.x;
  const int64_t b = blk / S;
  const int c = (int)(blk % S);
  const int t = threadIdx.x;

  // 1. A from the partials (fixed order over chunks)
  for (int e = t; e < SK_MP * (SK_MP + 1); e += SK_THREADS) (&As[0][0])[e] = 0.f;
  if (t == 0) {
    float inv = 1.f;
    if (first) {
      float v = 0.f;
      for (int q = 0; q < S; ++q) v += sp[b * S + q];
      const float den = sqrtf(v) + eps;
      inv = den > 0.f ? 1.f / den : 0.f;
    }
    inv_s = inv;
  }
  __syncthreads();
  const float inv = inv_s;
  const float scaleA = inv * inv;
  for (int idx = t; idx < T; idx += SK_THREADS) {
    float v = 0.f;
    const float* p = gp_in + b * S * (int64_t)T + idx;
    for (int q = 0; q < S; ++q) v += p[(int64_t)q * T];
    int r, s;
    tri_rc(idx, r, s);
    v *= scaleA;
    As[r][s] = v;
    As[s][r] = v;
  }
  __syncthreads();
  // 2. B = b A + c A A  (fp32)
  for (int e = t; e < MAXM * MAXM; e += SK_THREADS) {
    const int r = e / MAXM, s = e % MAXM;
    float acc = 0.f;
#pragma unroll 8
    for (int k = 0; k < MAXM; ++k) acc += As[r][k] * As[k][s];
    Bs[r][s] = cb * As[r][s] + cc * acc;
  }
  __syncthreads();

  // 3. X' = a X + B X on this thread's CPT columns
  float x[C::CPT][MAXM];
#pragma unroll
  for (int r = 0; r < MAXM; ++r) {
#pragma unroll
    for (int q = 0; q < C::CPT; ++q) {
      const int64_t j = (int64_t)c * C::L + t * C::CPT + q;
      x[q][r] = (r < m) ? ld_as_f32(xws, (b * m + r) * ldx + j) * inv : 0.f;
    }
  }
  if constexpr (!LAST) {
    for (int r = m; r < SK_MP; ++r) {
#pragma unroll
      for (int q = 0; q < C::CPT; ++q) lx[r * C::LDX + t * C::CPT + q] = (Op)0;
    }
  }
#pragma unroll
  for (int r = 0; r < MAXM; ++r) {
    float y[C::CPT];
#pragma unroll
    for (int q = 0; q < C::CPT; ++q) y[q] = ca * x[q][r];
#pragma unroll
    for (int s = 0; s < MAXM; ++s) {
      const float bv = Bs[r][s];
#pragma unroll
      for (int q = 0; q < C::CPT; ++q) y[q] += bv * x[q][s];
    }
    if (r < m) {
#pragma unroll
      for (int q = 0; q < C::CPT; ++q) {
        const int jl = t * C::CPT + q;
        const int64_t j = (int64_t)c * C::L + jl;
        if constexpr (!LAST) {
          st_from_f32(xws, (b * m + r) * ldx + j, y[q]);
          const float ys = round_to<XS>(y[q]);
          if constexpr (F32OP) lx[r * C::LDX + jl] = ys;
          else lx[r * C::LDX + jl] = f2bf(ys);
        } else if (j < n) {
          const int64_t si = b * (int64_t)m * n + stored_index(transposed, r, j, m, n);
          if (ns_out) ns_out[si] = y[q];
          if (param) {
            const float w = ld_as_f32(param, si);
            st_from_f32(param, si, apply_update(w, y[q], lr, wd, s_scale));
          }
        }
      }
    }
  }
  if constexpr (!LAST) {
    __syncthreads();
    gram_partial<F32OP>(lds_raw, gp_out + blk * T, T);
  }
}

template <bool F32OP, typename XS, typename GT>
hipError_t launch_first(const StepArgs& a, const WsLayout& L, int mode) {
  const BatchShape& sh = a.shape;
  dim3 grid((unsigned)(sh.count * L.S)), block(SK_THREADS);
  MUON_LAUNCH(mode == 0 ? "sk_momentum_norm_gram" : "sk_norm_gram", (sk_first<F32OP, XS, GT>), grid, block,
              a.stream, mode,
                     (const GT*)a.grad, a.mom, a.u_in, (XS*)(a.ws + L.x), (float*)(a.ws + L.gp0),
                     (float*)(a.ws + L.sp), (int)sh.m, sh.n, L.ldx, (int)L.S, (int)L.T,
                     (int)sh.transposed, a.mu, a.nesterov);
  return hipGetLastError();
}

template <int MAXM, bool F32OP, typename XS, typename PT>
hipError_t launch_iters(const StepArgs& a, const WsLayout& L) {
  const BatchShape& sh = a.shape;
  dim3 grid((unsigned)(sh.count * L.S)), block(SK_THREADS);
  float* gp[2] = {(float*)(a.ws + L.gp0), (float*)(a.ws + L.gp1)};
  PT* param = a.phase == PH_FULL ? (PT*)a.param : nullptr;
  for (int k = 0; k < a.steps; ++k) {
    const float ca = a.coeffs[3 * k], cb = a.coeffs[3 * k + 1], cc = a.coeffs[3 * k + 2];
    const bool last = (k == a.steps - 1);
    if (!last)
      MUON_LAUNCH("sk_ns_step", (sk_iter<MAXM, F32OP, XS, PT, false>), grid, block, a.stream,
                         (XS*)(a.ws + L.x), gp[k & 1], gp[(k + 1) & 1], (const float*)(a.ws + L.sp),
                         (int)(k == 0), a.eps, (int)sh.m, sh.n, L.ldx, (int)L.S, (int)L.T,
                         (int)sh.transposed, ca, cb, cc, param, a.ns_out, a.lr, a.wd, a.s);
    else
      MUON_LAUNCH("sk_ns_step_update", (sk_iter<MAXM, F32OP, XS, PT, true>), grid, block, a.stream,
                         (XS*)(a.ws + L.x), gp[k & 1], gp[(k + 1) & 1], (const float*)(a.ws + L.sp),
                         (int)(k == 0), a.eps, (int)sh.m, sh.n, L.ldx, (int)L.S, (int)L.T,
                         (int)sh.transposed, ca, cb, cc, param, a.ns_out, a.lr, a.wd, a.s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool F32OP, typename XS>
hipError_t run_mode(const StepArgs& a, const WsLayout& L) {
  hipError_t e;
  const int mode = a.phase == PH_FULL ? 0 : 1;
  if (a.grad_dtype == DT_BF16) e = launch_first<F32OP, XS, bf16_t>(a, L, mode);
  else e = launch_first<F32OP, XS, float>(a, L, mode);
  if (e != hipSuccess) return e;
  const int64_t m = a.shape.m;
  const bool pbf = (a.phase == PH_FULL && a.param_dtype == DT_BF16);
#define MUON_SK_ITERS(MM)                                                   \
  return pbf ? launch_iters<MM, F32OP, XS, bf16_t>(a, L)                    \
             : launch_iters<MM, F32OP, XS, float>(a, L);
  if (m <= 8) { MUON_SK_ITERS(8) }
  if (m <= 16) { MUON_SK_ITERS(16) }
  if (m <= 24) { MUON_SK_ITERS(24) }
  MUON_SK_ITERS(32)
#undef MUON_SK_ITERS
}

}  // namespace

hipError_t run_skinny(const StepArgs& a, const WsLayout& L) {
  switch (a.prec) {
    case PREC_BF16: return run_mode<false, bf16_t>(a, L);
    case PREC_BF16_X32: return run_mode<false, float>(a, L);
    default: return run_mode<true, float>(a, L);
  }
}

}  // namespace muon
