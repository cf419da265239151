// Skinny path, one workgroup per matrix: the "owner" kernel.
//
// For matrices whose short side m is at most 32, one workgroup (8 waves)
// owns one whole matrix and runs the entire step in a single launch (the
// owner-side step of DMuon architecture §2-3, shape-fused over the batch as
// in HyperParallel-FSDP §6.6):
//
//   phase 0   momentum M' = mu M + G, U = G + mu M' (or a given U), U into the
//             workspace, ||U||^2, and the Gram matrix U U^T;
//   step k    B' = a I + b A + c A A from the Gram matrix A of the previous
//             pass (HyperParallel-FSDP Eq. (1) as one product), then one pass
//             over X computing X' = B' X and, except on the last step, the
//             Gram matrix of X'; the last pass applies decay and update to W.
//
// Each wave streams its own 64-column slices of X through a
// private LDS slice (loads for the next slice are in flight while the current
// one is processed) and keeps its share of the Gram matrix in MFMA
// accumulators; the waves meet only at the end of a pass, through workgroup
// barriers, to add their shares in a fixed order.  No workgroup ever waits for
// another.  Operands and precisions are those of the chunked skinny kernels:
// fp32 A and B', B' X with B' as a bf16 hi + lo pair (fp32 on the check path).
#include "common.h"
#include "internal.h"

namespace muon {
namespace {

#ifndef MUON_OWNER_THREADS
#define MUON_OWNER_THREADS 512
#endif
constexpr int OW_THREADS = MUON_OWNER_THREADS;
constexpr int OW_WAVES = OW_THREADS / WAVE;
constexpr int OW_MP = 32;   // rows padded to one 32x32 MFMA block
constexpr int CW = 64;      // columns per wave slice

template <int MODE> struct OwCfg;
template <> struct OwCfg<0> { typedef bf16_t XS; static constexpr int LDW = CW + 8; };
template <> struct OwCfg<1> { typedef float XS; static constexpr int LDW = CW + 4; };
template <> struct OwCfg<2> { typedef float XS; static constexpr int LDW = CW + 4; };

template <int MODE> struct OwLds {
  typedef typename OwCfg<MODE>::XS XS;
  static constexpr int SLICE = OW_MP * OwCfg<MODE>::LDW;                  // elements per wave slice
  static constexpr int STAGE = OW_WAVES * SLICE * (int)sizeof(XS);        // bytes, all slices
  static constexpr int RED = OW_WAVES * OW_MP * (OW_MP + 1) * 4;          // Gram shares of the waves
  static constexpr int BYTES = STAGE > RED ? STAGE : RED;
  static constexpr int EPV = 16 / (int)sizeof(XS);                        // elements per 16 bytes
  static constexpr int VPR = CW / EPV;                                    // 16-byte vectors per slice row
  static constexpr int NV = OW_MP * VPR / WAVE;                           // vectors per lane (all 32 rows)
};

struct Coeffs {
  float c[3 * 64];
};

__device__ __forceinline__ void wave_sync() {
  // LDS accesses of one wave execute in order; keep the compiler from moving
  // them across this point either.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int64_t stored_index(bool transposed, int r, int64_t j, int m, int64_t n) {
  return transposed ? j * m + r : (int64_t)r * n + j;
}

// ---- slice helpers ----------------------------------------------------------
// X slice c (columns [64c, 64c+64) of rows < m) <-> registers <-> LDS slice.
template <int MODE> struct XRegs {
  u32x4 v[OwLds<MODE>::NV];
};

template <int MODE>
__device__ __forceinline__ void xslice_load(XRegs<MODE>& R, const typename OwCfg<MODE>::XS* xb, int64_t ldx,
                                            int64_t c, int m, int lane) {
  typedef OwLds<MODE> Q;
#pragma unroll
  for (int i = 0; i < Q::NV; ++i) {
    const int v = lane + WAVE * i;
    const int r = v / Q::VPR, cv = (v % Q::VPR) * Q::EPV;
    if (r < m) R.v[i] = *reinterpret_cast<const u32x4*>(xb + r * ldx + c * CW + cv);
  }
}

template <int MODE>
__device__ __forceinline__ void xslice_stage(const XRegs<MODE>& R, typename OwCfg<MODE>::XS* sl, int m, int lane) {
  typedef OwLds<MODE> Q;
#pragma unroll
  for (int i = 0; i < Q::NV; ++i) {
    const int v = lane + WAVE * i;
    const int r = v / Q::VPR, cv = (v % Q::VPR) * Q::EPV;
    if (r < m) *reinterpret_cast<u32x4*>(sl + r * OwCfg<MODE>::LDW + cv) = R.v[i];
  }
}

template <int MODE>
__device__ __forceinline__ void xslice_store(const typename OwCfg<MODE>::XS* sl, typename OwCfg<MODE>::XS* xb,
                                             int64_t ldx, int64_t c, int m, int lane) {
  typedef OwLds<MODE> Q;
#pragma unroll
  for (int i = 0; i < Q::NV; ++i) {
    const int v = lane + WAVE * i;
    const int r = v / Q::VPR, cv = (v % Q::VPR) * Q::EPV;
    if (r < m)
      *reinterpret_cast<u32x4*>(xb + r * ldx + c * CW + cv) =
          *reinterpret_cast<const u32x4*>(sl + r * OwCfg<MODE>::LDW + cv);
  }
}

// Gram share of the slice: acc += S S^T (32 x 32) over the slice's 64 columns.
template <int MODE>
__device__ __forceinline__ void xslice_gram(const typename OwCfg<MODE>::XS* sl, f32x16& acc, int lane) {
  constexpr int LDW = OwCfg<MODE>::LDW;
  const int row = lane & 31;
  if constexpr (MODE == 0) {
#pragma unroll
    for (int k0 = 0; k0 < CW; k0 += 16) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(sl + row * LDW + k0 + (lane >> 5) * 8);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, v, acc, 0, 0, 0);
    }
  } else if constexpr (MODE == 1) {
#pragma unroll
    for (int k0 = 0; k0 < CW; k0 += 16) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(sl + row * LDW + k0 + (lane >> 5) * 8);
      const f32x4 b = *reinterpret_cast<const f32x4*>(sl + row * LDW + k0 + (lane >> 5) * 8 + 4);
      bf16x8 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = __builtin_bit_cast(__bf16, f2bf(a[q]));
        v[q + 4] = __builtin_bit_cast(__bf16, f2bf(b[q]));
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, v, acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < CW; k0 += 2) {
      const float v = sl[row * LDW + k0 + (lane >> 5)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(v, v, acc, 0, 0, 0);
    }
  }
}

// B' operand fragments of one lane (see sk_bprime for the layout).
struct OwFrag {
  bf16x8 hi[2], lo[2];   // bf16 modes
  float f[16];           // fp32 mode
};

// X' = B' X on the slice, in place.
template <int MODE>
__device__ __forceinline__ void xslice_apply(typename OwCfg<MODE>::XS* sl, const OwFrag& fr, int lane) {
  constexpr int LDW = OwCfg<MODE>::LDW;
  const int row = lane & 31, hi8 = (lane >> 5) * 8;
#pragma unroll
  for (int jb = 0; jb < CW / 32; ++jb) {
    const int col = jb * 32 + row;
    f32x16 acc = {};
    if constexpr (MODE == 2) {
#pragma unroll
      for (int kb = 0; kb < 16; ++kb)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fr.f[kb], sl[(kb * 2 + (lane >> 5)) * LDW + col], acc, 0, 0, 0);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if constexpr (MODE == 0) {
          bf16x8 xv;
#pragma unroll
          for (int t = 0; t < 8; ++t) xv[t] = __builtin_bit_cast(__bf16, sl[(kb * 16 + hi8 + t) * LDW + col]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.hi[kb], xv, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.lo[kb], xv, acc, 0, 0, 0);
        } else {
          bf16x8 xh, xl;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float v = sl[(kb * 16 + hi8 + t) * LDW + col];
            const bf16_t h = f2bf(v);
            xh[t] = __builtin_bit_cast(__bf16, h);
            xl[t] = __builtin_bit_cast(__bf16, f2bf(v - bf2f(h)));
          }
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.hi[kb], xh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.hi[kb], xl, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.lo[kb], xh, acc, 0, 0, 0);
        }
      }
    }
    wave_sync();   // every lane has read the slice's column block before it is overwritten
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (MODE == 0) sl[mfma32_row(lane, r) * LDW + col] = f2bf(acc[r]);
      else sl[mfma32_row(lane, r) * LDW + col] = acc[r];
    }
  }
}

// ---- phase 0 helpers: momentum on one slice ---------------------------------
// Item (r, g): 8 consecutive columns [64c + 8g, +8) of row r; NI items per lane.
constexpr int P0_NI = OW_MP * (CW / 8) / WAVE;   // 4

template <typename GT> struct GMRegs {
  u32x4 g[P0_NI][sizeof(GT) == 2 ? 1 : 2];
  f32x4 mo[P0_NI][2];
};

template <typename GT>
__device__ __forceinline__ void gm_load(GMRegs<GT>& R, int mode, const GT* grad, const float* mom, const float* u_in,
                                        int64_t mat, int64_t c, int m, int64_t n, int lane) {
#pragma unroll
  for (int i = 0; i < P0_NI; ++i) {
    const int v = lane + WAVE * i;
    const int r = v / (CW / 8);
    const int64_t j = c * CW + (v % (CW / 8)) * 8;
    if (r < m && j < n) {
      const int64_t si = mat + (int64_t)r * n + j;
      if (mode == 0) {
        if constexpr (sizeof(GT) == 2) {
          R.g[i][0] = *reinterpret_cast<const u32x4*>(grad + si);
        } else {
          R.g[i][0] = *reinterpret_cast<const u32x4*>(grad + si);
          R.g[i][1] = *reinterpret_cast<const u32x4*>(grad + si + 4);
        }
        R.mo[i][0] = *reinterpret_cast<const f32x4*>(mom + si);
        R.mo[i][1] = *reinterpret_cast<const f32x4*>(mom + si + 4);
      } else {
        R.mo[i][0] = *reinterpret_cast<const f32x4*>(u_in + si);
        R.mo[i][1] = *reinterpret_cast<const f32x4*>(u_in + si + 4);
      }
    }
  }
}

// M' = mu M + G (stored), U into the LDS slice and the workspace, ss += U^2.
template <int MODE, typename GT>
__device__ __forceinline__ void gm_process(const GMRegs<GT>& R, int mode, float* mom, typename OwCfg<MODE>::XS* sl,
                                           typename OwCfg<MODE>::XS* xb, int64_t ldx, int64_t mat, int64_t c, int m,
                                           int64_t n, float mu, int nesterov, float& ss, int lane) {
  typedef typename OwCfg<MODE>::XS XS;
#pragma unroll
  for (int i = 0; i < P0_NI; ++i) {
    const int v = lane + WAVE * i;
    const int r = v / (CW / 8);
    const int jl = (v % (CW / 8)) * 8;
    const int64_t j = c * CW + jl;
    if (r >= m) continue;
    float u[8];
    if (j < n) {
      if (mode == 0) {
        float g[8];
        if constexpr (sizeof(GT) == 2) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            g[2 * q] = __uint_as_float(R.g[i][0][q] << 16);
            g[2 * q + 1] = __uint_as_float(R.g[i][0][q] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            g[q] = __uint_as_float(R.g[i][0][q]);
            g[q + 4] = __uint_as_float(R.g[i][1][q]);
          }
        }
        f32x4 m0 = R.mo[i][0], m1 = R.mo[i][1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a0 = mu * m0[q] + g[q];
          const float a1 = mu * m1[q] + g[q + 4];
          m0[q] = a0;
          m1[q] = a1;
          u[q] = nesterov ? g[q] + mu * a0 : a0;
          u[q + 4] = nesterov ? g[q + 4] + mu * a1 : a1;
        }
        const int64_t si = mat + (int64_t)r * n + j;
        *reinterpret_cast<f32x4*>(mom + si) = m0;
        *reinterpret_cast<f32x4*>(mom + si + 4) = m1;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u[q] = R.mo[i][0][q];
          u[q + 4] = R.mo[i][1][q];
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) u[q] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ss += u[q] * u[q];
      if constexpr (MODE == 0) sl[r * OwCfg<MODE>::LDW + jl + q] = f2bf(u[q]);
      else sl[r * OwCfg<MODE>::LDW + jl + q] = u[q];
    }
    // the stored U (X of the first step), 8 elements
    XS* dst = xb + r * ldx + j;
    if constexpr (MODE == 0) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (uint32_t)f2bf(u[2 * e]) | ((uint32_t)f2bf(u[2 * e + 1]) << 16);
      *reinterpret_cast<u32x4*>(dst) = w;
    } else {
      *reinterpret_cast<f32x4*>(dst) = f32x4{u[0], u[1], u[2], u[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{u[4], u[5], u[6], u[7]};
    }
  }
}

// Last step: O = X' of the slice, W' = W - lr (wd W + s O) in W's orientation.
template <int MODE, typename PT>
__device__ __forceinline__ void owner_update(const typename OwCfg<MODE>::XS* sl, int64_t c, int m, int64_t n,
                                             int64_t mat, int transposed, int vec, PT* __restrict__ param,
                                             float* __restrict__ ns_out, float lr, float wd, float s, int lane) {
  constexpr int LDW = OwCfg<MODE>::LDW;
  if (vec) {
#pragma unroll
    for (int i = 0; i < P0_NI; ++i) {
      const int v = lane + WAVE * i;
      const int r = v / (CW / 8);
      const int jl = (v % (CW / 8)) * 8;
      const int64_t j = c * CW + jl;
      if (r >= m || j >= n) continue;
      float o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if constexpr (MODE == 0) o[q] = bf2f(sl[r * LDW + jl + q]);
        else o[q] = sl[r * LDW + jl + q];
      }
      const int64_t si = mat + (int64_t)r * n + j;
      if (ns_out) {
        *reinterpret_cast<f32x4*>(ns_out + si) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(ns_out + si + 4) = f32x4{o[4], o[5], o[6], o[7]};
      }
      if (param) {
        if constexpr (sizeof(PT) == 2) {
          u32x4 wv = *reinterpret_cast<const u32x4*>(param + si);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float w0 = __uint_as_float(wv[e] << 16), w1 = __uint_as_float(wv[e] & 0xffff0000u);
            wv[e] = (uint32_t)f2bf(apply_update(w0, o[2 * e], lr, wd, s)) |
                    ((uint32_t)f2bf(apply_update(w1, o[2 * e + 1], lr, wd, s)) << 16);
          }
          *reinterpret_cast<u32x4*>(param + si) = wv;
        } else {
          f32x4 w0 = *reinterpret_cast<const f32x4*>(param + si);
          f32x4 w1 = *reinterpret_cast<const f32x4*>(param + si + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w0[e] = apply_update(w0[e], o[e], lr, wd, s);
            w1[e] = apply_update(w1[e], o[e + 4], lr, wd, s);
          }
          *reinterpret_cast<f32x4*>(param + si) = w0;
          *reinterpret_cast<f32x4*>(param + si + 4) = w1;
        }
      }
    }
  } else {
    for (int e = lane; e < m * CW; e += WAVE) {
      int r, jl;
      if (transposed) { jl = e / m; r = e % m; }
      else { r = e / CW; jl = e % CW; }
      const int64_t j = c * CW + jl;
      if (j >= n) continue;
      float o;
      if constexpr (MODE == 0) o = bf2f(sl[r * LDW + jl]);
      else o = sl[r * LDW + jl];
      const int64_t si = mat + stored_index(transposed, r, j, m, n);
      if (ns_out) ns_out[si] = o;
      if (param) st_from_f32(param, si, apply_update(ld_as_f32(param, si), o, lr, wd, s));
    }
  }
}

// ---- the kernel ---------------------------------------------------------------
template <int MODE, typename GT, typename PT>
__global__ void __launch_bounds__(OW_THREADS)
sk_owner(int mode, const GT* __restrict__ grad, float* __restrict__ mom, const float* __restrict__ u_in,
         typename OwCfg<MODE>::XS* __restrict__ xws, int m, int64_t n, int64_t ldx, int transposed, int vec,
         float mu, int nesterov, float eps, int steps, Coeffs cf, PT* __restrict__ param, float* __restrict__ ns_out,
         float lr, float wd, float s_scale) {
  typedef typename OwCfg<MODE>::XS XS;
  typedef OwLds<MODE> Q;
  constexpr int LDW = OwCfg<MODE>::LDW;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[Q::BYTES];
  __shared__ float As[OW_MP][OW_MP + 1];
  __shared__ float Bp[OW_MP][OW_MP + 1];
  __shared__ float wsum[OW_WAVES];

  const int t = threadIdx.x;
  const int lane = t & (WAVE - 1);
  const int w = t / WAVE;
  const int64_t b = blockIdx.x;
  const int64_t mat = b * (int64_t)m * n;
  const int64_t NC = ldx / CW;                   // slices of the matrix
  XS* xb = xws + b * (int64_t)m * ldx;
  XS* sl = reinterpret_cast<XS*>(lds_raw) + w * Q::SLICE;
  float* red = reinterpret_cast<float*>(lds_raw);

  // rows m..31 of every slice stay zero for the whole kernel
  for (int e = lane; e < (OW_MP - m) * LDW; e += WAVE) sl[m * LDW + e] = (XS)0;

  // ---------------- phase 0: momentum, U, ||U||^2 and U U^T ------------------
  f32x16 gacc = {};
  float ss = 0.f;
  if (vec) {
    GMRegs<GT> ra, rb;
    int64_t c = w;
    if (c < NC) gm_load<GT>(ra, mode, grad, mom, u_in, mat, c, m, n, lane);
    while (c < NC) {
      if (c + OW_WAVES < NC) gm_load<GT>(rb, mode, grad, mom, u_in, mat, c + OW_WAVES, m, n, lane);
      gm_process<MODE, GT>(ra, mode, mom, sl, xb, ldx, mat, c, m, n, mu, nesterov, ss, lane);
      wave_sync();
      xslice_gram<MODE>(sl, gacc, lane);
      wave_sync();
      c += OW_WAVES;
      if (c >= NC) break;
      if (c + OW_WAVES < NC) gm_load<GT>(ra, mode, grad, mom, u_in, mat, c + OW_WAVES, m, n, lane);
      gm_process<MODE, GT>(rb, mode, mom, sl, xb, ldx, mat, c, m, n, mu, nesterov, ss, lane);
      wave_sync();
      xslice_gram<MODE>(sl, gacc, lane);
      wave_sync();
      c += OW_WAVES;
    }
  } else {
    for (int64_t c = w; c < NC; c += OW_WAVES) {
      // element by element, walking the stored layout of the slice
      for (int e = lane; e < m * CW; e += WAVE) {
        int r, jl;
        if (transposed) { jl = e / m; r = e % m; }
        else { r = e / CW; jl = e % CW; }
        const int64_t j = c * CW + jl;
        float u = 0.f;
        if (j < n) {
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
        ss += u * u;
        st_from_f32(sl, r * LDW + jl, u);
      }
      wave_sync();
      xslice_store<MODE>(sl, xb, ldx, c, m, lane);
      xslice_gram<MODE>(sl, gacc, lane);
      wave_sync();
    }
  }

  // ---------------- reduce: ||U||, A = U U^T * inv^2 ---------------------------
  ss = wave_sum(ss);
  __syncthreads();   // all slices done: the staging area becomes the reduction area
  if (lane == 0) wsum[w] = ss;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    red[(w * OW_MP + mfma32_row(lane, r)) * (OW_MP + 1) + mfma32_col(lane)] = gacc[r];
  __syncthreads();
  float inv;
  {
    float v = 0.f;
    for (int q = 0; q < OW_WAVES; ++q) v += wsum[q];
    const float den = sqrtf(v) + eps;
    inv = den > 0.f ? 1.f / den : 0.f;
  }
  for (int e = t; e < OW_MP * OW_MP; e += OW_THREADS) {
    const int r = e / OW_MP, s = e % OW_MP;
    float v = 0.f;
    for (int q = 0; q < OW_WAVES; ++q) v += red[(q * OW_MP + r) * (OW_MP + 1) + s];
    As[r][s] = (r < m && s < m) ? v * inv * inv : 0.f;
  }
  __syncthreads();
  // restore the zero rows of the slices (the reduction used the same memory)
  for (int e = lane; e < (OW_MP - m) * LDW; e += WAVE) sl[m * LDW + e] = (XS)0;

  // ---------------- Newton-Schulz steps ------------------------------------------
  for (int k = 0; k < steps; ++k) {
    const bool last = k == steps - 1;
    const float ca = cf.c[3 * k], cb = cf.c[3 * k + 1], cc = cf.c[3 * k + 2];
    const float bscale = k == 0 ? inv : 1.f;
    if (w == 0) {
      f32x16 a2 = {};
#pragma unroll
      for (int kb = 0; kb < 16; ++kb)
        a2 = __builtin_amdgcn_mfma_f32_32x32x2f32(As[lane & 31][2 * kb + (lane >> 5)],
                                                  As[2 * kb + (lane >> 5)][lane & 31], a2, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = mfma32_row(lane, r), j = mfma32_col(lane);
        const float v = (i < m && j < m) ? cb * As[i][j] + cc * a2[r] + (i == j ? ca : 0.f) : 0.f;
        Bp[i][j] = v * bscale;
      }
    }
    __syncthreads();
    OwFrag fr;
    {
      const int row = lane & 31;
      if constexpr (MODE == 2) {
#pragma unroll
        for (int kb = 0; kb < 16; ++kb) fr.f[kb] = Bp[row][2 * kb + (lane >> 5)];
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float v = Bp[row][kb * 16 + (lane >> 5) * 8 + q];
            const bf16_t h = f2bf(v);
            fr.hi[kb][q] = __builtin_bit_cast(__bf16, h);
            fr.lo[kb][q] = __builtin_bit_cast(__bf16, f2bf(v - bf2f(h)));
          }
        }
      }
    }
    gacc = f32x16{};

    XRegs<MODE> xa, xc;
    int64_t c = w;
    if (c < NC) xslice_load<MODE>(xa, xb, ldx, c, m, lane);
    // process one slice held in registers R (column slice c)
#define MUON_OWNER_SLICE(R)                                                                          \
    do {                                                                                             \
      xslice_stage<MODE>(R, sl, m, lane);                                                            \
      wave_sync();                                                                                   \
      xslice_apply<MODE>(sl, fr, lane);                                                              \
      wave_sync();                                                                                   \
      if (!last) {                                                                                   \
        xslice_store<MODE>(sl, xb, ldx, c, m, lane);                                                 \
        xslice_gram<MODE>(sl, gacc, lane);                                                           \
      } else {                                                                                       \
        owner_update<MODE, PT>(sl, c, m, n, mat, transposed, vec, param, ns_out, lr, wd, s_scale, lane); \
      }                                                                                              \
      wave_sync();                                                                                   \
    } while (0)
    while (c < NC) {
      if (c + OW_WAVES < NC) xslice_load<MODE>(xc, xb, ldx, c + OW_WAVES, m, lane);
      MUON_OWNER_SLICE(xa);
      c += OW_WAVES;
      if (c >= NC) break;
      if (c + OW_WAVES < NC) xslice_load<MODE>(xa, xb, ldx, c + OW_WAVES, m, lane);
      MUON_OWNER_SLICE(xc);
      c += OW_WAVES;
    }
#undef MUON_OWNER_SLICE
    if (last) break;
    // A of the next step: the waves' shares, added in wave order
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r)
      red[(w * OW_MP + mfma32_row(lane, r)) * (OW_MP + 1) + mfma32_col(lane)] = gacc[r];
    __syncthreads();
    for (int e = t; e < OW_MP * OW_MP; e += OW_THREADS) {
      const int r = e / OW_MP, s = e % OW_MP;
      float v = 0.f;
      for (int q = 0; q < OW_WAVES; ++q) v += red[(q * OW_MP + r) * (OW_MP + 1) + s];
      As[r][s] = (r < m && s < m) ? v : 0.f;
    }
    __syncthreads();
    for (int e = lane; e < (OW_MP - m) * LDW; e += WAVE) sl[m * LDW + e] = (XS)0;
  }
}

template <int MODE, typename GT, typename PT>
hipError_t launch_owner(const StepArgs& a, const WsLayout& L) {
  typedef typename OwCfg<MODE>::XS XS;
  const BatchShape& sh = a.shape;
  if (L.ldx % CW != 0 || L.ldx < sh.n || a.steps > 64) return hipErrorInvalidValue;
  Coeffs cf = {};
  for (int i = 0; i < 3 * a.steps; ++i) cf.c[i] = a.coeffs[i];
  const int mode = a.phase == PH_FULL ? 0 : 1;
  const int vec = (!sh.transposed && sh.n % 8 == 0) ? 1 : 0;
  PT* param = a.phase == PH_FULL ? (PT*)a.param : nullptr;
  MUON_LAUNCH("sk_owner", (sk_owner<MODE, GT, PT>), dim3((unsigned)sh.count), dim3(OW_THREADS), a.stream, mode,
              (const GT*)a.grad, a.mom, a.u_in, (XS*)(a.ws + L.x), (int)sh.m, sh.n, L.ldx, (int)sh.transposed, vec,
              a.mu, a.nesterov, a.eps, a.steps, cf, param, a.ns_out, a.lr, a.wd, a.s);
  return hipGetLastError();
}

template <int MODE>
hipError_t owner_mode(const StepArgs& a, const WsLayout& L) {
  const bool gbf = a.grad_dtype == DT_BF16;
  const bool pbf = a.phase == PH_FULL && a.param_dtype == DT_BF16;
  if (gbf) return pbf ? launch_owner<MODE, bf16_t, bf16_t>(a, L) : launch_owner<MODE, bf16_t, float>(a, L);
  return pbf ? launch_owner<MODE, float, bf16_t>(a, L) : launch_owner<MODE, float, float>(a, L);
}

}  // namespace

hipError_t run_skinny_owner(const StepArgs& a, const WsLayout& L) {
  switch (a.prec) {
    case PREC_BF16: return owner_mode<0>(a, L);
    case PREC_BF16_X32: return owner_mode<1>(a, L);
    default: return owner_mode<2>(a, L);
  }
}

}  // namespace muon
