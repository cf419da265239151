// Tiled path of the Muon step: matrices whose short side m exceeds 32.
//
// Newton-Schulz runs on X (m x n, rows <= columns after the transpose-first
// rule of HyperParallel-FSDP §6.6) as three products per step, each an "NT"
// product C = P Q^T whose two operands are both contiguous along the
// reduction index, so both stream through LDS the same way:
//
//   Gram  A = X X^T          P = Q = X            lower-triangle tiles, mirrored
//   poly  B = b A + c A A    P = Q = A (A = A^T)  lower-triangle tiles, mirrored
//   apply X' = a X + B X     P = B, Q = X^T       all tiles
//
// (HyperParallel-FSDP Eq. (1), with the symmetric products computed on one
// triangle as DMuon-2 Appendix C.3 describes.)  The apply product needs X^T
// with the short index contiguous, so its epilogue writes X' in both
// layouts; the Gram of the next step reads X', the next apply reads X'^T.
// X and X^T are stored zero-padded to a multiple of 128 in both dimensions;
// the padding stays zero through every step (zero rows and columns map to
// zero), so no kernel needs a bounds check except where the final update
// touches the caller's W.
//
// Operands are bf16 on v_mfma_f32_32x32x16_bf16 with fp32 accumulation, or
// fp32 on v_mfma_f32_32x32x2f32 for the check path.
#include "common.h"
#include "internal.h"

namespace muon {
namespace {

constexpr int GM_THREADS = 256;
constexpr int BM = 128, BN = 128;

// ---------------------------------------------------------------------------
// momentum / norm partials
//   mode 0: M' = mu M + G in place; partial sum of U^2 (U = G + mu M' or M')
//   mode 1: partial sum of U^2 of a given U (u_in)
//   mode 2: M' = mu M + G in place and U written to u_out (no partials)
// ---------------------------------------------------------------------------
template <typename GT>
__global__ void __launch_bounds__(256)
tl_momentum(int mode, const GT* __restrict__ grad, float* __restrict__ mom, const float* __restrict__ u_in,
            float* __restrict__ u_out, float* __restrict__ ssp, int64_t elems, int64_t nparts,
            float mu, int nesterov) {
  __shared__ float wsum[4];
  const int64_t b = blockIdx.x / nparts;
  const int64_t p = blockIdx.x % nparts;
  const int64_t chunk = ((elems + nparts - 1) / nparts + 1023) / 1024 * 1024;
  const int64_t lo = p * chunk;
  const int64_t hi = lo + chunk < elems ? lo + chunk : elems;
  const int64_t base = b * elems;
  float ss = 0.f;
  for (int64_t e = lo + threadIdx.x; e < hi; e += 256) {
    const int64_t i = base + e;
    float u;
    if (mode == 1) {
      u = u_in[i];
    } else {
      const float g = ld_as_f32(grad, i);
      const float mn = mu * mom[i] + g;
      mom[i] = mn;
      u = nesterov ? g + mu * mn : mn;
      if (mode == 2) u_out[i] = u;
    }
    ss += u * u;
  }
  if (mode == 2) return;
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) ssp[blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// inv[b] = 1 / (sqrt(sum of partials) + eps), or 0 if that denominator is 0.
__global__ void __launch_bounds__(256)
tl_norm_finalize(const float* __restrict__ ssp, int64_t nparts, float eps, float* __restrict__ inv) {
  __shared__ float wsum[4];
  const int64_t b = blockIdx.x;
  float v = 0.f;
  for (int64_t q = threadIdx.x; q < nparts; q += 256) v += ssp[b * nparts + q];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float den = sqrtf(((wsum[0] + wsum[1]) + wsum[2]) + wsum[3]) + eps;
    inv[b] = den > 0.f ? 1.f / den : 0.f;
  }
}

// ---------------------------------------------------------------------------
// X0 = U * inv in both layouts (and the fp32 master), 64x64 tiles through LDS.
//   mode 0: U = G + mu M' (M' already updated) or M'
//   mode 1: U from u_in
// Tiles are in the Newton-Schulz orientation: (i, j), i < mp, j < np.
// ---------------------------------------------------------------------------
template <typename GT, typename XO>
__global__ void __launch_bounds__(256)
tl_layout(int mode, const GT* __restrict__ grad, const float* __restrict__ mom, const float* __restrict__ u_in,
          const float* __restrict__ inv, XO* __restrict__ X, XO* __restrict__ XT, float* __restrict__ X32,
          int64_t m, int64_t n, int64_t mp, int64_t np, int transposed, float mu, int nesterov) {
  __shared__ float tile[64][65];
  const int64_t tiles_j = np / 64;
  const int64_t tiles_per = (mp / 64) * tiles_j;
  const int64_t b = blockIdx.x / tiles_per;
  const int64_t tt = blockIdx.x % tiles_per;
  const int64_t i0 = (tt / tiles_j) * 64, j0 = (tt % tiles_j) * 64;
  const float sc = inv[b];
  const int64_t sbase = b * m * n;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    int li, lj;
    if (!transposed) { li = e >> 6; lj = e & 63; }   // stored rows are X rows
    else { lj = e >> 6; li = e & 63; }               // stored rows are X columns
    const int64_t i = i0 + li, j = j0 + lj;
    float v = 0.f;
    if (i < m && j < n) {
      const int64_t si = sbase + (transposed ? j * m + i : i * n + j);
      float u;
      if (mode == 1) {
        u = u_in[si];
      } else {
        const float g = ld_as_f32(grad, si);
        const float mn = mom[si];
        u = nesterov ? g + mu * mn : mn;
      }
      v = u * sc;
    }
    tile[li][lj] = v;
  }
  __syncthreads();
  const int64_t xb = b * mp * np;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int li = e >> 6, lj = e & 63;
    const float v = tile[li][lj];
    const int64_t xi = xb + (i0 + li) * np + j0 + lj;
    st_from_f32(X, xi, v);
    if (X32) X32[xi] = v;
  }
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int lj = e >> 6, li = e & 63;
    st_from_f32(XT, xb + (j0 + lj) * mp + i0 + li, tile[li][lj]);
  }
}

// ---------------------------------------------------------------------------
// NT product on MFMA with three epilogues.
// ---------------------------------------------------------------------------
enum { EPI_GRAM = 0, EPI_POLY = 1, EPI_APPLY = 2 };

struct GemmArgs {
  const void* P; const void* Q;
  int64_t ldp, ldq, strideP, strideQ, K;
  int64_t tiles_n, tiles_per_mat;   // tiles along the output columns; tiles per matrix
  // EPI_GRAM: A32 (+ A16) out.  EPI_POLY: A32 in, PB out.
  float* A32; bf16_t* A16; void* PB; int64_t lda, strideA;
  float ca, cb, cc;
  // EPI_APPLY
  void* X; float* X32; void* XT; int64_t ldx, ldxt, strideX;
  int last;
  void* param; int param_bf16; float* ns_out; float lr, wd, s;
  int64_t m, n; int transposed;
};

template <typename OP> struct OpCfg;
template <> struct OpCfg<bf16_t> { static constexpr int BK = 64, LD = 72; };   // 128 B rows + 16 B pad
template <> struct OpCfg<float> { static constexpr int BK = 32, LD = 36; };

__device__ __forceinline__ void tri_tile(int64_t t, int64_t& ti, int64_t& tj) {
  int64_t r = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (r * (r + 1) / 2 > t) --r;
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  ti = r;
  tj = t - r * (r + 1) / 2;
}

template <typename T>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float v) {
  st_from_f32(reinterpret_cast<T*>(base), i, v);
}

template <typename OP, int EPI, typename PT>
__global__ void __launch_bounds__(GM_THREADS)
tl_gemm(GemmArgs g) {
  typedef OpCfg<OP> C;
  __shared__ __attribute__((aligned(16))) OP Ps[BM * C::LD];
  __shared__ __attribute__((aligned(16))) OP Qs[BN * C::LD];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int64_t mat = blockIdx.x / g.tiles_per_mat;
  const int64_t tt = blockIdx.x % g.tiles_per_mat;
  int64_t ti, tj;
  if (EPI == EPI_APPLY) { ti = tt / g.tiles_n; tj = tt % g.tiles_n; }
  else tri_tile(tt, ti, tj);
  const int64_t i0 = ti * BM, j0 = tj * BN;

  const OP* P = reinterpret_cast<const OP*>(g.P) + mat * g.strideP + i0 * g.ldp;
  const OP* Q = reinterpret_cast<const OP*>(g.Q) + mat * g.strideQ + j0 * g.ldq;

  // global -> register staging: 4 x 16 B per thread per operand
  constexpr int VPR = C::BK * (int)sizeof(OP) / 16;   // 16-byte vectors per tile row (8)
  constexpr int EPV = 16 / (int)sizeof(OP);            // elements per 16-byte vector
  uint4 pr0, pr1, pr2, pr3, qr0, qr1, qr2, qr3;
  const int r0 = t / VPR, cv = (t % VPR) * EPV;       // rows r0 + 32*it, it = 0..3
  const OP* Pp = P + r0 * g.ldp + cv;
  const OP* Qp = Q + r0 * g.ldq + cv;
  const int64_t p32 = 32 * g.ldp, q32 = 32 * g.ldq;
#define MUON_GLOAD(k0)                                                      \
  do {                                                                      \
    pr0 = *reinterpret_cast<const uint4*>(Pp + (k0));                       \
    pr1 = *reinterpret_cast<const uint4*>(Pp + p32 + (k0));                 \
    pr2 = *reinterpret_cast<const uint4*>(Pp + 2 * p32 + (k0));             \
    pr3 = *reinterpret_cast<const uint4*>(Pp + 3 * p32 + (k0));             \
    qr0 = *reinterpret_cast<const uint4*>(Qp + (k0));                       \
    qr1 = *reinterpret_cast<const uint4*>(Qp + q32 + (k0));                 \
    qr2 = *reinterpret_cast<const uint4*>(Qp + 2 * q32 + (k0));             \
    qr3 = *reinterpret_cast<const uint4*>(Qp + 3 * q32 + (k0));             \
  } while (0)
  OP* Pl = &Ps[r0 * C::LD + cv];
  OP* Ql = &Qs[r0 * C::LD + cv];
  static_assert(GM_THREADS / VPR == 32, "staging assumes 32 rows per pass");

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  const int64_t KT = g.K / C::BK;
  MUON_GLOAD(0);
  for (int64_t kt = 0; kt < KT; ++kt) {
    __syncthreads();
    *reinterpret_cast<uint4*>(Pl) = pr0;
    *reinterpret_cast<uint4*>(Pl + 32 * C::LD) = pr1;
    *reinterpret_cast<uint4*>(Pl + 64 * C::LD) = pr2;
    *reinterpret_cast<uint4*>(Pl + 96 * C::LD) = pr3;
    *reinterpret_cast<uint4*>(Ql) = qr0;
    *reinterpret_cast<uint4*>(Ql + 32 * C::LD) = qr1;
    *reinterpret_cast<uint4*>(Ql + 64 * C::LD) = qr2;
    *reinterpret_cast<uint4*>(Ql + 96 * C::LD) = qr3;
    __syncthreads();
    if (kt + 1 < KT) MUON_GLOAD((kt + 1) * C::BK);
    if constexpr (sizeof(OP) == 2) {
#pragma unroll
      for (int kk = 0; kk < C::BK / 16; ++kk) {
        bf16x8 av[2], bv[2];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
          av[ib] = *reinterpret_cast<const bf16x8*>(&Ps[(wm * 64 + ib * 32 + (lane & 31)) * C::LD + kk * 16 + (lane >> 5) * 8]);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
          bv[jb] = *reinterpret_cast<const bf16x8*>(&Qs[(wn * 64 + jb * 32 + (lane & 31)) * C::LD + kk * 16 + (lane >> 5) * 8]);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int jb = 0; jb < 2; ++jb)
            acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ib], bv[jb], acc[ib][jb], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < C::BK / 2; ++kk) {
        float av[2], bv[2];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
          av[ib] = reinterpret_cast<const float*>(Ps)[(wm * 64 + ib * 32 + (lane & 31)) * C::LD + kk * 2 + (lane >> 5)];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
          bv[jb] = reinterpret_cast<const float*>(Qs)[(wn * 64 + jb * 32 + (lane & 31)) * C::LD + kk * 2 + (lane >> 5)];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int jb = 0; jb < 2; ++jb)
            acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[ib], bv[jb], acc[ib][jb], 0, 0, 0);
      }
    }
  }

#undef MUON_GLOAD

  // ---- epilogues -----------------------------------------------------------
  const bool diag = (EPI != EPI_APPLY) && (ti == tj);
#pragma unroll
  for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = i0 + wm * 64 + ib * 32 + mfma32_row(lane, r);
        const int64_t j = j0 + wn * 64 + jb * 32 + mfma32_col(lane);
        const float v = acc[ib][jb][r];
        if constexpr (EPI == EPI_GRAM) {
          const int64_t ab = mat * g.strideA;
          g.A32[ab + i * g.lda + j] = v;
          if (g.A16) g.A16[ab + i * g.lda + j] = f2bf(v);
          if (!diag) {
            g.A32[ab + j * g.lda + i] = v;
            if (g.A16) g.A16[ab + j * g.lda + i] = f2bf(v);
          }
        } else if constexpr (EPI == EPI_POLY) {
          const int64_t ab = mat * g.strideA;
          const float o = g.cb * g.A32[ab + i * g.lda + j] + g.cc * v;
          store_elem<OP>(g.PB, ab + i * g.lda + j, o);
          if (!diag) store_elem<OP>(g.PB, ab + j * g.lda + i, o);
        } else {
          const int64_t xi = mat * g.strideX + i * g.ldx + j;
          const float xo = g.X32 ? g.X32[xi] : ld_as_f32(reinterpret_cast<const OP*>(g.X), xi);
          const float o = g.ca * xo + v;
          if (!g.last) {
            store_elem<OP>(g.X, xi, o);
            if (g.X32) g.X32[xi] = o;
            store_elem<OP>(g.XT, mat * g.strideX + j * g.ldxt + i, o);
          } else if (i < g.m && j < g.n) {
            const int64_t si = mat * g.m * g.n + (g.transposed ? j * g.m + i : i * g.n + j);
            if (g.ns_out) g.ns_out[si] = o;
            if (g.param) {
              PT* W = reinterpret_cast<PT*>(g.param);
              st_from_f32(W, si, apply_update(ld_as_f32(W, si), o, g.lr, g.wd, g.s));
            }
          }
        }
      }
    }
  }
}

template <typename PT>
__global__ void __launch_bounds__(256)
tl_update(PT* __restrict__ W, const float* __restrict__ O, int64_t total, float lr, float wd, float s) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
    st_from_f32(W, i, apply_update(ld_as_f32(W, i), O[i], lr, wd, s));
}

// ---------------------------------------------------------------------------
template <typename GT>
hipError_t launch_momentum(const StepArgs& a, int mode, float* ssp, int64_t nparts) {
  const BatchShape& sh = a.shape;
  const int64_t elems = sh.M * sh.N;
  dim3 grid((unsigned)(sh.count * nparts)), block(256);
  MUON_LAUNCH(mode == 2 ? "momentum" : "tl_momentum_norm", (tl_momentum<GT>), grid, block, a.stream, mode, (const GT*)a.grad, a.mom, a.u_in,
                     a.u_out, ssp, elems, nparts, a.mu, a.nesterov);
  return hipGetLastError();
}

template <typename OP, typename GT, typename PT>
hipError_t tiled_impl(const StepArgs& a, const WsLayout& L) {
  const BatchShape& sh = a.shape;
  const int mode = a.phase == PH_FULL ? 0 : 1;
  float* ssp = (float*)(a.ws + L.ssp);
  float* inv = (float*)(a.ws + L.inv);
  hipError_t e = launch_momentum<GT>(a, mode, ssp, L.nparts);
  if (e != hipSuccess) return e;
  MUON_LAUNCH("tl_norm_finalize", tl_norm_finalize, dim3((unsigned)sh.count), dim3(256), a.stream, ssp, L.nparts,
              a.eps, inv);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  OP* X = (OP*)(a.ws + L.x);
  OP* XT[2] = {(OP*)(a.ws + L.xt0), (OP*)(a.ws + L.xt1)};
  float* X32 = a.prec == PREC_BF16_X32 ? (float*)(a.ws + L.x32) : nullptr;
  float* A32 = (float*)(a.ws + L.a32);
  bf16_t* A16 = a.prec == PREC_F32 ? nullptr : (bf16_t*)(a.ws + L.a16);
  OP* PB = (OP*)(a.ws + L.pb);
  const int64_t mp = L.mp, np = L.np;

  {
    const unsigned blocks = (unsigned)(sh.count * (mp / 64) * (np / 64));
    MUON_LAUNCH("tl_layout", (tl_layout<GT, OP>), dim3(blocks), dim3(256), a.stream, mode, (const GT*)a.grad,
                       (const float*)a.mom, a.u_in, (const float*)inv, X, XT[0], X32, sh.m, sh.n, mp, np,
                       (int)sh.transposed, a.mu, a.nesterov);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t tm = mp / BM, tn = np / BN;
  const int64_t tri = tm * (tm + 1) / 2;
  for (int k = 0; k < a.steps; ++k) {
    const float ca = a.coeffs[3 * k], cb = a.coeffs[3 * k + 1], cc = a.coeffs[3 * k + 2];
    GemmArgs g = {};
    // Gram: A = X X^T
    g.P = X; g.Q = X; g.ldp = np; g.ldq = np; g.strideP = mp * np; g.strideQ = mp * np; g.K = np;
    g.tiles_n = tm; g.tiles_per_mat = tri;
    g.A32 = A32; g.A16 = A16; g.lda = mp; g.strideA = mp * mp;
    MUON_LAUNCH("tl_gram", (tl_gemm<OP, EPI_GRAM, PT>), dim3((unsigned)(sh.count * tri)), dim3(GM_THREADS),
                a.stream, g);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // poly: B = b A + c A A
    g = GemmArgs{};
    if (a.prec == PREC_F32) { g.P = A32; g.Q = A32; } else { g.P = A16; g.Q = A16; }
    g.ldp = mp; g.ldq = mp; g.strideP = mp * mp; g.strideQ = mp * mp; g.K = mp;
    g.tiles_n = tm; g.tiles_per_mat = tri;
    g.A32 = A32; g.PB = PB; g.lda = mp; g.strideA = mp * mp; g.cb = cb; g.cc = cc;
    MUON_LAUNCH("tl_poly", (tl_gemm<OP, EPI_POLY, PT>), dim3((unsigned)(sh.count * tri)), dim3(GM_THREADS),
                a.stream, g);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // apply: X' = a X + B X, B X read as B (X^T)^T
    g = GemmArgs{};
    g.P = PB; g.Q = XT[k & 1]; g.ldp = mp; g.ldq = mp; g.strideP = mp * mp; g.strideQ = np * mp; g.K = mp;
    g.tiles_n = tn; g.tiles_per_mat = tm * tn;
    g.ca = ca; g.X = X; g.X32 = X32; g.XT = XT[(k + 1) & 1]; g.ldx = np; g.ldxt = mp; g.strideX = mp * np;
    g.last = (k == a.steps - 1);
    g.param = a.phase == PH_FULL ? a.param : nullptr; g.param_bf16 = a.param_dtype == DT_BF16;
    g.ns_out = a.ns_out; g.lr = a.lr; g.wd = a.wd; g.s = a.s;
    g.m = sh.m; g.n = sh.n; g.transposed = sh.transposed;
    MUON_LAUNCH(g.last ? "tl_apply_update" : "tl_apply", (tl_gemm<OP, EPI_APPLY, PT>),
                dim3((unsigned)(sh.count * tm * tn)), dim3(GM_THREADS), a.stream, g);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename OP>
hipError_t tiled_dispatch(const StepArgs& a, const WsLayout& L) {
  const bool gbf = a.grad_dtype == DT_BF16;
  const bool pbf = a.phase == PH_FULL && a.param_dtype == DT_BF16;
  if (gbf) return pbf ? tiled_impl<OP, bf16_t, bf16_t>(a, L) : tiled_impl<OP, bf16_t, float>(a, L);
  return pbf ? tiled_impl<OP, float, bf16_t>(a, L) : tiled_impl<OP, float, float>(a, L);
}

}  // namespace

hipError_t run_tiled(const StepArgs& a, const WsLayout& L) {
  if (a.prec == PREC_F32) return tiled_dispatch<float>(a, L);
  return tiled_dispatch<bf16_t>(a, L);
}

hipError_t run_momentum_only(const StepArgs& a) {
  const int64_t nparts = norm_parts(a.shape.M * a.shape.N);
  if (a.grad_dtype == DT_BF16) return launch_momentum<bf16_t>(a, 2, nullptr, nparts);
  return launch_momentum<float>(a, 2, nullptr, nparts);
}

hipError_t run_update_only(const StepArgs& a) {
  const int64_t total = a.shape.count * a.shape.M * a.shape.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (a.param_dtype == DT_BF16)
    MUON_LAUNCH("update", (tl_update<bf16_t>), dim3((unsigned)blocks), dim3(256), a.stream, (bf16_t*)a.param,
                a.o_in, total, a.lr, a.wd, a.s);
  else
    MUON_LAUNCH("update", (tl_update<float>), dim3((unsigned)blocks), dim3(256), a.stream, (float*)a.param,
                a.o_in, total, a.lr, a.wd, a.s);
  return hipGetLastError();
}

}  // namespace muon
