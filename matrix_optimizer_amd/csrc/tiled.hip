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
#include <cmath>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace muon {
namespace {


// ---------------------------------------------------------------------------
// Momentum stage alone (muon_stage_momentum): M' = mu M + G in place and U
// (G + mu M', or M') written to u_out.
// ---------------------------------------------------------------------------
template <typename GT>
__global__ void __launch_bounds__(256)
tl_momentum(const GT* __restrict__ grad, float* __restrict__ mom, float* __restrict__ u_out, int64_t total,
            float mu, int nesterov) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const float g = ld_as_f32(grad, i);
    const float mn = mu * mom[i] + g;
    mom[i] = mn;
    u_out[i] = nesterov ? g + mu * mn : mn;
  }
}

// inv[b] = 1 / (sqrt(sum of partials) + eps), or 0 if that denominator is 0.
// Block 0 also zeroes the nsched tile counters of the step's products.
__global__ void __launch_bounds__(256)
tl_norm_finalize(const float* __restrict__ ssp, int64_t nparts, float eps, float* __restrict__ inv,
                 unsigned* __restrict__ sched, int nsched) {
  __shared__ float wsum[4];
  const int64_t b = blockIdx.x;
  if (sched && b == 0)
    for (int i = threadIdx.x; i < nsched; i += 256) sched[i] = 0u;
  const float* p = ssp + b * nparts;
  float v = 0.f;
  // thread t adds partials t, t + 256, t + 512, ... in that order; 16 loads
  // in flight at a time (one workgroup per matrix, so the loads' latency, not
  // bandwidth, sets the time)
  int64_t q = threadIdx.x;
  for (; q + 15 * 256 < nparts; q += 16 * 256) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = p[q + i * 256];
#pragma unroll
    for (int i = 0; i < 16; ++i) v += x[i];
  }
  for (; q < nparts; q += 256) v += p[q];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float den = sqrtf(((wsum[0] + wsum[1]) + wsum[2]) + wsum[3]) + eps;
    inv[b] = den > 0.f ? 1.f / den : 0.f;
  }
}

// 8 consecutive elements at a 16-byte aligned address, as floats.
__device__ __forceinline__ void load8(const float* p, float* f) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) { f[q] = a[q]; f[q + 4] = b[q]; }
}
__device__ __forceinline__ void load8(const bf16_t* p, float* f) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int q = 0; q < 4; ++q) { f[2 * q] = __uint_as_float(v[q] << 16); f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u); }
}
__device__ __forceinline__ void store8(float* p, const float* f) {
  *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}
__device__ __forceinline__ void store8(bf16_t* p, const float* f) {
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = (uint32_t)f2bf(f[2 * q]) | ((uint32_t)f2bf(f[2 * q + 1]) << 16);
  *reinterpret_cast<u32x4*>(p) = v;
}
// The part of v that bf16 cannot hold: v - bf16(v), exact in fp32 (stored
// rounded to bf16, it makes bf16(v) + bf16(v - bf16(v)) a 16-bit-mantissa
// copy of v).
__device__ __forceinline__ float bf_res(float v) { return v - bf2f(f2bf(v)); }
__device__ __forceinline__ void store_res8(bf16_t* p, const float* f) {
  float r[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) r[q] = bf_res(f[q]);
  store8(p, r);
}

// ---------------------------------------------------------------------------
// First pass of the tiled path, one 64x64 tile (Newton-Schulz orientation)
// per workgroup: momentum and the Nesterov direction U (or a given U), the
// tile's share of ||U||_F^2, and U, unnormalised, row-major and transposed
// when the apply products read X^T (XT non-null).  With the master (R
// non-null) also the part of U that bf16 cannot hold, bf16(U - bf16(U)), in
// the layout in which the apply reads X: row-major, or transposed when XT is
// given.  The first Newton-Schulz step applies 1 / (||U||_F + eps): the Gram
// epilogue scales by its square, the apply epilogue by it.  One pass over G
// and M instead of two.
//   mode 0: M' = mu M + G (in place), U = G + mu M' or M'
//   mode 1: U from u_in
// ssp[blockIdx.x] = sum of U^2 over the tile (fixed order).
// vec (mode 0, no X^T, stored rows a multiple of 8 long): each lane moves
// runs of 8 consecutive stored elements, 16-byte accesses, and issues the
// loads of both its runs before any store; X comes straight from registers
// (through the LDS tile when the stored rows are X columns).  Stored rows
// that are X rows in a padded width that is a multiple of 256 are taken as
// 16 x 256 regions instead of 64 x 64: the same 4096 elements (and partial
// count), but 512-byte runs of each gradient row for the HBM pages.
// ---------------------------------------------------------------------------
template <typename GT, typename XO, bool ROWS>
__global__ void __launch_bounds__(256)
tl_first(int mode, int vec, const GT* __restrict__ grad, float* __restrict__ mom, const float* __restrict__ u_in,
         float* __restrict__ ssp, XO* __restrict__ X, XO* __restrict__ XT, bf16_t* __restrict__ R,
         int64_t m, int64_t n, int64_t mp, int64_t np, int transposed, float mu, int nesterov, MatTabs tabs) {
  __shared__ float tile[64][65];
  __shared__ float wsum[4];
  const bool wide = vec && !transposed && np % 256 == 0;
  const int rh = wide ? 16 : 64, rw = wide ? 256 : 64;   // region rows x columns
  const int lg = wide ? 5 : 3;                          // log2 of the 8-element runs per region row
  const int64_t tiles_j = np / rw;
  const int64_t tiles_per = (mp / rh) * tiles_j;
  const int64_t b = blockIdx.x / tiles_per;
  const int64_t tt = blockIdx.x % tiles_per;
  const int64_t i0 = (tt / tiles_j) * rh, j0 = (tt % tiles_j) * rw;
  const int64_t sbase = b * m * n;
  const int64_t xb = b * mp * np;
  grad = batch_view(grad, tabs.grad, b, m * n);
  mom = batch_view(mom, tabs.mom, b, m * n);
  float ss = 0.f;
  if (vec) {
    // run h of a lane: stored row sr of the region, elements sc .. sc + 7
    Raw8<GT> gr[2];
    Raw8<float> mr[2];
    bool ok[2];
    int64_t si[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = threadIdx.x + 256 * h, sr = v >> lg, sc = (v & ((1 << lg) - 1)) * 8;
      const int64_t i = transposed ? i0 + sc : i0 + sr, j = transposed ? j0 + sr : j0 + sc;
      ok[h] = i < m && j < n;   // whole runs: the stored row length is a multiple of 8
      si[h] = sbase + (transposed ? j * m + i : i * n + j);
      if (ok[h]) {
        if constexpr (ROWS)
          gr[h].load(row_of<const GT>(tabs.grad_rows, b, transposed ? n : m, transposed ? j : i) + (transposed ? i : j));
        else
          gr[h].load(grad + si[h]);
        mr[h].load(mom + si[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = threadIdx.x + 256 * h, sr = v >> lg, sc = (v & ((1 << lg) - 1)) * 8;
      float u[8];
      if (ok[h]) {
        float g[8], mo[8];
        gr[h].to_f32(g);
        mr[h].to_f32(mo);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          mo[q] = mu * mo[q] + g[q];
          u[q] = nesterov ? g[q] + mu * mo[q] : mo[q];
        }
        store8(mom + si[h], mo);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) u[q] = 0.f;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) ss += u[q] * u[q];
      if (transposed) {
#pragma unroll
        for (int q = 0; q < 8; ++q) tile[sc + q][sr] = u[q];
      } else {
        const int64_t xi = xb + (i0 + sr) * np + j0 + sc;
        store8(X + xi, u);
        if (R) store_res8(R + xi, u);
      }
    }
  } else {
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      int li, lj;
      if (!transposed) { li = e >> 6; lj = e & 63; }   // stored rows are X rows
      else { lj = e >> 6; li = e & 63; }               // stored rows are X columns
      const int64_t i = i0 + li, j = j0 + lj;
      float u = 0.f;
      if (i < m && j < n) {
        const int64_t si = sbase + (transposed ? j * m + i : i * n + j);
        if (mode == 1) {
          u = u_in[si];
        } else {
          float g;
          if constexpr (ROWS)
            g = ld_as_f32(row_of<const GT>(tabs.grad_rows, b, transposed ? n : m, transposed ? j : i),
                          transposed ? i : j);
          else
            g = ld_as_f32(grad, si);
          const float mn = mu * mom[si] + g;
          mom[si] = mn;
          u = nesterov ? g + mu * mn : mn;
        }
      }
      ss += u * u;
      tile[li][lj] = u;
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();   // also: the tile is complete
  if (threadIdx.x == 0) ssp[blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  if (!vec) {
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int li = e >> 6, lj = e & 63;
      const float v = tile[li][lj];
      const int64_t xi = xb + (i0 + li) * np + j0 + lj;
      st_from_f32(X, xi, v);
      if (R && !XT) st_from_f32(R, xi, bf_res(v));
    }
  } else if (transposed) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = threadIdx.x + 256 * h, li = v >> 3, lj = (v & 7) * 8;
      float u[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) u[q] = tile[li][lj + q];
      const int64_t xi = xb + (i0 + li) * np + j0 + lj;
      store8(X + xi, u);
      if (R) store_res8(R + xi, u);
    }
  }
  if (XT) {
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int lj = e >> 6, li = e & 63;
      const int64_t ti = xb + (j0 + lj) * mp + i0 + li;
      st_from_f32(XT, ti, tile[li][lj]);
      if (R) st_from_f32(R, ti, bf_res(tile[li][lj]));
    }
  }
}

// ---------------------------------------------------------------------------
// NT product on MFMA with three epilogues.
// ---------------------------------------------------------------------------
// EPI_APPLY writes X' (both layouts); EPI_LAST / EPI_LAST_T are the last
// step's apply for row-major / stored-transposed W, which update W (and
// write O) instead.
enum { EPI_GRAM = 0, EPI_POLY = 1, EPI_APPLY = 2, EPI_LAST = 3, EPI_LAST_T = 4 };

struct GemmArgs {
  const void* P; const void* Q;
  int64_t ldp, ldq, strideP, strideQ, K;
  int64_t tiles_n, tiles_per_mat;   // tiles along the output columns; tiles per matrix
  int64_t tiles_total;              // tiles of the launch (all matrices)
  const float* inv0;                // first step: per-matrix 1/(||U||+eps) (X holds U unscaled), else null
  // EPI_GRAM: A32 (+ A16) out.  EPI_POLY: A32 in, PB out.
  float* A32; bf16_t* A16; void* PB; int64_t lda, strideA;
  float ca, cb, cc;
  // EPI_APPLY
  void* X; void* XT; int64_t ldx, ldxt, strideX;
  // The master (bf16 modes): X = X~ + R with X~ = bf16(X) the product
  // operand and R = bf16(X - X~), R in the layout in which the apply reads X
  // (row-major on direct-load tiles, else as X^T).  Rin: the input's R,
  // added as a R in the epilogue; Rout: the output's R (null: none).
  // Compensated: k-slices kswitch .. of the K loop (K = 2 m) multiply B by
  // the input's R (Q2, Q's layout) instead of X~, and a R comes in with them.
  const bf16_t* Rin; bf16_t* Rout; const void* Q2; int64_t kswitch;
  int last;
  void* param; int param_bf16; float* ns_out; float lr, wd, s;
  const float* lrwd;   // optional device {lr, wd}
  MatTabs tabs;        // per-matrix W / O addresses (zero-copy batching), or null
  int64_t m, n; int transposed;
  unsigned* sched;     // dynamic tile order: this launch's 8 counters (zero at launch), or null
};

// Tile configuration of the NT product kernel: BM x BN output tile per
// workgroup, BK reduction slice per LDS stage, WAVES_M x WAVES_N waves, each
// owning a (BM/WAVES_M) x (BN/WAVES_N) sub-tile of 32x32 MFMA blocks.  LDS rows
// carry 16 bytes of padding so the MFMA fragment reads are bank-conflict free.
template <typename OP, int BM_, int BN_, int BK_, int WGM_, int WGN_, bool DIRECT_ = false>
struct GemmCfg {
  typedef OP Op;
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WGM_, WAVES_N = WGN_;
  static constexpr int THREADS = 64 * WGM_ * WGN_;
  static constexpr int WAVES = WGM_ * WGN_;
  // at least two waves per SIMD: 8-wave tiles by construction, 4-wave tiles
  // so that two workgroups share a CU (register budget 256 per lane)
  static constexpr int WAVES_PER_SIMD = 2;
  static constexpr int WTM = BM / WGM_, WTN = BN / WGN_;
  static constexpr int IB = WTM / 32, JB = WTN / 32;
  static constexpr int EPV = 16 / (int)sizeof(OP);
  // DIRECT: operand tiles go from global memory straight into LDS (no
  // register staging), rows unpadded with 16-byte chunk c of row r stored in
  // slot c ^ swz(r); else register-staged into rows padded by 16 bytes.
  static constexpr bool DIRECT = DIRECT_;
  static constexpr int LD = DIRECT ? BK : BK + EPV;
  static constexpr int VPR = BK / EPV;
  static constexpr int PV = BM * VPR / THREADS;
  static constexpr int QV = BN * VPR / THREADS;
  static constexpr int RPP = THREADS / VPR;          // tile rows per load pass
  static constexpr int STAGE = (BM + BN) * LD;       // elements per LDS stage
  // direct loads: one wave instruction fills RPI whole rows (1 KB); LPW
  // instructions per wave per stage, the first half in P's rows
  static constexpr int RPI = 64 / VPR;
  static constexpr int LPW = (BM + BN) / RPI / WAVES;
  static_assert(BM == BN || BM == 2 * BN, "symmetric products tile BM = BN or 2 BN");
  static_assert(BM * VPR % THREADS == 0 && BN * VPR % THREADS == 0, "load split");
  static_assert(!DIRECT || (sizeof(OP) == 2 && BK == 64 && BM == BN && (BM / RPI) % WAVES == 0),
                "direct loads: bf16, 8 chunks per row, P rows in whole instructions");
};
// bf16, 256x256 tiles, 8 waves of 128x64 (4x2 MFMA blocks): each fragment
// read from LDS feeds more MFMAs than in the 128x128 tile.  Needs rows and
// columns padded to 256.
typedef GemmCfg<bf16_t, 256, 256, 64, 2, 4, true> CfgBig;
typedef GemmCfg<bf16_t, 128, 128, 64, 2, 2> CfgSmall;

typedef GemmCfg<float, 128, 128, 32, 2, 2> CfgF32;

// Tiles of a symmetric product that cover its lower triangle, for tiles of
// BM = R x BN (R = 1 or 2): block row ti holds column tiles tj = 0 .. R ti +
// R - 1, the last R of them inside the diagonal block (computed whole, no
// mirror); tile t of a matrix in row-major order.
template <int R>
__device__ __forceinline__ void tri_tile(int64_t t, int64_t& ti, int64_t& tj) {
  // tiles before row r: R r (r + 1) / 2
  int64_t r = (int64_t)((sqrt(8.0 * (double)t / R + 1.0) - 1.0) * 0.5);
  while (r > 0 && R * r * (r + 1) / 2 > t) --r;
  while (R * (r + 1) * (r + 2) / 2 <= t) ++r;
  ti = r;
  tj = t - R * r * (r + 1) / 2;
}

// Lower-triangle tiles (BM = BN) in groups of GM tile rows, column by
// column, so the 32 tiles an XCD runs at once share few operand bands in its
// L2 (about 13 row / column bands instead of about 22 in row order): the
// tiles before group s are those of its first r0 = GM s rows, then come the
// group's full columns (GM tiles each), then its diagonal block column by
// column.  tm: tile rows of the matrix.
__device__ __forceinline__ void tri_tile_grouped(int64_t tt, int64_t tm, int64_t& ti, int64_t& tj) {
  constexpr int64_t GM = 4;
  int64_t r, c0;
  tri_tile<1>(tt, r, c0);
  const int64_t r0 = (r / GM) * GM;
  const int64_t gme = tm - r0 < GM ? tm - r0 : GM;
  int64_t o = tt - r0 * (r0 + 1) / 2;
  if (o < gme * r0) {
    ti = r0 + o % gme;
    tj = o / gme;
    return;
  }
  o -= gme * r0;
  int64_t c = 0;
  while (o >= gme - c) {   // at most GM - 1 rounds
    o -= gme - c;
    ++c;
  }
  ti = r0 + c + o;
  tj = r0 + c;
}

// Element i of a wave-uniform base, addressed by a 32-bit byte offset (the
// caller guarantees i * sizeof(T) < 2^32): the access takes the base from
// scalar registers and one offset register, instead of a 64-bit address per
// access (which, at full register use, serialises a group of loads).
template <typename T> __device__ __forceinline__ T* at32(T* base, uint32_t i) {
  typedef typename std::conditional<std::is_const<T>::value, const char, char>::type B;
  return reinterpret_cast<T*>(reinterpret_cast<B*>(base) + i * (uint32_t)sizeof(T));
}

// 32 consecutive bf16 elements starting at a 16-byte aligned address, as floats.
__device__ __forceinline__ void load_run32(const bf16_t* p, float* o) {
#pragma unroll
  for (int q = 0; q < 4; ++q) load8(p + 8 * q, o + 8 * q);
}

// 32 consecutive elements starting at a 16-byte aligned address, as 16-byte stores.
__device__ __forceinline__ void store_run32(float* p, const float* o) {
#pragma unroll
  for (int q = 0; q < 8; ++q) *reinterpret_cast<f32x4*>(p + 4 * q) = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
}
__device__ __forceinline__ void store_run32(bf16_t* p, const float* o) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (uint32_t)f2bf(o[8 * q + 2 * e]) | ((uint32_t)f2bf(o[8 * q + 2 * e + 1]) << 16);
    *reinterpret_cast<u32x4*>(p + 8 * q) = v;
  }
}

// Register staging of one k-slice of both operand tiles (16-byte vectors).
// W[0..31] -= lr (wd W + s O[0..31]) on 32 consecutive, 16-byte aligned elements.
__device__ __forceinline__ void update_run32(float* w, const float* o, float lr, float wd, float s) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    f32x4 v = *reinterpret_cast<const f32x4*>(w + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = apply_update(v[e], o[4 * q + e], lr, wd, s);
    *reinterpret_cast<f32x4*>(w + 4 * q) = v;
  }
}
__device__ __forceinline__ void update_run32(bf16_t* w, const float* o, float lr, float wd, float s) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u32x4 v = *reinterpret_cast<const u32x4*>(w + 8 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float w0 = __uint_as_float(v[e] << 16), w1 = __uint_as_float(v[e] & 0xffff0000u);
      v[e] = (uint32_t)f2bf(apply_update(w0, o[8 * q + 2 * e], lr, wd, s)) |
             ((uint32_t)f2bf(apply_update(w1, o[8 * q + 2 * e + 1], lr, wd, s)) << 16);
    }
    *reinterpret_cast<u32x4*>(w + 8 * q) = v;
  }
}

template <class C> struct StageRegs {
  u32x4 p[C::PV];
  u32x4 q[C::QV];
};

template <class C>
__device__ __forceinline__ void stage_load(StageRegs<C>& sr, const typename C::Op* Pp, const typename C::Op* Qp,
                                           int64_t pstep, int64_t qstep, int64_t k0) {
#pragma unroll
  for (int i = 0; i < C::PV; ++i) sr.p[i] = *reinterpret_cast<const u32x4*>(Pp + i * pstep + k0);
#pragma unroll
  for (int i = 0; i < C::QV; ++i) sr.q[i] = *reinterpret_cast<const u32x4*>(Qp + i * qstep + k0);
}

// pl: this thread's first slot of the P rows of a stage; the Q rows follow BM rows later
template <class C>
__device__ __forceinline__ void stage_store(const StageRegs<C>& sr, typename C::Op* pl) {
#pragma unroll
  for (int i = 0; i < C::PV; ++i) *reinterpret_cast<u32x4*>(pl + i * C::RPP * C::LD) = sr.p[i];
  typename C::Op* ql = pl + C::BM * C::LD;
#pragma unroll
  for (int i = 0; i < C::QV; ++i) *reinterpret_cast<u32x4*>(ql + i * C::RPP * C::LD) = sr.q[i];
}

// Tile (ti, tj) of matrix mat for launch-linear tile index lin.  Workgroups
// are dealt round-robin to the 8 XCDs, so with gridDim % 8 == 0 a workgroup's
// tiles stay on one XCD; each XCD gets a contiguous range of tiles so the
// operand panels its concurrent tiles share meet in its L2.
template <class C, int EPI>
__device__ __forceinline__ void tile_coords(const GemmArgs& g, int64_t bid, int64_t& mat, int64_t& ti, int64_t& tj) {
  mat = bid / g.tiles_per_mat;
  const int64_t tt = bid % g.tiles_per_mat;
  if (EPI >= EPI_APPLY) {
    // grouped order: GM tile rows at a time, column by column, so the 32
    // tiles an XCD runs at once form a GM x (32 / GM) block that shares few
    // operand panels in its L2.  Groups of 8 rows when a matrix is at most
    // 32 tiles wide (2048 x 7168 and 4096^2 applies 1.3-2.2% faster), else 4
    // (8 rows: 8192 x 28672 apply 2.8% slower)
    const int64_t GM = g.tiles_n <= 32 ? 8 : 4;
    const int64_t tmm = g.tiles_per_mat / g.tiles_n;
    const int64_t first = (tt / (GM * g.tiles_n)) * GM;
    const int64_t rows = tmm - first < GM ? tmm - first : GM;
    const int64_t tin = tt - first * g.tiles_n;
    ti = first + tin % rows;
    tj = tin / rows;
  } else {
    if constexpr (C::BM == C::BN) tri_tile_grouped(tt, g.tiles_n, ti, tj);
    else tri_tile<C::BM / C::BN>(tt, ti, tj);
  }
}

// Row-major X tile of the apply products (BK rows of BN = 256 columns, bf16):
// 16-byte chunk c of row k sits in slot c ^ qn_swz(k), which spreads the 4
// rows one transposing read touches per 16-lane group over all 64 banks.
__device__ __forceinline__ int qn_swz(int k) { return 4 * (k & 3); }
__device__ __forceinline__ int qn_index(int row, int col) {
  return row * 256 + ((((col >> 3) ^ qn_swz(row))) << 3) + (col & 7);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 4-element reads of lanes i / 4 + 4 q, q = 0..3 (measured).
// With lane s reading row k0 + s / 4 at columns c0 + 4 (s % 4) .. + 3, lane i
// gets column c0 + i at rows k0 .. k0 + 3: a transposed 4 x 16 block.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(__attribute__((address_space(3))) bf16_t*)p);
}

// Slot swizzle of the direct-load LDS tiles: 16-byte chunk c of row r sits in
// slot c ^ swz(r).  LDS serves a 16-byte read for 16 lanes per cycle (64
// banks); the 16 rows an MFMA fragment read touches per cycle (two 128-byte
// rows per bank sweep) then hit 16 different bank groups.  (r & 7 would
// leave rows r and r + 8 on the same banks: SQ_LDS_BANK_CONFLICT counted
// 1.0e8 cycles on an 8192^3 product with it, none with this one.)
__device__ __forceinline__ int lds_swz(int r) { return (r >> 1) & 7; }

// A wave-uniform 64-bit value moved to scalar registers (the compiler
// computes uniform divisions in vector registers; these stay live across a
// tile's main loop).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  // readfirstlane returns int: each half goes through uint32_t (no sign extension)
  return (int64_t)((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u) |
                   ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32)) << 32));
}
template <typename T> __device__ __forceinline__ T* uniform_ptr(T* p) {
  return reinterpret_cast<T*>((uintptr_t)uniform64((int64_t)(uintptr_t)p));
}

// Waits (on this wave's counter) until at most n vector-memory operations
// are outstanding.
__device__ __forceinline__ constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// 16 bytes per lane from global memory (uniform base + per-lane 32-bit byte
// offset) straight into LDS at lds_addr + 16 lane.  Written as asm: the
// compiler neither waits on it nor recycles its address registers early
// (either would serialise the prefetch); the caller waits with vmcnt before
// the data is read.
// M0 is written here and nowhere else in these kernels (the generated code
// holds no other use of it), so clobbering the reserved register is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  // base and lds_addr are wave-uniform; make that visible to the compiler
  const uint64_t b = (uint64_t)(uintptr_t)base;
  // (readfirstlane returns int: go through uint32_t so the low half is not
  // sign-extended into the high half)
  const uint64_t sb = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b) |
                      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32);
  const uint32_t sl = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sb), "s"(sl) : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier without the release/acquire fences of __syncthreads,
// which would also wait for every outstanding global store and LDS-DMA load;
// the caller waits for what it needs.  This wave's LDS accesses complete
// first, and the compiler moves no memory access across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Spreads a block of N MFMAs with V vector-memory reads and D LDS reads in
// between (one MFMA, then the next share of each).
template <int N, int V, int D, int I = 0>
__device__ __forceinline__ void sched_mfma_block() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int v = V * (I + 1) / N - V * I / N;
    constexpr int d = D * (I + 1) / N - D * I / N;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
    if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);
    sched_mfma_block<N, V, D, I + 1>();
  }
}

// ROWS (last step only): W comes through a row table.  COMP (apply
// products, compensated mode): the second half of K multiplies B by the
// input's R (k-slices g.kswitch ..).
template <class C, int EPI, typename PT, bool ROWS = false, bool COMP = false>
__global__ void __launch_bounds__(C::THREADS, C::WAVES_PER_SIMD)
tl_gemm(GemmArgs g) {
  typedef typename C::Op OP;
  // epilogue staging: one 32 x SLD fp32 block per wave; with direct loads it
  // sits above stage 0, which receives the next tile's first k-slice meanwhile
  constexpr int SLD = 72;   // staging row stride (floats): conflict-free writes and reads
  constexpr int STG_ELEMS = C::WAVES * 32 * SLD * 4 / (int)sizeof(OP);
  constexpr int STG_OFF = C::DIRECT ? C::STAGE : 0;
  constexpr int LDS_ELEMS = 2 * C::STAGE > STG_OFF + STG_ELEMS ? 2 * C::STAGE : STG_OFF + STG_ELEMS;
  __shared__ __attribute__((aligned(16))) OP lds[LDS_ELEMS];
  // The apply products on direct-load tiles read X row-major (an NN
  // product): the Q stage holds BK rows of X, BN columns each, and the MFMA
  // operand comes out of it through transposing LDS reads.
  constexpr bool QN = C::DIRECT && EPI >= EPI_APPLY;
  static_assert(!QN || (C::BK == 64 && C::BN == 256 && C::WAVES == 8), "row-major X operand: 64 x 256 Q stage");

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int wm = w / C::WAVES_N, wn = w % C::WAVES_N;
  // Persistent: each workgroup runs tiles until none are left; a tile's
  // epilogue stores drain while the next tile's main loop runs.  Tiles are
  // numbered so that XCD x (workgroups b with b % 8 == x, dealt round-robin)
  // has the contiguous range x total/8 .. and its concurrent tiles share
  // operand panels in its L2 (tile_coords' order).
  //  - static: workgroup b takes launch-linear tiles b, b + gridDim, ...
  //  - dynamic (Gram and poly on direct-load tiles, given counters: their
  //    triangles leave partial last rounds, and diagonal tiles, which load
  //    half the operands, run faster): workgroup b takes the next
  //    untaken tile of its XCD's range, then of the other ranges.  A workgroup
  //    that starts late (its CU still busy with another stream's kernel)
  //    takes fewer tiles instead of finishing last.  Wave 0 takes the next
  //    tile while the current one starts; the other threads read it from LDS
  //    after a k-slice barrier before the last slice.  Each tile is computed
  //    exactly as in the static order.
  const int64_t total = g.tiles_total;
  const bool xcd_map = (total & 7) == 0 && (gridDim.x & 7) == 0;
  const bool dyn = C::DIRECT && EPI < EPI_APPLY && g.sched != nullptr && xcd_map;
  __shared__ int64_t next_slot[2];
  auto static_tile = [&](int64_t l) -> int64_t {
    return l < total ? (xcd_map ? (l & 7) * (total >> 3) + (l >> 3) : l) : -1;
  };
  // Taking a tile: lane 0 of wave 0 adds 1 to its XCD's counter (own_try,
  // issued at the start of a tile, its result first used later); wave 0 then
  // resolves it (take_resolve): the tile own_try names, or, once its own
  // range is empty, another range's.  For that, lanes 0..7 read all counters
  // at once and lane 0 tries the first range with tiles left; a failed try
  // leaves that counter past its range, so at most 8 tries fail.  -1: every
  // range is exhausted.
  const int64_t per_range = total >> 3;
  const int home = blockIdx.x & 7;
  auto own_try = [&]() -> unsigned {
    return __hip_atomic_fetch_add(g.sched + home, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto take_resolve = [&](unsigned first) -> int64_t {
    const int64_t per = per_range;
    const int x = home;
    int64_t got = (lane == 0 && (int64_t)first < per) ? x * per + (int64_t)first : -1;
    got = __shfl(got, 0, 64);
    while (got < 0) {
      unsigned c = (unsigned)per;
      if (lane < 8) c = __hip_atomic_load(g.sched + ((x + lane) & 7), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned long long open = __ballot(lane < 8 && (int64_t)c < per);
      if (open == 0ull) break;
      const int xr = (x + __ffsll(open) - 1) & 7;
      if (lane == 0) {
        const unsigned i = __hip_atomic_fetch_add(g.sched + xr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int64_t)i < per) got = xr * per + (int64_t)i;
      }
      got = __shfl(got, 0, 64);
    }
    return got;
  };

  // direct loads: instruction i of this wave fills rows (w + i WAVES) RPI ..
  // + RPI - 1 of the stage (P's rows first, then Q's); the lane's byte offset
  // within its operand is the same for every instruction of that operand up
  // to a uniform multiple of WAVES RPI rows, which goes into the scalar base
  [[maybe_unused]] uint32_t voff_p = 0, voff_q = 0;
  if constexpr (C::DIRECT) {
    const int lrow = lane / C::VPR;
    // the lane's stage row is 8 (w + WAVES i) + lrow; its swizzle does not
    // depend on i
    const int lchunk = (lane % C::VPR) ^ lds_swz(8 * w + lrow);
    const int row = w * C::RPI + lrow;
    voff_p = (uint32_t)((row * g.ldp + lchunk * C::EPV) * (int64_t)sizeof(OP));
    if constexpr (QN) {
      // row-major X tile: one instruction fills 2 rows of BN columns; chunk
      // c of row k sits in slot c ^ qn_swz(k)
      const int qrow = 2 * w + lane / 32;
      voff_q = (uint32_t)((qrow * g.ldq + ((lane % 32) ^ qn_swz(qrow)) * C::EPV) * (int64_t)sizeof(OP));
    } else {
      voff_q = (uint32_t)((row * g.ldq + lchunk * C::EPV) * (int64_t)sizeof(OP));
    }
  }
  // direct loads of k-slice k0 of the tile whose operands start at pbase
  // (its first row) and qbase (first row, or first column when QN) into
  // stage st: this wave's instructions i0 .. i1 - 1 of LPW, the first half
  // in P's rows, the second in Q's
  // (qskip: P's rows only; Q's would repeat them)
  constexpr int HALF = C::LPW / 2;
  [[maybe_unused]] auto dma_slice = [&](int st, const OP* pbase, const OP* qbase, int64_t k0, bool qskip, int i0,
                                        int i1) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      if (i < i0 || i >= i1 || (i >= HALF && qskip)) continue;
      const int ins = w + i * C::WAVES;
      const int64_t rows = (int64_t)(i % HALF) * C::WAVES * C::RPI;
      const OP* src;
      int lofs;
      if (i < HALF) {
        src = pbase + rows * g.ldp + k0;
        lofs = ins * C::RPI * C::LD;
      } else if constexpr (QN) {   // k rows k0 + 16 (i - HALF) + 2 w + lane / 32
        const int qi = w + (i - HALF) * C::WAVES;
        src = qbase + (k0 + 16 * (i - HALF)) * g.ldq;
        lofs = C::BM * C::LD + qi * 2 * C::BN;
      } else {
        src = qbase + rows * g.ldq + k0;
        lofs = ins * C::RPI * C::LD;
      }
      const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) OP*)(lds + st * C::STAGE + lofs);
      lds_dma16(src, i < HALF ? voff_p : voff_q, la);
    }
  };
  bool stage0_ready = false;   // direct loads: stage 0 already holds this tile's first k-slice

  int64_t bid;
  if (dyn) {
    if (w == 0) {
      const int64_t first = take_resolve(lane == 0 ? own_try() : 0u);
      if (lane == 0) next_slot[0] = first;
    }
    __syncthreads();
    bid = next_slot[0];
  } else {
    bid = static_tile(blockIdx.x);
  }
  int64_t lin = blockIdx.x;
  int par = 0;   // next_slot[par ^ 1] receives the tile after this one
  while (bid >= 0) {
  int64_t mat, ti, tj;
  tile_coords<C, EPI>(g, bid, mat, ti, tj);
  int64_t nbid = dyn ? -1 : static_tile(lin + gridDim.x);
  [[maybe_unused]] unsigned tried = 0u;
  if (dyn && w == 0 && lane == 0) tried = own_try();
  mat = uniform64(mat); ti = uniform64(ti); tj = uniform64(tj);
  const int64_t i0 = ti * C::BM, j0 = tj * C::BN;

  f32x16 acc[C::IB][C::JB];
#pragma unroll
  for (int a = 0; a < C::IB; ++a)
#pragma unroll
    for (int b = 0; b < C::JB; ++b) acc[a][b] = f32x16{};
  const int64_t KT = g.K / C::BK;

  // a X term of the apply products: the Q stage holds X^T[j][k] = X[k][j]
  // for this k-slice; when the slice covers rows of this wave's output, add
  // a X[i][j] from LDS to the accumulators (no global read in the epilogue).
  // With the master, a R comes in the epilogue, or, compensated, from the
  // R slices of the second half of K (the caller passes their k).  The poly
  // product reads the same way: its Q stage holds A[j][k] = A[k][j], and
  // without an fp32 A (A32 null) it adds (b / c) A[i][j] here, the epilogue
  // scaling the sum by c.
  auto add_ax = [&](const OP* Qs, int64_t kt) {
    if constexpr (EPI >= EPI_APPLY || EPI == EPI_POLY) {
      if (EPI != EPI_POLY || g.A32 == nullptr) {
        const int64_t krel = kt * C::BK - (i0 + wm * C::WTM);
        if (krel > -C::BK && krel < C::WTM) {
#pragma unroll
          for (int ib = 0; ib < C::IB; ++ib) {
            const int off = ib * 32 - (int)krel;   // block row 0 relative to the slice
            if (off < 0 || off >= C::BK) continue;
            if constexpr (QN) {
              // Qs: the stage's row-major X rows; element (row, column) of
              // accumulator register r of this lane
#pragma unroll
              for (int jb = 0; jb < C::JB; ++jb) {
                const int col = wn * C::WTN + jb * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const int row = off + mfma32_row(lane, r);
                  const float xv = __uint_as_float((uint32_t)Qs[qn_index(row, col)] << 16);
                  acc[ib][jb][r] += g.ca * xv;
                }
              }
              continue;
            }
#pragma unroll
            for (int jb = 0; jb < C::JB; ++jb) {
              const OP* xrow = Qs + jb * 32 * C::LD;
#pragma unroll
              for (int qd = 0; qd < 4; ++qd) {
                // elements off + 8 qd + 4 (lane / 32) .. + 3 of the lane's row
                const int chunk = (off + 8 * qd) / C::EPV;
                const int within = (off + 8 * qd) % C::EPV + 4 * (lane >> 5);
                const int slot = C::DIRECT ? (chunk ^ lds_swz(lane & 31)) : chunk;
                const OP* xq = xrow + slot * C::EPV + within;
                float xv[4];
                if constexpr (sizeof(OP) == 2) {
                  const uint2 u = *reinterpret_cast<const uint2*>(xq);
                  xv[0] = __uint_as_float(u.x << 16);
                  xv[1] = __uint_as_float(u.x & 0xffff0000u);
                  xv[2] = __uint_as_float(u.y << 16);
                  xv[3] = __uint_as_float(u.y & 0xffff0000u);
                } else {
                  const f32x4 u = *reinterpret_cast<const f32x4*>(xq);
#pragma unroll
                  for (int e = 0; e < 4; ++e) xv[e] = u[e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[ib][jb][4 * qd + e] += g.ca * xv[e];
              }
            }
          }
        }
      }
    }
  };

  if constexpr (C::DIRECT) {
    // Two LDS stages; k-slice kt + 1 is loaded (direct) while slice kt is
    // multiplied, its loads and the fragment reads spread among the MFMAs.
    // The last slice of a tile loads the next tile's first slice instead, so
    // a tile starts without waiting for the previous epilogue's stores.
    // K is a multiple of 2 BK: slice kt uses stage kt & 1.
    // The Gram and poly products multiply a matrix by its own transpose: on
    // a diagonal tile the Q stage would repeat the P stage, so only P's rows
    // are loaded and Q's fragments are read from them (dq; ndq for the next
    // tile, whose first slice the last slice loads).
    const bool same_pq = (EPI == EPI_GRAM || EPI == EPI_POLY) && C::BM == C::BN && g.P == g.Q &&
                         g.ldp == g.ldq && g.strideP == g.strideQ;
    const bool dq = same_pq && ti == tj;
    bool ndq = false;
    const OP* pb = reinterpret_cast<const OP*>(g.P) + mat * g.strideP + i0 * g.ldp;
    const OP* qb = reinterpret_cast<const OP*>(g.Q) + mat * g.strideQ + (QN ? j0 : j0 * g.ldq);
    // compensated apply: the second half of K reads the input's R, which
    // has Q's layout, so its slices sit dq2 elements from X~'s (both lie in
    // the workspace; an offset rather than a second pointer keeps the
    // compiler from spilling the loop)
    const int64_t ksw = COMP && EPI >= EPI_APPLY ? g.kswitch : 0;
    const int64_t dq2 = ksw > 0 ? (reinterpret_cast<const OP*>(g.Q2) - reinterpret_cast<const OP*>(g.Q)) : 0;
    const OP* npb = pb;
    const OP* nqb = qb;
    // operands of the next tile, whose first slice the last slice loads
    auto set_next = [&](int64_t nb) {
      nbid = nb;
      if (nb >= 0) {
        int64_t nmat, nti, ntj;
        tile_coords<C, EPI>(g, nb, nmat, nti, ntj);
        ndq = same_pq && nti == ntj;
        npb = reinterpret_cast<const OP*>(g.P) + nmat * g.strideP + nti * C::BM * g.ldp;
        nqb = reinterpret_cast<const OP*>(g.Q) + nmat * g.strideQ + (QN ? ntj * C::BN : ntj * C::BN * g.ldq);
      }
      npb = uniform_ptr(npb);
      nqb = uniform_ptr(nqb);
    };
    if (!dyn) set_next(nbid);
    if (!stage0_ready) {
      dma_slice(0, pb, qb, 0, dq, 0, C::LPW);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
    }
    bf16x8 fa[2][C::IB], fb[2][C::JB];
    const OP* Pw = lds + (wm * C::WTM + (lane & 31)) * C::LD;
    const int qrow0 = dq ? 0 : C::BM;   // first stage row of the Q operand
    const OP* Qw = lds + (qrow0 + wn * C::WTN + (lane & 31)) * C::LD;
    auto read_frags = [&](int buf, int st, int kk) {
      const int slot = (2 * kk + (lane >> 5)) ^ lds_swz(lane & 31);
#pragma unroll
      for (int ib = 0; ib < C::IB; ++ib)
        fa[buf][ib] = *reinterpret_cast<const bf16x8*>(Pw + st * C::STAGE + ib * 32 * C::LD + slot * 8);
      if constexpr (QN) {
        // 16-lane group G, lane s: two transposing reads give k = 16 kk +
        // 8 (G / 2) + 0..7 of column 16 (G % 2) + s of the block
        const int G = lane >> 4, s4 = lane & 15;
#pragma unroll
        for (int jb = 0; jb < C::JB; ++jb) {
          bf16x4 h[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int row = 16 * kk + 8 * (G >> 1) + 4 * hh + (s4 >> 2);
            const int col = wn * C::WTN + jb * 32 + 16 * (G & 1) + 4 * (s4 & 3);
            h[hh] = lds_read_tr16(lds + st * C::STAGE + C::BM * C::LD + qn_index(row, col));
          }
          fb[buf][jb] = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
      } else {
#pragma unroll
        for (int jb = 0; jb < C::JB; ++jb)
          fb[buf][jb] = *reinterpret_cast<const bf16x8*>(Qw + st * C::STAGE + jb * 32 * C::LD + slot * 8);
      }
    };
    auto mfmas = [&](int buf) {
#pragma unroll
      for (int ib = 0; ib < C::IB; ++ib)
#pragma unroll
        for (int jb = 0; jb < C::JB; ++jb)
          acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][ib], fb[buf][jb], acc[ib][jb], 0, 0, 0);
    };
    read_frags(0, 0, 0);
    // slice whose barrier publishes the next tile (dynamic order): late
    // enough that thread 0's atomic has returned, before the last slice
    const int64_t kpub = KT >= 8 ? 4 : 0;
    // The next slice's loads are split between the first two MFMA steps:
    // P's rows as one burst at the head of the first step, Q's at the head
    // of the second (the loads are inline asm, which the scheduling hints
    // leave in place).  All of them at the head of the first step queue
    // behind each other in the load path and arrive later (every product
    // 2.5-4% slower); one instruction at a time between the MFMAs, or the
    // step's fragment reads issued before its burst, is slower still.
    auto slice = [&](int st, int64_t kt) {
      const bool last = kt + 1 == KT;
      const bool sw = ksw > 0 && kt + 1 >= ksw;   // the next slice is one of R's
      const OP* lp = last ? npb : pb;
      const int64_t kb = sw ? ksw : 0;
      const OP* lq = last ? nqb : qb + (sw ? dq2 : 0);
      const int64_t lk = last ? 0 : (kt + 1 - kb) * C::BK;
      const bool lskip = last ? ndq : dq;
      dma_slice(st ^ 1, lp, lq, lk, lskip, 0, HALF);
      read_frags(1, st, 1);
      mfmas(0);
      sched_mfma_block<C::IB * C::JB, HALF, C::IB + C::JB>();
      __builtin_amdgcn_sched_barrier(0);
      dma_slice(st ^ 1, lp, lq, lk, lskip, HALF, C::LPW);
      read_frags(0, st, 2);
      mfmas(1);
      sched_mfma_block<C::IB * C::JB, C::LPW - HALF, C::IB + C::JB>();
      __builtin_amdgcn_sched_barrier(0);
      read_frags(1, st, 3);
      mfmas(0);
      sched_mfma_block<C::IB * C::JB, 0, C::IB + C::JB>();
      __builtin_amdgcn_sched_barrier(0);
      mfmas(1);
      __builtin_amdgcn_sched_barrier(0);
      const int64_t ke = ksw > 0 && kt >= ksw ? kt - ksw : kt;   // k-slice within its half
      if constexpr (QN) add_ax(lds + st * C::STAGE + C::BM * C::LD, ke);
      else add_ax(lds + st * C::STAGE + (qrow0 + wn * C::WTN + (lane & 31)) * C::LD, ke);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this wave's loads of the next slice
      if (dyn && kt == kpub && w == 0) {
        const int64_t nb = take_resolve(tried);
        if (lane == 0) next_slot[par ^ 1] = nb;
      }
      lds_barrier();                               // everyone's; stage st is free again
      if (!last) read_frags(0, st ^ 1, 0);
    };
    for (int64_t kt = 0; kt < KT; kt += 2) {
      slice(0, kt);
      if (dyn && kt == kpub) set_next(next_slot[par ^ 1]);
      slice(1, kt + 1);
    }
    stage0_ready = nbid >= 0;
  } else {
  const int r0 = t / C::VPR, cv = (t % C::VPR) * C::EPV;
  const OP* Pp = reinterpret_cast<const OP*>(g.P) + mat * g.strideP + (i0 + r0) * g.ldp + cv;
  const OP* Qp = reinterpret_cast<const OP*>(g.Q) + mat * g.strideQ + (j0 + r0) * g.ldq + cv;
  const int64_t pstep = (int64_t)C::RPP * g.ldp, qstep = (int64_t)C::RPP * g.ldq;
  // compensated apply: the second half of K reads the input's R instead
  const int64_t ksw = COMP && EPI >= EPI_APPLY ? g.kswitch : 0;
  const OP* Qp2 = ksw > 0 ? reinterpret_cast<const OP*>(g.Q2) + mat * g.strideQ + (j0 + r0) * g.ldq + cv : Qp;

  StageRegs<C> sr;
  stage_load<C>(sr, Pp, Qp, pstep, qstep, 0);
  stage_store<C>(sr, lds + r0 * C::LD + cv);
  __syncthreads();
  for (int64_t kt = 0; kt < KT; ++kt) {
    const int st = (int)(kt & 1);
    if (kt + 1 < KT) {
      const bool sw = ksw > 0 && kt + 1 >= ksw;
      stage_load<C>(sr, Pp, sw ? Qp2 : Qp, pstep, qstep, (kt + 1 - (sw ? ksw : 0)) * C::BK);
    }
    const OP* Ps = lds + st * C::STAGE + (wm * C::WTM + (lane & 31)) * C::LD;
    const OP* Qs = lds + st * C::STAGE + (C::BM + wn * C::WTN + (lane & 31)) * C::LD;
    if constexpr (sizeof(OP) == 2) {
#pragma unroll
      for (int kk = 0; kk < C::BK / 16; ++kk) {
        bf16x8 av[C::IB], bv[C::JB];
#pragma unroll
        for (int ib = 0; ib < C::IB; ++ib)
          av[ib] = *reinterpret_cast<const bf16x8*>(Ps + ib * 32 * C::LD + kk * 16 + (lane >> 5) * 8);
#pragma unroll
        for (int jb = 0; jb < C::JB; ++jb)
          bv[jb] = *reinterpret_cast<const bf16x8*>(Qs + jb * 32 * C::LD + kk * 16 + (lane >> 5) * 8);
#pragma unroll
        for (int ib = 0; ib < C::IB; ++ib)
#pragma unroll
          for (int jb = 0; jb < C::JB; ++jb)
            acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ib], bv[jb], acc[ib][jb], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < C::BK / 2; ++kk) {
        float av[C::IB], bv[C::JB];
#pragma unroll
        for (int ib = 0; ib < C::IB; ++ib) av[ib] = Ps[ib * 32 * C::LD + kk * 2 + (lane >> 5)];
#pragma unroll
        for (int jb = 0; jb < C::JB; ++jb) bv[jb] = Qs[jb * 32 * C::LD + kk * 2 + (lane >> 5)];
#pragma unroll
        for (int ib = 0; ib < C::IB; ++ib)
#pragma unroll
          for (int jb = 0; jb < C::JB; ++jb)
            acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[ib], bv[jb], acc[ib][jb], 0, 0, 0);
      }
    }
    add_ax(Qs, ksw > 0 && kt >= ksw ? kt - ksw : kt);
    if (kt + 1 < KT) stage_store<C>(sr, lds + (st ^ 1) * C::STAGE + r0 * C::LD + cv);
    __syncthreads();
  }
  }

  // ---- epilogues -------------------------------------------------------------
  // Each wave stages one 32 x 64 block row of its sub-tile in its own LDS
  // region per round (the last main-loop barrier has retired every read of
  // the operand stages, so wave-level ordering suffices from here on); lane l
  // then owns column l of that block: row-major outputs are written 64 lanes
  // wide (coalesced) and transposed outputs as 16-byte vectors along the
  // lane's own 32 contiguous elements.  All global reads of a round are
  // issued before any of its stores, so their latencies overlap.  Offsets
  // inside one padded matrix fit in 32 bits (the planner caps a padded matrix
  // at 2^31 elements).
  static_assert(C::JB % 2 == 0, "epilogue stages 64-column blocks");
  float* stg = reinterpret_cast<float*>(lds + STG_OFF) + w * (32 * SLD);
  const bool diag = (EPI < EPI_APPLY) && (tj >= (C::BM / C::BN) * ti);   // inside the diagonal block
#pragma clang loop unroll(full)
  for (int rb = 0; rb < C::IB * C::JB / 2; ++rb) {
    const int ib = rb / (C::JB / 2), jp = rb % (C::JB / 2);
    const uint32_t jj = (uint32_t)(j0 + wn * C::WTN + jp * 64 + lane);
    if (rb > 0) wave_sync();   // this wave's reads of the previous round are done
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        stg[mfma32_row(lane, r) * SLD + jb * 32 + (lane & 31)] = acc[ib][2 * jp + jb][r];
    wave_sync();
    if constexpr (C::DIRECT && (EPI == EPI_APPLY || EPI == EPI_LAST_T)) {
      // the master (R row-major): a R joins the staged block, read by rows,
      // 8 columns per lane, so the four 16-byte loads of a lane are in flight
      // together (the column layout below would need 32 2-byte loads)
      if (g.Rin) {
        const bf16_t* Ri = g.Rin + mat * g.strideX;
        const int rr = lane >> 3, cc = (lane & 7) * 8;
        const uint32_t rw = (uint32_t)(i0 + wm * C::WTM + ib * 32 + rr);
        const uint32_t cw = (uint32_t)(j0 + wn * C::WTN + jp * 64 + cc);
        u32x4 raw[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
          raw[p] = *reinterpret_cast<const u32x4*>(at32(Ri, (rw + 8 * p) * (uint32_t)g.ldx + cw));
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          float* srow = stg + (rr + 8 * p) * SLD + cc;
          f32x4 lo = *reinterpret_cast<const f32x4*>(srow), hi = *reinterpret_cast<const f32x4*>(srow + 4);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            lo[2 * e] += g.ca * __uint_as_float(raw[p][e] << 16);
            lo[2 * e + 1] += g.ca * __uint_as_float(raw[p][e] & 0xffff0000u);
            hi[2 * e] += g.ca * __uint_as_float(raw[p][e + 2] << 16);
            hi[2 * e + 1] += g.ca * __uint_as_float(raw[p][e + 2] & 0xffff0000u);
          }
          *reinterpret_cast<f32x4*>(srow) = lo;
          *reinterpret_cast<f32x4*>(srow + 4) = hi;
        }
        wave_sync();
      }
    }
    float o[32];
    if constexpr (EPI != EPI_LAST) {   // lane l: column l of the block, 32 rows
#pragma unroll
      for (int q = 0; q < 32; ++q) o[q] = stg[q * SLD + lane];
    }
    const uint32_t ib0 = (uint32_t)(i0 + wm * C::WTM + ib * 32);
    if constexpr (EPI == EPI_GRAM) {
      if (g.inv0) {   // A = inv^2 U U^T
        const float sc = g.inv0[mat] * g.inv0[mat];
#pragma unroll
        for (int q = 0; q < 32; ++q) o[q] *= sc;
      }
      const uint32_t ld = (uint32_t)g.lda;
      // the fp32 copy feeds the poly epilogue (lower-triangle tiles only),
      // except on the fp32 path where it is also the full product operand;
      // none when the poly takes b A from its bf16 operand tiles
      if (g.A32) {
        float* A32 = g.A32 + mat * g.strideA;
#pragma unroll
        for (int q = 0; q < 32; ++q) A32[(ib0 + q) * ld + jj] = o[q];
        if (!diag && !g.A16) store_run32(A32 + jj * ld + ib0, o);
      }
      if (g.A16) {
        bf16_t* A16 = g.A16 + mat * g.strideA;
#pragma unroll
        for (int q = 0; q < 32; ++q) A16[(ib0 + q) * ld + jj] = f2bf(o[q]);
        if (!diag) store_run32(A16 + jj * ld + ib0, o);
      }
    } else if constexpr (EPI == EPI_POLY) {
      const uint32_t ld = (uint32_t)g.lda;
      OP* PB = reinterpret_cast<OP*>(g.PB) + mat * g.strideA;
      if (g.A32) {
        const float* A32 = g.A32 + mat * g.strideA;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float av[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) av[q] = A32[(ib0 + 16 * hh + q) * ld + jj];
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            o[16 * hh + q] = g.cb * av[q] + g.cc * o[16 * hh + q];
            st_from_f32(PB, (ib0 + 16 * hh + q) * ld + jj, o[16 * hh + q]);
          }
        }
      } else {   // the accumulators hold A A + (b / c) A
#pragma unroll
        for (int q = 0; q < 32; ++q) {
          o[q] *= g.cc;
          st_from_f32(PB, (ib0 + q) * ld + jj, o[q]);
        }
      }
      if (!diag) store_run32(PB + jj * ld + ib0, o);
    } else if constexpr (EPI == EPI_APPLY) {
      const uint32_t ldx = (uint32_t)g.ldx;
      OP* X = reinterpret_cast<OP*>(g.X) + mat * g.strideX;
      // a X~ is in the accumulators (compensated: a R and B R too); with the
      // master, a R is added here.  First step: X' = inv (a U + B U).
      const float sc = g.inv0 ? g.inv0[mat] : 1.f;
      if constexpr (QN) {
        // R row-major, like X (a R came in with the staged block).  By rows
        // of the staged block, 8 columns per lane: X' and R' leave as one
        // 16-byte store per 8 rows each (not 32 two-byte stores)
        bf16_t* Ro = g.Rout ? g.Rout + mat * g.strideX : nullptr;
        const int rr = lane >> 3, cc = (lane & 7) * 8;
        const uint32_t col = (uint32_t)(j0 + wn * C::WTN + jp * 64 + cc);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float* srow = stg + (rr + 8 * p) * SLD + cc;
          const f32x4 lo = *reinterpret_cast<const f32x4*>(srow), hi = *reinterpret_cast<const f32x4*>(srow + 4);
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) { v[e] = sc * lo[e]; v[e + 4] = sc * hi[e]; }
          const uint32_t idx = (ib0 + rr + 8 * p) * ldx + col;
          store8(at32(X, idx), v);
          if (Ro) store_res8(at32(Ro, idx), v);
        }
      } else {
        // the next apply reads X^T; R sits as X^T too, so the lane's 32 rows
        // of it are 32 contiguous elements
        const uint32_t tofs = jj * (uint32_t)g.ldxt + ib0;
        if (g.Rin) {
          float rv[32];
          load_run32(g.Rin + mat * g.strideX + tofs, rv);
#pragma unroll
          for (int q = 0; q < 32; ++q) o[q] += g.ca * rv[q];
        }
#pragma unroll
        for (int q = 0; q < 32; ++q) {
          o[q] *= sc;
          st_from_f32(X, (ib0 + q) * ldx + jj, o[q]);
        }
        store_run32(reinterpret_cast<OP*>(g.XT) + mat * g.strideX + tofs, o);
        if (g.Rout) {
          float r[32];
#pragma unroll
          for (int q = 0; q < 32; ++q) r[q] = bf_res(o[q]);
          store_run32(g.Rout + mat * g.strideX + tofs, r);
        }
      }
    } else {
      float ulr = g.lr, uwd = g.wd;
      update_scalars(g.lrwd, ulr, uwd);
      const uint32_t ldx = (uint32_t)g.ldx;
      const bf16_t* Ri = g.Rin ? g.Rin + mat * g.strideX : nullptr;   // the master: a R joins a X~
      PT* W = batch_view(reinterpret_cast<PT*>(g.param), g.tabs.param, mat, g.m * g.n);
      float* O = batch_view(g.ns_out, g.tabs.ns, mat, g.m * g.n);
      if (W) W += mat * g.m * g.n;
      if (O) O += mat * g.m * g.n;
      const uint32_t m = (uint32_t)g.m, n = (uint32_t)g.n;
      // W's stored element (row sr, column sc), rows of ncols elements: from
      // the row table when W is given row by row
      const bool has_w = ROWS || W != nullptr;
      auto w_at = [&](uint32_t sr, uint32_t sc, uint32_t ncols) -> PT* {
        if constexpr (ROWS) return row_of<PT>(g.tabs.param_rows, mat, EPI == EPI_LAST_T ? g.n : g.m, sr) + sc;
        else return W + sr * ncols + sc;
      };
      if constexpr (EPI == EPI_LAST) {
        // W row-major: the lane takes 8 consecutive columns of rows rr, rr + 8,
        // rr + 16, rr + 24 of the staged block, so W, the master's R and O move
        // as 16-byte vectors (8 lanes per 128-byte row segment), and all reads
        // of the round are issued before its stores.
        const int rr = lane >> 3, cc = (lane & 7) * 8;
        const uint32_t j = (uint32_t)(j0 + wn * C::WTN + jp * 64 + cc);
        const bool vec = (n % 8) == 0;   // aligned runs of 8 inside the matrix
        // The reads of W for all four row groups are issued before any store
        // of the round (the stores could alias the reads, so the compiler would
        // otherwise wait out one memory latency per row group); W stays in its
        // stored form until used (4 registers per group for bf16).
        Raw8<PT> wr[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t i = ib0 + rr + 8 * p;
          if (has_w && vec && i < m && j < n) wr[p].load(w_at(i, j, n));
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          float xv[8];
          if (Ri) {   // padded rows and columns: always readable
            if constexpr (C::DIRECT) {
              load8(at32(Ri, (ib0 + rr + 8 * p) * ldx + j), xv);
            } else {   // R as X^T
#pragma unroll
              for (int q = 0; q < 8; ++q) xv[q] = bf2f(Ri[(j + q) * (uint32_t)g.ldxt + ib0 + rr + 8 * p]);
            }
          }
          float ov[8];
          const f32x4 a = *reinterpret_cast<const f32x4*>(stg + (rr + 8 * p) * SLD + cc);
          const f32x4 b = *reinterpret_cast<const f32x4*>(stg + (rr + 8 * p) * SLD + cc + 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) { ov[q] = a[q]; ov[q + 4] = b[q]; }
          const uint32_t i = ib0 + rr + 8 * p;
          if (Ri) {
#pragma unroll
            for (int q = 0; q < 8; ++q) ov[q] = g.ca * xv[q] + ov[q];
          }
          if (g.inv0) {   // K = 1: X held U unscaled
            const float sc = g.inv0[mat];
#pragma unroll
            for (int q = 0; q < 8; ++q) ov[q] *= sc;
          }
          if (i >= m) continue;
          if (vec) {
            if (j >= n) continue;
            if (O) store8(O + i * n + j, ov);
            if (has_w) {
              float wv[8], nw[8];
              wr[p].to_f32(wv);
#pragma unroll
              for (int q = 0; q < 8; ++q) nw[q] = apply_update(wv[q], ov[q], ulr, uwd, g.s);
              store8(w_at(i, j, n), nw);
            }
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              if (j + q >= n) break;
              if (O) O[i * n + j + q] = ov[q];
              if (has_w) {
                PT* wp = w_at(i, j + q, n);
                st_from_f32(wp, 0, apply_update(ld_as_f32(wp, 0), ov[q], ulr, uwd, g.s));
              }
            }
          }
        }
      } else if (C::DIRECT && ib0 + 32 <= m && (m % 8) == 0) {
        // W is the transpose, its row j holding this block's column j: by W
        // rows, 8 elements per lane, four lanes per 32-element row piece and
        // 16 rows per round, so each access instruction covers 16 pieces of
        // 64 bytes (a lane per row would touch 64 rows with 16 bytes each);
        // the W reads of all four rounds go before their stores
        const float sc = g.inv0 ? g.inv0[mat] : 1.f;   // K = 1: X held U unscaled
        const int sub = lane & 3, jr = lane >> 2;
        const uint32_t jb = (uint32_t)(j0 + wn * C::WTN + jp * 64 + jr);
        Raw8<PT> wr[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
          if (has_w && jb + 16 * p < n) wr[p].load(w_at(jb + 16 * p, ib0 + 8 * sub, m));
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t j = jb + 16 * p;
          if (j >= n) continue;
          float ov[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) ov[q] = sc * stg[(8 * sub + q) * SLD + 16 * p + jr];
          if (O) store8(O + j * m + ib0 + 8 * sub, ov);
          if (has_w) {
            float wv[8], nw[8];
            wr[p].to_f32(wv);
#pragma unroll
            for (int q = 0; q < 8; ++q) nw[q] = apply_update(wv[q], ov[q], ulr, uwd, g.s);
            store8(w_at(j, ib0 + 8 * sub, m), nw);
          }
        }
      } else {
        if (jj < n) {
          if constexpr (!C::DIRECT) {   // (direct loads: a R came in with the staged block)
            if (Ri) {   // R as X^T: the lane's 32 rows are contiguous
              float rv[32];
              load_run32(Ri + jj * (uint32_t)g.ldxt + ib0, rv);
#pragma unroll
              for (int q = 0; q < 32; ++q) o[q] = g.ca * rv[q] + o[q];
            }
          }
          if (g.inv0) {   // K = 1: X held U unscaled
            const float sc = g.inv0[mat];
#pragma unroll
            for (int q = 0; q < 32; ++q) o[q] *= sc;
          }
          if (ib0 + 32 <= m && (m % 8) == 0) {
            // W is the transpose: this lane's 32 elements are contiguous and 16-byte aligned
            const uint32_t base = jj * m + ib0;
            if (O) store_run32(O + base, o);
            if (has_w) update_run32(w_at(jj, ib0, m), o, ulr, uwd, g.s);
          } else {
            for (uint32_t q = 0; q < 32 && ib0 + q < m; ++q) {
              const uint32_t si = jj * m + ib0 + q;
              if (O) O[si] = o[q];
              if (has_w) {
                PT* wp = w_at(jj, ib0 + q, m);
                st_from_f32(wp, 0, apply_update(ld_as_f32(wp, 0), o[q], ulr, uwd, g.s));
              }
            }
          }
        }
      }
    }
  }
  // every wave is done with its staging region before the next tile's
  // loads land there (no wait for this tile's stores)
  if constexpr (C::DIRECT) lds_barrier();
  else __syncthreads();
  lin += gridDim.x;
  par ^= 1;
  bid = nbid;
  }  // tiles
}

template <typename PT>
__global__ void __launch_bounds__(256)
tl_update(PT* __restrict__ W, const float* __restrict__ O, int64_t total, float lr, float wd, float s,
          const float* __restrict__ lrwd) {
  update_scalars(lrwd, lr, wd);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
    st_from_f32(W, i, apply_update(ld_as_f32(W, i), O[i], lr, wd, s));
}

// ---------------------------------------------------------------------------
// Persistent grid of tl_gemm<C, EPI, PT>: one wave of resident workgroups
// (a multiple of 8, so each stays on one XCD), or fewer if there are fewer
// tiles.
template <class C, int EPI, typename PT, bool ROWS = false, bool COMP = false>
unsigned gemm_grid(int64_t tiles) {
  static std::atomic<int> per_dev[kMaxDevices];   // resident workgroups of this kernel per device
  const int64_t slots = per_device_cached(per_dev, [](int dev) {
    int cus = 0, blocks = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, tl_gemm<C, EPI, PT, ROWS, COMP>, C::THREADS, 0) != hipSuccess ||
        blocks <= 0)
      blocks = 1;
    return cus * blocks;
  });
  return (unsigned)(tiles < slots ? tiles : slots);
}

// The K Newton-Schulz steps as three NT products each, on tile config C.
// X: the step's input X (row-major).  Direct-load tiles: X1 is the second
// row-major buffer, the apply reads X row-major and writes the next X to
// the other buffer.  Otherwise XT holds X^T (ping-pong) and X is updated in
// place.
// R (the master, else null): the residues bf16(X - bf16(X)) of step k's
// input in R[k & 1] and of its output in R[(k + 1) & 1], in the layout in
// which the apply reads X.  comp: the apply also multiplies B by the input's
// R (one launch over K = 2 m).
template <class C, typename PT>
hipError_t run_products_cfg(const StepArgs& a, const BatchShape& sh, typename C::Op* X, typename C::Op* X1,
                            typename C::Op* XT[2], bf16_t* const* R, bool comp, float* A32, bf16_t* A16,
                            typename C::Op* PB, int64_t mp, int64_t np, const float* inv, unsigned* sched) {
  typedef typename C::Op OP;
  hipError_t e;
  if (C::DIRECT ? X1 == nullptr : (XT[0] == nullptr || XT[1] == nullptr)) return hipErrorInvalidValue;
  OP* Xb[2] = {X, X1};
  const int64_t tm = mp / C::BM, tn = np / C::BN;
  const int64_t tri = (C::BM / C::BN) * tm * (tm + 1) / 2;   // triangle tiles
  for (int k = 0; k < a.steps; ++k) {
    const float ca = a.coeffs[3 * k], cb = a.coeffs[3 * k + 1], cc = a.coeffs[3 * k + 2];
    // bf16 products (with or without the master of X): the poly takes
    // b A from its bf16 A operand tiles in LDS, so B = b A + c A A is one
    // polynomial of the same bf16 A (b A from an fp32 copy makes B a
    // polynomial of two slightly different matrices, which costs accuracy),
    // and the Gram writes no fp32 copy of A.  It accumulates A A + (b / c) A
    // and scales by c, so c must not be tiny next to b (|b / c| <= 1e6 keeps
    // the sum far from overflow, |A| being about 1); otherwise b A comes from
    // fp32 A.
    const bool a_in_lds = sizeof(OP) == 2 && cc != 0.f && std::fabs(cc) >= 1e-6f * std::fabs(cb);
    OP* Xk = C::DIRECT ? Xb[k & 1] : X;
    GemmArgs g = {};
    // Gram: A = X X^T
    g.P = Xk; g.Q = Xk; g.ldp = np; g.ldq = np; g.strideP = mp * np; g.strideQ = mp * np; g.K = np;
    g.tiles_n = tm; g.tiles_per_mat = tri; g.tiles_total = sh.count * tri;
    g.inv0 = k == 0 ? inv : nullptr;
    g.A32 = a_in_lds ? nullptr : A32; g.A16 = A16; g.lda = mp; g.strideA = mp * mp;
    g.sched = sched ? sched + (2 * k) * kSchedPerLaunch : nullptr;
    MUON_LAUNCH("tl_gram", (tl_gemm<C, EPI_GRAM, PT>), dim3(gemm_grid<C, EPI_GRAM, PT>(g.tiles_total)),
                dim3(C::THREADS), a.stream, g);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // poly: B = b A + c A A
    g = GemmArgs{};
    if (sizeof(OP) == 4) { g.P = A32; g.Q = A32; } else { g.P = A16; g.Q = A16; }
    g.ldp = mp; g.ldq = mp; g.strideP = mp * mp; g.strideQ = mp * mp; g.K = mp;
    g.tiles_n = tm; g.tiles_per_mat = tri; g.tiles_total = sh.count * tri;
    g.A32 = a_in_lds ? nullptr : A32; g.PB = PB; g.lda = mp; g.strideA = mp * mp; g.cb = cb; g.cc = cc;
    g.ca = a_in_lds ? cb / cc : 0.f;   // the factor add_ax applies
    g.sched = sched ? sched + (2 * k + 1) * kSchedPerLaunch : nullptr;
    MUON_LAUNCH("tl_poly", (tl_gemm<C, EPI_POLY, PT>), dim3(gemm_grid<C, EPI_POLY, PT>(g.tiles_total)),
                dim3(C::THREADS), a.stream, g);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // apply: X' = a X + B X, with X read row-major (direct-load tiles) or as
    // (X^T)^T
    g = GemmArgs{};
    g.P = PB; g.ldp = mp; g.strideP = mp * mp; g.K = mp;
    if (C::DIRECT) {
      g.Q = Xk; g.ldq = np; g.strideQ = mp * np;
    } else {
      g.Q = XT[k & 1]; g.ldq = mp; g.strideQ = np * mp;
    }
    g.tiles_n = tn; g.tiles_per_mat = tm * tn; g.tiles_total = sh.count * tm * tn;
    g.inv0 = k == 0 ? inv : nullptr;
    g.ca = ca; g.ldx = np; g.ldxt = mp; g.strideX = mp * np;
    if (R) {
      if (comp) {   // K = 2 m: B X~ over the first half, B R over the second
        g.Q2 = R[k & 1]; g.kswitch = mp / C::BK; g.K = 2 * mp;
      } else {
        g.Rin = R[k & 1];
      }
      if (k + 1 < a.steps) g.Rout = R[(k + 1) & 1];
    }
    if (C::DIRECT) {
      g.X = Xb[(k + 1) & 1]; g.XT = nullptr;
    } else {
      g.X = X; g.XT = XT[(k + 1) & 1];
    }
    g.last = (k == a.steps - 1);
    g.param = a.phase == PH_FULL ? a.param : nullptr; g.param_bf16 = a.param_dtype == DT_BF16;
    g.ns_out = a.ns_out; g.lr = a.lr; g.wd = a.wd; g.s = a.s; g.lrwd = a.lrwd;
    g.tabs = a.phase == PH_FULL ? a.tabs : MatTabs{};
    g.m = sh.m; g.n = sh.n; g.transposed = sh.transposed;
    const bool rows = g.tabs.param_rows != nullptr;   // W through a row table
    auto launch = [&](auto comp_tag) {
      constexpr bool CP = decltype(comp_tag)::value;
      if (g.last && !sh.transposed && rows)
        MUON_LAUNCH("tl_apply_update", (tl_gemm<C, EPI_LAST, PT, true, CP>),
                    dim3(gemm_grid<C, EPI_LAST, PT, true, CP>(g.tiles_total)), dim3(C::THREADS), a.stream, g);
      else if (g.last && !sh.transposed)
        MUON_LAUNCH("tl_apply_update", (tl_gemm<C, EPI_LAST, PT, false, CP>),
                    dim3(gemm_grid<C, EPI_LAST, PT, false, CP>(g.tiles_total)), dim3(C::THREADS), a.stream, g);
      else if (g.last && rows)
        MUON_LAUNCH("tl_apply_update", (tl_gemm<C, EPI_LAST_T, PT, true, CP>),
                    dim3(gemm_grid<C, EPI_LAST_T, PT, true, CP>(g.tiles_total)), dim3(C::THREADS), a.stream, g);
      else if (g.last)
        MUON_LAUNCH("tl_apply_update", (tl_gemm<C, EPI_LAST_T, PT, false, CP>),
                    dim3(gemm_grid<C, EPI_LAST_T, PT, false, CP>(g.tiles_total)), dim3(C::THREADS), a.stream, g);
      else
        MUON_LAUNCH("tl_apply", (tl_gemm<C, EPI_APPLY, PT, false, CP>),
                    dim3(gemm_grid<C, EPI_APPLY, PT, false, CP>(g.tiles_total)), dim3(C::THREADS), a.stream, g);
    };
    if constexpr (sizeof(OP) == 2) {
      if (g.kswitch > 0) launch(std::true_type{});
      else launch(std::false_type{});
    } else {
      launch(std::false_type{});
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename OP, typename PT>
hipError_t run_products(const StepArgs& a, const BatchShape& sh, OP* X, OP* X1, OP* XT[2], bf16_t* const* R, bool comp,
                        float* A32, bf16_t* A16, OP* PB, int64_t mp, int64_t np, bool big_tiles, const float* inv,
                        unsigned* sched) {
  if constexpr (sizeof(OP) == 4) {
    if (big_tiles || R) return hipErrorInvalidValue;
    return run_products_cfg<CfgF32, PT>(a, sh, X, X1, XT, nullptr, false, A32, A16, PB, mp, np, inv, nullptr);
  } else {
    // the tile choice is the workspace's (use_big_tiles)
    if (big_tiles) {
      if (mp % CfgBig::BM != 0 || np % CfgBig::BN != 0) return hipErrorInvalidValue;
      return run_products_cfg<CfgBig, PT>(a, sh, X, X1, XT, R, comp, A32, A16, PB, mp, np, inv, sched);
    }
    return run_products_cfg<CfgSmall, PT>(a, sh, X, X1, XT, R, comp, A32, A16, PB, mp, np, inv, nullptr);
  }
}

template <typename OP, typename GT, typename PT>
hipError_t tiled_impl(const StepArgs& a, const WsLayout& L) {
  const BatchShape& sh = a.shape;
  const int mode = a.phase == PH_FULL ? 0 : 1;
  float* ssp = (float*)(a.ws + L.ssp);
  float* inv = (float*)(a.ws + L.inv);
  OP* X = (OP*)(a.ws + L.x);
  OP* X1 = L.big_tiles ? (OP*)(a.ws + L.x1) : nullptr;
  OP* XT[2] = {L.big_tiles ? nullptr : (OP*)(a.ws + L.xt0), L.big_tiles ? nullptr : (OP*)(a.ws + L.xt1)};
  bf16_t* Rbuf[2] = {(bf16_t*)(a.ws + L.r0), (bf16_t*)(a.ws + L.r1)};
  bf16_t* const* R = has_master(a.prec) ? Rbuf : nullptr;   // the master's residues
  float* A32 = (float*)(a.ws + L.a32);
  bf16_t* A16 = a.prec == PREC_F32 ? nullptr : (bf16_t*)(a.ws + L.a16);
  OP* PB = (OP*)(a.ws + L.pb);
  const int64_t mp = L.mp, np = L.np;
  if (L.nparts != (mp / 64) * (np / 64)) return hipErrorInvalidValue;   // one norm partial per 64x64 tile

  // vector form: 16-byte runs of a stored row (n elements, m when stored transposed)
  const int vec = mode == 0 && !XT[0] && (sh.transposed ? sh.m : sh.n) % 8 == 0;
  const MatTabs ftabs = a.phase == PH_FULL ? a.tabs : MatTabs{};
  bf16_t* R0 = R ? R[0] : nullptr;   // the first step's input residue
  if (ftabs.grad_rows)   // the gradient through a row table
    MUON_LAUNCH("tl_momentum_layout", (tl_first<GT, OP, true>), dim3((unsigned)(sh.count * L.nparts)), dim3(256),
                a.stream, mode, vec, (const GT*)a.grad, a.mom, a.u_in, ssp, X, XT[0], R0, sh.m, sh.n, mp, np,
                (int)sh.transposed, a.mu, a.nesterov, ftabs);
  else
    MUON_LAUNCH("tl_momentum_layout", (tl_first<GT, OP, false>), dim3((unsigned)(sh.count * L.nparts)), dim3(256),
                a.stream, mode, vec, (const GT*)a.grad, a.mom, a.u_in, ssp, X, XT[0], R0, sh.m, sh.n, mp, np,
                (int)sh.transposed, a.mu, a.nesterov, ftabs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned* sched = L.big_tiles ? (unsigned*)(a.ws + L.sched) : nullptr;
  MUON_LAUNCH("tl_norm_finalize", tl_norm_finalize, dim3((unsigned)sh.count), dim3(256), a.stream, ssp, L.nparts,
              a.eps, inv, sched, kSchedSlots * kSchedPerLaunch);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return run_products<OP, PT>(a, sh, X, X1, XT, R, a.prec == PREC_BF16_X32C, A32, A16, PB, mp, np, L.big_tiles, inv,
                              sched);
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
  const int64_t total = a.shape.count * a.shape.M * a.shape.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (a.grad_dtype == DT_BF16)
    MUON_LAUNCH("momentum", (tl_momentum<bf16_t>), dim3((unsigned)blocks), dim3(256), a.stream,
                (const bf16_t*)a.grad, a.mom, a.u_out, total, a.mu, a.nesterov);
  else
    MUON_LAUNCH("momentum", (tl_momentum<float>), dim3((unsigned)blocks), dim3(256), a.stream,
                (const float*)a.grad, a.mom, a.u_out, total, a.mu, a.nesterov);
  return hipGetLastError();
}

hipError_t run_update_only(const StepArgs& a) {
  const int64_t total = a.shape.count * a.shape.M * a.shape.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (a.param_dtype == DT_BF16)
    MUON_LAUNCH("update", (tl_update<bf16_t>), dim3((unsigned)blocks), dim3(256), a.stream, (bf16_t*)a.param,
                a.o_in, total, a.lr, a.wd, a.s, a.lrwd);
  else
    MUON_LAUNCH("update", (tl_update<float>), dim3((unsigned)blocks), dim3(256), a.stream, (float*)a.param,
                a.o_in, total, a.lr, a.wd, a.s, a.lrwd);
  return hipGetLastError();
}

}  // namespace muon
