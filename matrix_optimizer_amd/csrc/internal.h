// Internal host-side interface between the C ABI (abi.cpp) and the kernel
// launchers (skinny.hip, tiled.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <vector>

namespace muon {

// Per-device value that every caller computes the same way (resident
// workgroups of a kernel): read and published atomically, so concurrent first
// calls on a device race benignly (each stores the same value).
constexpr int kMaxDevices = 64;
template <class F>
int per_device_cached(std::atomic<int> (&cache)[kMaxDevices], F compute) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int v = cache[dev].load(std::memory_order_acquire);
  if (v == 0) {
    v = compute(dev);
    cache[dev].store(v, std::memory_order_release);
  }
  return v;
}

enum Dtype { DT_F32 = 0, DT_BF16 = 1 };
enum Prec { PREC_BF16 = 0, PREC_BF16_X32 = 1, PREC_F32 = 2, PREC_BF16_X32C = 3 };
// Precisions that keep a master of X on the tiled path: X = bf16(X) +
// bf16(X - bf16(X)), the second term (the residue) in its own buffer.
inline bool has_master(int prec) { return prec == PREC_BF16_X32 || prec == PREC_BF16_X32C; }

// Which part of the step a call runs.
enum Phase { PH_FULL = 0, PH_MOMENTUM = 1, PH_NS = 2, PH_UPDATE = 3 };

// Matrices with m = min(M, N) up to this many rows take the skinny path.
constexpr int64_t kSkinnyMaxRows = 32;

// Skinny path: columns of X handled by one workgroup (bf16-stored X, and
// fp32-stored X).  Both must be multiples of 64.
#ifndef MUON_SK_CHUNK_BF16
#define MUON_SK_CHUNK_BF16 512
#endif
#ifndef MUON_SK_CHUNK_F32
#define MUON_SK_CHUNK_F32 256
#endif
inline int64_t skinny_chunk(int prec) { return prec == PREC_BF16 ? MUON_SK_CHUNK_BF16 : MUON_SK_CHUNK_F32; }

// Tiled path: rows and columns of X are padded to this multiple.
constexpr int64_t kTilePad = 128;
// Tiled path: below this short side the bf16 placements (A and B rounded to
// bf16 as MFMA operands) lose too much accuracy, so products run on fp32
// operands whatever precision was asked for; the flops there are small.
constexpr int64_t kTiledBf16MinRows = 128;

// Precision the kernels actually run for a matrix with short side m.
inline int effective_prec(int64_t m, int prec) {
  if (m > kSkinnyMaxRows && m < kTiledBf16MinRows) return PREC_F32;
  // the skinny path's Gram-space products are fp32 already: the second
  // (compensating) product is a tiled-path placement
  if (m <= kSkinnyMaxRows && prec == PREC_BF16_X32C) return PREC_BF16_X32;
  return prec;
}
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct BatchShape {
  int64_t count, M, N;   // stored [count, M, N]
  int64_t m, n;          // Newton-Schulz orientation: m = min(M,N) rows, n = max(M,N) columns
  bool transposed;       // M > N
};

// Kernel family of a batch: tiled products (short side > 32), or the skinny
// chunk kernels with Newton-Schulz in Gram space (3 launches) or step by step
// (2K + 1 launches).
// PATH_SKINNY_FUSED: Gram space with the Newton-Schulz and the apply in one
// launch where the stored rows are U rows (the workspace of PATH_SKINNY_GRAM;
// reported to callers as path 1).
enum Path { PATH_TILED = 0, PATH_SKINNY_GRAM = 1, PATH_SKINNY_STEPWISE = 2, PATH_SKINNY_FUSED = 3 };

// Device workspace carve-up of one batch (offsets in bytes from the base).
struct WsLayout {
  bool skinny = false;
  int path = PATH_TILED;
  size_t total = 0;
  // skinny path
  int64_t ldx = 0, S = 0, T = 0;
  size_t x = 0, gp0 = 0, gp1 = 0, sp = 0, bfrag = 0;
  // tiled path.  With 256 x 256 tiles (big_tiles) the apply products read X
  // row-major, and X ping-pongs between x and x1; otherwise they read X^T,
  // kept in xt0 / xt1 beside x.
  int64_t mp = 0, np = 0, nparts = 0;
  bool big_tiles = false;
  size_t x1 = 0, xt0 = 0, xt1 = 0, a32 = 0, a16 = 0, pb = 0, ssp = 0, inv = 0;
  size_t r0 = 0, r1 = 0;   // the master: bf16 residues of X (X's layout, or X^T's)
  // tile counters of the 256 x 256 Gram and poly products: kSchedSlots
  // launches of a step (2 per Newton-Schulz step), 8 per launch (one per XCD
  // tile range)
  size_t sched = 0;
};

constexpr int kSchedPerLaunch = 8;
constexpr int kSchedSlots = 2 * 64;   // ns_steps <= 64

// The tiled products use 256 x 256 tiles (direct loads, row-major X operand
// of the apply) when both padded sides are multiples of 256 and the operands
// are bf16.
inline bool use_big_tiles(int64_t mp, int64_t np, int prec) {
  return prec != PREC_F32 && mp % 256 == 0 && np % 256 == 0;
}

WsLayout workspace_layout(const BatchShape& b, int prec, int path);

// Per-matrix addresses of a batch's caller buffers (zero-copy batching):
// device arrays of one pointer per matrix, or null where the buffer is one
// contiguous [count, M, N] region.  param_rows / grad_rows: one pointer per
// stored row instead ([count * M], row r of matrix b at b M + r, N elements
// each), for matrices that are row-level views of fused parameters.
struct MatTabs {
  const void* const* param;
  const void* const* grad;
  const void* const* mom;
  const void* const* ns;
  const void* const* param_rows;
  const void* const* grad_rows;
};

struct StepArgs {
  BatchShape shape;
  int phase;
  void* param; int param_dtype;
  const void* grad; int grad_dtype;
  float* mom;
  const float* u_in;     // PH_NS input
  float* u_out;          // PH_MOMENTUM output
  float* ns_out;         // O output (PH_FULL optional, PH_NS required)
  const float* o_in;     // PH_UPDATE input
  float lr, mu, wd, eps, s;
  const float* lrwd;     // optional device {lr, wd}, read by the update kernels
  MatTabs tabs = {};     // per-matrix pointer tables (PH_FULL), null for contiguous buffers
  int nesterov;
  int steps;
  std::vector<float> coeffs;   // 3 * steps (expanded)
  int prec;
  char* ws;
  hipStream_t stream;
};

// Launch tracing (trace.cpp): while muon_trace_start is active, hands out
// the start and stop events of the next traced launch (false otherwise).
bool trace_take(const char* name, hipEvent_t* start, hipEvent_t* stop);

// Launch a kernel.  While tracing, the launch goes through
// hipExtLaunchKernelGGL, whose start and stop events the runtime records with
// the dispatch itself, so they time the kernel's execution.
#define MUON_LAUNCH(NAME, KERNEL, GRID, BLOCK, STREAM, ...) \
  MUON_LAUNCH_SHM(NAME, KERNEL, GRID, BLOCK, 0, STREAM, __VA_ARGS__)

// Same, with SHM bytes of dynamic LDS.
#define MUON_LAUNCH_SHM(NAME, KERNEL, GRID, BLOCK, SHM, STREAM, ...)                                \
  do {                                                                                            \
    hipEvent_t muon_ev0_ = nullptr, muon_ev1_ = nullptr;                                          \
    if (::muon::trace_take(NAME, &muon_ev0_, &muon_ev1_))                                         \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHM, STREAM, muon_ev0_, muon_ev1_, 0u, __VA_ARGS__); \
    else                                                                                          \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHM, STREAM, __VA_ARGS__);                          \
  } while (0)

// Each returns hipSuccess or the first launch error.
hipError_t run_skinny(const StepArgs& a, const WsLayout& L);
hipError_t run_tiled(const StepArgs& a, const WsLayout& L);
hipError_t run_momentum_only(const StepArgs& a);
hipError_t run_update_only(const StepArgs& a);

}  // namespace muon
