// C ABI of libmuon: the host-side batch plan, argument validation, workspace
// layout and dispatch to the kernel launchers.  Declared in include/muon.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/muon.h"
#include "internal.h"

using namespace muon;

struct muon_plan {
  struct Batch {
    int64_t M, N, count;
    bool transposed;
    int path;
    std::vector<muon_segment> segs;
  };
  std::vector<Batch> batches;
};

namespace {

constexpr int64_t kDefaultCap = int64_t(1) << 29;
constexpr int64_t kMaxMatrixElems = int64_t(1) << 31;   // per padded matrix (32-bit safe tiles)

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

BatchShape shape_of(const muon_plan::Batch& b) {
  BatchShape s;
  s.count = b.count;
  s.M = b.M;
  s.N = b.N;
  s.m = std::min(b.M, b.N);
  s.n = std::max(b.M, b.N);
  s.transposed = b.M > b.N;
  return s;
}

}  // namespace

namespace muon {

WsLayout workspace_layout(const BatchShape& b, int prec, int path) {
  prec = effective_prec(b.m, prec);
  WsLayout L;
  L.path = path;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  if (path == PATH_SKINNY_GRAM || path == PATH_SKINNY_FUSED || path == PATH_SKINNY_STEPWISE) {
    L.skinny = true;
    const int64_t Lc = skinny_chunk(prec);
    L.ldx = round_up(b.n, Lc);
    L.S = L.ldx / Lc;
    L.T = b.m * (b.m + 1) / 2;
    const size_t xs = prec == PREC_BF16 ? 2 : 4;
    if (path != PATH_SKINNY_STEPWISE)   // U as 32-column x 8-row MFMA tiles
      L.x = take(size_t(b.count) * size_t((b.n + 31) / 32) * size_t((b.m + 7) / 8) * 256 * xs);
    else                            // X row-major, row stride ldx
      L.x = take(size_t(b.count) * b.m * L.ldx * xs);
    L.gp0 = take(size_t(b.count) * L.S * L.T * 4);
    if (path == PATH_SKINNY_STEPWISE) L.gp1 = take(size_t(b.count) * L.S * L.T * 4);
    L.sp = take(size_t(b.count) * L.S * 4);
    L.bfrag = take(size_t(b.count) * 64 * 64);   // B' or Q as MFMA fragments: 64 lanes x 64 bytes
  } else {
    L.skinny = false;
    L.mp = round_up(b.m, kTilePad);
    L.np = round_up(b.n, kTilePad);
    L.nparts = (L.mp / 64) * (L.np / 64);   // one ||U||^2 partial per 64x64 tile
    const size_t op = prec == PREC_F32 ? 4 : 2;
    const size_t xe = size_t(b.count) * L.mp * L.np;
    const size_t ae = size_t(b.count) * L.mp * L.mp;
    L.big_tiles = use_big_tiles(L.mp, L.np, prec);
    L.x = take(xe * op);
    if (L.big_tiles) {
      L.x1 = take(xe * op);
    } else {
      L.xt0 = take(xe * op);
      L.xt1 = take(xe * op);
    }
    // the master: the residues bf16(X - bf16(X)) of X, ping-pong (as X when
    // the apply reads X row-major, else as X^T)
    if (has_master(prec)) {
      L.r0 = take(xe * 2);
      L.r1 = take(xe * 2);
    }
    L.a32 = take(ae * 4);
    if (prec != PREC_F32) L.a16 = take(ae * 2);
    L.pb = take(ae * op);
    L.ssp = take(size_t(b.count) * L.nparts * 4);
    L.inv = take(size_t(b.count) * 4);
    if (L.big_tiles) L.sched = take(size_t(kSchedSlots) * kSchedPerLaunch * 4);
  }
  L.total = off;
  return L;
}

}  // namespace muon

namespace {

bool finite(float x) { return std::isfinite(x); }

muon_status check_hparams(const muon_hparams* hp, bool need_ns, bool need_update, bool need_mom) {
  if (!hp) return MUON_ERR_INVALID_ARG;
  if (need_mom) {
    if (!finite(hp->momentum) || hp->momentum < 0.f || hp->momentum > 1.f) return MUON_ERR_INVALID_ARG;
    if (hp->nesterov != 0 && hp->nesterov != 1) return MUON_ERR_INVALID_ARG;
  }
  if (need_ns) {
    if (hp->ns_steps < 1 || hp->ns_steps > 64) return MUON_ERR_INVALID_ARG;
    if (hp->num_coeff_sets != 1 && hp->num_coeff_sets != hp->ns_steps) return MUON_ERR_INVALID_ARG;
    if (!hp->coeffs) return MUON_ERR_INVALID_ARG;
    for (int i = 0; i < 3 * hp->num_coeff_sets; ++i)
      if (!finite(hp->coeffs[i])) return MUON_ERR_INVALID_ARG;
    if (!finite(hp->eps) || hp->eps < 0.f) return MUON_ERR_INVALID_ARG;
    if (hp->precision != MUON_PREC_BF16 && hp->precision != MUON_PREC_BF16_X32 && hp->precision != MUON_PREC_F32 &&
        hp->precision != MUON_PREC_BF16_X32C)
      return MUON_ERR_INVALID_ARG;
  }
  if (need_update) {
    if (!finite(hp->lr) || hp->lr < 0.f) return MUON_ERR_INVALID_ARG;
    if (!finite(hp->weight_decay) || hp->weight_decay < 0.f) return MUON_ERR_INVALID_ARG;
    if (hp->scale != MUON_SCALE_NONE && hp->scale != MUON_SCALE_RMS) return MUON_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(hp->lr_wd_device) & 3u) return MUON_ERR_INVALID_ARG;
  }
  return MUON_OK;
}

bool valid_dtype(muon_dtype d) { return d == MUON_F32 || d == MUON_BF16; }
size_t dsize(muon_dtype d) { return d == MUON_BF16 ? 2 : 4; }

struct Region {
  uintptr_t lo, hi;
};

// null -> invalid; 16-byte alignment; pairwise disjoint.
bool regions_ok(std::vector<Region> rs) {
  for (const Region& r : rs)
    if (r.lo == 0 || (r.lo & 15u)) return false;
  for (size_t i = 0; i < rs.size(); ++i)
    for (size_t j = i + 1; j < rs.size(); ++j)
      if (rs[i].lo < rs[j].hi && rs[j].lo < rs[i].hi) return false;
  return true;
}

Region region(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Region{a, a + bytes};
}

void fill_common(StepArgs& a, const muon_plan::Batch& b, const muon_hparams* hp, void* stream) {
  a.shape = shape_of(b);
  a.stream = reinterpret_cast<hipStream_t>(stream);
  a.param = nullptr; a.grad = nullptr; a.mom = nullptr; a.u_in = nullptr; a.u_out = nullptr;
  a.ns_out = nullptr; a.o_in = nullptr; a.ws = nullptr;
  a.param_dtype = DT_F32; a.grad_dtype = DT_F32;
  a.lr = hp->lr; a.mu = hp->momentum; a.wd = hp->weight_decay; a.eps = hp->eps;
  a.lrwd = hp->lr_wd_device;
  a.nesterov = hp->nesterov;
  a.s = hp->scale == MUON_SCALE_RMS ? float(0.2 * std::sqrt(double(std::max(b.M, b.N)))) : 1.0f;
  a.steps = hp->ns_steps;
  a.prec = effective_prec(std::min(b.M, b.N), hp->precision);
  a.coeffs.clear();
  if (hp->coeffs) {
    for (int k = 0; k < hp->ns_steps; ++k) {
      const float* c = hp->coeffs + 3 * (hp->num_coeff_sets == 1 ? 0 : k);
      a.coeffs.push_back(c[0]); a.coeffs.push_back(c[1]); a.coeffs.push_back(c[2]);
    }
  }
}

const muon_plan::Batch* get_batch(const muon_plan* plan, int32_t batch) {
  if (!plan || batch < 0 || batch >= (int32_t)plan->batches.size()) return nullptr;
  return &plan->batches[batch];
}

muon_status hip_status(hipError_t e) { return e == hipSuccess ? MUON_OK : MUON_ERR_HIP; }

// Failure injection (muon_debug_fail_dispatch): dispatches left before one
// fails without launching; -1 = off.
std::atomic<int> g_fail_after{-1};

hipError_t dispatch(const StepArgs& a, const WsLayout& L) {
  for (int n = g_fail_after.load(std::memory_order_relaxed); n >= 0;) {
    if (g_fail_after.compare_exchange_weak(n, n - 1, std::memory_order_relaxed)) {
      if (n == 0) return hipErrorInvalidValue;
      break;
    }
  }
  switch (L.path) {
    case PATH_SKINNY_GRAM:
    case PATH_SKINNY_FUSED:
    case PATH_SKINNY_STEPWISE: return run_skinny(a, L);
    default: return run_tiled(a, L);
  }
}

// ---- several batches on several streams -----------------------------------

// Estimated run time of a batch, only for ordering: tiled batches by the flops
// of K Gram, polynomial and apply products at 1 PFLOP/s, skinny ones by about
// 20 bytes per element at 6 TB/s.
double batch_cost(const muon_plan::Batch& b, int steps) {
  const double m = double(std::min(b.M, b.N)), n = double(std::max(b.M, b.N)), c = double(b.count);
  if (b.path == PATH_TILED) return c * steps * (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n) / 1.0e15;
  return c * m * n * 20.0 / 6.0e12;
}

// Lanes by longest estimated time first onto the least-loaded lane.  order
// receives positions into batches[] in that order.
void assign_lanes(const muon_plan* plan, int32_t n, const int32_t* batches, int steps, int32_t nlanes,
                  int32_t* lane_of, std::vector<int32_t>& order) {
  std::vector<double> cost(n);
  order.resize(n);
  for (int32_t i = 0; i < n; ++i) {
    cost[i] = batch_cost(plan->batches[batches[i]], steps);
    order[i] = i;
  }
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return cost[x] > cost[y]; });
  std::vector<double> load(nlanes, 0.0);
  for (int32_t i : order) {
    int32_t best = 0;
    for (int32_t l = 1; l < nlanes; ++l)
      if (load[l] < load[best]) best = l;
    lane_of[i] = best;
    load[best] += cost[i];
  }
}

// Common checks of muon_plan_lanes and muon_step_batches.
muon_status check_batch_list(const muon_plan* plan, int32_t n, const int32_t* batches, int32_t nstreams) {
  if (!plan || n < 1 || !batches || nstreams < 1 || nstreams > MUON_MAX_STREAMS) return MUON_ERR_INVALID_ARG;
  std::vector<bool> seen(plan->batches.size(), false);
  for (int32_t i = 0; i < n; ++i) {
    if (!get_batch(plan, batches[i]) || seen[batches[i]]) return MUON_ERR_INVALID_ARG;
    seen[batches[i]] = true;
  }
  return MUON_OK;
}

// Disjointness of many regions (null, misaligned or empty ones rejected).
bool regions_disjoint(std::vector<Region> rs) {
  for (const Region& r : rs)
    if (r.lo == 0 || (r.lo & 15u) || r.hi <= r.lo) return false;
  std::sort(rs.begin(), rs.end(), [](const Region& a, const Region& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < rs.size(); ++i)
    if (rs[i].lo < rs[i - 1].hi) return false;
  return true;
}

// Fork / join events, per device, created on first use and never released.
// Calls hold the lock from the first record to the last wait, so the events
// of concurrent calls are not re-recorded before their waits are enqueued.
std::mutex g_ev_mu;
std::map<int, std::vector<hipEvent_t>> g_events;

hipError_t device_events(int dev, size_t count, std::vector<hipEvent_t>*& out) {
  std::vector<hipEvent_t>& v = g_events[dev];
  while (v.size() < count) {
    hipEvent_t e;
    const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (err != hipSuccess) return err;
    v.push_back(e);
  }
  out = &v;
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t muon_abi_version(void) { return MUON_ABI_VERSION; }

const char* muon_status_str(muon_status s) {
  switch (s) {
    case MUON_OK: return "ok";
    case MUON_ERR_INVALID_ARG: return "invalid argument";
    case MUON_ERR_UNSUPPORTED: return "unsupported shape or combination";
    case MUON_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MUON_ERR_NO_MEMORY: return "host out of memory";
    case MUON_ERR_HIP: return "HIP launch error";
    case MUON_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

muon_status muon_plan_create(const muon_shape* shapes, int32_t n, const muon_plan_options* opt, muon_plan** out) {
  if (!out) return MUON_ERR_INVALID_ARG;
  *out = nullptr;
  if (!shapes || n < 1) return MUON_ERR_INVALID_ARG;
  int64_t cap = kDefaultCap;
  int32_t order = 0, skinny_kernel = 0;
  if (opt) {
    if (opt->max_batch_elems < 0 || (opt->order != 0 && opt->order != 1)) return MUON_ERR_INVALID_ARG;
    if (opt->skinny_kernel < 0 || opt->skinny_kernel > 3) return MUON_ERR_INVALID_ARG;
    if (opt->max_batch_elems > 0) cap = opt->max_batch_elems;
    order = opt->order;
    skinny_kernel = opt->skinny_kernel;
  }
  // core shape of every parameter (HyperParallel-FSDP §6.6: [A,B], [A,1,B], [N,A,B] -> (A,B))
  struct Core { int64_t nm, M, N; };
  std::vector<Core> cores;
  for (int32_t i = 0; i < n; ++i) {
    const muon_shape& s = shapes[i];
    if (s.ndim != 2 && s.ndim != 3) return MUON_ERR_UNSUPPORTED;
    for (int d = 0; d < s.ndim; ++d)
      if (s.dims[d] <= 0) return MUON_ERR_INVALID_ARG;
    Core c;
    if (s.ndim == 2) c = {1, s.dims[0], s.dims[1]};
    else if (s.dims[1] == 1) c = {1, s.dims[0], s.dims[2]};
    else c = {s.dims[0], s.dims[1], s.dims[2]};
    int64_t per, tot;
    if (!mul_ok(c.M, c.N, &per) || !mul_ok(per, c.nm, &tot)) return MUON_ERR_INVALID_ARG;
    // padded matrix must stay addressable with the kernels' tile arithmetic
    int64_t mp = round_up(std::min(c.M, c.N), kTilePad), np = round_up(std::max(c.M, c.N), kTilePad), pe;
    if (!mul_ok(mp, np, &pe) || pe > kMaxMatrixElems) return MUON_ERR_UNSUPPORTED;
    cores.push_back(c);
  }
  muon_plan* p = new (std::nothrow) muon_plan;
  if (!p) return MUON_ERR_NO_MEMORY;
  try {
    // buckets in first-seen order of (M, N)
    std::vector<std::pair<std::pair<int64_t, int64_t>, std::vector<std::pair<int32_t, int64_t>>>> buckets;
    for (int32_t i = 0; i < n; ++i) {
      auto key = std::make_pair(cores[i].M, cores[i].N);
      auto it = std::find_if(buckets.begin(), buckets.end(), [&](const auto& b) { return b.first == key; });
      if (it == buckets.end()) {
        buckets.push_back({key, {}});
        it = buckets.end() - 1;
      }
      for (int64_t e = 0; e < cores[i].nm; ++e) it->second.push_back({i, e});
    }
    for (auto& bk : buckets) {
      const int64_t M = bk.first.first, N = bk.first.second, per = M * N;
      const int64_t max_count = std::max<int64_t>(1, cap / per);
      const auto& mats = bk.second;
      // as few chunks as the cap allows, their sizes within one of each other (larger first)
      const int64_t total = (int64_t)mats.size();
      const int64_t chunks = (total + max_count - 1) / max_count;
      const int64_t base = total / chunks, extra = total % chunks;
      size_t start = 0;
      for (int64_t c = 0; c < chunks; ++c) {
        const size_t end = start + (size_t)(base + (c < extra ? 1 : 0));
        muon_plan::Batch b;
        b.M = M; b.N = N; b.count = (int64_t)(end - start); b.transposed = M > N;
        const int64_t m = std::min(M, N), n = std::max(M, N);
        if (m > kSkinnyMaxRows) b.path = PATH_TILED;
        else if (skinny_kernel == 2) b.path = PATH_SKINNY_STEPWISE;
        else if (skinny_kernel == 1) b.path = PATH_SKINNY_GRAM;
        else b.path = PATH_SKINNY_FUSED;
        for (size_t k = start; k < end; ++k) {
          const int32_t pi = mats[k].first;
          const int64_t mi = mats[k].second;
          if (!b.segs.empty() && b.segs.back().param_index == pi &&
              b.segs.back().first_matrix + b.segs.back().num_matrices == mi) {
            b.segs.back().num_matrices += 1;
          } else {
            muon_segment sg;
            sg.param_index = pi; sg.reserved = 0; sg.first_matrix = mi; sg.num_matrices = 1;
            sg.elem_offset = (int64_t)(k - start) * per;
            b.segs.push_back(sg);
          }
        }
        p->batches.push_back(std::move(b));
        start = end;
      }
    }
    if (order == 0)
      std::stable_sort(p->batches.begin(), p->batches.end(), [](const muon_plan::Batch& x, const muon_plan::Batch& y) {
        return x.count * x.M * x.N > y.count * y.M * y.N;
      });
  } catch (const std::bad_alloc&) {
    delete p;
    return MUON_ERR_NO_MEMORY;
  }
  *out = p;
  return MUON_OK;
}

void muon_plan_destroy(muon_plan* plan) { delete plan; }

int32_t muon_plan_num_batches(const muon_plan* plan) { return plan ? (int32_t)plan->batches.size() : -1; }

muon_status muon_plan_batch_info(const muon_plan* plan, int32_t batch, muon_batch_info* out) {
  const muon_plan::Batch* b = get_batch(plan, batch);
  if (!b || !out) return MUON_ERR_INVALID_ARG;
  out->M = b->M; out->N = b->N; out->count = b->count; out->transposed = b->transposed ? 1 : 0;
  out->num_segments = (int32_t)b->segs.size();
  out->path = b->path == PATH_SKINNY_FUSED ? PATH_SKINNY_GRAM : b->path;
  out->reserved = 0;
  return MUON_OK;
}

muon_status muon_plan_segments(const muon_plan* plan, int32_t batch, muon_segment* out, int32_t capacity) {
  const muon_plan::Batch* b = get_batch(plan, batch);
  if (!b || !out || capacity < 0) return MUON_ERR_INVALID_ARG;
  const int32_t k = std::min<int32_t>(capacity, (int32_t)b->segs.size());
  for (int32_t i = 0; i < k; ++i) out[i] = b->segs[i];
  return MUON_OK;
}

muon_status muon_workspace_bytes(const muon_plan* plan, int32_t batch, muon_precision precision, size_t* out) {
  const muon_plan::Batch* b = get_batch(plan, batch);
  if (!b || !out) return MUON_ERR_INVALID_ARG;
  if (precision != MUON_PREC_BF16 && precision != MUON_PREC_BF16_X32 && precision != MUON_PREC_F32 &&
      precision != MUON_PREC_BF16_X32C)
    return MUON_ERR_INVALID_ARG;
  *out = workspace_layout(shape_of(*b), precision, b->path).total;
  return MUON_OK;
}

muon_status muon_step(const muon_plan* plan, int32_t batch, const muon_batch_buffers* bufs, const muon_hparams* hp,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const muon_plan::Batch* b = get_batch(plan, batch);
  if (!b || !bufs) return MUON_ERR_INVALID_ARG;
  muon_status st = check_hparams(hp, true, true, true);
  if (st != MUON_OK) return st;
  if (!valid_dtype(bufs->param_dtype) || !valid_dtype(bufs->grad_dtype)) return MUON_ERR_INVALID_ARG;
  const size_t elems = size_t(b->count) * b->M * b->N;
  const WsLayout L = workspace_layout(shape_of(*b), hp->precision, b->path);
  if (workspace_bytes < L.total) return MUON_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MUON_ERR_INVALID_ARG;
  std::vector<Region> rs = {region(bufs->param, elems * dsize(bufs->param_dtype)),
                            region(bufs->grad, elems * dsize(bufs->grad_dtype)),
                            region(bufs->momentum, elems * 4), region(workspace, L.total)};
  if (bufs->ns_out) rs.push_back(region(bufs->ns_out, elems * 4));
  if (!regions_ok(rs)) return MUON_ERR_INVALID_ARG;

  StepArgs a;
  fill_common(a, *b, hp, stream);
  a.phase = PH_FULL;
  a.param = bufs->param; a.param_dtype = bufs->param_dtype == MUON_BF16 ? DT_BF16 : DT_F32;
  a.grad = bufs->grad; a.grad_dtype = bufs->grad_dtype == MUON_BF16 ? DT_BF16 : DT_F32;
  a.mom = bufs->momentum; a.ns_out = bufs->ns_out;
  a.ws = static_cast<char*>(workspace);
  return hip_status(dispatch(a, L));
}

muon_status muon_step_ptrs(const muon_plan* plan, int32_t batch, const muon_batch_ptrs* bufs, const muon_hparams* hp,
                           void* workspace, size_t workspace_bytes, void* stream) {
  const muon_plan::Batch* b = get_batch(plan, batch);
  if (!b || !bufs) return MUON_ERR_INVALID_ARG;
  muon_status st = check_hparams(hp, true, true, true);
  if (st != MUON_OK) return st;
  if (!valid_dtype(bufs->param_dtype) || !valid_dtype(bufs->grad_dtype)) return MUON_ERR_INVALID_ARG;
  if (!bufs->params || !bufs->grads || !bufs->momenta) return MUON_ERR_INVALID_ARG;
  const WsLayout L = workspace_layout(shape_of(*b), hp->precision, b->path);
  if (workspace_bytes < L.total) return MUON_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MUON_ERR_INVALID_ARG;
  const size_t tab_bytes = size_t(b->count) * sizeof(void*);
  std::vector<Region> rs = {region(bufs->params, tab_bytes), region(bufs->grads, tab_bytes),
                            region(bufs->momenta, tab_bytes), region(workspace, L.total)};
  if (bufs->ns_out) rs.push_back(region(bufs->ns_out, tab_bytes));
  if (!regions_ok(rs)) return MUON_ERR_INVALID_ARG;

  StepArgs a;
  fill_common(a, *b, hp, stream);
  a.phase = PH_FULL;
  a.param = nullptr; a.param_dtype = bufs->param_dtype == MUON_BF16 ? DT_BF16 : DT_F32;
  a.grad = nullptr; a.grad_dtype = bufs->grad_dtype == MUON_BF16 ? DT_BF16 : DT_F32;
  a.mom = nullptr; a.ns_out = nullptr;
  a.tabs.param = reinterpret_cast<const void* const*>(bufs->params);
  a.tabs.grad = bufs->grads;
  a.tabs.mom = reinterpret_cast<const void* const*>(bufs->momenta);
  a.tabs.ns = reinterpret_cast<const void* const*>(bufs->ns_out);
  a.ws = static_cast<char*>(workspace);
  return hip_status(dispatch(a, L));
}

muon_status muon_step_rows(const muon_plan* plan, int32_t batch, const muon_batch_rows* bufs, const muon_hparams* hp,
                           void* workspace, size_t workspace_bytes, void* stream) {
  const muon_plan::Batch* b = get_batch(plan, batch);
  if (!b || !bufs) return MUON_ERR_INVALID_ARG;
  muon_status st = check_hparams(hp, true, true, true);
  if (st != MUON_OK) return st;
  if (!valid_dtype(bufs->param_dtype) || !valid_dtype(bufs->grad_dtype)) return MUON_ERR_INVALID_ARG;
  if (!bufs->param_rows || !bufs->grad_rows || !bufs->momentum) return MUON_ERR_INVALID_ARG;
  const WsLayout L = workspace_layout(shape_of(*b), hp->precision, b->path);
  if (workspace_bytes < L.total) return MUON_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MUON_ERR_INVALID_ARG;
  const size_t elems = size_t(b->count) * b->M * b->N;
  const size_t tab_bytes = size_t(b->count) * b->M * sizeof(void*);
  std::vector<Region> rs = {region(bufs->param_rows, tab_bytes), region(bufs->grad_rows, tab_bytes),
                            region(bufs->momentum, elems * 4), region(workspace, L.total)};
  if (bufs->ns_out) rs.push_back(region(bufs->ns_out, elems * 4));
  if (!regions_ok(rs)) return MUON_ERR_INVALID_ARG;

  StepArgs a;
  fill_common(a, *b, hp, stream);
  a.phase = PH_FULL;
  a.param = nullptr; a.param_dtype = bufs->param_dtype == MUON_BF16 ? DT_BF16 : DT_F32;
  a.grad = nullptr; a.grad_dtype = bufs->grad_dtype == MUON_BF16 ? DT_BF16 : DT_F32;
  a.mom = bufs->momentum; a.ns_out = bufs->ns_out;
  a.tabs.param_rows = reinterpret_cast<const void* const*>(bufs->param_rows);
  a.tabs.grad_rows = bufs->grad_rows;
  a.ws = static_cast<char*>(workspace);
  return hip_status(dispatch(a, L));
}

muon_status muon_plan_lanes(const muon_plan* plan, int32_t n, const int32_t* batches, const muon_hparams* hp,
                            int32_t nstreams, int32_t* lane_of, size_t* lane_workspace_bytes) {
  muon_status st = check_batch_list(plan, n, batches, nstreams);
  if (st != MUON_OK) return st;
  if (!lane_of || !lane_workspace_bytes) return MUON_ERR_INVALID_ARG;
  st = check_hparams(hp, true, false, false);
  if (st != MUON_OK) return st;
  std::vector<int32_t> order;
  try {
    assign_lanes(plan, n, batches, hp->ns_steps, nstreams, lane_of, order);
  } catch (const std::bad_alloc&) {
    return MUON_ERR_NO_MEMORY;
  }
  for (int32_t l = 0; l < nstreams; ++l) lane_workspace_bytes[l] = 0;
  for (int32_t i = 0; i < n; ++i) {
    const muon_plan::Batch& b = plan->batches[batches[i]];
    const size_t need = workspace_layout(shape_of(b), hp->precision, b.path).total;
    lane_workspace_bytes[lane_of[i]] = std::max(lane_workspace_bytes[lane_of[i]], need);
  }
  return MUON_OK;
}

muon_status muon_step_batches(const muon_plan* plan, int32_t n, const int32_t* batches,
                              const muon_batch_buffers* bufs, const muon_hparams* hp, void* const* workspaces,
                              const size_t* workspace_bytes, void* const* streams, int32_t nstreams) {
  muon_status st = check_batch_list(plan, n, batches, nstreams);
  if (st != MUON_OK) return st;
  if (!bufs || !workspaces || !workspace_bytes || !streams) return MUON_ERR_INVALID_ARG;
  st = check_hparams(hp, true, true, true);
  if (st != MUON_OK) return st;
  try {
    std::vector<int32_t> lane_of(n), order;
    assign_lanes(plan, n, batches, hp->ns_steps, nstreams, lane_of.data(), order);
    std::vector<size_t> need(nstreams, 0);
    std::vector<Region> rs;
    for (int32_t i = 0; i < n; ++i) {
      const muon_plan::Batch& b = plan->batches[batches[i]];
      const muon_batch_buffers& f = bufs[i];
      if (!valid_dtype(f.param_dtype) || !valid_dtype(f.grad_dtype)) return MUON_ERR_INVALID_ARG;
      const size_t elems = size_t(b.count) * b.M * b.N;
      rs.push_back(region(f.param, elems * dsize(f.param_dtype)));
      rs.push_back(region(f.grad, elems * dsize(f.grad_dtype)));
      rs.push_back(region(f.momentum, elems * 4));
      if (f.ns_out) rs.push_back(region(f.ns_out, elems * 4));
      need[lane_of[i]] = std::max(need[lane_of[i]], workspace_layout(shape_of(b), hp->precision, b.path).total);
    }
    for (int32_t l = 0; l < nstreams; ++l) {
      if (need[l] == 0) continue;
      if (workspace_bytes[l] < need[l]) return MUON_ERR_WORKSPACE_TOO_SMALL;
      if (!workspaces[l] || (reinterpret_cast<uintptr_t>(workspaces[l]) & 255u)) return MUON_ERR_INVALID_ARG;
      rs.push_back(region(workspaces[l], need[l]));
    }
    if (!regions_disjoint(rs)) return MUON_ERR_INVALID_ARG;

    auto run_lane = [&](int32_t l) -> hipError_t {
      for (int32_t i : order) {
        if (lane_of[i] != l) continue;
        const muon_plan::Batch& b = plan->batches[batches[i]];
        const muon_batch_buffers& f = bufs[i];
        StepArgs a;
        fill_common(a, b, hp, streams[l]);
        a.phase = PH_FULL;
        a.param = f.param; a.param_dtype = f.param_dtype == MUON_BF16 ? DT_BF16 : DT_F32;
        a.grad = f.grad; a.grad_dtype = f.grad_dtype == MUON_BF16 ? DT_BF16 : DT_F32;
        a.mom = f.momentum; a.ns_out = f.ns_out;
        a.ws = static_cast<char*>(workspaces[l]);
        const hipError_t e = dispatch(a, workspace_layout(a.shape, hp->precision, b.path));
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    };
    int32_t used = 0;
    for (int32_t l = 1; l < nstreams; ++l) used += need[l] > 0;
    if (used == 0) return hip_status(run_lane(0));

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return MUON_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ev_mu);
    std::vector<hipEvent_t>* ev = nullptr;   // [0] fork, [l] join of lane l
    if ((e = device_events(dev, size_t(nstreams), ev)) != hipSuccess) return MUON_ERR_HIP;
    const hipStream_t s0 = reinterpret_cast<hipStream_t>(streams[0]);
    if ((e = hipEventRecord((*ev)[0], s0)) != hipSuccess) return MUON_ERR_HIP;
    // Every lane that waited on the fork is joined back into streams[0], also
    // when a launch fails part-way: eagerly, later work on the caller's stream
    // stays ordered after what the lanes did enqueue, and under graph capture
    // no side stream is left unjoined.
    std::vector<char> forked(size_t(nstreams), 0);
    auto join = [&]() -> hipError_t {
      hipError_t first = hipSuccess;
      for (int32_t l = 1; l < nstreams; ++l) {
        if (!forked[l]) continue;
        hipError_t r = hipEventRecord((*ev)[l], reinterpret_cast<hipStream_t>(streams[l]));
        if (r == hipSuccess) r = hipStreamWaitEvent(s0, (*ev)[l], 0);
        if (r != hipSuccess && first == hipSuccess) first = r;
      }
      return first;
    };
    for (int32_t l = 1; l < nstreams; ++l) {
      if (need[l] == 0) continue;
      if ((e = hipStreamWaitEvent(reinterpret_cast<hipStream_t>(streams[l]), (*ev)[0], 0)) != hipSuccess) {
        (void)join();
        return MUON_ERR_HIP;
      }
      forked[l] = 1;
    }
    for (int32_t l = 0; l < nstreams; ++l)
      if ((l == 0 || need[l] > 0) && (e = run_lane(l)) != hipSuccess) {
        (void)join();
        return MUON_ERR_HIP;
      }
    return join() == hipSuccess ? MUON_OK : MUON_ERR_HIP;
  } catch (const std::bad_alloc&) {
    return MUON_ERR_NO_MEMORY;
  }
}

muon_status muon_stage_momentum(const muon_plan* plan, int32_t batch, const void* grad, muon_dtype grad_dtype,
                                float* momentum, float* u_out, const muon_hparams* hp, void* stream) {
  const muon_plan::Batch* b = get_batch(plan, batch);
  if (!b) return MUON_ERR_INVALID_ARG;
  muon_status st = check_hparams(hp, false, false, true);
  if (st != MUON_OK) return st;
  if (!valid_dtype(grad_dtype)) return MUON_ERR_INVALID_ARG;
  const size_t elems = size_t(b->count) * b->M * b->N;
  if (!regions_ok({region(grad, elems * dsize(grad_dtype)), region(momentum, elems * 4), region(u_out, elems * 4)}))
    return MUON_ERR_INVALID_ARG;
  StepArgs a;
  fill_common(a, *b, hp, stream);
  a.phase = PH_MOMENTUM;
  a.grad = grad; a.grad_dtype = grad_dtype == MUON_BF16 ? DT_BF16 : DT_F32;
  a.mom = momentum; a.u_out = u_out;
  return hip_status(run_momentum_only(a));
}

muon_status muon_stage_ns(const muon_plan* plan, int32_t batch, const float* u_in, float* o_out, const muon_hparams* hp,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const muon_plan::Batch* b = get_batch(plan, batch);
  if (!b) return MUON_ERR_INVALID_ARG;
  muon_status st = check_hparams(hp, true, false, false);
  if (st != MUON_OK) return st;
  const size_t elems = size_t(b->count) * b->M * b->N;
  const WsLayout L = workspace_layout(shape_of(*b), hp->precision, b->path);
  if (workspace_bytes < L.total) return MUON_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return MUON_ERR_INVALID_ARG;
  if (!regions_ok({region(u_in, elems * 4), region(o_out, elems * 4), region(workspace, L.total)}))
    return MUON_ERR_INVALID_ARG;
  StepArgs a;
  fill_common(a, *b, hp, stream);
  a.phase = PH_NS;
  a.u_in = u_in; a.ns_out = o_out;
  a.ws = static_cast<char*>(workspace);
  return hip_status(dispatch(a, L));
}

muon_status muon_stage_update(const muon_plan* plan, int32_t batch, void* param, muon_dtype param_dtype,
                              const float* o_in, const muon_hparams* hp, void* stream) {
  const muon_plan::Batch* b = get_batch(plan, batch);
  if (!b) return MUON_ERR_INVALID_ARG;
  muon_status st = check_hparams(hp, false, true, false);
  if (st != MUON_OK) return st;
  if (!valid_dtype(param_dtype)) return MUON_ERR_INVALID_ARG;
  const size_t elems = size_t(b->count) * b->M * b->N;
  if (!regions_ok({region(param, elems * dsize(param_dtype)), region(o_in, elems * 4)})) return MUON_ERR_INVALID_ARG;
  StepArgs a;
  fill_common(a, *b, hp, stream);
  a.phase = PH_UPDATE;
  a.param = param; a.param_dtype = param_dtype == MUON_BF16 ? DT_BF16 : DT_F32;
  a.o_in = o_in;
  return hip_status(run_update_only(a));
}

void muon_debug_fail_dispatch(int32_t n) { g_fail_after.store(n < 0 ? -1 : n, std::memory_order_relaxed); }

}  // extern "C"
