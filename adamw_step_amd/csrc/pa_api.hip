// pa_api.hip -- host side of the C ABI declared in include/pa.h.
//
// Validation, the per-call scalars, the launch plan of a tensor list (a
// device table cached per distinct pointer/size list) and the launches.
// Nothing here computes the update; every element is handled by the kernels
// in kernels.hpp.  There is no CPU path.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstddef>
#include <cstring>
#include <list>
#include <mutex>
#include <type_traits>
#include <vector>

#include "../../include/pa.h"
#include "kernels.hpp"
#include "turbo.hpp"

namespace {

thread_local int g_last_hip_error = 0;

int hip_failed(hipError_t e) {
  g_last_hip_error = (int)e;
  return PA_ERR_DEVICE;
}

// ---------------------------------------------------------------- scalars

// lr, betas, eps and weight decay are host doubles; the bias corrections and
// the quotients that meet FP32 tensors are formed in double and each is
// rounded to binary32 once (the KBench reference computes them as Python
// floats and applies them to FP32 tensors).
int make_scalars(const pa_hyper* h, long long step, pa::Scalars* s) {
  if (h == nullptr || step < 1) return PA_ERR_ARG;
  const double lr = h->lr, b1 = h->beta1, b2 = h->beta2, eps = h->eps, wd = h->weight_decay;
  if (!std::isfinite(lr) || !std::isfinite(eps) || !std::isfinite(wd) || !std::isfinite(b1) ||
      !std::isfinite(b2))
    return PA_ERR_ARG;
  if (lr < 0.0 || eps < 0.0 || wd < 0.0) return PA_ERR_ARG;
  if (!(b1 >= 0.0 && b1 < 1.0) || !(b2 >= 0.0 && b2 < 1.0)) return PA_ERR_ARG;
  const double bc1 = 1.0 - std::pow(b1, (double)step);
  const double bc2 = 1.0 - std::pow(b2, (double)step);
  s->beta1 = (float)b1;
  s->one_m_beta1 = (float)(1.0 - b1);
  s->beta2 = (float)b2;
  s->one_m_beta2 = (float)(1.0 - b2);
  s->bc2 = (float)bc2;
  s->lr_over_bc1 = (float)(lr / bc1);
  s->decay = (float)(1.0 - lr * wd);
  s->eps = (float)eps;
  s->beta1_x2p112 = std::ldexp(s->beta1, 112);
  s->gmul = 1.0f;
  s->inv_bc2 = 1.0 / (double)s->bc2;
  s->gscale = h->grad_scale;
  s->skip = h->skip_if_nonzero;
  const uintptr_t gs = reinterpret_cast<uintptr_t>(h->grad_scale), sk = reinterpret_cast<uintptr_t>(h->skip_if_nonzero),
                  nf = reinterpret_cast<uintptr_t>(h->nonfinite);
  if (gs % 4 || sk % 8 || nf % 8) return PA_ERR_ALIGN;
  return PA_OK;
}


// ---------------------------------------------------------------- devices

struct DeviceInfo {
  int cus = 0;
  int blocks_per_cu = 0;      // elementwise kernels
  int bw_blocks_per_cu = 0;   // blockwise kernel
  int stats_blocks_per_cu = 0;   // gradient pre-pass
};

std::mutex g_dev_mu;
DeviceInfo g_dev[64];

int device_info(int* dev_out, DeviceInfo* info) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_failed(e);
  if (dev < 0 || dev >= 64) return PA_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (d.cus == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_failed(e);
    int per = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per, reinterpret_cast<const void*>(pa::elementwise_list<pa::kModeE4, pa::kF32, pa::kF32, false, false, pa::kUnroll>),
        pa::kThreads, 0);
    if (e != hipSuccess || per < 1) per = 4;
    int bw = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &bw, reinterpret_cast<const void*>(pa::blockwise_kernel<false, false, false>), pa::kThreads, 0);
    if (e != hipSuccess || bw < 1) bw = 2;
    d.cus = cus;
    d.blocks_per_cu = per;
    d.bw_blocks_per_cu = bw;
    int st = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &st, reinterpret_cast<const void*>(pa::grad_stats_list<pa::kF32, true>), pa::kThreads, 0);
    if (e != hipSuccess || st < 1) st = 4;
    d.stats_blocks_per_cu = st;
  }
  *dev_out = dev;
  *info = d;
  return PA_OK;
}

// Workgroups per CU of a persistent launch: the occupancy calculator's figure
// unless fixed at build time.
#ifndef PA_BLOCKS_PER_CU
#define PA_BLOCKS_PER_CU 0
#endif

long long grid_for(long long work_items, const DeviceInfo& d, int occupancy) {
  const long long per_cu = PA_BLOCKS_PER_CU > 0 ? PA_BLOCKS_PER_CU : occupancy;
  const long long cap = (long long)d.cus * per_cu;
  return std::max(1LL, std::min(work_items, cap));
}

// ---------------------------------------------------------------- checks

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  uintptr_t lo, hi;
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

// The device words named by a pa_hyper (counter, gradient scale, skip flag):
// none may overlap another or any tensor of the call, or a workgroup that
// starts late could read a value the call itself has changed.
void hyper_ranges(const pa_hyper* h, std::vector<Range>* out) {
  if (h->nonfinite) out->push_back(range_of(h->nonfinite, 8));
  if (h->grad_scale) out->push_back(range_of(h->grad_scale, 4));
  if (h->skip_if_nonzero) out->push_back(range_of(h->skip_if_nonzero, 8));
}

// True if r overlaps any range of `sorted` (sorted by start, disjoint).
bool hits_sorted(const std::vector<Range>& sorted, const Range& r) {
  auto it = std::upper_bound(sorted.begin(), sorted.end(), r.lo,
                             [](uintptr_t a, const Range& x) { return a < x.hi; });
  return it != sorted.end() && it->lo < r.hi;
}

// True if any two of the ranges overlap (empty ranges never do).
bool any_overlap(std::vector<Range>& r) {
  r.erase(std::remove_if(r.begin(), r.end(), [](const Range& x) { return x.hi == x.lo; }), r.end());
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < r.size(); ++i)
    if (r[i].lo < r[i - 1].hi) return true;
  return false;
}

// One tensor of an elementwise mode: pointers of the tensor, checked.
struct ElemTensor {
  void* p;
  const void* g;
  void* s0;
  float* s1;
  size_t n;
  int phase;
};

size_t dtype_size(int dt) { return dt == PA_DT_F32 ? 4 : 2; }
bool valid_dtype(int dt) { return dt == PA_DT_F32 || dt == PA_DT_BF16 || dt == PA_DT_F16; }

// Parameter/gradient element-type pairs with a kernel: equal types, or
// 16-bit parameters with FP32 gradients.
bool valid_dtype_pair(int pdt, int gdt) {
  return valid_dtype(pdt) && valid_dtype(gdt) && (pdt == gdt || gdt == PA_DT_F32);
}

int check_elem_tensor(int mode, int pdt, int gdt, void* p, const void* g, void* state, size_t n,
                      ElemTensor* out, std::vector<Range>* ranges) {
  out->p = p;
  out->g = g;
  out->n = n;
  out->s0 = nullptr;
  out->s1 = nullptr;
  out->phase = 0;
  if (n == 0) return PA_OK;
  if (p == nullptr || g == nullptr || state == nullptr) return PA_ERR_ARG;
  if (mode == PA_FP32) {
    const pa_fp32_state* st = static_cast<const pa_fp32_state*>(state);
    if (st->m == nullptr || st->v == nullptr) return PA_ERR_ARG;
    out->s0 = st->m;
    out->s1 = st->v;
  } else {
    out->s0 = state;
  }
  // Every buffer aligned to its element, and all at one phase in elements
  // modulo 4, so that elements 4k..4k+3 of every stream form one vector.
  const size_t ps = dtype_size(pdt), gs = dtype_size(gdt);
  const uintptr_t pa_ = reinterpret_cast<uintptr_t>(p), ga = reinterpret_cast<uintptr_t>(g);
  if (pa_ % ps || ga % gs) return PA_ERR_ALIGN;
  const uintptr_t ph = (pa_ / ps) & 3u;
  if (((ga / gs) & 3u) != ph) return PA_ERR_ALIGN;
  const void* st_bufs[2] = {out->s0, out->s1};
  const int ns = mode == PA_FP32 ? 2 : 1;
  for (int i = 0; i < ns; ++i) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(st_bufs[i]);
    if (a % 4 || ((a / 4) & 3u) != ph) return PA_ERR_ALIGN;
  }
  out->phase = (int)ph;
  ranges->push_back(range_of(p, n * ps));
  ranges->push_back(range_of(g, n * gs));
  for (int i = 0; i < ns; ++i) ranges->push_back(range_of(st_bufs[i], n * 4));
  return PA_OK;
}

pa::Entry make_entry(const ElemTensor& t, long long tile0) {
  pa::Entry e;
  e.p = t.p;
  e.g = t.g;
  e.s0 = t.s0;
  e.s1 = t.s1;
  e.n = (long long)t.n;
  e.tile0 = tile0;
  e.phase = t.phase;
  e.pad_ = 0;
  return e;
}

// Tiles of a tensor at `unroll` vectors per thread (1024 * unroll elements).
long long tiles_of(const pa::Entry& e, int unroll = pa::kUnroll) {
  const long long t = 1024LL * unroll;
  return (e.n + e.phase + t - 1) / t;
}

// The tile size of a list of `total` elements (see kSmallList).
int unroll_for(unsigned long long total) { return total < (unsigned long long)pa::kSmallList ? pa::kSmallUnroll : pa::kUnroll; }

// ---------------------------------------------------------------- launches

// Workgroups of one launch of the one-tile-per-workgroup kernels: a launch
// of more tiles is split into several (the dispatch packet counts work
// items in 32 bits).
constexpr long long kMaxLaunchTiles = 1LL << 22;

// One elementwise kernel over `tiles` tiles, one workgroup per tile, in
// launches of at most kMaxLaunchTiles workgroups; `launch(kernel, grid,
// tile_base)` issues one launch.
template <typename K, typename F>
hipError_t launch_tiles(long long tiles, K kernel, F&& launch) {
  for (long long base = 0; base < tiles; base += kMaxLaunchTiles) {
    launch(kernel, dim3((unsigned)std::min(kMaxLaunchTiles, tiles - base)), base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int MODE, int PT, int GT, bool COUNT, bool SCALE, int UNROLL>
hipError_t launch_one_v(const pa::Entry& e, long long tiles, const pa::Scalars& s, unsigned long long* nf,
                        hipStream_t st) {
  return launch_tiles(tiles, pa::elementwise_one<MODE, PT, GT, COUNT, SCALE, UNROLL>,
                      [&](auto k, dim3 grid, long long base) {
                        hipLaunchKernelGGL(k, grid, dim3(pa::kThreads), 0, st, e, base, s, nf);
                      });
}

// Kernel variant: with or without the non-finite counter, with or without
// a device gradient scale, and the tile size.
template <int MODE, int PT, int GT, int UNROLL>
hipError_t launch_one_u(const pa::Entry& e, long long tiles, const pa::Scalars& s, unsigned long long* nf,
                        hipStream_t st) {
  const bool sc = s.gscale != nullptr;
  if (nf && sc) return launch_one_v<MODE, PT, GT, true, true, UNROLL>(e, tiles, s, nf, st);
  if (nf) return launch_one_v<MODE, PT, GT, true, false, UNROLL>(e, tiles, s, nf, st);
  if (sc) return launch_one_v<MODE, PT, GT, false, true, UNROLL>(e, tiles, s, nf, st);
  return launch_one_v<MODE, PT, GT, false, false, UNROLL>(e, tiles, s, nf, st);
}

template <int MODE, int PT, int GT>
hipError_t launch_one(const pa::Entry& e, int unroll, long long tiles, const pa::Scalars& s, unsigned long long* nf,
                      hipStream_t st) {
  if (unroll == pa::kSmallUnroll) return launch_one_u<MODE, PT, GT, pa::kSmallUnroll>(e, tiles, s, nf, st);
  return launch_one_u<MODE, PT, GT, pa::kUnroll>(e, tiles, s, nf, st);
}

template <int MODE, int PT, int GT, bool COUNT, bool SCALE, int UNROLL>
hipError_t launch_list_v(const pa::Entry* table, int count, long long tiles, const pa::Scalars& s,
                         unsigned long long* nf, hipStream_t st) {
  return launch_tiles(tiles, pa::elementwise_list<MODE, PT, GT, COUNT, SCALE, UNROLL>,
                      [&](auto k, dim3 grid, long long base) {
                        hipLaunchKernelGGL(k, grid, dim3(pa::kThreads), 0, st, table, count, base, s, nf);
                      });
}

template <int MODE, int PT, int GT, int UNROLL>
hipError_t launch_list_u(const pa::Entry* table, int count, long long tiles, const pa::Scalars& s,
                         unsigned long long* nf, hipStream_t st) {
  const bool sc = s.gscale != nullptr;
  if (nf && sc) return launch_list_v<MODE, PT, GT, true, true, UNROLL>(table, count, tiles, s, nf, st);
  if (nf) return launch_list_v<MODE, PT, GT, true, false, UNROLL>(table, count, tiles, s, nf, st);
  if (sc) return launch_list_v<MODE, PT, GT, false, true, UNROLL>(table, count, tiles, s, nf, st);
  return launch_list_v<MODE, PT, GT, false, false, UNROLL>(table, count, tiles, s, nf, st);
}

template <int MODE, int PT, int GT>
hipError_t launch_list(const pa::Entry* table, int count, int unroll, long long tiles, const pa::Scalars& s,
                       unsigned long long* nf, hipStream_t st) {
  if (unroll == pa::kSmallUnroll) return launch_list_u<MODE, PT, GT, pa::kSmallUnroll>(table, count, tiles, s, nf, st);
  return launch_list_u<MODE, PT, GT, pa::kUnroll>(table, count, tiles, s, nf, st);
}

// One launch for a (mode, parameter type, gradient type) triple; `L` is
// launch_one or launch_list through the two lambdas below.
template <int MODE, typename F>
hipError_t by_types(int pdt, int gdt, F&& f) {
  if (pdt == PA_DT_F32) return f(std::integral_constant<int, MODE>(), std::integral_constant<int, pa::kF32>(),
                                 std::integral_constant<int, pa::kF32>());
  if (pdt == PA_DT_BF16 && gdt == PA_DT_BF16)
    return f(std::integral_constant<int, MODE>(), std::integral_constant<int, pa::kBF16>(),
             std::integral_constant<int, pa::kBF16>());
  if (pdt == PA_DT_BF16)
    return f(std::integral_constant<int, MODE>(), std::integral_constant<int, pa::kBF16>(),
             std::integral_constant<int, pa::kF32>());
  if (gdt == PA_DT_F16)
    return f(std::integral_constant<int, MODE>(), std::integral_constant<int, pa::kF16>(),
             std::integral_constant<int, pa::kF16>());
  return f(std::integral_constant<int, MODE>(), std::integral_constant<int, pa::kF16>(),
           std::integral_constant<int, pa::kF32>());
}

template <typename F>
hipError_t by_mode(int mode, int pdt, int gdt, F&& f) {
  switch (mode) {
    case PA_FP32: return by_types<pa::kModeFp32>(pdt, gdt, f);
    case PA_PACKED_E4: return by_types<pa::kModeE4>(pdt, gdt, f);
    default: return by_types<pa::kModeF16>(pdt, gdt, f);
  }
}

hipError_t dispatch_one(int mode, int pdt, int gdt, const pa::Entry& e, int unroll, long long tiles,
                        const pa::Scalars& s, unsigned long long* nf, hipStream_t st) {
  return by_mode(mode, pdt, gdt, [&](auto m, auto pt, auto gt) {
    return launch_one<decltype(m)::value, decltype(pt)::value, decltype(gt)::value>(e, unroll, tiles, s, nf, st);
  });
}

hipError_t dispatch_list(int mode, int pdt, int gdt, const pa::Entry* table, int count, int unroll, long long tiles,
                         const pa::Scalars& s, unsigned long long* nf, hipStream_t st) {
  return by_mode(mode, pdt, gdt, [&](auto m, auto pt, auto gt) {
    return launch_list<decltype(m)::value, decltype(pt)::value, decltype(gt)::value>(table, count, unroll, tiles, s,
                                                                                     nf, st);
  });
}

// Blockwise: check one tensor's buffers.
int check_blockwise(const float* p, const float* g, const void* state, size_t n, pa::BlockwiseArgs* a,
                    std::vector<Range>* ranges) {
  if (n == 0) return PA_OK;
  if (p == nullptr || g == nullptr || state == nullptr) return PA_ERR_ARG;
  const pa_blockwise_state* st = static_cast<const pa_blockwise_state*>(state);
  if (!st->m_code || !st->m_absmax || !st->v_code || !st->v_absmax || !st->qmap_m || !st->qmap_v ||
      !st->p_out_bf16)
    return PA_ERR_ARG;
  if (n % pa::kBlock != 0) return PA_ERR_SHAPE;
  if (!aligned(p, 16) || !aligned(g, 16) || !aligned(st->m_code, 4) || !aligned(st->v_code, 4) ||
      !aligned(st->m_absmax, 4) || !aligned(st->v_absmax, 4) || !aligned(st->qmap_m, 4) ||
      !aligned(st->qmap_v, 4) || !aligned(st->p_out_bf16, 8))
    return PA_ERR_ALIGN;
  const size_t nb = n / pa::kBlock;
  a->p = p;
  a->g = g;
  a->m_code = st->m_code;
  a->m_absmax = st->m_absmax;
  a->v_code = st->v_code;
  a->v_absmax = st->v_absmax;
  a->qmap_m = st->qmap_m;
  a->qmap_v = st->qmap_v;
  a->p_out = st->p_out_bf16;
  a->nblocks = (long long)nb;
  // Written buffers must not overlap anything; the read-only inputs (p, g,
  // the maps) may overlap one another.
  ranges->push_back(range_of(st->m_code, n));
  ranges->push_back(range_of(st->v_code, n));
  ranges->push_back(range_of(st->m_absmax, nb * 4));
  ranges->push_back(range_of(st->v_absmax, nb * 4));
  ranges->push_back(range_of(st->p_out_bf16, n * 2));
  return PA_OK;
}

int blockwise_inputs_clear(const pa::BlockwiseArgs& a, size_t n, std::vector<Range> written) {
  const Range ro[4] = {range_of(a.p, n * 4), range_of(a.g, n * 4), range_of(a.qmap_m, 1024),
                       range_of(a.qmap_v, 1024)};
  for (const Range& w : written)
    for (const Range& r : ro)
      if (w.hi > w.lo && r.lo < w.hi && w.lo < r.hi) return PA_ERR_ALIAS;
  return PA_OK;
}

// The blockwise tables of the ordered launch: one device buffer per (device,
// stream), built by blockwise_tables before each launch.  Calls ordered on one
// stream reuse its buffer in turn; calls on other streams have their own.  A
// call under graph capture takes the persistent launch, so no graph holds a
// buffer (which a later eviction could free).
struct BwBuffer {
  int dev;
  hipStream_t st;
  pa::BwTables* tabs;
};
std::mutex g_bw_mu;
std::list<BwBuffer> g_bw_buffers;   // guarded by g_bw_mu, most recent first
constexpr size_t kMaxBwBuffers = 16;
std::atomic<long long> g_bw_force{0};   // pa_debug_blockwise_path
// Blocks per workgroup of the ordered launch, and the workgroup rounds of a
// tensor below which it keeps the persistent launch.
constexpr long long kBwPerGroup = 12;
constexpr long long kBwMinRounds = 4;

bool capturing(hipStream_t st);

// The table buffer of (dev, st), allocated on first use; nullptr when the
// allocation fails (the caller then takes the persistent launch, which needs
// none).  The caller holds g_bw_mu until its launches are enqueued, so no
// other thread frees the buffer in between.
pa::BwTables* bw_tables_for(int dev, hipStream_t st) {
  for (auto it = g_bw_buffers.begin(); it != g_bw_buffers.end(); ++it)
    if (it->dev == dev && it->st == st) {
      g_bw_buffers.splice(g_bw_buffers.begin(), g_bw_buffers, it);
      return g_bw_buffers.front().tabs;
    }
  pa::BwTables* t = nullptr;
  if (hipMalloc(&t, sizeof(pa::BwTables)) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_bw_buffers.push_front(BwBuffer{dev, st, t});
  while (g_bw_buffers.size() > kMaxBwBuffers) {
    (void)hipFree(g_bw_buffers.back().tabs);   // waits for the work that reads it
    g_bw_buffers.pop_back();
  }
  return t;
}

// Persistent launch (tables built per workgroup) for small tensors, for
// pa_step_list_noalloc, under graph capture and when no table buffer can be
// had; otherwise the
// tables are built once into the stream's buffer and the ordered launch
// takes kBwPerGroup blocks per workgroup.
hipError_t launch_blockwise(const pa::BlockwiseArgs& a, const pa::Scalars& s, unsigned long long* nf,
                            hipStream_t st, int dev, const DeviceInfo& d, bool noalloc) {
  const bool sc = s.gscale != nullptr;
  const long long slots = (long long)d.cus * d.bw_blocks_per_cu;
  const long long force = g_bw_force.load();
  long long per = 0;
  if (force > 0) per = force;
  else if (force == 0 && a.nblocks >= kBwPerGroup * kBwMinRounds * slots) per = kBwPerGroup;
  std::unique_lock<std::mutex> lk(g_bw_mu, std::defer_lock);
  pa::BwTables* tabs = nullptr;
  if (per > 0 && !noalloc && !capturing(st)) {
    lk.lock();
    tabs = bw_tables_for(dev, st);
  }
  const dim3 block(pa::kThreads);
  if (tabs != nullptr) {
    hipLaunchKernelGGL(pa::blockwise_tables, dim3(1), block, 0, st, a.qmap_m, a.qmap_v, tabs);
    const dim3 grid((unsigned)((a.nblocks + per - 1) / per));
    const long long one = 1;
    if (nf && sc) hipLaunchKernelGGL((pa::blockwise_kernel<true, true, true>), grid, block, 0, st, a, s, nf, tabs, per, one);
    else if (nf) hipLaunchKernelGGL((pa::blockwise_kernel<true, false, true>), grid, block, 0, st, a, s, nf, tabs, per, one);
    else if (sc) hipLaunchKernelGGL((pa::blockwise_kernel<false, true, true>), grid, block, 0, st, a, s, nf, tabs, per, one);
    else hipLaunchKernelGGL((pa::blockwise_kernel<false, false, true>), grid, block, 0, st, a, s, nf, tabs, per, one);
    return hipGetLastError();
  }
  const long long g = grid_for(a.nblocks, d, d.bw_blocks_per_cu);
  const dim3 grid((unsigned)g);
  const pa::BwTables* none = nullptr;
  if (nf && sc) hipLaunchKernelGGL((pa::blockwise_kernel<true, true, false>), grid, block, 0, st, a, s, nf, none, 0LL, g);
  else if (nf) hipLaunchKernelGGL((pa::blockwise_kernel<true, false, false>), grid, block, 0, st, a, s, nf, none, 0LL, g);
  else if (sc) hipLaunchKernelGGL((pa::blockwise_kernel<false, true, false>), grid, block, 0, st, a, s, nf, none, 0LL, g);
  else hipLaunchKernelGGL((pa::blockwise_kernel<false, false, false>), grid, block, 0, st, a, s, nf, none, 0LL, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------- tables

// Validates the tensors of an elementwise list and builds its table: the
// tensors of length 0 left out, a sentinel whose tile0 is the total tile
// count appended (none for an empty list).  `ranges` receives every buffer
// of the list, sorted and checked disjoint.
int build_elem_table(int mode, int pdt, int gdt, size_t count, void* const* params, const void* const* grads,
                     void* const* states, const size_t* n, int unroll, std::vector<pa::Entry>* host,
                     std::vector<Range>* ranges, long long* tiles_out) {
  long long tiles = 0;
  for (size_t i = 0; i < count; ++i) {
    ElemTensor t;
    const int rc = check_elem_tensor(mode, pdt, gdt, params[i], grads[i], states[i], n[i], &t, ranges);
    if (rc) return rc;
    if (t.n == 0) continue;
    pa::Entry e = make_entry(t, tiles);
    tiles += tiles_of(e, unroll);
    host->push_back(e);
  }
  if (any_overlap(*ranges)) return PA_ERR_ALIAS;
  if (host->size() > (size_t)INT32_MAX) return PA_ERR_ARG;
  if (!host->empty()) {
    pa::Entry sentinel;
    std::memset(&sentinel, 0, sizeof(sentinel));
    sentinel.tile0 = tiles;
    host->push_back(sentinel);
  }
  *tiles_out = tiles;
  return PA_OK;
}

// The device words named by a pa_hyper against the list's buffers (sorted,
// disjoint) and against each other.
int hyper_clear(const pa_hyper* hyper, const std::vector<Range>& sorted) {
  std::vector<Range> hr;
  hyper_ranges(hyper, &hr);
  for (const Range& r : hr)
    if (hits_sorted(sorted, r)) return PA_ERR_ALIAS;
  if (any_overlap(hr)) return PA_ERR_ALIAS;
  return PA_OK;
}

// ---------------------------------------------------------------- no-allocation tables

// The tensor table of pa_step_list_noalloc lives in this array: each GPU the
// library runs on holds its own copy until the process ends.  Host code
// never uses the array's name as an address; it takes the device address
// from hipGetSymbolAddress, once per device (scratch_table).
static __device__ __align__(256) unsigned char scratch[(PA_NOALLOC_MAX_TENSORS + 1) * sizeof(pa::Entry)];

std::mutex g_scratch_mu;
pa::Entry* g_scratch_table[64] = {};

// The device address of `scratch` on device `dev` (the current device).
int scratch_table(int dev, pa::Entry** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_table[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return hip_failed(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch_table[dev] = static_cast<pa::Entry*>(ptr);
  }
  *out = g_scratch_table[dev];
  return PA_OK;
}

// Table entries written by kernels whose arguments carry them: the upload is
// ordered on the stream like the step that reads it, and keeps no host
// buffer alive past the call.
constexpr int kUploadEntries = 32;
struct EntryChunk {
  pa::Entry e[kUploadEntries];
};

__global__ void __launch_bounds__(64) upload_entries(pa::Entry* dst, EntryChunk chunk, int n) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = chunk.e[i];
}

hipError_t upload_table(pa::Entry* dst, const std::vector<pa::Entry>& host, hipStream_t st) {
  for (size_t i = 0; i < host.size(); i += kUploadEntries) {
    EntryChunk c;
    std::memset(&c, 0, sizeof(c));
    const int m = (int)std::min<size_t>(kUploadEntries, host.size() - i);
    std::memcpy(c.e, host.data() + i, (size_t)m * sizeof(pa::Entry));
    hipLaunchKernelGGL(upload_entries, dim3(1), dim3(64), 0, st, dst + i, c, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Gradient pointers written into a cached table by kernels whose arguments
// carry them, so that a list whose gradients move between calls (torch
// allocates fresh gradients after zero_grad(set_to_none=True)) keeps its
// plan: no allocation, no copy from host memory, no synchronisation, and
// the write is ordered on the stream before the step that reads it.
constexpr int kPatchPointers = 64;
struct PointerChunk {
  const void* v[kPatchPointers];
};

__global__ void __launch_bounds__(64) patch_pointers(char* base, long long stride, long long offset, PointerChunk c,
                                                     int n) {
  const int i = threadIdx.x;
  if (i < n) *reinterpret_cast<const void**>(base + (long long)i * stride + offset) = c.v[i];
}

// Writes vals[j] into the pointer field at `offset` of entries 0..vals.size()-1
// of a device table whose entries are `stride` bytes apart.
hipError_t patch_table(void* table, size_t stride, size_t offset, const std::vector<const void*>& vals,
                       hipStream_t st) {
  for (size_t j = 0; j < vals.size(); j += kPatchPointers) {
    PointerChunk c;
    std::memset(&c, 0, sizeof(c));
    const int m = (int)std::min<size_t>(kPatchPointers, vals.size() - j);
    for (int k = 0; k < m; ++k) c.v[k] = vals[j + k];
    hipLaunchKernelGGL(patch_pointers, dim3(1), dim3(64), 0, st, static_cast<char*>(table) + j * stride,
                       (long long)stride, (long long)offset, c, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Whether `st` is being captured into a graph (a failed query counts as no).
bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive;
}

// ---------------------------------------------------------------- plans

struct Plan {
  int device = -1;
  int mode = -1;
  int pdt = 0, gdt = 0;
  std::vector<uintptr_t> key;   // per tensor: p, s0, s1, n (pre-pass: n and phase); not the gradients
  pa::Entry* table = nullptr;   // device memory, count+1 entries (+ partials of a pre-pass plan)
  int count = 0;                // tensors in the table (the sentinel not counted)
  long long tiles = 0;
  std::vector<Range> ranges;    // the tensors' buffers, sorted and disjoint
  std::vector<Range> written;   // the written ones alone (sorted, disjoint)
  std::vector<const void*> grads;   // the gradient pointer of each table entry, as last written
  bool captured = false;        // a graph has captured a call on this plan
  double* part_sum = nullptr;   // pre-pass plans: per-workgroup partials, inside `table`'s block
  unsigned long long* part_bad = nullptr;
  int nparts = 0;
};

std::mutex g_plan_mu;
std::list<Plan> g_plans;       // most recently used first
constexpr size_t kMaxPlans = 16;

void free_plan(Plan& pl) {
  if (pl.table) {
    int cur = 0;
    if (hipGetDevice(&cur) == hipSuccess) {
      if (hipSetDevice(pl.device) == hipSuccess) (void)hipFree(pl.table);
      (void)hipSetDevice(cur);
    }
    pl.table = nullptr;
  }
}

bool valid_mode(int mode) { return mode >= PA_FP32 && mode <= PA_BLOCKWISE8; }

constexpr int kStatsPlanMode = 100;   // plan-cache tag of gradient pre-pass plans

// Sorted, disjoint union of the ranges (empty ones dropped).
std::vector<Range> merged(std::vector<Range> r) {
  r.erase(std::remove_if(r.begin(), r.end(), [](const Range& x) { return x.hi == x.lo; }), r.end());
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  std::vector<Range> out;
  for (const Range& x : r) {
    if (!out.empty() && x.lo <= out.back().hi) out.back().hi = std::max(out.back().hi, x.hi);
    else out.push_back(x);
  }
  return out;
}

// Gradient lists above this size read with nontemporal loads: the step that
// follows would miss the last-level cache (256 MB on MI355X) for them anyway,
// and streaming loads read HBM about 11% faster (7B list: 4.4 -> 3.95 ms).
constexpr double kStatsStreamBytes = 128.0 * 1024 * 1024;

template <int GT>
hipError_t launch_stats(const Plan& pl, double max_norm, double* sumsq, unsigned long long* nonfinite,
                        float* clip, hipStream_t st) {
  if (pl.nparts > 0) {
    const double bytes = (double)pl.tiles * pa::kTile * (GT == pa::kF32 ? 4 : 2);
    const dim3 grid((unsigned)pl.nparts), block(pa::kThreads);
    if (bytes > kStatsStreamBytes)
      hipLaunchKernelGGL((pa::grad_stats_list<GT, true>), grid, block, 0, st, pl.table, pl.tiles, pl.part_sum,
                         pl.part_bad);
    else
      hipLaunchKernelGGL((pa::grad_stats_list<GT, false>), grid, block, 0, st, pl.table, pl.tiles, pl.part_sum,
                         pl.part_bad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(pa::grad_stats_finalize, dim3(1), dim3(pa::kThreads), 0, st, pl.part_sum, pl.part_bad,
                     pl.nparts, max_norm, sumsq, nonfinite, clip);
  return hipGetLastError();
}

// ---------------------------------------------------------------- TurboAdam

// Table entries carry the element types as the kernels' type codes.
static_assert(PA_DT_F32 == pa::kF32 && PA_DT_BF16 == pa::kBF16 && PA_DT_F16 == pa::kF16, "dtype codes");

struct TurboPlan {
  int device = -1;
  std::vector<uintptr_t> key;
  pa::TurboEntry* table = nullptr;          // device: entries + sentinel, then the reduce list
  pa::TurboReduceEntry* reduce = nullptr;   // inside the same allocation
  long long tiles = 0;                      // 256-value tiles, or 1024-value ones on the general path
  int count = 0;                            // entries before the sentinel
  bool general = false;                     // turbo_general instead of turbo_list
  bool typed = false;                       // 16-bit parameters or gradients
  int blog = 7, glog = 6;                   // log2 of the 1Q block and of the UState group
  int nreduce = 0;
  long long nchunks = 0;                    // chunks of tile sums over all UState tensors
  size_t ws_bytes = 0;
  std::vector<Range> ranges;                // written buffers and gradients, merged
  std::vector<Range> written;               // the written buffers alone, merged
  std::vector<const void*> grads;           // the gradient pointer of each entry, as last written
  bool captured = false;                    // a graph has captured a call on this plan
};

std::list<TurboPlan> g_turbo_plans;         // guarded by g_plan_mu, most recent first

void free_turbo_plan(TurboPlan& pl) {
  if (pl.table) {
    int cur = 0;
    if (hipGetDevice(&cur) == hipSuccess) {
      if (hipSetDevice(pl.device) == hipSuccess) (void)hipFree(pl.table);
      (void)hipSetDevice(cur);
    }
    pl.table = nullptr;
  }
}

long long turbo_tiles(size_t n) { return (long long)((n + pa::kTurboTile - 1) / pa::kTurboTile); }
long long turbo_chunks_of(long long tiles) { return (tiles + pa::kTurboChunk - 1) / pa::kTurboChunk; }

// A layout the page's fused path takes: 2, 3, 4, 6 or 8 index bits, a
// power-of-two 1Q block from 32 to 1024 values, a power-of-two UState group
// dividing it.  The tuned kernel (turbo_list) covers 128-value blocks and
// 64-value groups at every width; turbo_general covers every layout.
struct TurboLayout {
  int bits = 4, block = 128, group = 64;
  bool general = false;
};

int log2_exact(int x) { return 31 - __builtin_clz((unsigned)x); }

bool layout_ok(int bits, int block, int group) {
  if (bits != 2 && bits != 3 && bits != 4 && bits != 6 && bits != 8) return false;
  if (block < 32 || block > 1024 || (block & (block - 1))) return false;
  return group >= 1 && group <= block && (group & (group - 1)) == 0;
}

int turbo_layout(const pa_turbo_config* c, TurboLayout* out) {
  out->bits = c->v_bits;
  out->block = c->block_size ? c->block_size : 128;
  out->group = c->m_block_size ? c->m_block_size : 64;
  if (!layout_ok(out->bits, out->block, out->group) || (c->path != 0 && c->path != 1)) return PA_ERR_ARG;
  out->general = c->path == 1 || out->block != 128 || out->group != 64;
  return PA_OK;
}

// Checks one tensor's buffers; appends the written ranges to `w` and the
// gradient range to `r`.
// The draws' counter words hold value index / 4 and the step in 32 bits.
constexpr size_t kTurboMaxValues = size_t(1) << 34;
constexpr long long kTurboMaxStep = 0xFFFFFFFFll;

int check_turbo_tensor(int pdt, int gdt, const void* p, const void* g, const pa_turbo_state& st, size_t n,
                       const TurboLayout& lay, std::vector<Range>* w, std::vector<Range>* r) {
  const size_t bits = (size_t)lay.bits, B = (size_t)lay.block, G = (size_t)lay.group;
  if (n == 0) return PA_OK;
  if (p == nullptr || g == nullptr) return PA_ERR_ARG;
  // A lane reads and writes four consecutive values as one vector.
  if (!aligned(p, 4 * dtype_size(pdt)) || !aligned(g, 4 * dtype_size(gdt))) return PA_ERR_ALIGN;
  w->push_back(range_of(p, n * dtype_size(pdt)));
  r->push_back(range_of(g, n * dtype_size(gdt)));
  if (st.compress_m) {
    if (!st.m_codes || !st.m_means || !st.scalars) return PA_ERR_ARG;
    if (!aligned(st.m_codes, 4) || !aligned(st.m_means, 2) || !aligned(st.scalars, 4)) return PA_ERR_ALIGN;
    w->push_back(range_of(st.m_codes, 4 * ((n + 15) / 16)));
    w->push_back(range_of(st.m_means, 2 * ((n + G - 1) / G)));
    w->push_back(range_of(st.scalars, 12));
  } else {
    if (!st.m_fp32) return PA_ERR_ARG;
    if (!aligned(st.m_fp32, 16)) return PA_ERR_ALIGN;
    w->push_back(range_of(st.m_fp32, n * 4));
  }
  if (st.compress_v) {
    if (!st.v_index || !st.v_ends) return PA_ERR_ARG;
    if (!aligned(st.v_index, 4) || !aligned(st.v_ends, 4)) return PA_ERR_ALIGN;
    w->push_back(range_of(st.v_index, 4 * ((n * bits + 31) / 32)));
    w->push_back(range_of(st.v_ends, 4 * ((n + B - 1) / B)));
  } else {
    if (!st.v_fp32) return PA_ERR_ARG;
    if (!aligned(st.v_fp32, 16)) return PA_ERR_ALIGN;
    w->push_back(range_of(st.v_fp32, n * 4));
  }
  return PA_OK;
}

// The residual sums' chunk pass and the per-tensor completion with the
// scale rotation, after either step kernel.
hipError_t launch_turbo_reduce(const TurboPlan& pl, const pa::Scalars& s, double* ws, double factor,
                               hipStream_t st) {
  if (pl.nreduce == 0) return hipSuccess;
  hipLaunchKernelGGL(pa::turbo_chunks, dim3((unsigned)pl.nchunks), dim3(pa::kThreads), 0, st, pl.reduce,
                     pl.nreduce, ws);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The reduce kernel checks the same skip flag: a skipped update leaves
  // the scales as they were.
  hipLaunchKernelGGL(pa::turbo_reduce, dim3((unsigned)pl.nreduce), dim3(pa::kThreads), 0, st, pl.reduce, ws, factor,
                     s.skip);
  return hipGetLastError();
}

// The tuned kernel: one wavefront per 256-value tile, four per workgroup,
// in launches of at most kMaxLaunchTiles workgroups.
template <int BITS, bool TYPED>
hipError_t launch_turbo_as(const TurboPlan& pl, const pa::Scalars& s, const pa::TurboScalars& ts, double* ws,
                           unsigned long long* nf, double factor, hipStream_t st) {
  constexpr long long kWaves = pa::kThreads / 64;
  const long long wgs = (pl.tiles + kWaves - 1) / kWaves;
  for (long long w0 = 0; w0 < wgs; w0 += kMaxLaunchTiles) {
    const long long nw = std::min(kMaxLaunchTiles, wgs - w0);
    if (nf)
      hipLaunchKernelGGL((pa::turbo_list<BITS, true, TYPED>), dim3((unsigned)nw), dim3(pa::kThreads), 0, st,
                         pl.table, pl.count, pl.tiles, w0 * kWaves, s, ts, ws, nf);
    else
      hipLaunchKernelGGL((pa::turbo_list<BITS, false, TYPED>), dim3((unsigned)nw), dim3(pa::kThreads), 0, st,
                         pl.table, pl.count, pl.tiles, w0 * kWaves, s, ts, ws, nf);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_turbo_reduce(pl, s, ws, factor, st);
}

template <int BITS>
hipError_t launch_turbo(const TurboPlan& pl, const pa::Scalars& s, const pa::TurboScalars& ts, double* ws,
                        unsigned long long* nf, double factor, hipStream_t st) {
  return pl.typed ? launch_turbo_as<BITS, true>(pl, s, ts, ws, nf, factor, st)
                  : launch_turbo_as<BITS, false>(pl, s, ts, ws, nf, factor, st);
}

// The general kernel: one workgroup per 1024-value tile, in launches of at
// most kMaxLaunchTiles workgroups.
template <int BITS, bool TYPED>
hipError_t launch_general_as(const TurboPlan& pl, const pa::Scalars& s, const pa::TurboScalars& ts, double* ws,
                             unsigned long long* nf, double factor, hipStream_t st) {
  for (long long t0 = 0; t0 < pl.tiles; t0 += kMaxLaunchTiles) {
    const long long nt = std::min(kMaxLaunchTiles, pl.tiles - t0);
    if (nf)
      hipLaunchKernelGGL((pa::turbo_general<BITS, true, TYPED>), dim3((unsigned)nt), dim3(pa::kThreads), 0, st,
                         pl.table, pl.count, t0, s, ts, pl.blog, pl.glog, ws, nf);
    else
      hipLaunchKernelGGL((pa::turbo_general<BITS, false, TYPED>), dim3((unsigned)nt), dim3(pa::kThreads), 0, st,
                         pl.table, pl.count, t0, s, ts, pl.blog, pl.glog, ws, nf);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_turbo_reduce(pl, s, ws, factor, st);
}

template <int BITS>
hipError_t launch_general(const TurboPlan& pl, const pa::Scalars& s, const pa::TurboScalars& ts, double* ws,
                          unsigned long long* nf, double factor, hipStream_t st) {
  return pl.typed ? launch_general_as<BITS, true>(pl, s, ts, ws, nf, factor, st)
                  : launch_general_as<BITS, false>(pl, s, ts, ws, nf, factor, st);
}

}  // namespace

// =================================================================== C ABI

extern "C" {

int pa_step_typed(int mode, int param_dtype, int grad_dtype, void* params, const void* grads, void* state,
                  size_t n, const pa_hyper* hyper, long long step, void* stream) {
  if (!valid_mode(mode) || !valid_dtype_pair(param_dtype, grad_dtype)) return PA_ERR_ARG;
  if (mode == PA_BLOCKWISE8 && (param_dtype != PA_DT_F32 || grad_dtype != PA_DT_F32)) return PA_ERR_ARG;
  pa::Scalars s;
  int rc = make_scalars(hyper, step, &s);
  if (rc) return rc;
  if (n == 0) return PA_OK;
  int dev;
  DeviceInfo d;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mode == PA_BLOCKWISE8) {
    pa::BlockwiseArgs a;
    std::vector<Range> w;
    rc = check_blockwise(static_cast<const float*>(params), static_cast<const float*>(grads), state, n, &a, &w);
    if (rc) return rc;
    hyper_ranges(hyper, &w);
    if (any_overlap(w)) return PA_ERR_ALIAS;
    rc = blockwise_inputs_clear(a, n, w);
    if (rc) return rc;
    rc = device_info(&dev, &d);
    if (rc) return rc;
    hipError_t e = launch_blockwise(a, s, hyper->nonfinite, st, dev, d, false);
    return e == hipSuccess ? PA_OK : hip_failed(e);
  }
  ElemTensor t;
  std::vector<Range> ranges;
  rc = check_elem_tensor(mode, param_dtype, grad_dtype, params, grads, state, n, &t, &ranges);
  if (rc) return rc;
  hyper_ranges(hyper, &ranges);
  if (any_overlap(ranges)) return PA_ERR_ALIAS;
  rc = device_info(&dev, &d);
  if (rc) return rc;
  const pa::Entry e = make_entry(t, 0);
  const int unroll = unroll_for(n);
  hipError_t err = dispatch_one(mode, param_dtype, grad_dtype, e, unroll, tiles_of(e, unroll), s, hyper->nonfinite, st);
  return err == hipSuccess ? PA_OK : hip_failed(err);
}

int pa_step(int mode, float* params, const float* grads, void* state, size_t n, const pa_hyper* hyper,
            long long step, void* stream) {
  return pa_step_typed(mode, PA_DT_F32, PA_DT_F32, params, grads, state, n, hyper, step, stream);
}

}  // extern "C"

namespace {

// pa_step_list_typed (noalloc false: the table in a cached plan) and
// pa_step_list_noalloc (noalloc true: the table in `scratch`).
// A cached elementwise plan called with gradients other than those in its
// table: they are checked as at the plan's creation (aligned to their
// element, at the parameters' phase, clear of every written buffer and of
// each other), and on success the plan's ranges and gradient list take them;
// the caller writes them into the device table.  Nothing changes on error.
int refresh_grads(Plan& pl, int pdt, int gdt, size_t count, void* const* params, const void* const* grads,
                  const size_t* n, bool* changed) {
  *changed = false;
  std::vector<const void*> g;
  g.reserve(pl.grads.size());
  for (size_t i = 0; i < count; ++i)
    if (n[i] > 0) g.push_back(grads[i]);
  if (g == pl.grads) return PA_OK;
  if (g.size() != pl.grads.size()) return PA_ERR_ARG;
  const size_t ps = dtype_size(pdt), gs = dtype_size(gdt);
  std::vector<Range> gr;
  for (size_t i = 0; i < count; ++i) {
    if (n[i] == 0) continue;
    if (grads[i] == nullptr) return PA_ERR_ARG;
    const uintptr_t ga = reinterpret_cast<uintptr_t>(grads[i]), pa_ = reinterpret_cast<uintptr_t>(params[i]);
    if (ga % gs || ((ga / gs) & 3u) != ((pa_ / ps) & 3u)) return PA_ERR_ALIGN;
    gr.push_back(range_of(grads[i], n[i] * gs));
  }
  {
    std::vector<Range> tmp = gr;
    if (any_overlap(tmp)) return PA_ERR_ALIAS;
  }
  for (const Range& r : gr)
    if (hits_sorted(pl.written, r)) return PA_ERR_ALIAS;
  std::vector<Range> all = pl.written;
  all.insert(all.end(), gr.begin(), gr.end());
  pl.ranges = merged(all);
  pl.grads = g;
  *changed = true;
  return PA_OK;
}

int step_list(bool noalloc, int mode, int param_dtype, int grad_dtype, size_t count, void* const* params,
              const void* const* grads, void* const* states, const size_t* n, const pa_hyper* hyper, long long step,
              void* stream) {
  if (!valid_mode(mode) || !valid_dtype_pair(param_dtype, grad_dtype)) return PA_ERR_ARG;
  if (mode == PA_BLOCKWISE8 && (param_dtype != PA_DT_F32 || grad_dtype != PA_DT_F32)) return PA_ERR_ARG;
  pa::Scalars s;
  int rc = make_scalars(hyper, step, &s);
  if (rc) return rc;
  if (count == 0) return PA_OK;
  if (params == nullptr || grads == nullptr || states == nullptr || n == nullptr) return PA_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev;
  DeviceInfo d;

  if (mode == PA_BLOCKWISE8) {
    std::vector<pa::BlockwiseArgs> args;
    std::vector<Range> written;
    for (size_t i = 0; i < count; ++i) {
      if (n[i] == 0) continue;
      pa::BlockwiseArgs a;
      std::vector<Range> w;
      rc = check_blockwise(static_cast<const float*>(params[i]), static_cast<const float*>(grads[i]), states[i],
                           n[i], &a, &w);
      if (rc) return rc;
      written.insert(written.end(), w.begin(), w.end());
      args.push_back(a);
    }
    hyper_ranges(hyper, &written);
    std::vector<Range> all = written;
    if (any_overlap(all)) return PA_ERR_ALIAS;
    for (size_t i = 0; i < args.size(); ++i) {
      rc = blockwise_inputs_clear(args[i], (size_t)args[i].nblocks * pa::kBlock, written);
      if (rc) return rc;
    }
    rc = device_info(&dev, &d);
    if (rc) return rc;
    for (const pa::BlockwiseArgs& a : args) {
      hipError_t e = launch_blockwise(a, s, hyper->nonfinite, st, dev, d, noalloc);
      if (e != hipSuccess) return hip_failed(e);
    }
    return PA_OK;
  }

  unsigned long long total = 0;
  for (size_t i = 0; i < count; ++i) total += n[i];
  const int unroll = unroll_for(total);
  if (noalloc) {
    std::vector<pa::Entry> host;
    std::vector<Range> ranges;
    long long tiles = 0;
    rc = build_elem_table(mode, param_dtype, grad_dtype, count, params, grads, states, n, unroll, &host, &ranges,
                          &tiles);
    if (rc) return rc;
    if (host.empty()) return PA_OK;
    if (host.size() > (size_t)PA_NOALLOC_MAX_TENSORS + 1) return PA_ERR_CAPACITY;
    rc = hyper_clear(hyper, ranges);
    if (rc) return rc;
    rc = device_info(&dev, &d);
    if (rc) return rc;
    pa::Entry* table = nullptr;
    rc = scratch_table(dev, &table);
    if (rc) return rc;
    hipError_t e = upload_table(table, host, st);
    if (e == hipSuccess)
      e = dispatch_list(mode, param_dtype, grad_dtype, table, (int)(host.size() - 1), unroll, tiles, s,
                        hyper->nonfinite, st);
    return e == hipSuccess ? PA_OK : hip_failed(e);
  }

  rc = device_info(&dev, &d);
  if (rc) return rc;

  // Key of this list: every pointer but the gradients', and every length,
  // in order.  The gradients are written into the table when they move.
  std::vector<uintptr_t> key;
  key.reserve(count * 4);
  for (size_t i = 0; i < count; ++i) {
    uintptr_t s0 = reinterpret_cast<uintptr_t>(states[i]), s1 = 0;
    if (mode == PA_FP32 && states[i] != nullptr) {
      const pa_fp32_state* fs = static_cast<const pa_fp32_state*>(states[i]);
      s0 = reinterpret_cast<uintptr_t>(fs->m);
      s1 = reinterpret_cast<uintptr_t>(fs->v);
    }
    key.push_back(reinterpret_cast<uintptr_t>(params[i]));
    key.push_back(s0);
    key.push_back(s1);
    key.push_back((uintptr_t)n[i]);
  }

  std::lock_guard<std::mutex> lk(g_plan_mu);
  auto it = std::find_if(g_plans.begin(), g_plans.end(), [&](const Plan& p) {
    return p.device == dev && p.mode == mode && p.pdt == param_dtype && p.gdt == grad_dtype && p.key == key;
  });
  bool changed = false;
  if (it == g_plans.end()) {
    // Validate and build the table once for this list.
    std::vector<pa::Entry> host;
    std::vector<Range> ranges;
    long long tiles = 0;
    rc = build_elem_table(mode, param_dtype, grad_dtype, count, params, grads, states, n, unroll, &host, &ranges,
                          &tiles);
    if (rc) return rc;
    if (host.empty()) return PA_OK;
    Plan pl;
    pl.device = dev;
    pl.mode = mode;
    pl.pdt = param_dtype;
    pl.gdt = grad_dtype;
    pl.key = key;
    pl.count = (int)(host.size() - 1);
    pl.tiles = tiles;
    pl.ranges = ranges;
    for (size_t j = 0; j + 1 < host.size(); ++j) pl.grads.push_back(host[j].g);
    {
      std::vector<Range> w;
      for (size_t i = 0; i < count; ++i) {
        ElemTensor t;
        std::vector<Range> r;
        (void)check_elem_tensor(mode, param_dtype, grad_dtype, params[i], grads[i], states[i], n[i], &t, &r);
        for (size_t k = 0; k < r.size(); ++k)
          if (k != 1) w.push_back(r[k]);   // every buffer but the gradients (the second)
      }
      pl.written = merged(w);
    }
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&pl.table), host.size() * sizeof(pa::Entry));
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return PA_ERR_NOMEM;
    }
    e = hipMemcpyAsync(pl.table, host.data(), host.size() * sizeof(pa::Entry), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      (void)hipFree(pl.table);
      return hip_failed(e);
    }
    g_plans.push_front(std::move(pl));
    while (g_plans.size() > kMaxPlans) {
      free_plan(g_plans.back());
      g_plans.pop_back();
    }
    it = g_plans.begin();
  } else {
    if (it != g_plans.begin()) {
      g_plans.splice(g_plans.begin(), g_plans, it);
      it = g_plans.begin();
    }
    rc = refresh_grads(*it, param_dtype, grad_dtype, count, params, grads, n, &changed);
    if (rc) return rc;
  }
  const bool cap = capturing(st);
  rc = hyper_clear(hyper, it->ranges);
  if (rc) return rc;
  if (changed || it->captured || cap) {
    // Gradients that moved are written into the table.  A replay rewrites
    // the table with the gradients it captured, so a plan that a graph
    // holds gets its gradients written on every call, and a captured call
    // writes its own.
    const hipError_t pe = patch_table(it->table, sizeof(pa::Entry), offsetof(pa::Entry, g), it->grads, st);
    if (pe != hipSuccess) return hip_failed(pe);
    it->captured = it->captured || cap;
  }
  hipError_t e =
      dispatch_list(mode, param_dtype, grad_dtype, it->table, it->count, unroll, it->tiles, s, hyper->nonfinite, st);
  return e == hipSuccess ? PA_OK : hip_failed(e);
}

}  // namespace

extern "C" {

int pa_step_list_typed(int mode, int param_dtype, int grad_dtype, size_t count, void* const* params,
                       const void* const* grads, void* const* states, const size_t* n, const pa_hyper* hyper,
                       long long step, void* stream) {
  return step_list(false, mode, param_dtype, grad_dtype, count, params, grads, states, n, hyper, step, stream);
}

int pa_step_list_noalloc(int mode, int param_dtype, int grad_dtype, size_t count, void* const* params,
                         const void* const* grads, void* const* states, const size_t* n, const pa_hyper* hyper,
                         long long step, void* stream) {
  return step_list(true, mode, param_dtype, grad_dtype, count, params, grads, states, n, hyper, step, stream);
}



int pa_step_list(int mode, size_t count, float* const* params, const float* const* grads, void* const* states,
                 const size_t* n, const pa_hyper* hyper, long long step, void* stream) {
  return pa_step_list_typed(mode, PA_DT_F32, PA_DT_F32, count, reinterpret_cast<void* const*>(params),
                            reinterpret_cast<const void* const*>(grads), states, n, hyper, step, stream);
}

int pa_grad_stats_list(int grad_dtype, size_t count, const void* const* grads, const size_t* n, double max_norm,
                       double* sumsq, unsigned long long* nonfinite, float* clip_scale, void* stream) {
  if (!valid_dtype(grad_dtype) || sumsq == nullptr) return PA_ERR_ARG;
  if (clip_scale != nullptr && !(std::isfinite(max_norm) && max_norm > 0.0)) return PA_ERR_ARG;
  if (count > 0 && (grads == nullptr || n == nullptr)) return PA_ERR_ARG;
  if (!aligned(sumsq, 8) || !aligned(nonfinite, 8) || !aligned(clip_scale, 4)) return PA_ERR_ALIGN;
  std::vector<Range> outs{range_of(sumsq, 8)};
  if (nonfinite) outs.push_back(range_of(nonfinite, 8));
  if (clip_scale) outs.push_back(range_of(clip_scale, 4));
  {
    std::vector<Range> tmp = outs;
    if (any_overlap(tmp)) return PA_ERR_ALIAS;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev;
  DeviceInfo d;
  int rc = device_info(&dev, &d);
  if (rc) return rc;

  // Key: the stream, and each gradient's length and phase (its position in
  // elements modulo 4, which the table's tiles follow).  The plan holds the
  // per-workgroup partials, so calls on different streams get plans of their
  // own and cannot overwrite each other's partials.  The gradient pointers
  // are written into the table when they move.
  const size_t es = dtype_size(grad_dtype);
  std::vector<uintptr_t> key;
  key.reserve(count * 2 + 1);
  key.push_back(reinterpret_cast<uintptr_t>(stream));
  std::vector<const void*> gnow;
  std::vector<Range> gr;
  for (size_t i = 0; i < count; ++i) {
    key.push_back((uintptr_t)n[i]);
    if (n[i] == 0) {
      key.push_back(0);
      continue;
    }
    if (grads[i] == nullptr) return PA_ERR_ARG;
    const uintptr_t a = reinterpret_cast<uintptr_t>(grads[i]);
    if (a % es) return PA_ERR_ALIGN;
    key.push_back((a / es) & 3u);
    gnow.push_back(grads[i]);
    gr.push_back(range_of(grads[i], n[i] * es));
  }
  std::lock_guard<std::mutex> lk(g_plan_mu);
  auto it = std::find_if(g_plans.begin(), g_plans.end(), [&](const Plan& p) {
    return p.device == dev && p.mode == kStatsPlanMode && p.gdt == grad_dtype && p.key == key;
  });
  bool changed = false;
  if (it == g_plans.end()) {
    std::vector<pa::Entry> host;
    std::vector<Range> ranges;
    long long tiles = 0;
    for (size_t i = 0; i < count; ++i) {
      if (n[i] == 0) continue;
      if (grads[i] == nullptr) return PA_ERR_ARG;
      const uintptr_t a = reinterpret_cast<uintptr_t>(grads[i]);
      if (a % es) return PA_ERR_ALIGN;
      pa::Entry e;
      std::memset(&e, 0, sizeof(e));
      e.g = grads[i];
      e.n = (long long)n[i];
      e.phase = (int)((a / es) & 3u);
      e.tile0 = tiles;
      tiles += tiles_of(e);
      host.push_back(e);
      ranges.push_back(range_of(grads[i], n[i] * es));
    }
    pa::Entry sentinel;
    std::memset(&sentinel, 0, sizeof(sentinel));
    sentinel.tile0 = tiles;
    host.push_back(sentinel);
    Plan pl;
    pl.device = dev;
    pl.mode = kStatsPlanMode;
    pl.pdt = -1;
    pl.gdt = grad_dtype;
    pl.key = key;
    pl.tiles = tiles;
    pl.ranges = merged(ranges);
    pl.grads = gnow;
    pl.nparts = tiles > 0 ? (int)grid_for(tiles, d, d.stats_blocks_per_cu) : 0;
    // One block: the table, then the partial sums and counts (at least one
    // slot each, so the finalizer always gets valid pointers).
    const size_t table_bytes = host.size() * sizeof(pa::Entry);
    const size_t slots = (size_t)std::max(pl.nparts, 1);
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&pl.table), table_bytes + slots * 16);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return PA_ERR_NOMEM;
    }
    pl.part_sum = reinterpret_cast<double*>(reinterpret_cast<char*>(pl.table) + table_bytes);
    pl.part_bad = reinterpret_cast<unsigned long long*>(pl.part_sum + slots);
    e = hipMemcpyAsync(pl.table, host.data(), table_bytes, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      (void)hipFree(pl.table);
      return hip_failed(e);
    }
    g_plans.push_front(std::move(pl));
    while (g_plans.size() > kMaxPlans) {
      free_plan(g_plans.back());
      g_plans.pop_back();
    }
    it = g_plans.begin();
  } else {
    if (it != g_plans.begin()) {
      g_plans.splice(g_plans.begin(), g_plans, it);
      it = g_plans.begin();
    }
    if (gnow != it->grads) {
      const std::vector<Range> mr = merged(gr);
      for (const Range& r : outs)
        if (hits_sorted(mr, r)) return PA_ERR_ALIAS;
      it->ranges = mr;
      it->grads = gnow;
      changed = true;
    }
  }
  for (const Range& r : outs)
    if (hits_sorted(it->ranges, r)) return PA_ERR_ALIAS;
  const bool cap = capturing(st);
  if (changed || it->captured || cap) {   // as for the list step: moved gradients, or a plan a graph holds
    const hipError_t pe = patch_table(it->table, sizeof(pa::Entry), offsetof(pa::Entry, g), it->grads, st);
    if (pe != hipSuccess) return hip_failed(pe);
    it->captured = it->captured || cap;
  }
  hipError_t e;
  switch (grad_dtype) {
    case PA_DT_F32: e = launch_stats<pa::kF32>(*it, max_norm, sumsq, nonfinite, clip_scale, st); break;
    case PA_DT_BF16: e = launch_stats<pa::kBF16>(*it, max_norm, sumsq, nonfinite, clip_scale, st); break;
    default: e = launch_stats<pa::kF16>(*it, max_norm, sumsq, nonfinite, clip_scale, st); break;
  }
  return e == hipSuccess ? PA_OK : hip_failed(e);
}

size_t pa_turbo_layout_bytes(int compress_m, int compress_v, int v_bits, int block_size, int m_block_size, size_t n) {
  if (!layout_ok(v_bits, block_size, m_block_size)) return 0;
  const size_t B = (size_t)block_size, G = (size_t)m_block_size;
  size_t b = 0;
  b += compress_m ? 4 * ((n + 15) / 16) + 2 * ((n + G - 1) / G) + 12 : 4 * n;
  b += compress_v ? 4 * ((n * (size_t)v_bits + 31) / 32) + 4 * ((n + B - 1) / B) : 4 * n;
  return b;
}

size_t pa_turbo_state_bytes(int compress_m, int compress_v, int v_bits, size_t n) {
  return pa_turbo_layout_bytes(compress_m, compress_v, v_bits, 128, 64, n);
}

size_t pa_turbo_workspace_bytes(size_t count, const pa_turbo_state* states, const size_t* n) {
  if (count == 0 || states == nullptr || n == nullptr) return 0;
  size_t b = 0;
  for (size_t i = 0; i < count; ++i)
    if (states[i].compress_m && n[i] > 0) {
      const long long t = turbo_tiles(n[i]);
      b += 8 * (size_t)(t + turbo_chunks_of(t));
    }
  return b;
}

int pa_turbo_step_list(size_t count, float* const* params, const float* const* grads, const pa_turbo_state* states,
                       const size_t* n, const pa_hyper* hyper, const pa_turbo_config* config, long long step,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return pa_turbo_step_list_typed(PA_DT_F32, PA_DT_F32, count, reinterpret_cast<void* const*>(params),
                                  reinterpret_cast<const void* const*>(grads), states, n, hyper, config, step,
                                  workspace, workspace_bytes, stream);
}

int pa_turbo_step_list_typed(int param_dtype, int grad_dtype, size_t count, void* const* params,
                             const void* const* grads, const pa_turbo_state* states, const size_t* n,
                             const pa_hyper* hyper, const pa_turbo_config* config, long long step, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!valid_dtype_pair(param_dtype, grad_dtype)) return PA_ERR_ARG;
  if (config == nullptr || !std::isfinite(config->m_step_factor) || !(config->m_step_factor > 0.0))
    return PA_ERR_ARG;
  TurboLayout lay;
  if (turbo_layout(config, &lay)) return PA_ERR_ARG;
  if (step > kTurboMaxStep) return PA_ERR_ARG;
  pa::Scalars s;
  int rc = make_scalars(hyper, step, &s);
  if (rc) return rc;
  if (count == 0) return PA_OK;
  if (params == nullptr || grads == nullptr || states == nullptr || n == nullptr) return PA_ERR_ARG;
  bool any_m = false;
  for (size_t i = 0; i < count; ++i) {
    if (n[i] > kTurboMaxValues) return PA_ERR_ARG;
    any_m = any_m || (states[i].compress_m && n[i] > 0);
  }
  if (any_m && !(hyper->beta1 * hyper->beta1 < hyper->beta2)) return PA_ERR_ARG;
  if (!aligned(workspace, 8)) return PA_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev;
  DeviceInfo d;
  rc = device_info(&dev, &d);
  if (rc) return rc;

  std::vector<uintptr_t> key;
  key.reserve(count * 13 + 7);
  key.push_back((uintptr_t)param_dtype);
  key.push_back((uintptr_t)grad_dtype);
  key.push_back((uintptr_t)lay.bits);
  key.push_back((uintptr_t)lay.block);
  key.push_back((uintptr_t)lay.group);
  key.push_back((uintptr_t)lay.general);
  key.push_back((uintptr_t)config->seed);
  // The gradients are not part of the key: they are written into the table
  // when they move.
  for (size_t i = 0; i < count; ++i) {
    const pa_turbo_state& t = states[i];
    for (const void* ptr : {(const void*)params[i], (const void*)t.m_codes,
                            (const void*)t.m_means, (const void*)t.m_fp32, (const void*)t.v_index,
                            (const void*)t.v_ends, (const void*)t.v_fp32, (const void*)t.scalars})
      key.push_back(reinterpret_cast<uintptr_t>(ptr));
    key.push_back((uintptr_t)n[i]);
    key.push_back((uintptr_t)t.tensor_id);
    key.push_back((uintptr_t)((t.compress_m ? 1 : 0) | (t.compress_v ? 2 : 0)));
  }
  std::lock_guard<std::mutex> lk(g_plan_mu);
  auto it = std::find_if(g_turbo_plans.begin(), g_turbo_plans.end(),
                         [&](const TurboPlan& p) { return p.device == dev && p.key == key; });
  bool changed = false;
  if (it == g_turbo_plans.end()) {
    std::vector<pa::TurboEntry> host;
    std::vector<pa::TurboReduceEntry> red;
    std::vector<Range> written, read;
    long long tiles = 0, ws_slots = 0;
    for (size_t i = 0; i < count; ++i) {
      const pa_turbo_state& t = states[i];
      rc = check_turbo_tensor(param_dtype, grad_dtype, params[i], grads[i], t, n[i], lay, &written, &read);
      if (rc) return rc;
      if (n[i] == 0) continue;
      pa::TurboEntry e;
      std::memset(&e, 0, sizeof(e));
      e.p = static_cast<float*>(params[i]);
      e.g = static_cast<const float*>(grads[i]);
      e.m_codes = t.compress_m ? t.m_codes : nullptr;
      e.m_means = t.compress_m ? t.m_means : nullptr;
      e.m_fp32 = t.compress_m ? nullptr : t.m_fp32;
      e.v_index = t.compress_v ? t.v_index : nullptr;
      e.v_ends = t.compress_v ? t.v_ends : nullptr;
      e.v_fp32 = t.compress_v ? nullptr : t.v_fp32;
      e.scal = t.compress_m ? t.scalars : nullptr;
      e.n = (long long)n[i];
      e.tile0 = tiles;                        // in units of the chosen kernel's tile
      e.ws0 = t.compress_m ? ws_slots : 0;    // in 256-value partial sums either way
      e.tensor_id = t.tensor_id;
      e.seed = config->seed;
      e.flags = (t.compress_m ? 1 : 0) | (t.compress_v ? 2 : 0) | (param_dtype << 2) | (grad_dtype << 4);
      const long long nt = turbo_tiles(n[i]);
      if (t.compress_m) {
        pa::TurboReduceEntry r{t.scalars, ws_slots, nt, (long long)n[i], 0, 0, turbo_chunks_of(nt)};
        red.push_back(r);
        ws_slots += nt;
      }
      tiles += lay.general ? (long long)((n[i] + pa::kGenTile - 1) / pa::kGenTile) : nt;
      host.push_back(e);
    }
    {
      std::vector<Range> w = written;
      if (any_overlap(w)) return PA_ERR_ALIAS;
      const std::vector<Range> wm = merged(written);
      for (const Range& r : read)
        if (hits_sorted(wm, r)) return PA_ERR_ALIAS;
    }
    if (host.empty()) return PA_OK;
    pa::TurboEntry sentinel;
    std::memset(&sentinel, 0, sizeof(sentinel));
    sentinel.tile0 = tiles;
    host.push_back(sentinel);
    long long chunk_slots = 0;                 // chunk sums follow the tile sums
    for (pa::TurboReduceEntry& r : red) {
      r.cs0 = ws_slots + chunk_slots;
      r.chunk0 = chunk_slots;
      chunk_slots += r.chunks;
    }
    TurboPlan pl;
    pl.device = dev;
    pl.key = key;
    pl.tiles = tiles;
    pl.count = (int)host.size() - 1;
    pl.general = lay.general;
    pl.typed = param_dtype != PA_DT_F32 || grad_dtype != PA_DT_F32;
    pl.blog = log2_exact(lay.block);
    pl.glog = log2_exact(lay.group);
    pl.nreduce = (int)red.size();
    pl.nchunks = chunk_slots;
    pl.ws_bytes = 8 * (size_t)(ws_slots + chunk_slots);
    pl.written = merged(written);
    for (size_t j = 0; j + 1 < host.size(); ++j) pl.grads.push_back(host[j].g);
    written.insert(written.end(), read.begin(), read.end());
    pl.ranges = merged(written);
    const size_t tb = host.size() * sizeof(pa::TurboEntry);
    const size_t rb = std::max<size_t>(red.size(), 1) * sizeof(pa::TurboReduceEntry);
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&pl.table), tb + rb);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return PA_ERR_NOMEM;
    }
    pl.reduce = reinterpret_cast<pa::TurboReduceEntry*>(reinterpret_cast<char*>(pl.table) + tb);
    e = hipMemcpyAsync(pl.table, host.data(), tb, hipMemcpyHostToDevice, st);
    if (e == hipSuccess && !red.empty())
      e = hipMemcpyAsync(pl.reduce, red.data(), red.size() * sizeof(pa::TurboReduceEntry), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      (void)hipFree(pl.table);
      return hip_failed(e);
    }
    g_turbo_plans.push_front(std::move(pl));
    while (g_turbo_plans.size() > kMaxPlans) {
      free_turbo_plan(g_turbo_plans.back());
      g_turbo_plans.pop_back();
    }
    it = g_turbo_plans.begin();
  } else {
    if (it != g_turbo_plans.begin()) {
      g_turbo_plans.splice(g_turbo_plans.begin(), g_turbo_plans, it);
      it = g_turbo_plans.begin();
    }
    // Gradients other than those in the table: checked as at the plan's
    // creation (aligned, clear of every written buffer), then written.
    std::vector<const void*> gnow;
    std::vector<Range> gr;
    const size_t gs = dtype_size(grad_dtype);
    for (size_t i = 0; i < count; ++i) {
      if (n[i] == 0) continue;
      gnow.push_back(grads[i]);
    }
    if (gnow != it->grads) {
      if (gnow.size() != it->grads.size()) return PA_ERR_ARG;
      for (size_t i = 0; i < count; ++i) {
        if (n[i] == 0) continue;
        if (grads[i] == nullptr) return PA_ERR_ARG;
        if (!aligned(grads[i], 4 * gs)) return PA_ERR_ALIGN;
        gr.push_back(range_of(grads[i], n[i] * gs));
      }
      for (const Range& r : gr)
        if (hits_sorted(it->written, r)) return PA_ERR_ALIAS;
      std::vector<Range> all = it->written;
      all.insert(all.end(), gr.begin(), gr.end());
      it->ranges = merged(all);
      it->grads = gnow;
      changed = true;
    }
  }
  if (workspace_bytes < it->ws_bytes || (it->ws_bytes > 0 && workspace == nullptr)) return PA_ERR_ARG;
  {
    std::vector<Range> hr;
    hyper_ranges(hyper, &hr);
    if (it->ws_bytes > 0) hr.push_back(range_of(workspace, it->ws_bytes));
    for (const Range& r : hr)
      if (hits_sorted(it->ranges, r)) return PA_ERR_ALIAS;
    if (any_overlap(hr)) return PA_ERR_ALIAS;
  }
  pa::TurboScalars ts;
  std::memset(&ts, 0, sizeof(ts));
  const double b1 = hyper->beta1, b2 = hyper->beta2;
  ts.bc1 = (float)(1.0 - std::pow(b1, (double)step));
  ts.bc1p = (float)(1.0 - std::pow(b1, (double)(step - 1)));
  ts.bc2p = (float)(1.0 - std::pow(b2, (double)(step - 1)));
  ts.inv_bc1 = 1.0 / (double)ts.bc1;
  ts.inv_bc2p = step > 1 ? 1.0 / (double)ts.bc2p : 0.0;
  ts.seed = config->seed;
  ts.step = step;
  hipError_t e;
  double* ws = static_cast<double*>(workspace);
  const double f = config->m_step_factor;
  unsigned long long* nf = hyper->nonfinite;
  const bool cap = capturing(st);
  if (changed || it->captured || cap) {   // as for the list step: moved gradients, or a plan a graph holds
    e = patch_table(it->table, sizeof(pa::TurboEntry), offsetof(pa::TurboEntry, g), it->grads, st);
    if (e != hipSuccess) return hip_failed(e);
    it->captured = it->captured || cap;
  }
  if (it->general) {
    switch (lay.bits) {
      case 2: e = launch_general<2>(*it, s, ts, ws, nf, f, st); break;
      case 3: e = launch_general<3>(*it, s, ts, ws, nf, f, st); break;
      case 4: e = launch_general<4>(*it, s, ts, ws, nf, f, st); break;
      case 6: e = launch_general<6>(*it, s, ts, ws, nf, f, st); break;
      default: e = launch_general<8>(*it, s, ts, ws, nf, f, st); break;
    }
  } else {
    switch (lay.bits) {
      case 2: e = launch_turbo<2>(*it, s, ts, ws, nf, f, st); break;
      case 3: e = launch_turbo<3>(*it, s, ts, ws, nf, f, st); break;
      case 4: e = launch_turbo<4>(*it, s, ts, ws, nf, f, st); break;
      case 6: e = launch_turbo<6>(*it, s, ts, ws, nf, f, st); break;
      default: e = launch_turbo<8>(*it, s, ts, ws, nf, f, st); break;
    }
  }
  return e == hipSuccess ? PA_OK : hip_failed(e);
}

size_t pa_state_bytes(int mode, size_t n) {
  switch (mode) {
    case PA_FP32: return 8 * n;
    case PA_PACKED_E4:
    case PA_PACKED_FP16: return 4 * n;
    case PA_BLOCKWISE8: return 2 * n + 8 * (n / pa::kBlock);
    default: return 0;
  }
}

int pa_format_info(int mode, pa_format* out) {
  if (out == nullptr || !valid_mode(mode)) return PA_ERR_ARG;
  std::memset(out, 0, sizeof(*out));
  out->mode = mode;
  switch (mode) {
    case PA_PACKED_E4:
      out->lanes = 2;
      out->m_sign_bits = 1; out->m_exp_bits = 4; out->m_mant_bits = 11; out->m_exp_bias = 15;
      out->r_sign_bits = 0; out->r_exp_bits = 4; out->r_mant_bits = 12; out->r_exp_bias = 15;
      out->m_max = std::ldexp(4095.0, -11);       // (2^12 - 1) * 2^-11
      out->m_min_normal = std::ldexp(1.0, -14);
      out->m_min_subnormal = std::ldexp(1.0, -25);
      out->r_max = std::ldexp(8191.0, -12);
      out->r_min_normal = std::ldexp(1.0, -14);
      out->r_min_subnormal = std::ldexp(1.0, -26);
      break;
    case PA_PACKED_FP16:
      out->lanes = 2;
      out->m_sign_bits = 1; out->m_exp_bits = 5; out->m_mant_bits = 10; out->m_exp_bias = 15;
      out->r_sign_bits = 1; out->r_exp_bits = 5; out->r_mant_bits = 10; out->r_exp_bias = 15;
      out->m_max = out->r_max = 65504.0;
      out->m_min_normal = out->r_min_normal = std::ldexp(1.0, -14);
      out->m_min_subnormal = out->r_min_subnormal = std::ldexp(1.0, -24);
      break;
    case PA_FP32:
      out->lanes = 2;
      out->m_sign_bits = out->r_sign_bits = 1;
      out->m_exp_bits = out->r_exp_bits = 8;
      out->m_mant_bits = out->r_mant_bits = 23;
      out->m_exp_bias = out->r_exp_bias = 127;
      out->m_max = out->r_max = 3.4028234663852886e38;
      out->m_min_normal = out->r_min_normal = std::ldexp(1.0, -126);
      out->m_min_subnormal = out->r_min_subnormal = std::ldexp(1.0, -149);
      break;
    case PA_BLOCKWISE8:
      out->lanes = 2;
      out->m_mant_bits = 8;   // 8-bit code into a 256-entry map
      out->r_mant_bits = 8;
      out->block = pa::kBlock;
      break;
  }
  return PA_OK;
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_ARG: return "invalid argument";
    case PA_ERR_ALIGN: return "misaligned buffer";
    case PA_ERR_SHAPE: return "length is not a multiple of the 2048-element block";
    case PA_ERR_ALIAS: return "buffers overlap";
    case PA_ERR_DEVICE: return "HIP runtime error";
    case PA_ERR_NOMEM: return "device allocation of the launch plan failed";
    case PA_ERR_CAPACITY: return "more tensors than the no-allocation table holds (PA_NOALLOC_MAX_TENSORS)";
    default: return "unknown status";
  }
}

int pa_last_hip_error(void) { return g_last_hip_error; }

void pa_release_plans(void) {
  std::lock_guard<std::mutex> lk(g_plan_mu);
  for (Plan& p : g_plans) free_plan(p);
  g_plans.clear();
  for (TurboPlan& p : g_turbo_plans) free_turbo_plan(p);
  g_turbo_plans.clear();
  std::lock_guard<std::mutex> lb(g_bw_mu);
  for (BwBuffer& b : g_bw_buffers) (void)hipFree(b.tabs);
  g_bw_buffers.clear();
}

int pa_debug_blockwise_path(long long blocks_per_workgroup) {
  if (blocks_per_workgroup < -1 || blocks_per_workgroup > (1LL << 20)) return PA_ERR_ARG;
  g_bw_force.store(blocks_per_workgroup);
  return PA_OK;
}

int pa_debug_plan_count(int* step_plans, int* stats_plans, int* turbo_plans) {
  if (step_plans == nullptr || stats_plans == nullptr || turbo_plans == nullptr) return PA_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_plan_mu);
  int a = 0, b = 0;
  for (const Plan& p : g_plans) (p.mode == kStatsPlanMode ? b : a) += 1;
  *step_plans = a;
  *stats_plans = b;
  *turbo_plans = (int)g_turbo_plans.size();
  return PA_OK;
}

int pa_debug_scalars(const pa_hyper* hyper, long long step, float* out, double* inv_bc2) {
  if (out == nullptr || inv_bc2 == nullptr) return PA_ERR_ARG;
  pa::Scalars s;
  const int rc = make_scalars(hyper, step, &s);
  if (rc) return rc;
  const float v[9] = {s.beta1, s.one_m_beta1, s.beta2, s.one_m_beta2, s.bc2,
                      s.lr_over_bc1, s.decay, s.eps, s.beta1_x2p112};
  std::memcpy(out, v, sizeof(v));
  *inv_bc2 = s.inv_bc2;
  return PA_OK;
}

int pa_debug_codec(int lane, int dir, const void* in, void* out, size_t n, void* stream) {
  if (lane < 0 || lane > 3 || dir < 0 || dir > 1) return PA_ERR_ARG;
  if (n == 0) return PA_OK;
  if (in == nullptr || out == nullptr) return PA_ERR_ARG;
  if (!aligned(in, dir == 0 ? 4 : 2) || !aligned(out, dir == 0 ? 2 : 4)) return PA_ERR_ALIGN;
  int dev;
  DeviceInfo d;
  int rc = device_info(&dev, &d);
  if (rc) return rc;
  const long long blocks = ((long long)n + pa::kThreads - 1) / pa::kThreads;
  const dim3 grid((unsigned)grid_for(blocks, d, d.blocks_per_cu)), block(pa::kThreads);
  hipLaunchKernelGGL(pa::codec_kernel, grid, block, 0, static_cast<hipStream_t>(stream), lane, dir, in, out,
                     (long long)n);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_failed(e);
}

int pa_debug_q1_ends(const float* in, uint32_t* out, size_t n, void* stream) {
  if (n == 0) return PA_OK;
  if (in == nullptr || out == nullptr) return PA_ERR_ARG;
  if (!aligned(in, 4) || !aligned(out, 4)) return PA_ERR_ALIGN;
  int dev;
  DeviceInfo d;
  int rc = device_info(&dev, &d);
  if (rc) return rc;
  const long long blocks = ((long long)n + pa::kThreads - 1) / pa::kThreads;
  const dim3 grid((unsigned)grid_for(blocks, d, d.blocks_per_cu)), block(pa::kThreads);
  hipLaunchKernelGGL(pa::q1_ends_kernel, grid, block, 0, static_cast<hipStream_t>(stream), in, out, (long long)n);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_failed(e);
}

int pa_debug_q1_levels(const uint32_t* ends, int bits, int exact, float* out, size_t n, void* stream) {
  if (bits != 2 && bits != 3 && bits != 4 && bits != 6 && bits != 8) return PA_ERR_ARG;
  if (n == 0) return PA_OK;
  if (ends == nullptr || out == nullptr || n > ((size_t)1 << 40)) return PA_ERR_ARG;
  if (!aligned(ends, 4) || !aligned(out, 4)) return PA_ERR_ALIGN;
  int dev;
  DeviceInfo d;
  int rc = device_info(&dev, &d);
  if (rc) return rc;
  // One half-wavefront per endpoint word: eight words per workgroup.
  const long long blocks = ((long long)n + 2 * (pa::kThreads / 64) - 1) / (2 * (pa::kThreads / 64));
  const dim3 grid((unsigned)grid_for(blocks, d, d.blocks_per_cu)), block(pa::kThreads);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int ex = exact ? 1 : 0;
  switch (bits) {
    case 2: hipLaunchKernelGGL(pa::q1_levels_kernel<2>, grid, block, 0, st, ends, ex, out, (long long)n); break;
    case 3: hipLaunchKernelGGL(pa::q1_levels_kernel<3>, grid, block, 0, st, ends, ex, out, (long long)n); break;
    case 4: hipLaunchKernelGGL(pa::q1_levels_kernel<4>, grid, block, 0, st, ends, ex, out, (long long)n); break;
    case 6: hipLaunchKernelGGL(pa::q1_levels_kernel<6>, grid, block, 0, st, ends, ex, out, (long long)n); break;
    default: hipLaunchKernelGGL(pa::q1_levels_kernel<8>, grid, block, 0, st, ends, ex, out, (long long)n); break;
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_failed(e);
}

int pa_debug_pow2_rn32(const double* x, int exact, float* out, size_t n, void* stream) {
  if (n == 0) return PA_OK;
  if (x == nullptr || out == nullptr) return PA_ERR_ARG;
  if (!aligned(x, 8) || !aligned(out, 4)) return PA_ERR_ALIGN;
  int dev;
  DeviceInfo d;
  int rc = device_info(&dev, &d);
  if (rc) return rc;
  const long long blocks = ((long long)n + pa::kThreads - 1) / pa::kThreads;
  const dim3 grid((unsigned)grid_for(blocks, d, d.blocks_per_cu)), block(pa::kThreads);
  hipLaunchKernelGGL(pa::pow2_rn32_kernel, grid, block, 0, static_cast<hipStream_t>(stream), x, exact ? 1 : 0, out,
                     (long long)n);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_failed(e);
}

int pa_debug_sqrt(const float* in, float* out, size_t n, void* stream) {
  if (n == 0) return PA_OK;
  if (in == nullptr || out == nullptr) return PA_ERR_ARG;
  if (!aligned(in, 4) || !aligned(out, 4)) return PA_ERR_ALIGN;
  int dev;
  DeviceInfo d;
  int rc = device_info(&dev, &d);
  if (rc) return rc;
  const long long blocks = ((long long)n + pa::kThreads - 1) / pa::kThreads;
  const dim3 grid((unsigned)grid_for(blocks, d, d.blocks_per_cu)), block(pa::kThreads);
  hipLaunchKernelGGL(pa::sqrt_kernel, grid, block, 0, static_cast<hipStream_t>(stream), in, out, (long long)n);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_failed(e);
}

}  // extern "C"
