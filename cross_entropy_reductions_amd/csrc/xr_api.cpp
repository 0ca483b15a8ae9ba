// xr_api.cpp -- the C ABI of libxr: argument validation, launch planning, kernel launches.
//
// Validation runs before any HIP call, so argument errors are reported without a device.
// Planning picks, from the row length, the dtype, the batch size and the device's compute
// unit count, one of three paths (row-resident, split row, stream); see include/xr.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/xr.h"
#include "xr_internal.h"

namespace xr {
namespace {

constexpr int32_t kVersion = 10400;  // 1.4.0
constexpr int64_t kMinChunkVecs = 256;
constexpr int64_t kMaxGrid = 0x7FFFFFFF;  // workgroups in one launch

// ----------------------------------------------------------------------------- options
// Process-wide overrides for tests and sweeps (xr_set_option); atomics, so that setting one
// while another thread launches work is not a data race (which value that launch sees is
// unspecified).
struct Options {
  std::atomic<int64_t> path{0}, split{0}, threads{0}, grid{0}, load_policy{0}, no_wait{0}, groups{0};
};
Options g_opt;

// Profiling hook: events recorded around the row kernel of each call (xr_set_profile_events).
std::atomic<hipEvent_t> g_ev_start{nullptr}, g_ev_stop{nullptr};

// ----------------------------------------------------------------------------- device cache
struct DeviceInfo {
  int cus = 0;
  int coop = 0;
  int model_per_cu = 0;  // > 0: a modelled device (xr_plan_model), holding this many
                         // workgroups of any shape per compute unit (no occupancy query)
};
std::mutex g_mu;
std::map<int, DeviceInfo> g_dev;
std::map<std::pair<int, const void*>, std::map<int, int>> g_occ;  // (device, kernel) -> threads -> blocks/CU

xr_status_t device_info(int* dev_out, DeviceInfo* info) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return XR_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_dev.find(dev);
  if (it == g_dev.end()) {
    DeviceInfo di;
    if (hipDeviceGetAttribute(&di.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        di.cus <= 0)
      return XR_ERR_DEVICE;
    if (hipDeviceGetAttribute(&di.coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess)
      di.coop = 0;
    it = g_dev.emplace(dev, di).first;
  }
  *dev_out = dev;
  *info = it->second;
  return XR_OK;
}

// Resident workgroups per compute unit for a kernel at a workgroup size.
int blocks_per_cu(int dev, const void* kernel, int threads) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_occ.find({dev, kernel});
    if (it != g_occ.end()) {
      auto jt = it->second.find(threads);
      if (jt != it->second.end()) return jt->second;
    }
  }
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, threads, 0) != hipSuccess)
    blocks = 0;
  std::lock_guard<std::mutex> lk(g_mu);
  g_occ[{dev, kernel}][threads] = blocks;
  return blocks;
}

// ----------------------------------------------------------------------------- helpers
int elt_bytes(xr_dtype_t dt) { return dt == XR_BF16 ? 2 : 4; }
int elts_per_vec(xr_dtype_t dt) { return dt == XR_BF16 ? 8 : 4; }
bool valid_dtype(int dt) { return dt == XR_F32 || dt == XR_BF16; }

// 16-byte vectors a row of n elements can touch, whatever its alignment.
int64_t row_vecs_max(int64_t n, xr_dtype_t dt) {
  const int64_t epv = elts_per_vec(dt);
  return (epv - 1 + n + epv - 1) / epv;
}

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Do two row-major matrices (M rows, n columns, strides in elements) overlap in memory?
bool overlaps(const void* a, int64_t lda, const void* b, int64_t ldb, int64_t M, int64_t n,
              int eb) {
  if (M == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  const uintptr_t a1 = a0 + (uintptr_t)(((M - 1) * lda + n) * eb);
  const uintptr_t b1 = b0 + (uintptr_t)(((M - 1) * ldb + n) * eb);
  return a0 < b1 && b0 < a1;
}
// Byte spans [a, a + abytes) and [b, b + bbytes) intersect.
bool spans_overlap(const void* a, uint64_t abytes, const void* b, uint64_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return abytes && bbytes && a0 < b0 + bbytes && b0 < a0 + abytes;
}
// Largest byte span of one operand, 2^48 bytes (256 TiB, far beyond any device's memory): a
// larger one is refused (XR_ERR_SHAPE) before any arithmetic on its sizes or addresses.
constexpr uint64_t kMaxSpanBytes = uint64_t(1) << 48;
// An [M, n] matrix of row stride ld (elements of eb bytes; 1 <= n <= ld) spans fewer than
// kMaxSpanBytes bytes; so does every product of its sizes computed later.
bool span_ok(int64_t M, int64_t ld, int64_t n, int eb) {
  const uint64_t lim = kMaxSpanBytes / (uint64_t)eb;  // in elements
  if ((uint64_t)ld >= lim || n > ld) return false;
  // (M - 1) ld + n < lim, with n <= ld < lim
  return M <= 1 || (uint64_t)(M - 1) <= (lim - (uint64_t)n - 1) / (uint64_t)ld;
}
// Bytes from the first element of an [M, n] matrix of row stride ld to past its last element.
uint64_t matrix_span(int64_t M, int64_t ld, int64_t n, int eb) {
  return M > 0 ? (uint64_t)((M - 1) * ld + n) * (uint64_t)eb : 0;
}
bool bad_alias(const void* out, int64_t ldo, const void* in, int64_t ldi, int64_t M, int64_t n,
               int eb) {
  if (out == in && ldo == ldi) return false;  // exactly in place
  return overlaps(out, ldo, in, ldi, M, n, eb);
}

// Every row of both matrices sits at the same address modulo 16 bytes.
bool same_lead(const void* a, int64_t lda, const void* b, int64_t ldb, int eb) {
  const intptr_t d = reinterpret_cast<intptr_t>(a) - reinterpret_cast<intptr_t>(b);
  return (d % 16) == 0 && (((lda - ldb) * eb) % 16) == 0;
}

// Smallest shape of the menu holding `vecs` vectors per workgroup (optionally a forced size).
const Shape* pick_shape(const Shape* menu, int count, int64_t vecs, int max_vpt = 0) {
  for (int i = 0; i < count; ++i) {
    const Shape& s = menu[i];
    if (g_opt.threads && s.threads != g_opt.threads) continue;
    if (max_vpt && s.vpt > max_vpt) continue;
    if ((int64_t)s.threads * s.vpt >= vecs) return &s;
  }
  return nullptr;
}

struct Plan {
  int path = kPathStream;
  Shape shape{kStreamThreads, 0};
  int S = 1;
  int64_t grid = 0;
  bool coop = false;
  int64_t chunk_vecs = 0;
  int group_rows = 1;  // cross-entropy split rows: adjacent rows written back together
  bool load_prio = false;  // softmax whole rows: raised wave priority for the row's loads
  const void* kernel = nullptr;
};

// Does every row of a matrix start on a 16-byte boundary?
bool rows_on_16(const void* p, int64_t ld, int64_t M, int eb) {
  return aligned_to(p, 16) && (M <= 1 || ((ld * eb) % 16) == 0);
}

const void* stream_kernel(int op, xr_dtype_t dt) {
  switch (op) {
    case kOpSoftmaxFwd: return softmax_fwd_stream_kernel_ptr(dt);
    case kOpSoftmaxBwd: return softmax_bwd_stream_kernel_ptr(dt);
    case kOpNllFwd: return nll_fwd_stream_kernel_ptr(dt);
    default: return xent_stream_kernel_ptr(dt);
  }
}

const void* split_kernel(int op, xr_dtype_t dt, Shape sh, bool nt) {
  switch (op) {
    case kOpSoftmaxFwd: return softmax_fwd_split_kernel_ptr(dt, sh, nt);
    case kOpSoftmaxBwd: return softmax_bwd_split_kernel_ptr(dt, sh, nt);
    default: return nll_split_kernel_ptr(dt, sh, nt);
  }
}

const void* row_kernel(int op, xr_dtype_t dt, Shape sh, bool nt) {
  switch (op) {
    case kOpSoftmaxFwd: return softmax_fwd_kernel_ptr(dt, sh, nt);
    case kOpSoftmaxBwd: return softmax_bwd_kernel_ptr(dt, sh, nt);
    case kOpNllFwd: return nll_fwd_kernel_ptr(dt, sh, nt);
    default: return xent_rows_kernel_ptr(dt, sh, nt);
  }
}

// op: an Op (softmax fwd / bwd, cross-entropy, negative log-softmax fwd). `aligned`: every
// operand row has the same address modulo 16; `on16`: moreover every row starts on a
// 16-byte boundary (then a row touches exactly ceil(N / elements-per-vector) vectors).
xr_status_t make_plan(int op, int64_t M, int64_t N, xr_dtype_t dt, bool aligned, bool on16,
                      Plan* plan, bool can_split = false, const DeviceInfo* model = nullptr) {
  if (!span_ok(M, N, N, elt_bytes(dt))) return XR_ERR_SHAPE;  // keeps M * S and the like exact
  int dev = 0;
  DeviceInfo di;
  if (model) di = *model;
  else if (xr_status_t st = device_info(&dev, &di)) return st;
  const bool bwd = op == kOpSoftmaxBwd;
  const Shape* menu = bwd ? kBwdShapes : kFwdShapes;
  const int nmenu = bwd ? kNumBwdShapes : kNumFwdShapes;
  const int64_t nvm = on16 ? (N + elts_per_vec(dt) - 1) / elts_per_vec(dt) : row_vecs_max(N, dt);
  const int64_t cap_max = (int64_t)menu[nmenu - 1].threads * menu[nmenu - 1].vpt;
  Plan p;
  p.grid = M;

  const int64_t want = g_opt.path;
  if (want == kPathStream || !aligned) {
    if (want && want != kPathStream) return XR_ERR_SHAPE;
    p.kernel = stream_kernel(op, dt);
    *plan = p;
    return XR_OK;
  }

  // Workgroups per row (cross-entropy, and the softmax forward / backward / negative
  // log-softmax when the call brings a workspace for the exchange; else their rows stay
  // whole): enough for the row to fit;
  // rows of 32 KB and more in several chunks, so that several workgroups share a compute
  // unit and one's reductions overlap another's memory traffic: ~16 KB chunks up to 64 KB
  // rows, ~64 KB chunks up to 512 KB rows (at most 8 chunks, so that their rows are still
  // written back in groups), ~128 KB chunks above (measured: 8192 x 32000 bf16 at 5.5 TB/s
  // in two chunks of 64 x 16 vectors, 5.65 in four; 16384 x 128256 bf16 at 5.6 TB/s whole,
  // 6.2 in two 128 KB chunks; then, with write groups, 6.15 in two, 6.24 in four 64 KB
  // chunks on 256 x 16, 6.20 in eight; 2048 x 256000 fp32 6.52 in eight 128 KB chunks, 6.28
  // in sixteen 64 KB ones); and enough chunks to give every compute unit work when the
  // batch is short.
  int64_t S = 1;
  if (op == kOpXent || can_split) {
    const int64_t s_cap = (nvm + cap_max - 1) / cap_max;
    const int64_t row_bytes = nvm * 16;
    // (the softmax backward holds two operands per thread: 64 KB chunks at every length;
    // measured on 4096 x 128256 bf16: 5.85 TB/s in two chunks, 6.29 in four. The softmax
    // forward over those rows: 5.70 in two 128 KB chunks, 5.91 in four 64 KB ones. The
    // negative log-softmax, writing a separate output, keeps 128 KB chunks: over the
    // 16384 x 128256 bf16 logits 0.3 % slower in 64 KB ones.)
    const bool chunks64 = op == kOpSoftmaxBwd || (op != kOpNllFwd && row_bytes <= (512 << 10));
    const int64_t big_chunk = chunks64 ? (64 << 10) : (128 << 10);
    const int64_t chunk_bytes = row_bytes <= (64 << 10) ? (16 << 10) : big_chunk;
    const int64_t s_bw = row_bytes >= (32 << 10)
                             ? std::max<int64_t>(2, (row_bytes + chunk_bytes - 1) / chunk_bytes)
                             : 1;
    int64_t s_par = 1;
    if (M > 0 && M < di.cus) {
      s_par = (di.cus + M - 1) / M;
      s_par = std::min(s_par, std::max<int64_t>(1, nvm / kMinChunkVecs));
    }
    S = std::max(std::max(s_cap, s_bw), s_par);
    if (g_opt.split) S = g_opt.split;
    if (want == kPathResident && g_opt.split == 0) S = s_cap;
    if (want == kPathSplit && g_opt.split == 0) S = std::max<int64_t>(2, S);
    if (want == kPathResident && S != 1) return XR_ERR_SHAPE;
    if (want == kPathSplit && S < 2) return XR_ERR_SHAPE;
  } else if (nvm > cap_max || want == kPathSplit) {
    if (want == kPathResident || want == kPathSplit) return XR_ERR_SHAPE;
    p.kernel = stream_kernel(op, dt);
    *plan = p;
    return XR_OK;
  }

  const int64_t chunk = (nvm + S - 1) / S;
  // Cross-entropy chunks of up to 32 KB take a shape of at most 8 vectors per thread when
  // one holds the chunk (more threads, fewer loads in flight per thread): measured on
  // 8192 x 32000 bf16, four 16 KB chunks per row at 5.62 TB/s on 64 threads x 16 vectors,
  // 5.80-5.84 on 128 x 8 (and two 32 KB chunks on 256 x 8 alike). Larger chunks take the
  // smallest shape that holds them: 16384 x 128256 bf16 in four 64 KB chunks at 6.24 TB/s
  // on 256 x 16, 6.13-6.17 on 512 x 8; the 128 KB chunks of longer rows 512 x 16.
  const Shape* sh = (op == kOpXent && chunk * 16 <= (32 << 10)) ? pick_shape(menu, nmenu, chunk, 8)
                                                                 : nullptr;
  if (!sh) sh = pick_shape(menu, nmenu, chunk);
  if (!sh) {
    if (want) return XR_ERR_SHAPE;
    p.kernel = stream_kernel(op, dt);
    *plan = p;
    return XR_OK;
  }
  p.shape = *sh;
  p.S = (int)S;
  p.chunk_vecs = chunk;
  // Row loads: non-temporal, except for whole rows of 128 KB and more, which measured
  // faster with the default policy (the cross-entropy over a 128256-wide bf16 vocabulary).
  bool nt_loads = !(S == 1 && nvm * 16 >= (128 << 10));
  if (g_opt.load_policy) nt_loads = g_opt.load_policy == 2;
  // the split forms of the ops other than the cross-entropy (no persistent form)
  const bool other_split = op != kOpXent && S > 1;
  p.kernel = other_split ? split_kernel(op, dt, *sh, nt_loads) : row_kernel(op, dt, *sh, nt_loads);
  if (!p.kernel) return XR_ERR_SHAPE;
  const int per_cu = di.model_per_cu > 0 ? di.model_per_cu : blocks_per_cu(dev, p.kernel, sh->threads);
  if (per_cu <= 0) return XR_ERR_DEVICE;
  const int64_t resident = (int64_t)di.cus * per_cu;
  if (S == 1) {
    // One workgroup per row by default (the hardware dispatcher balances the rows and
    // starts a row as soon as a compute unit frees up: measured faster than a persistent
    // grid); a persistent grid of `grid` workgroups per compute unit on request.
    p.path = kPathResident;
    int64_t g = M;
    if (g_opt.grid > 0) g = (int64_t)di.cus * std::min<int64_t>(g_opt.grid, per_cu);
    p.grid = std::max<int64_t>(1, std::min<int64_t>(M, g));
    // the backward's loop-free form when every row has a workgroup of its own
    if (bwd && p.grid >= M) p.kernel = softmax_bwd_kernel_ptr(dt, *sh, nt_loads, true);
    if (!p.kernel) return XR_ERR_SHAPE;
    // softmax rows issue their loads at a raised wave priority when the whole grid is
    // resident at once (measured faster there, slower on grids the GPU takes in rounds)
    p.load_prio = (op == kOpSoftmaxFwd || bwd) && p.grid <= resident;
  } else if (other_split || (g_opt.grid <= 0 && M * S <= 0x7FFFFFFF)) {
    // (only the cross-entropy has a persistent split form). A row's S chunks must be able
    // to be resident together, or its first chunks could wait for chunks that cannot start
    // until they finish: more chunks than the GPU holds workgroups of this shape (rows of
    // tens of MB) take the stream kernels.
    if (M * S > 0x7FFFFFFF || S > resident) {
      if (want) return XR_ERR_SHAPE;
      Plan q;
      q.grid = M;
      q.kernel = stream_kernel(op, dt);
      *plan = q;
      return XR_OK;
    }
    // One workgroup per row chunk, launched normally (measured faster than a persistent
    // cooperative grid): the S chunks of a row have consecutive workgroup ids, and the
    // dispatcher starts workgroups in id order, so a chunk only ever waits for chunks that
    // are resident or about to be; the wait is bounded in any case.
    p.path = kPathSplit;
    p.grid = M * S;
    // Split rows with chunks of 32 KiB and more, at most 8 per row, are written back in
    // groups of 8 adjacent rows: a chunk holds its stores until the chunks of the rows
    // around it have published (same-box A/B: cross-entropy over 16384 x 128256 bf16 in
    // 128 KB chunks 6.10-6.14 TB/s ungrouped, 6.22-6.23 grouped; 2048 x 256000 fp32, 8
    // chunks per row, 6.40-6.44 to 6.51-6.52; negative log-softmax 16384 x 128256 bf16
    // 6.11-6.18 to 6.39; softmax 4096 x 128256 bf16 forward 5.75-5.78 to 5.84-5.87, backward
    // in 62.6 KiB chunks 6.22 to 6.40; groups of 16 no better than 8; 8192 x 32000 bf16 in
    // 32 KB chunks no different, in 16 KB chunks 1-2 % slower; 16 rows of 2^20 fp32 in 32
    // or 64 chunks per row 2-7 % slower, a group then being hundreds of slots). A group's
    // chunks have consecutive workgroup ids, so in a normal launch a chunk waits only for
    // chunks resident or next in line; the group must fit the GPU many times over.
    const bool group_ok = S <= 8 && (int64_t)kWriteGroupRows * S * 4 <= resident;
    if (group_ok && (g_opt.groups == 2 || (g_opt.groups == 0 && chunk * 16 >= (32 << 10))))
      p.group_rows = kWriteGroupRows;
  } else {
    p.path = kPathSplit;
    if (!di.coop) return XR_ERR_DEVICE;
    int64_t slots = resident;
    if (g_opt.grid > 0) slots = (int64_t)di.cus * std::min<int64_t>(g_opt.grid, per_cu);
    const int64_t groups = std::min<int64_t>(std::max<int64_t>(M, 1), slots / S);
    if (groups < 1) {
      if (want) return XR_ERR_SHAPE;
      Plan q;
      q.grid = M;
      q.kernel = xent_stream_kernel_ptr(dt);
      *plan = q;
      return XR_OK;
    }
    p.grid = groups * S;
    p.coop = true;
  }
  *plan = p;
  return XR_OK;
}

xr_status_t launch(const Plan& p, void* params, hipStream_t stream, int threads) {
  void* args[] = {params};
  if (p.grid <= 0) return XR_OK;
  if (p.grid > 0x7FFFFFFF) return XR_ERR_SHAPE;
  const dim3 grid((unsigned)p.grid), block((unsigned)threads);
  const hipEvent_t ev0 = g_ev_start.load(), ev1 = g_ev_stop.load();
  if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return XR_ERR_LAUNCH;
  hipError_t e = p.coop ? hipLaunchCooperativeKernel(p.kernel, grid, block, args, 0, stream)
                        : hipLaunchKernel(p.kernel, grid, block, args, 0, stream);
  if (e != hipSuccess) return XR_ERR_LAUNCH;
  if (ev1 && hipEventRecord(ev1, stream) != hipSuccess) return XR_ERR_LAUNCH;
  return XR_OK;
}

// Layer norm launch plan. Row-resident kernels need every row of every matrix, w and b on
// 16-byte boundaries and N * element size a multiple of 16 (`resident_ok`), and a shape of
// the menu holding a row; anything else takes the stream kernels. Both kernels run a
// persistent grid: the forward keeps w and b in registers across its rows, the backward
// keeps its column sums (one partial row per workgroup, summed by the second stage).
struct LnPlan {
  const void* kernel = nullptr;
  int threads = kStreamThreads;
  int vpt = 0;
  int64_t grid = 0;
  bool stream = true;
};
constexpr int kLnBwdStreamPerCu = 4;  // stream backward: workgroups per compute unit

xr_status_t make_ln_plan(bool bwd, int64_t M, int64_t N, xr_dtype_t dt, bool resident_ok,
                         LnPlan* out) {
  int dev = 0;
  DeviceInfo di;
  if (xr_status_t st = device_info(&dev, &di)) return st;
  LnPlan p;
  const int64_t epv = 16 / elt_bytes(dt);
  const Shape* sh = nullptr;
  if (resident_ok && g_opt.path != kPathStream)
    sh = pick_shape(bwd ? kLnBwdShapes : kLnFwdShapes, bwd ? kNumLnBwdShapes : kNumLnFwdShapes,
                    N / epv);
  const bool nt = g_opt.load_policy ? g_opt.load_policy == 2 : true;
  const void* rk = nullptr;
  if (sh) rk = bwd ? ln_bwd_kernel_ptr(dt, *sh, nt) : ln_fwd_kernel_ptr(dt, *sh, nt);
  if (!rk) {
    if (g_opt.path == kPathResident || g_opt.path == kPathSplit) return XR_ERR_SHAPE;
    sh = nullptr;
  }
  if (sh) {
    p.kernel = rk;
    p.threads = sh->threads;
    p.vpt = sh->vpt;
    p.stream = false;
    int per_cu = blocks_per_cu(dev, p.kernel, sh->threads);
    if (per_cu <= 0) return XR_ERR_DEVICE;
    if (g_opt.grid > 0) per_cu = std::min<int>(per_cu, (int)g_opt.grid);
    p.grid = std::min<int64_t>(M, (int64_t)di.cus * per_cu);
  } else {
    p.kernel = bwd ? ln_bwd_stream_kernel_ptr(dt) : ln_fwd_stream_kernel_ptr(dt);
    p.grid = bwd ? std::min<int64_t>(M, (int64_t)di.cus * kLnBwdStreamPerCu) : M;
  }
  *out = p;
  return XR_OK;
}

int64_t ln_pstride(int64_t N) { return (N + 3) / 4 * 4; }

size_t xent_ws_bytes(const Plan& p, int64_t M) {
  return kWsPartials + (p.path == kPathSplit ? (size_t)M * (size_t)p.S * sizeof(uint64_t) : 0);
}

size_t align16(size_t b) { return (b + 15) & ~size_t(15); }

// Byte offset of the row losses kept in a cross-entropy workspace when the caller passes no
// row_loss: after the counts block and the plan's split slots, on a 16-byte boundary.
size_t xent_rowloss_offset(const Plan& p, int64_t M) { return align16(xent_ws_bytes(p, M)); }

// Every launch of a call fits the grid limit (checked before the call enqueues anything).
bool grid_fits(const Plan& p) { return p.grid <= kMaxGrid; }

// A byte span of a call's operands, for the overlap checks.
struct Span {
  const void* p;
  uint64_t bytes;
  bool written;
};
// Does any written span overlap another span of the list?
bool any_overlap(const Span* s, int n) {
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if ((s[i].written || s[j].written) && s[i].p && s[j].p &&
          spans_overlap(s[i].p, s[i].bytes, s[j].p, s[j].bytes))
        return true;
  return false;
}

// Split rows of the ops other than the cross-entropy: clear the flags and mark every slot of
// the exchange unpublished (the cross-entropy's target scan with no targets), on `s` before
// the row kernel. The workspace holds the counts block, then M * S slots.
xr_status_t prepare_exchange(char* ws, int64_t M, int S, int64_t N, hipStream_t s,
                             uint64_t** partials, int32_t** flags) {
  int32_t* ws_counts = reinterpret_cast<int32_t*>(ws + kWsCounts);
  *partials = reinterpret_cast<uint64_t*>(ws + kWsPartials);
  *flags = ws_counts + 2;
  const int64_t* tgt = nullptr;
  int64_t mm = 0, vv = N, ii = 0, nslots = M * S;
  int32_t init_flags = g_opt.no_wait ? kFlagExchangeTimeout : 0;
  void* args[] = {&tgt, &mm, &vv, &ii, &ws_counts, partials, &nslots, &init_flags};
  const int64_t fill_groups = std::min<int64_t>(64, std::max<int64_t>(1, nslots / 1024));
  if (hipLaunchKernel(xent_scan_kernel_ptr(), dim3((unsigned)fill_groups), dim3(kScanThreads),
                      args, 0, s) != hipSuccess)
    return XR_ERR_LAUNCH;
  return XR_OK;
}

// The workspace of a softmax / negative log-softmax call: checked against the plan's size
// and against the call's matrices (`spans`, none of which it may overlap), then, for split
// rows, the exchange is prepared on `s`; otherwise the row kernel only writes 0 to the
// status word. Nothing is enqueued on an error.
xr_status_t use_workspace(const Plan& p, int64_t M, int64_t N, void* workspace,
                          size_t workspace_bytes, const Span* spans, int nspans, hipStream_t s,
                          uint64_t** partials, int32_t** flags) {
  if (!workspace) return XR_OK;
  if (workspace_bytes < xent_ws_bytes(p, M)) return XR_ERR_WORKSPACE;
  for (int i = 0; i < nspans; ++i)
    if (spans_overlap(workspace, workspace_bytes, spans[i].p, spans[i].bytes)) return XR_ERR_ALIAS;
  char* ws = static_cast<char*>(workspace);
  if (p.path == kPathSplit) return prepare_exchange(ws, M, p.S, N, s, partials, flags);
  *flags = reinterpret_cast<int32_t*>(ws + kWsCounts) + 2;
  return XR_OK;
}

}  // namespace
}  // namespace xr

using namespace xr;

extern "C" {

const char* xr_status_string(xr_status_t s) {
  switch (s) {
    case XR_OK: return "ok";
    case XR_ERR_NULL: return "a required pointer is NULL";
    case XR_ERR_SHAPE: return "invalid or unsupported sizes";
    case XR_ERR_STRIDE: return "row stride smaller than the row length";
    case XR_ERR_DTYPE: return "unknown dtype";
    case XR_ERR_ALIAS: return "an output partially overlaps an input";
    case XR_ERR_WORKSPACE: return "workspace missing or too small";
    case XR_ERR_ALIGN: return "pointer not aligned to its element size";
    case XR_ERR_DEVICE: return "no usable HIP device";
    case XR_ERR_LAUNCH: return "kernel launch failed";
    case XR_ERR_OPTION: return "unknown option or value";
    case XR_ERR_VALUE: return "invalid argument value";
    case XR_ERR_TOO_LARGE: return "sizes need more scratch than the no-allocation entry point holds";
  }
  return "unknown status";
}

int32_t xr_version(void) { return kVersion; }

xr_status_t xr_set_option(xr_option_t option, int64_t value) {
  switch (option) {
    case XR_OPT_PATH:
      if (value < 0 || value > 3) return XR_ERR_OPTION;
      g_opt.path = value;
      return XR_OK;
    case XR_OPT_SPLIT:
      if (value < 0 || value == 1 || value > 4096) return XR_ERR_OPTION;
      g_opt.split = value;
      return XR_OK;
    case XR_OPT_THREADS:
      if (value != 0 && value != 64 && value != 128 && value != 256 && value != 512 && value != 1024)
        return XR_ERR_OPTION;
      g_opt.threads = value;
      return XR_OK;
    case XR_OPT_GRID:
      if (value < -1 || value > 64) return XR_ERR_OPTION;
      g_opt.grid = value;
      return XR_OK;
    case XR_OPT_LOAD_POLICY:
      if (value < 0 || value > 2) return XR_ERR_OPTION;
      g_opt.load_policy = value;
      return XR_OK;
    case XR_OPT_NO_WAIT:
      if (value < 0 || value > 1) return XR_ERR_OPTION;
      g_opt.no_wait = value;
      return XR_OK;
    case XR_OPT_GROUPS:
      if (value < 0 || value > 2) return XR_ERR_OPTION;
      g_opt.groups = value;
      return XR_OK;
  }
  return XR_ERR_OPTION;
}

xr_status_t xr_set_profile_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return XR_ERR_NULL;
  g_ev_start = static_cast<hipEvent_t>(start);
  g_ev_stop = static_cast<hipEvent_t>(stop);
  return XR_OK;
}

static xr_status_t plan_query(int32_t op, int64_t M, int64_t N, xr_dtype_t dtype, int32_t aligned,
                              xr_plan_t* out, const DeviceInfo* model) {
  if (!out) return XR_ERR_NULL;
  if (!valid_dtype(dtype)) return XR_ERR_DTYPE;
  if (op < 0 || op > 5 || M < 0 || N < 1) return XR_ERR_SHAPE;
  // ops 4 and 5: the softmax forward / backward with a workspace
  const bool with_ws = op >= kOpNllFwd;
  if (op > kOpNllFwd) op -= 4;
  Plan p;
  if (xr_status_t st = make_plan(op, M, N, dtype, op == 2 ? true : aligned != 0, aligned == 2, &p,
                                 with_ws, model))
    return st;
  out->path = p.path;
  out->threads = p.path == kPathStream ? kStreamThreads : p.shape.threads;
  out->vec_per_thread = p.path == kPathStream ? 0 : p.shape.vpt;
  out->split = p.S;
  out->grid = (int32_t)std::min<int64_t>(p.grid, kMaxGrid);
  out->cooperative = p.coop ? 1 : 0;
  out->chunk_vecs = p.chunk_vecs;
  out->group_rows = p.path == kPathSplit ? p.group_rows : 1;
  out->load_priority = p.load_prio ? 1 : 0;
  out->grid_total = p.grid;
  return XR_OK;
}

xr_status_t xr_plan(int32_t op, int64_t M, int64_t N, xr_dtype_t dtype, int32_t aligned,
                    xr_plan_t* out) {
  return plan_query(op, M, N, dtype, aligned, out, nullptr);
}

xr_status_t xr_plan_model(int32_t op, int64_t M, int64_t N, xr_dtype_t dtype, int32_t aligned,
                          int32_t compute_units, int32_t blocks_per_cu, xr_plan_t* out) {
  if (compute_units < 1 || blocks_per_cu < 1) return XR_ERR_VALUE;
  DeviceInfo model;
  model.cus = compute_units;
  model.coop = 1;
  model.model_per_cu = blocks_per_cu;
  return plan_query(op, M, N, dtype, aligned, out, &model);
}

size_t xr_softmax_workspace_bytes(int64_t M, int64_t N, xr_dtype_t dtype) {
  if (!valid_dtype(dtype) || M < 0 || N < 1) return 0;
  // the larger of the forward and backward needs, over the row alignments a call can have
  size_t need = 0;
  for (int op : {kOpSoftmaxFwd, kOpSoftmaxBwd})
    for (bool on16 : {false, true}) {
      Plan p;
      if (make_plan(op, M, N, dtype, true, on16, &p, true) == XR_OK)
        need = std::max(need, xent_ws_bytes(p, M));
    }
  return need;
}

xr_status_t xr_softmax_fwd_ex(void* y, int64_t ld_y, const void* x, int64_t ld_x, int64_t M,
                              int64_t N, xr_dtype_t dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return XR_ERR_DTYPE;
  if (M < 0 || N < 1) return XR_ERR_SHAPE;
  if (ld_x < N || ld_y < N) return XR_ERR_STRIDE;
  if (M == 0) return XR_OK;
  if (!span_ok(M, ld_x, N, elt_bytes(dtype)) || !span_ok(M, ld_y, N, elt_bytes(dtype)))
    return XR_ERR_SHAPE;
  if (!x || !y) return XR_ERR_NULL;
  const int eb = elt_bytes(dtype);
  if (!aligned_to(x, eb) || !aligned_to(y, eb)) return XR_ERR_ALIGN;
  if (bad_alias(y, ld_y, x, ld_x, M, N, eb)) return XR_ERR_ALIAS;
  if (workspace && !aligned_to(workspace, 8)) return XR_ERR_ALIGN;
  Plan p;
  const bool on16 = rows_on_16(x, ld_x, M, eb) && rows_on_16(y, ld_y, M, eb);
  if (xr_status_t st = make_plan(kOpSoftmaxFwd, M, N, dtype, same_lead(x, ld_x, y, ld_y, eb), on16,
                                 &p, workspace != nullptr))
    return st;
  if (!grid_fits(p)) return XR_ERR_SHAPE;
  SoftmaxFwdParams prm{static_cast<const char*>(x), ld_x * eb, static_cast<char*>(y), ld_y * eb, M, N,
                       nullptr, nullptr, p.S, p.chunk_vecs, nullptr, nullptr, p.group_rows,
                       p.load_prio ? 1 : 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Span mats[] = {{y, matrix_span(M, ld_y, N, eb), true}, {x, matrix_span(M, ld_x, N, eb), false}};
  if (xr_status_t st = use_workspace(p, M, N, workspace, workspace_bytes, mats, 2, s, &prm.partials,
                                     &prm.flags))
    return st;
  return launch(p, &prm, s, p.path == kPathStream ? kStreamThreads : p.shape.threads);
}

xr_status_t xr_softmax_fwd(void* y, int64_t ld_y, const void* x, int64_t ld_x, int64_t M,
                           int64_t N, xr_dtype_t dtype, void* stream) {
  return xr_softmax_fwd_ex(y, ld_y, x, ld_x, M, N, dtype, nullptr, 0, stream);
}

size_t xr_nll_fwd_workspace_bytes(int64_t M, int64_t N, xr_dtype_t dtype) {
  if (!valid_dtype(dtype) || M < 0 || N < 1) return 0;
  size_t need = 0;
  for (bool on16 : {false, true}) {
    Plan p;
    if (make_plan(kOpNllFwd, M, N, dtype, true, on16, &p, true) == XR_OK)
      need = std::max(need, xent_ws_bytes(p, M));
  }
  return need;
}

xr_status_t xr_nll_fwd(void* out, int64_t ld_out, const void* x, int64_t ld_x,
                       const int64_t* idx, float* loss, int64_t M, int64_t N, xr_dtype_t dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return XR_ERR_DTYPE;
  if (M < 0 || N < 1) return XR_ERR_SHAPE;
  if (ld_x < N || ld_out < N) return XR_ERR_STRIDE;
  if (M == 0) return XR_OK;
  if (!span_ok(M, ld_x, N, elt_bytes(dtype)) || !span_ok(M, ld_out, N, elt_bytes(dtype)))
    return XR_ERR_SHAPE;
  if (!x || !out || !idx || !loss) return XR_ERR_NULL;
  const int eb = elt_bytes(dtype);
  if (!aligned_to(x, eb) || !aligned_to(out, eb) || !aligned_to(idx, 8) || !aligned_to(loss, 4))
    return XR_ERR_ALIGN;
  if (bad_alias(out, ld_out, x, ld_x, M, N, eb)) return XR_ERR_ALIAS;
  // idx and loss must lie outside both matrices
  const uint64_t out_span = matrix_span(M, ld_out, N, eb);
  if (spans_overlap(out, out_span, idx, (uint64_t)M * 8) ||
      spans_overlap(out, out_span, loss, (uint64_t)M * 4) ||
      spans_overlap(x, matrix_span(M, ld_x, N, eb), loss, (uint64_t)M * 4) ||
      spans_overlap(idx, (uint64_t)M * 8, loss, (uint64_t)M * 4))
    return XR_ERR_ALIAS;
  if (workspace && !aligned_to(workspace, 8)) return XR_ERR_ALIGN;
  Plan p;
  const bool on16 = rows_on_16(x, ld_x, M, eb) && rows_on_16(out, ld_out, M, eb);
  if (xr_status_t st = make_plan(kOpNllFwd, M, N, dtype, same_lead(x, ld_x, out, ld_out, eb), on16,
                                 &p, workspace != nullptr))
    return st;
  if (!grid_fits(p)) return XR_ERR_SHAPE;
  SoftmaxFwdParams prm{static_cast<const char*>(x), ld_x * eb, static_cast<char*>(out), ld_out * eb,
                       M, N, idx, loss, p.S, p.chunk_vecs, nullptr, nullptr, p.group_rows};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Span mats[] = {{out, matrix_span(M, ld_out, N, eb), true},
                       {x, matrix_span(M, ld_x, N, eb), false},
                       {idx, (uint64_t)M * 8, false},
                       {loss, (uint64_t)M * 4, true}};
  if (xr_status_t st = use_workspace(p, M, N, workspace, workspace_bytes, mats, 4, s, &prm.partials,
                                     &prm.flags))
    return st;
  return launch(p, &prm, s, p.path == kPathStream ? kStreamThreads : p.shape.threads);
}

xr_status_t xr_layernorm_fwd(void* y, int64_t ld_y, const void* x, int64_t ld_x, const void* w,
                             const void* b, float* mean, float* rstd, int64_t M, int64_t N,
                             float eps, xr_dtype_t dtype, void* stream) {
  if (!valid_dtype(dtype)) return XR_ERR_DTYPE;
  if (M < 0 || N < 1) return XR_ERR_SHAPE;
  if (ld_x < N || ld_y < N) return XR_ERR_STRIDE;
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return XR_ERR_VALUE;
  if (M == 0) return XR_OK;
  if (!span_ok(M, ld_x, N, elt_bytes(dtype)) || !span_ok(M, ld_y, N, elt_bytes(dtype)))
    return XR_ERR_SHAPE;
  if (!y || !x || !w || !b || !mean || !rstd) return XR_ERR_NULL;
  const int eb = elt_bytes(dtype);
  if (!aligned_to(y, eb) || !aligned_to(x, eb) || !aligned_to(w, eb) || !aligned_to(b, eb) ||
      !aligned_to(mean, 4) || !aligned_to(rstd, 4))
    return XR_ERR_ALIGN;
  if (bad_alias(y, ld_y, x, ld_x, M, N, eb)) return XR_ERR_ALIAS;
  const uint64_t ys = matrix_span(M, ld_y, N, eb);
  if (spans_overlap(y, ys, w, (uint64_t)N * eb) || spans_overlap(y, ys, b, (uint64_t)N * eb) ||
      spans_overlap(y, ys, mean, (uint64_t)M * 4) || spans_overlap(y, ys, rstd, (uint64_t)M * 4) ||
      spans_overlap(mean, (uint64_t)M * 4, rstd, (uint64_t)M * 4))
    return XR_ERR_ALIAS;
  const bool resident_ok = rows_on_16(x, ld_x, M, eb) && rows_on_16(y, ld_y, M, eb) &&
                           aligned_to(w, 16) && aligned_to(b, 16) && (N * eb) % 16 == 0;
  LnPlan lp;
  if (xr_status_t st = make_ln_plan(false, M, N, dtype, resident_ok, &lp)) return st;
  LnFwdParams prm{static_cast<const char*>(x), ld_x * eb, static_cast<char*>(y), ld_y * eb,
                  static_cast<const char*>(w), static_cast<const char*>(b), mean, rstd, M, N, eps};
  Plan p;
  p.kernel = lp.kernel;
  p.grid = lp.grid;
  return launch(p, &prm, static_cast<hipStream_t>(stream), lp.threads);
}

size_t xr_layernorm_bwd_workspace_bytes(int64_t M, int64_t N, xr_dtype_t dtype) {
  if (!valid_dtype(dtype) || M < 0 || N < 1) return 0;
  // Rows may or may not qualify for the row-resident kernel: size for either plan (a plan
  // that cannot apply under the current options needs nothing).
  LnPlan a, b;
  const bool ok_a = make_ln_plan(true, M, N, dtype, true, &a) == XR_OK;
  const bool ok_b = make_ln_plan(true, M, N, dtype, false, &b) == XR_OK;
  if (!ok_a && !ok_b) return 0;
  const int64_t G = std::max<int64_t>(std::max(ok_a ? a.grid : 0, ok_b ? b.grid : 0), 1);
  return (size_t)(2 * G * ln_pstride(N)) * sizeof(float);
}

xr_status_t xr_layernorm_bwd(void* dx, int64_t ld_dx, const void* dy, int64_t ld_dy,
                             const void* x, int64_t ld_x, const void* w, const float* mean,
                             const float* rstd, void* dw, void* db, int64_t M, int64_t N,
                             xr_dtype_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!valid_dtype(dtype)) return XR_ERR_DTYPE;
  if (M < 0 || N < 1) return XR_ERR_SHAPE;
  if (ld_dx < N || ld_dy < N || ld_x < N) return XR_ERR_STRIDE;
  if (!span_ok(M, ld_dx, N, elt_bytes(dtype)) || !span_ok(M, ld_dy, N, elt_bytes(dtype)) ||
      !span_ok(M, ld_x, N, elt_bytes(dtype)))
    return XR_ERR_SHAPE;
  if (!w || !dw || !db || !workspace) return XR_ERR_NULL;
  if (M > 0 && (!dx || !dy || !x || !mean || !rstd)) return XR_ERR_NULL;
  const int eb = elt_bytes(dtype);
  if ((dx && !aligned_to(dx, eb)) || (dy && !aligned_to(dy, eb)) || (x && !aligned_to(x, eb)) ||
      !aligned_to(w, eb) || !aligned_to(dw, eb) || !aligned_to(db, eb) ||
      (mean && !aligned_to(mean, 4)) || (rstd && !aligned_to(rstd, 4)) ||
      !aligned_to(workspace, 16))
    return XR_ERR_ALIGN;
  if (M > 0 && (bad_alias(dx, ld_dx, dy, ld_dy, M, N, eb) || bad_alias(dx, ld_dx, x, ld_x, M, N, eb)))
    return XR_ERR_ALIAS;
  const uint64_t dxs = matrix_span(M, ld_dx, N, eb), vb = (uint64_t)N * eb;
  if (spans_overlap(dx, dxs, w, vb) || spans_overlap(dx, dxs, dw, vb) ||
      spans_overlap(dx, dxs, db, vb) || spans_overlap(dw, vb, db, vb) ||
      spans_overlap(dx, dxs, mean, (uint64_t)M * 4) || spans_overlap(dx, dxs, rstd, (uint64_t)M * 4))
    return XR_ERR_ALIAS;
  const bool resident_ok = M > 0 && rows_on_16(dx, ld_dx, M, eb) && rows_on_16(dy, ld_dy, M, eb) &&
                           rows_on_16(x, ld_x, M, eb) && aligned_to(w, 16) && (N * eb) % 16 == 0;
  LnPlan lp;
  if (xr_status_t st = make_ln_plan(true, M, N, dtype, resident_ok, &lp)) return st;
  const int64_t ps = ln_pstride(N);
  const int64_t G = lp.grid;
  if (workspace_bytes < (size_t)(2 * std::max<int64_t>(G, 1) * ps) * sizeof(float))
    return XR_ERR_WORKSPACE;
  float* part_dw = static_cast<float*>(workspace);
  float* part_db = part_dw + std::max<int64_t>(G, 1) * ps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t blocks = (N + kLnReduceCols - 1) / kLnReduceCols;
  if (blocks > kMaxGrid || G > kMaxGrid) return XR_ERR_SHAPE;
  if (G > 0) {
    LnBwdParams prm{static_cast<const char*>(dy), ld_dy * eb, static_cast<const char*>(x), ld_x * eb,
                    static_cast<char*>(dx), ld_dx * eb, static_cast<const char*>(w), mean, rstd,
                    part_dw, part_db, ps, M, N};
    Plan p;
    p.kernel = lp.kernel;
    p.grid = G;
    if (xr_status_t st = launch(p, &prm, s, lp.threads)) return st;
  }
  LnReduceParams rp{part_dw, part_db, ps, (int)G, static_cast<char*>(dw), static_cast<char*>(db), N};
  void* args[] = {&rp};
  if (hipLaunchKernel(ln_dwdb_kernel_ptr(dtype), dim3((unsigned)blocks), dim3(kLnReduceThreads),
                      args, 0, s) != hipSuccess)
    return XR_ERR_LAUNCH;
  return XR_OK;
}

xr_status_t xr_bsr_softmax_bwd(const void* y, int64_t stride_zy, void* dx, int64_t stride_zdx,
                               int64_t Z, const int32_t* lut, int64_t lut_len, int64_t n_brows,
                               int64_t n_blocks, int32_t block, float scale, xr_dtype_t dtype,
                               void* stream) {
  if (!valid_dtype(dtype)) return XR_ERR_DTYPE;
  const int eb = elt_bytes(dtype);
  const int epv = 16 / eb;
  if (Z < 0 || n_brows < 0 || n_blocks < 0 || block < epv || block > 64 * epv ||
      (block & (block - 1)) != 0)
    return XR_ERR_SHAPE;
  if (!(scale == scale)) return XR_ERR_VALUE;
  // one batch's blocks under 2 GiB (checked before the product can wrap)
  if ((uint64_t)n_blocks >= (1ull << 31) / ((uint64_t)block * (uint64_t)block * eb))
    return XR_ERR_SHAPE;
  const uint64_t batch_bytes = (uint64_t)n_blocks * (uint64_t)block * (uint64_t)block * eb;
  if (lut_len < 2 * n_brows || lut_len >= (1ll << 29)) return XR_ERR_SHAPE;
  if (stride_zy < n_blocks * block * block || stride_zdx < n_blocks * block * block)
    return XR_ERR_STRIDE;
  if (!span_ok(Z, stride_zy, n_blocks * block * block, eb) ||
      !span_ok(Z, stride_zdx, n_blocks * block * block, eb))
    return XR_ERR_SHAPE;
  if (Z == 0 || n_brows == 0 || n_blocks == 0) return XR_OK;
  if (!y || !dx || !lut) return XR_ERR_NULL;
  if (!aligned_to(y, 16) || !aligned_to(dx, 16) || !aligned_to(lut, 4) ||
      (stride_zy * eb) % 16 != 0 || (stride_zdx * eb) % 16 != 0)
    return XR_ERR_ALIGN;
  // y may be exactly dx; otherwise the two must not overlap, nor may the table
  const uint64_t ys = (uint64_t)((Z - 1) * stride_zy) * eb + batch_bytes;
  const uint64_t ds = (uint64_t)((Z - 1) * stride_zdx) * eb + batch_bytes;
  if (!(y == dx && stride_zy == stride_zdx) && spans_overlap(y, ys, dx, ds)) return XR_ERR_ALIAS;
  if (spans_overlap(dx, ds, lut, (uint64_t)lut_len * 4)) return XR_ERR_ALIAS;
  const int tpr = block / epv;
  const int rows = std::min<int>(block, std::max(1, kBsrThreads / tpr));
  const int chunks = (block + rows - 1) / rows;
  const int64_t grid = Z * n_brows * chunks;
  if (grid > 0x7FFFFFFF) return XR_ERR_SHAPE;
  BsrParams prm{static_cast<const char*>(y), stride_zy * eb, static_cast<char*>(dx),
                stride_zdx * eb, lut, lut_len, n_brows, (int32_t)n_blocks,
                (uint32_t)batch_bytes, block, rows, chunks, scale};
  Plan p;
  p.kernel = bsr_softmax_bwd_kernel_ptr(dtype);
  p.grid = grid;
  return launch(p, &prm, static_cast<hipStream_t>(stream), kBsrThreads);
}

xr_status_t xr_softmax_bwd(void* dx, int64_t ld_dx, const void* y, int64_t ld_y, const void* dy,
                           int64_t ld_dy, int64_t M, int64_t N, xr_dtype_t dtype, void* stream) {
  return xr_softmax_bwd_ex(dx, ld_dx, y, ld_y, dy, ld_dy, M, N, dtype, nullptr, 0, stream);
}

xr_status_t xr_softmax_bwd_ex(void* dx, int64_t ld_dx, const void* y, int64_t ld_y,
                              const void* dy, int64_t ld_dy, int64_t M, int64_t N,
                              xr_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!valid_dtype(dtype)) return XR_ERR_DTYPE;
  if (M < 0 || N < 1) return XR_ERR_SHAPE;
  if (ld_dx < N || ld_y < N || ld_dy < N) return XR_ERR_STRIDE;
  if (M == 0) return XR_OK;
  if (!span_ok(M, ld_dx, N, elt_bytes(dtype)) || !span_ok(M, ld_y, N, elt_bytes(dtype)) ||
      !span_ok(M, ld_dy, N, elt_bytes(dtype)))
    return XR_ERR_SHAPE;
  if (!dx || !y || !dy) return XR_ERR_NULL;
  const int eb = elt_bytes(dtype);
  if (!aligned_to(dx, eb) || !aligned_to(y, eb) || !aligned_to(dy, eb)) return XR_ERR_ALIGN;
  if (bad_alias(dx, ld_dx, y, ld_y, M, N, eb) || bad_alias(dx, ld_dx, dy, ld_dy, M, N, eb))
    return XR_ERR_ALIAS;
  const bool aligned = same_lead(y, ld_y, dy, ld_dy, eb) && same_lead(y, ld_y, dx, ld_dx, eb);
  const bool on16 = rows_on_16(y, ld_y, M, eb) && rows_on_16(dy, ld_dy, M, eb) &&
                    rows_on_16(dx, ld_dx, M, eb);
  if (workspace && !aligned_to(workspace, 8)) return XR_ERR_ALIGN;
  Plan p;
  if (xr_status_t st = make_plan(kOpSoftmaxBwd, M, N, dtype, aligned, on16, &p,
                                 workspace != nullptr))
    return st;
  if (!grid_fits(p)) return XR_ERR_SHAPE;
  SoftmaxBwdParams prm{static_cast<const char*>(y), ld_y * eb, static_cast<const char*>(dy),
                       ld_dy * eb, static_cast<char*>(dx), ld_dx * eb, M, N,
                       p.S, p.chunk_vecs, nullptr, nullptr, p.group_rows, p.load_prio ? 1 : 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Span mats[] = {{dx, matrix_span(M, ld_dx, N, eb), true},
                       {y, matrix_span(M, ld_y, N, eb), false},
                       {dy, matrix_span(M, ld_dy, N, eb), false}};
  if (xr_status_t st = use_workspace(p, M, N, workspace, workspace_bytes, mats, 3, s, &prm.partials,
                                     &prm.flags))
    return st;
  return launch(p, &prm, s, p.path == kPathStream ? kStreamThreads : p.shape.threads);
}

size_t xr_xent_workspace_bytes(int64_t M, int64_t V, xr_dtype_t dtype) {
  if (!valid_dtype(dtype) || M < 0 || V < 1) return 0;
  // Enough for the plan of either row alignment, with room for the row losses (used when
  // the caller passes no row_loss).
  size_t need = 0;
  bool any = false;
  for (bool on16 : {false, true}) {
    Plan p;
    if (make_plan(kOpXent, M, V, dtype, true, on16, &p) != XR_OK) continue;
    any = true;
    need = std::max(need, xent_rowloss_offset(p, M) + (size_t)M * sizeof(float));
  }
  return any ? need : 0;
}

xr_status_t xr_xent_fwd_bwd_ex(void* logits, int64_t ld, const int64_t* target, int64_t M,
                               int64_t V, int64_t ignore_index, xr_dtype_t dtype,
                               xr_reduction_t reduction, const float* grad_scale,
                               int64_t grad_scale_stride, float* row_loss, float* loss,
                               int32_t* counts, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!valid_dtype(dtype)) return XR_ERR_DTYPE;
  if (reduction != XR_REDUCTION_MEAN && reduction != XR_REDUCTION_SUM &&
      reduction != XR_REDUCTION_NONE)
    return XR_ERR_VALUE;
  if (grad_scale_stride < 0) return XR_ERR_VALUE;
  if (M < 0 || V < 1) return XR_ERR_SHAPE;
  if (ld < V) return XR_ERR_STRIDE;
  // the logits, and the upstream values read at i * grad_scale_stride
  if (!span_ok(M, ld, V, elt_bytes(dtype)) ||
      (grad_scale && !span_ok(M, std::max<int64_t>(grad_scale_stride, 1), 1, 4)))
    return XR_ERR_SHAPE;
  if (reduction != XR_REDUCTION_NONE && !loss) return XR_ERR_NULL;
  if (reduction == XR_REDUCTION_NONE) loss = nullptr;
  if (!workspace) return XR_ERR_NULL;
  // the row losses are the result of the none reduction; the others may keep them in the
  // workspace
  if (M > 0 && (!logits || !target || (reduction == XR_REDUCTION_NONE && !row_loss)))
    return XR_ERR_NULL;
  const int eb = elt_bytes(dtype);
  if ((logits && !aligned_to(logits, eb)) || (target && !aligned_to(target, 8)) ||
      (row_loss && !aligned_to(row_loss, 4)) || (loss && !aligned_to(loss, 4)) ||
      (counts && !aligned_to(counts, 4)) || (grad_scale && !aligned_to(grad_scale, 4)) ||
      !aligned_to(workspace, 8))
    return XR_ERR_ALIGN;
  // The written spans (logits, row losses, loss, counts, workspace) overlap nothing else
  // of the call.
  const Span spans[] = {
      {logits, matrix_span(M, ld, V, eb), true},
      {row_loss, row_loss ? (uint64_t)M * 4 : 0, true},
      {loss, 4, true},
      {counts, 12, true},
      {workspace, workspace_bytes, true},
      {target, (uint64_t)M * 8, false},
      {grad_scale, grad_scale && M > 0 ? (uint64_t)((M - 1) * grad_scale_stride + 1) * 4 : 0, false}};
  if (any_overlap(spans, 7)) return XR_ERR_ALIAS;
  Plan p;
  const bool on16 = logits == nullptr || rows_on_16(logits, ld, M, eb);
  if (xr_status_t st = make_plan(kOpXent, M, V, dtype, true, on16, &p)) return st;
  if (!grid_fits(p)) return XR_ERR_SHAPE;
  const size_t rl_off = xent_rowloss_offset(p, M);
  const size_t need = row_loss ? xent_ws_bytes(p, M) : rl_off + (size_t)M * sizeof(float);
  if (workspace_bytes < need) return XR_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* ws_counts = reinterpret_cast<int32_t*>(ws + kWsCounts);
  uint64_t* partials = reinterpret_cast<uint64_t*>(ws + kWsPartials);
  if (!row_loss) row_loss = reinterpret_cast<float*>(ws + rl_off);
  const int64_t nslots = p.path == kPathSplit ? M * p.S : 0;

  {
    const int64_t* tgt = target;
    int64_t mm = M, vv = V, ii = ignore_index;
    int32_t init_flags = g_opt.no_wait ? kFlagExchangeTimeout : 0;
    void* args[] = {&tgt, &mm, &vv, &ii, &ws_counts, &partials, const_cast<int64_t*>(&nslots),
                    &init_flags};
    // one workgroup counts; the slot fill is spread over up to 64 (8 KB of slots each)
    const int64_t fill_groups = std::min<int64_t>(64, std::max<int64_t>(1, nslots / 1024));
    if (hipLaunchKernel(xent_scan_kernel_ptr(), dim3((unsigned)fill_groups), dim3(kScanThreads),
                        args, 0, s) != hipSuccess)
      return XR_ERR_LAUNCH;
  }
  if (M > 0) {
    XentParams prm{static_cast<char*>(logits), ld * eb, target, M, V, ignore_index, row_loss,
                   ws_counts, ws_counts + 2, partials, p.chunk_vecs, p.S,
                   (int)(p.path == kPathSplit ? p.grid / p.S : p.grid), (int)reduction,
                   grad_scale, grad_scale_stride, p.group_rows};
    if (xr_status_t st = launch(p, &prm, s, p.path == kPathStream ? kStreamThreads : p.shape.threads))
      return st;
  }
  {
    const float* rl = row_loss;
    int64_t mm = M;
    const int32_t* wc = ws_counts;
    int red = (int)reduction;
    void* args[] = {&rl, &mm, &wc, &loss, &counts, &red};
    if (hipLaunchKernel(xent_mean_kernel_ptr(), dim3(1), dim3(kScanThreads), args, 0, s) != hipSuccess)
      return XR_ERR_LAUNCH;
  }
  return XR_OK;
}

xr_status_t xr_xent_fwd_bwd(void* logits, int64_t ld, const int64_t* target, int64_t M,
                            int64_t V, int64_t ignore_index, xr_dtype_t dtype, float* row_loss,
                            float* mean_loss, int32_t* counts, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return xr_xent_fwd_bwd_ex(logits, ld, target, M, V, ignore_index, dtype, XR_REDUCTION_MEAN,
                            nullptr, 0, row_loss, mean_loss, counts, workspace, workspace_bytes,
                            stream);
}

xr_status_t xr_element_mul(void* x, int64_t ld, int64_t M, int64_t N, xr_dtype_t dtype,
                           const float* grad_output, int64_t grad_output_stride, void* stream) {
  if (!valid_dtype(dtype)) return XR_ERR_DTYPE;
  if (grad_output_stride < 0) return XR_ERR_VALUE;
  if (M < 0 || N < 1) return XR_ERR_SHAPE;
  if (ld < N) return XR_ERR_STRIDE;
  if (M == 0) return XR_OK;
  if (!span_ok(M, ld, N, elt_bytes(dtype)) ||
      !span_ok(M, std::max<int64_t>(grad_output_stride, 1), 1, 4))
    return XR_ERR_SHAPE;
  if (!x || !grad_output) return XR_ERR_NULL;
  const int eb = elt_bytes(dtype);
  if (!aligned_to(x, eb) || !aligned_to(grad_output, 4)) return XR_ERR_ALIGN;
  {
    // grad_output must not lie inside the matrix's span
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x);
    const uintptr_t a1 = a0 + (uintptr_t)((M - 1) * ld + N) * (uintptr_t)eb;
    const uintptr_t g0 = reinterpret_cast<uintptr_t>(grad_output);
    const uintptr_t g1 = g0 + (uintptr_t)((M - 1) * grad_output_stride + 1) * 4u;
    if (g0 < a1 && a0 < g1) return XR_ERR_ALIAS;
  }
  // Vectors a row spans (one more when it does not start on a 16-byte boundary).
  const int64_t epv = 16 / eb;
  const int64_t nvm = (N + epv - 1) / epv + ((reinterpret_cast<uintptr_t>(x) & 15u) ||
                                             ((ld * eb) & 15) ? 1 : 0);
  const int64_t cv = (int64_t)kMulThreads * kMulVpt;
  const int64_t chunks = (nvm + cv - 1) / cv;
  if (M > INT64_MAX / chunks) return XR_ERR_SHAPE;
  const int64_t total = M * chunks;
  // One workgroup per row chunk, up to the grid limit; the kernel strides past it.
  const int64_t grid = std::min<int64_t>(total, 0x7FFFFFFF);
  bool nt = g_opt.load_policy == 0 ? true : g_opt.load_policy == 2;
  const void* kern = element_mul_kernel_ptr(dtype, nt);
  ElementMulParams prm{static_cast<char*>(x), ld * eb, M, N, grad_output, grad_output_stride,
                       cv, chunks};
  Plan p;
  p.kernel = kern;
  p.grid = grid;
  return launch(p, &prm, static_cast<hipStream_t>(stream), kMulThreads);
}

xr_status_t xr_probe_rows(void* out, int64_t ld_out, const void* in0, const void* in1,
                          int64_t ld_in, int64_t M, int64_t N, xr_dtype_t dtype, int32_t threads,
                          int32_t vpt, int32_t split, const int64_t* target,
                          int64_t ignore_index, void* stream) {
  if (!valid_dtype(dtype)) return XR_ERR_DTYPE;
  if (M < 0 || N < 1 || split < 1) return XR_ERR_SHAPE;
  if (ld_in < N || ld_out < N) return XR_ERR_STRIDE;
  if (M == 0) return XR_OK;
  if (!span_ok(M, ld_in, N, elt_bytes(dtype)) || !span_ok(M, ld_out, N, elt_bytes(dtype)))
    return XR_ERR_SHAPE;
  if (!out || !in0) return XR_ERR_NULL;
  const int eb = elt_bytes(dtype);
  // whole 16-byte vectors only: every row on a 16-byte boundary, N a whole number of vectors
  if (!rows_on_16(out, ld_out, M, eb) || !rows_on_16(in0, ld_in, M, eb) ||
      (in1 && !rows_on_16(in1, ld_in, M, eb)) || (N * eb) % 16 != 0 ||
      (target && !aligned_to(target, 8)))
    return XR_ERR_ALIGN;
  const Shape sh{threads, vpt};
  const void* kernel = probe_rows_kernel_ptr(dtype, sh, in1 ? 2 : 1);
  if (!kernel) return XR_ERR_SHAPE;
  const int64_t nv = N * eb / 16;
  const int64_t chunk = (nv + split - 1) / split;
  if (chunk > (int64_t)threads * vpt) return XR_ERR_SHAPE;
  Plan p;
  p.kernel = kernel;
  p.grid = M * split;
  if (!grid_fits(p)) return XR_ERR_SHAPE;
  ProbeParams prm{static_cast<const char*>(in0), static_cast<const char*>(in1), ld_in * eb,
                  static_cast<char*>(out), ld_out * eb, M, N, target, ignore_index, split, chunk};
  return launch(p, &prm, static_cast<hipStream_t>(stream), threads);
}

xr_status_t xr_probe_copy(void* out, const void* in, const void* in1, int64_t bytes,
                          int32_t workgroups, int32_t threads, void* stream) {
  if (bytes < 0 || (uint64_t)bytes >= kMaxSpanBytes || workgroups < 0) return XR_ERR_SHAPE;
  if (bytes == 0) return XR_OK;
  if (!out || !in) return XR_ERR_NULL;
  if (!aligned_to(out, 16) || !aligned_to(in, 16) || (in1 && !aligned_to(in1, 16)) ||
      bytes % 16 != 0)
    return XR_ERR_ALIGN;
  // in place: out == in exactly, one input, the copy kernel
  const bool in_place = out == in;
  if ((!in_place && spans_overlap(out, bytes, in, bytes)) ||
      (in1 && spans_overlap(out, bytes, in1, bytes)) || (in_place && workgroups == 0))
    return XR_ERR_ALIAS;
  if (in_place && in1) return XR_ERR_VALUE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (workgroups == 0) {  // the runtime's copy, bracketed by the profiling events like a kernel
    if (in1) return XR_ERR_VALUE;
    const hipEvent_t ev0 = g_ev_start.load(), ev1 = g_ev_stop.load();
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return XR_ERR_LAUNCH;
    if (hipMemcpyAsync(out, in, (size_t)bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return XR_ERR_LAUNCH;
    if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return XR_ERR_LAUNCH;
    return XR_OK;
  }
  Plan p;
  p.kernel = probe_copy_kernel_ptr(threads, in_place ? 0 : in1 ? 2 : 1);
  if (!p.kernel) return XR_ERR_SHAPE;
  p.grid = workgroups;
  CopyParams prm{static_cast<const char*>(in), static_cast<const char*>(in1),
                 static_cast<char*>(out), bytes / 16};
  return launch(p, &prm, s, threads);
}

xr_status_t xr_workspace_status(const void* workspace, size_t workspace_bytes, int32_t* status,
                                void* stream) {
  if (!workspace || !status) return XR_ERR_NULL;
  if (!aligned_to(workspace, 8) || !aligned_to(status, 4)) return XR_ERR_ALIGN;
  if (workspace_bytes < kWsPartials) return XR_ERR_WORKSPACE;
  const int32_t* word = reinterpret_cast<const int32_t*>(static_cast<const char*>(workspace) +
                                                         kWsCounts) + 2;
  if (spans_overlap(word, 4, status, 4)) return XR_ERR_ALIAS;
  if (hipMemcpyAsync(status, word, sizeof(int32_t), hipMemcpyDeviceToDevice,
                     static_cast<hipStream_t>(stream)) != hipSuccess)
    return XR_ERR_LAUNCH;
  return XR_OK;
}

}  // extern "C"
