// xr_kernels.hip -- HIP kernels for the numerically stable row-softmax family on gfx950.
//
// What is computed (the pages' definitions):
//   softmax forward  y_j = exp(x_j - m) / d, m = max_j x_j, d = sum_j exp(x_j - m)
//                    (page "python sum function examples", kernels softmax_kernel / _softmax)
//   softmax backward dx_j = y_j * (dy_j - sum_k y_k dy_k)
//                    (same page, kernel _backward, block-sparse scale taken as 1)
//   cross-entropy    loss_i = m + log d - x_{t_i}; the logits are overwritten with the gradient
//                    (softmax - onehot(t_i)) / n, n = #targets != ignore_index; ignored rows
//                    get zero gradient and zero loss; mean = sum_i loss_i / n
//                    (Liger-Kernel cross_entropy.py page, liger_cross_entropy_kernel steps 1-6,
//                    LigerCrossEntropyFunction.forward)
//
// Register budget: every row kernel is compiled for at least 4 waves per SIMD (128 VGPRs),
// so a 1024-thread workgroup fits a compute unit and smaller ones can share it.
//
// How, on MI355X:
//   * Row-resident kernels keep a whole row (or, for split rows, one chunk of it) in
//     registers as raw 16-byte vectors, so the logits are read from HBM exactly once:
//     max pass, then sum pass with that max (one exp per element, no online rescale),
//     then the output pass. The output is exp2(x*log2e - c) with c = m*log2e + log2(d*n),
//     which folds the division by d and by n into the exponent.
//   * The kernels are persistent: workgroup g handles rows g, g + G, g + 2G, ... and while
//     it writes row r it already issues the loads of row r + G into the registers it has
//     just written out ("rolling prefetch"), so a CU keeps reading while it stores.
//   * Rows longer than one workgroup's registers, or batches too short to fill the GPU,
//     are split over S workgroups. Each publishes its chunk's (m_c, d_c) pair as one
//     64-bit word; the chunks of a row combine them with the online-softmax rule
//     (m, d) + (m_c, d_c) -> (max, d e^(m - max) + d_c e^(m_c - max)), chunks whose max
//     is -inf being the identity. The grid is launched cooperatively so all chunk
//     workgroups are co-resident; the wait is bounded and reports a flag if it expires.
//   * Stream kernels (one workgroup per row, element-wise, several passes over global
//     memory) handle anything the row-resident kernels do not: rows whose operands are
//     not equally aligned, rows too long for the split grid.
#include "xr_device.h"
#include "xr_internal.h"

namespace xr {

const Shape kFwdShapes[kNumFwdShapes] = {{64, 4},   {64, 8},   {64, 16},  {128, 16},
                                         {256, 16}, {512, 16}, {1024, 16}};
const Shape kBwdShapes[kNumBwdShapes] = {{64, 4},  {64, 8},   {128, 8},
                                         {256, 8}, {512, 8}, {1024, 8}};

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kSpinLimit = 1 << 20;

__device__ __forceinline__ u32x4 splat(uint32_t w) { return (u32x4){w, w, w, w}; }

__device__ __forceinline__ uint64_t pack_pair(float m, float d) {
  return (uint64_t)as_u32(m) | ((uint64_t)as_u32(d) << 32);
}
__device__ __forceinline__ float pair_m(uint64_t w) { return as_f32((uint32_t)w); }
__device__ __forceinline__ float pair_d(uint64_t w) { return as_f32((uint32_t)(w >> 32)); }

// Issue the loads of a chunk: slot k of thread tid holds chunk vector k*THREADS + tid.
// Every slot is loaded, in slot order and without branches (so the compiler can wait for
// each slot's data separately); lanes past the chunk's end read zeros without a memory
// access, and the consumers below never look at them.
template <int D, int THREADS, int VPT>
__device__ __forceinline__ void issue_loads(u32x4 (&v)[VPT], const Chunk<D>& c) {
  const uint32_t off = threadIdx.x * 16u;
#pragma unroll
  for (int k = 0; k < VPT; ++k) v[k] = buf_load(c.slot(k * THREADS), off);
}

// How slot k relates to a chunk of nvec vectors (workgroup-uniform): every lane inside,
// some lanes inside (the last slot), or none.
enum SlotKind { kSlotFull, kSlotPart, kSlotNone };
template <int THREADS>
__device__ __forceinline__ SlotKind slot_kind(int k, int nvec) {
  const int s0 = k * THREADS;
  return s0 + THREADS <= nvec ? kSlotFull : (s0 < nvec ? kSlotPart : kSlotNone);
}

// Store slot k of a chunk with one 16-byte store per lane. Lanes past the chunk's end are
// dropped by the range check; the lane holding a partial first / last vector is pointed
// outside the resource, so it stores nothing here (see store_partials).
template <int D, int THREADS>
__device__ __forceinline__ void store_slot(const Chunk<D>& c, int k, const u32x4& bits) {
  const int s0 = k * THREADS;
  uint32_t off = threadIdx.x * 16u;
  const bool slot_has_partial = (c.head >= s0 && c.head < s0 + THREADS) ||
                                (c.tail >= s0 && c.tail < s0 + THREADS);
  if (slot_has_partial) {
    const int vi = s0 + (int)threadIdx.x;
    if (vi == c.head || vi == c.tail) off = kOffNone;
  }
  buf_store(c.slot(s0), off, bits);
}

// The in-row elements of the partial first / last vectors, which store_slot skipped:
// out[j] = f(x[j]) for the elements of the row inside those vectors. The inputs are
// re-read from `in` (16 bytes each; the elements have not been written yet, since only
// this workgroup writes them), by the thread that holds the vector.
template <int D, int THREADS, class F>
__device__ __forceinline__ void store_partials(const Chunk<D>& out, const Chunk<D>& in, F f) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int vi = q == 0 ? out.head : out.tail;
    if (vi < 0 || tid != vi % THREADS) continue;
    const uint32_t off = q == 0 ? out.hoff : out.toff;
    const int e0 = q == 0 ? out.h0 : out.t0, e1 = q == 0 ? out.h1 : out.t1;
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(in.rsrc, (int)off, 0, 0);
    OutVec<D> o;
#pragma unroll
    for (int e = 0; e < Elt<D>::kPerVec; ++e) o.v[e] = f(elem<D>(x, e));
    store_partial<D>(out.rsrc, off, o.bits(), e0, e1);
  }
}

// Compiler barriers on the register-resident vectors. Each pass widens the bf16 / fp32 bits
// of one slot right before using them: left alone, the compiler widens a whole row at once
// (or keeps an earlier pass's widened values), which doubles or triples the registers a row
// takes. pin() makes one slot opaque at its point of use; being volatile, the pins also keep
// the slots in order with the memory operations between them.
__device__ __forceinline__ void pin(u32x4& x) { asm volatile("" : "+v"(x)); }
// Per-slot pins matter for bf16, whose elements are widened by extra instructions; fp32
// elements are used as they are, and pinning copies of them only adds register moves.
template <int D> __device__ __forceinline__ void pin_slot(u32x4& x) {
  if (D == kBF16) pin(x);
}
template <int VPT> __device__ __forceinline__ void reg_barrier(u32x4 (&v)[VPT]) {
#pragma unroll
  for (int k = 0; k < VPT; ++k) pin(v[k]);
}

// Slot k of this thread as the reductions must see it: lanes past the chunk's end and the
// out-of-row elements of the partial first / last vectors hold `fill` (-inf for softmax
// rows: the identity of max and a zero term of the sum; 0 for the softmax-backward dot
// product). The registers themselves are left alone (the output pass needs no masking),
// and every test is workgroup-uniform except inside the rare slots that need one.
template <int D, int THREADS>
__device__ __forceinline__ u32x4 masked_slot(u32x4 x, int k, const Chunk<D>& c, uint32_t fill) {
  pin_slot<D>(x);
  const int s0 = k * THREADS;
  const int tid = threadIdx.x;
  if (s0 + THREADS > c.nvec) {
    asm volatile("" ::: "memory");  // a real branch: no speculated wait for the load
    if (s0 + tid >= c.nvec) x = splat(fill);
  }
  if (c.head >= s0 && c.head < s0 + THREADS) {
    asm volatile("" ::: "memory");
    if (tid == c.head - s0) x = mask_vec<D>(x, c.h0, c.h1, fill);
  }
  if (c.tail >= s0 && c.tail < s0 + THREADS) {
    asm volatile("" ::: "memory");
    if (tid == c.tail - s0) x = mask_vec<D>(x, c.t0, c.t1, fill);
  }
  return x;
}

// Maximum over the chunk elements this thread holds (-inf if none).
template <int D, int THREADS, int VPT>
__device__ __forceinline__ float thread_max(const u32x4 (&v)[VPT], const Chunk<D>& c) {
  constexpr int EPV = Elt<D>::kPerVec;
  float a = kNegInf, b = kNegInf;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (slot_kind<THREADS>(k, c.nvec) == kSlotNone) continue;
    const u32x4 x = masked_slot<D, THREADS>(v[k], k, c, Elt<D>::kNegInfWord);
#pragma unroll
    for (int e = 0; e < EPV; e += 2) {
      a = fmaxf(a, elem<D>(x, e));
      b = fmaxf(b, elem<D>(x, e + 1));
    }
  }
  return fmaxf(a, b);
}

// sum_j exp(x_j - m) over the chunk elements this thread holds, computed as
// exp2(x*log2e - m*log2e), four partial sums.
template <int D, int THREADS, int VPT>
__device__ __forceinline__ float thread_sum_exp(const u32x4 (&v)[VPT], const Chunk<D>& c, float mL) {
  constexpr int EPV = Elt<D>::kPerVec;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (slot_kind<THREADS>(k, c.nvec) == kSlotNone) continue;
    const u32x4 x = masked_slot<D, THREADS>(v[k], k, c, Elt<D>::kNegInfWord);
#pragma unroll
    for (int e = 0; e < EPV; ++e)
      s[e & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(elem<D>(x, e), kLog2e, -mL));
  }
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// exp2(x*log2e - coff) for every element of one slot, in the element type.
template <int D>
__device__ __forceinline__ u32x4 exp_slot(u32x4 v, float coff) {
  pin_slot<D>(v);
  OutVec<D> o;
#pragma unroll
  for (int e = 0; e < Elt<D>::kPerVec; ++e)
    o.v[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(elem<D>(v, e), kLog2e, -coff));
  return o.bits();
}

}  // namespace

// ============================================================================ cross-entropy
// Target scan: n = #{t != ignore_index}, bad = #{t != ignore_index, t outside [0, V)}.
// Also clears the error flags and marks every split-row (m, d) slot as unpublished.
__global__ __launch_bounds__(kScanThreads) void xent_scan_kernel(const int64_t* __restrict__ target,
                                                                 int64_t M, int64_t V,
                                                                 int64_t ignore_index,
                                                                 int32_t* __restrict__ ws_counts,
                                                                 uint64_t* __restrict__ partials,
                                                                 int64_t nslots) {
  __shared__ int red[2][kScanThreads / kWave];
  int n = 0, bad = 0;
  for (int64_t i = threadIdx.x; i < M; i += kScanThreads) {
    const int64_t t = target[i];
    if (t != ignore_index) {
      ++n;
      if (t < 0 || t >= V) ++bad;
    }
  }
  n = block_sum_int<kScanThreads>(n, red[0]);
  bad = block_sum_int<kScanThreads>(bad, red[1]);
  if (threadIdx.x == 0) {
    ws_counts[0] = n;
    ws_counts[1] = bad;
    ws_counts[2] = 0;
    ws_counts[3] = 0;
  }
  for (int64_t i = threadIdx.x; i < nslots; i += kScanThreads) partials[i] = kPartialEmpty;
}

// Mean over the row losses in a fixed order; copies the counts out.
__global__ __launch_bounds__(kScanThreads) void xent_mean_kernel(const float* __restrict__ row_loss,
                                                                 int64_t M,
                                                                 const int32_t* __restrict__ ws_counts,
                                                                 float* __restrict__ mean,
                                                                 int32_t* __restrict__ counts_out) {
  __shared__ float red[kScanThreads / kWave];
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < M; i += kScanThreads) s += row_loss[i];
  s = block_reduce<kScanThreads>(s, OpAdd(), red);
  if (threadIdx.x == 0) {
    const int32_t n = ws_counts[0];
    *mean = s / (float)n;  // n == 0: 0/0 = NaN
    if (counts_out) {
      counts_out[0] = n;
      counts_out[1] = ws_counts[1];
      counts_out[2] = ws_counts[2];
    }
  }
}

// Row-resident fused cross-entropy; S workgroups per row (S == 1: the whole row).
template <int D, int THREADS, int VPT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void xent_rows_kernel(XentParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int NW = THREADS / kWave;
  __shared__ float red[2][NW];
  __shared__ float bcast[2];

  const int tid = threadIdx.x;
  const int S = p.S;
  const int64_t grp = blockIdx.x / S;
  const int chunk = blockIdx.x % S;
  const int64_t lo = (int64_t)chunk * p.chunk_vecs;
  const int32_t n = p.ws_counts[0];
  const float inv_n = 1.0f / (float)n;
  const float log2n = log2f((float)n);

  auto skip = [&](int64_t t) { return t == p.ignore_index || t < 0 || t >= p.V; };
  auto row_ptr = [&](int64_t r) { return p.logits + r * p.ld_bytes; };

  u32x4 v[VPT];
  int64_t r = grp;
  int64_t t = (r < p.M) ? p.target[r] : p.ignore_index;
  if (r < p.M && !skip(t)) issue_loads<D, THREADS, VPT>(v, Chunk<D>(row_ptr(r), p.V, lo, p.chunk_vecs));

  while (r < p.M) {
    const int64_t rn = r + p.groups;
    const int64_t tn = (rn < p.M) ? p.target[rn] : p.ignore_index;
    const bool pf = rn < p.M && !skip(tn);
    const Chunk<D> c(row_ptr(r), p.V, lo, p.chunk_vecs);
    const bool ignored = skip(t);

    // The target logit, read by the thread holding its vector. Only this workgroup
    // writes this chunk, and it does so after the barriers below.
    const int64_t vt = c.lead + t - c.lo * EPV;  // chunk-local element index of the target
    const bool owner = !ignored && vt >= 0 && vt < (int64_t)c.nvec * EPV &&
                       tid == (int)(vt / EPV) % THREADS;
    float xt = 0.f;
    if (owner) xt = buf_load_elem<D>(c.rsrc, (uint32_t)(vt * Elt<D>::kBytes));

    float m = 0.f, d = 1.f, coff;
    if (ignored) {
      // Ignored (or out-of-range) target: the row was not loaded; with every input at
      // -inf and c = +inf the output pass below writes exact zeros.
#pragma unroll
      for (int k = 0; k < VPT; ++k) v[k] = splat(Elt<D>::kNegInfWord);
      coff = __builtin_inff();
    } else {
      // Chunk maximum.
      m = block_reduce<THREADS>(thread_max<D, THREADS, VPT>(v, c), OpMax(), red[0]);
      reg_barrier(v);

      // sum exp(x - m) over the chunk; an all -inf chunk contributes (-inf, 0).
      d = 0.f;
      if (m != kNegInf) d = thread_sum_exp<D, THREADS, VPT>(v, c, m * kLog2e);
      d = block_reduce<THREADS>(d, OpAdd(), red[1]);
      if (m == kNegInf) d = 0.f;
      reg_barrier(v);

      if (S > 1) {
        // Publish this chunk's pair, then combine the pairs of all chunks of the row in
        // chunk order (every chunk of the row computes the same (m, d)).
        if (tid == 0) {
          uint64_t* slot = p.partials + r * S;
          __hip_atomic_store(slot + chunk, pack_pair(m, d), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          float ms = kNegInf, ds = 0.f;
          bool ok = true;
          // One bounded wait for the whole row; after any timeout in this call no
          // workgroup waits again (the flag is set), so the kernel always drains.
          int budget = (__hip_atomic_load(p.ws_flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                        kFlagExchangeTimeout) ? 0 : kSpinLimit;
          for (int q = 0; q < S && ok; ++q) {
            uint64_t w;
            while ((w = __hip_atomic_load(slot + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) ==
                   kPartialEmpty) {
              if (--budget < 0) {
                ok = false;
                break;
              }
              __builtin_amdgcn_s_sleep(2);
            }
            if (!ok) break;
            const float mc = pair_m(w), dc = pair_d(w);
            if (mc == kNegInf) continue;
            const float mx = fmaxf(ms, mc);
            ds = ((ms == kNegInf) ? 0.f : ds * exp2f((ms - mx) * kLog2e)) +
                 dc * exp2f((mc - mx) * kLog2e);
            ms = mx;
          }
          if (!ok) {
            __hip_atomic_fetch_or(p.ws_flags, kFlagExchangeTimeout, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
            ms = __builtin_nanf("");
          }
          bcast[0] = ms;
          bcast[1] = ds;
        }
        __syncthreads();
        m = bcast[0];
        d = bcast[1];
      }
      // g_j = exp2(x_j*log2e - c) with c = m*log2e + log2(d) + log2(n) is p_j / n.
      coff = m * kLog2e + log2f(d) + log2n;
    }

    // Output pass, with the next row's loads issued into each slot once it is written out.
    if (pf) {
      const Chunk<D> cn(row_ptr(rn), p.V, lo, p.chunk_vecs);
      const uint32_t off = tid * 16u;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        store_slot<D, THREADS>(c, k, exp_slot<D>(v[k], coff));
        v[k] = buf_load(cn.slot(k * THREADS), off);
      }
    } else {
#pragma unroll
      for (int k = 0; k < VPT; ++k) store_slot<D, THREADS>(c, k, exp_slot<D>(v[k], coff));
    }
    store_partials<D, THREADS>(c, c, [coff, ignored](float x) {
      return ignored ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -coff));
    });
    if (owner) {
      // Target column: (p_t - 1)/n rounded once, stored after this thread's vector store.
      const float pt = exp2f((xt - m) * kLog2e) / d;
      store_elem<D>(c.rsrc, (uint32_t)(vt * Elt<D>::kBytes), (pt - 1.0f) * inv_n);
      p.row_loss[r] = m + logf(d) - xt;
    }
    if (ignored && chunk == 0 && tid == 0) p.row_loss[r] = 0.f;
    r = rn;
    t = tn;
  }
}

// Stream fallback: one workgroup per row, element-wise, max / sum / write passes over memory.
template <int D>
__global__ __launch_bounds__(kStreamThreads) void xent_stream_kernel(XentParams p) {
  __shared__ float red[2][kStreamThreads / kWave];
  const int64_t r = blockIdx.x;
  if (r >= p.M) return;
  const int64_t t = p.target[r];
  char* row = p.logits + r * p.ld_bytes;
  const int tid = threadIdx.x;
  auto ld = [&](int64_t j) -> float {
    if (D == kF32) return reinterpret_cast<const float*>(row)[j];
    return as_f32((uint32_t)reinterpret_cast<const uint16_t*>(row)[j] << 16);
  };
  auto st = [&](int64_t j, float val) {
    if (D == kF32) reinterpret_cast<float*>(row)[j] = val;
    else reinterpret_cast<uint16_t*>(row)[j] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
  };
  if (t == p.ignore_index || t < 0 || t >= p.V) {
    for (int64_t j = tid; j < p.V; j += kStreamThreads) st(j, 0.f);
    if (tid == 0) p.row_loss[r] = 0.f;
    return;
  }
  const int32_t n = p.ws_counts[0];
  const float xt = ld(t);
  float m = kNegInf;
  for (int64_t j = tid; j < p.V; j += kStreamThreads) m = fmaxf(m, ld(j));
  m = block_reduce<kStreamThreads>(m, OpMax(), red[0]);
  const float mL = m * kLog2e;
  float d = 0.f;
  for (int64_t j = tid; j < p.V; j += kStreamThreads)
    d += __builtin_amdgcn_exp2f(__builtin_fmaf(ld(j), kLog2e, -mL));
  d = block_reduce<kStreamThreads>(d, OpAdd(), red[1]);
  // Every thread has read xt and the row before the barrier inside the reductions.
  const float coff = mL + log2f(d) + log2f((float)n);
  for (int64_t j = tid; j < p.V; j += kStreamThreads) {
    const float g = (j == t) ? (exp2f((xt - m) * kLog2e) / d - 1.0f) / (float)n
                             : __builtin_amdgcn_exp2f(__builtin_fmaf(ld(j), kLog2e, -coff));
    st(j, g);
  }
  if (tid == 0) p.row_loss[r] = m + logf(d) - xt;
}

// ============================================================================ softmax forward
template <int D, int THREADS, int VPT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void softmax_fwd_kernel(SoftmaxFwdParams p) {
  constexpr int NW = THREADS / kWave;
  __shared__ float red[2][NW];
  const int64_t G = gridDim.x;
  const int64_t cv = p.N + Elt<D>::kPerVec;  // more vectors than any row has: whole rows

  u32x4 v[VPT];
  int64_t r = blockIdx.x;
  if (r < p.M) issue_loads<D, THREADS, VPT>(v, Chunk<D>(p.x + r * p.ldx_bytes, p.N, 0, cv));
  while (r < p.M) {
    const int64_t rn = r + G;
    const Chunk<D> cx(p.x + r * p.ldx_bytes, p.N, 0, cv);
    const Chunk<D> cy(p.y + r * p.ldy_bytes, p.N, 0, cv);  // same lead as cx (host-checked)
    const float m = block_reduce<THREADS>(thread_max<D, THREADS, VPT>(v, cx), OpMax(), red[0]);
    reg_barrier(v);
    const float mL = m * kLog2e;
    const float d =
        block_reduce<THREADS>(thread_sum_exp<D, THREADS, VPT>(v, cx, mL), OpAdd(), red[1]);
    reg_barrier(v);
    const float coff = mL + log2f(d);
    if (rn < p.M) {
      const Chunk<D> cn(p.x + rn * p.ldx_bytes, p.N, 0, cv);
      const uint32_t off = threadIdx.x * 16u;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        store_slot<D, THREADS>(cy, k, exp_slot<D>(v[k], coff));
        v[k] = buf_load(cn.slot(k * THREADS), off);
      }
    } else {
#pragma unroll
      for (int k = 0; k < VPT; ++k) store_slot<D, THREADS>(cy, k, exp_slot<D>(v[k], coff));
    }
    store_partials<D, THREADS>(cy, cx, [coff](float x) {
      return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -coff));
    });
    r = rn;
  }
}

template <int D>
__global__ __launch_bounds__(kStreamThreads) void softmax_fwd_stream_kernel(SoftmaxFwdParams p) {
  __shared__ float red[2][kStreamThreads / kWave];
  const int64_t r = blockIdx.x;
  if (r >= p.M) return;
  const char* row = p.x + r * p.ldx_bytes;
  char* out = p.y + r * p.ldy_bytes;
  const int tid = threadIdx.x;
  auto ld = [&](int64_t j) -> float {
    if (D == kF32) return reinterpret_cast<const float*>(row)[j];
    return as_f32((uint32_t)reinterpret_cast<const uint16_t*>(row)[j] << 16);
  };
  float m = kNegInf;
  for (int64_t j = tid; j < p.N; j += kStreamThreads) m = fmaxf(m, ld(j));
  m = block_reduce<kStreamThreads>(m, OpMax(), red[0]);
  const float mL = m * kLog2e;
  float d = 0.f;
  for (int64_t j = tid; j < p.N; j += kStreamThreads)
    d += __builtin_amdgcn_exp2f(__builtin_fmaf(ld(j), kLog2e, -mL));
  d = block_reduce<kStreamThreads>(d, OpAdd(), red[1]);
  // In place (y == x) is safe: every element's output depends only on itself and (m, d),
  // and all reads of the max / sum passes finished before the barrier above.
  const float coff = mL + log2f(d);
  for (int64_t j = tid; j < p.N; j += kStreamThreads) {
    const float val = __builtin_amdgcn_exp2f(__builtin_fmaf(ld(j), kLog2e, -coff));
    if (D == kF32) reinterpret_cast<float*>(out)[j] = val;
    else reinterpret_cast<uint16_t*>(out)[j] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
  }
}

// ============================================================================ softmax backward
template <int D, int THREADS, int VPT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void softmax_bwd_kernel(SoftmaxBwdParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int NW = THREADS / kWave;
  __shared__ float red[2][NW];
  const int64_t G = gridDim.x;
  const int64_t cv = p.N + EPV;

  u32x4 vy[VPT], vd[VPT];
  int64_t r = blockIdx.x;
  int buf = 0;
  if (r < p.M) {
    issue_loads<D, THREADS, VPT>(vy, Chunk<D>(p.y + r * p.ldy_bytes, p.N, 0, cv));
    issue_loads<D, THREADS, VPT>(vd, Chunk<D>(p.dy + r * p.lddy_bytes, p.N, 0, cv));
  }
  while (r < p.M) {
    const int64_t rn = r + G;
    // y, dy and dx rows share their alignment (host-checked), hence their vector layout.
    const Chunk<D> cy(p.y + r * p.ldy_bytes, p.N, 0, cv);
    const Chunk<D> cx(p.dx + r * p.lddx_bytes, p.N, 0, cv);
    // Out-of-row elements of both operands count as 0: they add nothing to the dot product.
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (slot_kind<THREADS>(k, cy.nvec) == kSlotNone) continue;
      const u32x4 a = masked_slot<D, THREADS>(vy[k], k, cy, 0u);
      const u32x4 b = masked_slot<D, THREADS>(vd[k], k, cy, 0u);
#pragma unroll
      for (int e = 0; e < EPV; ++e)
        s[e & 3] = __builtin_fmaf(elem<D>(a, e), elem<D>(b, e), s[e & 3]);
    }
    const float dot = block_reduce<THREADS>((s[0] + s[1]) + (s[2] + s[3]), OpAdd(), red[buf]);
    buf ^= 1;
    reg_barrier(vy);
    reg_barrier(vd);
    const bool pf = rn < p.M;
    const Chunk<D> cyn(p.y + (pf ? rn : r) * p.ldy_bytes, p.N, 0, cv);
    const Chunk<D> cdn(p.dy + (pf ? rn : r) * p.lddy_bytes, p.N, 0, cv);
    const uint32_t off = threadIdx.x * 16u;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      OutVec<D> o;
      u32x4 a = vy[k], b = vd[k];
      pin_slot<D>(a);
      pin_slot<D>(b);
#pragma unroll
      for (int e = 0; e < EPV; ++e) o.v[e] = elem<D>(a, e) * (elem<D>(b, e) - dot);
      store_slot<D, THREADS>(cx, k, o.bits());
      if (pf) {
        vy[k] = buf_load(cyn.slot(k * THREADS), off);
        vd[k] = buf_load(cdn.slot(k * THREADS), off);
      }
    }
    // Partial first / last vectors: re-read y and dy (this workgroup has not written them;
    // dx may be exactly y or dy) and store only the in-row elements.
    {
      const Chunk<D> cd(p.dy + r * p.lddy_bytes, p.N, 0, cv);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int vi = q == 0 ? cx.head : cx.tail;
        if (vi < 0 || (int)threadIdx.x != vi % THREADS) continue;
        const uint32_t po = q == 0 ? cx.hoff : cx.toff;
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(cy.rsrc, (int)po, 0, 0);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(cd.rsrc, (int)po, 0, 0);
        OutVec<D> o;
#pragma unroll
        for (int e = 0; e < EPV; ++e) o.v[e] = elem<D>(a, e) * (elem<D>(b, e) - dot);
        store_partial<D>(cx.rsrc, po, o.bits(), q == 0 ? cx.h0 : cx.t0, q == 0 ? cx.h1 : cx.t1);
      }
    }
    r = rn;
  }
}

template <int D>
__global__ __launch_bounds__(kStreamThreads) void softmax_bwd_stream_kernel(SoftmaxBwdParams p) {
  __shared__ float red[kStreamThreads / kWave];
  const int64_t r = blockIdx.x;
  if (r >= p.M) return;
  const char* yr = p.y + r * p.ldy_bytes;
  const char* dr = p.dy + r * p.lddy_bytes;
  char* out = p.dx + r * p.lddx_bytes;
  const int tid = threadIdx.x;
  auto ld = [&](const char* row, int64_t j) -> float {
    if (D == kF32) return reinterpret_cast<const float*>(row)[j];
    return as_f32((uint32_t)reinterpret_cast<const uint16_t*>(row)[j] << 16);
  };
  float s = 0.f;
  for (int64_t j = tid; j < p.N; j += kStreamThreads) s += ld(yr, j) * ld(dr, j);
  s = block_reduce<kStreamThreads>(s, OpAdd(), red);
  for (int64_t j = tid; j < p.N; j += kStreamThreads) {
    const float val = ld(yr, j) * (ld(dr, j) - s);
    if (D == kF32) reinterpret_cast<float*>(out)[j] = val;
    else reinterpret_cast<uint16_t*>(out)[j] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
  }
}

// ============================================================================ lookup tables
#define XR_SHAPES_FWD(X, D)                                                                     \
  X(D, 64, 4) X(D, 64, 8) X(D, 64, 16) X(D, 128, 16) X(D, 256, 16) X(D, 512, 16) X(D, 1024, 16)
#define XR_SHAPES_BWD(X, D) \
  X(D, 64, 4) X(D, 64, 8) X(D, 128, 8) X(D, 256, 8) X(D, 512, 8) X(D, 1024, 8)

#define XR_CASE_XENT(D, T, V) \
  if (s.threads == T && s.vpt == V) return reinterpret_cast<const void*>(&xent_rows_kernel<D, T, V>);
#define XR_CASE_SFWD(D, T, V) \
  if (s.threads == T && s.vpt == V) return reinterpret_cast<const void*>(&softmax_fwd_kernel<D, T, V>);
#define XR_CASE_SBWD(D, T, V) \
  if (s.threads == T && s.vpt == V) return reinterpret_cast<const void*>(&softmax_bwd_kernel<D, T, V>);

const void* xent_rows_kernel_ptr(int dtype, Shape s) {
  if (dtype == kF32) { XR_SHAPES_FWD(XR_CASE_XENT, kF32) }
  if (dtype == kBF16) { XR_SHAPES_FWD(XR_CASE_XENT, kBF16) }
  return nullptr;
}
const void* softmax_fwd_kernel_ptr(int dtype, Shape s) {
  if (dtype == kF32) { XR_SHAPES_FWD(XR_CASE_SFWD, kF32) }
  if (dtype == kBF16) { XR_SHAPES_FWD(XR_CASE_SFWD, kBF16) }
  return nullptr;
}
const void* softmax_bwd_kernel_ptr(int dtype, Shape s) {
  if (dtype == kF32) { XR_SHAPES_BWD(XR_CASE_SBWD, kF32) }
  if (dtype == kBF16) { XR_SHAPES_BWD(XR_CASE_SBWD, kBF16) }
  return nullptr;
}
const void* xent_stream_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&xent_stream_kernel<kF32>)
                       : reinterpret_cast<const void*>(&xent_stream_kernel<kBF16>);
}
const void* softmax_fwd_stream_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&softmax_fwd_stream_kernel<kF32>)
                       : reinterpret_cast<const void*>(&softmax_fwd_stream_kernel<kBF16>);
}
const void* softmax_bwd_stream_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&softmax_bwd_stream_kernel<kF32>)
                       : reinterpret_cast<const void*>(&softmax_bwd_stream_kernel<kBF16>);
}
const void* xent_scan_kernel_ptr() { return reinterpret_cast<const void*>(&xent_scan_kernel); }
const void* xent_mean_kernel_ptr() { return reinterpret_cast<const void*>(&xent_mean_kernel); }

}  // namespace xr
