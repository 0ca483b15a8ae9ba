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
// Slots wholly past the chunk are not loaded; lanes past its end read zeros (range check).
template <int D, int THREADS, int VPT>
__device__ __forceinline__ void issue_loads(u32x4 (&v)[VPT], const Chunk<D>& c) {
  const uint32_t off = threadIdx.x * 16u;
#pragma unroll
  for (int k = 0; k < VPT; ++k)
    if (k * THREADS < c.nvec) v[k] = buf_load(c.slot(k * THREADS), off);
}

// Before a chunk is used: every element outside the row becomes `fill` (-inf for the
// softmax rows: the identity of max and a zero term of the sum; 0 for the operands of the
// softmax-backward dot product). Only slots at the chunk's end and the thread holding a
// partial first / last vector do any work; every slot index is a compile-time constant.
template <int D, int THREADS, int VPT>
__device__ __forceinline__ void fixup(u32x4 (&v)[VPT], const Chunk<D>& c, uint32_t fill) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int s0 = k * THREADS;
    if (s0 >= c.nvec) {
      v[k] = splat(fill);
    } else if (s0 + THREADS > c.nvec) {
      if (s0 + tid >= c.nvec) v[k] = splat(fill);
    }
    if (c.head >= s0 && c.head < s0 + THREADS && tid == c.head - s0)
      v[k] = mask_vec<D>(v[k], c.h0, c.h1, fill);
    if (c.tail >= s0 && c.tail < s0 + THREADS && tid == c.tail - s0)
      v[k] = mask_vec<D>(v[k], c.t0, c.t1, fill);
  }
}

// Store slot k of a chunk with one 16-byte store per lane. Lanes past the chunk's end are
// dropped by the range check; the lane holding a partial first / last vector is pointed
// outside the resource, so it stores nothing here (see store_partials).
template <int D, int THREADS>
__device__ __forceinline__ void store_slot(const Chunk<D>& c, int k, const u32x4& bits) {
  const int s0 = k * THREADS;
  if (s0 >= c.nvec) return;
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

// Compiler barrier on the register-resident vectors: each pass re-widens the bf16 / fp32
// bits it needs instead of keeping the widened values of an earlier pass alive, which
// would double or triple the registers a row takes. Placed after the pass that first
// waits for the loads, so it never delays a load.
template <int VPT> __device__ __forceinline__ void reg_barrier(u32x4 (&v)[VPT]) {
#pragma unroll
  for (int k = 0; k < VPT; ++k) asm volatile("" : "+v"(v[k]));
}

template <int D, int VPT> __device__ __forceinline__ float thread_max(const u32x4 (&v)[VPT]) {
  constexpr int EPV = Elt<D>::kPerVec;
  float a = kNegInf, b = kNegInf;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
#pragma unroll
    for (int e = 0; e < EPV; e += 2) {
      a = fmaxf(a, elem<D>(v[k], e));
      b = fmaxf(b, elem<D>(v[k], e + 1));
    }
  }
  return fmaxf(a, b);
}

// sum_j exp(x_j - m), computed as exp2(x*log2e - m*log2e), four partial sums.
template <int D, int VPT>
__device__ __forceinline__ float thread_sum_exp(const u32x4 (&v)[VPT], float mL) {
  constexpr int EPV = Elt<D>::kPerVec;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
#pragma unroll
    for (int e = 0; e < EPV; ++e)
      s[e & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(elem<D>(v[k], e), kLog2e, -mL));
  }
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// exp2(x*log2e - coff) for every element of one slot, in the element type.
template <int D>
__device__ __forceinline__ u32x4 exp_slot(const u32x4& v, float coff) {
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
__global__ __launch_bounds__(THREADS) void xent_rows_kernel(XentParams p) {
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
      fixup<D, THREADS, VPT>(v, c, Elt<D>::kNegInfWord);

      // Chunk maximum.
      m = block_reduce<THREADS>(thread_max<D, VPT>(v), OpMax(), red[0]);
      reg_barrier(v);

      // sum exp(x - m) over the chunk; an all -inf chunk contributes (-inf, 0).
      d = 0.f;
      if (m != kNegInf) d = thread_sum_exp<D, VPT>(v, m * kLog2e);
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
    const Chunk<D> cn(row_ptr(pf ? rn : r), p.V, lo, p.chunk_vecs);
    const uint32_t off = tid * 16u;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      store_slot<D, THREADS>(c, k, exp_slot<D>(v[k], coff));
      if (pf && k * THREADS < cn.nvec) v[k] = buf_load(cn.slot(k * THREADS), off);
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
__global__ __launch_bounds__(THREADS) void softmax_fwd_kernel(SoftmaxFwdParams p) {
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
    fixup<D, THREADS, VPT>(v, cx, Elt<D>::kNegInfWord);
    const float m = block_reduce<THREADS>(thread_max<D, VPT>(v), OpMax(), red[0]);
    reg_barrier(v);
    const float mL = m * kLog2e;
    const float d = block_reduce<THREADS>(thread_sum_exp<D, VPT>(v, mL), OpAdd(), red[1]);
    reg_barrier(v);
    const float coff = mL + log2f(d);
    if (rn < p.M) {
      const Chunk<D> cn(p.x + rn * p.ldx_bytes, p.N, 0, cv);
      const uint32_t off = threadIdx.x * 16u;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        store_slot<D, THREADS>(cy, k, exp_slot<D>(v[k], coff));
        if (k * THREADS < cn.nvec) v[k] = buf_load(cn.slot(k * THREADS), off);
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
__global__ __launch_bounds__(THREADS) void softmax_bwd_kernel(SoftmaxBwdParams p) {
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
    // Out-of-row elements of both operands are 0, so they add nothing to the dot product.
    fixup<D, THREADS, VPT>(vy, cy, 0u);
    fixup<D, THREADS, VPT>(vd, cy, 0u);
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
      for (int e = 0; e < EPV; ++e)
        s[e & 3] = __builtin_fmaf(elem<D>(vy[k], e), elem<D>(vd[k], e), s[e & 3]);
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
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float a = elem<D>(vy[k], e), b = elem<D>(vd[k], e);
        o.v[e] = a * (b - dot);
      }
      store_slot<D, THREADS>(cx, k, o.bits());
      if (pf && k * THREADS < cyn.nvec) {
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
