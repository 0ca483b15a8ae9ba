// xr_xent.hip -- fused cross-entropy kernels (and the notes on every row kernel) for gfx950.
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
//                    LigerCrossEntropyFunction.forward). The sum reduction drops the 1/n,
//                    the none reduction keeps the row losses; an upstream gradient s_i
//                    multiplies row i's gradient as it is written (what the same page's
//                    backward does afterwards with element_mul, which is also here).
//
// Register budget: every row kernel is compiled for at least 4 waves per SIMD (128 VGPRs),
// so a 1024-thread workgroup fits a compute unit and smaller ones can share it.
//
// How, on MI355X:
//   * Row-resident kernels keep a whole row (or, for split rows, one chunk of it) in
//     registers as raw 16-byte vectors, so the logits are read from HBM exactly once:
//     max pass, then sum pass with that max (one exp per element, no online rescale),
//     then the output pass. The output is exp2((x - m)*log2e - log2(d*n)), which folds the
//     division by d and by n into the exponent; ordinary rows fold m into its constant too,
//     rows of large magnitude form x - m first (xr_rows.h).
//   * One workgroup per row, or per row chunk, by default: the dispatcher starts a new
//     workgroup as soon as one retires. A persistent form (workgroup g handles rows g,
//     g + G, ... and, once it has issued row r's stores, issues the loads of row r + G
//     into the same registers) is kept for grids set explicitly.
//   * Long rows, and batches too short to fill the GPU, are split over S workgroups. Each
//     publishes its chunk's (m_c, d_c) pair as one 64-bit word; the chunks of a row
//     combine them with the online-softmax rule
//     (m, d) + (m_c, d_c) -> (max, d e^(m - max) + d_c e^(m_c - max)), chunks whose max
//     is -inf being the identity. A row's chunks have consecutive workgroup ids, so in a
//     normal launch a chunk waits only for chunks already started or next in line (a
//     persistent grid is launched cooperatively); the wait is bounded and reports a flag
//     if it expires. Rows of a few large chunks are written back in groups of 8 adjacent
//     rows: after its own row's exchange a chunk also waits (bounded, deciding nothing)
//     for the other rows of its group to publish, so that their stores go out together.
//   * Stream kernels (one workgroup per row, element-wise, several passes over global
//     memory) handle anything the row-resident kernels do not: rows whose operands are
//     not equally aligned, rows too long for the split grid.
#include "xr_rows.h"

namespace xr {

// ============================================================================ cross-entropy
// Target scan: n = #{t != ignore_index}, bad = #{t != ignore_index, t outside [0, V)},
// counted by workgroup 0 (16-byte loads, two targets each, all issued before the sums),
// which also sets the error flags to `init_flags` (0; a test sets the exchange-timeout flag
// so that split rows do not wait); every workgroup marks its share of the split-row (m, d)
// slots as unpublished.
__global__ __launch_bounds__(kScanThreads) void xent_scan_kernel(const int64_t* __restrict__ target,
                                                                 int64_t M, int64_t V,
                                                                 int64_t ignore_index,
                                                                 int32_t* __restrict__ ws_counts,
                                                                 uint64_t* __restrict__ partials,
                                                                 int64_t nslots, int32_t init_flags) {
  __shared__ int red[2][kScanThreads / kWave];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    int n = 0, bad = 0;
    auto count = [&](int64_t t) {
      if (t != ignore_index) {
        ++n;
        if (t < 0 || t >= V) ++bad;
      }
    };
    const bool vec = (reinterpret_cast<uintptr_t>(target) & 15u) == 0;
    const int64_t pairs = vec ? M / 2 : 0;
    constexpr int U = 8;  // pairs per thread per round, loaded together
    for (int64_t base = 0; base < pairs; base += (int64_t)U * kScanThreads) {
      longlong2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kScanThreads + tid;
        v[u] = i < pairs ? reinterpret_cast<const longlong2*>(target)[i] : make_longlong2(ignore_index, ignore_index);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        count(v[u].x);
        count(v[u].y);
      }
    }
    for (int64_t i = 2 * pairs + tid; i < M; i += kScanThreads) count(target[i]);
    n = block_sum_int<kScanThreads>(n, red[0]);
    bad = block_sum_int<kScanThreads>(bad, red[1]);
    if (tid == 0) {
      ws_counts[0] = n;
      ws_counts[1] = bad;
      ws_counts[2] = init_flags;
      ws_counts[3] = 0;
    }
  }
  for (int64_t i = (int64_t)blockIdx.x * kScanThreads + tid; i < nslots;
       i += (int64_t)gridDim.x * kScanThreads)
    partials[i] = kPartialEmpty;
}

// Sum (or mean) of the row losses in a fixed order (16-byte loads issued together, then a
// fixed tree); copies the counts out.
__global__ __launch_bounds__(kScanThreads) void xent_mean_kernel(const float* __restrict__ row_loss,
                                                                 int64_t M,
                                                                 const int32_t* __restrict__ ws_counts,
                                                                 float* __restrict__ mean,
                                                                 int32_t* __restrict__ counts_out,
                                                                 int reduction) {
  __shared__ float red[kScanThreads / kWave];
  const int tid = threadIdx.x;
  float s = 0.f;
  const bool vec = (reinterpret_cast<uintptr_t>(row_loss) & 15u) == 0;
  const int64_t quads = vec ? M / 4 : 0;
  constexpr int U = 8;
  for (int64_t base = 0; base < quads; base += (int64_t)U * kScanThreads) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * kScanThreads + tid;
      v[u] = i < quads ? reinterpret_cast<const float4*>(row_loss)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) s += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  for (int64_t i = 4 * quads + tid; i < M; i += kScanThreads) s += row_loss[i];
  s = block_reduce<kScanThreads>(s, OpAdd(), red);
  if (tid == 0) {
    const int32_t n = ws_counts[0];
    if (mean) *mean = reduction == kReduceMean ? s / (float)n : s;  // n == 0: 0/0 = NaN
    if (counts_out) {
      counts_out[0] = n;
      counts_out[1] = ws_counts[1];
      counts_out[2] = ws_counts[2];
    }
  }
}

// Row-resident fused cross-entropy; S workgroups per row (S == 1: the whole row).
template <int D, int THREADS, int VPT, int LP>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void xent_rows_kernel(XentParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int NW = THREADS / kWave;
  __shared__ float2 red[2][NW];
  __shared__ float bcast[2];
  int buf = 0;

  const int tid = threadIdx.x;
  const int S = p.S;
  const int64_t grp = blockIdx.x / S;
  const int chunk = blockIdx.x % S;
  const int64_t lo = (int64_t)chunk * p.chunk_vecs;
  const int32_t n = p.ws_counts[0];
  const bool mean = p.reduction == kReduceMean;
  const float inv_n = mean ? 1.0f / (float)n : 1.0f;
  const float log2n = mean ? log2f((float)n) : 0.0f;

  auto skip = [&](int64_t t) { return t == p.ignore_index || t < 0 || t >= p.V; };
  auto row_ptr = [&](int64_t r) { return p.logits + r * p.ld_bytes; };

  u32x4 v[VPT];
  int64_t r = grp;
  int64_t t = (r < p.M) ? p.target[r] : p.ignore_index;
  if (r < p.M && !skip(t)) issue_loads<D, THREADS, VPT, LP>(v, Chunk<D>(row_ptr(r), p.V, lo, p.chunk_vecs));

  while (r < p.M) {
    const int64_t rn = r + p.groups;
    const int64_t tn = (rn < p.M) ? p.target[rn] : p.ignore_index;
    const bool pf = rn < p.M && !skip(tn);
    const Chunk<D> c(row_ptr(r), p.V, lo, p.chunk_vecs);
    const bool ignored = skip(t);
    // Upstream gradient of this row's loss (1 when none is given).
    const float sc = p.gscale ? p.gscale[r * p.gstride] : 1.0f;
    bool neg = false;

    // The target logit, read by the thread holding its vector. Only this workgroup
    // writes this chunk, and it does so after the barriers below.
    const int64_t vt = c.lead + t - c.lo * EPV;  // chunk-local element index of the target
    const bool owner = !ignored && vt >= 0 && vt < (int64_t)c.nvec * EPV &&
                       tid == (int)(vt / EPV) % THREADS;
    float xt = 0.f;
    if (owner) xt = buf_load_elem<D>(c.rsrc, (uint32_t)(vt * Elt<D>::kBytes));

    float m = 0.f, d = 1.f, off;  // outputs exp2((x - m) log2e - off)
    if (ignored) {
      // Ignored (or out-of-range) target: the row was not loaded; with every input at
      // -inf, m = 0 and off = +inf the output pass below writes exact zeros.
#pragma unroll
      for (int k = 0; k < VPT; ++k) v[k] = splat(Elt<D>::kNegInfWord);
      off = __builtin_inff();
    } else {
      // (m, d) of the chunk; an all -inf chunk gives (-inf, 0).
      const Stats st = block_reduce_stats<THREADS>(thread_stats<D, THREADS, VPT>(v, c), red[buf]);
      buf ^= 1;
      m = st.m;
      d = st.d;

      if (S > 1) {
        // every chunk of the row combines the same pairs in the same order
        const Stats row = exchange_row_stats<THREADS>({m, d}, p.partials + r * S, S, chunk,
                                                       p.ws_flags, bcast);
        m = row.m;
        d = row.d;
        if (p.group_rows > 1)
          wait_row_group<kWriteGroupRows>(p.partials, p.target, p.ignore_index, p.V, r, p.M, S,
                                         p.ws_flags);
      }
      // g_j = exp2((x_j - m) log2e - off) with off = log2(d) + log2(n) - log2|s| is
      // |s| p_j / n (n = 1 unless the reduction is the mean); the sign of s is applied to
      // the result bits.
      off = log2f(d) + log2n - log2f(fabsf(sc));
      neg = __builtin_signbit(sc) != 0;
    }

    // Output pass; then the next row's loads.
    const uint32_t sign = neg ? Elt<D>::kSignWord : 0u;
    const ExpForm f = exp_form(m, off);
    with_form(f, [&](auto form) {
      constexpr bool SC = decltype(form)::value;
#pragma unroll
      for (int k = 0; k < VPT; ++k) store_slot<D, THREADS>(c, k, exp_slot<D, SC>(v[k], f, sign));
      store_partials<D, THREADS>(c, c, [&f, ignored, neg](float x) {
        const float g = exp_of<SC>(x, f);
        return ignored ? 0.f : (neg ? -g : g);
      });
    });
    if (pf) {
      const Chunk<D> cn(row_ptr(rn), p.V, lo, p.chunk_vecs);
      const uint32_t voff = tid * 16u;
#pragma unroll
      for (int k = 0; k < VPT; ++k) v[k] = buf_load<LP>(cn.slot(k * THREADS), voff);
    }
    if (owner) {
      // Target column: s (p_t - 1)/n, stored after this thread's vector store. p_t's
      // numerator is formed as the sum pass forms the terms of d (in the row's form), so
      // that p_t near 1 keeps its accuracy (p_t - 1 cancels).
      const float et = f.scaled ? __builtin_fmaf(xt, kLog2e, -scaled_max(m)) : (xt - m) * kLog2e;
      const float pt = __builtin_amdgcn_exp2f(et) / d;
      store_elem<D>(c.rsrc, (uint32_t)(vt * Elt<D>::kBytes), (pt - 1.0f) * inv_n * sc);
      p.row_loss[r] = (m - xt) + logf(d);  // m - xt exact near the maximum, at any magnitude
    }
    if (ignored && chunk == 0 && tid == 0) p.row_loss[r] = 0.f;
    r = rn;
    t = tn;
  }
}

// Stream fallback (sizes no row-resident shape takes): one workgroup per row, two passes
// over memory in 16-byte vectors: per-thread online (m, d) pairs and their workgroup
// combine, then the gradient written over the logits (each vector re-read and written by
// the same thread).
template <int D>
__global__ __launch_bounds__(kStreamThreads) void xent_stream_kernel(XentParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int T = kStreamThreads;
  constexpr int U = kStreamUnroll;
  __shared__ float2 red[T / kWave];
  const int64_t r = blockIdx.x;
  if (r >= p.M) return;
  const int64_t t = p.target[r];
  char* row = p.logits + r * p.ld_bytes;
  const int tid = threadIdx.x;
  const int lead = (int)(((uintptr_t)row & 15u) / Elt<D>::kBytes);
  const int64_t nv = (lead + p.V + EPV - 1) / EPV;
  if (t == p.ignore_index || t < 0 || t >= p.V) {
    for (int64_t lo = 0; lo < nv; lo += kStreamWindow) {
      const Chunk<D> c(row, p.V, lo, kStreamWindow);
      for (int v = tid; v < c.nvec; v += T) store_vec<D>(c, v, splat(0u));
    }
    if (tid == 0) p.row_loss[r] = 0.f;
    return;
  }
  const bool mean = p.reduction == kReduceMean;
  const int32_t n = mean ? p.ws_counts[0] : 1;
  const float inv_n = mean ? 1.0f / (float)n : 1.0f;
  const float sc = p.gscale ? p.gscale[r * p.gstride] : 1.0f;
  const bool neg = __builtin_signbit(sc) != 0;
  // the target logit, read by every thread before the barrier below
  const float xt = D == kF32 ? reinterpret_cast<const float*>(row)[t]
                             : as_f32((uint32_t)reinterpret_cast<const uint16_t*>(row)[t] << 16);
  Stats st{kNegInf, 0.f};
  for (int64_t lo = 0; lo < nv; lo += kStreamWindow) {
    const Chunk<D> c(row, p.V, lo, kStreamWindow);
    for (int v0 = tid; v0 < c.nvec; v0 += U * T) {
      u32x4 a[U];
#pragma unroll
      for (int q = 0; q < U; ++q) a[q] = buf_load<kPolicyDefault>(c.rsrc, (uint32_t)(v0 + q * T) * 16u);
#pragma unroll
      for (int q = 0; q < U; ++q)
        online_add_vec<D>(st, vec_masked<D>(a[q], v0 + q * T, c, Elt<D>::kNegInfWord));
    }
  }
  st = block_reduce_stats<T>(st, red);
  const float m = st.m, d = st.d;
  // gradient exp2((x - m) log2e - off) = s p_j / n for j != target; s (p_t - 1) / n at the
  // target (p_t's numerator formed as the online sums form their terms)
  const ExpForm f = exp_form(m, log2f(d) + log2f((float)n) - log2f(fabsf(sc)));
  const float gt = (__builtin_amdgcn_exp2f((xt - m) * kLog2e) / d - 1.0f) * inv_n * sc;
  const int64_t tv = (lead + t) / EPV;  // the target's row vector and element in it
  const int te = (int)((lead + t) % EPV);
  with_form(f, [&](auto form) {
    constexpr bool SC = decltype(form)::value;
    for (int64_t lo = 0; lo < nv; lo += kStreamWindow) {
      const Chunk<D> c(row, p.V, lo, kStreamWindow);
      for (int v0 = tid; v0 < c.nvec; v0 += U * T) {
        u32x4 a[U];
#pragma unroll
        for (int q = 0; q < U; ++q) a[q] = buf_load<kPolicyNT>(c.rsrc, (uint32_t)(v0 + q * T) * 16u);
#pragma unroll
        for (int q = 0; q < U; ++q) {
          const int v = v0 + q * T;
          if (v >= c.nvec) break;
          OutVec<D> o;
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float g = exp_of<SC>(elem<D>(a[q], e), f);
            o.v[e] = neg ? -g : g;
          }
          if (lo + v == tv) {
#pragma unroll
            for (int e = 0; e < EPV; ++e)
              if (e == te) o.v[e] = gt;
          }
          store_vec<D>(c, v, o.bits());
        }
      }
    }
  });
  if (tid == 0) p.row_loss[r] = (m - xt) + logf(d);
}

// ============================================================================ element_mul
// The backward's scaling of a stored gradient by the upstream gradient, in place:
// x[i, 0:V) *= scale[i * sstride] (Liger-Kernel cross_entropy.py page, element_mul and
// LigerCrossEntropyFunction.backward). A row whose scale is exactly 1 is neither read nor
// written, which is what the page's skip of a unit upstream gradient amounts to, decided
// here on the device with no host synchronisation. Workgroup b handles chunk b % chunks of
// row b / chunks; 16-byte vectors, head / tail elements of unaligned rows element-wise.
template <int D, int LP>
__global__ __launch_bounds__(kMulThreads) void element_mul_kernel(ElementMulParams p) {
  const int64_t total = p.M * p.chunks;
  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    const int64_t r = b / p.chunks;
    const float sc = p.scale[r * p.sstride];
    if (sc == 1.0f) continue;
    const Chunk<D> c(p.x + r * p.ld_bytes, p.V, (b - r * p.chunks) * p.chunk_vecs, p.chunk_vecs);
    u32x4 v[kMulVpt];
    issue_loads<D, kMulThreads, kMulVpt, LP>(v, c);
#pragma unroll
    for (int k = 0; k < kMulVpt; ++k) store_slot<D, kMulThreads>(c, k, mul_slot<D>(v[k], sc));
    store_partials<D, kMulThreads>(c, c, [sc](float x) { return x * sc; });
  }
}

// ============================================================================ lookup tables
#define XR_CASE_XENT(D, T, V)                                                                  \
  if (s.threads == T && s.vpt == V)                                                              \
    return lp ? reinterpret_cast<const void*>(&xent_rows_kernel<D, T, V, kPolicyNT>)             \
              : reinterpret_cast<const void*>(&xent_rows_kernel<D, T, V, kPolicyDefault>);
const void* xent_rows_kernel_ptr(int dtype, Shape s, bool lp) {
  if (dtype == kF32) { XR_SHAPES_FWD(XR_CASE_XENT, kF32) }
  if (dtype == kBF16) { XR_SHAPES_FWD(XR_CASE_XENT, kBF16) }
  return nullptr;
}
const void* xent_stream_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&xent_stream_kernel<kF32>)
                       : reinterpret_cast<const void*>(&xent_stream_kernel<kBF16>);
}
const void* xent_scan_kernel_ptr() { return reinterpret_cast<const void*>(&xent_scan_kernel); }
const void* xent_mean_kernel_ptr() { return reinterpret_cast<const void*>(&xent_mean_kernel); }
const void* element_mul_kernel_ptr(int dtype, bool nt) {
  if (dtype == kF32)
    return nt ? reinterpret_cast<const void*>(&element_mul_kernel<kF32, kPolicyNT>)
              : reinterpret_cast<const void*>(&element_mul_kernel<kF32, kPolicyDefault>);
  return nt ? reinterpret_cast<const void*>(&element_mul_kernel<kBF16, kPolicyNT>)
            : reinterpret_cast<const void*>(&element_mul_kernel<kBF16, kPolicyDefault>);
}

}  // namespace xr
