// xr_softmax.hip -- softmax forward and backward kernels for gfx950 (the row-kernel design
// is described at the top of xr_xent.hip), and the negative log-softmax forward with a
// gathered loss (page "python sum function examples", Triton kernel _forward): the same
// row pass, writing -log p = m + log d - x instead of p, and loss[i] = the written element
// at idx[i].
#include "xr_rows.h"

namespace xr {

// In order of capacity (threads x vectors); of two shapes of equal capacity the one with
// fewer threads comes first, so the default pick of a whole row is the narrower workgroup.
const Shape kFwdShapes[kNumFwdShapes] = {{64, 4},   {64, 8},   {64, 16},  {128, 8},
                                         {128, 16}, {256, 8},  {256, 16}, {512, 8},
                                         {512, 16}, {1024, 16}};
const Shape kBwdShapes[kNumBwdShapes] = {{64, 4},  {64, 8},   {128, 8},
                                         {256, 8}, {512, 8}, {1024, 8}};

// -log p = nll_of<SCALED>(x, f) for every element of one slot, in the element type.
template <int D, bool SCALED>
__device__ __forceinline__ u32x4 nll_slot(u32x4 v, const ExpForm& f) {
  pin(v);  // fp32 too: the subtraction is cheap enough that, unpinned, the compiler computes
           // every slot's result at once and spills
  OutVec<D> o;
#pragma unroll
  for (int e = 0; e < Elt<D>::kPerVec; ++e) o.v[e] = nll_of<SCALED>(elem<D>(v, e), f);
  return o.bits();
}

// Wave priority while a row-resident softmax wave issues its row's loads (s_setprio; 0 is
// the default), when the plan asks for it (p.load_prio): the wave's requests then go out
// ahead of the arithmetic of the waves that already hold their rows. The plans ask for it
// only when the whole grid is resident at once (measured on 4096 x 4096 bf16: backward
// 19.0 -> 16.9 us, forward 12.0 -> 11.7 us; levels 1 to 3 alike); with more workgroups than
// the GPU holds, waves starting their rows at a raised priority hold back the output passes
// whose end frees the next workgroups' slots (2-7 % slower on four such shapes). Not used
// where chunks of a row exchange statistics (the cross-entropy, the split rows): slower.
constexpr int kLoadIssuePriority = 3;

// ============================================================================ softmax forward
// NLL = false: y = softmax(x). NLL = true: y = -log softmax(x) and loss[r] = y[r, idx[r]] as
// stored (NaN when idx[r] lies outside the row).
template <int D, int THREADS, int VPT, int LP, bool NLL>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void softmax_fwd_kernel(SoftmaxFwdParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int NW = THREADS / kWave;
  __shared__ float2 red[2][NW];
  int buf = 0;
  const int64_t G = gridDim.x;
  const int64_t cv = p.N + Elt<D>::kPerVec;  // more vectors than any row has: whole rows
  clear_status(p.flags);

  u32x4 v[VPT];
  int64_t r = blockIdx.x;
  if (p.load_prio) __builtin_amdgcn_s_setprio(kLoadIssuePriority);
  if (r < p.M) issue_loads<D, THREADS, VPT, LP>(v, Chunk<D>(p.x + r * p.ldx_bytes, p.N, 0, cv));
  __builtin_amdgcn_s_setprio(0);
  while (r < p.M) {
    const int64_t rn = r + G;
    const Chunk<D> cx(p.x + r * p.ldx_bytes, p.N, 0, cv);
    const Chunk<D> cy(p.y + r * p.ldy_bytes, p.N, 0, cv);  // same lead as cx (host-checked)
    // NLL: the gathered element, read by the thread holding its vector before any store of
    // this row (y may be exactly x).
    int64_t vi = -1;
    bool owner = false;
    float xi = 0.f;
    if (NLL) {
      const int64_t ix = p.idx[r];
      if (ix >= 0 && ix < p.N) vi = cx.lead + ix;
      owner = vi >= 0 && (int)threadIdx.x == (int)((vi / EPV) % THREADS);
      if (owner) xi = buf_load_elem<D>(cx.rsrc, (uint32_t)(vi * Elt<D>::kBytes));
    }
    const Stats st = block_reduce_stats<THREADS>(thread_stats<D, THREADS, VPT>(v, cx), red[buf]);
    buf ^= 1;
    // softmax: exp2((x - m) log2e - log2 d).  NLL: m + log d - x.
    const ExpForm f = NLL ? nll_form(st.m, logf(st.d)) : exp_form(st.m, log2f(st.d));
    with_form(f, [&](auto form) {
      constexpr bool SC = decltype(form)::value;
#pragma unroll
      for (int k = 0; k < VPT; ++k)
        store_slot<D, THREADS>(cy, k, NLL ? nll_slot<D, SC>(v[k], f) : exp_slot<D, SC>(v[k], f));
      store_partials<D, THREADS>(cy, cx, [&f](float x) {
        return NLL ? nll_of<SC>(x, f) : exp_of<SC>(x, f);
      });
      if (NLL && owner) p.loss[r] = round_elem<D>(nll_of<SC>(xi, f));
    });
    if (NLL && vi < 0 && threadIdx.x == 0) p.loss[r] = __builtin_nanf("");
    if (rn < p.M) {  // the next row's loads, once this row is written out
      const Chunk<D> cn(p.x + rn * p.ldx_bytes, p.N, 0, cv);
      const uint32_t off = threadIdx.x * 16u;
#pragma unroll
      for (int k = 0; k < VPT; ++k) v[k] = buf_load<LP>(cn.slot(k * THREADS), off);
    }
    r = rn;
  }
}

// Softmax (NLL = false) or negative log-softmax (NLL = true) over split rows: workgroup b
// handles chunk b % S of row b / S (long rows, or too few rows to fill the GPU). The chunks
// exchange their (m, d) pairs as the cross-entropy's split rows do; for NLL the chunk
// holding idx writes the loss.
template <int D, int THREADS, int VPT, int LP, bool NLL>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void softmax_split_kernel(SoftmaxFwdParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int NW = THREADS / kWave;
  __shared__ float2 red[NW];
  __shared__ float bcast[2];
  const int tid = threadIdx.x;
  const int S = p.S;
  const int64_t r = blockIdx.x / S;
  const int chunk = (int)(blockIdx.x - r * S);
  if (r >= p.M) return;
  const int64_t lo = (int64_t)chunk * p.chunk_vecs;
  const Chunk<D> cx(p.x + r * p.ldx_bytes, p.N, lo, p.chunk_vecs);
  const Chunk<D> cy(p.y + r * p.ldy_bytes, p.N, lo, p.chunk_vecs);  // same lead (host-checked)
  u32x4 v[VPT];
  issue_loads<D, THREADS, VPT, LP>(v, cx);
  // NLL: the gathered element, read by the thread holding its vector before any store of
  // this chunk (y may be exactly x; other chunks write only their own elements)
  const int64_t ix = NLL ? p.idx[r] : -1;
  const bool in_row = ix >= 0 && ix < p.N;
  const int64_t vt = cx.lead + ix - cx.lo * EPV;  // chunk-local element index
  const bool owner = in_row && vt >= 0 && vt < (int64_t)cx.nvec * EPV &&
                     tid == (int)((vt / EPV) % THREADS);
  float xi = 0.f;
  if (owner) xi = buf_load_elem<D>(cx.rsrc, (uint32_t)(vt * Elt<D>::kBytes));
  Stats st = block_reduce_stats<THREADS>(thread_stats<D, THREADS, VPT>(v, cx), red);
  st = exchange_row_stats<THREADS>(st, p.partials + r * S, S, chunk, p.flags, bcast);
  if (p.group_rows > 1)
    wait_row_group<kWriteGroupRows>(p.partials, nullptr, 0, 0, r, p.M, S, p.flags);
  // softmax: exp2((x - m) log2e - log2 d).  NLL: m + log d - x.
  const ExpForm f = NLL ? nll_form(st.m, logf(st.d)) : exp_form(st.m, log2f(st.d));
  with_form(f, [&](auto form) {
    constexpr bool SC = decltype(form)::value;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      store_slot<D, THREADS>(cy, k, NLL ? nll_slot<D, SC>(v[k], f) : exp_slot<D, SC>(v[k], f));
    store_partials<D, THREADS>(cy, cx, [&f](float x) {
      return NLL ? nll_of<SC>(x, f) : exp_of<SC>(x, f);
    });
    if (NLL && owner) p.loss[r] = round_elem<D>(nll_of<SC>(xi, f));
  });
  if (NLL && !in_row && chunk == 0 && tid == 0) p.loss[r] = __builtin_nanf("");
}

// Two-pass stream form (rows too long for the row-resident shapes, rows split over no
// workspace, or operands at different addresses modulo 16): one workgroup per row, a first
// pass folding every vector into per-thread online (m, d) pairs, the workgroup combine, then
// a second pass that re-reads the row and writes it. 16-byte vector loads in the input's own
// alignment; vector stores when the output shares it, element stores otherwise.
template <int D, bool NLL>
__global__ __launch_bounds__(kStreamThreads) void softmax_fwd_stream_kernel(SoftmaxFwdParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int T = kStreamThreads;
  constexpr int U = kStreamUnroll;
  __shared__ float2 red[T / kWave];
  clear_status(p.flags);
  const int64_t r = blockIdx.x;
  if (r >= p.M) return;
  const char* row = p.x + r * p.ldx_bytes;
  char* out = p.y + r * p.ldy_bytes;
  const int tid = threadIdx.x;
  const int lead = (int)(((uintptr_t)row & 15u) / Elt<D>::kBytes);
  const bool same = (((uintptr_t)row ^ (uintptr_t)out) & 15u) == 0;
  const int64_t nv = (lead + p.N + EPV - 1) / EPV;
  // NLL: the gathered element, read before the barrier below (y may be exactly x).
  const int64_t ix = NLL ? p.idx[r] : -1;
  const bool in_row = ix >= 0 && ix < p.N;
  float xi = 0.f;
  if (NLL && tid == 0 && in_row)
    xi = D == kF32 ? reinterpret_cast<const float*>(row)[ix]
                   : as_f32((uint32_t)reinterpret_cast<const uint16_t*>(row)[ix] << 16);
  Stats st{kNegInf, 0.f};
  for (int64_t lo = 0; lo < nv; lo += kStreamWindow) {
    const Chunk<D> cx(row, p.N, lo, kStreamWindow);
    for (int v0 = tid; v0 < cx.nvec; v0 += U * T) {
      u32x4 a[U];
#pragma unroll
      for (int q = 0; q < U; ++q) a[q] = buf_load<kPolicyDefault>(cx.rsrc, (uint32_t)(v0 + q * T) * 16u);
#pragma unroll
      for (int q = 0; q < U; ++q)
        online_add_vec<D>(st, vec_masked<D>(a[q], v0 + q * T, cx, Elt<D>::kNegInfWord));
    }
  }
  st = block_reduce_stats<T>(st, red);
  // In place (y == x) is safe: each vector is re-read and written by the same thread, and
  // all reads of the statistics pass finished before the barrier above.
  const ExpForm f = NLL ? nll_form(st.m, logf(st.d)) : exp_form(st.m, log2f(st.d));
  with_form(f, [&](auto form) {
    constexpr bool SC = decltype(form)::value;
    for (int64_t lo = 0; lo < nv; lo += kStreamWindow) {
      const Chunk<D> cx(row, p.N, lo, kStreamWindow);
      const Chunk<D> cy(out, p.N, lo, kStreamWindow);  // the output's geometry when `same`
      for (int v0 = tid; v0 < cx.nvec; v0 += U * T) {
        u32x4 a[U];
#pragma unroll
        for (int q = 0; q < U; ++q) a[q] = buf_load<kPolicyNT>(cx.rsrc, (uint32_t)(v0 + q * T) * 16u);
#pragma unroll
        for (int q = 0; q < U; ++q) {
          const int v = v0 + q * T;
          if (v >= cx.nvec) break;
          const u32x4 o = NLL ? nll_slot<D, SC>(a[q], f) : exp_slot<D, SC>(a[q], f);
          if (same) {
            store_vec<D>(cy, v, o);
          } else {
            // element stores at the output's own addresses
            const int e0 = v == cx.head ? cx.h0 : 0;
            const int e1 = v == cx.head ? cx.h1 : (v == cx.tail ? cx.t1 : EPV);
            const int64_t j0 = (lo + v) * EPV - lead;  // row index of the vector's element 0
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
              if (e < e0 || e >= e1) continue;
              if (D == kF32) reinterpret_cast<uint32_t*>(out)[j0 + e] = o[e];
              else reinterpret_cast<uint16_t*>(out)[j0 + e] = (uint16_t)(o[e >> 1] >> (16 * (e & 1)));
            }
          }
        }
      }
    }
    if (NLL && tid == 0 && in_row) p.loss[r] = round_elem<D>(nll_of<SC>(xi, f));
  });
  if (NLL && tid == 0 && !in_row) p.loss[r] = __builtin_nanf("");
}

// ============================================================================ softmax backward
// One row of the backward: vy / vd hold row r's y and dy (their loads issued in pairs);
// dx = y (dy - s), s = sum(y dy), formed as fma(-y, s, y dy) with the product y dy rounded
// once. Without PREFETCH (one row per workgroup) the products are kept in registers from the
// pass that sums them, so the pass that writes dx, which must wait for the last pair and
// the reduction, has one widening and one fma per element; with PREFETCH (the persistent
// loop, whose registers also carry the next row) they are formed again there, to the same
// bits. With PREFETCH, the loads of row rn (if rn < M) are issued as the slots of row r are
// stored.
template <int D, int THREADS, int VPT, int LP, bool PREFETCH>
__device__ __forceinline__ void softmax_bwd_row(const SoftmaxBwdParams& p, int64_t r, int64_t rn,
                                                u32x4 (&vy)[VPT], u32x4 (&vd)[VPT], float* red) {
  constexpr int EPV = Elt<D>::kPerVec;
  const int64_t cv = p.N + EPV;
  // y, dy and dx rows share their alignment (host-checked), hence their vector layout.
  const Chunk<D> cy(p.y + r * p.ldy_bytes, p.N, 0, cv);
  const Chunk<D> cx(p.dx + r * p.lddx_bytes, p.N, 0, cv);
  // Out-of-row elements of both operands count as 0: they add nothing to the dot product.
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  float prod[PREFETCH ? 1 : VPT][EPV];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (slot_kind<THREADS>(k, cy.nvec) == kSlotNone) {
      if constexpr (!PREFETCH) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) prod[k][e] = 0.f;
      }
      continue;
    }
    const u32x4 a = masked_slot<D, THREADS>(vy[k], k, cy, 0u);
    const u32x4 b = masked_slot<D, THREADS>(vd[k], k, cy, 0u);
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      s[e & 3] = __builtin_fmaf(elem<D>(a, e), elem<D>(b, e), s[e & 3]);
      if constexpr (!PREFETCH) prod[k][e] = elem<D>(a, e) * elem<D>(b, e);
    }
  }
  const float dot = block_reduce<THREADS>((s[0] + s[1]) + (s[2] + s[3]), OpAdd(), red);
  reg_barrier(vy);
  if constexpr (PREFETCH) reg_barrier(vd);  // (without it dy is dead once its products are formed)
  const bool pf = PREFETCH && rn < p.M;
  const Chunk<D> cyn(p.y + (pf ? rn : r) * p.ldy_bytes, p.N, 0, cv);
  const Chunk<D> cdn(p.dy + (pf ? rn : r) * p.lddy_bytes, p.N, 0, cv);
  const uint32_t off = threadIdx.x * 16u;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    OutVec<D> o;
    u32x4 a = vy[k];
    pin(a);  // fp32 too: unpinned, the fp32 shapes with 8 vectors per thread spill
    if constexpr (PREFETCH) {
      u32x4 b = vd[k];
      pin(b);
#pragma unroll
      for (int e = 0; e < EPV; ++e)
        o.v[e] = __builtin_fmaf(-elem<D>(a, e), dot, elem<D>(a, e) * elem<D>(b, e));
    } else {
      // lanes past the row hold masked products: their stores are dropped, and the
      // partial first / last vectors are written below
#pragma unroll
      for (int e = 0; e < EPV; ++e) o.v[e] = __builtin_fmaf(-elem<D>(a, e), dot, prod[k][e]);
    }
    store_slot<D, THREADS>(cx, k, o.bits());
    if (pf) {
      vy[k] = buf_load<LP>(cyn.slot(k * THREADS), off);
      vd[k] = buf_load<LP>(cdn.slot(k * THREADS), off);
    }
  }
  // Partial first / last vectors: re-read y and dy (this workgroup has not written them;
  // dx may be exactly y or dy) and store only the in-row elements.
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
    for (int e = 0; e < EPV; ++e)
      o.v[e] = __builtin_fmaf(-elem<D>(a, e), dot, elem<D>(a, e) * elem<D>(b, e));
    store_partial<D>(cx.rsrc, po, o.bits(), q == 0 ? cx.h0 : cx.t0, q == 0 ? cx.h1 : cx.t1);
  }
}

// Workgroup b handles rows b, b + G, ... (G = the grid). ONE_ROW: the grid covers the rows
// (G >= M, the plans' default; the host checks it), and the row is handled without the
// loop: the compiler's waits for the loads then follow the pairs as they arrive, where the
// loop's prefetch of the next row would merge them with that row's loads (and the two forms
// in one kernel would raise its register count until it spilled).
template <int D, int THREADS, int VPT, int LP, bool ONE_ROW>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void softmax_bwd_kernel(SoftmaxBwdParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int NW = THREADS / kWave;
  __shared__ float red[2][NW];
  const int64_t G = gridDim.x;
  const int64_t cv = p.N + EPV;
  clear_status(p.flags);

  u32x4 vy[VPT], vd[VPT];
  int64_t r = blockIdx.x;
  if (r >= p.M) return;
  if (p.load_prio) __builtin_amdgcn_s_setprio(kLoadIssuePriority);
  issue_loads2<D, THREADS, VPT, LP>(vy, Chunk<D>(p.y + r * p.ldy_bytes, p.N, 0, cv), vd,
                                    Chunk<D>(p.dy + r * p.lddy_bytes, p.N, 0, cv));
  __builtin_amdgcn_s_setprio(0);
  if constexpr (ONE_ROW) {
    softmax_bwd_row<D, THREADS, VPT, LP, false>(p, r, p.M, vy, vd, red[0]);
  } else {
    int buf = 0;
    while (r < p.M) {
      const int64_t rn = r + G;
      softmax_bwd_row<D, THREADS, VPT, LP, true>(p, r, rn, vy, vd, red[buf]);
      buf ^= 1;
      r = rn;
    }
  }
}

// Softmax backward over split rows: workgroup b handles chunk b % S of row b / S; the
// chunks exchange their partial dot products (summed in chunk order), then each writes its
// part of dx = y (dy - s). y, dy and dx rows share their alignment (host-checked).
template <int D, int THREADS, int VPT, int LP>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void softmax_bwd_split_kernel(SoftmaxBwdParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int NW = THREADS / kWave;
  __shared__ float red[NW];
  __shared__ float bcast[1];
  const int tid = threadIdx.x;
  const int S = p.S;
  const int64_t r = blockIdx.x / S;
  const int chunk = (int)(blockIdx.x - r * S);
  if (r >= p.M) return;
  const int64_t lo = (int64_t)chunk * p.chunk_vecs;
  const Chunk<D> cy(p.y + r * p.ldy_bytes, p.N, lo, p.chunk_vecs);
  const Chunk<D> cd(p.dy + r * p.lddy_bytes, p.N, lo, p.chunk_vecs);
  const Chunk<D> cx(p.dx + r * p.lddx_bytes, p.N, lo, p.chunk_vecs);
  u32x4 vy[VPT], vd[VPT];
  issue_loads<D, THREADS, VPT, LP>(vy, cy);
  issue_loads<D, THREADS, VPT, LP>(vd, cd);
  // out-of-row elements of both operands count as 0: they add nothing to the dot product
  float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (slot_kind<THREADS>(k, cy.nvec) == kSlotNone) continue;
    const u32x4 a = masked_slot<D, THREADS>(vy[k], k, cy, 0u);
    const u32x4 b = masked_slot<D, THREADS>(vd[k], k, cy, 0u);
#pragma unroll
    for (int e = 0; e < EPV; ++e) s4[e & 3] = __builtin_fmaf(elem<D>(a, e), elem<D>(b, e), s4[e & 3]);
  }
  const float part = block_reduce<THREADS>((s4[0] + s4[1]) + (s4[2] + s4[3]), OpAdd(), red);
  const float dot = exchange_row_sum<THREADS>(part, p.partials + r * S, S, chunk, p.flags, bcast);
  if (p.group_rows > 1)
    wait_row_group<kWriteGroupRows>(p.partials, nullptr, 0, 0, r, p.M, S, p.flags);
  reg_barrier(vy);
  reg_barrier(vd);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    OutVec<D> o;
    u32x4 a = vy[k], b = vd[k];
    pin(a);
    pin(b);
#pragma unroll
    for (int e = 0; e < EPV; ++e) o.v[e] = elem<D>(a, e) * (elem<D>(b, e) - dot);
    store_slot<D, THREADS>(cx, k, o.bits());
  }
  // partial first / last vectors: re-read y and dy (dx may be exactly y or dy; this chunk
  // has not written them) and store only the in-row elements
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int vi = q == 0 ? cx.head : cx.tail;
    if (vi < 0 || tid != vi % THREADS) continue;
    const uint32_t po = q == 0 ? cx.hoff : cx.toff;
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(cy.rsrc, (int)po, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(cd.rsrc, (int)po, 0, 0);
    OutVec<D> o;
#pragma unroll
    for (int e = 0; e < EPV; ++e) o.v[e] = elem<D>(a, e) * (elem<D>(b, e) - dot);
    store_partial<D>(cx.rsrc, po, o.bits(), q == 0 ? cx.h0 : cx.t0, q == 0 ? cx.h1 : cx.t1);
  }
}

// Two-pass stream form of the backward: the dot product, the workgroup sum, then a second
// pass that re-reads y and dy and writes dx. 16-byte vectors when y, dy and dx share their
// address modulo 16; element accesses otherwise.
template <int D>
__global__ __launch_bounds__(kStreamThreads) void softmax_bwd_stream_kernel(SoftmaxBwdParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int T = kStreamThreads;
  constexpr int U = kStreamUnroll;
  __shared__ float red[T / kWave];
  clear_status(p.flags);
  const int64_t r = blockIdx.x;
  if (r >= p.M) return;
  const char* yr = p.y + r * p.ldy_bytes;
  const char* dr = p.dy + r * p.lddy_bytes;
  char* out = p.dx + r * p.lddx_bytes;
  const int tid = threadIdx.x;
  const bool same = ((((uintptr_t)yr ^ (uintptr_t)dr) | ((uintptr_t)yr ^ (uintptr_t)out)) & 15u) == 0;
  if (!same) {
    auto ld = [&](const char* row, int64_t j) -> float {
      if (D == kF32) return reinterpret_cast<const float*>(row)[j];
      return as_f32((uint32_t)reinterpret_cast<const uint16_t*>(row)[j] << 16);
    };
    float s = 0.f;
    for (int64_t j = tid; j < p.N; j += T) s += ld(yr, j) * ld(dr, j);
    s = block_reduce<T>(s, OpAdd(), red);
    for (int64_t j = tid; j < p.N; j += T) {
      const float val = ld(yr, j) * (ld(dr, j) - s);
      if (D == kF32) reinterpret_cast<float*>(out)[j] = val;
      else reinterpret_cast<uint16_t*>(out)[j] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
    }
    return;
  }
  const int lead = (int)(((uintptr_t)yr & 15u) / Elt<D>::kBytes);
  const int64_t nv = (lead + p.N + EPV - 1) / EPV;
  float s4[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t lo = 0; lo < nv; lo += kStreamWindow) {
    const Chunk<D> cy(yr, p.N, lo, kStreamWindow);
    const Chunk<D> cd(dr, p.N, lo, kStreamWindow);
    for (int v0 = tid; v0 < cy.nvec; v0 += U * T) {
      u32x4 a[U], b[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        a[q] = buf_load<kPolicyDefault>(cy.rsrc, (uint32_t)(v0 + q * T) * 16u);
        b[q] = buf_load<kPolicyDefault>(cd.rsrc, (uint32_t)(v0 + q * T) * 16u);
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        // out-of-row elements count as 0 in both operands
        const u32x4 ya = vec_masked<D>(a[q], v0 + q * T, cy, 0u);
        const u32x4 da = vec_masked<D>(b[q], v0 + q * T, cy, 0u);
#pragma unroll
        for (int e = 0; e < EPV; ++e) s4[e & 3] = __builtin_fmaf(elem<D>(ya, e), elem<D>(da, e), s4[e & 3]);
      }
    }
  }
  const float s = block_reduce<T>((s4[0] + s4[1]) + (s4[2] + s4[3]), OpAdd(), red);
  // dx may be exactly y or dy: each vector is re-read and written by the same thread.
  for (int64_t lo = 0; lo < nv; lo += kStreamWindow) {
    const Chunk<D> cy(yr, p.N, lo, kStreamWindow);
    const Chunk<D> cd(dr, p.N, lo, kStreamWindow);
    const Chunk<D> cx(out, p.N, lo, kStreamWindow);
    for (int v0 = tid; v0 < cy.nvec; v0 += U * T) {
      u32x4 a[U], b[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        a[q] = buf_load<kPolicyNT>(cy.rsrc, (uint32_t)(v0 + q * T) * 16u);
        b[q] = buf_load<kPolicyNT>(cd.rsrc, (uint32_t)(v0 + q * T) * 16u);
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int v = v0 + q * T;
        if (v >= cy.nvec) break;
        OutVec<D> o;
#pragma unroll
        for (int e = 0; e < EPV; ++e) o.v[e] = elem<D>(a[q], e) * (elem<D>(b[q], e) - s);
        store_vec<D>(cx, v, o.bits());
      }
    }
  }
}

// ============================================================================ lookup tables
#define XR_CASE_SFWD(D, T, V)                                                                  \
  if (s.threads == T && s.vpt == V)                                                              \
    return lp ? reinterpret_cast<const void*>(&softmax_fwd_kernel<D, T, V, kPolicyNT, false>)    \
              : reinterpret_cast<const void*>(&softmax_fwd_kernel<D, T, V, kPolicyDefault, false>);
#define XR_CASE_NLL(D, T, V)                                                                   \
  if (s.threads == T && s.vpt == V)                                                              \
    return lp ? reinterpret_cast<const void*>(&softmax_fwd_kernel<D, T, V, kPolicyNT, true>)     \
              : reinterpret_cast<const void*>(&softmax_fwd_kernel<D, T, V, kPolicyDefault, true>);
#define XR_CASE_SBWD(D, T, V)                                                                  \
  if (s.threads == T && s.vpt == V) {                                                            \
    if (one_row)                                                                                 \
      return lp ? reinterpret_cast<const void*>(&softmax_bwd_kernel<D, T, V, kPolicyNT, true>)   \
                : reinterpret_cast<const void*>(&softmax_bwd_kernel<D, T, V, kPolicyDefault, true>); \
    return lp ? reinterpret_cast<const void*>(&softmax_bwd_kernel<D, T, V, kPolicyNT, false>)    \
              : reinterpret_cast<const void*>(&softmax_bwd_kernel<D, T, V, kPolicyDefault, false>); \
  }

const void* softmax_fwd_kernel_ptr(int dtype, Shape s, bool lp) {
  if (dtype == kF32) { XR_SHAPES_FWD(XR_CASE_SFWD, kF32) }
  if (dtype == kBF16) { XR_SHAPES_FWD(XR_CASE_SFWD, kBF16) }
  return nullptr;
}
const void* nll_fwd_kernel_ptr(int dtype, Shape s, bool lp) {
  if (dtype == kF32) { XR_SHAPES_FWD(XR_CASE_NLL, kF32) }
  if (dtype == kBF16) { XR_SHAPES_FWD(XR_CASE_NLL, kBF16) }
  return nullptr;
}
#define XR_CASE_NLLS(D, T, V)                                                                  \
  if (s.threads == T && s.vpt == V)                                                              \
    return lp ? reinterpret_cast<const void*>(&softmax_split_kernel<D, T, V, kPolicyNT, true>)   \
              : reinterpret_cast<const void*>(&softmax_split_kernel<D, T, V, kPolicyDefault, true>);
#define XR_CASE_SFWDS(D, T, V)                                                                 \
  if (s.threads == T && s.vpt == V)                                                              \
    return lp ? reinterpret_cast<const void*>(&softmax_split_kernel<D, T, V, kPolicyNT, false>)  \
              : reinterpret_cast<const void*>(&softmax_split_kernel<D, T, V, kPolicyDefault, false>);
#define XR_CASE_SBWDS(D, T, V)                                                                 \
  if (s.threads == T && s.vpt == V)                                                              \
    return lp ? reinterpret_cast<const void*>(&softmax_bwd_split_kernel<D, T, V, kPolicyNT>)     \
              : reinterpret_cast<const void*>(&softmax_bwd_split_kernel<D, T, V, kPolicyDefault>);
const void* nll_split_kernel_ptr(int dtype, Shape s, bool lp) {
  if (dtype == kF32) { XR_SHAPES_FWD(XR_CASE_NLLS, kF32) }
  if (dtype == kBF16) { XR_SHAPES_FWD(XR_CASE_NLLS, kBF16) }
  return nullptr;
}
const void* softmax_fwd_split_kernel_ptr(int dtype, Shape s, bool lp) {
  if (dtype == kF32) { XR_SHAPES_FWD(XR_CASE_SFWDS, kF32) }
  if (dtype == kBF16) { XR_SHAPES_FWD(XR_CASE_SFWDS, kBF16) }
  return nullptr;
}
const void* softmax_bwd_split_kernel_ptr(int dtype, Shape s, bool lp) {
  if (dtype == kF32) { XR_SHAPES_BWD(XR_CASE_SBWDS, kF32) }
  if (dtype == kBF16) { XR_SHAPES_BWD(XR_CASE_SBWDS, kBF16) }
  return nullptr;
}
const void* softmax_bwd_kernel_ptr(int dtype, Shape s, bool lp, bool one_row) {
  if (dtype == kF32) { XR_SHAPES_BWD(XR_CASE_SBWD, kF32) }
  if (dtype == kBF16) { XR_SHAPES_BWD(XR_CASE_SBWD, kBF16) }
  return nullptr;
}
const void* softmax_fwd_stream_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&softmax_fwd_stream_kernel<kF32, false>)
                       : reinterpret_cast<const void*>(&softmax_fwd_stream_kernel<kBF16, false>);
}
const void* nll_fwd_stream_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&softmax_fwd_stream_kernel<kF32, true>)
                       : reinterpret_cast<const void*>(&softmax_fwd_stream_kernel<kBF16, true>);
}
const void* softmax_bwd_stream_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&softmax_bwd_stream_kernel<kF32>)
                       : reinterpret_cast<const void*>(&softmax_bwd_stream_kernel<kBF16>);
}

}  // namespace xr
