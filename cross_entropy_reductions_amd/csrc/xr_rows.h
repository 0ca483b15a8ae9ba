// xr_rows.h -- building blocks of the row kernels (included by the kernel sources only).
#pragma once

#include "xr_device.h"
#include "xr_internal.h"

namespace xr {


inline constexpr float kNegInf = -__builtin_inff();
constexpr int kSpinLimit = 1 << 20;

// m log2e rounded once to fp32. The sum pass subtracts this value from every x log2e, and
// the output pass builds its exponent constant on the same value, so the rounding cancels
// between the two passes instead of entering every output (hence no contraction of the
// product into a neighbouring add).
__device__ __forceinline__ float scaled_max(float m) {
#pragma clang fp contract(off)
  return m * kLog2e;
}
// The output pass's exponent constant mL + small, where small (log2 d, plus log2 n and
// -log2|s| for the cross-entropy) is summed first: one rounding at the constant's magnitude.
// Measured by emulating the kernels' fp32 arithmetic over the 2048 x 256000 fp32 rows: the
// worst relative error of an output is 7.1e-6 this way, against 8.6e-6 with m log2e fused
// into the first add.
__device__ __forceinline__ float exp_offset(float mL, float small) {
#pragma clang fp contract(off)
  return mL + small;
}

__device__ __forceinline__ u32x4 splat(uint32_t w) { return (u32x4){w, w, w, w}; }

// A call given a workspace leaves the workspace's status word defined: rows that are not
// split exchange nothing and cannot time out, so the grid's first thread writes 0 (split
// rows have theirs written by the kernel that prepares the exchange).
__device__ __forceinline__ void clear_status(int32_t* flags) {
  if (flags != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *flags = 0;
}

__device__ __forceinline__ uint64_t pack_pair(float m, float d) {
  return (uint64_t)as_u32(m) | ((uint64_t)as_u32(d) << 32);
}
__device__ __forceinline__ float pair_m(uint64_t w) { return as_f32((uint32_t)w); }
__device__ __forceinline__ float pair_d(uint64_t w) { return as_f32((uint32_t)(w >> 32)); }

// Issue the loads of a chunk: slot k of thread tid holds chunk vector k*THREADS + tid.
// Every slot is loaded, in slot order and without branches (so the compiler can wait for
// each slot's data separately); lanes past the chunk's end read zeros without a memory
// access, and the consumers below never look at them.
template <int D, int THREADS, int VPT, int LP>
__device__ __forceinline__ void issue_loads(u32x4 (&v)[VPT], const Chunk<D>& c) {
  const uint32_t off = threadIdx.x * 16u;
#pragma unroll
  for (int k = 0; k < VPT; ++k) v[k] = buf_load<LP>(c.slot(k * THREADS), off);
}

// The loads of two chunks of the same layout, issued in pairs (a[0], b[0], a[1], b[1], ...):
// loads complete in issue order, so work on slot k can start once slot k of both has arrived
// (the scheduler would otherwise regroup them by resource).
template <int D, int THREADS, int VPT, int LP>
__device__ __forceinline__ void issue_loads2(u32x4 (&a)[VPT], const Chunk<D>& ca, u32x4 (&b)[VPT],
                                             const Chunk<D>& cb) {
  const uint32_t off = threadIdx.x * 16u;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    a[k] = buf_load<LP>(ca.slot(k * THREADS), off);
    b[k] = buf_load<LP>(cb.slot(k * THREADS), off);
    __builtin_amdgcn_sched_barrier(0);  // keep the pairs in this order
  }
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

// This thread's (m, d) over its chunk elements: its own maximum, then the sum of
// exp(x - m) with that maximum. No workgroup barrier sits between the two passes, so each
// wave streams through its slots as their loads land; the workgroup combines the pairs once.
template <int D, int THREADS, int VPT>
__device__ __forceinline__ Stats thread_stats(u32x4 (&v)[VPT], const Chunk<D>& c) {
  const float m = thread_max<D, THREADS, VPT>(v, c);
  reg_barrier(v);
  const float d = (m == kNegInf) ? 0.f : thread_sum_exp<D, THREADS, VPT>(v, c, scaled_max(m));
  reg_barrier(v);
  return {m, d};
}

// Wait for slot q of a split row's exchange (lane-private bounded poll): the published word,
// or kPartialEmpty with ok cleared once the budget runs out.
__device__ __forceinline__ uint64_t poll_slot(const uint64_t* slot, int& budget, bool& ok) {
  uint64_t w;
  while ((w = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) ==
         kPartialEmpty) {
    if (--budget < 0) {
      ok = false;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return w;
}

// Split rows: publish this chunk's (m, d) in its slot of the row's S slots (one 64-bit
// relaxed agent-scope store), then combine the pairs of all S chunks. The first wave reads
// the slots 64 at a time, one per lane (the polls overlap instead of queueing behind one
// another), and combines them with the fixed butterfly of wave_reduce_stats, blocks in slot
// order: the order never depends on timing, so every chunk of the row gets bit-identical
// (m, d). Slots hold kPartialEmpty until published. The wait is bounded: after kSpinLimit
// polls a lane gives up, the chunk sets kFlagExchangeTimeout in *flags and returns m = NaN,
// and once the flag is set no chunk waits again, so the grid always drains. Called by every
// thread of the workgroup (bcast is LDS).
template <int THREADS>
__device__ __forceinline__ Stats exchange_row_stats(Stats st, uint64_t* slots, int S, int chunk,
                                                    int32_t* flags, float* bcast) {
  const int tid = threadIdx.x;
  if (tid == 0)
    __hip_atomic_store(slots + chunk, pack_pair(st.m, st.d), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (tid < kWave) {
    int budget = (__hip_atomic_load(flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                  kFlagExchangeTimeout) ? 0 : kSpinLimit;
    bool ok = true;
    Stats acc{kNegInf, 0.f};
    for (int b = 0; b < S; b += kWave) {
      Stats mine{kNegInf, 0.f};
      if (b + tid < S && ok) {
        const uint64_t w = poll_slot(slots + b + tid, budget, ok);
        if (ok) mine = {pair_m(w), pair_d(w)};
      }
      acc = combine(acc, wave_reduce_stats(mine));
    }
    if (__any(!ok)) {
      if (tid == 0)
        __hip_atomic_fetch_or(flags, kFlagExchangeTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      acc.m = __builtin_nanf("");
    }
    if (tid == 0) {
      bcast[0] = acc.m;
      bcast[1] = acc.d;
    }
  }
  __syncthreads();
  return {bcast[0], bcast[1]};
}

// Write grouping of split rows: row r's chunks, once they have their (m, d), wait until the
// chunks of the other rows of its group of G adjacent rows (rows g0 .. g0 + G - 1, g0 a
// multiple of G, cut at M) have published their slots; for the cross-entropy (target given)
// only rows whose gradient is not zero (target neither ignore_index nor outside [0, V))
// publish, and only those are waited for. Nothing is combined: the wait only holds a
// chunk's stores until its neighbours' chunks are ready to store theirs too, so that
// adjacent rows are written back together. The first wave polls up to 64 slots at a time,
// one per lane (after loading the slot's row target, if any). The timeout flag is read only
// for a slot found unpublished: the wait is bounded like the exchange's, ends at once when
// the flag is set and, as it decides nothing, simply ends when its budget runs out. Called
// by every thread of the workgroup.
template <int G>
__device__ __forceinline__ void wait_row_group(const uint64_t* partials, const int64_t* target,
                                               int64_t ignore_index, int64_t V, int64_t r,
                                               int64_t M, int S, const int32_t* flags) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    const int64_t g0 = r - r % G;                         // G is a power of two
    const int rows = (int)(M - g0 < G ? M - g0 : G);
    const int n = rows * S;                               // slots of the group
    int budget = kSpinLimit;
    for (int b = 0; b < n; b += kWave) {
      const int q = b + tid;
      if (q >= n) continue;
      const int64_t rr = g0 + q / S;
      if (rr == r) continue;
      if (target) {  // cross-entropy: rows with a zero gradient publish nothing
        const int64_t t = target[rr];
        if (t == ignore_index || t < 0 || t >= V) continue;
      }
      const uint64_t* slot = partials + g0 * S + q;
      if (__hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != kPartialEmpty)
        continue;
      // not yet published: the timeout flag decides whether to wait at all
      if (__hip_atomic_load(flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
          kFlagExchangeTimeout)
        break;
      bool ok = true;
      (void)poll_slot(slot, budget, ok);
      if (!ok) break;
    }
  }
  __syncthreads();
}

// Split rows of the softmax backward: publish this chunk's partial dot product and add the
// S partials of the row, read by the first wave 64 at a time and summed with the fixed
// butterfly of wave_reduce (bit-identical sums in every chunk). A published word is the
// float's bits with 1 in the upper half, never kPartialEmpty. Same bounded wait and timeout
// flag as exchange_row_stats (the sum is NaN after a timeout).
template <int THREADS>
__device__ __forceinline__ float exchange_row_sum(float s, uint64_t* slots, int S, int chunk,
                                                  int32_t* flags, float* bcast) {
  const int tid = threadIdx.x;
  if (tid == 0)
    __hip_atomic_store(slots + chunk, (uint64_t)as_u32(s) | (1ull << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (tid < kWave) {
    int budget = (__hip_atomic_load(flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                  kFlagExchangeTimeout) ? 0 : kSpinLimit;
    bool ok = true;
    float acc = 0.f;
    for (int b = 0; b < S; b += kWave) {
      float mine = 0.f;
      if (b + tid < S && ok) {
        const uint64_t w = poll_slot(slots + b + tid, budget, ok);
        if (ok) mine = as_f32((uint32_t)w);
      }
      acc += wave_reduce(mine, OpAdd());
    }
    if (__any(!ok)) {
      if (tid == 0)
        __hip_atomic_fetch_or(flags, kFlagExchangeTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      acc = __builtin_nanf("");
    }
    if (tid == 0) bcast[0] = acc;
  }
  __syncthreads();
  return bcast[0];
}

// One element into a thread's running (m, d): the online-softmax rule, -inf elements adding
// nothing.
__device__ __forceinline__ void online_add(Stats& st, float x) {
  if (x > st.m) {
    st.d = (st.m == kNegInf ? 0.f : st.d * __builtin_amdgcn_exp2f((st.m - x) * kLog2e)) + 1.f;
    st.m = x;
  } else if (x != kNegInf) {
    st.d += __builtin_amdgcn_exp2f((x - st.m) * kLog2e);
  }
}

// ----------------------------------------------------------------------------- stream rows
// The stream kernels walk a row in windows of kStreamWindow vectors (one buffer resource
// each, so offsets stay 32-bit for rows of any length), kStreamUnroll vectors in flight
// per thread.
constexpr int64_t kStreamWindow = int64_t(1) << 26;  // 1 GiB
constexpr int kStreamUnroll = 4;

// Vector v of chunk c with its out-of-row elements replaced by `fill` (a vector at or past
// the chunk's end is all fill).
template <int D>
__device__ __forceinline__ u32x4 vec_masked(u32x4 x, int v, const Chunk<D>& c, uint32_t fill) {
  if (v >= c.nvec) return splat(fill);
  if (v == c.head) x = mask_vec<D>(x, c.h0, c.h1, fill);
  if (v == c.tail) x = mask_vec<D>(x, c.t0, c.t1, fill);
  return x;
}

// One vector folded into a running (m, d): the vector's maximum, one rescale of the running
// sum, then the vector's terms. -inf elements add nothing; NaN elements make d NaN.
template <int D>
__device__ __forceinline__ void online_add_vec(Stats& st, u32x4 x) {
  constexpr int EPV = Elt<D>::kPerVec;
  float vm = kNegInf;
#pragma unroll
  for (int e = 0; e < EPV; ++e) vm = fmaxf(vm, elem<D>(x, e));
  const float mn = fmaxf(st.m, vm);
  const float mnL = scaled_max(mn);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    const float xe = elem<D>(x, e);
    const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(xe, kLog2e, -mnL));
    s += xe == kNegInf ? 0.f : t;
  }
  st.d = (st.m == mn ? st.d : st.d * __builtin_amdgcn_exp2f((st.m - mn) * kLog2e)) + s;
  st.m = mn;
}

// Store vector v of an output chunk: whole, or only its in-row elements for the partial
// first / last vector.
template <int D>
__device__ __forceinline__ void store_vec(const Chunk<D>& c, int v, const u32x4& bits) {
  const uint32_t off = (uint32_t)v * 16u;
  if (v == c.head) store_partial<D>(c.rsrc, off, bits, c.h0, c.h1);
  else if (v == c.tail) store_partial<D>(c.rsrc, off, bits, c.t0, c.t1);
  else buf_store(c.rsrc, off, bits);
}

// exp2(x*log2e - coff) for every element of one slot, in the element type, XOR-ed with
// `sign` (0, or Elt<D>::kSignWord to negate every result: a negative upstream gradient).
template <int D>
__device__ __forceinline__ u32x4 exp_slot(u32x4 v, float coff, uint32_t sign = 0) {
  pin_slot<D>(v);
  OutVec<D> o;
#pragma unroll
  for (int e = 0; e < Elt<D>::kPerVec; ++e)
    o.v[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(elem<D>(v, e), kLog2e, -coff));
  return o.bits() ^ splat(sign);
}

// x * s for every element of one slot, in the element type (fp32 product, one rounding to
// bf16 for bf16 rows).
template <int D>
__device__ __forceinline__ u32x4 mul_slot(u32x4 v, float s) {
  pin_slot<D>(v);
  OutVec<D> o;
#pragma unroll
  for (int e = 0; e < Elt<D>::kPerVec; ++e) o.v[e] = elem<D>(v, e) * s;
  return o.bits();
}


// Instantiation lists of the row kernels (the shapes of kFwdShapes / kBwdShapes).
#define XR_SHAPES_FWD(X, D)                                                                     \
  X(D, 64, 4) X(D, 64, 8) X(D, 64, 16) X(D, 128, 8) X(D, 128, 16) X(D, 256, 8) X(D, 256, 16)  \
  X(D, 512, 8) X(D, 512, 16) X(D, 1024, 16)
#define XR_SHAPES_BWD(X, D) \
  X(D, 64, 4) X(D, 64, 8) X(D, 128, 8) X(D, 256, 8) X(D, 512, 8) X(D, 1024, 8)


}  // namespace xr
