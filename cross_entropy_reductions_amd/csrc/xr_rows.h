// xr_rows.h -- building blocks of the row kernels (included by the kernel sources only).
#pragma once

#include "xr_device.h"
#include "xr_internal.h"

namespace xr {


inline constexpr float kNegInf = -__builtin_inff();
constexpr int kSpinLimit = 1 << 20;

// Exponentials are taken relative to the row maximum m; the results must depend only on the
// differences x - m, not on m's magnitude (a row filled with a large negative mask value
// keeps the maximum's term at exactly 1).
//  * Sum pass: exp2(x log2e - mL), mL = m log2e rounded once (one fma per element), with a
//    per-thread correction of the sum where mL's rounding would matter (thread_sum_exp).
//  * Output pass, exp(x - m) / D = exp2 of (x - m) log2e - off with off = log2 D (log2 d,
//    plus log2 n and -log2|s| for the cross-entropy), in one of two forms:
//      scaled    exp2(x log2e - c), c = mL + off: one fma per element;
//      relative  exp2((x - m) log2e - off): one subtraction more.
//    The scaled form carries the roundings of mL and c into every exponent: at most 2^-18
//    (2.6e-6 relative in a result) while both stay under 2^7 in magnitude (|m| under about
//    88), growing with |m| past that (emulated over rows of 32000 fp32 logits with the
//    maximum near 1e3 / 1e5 / -1e6: 6.0e-5 / 4.2e-3 / 5.9e-2 relative, against 3.9e-6 in
//    the relative form); mL itself overflows past |m| = 2.4e38. The relative form instead
//    rounds x - m where x lies far below m: over the 2048 x 256000 fp32 cross-entropy rows
//    the emulated worst case is 9.3e-6 scaled, 1.0e-5 relative. So rows whose mL and c stay
//    under 2^7 take the scaled form and all others the relative one, the same choice in
//    every lane (one scalar branch around the pass).
// In the scaled form the thread holding the maximum forms its term and the output constant
// on the same mL, whose rounding then cancels: a one-column row gets p = 1 and a zero
// gradient exactly.
// m log2e rounded once to fp32 (no contraction into a neighbouring operation).
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
// Magnitude below which the scaled form's rounded values keep their error within 2^-18.
constexpr float kScaledLimit = 0x1p7f;
// |m| below which the sum pass splits m log2e into mL + lo with |lo| <= 32.
constexpr float kSplitLimit = 0x1p29f;

// How a row's outputs exp2((x - m) log2e - off) are evaluated; the same in every lane.
struct ExpForm {
  float m;      // the row maximum
  float c;      // scaled: exp_offset(scaled_max(m), off); relative: off
  bool scaled;
};
__device__ __forceinline__ ExpForm exp_form(float m, float off) {
  const float mL = scaled_max(m);
  const float c = exp_offset(mL, off);
  // m and off are the same in every lane: readfirstlane makes the choice a scalar one
  const bool scaled =
      __builtin_amdgcn_readfirstlane(fabsf(mL) < kScaledLimit && fabsf(c) < kScaledLimit) != 0;
  return {m, scaled ? c : off, scaled};
}
template <bool SCALED>
__device__ __forceinline__ float exp_of(float x, const ExpForm& f) {
  return __builtin_amdgcn_exp2f(SCALED ? __builtin_fmaf(x, kLog2e, -f.c)
                                       : __builtin_fmaf(x - f.m, kLog2e, -f.c));
}
// The negative log-softmax's -log p = m + log d - x in the same two forms: scaled c - x with
// c = m + log d (one rounding of c, at most 2^-18 while |c| < 2^7), relative
// log d - (x - m).
__device__ __forceinline__ ExpForm nll_form(float m, float lg) {
  const float c = m + lg;
  const bool scaled =
      __builtin_amdgcn_readfirstlane(fabsf(m) < kScaledLimit && fabsf(c) < kScaledLimit) != 0;
  return {m, scaled ? c : lg, scaled};
}
template <bool SCALED>
__device__ __forceinline__ float nll_of(float x, const ExpForm& f) {
  return SCALED ? f.c - x : f.c - (x - f.m);
}

// Runs body(Form<true>()) or body(Form<false>()) as the row's form says: each form gets a
// whole pass of straight-line code under one scalar branch. The row kernels issue their
// next row's loads after it, not inside the bodies: the compiler hoists loads common to both
// arms ahead of the branch, where two rows of registers are then live at once.
template <bool B> struct Form { static constexpr bool value = B; };
template <class F>
__device__ __forceinline__ void with_form(const ExpForm& f, F&& body) {
  if (f.scaled) body(Form<true>());
  else body(Form<false>());
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

// sum_j exp(x_j - m) over the chunk elements this thread holds, as the sum of
// exp2(x*k - hi), four partial sums; k and hi are chosen once per thread:
//   |m| < 2^29  k = log2e, hi = mL = m log2e rounded. Where |mL| < 2^7 that is the scaled
//               form as it stands; past it the sum is scaled once by 2^-lo, lo = m log2e - mL
//               exactly (an fma gives a product's rounding error exactly), which makes the
//               terms relative to m itself; |lo| <= 32 keeps every term in range.
//   otherwise   k is a power of two with k|m| in [2^40, 2^41), hi = k m (both exact): the
//               maximum's terms are exp2(0) = 1, and every other element lies at least
//               2^-25 |m| below m, where exp(x - m) is 0 in fp32 and exp2(k (x - m)) is too.
// One straight-line loop for every row (no branch: the maximum's reduction can overlap it).
template <int D, int THREADS, int VPT>
__device__ __forceinline__ float thread_sum_exp(const u32x4 (&v)[VPT], const Chunk<D>& c, float m) {
  constexpr int EPV = Elt<D>::kPerVec;
  const float mL = scaled_max(m);
  const bool split = fabsf(m) < kSplitLimit;
  // 2^(40 - e) for |m| in [2^e, 2^(e+1)): exponent field 167 - e
  const float kbig = as_f32(((127u + 40u + 127u) << 23) - (as_u32(m) & 0x7f800000u));
  const float k = split ? kLog2e : kbig;
  const float hi = split ? mL : kbig * m;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < VPT; ++q) {
    if (slot_kind<THREADS>(q, c.nvec) == kSlotNone) continue;
    const u32x4 x = masked_slot<D, THREADS>(v[q], q, c, Elt<D>::kNegInfWord);
#pragma unroll
    for (int e = 0; e < EPV; ++e) s[e & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(elem<D>(x, e), k, -hi));
  }
  const float sum = (s[0] + s[1]) + (s[2] + s[3]);
  const bool corr = split && !(fabsf(mL) < kScaledLimit);
  return corr ? sum * __builtin_amdgcn_exp2f(-__builtin_fmaf(m, kLog2e, -mL)) : sum;
}

// This thread's (m, d) over its chunk elements: its own maximum, then the sum of
// exp(x - m) with that maximum. No workgroup barrier sits between the two passes, so each
// wave streams through its slots as their loads land; the workgroup combines the pairs once.
template <int D, int THREADS, int VPT>
__device__ __forceinline__ Stats thread_stats(u32x4 (&v)[VPT], const Chunk<D>& c) {
  const float m = thread_max<D, THREADS, VPT>(v, c);
  reg_barrier(v);
  const float d = (m == kNegInf) ? 0.f : thread_sum_exp<D, THREADS, VPT>(v, c, m);
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
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    const float xe = elem<D>(x, e);
    const float t = __builtin_amdgcn_exp2f((xe - mn) * kLog2e);
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

// exp_of<SCALED>(x, f) for every element of one slot, in the element type, XOR-ed with
// `sign` (0, or Elt<D>::kSignWord to negate every result: a negative upstream gradient).
// The relative form pins the slot for fp32 too: its subtraction x - m is cheap enough that
// the compiler would otherwise form it for every slot of the row at once and spill.
template <int D, bool SCALED>
__device__ __forceinline__ u32x4 exp_slot(u32x4 v, const ExpForm& f, uint32_t sign = 0) {
  if (SCALED) pin_slot<D>(v);
  else pin(v);
  OutVec<D> o;
#pragma unroll
  for (int e = 0; e < Elt<D>::kPerVec; ++e) o.v[e] = exp_of<SCALED>(elem<D>(v, e), f);
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
