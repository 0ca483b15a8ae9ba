// xr_device.h -- device-side building blocks shared by the row kernels (gfx950, wave64).
//
// Rows are moved as 16-byte vectors (global_load_dwordx4 / global_store_dwordx4)
// and kept in registers as raw bits; elements are widened to fp32 when used.
// All arithmetic is fp32. Reductions are done inside a wave with DPP and
// ds_swizzle, then across the waves of a workgroup through LDS, in a fixed order
// so every run gives bit-identical results.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kWave = 64;

enum DType : int { kF32 = 0, kBF16 = 1 };

// Element traits: bytes per element, elements per 16-byte vector, the -inf
// bit pattern filling one 32-bit word.
template <int D> struct Elt;
template <> struct Elt<kF32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;
  static constexpr uint32_t kNegInfWord = 0xFF800000u;
  static constexpr uint32_t kSignWord = 0x80000000u;  // sign bit of every element of a word
};
template <> struct Elt<kBF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  static constexpr uint32_t kNegInfWord = 0xFF80FF80u;
  static constexpr uint32_t kSignWord = 0x80008000u;
};

__device__ __forceinline__ float as_f32(uint32_t b) { return __builtin_bit_cast(float, b); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// Element e (0 .. kPerVec-1) of a vector, widened to fp32 (exact for bf16).
template <int D> __device__ __forceinline__ float elem(const u32x4& v, int e);
template <> __device__ __forceinline__ float elem<kF32>(const u32x4& v, int e) {
  return as_f32(v[e]);
}
template <> __device__ __forceinline__ float elem<kBF16>(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? as_f32(w & 0xFFFF0000u) : as_f32(w << 16);
}

// Two fp32 values rounded to bf16 (nearest-even, v_cvt_pk_bf16_f32), packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 r = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// v rounded to the element type (as a store of v would leave it), widened back to fp32.
template <int D> __device__ __forceinline__ float round_elem(float v) {
  if (D == kF32) return v;
  return as_f32(pack_bf16x2(v, 0.f) << 16);
}

// A vector of kPerVec fp32 results stored back in the element type.
template <int D> struct OutVec;
template <> struct OutVec<kF32> {
  float v[4];
  __device__ __forceinline__ u32x4 bits() const {
    return (u32x4){as_u32(v[0]), as_u32(v[1]), as_u32(v[2]), as_u32(v[3])};
  }
};
template <> struct OutVec<kBF16> {
  float v[8];
  __device__ __forceinline__ u32x4 bits() const {
    return (u32x4){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
  }
};

// ----------------------------------------------------------------------------- memory
// Rows are read and written through buffer resources (V#) held in scalar registers:
// one 32-bit VGPR offset per access, and the hardware range check (an offset at or past
// num_records loads zeros and drops stores) guards every access past the chunk's end.
// The offset is always passed as the VGPR operand (soffset = 0) so it is range-checked.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family
// Cache-policy bits of the buffer instructions: 1 = sc0, 2 = nt, 16 = sc1. Row stores are
// non-temporal (nothing re-reads them); the load policy is a kernel template parameter,
// chosen per launch (see the plan in xr_api.cpp).
constexpr int kPolicyDefault = 0;
constexpr int kPolicyNT = 2;
#ifndef XR_STORE_POLICY
#define XR_STORE_POLICY 2
#endif
constexpr int kStorePolicy = XR_STORE_POLICY;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
template <int LP> __device__ __forceinline__ u32x4 buf_load(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, LP);
}
__device__ __forceinline__ void buf_store(Rsrc r, uint32_t off, const u32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kStorePolicy);
}
__device__ __forceinline__ void buf_store_b16(Rsrc r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, kStorePolicy);
}
__device__ __forceinline__ void buf_store_b32(Rsrc r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kStorePolicy);
}
// An offset no resource covers: the access is dropped (store) or reads zeros (load).
constexpr uint32_t kOffNone = 0x80000000u;

// One element of a row, widened to fp32.
template <int D> __device__ __forceinline__ float buf_load_elem(Rsrc r, uint32_t off) {
  if (D == kF32) return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
  const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  return __builtin_bit_cast(float, h << 16);
}

// Replace the elements of v outside [e0, e1) with the matching element of `fill`
// (a word holding one or two copies of the filler element: -inf or 0).
template <int D> __device__ __forceinline__ u32x4 mask_vec(u32x4 v, int e0, int e1, uint32_t fill) {
  if (D == kF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < e0 || e >= e1) v[e] = fill;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e < e0 || e >= e1) {
        const uint32_t half = (e & 1) ? 0xFFFF0000u : 0x0000FFFFu;
        v[e >> 1] = (v[e >> 1] & ~half) | (fill & half);
      }
    }
  }
  return v;
}

// Store only the elements [e0, e1) of the vector at byte offset off (element stores).
template <int D>
__device__ __forceinline__ void store_partial(Rsrc r, uint32_t off, const u32x4& v, int e0, int e1) {
  if (D == kF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e >= e0 && e < e1) buf_store_b32(r, off + 4u * e, v[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e >= e0 && e < e1)
        buf_store_b16(r, off + 2u * e, (uint16_t)((e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xFFFFu)));
  }
}

// One element value stored in the element type (bf16: rounded to nearest-even).
template <int D> __device__ __forceinline__ void store_elem(Rsrc r, uint32_t off, float val) {
  if (D == kF32) {
    buf_store_b32(r, off, as_u32(val));
  } else {
    buf_store_b16(r, off, (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu));
  }
}

// ----------------------------------------------------------------------------- wave reductions
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return as_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u32(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float swizzle_xor16(float x) {
  // ds_swizzle bit-mask mode: and 0x1F, or 0, xor 0x10 -> lane i reads lane i ^ 16 (within 32).
  return as_f32((uint32_t)__builtin_amdgcn_ds_swizzle((int)as_u32(x), 0x401F));
}
__device__ __forceinline__ float readlane(float x, int lane) {
  return as_f32((uint32_t)__builtin_amdgcn_readlane((int)as_u32(x), lane));
}

struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpAdd {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

// Butterfly over the 64 lanes; every lane ends with the same (wave-uniform) value.
//   xor 1, xor 2    : DPP quad_perm [1,0,3,2] and [2,3,0,1]
//   xor 4 (effect)  : DPP row_half_mirror (lane i <-> 7-i inside 8 lanes)
//   xor 8 (effect)  : DPP row_mirror (lane i <-> 15-i inside 16 lanes)
//   xor 16          : ds_swizzle
//   halves of 64    : readlane 0 and 32
template <class Op> __device__ __forceinline__ float wave_reduce(float x, Op op) {
  x = op(x, dpp<0xB1>(x));
  x = op(x, dpp<0x4E>(x));
  x = op(x, dpp<0x141>(x));
  x = op(x, dpp<0x140>(x));
  x = op(x, swizzle_xor16(x));
  return op(readlane(x, 0), readlane(x, 32));
}

// Workgroup reduction through LDS: one slot per wave, read back by every thread in
// wave order. `slots` must hold THREADS/64 floats; callers alternate buffers so that
// one barrier per reduction suffices (see the row kernels).
template <int THREADS, class Op>
__device__ __forceinline__ float block_reduce(float x, Op op, float* slots) {
  x = wave_reduce(x, op);
  if (THREADS == kWave) return x;
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) slots[wave] = x;
  __syncthreads();
  float r = slots[0];
#pragma unroll
  for (int w = 1; w < THREADS / kWave; ++w) r = op(r, slots[w]);
  return r;
}

// (m, d) statistics of a set of elements: m their maximum, d = sum exp(x - m). Two sets
// combine by the online-softmax rule; a set whose maximum is -inf (empty, or all -inf) is
// the identity. The combine is commutative bit for bit (fp add is), so a butterfly leaves
// the same pair on every lane.
struct Stats {
  float m, d;
};
__device__ __forceinline__ Stats combine(Stats a, Stats b) {
  const float mx = fmaxf(a.m, b.m);
  if (mx == -__builtin_inff()) return {mx, 0.f};
  return {mx, a.d * __builtin_amdgcn_exp2f((a.m - mx) * kLog2e) +
                  b.d * __builtin_amdgcn_exp2f((b.m - mx) * kLog2e)};
}
template <int CTRL> __device__ __forceinline__ Stats dpp_stats(Stats s) {
  return {dpp<CTRL>(s.m), dpp<CTRL>(s.d)};
}
__device__ __forceinline__ Stats wave_reduce_stats(Stats s) {
  s = combine(s, dpp_stats<0xB1>(s));
  s = combine(s, dpp_stats<0x4E>(s));
  s = combine(s, dpp_stats<0x141>(s));
  s = combine(s, dpp_stats<0x140>(s));
  s = combine(s, {swizzle_xor16(s.m), swizzle_xor16(s.d)});
  return combine({readlane(s.m, 0), readlane(s.d, 0)}, {readlane(s.m, 32), readlane(s.d, 32)});
}
// Workgroup combine through LDS (one slot per wave, read back in wave order). Callers
// alternate two slot buffers between consecutive calls, so one barrier per call suffices.
template <int THREADS>
__device__ __forceinline__ Stats block_reduce_stats(Stats s, float2* slots) {
  s = wave_reduce_stats(s);
  if (THREADS == kWave) return s;
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) slots[wave] = make_float2(s.m, s.d);
  __syncthreads();
  Stats r = {slots[0].x, slots[0].y};
#pragma unroll
  for (int w = 1; w < THREADS / kWave; ++w) r = combine(r, {slots[w].x, slots[w].y});
  return r;
}

// Integer sum across a workgroup (used by the target scan).
template <int THREADS>
__device__ __forceinline__ int block_sum_int(int x, int* slots) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) slots[wave] = x;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int w = 0; w < THREADS / kWave; ++w) r += slots[w];
  return r;
}

// ----------------------------------------------------------------------------- row chunks
// A row of `len` elements starting at byte address `row` is covered by the 16-byte-aligned
// vectors [0, nv) counted from align_down(row, 16); element j of the row sits at position
// lead + j of that vector space. A chunk is the vectors [lo, min(nv, lo + cv)) of the row;
// its buffer resource starts at vector lo, so chunk-local vector i is at byte 16 i.
// Every member is workgroup-uniform (scalar registers).
template <int D> struct Chunk {
  static constexpr int EPV = Elt<D>::kPerVec;
  uintptr_t base;  // byte address of chunk vector 0 (16-byte aligned)
  Rsrc rsrc;       // the whole chunk: [base, base + 16 nvec)
  int nvec;        // vectors in this chunk (0 when the chunk lies past the row end)
  int lead;        // elements between the aligned vector start and the row's first element
  int head;        // chunk-local index of the row's partial first vector, or -1
  int tail;        // chunk-local index of the row's partial last vector, or -1
  int h0, h1;      // valid elements [h0, h1) of the head vector
  int t0, t1;      // valid elements [t0, t1) of the tail vector
  uint32_t hoff;   // byte offsets of the head / tail vectors in the chunk
  uint32_t toff;
  int64_t lo;      // first row vector of the chunk

  __device__ __forceinline__ Chunk(const void* row, int64_t len, int64_t lo_, int64_t cv) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(row);
    lo = lo_;
    lead = (int)((a & 15u) / Elt<D>::kBytes);
    const int64_t nv = (lead + len + EPV - 1) / EPV;
    const int64_t hi = (nv < lo + cv) ? nv : lo + cv;
    nvec = hi > lo ? (int)(hi - lo) : 0;
    base = a - (a & 15u) + (uintptr_t)(lo * 16);
    rsrc = make_rsrc(reinterpret_cast<const void*>(base), (uint32_t)nvec * 16u);
    head = -1;
    tail = -1;
    h0 = t0 = 0;
    h1 = t1 = EPV;
    if (lead != 0 && lo == 0 && nvec > 0) {
      head = 0;
      h0 = lead;
      h1 = (lead + len < EPV) ? (int)(lead + len) : EPV;
    }
    const int tail_end = (int)((lead + len) % EPV);
    if (tail_end != 0 && nv - 1 >= lo && nv - 1 < hi) {
      const int ti = (int)(nv - 1 - lo);
      if (ti == head) {
        h1 = tail_end;  // the row fits in one vector: one partial vector [lead, lead + len)
      } else {
        tail = ti;
        t1 = tail_end;
      }
    }
    // Passed through readfirstlane so that, inside a branch on (lane vector == head), the
    // compiler cannot rewrite these scalar offsets into per-lane ones and keep a copy of
    // every slot's element offsets alive in vector registers.
    hoff = (uint32_t)__builtin_amdgcn_readfirstlane(head * 16);
    toff = (uint32_t)__builtin_amdgcn_readfirstlane(tail * 16);
  }

  // Resource for the slot starting at chunk vector s0: lane l addresses vector s0 + l at
  // byte 16 l, and lanes at or past the chunk's end fall outside num_records (loads give
  // zeros without touching memory, stores are dropped). Built in scalar registers at each
  // use; the clamp is a signed max (an unsigned saturating subtraction would be selected
  // as a vector instruction and make the compiler wrap every access in a loop over
  // distinct resources).
  __device__ __forceinline__ Rsrc slot(int s0) const {
    const int rem = (nvec - s0) * 16;  // signed: max() below is a scalar instruction
    return make_rsrc(reinterpret_cast<const void*>(base + (uint32_t)s0 * 16u),
                     (uint32_t)(rem > 0 ? rem : 0));
  }
};

}  // namespace xr
