// xr_probe.hip -- the memory-ceiling probe of the measurement: the row kernels' launch (the
// same workgroup shapes, chunks per row, buffer loads and non-temporal stores, every load of
// a chunk landed and a workgroup barrier before its first store), with none of their
// arithmetic, statistics exchange or row groups. Timed beside a row kernel on the same rows,
// it shows what that launch shape can move at that size.
#include "xr_rows.h"

namespace xr {

template <int D, int THREADS, int VPT, int NIN>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void probe_rows_kernel(ProbeParams p) {
  const int S = p.S;
  const int64_t r = blockIdx.x / S;
  const int64_t lo = (int64_t)(blockIdx.x % S) * p.chunk_vecs;
  const bool read = !(p.target != nullptr && p.target[r] == p.ignore_index);
  u32x4 a[VPT], b[VPT];
  if (read) {
    issue_loads<D, THREADS, VPT, kPolicyNT>(a, Chunk<D>(p.in0 + r * p.ldin_bytes, p.N, lo, p.chunk_vecs));
    if (NIN == 2)
      issue_loads<D, THREADS, VPT, kPolicyNT>(b, Chunk<D>(p.in1 + r * p.ldin_bytes, p.N, lo, p.chunk_vecs));
    reg_barrier(a);  // every load of the chunk has landed
    if (NIN == 2) reg_barrier(b);
  } else {
#pragma unroll
    for (int k = 0; k < VPT; ++k) a[k] = b[k] = splat(0u);
  }
  __syncthreads();
  const Chunk<D> co(p.out + r * p.ldout_bytes, p.N, lo, p.chunk_vecs);
#pragma unroll
  for (int k = 0; k < VPT; ++k) store_slot<D, THREADS>(co, k, NIN == 2 ? (a[k] ^ b[k]) : a[k]);
}

// The plain copy of the ceiling: a grid-stride loop over 16-byte vectors, kCopyUnroll vectors
// in flight per thread before their stores, non-temporal both ways; with two inputs the
// stored vector is in ^ in1 (two reads per write, as the softmax backward). nvec vectors.
template <int THREADS, int NIN>
__global__ __launch_bounds__(THREADS) void probe_copy_kernel(CopyParams p) {
  constexpr int U = kCopyUnroll;
  const u32x4* __restrict__ in = reinterpret_cast<const u32x4*>(p.in);
  const u32x4* __restrict__ in1 = reinterpret_cast<const u32x4*>(p.in1);
  u32x4* __restrict__ out = reinterpret_cast<u32x4*>(p.out);
  const int64_t nvec = p.nvec;
  const int64_t stride = (int64_t)gridDim.x * THREADS;
  int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
  for (; i + (U - 1) * stride < nvec; i += U * stride) {
    u32x4 v[U], w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = __builtin_nontemporal_load(in + i + u * stride);
      if (NIN == 2) w[u] = __builtin_nontemporal_load(in1 + i + u * stride);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      __builtin_nontemporal_store(NIN == 2 ? (v[u] ^ w[u]) : v[u], out + i + u * stride);
  }
  for (; i < nvec; i += stride) {
    u32x4 v = __builtin_nontemporal_load(in + i);
    if (NIN == 2) v ^= __builtin_nontemporal_load(in1 + i);
    __builtin_nontemporal_store(v, out + i);
  }
}

// The same stream in place: every vector read and written back to where it was, by the thread
// that read it (the traffic of a kernel that overwrites its input). A store of the value just
// loaded from the same address is a no-op to the compiler, which would drop the loop; the
// empty asm statement (no instruction) makes each vector opaque to it.
template <int THREADS>
__global__ __launch_bounds__(THREADS) void probe_inplace_kernel(CopyParams p) {
  constexpr int U = kCopyUnroll;
  u32x4* io = reinterpret_cast<u32x4*>(p.out);
  const int64_t nvec = p.nvec;
  const int64_t stride = (int64_t)gridDim.x * THREADS;
  int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
  for (; i + (U - 1) * stride < nvec; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(io + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      asm volatile("" : "+v"(v[u]));
      __builtin_nontemporal_store(v[u], io + i + u * stride);
    }
  }
  for (; i < nvec; i += stride) {
    u32x4 v = __builtin_nontemporal_load(io + i);
    asm volatile("" : "+v"(v));
    __builtin_nontemporal_store(v, io + i);
  }
}

const void* probe_copy_kernel_ptr(int threads, int inputs) {
  if (inputs == 0) {
    switch (threads) {
      case 256: return reinterpret_cast<const void*>(&probe_inplace_kernel<256>);
      case 512: return reinterpret_cast<const void*>(&probe_inplace_kernel<512>);
      case 1024: return reinterpret_cast<const void*>(&probe_inplace_kernel<1024>);
    }
  } else if (inputs == 1) {
    switch (threads) {
      case 256: return reinterpret_cast<const void*>(&probe_copy_kernel<256, 1>);
      case 512: return reinterpret_cast<const void*>(&probe_copy_kernel<512, 1>);
      case 1024: return reinterpret_cast<const void*>(&probe_copy_kernel<1024, 1>);
    }
  } else if (inputs == 2) {
    switch (threads) {
      case 256: return reinterpret_cast<const void*>(&probe_copy_kernel<256, 2>);
      case 512: return reinterpret_cast<const void*>(&probe_copy_kernel<512, 2>);
      case 1024: return reinterpret_cast<const void*>(&probe_copy_kernel<1024, 2>);
    }
  }
  return nullptr;
}

#define XR_CASE_PROBE1(D, T, V) \
  if (s.threads == T && s.vpt == V) return reinterpret_cast<const void*>(&probe_rows_kernel<D, T, V, 1>);
#define XR_CASE_PROBE2(D, T, V) \
  if (s.threads == T && s.vpt == V) return reinterpret_cast<const void*>(&probe_rows_kernel<D, T, V, 2>);
const void* probe_rows_kernel_ptr(int dtype, Shape s, int inputs) {
  if (inputs == 1) {
    if (dtype == kF32) { XR_SHAPES_FWD(XR_CASE_PROBE1, kF32) }
    if (dtype == kBF16) { XR_SHAPES_FWD(XR_CASE_PROBE1, kBF16) }
  } else if (inputs == 2) {
    if (dtype == kF32) { XR_SHAPES_BWD(XR_CASE_PROBE2, kF32) }
    if (dtype == kBF16) { XR_SHAPES_BWD(XR_CASE_PROBE2, kBF16) }
  }
  return nullptr;
}

}  // namespace xr
