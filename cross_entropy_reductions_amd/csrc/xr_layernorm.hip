// xr_layernorm.hip -- layer norm forward and backward for gfx950.
//
// What is computed (the Triton LayerNorm tutorial page, whose code is cut off in the copy
// at hand; the definitions follow its prose and the paper it cites, Ba, Kiros & Hinton 2016):
//   forward   mean_i = (1/N) sum_j x_ij, var_i = (1/N) sum_j (x_ij - mean_i)^2,
//             rstd_i = 1/sqrt(var_i + eps), y_ij = (x_ij - mean_i) rstd_i w_j + b_j;
//             mean and rstd are saved for the backward
//   backward  xhat = (x - mean) rstd, g = w dy, c1 = mean_j(xhat g), c2 = mean_j(g),
//             dx = rstd (g - (xhat c1 + c2)); dw_j = sum_i dy_ij xhat_ij, db_j = sum_i dy_ij
//
// The page reduces dw and db in two stages: each program adds its rows' partial sums into
// one of a few buffers (guarded by locks), and a second kernel sums the buffers. Here the
// same two stages run without locks: workgroup g of a persistent grid of G owns partial
// row g, accumulates the columns of its rows in registers, and writes that row once;
// the second kernel sums the G partial rows of every column in a fixed order, so the
// result does not depend on timing.
//
// Row-resident kernels (rows 16-byte aligned, N * element size a multiple of 16): thread t
// holds 16-byte vectors t, t + T, ... of its row, and of w (and b) for the whole grid's
// life; lanes past the row's last vector read zeros through the buffer range check. Other
// layouts go through element-wise stream kernels with the same partial-row contract.
#include "xr_rows.h"

namespace xr {

const Shape kLnFwdShapes[kNumLnFwdShapes] = {{64, 1},   {64, 2},   {64, 4},   {128, 4},
                                             {256, 4},  {512, 4},  {1024, 4}};
const Shape kLnBwdShapes[kNumLnBwdShapes] = {{64, 1},   {64, 2},   {128, 2},  {256, 2},
                                             {512, 2},  {1024, 2}, {1024, 4}};

// Resource over vectors [s0, nvec) of a row of nvec 16-byte vectors starting at `base`.
__device__ __forceinline__ Rsrc vec_rsrc(const void* base, int nvec, int s0) {
  const int rem = (nvec - s0) * 16;
  return make_rsrc(static_cast<const char*>(base) + (size_t)s0 * 16u, (uint32_t)(rem > 0 ? rem : 0));
}

// Sum of a pair over the workgroup (fixed order: waves, then wave slots in order).
template <int THREADS>
__device__ __forceinline__ float2 block_sum2(float a, float b, float2* slots) {
  a = wave_reduce(a, OpAdd());
  b = wave_reduce(b, OpAdd());
  if (THREADS == kWave) return make_float2(a, b);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) slots[wave] = make_float2(a, b);
  __syncthreads();
  float2 r = slots[0];
#pragma unroll
  for (int w = 1; w < THREADS / kWave; ++w) {
    r.x += slots[w].x;
    r.y += slots[w].y;
  }
  return r;
}

// ============================================================================ forward
template <int D, int THREADS, int VPT, int LP>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void ln_fwd_kernel(LnFwdParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int NW = THREADS / kWave;
  __shared__ float red[2][NW];
  int buf = 0;
  const int tid = threadIdx.x;
  const int nvec = (int)(p.N / EPV);
  const uint32_t off = tid * 16u;
  const float inv_n = 1.0f / (float)p.N;

  // w and b stay in registers for every row this workgroup handles.
  u32x4 wv[VPT], bv[VPT], v[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    wv[k] = buf_load<kPolicyDefault>(vec_rsrc(p.w, nvec, k * THREADS), off);
    bv[k] = buf_load<kPolicyDefault>(vec_rsrc(p.b, nvec, k * THREADS), off);
  }
  int64_t r = blockIdx.x;
  const int64_t G = gridDim.x;
  if (r < p.M) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) v[k] = buf_load<LP>(vec_rsrc(p.x + r * p.ldx_bytes, nvec, k * THREADS), off);
  }
  while (r < p.M) {
    const int64_t rn = r + G;
    // mean: lanes past the row read zeros and add nothing
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      u32x4 x = v[k];
      pin_slot<D>(x);
#pragma unroll
      for (int e = 0; e < EPV; ++e) s[e & 1] += elem<D>(x, e);
    }
    const float mean = block_reduce<THREADS>(s[0] + s[1], OpAdd(), red[buf]) * inv_n;
    buf ^= 1;
    // variance about that mean, from the registers; lanes past the row are left out
    float q[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (k * THREADS >= nvec) continue;
      u32x4 x = v[k];
      pin_slot<D>(x);
      float t[2] = {0.f, 0.f};
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float c = elem<D>(x, e) - mean;
        t[e & 1] = __builtin_fmaf(c, c, t[e & 1]);
      }
      // a lane past the row's last vector (last slot only) holds zeros, not row elements
      if ((k + 1) * THREADS <= nvec || k * THREADS + tid < nvec) {
        q[0] += t[0];
        q[1] += t[1];
      }
    }
    const float var = block_reduce<THREADS>(q[0] + q[1], OpAdd(), red[buf]) * inv_n;
    buf ^= 1;
    const float rstd = 1.0f / sqrtf(var + p.eps);
    if (tid == 0) {
      p.mean[r] = mean;
      p.rstd[r] = rstd;
    }
    // y = (x - mean) rstd w + b
    const char* yrow = p.y + r * p.ldy_bytes;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      u32x4 x = v[k], w = wv[k], b = bv[k];
      pin_slot<D>(x);
      pin_slot<D>(w);
      pin_slot<D>(b);
      OutVec<D> o;
#pragma unroll
      for (int e = 0; e < EPV; ++e)
        o.v[e] = __builtin_fmaf((elem<D>(x, e) - mean) * rstd, elem<D>(w, e), elem<D>(b, e));
      buf_store(vec_rsrc(yrow, nvec, k * THREADS), off, o.bits());
    }
    // the next row's loads after all of this row's stores (not interleaved with them)
    if (rn < p.M) {
#pragma unroll
      for (int k = 0; k < VPT; ++k)
        v[k] = buf_load<LP>(vec_rsrc(p.x + rn * p.ldx_bytes, nvec, k * THREADS), off);
    }
    r = rn;
  }
}

// Stream fallback: one workgroup per row, element-wise passes over memory.
template <int D>
__global__ __launch_bounds__(kStreamThreads) void ln_fwd_stream_kernel(LnFwdParams p) {
  __shared__ float red[2][kStreamThreads / kWave];
  const int64_t r = blockIdx.x;
  if (r >= p.M) return;
  const int tid = threadIdx.x;
  auto ld = [&](const char* base, int64_t j) -> float {
    if (D == kF32) return reinterpret_cast<const float*>(base)[j];
    return as_f32((uint32_t)reinterpret_cast<const uint16_t*>(base)[j] << 16);
  };
  const char* xr = p.x + r * p.ldx_bytes;
  char* yr = p.y + r * p.ldy_bytes;
  float s = 0.f;
  for (int64_t j = tid; j < p.N; j += kStreamThreads) s += ld(xr, j);
  const float mean = block_reduce<kStreamThreads>(s, OpAdd(), red[0]) / (float)p.N;
  float q = 0.f;
  for (int64_t j = tid; j < p.N; j += kStreamThreads) {
    const float c = ld(xr, j) - mean;
    q = __builtin_fmaf(c, c, q);
  }
  const float var = block_reduce<kStreamThreads>(q, OpAdd(), red[1]) / (float)p.N;
  const float rstd = 1.0f / sqrtf(var + p.eps);
  // y may be exactly x: every element is read by the thread that writes it, after the
  // reductions (whose barriers every read above precedes).
  for (int64_t j = tid; j < p.N; j += kStreamThreads) {
    const float val = __builtin_fmaf((ld(xr, j) - mean) * rstd, ld(p.w, j), ld(p.b, j));
    if (D == kF32) reinterpret_cast<float*>(yr)[j] = val;
    else reinterpret_cast<uint16_t*>(yr)[j] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
  }
  if (tid == 0) {
    p.mean[r] = mean;
    p.rstd[r] = rstd;
  }
}

// ============================================================================ backward, stage 1
// dx for rows g, g + G, ...; this workgroup's column sums of dy * xhat and dy go to partial
// row g (written once, at the end: every workgroup writes its row, zeros if it had no rows).
template <int D, int THREADS, int VPT, int LP>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void ln_bwd_kernel(LnBwdParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int NW = THREADS / kWave;
  __shared__ float2 red[2][NW];
  int buf = 0;
  const int tid = threadIdx.x;
  const int nvec = (int)(p.N / EPV);
  const uint32_t off = tid * 16u;
  const float inv_n = 1.0f / (float)p.N;

  u32x4 wv[VPT], vx[VPT], vd[VPT];
  float aw[VPT][EPV], ab[VPT][EPV];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    wv[k] = buf_load<kPolicyDefault>(vec_rsrc(p.w, nvec, k * THREADS), off);
#pragma unroll
    for (int e = 0; e < EPV; ++e) aw[k][e] = ab[k][e] = 0.f;
  }
  int64_t r = blockIdx.x;
  const int64_t G = gridDim.x;
  if (r < p.M) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      vx[k] = buf_load<LP>(vec_rsrc(p.x + r * p.ldx_bytes, nvec, k * THREADS), off);
      vd[k] = buf_load<LP>(vec_rsrc(p.dy + r * p.lddy_bytes, nvec, k * THREADS), off);
    }
  }
  while (r < p.M) {
    const int64_t rn = r + G;
    const float mu = p.mean[r], rs = p.rstd[r];
    // c1 = sum xhat * w * dy, c2 = sum w * dy (lanes past the row hold dy = 0: no terms)
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      u32x4 x = vx[k], d = vd[k], w = wv[k];
      pin_slot<D>(x);
      pin_slot<D>(d);
      pin_slot<D>(w);
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float g = elem<D>(w, e) * elem<D>(d, e);
        s1 = __builtin_fmaf((elem<D>(x, e) - mu) * rs, g, s1);
        s2 += g;
      }
    }
    const float2 c = block_sum2<THREADS>(s1, s2, red[buf]);
    buf ^= 1;
    const float c1 = c.x * inv_n, c2 = c.y * inv_n;
    char* dxrow = p.dx + r * p.lddx_bytes;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      u32x4 x = vx[k], d = vd[k], w = wv[k];
      pin_slot<D>(x);
      pin_slot<D>(d);
      pin_slot<D>(w);
      OutVec<D> o;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float xh = (elem<D>(x, e) - mu) * rs;
        const float dyv = elem<D>(d, e);
        const float g = elem<D>(w, e) * dyv;
        o.v[e] = (g - __builtin_fmaf(xh, c1, c2)) * rs;
        aw[k][e] = __builtin_fmaf(dyv, xh, aw[k][e]);
        ab[k][e] += dyv;
      }
      buf_store(vec_rsrc(dxrow, nvec, k * THREADS), off, o.bits());
    }
    // the next row's loads after all of this row's stores: interleaved with them, the
    // backward ran at 5.33-5.35 TB/s on 16384 x 8192 bf16, this way at 5.52-5.56
    if (rn < p.M) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        vx[k] = buf_load<LP>(vec_rsrc(p.x + rn * p.ldx_bytes, nvec, k * THREADS), off);
        vd[k] = buf_load<LP>(vec_rsrc(p.dy + rn * p.lddy_bytes, nvec, k * THREADS), off);
      }
    }
    r = rn;
  }
  // partial row g: fp32 columns, EPV per vector (range-checked: lanes past the row store nothing)
  float* pw = p.part_dw + blockIdx.x * p.pstride;
  float* pb = p.part_db + blockIdx.x * p.pstride;
  const Rsrc rpw = make_rsrc(pw, (uint32_t)p.N * 4u), rpb = make_rsrc(pb, (uint32_t)p.N * 4u);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t o = (uint32_t)((k * THREADS + tid) * EPV) * 4u;
#pragma unroll
    for (int h = 0; h < EPV; h += 4) {
      buf_store(rpw, o + h * 4u, (u32x4){as_u32(aw[k][h]), as_u32(aw[k][h + 1]),
                                         as_u32(aw[k][h + 2]), as_u32(aw[k][h + 3])});
      buf_store(rpb, o + h * 4u, (u32x4){as_u32(ab[k][h]), as_u32(ab[k][h + 1]),
                                         as_u32(ab[k][h + 2]), as_u32(ab[k][h + 3])});
    }
  }
}

// Stream fallback of stage 1: the same grid and partial rows, element-wise. Thread t of
// workgroup g owns columns t, t + T, ... of partial row g, so it alone updates them.
template <int D>
__global__ __launch_bounds__(kStreamThreads) void ln_bwd_stream_kernel(LnBwdParams p) {
  __shared__ float2 red[2][kStreamThreads / kWave];
  int buf = 0;
  const int tid = threadIdx.x;
  auto ld = [&](const char* base, int64_t j) -> float {
    if (D == kF32) return reinterpret_cast<const float*>(base)[j];
    return as_f32((uint32_t)reinterpret_cast<const uint16_t*>(base)[j] << 16);
  };
  float* pw = p.part_dw + blockIdx.x * p.pstride;
  float* pb = p.part_db + blockIdx.x * p.pstride;
  for (int64_t j = tid; j < p.N; j += kStreamThreads) pw[j] = pb[j] = 0.f;
  for (int64_t r = blockIdx.x; r < p.M; r += gridDim.x) {
    const char* xr = p.x + r * p.ldx_bytes;
    const char* dr = p.dy + r * p.lddy_bytes;
    char* dxr = p.dx + r * p.lddx_bytes;
    const float mu = p.mean[r], rs = p.rstd[r];
    float s1 = 0.f, s2 = 0.f;
    for (int64_t j = tid; j < p.N; j += kStreamThreads) {
      const float g = ld(p.w, j) * ld(dr, j);
      s1 = __builtin_fmaf((ld(xr, j) - mu) * rs, g, s1);
      s2 += g;
    }
    const float2 c = block_sum2<kStreamThreads>(s1, s2, red[buf]);
    buf ^= 1;
    const float c1 = c.x / (float)p.N, c2 = c.y / (float)p.N;
    // dx may be exactly x or dy: each element is read by the thread that writes it.
    for (int64_t j = tid; j < p.N; j += kStreamThreads) {
      const float xh = (ld(xr, j) - mu) * rs;
      const float dyv = ld(dr, j);
      const float val = (ld(p.w, j) * dyv - __builtin_fmaf(xh, c1, c2)) * rs;
      pw[j] = __builtin_fmaf(dyv, xh, pw[j]);
      pb[j] += dyv;
      if (D == kF32) reinterpret_cast<float*>(dxr)[j] = val;
      else reinterpret_cast<uint16_t*>(dxr)[j] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
    }
  }
}

// ============================================================================ backward, stage 2
// dw_j = sum_g part_dw[g][j], db_j likewise, g in order. A workgroup of kLnReduceThreads
// covers 64 columns: wave w sums g = w, w + W, ... for its lane's column, then the W
// partial sums are added in wave order.
template <int D>
__global__ __launch_bounds__(kLnReduceThreads) void ln_dwdb_kernel(LnReduceParams p) {
  constexpr int W = kLnReduceThreads / kWave;
  __shared__ float sw[W][kWave], sb[W][kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  static_assert(kLnReduceCols == kWave, "one column per lane");
  const int64_t j = (int64_t)blockIdx.x * kLnReduceCols + lane;
  float aw = 0.f, ab = 0.f;
  if (j < p.N) {
    for (int g = wave; g < p.G; g += W) {
      aw += p.part_dw[(int64_t)g * p.pstride + j];
      ab += p.part_db[(int64_t)g * p.pstride + j];
    }
  }
  sw[wave][lane] = aw;
  sb[wave][lane] = ab;
  __syncthreads();
  if (wave == 0 && j < p.N) {
    float tw = sw[0][lane], tb = sb[0][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) {
      tw += sw[w][lane];
      tb += sb[w][lane];
    }
    if (D == kF32) {
      reinterpret_cast<float*>(p.dw)[j] = tw;
      reinterpret_cast<float*>(p.db)[j] = tb;
    } else {
      reinterpret_cast<uint16_t*>(p.dw)[j] = (uint16_t)(pack_bf16x2(tw, 0.f) & 0xFFFFu);
      reinterpret_cast<uint16_t*>(p.db)[j] = (uint16_t)(pack_bf16x2(tb, 0.f) & 0xFFFFu);
    }
  }
}

// ============================================================================ lookup tables
#define XR_SHAPES_LN_FWD(X, D) \
  X(D, 64, 1) X(D, 64, 2) X(D, 64, 4) X(D, 128, 4) X(D, 256, 4) X(D, 512, 4) X(D, 1024, 4)
#define XR_SHAPES_LN_BWD(X, D) \
  X(D, 64, 1) X(D, 64, 2) X(D, 128, 2) X(D, 256, 2) X(D, 512, 2) X(D, 1024, 2) X(D, 1024, 4)
#define XR_CASE_LNF(D, T, V)                                                                   \
  if (s.threads == T && s.vpt == V)                                                              \
    return lp ? reinterpret_cast<const void*>(&ln_fwd_kernel<D, T, V, kPolicyNT>)                \
              : reinterpret_cast<const void*>(&ln_fwd_kernel<D, T, V, kPolicyDefault>);
#define XR_CASE_LNB(D, T, V)                                                                   \
  if (s.threads == T && s.vpt == V)                                                              \
    return lp ? reinterpret_cast<const void*>(&ln_bwd_kernel<D, T, V, kPolicyNT>)                \
              : reinterpret_cast<const void*>(&ln_bwd_kernel<D, T, V, kPolicyDefault>);

const void* ln_fwd_kernel_ptr(int dtype, Shape s, bool lp) {
  if (dtype == kF32) { XR_SHAPES_LN_FWD(XR_CASE_LNF, kF32) }
  if (dtype == kBF16) { XR_SHAPES_LN_FWD(XR_CASE_LNF, kBF16) }
  return nullptr;
}
// bf16 rows of more than 2048 vectors (16384 elements) are left to the stream kernel: four
// vectors of x, dy and w plus 64 fp32 column sums per thread do not fit 128 registers.
#define XR_SHAPES_LN_BWD_BF16(X, D) \
  X(D, 64, 1) X(D, 64, 2) X(D, 128, 2) X(D, 256, 2) X(D, 512, 2) X(D, 1024, 2)
const void* ln_bwd_kernel_ptr(int dtype, Shape s, bool lp) {
  if (dtype == kF32) { XR_SHAPES_LN_BWD(XR_CASE_LNB, kF32) }
  if (dtype == kBF16) { XR_SHAPES_LN_BWD_BF16(XR_CASE_LNB, kBF16) }
  return nullptr;
}
const void* ln_fwd_stream_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&ln_fwd_stream_kernel<kF32>)
                       : reinterpret_cast<const void*>(&ln_fwd_stream_kernel<kBF16>);
}
const void* ln_bwd_stream_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&ln_bwd_stream_kernel<kF32>)
                       : reinterpret_cast<const void*>(&ln_bwd_stream_kernel<kBF16>);
}
const void* ln_dwdb_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&ln_dwdb_kernel<kF32>)
                       : reinterpret_cast<const void*>(&ln_dwdb_kernel<kBF16>);
}

}  // namespace xr
