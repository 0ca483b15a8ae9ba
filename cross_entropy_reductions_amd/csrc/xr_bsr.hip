// xr_bsr.hip -- block-sparse softmax backward through a look-up table, for gfx950.
//
// What is computed (page "python sum function examples", Triton kernel _backward): the
// matrices hold Z batches of BLOCK x BLOCK blocks (row-major, block b of batch z at element
// z * stride_z + b * BLOCK^2). Row i of block-row r is the concatenation of row i of every
// block the table lists for r; along that row
//   dx <- y * (dx - sum(y * dx)) * scale
// with dx holding the incoming gradient on entry (overwritten, as on the page). Table
// layout, as that kernel reads it: words (size, offset) at 2 r, then the k-th listed block's
// index at word offset + 4 k.
//
// On MI355X: a workgroup takes R rows of one block-row (one batch), TPR = BLOCK / (elements
// per 16-byte vector) consecutive lanes per row, one vector of each listed block per lane:
// a wave reads 64 / TPR consecutive rows of a block, i.e. one contiguous span of it. Up to
// kBsrResident blocks per row stay in registers between the dot product and the write (one
// non-temporal read of y and dx, one write); longer rows are read twice. The dot product is a butterfly
// over the row's TPR lanes (the same bits on every lane, no LDS, no barrier). The table is
// read with scalar loads (it is uniform across the workgroup and read-only for the kernel,
// which the host checks: it may not overlap dx), every index bounded by the table length;
// data accesses go through buffer resources sized to one batch's blocks, so a bad block
// index reads zeros and writes nothing instead of faulting.
#include "xr_rows.h"

namespace xr {

// The table through the constant address space: uniform loads become scalar loads, which
// complete apart from the vector loads of the data (a wait for a table entry does not wait
// for data loads issued before it).
typedef const __attribute__((address_space(4))) int32_t ConstI32;

template <int D>
__global__ __launch_bounds__(kBsrThreads) __attribute__((amdgpu_waves_per_eu(4))) void bsr_softmax_bwd_kernel(BsrParams p) {
  constexpr int EPV = Elt<D>::kPerVec;
  constexpr int NB = kBsrResident;
  const int tid = threadIdx.x;
  const int block = p.block;
  const int tpr = block / EPV;                 // lanes per row segment (a power of two <= 64)
  const int R = p.rows_per_wg;                 // rows of the block-row per workgroup
  const int64_t b = blockIdx.x;
  const int64_t zr = b / p.row_chunks;
  const int rc = (int)(b - zr * p.row_chunks);
  const int64_t z = zr / p.n_brows;
  const int64_t br = zr - z * p.n_brows;
  const int i = rc * R + tid / tpr;            // row within the block
  const int lane = tid % tpr;
  const bool active = tid < R * tpr && i < block;

  // words 2 br and 2 br + 1 lie inside the table: the host checks lut_len >= 2 n_brows
  ConstI32* lut = (ConstI32*)p.lut;
  const int32_t size = lut[2 * br];
  const int32_t offset = lut[2 * br + 1];
  // listed blocks, bounded by the entries the table actually holds after `offset`
  const int64_t avail = offset >= 0 && offset <= p.lut_len ? (p.lut_len - offset) / 4 : 0;
  const int n = size > 0 ? (int)(size < avail ? size : avail) : 0;
  const Rsrc ry = make_rsrc(p.y + z * p.ldy_bytes, p.batch_bytes);
  const Rsrc rd = make_rsrc(p.dx + z * p.lddx_bytes, p.batch_bytes);
  const uint32_t in_block = (uint32_t)((i * block + lane * EPV) * Elt<D>::kBytes);
  const uint32_t block_bytes = (uint32_t)(block * block * Elt<D>::kBytes);

  // Byte offsets of this lane's vector in listed blocks k0 .. k0 + NB - 1 (kOffNone: no
  // access; n >= 1). The table entries are read without branches (indices clamped to the
  // last listed block, which lies inside the table) so the scalar loads issue together.
  auto vec_offs = [&](int k0, uint32_t (&vo)[NB]) {
    int32_t bid[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) bid[q] = lut[offset + 4 * min(k0 + q, n - 1)];
#pragma unroll
    for (int q = 0; q < NB; ++q)
      vo[q] = (!active || k0 + q >= n || bid[q] < 0 || bid[q] >= p.n_blocks)
                  ? kOffNone
                  : (uint32_t)bid[q] * block_bytes + in_block;
  };

  auto dot = [&](u32x4 a, u32x4 c, float acc) {
    pin_slot<D>(a);
    pin_slot<D>(c);
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc = __builtin_fmaf(elem<D>(a, e), elem<D>(c, e), acc);
    return acc;
  };
  auto out = [&](u32x4 a, u32x4 c, float s) {
    pin_slot<D>(a);
    pin_slot<D>(c);
    OutVec<D> o;
#pragma unroll
    for (int e = 0; e < EPV; ++e) o.v[e] = elem<D>(a, e) * (elem<D>(c, e) - s) * p.scale;
    return o.bits();
  };
  // the row's dot product: butterfly over its tpr lanes (lanes of other rows never mix)
  auto row_sum = [&](float s) {
    for (int m = 1; m < tpr; m <<= 1) s += __shfl_xor(s, m, kWave);
    return s;
  };

  if (n == 0) return;  // nothing listed: nothing to read or write
  if (n <= NB) {
    // every listed block's vector stays in registers: one read of y and dx, one write. The
    // loads are non-temporal (nothing reads these lines again; measured 4.96-4.98 TB/s with
    // the default policy, 5.61-5.62 non-temporal, on 32 causal 4096 x 4096 maps of 64-blocks)
    u32x4 vy[NB], vd[NB];
    uint32_t vo[NB];
    vec_offs(0, vo);
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      vy[q] = buf_load<kPolicyNT>(ry, vo[q]);
      vd[q] = buf_load<kPolicyNT>(rd, vo[q]);
    }
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NB; ++q) s = dot(vy[q], vd[q], s);
    s = row_sum(s);
#pragma unroll
    for (int q = 0; q < NB; ++q) buf_store(rd, vo[q], out(vy[q], vd[q], s));
  } else {
    // longer rows: the dot product over every listed block (default policy: the lines are
    // read again), then a second, non-temporal read to write, NB blocks at a time
    float s = 0.f;
    uint32_t vo[NB];
    for (int k0 = 0; k0 < n; k0 += NB) {
      vec_offs(k0, vo);
#pragma unroll
      for (int q = 0; q < NB; ++q)
        s = dot(buf_load<kPolicyDefault>(ry, vo[q]), buf_load<kPolicyDefault>(rd, vo[q]), s);
    }
    s = row_sum(s);
    for (int k0 = 0; k0 < n; k0 += NB) {
      vec_offs(k0, vo);
#pragma unroll
      for (int q = 0; q < NB; ++q)
        buf_store(rd, vo[q], out(buf_load<kPolicyNT>(ry, vo[q]), buf_load<kPolicyNT>(rd, vo[q]), s));
    }
  }
}

const void* bsr_softmax_bwd_kernel_ptr(int dtype) {
  return dtype == kF32 ? reinterpret_cast<const void*>(&bsr_softmax_bwd_kernel<kF32>)
                       : reinterpret_cast<const void*>(&bsr_softmax_bwd_kernel<kBF16>);
}

}  // namespace xr
