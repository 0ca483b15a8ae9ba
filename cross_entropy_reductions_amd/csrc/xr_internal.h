// xr_internal.h -- launch plans and kernel launchers shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xr {

// Byte offsets inside the cross-entropy workspace.
constexpr size_t kWsCounts = 0;      // int32[4]: n_non_ignore, n_bad_target, error flags, spare
constexpr size_t kWsPartials = 256;  // uint64[M * S]: (m, d) pairs of split rows

// Error flags (workspace int32 [2], copied to counts[2]).
constexpr int32_t kFlagExchangeTimeout = 1;

// Sentinel marking an unpublished (m, d) pair of a split row.
constexpr uint64_t kPartialEmpty = ~0ull;

enum Path : int { kPathAuto = 0, kPathResident = 1, kPathSplit = 2, kPathStream = 3 };

// Loss reductions (the values of xr_reduction_t).
enum Reduction : int { kReduceMean = 0, kReduceSum = 1, kReduceNone = 2 };

struct XentParams {
  char* logits;           // row 0 of the logits (overwritten by the gradient)
  int64_t ld_bytes;       // row pitch in bytes
  const int64_t* target;  // [M]
  int64_t M, V, ignore_index;
  float* row_loss;        // [M]
  const int32_t* ws_counts;  // workspace counts (n is read from [0])
  int32_t* ws_flags;         // workspace error flags
  uint64_t* partials;        // [M * S] when S > 1
  int64_t chunk_vecs;     // 16-byte vectors per chunk (the whole row when S == 1)
  int S;                  // workgroups per row
  int groups;             // row groups in the grid; grid = groups * S
  int reduction;          // Reduction: the mean divides the gradient by n
  const float* gscale;    // upstream gradient, row i at gscale[i * gstride]; nullptr = 1
  int64_t gstride;
  int group_rows;         // split rows written back in groups of kWriteGroupRows rows (or 1: none)
};

// Rows x[i, 0:V) scaled in place by scale[i * sstride]; chunk_vecs 16-byte vectors per
// workgroup, `chunks` workgroups per row.
struct ElementMulParams {
  char* x;
  int64_t ld_bytes;
  int64_t M, V;
  const float* scale;
  int64_t sstride;
  int64_t chunk_vecs;
  int64_t chunks;
};

struct SoftmaxFwdParams {
  const char* x;
  int64_t ldx_bytes;
  char* y;
  int64_t ldy_bytes;
  int64_t M, N;
  const int64_t* idx;  // negative log-softmax only: the index gathered into loss[] per row
  float* loss;
  // split rows (negative log-softmax with a workspace): S workgroups per row, chunk_vecs
  // 16-byte vectors each, exchanging (m, d) through partials[M * S]; flags as for xent
  int S;
  int64_t chunk_vecs;
  uint64_t* partials;
  int32_t* flags;
  int group_rows;  // split rows written back in groups of kWriteGroupRows rows (or 1: none)
  int load_prio = 0;  // whole rows: raise the wave priority while issuing the row's loads
};

// Layer norm forward: y = (x - mean) rstd w + b per row; mean and rstd saved.
struct LnFwdParams {
  const char* x;
  int64_t ldx_bytes;
  char* y;
  int64_t ldy_bytes;
  const char* w;
  const char* b;
  float* mean;
  float* rstd;
  int64_t M, N;
  float eps;
};

// Layer norm backward, stage 1: dx, and per-workgroup partial column sums of dy * xhat
// (part_dw) and dy (part_db), one row of pstride floats per workgroup of the grid.
struct LnBwdParams {
  const char* dy;
  int64_t lddy_bytes;
  const char* x;
  int64_t ldx_bytes;
  char* dx;
  int64_t lddx_bytes;
  const char* w;
  const float* mean;
  const float* rstd;
  float* part_dw;
  float* part_db;
  int64_t pstride;
  int64_t M, N;
};

// Layer norm backward, stage 2: dw / db = the sums of the G partial rows, in row order.
struct LnReduceParams {
  const float* part_dw;
  const float* part_db;
  int64_t pstride;
  int G;
  char* dw;
  char* db;
  int64_t N;
};

// Block-sparse softmax backward (see xr_bsr.hip): workgroup b handles rows
// [rc * rows_per_wg, ...) of block-row br of batch z, b = (z * n_brows + br) * row_chunks + rc.
struct BsrParams {
  const char* y;
  int64_t ldy_bytes;   // batch stride of y
  char* dx;
  int64_t lddx_bytes;  // batch stride of dx
  const int32_t* lut;
  int64_t lut_len;     // words
  int64_t n_brows;
  int32_t n_blocks;    // blocks stored per batch
  uint32_t batch_bytes;  // n_blocks * block^2 * element size (< 2^31)
  int32_t block;
  int32_t rows_per_wg;
  int32_t row_chunks;  // ceil(block / rows_per_wg)
  float scale;
};

// Memory-ceiling probe (xr_probe_rows): workgroup b moves chunk b % S of row b / S from in0
// (and in1) to out with the row kernels' access pattern and none of their arithmetic.
struct ProbeParams {
  const char* in0;
  const char* in1;  // nullptr: one input
  int64_t ldin_bytes;
  char* out;
  int64_t ldout_bytes;
  int64_t M, N;
  const int64_t* target;  // rows whose target is ignore_index are not read (zeros written)
  int64_t ignore_index;
  int S;
  int64_t chunk_vecs;
};

// The ceiling's plain copy (xr_probe_copy): nvec 16-byte vectors from in to out, or
// in ^ in1 when in1 is not null.
struct CopyParams {
  const char* in;
  const char* in1;
  char* out;
  int64_t nvec;
};

// Operations of the row kernels (also the `op` argument of xr_plan).
enum Op : int { kOpSoftmaxFwd = 0, kOpSoftmaxBwd = 1, kOpXent = 2, kOpNllFwd = 3 };

struct SoftmaxBwdParams {
  const char* y;
  int64_t ldy_bytes;
  const char* dy;
  int64_t lddy_bytes;
  char* dx;
  int64_t lddx_bytes;
  int64_t M, N;
  // split rows (with a workspace): S workgroups per row exchanging partial dot products
  int S;
  int64_t chunk_vecs;
  uint64_t* partials;
  int32_t* flags;
  int group_rows;  // split rows written back in groups of kWriteGroupRows rows (or 1: none)
  int load_prio = 0;  // whole rows: raise the wave priority while issuing the row's loads
};

// One kernel configuration: workgroup size and 16-byte vectors per thread.
struct Shape {
  int threads;
  int vpt;
};

// Kernel lookup (nullptr when the (dtype, shape) pair is not instantiated); nt_loads selects
// the instantiation whose row loads carry the non-temporal hint.
const void* xent_rows_kernel_ptr(int dtype, Shape s, bool nt_loads);
const void* softmax_fwd_kernel_ptr(int dtype, Shape s, bool nt_loads);
const void* nll_fwd_kernel_ptr(int dtype, Shape s, bool nt_loads);
const void* nll_split_kernel_ptr(int dtype, Shape s, bool nt_loads);
const void* softmax_fwd_split_kernel_ptr(int dtype, Shape s, bool nt_loads);
const void* softmax_bwd_split_kernel_ptr(int dtype, Shape s, bool nt_loads);
// one_row: the form for a grid of at least M workgroups (one row each, no loop).
const void* softmax_bwd_kernel_ptr(int dtype, Shape s, bool nt_loads, bool one_row = false);
const void* xent_stream_kernel_ptr(int dtype);
const void* softmax_fwd_stream_kernel_ptr(int dtype);
const void* nll_fwd_stream_kernel_ptr(int dtype);
const void* softmax_bwd_stream_kernel_ptr(int dtype);
const void* xent_scan_kernel_ptr();
const void* xent_mean_kernel_ptr();
const void* element_mul_kernel_ptr(int dtype, bool nt_loads);

const void* ln_fwd_kernel_ptr(int dtype, Shape s, bool nt_loads);
const void* ln_bwd_kernel_ptr(int dtype, Shape s, bool nt_loads);
const void* ln_fwd_stream_kernel_ptr(int dtype);
const void* ln_bwd_stream_kernel_ptr(int dtype);
const void* ln_dwdb_kernel_ptr(int dtype);

const void* bsr_softmax_bwd_kernel_ptr(int dtype);
const void* probe_rows_kernel_ptr(int dtype, Shape s, int inputs);
// The ceiling's plain copy (xr_probe_copy): 256, 512 or 1024 threads per workgroup, one or
// two inputs, or none (in place: the output read and written back).
const void* probe_copy_kernel_ptr(int threads, int inputs);
constexpr int kCopyUnroll = 4;  // 16-byte vectors in flight per thread of the plain copy
// Block-sparse backward: workgroup size, and listed blocks per row held in registers.
#ifndef XR_BSR_THREADS
#define XR_BSR_THREADS 256
#endif
#ifndef XR_BSR_RESIDENT
#define XR_BSR_RESIDENT 12
#endif
constexpr int kWriteGroupRows = 8;  // split-row write groups (rows, a power of two; see the plan)
constexpr int kBsrThreads = XR_BSR_THREADS;
constexpr int kBsrResident = XR_BSR_RESIDENT;

// Workgroup size of the stream, scan and mean kernels.
constexpr int kStreamThreads = 256;
constexpr int kScanThreads = 1024;
// element_mul: workgroup size and 16-byte vectors per thread.
#ifndef XR_MUL_THREADS
#define XR_MUL_THREADS 1024
#endif
#ifndef XR_MUL_VPT
#define XR_MUL_VPT 8
#endif
constexpr int kMulThreads = XR_MUL_THREADS;
constexpr int kMulVpt = XR_MUL_VPT;

// Shapes available to the row-resident kernels, smallest capacity first.
constexpr int kNumFwdShapes = 10;
extern const Shape kFwdShapes[kNumFwdShapes];  // xent and softmax forward
constexpr int kNumBwdShapes = 6;
extern const Shape kBwdShapes[kNumBwdShapes];  // softmax backward (two row operands)
constexpr int kNumLnFwdShapes = 7;
extern const Shape kLnFwdShapes[kNumLnFwdShapes];  // layer norm forward (w, b resident too)
constexpr int kNumLnBwdShapes = 7;
extern const Shape kLnBwdShapes[kNumLnBwdShapes];  // layer norm backward (fp32 column sums too)
// Layer norm stage-2 reduction: workgroup size, and columns per workgroup (one per lane).
constexpr int kLnReduceThreads = 1024;
constexpr int kLnReduceCols = 64;

}  // namespace xr
