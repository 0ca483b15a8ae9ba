/*
 * xr.h -- C ABI of libxr: numerically stable row softmax, softmax backward and fused
 * cross-entropy (loss + in-place gradient) for AMD Instinct MI355X (gfx950).
 *
 * Conventions for every entry point
 *   - Pointers named for tensors are DEVICE pointers (HIP device memory of the current
 *     device). Host pointers are marked as such.
 *   - Matrices are row-major: row i of a matrix starts at element i * ld of its pointer
 *     ("row stride", counted in ELEMENTS, ld >= number of columns); columns are unit stride.
 *     Columns [N, ld) of a row are padding: they are never read and never written.
 *   - dtype selects the floating type of every floating tensor argument of the call except
 *     row_loss / mean_loss, which are always fp32. bf16 values are rounded to nearest-even
 *     when stored. All arithmetic is fp32 whatever the storage type.
 *   - The softmax-family results depend on the differences x - max of a row, not on its
 *     magnitude: rows of large finite values (a row filled with a large negative mask value
 *     gives the uniform softmax, -log p = log N and the loss log N) keep the accuracy of
 *     ordinary rows, up to what fp32 holds of the differences themselves.
 *   - stream is a hipStream_t (NULL = the legacy default stream). Every entry point only
 *     enqueues work on it: nothing is synchronised, nothing is allocated or freed, and no
 *     device memory is read or written by the host.
 *   - Arguments, and the launch limits of the sizes given, are validated before anything is
 *     enqueued; on an error nothing is enqueued and the status says what is wrong. No C++
 *     exception crosses this ABI.
 *   - No operand may span 2^48 bytes or more from its first to past its last element (far
 *     beyond any device's memory): such sizes and strides return XR_ERR_SHAPE before any
 *     arithmetic on them, and the workspace queries return 0 for them.
 *   - Results are deterministic: the same inputs give bit-identical outputs on every run.
 *   - The library keeps no state across calls except a per-device cache of device
 *     properties, the process-wide overrides of xr_set_option() and the profiling events
 *     of xr_set_profile_events(). Workspaces are the caller's and hold nothing between
 *     calls.
 */
#ifndef XR_H_
#define XR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum xr_dtype {
  XR_F32 = 0,  /* IEEE binary32 */
  XR_BF16 = 1  /* bfloat16 (upper half of a binary32) */
} xr_dtype_t;

typedef enum xr_status {
  XR_OK = 0,
  XR_ERR_NULL = 1,      /* a required pointer is NULL */
  XR_ERR_SHAPE = 2,     /* M < 0, N (or V) < 1, or a size beyond what the library supports */
  XR_ERR_STRIDE = 3,    /* a row stride is smaller than the number of columns */
  XR_ERR_DTYPE = 4,     /* unknown dtype */
  XR_ERR_ALIAS = 5,     /* an output overlaps an input without being exactly the same matrix */
  XR_ERR_WORKSPACE = 6, /* a required workspace is NULL or smaller than its *_bytes() query */
  XR_ERR_ALIGN = 7,     /* a tensor pointer is not aligned to its element size */
  XR_ERR_DEVICE = 8,    /* no usable HIP device, or a device query failed */
  XR_ERR_LAUNCH = 9,    /* a kernel launch failed (the HIP error is reported by HIP) */
  XR_ERR_OPTION = 10,   /* unknown option or value in xr_set_option() */
  XR_ERR_VALUE = 11,    /* an argument has an invalid value (reduction, negative stride) */
  XR_ERR_TOO_LARGE = 12 /* the sizes need more scratch than xr_xent_fwd_bwd_noalloc() has */
} xr_status_t;

/*
 * Softmax forward, one row at a time:
 *   y[i, j] = exp(x[i, j] - m_i) / d_i,  m_i = max_j x[i, j],  d_i = sum_j exp(x[i, j] - m_i)
 * The safe softmax of the Triton fused-softmax kernels `softmax_kernel` and `_softmax` on
 * the page "python sum function examples" (subtract the row max, exponentiate, divide by
 * the row sum; masked lanes are -inf, so -inf inputs get probability 0).
 *   y, ld_y   output [M, N] of dtype; may be exactly x (y == x and ld_y == ld_x, in place)
 *   x, ld_x   input  [M, N] of dtype
 *   M >= 0 (M == 0 enqueues nothing), N >= 1
 * A row that is entirely -inf, or holds NaN or +inf, gives NaN outputs.
 */
xr_status_t xr_softmax_fwd(void* y, int64_t ld_y, const void* x, int64_t ld_x, int64_t M,
                           int64_t N, xr_dtype_t dtype, void* stream);

/*
 * xr_softmax_fwd / xr_softmax_bwd with a workspace: the same results, but long rows (and
 * rows too few to give every compute unit work) are split over several workgroups that
 * exchange their partial statistics through the workspace: the (max, sum) pairs of the
 * online-softmax combine for the forward (the pairs the cross-entropy's split rows
 * exchange), the partial dot products sum(y * dy) for the backward, each added in chunk
 * order, so the results do not depend on timing. Rows of a few large chunks are also
 * written back in groups of adjacent rows (a chunk holds its stores until its neighbours'
 * chunks have published: a bounded wait that never changes a result).
 * A chunk's wait for its row's partners is bounded too: should it expire, the row's
 * outputs are NaN and the workspace's status word gets bit 0 (xr_workspace_status()).
 * Every call given a workspace leaves that word defined (0 when nothing timed out).
 *   workspace  device scratch of at least xr_softmax_workspace_bytes(M, N, dtype) bytes
 *              (covers both directions), 8-byte aligned, or NULL (rows handled whole, as
 *              without _ex); no initialisation needed; scratch between calls; it must not
 *              overlap any matrix of the call (XR_ERR_ALIAS)
 *   workspace_bytes  its size; too small for the plan the call takes: XR_ERR_WORKSPACE
 * Calls that share a workspace must not run concurrently.
 */
size_t xr_softmax_workspace_bytes(int64_t M, int64_t N, xr_dtype_t dtype);
xr_status_t xr_softmax_fwd_ex(void* y, int64_t ld_y, const void* x, int64_t ld_x, int64_t M,
                              int64_t N, xr_dtype_t dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Softmax backward, one row at a time:
 *   dx[i, j] = y[i, j] * (dy[i, j] - s_i),  s_i = sum_k y[i, k] * dy[i, k]
 * The fused softmax backward of the Triton kernel `_backward` on the page "python sum
 * function examples", with its block-sparse scale taken as 1 and dense rows.
 *   dx, ld_dx  output [M, N] of dtype; may be exactly y or exactly dy (in place)
 *   y, ld_y    the softmax output [M, N];  dy, ld_dy  the upstream gradient [M, N]
 *   M >= 0 (M == 0 enqueues nothing), N >= 1
 */
xr_status_t xr_softmax_bwd(void* dx, int64_t ld_dx, const void* y, int64_t ld_y, const void* dy,
                           int64_t ld_dy, int64_t M, int64_t N, xr_dtype_t dtype, void* stream);
xr_status_t xr_softmax_bwd_ex(void* dx, int64_t ld_dx, const void* y, int64_t ld_y,
                              const void* dy, int64_t ld_dy, int64_t M, int64_t N,
                              xr_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Block-sparse softmax backward through a look-up table (the Triton kernel `_backward` on
 * the page "python sum function examples"). y (the softmax output) and dx (the incoming
 * gradient on entry, the result on return, as on the page) hold Z batches of n_blocks
 * blocks of block x block elements, row-major within a block, block b of batch z at element
 * z * stride_z + b * block^2 (stride_zy for y, stride_zdx for dx). Row i of block-row r is
 * row i of every block the table lists for r, in table order; along it
 *   dx <- y * (dx - sum(y * dx)) * scale          (fp32 arithmetic, one rounding to dtype)
 * Table (int32, device, lut_len words), as that kernel reads it: words 2 r and 2 r + 1 are
 * the number of listed blocks and the word offset of the list for block-row r; the k-th
 * listed block's index is word offset + 4 k (the other three words of an entry are not
 * read). A list that runs past the table is cut at its end; a block index outside
 * [0, n_blocks) reads as zeros and is not written. A block listed for several block-rows
 * gives unspecified results (as on the page).
 *   block: a power of two, 8..512 for bf16, 4..256 for fp32;  Z, n_brows, n_blocks >= 0
 *   y, dx 16-byte aligned, stride_z * element size a multiple of 16; one batch's blocks
 *   under 2 GiB; y may be exactly dx, otherwise no overlap (nor with the table).
 */
xr_status_t xr_bsr_softmax_bwd(const void* y, int64_t stride_zy, void* dx, int64_t stride_zdx,
                               int64_t Z, const int32_t* lut, int64_t lut_len, int64_t n_brows,
                               int64_t n_blocks, int32_t block, float scale, xr_dtype_t dtype,
                               void* stream);

/*
 * Negative log-softmax forward with the loss gathered at one index per row (the Triton
 * kernel `_forward` on the page "python sum function examples"):
 *   out[i, j] = log d_i - (x[i, j] - m_i)   (= -log softmax(x[i, :])_j; +inf where x is -inf)
 *   loss[i]   = out[i, idx[i]] as stored, i.e. rounded to dtype (the page reads the loss back
 *               from the output), widened to fp32; NaN when idx[i] lies outside [0, N)
 *   out, ld_out  output [M, N] of dtype; may be exactly x (in place)
 *   x, ld_x      input [M, N] of dtype
 *   idx          int64 [M], device;  loss  fp32 [M], device
 *   workspace    device scratch of at least xr_nll_fwd_workspace_bytes(M, N, dtype) bytes, or
 *                NULL: with it, long rows are split over several workgroups that exchange
 *                their (max, sum) pairs through it, as the cross-entropy's split rows do
 *                (no initialisation needed; scratch between calls; its status word is
 *                reported by xr_workspace_status() as for xr_softmax_fwd_ex); without it
 *                every row is handled whole
 *   M >= 0 (M == 0 enqueues nothing), N >= 1
 * idx, loss and the workspace must not overlap the matrices or each other (XR_ERR_ALIAS).
 */
size_t xr_nll_fwd_workspace_bytes(int64_t M, int64_t N, xr_dtype_t dtype);
xr_status_t xr_nll_fwd(void* out, int64_t ld_out, const void* x, int64_t ld_x,
                       const int64_t* idx, float* loss, int64_t M, int64_t N, xr_dtype_t dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Layer norm forward (the Triton LayerNorm tutorial page, translated; its code is cut off,
 * so the definition follows its prose and the paper it cites, Ba, Kiros & Hinton 2016):
 *   mean[i] = (1/N) sum_j x[i, j],  var_i = (1/N) sum_j (x[i, j] - mean[i])^2,
 *   rstd[i] = 1 / sqrt(var_i + eps),  y[i, j] = (x[i, j] - mean[i]) * rstd[i] * w[j] + b[j]
 * computed in fp32 (two passes over the row held in registers), y rounded once to dtype.
 *   y, ld_y        output [M, N] of dtype; may be exactly x (in place)
 *   x, ld_x        input [M, N] of dtype;  w, b  [N] of dtype, device
 *   mean, rstd     fp32 [M], device: saved for xr_layernorm_bwd()
 *   eps >= 0 and finite, else XR_ERR_VALUE;  M >= 0 (M == 0 enqueues nothing), N >= 1
 * Fastest when every row, w and b start on 16-byte boundaries and N * element size is a
 * multiple of 16 (contiguous tensors with N a multiple of 8); other layouts are accepted
 * and run element-wise. y must not overlap w, b, mean or rstd (XR_ERR_ALIAS).
 */
xr_status_t xr_layernorm_fwd(void* y, int64_t ld_y, const void* x, int64_t ld_x, const void* w,
                             const void* b, float* mean, float* rstd, int64_t M, int64_t N,
                             float eps, xr_dtype_t dtype, void* stream);

/*
 * Bytes of device workspace xr_layernorm_bwd() needs for these sizes on the current device
 * (host query; 0 if the sizes are invalid): the partial dw / db rows of the first stage.
 */
size_t xr_layernorm_bwd_workspace_bytes(int64_t M, int64_t N, xr_dtype_t dtype);

/*
 * Layer norm backward: the derivative of xr_layernorm_fwd()'s y, contracted with dy.
 * With xhat = (x - mean) * rstd and g = w * dy (per row i, column j):
 *   dx[i, j] = rstd[i] * (g[i, j] - (xhat[i, j] * c1_i + c2_i)),
 *       c1_i = (1/N) sum_j xhat[i, j] g[i, j],  c2_i = (1/N) sum_j g[i, j]
 *   dw[j] = sum_i dy[i, j] xhat[i, j],  db[j] = sum_i dy[i, j]
 * The column sums run in two stages, as on the page: a persistent grid of G workgroups each
 * sums its rows' columns into its own partial row of the workspace (no locks), then a
 * second kernel sums the G partial rows of each column in a fixed order (deterministic for
 * a given device and plan). All sums in fp32; dx, dw and db rounded once to dtype.
 *   dx, ld_dx          output [M, N] of dtype; may be exactly dy or exactly x
 *   dy, x              [M, N] of dtype (row strides ld_dy, ld_x);  w  [N] of dtype
 *   mean, rstd         fp32 [M] from xr_layernorm_fwd()
 *   dw, db             outputs [N] of dtype (M == 0 writes zeros)
 *   workspace          device, 16-byte aligned, >= xr_layernorm_bwd_workspace_bytes(M, N, dtype)
 * Outputs must not overlap each other, w, mean or rstd (XR_ERR_ALIAS).
 */
xr_status_t xr_layernorm_bwd(void* dx, int64_t ld_dx, const void* dy, int64_t ld_dy,
                             const void* x, int64_t ld_x, const void* w, const float* mean,
                             const float* rstd, void* dw, void* db, int64_t M, int64_t N,
                             xr_dtype_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Bytes of device workspace xr_xent_fwd_bwd() needs for these sizes on the current device
 * (host query; 0 if the sizes are invalid), with room for the row losses of a call that
 * passes no row_loss. The caller owns the workspace; its contents need no initialisation
 * and are scratch between calls.
 */
size_t xr_xent_workspace_bytes(int64_t M, int64_t V, xr_dtype_t dtype);

/*
 * Fused cross-entropy loss and gradient (hard labels, mean over non-ignored rows), from
 * Liger-Kernel `cross_entropy.py`: `liger_cross_entropy_kernel` steps 1-6 and
 * `LigerCrossEntropyFunction.forward`. With n = #{i : target[i] != ignore_index}:
 *   row_loss[i] = m_i + log d_i - logits[i, t_i]               (0 for ignored rows)
 *   logits[i, j] <- (softmax(logits[i, :])_j - [j == t_i]) / n   (0 for ignored rows)
 *   *mean_loss   = (sum_i row_loss[i]) / n                       (NaN when n == 0)
 *   logits, ld     [M, V] of dtype, overwritten IN PLACE by the gradient; columns [V, ld)
 *                  are never touched
 *   target         int64 [M], device; ignore_index is compared first, so an ignore_index
 *                  inside [0, V) still ignores its rows
 *   row_loss       fp32 [M], device, or NULL (the row losses are then kept in the workspace)
 *   mean_loss      fp32 [1], device, required
 *   counts         int32 [3], device, or NULL: counts[0] = n, counts[1] = targets that are
 *                  neither ignore_index nor inside [0, V) (their rows get zero gradient and
 *                  zero loss, but still count in n), counts[2] = error flags (0 = none;
 *                  bit 0: a split-row exchange timed out and the row holds NaN)
 *   workspace      device scratch of at least xr_xent_workspace_bytes(M, V, dtype) bytes
 *   M >= 0 (M == 0 still writes mean_loss = NaN and counts = {0, 0, 0}), V >= 1
 * Rows whose only finite logits are missing (all -inf), or a target logit of -inf, give
 * NaN / +inf; a NaN or +inf logit in a row that is not ignored makes that row's gradient and
 * loss NaN (and so the mean or sum); an ignored row is never read, whatever it holds.
 * No written buffer (logits, row_loss, mean_loss, counts, the workspace) may overlap another
 * buffer of the call (XR_ERR_ALIAS); target and grad_scale are only read.
 */
xr_status_t xr_xent_fwd_bwd(void* logits, int64_t ld, const int64_t* target, int64_t M,
                            int64_t V, int64_t ignore_index, xr_dtype_t dtype, float* row_loss,
                            float* mean_loss, int32_t* counts, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Loss reductions of xr_xent_fwd_bwd_ex(). */
typedef enum {
  XR_REDUCTION_MEAN = 0, /* sum_i row_loss[i] / n: the pages' kernel */
  XR_REDUCTION_SUM = 1,  /* sum_i row_loss[i] */
  XR_REDUCTION_NONE = 2  /* the row losses themselves */
} xr_reduction_t;

/*
 * xr_xent_fwd_bwd() with a choice of reduction and the upstream gradient folded into the
 * gradient write. The Liger-Kernel `cross_entropy.py` kernel documents the mean reduction
 * only; the sum and none reductions are those of the loss definition its docstring links
 * to. `LigerCrossEntropyFunction.backward` multiplies the stored gradient by the upstream
 * gradient in a second pass (`element_mul`); a caller that knows that gradient before the
 * forward (a loss scale, a per-token weight) passes it here and saves the pass:
 *   logits[i, j] <- s_i * (softmax(logits[i, :])_j - [j == t_i]) / n_r   (0 for ignored rows)
 *   with n_r = n for XR_REDUCTION_MEAN and 1 otherwise, s_i = grad_scale[i * grad_scale_stride]
 *   (s_i = 1 when grad_scale is NULL).
 *   reduction          an xr_reduction_t; anything else returns XR_ERR_VALUE
 *   grad_scale         fp32, device, or NULL; grad_scale_stride >= 0 (0: one value for all
 *                      rows, the usual case for the mean and sum; 1: one value per row,
 *                      the none reduction's upstream gradient); negative returns XR_ERR_VALUE
 *   loss               fp32 [1], device: the mean (XR_REDUCTION_MEAN, NaN when n == 0) or
 *                      the sum (XR_REDUCTION_SUM, 0 when M == 0); required for those two,
 *                      ignored and may be NULL for XR_REDUCTION_NONE
 *   row_loss           fp32 [M], device: the unscaled row losses (0 for ignored rows);
 *                      required for XR_REDUCTION_NONE (they are its result), may be NULL
 *                      for the other two (then kept in the workspace)
 * Everything else is as in xr_xent_fwd_bwd(), which equals this call with
 * XR_REDUCTION_MEAN and grad_scale NULL.
 */
xr_status_t xr_xent_fwd_bwd_ex(void* logits, int64_t ld, const int64_t* target, int64_t M,
                               int64_t V, int64_t ignore_index, xr_dtype_t dtype,
                               xr_reduction_t reduction, const float* grad_scale,
                               int64_t grad_scale_stride, float* row_loss, float* loss,
                               int32_t* counts, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * xr_xent_fwd_bwd_ex() for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): no workspace argument; the
 * call's scratch (the counts, the split rows' exchange slots and, when row_loss is NULL, the
 * row losses) lives in a static device array of the library, XR_NOALLOC_SCRATCH_BYTES on
 * each device it runs on, held until the process ends. Sizes whose scratch would not fit
 * return XR_ERR_TOO_LARGE with nothing enqueued (xr_xent_workspace_bytes() tells the need;
 * for instance 16384 x 128256 bf16, four chunks per row, needs 256 + 16384 x 4 x 8 bytes,
 * plus 4 per row without row_loss). Nothing is allocated, freed or synchronised; the kernels initialise what must
 * start at zero. Every call on a device shares that device's array and leaves its contents
 * behind: calls that overlap in time on one device (several streams, several threads) race
 * and must not be made. Arguments and results are otherwise those of xr_xent_fwd_bwd_ex().
 */
#define XR_NOALLOC_SCRATCH_BYTES (4u << 20)
xr_status_t xr_xent_fwd_bwd_noalloc(void* logits, int64_t ld, const int64_t* target, int64_t M,
                                    int64_t V, int64_t ignore_index, xr_dtype_t dtype,
                                    xr_reduction_t reduction, const float* grad_scale,
                                    int64_t grad_scale_stride, float* row_loss, float* loss,
                                    int32_t* counts, void* stream);

/*
 * The backward's scaling of a stored cross-entropy gradient by the upstream gradient, in
 * place (Liger-Kernel `cross_entropy.py`: `element_mul`, called by
 * `LigerCrossEntropyFunction.backward`):
 *   x[i, j] <- x[i, j] * grad_output[i * grad_output_stride]   for j < N
 * computed in fp32 and rounded once to dtype. A row whose factor is exactly 1.0 is neither
 * read nor written: the page skips the multiplication for a unit upstream gradient after a
 * host-side comparison, which this decides on the device, with no synchronisation.
 *   x, ld              [M, N] of dtype, device, modified in place; columns [N, ld) untouched
 *   grad_output        fp32, device, required; grad_output_stride >= 0 (0: one factor for
 *                      every row, a scalar loss's upstream gradient; 1: one per row)
 *   M >= 0 (M == 0 enqueues nothing), N >= 1
 * grad_output must not overlap x.
 */
xr_status_t xr_element_mul(void* x, int64_t ld, int64_t M, int64_t N, xr_dtype_t dtype,
                           const float* grad_output, int64_t grad_output_stride, void* stream);

/*
 * Status word of a workspace, written by the last call that used it (xr_softmax_fwd_ex,
 * xr_softmax_bwd_ex, xr_nll_fwd, xr_xent_fwd_bwd / _ex): 0, or bit 0 when a split row's
 * exchange timed out (its row then holds NaN). Enqueues on `stream` a 4-byte device copy of
 * the word into *status, a DEVICE int32 (no synchronisation): read it after that stream's
 * work is done. The cross-entropy reports the same word in counts[2].
 *   workspace, workspace_bytes  the workspace as passed to that call (>= 256 bytes)
 */
xr_status_t xr_workspace_status(const void* workspace, size_t workspace_bytes, int32_t* status,
                                void* stream);

/*
 * Memory-ceiling probe, for measurement (what a row kernel's launch can move at a given
 * size): the row kernels' loads and stores with none of their arithmetic. Each of `split`
 * workgroups per row, of `threads` threads holding `vpt` 16-byte vectors each per input,
 * loads its chunk of the row from in0 (and from in1 when in1 is not NULL) with non-temporal
 * loads, waits for every load and a workgroup barrier, then stores the chunk (in0 ^ in1 with
 * two inputs) to out with non-temporal stores. Rows whose target equals ignore_index (target
 * may be NULL) are not read and are written with zeros, as the cross-entropy does with
 * ignored rows. out may be exactly in0 (in place).
 *   M rows of N elements of dtype; in0 / in1 with row stride ld_in, out with ld_out; every
 *   row on a 16-byte boundary and N * element size a multiple of 16, else XR_ERR_ALIGN
 *   threads x vpt: a shape of the row kernels (one input: 64x4, 64x8, 64x16, 128x8, 128x16,
 *   256x8, 256x16, 512x8, 512x16, 1024x16; two inputs: 64x4, 64x8, 128x8, 256x8, 512x8,
 *   1024x8) holding a chunk of ceil(vectors per row / split) vectors, else XR_ERR_SHAPE
 * Enqueued like the other calls (the profiling events of xr_set_profile_events() bracket it).
 */
xr_status_t xr_probe_rows(void* out, int64_t ld_out, const void* in0, const void* in1,
                          int64_t ld_in, int64_t M, int64_t N, xr_dtype_t dtype, int32_t threads,
                          int32_t vpt, int32_t split, const int64_t* target, int64_t ignore_index,
                          void* stream);

/*
 * Copy ceiling, for measurement: what a plain stream of `bytes` bytes moves (the achievable
 * rate of that traffic, against which a row kernel's rate is read). With in1 NULL, one read
 * and one write per byte (out = in); with in1, two reads per write (out = in ^ in1, the
 * softmax backward's mix). workgroups > 0: a grid-stride kernel of that many workgroups of
 * `threads` threads (256, 512 or 1024, else XR_ERR_SHAPE), 16-byte non-temporal loads and
 * stores, four vectors in flight per thread; workgroups == 0: the runtime's device-to-device
 * copy (hipMemcpyAsync; in1 must be NULL, else XR_ERR_VALUE). Either is bracketed by the
 * events of xr_set_profile_events(). out == in (exactly) with in1 NULL and workgroups > 0 is
 * the same kernel stream in place, every vector read and written back (the traffic of a
 * kernel that overwrites its input, as the cross-entropy's gradient does).
 *   in, in1, out: device memory on 16-byte boundaries, bytes a multiple of 16 (else
 *   XR_ERR_ALIGN); out must not overlap an input other than as that exact in-place call
 *   (XR_ERR_ALIAS; in place with workgroups == 0 too); in place with in1: XR_ERR_VALUE;
 *   bytes == 0 enqueues nothing
 */
xr_status_t xr_probe_copy(void* out, const void* in, const void* in1, int64_t bytes,
                          int32_t workgroups, int32_t threads, void* stream);

/* Static, human-readable text for a status code (host). */
const char* xr_status_string(xr_status_t status);

/* ABI version: major * 10000 + minor * 100 + patch. */
int32_t xr_version(void);

/*
 * How a call is carried out (host query, nothing enqueued). path: 1 = row-resident
 * (a row or a row chunk per workgroup, held in registers: one read of the input),
 * 2 = split row (S > 1 workgroups per row exchanging (max, sum) pairs or partial sums),
 * 3 = stream (one workgroup per row, two passes over global memory: the row statistics,
 * then the outputs).
 * op: 0 = softmax forward, 1 = softmax backward (both without a workspace),
 * 2 = cross-entropy, 3 = negative log-softmax forward (with a workspace), 4 = softmax
 * forward and 5 = softmax backward with a workspace (xr_softmax_fwd_ex / _bwd_ex).
 * aligned: 0 = the operand rows sit at different addresses modulo 16 bytes (stream path),
 * 1 = they share their address modulo 16 (rows may start anywhere), 2 = moreover every row
 * starts on a 16-byte boundary (the usual contiguous tensors). The cross-entropy has one
 * operand, so 0 is read as 1 for it.
 */
typedef struct xr_plan {
  int32_t path;
  int32_t threads;         /* workgroup size */
  int32_t vec_per_thread;  /* 16-byte vectors held per thread and operand */
  int32_t split;           /* workgroups per row (S) */
  int32_t grid;            /* workgroups launched (capped at INT32_MAX; see grid_total) */
  int32_t cooperative;     /* 1 if launched as a cooperative grid */
  int64_t chunk_vecs;      /* 16-byte vectors per workgroup chunk of a row */
  int32_t group_rows;      /* split rows: adjacent rows whose chunks store together (1: none) */
  int32_t load_priority;   /* 1 if the row kernel raises its wave priority for the row's loads
                              (whole softmax rows whose grid the device holds at once) */
  int64_t grid_total;      /* workgroups the plan asks for (above INT32_MAX the call fails) */
} xr_plan_t;

xr_status_t xr_plan(int32_t op, int64_t M, int64_t N, xr_dtype_t dtype, int32_t aligned,
                    xr_plan_t* plan /* host */);

/*
 * xr_plan() for a modelled device instead of the current one (host only, no device needed):
 * compute_units compute units, each holding blocks_per_cu workgroups of the planned shape
 * at once (the occupancy a real device reports per kernel), cooperative launch available.
 * For planning and for checking the launch plans' residency conditions without a GPU.
 * compute_units or blocks_per_cu below 1 returns XR_ERR_VALUE.
 */
xr_status_t xr_plan_model(int32_t op, int64_t M, int64_t N, xr_dtype_t dtype, int32_t aligned,
                          int32_t compute_units, int32_t blocks_per_cu, xr_plan_t* plan /* host */);

/*
 * Process-wide overrides for tests and benchmarks. Setting one while another thread
 * launches work is safe, but which value that launch sees is unspecified. Value 0 restores
 * the automatic choice.
 *   XR_OPT_PATH     1 resident, 2 split, 3 stream (a forced path the sizes cannot take
 *                   returns XR_ERR_SHAPE from the entry point); layer norm: 1 row-resident,
 *                   3 element-wise
 *   XR_OPT_SPLIT    workgroups per row for the split path (>= 2): cross-entropy, and the
 *                   softmax forward / backward and negative log-softmax with a workspace
 *   XR_OPT_THREADS  workgroup size of the row-resident kernels (64 .. 1024)
 *   XR_OPT_GRID     0 or -1 = one workgroup per row (or per row chunk), launched normally;
 *                   k >= 1 = a persistent grid of k workgroups per compute unit (launched
 *                   cooperatively for split cross-entropy rows); layer norm: at most k
 *                   workgroups per compute unit in its persistent grids
 *   XR_OPT_LOAD_POLICY  row loads: 1 = default cache policy, 2 = non-temporal
 *   XR_OPT_NO_WAIT  1 = split-row exchanges start as if a wait had already timed out: a chunk
 *                   reads each partner's slot once and, if it is not yet published, gives
 *                   up (its row's outputs and loss become NaN; the cross-entropy reports
 *                   the timeout flag in counts[2], set from the start); the waits that
 *                   group adjacent rows' stores end at once. For testing the bounded-wait
 *                   path; never faster.
 *   XR_OPT_GROUPS   write groups of split rows: 1 = never, 2 = whenever the plan's
 *                   residency condition allows them (chunks of any size); 0 = the automatic
 *                   choice (chunks of 32 KiB and more)
 */
typedef enum xr_option {
  XR_OPT_PATH = 1,
  XR_OPT_SPLIT = 2,
  XR_OPT_THREADS = 3,
  XR_OPT_GRID = 4,
  XR_OPT_LOAD_POLICY = 5,
  XR_OPT_NO_WAIT = 6,
  XR_OPT_GROUPS = 7
} xr_option_t;

xr_status_t xr_set_option(xr_option_t option, int64_t value);

/*
 * Profiling hook (process-wide): while set, every entry point records
 * hipEvent_t `start` on its stream right before launching its row kernel (the kernel that
 * reads and writes the rows; not the small target-scan and mean kernels of the
 * cross-entropy) and `stop` right after it, so hipEventElapsedTime(start, stop) is that
 * kernel's duration. The events are created and owned by the caller. Both NULL clears the
 * hook; exactly one NULL is XR_ERR_NULL.
 */
xr_status_t xr_set_profile_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* XR_H_ */
