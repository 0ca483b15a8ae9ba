/*
 * xr_oracle.c -- plain float64 CPU oracle for the row-softmax family.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product path (the
 * HIP library under cross_entropy_reductions_amd/) never links, imports or
 * calls it, and this file shares no source with it.
 *
 * Every routine is the plain definition, computed in double precision, one
 * row after another within a thread, with no blocking, fusion or reordering
 * beyond what the definition states:
 *
 *   softmax forward   -- the "safe softmax" of the Triton fused-softmax
 *                        examples on the page "python sum function examples"
 *                        (kernels `softmax_kernel` and `_softmax`): subtract
 *                        the row maximum, exponentiate, divide by the row sum.
 *   softmax backward  -- the fused softmax backward of the `_backward` kernel
 *                        on the same page, with its block-sparse scale taken
 *                        as 1: dx_j = y_j * (dy_j - sum_k y_k * dy_k).
 *   block-sparse softmax backward -- the `_backward` kernel on the same page in
 *                        full: each row of a block-sparse matrix is the row's
 *                        segment in each of the blocks its look-up table lists;
 *                        dx = y * (dy - sum(y * dy)) * scale along that row,
 *                        written over dy. Table layout, as the kernel reads
 *                        it: two words (size, offset) per block-row, then at
 *                        word offset + 4 k the k-th block's index into the
 *                        block storage (the other three words of an entry are
 *                        not read). Block b of batch z holds BLOCK x BLOCK
 *                        elements, row-major, at z * stride_z + b * BLOCK^2.
 *   negative log-softmax with a gathered loss -- the Triton kernel `_forward`
 *                        on the same page: each output element is
 *                        log(sum_k exp(x_k - m)) - (x_j - m) = -log p_j, and
 *                        the row's loss is the output element at the row's
 *                        index as stored (the kernel reads it back from the
 *                        output), i.e. rounded to the output type.
 *   layer norm        -- the Triton LayerNorm tutorial page (translated; its code is
 *                        cut off, so the definitions come from its prose and the
 *                        cited paper, Ba, Kiros & Hinton 2016): per row, mean
 *                        and variance over the N features, rstd = 1/sqrt(var +
 *                        eps), y = (x - mean) * rstd * w + b; the backward is the
 *                        derivative of that definition, with dw and db summed
 *                        over all rows (the page's two-stage reduction reaches
 *                        the same sums).
 *   cross-entropy     -- Liger-Kernel `cross_entropy.py`,
 *                        `liger_cross_entropy_kernel` steps 1-6 and
 *                        `LigerCrossEntropyFunction.forward`: per-row loss
 *                        m + log d - x_y, gradient (softmax - onehot)/n where
 *                        n counts the targets that differ from ignore_index,
 *                        zero rows (gradient and loss) for ignored targets,
 *                        and the mean of the row losses over n.
 *   reductions and    -- the same page's kernel documents only the mean
 *   upstream gradient    reduction; the sum and none reductions are read from
 *                        the definition of the loss it links to: "sum" is
 *                        sum_i loss_i, whose gradient is softmax - onehot (no
 *                        1/n), and "none" returns the row losses, the gradient
 *                        of row i being weighted by its own upstream value.
 *                        `LigerCrossEntropyFunction.backward` and its
 *                        `element_mul` kernel multiply the stored gradient by
 *                        the upstream gradient of the loss; the forward here
 *                        can apply that factor while it writes the gradient.
 *
 * The oracle deliberately uses the two-pass safe form (max first, then the
 * sum with that max), not the online running max/sum of the GPU path; both
 * reach the same value up to rounding.
 *
 * Readings of points the pages leave open (each one is stated where it acts):
 *   - bf16 inputs are decoded exactly: bits << 16 reinterpreted as a float.
 *   - a target outside [0, V) that is not ignore_index is counted as a bad
 *     target; its row gets a zero gradient and a zero loss (Liger reads such
 *     a target unchecked).
 *   - n counts every target that is not ignore_index (bad targets included),
 *     exactly as `(target != ignore_index).sum()` does on the Liger page.
 *   - n == 0 gives mean = 0/0 = NaN.
 *   - ignore_index is compared before any range check, so an ignore_index
 *     that lies inside [0, V) still ignores its rows.
 *
 * Parallelism: rows are independent, so rows are spread over OpenMP threads.
 * Within a row every sum runs left to right in double. The mean is a serial
 * left-to-right sum in row order.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { XRO_F32 = 0, XRO_BF16 = 1 };
enum { XRO_MEAN = 0, XRO_SUM = 1, XRO_NONE = 2 };

/* Element idx (in elements from base) of a bf16 or fp32 buffer, as double. */
static double load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == XRO_BF16) {
    uint16_t h;
    memcpy(&h, (const char*)base + 2 * idx, 2);
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
  } else {
    float f;
    memcpy(&f, (const char*)base + 4 * idx, 4);
    return (double)f;
  }
}

int xro_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void xro_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Safe softmax of one row: y[j] = exp(x_j - max) / sum_k exp(x_k - max). */
static void softmax_row(const void* x, int64_t row_off, int64_t N, int dtype, double* y) {
  double m = -INFINITY;
  for (int64_t j = 0; j < N; ++j) {
    double v = load_elem(x, row_off + j, dtype);
    if (v > m) m = v;
  }
  double d = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    double e = exp(load_elem(x, row_off + j, dtype) - m);
    y[j] = e;
    d += e;
  }
  for (int64_t j = 0; j < N; ++j) y[j] = y[j] / d;
}

/* y[M][N] (contiguous doubles) = softmax over each row of x (row stride ld_x). */
void xro_softmax_fwd(const void* x, int64_t ld_x, int64_t M, int64_t N, int dtype, double* y) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < M; ++i) softmax_row(x, i * ld_x, N, dtype, y + i * N);
}

/* dx[M][N] = y * (dy - sum_k y_k dy_k) per row; y and dy are read in dtype. */
void xro_softmax_bwd(const void* y, int64_t ld_y, const void* dy, int64_t ld_dy, int64_t M,
                     int64_t N, int dtype, double* dx) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < M; ++i) {
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j)
      s += load_elem(y, i * ld_y + j, dtype) * load_elem(dy, i * ld_dy + j, dtype);
    for (int64_t j = 0; j < N; ++j)
      dx[i * N + j] = load_elem(y, i * ld_y + j, dtype) * (load_elem(dy, i * ld_dy + j, dtype) - s);
  }
}

/*
 * v rounded to the nearest value of the element type, ties to even: fp32 by the C
 * conversion (round to nearest even), bf16 by keeping 8 significant bits of v with
 * nearbyint (the default rounding mode: to nearest, ties to even). Finite, normal v only.
 */
static double round_to_dtype(double v, int dtype) {
  if (dtype == XRO_F32) return (double)(float)v;
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  double f = frexp(v, &e); /* v = f * 2^e, 0.5 <= |f| < 1 */
  return ldexp(nearbyint(ldexp(f, 8)), e - 8);
}

/*
 * out[M][N] (contiguous doubles) = -log softmax of each row of x (row stride ld_x);
 * loss[i] = out[i][idx[i]] rounded to dtype, NaN when idx[i] lies outside [0, N).
 */
void xro_nll_fwd(const void* x, int64_t ld_x, const int64_t* idx, int64_t M, int64_t N,
                 int dtype, double* out, double* loss) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < M; ++i) {
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j) {
      double v = load_elem(x, i * ld_x + j, dtype);
      if (v > m) m = v;
    }
    double d = 0.0;
    for (int64_t j = 0; j < N; ++j) d += exp(load_elem(x, i * ld_x + j, dtype) - m);
    double lse = log(d);
    for (int64_t j = 0; j < N; ++j) out[i * N + j] = lse - (load_elem(x, i * ld_x + j, dtype) - m);
    loss[i] = (idx[i] >= 0 && idx[i] < N) ? round_to_dtype(out[i * N + idx[i]], dtype) : NAN;
  }
}

/*
 * Layer norm forward. x [M, N] (row stride ld_x), w and b [N], all in dtype.
 * y [M][N] contiguous doubles; mean [M], rstd [M] doubles.
 *   mean_i = (1/N) sum_j x_ij,  var_i = (1/N) sum_j (x_ij - mean_i)^2,
 *   rstd_i = 1 / sqrt(var_i + eps),  y_ij = (x_ij - mean_i) * rstd_i * w_j + b_j
 */
void xro_layernorm_fwd(const void* x, int64_t ld_x, const void* w, const void* b, int64_t M,
                       int64_t N, double eps, int dtype, double* y, double* mean, double* rstd) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < M; ++i) {
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j) s += load_elem(x, i * ld_x + j, dtype);
    double mu = s / (double)N;
    double v = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      double c = load_elem(x, i * ld_x + j, dtype) - mu;
      v += c * c;
    }
    double r = 1.0 / sqrt(v / (double)N + eps);
    mean[i] = mu;
    rstd[i] = r;
    for (int64_t j = 0; j < N; ++j)
      y[i * N + j] = (load_elem(x, i * ld_x + j, dtype) - mu) * r * load_elem(w, j, dtype) +
                     load_elem(b, j, dtype);
  }
}

/*
 * Layer norm backward: the derivative of xro_layernorm_fwd's y with respect to x, w and b,
 * contracted with dy [M, N] (row stride ld_dy). mean and rstd are recomputed from x in
 * double. With xhat_ij = (x_ij - mean_i) * rstd_i and g_ij = w_j * dy_ij:
 *   dx_ij = rstd_i * (g_ij - (xhat_ij * c1_i + c2_i)),
 *       c1_i = (1/N) sum_j xhat_ij g_ij,  c2_i = (1/N) sum_j g_ij
 *   dw_j = sum_i dy_ij xhat_ij,  db_j = sum_i dy_ij      (sums in row order)
 * dx [M][N] contiguous doubles, dw [N], db [N] doubles.
 */
void xro_layernorm_bwd(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x, const void* w,
                       int64_t M, int64_t N, double eps, int dtype, double* dx, double* dw,
                       double* db) {
  double* mu = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
  double* rs = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < M; ++i) {
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j) s += load_elem(x, i * ld_x + j, dtype);
    double m = s / (double)N;
    double v = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      double c = load_elem(x, i * ld_x + j, dtype) - m;
      v += c * c;
    }
    double r = 1.0 / sqrt(v / (double)N + eps);
    mu[i] = m;
    rs[i] = r;
    double c1 = 0.0, c2 = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      double xh = (load_elem(x, i * ld_x + j, dtype) - m) * r;
      double g = load_elem(w, j, dtype) * load_elem(dy, i * ld_dy + j, dtype);
      c1 += xh * g;
      c2 += g;
    }
    c1 /= (double)N;
    c2 /= (double)N;
    for (int64_t j = 0; j < N; ++j) {
      double xh = (load_elem(x, i * ld_x + j, dtype) - m) * r;
      double g = load_elem(w, j, dtype) * load_elem(dy, i * ld_dy + j, dtype);
      dx[i * N + j] = r * (g - (xh * c1 + c2));
    }
  }
  /* dw and db: column sums over the rows, in row order */
  int64_t j;
#pragma omp parallel for schedule(static)
  for (j = 0; j < N; ++j) {
    double sw = 0.0, sb = 0.0;
    for (int64_t r = 0; r < M; ++r) {
      double d = load_elem(dy, r * ld_dy + j, dtype);
      sw += d * ((load_elem(x, r * ld_x + j, dtype) - mu[r]) * rs[r]);
      sb += d;
    }
    dw[j] = sw;
    db[j] = sb;
  }
  free(mu);
  free(rs);
}

/*
 * Block-sparse softmax backward. y and dy hold Z batches of n_blocks blocks of block x block
 * elements (batch z at element z * stride_z); lut as described above, for n_brows
 * block-rows. out is a copy of dy (Z * stride_z doubles) that receives, for every row
 * (z, block-row r, row i of the block) and every block k < size_r of its table entry list:
 *   out[z][b_k][i][c] = y * (dy - s) * scale,   s = sum over k', c' of y * dy along the row
 * Elements of blocks the table does not list for a row stay as in dy.
 */
void xro_bsr_softmax_bwd(const void* y, const void* dy, int64_t stride_z, int64_t Z,
                         const int32_t* lut, int64_t n_brows, int64_t block, double scale,
                         int dtype, double* out) {
  int64_t zr;
#pragma omp parallel for schedule(dynamic, 1)
  for (zr = 0; zr < Z * n_brows; ++zr) {
    int64_t z = zr / n_brows, r = zr % n_brows;
    int32_t size = lut[2 * r], offset = lut[2 * r + 1];
    for (int64_t i = 0; i < block; ++i) {
      double s = 0.0;
      for (int32_t k = 0; k < size; ++k) {
        int64_t base = z * stride_z + (int64_t)lut[offset + 4 * k] * block * block + i * block;
        for (int64_t c = 0; c < block; ++c)
          s += load_elem(y, base + c, dtype) * load_elem(dy, base + c, dtype);
      }
      for (int32_t k = 0; k < size; ++k) {
        int64_t base = z * stride_z + (int64_t)lut[offset + 4 * k] * block * block + i * block;
        for (int64_t c = 0; c < block; ++c)
          out[base + c] = load_elem(y, base + c, dtype) * (load_elem(dy, base + c, dtype) - s) * scale;
      }
    }
  }
}

/* counts[0] = #{i : t_i != ignore_index}; counts[1] = those among them outside [0, V). */
void xro_xent_count(const int64_t* target, int64_t M, int64_t V, int64_t ignore_index,
                    int64_t* counts) {
  int64_t n = 0, bad = 0;
  for (int64_t i = 0; i < M; ++i) {
    if (target[i] == ignore_index) continue;
    ++n;
    if (target[i] < 0 || target[i] >= V) ++bad;
  }
  counts[0] = n;
  counts[1] = bad;
}

/*
 * Cross-entropy loss and gradient for a list of rows.
 *   rows         : row indices into logits/target, or NULL for rows 0..nrows-1
 *   reduction    : XRO_MEAN (gradient of sum_i loss_i / n), XRO_SUM (gradient of
 *                  sum_i loss_i) or XRO_NONE (gradient of the row losses)
 *   n            : the batch's non-ignored count (from xro_xent_count)
 *   scale        : upstream gradient; row i's gradient is multiplied by
 *                  scale[i * scale_stride] (stride 0: one value for every row);
 *                  NULL means 1. Ignored rows stay exactly zero.
 *   grad         : [nrows][V] contiguous doubles, or NULL to skip the gradient
 *   loss         : [nrows] doubles
 */
void xro_xent_rows_ex(const void* logits, int64_t ld, const int64_t* target, const int64_t* rows,
                      int64_t nrows, int64_t V, int64_t ignore_index, int dtype, int reduction,
                      int64_t n, const double* scale, int64_t scale_stride, double* grad,
                      double* loss) {
  int64_t r;
#pragma omp parallel for schedule(dynamic, 4)
  for (r = 0; r < nrows; ++r) {
    int64_t i = rows ? rows[r] : r;
    int64_t t = target[i];
    double* g = grad ? grad + r * V : NULL;
    if (t == ignore_index || t < 0 || t >= V) {
      loss[r] = 0.0;
      if (g)
        for (int64_t j = 0; j < V; ++j) g[j] = 0.0;
      continue;
    }
    int64_t off = i * ld;
    double m = -INFINITY;
    for (int64_t j = 0; j < V; ++j) {
      double v = load_elem(logits, off + j, dtype);
      if (v > m) m = v;
    }
    double d = 0.0;
    for (int64_t j = 0; j < V; ++j) d += exp(load_elem(logits, off + j, dtype) - m);
    double xt = load_elem(logits, off + t, dtype);
    /* logsumexp - x_t with the difference first: float64 keeps log d at any magnitude
       of m (m + log d rounds log d away once |m| passes about 1e16) */
    loss[r] = (m - xt) + log(d);
    if (g) {
      /* d(loss_i)/d(x_ij) = p_j - [j == t]; the reduction and the upstream value scale it. */
      double w = scale ? scale[i * scale_stride] : 1.0;
      if (reduction == XRO_MEAN) w = w / (double)n;
      for (int64_t j = 0; j < V; ++j) {
        double p = exp(load_elem(logits, off + j, dtype) - m) / d;
        g[j] = w * ((j == t) ? p - 1.0 : p);
      }
    }
  }
}

/* The mean-reduction case with upstream gradient 1 (the pages' own kernel). */
void xro_xent_rows(const void* logits, int64_t ld, const int64_t* target, const int64_t* rows,
                   int64_t nrows, int64_t V, int64_t ignore_index, int dtype, int64_t n,
                   double* grad, double* loss) {
  xro_xent_rows_ex(logits, ld, target, rows, nrows, V, ignore_index, dtype, XRO_MEAN, n, NULL, 0,
                   grad, loss);
}

/* sum_i loss_i, left to right in row order. */
double xro_sum(const double* loss, int64_t M) {
  double s = 0.0;
  for (int64_t i = 0; i < M; ++i) s += loss[i];
  return s;
}

/*
 * The backward's `element_mul`: out[i][j] = x[i][j] * scale[i * scale_stride] for the V
 * columns of each row of x (row stride ld, read in dtype); out is [M][V] contiguous doubles.
 */
void xro_element_mul(const void* x, int64_t ld, int64_t M, int64_t V, int dtype,
                     const double* scale, int64_t scale_stride, double* out) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < M; ++i) {
    double w = scale[i * scale_stride];
    for (int64_t j = 0; j < V; ++j) out[i * V + j] = load_elem(x, i * ld + j, dtype) * w;
  }
}

/* mean = (sum_i loss_i) / n, summed left to right in row order; n == 0 gives NaN. */
double xro_mean(const double* loss, int64_t M, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < M; ++i) s += loss[i];
  return s / (double)n;
}

/* The whole fused cross-entropy on M rows; grad may be NULL. */
double xro_xent(const void* logits, int64_t ld, const int64_t* target, int64_t M, int64_t V,
                int64_t ignore_index, int dtype, double* grad, double* loss, int64_t* counts) {
  xro_xent_count(target, M, V, ignore_index, counts);
  xro_xent_rows(logits, ld, target, NULL, M, V, ignore_index, dtype, counts[0], grad, loss);
  return xro_mean(loss, M, counts[0]);
}
