/*
 * nbw_oracle.c -- plain, slow, fp64 CPU oracle for sliced r-bit qgemm over
 * nested bit-plane weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or constant with the HIP library; it is written from the
 * method's definitions alone, one step at a time, with no blocking or fusion.
 *
 * What it computes, and where each step comes from:
 *
 *  - One 8-bit "sliceable" parent code c in [0,255] per weight.  An r-bit child
 *    is obtained by keeping the most significant bits of every parent code
 *    (MatGPTQ: Accurate and Efficient Post-Training Matryoshka Quantization,
 *    abstract: serving several precisions by slicing the MSBs at inference
 *    time; MatGPTQ: Efficient and Accurate Inference over Nested Quantized
 *    Models, Abstract: lower precisions are read as fewer bits of the weights):
 *        q_r = c >> (8 - r).
 *  - "An r-bit model reads exactly r bits" (same page, Abstract and Table 1,
 *    row "Exact r-bit loading"): codes are stored as eight bit-planes, plane 0
 *    holding the most significant bit, so the r-bit child is the first r
 *    planes.  The order of bits inside a plane is this library's own layout
 *    definition (the pages do not give one):
 *        rows are padded to a multiple of 16 (padding bits are 0);
 *        plane_bytes = ceil(n/16)*16 * k/8;
 *        the 16-byte chunk for (plane p, row i, scale group g = j/128) starts at
 *          p*plane_bytes + ((i/16)*(k/128) + g)*256 + (i%16)*16;
 *        inside a chunk, column c = j%128 lives in little-endian 32-bit word
 *          c/32, at bit  (c%32)/2 + 16*(c%2)   (even columns in bits 0..15,
 *          odd columns in bits 16..31).
 *  - Dequantisation of a child code (the pages give no formula; this library
 *    uses the symmetric mid-point grid): with the bf16 scale s of the row's
 *    128-wide group along k,
 *        w = s * 2^(8-r) * (q_r + 1/2 - 2^(r-1)).
 *  - The product (MatGPTQ v2, Abstract: kernels for batch sizes beyond one;
 *    Figure 1: the kernels are timed against a dense matmul):
 *        Y[b][i] = sum_j X[b][j] * w[i][j],   X bf16 [batch][k], W [n][k].
 *
 * All floating point here is IEEE double.  bf16 inputs are widened exactly.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

/* ---- geometry of the bit-plane layout ---------------------------------- */

static int64_t padded_rows(int64_t n) { return (n + 15) / 16 * 16; }

int64_t nbwo_plane_bytes(int64_t n, int64_t k) { return padded_rows(n) * (k / 8); }

/* Byte offset and bit number of (plane p, row i, column j). */
static void locate(int64_t n, int64_t k, int p, int64_t i, int64_t j,
                   int64_t *byte_off, int *bit) {
    int64_t groups = k / 128;
    int64_t g = j / 128;
    int64_t c = j % 128;
    int64_t word = c / 32;
    int64_t e = c % 32;
    int pos = (int)(e / 2 + 16 * (e % 2)); /* bit inside the 32-bit word */
    int64_t chunk = ((i / 16) * groups + g) * 256 + (i % 16) * 16;
    *byte_off = (int64_t)p * nbwo_plane_bytes(n, k) + chunk + 4 * word + pos / 8;
    *bit = pos % 8;
}

static int read_bit(const uint8_t *planes, int64_t n, int64_t k, int p, int64_t i, int64_t j) {
    int64_t off;
    int bit;
    locate(n, k, p, i, j, &off, &bit);
    return (planes[off] >> bit) & 1;
}

/* ---- bf16 widening (exact) --------------------------------------------- */

double nbwo_bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---- pack: parent codes -> 8 MSB-first bit-planes ---------------------- */

/* codes: [n][k] row-major.  planes: 8*nbwo_plane_bytes(n,k) bytes, written in full. */
void nbwo_pack(const uint8_t *codes, int64_t n, int64_t k, uint8_t *planes) {
    memset(planes, 0, (size_t)(8 * nbwo_plane_bytes(n, k)));
    for (int p = 0; p < 8; ++p)
        for (int64_t i = 0; i < n; ++i)
            for (int64_t j = 0; j < k; ++j) {
                int b = (codes[i * k + j] >> (7 - p)) & 1; /* plane 0 = bit 7 */
                if (b) {
                    int64_t off;
                    int bit;
                    locate(n, k, p, i, j, &off, &bit);
                    planes[off] |= (uint8_t)(1u << bit);
                }
            }
}

/* ---- slice + unpack: read only planes 0..r-1 --------------------------- */

/* q[i][j] = sum_{p<r} bit_p(i,j) * 2^(r-1-p).  Planes r..7 are never read. */
void nbwo_unpack(const uint8_t *planes, int64_t n, int64_t k, int r, uint8_t *q) {
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < k; ++j) {
            int v = 0;
            for (int p = 0; p < r; ++p)
                v = 2 * v + read_bit(planes, n, k, p, i, j);
            q[i * k + j] = (uint8_t)v;
        }
}

/* ---- dequant ------------------------------------------------------------ */

double nbwo_dequant_value(double s, int q, int r) {
    return s * ldexp(1.0, 8 - r) * ((double)q + 0.5 - ldexp(1.0, r - 1));
}

/* w[i][j] for the r-bit child; scales bf16 [n][k/128]. */
void nbwo_dequant(const uint8_t *planes, const uint16_t *scales, int64_t n, int64_t k, int r,
                  double *w) {
    int64_t groups = k / 128;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < k; ++j) {
            int q = 0;
            for (int p = 0; p < r; ++p)
                q = 2 * q + read_bit(planes, n, k, p, i, j);
            double s = nbwo_bf16_to_double(scales[i * groups + j / 128]);
            w[i * k + j] = nbwo_dequant_value(s, q, r);
        }
}

/* ---- qgemm -------------------------------------------------------------- */

/* One output row i for every batch row: dequantise row i of the child, then a
 * plain dot product in k order for each batch row.  Result b goes to out[b*stride]. */
static void qgemm_row(const uint16_t *x, int64_t batch, const uint8_t *planes,
                      const uint16_t *scales, int64_t n, int64_t k, int r, int64_t i,
                      double *wrow, double *out, int64_t stride) {
    int64_t groups = k / 128;
    for (int64_t j = 0; j < k; ++j) {
        int q = 0;
        for (int p = 0; p < r; ++p)
            q = 2 * q + read_bit(planes, n, k, p, i, j);
        double s = nbwo_bf16_to_double(scales[i * groups + j / 128]);
        wrow[j] = nbwo_dequant_value(s, q, r);
    }
    for (int64_t b = 0; b < batch; ++b) {
        double acc = 0.0;
        for (int64_t j = 0; j < k; ++j)
            acc += nbwo_bf16_to_double(x[b * k + j]) * wrow[j];
        out[b * stride] = acc;
    }
}

/* Y[b][i] = sum_j X[b][j] * w[i][j];  y is [batch][n] row-major, fp64.
 * Returns 0, or -1 if a row buffer could not be allocated. */
int nbwo_qgemm(const uint16_t *x, int64_t batch, const uint8_t *planes, const uint16_t *scales,
               int64_t n, int64_t k, int r, double *y) {
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n; ++i) {
        double *wrow = (double *)malloc((size_t)k * sizeof(double));
        if (!wrow) {
#pragma omp atomic write
            fail = 1;
            continue;
        }
        qgemm_row(x, batch, planes, scales, n, k, r, i, wrow, y + i, n);
        free(wrow);
    }
    return fail ? -1 : 0;
}

/* The same product for selected output rows only (for outputs sampled from
 * shapes too large to compute in full).  y is [batch][nrows]: y[b*nrows + t]
 * is output row rows[t]. */
int nbwo_qgemm_rows(const uint16_t *x, int64_t batch, const uint8_t *planes,
                    const uint16_t *scales, int64_t n, int64_t k, int r, const int64_t *rows,
                    int64_t nrows, double *y) {
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < nrows; ++t) {
        double *wrow = (double *)malloc((size_t)k * sizeof(double));
        if (!wrow) {
#pragma omp atomic write
            fail = 1;
            continue;
        }
        qgemm_row(x, batch, planes, scales, n, k, r, rows[t], wrow, y + t, nrows);
        free(wrow);
    }
    return fail ? -1 : 0;
}

/* ---- asymmetric children ------------------------------------------------ */
/*
 * The pages evaluate an asymmetric variant (MatGPTQ: Efficient and Accurate
 * Inference over Nested Quantized Models, Tables 4-7, "asymmetric MatGPTQ")
 * without stating its formula.  Reading used here: the parent grid is
 * s * (c - z) with a per-(row, group) zero point z, and an r-bit child takes
 * the mean of its 2^(8-r) parent values, exactly as the symmetric grid does:
 *     w = s * (2^(8-r) * (q_r + 1/2) - 1/2 - z).
 * With z = 127.5 this is the symmetric closed form above.
 */
double nbwo_dequant_value_asym(double s, double z, int q, int r) {
    return s * (ldexp(1.0, 8 - r) * ((double)q + 0.5) - 0.5 - z);
}

static void qgemm_row_asym(const uint16_t *x, int64_t batch, const uint8_t *planes,
                           const uint16_t *scales, const uint16_t *zeros, int64_t n, int64_t k,
                           int r, int64_t i, double *wrow, double *out, int64_t stride) {
    int64_t groups = k / 128;
    for (int64_t j = 0; j < k; ++j) {
        int q = 0;
        for (int p = 0; p < r; ++p)
            q = 2 * q + read_bit(planes, n, k, p, i, j);
        double s = nbwo_bf16_to_double(scales[i * groups + j / 128]);
        double z = nbwo_bf16_to_double(zeros[i * groups + j / 128]);
        wrow[j] = nbwo_dequant_value_asym(s, z, q, r);
    }
    for (int64_t b = 0; b < batch; ++b) {
        double acc = 0.0;
        for (int64_t j = 0; j < k; ++j)
            acc += wrow[j] * nbwo_bf16_to_double(x[b * k + j]);
        out[b * stride] = acc;
    }
}

/* Asymmetric product for selected output rows (all rows: rows = 0..n-1);
 * zeros bf16 [n][k/128] like the scales.  y is [batch][nrows]. */
int nbwo_qgemm_asym_rows(const uint16_t *x, int64_t batch, const uint8_t *planes,
                         const uint16_t *scales, const uint16_t *zeros, int64_t n, int64_t k,
                         int r, const int64_t *rows, int64_t nrows, double *y) {
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < nrows; ++t) {
        double *wrow = (double *)malloc((size_t)k * sizeof(double));
        if (!wrow) {
#pragma omp atomic write
            fail = 1;
            continue;
        }
        qgemm_row_asym(x, batch, planes, scales, zeros, n, k, r, rows[t], wrow, y + t, nrows);
        free(wrow);
    }
    return fail ? -1 : 0;
}

/* ---- data-free multi-precision code choice ----------------------------- */
/*
 * For each weight w (fp32) with its group scale s, choose the parent code
 * c in [0, 255] that minimises the weighted squared error of the children it
 * serves (MatGPTQ: Accurate and Efficient Post-Training Matryoshka
 * Quantization, abstract: one parent serves several precisions; MatGPTQ:
 * Efficient and Accurate Inference over Nested Quantized Models, captions of
 * Tables 6 and 7, which name the per-precision weights lambda_3, lambda_4,
 * lambda_8):
 *     loss(c) = sum_t lambda_t * (w - dequant(s, c >> (8 - r_t), r_t))^2,
 * for the widths r_t in `widths` (nw of them).  Every code is tried in order
 * 0..255; the first code with the smallest loss wins.  All arithmetic is
 * IEEE double, one operation at a time, in this order: e = w - d; e2 = e * e;
 * term = lambda * e2; loss accumulated left to right over `widths`.
 */
void nbwo_choose_codes(const float *w, int64_t n, int64_t k, const uint16_t *scales,
                       const int *widths, const double *lambdas, int nw, uint8_t *codes) {
    int64_t groups = k / 128;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < k; ++j) {
            double wv = (double)w[i * k + j];
            double s = nbwo_bf16_to_double(scales[i * groups + j / 128]);
            int best = 0;
            double best_loss = 0.0;
            for (int c = 0; c < 256; ++c) {
                double loss = 0.0;
                for (int t = 0; t < nw; ++t) {
                    int r = widths[t];
                    double d = nbwo_dequant_value(s, c >> (8 - r), r);
                    double e = wv - d;
                    double e2 = e * e;
                    double term = lambdas[t] * e2;
                    loss = loss + term;
                }
                if (c == 0 || loss < best_loss) {
                    best = c;
                    best_loss = loss;
                }
            }
            codes[i * k + j] = (uint8_t)best;
        }
}
