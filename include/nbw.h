/*
 * nbw.h -- C ABI of libnbw: sliced r-bit qgemm over nested bit-plane weights
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (MatGPTQ: Efficient and Accurate Inference over Nested Quantized
 * Models; MatGPTQ: Accurate and Efficient Post-Training Matryoshka
 * Quantization) serves one 8-bit "sliceable" parent checkpoint at several
 * precisions: the r-bit child keeps the most significant bits of every parent
 * code (v1 abstract; v2 Abstract), reads exactly r bits of weight data (v2
 * Abstract; Table 1, row "Exact r-bit loading"), and is executed by kernels
 * that support batch sizes beyond one (v2 Abstract; Figure 1, kernel speed-up
 * over a dense matmul across bit-widths, shapes and batch sizes).
 *
 * Conventions for every entry point
 *  - Every pointer argument that names tensor data is a DEVICE pointer,
 *    allocated and owned by the caller, who keeps it alive until the work
 *    queued on `stream` has completed.  The library keeps no pointer beyond
 *    the call.  `stream` is a hipStream_t passed as void* (NULL = default
 *    stream); work is queued asynchronously on it.
 *  - Errors are returned as nbw_status.  All argument checks run on the host
 *    before any device work is queued; on error nothing is queued.  NBW_EHIP
 *    means a HIP runtime call failed: nbw_last_hip_error() returns its
 *    hipError_t for the calling thread.  Faults inside a kernel surface at the
 *    caller's next synchronisation, as with any HIP launch.
 *  - Calls are thread-safe.  Calls queued on different streams may overlap;
 *    they share no library state apart from one device-property cache.
 *
 * Data formats
 *  - Parent codes: uint8 [n][k] row-major, c in [0, 255].
 *  - Child codes: q_r = c >> (8 - r), r in 1..8 (the MatGPTQ pages run 2..8).
 *  - Bit-planes (layout NBW_LAYOUT_T16): eight planes, plane p holding bit
 *    (7 - p) of every code, so plane 0 is the MSB and the r-bit child is the
 *    byte prefix of r planes.  Rows are padded to a multiple of 16 (padding
 *    bits 0); plane_bytes = ceil(n/16)*16 * k/8.  The 16-byte chunk of
 *    (plane p, row i, group g = j/128) starts at
 *        p*plane_bytes + ((i/16)*(k/128) + g)*256 + (i%16)*16,
 *    and column c = j%128 of that chunk sits in little-endian 32-bit word c/32
 *    at bit (c%32)/2 + 16*(c%2): even columns in bits 0..15, odd columns in
 *    bits 16..31 of each word.  So one 16-row tile of one group is 256
 *    contiguous bytes per plane, and the two columns of a bf16 pair sit at
 *    the same bit of the two 16-bit halves of a word.
 *  - Scales: bf16 [n][k/128] row-major, one per row and 128-wide group of k.
 *  - Dequantisation of a child code (the pages state no formula; this library
 *    uses the symmetric mid-point grid, which puts the child value at the
 *    mean of its parent bucket):
 *        w = s * 2^(8-r) * (q_r + 1/2 - 2^(r-1)).
 *  - X: bf16 [batch][k] row-major.  Y: fp32 [batch][n] row-major,
 *        Y[b][i] = sum_j X[b][j] * w[i][j]   (fp32 accumulation).
 *  - k must be a positive multiple of 128; n >= 1; batch >= 0.
 *
 * Alignment: planes, X and Y 16 bytes; scales 4 bytes; codes 16 bytes.
 */
#ifndef NBW_H
#define NBW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nbw_status {
    NBW_OK = 0,
    NBW_EINVAL = 1,       /* null pointer, bad size, k not a multiple of 128, batch < 1 */
    NBW_EALIGN = 2,       /* a pointer misses its required alignment */
    NBW_ERANGE = 3,       /* r outside 1..8, or r larger than the planes present */
    NBW_EUNSUPPORTED = 4, /* unknown layout or kernel selector */
    NBW_EHIP = 5,         /* a HIP runtime call failed (see nbw_last_hip_error) */
    NBW_ESCRATCH = 6      /* nbw_qgemm_noalloc: the problem needs more scratch than
                             NBW_NOALLOC_SCRATCH_BYTES */
} nbw_status;

#define NBW_LAYOUT_T16 1

/* A view of packed weights: `nplanes` consecutive planes of `plane_bytes`
 * each, starting at device pointer `planes` (plane 0 = MSB).  A parent view
 * has nplanes = 8; an r-bit child view has nplanes = r and the same base. */
typedef struct nbw_wview {
    const void *planes;
    int64_t n;           /* rows (output features) */
    int64_t k;           /* columns (input features), multiple of 128 */
    int32_t nplanes;     /* planes present at `planes` */
    int32_t layout;      /* NBW_LAYOUT_T16 */
    int64_t plane_bytes; /* ceil(n/16)*16*k/8 */
} nbw_wview;

/* Kernel selectors for nbw_qgemm_kernel.  NBW_KERNEL_AUTO picks by batch:
 * 1..4 -> GEMV; otherwise SMALLB while it needs one pass over the planes, or
 * two passes and k <= 8192 (a pass covers 32 batch rows for r <= 4 when the
 * workgroups' tile runs are short, else 16); otherwise GEMM.  Batches 5..16
 * always take SMALLB and batches above 64 always GEMM. */
typedef enum nbw_kernel {
    NBW_KERNEL_AUTO = 0,
    NBW_KERNEL_GEMV = 1,   /* streaming dequant feeding MFMA, 4 batch rows per launch */
    NBW_KERNEL_SMALLB = 2, /* in-register dequant feeding MFMA, 16 or 32 batch rows per pass */
    NBW_KERNEL_GEMM = 3    /* large-batch MFMA kernel */
} nbw_kernel;

/* Bytes of one plane for an n x k matrix, or -1 if n < 1 or k is not a
 * positive multiple of 128. */
int64_t nbw_plane_bytes(int64_t n, int64_t k);

/* Bytes read by an r-bit child: r * nbw_plane_bytes(n, k) (-1 on bad input). */
int64_t nbw_packed_bytes(int64_t n, int64_t k, int32_t r);

/* Pack parent codes into the 8 MSB-first bit-planes of layout NBW_LAYOUT_T16
 * (MatGPTQ v2, Abstract and Table 1: one checkpoint whose r-bit child reads
 * exactly r bits).  codes: device uint8 [n][k]; planes_out: device buffer of
 * planes_out_bytes >= 8*nbw_plane_bytes(n, k), fully written (padding rows
 * included).  Bit-exact; runs on `stream`. */
nbw_status nbw_pack_bitplanes(const uint8_t *codes, int64_t n, int64_t k, void *planes_out,
                              int64_t planes_out_bytes, void *stream);

/* Describe `nplanes` planes (1..8) of an n x k matrix at device pointer
 * `planes`.  Host only; no device work. */
nbw_status nbw_make_view(const void *planes, int64_t n, int64_t k, int32_t nplanes,
                         nbw_wview *out);

/* The r-bit child of a view: same base pointer, nplanes = r (MatGPTQ v1
 * abstract: lower precisions by slicing the most significant bits).  Host
 * only; no device work, no data read.  NBW_ERANGE if r < 1 or
 * r > parent->nplanes. */
nbw_status nbw_slice_view(const nbw_wview *parent, int32_t r, nbw_wview *child);

/* Y = X . dequant_r(W)^T for the r-bit child of `w` (MatGPTQ: Efficient and
 * Accurate Inference over Nested Quantized Models, Abstract: an r-bit model
 * reads exactly r bits, and the kernels serve batch sizes beyond one; Table 1,
 * row "Exact r-bit loading").  Reads planes 0..r-1 only, plus the scales and
 * X.  x_bf16: [batch][k]; scales_bf16: [n][k/128]; y: fp32 [batch][n], fully
 * written.  batch == 0 is an empty product: NBW_OK, nothing queued,
 * x/scales/y unused.  The kernel is chosen by batch size.  No workspace is
 * used, so a large-batch launch runs unsplit; Y is deterministic (the same
 * inputs give bit-identical Y).  Allocates nothing.  Runs on `stream`. */
nbw_status nbw_qgemm(const void *x_bf16, int64_t batch, const nbw_wview *w,
                     const void *scales_bf16, int32_t r, float *y, void *stream);

/* nbw_qgemm with an explicit kernel choice (every kernel accepts every batch
 * size; used to test and time each kernel on its own). */
nbw_status nbw_qgemm_kernel(const void *x_bf16, int64_t batch, const nbw_wview *w,
                            const void *scales_bf16, int32_t r, float *y, nbw_kernel kernel,
                            void *stream);

/* Output element type of nbw_qgemm_ex. */
typedef enum nbw_ydtype {
    NBW_Y_F32 = 0,  /* fp32 (the accumulation itself) */
    NBW_Y_BF16 = 1  /* bf16, the fp32 result rounded to nearest even */
} nbw_ydtype;

/* Options of nbw_qgemm_ex.  A zero-filled struct gives nbw_qgemm's
 * behaviour (dense X and Y, fp32 Y, symmetric children, automatic kernel). */
typedef struct nbw_qgemm_opts {
    int64_t ldx;        /* elements from one X row to the next: 0 (= k) or >= k,
                           a multiple of 8 (X rows stay 16-byte aligned) */
    int64_t ldy;        /* elements from one Y row to the next: 0 (= n) or >= n */
    int32_t y_dtype;    /* nbw_ydtype */
    int32_t kernel;     /* nbw_kernel */
    const void *zeros_bf16; /* NULL: symmetric children.  Otherwise asymmetric
                           children, bf16 zero points [n][k/128] (4-byte
                           aligned, the scales' layout): the parent grid is
                           s * (c - z) and an r-bit child is the mean of its
                           parent bucket, w = s * (2^(8-r) * (q_r + 1/2) - 1/2 - z)
                           (the pages evaluate an asymmetric variant, MatGPTQ v2
                           Tables 4-7, without stating its formula; z = 127.5
                           gives the symmetric child exactly). */
    void *workspace;    /* NULL, or caller-owned device scratch (256-byte
                           aligned) of workspace_bytes bytes; no initial
                           contents are needed.  When it holds at least
                           nbw_qgemm_workspace_bytes(...) bytes, a large-batch
                           launch whose output tiles leave compute units idle
                           splits k and meets its splits there: each split
                           stores its fp32 partial tile and a second launch on
                           the same stream adds them in a fixed order.
                           Without it (NULL or too small) the launch runs
                           unsplit.  Either way the result is deterministic:
                           the same inputs give bit-identical Y on every call.
                           Calls that overlap in time must not share a
                           workspace. */
    int64_t workspace_bytes;
} nbw_qgemm_opts;

/* Bytes of workspace nbw_qgemm_ex uses for this problem and kernel choice
 * (0: the launch does not split k, or batch is 0, and needs none), or -1 on
 * bad arguments.
 * Host only; queries the device's compute-unit count once. */
int64_t nbw_qgemm_workspace_bytes(int64_t batch, int64_t n, int64_t k, int32_t r, nbw_kernel kernel);

/* nbw_qgemm with row strides, a bf16 output, asymmetric children and a
 * split-k workspace (opts == NULL: as nbw_qgemm).  y points at fp32 or bf16
 * elements per opts->y_dtype; only the first n elements of each Y row are
 * written.  Same errors as nbw_qgemm, plus NBW_EINVAL for a stride below k or
 * n or a negative workspace_bytes, NBW_EALIGN for a stride that breaks the row
 * alignment or a misaligned workspace; NBW_EUNSUPPORTED for an unknown
 * y_dtype or kernel. */
nbw_status nbw_qgemm_ex(const void *x_bf16, int64_t batch, const nbw_wview *w,
                        const void *scales_bf16, int32_t r, void *y, const nbw_qgemm_opts *opts,
                        void *stream);

/* Size of the static device scratch behind nbw_qgemm_noalloc (64 MiB per
 * device that runs it, held until the process ends). */
#define NBW_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)

/* nbw_qgemm_ex for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It calls no
 * hipMalloc, hipFree or other allocating routine.  Where a large-batch launch
 * splits k, its partial tiles go to a static device scratch array of the
 * library (NBW_NOALLOC_SCRATCH_BYTES, one per device, its address looked up
 * once per device on the first call there) instead of a caller workspace;
 * results are bit-identical to nbw_qgemm_ex given a large enough workspace.
 * Same arguments and errors as nbw_qgemm_ex, except: opts->workspace must be
 * NULL and opts->workspace_bytes 0 (NBW_EINVAL otherwise), and a problem
 * whose split needs more than NBW_NOALLOC_SCRATCH_BYTES
 * (nbw_qgemm_workspace_bytes) returns NBW_ESCRATCH with nothing queued.  Every
 * call on a device shares that device's scratch and leaves it holding its
 * partial tiles (no initial contents are needed): calls that overlap in time
 * on one device -- on two streams, or from two threads -- race on it and must
 * be serialised by the caller. */
nbw_status nbw_qgemm_noalloc(const void *x_bf16, int64_t batch, const nbw_wview *w,
                             const void *scales_bf16, int32_t r, void *y,
                             const nbw_qgemm_opts *opts, void *stream);

/* Data-free parent-code choice: for every fp32 weight w[i][j] (device, [n][k])
 * with group scale s[i][j/128] (device bf16 [n][k/128]), the code c in 0..255
 * minimising sum_t lambdas[t] * (w - dequant_{widths[t]}(c))^2 over the
 * children r = widths[t] (symmetric closed form above); the first code with
 * the smallest loss wins (MatGPTQ v2, captions of Tables 6 and 7: per-precision
 * weights lambda_r; MatGPTQ v1 abstract: one parent serves every sliced width).  Every
 * code is tried in IEEE double, one rounded operation at a time.  widths and
 * lambdas are HOST arrays of nw (1..8) entries; widths in 1..8, lambdas >= 0
 * and finite.  codes_out: device uint8 [n][k] (ready for nbw_pack_bitplanes).
 * Runs on `stream`. */
nbw_status nbw_choose_codes(const float *w, int64_t n, int64_t k, const void *scales_bf16,
                            const int32_t *widths, const double *lambdas, int32_t nw,
                            uint8_t *codes_out, void *stream);

/* One product of a grouped call: Y = X . dequant_r(W)^T for the r-bit child
 * of `w`, with the same arguments as nbw_qgemm. */
typedef struct nbw_problem {
    const void *x_bf16;      /* [batch][k] */
    int64_t batch;
    nbw_wview w;             /* weights (a parent or child view) */
    const void *scales_bf16; /* [n][k/128] */
    int32_t r;               /* child width, 1..w.nplanes */
    float *y;                /* [batch][n] */
} nbw_problem;

/* Several products queued as few dispatches as possible -- for example the
 * linears of one decoder layer, each sliced to its own r (MatGPTQ: Accurate
 * and Efficient Post-Training Matryoshka Quantization, abstract: mixed-
 * precision execution over heterogeneous per-layer bit-widths).  Results are
 * those of calling nbw_qgemm on each problem in order on `stream`; since the
 * problems may run concurrently, no problem's output may overlap another's
 * inputs or output.  Batch 1..4 problems run as grouped launches of the
 * streaming kernel (one for batch 1, one for batch 2..4) and batch-5..16
 * problems as one grouped launch of the small-batch kernel (k/128 a multiple
 * of 4; up to 32 products per launch), each bit-identical to its single call;
 * others are queued one by one.
 * Every problem is validated before anything is queued. */
nbw_status nbw_qgemm_grouped(const nbw_problem *problems, int32_t count, void *stream);

/* Child codes q_r = c >> (8 - r) read back from planes 0..r-1 of `w`, through
 * the same in-register plane decode the qgemm kernels use (MatGPTQ: Accurate
 * and Efficient Post-Training Matryoshka Quantization, abstract: a lower
 * precision is the parent's most significant bits; MatGPTQ: Efficient and
 * Accurate Inference over Nested Quantized Models, Abstract: reading fewer
 * bits of the weights).  codes_out: device uint8 [n][k], fully written.  A
 * test hook for the bit-exact slicing check.  Errors: NBW_EINVAL (null
 * pointer or bad view), NBW_ERANGE (r outside 1..w->nplanes), NBW_EALIGN
 * (codes_out not 16-byte aligned), NBW_EHIP.  Runs on `stream`. */
nbw_status nbw_unpack_codes(const nbw_wview *w, int32_t r, uint8_t *codes_out, void *stream);

/* Bandwidth reference for the batch-1 products (MatGPTQ: Efficient and
 * Accurate Inference over Nested Quantized Models, Table 1: an r-bit child
 * loads r/8 bytes per weight, so a batch-1 product is a single pass over its
 * plane bytes): one launch that reads the device range [src, src + bytes)
 * with 16-byte loads and does nothing else, i.e. the time floor a product
 * of that many plane bytes is measured against.
 * src: device pointer, 16-byte aligned; bytes: a multiple of 16, >= 0.
 * sink: device uint32 array of nbw_stream_sink_words() words (caller-owned),
 * fully written: word i is the XOR of the 32-bit words wave i read, so the
 * XOR of all sink words is the XOR of every 32-bit word of the range.
 * Errors: NBW_EINVAL (null pointer, negative or non-multiple-of-16 bytes),
 * NBW_EALIGN (src or sink misaligned), NBW_EHIP (launch failed).  Asynchronous
 * on `stream`. */
int32_t nbw_stream_sink_words(void);
nbw_status nbw_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);

/* Matrix-unit reference for the products beyond batch one (MatGPTQ:
 * Efficient and Accurate Inference over Nested Quantized Models, Abstract:
 * kernels that serve batch sizes beyond one; at batch 128-256 the products
 * are bound by v_mfma_f32_32x32x16_bf16): one launch of `iters` rounds in
 * which every wave issues 64 of those instructions and nothing else (four
 * independent accumulator chains, two waves per SIMD, one workgroup of 8
 * waves per compute unit), the operands cycling through 8 A and 8 B
 * fragments held in registers.  Its rate is the ceiling the products are
 * measured against on the same chip and operand data.
 * ops: device pointer, 16-byte aligned, 16 KB: fragment f (0..15) of lane l
 * (0..63) is the 16 bytes at (f * 64 + l) * 16, eight bf16 values in the
 * instruction's operand layout; f < 8 are A operands, f >= 8 B operands.
 * Round MFMA s (0..63) multiplies A fragment s % 8 by B fragment (s / 8) % 8
 * into accumulator s % 4.  iters >= 1.
 * sink: device float array of nbw_mfma_rate_sink_floats() floats
 * (caller-owned), fully written: float t is thread t's sum of its four
 * accumulators (every wave computes the same values).  A launch performs
 * (nbw_mfma_rate_sink_floats() / 64) * iters * 64 * 32768 flops.
 * Errors: NBW_EINVAL (null pointer, iters < 1), NBW_EALIGN, NBW_EHIP (no
 * device or launch failed; nbw_mfma_rate_sink_floats then returns -1).
 * Asynchronous on `stream`. */
int64_t nbw_mfma_rate_sink_floats(void);
nbw_status nbw_mfma_rate(const void *ops, int32_t iters, float *sink, void *stream);

/* On-disk form of a sliceable parent (host only, no device work).  The r-bit
 * child loads exactly r bits per weight (MatGPTQ: Efficient and Accurate
 * Inference over Nested Quantized Models, Abstract; Table 1, row "Exact r-bit
 * loading"), so the file keeps the scales ahead of the planes and the planes
 * MSB first: the first nbw_file_prefix_bytes(n, k, r) bytes of a parent file
 * hold everything an r-bit child needs, and a file cut after them is itself a
 * valid child file.  Layout (integers little-endian):
 *   [0, NBW_FILE_HEADER_BYTES)  header, written by nbw_file_header
 *   scales_offset               bf16 scales [n][k/128] row-major
 *   planes_offset               plane p at planes_offset + p*plane_bytes
 *                               (p = 0..7, plane 0 = MSB), byte for byte the
 *                               device layout NBW_LAYOUT_T16
 * planes_offset = NBW_FILE_HEADER_BYTES + the scale bytes rounded up to a
 * multiple of 4096. */
#define NBW_FILE_HEADER_BYTES 4096

typedef struct nbw_file_info {
    int64_t n, k;
    int32_t nplanes;        /* planes the writer stored (8 for a parent) */
    int32_t layout;         /* NBW_LAYOUT_T16 */
    int64_t plane_bytes;    /* nbw_plane_bytes(n, k) */
    int64_t scales_offset;  /* NBW_FILE_HEADER_BYTES */
    int64_t scales_bytes;   /* n * (k/128) * 2 */
    int64_t planes_offset;
    int32_t planes_present; /* whole planes within the first file_bytes bytes (0..nplanes) */
    int32_t reserved;
} nbw_file_info;

/* Bytes of a parent file's prefix that holds the header, the scales and
 * planes 0..r-1 (r = 0..8; r = 0 gives planes_offset), or -1 on bad input. */
int64_t nbw_file_prefix_bytes(int64_t n, int64_t k, int32_t r);

/* Writes the NBW_FILE_HEADER_BYTES-byte header of an 8-plane parent file for
 * an n x k matrix into the host buffer header_out (caller-owned).
 * Errors: NBW_EINVAL (null buffer, bad shape). */
nbw_status nbw_file_header(int64_t n, int64_t k, void *header_out);

/* Checks a header (host buffer of NBW_FILE_HEADER_BYTES bytes) and describes
 * the file, given that its first file_bytes bytes are available (the whole
 * file, or a prefix of it): info->planes_present says how many whole planes
 * that prefix holds, so a child of r <= planes_present can be loaded.
 * Errors: NBW_EINVAL (null pointer, wrong magic or header size, a field that
 * disagrees with the layout), NBW_EUNSUPPORTED (unknown layout, scale type or
 * group size), NBW_ERANGE (the prefix ends before the planes start). */
nbw_status nbw_file_parse(const void *header, int64_t file_bytes, nbw_file_info *info);

/* Name of the kernel template instance nbw_qgemm_kernel would launch for
 * this problem on the current device (for example "nbw::gemv_kernel<4, 1, 2>",
 * as profilers print it without the parameter list), or "" on bad input.  The
 * string lives until the calling thread's next call.  Host only; queries the
 * device's compute-unit count once. */
const char *nbw_kernel_name(int64_t batch, int64_t n, int64_t k, int32_t r, nbw_kernel kernel);

/* Static text for a status code. */
const char *nbw_status_str(nbw_status s);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int32_t nbw_last_hip_error(void);

/* Library version string. */
const char *nbw_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NBW_H */
