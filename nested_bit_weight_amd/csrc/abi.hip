// abi.hip -- the extern "C" entry points of libnbw (see include/nbw.h).
//
// Host code only: argument validation, weight views, kernel choice by batch
// size, and launches on the caller's stream.  Every check runs before any
// HIP call, so a rejected call queues nothing.
#include <climits>
#include <mutex>
#include <vector>

#include "launch.h"
#include "nbw.h"

// Scratch of nbw_qgemm_noalloc: the split-k partial tiles of a large-batch
// launch live here instead of in a caller workspace.  One copy per device,
// held until the process ends; its device address is taken once per device
// (scratch_ptr below) -- the name itself is a host-side stand-in.
static __device__ __align__(256) unsigned char scratch[NBW_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int32_t g_last_hip_error = 0;

nbw_status hip_failed(hipError_t e) {
    g_last_hip_error = (int32_t)e;
    return NBW_EHIP;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool shape_ok(int64_t n, int64_t k) {
    return n >= 1 && n <= INT_MAX - 16 && k >= 128 && k % 128 == 0 && k <= INT_MAX;
}

// Compute-unit count of the current device, cached per device.
nbw_status cu_count(int *out) {
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_failed(e);
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
    if (cache[dev] == 0) {
        int v = 0;
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_failed(e);
        cache[dev] = v > 0 ? v : 1;
    }
    *out = cache[dev];
    return NBW_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and cached.
nbw_status scratch_ptr(void **out) {
    static std::mutex mu;
    static std::vector<void *> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_failed(e);
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1, nullptr);
    if (!cache[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_failed(e);
        if (!p) return NBW_EHIP;
        cache[dev] = p;
    }
    *out = cache[dev];
    return NBW_OK;
}

nbw_status check_view(const nbw_wview *w) {
    if (!w || !w->planes) return NBW_EINVAL;
    if (!shape_ok(w->n, w->k)) return NBW_EINVAL;
    if (w->layout != NBW_LAYOUT_T16) return NBW_EUNSUPPORTED;
    if (w->nplanes < 1 || w->nplanes > 8) return NBW_ERANGE;
    if (w->plane_bytes != nbw_plane_bytes(w->n, w->k)) return NBW_EINVAL;
    if (!aligned(w->planes, 16)) return NBW_EALIGN;
    return NBW_OK;
}

// NBW_KERNEL_AUTO: batch 1..4 -> GEMV (up to four batch rows ride in one
// launch at about the cost of one; measured on the 70B, Qwen3-8B and
// Llama-3.1-8B linears at batch 2 and 4: 3-20% faster than the small-batch
// kernel).  Otherwise the small-batch kernel while
// it needs at most two passes over the planes (16 or 32 batch rows a pass)
// and, for two, k <= 8192; else the large-batch GEMM, which reads the planes
// about once at any batch.  (Measured on the Llama-3.1-8B linears at r = 2..8:
// two passes beat the GEMM except on down, k = 14336, where every workgroup
// reads the whole of X each pass; four passes lose.)  Batches up to 16 and
// above 64 need no device query.
nbw_status auto_kernel(int64_t batch, int64_t n, int64_t k, int32_t r, int *kernel) {
    if (batch <= nbw::gemv_max_batch()) {
        *kernel = NBW_KERNEL_GEMV;
        return NBW_OK;
    }
    if (batch <= 16 || batch > 64) {
        *kernel = batch <= 16 ? NBW_KERNEL_SMALLB : NBW_KERNEL_GEMM;
        return NBW_OK;
    }
    int cus = 0;
    const nbw_status st = cu_count(&cus);
    if (st != NBW_OK) return st;
    const int64_t rows = nbw::smallb_pass_rows(r, (int)n, cus);
    const int64_t passes = (batch + rows - 1) / rows;
    *kernel = passes == 1 || (passes == 2 && k <= 8192) ? NBW_KERNEL_SMALLB : NBW_KERNEL_GEMM;
    return NBW_OK;
}

}  // namespace

extern "C" {

int64_t nbw_plane_bytes(int64_t n, int64_t k) {
    if (!shape_ok(n, k)) return -1;
    return (n + 15) / 16 * 16 * (k / 8);
}

int64_t nbw_packed_bytes(int64_t n, int64_t k, int32_t r) {
    const int64_t pb = nbw_plane_bytes(n, k);
    if (pb < 0 || r < 1 || r > 8) return -1;
    return r * pb;
}

nbw_status nbw_pack_bitplanes(const uint8_t *codes, int64_t n, int64_t k, void *planes_out,
                              int64_t planes_out_bytes, void *stream) {
    if (!codes || !planes_out) return NBW_EINVAL;
    if (!shape_ok(n, k)) return NBW_EINVAL;
    const int64_t pb = nbw_plane_bytes(n, k);
    if (planes_out_bytes < 8 * pb) return NBW_EINVAL;
    if (!aligned(codes, 16) || !aligned(planes_out, 16)) return NBW_EALIGN;
    hipError_t e = nbw::launch_pack(codes, (int)n, (int)k, (uint8_t *)planes_out, pb,
                                    (hipStream_t)stream);
    return e == hipSuccess ? NBW_OK : hip_failed(e);
}

nbw_status nbw_make_view(const void *planes, int64_t n, int64_t k, int32_t nplanes,
                         nbw_wview *out) {
    if (!out || !planes) return NBW_EINVAL;
    if (!shape_ok(n, k)) return NBW_EINVAL;
    if (nplanes < 1 || nplanes > 8) return NBW_ERANGE;
    if (!aligned(planes, 16)) return NBW_EALIGN;
    out->planes = planes;
    out->n = n;
    out->k = k;
    out->nplanes = nplanes;
    out->layout = NBW_LAYOUT_T16;
    out->plane_bytes = nbw_plane_bytes(n, k);
    return NBW_OK;
}

nbw_status nbw_slice_view(const nbw_wview *parent, int32_t r, nbw_wview *child) {
    if (!child) return NBW_EINVAL;
    nbw_status st = check_view(parent);
    if (st != NBW_OK) return st;
    if (r < 1 || r > parent->nplanes) return NBW_ERANGE;
    *child = *parent;
    child->nplanes = r;
    return NBW_OK;
}

nbw_status nbw_qgemm_ex(const void *x_bf16, int64_t batch, const nbw_wview *w,
                        const void *scales_bf16, int32_t r, void *y, const nbw_qgemm_opts *opts,
                        void *stream) {
    nbw_qgemm_opts o = {};
    if (opts) o = *opts;
    nbw_status st = check_view(w);
    if (st != NBW_OK) return st;
    if (batch < 0) return NBW_EINVAL;
    if (r < 1 || r > 8 || r > w->nplanes) return NBW_ERANGE;
    if (o.kernel < NBW_KERNEL_AUTO || o.kernel > NBW_KERNEL_GEMM) return NBW_EUNSUPPORTED;
    if (o.y_dtype != NBW_Y_F32 && o.y_dtype != NBW_Y_BF16) return NBW_EUNSUPPORTED;
    const int64_t ldx = o.ldx ? o.ldx : w->k, ldy = o.ldy ? o.ldy : w->n;
    if (ldx < w->k || ldy < w->n) return NBW_EINVAL;
    if (batch == 0) return NBW_OK;  // empty product: nothing to read or write
    if (!x_bf16 || !scales_bf16 || !y) return NBW_EINVAL;
    const bool ybf16 = o.y_dtype == NBW_Y_BF16;
    if (!aligned(x_bf16, 16) || !aligned(y, 16) || !aligned(scales_bf16, 4)) return NBW_EALIGN;
    if (o.zeros_bf16 && !aligned(o.zeros_bf16, 4)) return NBW_EALIGN;
    if (ldx % 8 != 0) return NBW_EALIGN;  // X rows are read with 16-byte loads
    if (o.workspace_bytes < 0) return NBW_EINVAL;
    if (o.workspace && !aligned(o.workspace, 256)) return NBW_EALIGN;
    int cus = 0;
    st = cu_count(&cus);
    if (st != NBW_OK) return st;
    int kernel = o.kernel;
    if (kernel == NBW_KERNEL_AUTO) {
        st = auto_kernel(batch, w->n, w->k, r, &kernel);
        if (st != NBW_OK) return st;
    }
    nbw::QgemmArgs a;
    a.x = (const uint16_t *)x_bf16;
    a.batch = batch;
    a.planes = (const uint8_t *)w->planes;
    a.plane_bytes = w->plane_bytes;
    a.scales = (const uint16_t *)scales_bf16;
    a.n = (int)w->n;
    a.k = (int)w->k;
    a.y = (float *)y;
    a.ldx = ldx;
    a.ldy = ldy;
    a.ybf16 = ybf16 ? 1 : 0;
    a.zeros = (const uint16_t *)o.zeros_bf16;
    a.ws = o.workspace;
    a.ws_bytes = o.workspace ? o.workspace_bytes : 0;
    hipError_t e;
    switch (kernel) {
    case NBW_KERNEL_GEMV: e = nbw::launch_gemv(r, a, cus, (hipStream_t)stream); break;
    case NBW_KERNEL_SMALLB: e = nbw::launch_smallb(r, a, cus, (hipStream_t)stream); break;
    default: e = nbw::launch_gemm(r, a, cus, (hipStream_t)stream); break;
    }
    return e == hipSuccess ? NBW_OK : hip_failed(e);
}

nbw_status nbw_qgemm_noalloc(const void *x_bf16, int64_t batch, const nbw_wview *w,
                             const void *scales_bf16, int32_t r, void *y,
                             const nbw_qgemm_opts *opts, void *stream) {
    nbw_qgemm_opts o = {};
    if (opts) o = *opts;
    if (o.workspace || o.workspace_bytes) return NBW_EINVAL;  // the scratch replaces it
    const nbw_status st = check_view(w);
    if (st != NBW_OK) return st;
    if (r < 1 || r > 8 || r > w->nplanes) return NBW_ERANGE;
    if (o.kernel < NBW_KERNEL_AUTO || o.kernel > NBW_KERNEL_GEMM) return NBW_EUNSUPPORTED;
    const int64_t need = nbw_qgemm_workspace_bytes(batch, w->n, w->k, r, (nbw_kernel)o.kernel);
    if (need < 0) return NBW_EINVAL;
    if (need > NBW_NOALLOC_SCRATCH_BYTES) return NBW_ESCRATCH;
    if (need > 0) {
        void *p = nullptr;
        const nbw_status sp = scratch_ptr(&p);
        if (sp != NBW_OK) return sp;
        o.workspace = p;
        o.workspace_bytes = NBW_NOALLOC_SCRATCH_BYTES;
    }
    return nbw_qgemm_ex(x_bf16, batch, w, scales_bf16, r, y, &o, stream);
}

nbw_status nbw_qgemm_kernel(const void *x_bf16, int64_t batch, const nbw_wview *w,
                            const void *scales_bf16, int32_t r, float *y, nbw_kernel kernel,
                            void *stream) {
    nbw_qgemm_opts o = {};
    o.kernel = kernel;
    return nbw_qgemm_ex(x_bf16, batch, w, scales_bf16, r, y, &o, stream);
}

nbw_status nbw_choose_codes(const float *w, int64_t n, int64_t k, const void *scales_bf16,
                            const int32_t *widths, const double *lambdas, int32_t nw,
                            uint8_t *codes_out, void *stream) {
    if (!w || !scales_bf16 || !codes_out || !widths || !lambdas) return NBW_EINVAL;
    if (!shape_ok(n, k)) return NBW_EINVAL;
    if (nw < 1 || nw > 8) return NBW_EINVAL;
    nbw::ChooseSpec spec = {};
    spec.nw = nw;
    for (int t = 0; t < nw; ++t) {
        if (widths[t] < 1 || widths[t] > 8) return NBW_ERANGE;
        // lambdas must be finite and >= 0 (this also rejects NaN)
        if (!(lambdas[t] >= 0.0 && lambdas[t] <= 1.7976931348623157e308)) return NBW_EINVAL;
        spec.widths[t] = widths[t];
        spec.lambdas[t] = lambdas[t];
    }
    if (!aligned(w, 4) || !aligned(scales_bf16, 2)) return NBW_EALIGN;
    hipError_t e = nbw::launch_choose(w, n, (int)k, (const uint16_t *)scales_bf16, spec, codes_out,
                                      (hipStream_t)stream);
    return e == hipSuccess ? NBW_OK : hip_failed(e);
}

nbw_status nbw_qgemm_grouped(const nbw_problem *problems, int32_t count, void *stream) {
    if (count < 0 || (count > 0 && !problems)) return NBW_EINVAL;
    // Validate everything before queuing anything.
    for (int32_t j = 0; j < count; ++j) {
        const nbw_problem &pr = problems[j];
        nbw_status st = check_view(&pr.w);
        if (st != NBW_OK) return st;
        if (pr.batch < 0) return NBW_EINVAL;
        if (pr.r < 1 || pr.r > 8 || pr.r > pr.w.nplanes) return NBW_ERANGE;
        if (pr.batch == 0) continue;
        if (!pr.x_bf16 || !pr.scales_bf16 || !pr.y) return NBW_EINVAL;
        if (!aligned(pr.x_bf16, 16) || !aligned(pr.y, 16) || !aligned(pr.scales_bf16, 4))
            return NBW_EALIGN;
    }
    int cus = 0;
    nbw_status st = cu_count(&cus);
    if (st != NBW_OK) return st;
    // Batch 1..4 products go to the streaming kernel's grouped launch, batch
    // 5..16 ones to the small-batch kernel's; each flushes when full.
    std::vector<nbw::QgemmArgs> group, sgroup;
    std::vector<int> rs, srs;
    const int cap = nbw::gemv_group_capacity(), scap = nbw::smallb_group_capacity();
    auto flush = [&]() -> nbw_status {
        if (group.empty()) return NBW_OK;
        hipError_t e = nbw::launch_gemv_group(group.data(), rs.data(), (int)group.size(), cus,
                                              (hipStream_t)stream);
        group.clear();
        rs.clear();
        return e == hipSuccess ? NBW_OK : hip_failed(e);
    };
    auto sflush = [&]() -> nbw_status {
        if (sgroup.empty()) return NBW_OK;
        hipError_t e = nbw::launch_smallb_group(sgroup.data(), srs.data(), (int)sgroup.size(), cus,
                                                (hipStream_t)stream);
        sgroup.clear();
        srs.clear();
        return e == hipSuccess ? NBW_OK : hip_failed(e);
    };
    for (int32_t j = 0; j < count; ++j) {
        const nbw_problem &pr = problems[j];
        if (pr.batch == 0) continue;
        nbw::QgemmArgs a;
        a.x = (const uint16_t *)pr.x_bf16;
        a.batch = pr.batch;
        a.planes = (const uint8_t *)pr.w.planes;
        a.plane_bytes = pr.w.plane_bytes;
        a.scales = (const uint16_t *)pr.scales_bf16;
        a.n = (int)pr.w.n;
        a.k = (int)pr.w.k;
        a.y = pr.y;
        if (nbw::gemv_group_eligible(a)) {
            group.push_back(a);
            rs.push_back(pr.r);
            if ((int)group.size() == cap && (st = flush()) != NBW_OK) return st;
        } else if (nbw::smallb_group_eligible(a)) {
            sgroup.push_back(a);
            srs.push_back(pr.r);
            if ((int)sgroup.size() == scap && (st = sflush()) != NBW_OK) return st;
        } else {
            st = nbw_qgemm(pr.x_bf16, pr.batch, &pr.w, pr.scales_bf16, pr.r, pr.y, stream);
            if (st != NBW_OK) return st;
        }
    }
    if ((st = flush()) != NBW_OK) return st;
    return sflush();
}

nbw_status nbw_qgemm(const void *x_bf16, int64_t batch, const nbw_wview *w,
                     const void *scales_bf16, int32_t r, float *y, void *stream) {
    return nbw_qgemm_kernel(x_bf16, batch, w, scales_bf16, r, y, NBW_KERNEL_AUTO, stream);
}

nbw_status nbw_unpack_codes(const nbw_wview *w, int32_t r, uint8_t *codes_out, void *stream) {
    if (!codes_out) return NBW_EINVAL;
    nbw_status st = check_view(w);
    if (st != NBW_OK) return st;
    if (r < 1 || r > 8 || r > w->nplanes) return NBW_ERANGE;
    if (!aligned(codes_out, 16)) return NBW_EALIGN;
    hipError_t e = nbw::launch_unpack(r, (const uint8_t *)w->planes, w->plane_bytes, (int)w->n,
                                      (int)w->k, codes_out, (hipStream_t)stream);
    return e == hipSuccess ? NBW_OK : hip_failed(e);
}

int64_t nbw_qgemm_workspace_bytes(int64_t batch, int64_t n, int64_t k, int32_t r, nbw_kernel kernel) {
    if (!shape_ok(n, k) || batch < 0 || r < 1 || r > 8 || kernel < NBW_KERNEL_AUTO ||
        kernel > NBW_KERNEL_GEMM)
        return -1;
    if (batch == 0) return 0;
    int kn = kernel;
    if (kn == NBW_KERNEL_AUTO && auto_kernel(batch, n, k, r, &kn) != NBW_OK) return -1;
    if (kn != NBW_KERNEL_GEMM) return 0;
    int cus = 0;
    if (cu_count(&cus) != NBW_OK) return -1;
    nbw::QgemmArgs a = {};
    a.batch = batch;
    a.n = (int)n;
    a.k = (int)k;
    return nbw::gemm_workspace_bytes(a, cus);
}

int32_t nbw_stream_sink_words(void) { return nbw::stream_sink_words(); }

nbw_status nbw_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream) {
    if (!src || !sink || bytes < 0 || bytes % 16) return NBW_EINVAL;
    if (!aligned(src, 16) || !aligned(sink, 4)) return NBW_EALIGN;
    hipError_t e = nbw::launch_stream_read(src, bytes, sink, (hipStream_t)stream);
    return e == hipSuccess ? NBW_OK : hip_failed(e);
}

int64_t nbw_mfma_rate_sink_floats(void) {
    int cus = 0;
    if (cu_count(&cus) != NBW_OK) return -1;
    return nbw::mfma_rate_threads(cus);
}

nbw_status nbw_mfma_rate(const void *ops, int32_t iters, float *sink, void *stream) {
    if (!ops || !sink || iters < 1) return NBW_EINVAL;
    if (!aligned(ops, 16) || !aligned(sink, 4)) return NBW_EALIGN;
    int cus = 0;
    const nbw_status st = cu_count(&cus);
    if (st != NBW_OK) return st;
    hipError_t e = nbw::launch_mfma_rate(ops, iters, sink, cus, (hipStream_t)stream);
    return e == hipSuccess ? NBW_OK : hip_failed(e);
}

const char *nbw_kernel_name(int64_t batch, int64_t n, int64_t k, int32_t r, nbw_kernel kernel) {
    thread_local char buf[96];
    if (!shape_ok(n, k) || batch < 1 || r < 1 || r > 8 || kernel < NBW_KERNEL_AUTO ||
        kernel > NBW_KERNEL_GEMM)
        return "";
    int cus = 0;
    if (cu_count(&cus) != NBW_OK) return "";
    int kn = kernel;
    if (kn == NBW_KERNEL_AUTO && auto_kernel(batch, n, k, r, &kn) != NBW_OK) return "";
    nbw::QgemmArgs a = {};
    a.batch = batch;
    a.n = (int)n;
    a.k = (int)k;
    switch (kn) {
    case NBW_KERNEL_GEMV: nbw::gemv_name(r, a, cus, buf, sizeof buf); break;
    case NBW_KERNEL_SMALLB: nbw::smallb_name(r, a, cus, buf, sizeof buf); break;
    default: nbw::gemm_name(r, a, cus, buf, sizeof buf); break;
    }
    return buf;
}

const char *nbw_status_str(nbw_status s) {
    switch (s) {
    case NBW_OK: return "ok";
    case NBW_EINVAL: return "invalid argument";
    case NBW_EALIGN: return "misaligned pointer";
    case NBW_ERANGE: return "bit-width out of range";
    case NBW_EUNSUPPORTED: return "unsupported layout or kernel";
    case NBW_EHIP: return "HIP runtime error";
    case NBW_ESCRATCH: return "problem needs more scratch than the library's static buffer holds";
    }
    return "unknown status";
}

int32_t nbw_last_hip_error(void) { return g_last_hip_error; }

const char *nbw_version(void) { return "nbw 0.1.0 gfx950"; }

}  // extern "C"
