// api.hip -- the C ABI of libm3scan (declared in include/m3scan.h): argument validation, the
// gfx950 device check, workspace sizing, and dispatch to the kernels.  Nothing here computes
// any part of the method; every call validates, then only enqueues kernels on the caller's
// stream.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "m3_device.h"
#include "m3_launch.h"
#include "m3scan.h"

namespace {

thread_local char g_err[512] = "";

m3_status fail(m3_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

// 0 = not checked yet, 1 = gfx950, 2 = something else
std::atomic<int> g_dev_ok[256];

m3_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(M3_E_NODEVICE, "no current HIP device");
    if (dev < 256) {
        const int s = g_dev_ok[dev].load(std::memory_order_relaxed);
        if (s == 1) return M3_OK;
        if (s == 2) return fail(M3_E_NODEVICE, "HIP device %d is not a gfx950 GPU", dev);
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(M3_E_NODEVICE, "cannot query HIP device %d", dev);
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 256) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    if (!ok) return fail(M3_E_NODEVICE, "HIP device %d is %s, not gfx950", dev, prop.gcnArchName);
    return M3_OK;
}

size_t io_size(const m3_dims* d) { return d->io == M3_BF16 ? 2 : 4; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// [p, p + n) and [q, q + m) overlap (both non-empty)
bool overlap(const void* p, size_t n, const void* q, size_t m) {
    if (!p || !q || n == 0 || m == 0) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + m && b < a + n;
}

struct Buf {
    const void* p;
    size_t bytes;
    const char* name;
};

m3_status check_common_dims(const m3_dims* d) {
    if (!d) return fail(M3_E_NULL, "dims is NULL");
    if (d->io != M3_F32 && d->io != M3_BF16) return fail(M3_E_DTYPE, "dims->io = %d is not M3_F32 or M3_BF16", d->io);
    const int64_t lim = (int64_t)1 << 31;
    if (d->batch < 0 || d->seqlen < 0 || d->nheads < 0 || d->headdim < 0 || d->dstate < 0 || d->rank < 1 ||
        d->chunk < 0)
        return fail(M3_E_DIMS, "negative size, or rank < 1");
    if (d->batch >= lim || d->seqlen >= lim || d->nheads >= lim || d->headdim > 4096 || d->dstate > 4096 ||
        d->rank > 64)
        return fail(M3_E_DIMS, "size out of range");
    if (d->dstate % 2 != 0) return fail(M3_E_DIMS, "dstate N = %lld must be even", (long long)d->dstate);
    if (d->ngroups < 0 || d->ngroups > d->nheads || (d->ngroups > 0 && d->nheads % d->ngroups != 0))
        return fail(M3_E_DIMS, "ngroups G = %lld must be 0 or divide nheads H = %lld", (long long)d->ngroups,
                    (long long)d->nheads);
    return M3_OK;
}

// head slots of raw B and C (G; H when every head has its own), and the kernels' group field
// (0 for one slot per head)
int64_t bc_groups(const m3_dims* d) { return d->ngroups > 0 ? d->ngroups : d->nheads; }
int kernel_groups(const m3_dims* d) { return d->ngroups > 0 && d->ngroups < d->nheads ? (int)d->ngroups : 0; }

// the calls that take rotated, per-head Bbar and Cbar
m3_status check_per_head(const m3_dims* d, const char* fn) {
    if (bc_groups(d) != d->nheads)
        return fail(M3_E_DIMS, "%s takes per-head Bbar and Cbar: dims->ngroups must be 0 or nheads", fn);
    return M3_OK;
}

// outputs must not overlap inputs, nor each other
m3_status check_alias(const Buf* outs, int nout, const Buf* ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i].p, outs[i].bytes, ins[j].p, ins[j].bytes))
                return fail(M3_E_ALIAS, "output %s overlaps input %s", outs[i].name, ins[j].name);
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
                return fail(M3_E_ALIAS, "outputs %s and %s overlap", outs[i].name, outs[j].name);
    }
    return M3_OK;
}

m3_status check_required(const Buf* bufs, int n) {
    for (int i = 0; i < n; ++i)
        if (!bufs[i].p && bufs[i].bytes > 0) return fail(M3_E_NULL, "%s is NULL", bufs[i].name);
    return M3_OK;
}

m3_status check_align(const Buf* bufs, int n, size_t a) {
    for (int i = 0; i < n; ++i)
        if (bufs[i].p && !aligned(bufs[i].p, a))
            return fail(M3_E_ALIGN, "%s is not %zu-byte aligned", bufs[i].name, a);
    return M3_OK;
}

m3_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(M3_E_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return M3_OK;
}

// dst[i] = src ? src[i] : 0 over n 16-bit words (the sizes used here are all even in bytes)
__global__ void copy_or_zero_kernel(uint16_t* dst, const uint16_t* src, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : (uint16_t)0;
}

__global__ void wrap_angle_kernel(float* dst, const float* src, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src ? m3::wrap_angle(src[i]) : 0.0f;
}

hipError_t copy_or_zero(void* dst, const void* src, size_t bytes, hipStream_t s) {
    if (!dst || bytes == 0) return hipSuccess;
    const int64_t n = (int64_t)(bytes / 2);
    const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3(blocks), dim3(256), 0, s, (uint16_t*)dst, (const uint16_t*)src, n);
    return hipGetLastError();
}

// Compute units of the current device (256 when there is none to ask), cached per device.
std::atomic<int> g_cus[256];
int device_cus() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return 256;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Sequence split of a prefill call (m3_prefill, m3_layer_prefill): when the (b, h) pairs are too
// few to give every compute unit two workgroups, each sequence is cut into segments of a
// multiple of 512 steps (at least 1024 each) that run in parallel, then are chained (see
// PrefillArgs).  Workspace: the segments' end states, the rotated Bbar of their last steps, their
// log2 decays, the steps of each segment to rerun and, fused, each segment's end angle from the
// first pass and its true start angle.
struct SplitPlan {
    int nseg = 1;
    int64_t seglen = 0;
    size_t off_state = 0, off_bbar = 0, off_l2 = 0, off_fix = 0, off_phiend = 0, off_phi = 0, total = 0;
};
constexpr int64_t kSplitAlign = 512, kSplitMin = 1024;

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

SplitPlan split_plan(const m3_dims* d, int64_t Q, bool fused, bool packed) {
    SplitPlan sp;
    const int64_t b = d->batch, L = d->seqlen, H = d->nheads, N = d->dstate, P = d->headdim, R = d->rank;
    const int64_t pairs = b * H, target = 2 * (int64_t)device_cus();
    if (packed || pairs <= 0 || pairs >= target || Q <= 0 || kSplitAlign % Q != 0) return sp;
    int64_t nseg = (target + pairs - 1) / pairs;
    if (nseg > L / kSplitMin) nseg = L / kSplitMin;
    if (nseg < 2) return sp;
    int64_t seglen = (L + nseg - 1) / nseg;
    seglen = (seglen + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
    nseg = (L + seglen - 1) / seglen;
    if (nseg < 2) return sp;
    sp.nseg = (int)nseg;
    sp.seglen = seglen;
    const size_t es = d->io == M3_BF16 ? 2 : 4;
    sp.off_state = 0;
    sp.off_bbar = align256((size_t)(pairs * nseg * N * P) * 4);
    sp.off_l2 = sp.off_bbar + align256((size_t)(pairs * nseg * R * N) * es);
    sp.off_fix = sp.off_l2 + align256((size_t)(pairs * nseg) * 4);
    sp.total = sp.off_fix + align256((size_t)(pairs * nseg) * 4);
    if (fused) {
        sp.off_phiend = sp.total;
        sp.off_phi = sp.off_phiend + align256((size_t)(pairs * nseg * (N / 2)) * 4);
        sp.total = sp.off_phi + align256((size_t)(pairs * nseg * (N / 2)) * 4);
    }
    return sp;
}

// The workspace a split call uses: NULL (or a split that does not pay) runs one pass; otherwise it
// must hold the plan's bytes, be 16-byte aligned and overlap none of the call's buffers.
m3_status check_split_workspace(const SplitPlan& sp, const void* ws, size_t ws_bytes, const Buf* bufs, int n,
                                const char* fn) {
    if (!ws || sp.nseg < 2) return M3_OK;
    if (ws_bytes < sp.total)
        return fail(M3_E_WORKSPACE, "%s needs %zu workspace bytes, got %zu", fn, sp.total, ws_bytes);
    if (!aligned(ws, 16)) return fail(M3_E_ALIGN, "workspace is not 16-byte aligned");
    for (int i = 0; i < n; ++i)
        if (overlap(ws, sp.total, bufs[i].p, bufs[i].bytes)) return fail(M3_E_ALIAS, "workspace overlaps %s", bufs[i].name);
    return M3_OK;
}

// A split prefill: pass 1 (every segment; the later ones from zero state and, fused, zero
// angle), chaining (true start angles, entering states, h_out, Bbar_last, phi_out), pass 2 (the
// later segments' first steps again, from their entering state, until the carry's share of y has
// decayed below float rounding)
hipError_t run_split(m3::PrefillArgs a, const SplitPlan& sp, void* ws, bool fused, bool bf16, hipStream_t s) {
    char* w = (char*)ws;
    a.nseg = sp.nseg;
    a.seglen = sp.seglen;
    a.ws_state = (float*)(w + sp.off_state);
    a.ws_bbar = w + sp.off_bbar;
    a.ws_l2 = (float*)(w + sp.off_l2);
    a.ws_fix = (int*)(w + sp.off_fix);
    a.ws_phiend = fused ? (float*)(w + sp.off_phiend) : nullptr;
    a.seg_phi = fused ? (float*)(w + sp.off_phi) : nullptr;
    auto run = [&](const m3::PrefillArgs& pa) {
        return fused ? m3::launch_layer(pa, bf16, s) : m3::launch_prefill(pa, bf16, s);
    };
    a.pass = 1;
    hipError_t e = run(a);
    if (e == hipSuccess) e = m3::launch_segment_combine(a, bf16, s);
    a.pass = 2;
    if (e == hipSuccess) e = run(a);
    return e;
}

}  // namespace

namespace {

// m3_layer_prefill and its packed form: with cu_seqlens the sequence tensors are [T, H, ...] with
// T = dims->seqlen tokens, and dims->batch sequences; per-sequence tensors stay [b, H, ...]
m3_status layer_prefill(const m3_dims* d, bool packed, const int32_t* cu_seqlens, const void* x, const void* B,
                        const void* C, const void* dt, const void* theta, const float* normw_B, const float* normw_C,
                        const float* bias_B, const float* bias_C, const float* A, const void* lam,
                        const float* w_out, const float* phi_in, const float* h_in, const void* Bbar_prev,
                        const void* x_prev, void* y, float* h_out, float* phi_out, void* Bbar_last, void* x_last,
                        void* workspace, size_t workspace_bytes, hipStream_t stream, const char* fn) {
    m3_status s = check_common_dims(d);
    if (s != M3_OK) return s;
    const int64_t b = d->batch, H = d->nheads, N = d->dstate, P = d->headdim, R = d->rank;
    // tokens per sequence tensor: b * L dense, T packed
    const int64_t L = d->seqlen, BL = packed ? L : b * L;
    const int64_t Q = d->chunk > 0 ? d->chunk : (32 / R > 0 ? 32 / R : 1);
    const size_t es = io_size(d);
    const size_t nX = (size_t)(BL * H * R * P) * es, nBC = (size_t)(BL * bc_groups(d) * R * N) * es;
    const size_t nStep = (size_t)(BL * H) * es, nA = (size_t)H * 4;
    const size_t nTh = (size_t)(BL * H * (N / 2)) * es, nPhi = (size_t)(b * H * (N / 2)) * 4;
    const size_t nY = (size_t)(BL * H * (w_out ? 1 : R) * P) * es, nH = (size_t)(b * H * N * P) * 4;
    const size_t nBp = (size_t)(b * H * R * N) * es, nXp = (size_t)(b * H * R * P) * es;
    const size_t nWo = (size_t)(H * R * P) * 4, nW = (size_t)(H * N) * 4, nBias = (size_t)(H * R * N) * 4;
    const Buf req[] = {{x, nX, "x"}, {B, nBC, "B"}, {C, nBC, "C"}, {dt, nStep, "dt"}, {theta, nTh, "theta"},
                       {A, nA, "A"}, {lam, nStep, "lam"}, {y, nY, "y"}, {h_out, nH, "h_out"},
                       {phi_out, nPhi, "phi_out"}};
    if ((s = check_required(req, 10)) != M3_OK) return s;
    if (packed && cu_seqlens == nullptr) return fail(M3_E_NULL, "cu_seqlens is NULL");
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(M3_E_ALIGN, "cu_seqlens is not 4-byte aligned");
    if (Q * R > 64 || !m3::layer_supported((int)N, (int)P, (int)R, (int)(Q * R), d->io == M3_BF16))
        return fail(M3_E_UNSUPPORTED,
                    "%s: no kernel for N = %lld, P = %lld, R = %lld, chunk*R = %lld (supported: (N,P) "
                    "in {(16,16),(64,64),(128,64)}, R in {1,2,4,8,16}, chunk*R in {16,32,64})",
                    fn, (long long)N, (long long)P, (long long)R, (long long)(Q * R));
    // the kernel addresses a sequence's rows with 32-bit byte offsets (a packed sequence is at most
    // the L = T packed tokens long)
    if ((L + 3 * Q) * H * R * (N > P ? N : P) * (int64_t)es >= ((int64_t)1 << 31))
        return fail(M3_E_DIMS,
                    "%s: one sequence spans %lld bytes per tensor, the limit is 2^31 (split the sequence: the "
                    "carried state, angle and last step make the split exact)",
                    fn, (long long)(L * H * R * (N > P ? N : P) * (int64_t)es));
    const Buf a16[] = {{x, 1, "x"}, {B, 1, "B"}, {C, 1, "C"}, {theta, 1, "theta"}, {y, 1, "y"},
                       {h_out, 1, "h_out"}, {h_in, 1, "h_in"}};
    if ((s = check_align(a16, 7, 16)) != M3_OK) return s;
    const Buf aes[] = {{dt, 1, "dt"}, {lam, 1, "lam"}, {Bbar_prev, 1, "Bbar_prev"}, {x_prev, 1, "x_prev"},
                       {Bbar_last, 1, "Bbar_last"}, {x_last, 1, "x_last"}};
    if ((s = check_align(aes, 6, es)) != M3_OK) return s;
    const Buf a4[] = {{A, 1, "A"}, {w_out, 1, "w_out"}, {normw_B, 1, "normw_B"}, {normw_C, 1, "normw_C"},
                      {bias_B, 1, "bias_B"}, {bias_C, 1, "bias_C"}, {phi_in, 1, "phi_in"}, {phi_out, 1, "phi_out"}};
    if ((s = check_align(a4, 8, 4)) != M3_OK) return s;
    const Buf ins[] = {{x, nX, "x"}, {B, nBC, "B"}, {C, nBC, "C"}, {dt, nStep, "dt"}, {theta, nTh, "theta"},
                       {A, nA, "A"}, {lam, nStep, "lam"}, {w_out, nWo, "w_out"}, {normw_B, nW, "normw_B"},
                       {normw_C, nW, "normw_C"}, {bias_B, nBias, "bias_B"}, {bias_C, nBias, "bias_C"},
                       {Bbar_prev, nBp, "Bbar_prev"}, {x_prev, nXp, "x_prev"}};
    const Buf outs[] = {{y, nY, "y"}, {h_out, nH, "h_out"}, {phi_out, nPhi, "phi_out"},
                        {Bbar_last, nBp, "Bbar_last"}, {x_last, nXp, "x_last"}};
    if ((s = check_alias(outs, 5, ins, 14)) != M3_OK) return s;
    for (int o = 0; o < 5; ++o)
        if (overlap(cu_seqlens, (size_t)(b + 1) * 4, outs[o].p, outs[o].bytes))
            return fail(M3_E_ALIAS, "cu_seqlens overlaps %s", outs[o].name);
    if (h_in && h_in != h_out && overlap(h_in, nH, h_out, nH)) return fail(M3_E_ALIAS, "h_out partially overlaps h_in");
    if (phi_in && phi_in != phi_out && overlap(phi_in, nPhi, phi_out, nPhi))
        return fail(M3_E_ALIAS, "phi_out partially overlaps phi_in");
    const Buf carried[] = {{h_in, nH, "h_in"}, {phi_in, nPhi, "phi_in"}};
    for (int i = 0; i < 2; ++i)
        for (int o = 0; o < 5; ++o) {
            const bool same_buffer = (i == 0 && o == 1 && h_in == h_out) || (i == 1 && o == 2 && phi_in == phi_out);
            if (!same_buffer && overlap(carried[i].p, carried[i].bytes, outs[o].p, outs[o].bytes))
                return fail(M3_E_ALIAS, "%s overlaps %s", carried[i].name, outs[o].name);
        }
    if ((s = check_device()) != M3_OK) return s;
    if (b == 0 || H == 0) return M3_OK;
    if (L == 0) {   // no tokens at all (dense L = 0, or a packed batch of empty sequences)
        // nothing to scan: the carried state and angle pass through unchanged
        hipError_t e = copy_or_zero(h_out, h_in == h_out ? h_out : h_in, nH, stream);
        if (e == hipSuccess) e = copy_or_zero(Bbar_last, Bbar_prev, nBp, stream);
        if (e == hipSuccess) e = copy_or_zero(x_last, x_prev, nXp, stream);
        if (e == hipSuccess) {
            const int64_t n = b * H * (N / 2);
            hipLaunchKernelGGL(wrap_angle_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, phi_out,
                               phi_in, n);
            e = hipGetLastError();
        }
        return launched(e, fn);
    }
    m3::PrefillArgs a;
    a.x = x; a.Bbar = B; a.Cbar = C; a.dt = dt; a.A = A; a.lam = lam; a.w_out = w_out;
    a.h_in = h_in; a.Bbar_prev = Bbar_prev; a.x_prev = x_prev;
    a.y = y; a.h_out = h_out; a.Bbar_last = Bbar_last; a.x_last = x_last;
    a.b = b; a.L = L; a.H = (int)H; a.N = (int)N; a.P = (int)P; a.R = (int)R; a.Q = (int)Q;
    a.theta = theta; a.normw_B = normw_B; a.normw_C = normw_C; a.bias_B = bias_B; a.bias_C = bias_C;
    a.phi_in = phi_in; a.phi_out = phi_out;
    a.bcnorm = (d->flags & M3_BCNORM) ? 1 : 0;
    a.eps = d->eps;
    a.G = kernel_groups(d);
    if (packed) {
        a.cu_seqlens = cu_seqlens;
        a.T = L;
        a.L = 0;
    }
    const SplitPlan sp = split_plan(d, Q, true, packed);
    const Buf all[] = {{x, nX, "x"}, {B, nBC, "B"}, {C, nBC, "C"}, {dt, nStep, "dt"}, {theta, nTh, "theta"},
                       {A, nA, "A"}, {lam, nStep, "lam"}, {w_out, nWo, "w_out"}, {normw_B, nW, "normw_B"},
                       {normw_C, nW, "normw_C"}, {bias_B, nBias, "bias_B"}, {bias_C, nBias, "bias_C"},
                       {Bbar_prev, nBp, "Bbar_prev"}, {x_prev, nXp, "x_prev"}, {y, nY, "y"}, {h_out, nH, "h_out"},
                       {phi_out, nPhi, "phi_out"}, {Bbar_last, nBp, "Bbar_last"}, {x_last, nXp, "x_last"},
                       {h_in, nH, "h_in"}, {phi_in, nPhi, "phi_in"}};
    if ((s = check_split_workspace(sp, workspace, workspace_bytes, all, 21, fn)) != M3_OK) return s;
    if (workspace && sp.nseg >= 2) return launched(run_split(a, sp, workspace, true, d->io == M3_BF16, stream), fn);
    return launched(m3::launch_layer(a, d->io == M3_BF16, stream), fn);
}


// backward pass: chunk and workspace layout (states, angles, per-(b, h) partial sums, per-chunk
// step sums, each starting on a 256-byte boundary)
struct BwdLayout {
    int64_t Q = 0, nchunk = 0;
    int rec = 0;
    size_t st_bytes = 0, phi_off = 0, phi_bytes = 0, part_off = 0, part_bytes = 0, sc_off = 0, sc_bytes = 0;
    size_t total = 0;
    // head groups: per-head dB and dC rows (H / G planes of the grouped layout each)
    size_t gB_off = 0, gC_off = 0, g_bytes = 0;
};

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

bool bwd_layout(const m3_dims* d, BwdLayout* o) {
    if (!d || (d->io != M3_F32 && d->io != M3_BF16) || d->rank < 1 || d->batch < 0 || d->seqlen < 0 ||
        d->nheads < 0 || d->ngroups < 0 || d->ngroups > d->nheads ||
        (d->ngroups > 0 && d->nheads % d->ngroups != 0))
        return false;
    if (!m3::backward_supported((int)d->dstate, (int)d->headdim, (int)d->rank)) return false;
    const int64_t rows = m3::backward_chunk_rows((int)d->headdim, d->io == M3_BF16);
    o->Q = rows / d->rank;
    o->nchunk = (d->seqlen + o->Q - 1) / o->Q;
    const int64_t b = d->batch, H = d->nheads, N = d->dstate, P = d->headdim, R = d->rank;
    o->rec = (int)(1 + R * P + 2 * N + 2 * R * N);
    o->st_bytes = (size_t)(b * H * o->nchunk * P * N) * io_size(d);
    o->phi_off = round256(o->st_bytes);
    o->phi_bytes = (size_t)(b * H * o->nchunk * (N / 2)) * 4;
    o->part_off = o->phi_off + round256(o->phi_bytes);
    o->part_bytes = (size_t)(b * H * o->rec) * 4;
    o->sc_off = o->part_off + round256(o->part_bytes);
    o->sc_bytes = (size_t)(b * H * o->nchunk * (5 * o->Q + 3)) * 4;
    o->total = o->sc_off + round256(o->sc_bytes);
    if (kernel_groups(d) > 0) {
        o->g_bytes = (size_t)(b * d->seqlen * H * R * N) * io_size(d);
        o->gB_off = o->total;
        o->gC_off = o->gB_off + round256(o->g_bytes);
        o->total = o->gC_off + round256(o->g_bytes);
    }
    return true;
}

}  // namespace

extern "C" {

const char* m3_last_error(void) { return g_err; }

const char* m3_version(void) { return "libm3scan 0.2.0 gfx950"; }

size_t m3_bcnorm_rope_workspace_bytes(const m3_dims* d) {
    if (!d || d->batch <= 0 || d->nheads <= 0 || d->seqlen <= 0 || d->dstate <= 0) return 0;
    const int64_t seg = m3::bcnorm_rope_seglen();
    const int64_t nseg = (d->seqlen + seg - 1) / seg;
    if (nseg <= 1) return 0;
    return (size_t)(d->batch * d->nheads * nseg * m3::bcnorm_rope_parts() * (d->dstate / 2)) * sizeof(float);
}

size_t m3_prefill_workspace_bytes(const m3_dims* d) {
    if (check_common_dims(d) != M3_OK) return 0;
    const int64_t R = d->rank, Q = d->chunk > 0 ? d->chunk : (64 / R > 0 ? 64 / R : 1);
    return split_plan(d, Q, false, false).total;
}

size_t m3_layer_prefill_workspace_bytes(const m3_dims* d) {
    if (check_common_dims(d) != M3_OK) return 0;
    const int64_t R = d->rank, Q = d->chunk > 0 ? d->chunk : (32 / R > 0 ? 32 / R : 1);
    return split_plan(d, Q, true, false).total;
}

m3_status m3_bcnorm_rope(const m3_dims* d, const void* B, const void* C, const void* dt, const void* theta,
                         const float* normw_B, const float* normw_C, const float* bias_B, const float* bias_C,
                         const float* phi_in, void* Bbar, void* Cbar, float* phi_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    m3_status s = check_common_dims(d);
    if (s != M3_OK) return s;
    const int64_t b = d->batch, L = d->seqlen, H = d->nheads, N = d->dstate, R = d->rank;
    const size_t es = io_size(d);
    const size_t nBC = (size_t)(b * L * H * R * N) * es, nStep = (size_t)(b * L * H) * es;
    const size_t nIn = (size_t)(b * L * bc_groups(d) * R * N) * es;   // raw B, C: G head slots
    const size_t nTh = (size_t)(b * L * H * (N / 2)) * es, nPhi = (size_t)(b * H * (N / 2)) * 4;
    const Buf req[] = {{B, nIn, "B"}, {C, nIn, "C"}, {dt, nStep, "dt"}, {theta, nTh, "theta"},
                       {Bbar, nBC, "Bbar"}, {Cbar, nBC, "Cbar"}, {phi_out, nPhi, "phi_out"}};
    if ((s = check_required(req, 7)) != M3_OK) return s;
    if (!m3::bcnorm_rope_supported((int)N, (int)R))
        return fail(M3_E_UNSUPPORTED, "m3_bcnorm_rope: N = %lld (need 16, 32, 64, 128 or 256), R = %lld",
                    (long long)N, (long long)R);
    const Buf a16[] = {{B, 1, "B"}, {C, 1, "C"}, {theta, 1, "theta"}, {Bbar, 1, "Bbar"}, {Cbar, 1, "Cbar"}};
    if ((s = check_align(a16, 5, 16)) != M3_OK) return s;
    const Buf a4[] = {{normw_B, 1, "normw_B"}, {normw_C, 1, "normw_C"}, {bias_B, 1, "bias_B"},
                      {bias_C, 1, "bias_C"}, {phi_in, 1, "phi_in"}, {phi_out, 1, "phi_out"},
                      {workspace, 1, "workspace"}};
    if ((s = check_align(a4, 7, 4)) != M3_OK) return s;
    if ((s = check_align(&req[2], 1, es)) != M3_OK) return s;
    if (normw_B && !aligned(normw_B, 16)) return fail(M3_E_ALIGN, "normw_B is not 16-byte aligned");
    if (normw_C && !aligned(normw_C, 16)) return fail(M3_E_ALIGN, "normw_C is not 16-byte aligned");
    if (bias_B && !aligned(bias_B, 16)) return fail(M3_E_ALIGN, "bias_B is not 16-byte aligned");
    if (bias_C && !aligned(bias_C, 16)) return fail(M3_E_ALIGN, "bias_C is not 16-byte aligned");
    const size_t nW = (size_t)(H * N) * 4, nBias = (size_t)(H * R * N) * 4;
    const Buf ins[] = {{B, nIn, "B"}, {C, nIn, "C"}, {dt, nStep, "dt"}, {theta, nTh, "theta"},
                       {normw_B, nW, "normw_B"}, {normw_C, nW, "normw_C"}, {bias_B, nBias, "bias_B"},
                       {bias_C, nBias, "bias_C"}};
    const size_t need = m3_bcnorm_rope_workspace_bytes(d);
    const Buf outs[] = {{Bbar, nBC, "Bbar"}, {Cbar, nBC, "Cbar"}, {phi_out, nPhi, "phi_out"},
                        {workspace, need, "workspace"}};
    if ((s = check_alias(outs, 4, ins, 8)) != M3_OK) return s;
    if (phi_in && phi_in != phi_out && overlap(phi_in, nPhi, phi_out, nPhi))
        return fail(M3_E_ALIAS, "phi_out partially overlaps phi_in");
    if (overlap(phi_in, nPhi, Bbar, nBC) || overlap(phi_in, nPhi, Cbar, nBC) || overlap(phi_in, nPhi, workspace, need))
        return fail(M3_E_ALIAS, "phi_in overlaps an output");
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(M3_E_WORKSPACE, "m3_bcnorm_rope needs %zu workspace bytes, got %zu", need, workspace_bytes);
    if ((s = check_device()) != M3_OK) return s;
    if (b == 0 || H == 0 || N == 0) return M3_OK;
    if (L == 0) {
        const int64_t n = b * H * (N / 2);
        hipLaunchKernelGGL(wrap_angle_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, phi_out,
                           phi_in, n);
        return launched(hipGetLastError(), "m3_bcnorm_rope");
    }
    const int64_t seg = m3::bcnorm_rope_seglen();
    const int64_t nseg = (L + seg - 1) / seg;
    if (b * H * nseg >= ((int64_t)1 << 31) / 256) return fail(M3_E_DIMS, "m3_bcnorm_rope: grid too large");
    m3::BcnormRopeArgs a;
    a.B = B; a.C = C; a.dt = dt; a.theta = theta;
    a.normw_B = normw_B; a.normw_C = normw_C; a.bias_B = bias_B; a.bias_C = bias_C;
    a.phi_in = phi_in;
    a.seg_phi = nseg > 1 ? (float*)workspace : nullptr;
    a.Bbar = Bbar; a.Cbar = Cbar; a.phi_out = phi_out;
    a.b = b; a.L = L; a.H = (int)H; a.N = (int)N; a.R = (int)R;
    a.seglen = seg; a.nseg = (int)nseg;
    a.bcnorm = (d->flags & M3_BCNORM) ? 1 : 0;
    a.eps = d->eps;
    a.G = kernel_groups(d);
    return launched(m3::launch_bcnorm_rope(a, d->io == M3_BF16, stream), "m3_bcnorm_rope");
}

m3_status m3_prefill(const m3_dims* d, const void* x, const void* Bbar, const void* Cbar, const void* dt,
                     const float* A, const void* lam, const float* w_out, const float* h_in, const void* Bbar_prev,
                     const void* x_prev, void* y, float* h_out, void* Bbar_last, void* x_last, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    m3_status s = check_common_dims(d);
    if (s != M3_OK) return s;
    if ((s = check_per_head(d, "m3_prefill")) != M3_OK) return s;
    const int64_t b = d->batch, L = d->seqlen, H = d->nheads, N = d->dstate, P = d->headdim, R = d->rank;
    const int64_t Q = d->chunk > 0 ? d->chunk : (64 / R > 0 ? 64 / R : 1);
    const size_t es = io_size(d);
    const size_t nX = (size_t)(b * L * H * R * P) * es, nBC = (size_t)(b * L * H * R * N) * es;
    const size_t nStep = (size_t)(b * L * H) * es, nA = (size_t)H * 4;
    const size_t nY = (size_t)(b * L * H * (w_out ? 1 : R) * P) * es, nH = (size_t)(b * H * N * P) * 4;
    const size_t nBp = (size_t)(b * H * R * N) * es, nXp = (size_t)(b * H * R * P) * es;
    const size_t nWo = (size_t)(H * R * P) * 4;
    const Buf req[] = {{x, nX, "x"}, {Bbar, nBC, "Bbar"}, {Cbar, nBC, "Cbar"}, {dt, nStep, "dt"}, {A, nA, "A"},
                       {lam, nStep, "lam"}, {y, nY, "y"}, {h_out, nH, "h_out"}};
    if ((s = check_required(req, 8)) != M3_OK) return s;
    if (Q * R > 64 || !m3::prefill_supported((int)N, (int)P, (int)R, (int)(Q * R), d->io == M3_BF16))
        return fail(M3_E_UNSUPPORTED,
                    "m3_prefill: no kernel for N = %lld, P = %lld, R = %lld, chunk*R = %lld (supported: (N,P) in "
                    "{(16,16),(64,64),(128,64)}, R in {1,2,4,8,16}, chunk*R in {16,32,48,64})",
                    (long long)N, (long long)P, (long long)R, (long long)(Q * R));
    // the kernel addresses a sequence's rows with 32-bit byte offsets
    if ((L + 3 * Q) * H * R * (N > P ? N : P) * (int64_t)es >= ((int64_t)1 << 31))
        return fail(M3_E_DIMS,
                    "m3_prefill: one sequence spans %lld bytes per tensor, the limit is 2^31 (split the sequence: "
                    "the carried state and last step make the split exact)",
                    (long long)(L * H * R * (N > P ? N : P) * (int64_t)es));
    const Buf a16[] = {{x, 1, "x"}, {Bbar, 1, "Bbar"}, {Cbar, 1, "Cbar"}, {y, 1, "y"}, {h_out, 1, "h_out"},
                       {h_in, 1, "h_in"}};
    if ((s = check_align(a16, 6, 16)) != M3_OK) return s;
    const Buf aes[] = {{dt, 1, "dt"}, {lam, 1, "lam"}, {Bbar_prev, 1, "Bbar_prev"}, {x_prev, 1, "x_prev"},
                       {Bbar_last, 1, "Bbar_last"}, {x_last, 1, "x_last"}};
    if ((s = check_align(aes, 6, es)) != M3_OK) return s;
    const Buf a4[] = {{A, 1, "A"}, {w_out, 1, "w_out"}};
    if ((s = check_align(a4, 2, 4)) != M3_OK) return s;
    const Buf ins[] = {{x, nX, "x"}, {Bbar, nBC, "Bbar"}, {Cbar, nBC, "Cbar"}, {dt, nStep, "dt"}, {A, nA, "A"},
                       {lam, nStep, "lam"}, {w_out, nWo, "w_out"}, {Bbar_prev, nBp, "Bbar_prev"},
                       {x_prev, nXp, "x_prev"}};
    const Buf outs[] = {{y, nY, "y"}, {h_out, nH, "h_out"}, {Bbar_last, nBp, "Bbar_last"}, {x_last, nXp, "x_last"}};
    if ((s = check_alias(outs, 4, ins, 9)) != M3_OK) return s;
    if (h_in && h_in != h_out && overlap(h_in, nH, h_out, nH)) return fail(M3_E_ALIAS, "h_out partially overlaps h_in");
    if (overlap(h_in, nH, y, nY) || overlap(h_in, nH, Bbar_last, nBp) || overlap(h_in, nH, x_last, nXp))
        return fail(M3_E_ALIAS, "h_in overlaps an output");
    if ((s = check_device()) != M3_OK) return s;
    if (b == 0 || H == 0) return M3_OK;
    if (L == 0) {
        // nothing to scan: the carried state passes through unchanged
        hipError_t e = copy_or_zero(h_out, h_in == h_out ? h_out : h_in, nH, stream);
        if (e == hipSuccess) e = copy_or_zero(Bbar_last, Bbar_prev, nBp, stream);
        if (e == hipSuccess) e = copy_or_zero(x_last, x_prev, nXp, stream);
        return launched(e, "m3_prefill");
    }
    m3::PrefillArgs a;
    a.x = x; a.Bbar = Bbar; a.Cbar = Cbar; a.dt = dt; a.A = A; a.lam = lam; a.w_out = w_out;
    a.h_in = h_in; a.Bbar_prev = Bbar_prev; a.x_prev = x_prev;
    a.y = y; a.h_out = h_out; a.Bbar_last = Bbar_last; a.x_last = x_last;
    a.b = b; a.L = L; a.H = (int)H; a.N = (int)N; a.P = (int)P; a.R = (int)R; a.Q = (int)Q;
    const SplitPlan sp = split_plan(d, Q, false, false);
    const Buf all[] = {{x, nX, "x"}, {Bbar, nBC, "Bbar"}, {Cbar, nBC, "Cbar"}, {dt, nStep, "dt"}, {A, nA, "A"},
                       {lam, nStep, "lam"}, {w_out, nWo, "w_out"}, {Bbar_prev, nBp, "Bbar_prev"},
                       {x_prev, nXp, "x_prev"}, {y, nY, "y"}, {h_out, nH, "h_out"}, {Bbar_last, nBp, "Bbar_last"},
                       {x_last, nXp, "x_last"}, {h_in, nH, "h_in"}};
    if ((s = check_split_workspace(sp, workspace, workspace_bytes, all, 14, "m3_prefill")) != M3_OK) return s;
    if (workspace && sp.nseg >= 2)
        return launched(run_split(a, sp, workspace, false, d->io == M3_BF16, stream), "m3_prefill");
    return launched(m3::launch_prefill(a, d->io == M3_BF16, stream), "m3_prefill");
}

m3_status m3_layer_prefill(const m3_dims* d, const void* x, const void* B, const void* C, const void* dt,
                           const void* theta, const float* normw_B, const float* normw_C, const float* bias_B,
                           const float* bias_C, const float* A, const void* lam, const float* w_out,
                           const float* phi_in, const float* h_in, const void* Bbar_prev, const void* x_prev,
                           void* y, float* h_out, float* phi_out, void* Bbar_last, void* x_last, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    return layer_prefill(d, false, nullptr, x, B, C, dt, theta, normw_B, normw_C, bias_B, bias_C, A, lam, w_out, phi_in,
                         h_in, Bbar_prev, x_prev, y, h_out, phi_out, Bbar_last, x_last, workspace, workspace_bytes,
                         stream, "m3_layer_prefill");
}

m3_status m3_layer_prefill_varlen(const m3_dims* d, const int32_t* cu_seqlens, const void* x, const void* B,
                                  const void* C, const void* dt, const void* theta, const float* normw_B,
                                  const float* normw_C, const float* bias_B, const float* bias_C, const float* A,
                                  const void* lam, const float* w_out, const float* phi_in, const float* h_in,
                                  const void* Bbar_prev, const void* x_prev, void* y, float* h_out, float* phi_out,
                                  void* Bbar_last, void* x_last, hipStream_t stream) {
    return layer_prefill(d, true, cu_seqlens, x, B, C, dt, theta, normw_B, normw_C, bias_B, bias_C, A, lam, w_out,
                         phi_in, h_in, Bbar_prev, x_prev, y, h_out, phi_out, Bbar_last, x_last, nullptr, 0,
                         stream, "m3_layer_prefill_varlen");
}

m3_status m3_decode_step(const m3_dims* d, float* h, const void* Bbar_prev, const void* x_prev, const void* x,
                         const void* Bbar, const void* Cbar, const void* dt, const float* A, const void* lam,
                         const float* w_out, void* y, hipStream_t stream) {
    m3_status s = check_common_dims(d);
    if (s != M3_OK) return s;
    if (d->seqlen != 1) return fail(M3_E_DIMS, "m3_decode_step: dims->seqlen must be 1, got %lld", (long long)d->seqlen);
    if ((s = check_per_head(d, "m3_decode_step")) != M3_OK) return s;
    const int64_t b = d->batch, H = d->nheads, N = d->dstate, P = d->headdim, R = d->rank;
    const size_t es = io_size(d);
    const size_t nH = (size_t)(b * H * N * P) * 4, nBp = (size_t)(b * H * R * N) * es;
    const size_t nXp = (size_t)(b * H * R * P) * es, nStep = (size_t)(b * H) * es, nA = (size_t)H * 4;
    const size_t nY = (size_t)(b * H * (w_out ? 1 : R) * P) * es, nWo = (size_t)(H * R * P) * 4;
    const Buf req[] = {{h, nH, "h"}, {Bbar_prev, nBp, "Bbar_prev"}, {x_prev, nXp, "x_prev"}, {x, nXp, "x"},
                       {Bbar, nBp, "Bbar"}, {Cbar, nBp, "Cbar"}, {dt, nStep, "dt"}, {A, nA, "A"},
                       {lam, nStep, "lam"}, {y, nY, "y"}};
    if ((s = check_required(req, 10)) != M3_OK) return s;
    if (!m3::decode_supported((int)N, (int)P, (int)R))
        return fail(M3_E_UNSUPPORTED,
                    "m3_decode_step: no kernel for N = %lld, P = %lld, R = %lld (need P a power of two in [4, 256], "
                    "N <= 256, R in {1,2,4,8})",
                    (long long)N, (long long)P, (long long)R);
    if (!aligned(h, 16)) return fail(M3_E_ALIGN, "h is not 16-byte aligned");
    const Buf aes[] = {{Bbar_prev, 1, "Bbar_prev"}, {x_prev, 1, "x_prev"}, {x, 1, "x"}, {Bbar, 1, "Bbar"},
                       {Cbar, 1, "Cbar"}, {dt, 1, "dt"}, {lam, 1, "lam"}, {y, 1, "y"}};
    if ((s = check_align(aes, 8, es)) != M3_OK) return s;
    const Buf a4[] = {{A, 1, "A"}, {w_out, 1, "w_out"}};
    if ((s = check_align(a4, 2, 4)) != M3_OK) return s;
    const Buf ins[] = {{Bbar_prev, nBp, "Bbar_prev"}, {x_prev, nXp, "x_prev"}, {x, nXp, "x"}, {Bbar, nBp, "Bbar"},
                       {Cbar, nBp, "Cbar"}, {dt, nStep, "dt"}, {A, nA, "A"}, {lam, nStep, "lam"},
                       {w_out, nWo, "w_out"}};
    const Buf outs[] = {{h, nH, "h"}, {y, nY, "y"}};
    if ((s = check_alias(outs, 2, ins, 9)) != M3_OK) return s;
    if ((s = check_device()) != M3_OK) return s;
    if (b == 0 || H == 0) return M3_OK;
    if (b * H >= ((int64_t)1 << 31) / 256) return fail(M3_E_DIMS, "m3_decode_step: grid too large");
    m3::DecodeArgs a;
    a.h = h; a.Bbar_prev = Bbar_prev; a.x_prev = x_prev; a.x = x; a.Bbar = Bbar; a.Cbar = Cbar;
    a.dt = dt; a.A = A; a.lam = lam; a.w_out = w_out; a.y = y;
    a.b = b; a.H = (int)H; a.N = (int)N; a.P = (int)P; a.R = (int)R;
    return launched(m3::launch_decode(a, d->io == M3_BF16, stream), "m3_decode_step");
}

m3_status m3_layer_decode_step(const m3_dims* d, float* h, float* phi, const void* Bbar_prev, const void* x_prev,
                               const void* x, const void* B, const void* C, const void* dt, const void* theta,
                               const float* normw_B, const float* normw_C, const float* bias_B,
                               const float* bias_C, const float* A, const void* lam, const float* w_out, void* y,
                               void* Bbar_out, hipStream_t stream) {
    m3_status s = check_common_dims(d);
    if (s != M3_OK) return s;
    if (d->seqlen != 1)
        return fail(M3_E_DIMS, "m3_layer_decode_step: dims->seqlen must be 1, got %lld", (long long)d->seqlen);
    const int64_t b = d->batch, H = d->nheads, N = d->dstate, P = d->headdim, R = d->rank;
    const size_t es = io_size(d);
    const size_t nH = (size_t)(b * H * N * P) * 4, nBp = (size_t)(b * H * R * N) * es;
    const size_t nXp = (size_t)(b * H * R * P) * es, nStep = (size_t)(b * H) * es, nA = (size_t)H * 4;
    const size_t nY = (size_t)(b * H * (w_out ? 1 : R) * P) * es, nWo = (size_t)(H * R * P) * 4;
    const size_t nTh = (size_t)(b * H * (N / 2)) * es, nPhi = (size_t)(b * H * (N / 2)) * 4;
    const size_t nW = (size_t)(H * N) * 4, nBias = (size_t)(H * R * N) * 4;
    const size_t nIn = (size_t)(b * bc_groups(d) * R * N) * es;   // raw B, C: G head slots
    const Buf req[] = {{h, nH, "h"}, {phi, nPhi, "phi"}, {Bbar_prev, nBp, "Bbar_prev"}, {x_prev, nXp, "x_prev"},
                       {x, nXp, "x"}, {B, nIn, "B"}, {C, nIn, "C"}, {dt, nStep, "dt"}, {theta, nTh, "theta"},
                       {A, nA, "A"}, {lam, nStep, "lam"}, {y, nY, "y"}, {Bbar_out, nBp, "Bbar_out"}};
    if ((s = check_required(req, 13)) != M3_OK) return s;
    if (!m3::decode_supported((int)N, (int)P, (int)R))
        return fail(M3_E_UNSUPPORTED,
                    "m3_layer_decode_step: no kernel for N = %lld, P = %lld, R = %lld (need P a power of two in "
                    "[4, 256], N <= 256, R in {1,2,4,8})",
                    (long long)N, (long long)P, (long long)R);
    if (!aligned(h, 16)) return fail(M3_E_ALIGN, "h is not 16-byte aligned");
    const Buf aes[] = {{Bbar_prev, 1, "Bbar_prev"}, {x_prev, 1, "x_prev"}, {x, 1, "x"}, {B, 1, "B"},
                       {C, 1, "C"}, {dt, 1, "dt"}, {theta, 1, "theta"}, {lam, 1, "lam"}, {y, 1, "y"},
                       {Bbar_out, 1, "Bbar_out"}};
    if ((s = check_align(aes, 10, es)) != M3_OK) return s;
    const Buf a4[] = {{A, 1, "A"}, {w_out, 1, "w_out"}, {phi, 1, "phi"}, {normw_B, 1, "normw_B"},
                      {normw_C, 1, "normw_C"}, {bias_B, 1, "bias_B"}, {bias_C, 1, "bias_C"}};
    if ((s = check_align(a4, 7, 4)) != M3_OK) return s;
    const Buf ins[] = {{Bbar_prev, nBp, "Bbar_prev"}, {x_prev, nXp, "x_prev"}, {x, nXp, "x"}, {B, nIn, "B"},
                       {C, nIn, "C"}, {dt, nStep, "dt"}, {theta, nTh, "theta"}, {A, nA, "A"}, {lam, nStep, "lam"},
                       {w_out, nWo, "w_out"}, {normw_B, nW, "normw_B"}, {normw_C, nW, "normw_C"},
                       {bias_B, nBias, "bias_B"}, {bias_C, nBias, "bias_C"}};
    const Buf outs[] = {{h, nH, "h"}, {phi, nPhi, "phi"}, {y, nY, "y"}, {Bbar_out, nBp, "Bbar_out"}};
    if ((s = check_alias(outs, 4, ins, 14)) != M3_OK) return s;
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
                return fail(M3_E_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
    if ((s = check_device()) != M3_OK) return s;
    if (b == 0 || H == 0) return M3_OK;
    if (b * H >= ((int64_t)1 << 31) / 256) return fail(M3_E_DIMS, "m3_layer_decode_step: grid too large");
    m3::DecodeArgs a;
    a.h = h; a.Bbar_prev = Bbar_prev; a.x_prev = x_prev; a.x = x; a.Bbar = B; a.Cbar = C;
    a.dt = dt; a.A = A; a.lam = lam; a.w_out = w_out; a.y = y;
    a.b = b; a.H = (int)H; a.N = (int)N; a.P = (int)P; a.R = (int)R;
    a.theta = theta; a.normw_B = normw_B; a.normw_C = normw_C; a.bias_B = bias_B; a.bias_C = bias_C;
    a.phi = phi; a.Bbar_out = Bbar_out;
    a.bcnorm = (d->flags & M3_BCNORM) ? 1 : 0;
    a.eps = d->eps;
    a.G = kernel_groups(d);
    return launched(m3::launch_layer_decode(a, d->io == M3_BF16, stream), "m3_layer_decode_step");
}

int64_t m3_layer_backward_chunk(const m3_dims* d) {
    BwdLayout lay;
    return bwd_layout(d, &lay) ? lay.Q : 0;
}

size_t m3_layer_backward_workspace_bytes(const m3_dims* d) {
    BwdLayout lay;
    return bwd_layout(d, &lay) ? lay.total : 0;
}

m3_status m3_layer_chunk_states(const m3_dims* d, const void* x, const void* B, const void* dt, const void* theta,
                                const float* normw_B, const float* bias_B, const float* A, const void* lam,
                                const float* phi_in, const float* h_in, const void* Bbar_prev, const void* x_prev,
                                void* states, float* phis, hipStream_t stream) {
    m3_status s = check_common_dims(d);
    if (s != M3_OK) return s;
    const int64_t b = d->batch, L = d->seqlen, H = d->nheads, N = d->dstate, P = d->headdim, R = d->rank;
    BwdLayout lay;
    if (!bwd_layout(d, &lay))
        return fail(M3_E_UNSUPPORTED,
                    "m3_layer_chunk_states: no kernel for N = %lld, P = %lld, R = %lld (supported: (N,P) in "
                    "{(16,16),(64,64),(128,64)}, R in {1,2,4})", (long long)N, (long long)P, (long long)R);
    const size_t es = io_size(d);
    const size_t nX = (size_t)(b * L * H * R * P) * es, nBC = (size_t)(b * L * bc_groups(d) * R * N) * es;
    const size_t nStep = (size_t)(b * L * H) * es, nA = (size_t)H * 4;
    const size_t nTh = (size_t)(b * L * H * (N / 2)) * es, nPhi = (size_t)(b * H * (N / 2)) * 4;
    const size_t nH = (size_t)(b * H * N * P) * 4, nBp = (size_t)(b * H * R * N) * es;
    const size_t nXp = (size_t)(b * H * R * P) * es, nW = (size_t)(H * N) * 4, nBias = (size_t)(H * R * N) * 4;
    const Buf req[] = {{x, nX, "x"}, {B, nBC, "B"}, {dt, nStep, "dt"}, {theta, nTh, "theta"}, {A, nA, "A"},
                       {lam, nStep, "lam"}, {states, lay.st_bytes, "states"}, {phis, lay.phi_bytes, "phis"}};
    if ((s = check_required(req, 8)) != M3_OK) return s;
    if (lay.Q * H * R * (N > P ? N : P) * (int64_t)es >= ((int64_t)1 << 31))
        return fail(M3_E_DIMS, "m3_layer_chunk_states: nheads * rank = %lld is too large for one chunk",
                    (long long)(H * R));
    const Buf a16[] = {{x, 1, "x"}, {B, 1, "B"}, {theta, 1, "theta"}, {states, 1, "states"}};
    if ((s = check_align(a16, 4, 16)) != M3_OK) return s;
    const Buf aes[] = {{dt, 1, "dt"}, {lam, 1, "lam"}, {Bbar_prev, 1, "Bbar_prev"}, {x_prev, 1, "x_prev"}};
    if ((s = check_align(aes, 4, es)) != M3_OK) return s;
    const Buf a4[] = {{A, 1, "A"}, {normw_B, 1, "normw_B"}, {bias_B, 1, "bias_B"}, {phi_in, 1, "phi_in"},
                      {h_in, 1, "h_in"}, {phis, 1, "phis"}};
    if ((s = check_align(a4, 6, 4)) != M3_OK) return s;
    const Buf ins[] = {{x, nX, "x"}, {B, nBC, "B"}, {dt, nStep, "dt"}, {theta, nTh, "theta"}, {A, nA, "A"},
                       {lam, nStep, "lam"}, {normw_B, nW, "normw_B"}, {bias_B, nBias, "bias_B"},
                       {phi_in, nPhi, "phi_in"}, {h_in, nH, "h_in"}, {Bbar_prev, nBp, "Bbar_prev"},
                       {x_prev, nXp, "x_prev"}};
    const Buf outs[] = {{states, lay.st_bytes, "states"}, {phis, lay.phi_bytes, "phis"}};
    if ((s = check_alias(outs, 2, ins, 12)) != M3_OK) return s;
    if ((s = check_device()) != M3_OK) return s;
    if (b == 0 || H == 0 || L == 0) return M3_OK;
    m3::BackwardArgs a = {};
    a.x = x; a.B = B; a.dt = dt; a.theta = theta; a.A = A; a.lam = lam; a.normw_B = normw_B; a.bias_B = bias_B;
    a.phi_in = phi_in; a.h_in = h_in; a.Bbar_prev = Bbar_prev; a.x_prev = x_prev;
    a.ws_states = states; a.ws_phi = phis;
    a.b = b; a.L = L; a.H = (int)H; a.N = (int)N; a.P = (int)P; a.R = (int)R;
    a.bcnorm = (d->flags & M3_BCNORM) ? 1 : 0;
    a.eps = d->eps;
    a.G = kernel_groups(d);
    return launched(m3::launch_chunk_states(a, d->io == M3_BF16, stream), "m3_layer_chunk_states");
}

m3_status m3_layer_backward(const m3_dims* d, const void* x, const void* B, const void* C, const void* dt,
                            const void* theta, const float* normw_B, const float* normw_C, const float* bias_B,
                            const float* bias_C, const float* A, const void* lam, const float* w_out,
                            const float* phi_in, const float* h_in, const void* Bbar_prev, const void* x_prev,
                            const void* dy, const float* dh_out, const float* dphi_out, void* dx, void* dB,
                            void* dC, void* ddt, void* dtheta, float* dA, void* dlam, float* dnormw_B,
                            float* dnormw_C, float* dbias_B, float* dbias_C, float* dw_out, float* dphi_in,
                            float* dh_in, void* dBbar_prev, void* dx_prev, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    m3_status s = check_common_dims(d);
    if (s != M3_OK) return s;
    const int64_t b = d->batch, L = d->seqlen, H = d->nheads, N = d->dstate, P = d->headdim, R = d->rank;
    BwdLayout lay;
    if (!bwd_layout(d, &lay))
        return fail(M3_E_UNSUPPORTED,
                    "m3_layer_backward: no kernel for N = %lld, P = %lld, R = %lld (supported: (N,P) in "
                    "{(16,16),(64,64),(128,64)}, R in {1,2,4})", (long long)N, (long long)P, (long long)R);
    if (d->chunk != 0 && d->chunk != lay.Q)
        return fail(M3_E_UNSUPPORTED, "m3_layer_backward: chunk must be 0 or %lld for these dims",
                    (long long)lay.Q);
    const size_t es = io_size(d);
    const size_t nX = (size_t)(b * L * H * R * P) * es, nBC = (size_t)(b * L * bc_groups(d) * R * N) * es;
    const size_t nStep = (size_t)(b * L * H) * es, nA = (size_t)H * 4;
    const size_t nTh = (size_t)(b * L * H * (N / 2)) * es, nPhi = (size_t)(b * H * (N / 2)) * 4;
    const size_t nY = (size_t)(b * L * H * (w_out ? 1 : R) * P) * es, nH = (size_t)(b * H * N * P) * 4;
    const size_t nBp = (size_t)(b * H * R * N) * es, nXp = (size_t)(b * H * R * P) * es;
    const size_t nWo = (size_t)(H * R * P) * 4, nW = (size_t)(H * N) * 4, nBias = (size_t)(H * R * N) * 4;
    const Buf req[] = {{x, nX, "x"}, {B, nBC, "B"}, {C, nBC, "C"}, {dt, nStep, "dt"}, {theta, nTh, "theta"},
                       {A, nA, "A"}, {lam, nStep, "lam"}, {dy, nY, "dy"}, {dx, nX, "dx"}, {dB, nBC, "dB"},
                       {dC, nBC, "dC"}, {ddt, nStep, "ddt"}, {dtheta, nTh, "dtheta"}, {dA, nA, "dA"},
                       {dlam, nStep, "dlam"}, {dphi_in, nPhi, "dphi_in"}, {dh_in, nH, "dh_in"}};
    if ((s = check_required(req, 17)) != M3_OK) return s;
    if (!workspace && lay.total > 0) return fail(M3_E_WORKSPACE, "m3_layer_backward: workspace is NULL");
    if (workspace_bytes < lay.total)
        return fail(M3_E_WORKSPACE, "m3_layer_backward: workspace has %zu bytes, needs %zu", workspace_bytes,
                    lay.total);
    if (lay.Q * H * R * (N > P ? N : P) * (int64_t)es >= ((int64_t)1 << 31))
        return fail(M3_E_DIMS, "m3_layer_backward: nheads * rank = %lld is too large for one chunk",
                    (long long)(H * R));
    const Buf a16[] = {{x, 1, "x"}, {B, 1, "B"}, {C, 1, "C"}, {theta, 1, "theta"}, {dy, 1, "dy"},
                       {dx, 1, "dx"}, {dB, 1, "dB"}, {dC, 1, "dC"}, {dtheta, 1, "dtheta"},
                       {workspace, 1, "workspace"}};
    if ((s = check_align(a16, 10, 16)) != M3_OK) return s;
    const Buf aes[] = {{dt, 1, "dt"}, {lam, 1, "lam"}, {Bbar_prev, 1, "Bbar_prev"}, {x_prev, 1, "x_prev"},
                       {ddt, 1, "ddt"}, {dlam, 1, "dlam"}, {dBbar_prev, 1, "dBbar_prev"}, {dx_prev, 1, "dx_prev"}};
    if ((s = check_align(aes, 8, es)) != M3_OK) return s;
    const Buf a4[] = {{A, 1, "A"}, {w_out, 1, "w_out"}, {normw_B, 1, "normw_B"}, {normw_C, 1, "normw_C"},
                      {bias_B, 1, "bias_B"}, {bias_C, 1, "bias_C"}, {phi_in, 1, "phi_in"}, {h_in, 1, "h_in"},
                      {dh_out, 1, "dh_out"}, {dphi_out, 1, "dphi_out"}, {dA, 1, "dA"}, {dnormw_B, 1, "dnormw_B"},
                      {dnormw_C, 1, "dnormw_C"}, {dbias_B, 1, "dbias_B"}, {dbias_C, 1, "dbias_C"},
                      {dw_out, 1, "dw_out"}, {dphi_in, 1, "dphi_in"}, {dh_in, 1, "dh_in"}};
    if ((s = check_align(a4, 18, 4)) != M3_OK) return s;
    const Buf ins[] = {{x, nX, "x"}, {B, nBC, "B"}, {C, nBC, "C"}, {dt, nStep, "dt"}, {theta, nTh, "theta"},
                       {A, nA, "A"}, {lam, nStep, "lam"}, {w_out, nWo, "w_out"}, {normw_B, nW, "normw_B"},
                       {normw_C, nW, "normw_C"}, {bias_B, nBias, "bias_B"}, {bias_C, nBias, "bias_C"},
                       {phi_in, nPhi, "phi_in"}, {h_in, nH, "h_in"}, {Bbar_prev, nBp, "Bbar_prev"},
                       {x_prev, nXp, "x_prev"}, {dy, nY, "dy"}, {dh_out, nH, "dh_out"},
                       {dphi_out, nPhi, "dphi_out"}, {workspace, lay.total, "workspace"}};
    const Buf outs[] = {{dx, nX, "dx"}, {dB, nBC, "dB"}, {dC, nBC, "dC"}, {ddt, nStep, "ddt"},
                        {dtheta, nTh, "dtheta"}, {dA, nA, "dA"}, {dlam, nStep, "dlam"}, {dnormw_B, nW, "dnormw_B"},
                        {dnormw_C, nW, "dnormw_C"}, {dbias_B, nBias, "dbias_B"}, {dbias_C, nBias, "dbias_C"},
                        {dw_out, w_out ? nWo : 0, "dw_out"}, {dphi_in, nPhi, "dphi_in"}, {dh_in, nH, "dh_in"},
                        {dBbar_prev, nBp, "dBbar_prev"}, {dx_prev, nXp, "dx_prev"}};
    if ((s = check_alias(outs, 16, ins, 20)) != M3_OK) return s;
    if ((s = check_device()) != M3_OK) return s;
    if (b == 0 || H == 0) return M3_OK;
    m3::BackwardArgs a = {};
    a.x = x; a.B = B; a.C = C; a.dt = dt; a.theta = theta; a.A = A; a.lam = lam;
    a.normw_B = normw_B; a.normw_C = normw_C; a.bias_B = bias_B; a.bias_C = bias_C; a.w_out = w_out;
    a.phi_in = phi_in; a.h_in = h_in; a.Bbar_prev = Bbar_prev; a.x_prev = x_prev;
    a.dy = dy; a.dh_out = dh_out; a.dphi_out = dphi_out;
    a.dx = dx; a.dB = dB; a.dC = dC; a.ddt = ddt; a.dtheta = dtheta; a.dlam = dlam; a.dA = dA;
    a.dnormw_B = dnormw_B; a.dnormw_C = dnormw_C; a.dbias_B = dbias_B; a.dbias_C = dbias_C;
    a.dw_out = w_out ? dw_out : nullptr;
    a.dphi_in = dphi_in; a.dh_in = dh_in; a.dBbar_prev = dBbar_prev; a.dx_prev = dx_prev;
    a.ws_states = workspace;
    a.ws_phi = (float*)((char*)workspace + lay.phi_off);
    a.ws_part = (float*)((char*)workspace + lay.part_off);
    a.ws_scal = (float*)((char*)workspace + lay.sc_off);
    a.rec = lay.rec;
    a.b = b; a.L = L; a.H = (int)H; a.N = (int)N; a.P = (int)P; a.R = (int)R;
    a.bcnorm = (d->flags & M3_BCNORM) ? 1 : 0;
    a.eps = d->eps;
    a.G = kernel_groups(d);
    if (a.G > 0) {
        a.ws_dB = (char*)workspace + lay.gB_off;
        a.ws_dC = (char*)workspace + lay.gC_off;
    }
    return launched(m3::launch_backward(a, d->io == M3_BF16, stream), "m3_layer_backward");
}


}  // extern "C"

// ---------------------------------------------------------------------------------------------
// m3_layer_prefill_noalloc: m3_layer_prefill whose sequence-split workspace is a library-held
// device array instead of caller memory, for callers that cannot allocate (code under graph
// capture, serving loops).  The array lives in this file's code object: each GPU the library
// runs on holds its own copy (kNoAllocScratchBytes) from the module's load until the process
// ends.  Host code never uses the array's name as a device address; its address on each device
// is taken once with hipGetSymbolAddress, with that device current, and kept per device.
// ---------------------------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = M3_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kScratchDevices = 256;
std::atomic<void*> g_scratch_ptr[kScratchDevices];

// the scratch array's address on the current device, taken once per device (with that device
// current) and kept
m3_status scratch_on_current_device(const char* fn, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices)
        return fail(M3_E_NODEVICE, "%s: no current HIP device", fn);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(M3_E_LAUNCH, "%s: cannot get the scratch array's address on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return M3_OK;
}

}  // namespace

extern "C" {

m3_status m3_layer_prefill_noalloc(const m3_dims* d, const void* x, const void* B, const void* C,
                                   const void* dt, const void* theta, const float* normw_B,
                                   const float* normw_C, const float* bias_B, const float* bias_C,
                                   const float* A, const void* lam, const float* w_out,
                                   const float* phi_in, const float* h_in, const void* Bbar_prev,
                                   const void* x_prev, void* y, float* h_out, float* phi_out,
                                   void* Bbar_last, void* x_last, hipStream_t stream) {
    const char* fn = "m3_layer_prefill_noalloc";
    m3_status s = check_common_dims(d);
    if (s != M3_OK) return s;
    // the workspace m3_layer_prefill would take for these dims on this device (0: no split)
    const size_t need = m3_layer_prefill_workspace_bytes(d);
    if (need > kNoAllocScratchBytes)
        return fail(M3_E_WORKSPACE,
                    "%s: these dims split each sequence and need %zu bytes of scratch; the library holds %zu "
                    "(call m3_layer_prefill with a workspace instead)",
                    fn, need, kNoAllocScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        if ((s = check_device()) != M3_OK) return s;
        if ((s = scratch_on_current_device(fn, &ws)) != M3_OK) return s;
    }
    return layer_prefill(d, false, nullptr, x, B, C, dt, theta, normw_B, normw_C, bias_B, bias_C, A, lam, w_out,
                         phi_in, h_in, Bbar_prev, x_prev, y, h_out, phi_out, Bbar_last, x_last, ws, need, stream, fn);
}

}  // extern "C"
