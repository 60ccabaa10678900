// C-ABI layer of libtitans_mem: host-side validation, workspace sizing and
// kernel dispatch.  Every check runs before any HIP call, so an invalid call
// enqueues nothing and writes nothing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "titans_internal.h"

namespace {

thread_local char g_last_error[512] = "";

titans_status fail(titans_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

// Byte interval [lo, hi) touched by a strided tensor; empty tensors touch nothing.
struct Span {
    uintptr_t lo = 0, hi = 0;
    bool empty() const { return hi <= lo; }
};

Span span_of(const void* p, const int64_t* sizes, const int64_t* strides, int nd, size_t elem) {
    Span s;
    int64_t last = 0;
    for (int i = 0; i < nd; ++i) {
        if (sizes[i] == 0) return s;
        last += (sizes[i] - 1) * strides[i];
    }
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + (uintptr_t)((last + 1) * (int64_t)elem);
    return s;
}

bool overlaps(const Span& a, const Span& b) {
    if (a.empty() || b.empty()) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// True when distinct indices map to distinct elements (required of outputs).
bool non_self_overlapping(const int64_t* sizes, const int64_t* strides, int nd) {
    std::vector<std::pair<int64_t, int64_t>> dims;  // (stride, size)
    for (int i = 0; i < nd; ++i) {
        if (sizes[i] == 0) return true;
        if (sizes[i] > 1) dims.push_back({strides[i], sizes[i]});
    }
    std::sort(dims.begin(), dims.end());
    int64_t extent = 1;  // elements spanned by the inner dims
    for (auto& ds : dims) {
        if (ds.first < extent) return false;
        extent = ds.first * (ds.second - 1) + extent;
    }
    return true;
}

bool strides_nonneg(const int64_t* s, int n) {
    for (int i = 0; i < n; ++i)
        if (s[i] < 0) return false;
    return true;
}

titans_status check_mlp(const titans_mlp_desc* mlp, titans::ScanArgs& a) {
    if (!mlp) return fail(TITANS_ERR_INVALID_ARGUMENT, "mlp descriptor is NULL");
    if (mlp->n_layers < 1 || mlp->n_layers > TITANS_MAX_LAYERS)
        return fail(TITANS_ERR_INVALID_ARGUMENT, "n_layers=%d outside 1..%d", mlp->n_layers,
                    TITANS_MAX_LAYERS);
    a.L = mlp->n_layers;
    for (int l = 0; l <= a.L; ++l) {
        if (mlp->width[l] < 1)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "width[%d]=%d must be >= 1", l, mlp->width[l]);
        a.n[l] = mlp->width[l];
    }
    for (int l = a.L + 1; l <= TITANS_MAX_LAYERS; ++l) a.n[l] = 0;
    if (a.n[0] != a.n[a.L])
        return fail(TITANS_ERR_INVALID_ARGUMENT, "width[0]=%d must equal width[L]=%d (d)", a.n[0],
                    a.n[a.L]);
    a.P = 0;
    a.off[0] = 0;
    for (int l = 1; l <= a.L; ++l) {
        a.off[l] = a.P;
        a.P += (int64_t)a.n[l] * a.n[l - 1];
    }
    a.off[a.L + 1] = a.P;
    return TITANS_OK;
}

titans_status check_shape_support(const titans::ScanArgs& a, bool scan) {
    if (a.n[0] > 128)
        return fail(TITANS_ERR_UNSUPPORTED, "d=%d > 128 is not compiled", a.n[0]);
    for (int l = 1; l < a.L; ++l)
        if (a.n[l] > 512) return fail(TITANS_ERR_UNSUPPORTED, "width[%d]=%d > 512", l, a.n[l]);
    if (scan && a.C > 256) return fail(TITANS_ERR_UNSUPPORTED, "chunk=%d > 256", a.C);
    if (a.B * a.H > 65535)
        return fail(TITANS_ERR_UNSUPPORTED, "batch*heads=%lld > 65535",
                    (long long)(a.B * a.H));
    return TITANS_OK;
}

titans_status check_desc_common(const titans_scan_desc* desc, titans::ScanArgs& a) {
    if (!desc) return fail(TITANS_ERR_INVALID_ARGUMENT, "scan descriptor is NULL");
    if (desc->batch < 0 || desc->seq_len < 0 || desc->heads < 0)
        return fail(TITANS_ERR_INVALID_ARGUMENT, "negative size (B=%lld T=%lld H=%lld)",
                    (long long)desc->batch, (long long)desc->seq_len, (long long)desc->heads);
    if (desc->io_dtype != TITANS_F32 && desc->io_dtype != TITANS_BF16)
        return fail(TITANS_ERR_INVALID_ARGUMENT, "io_dtype=%d is neither F32 nor BF16",
                    desc->io_dtype);
    a.B = desc->batch;
    a.T = desc->seq_len;
    a.H = desc->heads;
    a.C = desc->chunk;
    a.io = desc->io_dtype;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = desc->qkv_stride[i];
        a.ys[i] = desc->y_stride[i];
        a.gs[i] = desc->gate_stride[i];
    }
    for (int i = 0; i < 2; ++i) {
        a.ss[i] = desc->state_stride[i];
        a.s0s[i] = desc->state0_stride[i];
    }
    if (!strides_nonneg(a.qs, 3) || !strides_nonneg(a.ys, 3) || !strides_nonneg(a.gs, 3) ||
        !strides_nonneg(a.ss, 2) || !strides_nonneg(a.s0s, 2))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "negative stride");
    return TITANS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

titans_status check_io_alignment(const titans::ScanArgs& a, const void* p, const int64_t* st,
                                 const char* name) {
    const int64_t vec = a.io == TITANS_BF16 ? 8 : 4;  // elements per 16 bytes
    if (a.n[0] % vec)
        return fail(TITANS_ERR_UNSUPPORTED, "d=%d must be a multiple of %lld for this dtype",
                    a.n[0], (long long)vec);
    if (!aligned16(p)) return fail(TITANS_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
    for (int i = 0; i < 3; ++i)
        if (st[i] % vec)
            return fail(TITANS_ERR_INVALID_ARGUMENT,
                        "%s stride[%d]=%lld is not a multiple of 16 bytes", name, i,
                        (long long)st[i]);
    return TITANS_OK;
}

titans_status check_state_alignment(const float* p, const int64_t* st, const char* name) {
    if (!aligned16(p)) return fail(TITANS_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
    for (int i = 0; i < 2; ++i)
        if (st[i] % 4)
            return fail(TITANS_ERR_INVALID_ARGUMENT,
                        "%s stride[%d]=%lld is not a multiple of 16 bytes", name, i,
                        (long long)st[i]);
    return TITANS_OK;
}

titans_status hip_fail(hipError_t e, const char* what) {
    return fail(TITANS_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

}  // namespace

extern "C" {

int titans_abi_version(void) { return TITANS_MEM_ABI_VERSION; }

const char* titans_status_string(int status) {
    switch (status) {
        case TITANS_OK: return "TITANS_OK";
        case TITANS_ERR_INVALID_ARGUMENT: return "TITANS_ERR_INVALID_ARGUMENT";
        case TITANS_ERR_UNSUPPORTED: return "TITANS_ERR_UNSUPPORTED";
        case TITANS_ERR_WORKSPACE: return "TITANS_ERR_WORKSPACE";
        case TITANS_ERR_HIP: return "TITANS_ERR_HIP";
        default: return "TITANS_ERR_UNKNOWN";
    }
}

const char* titans_last_error(void) { return g_last_error; }

int64_t titans_mem_param_count(const titans_mlp_desc* mlp) {
    titans::ScanArgs a{};
    if (check_mlp(mlp, a) != TITANS_OK) return -1;
    return a.P;
}

static titans_status prepare_scan(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                  titans::ScanArgs& a) {
    titans_status st = check_desc_common(desc, a);
    if (st) return st;
    if ((st = check_mlp(mlp, a))) return st;
    if (a.C < 1) return fail(TITANS_ERR_INVALID_ARGUMENT, "chunk=%d must be >= 1", a.C);
    a.bias = desc->bias;
    a.bias_param = desc->bias_param;
    if (a.bias == TITANS_BIAS_HUBER && !(a.bias_param > 0.f))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "Huber delta=%g must be > 0", (double)a.bias_param);
    if (a.bias == TITANS_BIAS_LP && !(a.bias_param >= 1.f && a.bias_param < INFINITY))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "l_p exponent p=%g must be finite and >= 1",
                    (double)a.bias_param);
    if (a.bias != TITANS_BIAS_L2 && a.bias != TITANS_BIAS_HUBER && a.bias != TITANS_BIAS_LP)
        return fail(TITANS_ERR_INVALID_ARGUMENT, "bias=%d is not a titans_bias", a.bias);
    return check_shape_support(a, true);
}

// Compute units of the current device; 256 (an MI355X) when no device is visible, so
// host-only queries answer as they would on that GPU.
static int64_t device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    return n;
}

enum class Path { Generic, Phased, Fused, Pair, Linear };

// Testing overrides.  The TITANS_MEM_* switches below (kernel family, generic member,
// linear path, fused kernel, the pair path's failure hook) are read only while
// TITANS_MEM_DEBUG=1 is set as well, so a stray variable cannot move production calls
// onto another path; titans_mem_scan_path reports the path a call would take, overrides
// included.
static const char* debug_env(const char* name) {
    const char* on = getenv("TITANS_MEM_DEBUG");
    if (!on || on[0] != '1') return nullptr;
    return getenv(name);
}

// Within the generic family: the chain of GPU-wide launches for memories with a layer of
// 128 or more units (their chunk products span several 64 x 64 tiles), else one workgroup
// per memory.  TITANS_MEM_GENERIC_MODE=single / phased picks one for testing (with
// TITANS_MEM_DEBUG=1).
static Path generic_path(const titans::ScanArgs& a) {
    const char* env = debug_env("TITANS_MEM_GENERIC_MODE");
    if (env && strcmp(env, "single") == 0) return Path::Generic;
    if (env && strcmp(env, "phased") == 0) return Path::Phased;
    int maxw = 0;
    for (int l = 0; l <= a.L; ++l) maxw = a.n[l] > maxw ? a.n[l] : maxw;
    return maxw >= 128 ? Path::Phased : Path::Generic;
}

// Which kernel serves a (validated) problem.  The 64-256-64 bf16 memory runs on pairs of
// workgroups (any chunk length that is a multiple of 64) while the pairs fit the device at
// one workgroup per compute unit, else on one workgroup per memory (C = 64 only).  A linear
// memory (L = 1) with the squared-error bias and enough chunks takes the sequence-parallel
// linear path.  Testing switches (read with TITANS_MEM_DEBUG=1 only):
// TITANS_MEM_FORCE_GENERIC=1 routes every call through the generic family,
// TITANS_MEM_LINEAR=0 keeps linear memories on it too, TITANS_MEM_FUSED_SINGLE=1 keeps the
// fused shape on one workgroup per memory.
static Path choose_path(const titans::ScanArgs& a) {
    const char* env = debug_env("TITANS_MEM_FORCE_GENERIC");
    if (env && env[0] == '1') return generic_path(a);
    env = debug_env("TITANS_MEM_GENERIC_MODE");  // a chosen member of the generic family
    if (env && env[0]) return generic_path(a);
    env = debug_env("TITANS_MEM_LINEAR");
    if (!(env && env[0] == '0') && titans::scan_linear_supported(a)) return Path::Linear;
    env = debug_env("TITANS_MEM_FUSED_SINGLE");
    const bool single = env && env[0] == '1';
    if (!single && titans::scan_pair_supported(a) &&
        titans::scan_pair_workgroups(a) <= device_cus())
        return Path::Pair;
    return titans::scan_mfma_supported(a) ? Path::Fused : generic_path(a);
}

// Workgroups per memory on the pair path: quads (four workgroups per memory, 16 hidden
// units per wave) while 4 * ceil(B*H/8) * 8 of them fit the device at one per compute unit
// and no per-token surprise is asked for (its shares are laid out for pairs), else pairs.
// TITANS_MEM_PAIR_SIDES=2 keeps pairs (a testing switch, with TITANS_MEM_DEBUG=1).
static int pair_sides(const titans::ScanArgs& a, bool surprise) {
    const char* env = debug_env("TITANS_MEM_PAIR_SIDES");
    if (surprise || (env && env[0] == '2')) return 2;
    titans::ScanArgs b = a;
    b.sides = 4;
    return titans::scan_pair_workgroups(b) <= device_cus() ? 4 : 2;
}

static const char* path_name(Path p, const titans::ScanArgs& a, bool surprise = false) {
    switch (p) {
        case Path::Pair: return pair_sides(a, surprise) == 4 ? "fused_quad" : "fused_pair";
        case Path::Fused: return "fused_mfma";
        case Path::Phased: return a.io == TITANS_BF16 ? "phased_mfma" : "phased_fp32";
        case Path::Linear: return a.io == TITANS_BF16 ? "linear_mfma" : "linear_fp32";
        default: return a.io == TITANS_BF16 ? "generic_mfma" : "generic_fp32";
    }
}

const char* titans_mem_scan_path(const titans_scan_desc* desc, const titans_mlp_desc* mlp) {
    titans::ScanArgs a{};
    if (prepare_scan(desc, mlp, a) != TITANS_OK) return nullptr;
    return path_name(choose_path(a), a);
}

// The path of a call; the per-token surprise output is computed by the pair path and the
// generic family (the single-workgroup fused and the linear paths do not produce it).
static Path scan_path_of(const titans::ScanArgs& a, bool surprise) {
    const Path p = choose_path(a);
    if (!surprise || p == Path::Pair) return p;
    return generic_path(a);
}

static size_t workspace_of(const titans::ScanArgs& a, bool surprise) {
    if (a.B * a.H == 0 || a.T == 0) return 0;
    switch (scan_path_of(a, surprise)) {
        case Path::Pair: {
            titans::ScanArgs b = a;
            b.sides = pair_sides(a, surprise);
            return titans::scan_pair_workspace_bytes(b) +
                   (surprise ? titans::scan_pair_surprise_bytes(b) : 0);
        }
        case Path::Fused: return 0;
        case Path::Phased: return titans::scan_phased_workspace_bytes(a);
        case Path::Linear: return titans::scan_linear_workspace_bytes(a);
        default: return titans::scan_generic_workspace_bytes(a);
    }
}

size_t titans_mem_scan_workspace_size(const titans_scan_desc* desc, const titans_mlp_desc* mlp) {
    titans::ScanArgs a{};
    if (prepare_scan(desc, mlp, a) != TITANS_OK) return SIZE_MAX;
    return workspace_of(a, false);
}

const char* titans_mem_scan_surprise_path(const titans_scan_desc* desc, const titans_mlp_desc* mlp) {
    titans::ScanArgs a{};
    if (prepare_scan(desc, mlp, a) != TITANS_OK) return nullptr;
    return path_name(scan_path_of(a, true), a, true);
}

size_t titans_mem_scan_surprise_workspace_size(const titans_scan_desc* desc,
                                               const titans_mlp_desc* mlp) {
    titans::ScanArgs a{};
    if (prepare_scan(desc, mlp, a) != TITANS_OK) return SIZE_MAX;
    return workspace_of(a, true);
}

// The pair path run as a chain of calls over segments of the sequence, each within the
// static scratch array (no caller workspace, nothing allocated): segment 1 reads theta0 /
// s0, every later one continues in place from theta_T / s_T.  Segments are whole gradient
// chunks, so the chain equals one call bitwise (calls chain exactly).
static titans_status scan_pair_noalloc(titans::ScanArgs a, hipStream_t hs) {
    const size_t cap = titans::scan_pair_scratch_capacity();
    const size_t fixed = titans::scan_pair_scratch_exchange_bytes(a);
    const size_t per_chunk = titans::scan_pair_scratch_chunk_bytes(a);
    if (fixed + per_chunk > cap)
        return fail(TITANS_ERR_UNSUPPORTED,
                    "titans_mem_scan_noalloc: B*H=%lld with C=%d needs %zu bytes of scratch for one "
                    "chunk, more than the %zu-byte static array",
                    (long long)(a.B * a.H), a.C, fixed + per_chunk, cap);
    void* ws = nullptr;
    hipError_t e = titans::scan_pair_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "scratch address (hipGetSymbolAddress)");
    const int64_t seg = (int64_t)((cap - fixed) / per_chunk) * a.C;  // tokens per segment
    const size_t esz = a.io == TITANS_BF16 ? 2 : 4;
    titans::ScanArgs s = a;
    s.ws = ws;
    for (int64_t t0 = 0; t0 < a.T; t0 += seg) {
        s.T = a.T - t0 < seg ? a.T - t0 : seg;
        const size_t qo = (size_t)(t0 * a.qs[1]) * esz, yo = (size_t)(t0 * a.ys[1]) * esz;
        s.q = static_cast<const char*>(a.q) + qo;
        s.k = static_cast<const char*>(a.k) + qo;
        s.v = static_cast<const char*>(a.v) + qo;
        s.y = static_cast<char*>(a.y) + yo;
        s.alpha = a.alpha + t0 * a.gs[1];
        s.eta = a.eta + t0 * a.gs[1];
        s.beta = a.beta + t0 * a.gs[1];
        if (t0 > 0) {  // continue from the previous segment's state, in place
            s.theta0 = a.thetaT;
            s.s0 = a.sT;
            s.s0s[0] = a.ss[0];
            s.s0s[1] = a.ss[1];
        }
        e = titans::launch_scan_pair(s, hs);
        if (e != hipSuccess) return hip_fail(e, "scan launch");
    }
    return TITANS_OK;
}

static titans_status scan_impl(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                               const void* q, const void* k, const void* v, const float* alpha,
                               const float* eta, const float* beta, const float* theta0,
                               const float* s0, void* y, float* theta_T, float* s_T,
                               float* surprise, bool want_surprise, void* workspace,
                               size_t workspace_bytes, void* stream, bool noalloc = false) {
    g_last_error[0] = '\0';
    titans::ScanArgs a{};
    titans_status st = prepare_scan(desc, mlp, a);
    if (st) return st;
    const int64_t nseq = a.B * a.H;
    const bool have_tokens = nseq > 0 && a.T > 0;
    if (nseq > 0) {
        if (!theta0 || !s0 || !theta_T || !s_T)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "theta0, s0, theta_T and s_T must be non-NULL");
        if ((st = check_state_alignment(theta0, a.s0s, "theta0"))) return st;
        if ((st = check_state_alignment(s0, a.s0s, "s0"))) return st;
        if ((st = check_state_alignment(theta_T, a.ss, "theta_T"))) return st;
        if ((st = check_state_alignment(s_T, a.ss, "s_T"))) return st;
    }
    if (have_tokens) {
        if (!q || !k || !v || !alpha || !eta || !beta || !y)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "q, k, v, alpha, eta, beta and y must be non-NULL");
        if ((st = check_io_alignment(a, q, a.qs, "q"))) return st;
        if ((st = check_io_alignment(a, k, a.qs, "k"))) return st;
        if ((st = check_io_alignment(a, v, a.qs, "v"))) return st;
        if ((st = check_io_alignment(a, y, a.ys, "y"))) return st;
        if (want_surprise && !surprise)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "surprise must be non-NULL");
        if (want_surprise && (reinterpret_cast<uintptr_t>(surprise) & 3u) != 0)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "surprise is not 4-byte aligned");
    }
    // ---- aliasing rules
    const size_t esz = a.io == TITANS_BF16 ? 2 : 4;
    const int64_t io_sz[4] = {a.B, a.T, a.H, a.n[0]};
    const int64_t qst[4] = {a.qs[0], a.qs[1], a.qs[2], 1};
    const int64_t yst[4] = {a.ys[0], a.ys[1], a.ys[2], 1};
    const int64_t g_sz[3] = {a.B, a.T, a.H};
    const int64_t st_sz[3] = {a.B, a.H, a.P};
    const int64_t sst[3] = {a.ss[0], a.ss[1], 1};
    const int64_t s0st[3] = {a.s0s[0], a.s0s[1], 1};
    if (!non_self_overlapping(io_sz, yst, 4))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "y strides make distinct elements alias");
    if (!non_self_overlapping(st_sz, sst, 3))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "theta_T/s_T strides make distinct elements alias");
    if (want_surprise && have_tokens && !non_self_overlapping(g_sz, a.gs, 3))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "gate strides make distinct surprise elements alias");
    const Span ssur = (want_surprise && have_tokens) ? span_of(surprise, g_sz, a.gs, 3, 4) : Span{};
    Span sy = have_tokens ? span_of(y, io_sz, yst, 4, esz) : Span{};
    Span sth = span_of(theta_T, st_sz, sst, 3, 4), ssT = span_of(s_T, st_sz, sst, 3, 4);
    Span ins[8];
    int nin = 0;
    if (have_tokens) {
        ins[nin++] = span_of(q, io_sz, qst, 4, esz);
        ins[nin++] = span_of(k, io_sz, qst, 4, esz);
        ins[nin++] = span_of(v, io_sz, qst, 4, esz);
        ins[nin++] = span_of(alpha, g_sz, a.gs, 3, 4);
        ins[nin++] = span_of(eta, g_sz, a.gs, 3, 4);
        ins[nin++] = span_of(beta, g_sz, a.gs, 3, 4);
    }
    Span sth0 = span_of(theta0, st_sz, s0st, 3, 4), ss0 = span_of(s0, st_sz, s0st, 3, 4);
    const bool same_strides = a.ss[0] == a.s0s[0] && a.ss[1] == a.s0s[1];
    const bool theta_inplace = theta_T == theta0 && same_strides;
    const bool s_inplace = s_T == s0 && same_strides;
    for (int i = 0; i < nin; ++i) {
        if (overlaps(sy, ins[i]) || overlaps(sth, ins[i]) || overlaps(ssT, ins[i]))
            return fail(TITANS_ERR_INVALID_ARGUMENT, "an output overlaps an input");
    }
    if (overlaps(sy, sth) || overlaps(sy, ssT) || overlaps(sth, ssT) || overlaps(sy, sth0) ||
        overlaps(sy, ss0))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "outputs y, theta_T and s_T must not overlap");
    for (int i = 0; i < nin; ++i)
        if (overlaps(ssur, ins[i])) return fail(TITANS_ERR_INVALID_ARGUMENT, "surprise overlaps an input");
    if (overlaps(ssur, sy) || overlaps(ssur, sth) || overlaps(ssur, ssT) || overlaps(ssur, sth0) ||
        overlaps(ssur, ss0))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "surprise overlaps a state or output buffer");
    if (!theta_inplace && (overlaps(sth, sth0) || overlaps(sth, ss0)))
        return fail(TITANS_ERR_INVALID_ARGUMENT,
                    "theta_T overlaps theta0/s0 without being exactly theta0");
    if (!s_inplace && (overlaps(ssT, ss0) || overlaps(ssT, sth0)))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "s_T overlaps theta0/s0 without being exactly s0");
    if (theta_inplace && overlaps(sth, ss0) && !s_inplace)
        return fail(TITANS_ERR_INVALID_ARGUMENT, "theta_T overlaps s0");
    // ---- workspace (the allocation-free call has none: the pair path only, see below)
    if (noalloc && a.T > 0 && nseq > 0 && scan_path_of(a, false) != Path::Pair)
        return fail(TITANS_ERR_UNSUPPORTED,
                    "titans_mem_scan_noalloc serves the shapes titans_mem_scan runs on the pair path "
                    "(\"fused_pair\" / \"fused_quad\": the 64-256-64 memory, bf16 I/O, C a multiple "
                    "of 64, 2*ceil(B*H/8)*8 workgroups within the device's compute units); this one "
                    "takes \"%s\"",
                    path_name(scan_path_of(a, false), a));
    a.sides = pair_sides(a, want_surprise);
    size_t need = noalloc ? 0 : workspace_of(a, want_surprise);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(TITANS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                        workspace ? workspace_bytes : (size_t)0);
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
        Span sw{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
        for (int i = 0; i < nin; ++i)
            if (overlaps(sw, ins[i])) return fail(TITANS_ERR_INVALID_ARGUMENT, "workspace overlaps an input");
        if (overlaps(sw, sy) || overlaps(sw, sth) || overlaps(sw, ssT) || overlaps(sw, sth0) ||
            overlaps(sw, ss0) || overlaps(sw, ssur))
            return fail(TITANS_ERR_INVALID_ARGUMENT, "workspace overlaps a state or output buffer");
    }
    if (nseq == 0) return TITANS_OK;
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.eta = eta; a.beta = beta;
    a.theta0 = theta0; a.s0 = s0;
    a.y = y; a.thetaT = theta_T; a.sT = s_T;
    a.surprise = want_surprise ? surprise : nullptr;
    a.ws = workspace;
    // Test hook for the pair path's failure handling: side 1 of every memory never posts
    // its exchange flags and every wait gives up after a few polls, so the other sides time
    // out and every output of the memory comes out NaN while every kernel still ends
    // normally.
    const char* hook = debug_env("TITANS_MEM_TEST_PAIR_TIMEOUT");
    a.debug = (hook && hook[0] == '1') ? 1 : 0;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (noalloc && a.T > 0) return scan_pair_noalloc(a, hs);
    const Path path = a.T > 0 ? scan_path_of(a, want_surprise) : Path::Generic;
    hipError_t e = path == Path::Pair    ? titans::launch_scan_pair(a, hs)
                   : path == Path::Fused ? titans::launch_scan_mfma(a, hs)
                   : path == Path::Phased ? titans::launch_scan_phased(a, hs)
                   : path == Path::Linear ? titans::launch_scan_linear(a, hs)
                                          : titans::launch_scan_generic(a, hs);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
    return TITANS_OK;
}

titans_status titans_mem_scan(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                              const void* q, const void* k, const void* v, const float* alpha,
                              const float* eta, const float* beta, const float* theta0,
                              const float* s0, void* y, float* theta_T, float* s_T,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return scan_impl(desc, mlp, q, k, v, alpha, eta, beta, theta0, s0, y, theta_T, s_T, nullptr,
                     false, workspace, workspace_bytes, stream);
}

titans_status titans_mem_scan_noalloc(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                      const void* q, const void* k, const void* v,
                                      const float* alpha, const float* eta, const float* beta,
                                      const float* theta0, const float* s0, void* y,
                                      float* theta_T, float* s_T, void* stream) {
    return scan_impl(desc, mlp, q, k, v, alpha, eta, beta, theta0, s0, y, theta_T, s_T, nullptr,
                     false, nullptr, 0, stream, true);
}

titans_status titans_mem_scan_surprise(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                       const void* q, const void* k, const void* v,
                                       const float* alpha, const float* eta, const float* beta,
                                       const float* theta0, const float* s0, void* y,
                                       float* theta_T, float* s_T, float* surprise,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    return scan_impl(desc, mlp, q, k, v, alpha, eta, beta, theta0, s0, y, theta_T, s_T, surprise,
                     true, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- reverse pass

static titans_status prepare_backward(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                      titans::ScanArgs& a) {
    titans_status st = prepare_scan(desc, mlp, a);
    if (st) return st;
    if (a.bias == TITANS_BIAS_LP && a.bias_param < 2.f)
        return fail(TITANS_ERR_UNSUPPORTED,
                    "the reverse pass needs the l_p loss twice differentiable (p=%g < 2)",
                    (double)a.bias_param);
    return TITANS_OK;
}

size_t titans_mem_scan_backward_workspace_size(const titans_scan_desc* desc,
                                               const titans_mlp_desc* mlp) {
    titans::ScanArgs a{};
    if (prepare_backward(desc, mlp, a) != TITANS_OK) return SIZE_MAX;
    if (a.B * a.H == 0 || a.T == 0) return 0;
    return titans::scan_backward_workspace_bytes(a);
}

titans_status titans_mem_scan_backward(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                       const void* q, const void* k, const void* v,
                                       const float* alpha, const float* eta, const float* beta,
                                       const float* theta0, const float* s0, const void* dy,
                                       const float* dtheta_T, const float* ds_T, void* dq,
                                       void* dk, void* dv, float* dalpha, float* deta,
                                       float* dbeta, float* dtheta0, float* ds0,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    titans::ScanArgs a{};
    titans_status st = prepare_backward(desc, mlp, a);
    if (st) return st;
    const int64_t nseq = a.B * a.H;
    const bool have_tokens = nseq > 0 && a.T > 0;
    if (nseq > 0) {
        if (!theta0 || !s0 || !dtheta0 || !ds0)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "theta0, s0, dtheta0 and ds0 must be non-NULL");
        if ((st = check_state_alignment(theta0, a.s0s, "theta0"))) return st;
        if ((st = check_state_alignment(s0, a.s0s, "s0"))) return st;
        if ((st = check_state_alignment(dtheta0, a.ss, "dtheta0"))) return st;
        if ((st = check_state_alignment(ds0, a.ss, "ds0"))) return st;
        if (dtheta_T && (st = check_state_alignment(dtheta_T, a.ss, "dtheta_T"))) return st;
        if (ds_T && (st = check_state_alignment(ds_T, a.ss, "ds_T"))) return st;
    }
    if (have_tokens) {
        if (!q || !k || !v || !alpha || !eta || !beta || !dy || !dq || !dk || !dv || !dalpha ||
            !deta || !dbeta)
            return fail(TITANS_ERR_INVALID_ARGUMENT,
                        "q, k, v, the gates, dy and every token cotangent must be non-NULL");
        const void* io_ptrs[6] = {q, k, v, dq, dk, dv};
        const char* io_names[6] = {"q", "k", "v", "dq", "dk", "dv"};
        for (int i = 0; i < 6; ++i)
            if ((st = check_io_alignment(a, io_ptrs[i], a.qs, io_names[i]))) return st;
        if ((st = check_io_alignment(a, dy, a.ys, "dy"))) return st;
        const float* g_ptrs[3] = {dalpha, deta, dbeta};
        for (int i = 0; i < 3; ++i)
            if ((reinterpret_cast<uintptr_t>(g_ptrs[i]) & 3u) != 0)
                return fail(TITANS_ERR_INVALID_ARGUMENT, "gate cotangents must be 4-byte aligned");
    }
    // ---- aliasing: outputs distinct from each other, from every input and the workspace;
    // dtheta0 may be exactly dtheta_T and ds0 exactly ds_T (in place)
    const size_t esz = a.io == TITANS_BF16 ? 2 : 4;
    const int64_t io_sz[4] = {a.B, a.T, a.H, a.n[0]};
    const int64_t qst[4] = {a.qs[0], a.qs[1], a.qs[2], 1};
    const int64_t yst[4] = {a.ys[0], a.ys[1], a.ys[2], 1};
    const int64_t g_sz[3] = {a.B, a.T, a.H};
    const int64_t st_sz[3] = {a.B, a.H, a.P};
    const int64_t sst[3] = {a.ss[0], a.ss[1], 1};
    const int64_t s0st[3] = {a.s0s[0], a.s0s[1], 1};
    if (have_tokens && !non_self_overlapping(io_sz, qst, 4))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "q/k/v strides make distinct dq/dk/dv elements alias");
    if (have_tokens && !non_self_overlapping(g_sz, a.gs, 3))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "gate strides make distinct gate cotangents alias");
    if (!non_self_overlapping(st_sz, sst, 3))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "state strides make distinct dtheta0/ds0 elements alias");
    Span outs[8], ins[10];
    int nout = 0, nin = 0;
    if (have_tokens) {
        outs[nout++] = span_of(dq, io_sz, qst, 4, esz);
        outs[nout++] = span_of(dk, io_sz, qst, 4, esz);
        outs[nout++] = span_of(dv, io_sz, qst, 4, esz);
        outs[nout++] = span_of(dalpha, g_sz, a.gs, 3, 4);
        outs[nout++] = span_of(deta, g_sz, a.gs, 3, 4);
        outs[nout++] = span_of(dbeta, g_sz, a.gs, 3, 4);
        ins[nin++] = span_of(q, io_sz, qst, 4, esz);
        ins[nin++] = span_of(k, io_sz, qst, 4, esz);
        ins[nin++] = span_of(v, io_sz, qst, 4, esz);
        ins[nin++] = span_of(alpha, g_sz, a.gs, 3, 4);
        ins[nin++] = span_of(eta, g_sz, a.gs, 3, 4);
        ins[nin++] = span_of(beta, g_sz, a.gs, 3, 4);
        ins[nin++] = span_of(dy, io_sz, yst, 4, esz);
    }
    const Span sdth = span_of(dtheta0, st_sz, sst, 3, 4), sds = span_of(ds0, st_sz, sst, 3, 4);
    const Span sdT = dtheta_T ? span_of(dtheta_T, st_sz, sst, 3, 4) : Span{};
    const Span ssT = ds_T ? span_of(ds_T, st_sz, sst, 3, 4) : Span{};
    outs[nout++] = sdth;
    outs[nout++] = sds;
    ins[nin++] = span_of(theta0, st_sz, s0st, 3, 4);
    ins[nin++] = span_of(s0, st_sz, s0st, 3, 4);
    for (int i = 0; i < nout; ++i) {
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(TITANS_ERR_INVALID_ARGUMENT, "two cotangent outputs overlap");
        for (int j = 0; j < nin; ++j)
            if (overlaps(outs[i], ins[j]))
                return fail(TITANS_ERR_INVALID_ARGUMENT, "a cotangent output overlaps an input");
    }
    const bool th_inplace = dtheta_T == dtheta0;
    const bool s_inplace = ds_T == ds0;
    for (int i = 0; i < nout; ++i) {
        const bool is_dth = i == nout - 2, is_ds = i == nout - 1;
        if (overlaps(outs[i], sdT) && !(is_dth && th_inplace))
            return fail(TITANS_ERR_INVALID_ARGUMENT,
                        "dtheta_T overlaps an output without being exactly dtheta0");
        if (overlaps(outs[i], ssT) && !(is_ds && s_inplace))
            return fail(TITANS_ERR_INVALID_ARGUMENT, "ds_T overlaps an output without being exactly ds0");
    }
    const size_t need = have_tokens ? titans::scan_backward_workspace_bytes(a) : 0;
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(TITANS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                        workspace ? workspace_bytes : (size_t)0);
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
        const Span sw{reinterpret_cast<uintptr_t>(workspace),
                      reinterpret_cast<uintptr_t>(workspace) + need};
        for (int i = 0; i < nout; ++i)
            if (overlaps(sw, outs[i])) return fail(TITANS_ERR_INVALID_ARGUMENT, "workspace overlaps an output");
        for (int i = 0; i < nin; ++i)
            if (overlaps(sw, ins[i])) return fail(TITANS_ERR_INVALID_ARGUMENT, "workspace overlaps an input");
        if (overlaps(sw, sdT) || overlaps(sw, ssT))
            return fail(TITANS_ERR_INVALID_ARGUMENT, "workspace overlaps dtheta_T or ds_T");
    }
    if (nseq == 0) return TITANS_OK;
    titans::BwdArgs b{};
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.eta = eta; a.beta = beta;
    a.theta0 = theta0; a.s0 = s0;
    a.ws = workspace;
    b.a = a;
    b.dy = dy;
    b.dthetaT = dtheta_T;
    b.dsT = ds_T;
    b.dq = dq; b.dk = dk; b.dv = dv;
    b.dalpha = dalpha; b.deta = deta; b.dbeta = dbeta;
    b.dtheta0 = dtheta0;
    b.ds0 = ds0;
    const hipError_t e = titans::launch_scan_backward(b, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return TITANS_OK;
}

static titans_status prepare_retrieve(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                      titans::ScanArgs& a) {
    titans_status st = check_desc_common(desc, a);
    if (st) return st;
    if ((st = check_mlp(mlp, a))) return st;
    return check_shape_support(a, false);
}

enum class RPath { Fused, Wide, Generic };

// The 64-256-64 bf16 memory keeps its weights in LDS ("fused_mfma"); other bf16 memories
// with widths that are multiples of 16 stream them ("wide_mfma"); the rest, and fp32 I/O,
// take the generic kernel.  TITANS_MEM_FORCE_GENERIC=1 (with TITANS_MEM_DEBUG=1) forces
// the generic kernel.
static RPath retrieve_path_of(const titans::ScanArgs& a) {
    const char* env = debug_env("TITANS_MEM_FORCE_GENERIC");
    if (env && env[0] == '1') return RPath::Generic;
    if (titans::retrieve_mfma_supported(a)) return RPath::Fused;
    return titans::retrieve_wide_supported(a) ? RPath::Wide : RPath::Generic;
}

const char* titans_mem_retrieve_path(const titans_scan_desc* desc, const titans_mlp_desc* mlp) {
    titans::ScanArgs a{};
    if (prepare_retrieve(desc, mlp, a) != TITANS_OK) return nullptr;
    switch (retrieve_path_of(a)) {
        case RPath::Fused: return "fused_mfma";
        case RPath::Wide: return "wide_mfma";
        default: return a.io == TITANS_BF16 ? "generic_mfma" : "generic_fp32";
    }
}

titans_status titans_mem_retrieve(const titans_scan_desc* desc, const titans_mlp_desc* mlp,
                                  const void* q, const float* theta, void* y, void* stream) {
    g_last_error[0] = '\0';
    titans::ScanArgs a{};
    titans_status st = prepare_retrieve(desc, mlp, a);
    if (st) return st;
    const int64_t nseq = a.B * a.H;
    if (nseq == 0 || a.T == 0) return TITANS_OK;
    if (!q || !theta || !y)
        return fail(TITANS_ERR_INVALID_ARGUMENT, "q, theta and y must be non-NULL");
    if ((st = check_io_alignment(a, q, a.qs, "q"))) return st;
    if ((st = check_io_alignment(a, y, a.ys, "y"))) return st;
    if ((st = check_state_alignment(theta, a.ss, "theta"))) return st;
    const size_t esz = a.io == TITANS_BF16 ? 2 : 4;
    const int64_t io_sz[4] = {a.B, a.T, a.H, a.n[0]};
    const int64_t qst[4] = {a.qs[0], a.qs[1], a.qs[2], 1};
    const int64_t yst[4] = {a.ys[0], a.ys[1], a.ys[2], 1};
    const int64_t st_sz[3] = {a.B, a.H, a.P};
    const int64_t sst[3] = {a.ss[0], a.ss[1], 1};
    if (!non_self_overlapping(io_sz, yst, 4))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "y strides make distinct elements alias");
    Span sy = span_of(y, io_sz, yst, 4, esz);
    if (overlaps(sy, span_of(q, io_sz, qst, 4, esz)) || overlaps(sy, span_of(theta, st_sz, sst, 3, 4)))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "y overlaps q or theta");
    a.q = q;
    a.thetaT = const_cast<float*>(theta);
    a.y = y;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const RPath rp = retrieve_path_of(a);
    hipError_t e = rp == RPath::Fused  ? titans::launch_retrieve_mfma(a, device_cus(), hs)
                   : rp == RPath::Wide ? titans::launch_retrieve_wide(a, hs)
                                       : titans::launch_retrieve_generic(a, hs);
    if (e != hipSuccess) return hip_fail(e, "retrieve launch");
    return TITANS_OK;
}

// ---------------------------------------------------------------- MAG block

static Span contiguous(const void* p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, p ? lo + bytes : lo};
}

// The memory scan of the block: bf16 [B, T, H, d] q / k / v / y, [B, T, H] gates,
// contiguous [B, H, P] states, the squared-error bias.
static titans_scan_desc mag_scan_desc(const titans_mag_desc* desc, int d, int64_t P) {
    titans_scan_desc s{};
    const int64_t B = desc->batch, T = desc->seq_len, H = desc->heads, D = H * d;
    s.batch = B;
    s.seq_len = T;
    s.heads = H;
    s.chunk = desc->chunk;
    s.io_dtype = TITANS_BF16;
    s.qkv_stride[0] = s.y_stride[0] = T * D;
    s.qkv_stride[1] = s.y_stride[1] = D;
    s.qkv_stride[2] = s.y_stride[2] = d;
    s.gate_stride[0] = T * H;
    s.gate_stride[1] = H;
    s.gate_stride[2] = 1;
    s.state_stride[0] = s.state0_stride[0] = H * P;
    s.state_stride[1] = s.state0_stride[1] = P;
    s.bias = TITANS_BIAS_L2;
    s.bias_param = 0.f;
    return s;
}

static titans_status prepare_mag(const titans_mag_desc* desc, const titans_mlp_desc* mlp,
                                 titans::MagArgs& g, titans_scan_desc& sd, titans::ScanArgs& a) {
    if (!desc || !mlp) return fail(TITANS_ERR_INVALID_ARGUMENT, "desc and mlp must be non-NULL");
    if (desc->batch < 0 || desc->seq_len < 0 || desc->heads < 1)
        return fail(TITANS_ERR_INVALID_ARGUMENT, "need batch >= 0, seq_len >= 0, heads >= 1");
    if (desc->chunk < 1) return fail(TITANS_ERR_INVALID_ARGUMENT, "chunk=%d must be >= 1", desc->chunk);
    if (desc->window < 1)
        return fail(TITANS_ERR_INVALID_ARGUMENT, "window=%d must be >= 1", desc->window);
    if (!(desc->eta_scale >= 0.f && desc->eta_scale < INFINITY))
        return fail(TITANS_ERR_INVALID_ARGUMENT, "eta_scale=%g must be finite and >= 0",
                    (double)desc->eta_scale);
    if (desc->reserved != 0) return fail(TITANS_ERR_INVALID_ARGUMENT, "reserved must be 0");
    titans::ScanArgs m{};
    titans_status st = check_mlp(mlp, m);
    if (st) return st;
    const int d = m.n[0];
    if (m.n[m.L] != d)
        return fail(TITANS_ERR_INVALID_ARGUMENT,
                    "the memory's output width %d must equal its input width %d", m.n[m.L], d);
    if (!titans::mag_head_dim_supported(d))
        return fail(TITANS_ERR_UNSUPPORTED, "head width d=%d: the attention takes 32, 64 or 128", d);
    if (desc->heads > 65536 / d)
        return fail(TITANS_ERR_UNSUPPORTED, "heads * d = %lld exceeds 65536",
                    (long long)(desc->heads * d));
    const int64_t nqb = (desc->seq_len + 63) / 64;
    const int64_t tiles_m = (desc->batch * desc->seq_len + 127) / 128;
    const int64_t tiles_n = (3 * desc->heads * d + 3 * desc->heads + 127) / 128;
    if (desc->batch * desc->heads * nqb > 0xffffffffLL || tiles_m * tiles_n > 0xffffffffLL ||
        desc->batch * desc->seq_len > 0xffffffffLL || desc->seq_len >= (1LL << 30))
        return fail(TITANS_ERR_UNSUPPORTED,
                    "seq_len >= 2^30 or batch * seq_len too large for one launch");
    sd = mag_scan_desc(desc, d, m.P);
    if ((st = prepare_scan(&sd, mlp, a))) return st;
    g = titans::MagArgs{};
    g.B = desc->batch;
    g.T = desc->seq_len;
    g.H = desc->heads;
    g.d = d;
    g.window = desc->window;
    g.eta_scale = desc->eta_scale;
    return TITANS_OK;
}

// The block's own pieces, then the scan's workspace (256-byte aligned offset).
static size_t mag_own_bytes(const titans::MagArgs& g) {
    return (titans::mag_workspace_bytes(g) + 255) / 256 * 256;
}

size_t titans_mag_workspace_size(const titans_mag_desc* desc, const titans_mlp_desc* mlp) {
    titans::MagArgs g;
    titans_scan_desc sd;
    titans::ScanArgs a{};
    if (prepare_mag(desc, mlp, g, sd, a) != TITANS_OK) return SIZE_MAX;
    return mag_own_bytes(g) + workspace_of(a, false);
}

// Pointers, alignment, overlap and workspace of a block call (MAG or MAC): x [B, T, D],
// W_in [3D + 3H, D], W_out [D, D] bf16, b_gate [3H], contiguous [B, H, P] states.
static titans_status check_block_args(const titans::MagArgs& g, const titans::ScanArgs& a,
                                      const void* x, const void* w_in, const float* b_gate,
                                      const void* w_out, const float* theta0, const float* s0,
                                      const void* out, const float* theta_T, const float* s_T,
                                      const void* workspace, size_t workspace_bytes, size_t need) {
    const int64_t B = g.B, H = g.H, D = H * g.d, M = B * g.T, P = a.P;
    const bool tokens = M > 0;
    titans_status st;
    if (B > 0) {
        if (!theta0 || !s0 || !theta_T || !s_T)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "theta0, s0, theta_T and s_T must be non-NULL");
        if ((st = check_state_alignment(theta0, a.s0s, "theta0"))) return st;
        if ((st = check_state_alignment(s0, a.s0s, "s0"))) return st;
        if ((st = check_state_alignment(theta_T, a.ss, "theta_T"))) return st;
        if ((st = check_state_alignment(s_T, a.ss, "s_T"))) return st;
    }
    // x and the weights are read only when there are tokens
    if (tokens) {
        if (!x || !w_in || !b_gate || !w_out || !out)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "x, w_in, b_gate, w_out and out must be non-NULL");
        const void* a16[3] = {x, w_in, w_out};
        const char* n16[3] = {"x", "w_in", "w_out"};
        for (int i = 0; i < 3; ++i)
            if (reinterpret_cast<uintptr_t>(a16[i]) & 15u)
                return fail(TITANS_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n16[i]);
        if (reinterpret_cast<uintptr_t>(out) & 7u)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "out is not 8-byte aligned");
        if (reinterpret_cast<uintptr_t>(b_gate) & 3u)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "b_gate is not 4-byte aligned");
    }
    const size_t state_bytes = static_cast<size_t>(B * H * P) * 4;
    const Span ins[6] = {tokens ? contiguous(x, static_cast<size_t>(M * D) * 2) : Span{},
                         tokens ? contiguous(w_in, static_cast<size_t>((3 * D + 3 * H) * D) * 2) : Span{},
                         tokens ? contiguous(b_gate, static_cast<size_t>(3 * H) * 4) : Span{},
                         tokens ? contiguous(w_out, static_cast<size_t>(D * D) * 2) : Span{},
                         contiguous(theta0, state_bytes), contiguous(s0, state_bytes)};
    const Span outs[4] = {tokens ? contiguous(out, static_cast<size_t>(M * D) * 2) : Span{},
                          contiguous(theta_T, state_bytes), contiguous(s_T, state_bytes),
                          need ? contiguous(workspace, need) : Span{}};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], ins[j]))
                return fail(TITANS_ERR_INVALID_ARGUMENT,
                            "out, theta_T, s_T and the workspace must not overlap an input");
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(TITANS_ERR_INVALID_ARGUMENT,
                            "out, theta_T, s_T and the workspace must not overlap each other");
    }
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(TITANS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                        workspace ? workspace_bytes : (size_t)0);
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return fail(TITANS_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    }
    return TITANS_OK;
}

titans_status titans_mag_forward(const titans_mag_desc* desc, const titans_mlp_desc* mlp,
                                 const void* x, const void* w_in, const float* b_gate,
                                 const void* w_out, const float* theta0, const float* s0,
                                 void* out, float* theta_T, float* s_T, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    titans::MagArgs g;
    titans_scan_desc sd;
    titans::ScanArgs a{};
    titans_status st = prepare_mag(desc, mlp, g, sd, a);
    if (st) return st;
    const bool tokens = g.B * g.T > 0;
    const size_t own = tokens ? mag_own_bytes(g) : 0;
    const size_t scan_ws = workspace_of(a, false);
    const size_t need = tokens ? own + scan_ws : 0;
    if ((st = check_block_args(g, a, x, w_in, b_gate, w_out, theta0, s0, out, theta_T, s_T,
                               workspace, workspace_bytes, need)))
        return st;
    if (g.B == 0) return TITANS_OK;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (!tokens)  // no tokens: the memory passes through unchanged
        return scan_impl(&sd, mlp, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, theta0, s0,
                         nullptr, theta_T, s_T, nullptr, false, nullptr, 0, stream);
    g.x = static_cast<const __bf16*>(x);
    g.w_in = static_cast<const __bf16*>(w_in);
    g.b_gate = b_gate;
    g.w_out = static_cast<const __bf16*>(w_out);
    g.out = static_cast<__bf16*>(out);
    titans::mag_place(g, workspace);
    hipError_t e = titans::launch_mag_front(g, hs);
    if (e != hipSuccess) return hip_fail(e, "MAG front-end launch");
    st = scan_impl(&sd, mlp, g.q, g.k, g.v, g.alpha, g.eta, g.beta, theta0, s0, g.ymem, theta_T,
                   s_T, nullptr, false, scan_ws ? static_cast<char*>(workspace) + own : nullptr,
                   scan_ws, stream);
    if (st) return st;
    if ((e = titans::launch_mag_attention(g, hs)) != hipSuccess)
        return hip_fail(e, "MAG attention launch");
    if ((e = titans::launch_mag_out(g, hs)) != hipSuccess)
        return hip_fail(e, "MAG output projection launch");
    return TITANS_OK;
}

// ---------------------------------------------------------------- MAC block

static titans_mag_desc mac_as_mag(const titans_mac_desc* d) {
    titans_mag_desc m{};
    m.batch = d->batch;
    m.seq_len = d->seq_len;
    m.heads = d->heads;
    m.chunk = d->chunk;
    m.window = d->segment;  // validated as >= 1 like a window
    m.eta_scale = d->eta_scale;
    m.reserved = d->reserved;
    return m;
}

// The MAG layout, then the memory reads h (bf16 [B, T, H, d]), then the scan's workspace
// for one segment; `seg` receives the scan descriptor of a segment of `len` tokens.
struct MacPlan {
    titans::MagArgs g;
    titans_scan_desc sd;
    titans::ScanArgs a;
    int64_t S;
    size_t own, scan_ws;
};

static titans_status prepare_mac(const titans_mac_desc* desc, const titans_mlp_desc* mlp,
                                 MacPlan& p) {
    if (!desc) return fail(TITANS_ERR_INVALID_ARGUMENT, "desc and mlp must be non-NULL");
    const titans_mag_desc md = mac_as_mag(desc);
    p.a = titans::ScanArgs{};
    titans_status st = prepare_mag(&md, mlp, p.g, p.sd, p.a);
    if (st) return st;
    p.S = desc->segment;
    const int64_t M = p.g.B * p.g.T, D = p.g.H * p.g.d;
    p.own = M > 0 ? mag_own_bytes(p.g) + static_cast<size_t>((M * D * 2 + 255) / 256 * 256) : 0;
    p.scan_ws = 0;
    // the segments' scans (the first is the longest; the last may be shorter)
    const int64_t T = p.g.T;
    const int64_t lens[2] = {T < p.S ? T : p.S, T % p.S};
    for (int i = 0; i < 2; ++i) {
        if (lens[i] == 0) continue;
        titans_scan_desc sdi = p.sd;
        sdi.seq_len = lens[i];
        titans::ScanArgs ai{};
        if ((st = prepare_scan(&sdi, mlp, ai))) return st;
        const size_t w = workspace_of(ai, false);
        p.scan_ws = w > p.scan_ws ? w : p.scan_ws;
    }
    return TITANS_OK;
}

size_t titans_mac_workspace_size(const titans_mac_desc* desc, const titans_mlp_desc* mlp) {
    MacPlan p;
    if (prepare_mac(desc, mlp, p) != TITANS_OK) return SIZE_MAX;
    return p.g.B * p.g.T > 0 ? p.own + p.scan_ws : 0;
}

titans_status titans_mac_forward(const titans_mac_desc* desc, const titans_mlp_desc* mlp,
                                 const void* x, const void* w_in, const float* b_gate,
                                 const void* w_out, const float* theta0, const float* s0,
                                 void* out, float* theta_T, float* s_T, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    MacPlan p;
    titans_status st = prepare_mac(desc, mlp, p);
    if (st) return st;
    titans::MagArgs& g = p.g;
    const int64_t T = g.T, H = g.H, D = H * g.d;
    const bool tokens = g.B * T > 0;
    const size_t need = tokens ? p.own + p.scan_ws : 0;
    if ((st = check_block_args(g, p.a, x, w_in, b_gate, w_out, theta0, s0, out, theta_T, s_T,
                               workspace, workspace_bytes, need)))
        return st;
    if (g.B == 0) return TITANS_OK;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (!tokens)
        return scan_impl(&p.sd, mlp, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, theta0,
                         s0, nullptr, theta_T, s_T, nullptr, false, nullptr, 0, stream);
    g.x = static_cast<const __bf16*>(x);
    g.w_in = static_cast<const __bf16*>(w_in);
    g.b_gate = b_gate;
    g.w_out = static_cast<const __bf16*>(w_out);
    g.out = static_cast<__bf16*>(out);
    titans::mag_place(g, workspace);
    __bf16* hbuf = reinterpret_cast<__bf16*>(static_cast<char*>(workspace) + mag_own_bytes(g));
    void* scan_ws = p.scan_ws ? static_cast<char*>(workspace) + p.own : nullptr;
    hipError_t e = titans::launch_mag_front(g, hs);
    if (e != hipSuccess) return hip_fail(e, "MAC front-end launch");
    for (int64_t t0 = 0; t0 < T; t0 += p.S) {
        const int64_t len = T - t0 < p.S ? T - t0 : p.S;
        const float* th = t0 == 0 ? theta0 : theta_T;
        const float* sg = t0 == 0 ? s0 : s_T;
        titans_scan_desc sdi = p.sd;
        sdi.seq_len = len;
        // the segment's memory reads at the state before it, then its writes (in place
        // on theta_T / s_T after the first segment), then its attention
        if ((st = titans_mem_retrieve(&sdi, mlp, g.q + t0 * D, th, hbuf + t0 * D, stream)))
            return st;
        if ((st = scan_impl(&sdi, mlp, g.q + t0 * D, g.k + t0 * D, g.v + t0 * D, g.alpha + t0 * H,
                            g.eta + t0 * H, g.beta + t0 * H, th, sg, g.ymem + t0 * D, theta_T,
                            s_T, nullptr, false, scan_ws, p.scan_ws, stream)))
            return st;
        if ((e = titans::launch_mac_attention(g, hbuf, t0, len, hs)) != hipSuccess)
            return hip_fail(e, "MAC attention launch");
    }
    if ((e = titans::launch_mag_out(g, hs)) != hipSuccess)
        return hip_fail(e, "MAC output projection launch");
    return TITANS_OK;
}

}  // extern "C"
