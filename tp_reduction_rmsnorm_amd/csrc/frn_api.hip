// frn_api.hip -- the extern "C" entry points of include/fused_reduce_norm.h:
// argument checks, the decline rule and kernel launches.  Every check runs
// before the first launch, so a rejected call leaves every output untouched
// (the fail-closed contract of vLLM PR #62366 "Details" and SGLang PR
// #34134: a call that cannot be served says so instead of silently skipping
// the reduction).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "frn_internal.h"

#define FRN_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[256] = "";

frn_status fail(frn_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

bool force_decline() {
    static const bool forced = [] {
        const char* e = getenv("FRN_FORCE_DECLINE");
        return e != nullptr && e[0] == '1';
    }();
    return forced;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};

Span span(const char* name, const void* p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{name, lo, lo + bytes};
}

bool overlap(const Span& a, const Span& b) {
    return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

// Sizes that are malformed (INVALID) or outside what the kernels serve
// (UNSUPPORTED).  k == 0: no finalize.
frn_status check_sizes(int32_t R, int32_t k, int64_t T, int64_t H, int32_t epilogue) {
    if (R < 1) return fail(FRN_ERR_INVALID, "R must be >= 1 (got %d)", R);
    if (k < 0) return fail(FRN_ERR_INVALID, "k must be >= 0 (got %d)", k);
    if (T < 0) return fail(FRN_ERR_INVALID, "T must be >= 0 (got %lld)", (long long)T);
    if (H <= 0) return fail(FRN_ERR_INVALID, "H must be > 0 (got %lld)", (long long)H);
    if (epilogue != FRN_EPI_RMSNORM && epilogue != FRN_EPI_SANDWICH && epilogue != frn::kStoreSum)
        return fail(FRN_ERR_INVALID, "unknown epilogue %d", epilogue);
    if (force_decline()) return fail(FRN_ERR_UNSUPPORTED, "declined: FRN_FORCE_DECLINE=1");
    if (R > FRN_MAX_R) return fail(FRN_ERR_UNSUPPORTED, "R=%d exceeds %d", R, FRN_MAX_R);
    if (k > FRN_MAX_K) return fail(FRN_ERR_UNSUPPORTED, "k=%d exceeds %d", k, FRN_MAX_K);
    if (H % 8 != 0)
        return fail(FRN_ERR_UNSUPPORTED, "H=%lld is not a multiple of 8", (long long)H);
    if (H < 8 || H > FRN_MAX_H)
        return fail(FRN_ERR_UNSUPPORTED, "H=%lld outside [8, %d]", (long long)H, FRN_MAX_H);
    if (T > FRN_MAX_T)
        return fail(FRN_ERR_UNSUPPORTED, "T=%lld exceeds %d rows", (long long)T, FRN_MAX_T);
    return FRN_OK;
}

// Pointer checks shared by every call.
struct Call {
    frn::RowArgs a;
    Span in[3 * FRN_MAX_R + 6];
    int n_in = 0;
    Span outs[FRN_MAX_R + 4];
    int n_out = 0;
};

frn_status add_in(Call& c, const char* name, const void* p, size_t bytes, bool need16 = true) {
    if (p == nullptr) return fail(FRN_ERR_INVALID, "%s is NULL", name);
    if (need16 && !aligned16(p))
        return fail(FRN_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
    if (!need16 && (reinterpret_cast<uintptr_t>(p) & 3u))
        return fail(FRN_ERR_UNSUPPORTED, "%s is not 4-byte aligned", name);
    c.in[c.n_in++] = span(name, p, bytes);
    return FRN_OK;
}

frn_status add_out(Call& c, const char* name, void* p, size_t bytes) {
    if (p == nullptr) return fail(FRN_ERR_INVALID, "%s is NULL", name);
    if (!aligned16(p)) return fail(FRN_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
    c.outs[c.n_out++] = span(name, p, bytes);
    return FRN_OK;
}

// Outputs may not overlap inputs or each other; the one exception is the
// residual updated in place (residual_out == residual_in, same extent).
frn_status check_alias(const Call& c) {
    for (int o = 0; o < c.n_out; ++o) {
        for (int i = 0; i < c.n_in; ++i) {
            const bool in_place = strcmp(c.outs[o].name, "residual_out") == 0 &&
                                  strcmp(c.in[i].name, "residual_in") == 0 &&
                                  c.outs[o].lo == c.in[i].lo && c.outs[o].hi == c.in[i].hi;
            if (!in_place && overlap(c.outs[o], c.in[i]))
                return fail(FRN_ERR_INVALID, "%s overlaps %s", c.outs[o].name, c.in[i].name);
        }
        for (int p = o + 1; p < c.n_out; ++p)
            if (overlap(c.outs[o], c.outs[p]))
                return fail(FRN_ERR_INVALID, "%s overlaps %s", c.outs[o].name, c.outs[p].name);
    }
    return FRN_OK;
}

// Top-k routing of a finalize: the weights [T,k] shared by every rank, and
// per rank the row-index array [T,k] and the row count of its expert buffer.
// Under TP every rank gets the same index array and row count; under
// expert-parallel routing (ep) each rank has its own, a negative index marks
// another rank's slot, and a rank may own no rows (its buffer may be NULL).
struct Routing {
    const float* topk_w = nullptr;
    const int32_t* rows[FRN_MAX_R] = {};
    int64_t num_rows[FRN_MAX_R] = {};
    bool ep = false;
};

Routing tp_routing(int32_t R, const float* topk_w, const int32_t* topk_row, int64_t num_rows) {
    Routing g;
    g.topk_w = topk_w;
    for (int r = 0; r < R && r < FRN_MAX_R; ++r) {
        g.rows[r] = topk_row;
        g.num_rows[r] = num_rows;
    }
    return g;
}

frn_status ep_routing(Routing& g, int32_t R, const float* topk_w,
                      const int32_t* const* topk_rows, const int64_t* num_rows) {
    if (topk_rows == nullptr) return fail(FRN_ERR_INVALID, "topk_rows pointer array is NULL");
    if (num_rows == nullptr) return fail(FRN_ERR_INVALID, "num_rows array is NULL");
    g.topk_w = topk_w;
    g.ep = true;
    for (int r = 0; r < R && r < FRN_MAX_R; ++r) {
        g.rows[r] = topk_rows[r];
        g.num_rows[r] = num_rows[r];
    }
    return FRN_OK;
}

// Fill the source part of the argument block: partials (k == 0) or the
// finalize operands (k > 0).
frn_status set_sources(Call& c, const void* const* src, const void* const* shared, int32_t R,
                       const Routing& g, int32_t k, int64_t T, int64_t H) {
    static const char* const kSrcNames[FRN_MAX_R] = {
        "src[0]", "src[1]", "src[2]", "src[3]", "src[4]", "src[5]", "src[6]", "src[7]",
        "src[8]", "src[9]", "src[10]", "src[11]", "src[12]", "src[13]", "src[14]", "src[15]"};
    static const char* const kSharedNames[FRN_MAX_R] = {
        "shared[0]", "shared[1]", "shared[2]", "shared[3]", "shared[4]", "shared[5]",
        "shared[6]", "shared[7]", "shared[8]", "shared[9]", "shared[10]", "shared[11]",
        "shared[12]", "shared[13]", "shared[14]", "shared[15]"};
    static const char* const kRowNames[FRN_MAX_R] = {
        "topk_rows[0]", "topk_rows[1]", "topk_rows[2]", "topk_rows[3]", "topk_rows[4]",
        "topk_rows[5]", "topk_rows[6]", "topk_rows[7]", "topk_rows[8]", "topk_rows[9]",
        "topk_rows[10]", "topk_rows[11]", "topk_rows[12]", "topk_rows[13]", "topk_rows[14]",
        "topk_rows[15]"};
    if (src == nullptr) return fail(FRN_ERR_INVALID, "source pointer array is NULL");
    const size_t row_bytes = (size_t)H * 2;
    frn_status st;
    c.a.ep = 0;
    if (k > 0) {
        if ((st = add_in(c, "topk_w", g.topk_w, (size_t)T * k * 4, false)) != FRN_OK) return st;
        c.a.topk_w = g.topk_w;
        c.a.ep = g.ep ? 1 : 0;
        for (int r = 0; r < R; ++r) {
            const int64_t n = g.num_rows[r];
            if (n < (g.ep ? 0 : 1))
                return fail(FRN_ERR_INVALID, g.ep ? "num_rows[%d] is negative"
                                                  : "num_rows must be >= 1", r);
            if (n > (int64_t)0x7fffffff)
                return fail(FRN_ERR_UNSUPPORTED, "num_rows exceeds int32 indexing");
            if (g.ep || r == 0) {
                st = add_in(c, g.ep ? kRowNames[r] : "topk_row", g.rows[r], (size_t)T * k * 4,
                            false);
                if (st != FRN_OK) return st;
            }
            c.a.topk_row[r] = g.rows[r];
            c.a.num_rows[r] = n;
        }
    }
    for (int r = 0; r < R; ++r) {
        c.a.src[r] = static_cast<const uint4*>(src[r]);
        c.a.shared[r] = nullptr;
        // an expert-parallel rank without rows never has its buffer read
        if (k > 0 && g.ep && g.num_rows[r] == 0 && src[r] == nullptr) continue;
        const size_t bytes = (k > 0 ? (size_t)g.num_rows[r] : (size_t)T) * row_bytes;
        if ((st = add_in(c, kSrcNames[r], src[r], bytes)) != FRN_OK) return st;
    }
    if (k > 0 && shared != nullptr) {
        for (int r = 0; r < R; ++r) {
            if (g.ep && shared[r] == nullptr) continue;  // this rank holds no shared expert
            if ((st = add_in(c, kSharedNames[r], shared[r], (size_t)T * row_bytes)) != FRN_OK)
                return st;
            c.a.shared[r] = static_cast<const uint4*>(shared[r]);
        }
    }
    c.a.R = R;
    c.a.k = k;
    c.a.T = T;
    c.a.nvec = (int32_t)(H / 8);
    c.a.H = (int32_t)H;
    return FRN_OK;
}

frn_status set_epilogue(Call& c, int32_t epilogue, const void* residual_in, const float* g1,
                        const float* g2, float eps, int64_t T, int64_t H, void* out,
                        void* residual_out) {
    frn_status st;
    if (!(eps >= 0.0f) || !__builtin_isfinite(eps))
        return fail(FRN_ERR_INVALID, "eps must be finite and >= 0");
    const size_t tensor = (size_t)T * H * 2;
    if ((st = add_in(c, "residual_in", residual_in, tensor)) != FRN_OK) return st;
    if ((st = add_in(c, "gamma1", g1, (size_t)H * 4)) != FRN_OK) return st;
    if (epilogue == FRN_EPI_SANDWICH) {
        if ((st = add_in(c, "gamma2", g2, (size_t)H * 4)) != FRN_OK) return st;
    }
    if ((st = add_out(c, "out", out, tensor)) != FRN_OK) return st;
    if ((st = add_out(c, "residual_out", residual_out, tensor)) != FRN_OK) return st;
    c.a.residual = static_cast<const uint4*>(residual_in);
    c.a.gamma1 = reinterpret_cast<const float4*>(g1);
    c.a.gamma2 = reinterpret_cast<const float4*>(epilogue == FRN_EPI_SANDWICH ? g2 : g1);
    c.a.out = static_cast<uint4*>(out);
    c.a.residual_out = static_cast<uint4*>(residual_out);
    c.a.eps = eps;
    return FRN_OK;
}

frn_status run(const Call& c, int32_t epilogue, int64_t T, void* stream) {
    if (T == 0) return FRN_OK;
    const hipError_t e = frn::launch_rows(c.a, epilogue, T, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FRN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return FRN_OK;
}

// The optional workspace serves the split-row finalize where that is the
// chosen path for this call; a call that does not take it ignores the
// workspace (the one-row kernel needs none).  A workspace too small for the
// chosen mode declines the call, as a misaligned one does.
frn_status set_workspace(Call& c, void* workspace, size_t workspace_bytes, int32_t k, int64_t T,
                         int64_t H, int32_t R, int32_t epilogue) {
    c.a.ws_sum = nullptr;
    if (k == 0 || workspace == nullptr) return FRN_OK;
    if (!frn::use_split_rows(R, H, k, c.a.ep != 0, epilogue, T)) return FRN_OK;
    const size_t need = frn::split_workspace_bytes(T, H);
    if (workspace_bytes < need)
        return fail(FRN_ERR_UNSUPPORTED,
                    "workspace of %zu bytes is smaller than the %zu bytes the split-row "
                    "finalize needs at T=%lld (frn_workspace_bytes)",
                    workspace_bytes, need, (long long)T);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(FRN_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
    frn_status st = add_out(c, "workspace", workspace, need);
    if (st != FRN_OK) return st;
    c.a.ws_sum = static_cast<float4*>(workspace);
    c.a.ws_ss = reinterpret_cast<double*>(static_cast<char*>(workspace) +
                                          frn::split_ss_offset(T, H));
    return FRN_OK;
}

frn_status fused(const void* const* src, const void* const* shared, int32_t R,
                 const Routing& g, int32_t k, int32_t epilogue, const void* residual_in,
                 const float* g1, const float* g2, float eps, int64_t T, int64_t H, void* out,
                 void* residual_out, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    frn_status st = check_sizes(R, k, T, H, epilogue);
    if (st != FRN_OK || T == 0) return st;  // empty tensors may carry null pointers
    Call c{};
    if ((st = set_sources(c, src, shared, R, g, k, T, H)) != FRN_OK) return st;
    if ((st = set_epilogue(c, epilogue, residual_in, g1, g2, eps, T, H, out, residual_out)) !=
        FRN_OK)
        return st;
    if ((st = set_workspace(c, workspace, workspace_bytes, k, T, H, R, epilogue)) != FRN_OK)
        return st;
    if ((st = check_alias(c)) != FRN_OK) return st;
    return run(c, epilogue, T, stream);
}

// Checks of a finalize call's k and epilogue that come before the sizes.
frn_status check_finalize_call(int32_t k, int32_t epilogue) {
    if (k < 1) return fail(FRN_ERR_INVALID, "k must be >= 1 for the finalize (got %d)", k);
    if (epilogue != FRN_EPI_RMSNORM && epilogue != FRN_EPI_SANDWICH)
        return fail(FRN_ERR_INVALID, "unknown epilogue %d", epilogue);
    return FRN_OK;
}

frn_status pass1(const void* const* src, const void* const* shared, int32_t R,
                 const Routing& g, int32_t k, int64_t T, int64_t H, void* sum_out,
                 void* stream) {
    g_last_error[0] = '\0';
    frn_status st = check_sizes(R, k, T, H, frn::kStoreSum);
    if (st != FRN_OK || T == 0) return st;
    Call c{};
    if ((st = set_sources(c, src, shared, R, g, k, T, H)) != FRN_OK) return st;
    if ((st = add_out(c, "sum_out", sum_out, (size_t)T * H * 2)) != FRN_OK) return st;
    if ((st = check_alias(c)) != FRN_OK) return st;
    c.a.out = static_cast<uint4*>(sum_out);
    return run(c, frn::kStoreSum, T, stream);
}

}  // namespace

FRN_API frn_status frn_reduce_residual_rmsnorm(const void* const* partials, int32_t R,
                                               const void* residual_in, const float* gamma,
                                               float eps, int64_t T, int64_t H, void* out,
                                               void* residual_out, void* workspace,
                                               size_t workspace_bytes, void* stream) {
    return fused(partials, nullptr, R, Routing{}, 0, FRN_EPI_RMSNORM, residual_in,
                 gamma, nullptr, eps, T, H, out, residual_out, workspace, workspace_bytes,
                 stream);
}

FRN_API frn_status frn_reduce_sandwich_norm(const void* const* partials, int32_t R,
                                            const void* residual_in, const float* gamma1,
                                            const float* gamma2, float eps, int64_t T,
                                            int64_t H, void* out, void* residual_out,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream) {
    return fused(partials, nullptr, R, Routing{}, 0, FRN_EPI_SANDWICH, residual_in,
                 gamma1, gamma2, eps, T, H, out, residual_out, workspace, workspace_bytes,
                 stream);
}

FRN_API frn_status frn_moe_finalize_reduce_norm(
    const void* const* expert_rows, const void* const* shared, int32_t R, const float* topk_w,
    const int32_t* topk_row, int32_t k, int64_t num_rows, int32_t epilogue,
    const void* residual_in, const float* gamma1, const float* gamma2, float eps, int64_t T,
    int64_t H, void* out, void* residual_out, void* workspace, size_t workspace_bytes,
    void* stream) {
    g_last_error[0] = '\0';
    const frn_status st = check_finalize_call(k, epilogue);
    if (st != FRN_OK) return st;
    return fused(expert_rows, shared, R, tp_routing(R, topk_w, topk_row, num_rows), k, epilogue,
                 residual_in, gamma1, gamma2, eps, T, H, out, residual_out, workspace,
                 workspace_bytes, stream);
}

// ------------------------------------------- the no-allocation entry point --- //

// Scratch memory of frn_moe_finalize_reduce_norm_noalloc: the split-row
// finalize's workspace (T x H FP32 rows, then the FP64 slice sums), for
// callers that cannot allocate.
// Each GPU the library runs on holds its own copy of this array until the
// process ends.  Host code never uses the array's name as an address (on
// the host it is a stand-in, not device memory): it uses the address that
// hipGetSymbolAddress returns for the device, kept per device below.
static __device__ __align__(256) uint8_t scratch[FRN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, under the mutex

// The device address of `scratch` on the device that runs `stream`, looked
// up once per device with that device current.
frn_status scratch_address(void* stream, void** out) {
    int dev = -1;
    hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess)
        return fail(FRN_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(FRN_ERR_UNSUPPORTED, "device %d: the scratch table holds %d devices", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return fail(FRN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(FRN_ERR_HIP, "hipSetDevice(%d) failed: %s", dev, hipGetErrorString(e));
        void* ptr = nullptr;
        const hipError_t es = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess)
            return fail(FRN_ERR_HIP, "hipSetDevice(%d) failed: %s", cur, hipGetErrorString(e));
        if (es != hipSuccess || ptr == nullptr)
            return fail(FRN_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(es));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FRN_OK;
}

}  // namespace

FRN_API frn_status frn_moe_finalize_reduce_norm_noalloc(
    const void* const* expert_rows, const void* const* shared, int32_t R, const float* topk_w,
    const int32_t* topk_row, int32_t k, int64_t num_rows, int32_t epilogue,
    const void* residual_in, const float* gamma1, const float* gamma2, float eps, int64_t T,
    int64_t H, void* out, void* residual_out, void* stream) {
    g_last_error[0] = '\0';
    frn_status st = check_finalize_call(k, epilogue);
    if (st != FRN_OK) return st;
    if ((st = check_sizes(R, k, T, H, epilogue)) != FRN_OK || T == 0) return st;
    Call c{};
    if ((st = set_sources(c, expert_rows, shared, R, tp_routing(R, topk_w, topk_row, num_rows), k,
                          T, H)) != FRN_OK)
        return st;
    if ((st = set_epilogue(c, epilogue, residual_in, gamma1, gamma2, eps, T, H, out,
                           residual_out)) != FRN_OK)
        return st;
    if ((st = check_alias(c)) != FRN_OK) return st;
    c.a.ws_sum = nullptr;
    if (frn::use_split_rows(R, H, k, false, epilogue, T)) {
        const size_t need = frn::split_workspace_bytes(T, H);
        if (need > (size_t)FRN_NOALLOC_SCRATCH_BYTES)
            return fail(FRN_ERR_UNSUPPORTED,
                        "the split-row finalize needs %zu bytes of scratch at R=%d T=%lld "
                        "H=%lld; this entry point holds %zu (FRN_NOALLOC_SCRATCH_BYTES)",
                        need, R, (long long)T, (long long)H,
                        (size_t)FRN_NOALLOC_SCRATCH_BYTES);
        void* p = nullptr;
        if ((st = scratch_address(stream, &p)) != FRN_OK) return st;
        c.a.ws_sum = static_cast<float4*>(p);
        c.a.ws_ss = reinterpret_cast<double*>(static_cast<char*>(p) + frn::split_ss_offset(T, H));
    }
    return run(c, epilogue, T, stream);
}

FRN_API frn_status frn_reduce_bf16(const void* const* partials, int32_t R, int64_t T, int64_t H,
                                   void* sum_out, void* stream) {
    return pass1(partials, nullptr, R, Routing{}, 0, T, H, sum_out, stream);
}

FRN_API frn_status frn_moe_finalize_reduce_bf16(const void* const* expert_rows,
                                                const void* const* shared, int32_t R,
                                                const float* topk_w, const int32_t* topk_row,
                                                int32_t k, int64_t num_rows, int64_t T,
                                                int64_t H, void* sum_out, void* stream) {
    if (k < 1) {
        g_last_error[0] = '\0';
        return fail(FRN_ERR_INVALID, "k must be >= 1 for the finalize (got %d)", k);
    }
    return pass1(expert_rows, shared, R, tp_routing(R, topk_w, topk_row, num_rows), k, T, H,
                 sum_out, stream);
}

FRN_API frn_status frn_split_reduce_norm(const void* const* src, const void* const* shared,
                                         int32_t R, const float* topk_w,
                                         const int32_t* topk_row, int32_t k, int64_t num_rows,
                                         int32_t epilogue, const void* residual_in,
                                         const float* gamma1, const float* gamma2, float eps,
                                         int64_t T, int64_t H, void* scratch, void* out,
                                         void* residual_out, void* stream) {
    g_last_error[0] = '\0';
    if (epilogue != FRN_EPI_RMSNORM && epilogue != FRN_EPI_SANDWICH)
        return fail(FRN_ERR_INVALID, "unknown epilogue %d", epilogue);
    // Check both passes completely before launching either.
    frn_status st = check_sizes(R, k, T, H, epilogue);
    if (st != FRN_OK || T == 0) return st;
    Call c1{};
    if ((st = set_sources(c1, src, shared, R, tp_routing(R, topk_w, topk_row, num_rows), k, T,
                          H)) != FRN_OK)
        return st;
    if ((st = add_out(c1, "scratch", scratch, (size_t)T * H * 2)) != FRN_OK) return st;
    // the scratch tensor must not overlap the pass-2 operands either
    if ((st = set_epilogue(c1, epilogue, residual_in, gamma1, gamma2, eps, T, H, out,
                           residual_out)) != FRN_OK)
        return st;
    if ((st = check_alias(c1)) != FRN_OK) return st;
    c1.a.out = static_cast<uint4*>(scratch);
    Call c2{};
    const void* one[1] = {scratch};
    if ((st = set_sources(c2, one, nullptr, 1, Routing{}, 0, T, H)) != FRN_OK) return st;
    if ((st = set_epilogue(c2, epilogue, residual_in, gamma1, gamma2, eps, T, H, out,
                           residual_out)) != FRN_OK)
        return st;
    if ((st = run(c1, frn::kStoreSum, T, stream)) != FRN_OK) return st;
    return run(c2, epilogue, T, stream);
}

namespace {

// The per-rank finalize alone, materialized into R BF16 tensors.
frn_status finalize_only(const void* const* expert_rows, const void* const* shared, int32_t R,
                         const Routing& g, int32_t k, int64_t T, int64_t H,
                         void* const* partials_out, void* stream) {
    static const char* const kOutNames[FRN_MAX_R] = {
        "partials_out[0]", "partials_out[1]", "partials_out[2]", "partials_out[3]",
        "partials_out[4]", "partials_out[5]", "partials_out[6]", "partials_out[7]",
        "partials_out[8]", "partials_out[9]", "partials_out[10]", "partials_out[11]",
        "partials_out[12]", "partials_out[13]", "partials_out[14]", "partials_out[15]"};
    frn_status st;
    Call c{};
    if ((st = set_sources(c, expert_rows, shared, R, g, k, T, H)) != FRN_OK) return st;
    if (partials_out == nullptr) return fail(FRN_ERR_INVALID, "partials_out array is NULL");
    for (int r = 0; r < R; ++r) {
        if ((st = add_out(c, kOutNames[r], partials_out[r], (size_t)T * H * 2)) != FRN_OK)
            return st;
        c.a.part_out[r] = static_cast<uint4*>(partials_out[r]);
    }
    if ((st = check_alias(c)) != FRN_OK) return st;
    const hipError_t e = frn::launch_finalize(c.a, T, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FRN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return FRN_OK;
}

}  // namespace

FRN_API frn_status frn_moe_finalize(const void* const* expert_rows, const void* const* shared,
                                    int32_t R, const float* topk_w, const int32_t* topk_row,
                                    int32_t k, int64_t num_rows, int64_t T, int64_t H,
                                    void* const* partials_out, void* stream) {
    g_last_error[0] = '\0';
    if (k < 1) return fail(FRN_ERR_INVALID, "k must be >= 1 for the finalize (got %d)", k);
    frn_status st = check_sizes(R, k, T, H, frn::kStoreSum);
    if (st != FRN_OK || T == 0) return st;
    return finalize_only(expert_rows, shared, R, tp_routing(R, topk_w, topk_row, num_rows), k,
                         T, H, partials_out, stream);
}

FRN_API frn_status frn_ep_moe_finalize_reduce_norm(
    const void* const* expert_rows, const void* const* shared, int32_t R, const float* topk_w,
    const int32_t* const* topk_rows, int32_t k, const int64_t* num_rows, int32_t epilogue,
    const void* residual_in, const float* gamma1, const float* gamma2, float eps, int64_t T,
    int64_t H, void* out, void* residual_out, void* workspace, size_t workspace_bytes,
    void* stream) {
    g_last_error[0] = '\0';
    if (k < 1) return fail(FRN_ERR_INVALID, "k must be >= 1 for the finalize (got %d)", k);
    if (epilogue != FRN_EPI_RMSNORM && epilogue != FRN_EPI_SANDWICH)
        return fail(FRN_ERR_INVALID, "unknown epilogue %d", epilogue);
    frn_status st = check_sizes(R, k, T, H, epilogue);
    if (st != FRN_OK || T == 0) return st;
    Routing g;
    if ((st = ep_routing(g, R, topk_w, topk_rows, num_rows)) != FRN_OK) return st;
    return fused(expert_rows, shared, R, g, k, epilogue, residual_in, gamma1, gamma2, eps, T, H,
                 out, residual_out, workspace, workspace_bytes, stream);
}

FRN_API frn_status frn_ep_moe_finalize(const void* const* expert_rows,
                                       const void* const* shared, int32_t R,
                                       const float* topk_w, const int32_t* const* topk_rows,
                                       int32_t k, const int64_t* num_rows, int64_t T, int64_t H,
                                       void* const* partials_out, void* stream) {
    g_last_error[0] = '\0';
    if (k < 1) return fail(FRN_ERR_INVALID, "k must be >= 1 for the finalize (got %d)", k);
    frn_status st = check_sizes(R, k, T, H, frn::kStoreSum);
    if (st != FRN_OK || T == 0) return st;
    Routing g;
    if ((st = ep_routing(g, R, topk_w, topk_rows, num_rows)) != FRN_OK) return st;
    return finalize_only(expert_rows, shared, R, g, k, T, H, partials_out, stream);
}

FRN_API frn_status frn_set_launch_table(const char* text) {
    g_last_error[0] = '\0';
    const char* err = frn::set_launch_table(text);
    if (err != nullptr) return fail(FRN_ERR_INVALID, "%s", err);
    return FRN_OK;
}

FRN_API frn_status frn_launch_shape(int32_t R, int32_t k, int64_t T, int64_t H, int32_t epilogue,
                                    int32_t* threads, int32_t* vectors) {
    g_last_error[0] = '\0';
    const bool ep = (epilogue & FRN_SHAPE_EP) != 0;
    epilogue &= ~FRN_SHAPE_EP;
    if (ep && (k < 1 || epilogue == frn::kStoreSum))
        return fail(FRN_ERR_INVALID, "FRN_SHAPE_EP needs k >= 1 and a norm epilogue");
    frn_status st = check_sizes(R, k, T, H, epilogue);
    if (st != FRN_OK) return st;
    if (threads == nullptr || vectors == nullptr)
        return fail(FRN_ERR_INVALID, "threads and vectors must not be NULL");
    const int fin = k == 0 ? frn::kNoFinalize : (ep ? frn::kEpFinalize : frn::kTpFinalize);
    const frn::LaunchShape sh = frn::choose_shape((int)(H / 8), fin, T, epilogue, R, k);
    *threads = sh.threads;
    *vectors = sh.vec;
    return FRN_OK;
}

FRN_API frn_status frn_query(int32_t R, int32_t k, int64_t T, int64_t H, int32_t epilogue) {
    g_last_error[0] = '\0';
    return check_sizes(R, k, T, H, epilogue);
}

FRN_API size_t frn_workspace_bytes(int64_t max_T, int64_t H, int32_t R, int32_t k) {
    if (k < 1 || k > FRN_MAX_K || R < 1 || R > FRN_MAX_R || H < 8 || H > FRN_MAX_H ||
        H % 8 != 0 || max_T < 1)
        return 0;
    const int64_t cap = frn::split_rows_cap(R, H, k);
    const int64_t t = max_T < cap ? max_T : cap;
    return t < 1 ? 0 : frn::split_workspace_bytes(t, H);
}

FRN_API int32_t frn_split_rows(int32_t R, int32_t k, int64_t T, int64_t H, int32_t epilogue) {
    const bool ep = (epilogue & FRN_SHAPE_EP) != 0;
    epilogue &= ~FRN_SHAPE_EP;
    if (k < 1 || (epilogue != FRN_EPI_RMSNORM && epilogue != FRN_EPI_SANDWICH)) return 0;
    if (R < 1 || R > FRN_MAX_R || k > FRN_MAX_K || H < 8 || H > FRN_MAX_H || H % 8 != 0)
        return 0;
    return frn::use_split_rows(R, H, k, ep, epilogue, T) ? 1 : 0;
}

FRN_API int32_t frn_launch_pipelined(int32_t R, int32_t k, int64_t T, int64_t H,
                                     int32_t epilogue) {
    if (k != 0 || (epilogue != FRN_EPI_RMSNORM && epilogue != FRN_EPI_SANDWICH)) return 0;
    if (R < 1 || R > FRN_MAX_R || H < 8 || H > FRN_MAX_H || H % 8 != 0 || T < 1 ||
        T > FRN_MAX_T)
        return 0;
    return frn::choose_shape((int)(H / 8), frn::kNoFinalize, T, epilogue, R, 0).pipelined ? 1
                                                                                         : 0;
}

FRN_API const char* frn_status_string(frn_status s) {
    switch (s) {
        case FRN_OK: return "FRN_OK";
        case FRN_ERR_INVALID: return "FRN_ERR_INVALID: malformed arguments";
        case FRN_ERR_UNSUPPORTED: return "FRN_ERR_UNSUPPORTED: call declined";
        case FRN_ERR_HIP: return "FRN_ERR_HIP: HIP launch failed";
    }
    return "unknown frn_status";
}

FRN_API const char* frn_last_error(void) { return g_last_error; }

FRN_API const char* frn_version(void) { return FRN_VERSION_STRING; }
