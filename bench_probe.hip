// bench_probe.hip -- the boundary's memory access pattern alone, for bench.py.
//
// Per token row, one workgroup reads `nsrc` rows of H BF16 values with
// non-temporal 16-byte loads and writes `ndst` rows with non-temporal
// stores: the row-major layout and the lane mapping of the library's
// one-row kernel (lane l owns vectors l, l + threads, ...), with no
// arithmetic beyond an XOR that keeps every load live and no row-wide sums.
// Its rate is what this GPU delivers to the access pattern itself, the
// reference the fused kernel's rate is read against.  Measurement
// infrastructure only; not part of the library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMaxSrc = 17;
constexpr int kMaxDst = 2;

struct ProbeArgs {
    const uint4* src[kMaxSrc];
    uint4* dst[kMaxDst];
    int nsrc, ndst, nvec;
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void st_nt(uint4* p, const uint4& q) {
    const u32x4_t v = {q.x, q.y, q.z, q.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

template <int V>
__global__ __launch_bounds__(1024) void probe_rows_kernel(const ProbeArgs a) {
    const int64_t row = (int64_t)blockIdx.x * a.nvec;
    int vi[V];
    bool ok[V];
    uint4 acc[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        vi[j] = threadIdx.x + j * blockDim.x;
        ok[j] = vi[j] < a.nvec;
        acc[j] = make_uint4(0, 0, 0, 0);
    }
    // every load of a chunk issued before any is consumed, as in the kernel
    // (5 rows -- partials and residual of the headline call -- in one chunk)
    constexpr int CH = V == 4 ? 5 : 8;
    for (int r0 = 0; r0 < a.nsrc; r0 += CH) {
        uint4 q[CH][V];
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int j = 0; j < V; ++j) {
                q[c][j] = make_uint4(0, 0, 0, 0);
                if (r0 + c < a.nsrc && ok[j]) q[c][j] = ld_nt(a.src[r0 + c] + row + vi[j]);
            }
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int j = 0; j < V; ++j) {
                acc[j].x ^= q[c][j].x;
                acc[j].y ^= q[c][j].y;
                acc[j].z ^= q[c][j].z;
                acc[j].w ^= q[c][j].w;
            }
    }
    for (int d = 0; d < a.ndst; ++d)
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (ok[j]) st_nt(a.dst[d] + row + vi[j], acc[j]);
}

}  // namespace

// src: nsrc device pointers to [T,H] BF16; dst: ndst device pointers to
// [T,H] BF16; vec: vectors per lane (1, 2 or 4).  Returns 0 on success, 1 on
// bad arguments, 2 if the launch failed.
extern "C" __attribute__((visibility("default"))) int probe_rows(
    const void* const* src, int nsrc, void* const* dst, int ndst, int64_t T, int64_t H, int vec,
    void* stream) {
    if (nsrc < 1 || nsrc > kMaxSrc || ndst < 0 || ndst > kMaxDst || T < 1 || H < 8 ||
        H % 8 != 0 || H > 16384 || T > 4194303 || !(vec == 1 || vec == 2 || vec == 4))
        return 1;
    ProbeArgs a{};
    for (int r = 0; r < nsrc; ++r) {
        if (src[r] == nullptr) return 1;
        a.src[r] = static_cast<const uint4*>(src[r]);
    }
    for (int d = 0; d < ndst; ++d) {
        if (dst[d] == nullptr) return 1;
        a.dst[d] = static_cast<uint4*>(dst[d]);
    }
    a.nsrc = nsrc;
    a.ndst = ndst;
    a.nvec = (int)(H / 8);
    const int lanes = (a.nvec + vec - 1) / vec;
    const int threads = ((lanes + 63) / 64) * 64;
    if (threads > 1024) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (vec == 1)
        hipLaunchKernelGGL(probe_rows_kernel<1>, dim3((unsigned)T), dim3(threads), 0, s, a);
    else if (vec == 2)
        hipLaunchKernelGGL(probe_rows_kernel<2>, dim3((unsigned)T), dim3(threads), 0, s, a);
    else
        hipLaunchKernelGGL(probe_rows_kernel<4>, dim3((unsigned)T), dim3(threads), 0, s, a);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
