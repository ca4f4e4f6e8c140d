// frn_internal.h -- what the host entry points and the gfx950 kernels share:
// the kernel argument block and the launch functions.  Not installed; the
// public interface is include/fused_reduce_norm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fused_reduce_norm.h"

namespace frn {

// Which epilogue a kernel runs after the FP32 reduction.
enum Epilogue : int {
    kRmsNorm = FRN_EPI_RMSNORM,    // h = s + x; y = norm(h) * g1
    kSandwich = FRN_EPI_SANDWICH,  // a = norm(s) * g1; h = a + x; y = norm(h) * g2
    kStoreSum = 2,                 // split pass 1: sum_out = bf16(s)
};

// Everything one launch needs, passed by value as the kernel argument.
// All tensors are addressed in 16-byte vectors of 8 BF16 values (or 4 FP32
// values for gamma); nvec = H / 8 vectors per row.
struct RowArgs {
    const uint4* src[FRN_MAX_R];     // partials [T,H], or expert rows [num_rows,H]
    const uint4* shared[FRN_MAX_R];  // shared-expert rows [T,H] per rank (finalize), or null
    const float* topk_w;             // [T,k]
    const int32_t* topk_row[FRN_MAX_R];  // [T,k] per rank (the same array for every rank
                                         // unless routing is expert-parallel)
    const uint4* residual;           // [T,H]
    const float4* gamma1;            // [H]
    const float4* gamma2;            // [H]
    uint4* out;                      // [T,H] normed output, or the pass-1 sum
    uint4* residual_out;             // [T,H]
    int64_t num_rows[FRN_MAX_R];     // rows in each rank's expert buffer
    int64_t T;                       // token rows of the call
    float4* ws_sum;                  // split-row finalize: [T,H] FP32 rank sums (residual +
                                     // RMSNorm: the row h), or null
    double* ws_ss;                   // split-row finalize: [T,S] slice sums of squares
    uint4* part_out[FRN_MAX_R];      // finalize_slices_kernel: [T,H] BF16 output per rank
    int32_t R;                       // ranks
    int32_t k;                       // top-k slots (0: no finalize)
    int32_t nvec;                    // H / 8
    int32_t H;
    float eps;
    int32_t ep;                      // expert-parallel routing: a negative row index
                                     // marks a slot of another rank's expert
};

// Standalone finalize: workgroup size (one slice of one rank's row).
constexpr int kSplitThreads = 256;

// Split-row finalize (small T): the largest T any call may take it at, the
// 64-vector column slices of a row, and its workspace: the T x H FP32 sums
// of the R finalized partials, then T x S FP64 slice sums of squares (no
// other state: the workspace needs no initialisation and keeps nothing
// between calls).
constexpr int64_t kSplitCapT = 256;

inline int split_row_slices(int nvec) { return (nvec + 63) / 64; }

// Workspace bytes the split-row finalize needs for T rows, and where its
// sums of squares start.
inline size_t split_ss_offset(int64_t T, int64_t H) { return (size_t)T * (size_t)H * 4; }
inline size_t split_workspace_bytes(int64_t T, int64_t H) {
    return split_ss_offset(T, H) + (size_t)T * (size_t)split_row_slices((int)(H / 8)) * 8;
}

// Whether a finalize call (k >= 1) that is given a large enough workspace
// takes the split-row finalize: the first matching split/fused rule of the
// tuned table, else the built-in rule.  ep: expert-parallel routing.
// Thread-safe.
bool use_split_rows(int32_t R, int64_t H, int32_t k, bool ep, int epilogue, int64_t T);

// The largest T at which use_split_rows can hold for these sizes, under
// either routing and any epilogue (at most kSplitCapT): what a workspace
// must cover.  Thread-safe.
int64_t split_rows_cap(int32_t R, int64_t H, int32_t k);

// Column slices of one row in the standalone finalize.
int split_slices(int nvec);

// Launch shape of one call: `threads` lanes per row, each lane owning `vec`
// 16-byte vectors of the row.  pipelined = false: row_kernel, one token row
// per workgroup; true: rows_pipelined_kernel, one workgroup per compute
// unit walking rows (threads * vec == H / 8 exactly).
struct LaunchShape {
    int threads;
    int vec;
    bool pipelined;
};

// Compute units of the current device (queried once per device).
int64_t compute_units();

// Finalize kind of a call: none, TP routing, or expert-parallel routing.
enum FinKind { kNoFinalize = 0, kTpFinalize = 1, kEpFinalize = 2 };

// Launch shape of row_kernel for a call: the first matching rule of the
// tuned table (frn_set_launch_table / FRN_LAUNCH_TABLE) that fits the call,
// else the built-in rule.  fin: a FinKind.  Thread-safe.
LaunchShape choose_shape(int nvec, int fin, int64_t T, int epilogue, int R, int k);

// Replace the tuned table (text as documented at frn_set_launch_table; NULL
// clears it).  Returns nullptr on success, else a message naming the line.
const char* set_launch_table(const char* text);

// Enqueue the boundary kernel for T rows.  Returns the HIP launch status.
hipError_t launch_rows(const RowArgs& a, int epilogue, int64_t T, hipStream_t stream);

// Enqueue the per-rank finalize alone: a.part_out[r][t] = bf16(finalize of
// rank r, token t) for all R ranks and T tokens.
hipError_t launch_finalize(const RowArgs& a, int64_t T, hipStream_t stream);

}  // namespace frn
