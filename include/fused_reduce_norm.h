/*
 * fused_reduce_norm.h -- C ABI of the fused reduce + norm boundary for one
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the layer boundary of a tensor-parallel transformer: R
 * BF16 partial-sum tensors [T,H] (one per TP rank) are summed in FP32 and
 * followed by residual add + RMSNorm, or by the FP32 norm -> residual add ->
 * norm "sandwich" (vLLM PR #62366, "Overview" and "Claims"; SGLang PR
 * #34134, first commit message, first fusion pattern).  An optional MoE
 * top-k finalize -- the weighted sum of each token's k expert output rows
 * plus a shared-expert row, rounded to BF16 on each rank -- runs ahead of
 * the reduction (vLLM PR #62366 "Claims"; SGLang PR #34134, second fusion
 * pattern).  For large batches a two-pass path first reduces to a BF16
 * tensor and then runs the boundary on it (vLLM PR #62366 "Claims").  All
 * FP32 arithmetic is uncontracted: no multiply-add is fused into an FMA
 * (vLLM PR #62366 "Details").
 *
 * Here the R rank shares are R buffers resident in the one GPU's HBM.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - BF16 tensors are passed as raw device pointers to row-major [rows, H]
 *   arrays of 16-bit bfloat16 values, row stride H elements.  FP32 vectors
 *   (gamma) and top-k weights are float; top-k rows are int32.
 * - Pointer arrays (partials, expert_rows, shared) are HOST arrays of R
 *   device pointers; the library copies them into the kernel arguments, so
 *   the host array may be freed as soon as the call returns.
 * - Every device pointer must be 16-byte aligned and H must be a multiple
 *   of 8 (one 128-bit vector holds 8 BF16 values); otherwise the call
 *   returns FRN_ERR_UNSUPPORTED.  1 <= R <= FRN_MAX_R, 1 <= k <= FRN_MAX_K,
 *   8 <= H <= FRN_MAX_H, 0 <= T <= FRN_MAX_T.
 * - stream is a hipStream_t passed as void*; NULL is the null stream.  Calls
 *   are asynchronous: they enqueue kernels and return.  They never
 *   synchronize, never read device memory from the host and never allocate,
 *   so they may be captured into a HIP graph.
 * - The caller owns every buffer.  The library keeps no per-call state.
 * - Aliasing: residual_out may be the same pointer as residual_in (the
 *   residual stream updated in place).  Any other overlap between an
 *   output and any input or other output is FRN_ERR_INVALID.
 * - Errors are return codes; nothing is thrown across the ABI.  All
 *   arguments are checked before anything is launched, so on any error the
 *   outputs are untouched.  T == 0 returns FRN_OK once the sizes are
 *   valid, without looking at the pointers and without a launch.
 *   FRN_ERR_HIP means the launch itself failed; frn_last_error() has text.
 * - Numerics: per element, the finalize accumulates j = 0..k-1 in order
 *   (each product and sum one FP32 rounding), adds the shared row last and
 *   rounds to BF16 (nearest-even); the reduction adds ranks r = 0..R-1 in
 *   order in FP32; the inverse RMS uses an FP64 sum of the squares, divides
 *   by H, rounds to FP32, adds eps in FP32 and takes a correctly rounded
 *   square root and reciprocal; the normalized value is (x * rinv) * gamma.
 *   Outputs are rounded to BF16, nearest-even.
 */
#ifndef FUSED_REDUCE_NORM_H
#define FUSED_REDUCE_NORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FRN_VERSION_STRING "0.1.0"

#define FRN_MAX_R 16     /* partials (TP ranks) per call */
#define FRN_MAX_K 16     /* top-k slots per token */
#define FRN_MAX_H 16384  /* hidden size */
#define FRN_MAX_T 4194303 /* token rows per call (a row's workgroup has up to
                             1024 lanes, and a dispatch holds < 2^32 lanes) */
#define FRN_NOALLOC_SCRATCH_BYTES (17u << 20) /* scratch per GPU of
                             frn_moe_finalize_reduce_norm_noalloc (17 MiB) */

typedef enum frn_status {
    FRN_OK = 0,
    FRN_ERR_INVALID = 1,     /* malformed arguments (null pointer, R < 1, ...) */
    FRN_ERR_UNSUPPORTED = 2, /* well-formed, but outside what the library serves */
    FRN_ERR_HIP = 3          /* the HIP launch failed */
} frn_status;

typedef enum frn_epilogue {
    FRN_EPI_RMSNORM = 0,  /* residual add + RMSNorm(gamma1) */
    FRN_EPI_SANDWICH = 1  /* RMSNorm(gamma1) -> residual add -> RMSNorm(gamma2) */
} frn_epilogue;

/*
 * Reduce + residual add + RMSNorm (vLLM PR #62366, kernel microbenchmark
 * table; SGLang PR #34134, first fusion pattern).  Per token row t:
 *   s = sum_r partials[r][t]          (FP32, r ascending)
 *   h = s + residual_in[t]            (FP32)
 *   residual_out[t] = bf16(h)
 *   out[t] = bf16((h * rinv(h)) * gamma)
 * partials: R device pointers to [T,H] BF16.  residual_in/out, out: [T,H]
 * BF16.  gamma: [H] FP32.  eps >= 0, finite.  workspace/workspace_bytes:
 * optional scratch, NULL/0 allowed (see frn_workspace_bytes; unused
 * without the finalize).
 */
frn_status frn_reduce_residual_rmsnorm(const void* const* partials, int32_t R,
                                       const void* residual_in, const float* gamma,
                                       float eps, int64_t T, int64_t H, void* out,
                                       void* residual_out, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Reduce + Beam's FP32 sandwich norm (vLLM PR #62366, "Overview", "Claims").
 * Per token row t:
 *   s = sum_r partials[r][t]           (FP32)
 *   a = (s * rinv(s)) * gamma1         (FP32, never rounded to BF16)
 *   h = a + residual_in[t]             (FP32)
 *   residual_out[t] = bf16(h)
 *   out[t] = bf16((h * rinv(h)) * gamma2)
 * Arguments as for frn_reduce_residual_rmsnorm; gamma1, gamma2: [H] FP32.
 */
frn_status frn_reduce_sandwich_norm(const void* const* partials, int32_t R,
                                    const void* residual_in, const float* gamma1,
                                    const float* gamma2, float eps, int64_t T, int64_t H,
                                    void* out, void* residual_out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * MoE top-k finalize (+ shared expert) folded ahead of the reduction, then
 * the chosen epilogue (vLLM PR #62366 "Claims": the finalize is deferred
 * into the fused all-reduce and keeps its per-rank BF16 rounding; SGLang PR
 * #34134, second fusion pattern: finalize + shared-expert add + all-reduce
 * + residual + RMSNorm).  Per rank r, token t, element i:
 *   acc = 0; for j = 0..k-1: acc = acc + topk_w[t,j] * E_r[topk_row[t,j], i]
 *   if shared: acc = acc + S_r[t, i]
 *   P_r[t, i] = bf16(acc)
 * then the epilogue runs on s = sum_r P_r exactly as in the calls above.
 * expert_rows: R device pointers to [num_rows,H] BF16 (each rank's expert
 * outputs, one row per (token, slot) in any order).  shared: NULL, or R
 * device pointers to [T,H] BF16.  topk_w: [T,k] FP32; topk_row: [T,k]
 * int32, the row of E_r holding token t's j-th expert output; routing is
 * the same on every rank.  A row index outside [0, num_rows) is never
 * dereferenced: that slot reads as NaN, so the token's whole output row
 * becomes NaN (visible, and no memory fault).  epilogue: FRN_EPI_RMSNORM
 * (gamma1 used, gamma2 ignored and may be NULL) or FRN_EPI_SANDWICH.
 */
frn_status frn_moe_finalize_reduce_norm(const void* const* expert_rows,
                                        const void* const* shared, int32_t R,
                                        const float* topk_w, const int32_t* topk_row,
                                        int32_t k, int64_t num_rows, int32_t epilogue,
                                        const void* residual_in, const float* gamma1,
                                        const float* gamma2, float eps, int64_t T,
                                        int64_t H, void* out, void* residual_out,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * frn_moe_finalize_reduce_norm for callers that cannot allocate device
 * memory or hand in a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, results
 * and checks as frn_moe_finalize_reduce_norm, without workspace and
 * workspace_bytes: where that call would take the split-row finalize (see
 * frn_split_rows), this one puts that call's workspace (see
 * frn_workspace_bytes) in a scratch array that the library holds in device
 * memory, FRN_NOALLOC_SCRATCH_BYTES per GPU, kept until the process ends;
 * elsewhere it runs the one-row kernel and uses no scratch.  It calls no
 * allocation routine.  The array covers the largest call any launch table
 * can route to the split-row finalize (T = 256 at H = 16384: 16 MiB of FP32
 * rows and 64 KiB of sums); a larger need would return FRN_ERR_UNSUPPORTED
 * without launching, with both sizes in frn_last_error().  The scratch needs no initialisation and its contents
 * from the previous call are never read.  Every call on one GPU shares that GPU's
 * array: calls that may overlap in time on one GPU (different streams,
 * concurrent graph replays) race and give wrong results; serialise them.
 * The first call on each GPU looks up the array's device address
 * (hipGetSymbolAddress, with that GPU current); make it once before any
 * graph capture.  The kernels run on the device of `stream`.
 */
frn_status frn_moe_finalize_reduce_norm_noalloc(const void* const* expert_rows,
                                                const void* const* shared, int32_t R,
                                                const float* topk_w, const int32_t* topk_row,
                                                int32_t k, int64_t num_rows, int32_t epilogue,
                                                const void* residual_in, const float* gamma1,
                                                const float* gamma2, float eps, int64_t T,
                                                int64_t H, void* out, void* residual_out,
                                                void* stream);

/*
 * Split path, pass 1 (vLLM PR #62366 "Claims": for large batches the
 * all-reduce alone produces a BF16 tensor): sum_out[t] = bf16(sum_r
 * partials[r][t]).  sum_out: [T,H] BF16.  Pass 2 is
 * frn_reduce_residual_rmsnorm / frn_reduce_sandwich_norm with R = 1 and
 * partials = {sum_out}.
 */
frn_status frn_reduce_bf16(const void* const* partials, int32_t R, int64_t T, int64_t H,
                           void* sum_out, void* stream);

/* Split path, pass 1 with the finalize folded in: sum_out[t] =
 * bf16(sum_r P_r[t]), P_r as in frn_moe_finalize_reduce_norm. */
frn_status frn_moe_finalize_reduce_bf16(const void* const* expert_rows,
                                        const void* const* shared, int32_t R,
                                        const float* topk_w, const int32_t* topk_row,
                                        int32_t k, int64_t num_rows, int64_t T, int64_t H,
                                        void* sum_out, void* stream);

/*
 * Both passes of the split path on one stream (vLLM PR #62366 "Claims":
 * two-shot reduction to BF16, then the boundary kernel).  k == 0: src holds
 * R partials [T,H] and shared/topk_w/topk_row are ignored; k > 0: src holds
 * R expert-row buffers [num_rows,H] as in frn_moe_finalize_reduce_norm.
 * scratch: caller-owned [T,H] BF16 device buffer for the pass-1 tensor; it
 * must not overlap any other argument.
 */
frn_status frn_split_reduce_norm(const void* const* src, const void* const* shared,
                                 int32_t R, const float* topk_w, const int32_t* topk_row,
                                 int32_t k, int64_t num_rows, int32_t epilogue,
                                 const void* residual_in, const float* gamma1,
                                 const float* gamma2, float eps, int64_t T, int64_t H,
                                 void* scratch, void* out, void* residual_out, void* stream);

/*
 * The MoE top-k finalize alone, materialized per rank: for r = 0..R-1,
 * partials_out[r][t] = P_r[t] with P_r exactly as in
 * frn_moe_finalize_reduce_norm (j ascending, shared expert last, BF16
 * rounding).  This is the standalone finalize kernel the fused path
 * replaces (SGLang PR #34134, first commit message: a separate finalize
 * kernel, and the rule that a deferred finalize reaching a non-fusing path
 * is materialized in place): a caller whose reduction runs elsewhere
 * finalizes with this and reduces the R tensors itself.  Reducing the R
 * outputs with frn_reduce_residual_rmsnorm / frn_reduce_sandwich_norm gives
 * bit for bit the fused call's results.  partials_out: HOST array of R
 * device pointers to [T,H] BF16 buffers, which must not overlap each other
 * or any input.  Other arguments as in frn_moe_finalize_reduce_norm.
 */
frn_status frn_moe_finalize(const void* const* expert_rows, const void* const* shared,
                            int32_t R, const float* topk_w, const int32_t* topk_row, int32_t k,
                            int64_t num_rows, int64_t T, int64_t H, void* const* partials_out,
                            void* stream);

/*
 * Expert-parallel variant of frn_moe_finalize_reduce_norm: the
 * replicated-token deferral for TP = 1, EP > 1 that vLLM PR #62366 names in
 * "Overview" and "Details" (built on the same fused boundary).  Every rank
 * holds all T tokens and the same top-k weights, but expert outputs only
 * for its own experts, so each rank has its own row-index array:
 *   topk_rows[r][t,j] >= 0   the row of E_r holding token t's j-th expert
 *                            output (that expert lives on rank r);
 *   topk_rows[r][t,j] <  0   slot j's expert lives on another rank: the
 *                            slot takes no part in rank r's sum (skipped,
 *                            not added as zero).
 * Per rank r, token t, element i:
 *   acc = 0; for j = 0..k-1 with topk_rows[r][t,j] >= 0:
 *       acc = acc + topk_w[t,j] * E_r[topk_rows[r][t,j], i]
 *   if shared[r]: acc = acc + S_r[t, i]
 *   P_r[t, i] = bf16(acc)
 * then the reduction and epilogue exactly as in the calls above.
 * expert_rows: R device pointers, E_r = [num_rows[r], H] BF16; an entry may
 * be NULL when num_rows[r] == 0.  num_rows: HOST array of R counts (>= 0).
 * topk_rows: HOST array of R device pointers to [T,k] int32 (4-byte
 * aligned).  shared: NULL, or a HOST array of R entries, each NULL (that
 * rank holds no shared-expert row) or a device pointer to [T,H] BF16.
 * topk_w: [T,k] FP32, the same for every rank.  An index at or past
 * num_rows[r] is never dereferenced: that slot reads as NaN and the token's
 * output row becomes NaN.  Workspace, epilogue, aliasing and errors as in
 * frn_moe_finalize_reduce_norm.  With one rank owning every slot this is
 * frn_moe_finalize_reduce_norm bit for bit.
 */
frn_status frn_ep_moe_finalize_reduce_norm(const void* const* expert_rows,
                                           const void* const* shared, int32_t R,
                                           const float* topk_w,
                                           const int32_t* const* topk_rows, int32_t k,
                                           const int64_t* num_rows, int32_t epilogue,
                                           const void* residual_in, const float* gamma1,
                                           const float* gamma2, float eps, int64_t T,
                                           int64_t H, void* out, void* residual_out,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream);

/*
 * The expert-parallel finalize alone, materialized per rank:
 * partials_out[r][t] = P_r[t] with P_r as in
 * frn_ep_moe_finalize_reduce_norm.  The deferred finalize reaching a
 * non-fusing path is materialized this way (SGLang PR #34134, first commit
 * message); reducing the R outputs with frn_reduce_residual_rmsnorm /
 * frn_reduce_sandwich_norm gives the fused call's results bit for bit.
 * partials_out as in frn_moe_finalize; other arguments as in
 * frn_ep_moe_finalize_reduce_norm.
 */
frn_status frn_ep_moe_finalize(const void* const* expert_rows, const void* const* shared,
                               int32_t R, const float* topk_w,
                               const int32_t* const* topk_rows, int32_t k,
                               const int64_t* num_rows, int64_t T, int64_t H,
                               void* const* partials_out, void* stream);

/*
 * Capability check without launching anything: FRN_OK if a call with these
 * sizes is served, FRN_ERR_UNSUPPORTED if it would be declined, and
 * FRN_ERR_INVALID for malformed sizes (the analogue of a workspace factory
 * that returns nothing for unsupported shapes, vLLM PR #62366 "Details").
 * k == 0 means no finalize.  Setting the environment variable
 * FRN_FORCE_DECLINE=1 before the first call makes every entry point return
 * FRN_ERR_UNSUPPORTED (for testing callers' fallback paths).
 */
frn_status frn_query(int32_t R, int32_t k, int64_t T, int64_t H, int32_t epilogue);

/*
 * Tuned launch shapes.  A call launches either one workgroup per token row
 * (the one-row kernel) or, without finalize, one workgroup per compute
 * unit that walks the rows with the next row's loads in flight (the
 * row-pipelined kernel, see frn_launch_pipelined); the lanes own 1, 2 or 4
 * vectors of 8 BF16 values ("vec").  The best choice depends on H, R, k,
 * the epilogue and T, and shapes tuned for one hidden size do not carry
 * over to another (SGLang PR #34134: the shipped H=8192 profiles misfit
 * H=6144).  Three layers of rules decide, the first with a rule for the
 * call winning: the caller's table (this call, or FRN_LAUNCH_TABLE); the
 * table measured on MI355X for the shapes of the pages' workloads and for
 * residual + RMSNorm at common hidden sizes and TP degrees, which the
 * library carries compiled in; and a hand-fitted rule, also measured on
 * MI355X, for every other shape.  Table text: one rule per line, '#'
 * starts a comment:
 *     H  R  k  epilogue  Tmin  Tmax  vec
 * H, R, k, Tmin, Tmax: integers or '*' (any); k = 0 means no finalize;
 * epilogue: rmsnorm | sandwich | sum (split pass 1) for calls without
 * expert-parallel routing, ep-rmsnorm | ep-sandwich | ep-* for
 * frn_ep_moe_finalize_reduce_norm, or * (every call); vec: 1 | 2 | 4,
 * p1 | p2, split | fused, or builtin.  A numeric vec sets the one-row kernel's
 * shape, p1 / p2 the row-pipelined kernel with 1 / 2 vectors per lane: the
 * first such rule that matches a call and fits it decides (one-row kernel:
 * at most 1024 lanes, vec 4 only without finalize and outside split pass 1;
 * row-pipelined kernel: see frn_launch_pipelined).  split / fused
 * decide, for a finalize call (k >= 1) given a large enough workspace,
 * whether it takes the split-row finalize (see frn_workspace_bytes) or the
 * one-row kernel: the first such rule that matches decides, and T above 256
 * is never split.  builtin: the calls the rule matches take the
 * hand-fitted rule for both questions, whatever later rules and the
 * compiled-in table say ("* * * * 0 * builtin" alone turns the measured
 * table off).  Only speed changes: the one FP64 sum of squares per row is
 * added in an order that depends on the shape, and FP64 holds each FP32
 * square exactly, so the FP32 mean it rounds to has not changed in any of
 * the parity sweeps.  tp_reduction_rmsnorm_amd/tune.py measures a table.
 * frn_set_launch_table(NULL) removes the caller's table (the compiled-in
 * table and the hand-fitted rule then decide); an unparsable text returns
 * FRN_ERR_INVALID (the line is in frn_last_error) and leaves the table as
 * it was.  If no table was set
 * before the first launch, the file named by the environment variable
 * FRN_LAUNCH_TABLE (if any) is loaded.  Thread-safe; affects later launches
 * only.
 */
frn_status frn_set_launch_table(const char* text);

/* The shape (lanes per workgroup, vectors per lane) a call of these sizes
 * gets, without launching: that of the row-pipelined kernel where the call
 * takes it (frn_launch_pipelined), else that of the one-row kernel.  epilogue: FRN_EPI_RMSNORM,
 * FRN_EPI_SANDWICH or 2 (split pass 1), OR'ed with FRN_SHAPE_EP for a call
 * of frn_ep_moe_finalize_reduce_norm (k >= 1).  threads, vectors: host
 * pointers to receive the values. */
#define FRN_SHAPE_EP 16
frn_status frn_launch_shape(int32_t R, int32_t k, int64_t T, int64_t H, int32_t epilogue,
                            int32_t* threads, int32_t* vectors);

/*
 * Bytes of the optional workspace argument of the fused calls for calls of
 * up to max_T tokens (0: no call of these sizes uses one).  Only the MoE
 * finalize (k > 0) uses it, at small T: each (token, 512-column slice) then
 * runs in a workgroup of its own with one wave per rank, the R finalized
 * BF16 partials are summed in LDS, and the FP32 sum goes to the workspace
 * (residual + RMSNorm: the residual is added there too, residual_out
 * written, and the slice's FP64 sum of squares kept); a second kernel on the
 * same stream reads it back and runs the rest of the epilogue, per slice
 * (residual + RMSNorm) or per token (sandwich).  This spreads a token's row
 * over many workgroups at small batch, the analogue of the pages' row
 * spread over several blocks (SGLang PR #34134, the publish-granularity
 * discussion).  Which calls take it is frn_split_rows; the size returned
 * covers both routings and every epilogue under the current launch table.
 * Results are the same as without it: the same BF16 partials summed in the
 * same order, the FP32 sums stored exactly, and the slice sums of squares
 * added in slice order, which is the one-row kernel's order when it runs
 * one vector per lane (other shapes add the same FP64 terms in another
 * order, as launch shapes do; see frn_set_launch_table).  Layout: T x H
 * FP32 rows, then T x ceil(H / 512) FP64 sums.  The caller allocates it
 * (256-byte aligned); it needs no initialisation and holds nothing between
 * calls.  Calls that share one workspace must not run concurrently.  A
 * workspace that is NULL, or given to a call that does not take the
 * split-row finalize, is ignored (the call then uses the
 * one-row-per-workgroup kernel).  A workspace given to a call that takes it
 * must cover that call (frn_workspace_bytes(T, ...)) and be 256-byte
 * aligned, else the call returns FRN_ERR_UNSUPPORTED without launching; it
 * must not overlap any other argument (FRN_ERR_INVALID).
 */
size_t frn_workspace_bytes(int64_t max_T, int64_t H, int32_t R, int32_t k);

/*
 * 1 if a finalize call of these sizes that is given a large enough
 * workspace takes the split-row finalize, else 0 (also for k = 0 and for
 * sizes outside what the library serves).  epilogue: FRN_EPI_RMSNORM or
 * FRN_EPI_SANDWICH, OR'ed with FRN_SHAPE_EP for a call of
 * frn_ep_moe_finalize_reduce_norm.  The split-row finalize writes and
 * re-reads one FP32 row per token and adds a second launch, so it pays only
 * while the one-row kernel is bound by its memory round trips.  The
 * compiled-in measured table decides the shapes it covers; the hand-fitted
 * rule, measured on MI355X, takes it up to 32 to 256 tokens depending on R,
 * H, k and the routing (never at R = 1 under TP routing); a caller's split /
 * fused rules override both (see frn_set_launch_table).
 */
int32_t frn_split_rows(int32_t R, int32_t k, int64_t T, int64_t H, int32_t epilogue);

/*
 * 1 if a call of these sizes without finalize (k = 0; epilogue
 * FRN_EPI_RMSNORM or FRN_EPI_SANDWICH) runs the row-pipelined kernel, else
 * 0 (also for k > 0, split pass 1 and sizes outside what the library
 * serves).  That kernel launches one workgroup per compute unit; each walks
 * the rows b, b + G, b + 2G, ... with the gamma rows held in LDS and the
 * next row's residual and partials in flight during the current row's
 * epilogue, so a CU keeps reading while it writes (with one row per
 * workgroup, the reads of all resident rows come first and the writes
 * after).  It serves 1 <= R <= 4, H/8 a multiple of 64 * vec (at most 1024
 * lanes with one vector per lane, 512 with two) and gamma rows of at most
 * 64 KiB.  The compiled-in measured table decides the shapes it covers;
 * the hand-fitted rule, measured on MI355X,
 * takes it with two vectors per lane from T = 1536 for 4096 < H < 8192,
 * for the sandwich epilogue (at R >= 3 and H >= 6144 up to T = 4096) and
 * for residual + RMSNorm at R = 1, and with
 * one vector per lane for 1536 <= T <= 4096 and 4096 <= H <= 8192 for
 * residual + RMSNorm at R = 2 (where it measured faster or even); a
 * caller's p1 / p2 and numeric vec rules
 * override both.  Results are bit-identical either way: the same
 * arithmetic in the same order, row by row.
 */
int32_t frn_launch_pipelined(int32_t R, int32_t k, int64_t T, int64_t H, int32_t epilogue);

/* Static text for a status code. */
const char* frn_status_string(frn_status s);

/* Text describing the last error returned on the calling thread ("" if
 * none).  Valid until the next call on that thread. */
const char* frn_last_error(void);

/* Library version, FRN_VERSION_STRING. */
const char* frn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FUSED_REDUCE_NORM_H */
