// frn_kernels.hip -- gfx950 kernels of the fused reduce + norm boundary.
//
// Five kernels (row_kernel, rows_pipelined_kernel,
// finalize_sum_slices_kernel, norm_slices_kernel and finalize_slices_kernel,
// most in several instantiations) share the per-row building blocks below.
//
// row_kernel: one token row per workgroup.  Each lane owns V 16-byte vectors
// of the row (8 BF16 values each), placed `threads` vectors apart so every
// wave instruction touches 64 consecutive vectors (1 KiB) of a row.  A lane
// issues all loads of a chunk -- of ranks, of one rank's top-k slots, or
// (expert-parallel routing) of the token's live rows across ranks -- before
// it consumes any of them, keeps the FP32 row slice in registers through the
// epilogue, and writes each output exactly once; with two or four vectors
// per lane no load follows its first store (see epilogue).
//
// rows_pipelined_kernel: for calls without finalize at large T.  One
// workgroup per compute unit walks rows b, b + G, b + 2G, ...; the gamma
// rows sit in LDS for the workgroup's lifetime, and the next row's residual
// and partials are in flight while the current row runs its epilogue, so
// every CU keeps reading while it writes.
//
// finalize_sum_slices_kernel: for the MoE finalize at small T, where one
// workgroup per token would walk the R ranks one memory round trip after
// another.  Workgroup (t, c) takes a 64-vector slice of token t with one
// wave per rank: each wave finalizes its rank's slice, the R BF16 partials
// meet in LDS and are summed in rank order, and the FP32 sum goes to the
// caller's workspace.  norm_slices_kernel (residual + RMSNorm, from the
// slices' sums of squares) or row_kernel (sandwich) then reads it back and
// finishes the epilogue.  The kernel boundary orders the two, so no
// workgroup waits for another and no cross-XCD cache maintenance is issued
// inside a kernel (a device-scope fence per workgroup writes back and
// invalidates the whole L2 of its XCD, which measured far slower).
//
// finalize_slices_kernel: the standalone per-rank finalize.  Workgroup
// (t, r, c) finalizes slice c of rank r of token t and stores the BF16
// partial to rank r's output.
//
// Row-wide sums of squares are FP64: per lane, then within each wave (DPP
// swaps and four lane reads in a fixed order), then one LDS slot per wave
// summed in wave order, so every lane sees the same bits and the result does
// not depend on scheduling.
//
// Arithmetic (vLLM PR #62366 "Claims": FP32 reduction, FP32 epilogue,
// per-rank BF16 rounding of the finalize; "Details": no FMA contraction --
// this file is built with -ffp-contract=off):
//   finalize   acc = 0; acc = acc + w_j * e_j for j ascending; acc = acc + shared;
//              P_r = bf16(acc)  (expert-parallel routing: j over rank r's own
//              slots, shared only where rank r holds a shared-expert row)
//   reduce     s = P_0; s = s + P_r for r ascending
//   rinv(x)    ms = (float)(sum x^2 (FP64) / H); v = ms + eps; rinv = 1 / sqrt(v)
//   rmsnorm    h = s + x; y = (h * rinv(h)) * gamma
//   sandwich   a = (s * rinv(s)) * gamma1; h = a + x; y = (h * rinv(h)) * gamma2
// No MFMA: nothing here is a dense contraction; the kernels are bound by HBM.
#include <type_traits>

#include "frn_internal.h"

namespace frn {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streamed tensors (partials, expert rows, residual, outputs) are touched
// once: load and store them non-temporally so they do not displace the
// reused gamma rows from the caches.  Worth ~10% of HBM bandwidth on gfx950.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The same load from a pointer rebuilt from integers (the expert-parallel
// work list reads row addresses out of lanes): the compiler cannot tell that
// such a pointer is global, so say so, or it emits flat loads -- which also
// count against the scalar-load counter and so serialise with s_load waits.
typedef __attribute__((address_space(1))) const u32x4_t global_u32x4_t;

__device__ __forceinline__ uint4 ld_stream_global(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load((global_u32x4_t*)(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void st_stream(uint4* p, const uint4& q) {
    const u32x4_t v = {q.x, q.y, q.z, q.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// BF16 -> FP32 is exact: the BF16 bits are the high half of the FP32 bits.
__device__ __forceinline__ void widen(const uint4& q, float (&f)[8]) {
    f[0] = __uint_as_float(q.x << 16);
    f[1] = __uint_as_float(q.x & 0xffff0000u);
    f[2] = __uint_as_float(q.y << 16);
    f[3] = __uint_as_float(q.y & 0xffff0000u);
    f[4] = __uint_as_float(q.z << 16);
    f[5] = __uint_as_float(q.z & 0xffff0000u);
    f[6] = __uint_as_float(q.w << 16);
    f[7] = __uint_as_float(q.w & 0xffff0000u);
}

// FP32 -> BF16, round to nearest even (one v_cvt_pk_bf16_f32 per pair).
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint4 narrow(const float (&f)[8]) {
    uint4 q;
    q.x = pack2(f[0], f[1]);
    q.y = pack2(f[2], f[3]);
    q.z = pack2(f[4], f[5]);
    q.w = pack2(f[6], f[7]);
    return q;
}

__device__ __forceinline__ void load_gamma(const float4* g, int v, float (&out)[8]) {
    const float4 a = g[2 * v];
    const float4 b = g[2 * v + 1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// One DPP lane permutation applied to a double (two 32-bit DPP moves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), lane);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), lane);
    return __hiloint2double(hi, lo);
}

// Sum of one double per lane over the wave (wave_sum) or the workgroup
// (block_sum), the same bits in every lane.  Within a 16-lane row: DPP swaps
// (lane ^ 1, ^ 2, then the half-row and row mirrors), each step adding two
// equal partial sums in either order, so all 16 lanes hold identical bits;
// the four row sums are then read out and added in row order; the waves'
// sums meet in LDS and are added in wave order.  nw: waves in the workgroup.
__device__ __forceinline__ double wave_sum(double v) {
    v = v + dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
    v = v + dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
    v = v + dpp_f64<0x141>(v);  // row_half_mirror
    v = v + dpp_f64<0x140>(v);  // row_mirror
    return ((readlane_f64(v, 0) + readlane_f64(v, 16)) + readlane_f64(v, 32)) + readlane_f64(v, 48);
}

__device__ __forceinline__ double block_sum(double v, double* slots, int nw) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (lane == 0) slots[wave] = v;
    __syncthreads();
    double t = slots[0];
    for (int w = 1; w < nw; ++w) t += slots[w];
    return t;
}

// Inverse RMS from the FP64 sum of squares: eps inside the root, each FP32
// step correctly rounded (hipcc's default sqrt and divide are).
__device__ __forceinline__ float inv_rms(double ss, int H, float eps) {
    const float ms = (float)(ss / (double)H);
    const float v = ms + eps;
    const float d = sqrtf(v);
    return 1.0f / d;
}

// The vectors of a row that one lane owns: V of them, blockDim.x apart.
template <int V>
struct Lanes {
    int vi[V];
    bool ok[V];
    __device__ __forceinline__ explicit Lanes(int nvec) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            vi[j] = threadIdx.x + j * blockDim.x;
            ok[j] = vi[j] < nvec;
        }
    }
};

template <int V>
__device__ __forceinline__ double sum_squares(const float (&x)[V][8], const Lanes<V>& L) {
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        if (!L.ok[j]) continue;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double d = (double)x[j][i];
            ss = __fma_rn(d, d, ss);  // d*d is exact in FP64, so this is one rounding
        }
    }
    return ss;
}

template <int V>
__device__ __forceinline__ void load_residual(const RowArgs& a, int64_t row, const Lanes<V>& L,
                                              uint4 (&xr)[V]) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
        xr[j] = make_uint4(0, 0, 0, 0);
        if (L.ok[j]) xr[j] = ld_stream(a.residual + row + L.vi[j]);
    }
}

// s = P_0 + P_1 + ... + P_{R-1} (FP32, rank order) over the lane's vectors.
// rank_row(r) gives rank r's row as a vector pointer; ranks are loaded in
// chunks of C, every load of a chunk issued before any is consumed.
template <int V, int C, bool STREAM, typename RankRow>
__device__ __forceinline__ void reduce_ranks(RankRow rank_row, int R, const Lanes<V>& L,
                                             float (&s)[V][8]) {
    for (int r0 = 0; r0 < R; r0 += C) {
        uint4 q[C][V];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (r0 + c < R) {
                const uint4* p = rank_row(r0 + c);
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    q[c][j] = make_uint4(0, 0, 0, 0);
                    if (L.ok[j]) q[c][j] = STREAM ? ld_stream(p + L.vi[j]) : p[L.vi[j]];
                }
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (r0 + c < R) {
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    float f[8];
                    widen(q[c][j], f);
                    if (r0 + c == 0) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) s[j][i] = f[i];
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) s[j][i] = s[j][i] + f[i];
                    }
                }
            }
        }
    }
}

// Finalize of one rank for token t over the lane's vectors, before the BF16
// rounding: acc = sum_j w_j * E[row_j] (+ shared), j in order, top-k slots
// loaded in chunks of C.  A row index outside [0, num_rows) is never
// dereferenced; its slot reads as NaN -- except that with expert-parallel
// routing (a.ep) a negative index marks a slot of another rank's expert,
// which takes no part in this rank's sum.
template <int V, int C, bool EARLY_SHARED>
__device__ __forceinline__ void finalize_rank(const RowArgs& a, int r, int64_t t,
                                              const Lanes<V>& L, float (&acc)[V][8]) {
    const int k = a.k;
    const int32_t* rows_t = a.topk_row[r] + t * k;
    const int64_t num_rows = a.num_rows[r];
    const float* w_t = a.topk_w + t * k;
    const uint4 nan8 = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
    const uint4* E = a.src[r];
    const int nvec = a.nvec;
    // EARLY_SHARED: the shared row is loaded with the first chunk of slots
    // (it is added last, but waiting for it separately costs a memory round
    // trip); otherwise after the slots (four fewer VGPRs per vector).
    const uint4* S = a.shared[r];
    uint4 sh[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        sh[j] = make_uint4(0, 0, 0, 0);
        if (EARLY_SHARED && S != nullptr && L.ok[j]) sh[j] = ld_stream(S + t * nvec + L.vi[j]);
    }
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += C) {
        uint4 e[C][V];
        float w[C];
        bool use[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            w[c] = 0.0f;
            use[c] = false;
            if (j0 + c < k) {
                const int32_t er = rows_t[j0 + c];
                w[c] = w_t[j0 + c];
                use[c] = !(a.ep && er < 0);
                const bool in = er >= 0 && (int64_t)er < num_rows;
                const int64_t base = (int64_t)(in ? er : 0) * nvec;
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    e[c][j] = nan8;
                    if (in && L.ok[j]) e[c][j] = ld_stream(E + base + L.vi[j]);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (use[c]) {
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    float f[8];
                    widen(e[c][j], f);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float prod = w[c] * f[i];
                        acc[j][i] = acc[j][i] + prod;
                    }
                }
            }
        }
    }
    if (S != nullptr) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            if (!EARLY_SHARED && L.ok[j]) sh[j] = ld_stream(S + t * nvec + L.vi[j]);
            float f[8];
            widen(sh[j], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] = acc[j][i] + f[i];
        }
    }
}

// The finalize of every rank for token t, then the FP32 sum of the R
// rounded partials, as a work list that crosses rank boundaries.
//
// The token's rows are numbered as pairs p = r * (k + 1) + j: slot j < k of
// rank r, and j == k for rank r's shared-expert row.  A pair is live when
// its row enters the sum: a slot under TP routing always (an index out of
// range then reads as NaN), under expert-parallel routing when its index is
// >= 0; a shared row when rank r has one.  Each wave finds the live pairs of
// a 64-pair word with one ballot (every wave computes the same masks, so no
// LDS or barrier is needed), and the lane of pair p keeps its row index and
// weight for a readlane.  Live pairs are loaded C at a time in pair order,
// across rank boundaries, and consumed in the same order: rank r's
// accumulator takes its slots in j order and its shared row last, then is
// rounded to BF16 and added to s when the list moves past rank r.  This is
// the arithmetic of finalize_rank followed by the rank sum, with the loads
// of several ranks in flight at once.
struct PairWord {
    uint64_t live;      // uniform: bit l = pair 64 * word + l is live
    const uint4* row;   // lane l: start of its pair's row, or null (index out of range)
    float w;            // lane l: weight of its pair (slots)
    int32_t meta;       // lane l: its rank, plus kSharedPair for a shared-expert row
};

// A word of pairs whose indices and weights are still on their way.
struct PairLoad {
    int32_t row;   // lane l: its slot's row index (slots)
    float w;       // lane l: its slot's weight (slots)
    int32_t meta;  // lane l: rank, plus kSharedPair for a shared row; -1 past the last pair
};

constexpr int32_t kSharedPair = 256;

// A kernel argument read as a wave-uniform value.  The per-rank arrays of
// RowArgs are picked from per lane (pick below); reading each rank's entry
// uniformly keeps those reads scalar loads of the kernel arguments, where the
// compiler would otherwise fold the selection into a per-lane vector load --
// a memory round trip in front of every index load.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// arr[r] with r per lane (0 <= r < R); call in wave-uniform control flow.
// Entries are read kPickBatch at a time (one scalar load of the batch).
constexpr int kPickBatch = 4;
static_assert(FRN_MAX_R % kPickBatch == 0, "pick reads whole batches");

template <class P>
__device__ __forceinline__ P pick(const P (&arr)[FRN_MAX_R], int R, int r) {
    uint64_t out = 0;
    for (int r0 = 0; r0 < R; r0 += kPickBatch) {
#pragma unroll
        for (int q = 0; q < kPickBatch; ++q) {
            const uint64_t v = uniform_u64(__builtin_bit_cast(uint64_t, arr[r0 + q]));
            out = r == r0 + q ? v : out;
        }
    }
    return __builtin_bit_cast(P, out);
}

typedef __attribute__((address_space(1))) const int32_t global_i32_t;

// Issue the index and weight loads of one word of token t's pairs (see
// finalize_reduce); resolve_pairs turns them into a PairWord once they land.
__device__ __forceinline__ PairLoad load_pairs(const RowArgs& a, int64_t t, int word) {
    const int k = a.k;
    const int k1 = k + 1;
    const int p = word * 64 + (int)(threadIdx.x & 63);
    const int r = p / k1 < a.R ? p / k1 : a.R - 1;
    const int j = p - r * k1;
    const int32_t* rows = pick(a.topk_row, a.R, r);
    PairLoad pl;
    pl.row = 0;
    pl.w = 0.0f;
    pl.meta = -1;
    if (p < a.R * k1) {
        if (j < k) {
            pl.row = *((global_i32_t*)rows + t * k + j);
            pl.w = a.topk_w[t * k + j];
            pl.meta = r;
        } else {
            pl.meta = r | kSharedPair;
        }
    }
    return pl;
}

// Each lane resolves its pair's row address, so the loop that loads the rows
// only reads lanes.
__device__ __forceinline__ PairWord resolve_pairs(const RowArgs& a, int64_t t,
                                                  const PairLoad& pl) {
    const int r = pl.meta < 0 ? 0 : (pl.meta & (kSharedPair - 1));
    const uint4* src = pick(a.src, a.R, r);
    const uint4* shared = pick(a.shared, a.R, r);
    const int64_t num_rows = pick(a.num_rows, a.R, r);
    bool live = false;
    PairWord pw;
    pw.row = nullptr;
    pw.w = pl.w;
    pw.meta = pl.meta;
    if (pl.meta >= 0) {
        if ((pl.meta & kSharedPair) == 0) {
            live = !a.ep || pl.row >= 0;
            if (pl.row >= 0 && (int64_t)pl.row < num_rows) pw.row = src + (int64_t)pl.row * a.nvec;
        } else {
            live = shared != nullptr;
            if (live) pw.row = shared + t * a.nvec;
        }
    }
    pw.live = __ballot(live);
    return pw;
}

template <int V>
__device__ __forceinline__ void add_partial(int r, float (&acc)[V][8], float (&s)[V][8]) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
        float q[8];
        widen(narrow(acc[j]), q);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[j][i] = (r == 0) ? q[i] : s[j][i] + q[i];
            acc[j][i] = 0.0f;
        }
    }
}

// Up to C live pairs of one token, loaded and waiting to be consumed.
template <int C, int V>
struct Chunk {
    uint4 e[C][V];
    float w[C];
    int rank[C];
    bool slot[C], has[C];
};

// Issue the loads of the next (up to) C live pairs of word `pw`, taking them
// off the mask m in pair order.
template <int C, int V>
__device__ __forceinline__ void gather(const PairWord& pw, uint64_t& m, const Lanes<V>& L,
                                       Chunk<C, V>& ch) {
    const uint4 nan8 = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
#pragma unroll
    for (int c = 0; c < C; ++c) {
        ch.has[c] = m != 0;
        ch.slot[c] = false;
        ch.w[c] = 0.0f;
        ch.rank[c] = 0;
        if (ch.has[c]) {
            const int bit = __builtin_ctzll(m);
            m &= m - 1;
            const int meta = __builtin_amdgcn_readlane(pw.meta, bit);
            const uintptr_t addr = pw.row == nullptr ? 0 : (uintptr_t)pw.row;
            const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)addr, bit);
            const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(addr >> 32), bit);
            const uint4* E = (const uint4*)(((uint64_t)hi << 32) | lo);
            ch.rank[c] = meta & (kSharedPair - 1);
            ch.slot[c] = (meta & kSharedPair) == 0;
            ch.w[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw.w), bit));
#pragma unroll
            for (int j = 0; j < V; ++j) {
                ch.e[c][j] = nan8;
                if (E != nullptr && L.ok[j]) ch.e[c][j] = ld_stream_global(E + L.vi[j]);
            }
        }
    }
}

// Consume a chunk in pair order: close (round and add) every rank before the
// pair's rank, then add the pair into the open rank's accumulator.
template <int C, int V>
__device__ __forceinline__ void consume(const Chunk<C, V>& ch, int& cur, float (&acc)[V][8],
                                        float (&s)[V][8]) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (!ch.has[c]) continue;
        while (cur < ch.rank[c]) add_partial<V>(cur++, acc, s);
#pragma unroll
        for (int j = 0; j < V; ++j) {
            float f[8];
            widen(ch.e[c][j], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (ch.slot[c]) {
                    const float prod = ch.w[c] * f[i];
                    acc[j][i] = acc[j][i] + prod;
                } else {
                    acc[j][i] = acc[j][i] + f[i];
                }
            }
        }
    }
}

template <int V, int C>
__device__ __forceinline__ void finalize_reduce(const RowArgs& a, int64_t t, const Lanes<V>& L,
                                                float (&s)[V][8]) {
    const int words = (a.R * (a.k + 1) + 63) >> 6;
    float acc[V][8];
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;
    int cur = 0;  // rank whose accumulator is open
    // The indices and weights of the first two words go out together, and
    // each later word's one word ahead of its use: the first row loads wait
    // for one memory round trip, and loads complete in order, so a word's
    // indices have landed by the time the previous word's rows are consumed.
    PairLoad cur_load = load_pairs(a, t, 0);
    PairLoad next_load = load_pairs(a, t, 1);  // no lane loads if there is one word
    for (int word = 0; word < words; ++word) {
        const PairWord pw = resolve_pairs(a, t, cur_load);
        cur_load = next_load;
        if (word + 2 < words) next_load = load_pairs(a, t, word + 2);
        uint64_t m = pw.live;
        while (m != 0) {
            Chunk<C, V> ch;
            gather<C, V>(pw, m, L, ch);
            consume<C, V>(ch, cur, acc, s);
        }
    }
    while (cur < a.R) add_partial<V>(cur++, acc, s);
}

// Epilogue of one row: residual add and norm(s), stores of out and
// residual_out (or the pass-1 sum).  Every lane of the workgroup takes part
// (the row-wide sums synchronise the workgroup).
//
// A wave's vector memory operations complete in issue order (one counter
// covers loads and stores), so a load issued behind a store also waits for
// that store to be acknowledged.  With two or four vectors per lane, loading
// each vector's last gamma after the previous vector's stores would chain V
// such waits; there every gamma load goes out before the last row sum and
// residual_out and out are both stored after it.  Measured on MI355X (graph
// replay, inputs rotated over 1 GiB): sandwich H=5120 R=4 T=1024 14.7 ->
// 13.3 us, H=8192 R=8 T=64 7.4 -> 7.2 us, even elsewhere.  With one vector
// per lane (one such wait) storing residual_out ahead of the last row sum
// stays 2-4% faster at T <= 256.
template <int EPI, int V>
__device__ __forceinline__ void epilogue(const RowArgs& a, int64_t row, const Lanes<V>& L,
                                         float (&s)[V][8], const uint4 (&xr)[V],
                                         double (&slots)[2][16], const float4* gamma1,
                                         const float4* gamma2) {
    if constexpr (EPI == kStoreSum) {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (L.ok[j]) st_stream(a.out + row + L.vi[j], narrow(s[j]));
    } else {
        const float eps = a.eps;
        const int H = a.H;
        // h overwrites s in place
        const int nw = blockDim.x >> 6;
        if constexpr (EPI == kSandwich) {
            const float r1 = inv_rms(block_sum(sum_squares<V>(s, L), slots[0], nw), H, eps);
#pragma unroll
            for (int j = 0; j < V; ++j) {
                float g[8], x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) g[i] = 0.0f;
                if (L.ok[j]) load_gamma(gamma1, L.vi[j], g);
                widen(xr[j], x);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float n = s[j][i] * r1;
                    const float av = n * g[i];
                    s[j][i] = av + x[i];
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < V; ++j) {
                float x[8];
                widen(xr[j], x);
#pragma unroll
                for (int i = 0; i < 8; ++i) s[j][i] = s[j][i] + x[i];
            }
        }
        const float4* g2 = (EPI == kSandwich) ? gamma2 : gamma1;
        if constexpr (V == 1) {
            if (L.ok[0]) st_stream(a.residual_out + row + L.vi[0], narrow(s[0]));
            const float r2 = inv_rms(block_sum(sum_squares<V>(s, L), slots[1], nw), H, eps);
            if (!L.ok[0]) return;
            float g[8], y[8];
            load_gamma(g2, L.vi[0], g);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float n = s[0][i] * r2;
                y[i] = n * g[i];
            }
            st_stream(a.out + row + L.vi[0], narrow(y));
        } else {
            const double ss = sum_squares<V>(s, L);
            float g[V][8];
#pragma unroll
            for (int j = 0; j < V; ++j) {
#pragma unroll
                for (int i = 0; i < 8; ++i) g[j][i] = 0.0f;
                if (L.ok[j]) load_gamma(g2, L.vi[j], g[j]);
            }
            const float r2 = inv_rms(block_sum(ss, slots[1], nw), H, eps);
            // one wait for all of the gamma loads, ahead of the first store
            // (a wait inside the per-vector branches below would also cover
            // the stores issued before it)
#pragma unroll
            for (int j = 0; j < V; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(g[j][i]));
#pragma unroll
            for (int j = 0; j < V; ++j) {
                if (!L.ok[j]) continue;
                float y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float n = s[j][i] * r2;
                    y[i] = n * g[j][i];
                }
                st_stream(a.residual_out + row + L.vi[j], narrow(s[j]));
                st_stream(a.out + row + L.vi[j], narrow(y));
            }
        }
    }
}

// ------------------------------------------------------------ kernels --- //

// Finalize variants of the one-row kernel.
enum Fin { kNoFin = 0, kFinTp = 1, kFinEp = 2, kFinSum = 3 };

// One token row per workgroup.  EPI: epilogue; FIN: top-k finalize ahead of
// the reduction (kFinTp: every rank routes every slot, one rank after the
// other; kFinEp: expert-parallel routing, the work list across ranks;
// kFinSum: the rank sum already formed by finalize_sum_slices_kernel, read
// back as FP32); V: vectors per lane; C: ranks (no finalize), top-k slots
// (kFinTp) or live rows (kFinEp) loaded per chunk.
template <int EPI, int FIN, int V, int C>
__global__ __launch_bounds__(1024) void row_kernel(const RowArgs a) {
    __shared__ double slots[2][16];
    const int64_t t = blockIdx.x;
    const int64_t row = t * (int64_t)a.nvec;
    const Lanes<V> L(a.nvec);

    // The residual does not depend on the reduction: start its loads first.
    uint4 xr[V];
    if constexpr (EPI != kStoreSum) load_residual<V>(a, row, L, xr);

    float s[V][8];
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) s[j][i] = 0.0f;

    if constexpr (FIN == kNoFin) {
        reduce_ranks<V, C, true>([&](int r) { return a.src[r] + row; }, a.R, L, s);
    } else if constexpr (FIN == kFinSum) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            if (!L.ok[j]) continue;
            const float4* p = a.ws_sum + 2 * (row + L.vi[j]);
            const float4 lo = p[0];
            const float4 hi = p[1];
            s[j][0] = lo.x; s[j][1] = lo.y; s[j][2] = lo.z; s[j][3] = lo.w;
            s[j][4] = hi.x; s[j][5] = hi.y; s[j][6] = hi.z; s[j][7] = hi.w;
        }
    } else if constexpr (FIN == kFinEp) {
        // a rank owns few of the token's slots: keep several ranks' rows in flight
        finalize_reduce<V, C>(a, t, L, s);
    } else {
        for (int r = 0; r < a.R; ++r) {
            float acc[V][8];
            finalize_rank<V, C, true>(a, r, t, L, acc);
            // The rank's finalized partial is a BF16 tensor: round, then sum.
            add_partial<V>(r, acc, s);
        }
    }
    epilogue<EPI, V>(a, row, L, s, xr, slots, a.gamma1, a.gamma2);
}

// Per-rank MoE finalize of T rows, one row slice of one rank per workgroup:
// workgroup (t, r, c) writes bf16(finalize) of vectors [c * kSplitThreads,
// (c + 1) * kSplitThreads) of rank r, token t to row t of part_out[r].  C:
// top-k slots loaded per chunk (the launch takes C >= k, so all of a rank's
// rows go out in one memory round trip).
template <bool EARLY_SHARED, int C>
__global__ __launch_bounds__(kSplitThreads) void finalize_slices_kernel(const RowArgs a, int S,
                                                                        int64_t t0) {
    const int c = blockIdx.x % S;
    const int r = (blockIdx.x / S) % a.R;
    const int64_t t = t0 + blockIdx.x / (S * a.R);
    Lanes<1> L(a.nvec);
    L.vi[0] = c * kSplitThreads + threadIdx.x;
    L.ok[0] = L.vi[0] < a.nvec;
    float acc[1][8];
    finalize_rank<1, C, EARLY_SHARED>(a, r, t, L, acc);
    if (L.ok[0]) a.part_out[r][t * a.nvec + L.vi[0]] = narrow(acc[0]);
}

// Split-row finalize, first kernel: workgroup (t, c) takes vectors
// [64c, 64c + 64) of token t, one wave per rank.  Wave r finalizes rank r's
// slice (all of its top-k rows in one chunk of C >= k loads) and parks the
// BF16-rounded partial in LDS; after the barrier wave 0 adds the R partials
// in rank order -- bit for bit the sum the one-row kernel holds before its
// epilogue.  The R partials never reach HBM.
//  - Residual + RMSNorm: wave 0 also adds the residual (loaded before the
//    finalize), stores residual_out, the FP32 row h to the workspace and
//    its slice's sum of squares (per lane, then wave_sum: exactly the wave
//    term the one-row kernel with one vector per lane forms for these 64
//    vectors); norm_slices_kernel finishes the row.
//  - Sandwich: wave 0 stores the FP32 sum s; row_kernel<kSandwich, kFinSum>
//    runs the epilogue, one workgroup per token (its two row-wide sums need
//    the whole row).
template <int EPI, bool EARLY_SHARED, int C>
__global__ __launch_bounds__(64 * FRN_MAX_R) void finalize_sum_slices_kernel(const RowArgs a,
                                                                             int S) {
    __shared__ uint4 part[FRN_MAX_R][64];
    const int lane = threadIdx.x & 63;
    const int r = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = blockIdx.x % S;
    const int64_t t = blockIdx.x / S;
    Lanes<1> L(a.nvec);
    L.vi[0] = c * 64 + lane;
    L.ok[0] = L.vi[0] < a.nvec;
    const int64_t v = t * a.nvec + L.vi[0];
    uint4 xr = make_uint4(0, 0, 0, 0);
    if (EPI == kRmsNorm && r == 0 && L.ok[0]) xr = ld_stream(a.residual + v);
    float acc[1][8];
    finalize_rank<1, C, EARLY_SHARED>(a, r, t, L, acc);
    part[r][lane] = narrow(acc[0]);
    __syncthreads();
    if (r != 0) return;
    float h[8];
    widen(part[0][lane], h);
    for (int q = 1; q < a.R; ++q) {
        float f[8];
        widen(part[q][lane], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = h[i] + f[i];
    }
    if constexpr (EPI == kRmsNorm) {
        float x[8];
        widen(xr, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = h[i] + x[i];
        double ss = 0.0;
        if (L.ok[0]) {
            st_stream(a.residual_out + v, narrow(h));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double d = (double)h[i];
                ss = __fma_rn(d, d, ss);
            }
        }
        ss = wave_sum(ss);
        if (lane == 0) a.ws_ss[t * S + c] = ss;
    }
    if (!L.ok[0]) return;
    float4* out = a.ws_sum + 2 * v;
    out[0] = make_float4(h[0], h[1], h[2], h[3]);
    out[1] = make_float4(h[4], h[5], h[6], h[7]);
}

// Split-row finalize, second kernel (residual + RMSNorm): workgroup (t, c)
// adds token t's S slice sums of squares in slice order -- the one-row
// kernel's wave order -- and normalizes its 64 vectors of h.  Lane q < S
// loads slice q's sum, so all S arrive in one memory round trip, together
// with the lane's h and gamma.
__global__ __launch_bounds__(64) void norm_slices_kernel(const RowArgs a, int S) {
    const int lane = threadIdx.x;
    const int c = blockIdx.x % S;
    const int64_t t = blockIdx.x / S;
    const int vi = c * 64 + lane;
    const bool ok = vi < a.nvec;
    const int64_t v = t * a.nvec + vi;
    float4 lo = make_float4(0.0f, 0.0f, 0.0f, 0.0f), hi = lo;
    float g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = 0.0f;
    if (ok) {
        lo = a.ws_sum[2 * v];
        hi = a.ws_sum[2 * v + 1];
        load_gamma(a.gamma1, vi, g);
    }
    const double mine = lane < S ? a.ws_ss[t * S + lane] : 0.0;
    double ss = readlane_f64(mine, 0);
    for (int q = 1; q < S; ++q) ss += readlane_f64(mine, q);
    const float rinv = inv_rms(ss, a.H, a.eps);
    if (!ok) return;
    const float h[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float n = h[i] * rinv;
        y[i] = n * g[i];
    }
    st_stream(a.out + v, narrow(y));
}

// Calls f(std::integral_constant<int, C>) with the top-k chunk for k slots:
// the smallest of 4, 8, 12, 16 that holds all k.  A chunk's loads are
// registers whether or not a slot is used, so a chunk sized to k keeps the
// register count, and with it the workgroups resident per CU, as high as
// one round trip for all of a rank's rows allows.
template <class F>
__device__ __host__ auto with_topk_chunk(int k, F f) {
    if (k <= 4) return f(std::integral_constant<int, 4>{});
    if (k <= 8) return f(std::integral_constant<int, 8>{});
    if (k <= 12) return f(std::integral_constant<int, 12>{});
    return f(std::integral_constant<int, 16>{});
}

// Gamma rows staged in LDS (rows_pipelined_kernel): FP32 vectors in the
// LDS address space, so the reads are ds_read and never wait on the vector
// memory counter that the in-flight row loads hold.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// A gamma row in LDS is two planes of nvec FP32 vectors: plane 0 holds the
// first four values of each 8-value vector, plane 1 the last four, so the
// lanes of a wave read 16-byte words at a 16-byte stride (no bank
// conflicts; one interleaved row would put them 32 bytes apart).
__device__ __forceinline__ void load_gamma(const lds_f32x4_t* g, int nvec, int v,
                                           float (&out)[8]) {
    const f32x4_t a = g[v];
    const f32x4_t b = g[nvec + v];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// The residual and the R partial rows of one token: the residual loads go
// out first (the compiler barrier keeps them ahead of the partials, so a
// wait for the partials covers them too).
template <int V, int R>
__device__ __forceinline__ void issue_row(const RowArgs& a, int64_t row, const Lanes<V>& L,
                                          uint4 (&xr)[V], uint4 (&q)[R][V]) {
    load_residual<V>(a, row, L, xr);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < V; ++j) q[r][j] = ld_stream(a.src[r] + row + L.vi[j]);
}

// s = P_0 + P_1 + ... + P_{R-1} (FP32, rank order), consuming each rank's
// loads as they land.
template <int V, int R>
__device__ __forceinline__ void sum_ranks(const uint4 (&q)[R][V], float (&s)[V][8]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < V; ++j) {
            float f[8];
            widen(q[r][j], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) s[j][i] = (r == 0) ? f[i] : s[j][i] + f[i];
        }
}

// The epilogue of `epilogue` with the gamma rows read from LDS.  Same
// arithmetic, in the same order.  Slot arrays: the sandwich's two row sums
// take slots[0] and slots[1]; residual + RMSNorm's one row sum takes
// slots[P], so that the caller can alternate them from row to row.
template <int EPI, int V, int P>
__device__ __forceinline__ void epilogue_lds(const RowArgs& a, int64_t row, const Lanes<V>& L,
                                             float (&s)[V][8], const uint4 (&xr)[V],
                                             double (&slots)[2][16], const lds_f32x4_t* gamma1,
                                             const lds_f32x4_t* gamma2) {
    const float eps = a.eps;
    const int H = a.H;
    // waves per workgroup, from the kernel arguments (a scalar load): the
    // launch sizes the workgroup to the row, blockDim.x * V == nvec
    const int nw = a.nvec / (64 * V);
    if constexpr (EPI == kSandwich) {
        const float r1 = inv_rms(block_sum(sum_squares<V>(s, L), slots[0], nw), H, eps);
#pragma unroll
        for (int j = 0; j < V; ++j) {
            float g[8], x[8];
            load_gamma(gamma1, a.nvec, L.vi[j], g);
            widen(xr[j], x);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float n = s[j][i] * r1;
                const float av = n * g[i];
                s[j][i] = av + x[i];
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            float x[8];
            widen(xr[j], x);
#pragma unroll
            for (int i = 0; i < 8; ++i) s[j][i] = s[j][i] + x[i];
        }
    }
#pragma unroll
    for (int j = 0; j < V; ++j) st_stream(a.residual_out + row + L.vi[j], narrow(s[j]));
    const float r2 =
        inv_rms(block_sum(sum_squares<V>(s, L), slots[EPI == kSandwich ? 1 : P], nw), H, eps);
    const lds_f32x4_t* g2 = (EPI == kSandwich) ? gamma2 : gamma1;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        float g[8], y[8];
        load_gamma(g2, a.nvec, L.vi[j], g);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float n = s[j][i] * r2;
            y[i] = n * g[i];
        }
        st_stream(a.out + row + L.vi[j], narrow(y));
    }
}

// Row-pipelined boundary kernel: workgroup b takes rows b, b + G, b + 2G,
// ... (G = gridDim.x, one workgroup per CU).  The gamma rows are copied to
// LDS once, straight from global memory (global_load_lds, no registers),
// and the next row's loads are issued before the current row's epilogue.
// The launch guarantees blockDim.x * V == nvec (no tail lanes, so no lane
// predicate hides a load or store from the compiler's wait counting), R
// ranks exactly, and gridDim.x <= T.  Dynamic LDS: 16 * 2 * nvec bytes per
// gamma row.
template <int EPI, int V, int R>
__global__ __launch_bounds__(V == 1 ? 1024 : 512) void rows_pipelined_kernel(const RowArgs a) {
    extern __shared__ f32x4_t gamma_lds_raw[];
    __shared__ double slots[2][16];
    lds_f32x4_t* gamma_lds = (lds_f32x4_t*)gamma_lds_raw;
    const int nvec = a.nvec;
    const int n4 = 2 * nvec;  // FP32 vectors per gamma row (two planes of nvec, a multiple of 64)
    Lanes<V> L(nvec);
#pragma unroll
    for (int j = 0; j < V; ++j) L.ok[j] = true;  // no tail lanes (see above)
    {
        // lane l of an instruction copies word (base + l) of one plane: the
        // global FP32 vector 2 (base + l) (plane 0) or 2 (base + l) + 1 (plane 1)
        const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
        for (int base = w * 64; base < nvec; base += nw * 64) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                __builtin_amdgcn_global_load_lds(
                    (const void*)(a.gamma1 + 2 * (base + lane) + half),
                    (lds_void_t*)(gamma_lds + half * nvec + base), 16, 0, 0);
                if constexpr (EPI == kSandwich)
                    __builtin_amdgcn_global_load_lds(
                        (const void*)(a.gamma2 + 2 * (base + lane) + half),
                        (lds_void_t*)(gamma_lds + n4 + half * nvec + base), 16, 0, 0);
            }
        }
    }
    int64_t t = blockIdx.x;
    uint4 xr[V];
    uint4 q[R][V];
    issue_row<V, R>(a, t * nvec, L, xr, q);
    float s[V][8];
    sum_ranks<V, R>(q, s);
    // Make the first row's residual land here too: otherwise the loop's
    // epilogue would carry a wait for it into every later row.
#pragma unroll
    for (int j = 0; j < V; ++j)
        asm volatile("" ::"v"(xr[j].x), "v"(xr[j].y), "v"(xr[j].z), "v"(xr[j].w));
    __syncthreads();  // the gamma rows are in LDS (the compiler waits for the copies here)
    // One row: the next row's loads go out, then this row's epilogue runs;
    // false once this was the workgroup's last row.
    auto step = [&](auto parity) -> bool {
        const int64_t tn = t + gridDim.x;
        const bool more = tn < a.T;
        uint4 xn[V];
        if (more) issue_row<V, R>(a, tn * nvec, L, xn, q);
        epilogue_lds<EPI, V, decltype(parity)::value>(a, t * nvec, L, s, xr, slots, gamma_lds,
                                                      gamma_lds + n4);
        if (!more) return false;
        sum_ranks<V, R>(q, s);
        for (int j = 0; j < V; ++j) xr[j] = xn[j];
        t = tn;
        return true;
    };
    // A row sum's slot array is written by one lane per wave before a
    // barrier and read by every lane after it, with no second barrier: the
    // next write to the same array must come after a later barrier, which no
    // wave passes before every wave has read it.  The sandwich's two sums per
    // row alternate the two arrays; residual + RMSNorm has one sum per row, so
    // consecutive rows alternate them (two rows per iteration).
    if constexpr (EPI == kSandwich) {
        while (step(std::integral_constant<int, 0>{})) {
        }
    } else {
        while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
        }
    }
}

template <int EPI, int V, int R>
hipError_t launch_pipelined(const RowArgs& a, int threads, int64_t groups, hipStream_t stream) {
    const size_t lds = (size_t)(EPI == kSandwich ? 2 : 1) * 2 * a.nvec * 16;
    hipLaunchKernelGGL((rows_pipelined_kernel<EPI, V, R>), dim3((unsigned)groups),
                       dim3(threads), lds, stream, a);
    return hipGetLastError();
}

template <int EPI, int V>
hipError_t launch_pipelined_r(const RowArgs& a, int threads, int64_t groups,
                              hipStream_t stream) {
    switch (a.R) {
        case 1: return launch_pipelined<EPI, V, 1>(a, threads, groups, stream);
        case 2: return launch_pipelined<EPI, V, 2>(a, threads, groups, stream);
        case 3: return launch_pipelined<EPI, V, 3>(a, threads, groups, stream);
        case 4: return launch_pipelined<EPI, V, 4>(a, threads, groups, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int EPI>
hipError_t launch_pipelined_v(const RowArgs& a, int64_t T, LaunchShape sh, hipStream_t stream) {
    const int64_t cus = compute_units();
    const int64_t groups = T < cus ? T : cus;
    if (sh.vec == 1) return launch_pipelined_r<EPI, 1>(a, sh.threads, groups, stream);
    return launch_pipelined_r<EPI, 2>(a, sh.threads, groups, stream);
}

template <int EPI, int FIN, int V, int C>
hipError_t launch(const RowArgs& a, int64_t T, int threads, hipStream_t stream) {
    hipLaunchKernelGGL((row_kernel<EPI, FIN, V, C>), dim3((unsigned)T), dim3(threads), 0,
                       stream, a);
    return hipGetLastError();
}

// Ranks (or top-k slots, or live rows) per load chunk: at most 64 VGPRs of
// loads in flight per lane (32 for a two-vector finalize, which holds more
// live state and would otherwise spill or lose occupancy).  The
// expert-parallel work list takes five live rows a chunk: 62 VGPRs, eight
// waves per SIMD, where eight rows take 74 and six waves -- one workgroup
// fewer per CU at 512 and 896 lanes.  Measured on MI355X against eight
// (graph replay, R=8 H=6144 k=10 of 256 experts): 2-5% faster at T=64 to
// 256, 1-2% at T=1024 to 16384; 8% faster at R=4 H=4096 k=8 T=1024 and 6%
// at R=16 H=7168 k=8 T=1024; at most 1% slower over k=2 to 16 at
// H=6144 R=8.
template <int EPI, int FIN, int V>
hipError_t launch_c(const RowArgs& a, int64_t T, int threads, hipStream_t stream) {
    constexpr int CMAX = 16 / V;
    if constexpr (FIN == kFinTp) {
        // Split pass 1 keeps the 16-slot chunk: sized to k (more tokens per
        // CU) it measured 4% slower (H=7168 R=2 k=8 T=4096), the fused
        // calls 0-2% faster.
        if constexpr (V == 1 && EPI != kStoreSum) {
            return with_topk_chunk(a.k, [&](auto c) {
                return launch<EPI, FIN, V, decltype(c)::value>(a, T, threads, stream);
            });
        } else {
            return launch<EPI, FIN, V, (V == 1 ? 16 : 4)>(a, T, threads, stream);
        }
    } else if constexpr (FIN == kFinEp) {
        return launch<EPI, FIN, V, (V == 1 ? 5 : 4)>(a, T, threads, stream);
    } else {
        if (a.R <= 2) return launch<EPI, FIN, V, 2>(a, T, threads, stream);
        if (a.R <= 4) return launch<EPI, FIN, V, 4>(a, T, threads, stream);
        if (a.R <= 8 || CMAX == 8) return launch<EPI, FIN, V, 8>(a, T, threads, stream);
        return launch<EPI, FIN, V, CMAX>(a, T, threads, stream);
    }
}

template <int EPI, int FIN>
hipError_t launch_v(const RowArgs& a, int64_t T, LaunchShape sh, hipStream_t stream) {
    if (sh.vec == 1) return launch_c<EPI, FIN, 1>(a, T, sh.threads, stream);
    if constexpr (FIN == kNoFin && EPI != kStoreSum) {
        if (sh.vec == 4) return launch<EPI, FIN, 4, 4>(a, T, sh.threads, stream);
    }
    return launch_c<EPI, FIN, 2>(a, T, sh.threads, stream);
}

template <int EPI>
hipError_t launch_fin(const RowArgs& a, int64_t T, LaunchShape sh, hipStream_t stream) {
    if (a.k == 0) return launch_v<EPI, kNoFin>(a, T, sh, stream);
    if (a.ep) return launch_v<EPI, kFinEp>(a, T, sh, stream);
    return launch_v<EPI, kFinTp>(a, T, sh, stream);
}

// Split-row finalize: finalize_sum_slices_kernel (a workgroup per token and
// 64-vector slice, a wave per rank), then the epilogue: norm_slices_kernel
// (residual + RMSNorm, a workgroup per token and slice) or row_kernel<EPI,
// kFinSum> (sandwich, one workgroup per token; one vector per lane up to
// 1024 lanes, two above).  The caller keeps T at or below kSplitCapT, so
// the grids stay far below their limit.
template <int EPI>
hipError_t launch_split_rows(const RowArgs& a, int64_t T, hipStream_t stream) {
    if (T > kSplitCapT) return hipErrorInvalidValue;
    const int S = split_row_slices(a.nvec);
    const dim3 grid((unsigned)(T * S));
    const dim3 block((unsigned)(64 * a.R));
    // Under expert-parallel routing most ranks hold no shared row, and the
    // registers of an early shared load would cost occupancy for nothing.
    with_topk_chunk(a.k, [&](auto c) {
        constexpr int C = decltype(c)::value;
        if (a.ep)
            hipLaunchKernelGGL((finalize_sum_slices_kernel<EPI, false, C>), grid, block, 0,
                               stream, a, S);
        else
            hipLaunchKernelGGL((finalize_sum_slices_kernel<EPI, true, C>), grid, block, 0,
                               stream, a, S);
        return 0;
    });
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (EPI == kRmsNorm) {
        hipLaunchKernelGGL(norm_slices_kernel, grid, dim3(64), 0, stream, a, S);
        return hipGetLastError();
    } else {
        const int vec = a.nvec > 1024 ? 2 : 1;
        const int threads = ((a.nvec + vec - 1) / vec + 63) / 64 * 64;
        if (vec == 1) return launch<EPI, kFinSum, 1, 1>(a, T, threads, stream);
        return launch<EPI, kFinSum, 2, 1>(a, T, threads, stream);
    }
}

}  // namespace

int split_slices(int nvec) { return (nvec + kSplitThreads - 1) / kSplitThreads; }

hipError_t launch_finalize(const RowArgs& a, int64_t T, hipStream_t stream) {
    const int S = split_slices(a.nvec);
    // A dispatch holds fewer than 2^32 lanes: launch large T in token ranges.
    const int64_t per_token = (int64_t)a.R * S;
    const int64_t max_groups = 0xffffffffLL / kSplitThreads;
    const int64_t chunk = max_groups / per_token;
    for (int64_t t0 = 0; t0 < T; t0 += chunk) {
        const int64_t n = (T - t0 < chunk ? T - t0 : chunk) * per_token;
        // Under expert-parallel routing most ranks hold no shared row, and the
        // registers of an early shared load would cost occupancy for nothing.
        with_topk_chunk(a.k, [&](auto c) {
            constexpr int C = decltype(c)::value;
            if (a.ep)
                hipLaunchKernelGGL((finalize_slices_kernel<false, C>), dim3((unsigned)n),
                                   dim3(kSplitThreads), 0, stream, a, S, t0);
            else
                hipLaunchKernelGGL((finalize_slices_kernel<true, C>), dim3((unsigned)n),
                                   dim3(kSplitThreads), 0, stream, a, S, t0);
            return 0;
        });
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_rows(const RowArgs& a, int epilogue, int64_t T, hipStream_t stream) {
    if (a.k > 0 && a.ws_sum != nullptr) {
        switch (epilogue) {
            case kRmsNorm: return launch_split_rows<kRmsNorm>(a, T, stream);
            case kSandwich: return launch_split_rows<kSandwich>(a, T, stream);
            default: return hipErrorInvalidValue;
        }
    }
    const int fin = a.k == 0 ? kNoFinalize : (a.ep ? kEpFinalize : kTpFinalize);
    const LaunchShape sh = choose_shape(a.nvec, fin, T, epilogue, a.R, a.k);
    if (sh.pipelined) {
        if (epilogue == kSandwich) return launch_pipelined_v<kSandwich>(a, T, sh, stream);
        return launch_pipelined_v<kRmsNorm>(a, T, sh, stream);
    }
    switch (epilogue) {
        case kRmsNorm: return launch_fin<kRmsNorm>(a, T, sh, stream);
        case kSandwich: return launch_fin<kSandwich>(a, T, sh, stream);
        case kStoreSum: return launch_fin<kStoreSum>(a, T, sh, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace frn
