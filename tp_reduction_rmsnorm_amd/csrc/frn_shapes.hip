// frn_shapes.hip -- launch shapes of row_kernel and the choice between the
// split-row and the one-row finalize.  Three layers of rules, the first
// that has a rule for a call deciding it: a caller's table
// (frn_set_launch_table, FRN_LAUNCH_TABLE), the table measured on MI355X
// that is compiled in (frn_tuned_mi355x.inc), and the hand-fitted rules
// below for every shape the measured table does not cover.  Launch profiles
// tuned for one hidden size do not carry over to another (SGLang PR #34134:
// shipped profiles for H=8192 misfit H=6144), so a deployment can measure
// its own shapes (tp_reduction_rmsnorm_amd/tune.py) and load them.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "frn_internal.h"

namespace frn {
namespace {

// One tuned rule; -1 in H, R, k, epilogue, ep means "any".  T in [tmin,
// tmax].  ep: 1 for calls with expert-parallel routing, 0 for the others.
// vec 1, 2 or 4: vectors per lane of row_kernel, or with pipe set, of
// rows_pipelined_kernel (1 or 2); kSplitRule / kFusedRule: a finalize call
// given a workspace takes the split-row / the one-row finalize;
// kBuiltinRule: the calls it matches take the hand-fitted rules for both
// questions, whatever the later rules and the compiled-in table say.
struct Rule {
    int64_t H, R, k, epilogue, ep;
    int64_t tmin, tmax;
    int vec;
    bool pipe;
};

constexpr int kSplitRule = -1;
constexpr int kFusedRule = -2;
constexpr int kBuiltinRule = -3;

std::mutex g_mu;
std::vector<Rule> g_rules;   // the caller's table
std::vector<Rule> g_tuned;   // the compiled-in measured table
bool g_env_checked = false;
bool g_tuned_parsed = false;
std::string g_parse_error;

const char kTunedTable[] =
#include "frn_tuned_mi355x.inc"
    ;

bool parse_field(const char* tok, int64_t* out) {
    if (strcmp(tok, "*") == 0) {
        *out = -1;
        return true;
    }
    char* end = nullptr;
    const long long v = strtoll(tok, &end, 10);
    if (end == tok || *end != '\0' || v < 0) return false;
    *out = v;
    return true;
}

// "rmsnorm" | "sandwich" | "sum" match calls without expert-parallel
// routing; "ep-rmsnorm" | "ep-sandwich" | "ep-*" match the expert-parallel
// finalize; "*" matches every call.
bool parse_epilogue(const char* tok, int64_t* out, int64_t* ep) {
    if (strcmp(tok, "*") == 0) {
        *out = -1;
        *ep = -1;
        return true;
    }
    *ep = 0;
    if (strncmp(tok, "ep-", 3) == 0) {
        *ep = 1;
        tok += 3;
        if (strcmp(tok, "*") == 0) {
            *out = -1;
            return true;
        }
    }
    if (strcmp(tok, "rmsnorm") == 0) *out = kRmsNorm;
    else if (strcmp(tok, "sandwich") == 0) *out = kSandwich;
    else if (strcmp(tok, "sum") == 0 && *ep == 0) *out = kStoreSum;
    else return false;
    return true;
}

// Parse the whole text into `out`; on error return false with a message.
bool parse(const char* text, std::vector<Rule>& out, std::string& err) {
    out.clear();
    int lineno = 0;
    const char* p = text;
    while (*p) {
        const char* eol = strchr(p, '\n');
        std::string line = eol ? std::string(p, eol - p) : std::string(p);
        p = eol ? eol + 1 : p + line.size();
        ++lineno;
        const size_t hash = line.find('#');
        if (hash != std::string::npos) line.resize(hash);
        std::vector<std::string> tok;
        size_t i = 0;
        while (i < line.size()) {
            while (i < line.size() && (line[i] == ' ' || line[i] == '\t' || line[i] == '\r')) ++i;
            size_t j = i;
            while (j < line.size() && line[j] != ' ' && line[j] != '\t' && line[j] != '\r') ++j;
            if (j > i) tok.push_back(line.substr(i, j - i));
            i = j;
        }
        if (tok.empty()) continue;
        Rule r{};
        int64_t vec = 0;
        const bool last_ok =
            tok.size() == 7 &&
            (tok[6] == "split"     ? (vec = kSplitRule, true)
             : tok[6] == "fused"   ? (vec = kFusedRule, true)
             : tok[6] == "builtin" ? (vec = kBuiltinRule, true)
             : tok[6] == "p1"    ? (vec = 1, r.pipe = true, true)
             : tok[6] == "p2"    ? (vec = 2, r.pipe = true, true)
                                 : parse_field(tok[6].c_str(), &vec) &&
                                       (vec == 1 || vec == 2 || vec == 4));
        if (!last_ok || !parse_field(tok[0].c_str(), &r.H) ||
            !parse_field(tok[1].c_str(), &r.R) || !parse_field(tok[2].c_str(), &r.k) ||
            !parse_epilogue(tok[3].c_str(), &r.epilogue, &r.ep) ||
            !parse_field(tok[4].c_str(), &r.tmin) || !parse_field(tok[5].c_str(), &r.tmax)) {
            err = "launch table line " + std::to_string(lineno) +
                  ": expected 'H R k epilogue Tmin Tmax vec' (numbers or *, epilogue "
                  "rmsnorm|sandwich|sum|ep-rmsnorm|ep-sandwich|ep-*|*, vec "
                  "1|2|4|p1|p2|split|fused|builtin)";
            return false;
        }
        if (r.tmin < 0) r.tmin = 0;
        if (r.tmax < 0) r.tmax = INT64_MAX;
        r.vec = (int)vec;
        out.push_back(r);
    }
    return true;
}

// FRN_LAUNCH_TABLE names a table file read at the first launch, unless a
// table was set through the API first.  A file that does not parse is
// ignored, with one line on stderr.
void load_env_table_locked() {
    if (g_env_checked) return;
    g_env_checked = true;
    const char* path = getenv("FRN_LAUNCH_TABLE");
    if (path == nullptr || path[0] == '\0') return;
    FILE* f = fopen(path, "rb");
    if (f == nullptr) {
        fprintf(stderr,
                "fused_reduce_norm: cannot open FRN_LAUNCH_TABLE=%s; using built-in shapes\n",
                path);
        return;
    }
    std::string text;
    char buf[4096];
    size_t n;
    while ((n = fread(buf, 1, sizeof buf, f)) > 0) text.append(buf, n);
    fclose(f);
    std::vector<Rule> rules;
    std::string err;
    if (!parse(text.c_str(), rules, err)) {
        fprintf(stderr, "fused_reduce_norm: %s (%s); using built-in shapes\n", err.c_str(), path);
        return;
    }
    g_rules.swap(rules);
}

// The compiled-in measured table, parsed at the first use (it is checked by
// a test; a table that failed to parse would leave the hand-fitted rules).
void load_tuned_locked() {
    if (g_tuned_parsed) return;
    g_tuned_parsed = true;
    std::string err;
    if (!parse(kTunedTable, g_tuned, err)) {
        fprintf(stderr, "fused_reduce_norm: compiled-in launch table: %s\n", err.c_str());
        g_tuned.clear();
    }
}

// Both tables, caller's first, ready under g_mu.
void load_tables_locked() {
    load_env_table_locked();
    load_tuned_locked();
}

// The hand-fitted rule, from graph-replay sweeps on MI355X (the sandwich
// workloads by hand, then tune.py over nine and later twenty shapes with
// inputs rotated over 1 GiB, the disputed cells A/B/B/A-interleaved):
//  - small T (T <= 256, latency-bound): one vector per lane up to 896
//    lanes, else two -- more lanes issue the row's loads at once (H=6144
//    R=8 T=1: 3.8 us with one vector, 4.2 with two; H=5120 T=64: 5.0
//    against 5.3); at 1024 lanes (H=8192) it is a wash at T <= 64, 1.5%
//    either way with hot or cold inputs, and two vectors win at T = 256
//    (10.6 against 10.9 us);
//  - larger T without finalize: four vectors per lane for rows of 1024+
//    vectors from T = 257 and of 512+ vectors from T = 513, up to T = 1024,
//    and for rows of 768+ vectors (H >= 6144) up to T = 4096 -- fewer waves
//    per row to synchronise (H=5120 T=1024: 16.0 -> 15.3 us; H=8192 T=512:
//    18.8 -> 17.7 us); two vectors below 1024 vectors at T <= 512 (H=5120:
//    9.1 -> 8.7 us, H=7168 R=2: 8.7 -> 8.3 us at T=512); beyond that two
//    vectors for rows over 512 vectors (H=5120 at T=2048 and 4096: two
//    vectors 29.1 and 51.9 us, four 29.5 and 52.0 us);
//  - with finalize, one vector per lane up to 1024 lanes, except two for
//    256 < T <= 1024 at R <= 2 and for split pass 1, and for 256 < T <= 512
//    at R > 2 (H=7168 R=2 k=8: T=512 29.0 -> 27.6 us, T=1024 57.4 -> 53.4
//    us; H=6144 R=8 k=10: T=512 91.9 -> 88.8 us with two, T=1024 195.9 ->
//    181.9 us with one);
//  - with the expert-parallel finalize, one vector per lane up to 1024
//    lanes except two for 256 < T <= 512: its work list is short per rank,
//    and more tokens in flight per CU matter more (H=6144 R=8 k=10: T=4096
//    131 against 145 us with two; T=512 21.1 against 20.4).
//  - beyond T = 4096 without finalize, one vector per lane up to 1024 lanes:
//    with the epilogue issuing every load before its first store, tune.py
//    over the sixteen measured shapes without finalize put one vector within
//    1% of the fastest one-row choice at T = 16384 in 14 of them, and ahead
//    of two vectors by 1-5% at R = 8 (H=8192 sandwich: 469.6 against 493.8
//    us; H=8192 R=8 residual + RMSNorm: 487.7 against 501.3).
// Four vectors are never used with the finalize (too many live registers)
// or for split pass 1 (it spills).
int builtin_vec(int nvec, int fin, int64_t T, int epilogue, int R) {
    if (fin == kEpFinalize) {
        if (T > 256 && T <= 512 && nvec <= 2048) return 2;
        return nvec <= 1024 ? 1 : 2;
    }
    if (fin == kTpFinalize) {
        const int64_t two_up_to = (epilogue == kStoreSum || R <= 2) ? 1024 : 512;
        if (T > 256 && T <= two_up_to && nvec <= 2048) return 2;
        return nvec <= 1024 ? 1 : 2;
    }
    if (T <= 256) return nvec <= 896 ? 1 : 2;
    if (epilogue != kStoreSum && nvec >= 512) {
        if (T <= 512) return nvec >= 1024 ? 4 : 2;
        if (T <= 1024 || (nvec >= 768 && T <= 4096)) return 4;
    }
    if (epilogue != kStoreSum && T > 4096) return nvec <= 1024 ? 1 : 2;
    return nvec <= 512 ? 1 : 2;
}

// A tuned vec must fit the kernels that exist: at most 1024 lanes, and four
// vectors only without finalize and outside split pass 1.
bool vec_fits(int vec, int nvec, bool finalize, int epilogue) {
    if ((nvec + vec - 1) / vec > 1024) return false;
    if (vec == 4 && (finalize || epilogue == kStoreSum)) return false;
    return true;
}

// Whether rows_pipelined_kernel serves a call with `vec` vectors per lane:
// no finalize, the residual + RMSNorm or sandwich epilogue, 1 <= R <= 4
// (the next row's loads stay in registers), rows that split into whole
// waves (H/8 a multiple of 64 * vec, so no lane is idle), at most 1024
// lanes with one vector and 512 with two (the register budget of two), and
// gamma rows that fit in 64 KiB of LDS.
bool pipe_fits(int vec, int nvec, int fin, int epilogue, int R) {
    if (fin != kNoFinalize || (epilogue != kRmsNorm && epilogue != kSandwich)) return false;
    if (R < 1 || R > 4 || (vec != 1 && vec != 2)) return false;
    if (nvec % (64 * vec) != 0 || nvec / vec > (vec == 1 ? 1024 : 512)) return false;
    const int64_t gamma_bytes = (int64_t)(epilogue == kSandwich ? 2 : 1) * nvec * 32;
    return gamma_bytes <= 65536;
}

// The built-in choice of rows_pipelined_kernel, from graph-replay runs on
// MI355X with inputs rotated over 1 GiB, each graph replayed for a warm-up
// first (bit-identical outputs either way).  With two vectors per lane and
// one workgroup per CU it beat one row per workgroup from T = 1536 on rows
// of 640 to 896 vectors with the sandwich epilogue, whose two row sums and
// two gamma rows it overlaps with the next row's loads -- H=5120 R=4
// (A/B/B/A): T=1536 22.1 against 23.6 us, T=2048 27.1-27.7 against
// 28.8-29.0, T=4096 49.7-50.5 against 51.5-51.9, T=8192 94.4 against 97.7,
// T=16384 185.9 against 191.2; H=6144 R=2 T=2048 24.7 against 26.6 -- and
// with the residual + RMSNorm epilogue at R = 1 (the split path's pass 2,
// H=7168: T=4096 40.2 against 41.0 us, T=16384 154.1 either way).  With
// that lighter epilogue at R >= 2 it came out even or behind (H=7168 R=2:
// T=8192 even, T=16384 195.7 against 187.4 us; H=6144 R=4 T=4096 60.3
// against 59.0).  It lost at T <= 1024 (H=5120: 15.6 against 14.7 us; every
// row is resident at once there already), with two or three workgroups per
// CU (up to 1.06x slower), at R=8 (H=8192 T=4096: 125-128 against 119 us),
// and on rows of 512 and 1024 vectors, where the one-row kernel's four
// vectors per lane fit the row in few waves (H=4096 R=2 T=1536-2048: 3-7%
// behind; H=8192 R=4: 1-3% behind).  Returns the vec, or 0 for the one-row
// kernel.
//  Residual + RMSNorm at R = 2 is the exception, re-measured after the
//  one-row kernel's epilogue began issuing every load before its first
//  store: for 1536 <= T <= 4096 the row-pipelined kernel with one vector per
//  lane beat the one-row kernel on all four shapes measured, rows of 512 to
//  1024 vectors included (T=2048 / 4096: H=4096 16.3 / 29.1 against 16.9 /
//  30.1 us, H=5120 19.8 / 36.0 against 20.8 / 36.9, H=7168 26.7 / 49.1
//  against 27.0 / 50.0, H=8192 29.9 / 55.7 against 30.1 / 56.0) and lost at
//  T=16384 (107.5 against 110.3 us at H=4096).
//  The sandwich at R >= 3 on rows of 768+ vectors stops at T = 4096: at
//  R = 4 it lost from T = 8192 on both shapes measured (H=6144: T=8192 121.4
//  against 116.9 us, T=16384 245.3 against 227.1; H=7168: 137.7 against
//  135.0, 281.4 against 267.2), while at R = 2, and at H=5120 R=4, it won
//  through T = 16384 (H=7168 R=2: 196.0 against 197.9 us; H=5120 R=4: 186.6
//  against 190.7).
int builtin_pipe_vec(int nvec, int fin, int64_t T, int epilogue, int R) {
    if (T < 1536) return 0;
    if (epilogue == kRmsNorm && R == 2) {
        if (T > 4096 || nvec < 512 || nvec > 1024) return 0;
        return pipe_fits(1, nvec, fin, epilogue, R) ? 1 : 0;
    }
    if (nvec <= 512 || nvec >= 1024) return 0;
    if (epilogue == kRmsNorm && R != 1) return 0;
    if (epilogue == kSandwich && R >= 3 && nvec >= 768 && T > 4096) return 0;
    if (pipe_fits(2, nvec, fin, epilogue, R)) return 2;
    if (pipe_fits(1, nvec, fin, epilogue, R)) return 1;
    return 0;
}

// The built-in choice of the split-row finalize (a workgroup per token and
// 512-column slice with a wave per rank, summing the R rounded partials in
// LDS into one FP32 row of the workspace, then the epilogue kernel) over the
// one-row finalize, from graph-replay sweeps on MI355X with inputs rotated
// over 1 GiB.  With one workgroup per token, all R * (k + 1) rows of a token
// pass through one CU, whose throughput bounds the one-row kernel at small T
// (about 37 GB/s per CU at T=16, R=8, k=10), so its time is nearly flat in
// T; the split-row finalize spreads a token over many workgroups but writes
// and re-reads one FP32 row per token and adds a second launch, so its time
// grows with T from a lower start.
// Largest T at which the split-row finalize still won (25 shapes, T = 1, 8,
// 16, 32, 48, 64, 96, 128, 160, 192, 224, 256):
//  - TP routing, R = 1: none (H=7168 k=8: 6.2 us either way at T=1);
//  - TP routing, R = 2: 64 at H*k >= 32768 (H=7168 k=8: 8.9 against 9.9 us
//    at T=64, 10.3 against 10.2 at T=96), 96 at H*k >= 65536 (H=5120 k=16:
//    11.5 against 12.7 us at T=96, 13.2 against 13.1 at T=128); none below
//    (H=4096 k=4: 5.6 against 5.4 us at T=1; H=2048 k=8 within 5% either
//    way);
//  - TP routing, 3 <= R: 256 at H <= 2048 (R=4 k=8: 11.7 against 12.6 us at
//    T=256), 224 at H <= 3072 (R=8 k=8: 22.7 against 24.0 us at T=224, 24.7
//    against 24.6 at T=256), 192 at H <= 4096 (R=8 k=8: 24.5 against 24.9 us
//    at T=192, 27.4 against 26.2 at T=224; R=16 the same); above, 128 at
//    R >= 5 (H=6144 R=8 k=10: 28.3 against 30.2 us at T=128, 34.8 against
//    32.3 at T=160; k=4, H=7168 R=8 and R=16 the same, H=16384 R=8 a tie at
//    128) and 192 for k <= 2 (H=6144 R=8 k=2: 16.4 against 16.8 us at T=192,
//    18.3 against 17.4 at T=224); at R = 4, 128 up to H=6144 (H=5120 k=8:
//    13.2 against 14.4 us at T=128, 15.7 against 14.8 at T=160) and 96 above
//    (H=8192 k=8: 15.1 against 17.0 at T=96, 19.0 against 17.8 at T=128);
//    R = 3 taken as 96;
//  - expert-parallel routing, where the one-row kernel already keeps
//    several ranks' rows in flight and the split kernel's waves of ranks
//    without a live slot idle: 64 at R <= 2 (H=6144 k=8: 7.6 against 7.8 us
//    at T=64, 8.4 against 7.9 at T=96); 32 at k <= 4 (H=6144 R=8 k=4: 6.9
//    against 7.5 at T=32, 7.5 each at T=48); 256 at H <= 2048 (R=8 k=8: 8.8
//    against 9.5 us at T=256); at R >= 16, 128 at H <= 4096 (H=4096 k=8:
//    12.7 against 13.9 us at T=128, 14.5 against 14.1 at T=160; H=3072 k=6
//    10.3 against 11.2) and 96 above; else 64 (H=6144 R=8 k=10: 8.7 against
//    11.1 us at T=64, 11.9 against 11.1 at T=96; H=7168 R=4 k=8: 8.0
//    against 9.2 at T=64, 9.2 each at T=96).
int64_t builtin_split_max_t(int32_t R, int64_t H, int32_t k, bool ep) {
    if (ep) {
        if (R <= 2) return 64;
        if (k <= 4) return 32;
        if (H <= 2048) return 256;
        if (R >= 16) return H <= 4096 ? 128 : 96;
        return 64;
    }
    if (R == 1) return 0;
    if (R == 2) return H * k >= 65536 ? 96 : H * k >= 32768 ? 64 : 0;
    if (H <= 2048) return 256;
    if (H <= 3072) return 224;
    if (H <= 4096) return 192;
    if (R == 3) return 96;
    if (R == 4) return H <= 6144 ? 128 : 96;
    return k <= 2 ? 192 : 128;
}

bool matches(const Rule& r, int64_t H, int64_t R, int64_t k, int64_t epilogue, int64_t ep) {
    return (r.H < 0 || r.H == H) && (r.R < 0 || r.R == R) && (r.k < 0 || r.k == k) &&
           (r.epilogue < 0 || r.epilogue == epilogue) && (r.ep < 0 || r.ep == ep);
}

}  // namespace

bool use_split_rows(int32_t R, int64_t H, int32_t k, bool ep, int epilogue, int64_t T) {
    if (k < 1 || T < 1 || T > kSplitCapT) return false;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        load_tables_locked();
        bool builtin = false;
        for (const std::vector<Rule>* table : {&g_rules, &g_tuned}) {
            for (const Rule& r : *table) {
                if (r.vec >= 0 || !matches(r, H, R, k, epilogue, ep ? 1 : 0)) continue;
                if (T < r.tmin || T > r.tmax) continue;
                if (r.vec == kBuiltinRule) {
                    builtin = true;
                    break;
                }
                return r.vec == kSplitRule;
            }
            if (builtin) break;
        }
    }
    return T <= builtin_split_max_t(R, H, k, ep);
}

int64_t split_rows_cap(int32_t R, int64_t H, int32_t k) {
    if (k < 1) return 0;
    int64_t cap = builtin_split_max_t(R, H, k, false);
    const int64_t cap_ep = builtin_split_max_t(R, H, k, true);
    if (cap_ep > cap) cap = cap_ep;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        load_tables_locked();
        for (const std::vector<Rule>* table : {&g_rules, &g_tuned})
            for (const Rule& r : *table)
                if (r.vec == kSplitRule && (r.H < 0 || r.H == H) && (r.R < 0 || r.R == R) &&
                    (r.k < 0 || r.k == k) && r.tmax > cap)
                    cap = r.tmax;
    }
    return cap < kSplitCapT ? cap : kSplitCapT;
}

LaunchShape choose_shape(int nvec, int fin, int64_t T, int epilogue, int R, int k) {
    const bool finalize = fin != kNoFinalize;
    const int64_t ep = fin == kEpFinalize ? 1 : 0;
    int vec = 0;
    bool pipe = false;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        load_tables_locked();
        const int64_t H = (int64_t)nvec * 8;
        bool builtin = false;
        for (const std::vector<Rule>* table : {&g_rules, &g_tuned}) {
            for (const Rule& r : *table) {
                const bool shape_rule = r.vec > 0 || r.vec == kBuiltinRule;
                if (!shape_rule || !matches(r, H, R, k, epilogue, ep) || T < r.tmin ||
                    T > r.tmax)
                    continue;
                if (r.vec == kBuiltinRule) {
                    builtin = true;
                    break;
                }
                if (r.pipe ? pipe_fits(r.vec, nvec, fin, epilogue, R)
                           : vec_fits(r.vec, nvec, finalize, epilogue)) {
                    vec = r.vec;
                    pipe = r.pipe;
                    break;
                }
            }
            if (vec != 0 || builtin) break;
        }
    }
    if (vec == 0) {
        vec = builtin_pipe_vec(nvec, fin, T, epilogue, R);
        pipe = vec != 0;
    }
    if (vec == 0) vec = builtin_vec(nvec, fin, T, epilogue, R);
    LaunchShape sh;
    sh.vec = vec;
    sh.pipelined = pipe;
    const int lanes = (nvec + vec - 1) / vec;
    sh.threads = ((lanes + 63) / 64) * 64;
    return sh;
}

int64_t compute_units() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
    int v = dev >= 0 ? cus[dev].load(std::memory_order_relaxed) : 0;
    if (v <= 0) {
        if (dev < 0 ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;  // MI355X
        if (dev >= 0) cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

const char* set_launch_table(const char* text) {
    std::lock_guard<std::mutex> lock(g_mu);
    g_env_checked = true;  // an explicit table replaces the environment's
    if (text == nullptr) {
        g_rules.clear();
        return nullptr;
    }
    std::vector<Rule> rules;
    if (!parse(text, rules, g_parse_error)) return g_parse_error.c_str();
    g_rules.swap(rules);
    return nullptr;
}

}  // namespace frn
