// Host side of the C ABI: argument checks, workspace planning, launch order.
// Every check runs before any device call; launches go in order on the
// caller's stream and nothing here waits for the device (except growing a
// cached workspace, which synchronises that stream once).
//
// Conventions follow "UForm for Swift", sections "Errors" and "Design" (one
// C verb per operation, statuses spelled like "invalid-argument"); the loss
// follows "Scaling-Up Contrastive Learning over NVLink Multicast", section
// "One Set or Two".
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "common.h"
#include "uform_contrastive.h"

namespace {

using namespace uform;

thread_local std::string g_last_error;

uform_status_t fail(uform_status_t st, const std::string &msg) {
    g_last_error = msg;
    return st;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
    int64_t R, N, D, P, off;
    int kind;
    bool want_dq, want_dk;
    uint32_t mask;
    bool gen;                          // the generic backward (ladders without a compiled kernel, D > 1024)
    int gen_nq;                        // its 32-wide steps per wave
    int64_t nIt, nJt;                  // forward tiles
    int64_t nsplit_row, nsplit_col;    // backward inner splits
    int64_t bps_row, bps_col;          // inner blocks per split
    int64_t slots_a, slots_b, nslots;  // loss partial slots
    // workspace offsets (bytes)
    size_t o_invq, o_invk, o_qA, o_kA, o_posdot, o_qH, o_kH;
    size_t o_qIYR, o_kIYR, o_sigq, o_sigk, o_gamq, o_gamk;
    size_t o_qC, o_qRho, o_qKap, o_kC, o_kRho, o_kKap, o_negfrac, o_kNegfrac, o_diagA, o_gmax;
    size_t o_rowpart, o_colpart, o_part, o_Cpart, o_loss, o_tsum, o_bias;
    int64_t npos;                      // listed extra positives
    bool pos_cols;                     // the column lists are needed (two-set sigmoid with dk)
    size_t o_plist, o_pparts;           // extra positives: lists and mask tables (ListWords), partial sums
    size_t total;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Word offsets (int32) of the extra-positive region of the workspace, at most npos cells:
// row lists [R + 1 | npos]; column lists [N + 1 | npos] (for dk); then per backward pass the
// outer blocks' entry ranges [blocks + 1] and at most npos ListEnt entries (8-byte aligned).
struct ListWords {
    size_t rows, cols, lptr_r, ent_r, lptr_c, ent_c, total;
    ListWords(int64_t R, int64_t N, int64_t npos, bool pos_cols) {
        const size_t n = npos > 0 ? (size_t)npos : 0;
        auto even = [](size_t w) { return (w + 1) & ~(size_t)1; };
        rows = 0;
        cols = rows + (size_t)R + 1 + n;
        lptr_r = cols + (pos_cols ? (size_t)N + 1 + n : 0);
        ent_r = even(lptr_r + (size_t)((R + kBwdOuter - 1) / kBwdOuter) + 1);
        lptr_c = ent_r + n * kListEntWords;
        ent_c = even(lptr_c + (pos_cols ? (size_t)((N + kBwdOuter - 1) / kBwdOuter) + 1 : 0));
        total = ent_c + (pos_cols ? n * kListEntWords : 0);
    }
};

// Mask tables of one backward pass from its outer rows' CSR lists (ptr [NO + 1], idx): per block
// of kBwdOuter outer rows, one ListEnt per inner block that holds listed cells, sorted by nb.
void build_list_ents(int64_t NO, const int32_t *ptr, const int32_t *idx, int32_t *lptr, std::vector<ListEnt> &ents) {
    const int64_t nob = (NO + kBwdOuter - 1) / kBwdOuter;
    std::vector<std::pair<int32_t, int32_t>> cells;  // (inner block, row in block * 64 + outer lane)
    lptr[0] = 0;
    for (int64_t ob = 0; ob < nob; ++ob) {
        cells.clear();
        const int64_t o1 = std::min(NO, (ob + 1) * kBwdOuter);
        for (int64_t o = ob * kBwdOuter; o < o1; ++o)
            for (int32_t e = ptr[o]; e < ptr[o + 1]; ++e)
                cells.emplace_back(idx[e] / kBwdInner, (idx[e] % kBwdInner) * 64 + (int32_t)(o - ob * kBwdOuter));
        std::sort(cells.begin(), cells.end());
        for (size_t c = 0; c < cells.size(); ++c) {
            if (c == 0 || cells[c].first != cells[c - 1].first) {
                ents.push_back(ListEnt{});
                ents.back().nb = cells[c].first;
            }
            ents.back().m[cells[c].second / 64] |= 1ull << (cells[c].second % 64);
        }
        lptr[ob + 1] = (int32_t)ents.size();
    }
}

// Inner splits so that a pass launches enough workgroups for 256 CUs.
void choose_split(int64_t NO, int64_t NI, int64_t bo, int64_t &nsplit, int64_t &bps) {
    const int64_t wgs = cdiv(NO, bo);
    const int64_t nblocks = cdiv(NI, kBwdInner);
    int64_t want = cdiv(256, wgs);  // one round of workgroups: one per CU (a workgroup fills its CU)
    if (want < 1) want = 1;
    if (want > nblocks) want = nblocks;
    bps = cdiv(nblocks, want);
    nsplit = cdiv(nblocks, bps);
}

// Bit ds set: a prefix ends at 32 (ds + 1).  Ladders wider than 1024 have no compiled backward
// (mask 0).
uint32_t ladder_mask(const int32_t *pw, int32_t n) {
    if (pw[n - 1] > 1024) return 0u;
    uint32_t m = 0;
    for (int32_t i = 0; i < n; ++i) m |= 1u << (pw[i] / 32 - 1);
    return m;
}

// 32-wide steps per wave of the generic backward: the least power of two with 4 waves covering
// the widest prefix.
int gen_nq_for(int32_t widest) {
    const int steps = widest / 32;
    int nq = 1;
    while (4 * nq < steps) nq *= 2;
    return nq;
}

GenTabs make_gen_tabs(const int32_t *pw, int32_t P, int nq) {
    GenTabs t{};
    for (int j = 0; j < kMaxSteps; ++j) {
        t.snap_at[j] = -1;
        int band = P;
        for (int p = P - 1; p >= 0; --p)
            if (pw[p] > 32 * j) band = p;
        t.band_of[j] = (int8_t)band;
    }
    int interior = 0;
    for (int p = 0; p < P; ++p) {
        const int e = pw[p] / 32 - 1;  // the prefix's last step
        t.wave_of[p] = (int8_t)(e / nq);
        if ((e + 1) % nq == 0) {
            t.snap_slot[p] = (int8_t)(e / nq);
        } else {
            t.snap_slot[p] = (int8_t)(4 + interior);
            t.snap_at[e] = (int8_t)(4 + interior);
            ++interior;
        }
    }
    t.nslot = 4 + interior;
    return t;
}

// Which backward a ladder takes: the compiled one (k_bwd), or the generic one if its tables fit.
bool bwd_compiled(int64_t D, const int32_t *pw, int32_t P) {
    return D <= 1024 && bwd_mask_supported(ladder_mask(pw, P));
}
bool bwd_generic_fits(const int32_t *pw, int32_t P) {
    const int nq = gen_nq_for(pw[P - 1]);
    return make_gen_tabs(pw, P, nq).nslot <= gen_max_slots(nq) && P + 1 <= gen_max_bands(nq);
}

Plan make_plan(int64_t R, int64_t N, int64_t D, const int32_t *pw, int32_t P, int kind, int64_t off, bool want_dq,
               bool want_dk, bool one_split = false, int64_t npos = -1, int force_gen = -1) {
    Plan p{};
    p.R = R;
    p.N = N;
    p.D = D;
    p.P = P;
    p.off = off;
    p.kind = kind;
    p.want_dq = want_dq;
    p.want_dk = want_dk;
    p.mask = ladder_mask(pw, P);
    p.gen = force_gen >= 0 ? force_gen != 0 : !bwd_compiled(D, pw, P);
    p.gen_nq = gen_nq_for(pw[P - 1]);
    const int64_t bo = p.gen ? kGenOuter : kBwdOuter;  // outer rows per backward workgroup
    const bool softmax = kind != kSiglip;
    p.nIt = cdiv(R, kFwdTile);
    p.nJt = cdiv(N, kFwdTile);
    choose_split(R, N, bo, p.nsplit_row, p.bps_row);
    choose_split(N, R, bo, p.nsplit_col, p.bps_col);
    if (one_split) {
        p.nsplit_row = p.nsplit_col = 1;
        p.bps_row = cdiv(N, kBwdInner);
        p.bps_col = cdiv(R, kBwdInner);
    }
    // loss slots: softmax = row stats blocks + column stats blocks;
    // sigmoid = positive-cell blocks + row-pass workgroups
    if (softmax) {
        p.slots_a = cdiv(R, kStatRows);
        p.slots_b = cdiv(N, kStatRows);
    } else {
        p.slots_a = cdiv(R + N, 256);
        p.slots_b = cdiv(R, bo) * p.nsplit_row;
    }
    p.nslots = p.slots_a + p.slots_b;

    size_t off_b = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off_b;
        off_b += align_up(bytes);
        return o;
    };
    const size_t fR = sizeof(float) * P * R, fN = sizeof(float) * P * N;
    p.o_invq = take(fR);
    p.o_invk = take(fN);
    p.o_qA = take(fR);
    p.o_kA = take(fN);
    p.o_posdot = take(fR);
    p.o_qIYR = take(fR);
    p.o_kIYR = take(fN);
    p.o_sigq = take(sizeof(float) * R);
    p.o_sigk = take(sizeof(float) * N);
    p.o_gamq = take(sizeof(float) * R);
    p.o_gamk = take(sizeof(float) * N);
    p.o_qC = take(fR);
    p.o_qRho = take(fR);
    p.o_qKap = take(fR);
    p.o_kC = take(fN);
    p.o_kRho = take(fN);
    p.o_kKap = take(fN);
    p.o_negfrac = take(fR);
    p.o_kNegfrac = take(fN);
    p.o_gmax = take(sizeof(float) * 4 * P);
    p.o_diagA = take(fR);
    const bool bwd = want_dq || want_dk || !softmax;  // some backward pass runs
    p.o_qH = take(bwd ? sizeof(u16) * bwd_padded_rows(R) * D : 0);
    p.o_kH = take(bwd ? sizeof(u16) * bwd_padded_rows(N) * D : 0);
    // forward partials: one per tile (row partials per column tile, column partials per row tile)
    p.o_rowpart = take(softmax ? sizeof(float) * p.nJt * P * R : 0);
    p.o_colpart = take(softmax ? sizeof(float) * p.nIt * P * N : 0);
    // gradient partials only with inner splits (one split: the backward finishes the rows in place;
    // the generic backward always leaves its rows to k_finalize)
    const size_t part_row = (want_dq && (p.nsplit_row > 1 || p.gen)) ? sizeof(float) * p.nsplit_row * R * D : 0;
    const size_t part_col = (want_dk && (p.nsplit_col > 1 || p.gen)) ? sizeof(float) * p.nsplit_col * N * D : 0;
    p.o_part = take(part_row > part_col ? part_row : part_col);
    const size_t c_row = sizeof(float) * p.nsplit_row * P * R, c_col = sizeof(float) * p.nsplit_col * P * N;
    p.o_Cpart = take(c_row > c_col ? c_row : c_col);
    p.o_loss = take(sizeof(float) * p.nslots * P);
    // per-row radial sums of one gradient pass (dL/dscale); sigmoid bias partials (dL/dbias)
    p.o_tsum = take((want_dq || want_dk) ? sizeof(float) * (R > N ? R : N) : 0);
    p.o_bias = take((want_dq || want_dk) && !softmax ? sizeof(float) * p.nslots * P : 0);
    // extra positives (npos >= 0: a list is given), int32 in one region (one copy): the row lists
    // [R + 1 | npos], then, for dk of the two-set form, the column lists [N + 1 | npos]; then
    // the pass's partial sums
    p.npos = npos;
    p.pos_cols = npos >= 0 && want_dk;
    p.o_plist = take(npos >= 0 ? sizeof(int32_t) * ListWords(R, N, npos, p.pos_cols).total : 0);
    p.o_pparts = take(npos >= 0 ? sizeof(float) * kPosBlocks * 3 * P : 0);
    p.total = off_b;
    return p;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

uform_status_t validate(const void *q, const void *k, int64_t R, int64_t N, int64_t D, const int32_t *prefixes,
                        int32_t n_prefixes, float scale, float bias, int32_t kind, const float *loss_out,
                        const float *dq, const float *dk, const uform_contrastive_options_t *opt) {
    g_last_error.clear();
    if (!q || !k) return fail(uform_status_invalid_argument_k, "q and k must be device pointers");
    if (!loss_out) return fail(uform_status_invalid_argument_k, "loss_out must be a device pointer");
    if (!aligned(q, 16) || !aligned(k, 16)) return fail(uform_status_invalid_argument_k, "q and k must be 16-byte aligned");
    if (!aligned(loss_out, 4)) return fail(uform_status_invalid_argument_k, "loss_out must be 4-byte aligned");
    if ((dq && !aligned(dq, 16)) || (dk && !aligned(dk, 16)))
        return fail(uform_status_invalid_argument_k, "dq and dk must be 16-byte aligned");
    if (R < 1 || N < 1 || D < 1) return fail(uform_status_invalid_argument_k, "R, N and D must be positive");
    if (R > N) return fail(uform_status_invalid_argument_k, "R must not exceed N");
    if (kind < kInfonce || kind > kOnesetEdges) return fail(uform_status_invalid_argument_k, "unknown kind");
    const int64_t off = opt ? opt->row_offset : 0;
    if (off < 0 || off + R > N) return fail(uform_status_invalid_argument_k, "need 0 <= row_offset and row_offset + R <= N");
    const bool oneset = kind == kOneset || kind == kOnesetEdges;
    if (kind == kOneset && N % 2 != 0)
        return fail(uform_status_invalid_argument_k, "the one-set form with pairs needs an even set (rows 2m, 2m + 1 pair up)");
    if (oneset) {
        if ((const char *)q != (const char *)k + off * D * 2)
            return fail(uform_status_invalid_argument_k, "the one-set forms need q = k + row_offset * D (its rows of the set)");
        if (dk) return fail(uform_status_invalid_argument_k, "the one-set forms have one gradient, dq (pass dk = NULL)");
    }
    if (kind == kOnesetEdges && opt && opt->pos_logit_out)
        return fail(uform_status_invalid_argument_k, "the one-set form with listed relations has no single positive logit");
    if (kind == kInfonce && (R != N || off != 0))
        return fail(uform_status_invalid_argument_k, "symmetric InfoNCE needs R == N and row_offset == 0");
    if (!prefixes) return fail(uform_status_invalid_argument_k, "prefixes must be a host array");
    if (n_prefixes < 1 || n_prefixes > kMaxP) return fail(uform_status_invalid_argument_k, "n_prefixes must be in [1, 8]");
    for (int32_t i = 0; i < n_prefixes; ++i) {
        if (prefixes[i] < 32 || prefixes[i] % 32 != 0)
            return fail(uform_status_invalid_argument_k, "prefix widths must be positive multiples of 32");
        if (i > 0 && prefixes[i] <= prefixes[i - 1])
            return fail(uform_status_invalid_argument_k, "prefix widths must be strictly increasing");
    }
    if (prefixes[n_prefixes - 1] > D) return fail(uform_status_invalid_argument_k, "the widest prefix exceeds D");
    if (!std::isfinite(scale) || !std::isfinite(bias)) return fail(uform_status_invalid_argument_k, "scale and bias must be finite");
    if (scale == 0.0f) return fail(uform_status_invalid_argument_k, "scale must be nonzero");
    if (opt && opt->prefix_weights) {
        for (int32_t i = 0; i < n_prefixes; ++i)
            if (!(opt->prefix_weights[i] > 0.0f) || !std::isfinite(opt->prefix_weights[i]))
                return fail(uform_status_invalid_argument_k, "prefix weights must be finite and positive");
    }
    if (opt && opt->workspace && !aligned(opt->workspace, 256))
        return fail(uform_status_invalid_argument_k, "workspace must be 256-byte aligned");
    if (opt && (opt->dscale_out || opt->dbias_out)) {
        if (!dq && !dk)
            return fail(uform_status_invalid_argument_k, "dscale_out and dbias_out come from a gradient pass: give dq or dk");
        if ((opt->dscale_out && !aligned(opt->dscale_out, 4)) || (opt->dbias_out && !aligned(opt->dbias_out, 4)))
            return fail(uform_status_invalid_argument_k, "dscale_out and dbias_out must be 4-byte aligned");
    }
    if (opt && opt->pos_row_ptr) {
        if (kind != kSiglip && !oneset)
            return fail(uform_status_invalid_argument_k, "listed positives are defined for the sigmoid kinds");
        const int64_t *rp = opt->pos_row_ptr;
        if (rp[0] != 0) return fail(uform_status_invalid_argument_k, "pos_row_ptr[0] must be 0");
        for (int64_t i = 0; i < R; ++i)
            if (rp[i + 1] < rp[i]) return fail(uform_status_invalid_argument_k, "pos_row_ptr must not decrease");
        if (rp[R] > 0 && !opt->pos_col)
            return fail(uform_status_invalid_argument_k, "pos_col must be a host array when positives are listed");
        if (rp[R] >= ((int64_t)1 << 31) - 1)
            return fail(uform_status_unsupported_k, "at most 2^31 - 2 extra positives per call");
        for (int64_t i = 0; i < R; ++i) {
            const int64_t g = off + i, own = kind == kSiglip ? g : kind == kOneset ? (g ^ 1) : -1;
            for (int64_t e = rp[i]; e < rp[i + 1]; ++e) {
                const int64_t j = opt->pos_col[e];
                if (j < 0 || j >= N || (e > rp[i] && j <= opt->pos_col[e - 1]) || j == own || (oneset && j == g))
                    return fail(uform_status_invalid_argument_k,
                                "row " + std::to_string(i) + ": listed positives must be increasing columns in [0, N), "
                                "none of them the row's own positive (nor, in the one-set forms, the row itself)");
            }
        }
        if (oneset) {  // mirrored cells carry one label: a pair of two rows of the share is listed both ways
            for (int64_t i = 0; i < R; ++i)
                for (int64_t e = rp[i]; e < rp[i + 1]; ++e) {
                    const int64_t j = opt->pos_col[e] - off;
                    if (j < 0 || j >= R) continue;
                    const int32_t *b = opt->pos_col + rp[j], *en = opt->pos_col + rp[j + 1];
                    if (!std::binary_search(b, en, (int32_t)(off + i)))
                        return fail(uform_status_invalid_argument_k,
                                    "rows " + std::to_string(off + i) + " and " + std::to_string(off + j) +
                                        ": a one-set pair must be listed both ways");
                }
        }
    }
    if (D % 64 != 0 || D > kMaxD) return fail(uform_status_unsupported_k, "D must be a multiple of 64 and at most 2048");
    const bool sigmoid_kind = kind == kSiglip || oneset;
    if (!sigmoid_kind && std::fabs(scale) > UFORM_CONTRASTIVE_MAX_SOFTMAX_SCALE)
        return fail(uform_status_unsupported_k, "softmax kinds support |scale| <= 40");
    if ((dq || dk || sigmoid_kind) && !bwd_compiled(D, prefixes, n_prefixes) && !bwd_generic_fits(prefixes, n_prefixes))
        return fail(uform_status_unsupported_k,
                    "this prefix ladder needs more snapshot slots or bands than the backward's LDS holds at this width");
    if (N > (int64_t)1 << 31) return fail(uform_status_unsupported_k, "N must be below 2^31");
    return uform_status_success_k;
}

// ---------------------------------------------------------------- workspace cache

struct Cached {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Cached> g_cache;

// Pinned host staging of the extra-positive lists, one per device and stream.  The copy out of
// it is enqueued on the stream; an event after the copy guards the buffer's next refill.
struct Staging {
    int32_t *host = nullptr;
    size_t count = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
};
std::map<std::pair<int, hipStream_t>, Staging> g_staging;

// Fill the pinned staging buffer of (device, stream) through fill(buf) and enqueue its copy to dst.
template <class Fill>
uform_status_t stage_and_copy(hipStream_t s, int32_t *dst, size_t count, Fill fill) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(uform_status_device_error_k, "hipGetDevice failed");
    std::lock_guard<std::mutex> lock(g_mu);
    Staging &st = g_staging[{dev, s}];
    if (!st.ev && hipEventCreateWithFlags(&st.ev, hipEventDisableTiming) != hipSuccess) {
        st.ev = nullptr;
        return fail(uform_status_device_error_k, "hipEventCreate failed");
    }
    if (st.pending && hipEventSynchronize(st.ev) != hipSuccess)  // the previous copy out of the buffer is done
        return fail(uform_status_device_error_k, "waiting for the previous list copy failed");
    st.pending = false;
    if (st.count < count) {
        if (st.host) (void)hipHostFree(st.host);
        st.host = nullptr;
        st.count = 0;
        if (hipHostMalloc((void **)&st.host, sizeof(int32_t) * count, hipHostMallocDefault) != hipSuccess || !st.host) {
            (void)hipGetLastError();
            st.host = nullptr;
            return fail(uform_status_out_of_memory_k, "pinned staging allocation failed");
        }
        st.count = count;
    }
    fill(st.host);
    if (hipMemcpyAsync(dst, st.host, sizeof(int32_t) * count, hipMemcpyHostToDevice, s) != hipSuccess ||
        hipEventRecord(st.ev, s) != hipSuccess)
        return fail(uform_status_device_error_k, "enqueueing the list copy failed");
    st.pending = true;
    return uform_status_success_k;
}

uform_status_t get_workspace(hipStream_t s, size_t need, void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(uform_status_device_error_k, "hipGetDevice failed");
    std::lock_guard<std::mutex> lock(g_mu);
    Cached &c = g_cache[{dev, s}];
    if (c.bytes < need) {
        if (c.ptr) {
            if (hipStreamSynchronize(s) != hipSuccess) return fail(uform_status_device_error_k, "stream sync failed");
            (void)hipFree(c.ptr);
            c.ptr = nullptr;
            c.bytes = 0;
        }
        void *p = nullptr;
        if (hipMalloc(&p, need) != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(uform_status_out_of_memory_k, "workspace allocation failed");
        }
        c.ptr = p;
        c.bytes = need;
    }
    *out = c.ptr;
    return uform_status_success_k;
}

// ---------------------------------------------------------------- opt-in kernel timing
// With UFORM_CONTRASTIVE_PROFILE set, every launch of a call is bracketed by a
// pair of events recorded on the caller's stream; uform_contrastive_profile()
// waits for them and returns the summed time per kernel since the last read.
struct ProfRec {
    const char *name;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;  // guards g_prof_live and g_prof_pool; a profiled call holds it throughout
std::vector<ProfRec> g_prof_live;
std::vector<hipEvent_t> g_prof_pool;

// Per-call profiling state, passed down by value: a call without the flag never touches the
// shared records, so it needs no lock.
struct ProfCtx {
    bool on = false;
    hipStream_t stream = nullptr;
};

hipEvent_t prof_event() {
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

struct ProfScope {
    ProfRec rec{};
    ProfCtx ctx;
    ProfScope(const ProfCtx &c, const char *name) : ctx(c) {
        if (!ctx.on) return;
        rec.name = name;
        rec.a = prof_event();
        rec.b = prof_event();
        if (rec.a) (void)hipEventRecord(rec.a, ctx.stream);
    }
    ~ProfScope() {
        if (!ctx.on) return;
        if (rec.b) (void)hipEventRecord(rec.b, ctx.stream);
        if (rec.a && rec.b) g_prof_live.push_back(rec);
    }
};

#define LAUNCH_NAMED(name, expr)                                                                     \
    do {                                                                                             \
        ProfScope prof_(prof, name);                                                                 \
        hipError_t e_ = (expr);                                                                      \
        if (e_ != hipSuccess) return fail(uform_status_device_error_k, std::string("launch failed: ") + \
                                                                          hipGetErrorString(e_));      \
    } while (0)
#define LAUNCH(expr) LAUNCH_NAMED(#expr, expr)

// ---------------------------------------------------------------- allocation-free workspace
// One fixed device array per GPU for the entry point that allocates nothing: the runtime
// places a copy on every device the library's code is loaded on, and it stays until the
// process ends.  Host code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): its device address comes from hipGetSymbolAddress, once per
// device, with that device current.
static __device__ __align__(256) unsigned char scratch[UFORM_CONTRASTIVE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;  // device -> device address of that device's scratch

uform_status_t scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(uform_status_device_error_k, "hipGetDevice failed");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(uform_status_device_error_k, "hipGetSymbolAddress of the allocation-free scratch failed");
        }
        it = g_scratch_ptr.emplace(dev, ptr).first;
    }
    *out = it->second;
    return uform_status_success_k;
}

// The workspace plan of a call (as run() lays it out).
Plan call_plan(int64_t R, int64_t N, int64_t D, const int32_t *prefixes, int32_t P, int32_t kind_in, const float *dq,
               const float *dk, const uform_contrastive_options_t *opt) {
    const int32_t kind = (kind_in == kOneset || kind_in == kOnesetEdges) ? kSiglip : kind_in;
    const int64_t npos = (opt && opt->pos_row_ptr) ? opt->pos_row_ptr[R] : -1;
    return make_plan(R, N, D, prefixes, P, kind, opt ? opt->row_offset : 0, dq != nullptr, dk != nullptr,
                     opt && (opt->flags & UFORM_CONTRASTIVE_ONE_SPLIT), npos);
}

uform_status_t run(const void *q_, const void *k_, int64_t R, int64_t N, int64_t D, const int32_t *prefixes,
                   int32_t P, float scale, float bias, int32_t kind_in, float *loss_out, float *dq, float *dk,
                   hipStream_t s, const uform_contrastive_options_t *opt, const ProfCtx &prof) {
    const u16 *q = (const u16 *)q_, *k = (const u16 *)k_;
    // the one-set forms run as the sigmoid kind whose cell (g, g) is not scored and whose row
    // gradients count both mirrored cells; with pairs the positive of row g is g ^ 1, with listed
    // relations no cell is an implicit positive (pxor = 0 points the positive at the self cell,
    // which the masks already leave out, and nopos gives it no terms)
    const bool oneset = kind_in == kOneset || kind_in == kOnesetEdges;
    const bool nopos = kind_in == kOnesetEdges;
    const int32_t kind = oneset ? kSiglip : kind_in;
    const int pxor = kind_in == kOneset ? 1 : 0;
    const float mirror = oneset ? 2.0f : 1.0f;
    const int64_t off = opt ? opt->row_offset : 0;
    const bool softmax = kind != kSiglip;
    const int64_t npos = (opt && opt->pos_row_ptr) ? opt->pos_row_ptr[R] : -1;
    Plan pl = call_plan(R, N, D, prefixes, P, kind_in, dq, dk, opt);

    void *ws = nullptr;
    if (opt && opt->workspace) {
        if (opt->workspace_bytes < pl.total) return fail(uform_status_invalid_argument_k, "workspace too small");
        ws = opt->workspace;
    } else {
        uform_status_t st = get_workspace(s, pl.total, &ws);
        if (st != uform_status_success_k) return st;
    }
    char *base = (char *)ws;
    auto F = [&](size_t o) { return (float *)(base + o); };
    int32_t *const plist = npos >= 0 ? (int32_t *)(base + pl.o_plist) : nullptr;
    const ListWords lw(R, N, npos, pl.pos_cols);
    int32_t *const clist = pl.pos_cols ? plist + lw.cols : nullptr;
    if (npos >= 0) {
        // row lists as given; column lists (rows ascending per column) by a counting pass; the
        // backward passes' mask tables of the listed cells
        const int64_t *rp = opt->pos_row_ptr;
        const int32_t *pc = opt->pos_col;
        std::vector<int32_t> h(lw.total, 0);
        for (int64_t i = 0; i <= R; ++i) h[lw.rows + i] = (int32_t)rp[i];
        for (int64_t e = 0; e < npos; ++e) h[lw.rows + R + 1 + e] = pc[e];
        std::vector<ListEnt> ents;
        build_list_ents(R, h.data() + lw.rows, h.data() + lw.rows + R + 1, h.data() + lw.lptr_r, ents);
        std::memcpy(h.data() + lw.ent_r, ents.data(), ents.size() * sizeof(ListEnt));
        if (pl.pos_cols) {
            int32_t *cp = h.data() + lw.cols, *cr = cp + N + 1;
            for (int64_t e = 0; e < npos; ++e) ++cp[pc[e] + 1];
            for (int64_t j = 0; j < N; ++j) cp[j + 1] += cp[j];
            std::vector<int32_t> fill((size_t)N, 0);
            for (int64_t i = 0; i < R; ++i)
                for (int64_t e = rp[i]; e < rp[i + 1]; ++e) {
                    const int32_t j = pc[e];
                    cr[cp[j] + fill[j]++] = (int32_t)i;
                }
            ents.clear();
            build_list_ents(N, cp, cr, h.data() + lw.lptr_c, ents);
            std::memcpy(h.data() + lw.ent_c, ents.data(), ents.size() * sizeof(ListEnt));
        }
        uform_status_t st = stage_and_copy(s, plist, h.size(), [&](int32_t *dst) {
            std::memcpy(dst, h.data(), h.size() * sizeof(int32_t));
        });
        if (st != uform_status_success_k) return st;
    }

    Prefixes pf{};
    pf.n = P;
    for (int i = 0; i < P; ++i) pf.w[i] = prefixes[i];
    float wsum = 0.f;
    float wnorm[kMaxP] = {};
    for (int i = 0; i < P; ++i) wsum += (opt && opt->prefix_weights) ? opt->prefix_weights[i] : 1.0f;
    for (int i = 0; i < P; ++i) wnorm[i] = ((opt && opt->prefix_weights) ? opt->prefix_weights[i] : 1.0f) / wsum;

    const float abs_s = std::fabs(scale);
    const float cshift = -abs_s * kLog2e;
    const float sgn = scale > 0 ? 1.0f : -1.0f;
    const double den = kind == kInfonce ? 2.0 * (double)N : (double)N;
    const int Di = (int)D;

    float *invq = F(pl.o_invq), *invk = F(pl.o_invk), *qA = F(pl.o_qA), *kA = F(pl.o_kA), *posdot = F(pl.o_posdot);
    float *qIYR = F(pl.o_qIYR), *kIYR = F(pl.o_kIYR), *sigq = F(pl.o_sigq), *sigk = F(pl.o_sigk);
    float *gamq = F(pl.o_gamq), *gamk = F(pl.o_gamk);
    _Float16 *qH = (_Float16 *)(base + pl.o_qH), *kH = (_Float16 *)(base + pl.o_kH);
    float *lossparts = F(pl.o_loss);

    PrepArgs pa{};
    pa.q = q;
    pa.k = k;
    pa.R = R;
    pa.N = N;
    pa.off = off;
    pa.D = Di;
    pa.pf = pf;
    pa.a_scale = scale * kLog2e;
    pa.gam_scale = (float)(mirror * abs_s / den);
    pa.pxor = pxor;
    pa.want_pos = softmax ? 0 : 1;  // the softmax kinds' forward writes posdot from its diagonal tiles
    pa.invq = invq;
    pa.invk = invk;
    pa.qA = qA;
    pa.kA = kA;
    pa.qIYR = qIYR;
    pa.kIYR = kIYR;
    pa.posdot = posdot;
    pa.sigq = sigq;
    pa.sigk = sigk;
    pa.gamq = gamq;
    pa.gamk = gamk;
    pa.gmax = F(pl.o_gmax);
    const bool half = dq || dk || !softmax;  // some backward pass runs: k_prep writes its FP16 copies
    pa.qH = half ? qH : nullptr;
    pa.kH = half ? kH : nullptr;
    pa.Rpad = bwd_padded_rows(R);
    pa.Npad = bwd_padded_rows(N);
    LAUNCH_NAMED("k_prep", launch_prep(pa, s));

    StatsArgs sa{};
    sa.R = R;
    sa.N = N;
    sa.off = off;
    sa.pxor = pxor;
    sa.nopos = nopos ? 1 : 0;
    sa.mirror = mirror;
    sa.nJt = pl.nJt;  // partials per row: one per column tile
    sa.nIt = pl.nIt;
    sa.pf = pf;
    sa.kind = kind;
    sa.scale = scale;
    sa.bias = bias;
    sa.cshift = cshift;
    sa.lse_offset = abs_s + bias;
    sa.inv_den = (float)(1.0 / den);
    sa.sgn = sgn;
    for (int i = 0; i < kMaxP; ++i) sa.wnorm[i] = wnorm[i];
    sa.rowpart = F(pl.o_rowpart);
    sa.colpart = F(pl.o_colpart);
    sa.invq = invq;
    sa.invk = invk;
    sa.posdot = posdot;
    sa.qA = qA;
    sa.qIYR = qIYR;
    sa.kIYR = kIYR;
    sa.row_lse_out = opt ? opt->row_lse_out : nullptr;
    sa.col_lse_out = opt ? opt->col_lse_out : nullptr;
    sa.pos_logit_out = opt ? opt->pos_logit_out : nullptr;
    sa.negfrac = F(pl.o_negfrac);
    sa.kNegfrac = F(pl.o_kNegfrac);
    sa.qC = F(pl.o_qC);
    sa.qRho = F(pl.o_qRho);
    sa.qKap = F(pl.o_qKap);
    sa.kC = F(pl.o_kC);
    sa.kRho = F(pl.o_kRho);
    sa.kKap = F(pl.o_kKap);
    sa.diagA = F(pl.o_diagA);
    sa.lossparts = lossparts;
    float *const dscale_out = opt ? opt->dscale_out : nullptr, *const dbias_out = opt ? opt->dbias_out : nullptr;
    float *const biasparts = (!softmax && dbias_out) ? F(pl.o_bias) : nullptr;
    float *const tsum = dscale_out ? F(pl.o_tsum) : nullptr;
    sa.biasparts = biasparts;

    if (softmax) {
        LAUNCH_NAMED("k_fwd", launch_fwd(q, k, R, N, Di, pf, off, qA, invk, cshift, F(pl.o_rowpart),
                                         F(pl.o_colpart), posdot, s));
        sa.slot0 = 0;
        LAUNCH_NAMED("k_rowstats", launch_rowstats(sa, s));
        sa.slot0 = pl.slots_a;
        LAUNCH_NAMED("k_colstats", launch_colstats(sa, s));
    } else {
        sa.slot0 = 0;
        LAUNCH_NAMED("k_siglip_tabs", launch_siglip_tabs(sa, s));
    }
    float *gmax = F(pl.o_gmax);  // [4][P]: max q inv/sig, max k inv/sig, max row neg mass, max column neg mass
    LAUNCH_NAMED("k_maxes", launch_maxes(qIYR, kIYR, softmax ? sa.negfrac : nullptr,
                                         kind == kInfonce ? sa.kNegfrac : nullptr, R, N, R, N, P, gmax, s));

    auto pass = [&](bool rowpass, float *out) -> uform_status_t {
        BwdArgs ba{};
        ba.X16 = rowpass ? qH : kH;
        ba.Y16 = rowpass ? kH : qH;
        ba.oSig = rowpass ? sigq : sigk;
        ba.NO = rowpass ? R : N;
        ba.NI = rowpass ? N : R;
        ba.D = Di;
        ba.oA = rowpass ? qA : kA;
        ba.oC = rowpass ? sa.qC : sa.kC;
        ba.oRho = rowpass ? sa.qRho : sa.kRho;
        ba.iI = rowpass ? kIYR : qIYR;
        ba.iKap = rowpass ? sa.kKap : sa.qKap;
        ba.b2 = bias * kLog2e;
        ba.oInv = rowpass ? invq : invk;
        ba.iyrmax = gmax + (rowpass ? 1 : 0) * P;
        for (int i = 0; i < kMaxP; ++i) ba.wnorm[i] = wnorm[i];
        if (!softmax) {  // sigmoid: every cell is bounded by sigma(|s| + b)
            const float smax = 1.0f / (1.0f + std::exp(-(abs_s + bias)));
            ba.oNeg = nullptr;
            ba.gterm = nullptr;
            for (int i = 0; i < kMaxP; ++i) ba.gterm_val[i] = smax;
        } else if (kind == kInfonce) {  // row and column softmax terms
            ba.oNeg = rowpass ? sa.negfrac : sa.kNegfrac;
            ba.gterm = gmax + (rowpass ? 3 : 2) * P;
        } else if (rowpass) {  // rows: the row softmax only
            ba.oNeg = sa.negfrac;
            ba.gterm = nullptr;
        } else {  // rows, column pass: the inner rows' softmax only
            ba.oNeg = nullptr;
            ba.gterm = gmax + 2 * P;
        }
        if (npos >= 0) {  // listed cells leave the dense pass (the extra-positive pass takes them)
            ba.lptr = plist + (rowpass ? lw.lptr_r : lw.lptr_c);
            ba.lent = (const ListEnt *)(plist + (rowpass ? lw.ent_r : lw.ent_c));
        }
        ba.diag_shift = rowpass ? off : -off;
        ba.pxor = pxor;
        ba.blocks_per_split = rowpass ? pl.bps_row : pl.bps_col;
        ba.do_update = out != nullptr;
        ba.want_loss = (!softmax && rowpass) ? 1 : 0;
        ba.part = F(pl.o_part);
        ba.Cpart = F(pl.o_Cpart);
        ba.lossparts = lossparts;
        ba.loss_slot0 = pl.slots_a;
        ba.biasparts = biasparts;
        // the radial sums of the first gradient pass give dL/dscale
        float *const ts = (out && (rowpass || !dq)) ? tsum : nullptr;
        ba.tsum = ts;
        const int64_t nsplit = rowpass ? pl.nsplit_row : pl.nsplit_col;
        const bool fuse = out && nsplit == 1 && !pl.gen;  // one split: the compiled backward finishes the rows itself
        if (fuse) {
            ba.fin_out = out;
            ba.finX = rowpass ? q : k;
            ba.finY = rowpass ? k : q;
            ba.diagA = sa.diagA;
            ba.posdot = posdot;
            ba.invx = rowpass ? invq : invk;
            ba.gam = rowpass ? gamq : gamk;
            ba.R = R;
            ba.pos_shift = rowpass ? 0 : -off;
            ba.accumulate = (opt && (opt->flags & UFORM_CONTRASTIVE_ACCUMULATE)) ? 1 : 0;
        }
        if (pl.gen) {
            ba.pf = pf;
            ba.gt = make_gen_tabs(prefixes, P, pl.gen_nq);
            LAUNCH_NAMED("k_bwd_gen", launch_bwd_gen(ba, pl.gen_nq, !softmax, nsplit, s));
        } else {
            LAUNCH_NAMED("k_bwd", launch_bwd(ba, pl.mask, !softmax, nsplit, s));
        }
        if (out && !fuse) {
            FinArgs fa{};
            fa.X = rowpass ? q : k;
            fa.Y = rowpass ? k : q;
            fa.NO = ba.NO;
            fa.R = R;
            fa.D = Di;
            fa.pf = pf;
            fa.part = ba.part;
            fa.Cpart = ba.Cpart;
            fa.diagA = sa.diagA;
            fa.posdot = posdot;
            fa.invx = rowpass ? invq : invk;
            fa.gam = rowpass ? gamq : gamk;
            fa.nsplit = nsplit;
            fa.diag_shift = ba.diag_shift;
            fa.pxor = pxor;
            fa.pos_shift = rowpass ? 0 : -off;
            fa.accumulate = (opt && (opt->flags & UFORM_CONTRASTIVE_ACCUMULATE)) ? 1 : 0;
            fa.out = out;
            fa.tsum = ts;
            LAUNCH_NAMED("k_finalize", launch_finalize(fa, s));
        }
        return uform_status_success_k;
    };
    if (dq || !softmax) {
        uform_status_t st = pass(true, dq);
        if (st != uform_status_success_k) return st;
    }
    if (dk) {
        uform_status_t st = pass(false, dk);
        if (st != uform_status_success_k) return st;
    }
    int64_t pos_blocks = 0;
    if (npos >= 0) {
        // listed cells: loss and row gradients over the row lists, column gradients over the column lists
        PosArgs pa2{};
        pa2.D = Di;
        pa2.pf = pf;
        pa2.t = scale;
        pa2.b = bias;
        pa2.x = q;
        pa2.y = k;
        pa2.invx = invq;
        pa2.invy = invk;
        pa2.NO = R;
        pa2.NI = N;
        pa2.ptr = plist + lw.rows;
        pa2.idx = plist + lw.rows + R + 1;
        for (int i = 0; i < P; ++i) pa2.gc[i] = (float)(-(double)mirror * wnorm[i] * scale / den);
        pa2.out = dq;
        pa2.parts = F(pl.o_pparts);
        LAUNCH_NAMED("k_pos", launch_pos(pa2, s, &pos_blocks));
        if (dk) {
            pa2.x = k;
            pa2.y = q;
            pa2.invx = invk;
            pa2.invy = invq;
            pa2.NO = N;
            pa2.NI = R;
            pa2.ptr = clist;
            pa2.idx = clist + N + 1;
            for (int i = 0; i < P; ++i) pa2.gc[i] = (float)(-(double)wnorm[i] * scale / den);
            pa2.out = dk;
            pa2.parts = nullptr;
            LAUNCH_NAMED("k_pos", launch_pos(pa2, s, nullptr));
        }
    }

    LossArgs la{};
    la.pf = pf;
    la.lossparts = lossparts;
    la.nslots = pl.nslots;
    la.norm = 1.0 / den;
    for (int i = 0; i < kMaxP; ++i) la.wnorm[i] = wnorm[i];
    la.loss_out = loss_out;
    la.prefix_losses_out = opt ? opt->prefix_losses_out : nullptr;
    la.tsum = tsum;
    la.ntsum = dq ? R : N;
    la.inv_scale = 1.0f / (mirror * scale);  // the radial sums count both mirrored cells; dL/ds counts each once
    la.biasparts = biasparts;
    la.dscale_out = dscale_out;
    la.dbias_out = dbias_out;
    LAUNCH_NAMED("k_loss", launch_loss(la, s));
    if (npos >= 0) {
        PosFoldArgs fa{};
        fa.parts = F(pl.o_pparts);
        fa.nblk = pos_blocks;
        fa.pf = pf;
        fa.norm = 1.0 / den;
        for (int i = 0; i < kMaxP; ++i) fa.wnorm[i] = wnorm[i];
        fa.loss_out = loss_out;
        fa.prefix_losses_out = la.prefix_losses_out;
        fa.dscale_out = dscale_out;
        fa.dbias_out = dbias_out;
        LAUNCH_NAMED("k_pos_fold", launch_pos_fold(fa, s));
    }
    return uform_status_success_k;
}

}  // namespace

extern "C" {

uform_status_t uform_contrastive_fwd_bwd_ex(const void *q, const void *k, int64_t R, int64_t N, int64_t D,
                                            const int32_t *prefixes, int32_t n_prefixes, float scale, float bias,
                                            int32_t kind, float *loss_out, float *dq, float *dk, hipStream_t stream,
                                            const uform_contrastive_options_t *options) {
    uform_status_t st = validate(q, k, R, N, D, prefixes, n_prefixes, scale, bias, kind, loss_out, dq, dk, options);
    if (st != uform_status_success_k) return st;
    ProfCtx prof;
    prof.on = options && (options->flags & UFORM_CONTRASTIVE_PROFILE);
    prof.stream = stream;
    std::unique_lock<std::mutex> lock(g_prof_mu, std::defer_lock);
    if (prof.on) lock.lock();
    return run(q, k, R, N, D, prefixes, n_prefixes, scale, bias, kind, loss_out, dq, dk, stream, options, prof);
}

uform_status_t uform_contrastive_fwd_bwd_noalloc(const void *q, const void *k, int64_t R, int64_t N, int64_t D,
                                                 const int32_t *prefixes, int32_t n_prefixes, float scale, float bias,
                                                 int32_t kind, float *loss_out, float *dq, float *dk,
                                                 hipStream_t stream, const uform_contrastive_options_t *options) {
    uform_status_t st = validate(q, k, R, N, D, prefixes, n_prefixes, scale, bias, kind, loss_out, dq, dk, options);
    if (st != uform_status_success_k) return st;
    if (options && options->workspace)
        return fail(uform_status_invalid_argument_k,
                    "the allocation-free entry point uses its own scratch: pass workspace = NULL "
                    "(uform_contrastive_fwd_bwd_ex takes a caller workspace)");
    if (options && options->pos_row_ptr)
        return fail(uform_status_unsupported_k,
                    "the allocation-free entry point takes no positive lists (they are staged through pinned memory)");
    if (options && (options->flags & UFORM_CONTRASTIVE_PROFILE))
        return fail(uform_status_unsupported_k, "the allocation-free entry point does not profile (events are allocated)");
    const size_t need = call_plan(R, N, D, prefixes, n_prefixes, kind, dq, dk, options).total;
    if (need > (size_t)UFORM_CONTRASTIVE_NOALLOC_SCRATCH_BYTES)
        return fail(uform_status_unsupported_k,
                    "this call needs " + std::to_string(need) + " bytes of scratch; the allocation-free entry point holds " +
                        std::to_string((size_t)UFORM_CONTRASTIVE_NOALLOC_SCRATCH_BYTES) +
                        " (use uform_contrastive_fwd_bwd_ex with a workspace)");
    void *ptr = nullptr;
    st = scratch_address(&ptr);
    if (st != uform_status_success_k) return st;
    uform_contrastive_options_t opt{};
    if (options) opt = *options;
    opt.workspace = ptr;
    opt.workspace_bytes = (size_t)UFORM_CONTRASTIVE_NOALLOC_SCRATCH_BYTES;
    return run(q, k, R, N, D, prefixes, n_prefixes, scale, bias, kind, loss_out, dq, dk, stream, &opt, ProfCtx{});
}

int32_t uform_contrastive_profile(const char **names, float *ms, int32_t cap) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    std::vector<std::pair<const char *, float>> sums;
    for (const ProfRec &r : g_prof_live) {
        float t = 0.f;
        if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
            bool found = false;
            for (auto &kv : sums)
                if (std::strcmp(kv.first, r.name) == 0) {
                    kv.second += t;
                    found = true;
                }
            if (!found) sums.emplace_back(r.name, t);
        }
        g_prof_pool.push_back(r.a);
        g_prof_pool.push_back(r.b);
    }
    g_prof_live.clear();
    int32_t n = 0;
    for (auto &kv : sums) {
        if (n < cap) {
            if (names) names[n] = kv.first;
            if (ms) ms[n] = kv.second;
        }
        ++n;
    }
    return n;
}

uform_status_t uform_contrastive_fwd_bwd(const void *q, const void *k, int64_t R, int64_t N, int64_t D,
                                         const int32_t *prefixes, int32_t n_prefixes, float scale, float bias,
                                         int32_t kind, float *loss_out, float *dq, float *dk, hipStream_t stream) {
    return uform_contrastive_fwd_bwd_ex(q, k, R, N, D, prefixes, n_prefixes, scale, bias, kind, loss_out, dq, dk,
                                        stream, nullptr);
}

size_t uform_contrastive_workspace_bytes(int64_t R, int64_t N, int64_t D, int32_t n_prefixes, int32_t kind) {
    return uform_contrastive_workspace_bytes_ex(R, N, D, n_prefixes, kind, -1);
}

size_t uform_contrastive_workspace_bytes_ex(int64_t R, int64_t N, int64_t D, int32_t n_prefixes, int32_t kind,
                                            int64_t n_positives) {
    if (n_positives >= 0 && kind != kSiglip && kind != kOneset && kind != kOnesetEdges) return 0;
    if (R < 1 || N < 1 || R > N || D < 64 || D % 64 != 0 || D > kMaxD || n_prefixes < 1 || n_prefixes > kMaxP)
        return 0;
    if (kind < kInfonce || kind > kOnesetEdges) return 0;
    int32_t pw[kMaxP];
    for (int32_t i = 0; i < n_prefixes; ++i) pw[i] = (int32_t)(D - 32 * (n_prefixes - 1 - i));  // any ladder ending at D
    const int64_t npos = n_positives < 0 ? -1 : n_positives;
    // enough for either backward (the size depends on the ladder's count and width, not its steps)
    const bool oneset = kind == kOneset || kind == kOnesetEdges;
    size_t need = 0;
    for (int g = 0; g < 2; ++g) {
        const Plan pl = make_plan(R, N, D, pw, n_prefixes, oneset ? kSiglip : kind, 0, true, !oneset, false, npos, g);
        need = pl.total > need ? pl.total : need;
    }
    return need;
}

uform_status_t uform_contrastive_supported(int64_t D, const int32_t *prefixes, int32_t n_prefixes, int32_t kind,
                                          int32_t with_gradients) {
    g_last_error.clear();
    if (!prefixes || n_prefixes < 1 || n_prefixes > kMaxP)
        return fail(uform_status_invalid_argument_k, "prefixes must be a host array of 1..8 widths");
    if (kind < kInfonce || kind > kOnesetEdges) return fail(uform_status_invalid_argument_k, "unknown kind");
    for (int32_t i = 0; i < n_prefixes; ++i) {
        if (prefixes[i] < 32 || prefixes[i] % 32 != 0 || (i > 0 && prefixes[i] <= prefixes[i - 1]))
            return fail(uform_status_invalid_argument_k, "prefix widths must be increasing multiples of 32");
    }
    if (D < 1 || prefixes[n_prefixes - 1] > D) return fail(uform_status_invalid_argument_k, "the widest prefix exceeds D");
    if (D % 64 != 0 || D > kMaxD) return fail(uform_status_unsupported_k, "D must be a multiple of 64 and at most 2048");
    if ((with_gradients || kind == kSiglip || kind == kOneset || kind == kOnesetEdges) &&
        !bwd_compiled(D, prefixes, n_prefixes) && !bwd_generic_fits(prefixes, n_prefixes))
        return fail(uform_status_unsupported_k,
                    "this prefix ladder needs more snapshot slots or bands than the backward's LDS holds at this width");
    return uform_status_success_k;
}

const char *uform_status_name(uform_status_t status) {
    switch (status) {
        case uform_status_success_k: return "success";
        case uform_status_invalid_argument_k: return "invalid-argument";
        case uform_status_unsupported_k: return "unsupported";
        case uform_status_out_of_memory_k: return "out-of-memory";
        case uform_status_device_error_k: return "device-error";
    }
    return "unknown";
}

const char *uform_contrastive_last_error(void) { return g_last_error.c_str(); }

void uform_contrastive_release(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    for (auto &kv : g_cache) {
        if (kv.second.ptr) {
            (void)hipStreamSynchronize(kv.first.second);
            (void)hipFree(kv.second.ptr);
        }
    }
    g_cache.clear();
    for (auto &kv : g_staging) {
        if (kv.second.ev) {
            (void)hipEventSynchronize(kv.second.ev);
            (void)hipEventDestroy(kv.second.ev);
        }
        if (kv.second.host) (void)hipHostFree(kv.second.host);
    }
    g_staging.clear();
}

}  // extern "C"
