// Host runtime of the Muon step library: argument validation, same-shape
// grouping, workspace planning, descriptor upload and the launch sequence
// behind the C ABI declared in include/muon_step.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <map>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/muon_step.h"
#include "common.hpp"
#include "kernels.hpp"

using muon::Geom;
using muon::MatDesc;
using muon::Work;

namespace {

constexpr int64_t kMaxNsSteps = 64;
constexpr int64_t kMaxDim = int64_t(1) << 31;   // rows, cols
constexpr int64_t kMaxElems = int64_t(1) << 40; // rows * cols
// Groups whose smaller side is at most this run the fp32 Newton-Schulz
// products even when bf16 is requested: with so few singular directions the
// bf16 rounding of X does not average out, and their cost is negligible.
constexpr int64_t kThinF32Side = 16;
// Matrices one muon_step_noalloc call may take (its descriptor table is
// staged through a pinned buffer of this many entries, allocated at creation).
constexpr int64_t kNoAllocMaxMatrices = 16384;

bool use_bf16(int32_t precision, int64_t s) { return precision == MUON_NS_BF16 && s > kThinF32Side; }

void set_msg(char *msg, size_t cap, const char *fmt, ...) {
    if (!msg || cap == 0) return;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, cap, fmt, ap);
    va_end(ap);
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

bool finite(double v) { return std::isfinite(v); }

struct Interval {
    uintptr_t lo, hi;
    bool writable;
    int64_t owner;
    const char *what;
};

// Returns the index pair of the first conflicting overlap (a writable range
// overlapping any other range), or false.
bool find_overlap(std::vector<Interval> &iv, const Interval **a, const Interval **b) {
    std::sort(iv.begin(), iv.end(), [](const Interval &x, const Interval &y) { return x.lo < y.lo; });
    const Interval *max_all = nullptr, *max_w = nullptr;
    for (const Interval &cur : iv) {
        if (cur.writable && max_all && cur.lo < max_all->hi) { *a = max_all; *b = &cur; return true; }
        if (!cur.writable && max_w && cur.lo < max_w->hi) { *a = max_w; *b = &cur; return true; }
        if (!max_all || cur.hi > max_all->hi) max_all = &cur;
        if (cur.writable && (!max_w || cur.hi > max_w->hi)) max_w = &cur;
    }
    return false;
}

size_t dtype_size(int32_t dt) { return dt == MUON_BF16 ? 2 : 4; }

muon_status check_hparams(const muon_hparams *hp, char *msg, size_t cap) {
    if (!hp) { set_msg(msg, cap, "hparams is NULL"); return MUON_ERR_INVALID_ARGUMENT; }
    if (!finite(hp->lr) || !finite(hp->momentum) || !finite(hp->weight_decay) || !finite(hp->gamma)) {
        set_msg(msg, cap, "lr, momentum, weight_decay and gamma must be finite");
        return MUON_ERR_INVALID_ARGUMENT;
    }
    if (hp->num_ns_steps < 0 || hp->num_ns_steps > kMaxNsSteps) {
        set_msg(msg, cap, "num_ns_steps=%d outside [0, %lld]", hp->num_ns_steps, (long long)kMaxNsSteps);
        return MUON_ERR_INVALID_ARGUMENT;
    }
    if (hp->num_ns_steps > 0 && !hp->schedule) {
        set_msg(msg, cap, "schedule is NULL with num_ns_steps=%d", hp->num_ns_steps);
        return MUON_ERR_INVALID_ARGUMENT;
    }
    for (int i = 0; i < hp->num_ns_steps; ++i) {
        const muon_ns_coeff &c = hp->schedule[i];
        if (!finite(c.a) || !finite(c.b) || !finite(c.c)) {
            set_msg(msg, cap, "schedule[%d] has a non-finite coefficient", i);
            return MUON_ERR_INVALID_ARGUMENT;
        }
    }
    if (hp->nesterov != 0 && hp->nesterov != 1) {
        set_msg(msg, cap, "nesterov must be 0 or 1");
        return MUON_ERR_INVALID_ARGUMENT;
    }
    if (hp->ns_precision != MUON_NS_BF16 && hp->ns_precision != MUON_NS_F32) {
        set_msg(msg, cap, "unknown ns_precision %d", hp->ns_precision);
        return MUON_ERR_INVALID_ARGUMENT;
    }
    if (hp->scale_mode != MUON_SCALE_SQRT_MAX && hp->scale_mode != MUON_SCALE_UNIT_RMS) {
        set_msg(msg, cap, "unknown scale_mode %d", hp->scale_mode);
        return MUON_ERR_INVALID_ARGUMENT;
    }
    return MUON_OK;
}

muon_status check_shape(int64_t rows, int64_t cols, char *msg, size_t cap, int64_t idx) {
    if (rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim || rows * cols > kMaxElems) {
        set_msg(msg, cap, "matrix %lld: unsupported shape %lld x %lld", (long long)idx, (long long)rows,
                (long long)cols);
        return MUON_ERR_INVALID_ARGUMENT;
    }
    return MUON_OK;
}

muon_status check_step(const muon_matrix *mats, int64_t count, const muon_hparams *hp, char *msg, size_t cap) {
    if (count < 0) { set_msg(msg, cap, "count < 0"); return MUON_ERR_INVALID_ARGUMENT; }
    if (count > 0 && !mats) { set_msg(msg, cap, "mats is NULL"); return MUON_ERR_INVALID_ARGUMENT; }
    muon_status s = check_hparams(hp, msg, cap);
    if (s != MUON_OK) return s;
    std::vector<Interval> iv;
    iv.reserve(static_cast<size_t>(count) * 4);
    for (int64_t i = 0; i < count; ++i) {
        const muon_matrix &m = mats[i];
        if (!m.param || !m.grad || !m.momentum) {
            set_msg(msg, cap, "matrix %lld: param, grad and momentum must be non-NULL", (long long)i);
            return MUON_ERR_INVALID_ARGUMENT;
        }
        if ((m.param_dtype != MUON_F32 && m.param_dtype != MUON_BF16) ||
            (m.grad_dtype != MUON_F32 && m.grad_dtype != MUON_BF16)) {
            set_msg(msg, cap, "matrix %lld: unknown dtype", (long long)i);
            return MUON_ERR_INVALID_ARGUMENT;
        }
        s = check_shape(m.rows, m.cols, msg, cap, i);
        if (s != MUON_OK) return s;
        const uintptr_t n = static_cast<uintptr_t>(m.rows * m.cols);
        auto add = [&](const void *p, size_t es, bool wr, const char *what) {
            const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
            iv.push_back(Interval{lo, lo + n * es, wr, i, what});
        };
        add(m.param, dtype_size(m.param_dtype), true, "param");
        add(m.grad, dtype_size(m.grad_dtype), false, "grad");
        add(m.momentum, 4, true, "momentum");
        if (m.ns_out) add(m.ns_out, 4, true, "ns_out");
    }
    const Interval *a = nullptr, *b = nullptr;
    if (find_overlap(iv, &a, &b)) {
        set_msg(msg, cap, "memory of matrix %lld %s overlaps matrix %lld %s", (long long)a->owner, a->what,
                (long long)b->owner, b->what);
        return MUON_ERR_INVALID_ARGUMENT;
    }
    return MUON_OK;
}

muon_status check_adamw(const muon_adamw_tensor *ts, int64_t count, const muon_adamw_hparams *hp, char *msg,
                        size_t cap) {
    if (count < 0) { set_msg(msg, cap, "count < 0"); return MUON_ERR_INVALID_ARGUMENT; }
    if (count > 0 && !ts) { set_msg(msg, cap, "tensors is NULL"); return MUON_ERR_INVALID_ARGUMENT; }
    if (count > (int64_t(1) << 31) - 1) { set_msg(msg, cap, "too many tensors"); return MUON_ERR_INVALID_ARGUMENT; }
    if (!hp) { set_msg(msg, cap, "hparams is NULL"); return MUON_ERR_INVALID_ARGUMENT; }
    if (!finite(hp->lr) || !finite(hp->beta1) || !finite(hp->beta2) || !finite(hp->eps) ||
        !finite(hp->weight_decay)) {
        set_msg(msg, cap, "lr, beta1, beta2, eps and weight_decay must be finite");
        return MUON_ERR_INVALID_ARGUMENT;
    }
    if (hp->step < 1) { set_msg(msg, cap, "step must be >= 1"); return MUON_ERR_INVALID_ARGUMENT; }
    std::vector<Interval> iv;
    for (int64_t i = 0; i < count; ++i) {
        const muon_adamw_tensor &t = ts[i];
        if (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq) {
            set_msg(msg, cap, "tensor %lld: pointers must be non-NULL", (long long)i);
            return MUON_ERR_INVALID_ARGUMENT;
        }
        if (t.numel < 0 || t.numel > kMaxElems) {
            set_msg(msg, cap, "tensor %lld: numel %lld out of range", (long long)i, (long long)t.numel);
            return MUON_ERR_INVALID_ARGUMENT;
        }
        if ((t.param_dtype != MUON_F32 && t.param_dtype != MUON_BF16) ||
            (t.grad_dtype != MUON_F32 && t.grad_dtype != MUON_BF16)) {
            set_msg(msg, cap, "tensor %lld: unknown dtype", (long long)i);
            return MUON_ERR_INVALID_ARGUMENT;
        }
        if (t.param_dtype != MUON_F32 || t.grad_dtype != MUON_F32) {
            set_msg(msg, cap, "tensor %lld: AdamW supports fp32 param and grad only", (long long)i);
            return MUON_ERR_UNSUPPORTED;
        }
        const uintptr_t nb = static_cast<uintptr_t>(t.numel) * 4;
        auto add = [&](const void *p, bool wr, const char *what) {
            const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
            iv.push_back(Interval{lo, lo + nb, wr, i, what});
        };
        add(t.param, true, "param");
        add(t.grad, false, "grad");
        add(t.exp_avg, true, "exp_avg");
        add(t.exp_avg_sq, true, "exp_avg_sq");
    }
    const Interval *a = nullptr, *b = nullptr;
    if (find_overlap(iv, &a, &b)) {
        set_msg(msg, cap, "memory of tensor %lld %s overlaps tensor %lld %s", (long long)a->owner, a->what,
                (long long)b->owner, b->what);
        return MUON_ERR_INVALID_ARGUMENT;
    }
    return MUON_OK;
}

// ---------------------------------------------------------------- planning

Geom make_geom(int64_t rows, int64_t cols) {
    Geom g{};
    g.rows = rows;
    g.cols = cols;
    g.transposed = rows > cols ? 1 : 0;
    g.s = std::min(rows, cols);
    g.l = std::max(rows, cols);
    g.sp = round_up(g.s, muon::kTile);
    g.lp = round_up(g.l, muon::kTile);
    return g;
}

// Split-K of the bf16 Gram, A^2 and apply products of a group (all 1 on the fp32
// path).  The group's lower-triangle tiles, counted in the order (matrix,
// tile of the matrix) over all its matrices, from `from` on run with K split
// into ranges (gram / poly of them, of gram_units / poly_units x 128), their
// fp32 partial tiles (kpart(n) bytes in a chunk of n matrices) summed in range order
// by a reduce.  Depends only on the shape and the group size, so every
// chunking of a group (and muon_step_noalloc) splits the same tiles alike.
struct Splits {
    int gram = 1, gram_units = 0, poly = 1, poly_units = 0;
    int64_t from = 0;
    // a X + B X of the intermediate steps, over its own tiles (sp/256 x lp/256
    // per matrix, in ns_apply_kernel's order), from apply_from on
    int apply = 1, apply_units = 0;
    int64_t apply_from = 0;
    size_t per_matrix = 0;  // partial bytes per matrix of a chunk (every tile split)
    size_t fixed = 0;       // partial bytes of a chunk holding the split tail tiles
    size_t kpart(int64_t n) const { return per_matrix * static_cast<size_t>(n) + fixed; }
};

int64_t sym_tiles(const Geom &g) {
    const int64_t nt = g.sp / muon::kTile;
    return nt * (nt + 1) / 2;
}
int64_t apply_tiles(const Geom &g) { return (g.sp / muon::kTile) * (g.lp / muon::kTile); }

constexpr size_t kPartTileBytes = size_t(256) * 256 * 4;  // one fp32 partial tile
constexpr int64_t kCUs = 256;                              // workgroups in one wave (one per CU)

// Ranges for `count` tiles of K extent `units` x 128 that otherwise run as
// the last, partial wave of a launch (whole: as the whole launch).  Model in
// microseconds, from the kernels' measured rates: a 256 x 256 tile takes 3.5
// per 128 of K; a split piece adds 3 to start and 13 to store its fp32
// partial tile (a wave of 256 pieces moves 64 MB); the reduce costs 5 plus
// 0.055 per piece; splitting only the tail waits for the whole tiles' launch
// to drain (0.1 tile).  The S (at most max_splits, each range at least 512 of
// K) with the least time is taken if it saves a tenth of a tile (of the one
// wave when whole), else 1.  *ups receives the range length (x 128).
int tail_splits(int64_t count, int64_t units, int64_t max_splits, bool whole, int *ups) {
    const double tile = 3.5 * static_cast<double>(units);
    int best = 1;
    double best_t = 0.9 * tile;
    for (int64_t sp = 2; sp <= std::min<int64_t>(max_splits, units / 4); ++sp) {
        const int64_t u = (units + sp - 1) / sp;
        const int64_t real = (units + u - 1) / u;  // ranges actually used
        const double waves = static_cast<double>((count * real + kCUs - 1) / kCUs);
        const double t = waves * (tile / static_cast<double>(real) + 16.0) + 5.0 +
                         0.055 * static_cast<double>(count * real) + (whole ? 0.0 : 0.1 * tile);
        if (t < best_t) {
            best_t = t;
            best = static_cast<int>(real);
        }
    }
    *ups = static_cast<int>(best > 1 ? (units + best - 1) / best : units);
    return best;
}

Splits plan_splits(const Geom &g, bool bf16, int64_t group_n) {
    Splits sp;
    if (!bf16) return sp;
    // K extents of the loops (the true length rounded up to 128), in units of 128
    const int64_t gram_k = std::min(g.lp, round_up(g.l, 128)) / 128;
    const int64_t s_k = std::min(g.sp, round_up(g.s, 128)) / 128;  // A^2 and a X + B X
    // partial tiles take at most half of a matrix's own workspace: per matrix
    // when every tile of the group is split, in all when only the tail is; the
    // Gram, A^2 and apply partials share the space (their reduces run in turn)
    const size_t x = static_cast<size_t>(g.sp * g.lp), a = static_cast<size_t>(g.sp * g.sp);
    const int64_t max_pieces = static_cast<int64_t>((x * 5 + a * 4) / 2 / kPartTileBytes);
    // a group under half a wave splits every tile; a larger one only the tiles
    // of its last, partial wave
    auto plan = [&](int64_t tiles, int64_t *count, bool *whole, int64_t *max_splits) {
        const int64_t w = tiles * group_n;
        *whole = w < kCUs / 2;
        *count = *whole ? w : w % kCUs;
        *max_splits = *whole ? max_pieces / tiles : (*count > 0 ? max_pieces / *count : 0);
        return w;
    };
    int64_t count, max_splits;
    bool whole;
    const int64_t st = sym_tiles(g);
    const int64_t w = plan(st, &count, &whole, &max_splits);
    sp.from = w;
    if (count > 0 && max_splits >= 2) {
        sp.gram = tail_splits(count, gram_k, max_splits, whole, &sp.gram_units);
        sp.poly = tail_splits(count, s_k, max_splits, whole, &sp.poly_units);
        if (sp.gram > 1 || sp.poly > 1) {
            const size_t piece = static_cast<size_t>(std::max(sp.gram, sp.poly)) * kPartTileBytes;
            sp.from = w - count;
            if (whole)
                sp.per_matrix = static_cast<size_t>(st) * piece;
            else
                sp.fixed = static_cast<size_t>(count) * piece;
        }
    }
    const int64_t at = apply_tiles(g);
    const int64_t aw = plan(at, &count, &whole, &max_splits);
    sp.apply_from = aw;
    if (count > 0 && max_splits >= 2) {
        sp.apply = tail_splits(count, s_k, max_splits, whole, &sp.apply_units);
        if (sp.apply > 1) {
            const size_t piece = static_cast<size_t>(sp.apply) * kPartTileBytes;
            sp.apply_from = aw - count;
            if (whole)
                sp.per_matrix = std::max(sp.per_matrix, static_cast<size_t>(at) * piece);
            else
                sp.fixed = std::max(sp.fixed, static_cast<size_t>(count) * piece);
        }
    }
    return sp;
}

// One group: every matrix with the same (min, max) of its shape and the same
// dtypes.  The Newton-Schulz stages see only X (s x l), so both orientations
// of a shape share their launches; the momentum pass and the update, which
// touch W's layout, run once per orientation ("run").  members lists the
// matrices with rows <= cols first (n_flat of them), then those with
// rows > cols (X = W^T), each in call order.
struct GroupPlan {
    Geom g;                       // X geometry: rows = s, cols = l, untransposed
    bool bf16;                    // bf16 Newton-Schulz products for this group
    int32_t param_dtype, grad_dtype;
    std::vector<int64_t> members; // indices into the caller's list
    int64_t n_flat = 0;           // members with rows <= cols (a prefix)
    int64_t chunk = 0;            // matrices per chunk
    int bpm = 0;                  // stage-1 blocks per matrix (the larger of the two orientations)
    Splits splits;
};

// Geometry of W for a member of the group: rows <= cols (flat) or rows > cols.
Geom run_geom(const Geom &g, bool tall) { return tall ? make_geom(g.l, g.s) : make_geom(g.s, g.l); }

// Bytes of NS workspace one matrix of geometry g needs (without split-K partials).
size_t per_matrix_bytes(const Geom &g, bool bf16) {
    const size_t x = static_cast<size_t>(g.sp * g.lp), a = static_cast<size_t>(g.sp * g.sp);
    return bf16 ? (x * (2 + 2 + 1) + a * (2 + 2)) : (x * (4 + 4) + a * (4 + 4 + 4));
}

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

struct Layout {
    size_t xf0, xf1, xb0, xb1, xl, af, ab, bb, kp, total;
    bool has_xf, has_kp;
};

Layout chunk_layout(const Geom &g, bool bf16, int64_t n, size_t kpart_bytes) {
    const size_t x = static_cast<size_t>(g.sp * g.lp) * n, a = static_cast<size_t>(g.sp * g.sp) * n;
    Layout L{};
    size_t off = 0;
    if (bf16) {
        // X as hi (bf16, ping-pong) + its 8-bit residual lo (in place); no fp32 X
        // and no fp32 A (A lives in bf16 only).
        L.has_xf = false;
        L.xb0 = off; off = align_up(off + x * 2);
        L.xb1 = off; off = align_up(off + x * 2);
        L.xl = off; off = align_up(off + x * 1);
        L.af = 0;
        L.ab = off; off = align_up(off + a * 2);
        L.bb = off; off = align_up(off + a * 2);
    } else {
        L.has_xf = true;
        L.xf0 = off; off = align_up(off + x * 4);
        L.xf1 = off; off = align_up(off + x * 4);
        L.xb0 = L.xb1 = L.xl = 0;
        L.af = off; off = align_up(off + a * 4);
        L.ab = off; off = align_up(off + a * 4);
        L.bb = off; off = align_up(off + a * 4);
    }
    L.has_kp = kpart_bytes > 0;
    L.kp = off; off = align_up(off + kpart_bytes);
    L.total = off;
    return L;
}

muon_status plan_groups(const muon_matrix *mats, int64_t count, int32_t precision, size_t cap, std::vector<GroupPlan> *out,
                        size_t *ws_bytes, size_t *partial_count, int64_t *max_chunk, char *msg, size_t msg_cap) {
    std::map<std::tuple<int64_t, int64_t, int32_t, int32_t>, size_t> index;
    out->clear();
    std::vector<std::vector<int64_t>> tall;  // per group: members with rows > cols
    for (int64_t i = 0; i < count; ++i) {
        const int64_t s = std::min(mats[i].rows, mats[i].cols), l = std::max(mats[i].rows, mats[i].cols);
        const auto key = std::make_tuple(s, l, mats[i].param_dtype, mats[i].grad_dtype);
        auto it = index.find(key);
        size_t gi;
        if (it == index.end()) {
            GroupPlan gp;
            gp.g = make_geom(s, l);
            gp.bf16 = use_bf16(precision, s);
            gp.param_dtype = mats[i].param_dtype;
            gp.grad_dtype = mats[i].grad_dtype;
            gi = out->size();
            index.emplace(key, gi);
            out->push_back(gp);
            tall.emplace_back();
        } else {
            gi = it->second;
        }
        if (mats[i].rows > mats[i].cols)
            tall[gi].push_back(i);
        else
            (*out)[gi].members.push_back(i);
    }
    for (size_t gi = 0; gi < out->size(); ++gi) {
        GroupPlan &gp = (*out)[gi];
        gp.n_flat = static_cast<int64_t>(gp.members.size());
        gp.members.insert(gp.members.end(), tall[gi].begin(), tall[gi].end());
    }
    *ws_bytes = 0;
    *partial_count = 0;
    *max_chunk = 0;
    for (GroupPlan &gp : *out) {
        const bool bf16 = gp.bf16;
        const int64_t n_all = static_cast<int64_t>(gp.members.size());
        gp.splits = plan_splits(gp.g, bf16, n_all);
        const Splits &sm = gp.splits;
        const size_t per = per_matrix_bytes(gp.g, bf16) + sm.per_matrix;
        int64_t n = n_all;
        if (cap) {
            const size_t one = chunk_layout(gp.g, bf16, 1, sm.kpart(1)).total;
            if (one > cap) {
                set_msg(msg, msg_cap, "a %lld x %lld matrix needs %zu bytes of workspace, above the cap %zu",
                        (long long)gp.g.s, (long long)gp.g.l, one, cap);
                return MUON_ERR_OUT_OF_MEMORY;
            }
            n = std::min<int64_t>(n, std::max<int64_t>(1, static_cast<int64_t>((cap > sm.fixed ? cap - sm.fixed : 0) / per)));
            while (n > 1 && chunk_layout(gp.g, bf16, n, sm.kpart(n)).total > cap) --n;
        }
        // Keep every grouped launch inside a 32-bit grid.
        const int64_t apply_tiles = (gp.g.sp / muon::kTile) * (gp.g.lp / muon::kTile);
        n = std::min<int64_t>(n, std::max<int64_t>(1, ((int64_t(1) << 31) - 1) / apply_tiles));
        int tc = 0;
        gp.bpm = std::max(muon::nesterov_blocks_per_mat(run_geom(gp.g, false), &tc),
                          muon::nesterov_blocks_per_mat(run_geom(gp.g, true), &tc));
        n = std::min<int64_t>(n, std::max<int64_t>(1, ((int64_t(1) << 31) - 1) / gp.bpm));
        gp.chunk = n;
        *ws_bytes = std::max(*ws_bytes, chunk_layout(gp.g, bf16, n, sm.kpart(n)).total);
        *partial_count = std::max(*partial_count, static_cast<size_t>(n) * gp.bpm);
        *max_chunk = std::max(*max_chunk, n);
    }
    return MUON_OK;
}

}  // namespace

// ------------------------------------------------------------------ context

struct DevBuf {
    void *p = nullptr;
    size_t n = 0;
};

struct muon_context {
    int device = 0;
    size_t cap = 0;
    std::string err;
    DevBuf ws;        // Newton-Schulz workspace
    DevBuf tabs;      // partials | nrm2 | inv_norm
    DevBuf call_nrm2; // per call matrix
    DevBuf mat_desc;  // MatDesc table
    DevBuf adamw_desc;
    void *pinned = nullptr;
    size_t pinned_n = 0;
    hipEvent_t upload_done = nullptr;
    bool upload_recorded = false;
    std::vector<unsigned char> mat_cache, adamw_cache;
    hipStream_t last_stream = nullptr;
    int64_t last_count = 0;
    const double *last_nrm2 = nullptr;  // device: the last step's per-matrix ||N||^2
    // allocation-free step: this device's copy of the static scratch (from
    // hipGetSymbolAddress at creation; nullptr if that failed, with the reason
    // kept in scratch_err) and a pinned staging buffer for its descriptor
    // table, both set up by muon_create
    char *scratch = nullptr;
    std::string scratch_err;
    void *noalloc_pinned = nullptr;
    hipEvent_t noalloc_upload_done = nullptr;
    bool noalloc_upload_recorded = false;
    // concurrent groups: side streams (default priority) forked from the
    // caller's stream and joined back to it, created on first use
    static constexpr int kSide = 3;
    hipStream_t side[kSide] = {};
    hipEvent_t fork_ev = nullptr, join_ev[kSide] = {};
    bool concurrent = true;
    // per-stage timing
    bool prof_on = false;
    std::vector<hipEvent_t> ev_pool;
    size_t ev_used = 0;
    struct Rec {
        int stage;
        hipEvent_t a, b;
        double flops, bytes;
    };
    std::vector<Rec> recs;
};

namespace {

struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) (void)hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

muon_status fail(muon_context *ctx, muon_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    ctx->err = buf;
    return st;
}

muon_status hip_fail(muon_context *ctx, hipError_t e, const char *where) {
    return fail(ctx, MUON_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

enum Stage {
    ST_MOMENTUM = 0, ST_FINALIZE, ST_NORMALIZE, ST_GRAM, ST_POLY, ST_APPLY, ST_APPLY_UPDATE, ST_UPDATE,
    ST_ADAMW, ST_IMPORT, ST_EXPORT, ST_UNIT_RMS, ST_PRENORM, ST_PROBE, ST_COUNT
};
const char *const kStageNames[ST_COUNT] = {"momentum_nesterov", "norm_finalize", "normalize", "gram", "poly",
                                           "apply", "apply_update", "update", "adamw", "import", "export",
                                           "unit_rms", "prenormalize", "stream_probe"};

hipError_t take_event(muon_context *ctx, hipEvent_t *ev) {
    if (ctx->ev_used == ctx->ev_pool.size()) {
        hipEvent_t e = nullptr;
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return err;
        ctx->ev_pool.push_back(e);
    }
    *ev = ctx->ev_pool[ctx->ev_used++];
    return hipSuccess;
}

// Launches through `fn` (returns hipError_t); with timing enabled the launch
// is bracketed by two events on stream st and its algorithmic work recorded.
template <class F>
hipError_t timed(muon_context *ctx, int stage, double flops, double bytes, hipStream_t st, F fn) {
    if (!ctx->prof_on) return fn();
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = take_event(ctx, &a);
    if (e == hipSuccess) e = take_event(ctx, &b);
    if (e == hipSuccess) e = hipEventRecord(a, st);
    if (e != hipSuccess) return e;
    e = fn();
    if (e != hipSuccess) return e;
    e = hipEventRecord(b, st);
    if (e != hipSuccess) return e;
    ctx->recs.push_back(muon_context::Rec{stage, a, b, flops, bytes});
    return hipSuccess;
}

// Grows a device buffer to at least n bytes.  Outstanding work may still use
// the old buffer, so the device is synchronised before it is freed.
muon_status ensure(muon_context *ctx, DevBuf &b, size_t n, const char *what) {
    if (b.n >= n && b.p) return MUON_OK;
    if (b.p) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(ctx, e, "hipDeviceSynchronize");
        (void)hipFree(b.p);
        b.p = nullptr;
        b.n = 0;
    }
    const size_t want = std::max<size_t>(n, 256);
    hipError_t e = hipMalloc(&b.p, want);
    if (e != hipSuccess) {
        b.p = nullptr;
        (void)hipGetLastError();
        return fail(ctx, MUON_ERR_OUT_OF_MEMORY, "hipMalloc of %zu bytes for %s failed", want, what);
    }
    b.n = want;
    return MUON_OK;
}

// Uploads a host table to a device buffer through pinned staging, skipping the
// copy when the bytes equal the previous upload of the same table.
muon_status upload(muon_context *ctx, DevBuf &dst, std::vector<unsigned char> &cache, const void *src, size_t n,
                   hipStream_t st, const char *what) {
    if (n == 0) return MUON_OK;
    if (cache.size() == n && dst.p && dst.n >= n && std::memcmp(cache.data(), src, n) == 0) return MUON_OK;
    muon_status s = ensure(ctx, dst, n, what);
    if (s != MUON_OK) return s;
    hipError_t e;
    if (ctx->upload_recorded) {
        e = hipEventSynchronize(ctx->upload_done);  // the staging buffer is free again
        if (e != hipSuccess) return hip_fail(ctx, e, "hipEventSynchronize");
    }
    if (ctx->pinned_n < n) {
        if (ctx->pinned) (void)hipHostFree(ctx->pinned);
        ctx->pinned = nullptr;
        ctx->pinned_n = 0;
        const size_t want = std::max<size_t>(n, 4096);
        e = hipHostMalloc(&ctx->pinned, want, hipHostMallocDefault);
        if (e != hipSuccess) {
            ctx->pinned = nullptr;
            return fail(ctx, MUON_ERR_OUT_OF_MEMORY, "hipHostMalloc of %zu bytes failed", want);
        }
        ctx->pinned_n = want;
    }
    std::memcpy(ctx->pinned, src, n);
    e = hipMemcpyAsync(dst.p, ctx->pinned, n, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpyAsync");
    e = hipEventRecord(ctx->upload_done, st);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipEventRecord");
    ctx->upload_recorded = true;
    cache.assign(static_cast<const unsigned char *>(src), static_cast<const unsigned char *>(src) + n);
    return MUON_OK;
}

void muon_scalars(const muon_hparams *hp, int64_t rows, int64_t cols, float *d, float *s) {
    *d = static_cast<float>(1.0 - hp->lr * hp->weight_decay);
    *s = static_cast<float>(hp->lr * hp->gamma * std::sqrt(static_cast<double>(std::max(rows, cols))));
}

// Device memory of one muon_step call: the Newton-Schulz workspace, the norm
// tables (partials | nrm2 | inv_norm) and the per-call norm output.  Either
// the context's own buffers or the fixed scratch of the allocation-free step.
struct CallMem {
    char *ws;
    char *tabs;
    double *call_nrm2;
};

// Work view of a chunk laid out at the workspace base.
Work chunk_work(const CallMem &mem, const Geom &g, bool bf16, int64_t n, int bpm, size_t kpart_bytes) {
    const Layout L = chunk_layout(g, bf16, n, kpart_bytes);
    char *base = mem.ws;
    Work w{};
    w.xf = L.has_xf ? reinterpret_cast<float *>(base + L.xf0) : nullptr;
    w.xf_next = L.has_xf ? reinterpret_cast<float *>(base + L.xf1) : nullptr;
    w.xb = bf16 ? static_cast<void *>(base + L.xb0) : nullptr;
    w.xb_next = bf16 ? static_cast<void *>(base + L.xb1) : nullptr;
    w.xl = bf16 ? static_cast<void *>(base + L.xl) : nullptr;
    w.af = bf16 ? nullptr : reinterpret_cast<float *>(base + L.af);
    w.ab = base + L.ab;
    w.bb = base + L.bb;
    w.x_stride = g.sp * g.lp;
    w.a_stride = g.sp * g.sp;
    char *t = mem.tabs;
    w.partials = reinterpret_cast<double *>(t);
    const size_t np = align_up(static_cast<size_t>(n) * bpm * sizeof(double));
    w.nrm2 = reinterpret_cast<double *>(t + np);
    w.inv_norm = reinterpret_cast<float *>(t + np + align_up(static_cast<size_t>(n) * sizeof(double)));
    w.call_nrm2 = mem.call_nrm2;
    w.kpart = L.has_kp ? reinterpret_cast<float *>(base + L.kp) : nullptr;
    return w;
}

// The view of matrices k, k+1, ... of a chunk (a run of one orientation):
// per-matrix workspace and tables shifted by k, stage-1 partial sums by
// partial_off.
Work offset_work(const Work &w, int64_t k, bool bf16, int64_t partial_off) {
    Work o = w;
    const int64_t xo = k * w.x_stride, ao = k * w.a_stride;
    if (o.xf) o.xf += xo;
    if (o.xf_next) o.xf_next += xo;
    if (o.xb) o.xb = static_cast<uint16_t *>(o.xb) + xo;
    if (o.xb_next) o.xb_next = static_cast<uint16_t *>(o.xb_next) + xo;
    if (o.xl) o.xl = static_cast<uint8_t *>(o.xl) + xo;
    if (o.af) o.af += ao;
    o.ab = static_cast<char *>(o.ab) + ao * (bf16 ? 2 : 4);
    o.bb = static_cast<char *>(o.bb) + ao * (bf16 ? 2 : 4);
    o.partials += partial_off;
    o.nrm2 += k;
    o.inv_norm += k;
    if (o.uscale) o.uscale += k;
    o.kpart = nullptr;
    return o;
}

// Matrices [k0, k0 + n) of a chunk that share W's orientation, g their W
// geometry (transposed when rows > cols).
struct Run {
    int64_t k0, n;
    Geom g;
};

size_t tabs_bytes(size_t partials, int64_t max_chunk) {
    return align_up(partials * sizeof(double)) + align_up(static_cast<size_t>(max_chunk) * sizeof(double)) +
           align_up(static_cast<size_t>(max_chunk) * sizeof(float));
}

// Algorithmic work of one Newton-Schulz stage over n matrices of geometry g:
// FLOPs counting one triangle of the symmetric products, and the bytes a
// kernel must move at least once (operands, X for the aX term, outputs).
void ns_work(int stage, const Geom &g, bool bf16, int n, bool ns_out, int psize, double *flops, double *bytes) {
    const double s = static_cast<double>(g.s), l = static_cast<double>(g.l), es = bf16 ? 2.0 : 4.0;
    switch (stage) {
        case ST_GRAM:
            // X read; A written (fp32 path: lower triangle in fp32 plus the operand copy)
            *flops = l * s * (s + 1);
            *bytes = s * l * es + (bf16 ? 0.0 : s * (s + 1) / 2 * 4) + s * s * es;
            break;
        case ST_POLY:
            *flops = s * s * (s + 1);
            *bytes = s * s * es + (bf16 ? 0.0 : s * (s + 1) / 2 * 4) + s * s * es;
            break;
        case ST_APPLY:
            // B, X operand, then X_lo in and (X_hi, X_lo) out (2 + 1 bytes); fp32 path: X in, X out
            *flops = 2 * s * s * l;
            *bytes = s * s * es + s * l * es + (bf16 ? s * l * 4 : s * l * 8);
            break;
        default:  // ST_APPLY_UPDATE
            *flops = 2 * s * s * l;
            *bytes = s * s * es + s * l * es + s * l * (bf16 ? 1 : 4) + s * l * 2.0 * psize + (ns_out ? s * l * 4 : 0);
            break;
    }
    *flops *= n;
    *bytes *= n;
}

// Runs normalisation + the NS schedule (+ the decay and update when
// `update`) on one chunk whose first stage already wrote X = N and the norms.
// gx is X's geometry (s x l); runs[] split the chunk into its matrices with
// rows <= cols and those with rows > cols (W = X^T), runs[k].g being W's
// geometry.  The products see only X, so one launch per stage covers both
// runs; a chunk of one run may fuse the update into the last product, a
// chunk of two runs updates each run in a pass of its own.  Returns the
// workspace view holding the final X in xf (fp32 path) or xb + xl (bf16
// path), meaningful when !update.  In the unit-RMS scale mode the last step
// writes X like the others; ||X||^2 per matrix is then reduced (partial_bpm
// partial sums per matrix fit in w.partials) into a per-matrix scale, and a
// separate pass applies the decay + update.
muon_status run_ns(muon_context *ctx, const MatDesc *descs, int nmat, const Geom &gx, Work &w, bool bf16,
                   const muon_hparams *hp, bool update, int param_bf16, bool any_ns_out, float d, float s,
                   hipStream_t st, const Splits &sp, const Run *runs, int nruns, int64_t chunk_m0 = 0,
                   bool params_aligned16 = false, int partial_bpm = 0, bool outs_aligned16 = false) {
    const bool unit_rms = update && hp->scale_mode == MUON_SCALE_UNIT_RMS;
    // the geometry the product launches see: W's own for a chunk of one run (the
    // fused update needs its orientation), X's otherwise
    const Geom &g = nruns == 1 ? runs[0].g : gx;
    // bf16 parameters whose tiles allow staging W through LDS keep the update
    // fused into the last product.  Other shapes whose W rows allow 8-wide
    // access run the last step as a plain product plus a separate update
    // pass, which costs less than the per-element fused epilogue there, and
    // so does a chunk of both orientations.
    const bool w_staged = nruns == 1 && param_bf16 && params_aligned16 && outs_aligned16 && !g.transposed &&
                          g.s % muon::kTile == 0 && g.l % muon::kTile == 0;
    const bool split_update =
        update && !unit_rms &&
        (nruns > 1 || (bf16 && !w_staged && params_aligned16 && outs_aligned16 &&
                       (g.transposed ? g.cols % 8 == 0 : g.l % 8 == 0)));
    const double xe = static_cast<double>(g.s) * g.l * nmat;
    // bf16 path with a schedule: X stays N and the first step applies 1/||N||
    // (only the padding needs zeros), except for the matrices whose norm lies
    // outside the fold range, which a pre-normalisation pass scales first
    // (its blocks return at once for the others); otherwise a normalisation
    // pass over every matrix.
    const bool fold = bf16 && hp->num_ns_steps > 0;
    hipError_t e = hipSuccess;
    if (!fold) {
        e = timed(ctx, ST_NORMALIZE, 0.0, xe * (bf16 ? 6.0 : 8.0), st,
                  [&] { return muon::launch_normalize(nmat, g, w, 0, st); });
    } else {
        if (g.sp > g.s || g.lp > g.l) {
            const double pad = (static_cast<double>(g.sp) * g.lp - static_cast<double>(g.s) * g.l) * nmat;
            e = timed(ctx, ST_NORMALIZE, 0.0, pad * 3.0, st, [&] { return muon::launch_pad_zero(nmat, g, w, st); });
        }
        // no algorithmic bytes: only matrices with an extreme norm are touched
        if (e == hipSuccess)
            e = timed(ctx, ST_PRENORM, 0.0, 0.0, st, [&] { return muon::launch_normalize(nmat, g, w, 1, st); });
    }
    if (e != hipSuccess) return hip_fail(ctx, e, "normalize launch");
    const int psize = param_bf16 ? 2 : 4;
    for (int it = 0; it < hp->num_ns_steps; ++it) {
        muon::NsStep p{};
        p.a = static_cast<float>(hp->schedule[it].a);
        p.b = static_cast<float>(hp->schedule[it].b);
        p.c = static_cast<float>(hp->schedule[it].c);
        p.final_update = (update && !unit_rms && !split_update && it == hp->num_ns_steps - 1) ? 1 : 0;
        p.param_bf16 = param_bf16;
        p.dscale = d;
        p.sscale = s;
        p.unnormalized = (fold && it == 0) ? 1 : 0;
        p.w_staged = w_staged ? 1 : 0;
        p.vec_ok = params_aligned16 && outs_aligned16 ? 1 : 0;
        p.gram_splits = sp.gram;
        p.gram_units = sp.gram_units;
        p.poly_splits = sp.poly;
        p.poly_units = sp.poly_units;
        // the group's first split tiles, counted from the chunk's first matrix
        // chunk_m0 (the launches clamp them to the chunk)
        p.split_from = sp.from - chunk_m0 * sym_tiles(g);
        p.apply_splits = sp.apply;
        p.apply_units = sp.apply_units;
        p.apply_split_from = sp.apply_from - chunk_m0 * apply_tiles(g);
        for (int kind = 0; kind < 3; ++kind) {
            const int stage = kind == 0 ? ST_GRAM : kind == 1 ? ST_POLY : (p.final_update ? ST_APPLY_UPDATE : ST_APPLY);
            double fl = 0, by = 0;
            ns_work(stage, g, bf16, nmat, any_ns_out, psize, &fl, &by);
            e = timed(ctx, stage, fl, by, st,
                      [&] { return muon::launch_ns_stage(kind, bf16, descs, nmat, g, w, p, st); });
            if (e != hipSuccess) return hip_fail(ctx, e, "Newton-Schulz launch");
        }
        std::swap(w.xf, w.xf_next);
        std::swap(w.xb, w.xb_next);
    }
    if (unit_rms) {
        const int nbx = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(partial_bpm, g.s)));
        const double gsq = hp->gamma * std::sqrt(static_cast<double>(g.rows) * static_cast<double>(g.cols));
        e = timed(ctx, ST_UNIT_RMS, 0.0, xe * (bf16 ? 3.0 : 4.0), st, [&] {
            return muon::launch_unit_rms_scale(nmat, g, w, nullptr, nbx, hp->lr, gsq, w.inv_norm, st);
        });
        if (e != hipSuccess) return hip_fail(ctx, e, "unit-RMS norm launch");
        w.uscale = w.inv_norm;
    }
    if (update && (hp->num_ns_steps == 0 || unit_rms || split_update)) {
        for (int r = 0; r < nruns; ++r) {
            const Run &run = runs[r];
            const Work wr = offset_work(w, run.k0, bf16, 0);
            const double by = static_cast<double>(g.s) * g.l * run.n *
                              ((bf16 ? 3.0 : 4.0) + 2.0 * psize + (any_ns_out ? 4.0 : 0.0));
            e = timed(ctx, ST_UPDATE, 0.0, by, st, [&] {
                return muon::launch_update_from_work(descs + run.k0, static_cast<int>(run.n), run.g, wr, param_bf16,
                                                     d, s, params_aligned16 && outs_aligned16, st);
            });
            if (e != hipSuccess) return hip_fail(ctx, e, "update launch");
        }
    }
    return MUON_OK;
}

// Concurrent groups.  Groups share only the descriptor table and the
// per-call norms, so they may run at the same time: lane 0 is the caller's
// stream, lanes 1.. side streams forked from it and joined back to it.  A
// group too small to fill the chip, or the last partial wave of a group's
// launch, then leaves CUs that another group's work takes.  A large group
// (an apply launch of 8 waves of the chip or more) has few such CUs and
// loses L2 locality when another large group shares the chip (the
// 2048 x 7168 batch split in two concurrent halves runs 3% slower), so the
// large groups run in turn on lane 0 and only the others go to side lanes,
// longest first (by Newton-Schulz FLOPs) onto the least loaded lane (lane 0
// too when no group is large).  A lane runs its groups in turn in a slice
// of the workspace (ws_off) and of the norm tables (tb_off) of its own,
// sized for its largest chunk.  One lane (every group in turn on the
// caller's stream, in one shared slice) when fewer than two groups are
// left to share the chip, or when the slices side by side exceed a nonzero
// cap.
struct Lanes {
    int n = 1;
    std::vector<int> lane_of;          // per group
    std::vector<size_t> ws_off{0, 0};  // lane l's workspace slice: [ws_off[l], ws_off[l + 1])
    std::vector<size_t> tb_off{0, 0};  // lane l's norm-table slice
};

Lanes plan_lanes(const std::vector<GroupPlan> &plan, int max_lanes, size_t cap) {
    Lanes L;
    const size_t ng = plan.size();
    L.lane_of.assign(ng, 0);
    if (ng < 2 || max_lanes < 2) return L;
    auto work = [&](size_t i) {
        const double sd = static_cast<double>(plan[i].g.s), ld = static_cast<double>(plan[i].g.l);
        return static_cast<double>(plan[i].members.size()) * (3.0 * ld * sd * sd + sd * sd * sd);
    };
    auto large = [&](size_t i) {
        return apply_tiles(plan[i].g) * static_cast<int64_t>(plan[i].members.size()) >= 8 * kCUs;
    };
    std::vector<size_t> order;
    bool any_large = false;
    for (size_t i = 0; i < ng; ++i) {
        if (large(i))
            any_large = true;  // lane 0
        else
            order.push_back(i);
    }
    // lane 0 for the large groups (if any), one more per remaining group
    const int n = static_cast<int>(std::min<size_t>(order.size() + (any_large ? 1 : 0), static_cast<size_t>(max_lanes)));
    if (order.empty() || n < 2) return L;
    std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return work(a) > work(b); });
    std::vector<double> load(static_cast<size_t>(n), 0.0);
    if (any_large) load[0] = std::numeric_limits<double>::infinity();
    for (size_t i : order) {
        const size_t l = static_cast<size_t>(std::min_element(load.begin(), load.end()) - load.begin());
        L.lane_of[i] = static_cast<int>(l);
        load[l] += work(i);
    }
    std::vector<size_t> lws(static_cast<size_t>(n), 0), ltb(static_cast<size_t>(n), 0);
    for (size_t i = 0; i < ng; ++i) {
        const GroupPlan &gp = plan[i];
        const size_t l = static_cast<size_t>(L.lane_of[i]);
        lws[l] = std::max(lws[l], chunk_layout(gp.g, gp.bf16, gp.chunk, gp.splits.kpart(gp.chunk)).total);
        ltb[l] = std::max(ltb[l], align_up(tabs_bytes(static_cast<size_t>(gp.chunk) * gp.bpm, gp.chunk)));
    }
    L.ws_off.assign(static_cast<size_t>(n) + 1, 0);
    L.tb_off.assign(static_cast<size_t>(n) + 1, 0);
    for (size_t l = 0; l < static_cast<size_t>(n); ++l) {
        L.ws_off[l + 1] = L.ws_off[l] + align_up(lws[l]);
        L.tb_off[l + 1] = L.tb_off[l] + ltb[l];
    }
    if (cap && L.ws_off.back() > cap) return Lanes{1, std::vector<int>(ng, 0)};
    L.n = n;
    return L;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Copies the descriptor table into the fixed scratch through the context's
// pinned staging buffer (allocated by muon_create), once the previous copy
// from it has been consumed.  Nothing is allocated.
muon_status upload_fixed(muon_context *ctx, void *dst, const void *src, size_t n, hipStream_t st) {
    hipError_t e;
    if (ctx->noalloc_upload_recorded) {
        e = hipEventSynchronize(ctx->noalloc_upload_done);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipEventSynchronize");
    }
    std::memcpy(ctx->noalloc_pinned, src, n);
    e = hipMemcpyAsync(dst, ctx->noalloc_pinned, n, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpyAsync");
    e = hipEventRecord(ctx->noalloc_upload_done, st);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipEventRecord");
    ctx->noalloc_upload_recorded = true;
    return MUON_OK;
}

// muon_step and muon_step_noalloc.  fixed: every buffer of the call lives in
// the device's static scratch (descriptor table | per-call norms | norm tables
// | workspace), the groups are chunked to fit it, and nothing is allocated;
// otherwise the context's grow-only buffers are used.
muon_status step_impl(muon_context *ctx, const muon_matrix *mats, int64_t count, const muon_hparams *hp,
                      void *hip_stream, bool fixed) {
    if (!ctx) return MUON_ERR_INVALID_ARGUMENT;
    char msg[512];
    muon_status s = check_step(mats, count, hp, msg, sizeof msg);
    if (s != MUON_OK) return fail(ctx, s, "%s", msg);
    if (count == 0) { ctx->err.clear(); return MUON_OK; }
    std::vector<GroupPlan> plan;
    size_t ws = 0, parts = 0;
    int64_t max_chunk = 0;
    CallMem mem{};
    MatDesc *desc_dst = nullptr;
    if (!fixed) {
        s = plan_groups(mats, count, hp->ns_precision, ctx->cap, &plan, &ws, &parts, &max_chunk, msg, sizeof msg);
        if (s != MUON_OK) return fail(ctx, s, "%s", msg);
    } else {
        if (!ctx->scratch || !ctx->noalloc_pinned)
            return fail(ctx, MUON_ERR_DEVICE, "the fixed scratch is not available: %s", ctx->scratch_err.c_str());
        if (count > kNoAllocMaxMatrices)
            return fail(ctx, MUON_ERR_OUT_OF_MEMORY, "muon_step_noalloc takes at most %lld matrices per call, got %lld",
                        (long long)kNoAllocMaxMatrices, (long long)count);
        const size_t desc_b = align_up(static_cast<size_t>(count) * sizeof(MatDesc));
        const size_t head = desc_b + align_up(static_cast<size_t>(count) * sizeof(double));
        const size_t room = muon::kScratchBytes - head;
        size_t cap = room;
        for (int tries = 0;; ++tries) {
            s = plan_groups(mats, count, hp->ns_precision, cap, &plan, &ws, &parts, &max_chunk, msg, sizeof msg);
            if (s != MUON_OK)
                return fail(ctx, s, "muon_step_noalloc: %s (the fixed scratch holds %zu bytes)", msg,
                            static_cast<size_t>(muon::kScratchBytes));
            const size_t tb = align_up(tabs_bytes(parts, max_chunk));
            if (ws + tb <= room) {
                mem.call_nrm2 = reinterpret_cast<double *>(ctx->scratch + desc_b);
                mem.tabs = ctx->scratch + head;
                mem.ws = ctx->scratch + head + tb;
                break;
            }
            if (tries == 3 || tb >= room)
                return fail(ctx, MUON_ERR_OUT_OF_MEMORY,
                            "muon_step_noalloc: the call needs %zu bytes, the fixed scratch holds %zu", head + ws + tb,
                            static_cast<size_t>(muon::kScratchBytes));
            cap = room - tb;
        }
        desc_dst = reinterpret_cast<MatDesc *>(ctx->scratch);
    }
    DeviceGuard guard(ctx->device);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    // groups on concurrent lanes (plan_lanes), except in the allocation-free
    // step and under per-stage timing, which run them in turn
    Lanes lanes;
    if (!fixed && !ctx->prof_on && ctx->concurrent) {
        lanes = plan_lanes(plan, 1 + muon_context::kSide, ctx->cap);
        // the side streams and the fork / join events, made once per context
        for (int i = 0; lanes.n > 1 && i < lanes.n - 1; ++i) {
            hipError_t e = hipSuccess;
            if (!ctx->side[i]) e = hipStreamCreateWithFlags(&ctx->side[i], hipStreamNonBlocking);
            if (e == hipSuccess && !ctx->join_ev[i])
                e = hipEventCreateWithFlags(&ctx->join_ev[i], hipEventDisableTiming);
            if (e == hipSuccess && !ctx->fork_ev) e = hipEventCreateWithFlags(&ctx->fork_ev, hipEventDisableTiming);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                lanes = Lanes{};
            }
        }
    }
    if (lanes.n == 1) lanes.lane_of.assign(plan.size(), 0);
    const int nlanes = lanes.n;
    const size_t tabs_total = nlanes > 1 ? lanes.tb_off.back() : tabs_bytes(parts, max_chunk);
    if (nlanes > 1) ws = lanes.ws_off.back();
    if (!fixed) {
        if ((s = ensure(ctx, ctx->ws, ws, "workspace")) != MUON_OK) return s;
        if ((s = ensure(ctx, ctx->tabs, tabs_total, "norm tables")) != MUON_OK) return s;
        if ((s = ensure(ctx, ctx->call_nrm2, static_cast<size_t>(count) * sizeof(double), "norm output")) != MUON_OK)
            return s;
        mem = CallMem{static_cast<char *>(ctx->ws.p), static_cast<char *>(ctx->tabs.p),
                      static_cast<double *>(ctx->call_nrm2.p)};
    }
    // Descriptor table in group order: every chunk is a contiguous slice.
    std::vector<MatDesc> descs;
    descs.reserve(static_cast<size_t>(count));
    for (const GroupPlan &gp : plan)
        for (int64_t i : gp.members) {
            MatDesc d{};
            d.param = mats[i].param;
            d.grad = mats[i].grad;
            d.mom = mats[i].momentum;
            d.ns_out = mats[i].ns_out;
            d.call_index = i;
            descs.push_back(d);
        }
    const size_t desc_bytes = descs.size() * sizeof(MatDesc);
    if (fixed) {
        s = upload_fixed(ctx, desc_dst, descs.data(), desc_bytes, st);
        if (s != MUON_OK) return s;
    } else {
        s = upload(ctx, ctx->mat_desc, ctx->mat_cache, descs.data(), desc_bytes, st, "matrix descriptors");
        if (s != MUON_OK) return s;
        desc_dst = static_cast<MatDesc *>(ctx->mat_desc.p);
    }
    const MatDesc *ddev = desc_dst;
    const float mu = static_cast<float>(hp->momentum);
    // one group, on stream st, in the workspace and tables of `gm`; pos is its
    // first entry in the descriptor table
    auto run_group = [&](const GroupPlan &gp, size_t pos, const CallMem &gm, hipStream_t st) -> muon_status {
        muon_status s = MUON_OK;
        const CallMem &mem = gm;
        const bool bf16 = gp.bf16;
        float d = 0.f, sc = 0.f;
        muon_scalars(hp, gp.g.rows, gp.g.cols, &d, &sc);
        const int64_t n_all = static_cast<int64_t>(gp.members.size());
        for (int64_t c0 = 0; c0 < n_all; c0 += gp.chunk) {
            const int n = static_cast<int>(std::min<int64_t>(gp.chunk, n_all - c0));
            const MatDesc *dd = ddev + pos + c0;
            bool params_aligned = true, outs_aligned = true, any_out = false;
            for (int k = 0; k < n; ++k) {
                const muon_matrix &m = mats[gp.members[c0 + k]];
                params_aligned = params_aligned && aligned16(m.param);
                outs_aligned = outs_aligned && (!m.ns_out || aligned16(m.ns_out));
                any_out = any_out || m.ns_out != nullptr;
            }
            // the chunk's runs: members with rows <= cols, then those with rows > cols
            Run runs[2];
            int nruns = 0;
            if (c0 < gp.n_flat) runs[nruns++] = Run{0, std::min<int64_t>(c0 + n, gp.n_flat) - c0, run_geom(gp.g, false)};
            if (c0 + n > gp.n_flat) {
                const int64_t k0 = std::max<int64_t>(c0, gp.n_flat) - c0;
                runs[nruns++] = Run{k0, n - k0, run_geom(gp.g, true)};
            }
            Work w = chunk_work(mem, gp.g, bf16, n, gp.bpm, gp.splits.kpart(n));
            const double gsz = gp.grad_dtype == MUON_BF16 ? 2.0 : 4.0;
            for (int r = 0; r < nruns; ++r) {
                const Run &run = runs[r];
                const MatDesc *dr = dd + run.k0;
                const Work wr = offset_work(w, run.k0, bf16, run.k0 * gp.bpm);
                bool vec_ok = true;
                for (int64_t k = run.k0; k < run.k0 + run.n; ++k) {
                    const muon_matrix &m = mats[gp.members[c0 + k]];
                    vec_ok = vec_ok && aligned16(m.momentum) && aligned16(m.grad);
                }
                int tc = 0;
                const int bpm = muon::nesterov_blocks_per_mat(run.g, &tc);
                const double elems = static_cast<double>(gp.g.s) * gp.g.l * run.n;
                // M read and written (8), N written: fp32 (4) or hi + residual (3)
                hipError_t e = timed(ctx, ST_MOMENTUM, 0.0, elems * (gsz + (bf16 ? 11.0 : 12.0)), st, [&] {
                    return muon::launch_nesterov(dr, static_cast<int>(run.n), run.g, wr, mu, hp->nesterov,
                                                 gp.grad_dtype == MUON_BF16, vec_ok, st);
                });
                if (e != hipSuccess) return hip_fail(ctx, e, "momentum launch");
                e = timed(ctx, ST_FINALIZE, 0.0, static_cast<double>(run.n) * bpm * 8.0, st,
                          [&] { return muon::launch_norm_finalize(dr, static_cast<int>(run.n), wr, bpm, st); });
                if (e != hipSuccess) return hip_fail(ctx, e, "norm launch");
            }
            s = run_ns(ctx, dd, n, gp.g, w, bf16, hp, true, gp.param_dtype == MUON_BF16, any_out, d, sc, st,
                       gp.splits, runs, nruns, c0, params_aligned, gp.bpm, outs_aligned);
            if (s != MUON_OK) return s;
        }
        return s;
    };
    std::vector<hipStream_t> lane_st(static_cast<size_t>(nlanes), st);
    int forked = 0;  // side streams that wait for the fork
    if (nlanes > 1) {
        hipError_t e = hipEventRecord(ctx->fork_ev, st);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipEventRecord");
        for (int i = 0; i < nlanes - 1 && s == MUON_OK; ++i) {
            e = hipStreamWaitEvent(ctx->side[i], ctx->fork_ev, 0);
            if (e != hipSuccess) {
                s = hip_fail(ctx, e, "hipStreamWaitEvent");
                break;
            }
            lane_st[static_cast<size_t>(i) + 1] = ctx->side[i];
            ++forked;
        }
    }
    size_t pos = 0;
    for (size_t i = 0; i < plan.size() && s == MUON_OK; ++i) {
        const size_t l = static_cast<size_t>(lanes.lane_of[i]);
        const CallMem gm{mem.ws + lanes.ws_off[l], mem.tabs + lanes.tb_off[l], mem.call_nrm2};
        s = run_group(plan[i], pos, gm, lane_st[l]);
        pos += plan[i].members.size();
    }
    // every forked side stream joins the caller's stream, also after a failure
    for (int i = 0; i < forked; ++i) {
        hipError_t e = hipEventRecord(ctx->join_ev[i], ctx->side[i]);
        if (e == hipSuccess) e = hipStreamWaitEvent(st, ctx->join_ev[i], 0);
        if (e != hipSuccess && s == MUON_OK) s = hip_fail(ctx, e, "stream join");
    }
    if (s != MUON_OK) return s;
    ctx->last_stream = st;
    ctx->last_count = count;
    ctx->last_nrm2 = mem.call_nrm2;
    ctx->err.clear();
    return MUON_OK;
}


}  // namespace

// ===================================================================== C ABI

extern "C" {

int32_t muon_abi_version(void) { return MUON_STEP_ABI_VERSION; }

const char *muon_status_string(muon_status status) {
    // Callers in C (or through a foreign-function layer) may pass any 32-bit
    // value; reading it as the enum would be undefined for values outside the
    // enumerators' range, so the bytes are read as an integer.
    int32_t v = 0;
    static_assert(sizeof(status) == sizeof(v), "muon_status is 32 bits");
    std::memcpy(&v, &status, sizeof v);
    switch (v) {
        case MUON_OK: return "ok";
        case MUON_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MUON_ERR_UNSUPPORTED: return "unsupported";
        case MUON_ERR_OUT_OF_MEMORY: return "out of memory";
        case MUON_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

int64_t muon_schedule(const char *name, muon_ns_coeff *out, int64_t capacity) {
    if (!name) return -1;
    const muon_ns_coeff aggressive{3.4445, -4.7750, 2.0315};
    const muon_ns_coeff standard{2.0, -1.5, 0.5};
    std::vector<muon_ns_coeff> s;
    if (std::strcmp(name, "deepseekv4") == 0) {
        s.assign(8, aggressive);
        s.push_back(standard);
        s.push_back(standard);
    } else if (std::strcmp(name, "quintic") == 0) {
        s.assign(5, aggressive);
    } else {
        return -1;
    }
    if (out)
        for (int64_t i = 0; i < std::min<int64_t>(capacity, static_cast<int64_t>(s.size())); ++i) out[i] = s[i];
    return static_cast<int64_t>(s.size());
}

muon_status muon_check_step_args(const muon_matrix *mats, int64_t count, const muon_hparams *hp, char *msg,
                                 size_t msg_cap) {
    set_msg(msg, msg_cap, "%s", "");
    return check_step(mats, count, hp, msg, msg_cap);
}

muon_status muon_check_adamw_args(const muon_adamw_tensor *ts, int64_t count, const muon_adamw_hparams *hp,
                                  char *msg, size_t msg_cap) {
    set_msg(msg, msg_cap, "%s", "");
    return check_adamw(ts, count, hp, msg, msg_cap);
}

muon_status muon_workspace_bytes(const muon_matrix *mats, int64_t count, const muon_hparams *hp,
                                 size_t *bytes_out) {
    if (!bytes_out) return MUON_ERR_INVALID_ARGUMENT;
    muon_status s = check_step(mats, count, hp, nullptr, 0);
    if (s != MUON_OK) return s;
    std::vector<GroupPlan> plan;
    size_t ws = 0, parts = 0;
    int64_t mc = 0;
    s = plan_groups(mats, count, hp->ns_precision, 0, &plan, &ws, &parts, &mc, nullptr, 0);
    if (s != MUON_OK) return s;
    const Lanes lanes = plan_lanes(plan, 1 + muon_context::kSide, 0);
    const size_t tabs = lanes.n > 1 ? lanes.tb_off.back() : tabs_bytes(parts, mc);
    if (lanes.n > 1) ws = lanes.ws_off.back();
    *bytes_out = ws + tabs + align_up(static_cast<size_t>(count) * sizeof(double)) +
                 align_up(static_cast<size_t>(count) * sizeof(MatDesc));
    return MUON_OK;
}

muon_status muon_create(muon_context **out, int32_t hip_device, size_t workspace_cap_bytes) {
    if (!out) return MUON_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return MUON_ERR_DEVICE;
    }
    if (hip_device < 0 || hip_device >= n) return MUON_ERR_INVALID_ARGUMENT;
    muon_context *ctx = new (std::nothrow) muon_context();
    if (!ctx) return MUON_ERR_OUT_OF_MEMORY;
    ctx->device = hip_device;
    ctx->cap = workspace_cap_bytes;
    DeviceGuard guard(hip_device);
    if (hipEventCreateWithFlags(&ctx->upload_done, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ctx->noalloc_upload_done, hipEventDisableTiming) != hipSuccess) {
        (void)hipGetLastError();
        if (ctx->upload_done) (void)hipEventDestroy(ctx->upload_done);
        delete ctx;
        return MUON_ERR_DEVICE;
    }
    // The allocation-free step's memory: this device's copy of the static
    // scratch (its address, with this device current) and the pinned staging
    // of its descriptor table.  A failure here only disables that entry point.
    void *sp = nullptr;
    hipError_t e = muon::scratch_address(&sp);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        ctx->scratch_err = std::string("hipGetSymbolAddress: ") + hipGetErrorString(e);
    } else {
        ctx->scratch = static_cast<char *>(sp);
        e = hipHostMalloc(&ctx->noalloc_pinned, static_cast<size_t>(kNoAllocMaxMatrices) * sizeof(MatDesc),
                          hipHostMallocDefault);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            ctx->noalloc_pinned = nullptr;
            ctx->scratch_err = std::string("hipHostMalloc: ") + hipGetErrorString(e);
        }
    }
    *out = ctx;
    return MUON_OK;
}

muon_status muon_destroy(muon_context *ctx) {
    if (!ctx) return MUON_OK;
    DeviceGuard guard(ctx->device);
    (void)hipDeviceSynchronize();
    for (DevBuf *b : {&ctx->ws, &ctx->tabs, &ctx->call_nrm2, &ctx->mat_desc, &ctx->adamw_desc})
        if (b->p) (void)hipFree(b->p);
    if (ctx->pinned) (void)hipHostFree(ctx->pinned);
    if (ctx->noalloc_pinned) (void)hipHostFree(ctx->noalloc_pinned);
    if (ctx->upload_done) (void)hipEventDestroy(ctx->upload_done);
    if (ctx->noalloc_upload_done) (void)hipEventDestroy(ctx->noalloc_upload_done);
    for (hipEvent_t e : ctx->ev_pool) (void)hipEventDestroy(e);
    for (int i = 0; i < muon_context::kSide; ++i) {
        if (ctx->side[i]) (void)hipStreamDestroy(ctx->side[i]);
        if (ctx->join_ev[i]) (void)hipEventDestroy(ctx->join_ev[i]);
    }
    if (ctx->fork_ev) (void)hipEventDestroy(ctx->fork_ev);
    delete ctx;
    return MUON_OK;
}

const char *muon_last_error(const muon_context *ctx) { return ctx ? ctx->err.c_str() : "null context"; }

muon_status muon_step(muon_context *ctx, const muon_matrix *mats, int64_t count, const muon_hparams *hp,
                      void *hip_stream) {
    return step_impl(ctx, mats, count, hp, hip_stream, false);
}

muon_status muon_step_noalloc(muon_context *ctx, const muon_matrix *mats, int64_t count, const muon_hparams *hp,
                              void *hip_stream) {
    return step_impl(ctx, mats, count, hp, hip_stream, true);
}

muon_status muon_ns_only(muon_context *ctx, const float *n_in, float *x_out, int64_t rows, int64_t cols,
                         const muon_hparams *hp, void *hip_stream) {
    if (!ctx) return MUON_ERR_INVALID_ARGUMENT;
    char msg[512];
    if (!n_in || !x_out) return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "n_in and x_out must be non-NULL");
    muon_status s = check_shape(rows, cols, msg, sizeof msg, 0);
    if (s != MUON_OK) return fail(ctx, s, "%s", msg);
    if ((s = check_hparams(hp, msg, sizeof msg)) != MUON_OK) return fail(ctx, s, "%s", msg);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(n_in), b0 = reinterpret_cast<uintptr_t>(x_out);
    const uintptr_t nb = static_cast<uintptr_t>(rows * cols) * 4;
    if (a0 < b0 + nb && b0 < a0 + nb) return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "n_in and x_out overlap");
    const Geom g = make_geom(rows, cols);
    const bool bf16 = use_bf16(hp->ns_precision, g.s);
    const Splits sp = plan_splits(g, bf16, 1);
    const size_t need = chunk_layout(g, bf16, 1, sp.kpart(1)).total;
    if (ctx->cap && need > ctx->cap)
        return fail(ctx, MUON_ERR_OUT_OF_MEMORY, "matrix needs %zu bytes of workspace, above the cap", need);
    DeviceGuard guard(ctx->device);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const int tc = static_cast<int>((cols + 63) / 64);
    const int nb_blocks = static_cast<int>(((rows + 63) / 64) * tc);
    if ((s = ensure(ctx, ctx->ws, need, "workspace")) != MUON_OK) return s;
    if ((s = ensure(ctx, ctx->tabs, tabs_bytes(static_cast<size_t>(nb_blocks), 1), "norm tables")) != MUON_OK)
        return s;
    if ((s = ensure(ctx, ctx->call_nrm2, sizeof(double), "norm output")) != MUON_OK) return s;
    MatDesc d{};
    s = upload(ctx, ctx->mat_desc, ctx->mat_cache, &d, sizeof d, st, "matrix descriptors");
    if (s != MUON_OK) return s;
    const MatDesc *ddev = static_cast<const MatDesc *>(ctx->mat_desc.p);
    Work w = chunk_work(CallMem{static_cast<char *>(ctx->ws.p), static_cast<char *>(ctx->tabs.p),
                                static_cast<double *>(ctx->call_nrm2.p)},
                        g, bf16, 1, nb_blocks, sp.kpart(1));
    const double elems = static_cast<double>(rows) * cols;
    hipError_t e = timed(ctx, ST_IMPORT, 0.0, elems * 8.0, st, [&] { return muon::launch_import_n(n_in, g, w, st); });
    if (e != hipSuccess) return hip_fail(ctx, e, "import launch");
    e = timed(ctx, ST_FINALIZE, 0.0, nb_blocks * 8.0, st,
              [&] { return muon::launch_norm_finalize(ddev, 1, w, nb_blocks, st); });
    if (e != hipSuccess) return hip_fail(ctx, e, "norm launch");
    const Run run{0, 1, g};
    s = run_ns(ctx, ddev, 1, g, w, bf16, hp, false, 0, false, 0.f, 0.f, st, sp, &run, 1);
    if (s != MUON_OK) return s;
    e = timed(ctx, ST_EXPORT, 0.0, elems * 8.0, st, [&] { return muon::launch_export_x(g, w, x_out, st); });
    if (e != hipSuccess) return hip_fail(ctx, e, "export launch");
    ctx->last_stream = st;
    ctx->last_count = 1;
    ctx->last_nrm2 = w.call_nrm2;
    ctx->err.clear();
    return MUON_OK;
}

muon_status muon_apply_update(muon_context *ctx, void *param, int32_t param_dtype, const float *x, int64_t rows,
                              int64_t cols, const muon_hparams *hp, void *hip_stream) {
    if (!ctx) return MUON_ERR_INVALID_ARGUMENT;
    char msg[512];
    if (!param || !x) return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "param and x must be non-NULL");
    if (param_dtype != MUON_F32 && param_dtype != MUON_BF16)
        return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "unknown param dtype");
    muon_status s = check_shape(rows, cols, msg, sizeof msg, 0);
    if (s != MUON_OK) return fail(ctx, s, "%s", msg);
    if ((s = check_hparams(hp, msg, sizeof msg)) != MUON_OK) return fail(ctx, s, "%s", msg);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(param), b0 = reinterpret_cast<uintptr_t>(x);
    const uintptr_t na = static_cast<uintptr_t>(rows * cols) * dtype_size(param_dtype);
    const uintptr_t nx = static_cast<uintptr_t>(rows * cols) * 4;
    if (a0 < b0 + nx && b0 < a0 + na) return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "param and x overlap");
    float d = 0.f, sc = 0.f;
    muon_scalars(hp, rows, cols, &d, &sc);
    DeviceGuard guard(ctx->device);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const double by = static_cast<double>(rows) * cols * (4.0 + 2.0 * dtype_size(param_dtype));
    const float *s_dev = nullptr;
    hipError_t e = hipSuccess;
    if (hp->scale_mode == MUON_SCALE_UNIT_RMS) {
        // ||x||^2 over the plain rows x cols matrix: rows reduced in up to 1024
        // blocks, the scale written after the partial sums.
        const int nbx = static_cast<int>(std::min<int64_t>(rows, 1024));
        const size_t part = align_up(static_cast<size_t>(nbx) * sizeof(double));
        if ((s = ensure(ctx, ctx->tabs, part + sizeof(float), "norm tables")) != MUON_OK) return s;
        Geom g{};
        g.rows = g.s = g.sp = rows;
        g.cols = g.l = g.lp = cols;
        Work w{};
        w.partials = static_cast<double *>(ctx->tabs.p);
        float *sd = reinterpret_cast<float *>(static_cast<char *>(ctx->tabs.p) + part);
        const double gsq = hp->gamma * std::sqrt(static_cast<double>(rows) * static_cast<double>(cols));
        e = timed(ctx, ST_UNIT_RMS, 0.0, static_cast<double>(rows) * cols * 4.0, st, [&] {
            return muon::launch_unit_rms_scale(1, g, w, x, nbx, hp->lr, gsq, sd, st);
        });
        if (e != hipSuccess) return hip_fail(ctx, e, "unit-RMS norm launch");
        s_dev = sd;
    }
    e = timed(ctx, ST_UPDATE, 0.0, by, st, [&] {
        return muon::launch_update_plain(param, param_dtype == MUON_BF16, x, rows * cols, d, sc, s_dev, st);
    });
    if (e != hipSuccess) return hip_fail(ctx, e, "update launch");
    ctx->err.clear();
    return MUON_OK;
}

muon_status muon_adamw_step(muon_context *ctx, const muon_adamw_tensor *ts, int64_t count,
                            const muon_adamw_hparams *hp, void *hip_stream) {
    if (!ctx) return MUON_ERR_INVALID_ARGUMENT;
    char msg[512];
    muon_status s = check_adamw(ts, count, hp, msg, sizeof msg);
    if (s != MUON_OK) return fail(ctx, s, "%s", msg);
    muon::AdamwScalars k{};
    k.decay = static_cast<float>(1.0 - hp->lr * hp->weight_decay);
    k.beta1 = static_cast<float>(hp->beta1);
    k.beta2 = static_cast<float>(hp->beta2);
    k.one_minus_beta1 = static_cast<float>(1.0 - hp->beta1);
    k.one_minus_beta2 = static_cast<float>(1.0 - hp->beta2);
    k.bias_corr1 = static_cast<float>(1.0 - std::pow(hp->beta1, static_cast<double>(hp->step)));
    k.bias_corr2 = static_cast<float>(1.0 - std::pow(hp->beta2, static_cast<double>(hp->step)));
    k.lr = static_cast<float>(hp->lr);
    k.eps = static_cast<float>(hp->eps);
    const size_t ds = muon::adamw_desc_size();
    std::vector<unsigned char> table;
    int64_t blocks = 0;
    int n = 0;
    for (int64_t i = 0; i < count; ++i) {
        if (ts[i].numel == 0) continue;
        table.resize(table.size() + ds);
        muon::adamw_fill_desc(table.data() + table.size() - ds, static_cast<float *>(ts[i].param),
                              static_cast<const float *>(ts[i].grad), ts[i].exp_avg, ts[i].exp_avg_sq, ts[i].numel,
                              blocks);
        blocks += muon::adamw_blocks(ts[i].numel);
        ++n;
    }
    if (n == 0) { ctx->err.clear(); return MUON_OK; }
    if (blocks > (int64_t(1) << 31) - 1) return fail(ctx, MUON_ERR_UNSUPPORTED, "AdamW call too large for one grid");
    DeviceGuard guard(ctx->device);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    s = upload(ctx, ctx->adamw_desc, ctx->adamw_cache, table.data(), table.size(), st, "AdamW descriptors");
    if (s != MUON_OK) return s;
    double elems = 0;
    for (int64_t i = 0; i < count; ++i) elems += static_cast<double>(ts[i].numel);
    hipError_t e = timed(ctx, ST_ADAMW, 0.0, elems * 28.0, st,
                         [&] { return muon::launch_adamw(ctx->adamw_desc.p, n, blocks, k, st); });
    if (e != hipSuccess) return hip_fail(ctx, e, "AdamW launch");
    ctx->err.clear();
    return MUON_OK;
}

muon_status muon_ns_stage(muon_context *ctx, int32_t stage, const float *x, const float *m, float *out, int64_t s,
                          int64_t l, double a, double b, double c, void *hip_stream) {
    if (!ctx) return MUON_ERR_INVALID_ARGUMENT;
    if (stage != MUON_STAGE_GRAM && stage != MUON_STAGE_POLY && stage != MUON_STAGE_APPLY)
        return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "unknown stage %d", stage);
    if (!out || (stage != MUON_STAGE_POLY && !x) || (stage != MUON_STAGE_GRAM && !m))
        return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "missing operand or output");
    if (s < 1 || l < s || l > kMaxDim || s * l > kMaxElems)
        return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "unsupported shape %lld x %lld (need 1 <= s <= l)", (long long)s,
                    (long long)l);
    if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c))
        return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "non-finite coefficient");
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(out);
    const uintptr_t on = static_cast<uintptr_t>(stage == MUON_STAGE_APPLY ? s * l : s * s) * 4;
    for (const float *in : {x, m}) {
        if (!in) continue;
        const uintptr_t i0 = reinterpret_cast<uintptr_t>(in);
        const uintptr_t in_n = static_cast<uintptr_t>(in == x ? s * l : s * s) * 4;
        if (i0 < o0 + on && o0 < i0 + in_n) return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "an operand overlaps out");
    }
    const Geom g = make_geom(s, l);
    const Splits sp = plan_splits(g, true, 1);
    const size_t need = chunk_layout(g, true, 1, sp.kpart(1)).total;
    if (ctx->cap && need > ctx->cap)
        return fail(ctx, MUON_ERR_OUT_OF_MEMORY, "matrix needs %zu bytes of workspace, above the cap", need);
    DeviceGuard guard(ctx->device);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    muon_status rs;
    if ((rs = ensure(ctx, ctx->ws, need, "workspace")) != MUON_OK) return rs;
    if ((rs = ensure(ctx, ctx->tabs, tabs_bytes(1, 1), "norm tables")) != MUON_OK) return rs;
    if ((rs = ensure(ctx, ctx->call_nrm2, sizeof(double), "norm output")) != MUON_OK) return rs;
    Work w = chunk_work(CallMem{static_cast<char *>(ctx->ws.p), static_cast<char *>(ctx->tabs.p),
                                static_cast<double *>(ctx->call_nrm2.p)},
                        g, true, 1, 1, sp.kpart(1));
    muon::NsStep p{};
    p.a = static_cast<float>(a);
    p.b = static_cast<float>(b);
    p.c = static_cast<float>(c);
    p.gram_splits = sp.gram;
    p.gram_units = sp.gram_units;
    p.poly_splits = sp.poly;
    p.poly_units = sp.poly_units;
    p.split_from = sp.from;
    p.apply_splits = sp.apply;
    p.apply_units = sp.apply_units;
    p.apply_split_from = sp.apply_from;
    hipError_t e = hipSuccess;
    if (stage != MUON_STAGE_POLY) e = muon::launch_import_pair(g, x, w, st);
    if (e == hipSuccess && stage != MUON_STAGE_GRAM)
        e = muon::launch_import_bf16_square(s, g.sp, m, stage == MUON_STAGE_POLY ? w.ab : w.bb, st);
    if (e != hipSuccess) return hip_fail(ctx, e, "operand import");
    const int kind = stage == MUON_STAGE_GRAM ? 0 : stage == MUON_STAGE_POLY ? 1 : 2;
    double fl = 0, by = 0;
    ns_work(kind == 0 ? ST_GRAM : kind == 1 ? ST_POLY : ST_APPLY, g, true, 1, false, 2, &fl, &by);
    e = timed(ctx, kind == 0 ? ST_GRAM : kind == 1 ? ST_POLY : ST_APPLY, fl, by, st,
              [&] { return muon::launch_ns_stage_bf16(kind, nullptr, 1, g, w, p, st); });
    if (e != hipSuccess) return hip_fail(ctx, e, "Newton-Schulz launch");
    if (stage == MUON_STAGE_APPLY) {
        std::swap(w.xb, w.xb_next);
        e = muon::launch_export_x(g, w, out, st);
    } else {
        e = muon::launch_export_bf16_square(s, g.sp, stage == MUON_STAGE_GRAM ? w.ab : w.bb, out, st);
    }
    if (e != hipSuccess) return hip_fail(ctx, e, "export launch");
    ctx->err.clear();
    return MUON_OK;
}

muon_status muon_stream_probe(muon_context *ctx, const void *src, void *dst, int64_t stream_bytes,
                              int64_t pitch_bytes, int32_t reads, int32_t writes, void *hip_stream) {
    if (!ctx) return MUON_ERR_INVALID_ARGUMENT;
    if (!src || !dst || stream_bytes <= 0 || stream_bytes % 16 != 0 || pitch_bytes < stream_bytes ||
        pitch_bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
        return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "src and dst must be 16-byte aligned, stream_bytes a positive "
                                                    "multiple of 16, pitch_bytes a multiple of 16 >= stream_bytes");
    if (!((reads == 6 && writes == 7) || (reads == 4 && writes == 3) || (reads == 5 && writes == 2) ||
          (reads == 1 && writes == 1)))
        return fail(ctx, MUON_ERR_UNSUPPORTED, "no probe for %d reads : %d writes", reads, writes);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(src), b0 = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t na = static_cast<uintptr_t>(pitch_bytes) * (reads - 1) + static_cast<uintptr_t>(stream_bytes);
    const uintptr_t nb = static_cast<uintptr_t>(pitch_bytes) * (writes - 1) + static_cast<uintptr_t>(stream_bytes);
    if (a0 < b0 + nb && b0 < a0 + na) return fail(ctx, MUON_ERR_INVALID_ARGUMENT, "src and dst overlap");
    DeviceGuard guard(ctx->device);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    hipError_t e = timed(ctx, ST_PROBE, 0.0, static_cast<double>(stream_bytes) * (reads + writes), st, [&] {
        return muon::launch_stream_probe(src, dst, stream_bytes / 16, pitch_bytes / 16, reads, writes, st);
    });
    if (e != hipSuccess) return hip_fail(ctx, e, "probe launch");
    ctx->err.clear();
    return MUON_OK;
}

muon_status muon_last_norms(muon_context *ctx, double *out, int64_t capacity, int64_t *count_out) {
    if (!ctx || !count_out || capacity < 0 || (capacity > 0 && !out)) return MUON_ERR_INVALID_ARGUMENT;
    *count_out = ctx->last_count;
    const int64_t n = std::min(capacity, ctx->last_count);
    if (n == 0) return MUON_OK;
    DeviceGuard guard(ctx->device);
    hipError_t e = hipStreamSynchronize(ctx->last_stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamSynchronize");
    e = hipMemcpy(out, ctx->last_nrm2, static_cast<size_t>(n) * sizeof(double), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpy");
    return MUON_OK;
}

muon_status muon_set_concurrent_groups(muon_context *ctx, int32_t enable) {
    if (!ctx || (enable != 0 && enable != 1)) return MUON_ERR_INVALID_ARGUMENT;
    ctx->concurrent = enable != 0;
    return MUON_OK;
}

muon_status muon_profile_enable(muon_context *ctx, int32_t enable) {
    if (!ctx || (enable != 0 && enable != 1)) return MUON_ERR_INVALID_ARGUMENT;
    ctx->prof_on = enable != 0;
    ctx->recs.clear();
    ctx->ev_used = 0;
    return MUON_OK;
}

muon_status muon_profile_read(muon_context *ctx, muon_stage_stats *out, int32_t capacity, int32_t *count) {
    if (!ctx || !count || capacity < 0 || (capacity > 0 && !out)) return MUON_ERR_INVALID_ARGUMENT;
    DeviceGuard guard(ctx->device);
    std::vector<int> order;
    std::vector<muon_stage_stats> agg(ST_COUNT);
    for (int i = 0; i < ST_COUNT; ++i) {
        std::memset(&agg[i], 0, sizeof agg[i]);
        std::snprintf(agg[i].name, sizeof agg[i].name, "%s", kStageNames[i]);
    }
    for (const auto &r : ctx->recs) {
        hipError_t e = hipEventSynchronize(r.b);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipEventSynchronize");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipEventElapsedTime");
        if (agg[r.stage].launches == 0) order.push_back(r.stage);
        agg[r.stage].launches += 1;
        agg[r.stage].total_ms += ms;
        agg[r.stage].flops += r.flops;
        agg[r.stage].bytes += r.bytes;
    }
    *count = static_cast<int32_t>(order.size());
    for (int i = 0; i < static_cast<int>(order.size()) && i < capacity; ++i) out[i] = agg[order[i]];
    ctx->recs.clear();
    ctx->ev_used = 0;
    return MUON_OK;
}

}  // extern "C"
