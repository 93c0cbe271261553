// Host runtime of the Muon step library: argument validation, same-shape
// grouping, workspace planning, descriptor upload and the launch sequence
// behind the C ABI declared in include/muon_step.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
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

struct GroupPlan {
    Geom g;
    bool bf16;                    // bf16 Newton-Schulz products for this group
    int32_t param_dtype, grad_dtype;
    std::vector<int64_t> members; // indices into the caller's list
    int64_t chunk = 0;            // matrices per chunk
    int bpm = 0;                  // stage-1 blocks per matrix
};

// Bytes of NS workspace one matrix of geometry g needs.
size_t per_matrix_bytes(const Geom &g, bool bf16) {
    const size_t x = static_cast<size_t>(g.sp * g.lp), a = static_cast<size_t>(g.sp * g.sp);
    return bf16 ? (x * (2 + 2 + 1) + a * (2 + 2)) : (x * (4 + 4) + a * (4 + 4 + 4));
}

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

struct Layout {
    size_t xf0, xf1, xb0, xb1, xl, af, ab, bb, total;
    bool has_xf;
};

Layout chunk_layout(const Geom &g, bool bf16, int64_t n) {
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
    L.total = off;
    return L;
}

muon_status plan_groups(const muon_matrix *mats, int64_t count, int32_t precision, size_t cap, std::vector<GroupPlan> *out,
                        size_t *ws_bytes, size_t *partial_count, int64_t *max_chunk, char *msg, size_t msg_cap) {
    std::map<std::tuple<int64_t, int64_t, int32_t, int32_t>, size_t> index;
    out->clear();
    for (int64_t i = 0; i < count; ++i) {
        const auto key = std::make_tuple(mats[i].rows, mats[i].cols, mats[i].param_dtype, mats[i].grad_dtype);
        auto it = index.find(key);
        if (it == index.end()) {
            GroupPlan gp;
            gp.g = make_geom(mats[i].rows, mats[i].cols);
            gp.bf16 = use_bf16(precision, gp.g.s);
            gp.param_dtype = mats[i].param_dtype;
            gp.grad_dtype = mats[i].grad_dtype;
            index.emplace(key, out->size());
            out->push_back(gp);
            out->back().members.push_back(i);
        } else {
            (*out)[it->second].members.push_back(i);
        }
    }
    *ws_bytes = 0;
    *partial_count = 0;
    *max_chunk = 0;
    for (GroupPlan &gp : *out) {
        const bool bf16 = gp.bf16;
        const size_t per = per_matrix_bytes(gp.g, bf16);
        int64_t n = static_cast<int64_t>(gp.members.size());
        if (cap) {
            if (chunk_layout(gp.g, bf16, 1).total > cap) {
                set_msg(msg, msg_cap, "a %lld x %lld matrix needs %zu bytes of workspace, above the cap %zu",
                        (long long)gp.g.rows, (long long)gp.g.cols, chunk_layout(gp.g, bf16, 1).total, cap);
                return MUON_ERR_OUT_OF_MEMORY;
            }
            n = std::min<int64_t>(n, std::max<int64_t>(1, static_cast<int64_t>(cap / per)));
            while (n > 1 && chunk_layout(gp.g, bf16, n).total > cap) --n;
        }
        // Keep every grouped launch inside a 32-bit grid.
        const int64_t apply_tiles = (gp.g.sp / muon::kTile) * (gp.g.lp / muon::kTile);
        n = std::min<int64_t>(n, std::max<int64_t>(1, ((int64_t(1) << 31) - 1) / apply_tiles));
        int rpb = 0, tc = 0;
        gp.bpm = muon::nesterov_blocks_per_mat(gp.g, &rpb, &tc);
        n = std::min<int64_t>(n, std::max<int64_t>(1, ((int64_t(1) << 31) - 1) / gp.bpm));
        gp.chunk = n;
        *ws_bytes = std::max(*ws_bytes, chunk_layout(gp.g, bf16, n).total);
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
    ST_ADAMW, ST_IMPORT, ST_EXPORT, ST_UNIT_RMS, ST_COUNT
};
const char *const kStageNames[ST_COUNT] = {"momentum_nesterov", "norm_finalize", "normalize", "gram", "poly",
                                           "apply", "apply_update", "update", "adamw", "import", "export",
                                           "unit_rms"};

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

// Work view of a chunk laid out at the workspace base.
Work chunk_work(muon_context *ctx, const Geom &g, bool bf16, int64_t n, int bpm, size_t call_count) {
    (void)call_count;
    const Layout L = chunk_layout(g, bf16, n);
    char *base = static_cast<char *>(ctx->ws.p);
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
    char *t = static_cast<char *>(ctx->tabs.p);
    w.partials = reinterpret_cast<double *>(t);
    const size_t np = align_up(static_cast<size_t>(n) * bpm * sizeof(double));
    w.nrm2 = reinterpret_cast<double *>(t + np);
    w.inv_norm = reinterpret_cast<float *>(t + np + align_up(static_cast<size_t>(n) * sizeof(double)));
    w.call_nrm2 = static_cast<double *>(ctx->call_nrm2.p);
    return w;
}

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

// Runs normalisation + the NS schedule (+ the fused update when `update`) on
// one chunk whose first stage already wrote X = N and the norms.  Returns the
// workspace view holding the final X in xf (fp32 path) or xb + xl (bf16 path),
// meaningful when !update.  In the unit-RMS scale mode the last step writes X
// like the others; ||X||^2 per matrix is then reduced (partial_bpm partial
// sums per matrix fit in w.partials) into a per-matrix scale, and a separate
// pass applies the decay + update.
muon_status run_ns(muon_context *ctx, const MatDesc *descs, int nmat, const Geom &g, Work &w, bool bf16,
                   const muon_hparams *hp, bool update, int param_bf16, bool any_ns_out, float d, float s,
                   hipStream_t st, bool params_aligned16 = false, int partial_bpm = 0, bool outs_aligned16 = false) {
    const bool unit_rms = update && hp->scale_mode == MUON_SCALE_UNIT_RMS;
    // bf16 parameters whose tiles allow staging W through LDS keep the update
    // fused into the last product.  Other shapes whose W rows allow 8-wide
    // access run the last step as a plain product plus a separate update
    // pass, which costs less than the per-element fused epilogue there.
    const bool w_staged = param_bf16 && params_aligned16 && !g.transposed && g.s % muon::kTile == 0 &&
                          g.l % muon::kTile == 0;
    const bool split_update = update && !unit_rms && bf16 && !w_staged && params_aligned16 && outs_aligned16 &&
                              (g.transposed ? g.cols % 8 == 0 : g.l % 8 == 0);
    const double xe = static_cast<double>(g.s) * g.l * nmat;
    // bf16 path with a schedule: X stays N and the first step applies 1/||N||
    // (only the padding needs zeros); otherwise a normalisation pass.
    const bool fold = bf16 && hp->num_ns_steps > 0;
    hipError_t e = hipSuccess;
    if (!fold) {
        e = timed(ctx, ST_NORMALIZE, 0.0, xe * (bf16 ? 6.0 : 8.0), st, [&] { return muon::launch_normalize(nmat, g, w, st); });
    } else if (g.sp > g.s || g.lp > g.l) {
        const double pad = (static_cast<double>(g.sp) * g.lp - static_cast<double>(g.s) * g.l) * nmat;
        e = timed(ctx, ST_NORMALIZE, 0.0, pad * 3.0, st, [&] { return muon::launch_pad_zero(nmat, g, w, st); });
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
        const double by = xe * ((bf16 ? 3.0 : 4.0) + 2.0 * psize + (any_ns_out ? 4.0 : 0.0));
        e = timed(ctx, ST_UPDATE, 0.0, by, st,
                  [&] {
                      return muon::launch_update_from_work(descs, nmat, g, w, param_bf16, d, s,
                                                           params_aligned16 && outs_aligned16, st);
                  });
        if (e != hipSuccess) return hip_fail(ctx, e, "update launch");
    }
    return MUON_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

// ===================================================================== C ABI

extern "C" {

int32_t muon_abi_version(void) { return MUON_STEP_ABI_VERSION; }

const char *muon_status_string(muon_status status) {
    switch (status) {
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
    *bytes_out = ws + tabs_bytes(parts, mc) + align_up(static_cast<size_t>(count) * sizeof(double)) +
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
    if (hipEventCreateWithFlags(&ctx->upload_done, hipEventDisableTiming) != hipSuccess) {
        delete ctx;
        return MUON_ERR_DEVICE;
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
    if (ctx->upload_done) (void)hipEventDestroy(ctx->upload_done);
    for (hipEvent_t e : ctx->ev_pool) (void)hipEventDestroy(e);
    delete ctx;
    return MUON_OK;
}

const char *muon_last_error(const muon_context *ctx) { return ctx ? ctx->err.c_str() : "null context"; }

muon_status muon_step(muon_context *ctx, const muon_matrix *mats, int64_t count, const muon_hparams *hp,
                      void *hip_stream) {
    if (!ctx) return MUON_ERR_INVALID_ARGUMENT;
    char msg[512];
    muon_status s = check_step(mats, count, hp, msg, sizeof msg);
    if (s != MUON_OK) return fail(ctx, s, "%s", msg);
    if (count == 0) { ctx->err.clear(); return MUON_OK; }
    std::vector<GroupPlan> plan;
    size_t ws = 0, parts = 0;
    int64_t max_chunk = 0;
    s = plan_groups(mats, count, hp->ns_precision, ctx->cap, &plan, &ws, &parts, &max_chunk, msg, sizeof msg);
    if (s != MUON_OK) return fail(ctx, s, "%s", msg);
    DeviceGuard guard(ctx->device);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if ((s = ensure(ctx, ctx->ws, ws, "workspace")) != MUON_OK) return s;
    if ((s = ensure(ctx, ctx->tabs, tabs_bytes(parts, max_chunk), "norm tables")) != MUON_OK) return s;
    if ((s = ensure(ctx, ctx->call_nrm2, static_cast<size_t>(count) * sizeof(double), "norm output")) != MUON_OK)
        return s;
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
    s = upload(ctx, ctx->mat_desc, ctx->mat_cache, descs.data(), descs.size() * sizeof(MatDesc), st,
               "matrix descriptors");
    if (s != MUON_OK) return s;
    const MatDesc *ddev = static_cast<const MatDesc *>(ctx->mat_desc.p);
    const float mu = static_cast<float>(hp->momentum);
    size_t pos = 0;
    for (const GroupPlan &gp : plan) {
        const bool bf16 = gp.bf16;
        float d = 0.f, sc = 0.f;
        muon_scalars(hp, gp.g.rows, gp.g.cols, &d, &sc);
        const int64_t n_all = static_cast<int64_t>(gp.members.size());
        for (int64_t c0 = 0; c0 < n_all; c0 += gp.chunk) {
            const int n = static_cast<int>(std::min<int64_t>(gp.chunk, n_all - c0));
            const MatDesc *dd = ddev + pos + c0;
            bool vec_ok = true, params_aligned = true, outs_aligned = true;
            for (int k = 0; k < n; ++k) {
                const muon_matrix &m = mats[gp.members[c0 + k]];
                vec_ok = vec_ok && aligned16(m.momentum) && aligned16(m.grad);
                params_aligned = params_aligned && aligned16(m.param);
                outs_aligned = outs_aligned && (!m.ns_out || aligned16(m.ns_out));
            }
            bool any_out = false;
            for (int k = 0; k < n; ++k) any_out = any_out || mats[gp.members[c0 + k]].ns_out != nullptr;
            Work w = chunk_work(ctx, gp.g, bf16, n, gp.bpm, count);
            const double elems = static_cast<double>(gp.g.rows) * gp.g.cols * n;
            const double gsz = gp.grad_dtype == MUON_BF16 ? 2.0 : 4.0;
            // M read and written (8), N written: fp32 (4) or hi + residual (3)
            hipError_t e = timed(ctx, ST_MOMENTUM, 0.0, elems * (gsz + (bf16 ? 11.0 : 12.0)), st, [&] {
                return muon::launch_nesterov(dd, n, gp.g, w, mu, hp->nesterov, gp.grad_dtype == MUON_BF16, vec_ok,
                                             st);
            });
            if (e != hipSuccess) return hip_fail(ctx, e, "momentum launch");
            e = timed(ctx, ST_FINALIZE, 0.0, static_cast<double>(n) * gp.bpm * 8.0, st,
                      [&] { return muon::launch_norm_finalize(dd, n, w, gp.bpm, st); });
            if (e != hipSuccess) return hip_fail(ctx, e, "norm launch");
            s = run_ns(ctx, dd, n, gp.g, w, bf16, hp, true, gp.param_dtype == MUON_BF16, any_out, d, sc, st,
                       params_aligned, gp.bpm, outs_aligned);
            if (s != MUON_OK) return s;
        }
        pos += static_cast<size_t>(n_all);
    }
    ctx->last_stream = st;
    ctx->last_count = count;
    ctx->err.clear();
    return MUON_OK;
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
    const size_t need = chunk_layout(g, bf16, 1).total;
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
    Work w = chunk_work(ctx, g, bf16, 1, nb_blocks, 1);
    const double elems = static_cast<double>(rows) * cols;
    hipError_t e = timed(ctx, ST_IMPORT, 0.0, elems * 8.0, st, [&] { return muon::launch_import_n(n_in, g, w, st); });
    if (e != hipSuccess) return hip_fail(ctx, e, "import launch");
    e = timed(ctx, ST_FINALIZE, 0.0, nb_blocks * 8.0, st,
              [&] { return muon::launch_norm_finalize(ddev, 1, w, nb_blocks, st); });
    if (e != hipSuccess) return hip_fail(ctx, e, "norm launch");
    s = run_ns(ctx, ddev, 1, g, w, bf16, hp, false, 0, false, 0.f, 0.f, st);
    if (s != MUON_OK) return s;
    e = timed(ctx, ST_EXPORT, 0.0, elems * 8.0, st, [&] { return muon::launch_export_x(g, w, x_out, st); });
    if (e != hipSuccess) return hip_fail(ctx, e, "export launch");
    ctx->last_stream = st;
    ctx->last_count = 1;
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

muon_status muon_last_norms(muon_context *ctx, double *out, int64_t capacity, int64_t *count_out) {
    if (!ctx || !count_out || capacity < 0 || (capacity > 0 && !out)) return MUON_ERR_INVALID_ARGUMENT;
    *count_out = ctx->last_count;
    const int64_t n = std::min(capacity, ctx->last_count);
    if (n == 0) return MUON_OK;
    DeviceGuard guard(ctx->device);
    hipError_t e = hipStreamSynchronize(ctx->last_stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamSynchronize");
    e = hipMemcpy(out, ctx->call_nrm2.p, static_cast<size_t>(n) * sizeof(double), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpy");
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
