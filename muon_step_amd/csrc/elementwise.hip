// Elementwise and reduction kernels of the Muon step (HBM-bound).
//
//  * nesterov_*      : M_t = mu M_{t-1} + G_t, N_t = mu M_t + G_t (deep-dive page,
//                      "V4 的完整更新公式" steps 1-2; DeepSeek-V4 book ch. 6 §5),
//                      N_t written into the X workspace in the s x l orientation
//                      (transposed through LDS when rows > cols) as fp32, or on the
//                      bf16 path as the bf16 pair (hi, lo) the first Newton-Schulz
//                      step reads directly, per-block sums of N_t^2 in fp64.
//  * norm_finalize   : ||N_t||_F^2 per matrix from the block sums, fixed order.
//  * normalize       : X_0 = N_t / ||N_t||_F (book ch. 6 §5, normalisation line),
//                      fp32 (fp32 path) or the bf16 pair (hi, lo), zero padding.
//  * update_*        : W_t = (1 - lr wd) W_{t-1} - lr gamma sqrt(max) X (deep-dive
//                      page step 4-5), fl32 ops in exactly that order.
//  * adamw           : the AdamW step of embedding/head tensors (division is the
//                      IEEE div_scale/div_fmas/div_fixup sequence the build selects
//                      with -fhip-fp32-correctly-rounded-divide-sqrt; sqrt_rn below).
//
// All float arithmetic here is compiled with -ffp-contract=off so every
// multiply and add rounds once, matching the fp32 bookkeeping reference.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace muon {

template <typename T> __device__ __forceinline__ float load_val(const T *p, int64_t i);
template <> __device__ __forceinline__ float load_val<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_val<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_bits_to_float(p[i]);
}
template <typename T> __device__ __forceinline__ void store_val(T *p, int64_t i, float v);
template <> __device__ __forceinline__ void store_val<float>(float *p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void store_val<uint16_t>(uint16_t *p, int64_t i, float v) {
    p[i] = float_to_bf16_bits(v);
}

// Correctly rounded fp32 square root.  The hardware estimate v_sqrt_f32
// (within 1 ulp) is corrected by the signs of the exact FMA residuals
// x - s*pred(s) and x - s*succ(s): the true root lies below the midpoint
// (s + pred(s))/2 iff x <= s*pred(s), because no float x falls strictly between
// s*pred(s) and the square of that midpoint (Markstein's FMA-based square-root
// rounding; Muller et al., Handbook of Floating-Point Arithmetic, square-root
// chapter).  Inputs below 2^-96 are scaled by 2^32 so the residuals cannot
// underflow; zeros, infinities, NaN and negative inputs take the hardware result.
__device__ __forceinline__ float sqrt_rn(float x) {
    if (!(x > 0.0f) || x == __builtin_inff()) return __builtin_amdgcn_sqrtf(x);
    const bool tiny = x < 0x1p-96f;
    const float xs = tiny ? x * 0x1p32f : x;
    float s = __builtin_amdgcn_sqrtf(xs);
    for (int i = 0; i < 2; ++i) {
        const float dn = __uint_as_float(__float_as_uint(s) - 1u);
        const float up = __uint_as_float(__float_as_uint(s) + 1u);
        const float r_dn = __builtin_fmaf(-dn, s, xs);
        const float r_up = __builtin_fmaf(-up, s, xs);
        if (r_dn <= 0.0f) s = dn;
        else if (r_up > 0.0f) s = up;
    }
    return tiny ? s * 0x1p-16f : s;
}

// Deterministic block reduction of one double per thread (fixed tree order).
template <int NT>
__device__ __forceinline__ double block_sum(double v, double *sh) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) sh[wid] = v;
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0) {
        for (int w = 0; w < NT / 64; ++w) r += sh[w];
    }
    return r;  // valid in thread 0
}

// Read access to one matrix's workspace X: fp32, or the bf16 pair (hi, lo).
struct XView {
    const float *xf;  // fp32 path; nullptr on the bf16 path
    const uint16_t *xh;
    const uint8_t *xl;
    __device__ __forceinline__ float at(int64_t i) const { return xf ? xf[i] : join_bf16(xh[i], xl[i]); }
};

// N into the first matrix's workspace slot (fp32, or the bf16 pair in (xb, xl)).
__device__ __forceinline__ void store_n(const Work &w, int64_t i, float v) {
    if (w.xf)
        w.xf[i] = v;
    else
        split_bf16(v, static_cast<uint16_t *>(w.xb) + i, static_cast<uint8_t *>(w.xl) + i);
}

// ---------------------------------------------------------------------------
// Stage 1, rows <= cols: X = N (no transpose).  Block (e, b) handles elements
// [b * kMomElems, (b + 1) * kMomElems) of matrix e in row-major order, where G
// and M are contiguous (X rows have pitch lp).  VEC (16-byte aligned G and M,
// cols and lp multiples of 4): each lane loads its four vectors of four
// elements (4 x 24 or 32 bytes in flight) before it computes, and every
// access is a non-temporal stream; a vector never straddles a row.  Blocks
// this short (one pass per lane) stream about 15% faster than blocks of whole
// rows that loop.  Each lane sums N^2 over its elements in index order.
constexpr int kMomElems = 4096;

template <typename GradT, bool VEC>
__global__ __launch_bounds__(256) void nesterov_rows_kernel(const MatDesc *__restrict__ descs,
                                                            Geom g, Work w, float mu,
                                                            int nesterov, int blocks_per_mat) {
    __shared__ double sh[4];
    const int64_t e = blockIdx.x / blocks_per_mat;
    const int64_t b = blockIdx.x % blocks_per_mat;
    const MatDesc d = descs[e];
    const int64_t cols = g.cols;
    const int64_t k0 = b * kMomElems;
    const GradT *__restrict__ gp = static_cast<const GradT *>(d.grad) + k0;
    float *__restrict__ mp = d.mom + k0;
    float *__restrict__ xf = w.xf ? w.xf + e * w.x_stride : nullptr;  // fp32 path
    uint16_t *__restrict__ xh = static_cast<uint16_t *>(w.xb) + e * w.x_stride;  // bf16 path
    uint8_t *__restrict__ xl = static_cast<uint8_t *>(w.xl) + e * w.x_stride;
    const int total = static_cast<int>(min<int64_t>(kMomElems, g.rows * cols - k0));
    // row and column of the block's first element; element t of the block then
    // lies at column j0 + t of row i0 (32-bit: j0 + t < cols + kMomElems)
    const int64_t i0 = k0 / cols;
    const uint32_t j0 = static_cast<uint32_t>(k0 - i0 * cols), ucols = static_cast<uint32_t>(cols);
    auto xidx = [&](int t) {
        const uint32_t jj = j0 + static_cast<uint32_t>(t);
        const uint32_t ii = jj / ucols;
        return (i0 + ii) * g.lp + (jj - ii * ucols);
    };
    double acc = 0.0;
    if (VEC) {
        constexpr int U = kMomElems / 4 / 256;
        float gv[U][4];
        floatx4 m[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = threadIdx.x + 256 * u;  // vector t: elements 4t .. 4t+3
            if (4 * t >= total) break;
            if constexpr (sizeof(GradT) == 2) {
                const u32x2 raw = __builtin_nontemporal_load(as_global(reinterpret_cast<const u32x2 *>(gp) + t));
                gv[u][0] = __uint_as_float(raw[0] << 16);
                gv[u][1] = __uint_as_float(raw[0] & 0xffff0000u);
                gv[u][2] = __uint_as_float(raw[1] << 16);
                gv[u][3] = __uint_as_float(raw[1] & 0xffff0000u);
            } else {
                const floatx4 raw = __builtin_nontemporal_load(as_global(reinterpret_cast<const floatx4 *>(gp) + t));
                gv[u][0] = raw[0]; gv[u][1] = raw[1]; gv[u][2] = raw[2]; gv[u][3] = raw[3];
            }
            m[u] = __builtin_nontemporal_load(as_global(reinterpret_cast<const floatx4 *>(mp) + t));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = threadIdx.x + 256 * u;
            if (4 * t >= total) break;
            floatx4 mo, no;
            for (int q = 0; q < 4; ++q) {
                const float m1 = mu * m[u][q] + gv[u][q];
                const float n = nesterov ? (mu * m1 + gv[u][q]) : m1;
                mo[q] = m1;
                no[q] = n;
                acc += static_cast<double>(n) * static_cast<double>(n);
            }
            __builtin_nontemporal_store(mo, as_global(reinterpret_cast<floatx4 *>(mp) + t));
            const int64_t dst = xidx(4 * t);
            if (xf) {
                __builtin_nontemporal_store(no, as_global(reinterpret_cast<floatx4 *>(xf + dst)));
            } else {
                u32x2 h;
                uint32_t l;
                split_bf16x4(no, &h, &l);
                __builtin_nontemporal_store(h, as_global(reinterpret_cast<u32x2 *>(xh + dst)));
                __builtin_nontemporal_store(l, as_global(reinterpret_cast<uint32_t *>(xl + dst)));
            }
        }
    } else {
        for (int t = threadIdx.x; t < total; t += 256) {
            const float gv = load_val<GradT>(gp, t);
            const float m1 = mu * mp[t] + gv;
            const float n = nesterov ? (mu * m1 + gv) : m1;
            mp[t] = m1;
            const int64_t dst = xidx(t);
            if (xf)
                xf[dst] = n;
            else
                split_bf16(n, xh + dst, xl + dst);
            acc += static_cast<double>(n) * static_cast<double>(n);
        }
    }
    const double s = block_sum<256>(acc, sh);
    if (threadIdx.x == 0) w.partials[blockIdx.x] = s;
}

// Four consecutive gradient values as floats, one non-temporal 8-byte (bf16)
// or 16-byte (fp32) load of a stream read once.
template <typename GradT> __device__ __forceinline__ floatx4 load4_nt(const GradT *p);
template <> __device__ __forceinline__ floatx4 load4_nt<float>(const float *p) {
    return __builtin_nontemporal_load(as_global(reinterpret_cast<const floatx4 *>(p)));
}
template <> __device__ __forceinline__ floatx4 load4_nt<uint16_t>(const uint16_t *p) {
    const u32x2 h = __builtin_nontemporal_load(as_global(reinterpret_cast<const u32x2 *>(p)));
    return floatx4{__uint_as_float(h[0] << 16), __uint_as_float(h[0] & 0xffff0000u), __uint_as_float(h[1] << 16),
                   __uint_as_float(h[1] & 0xffff0000u)};
}

// Non-temporal vector load and store (streams touched once).
template <class T> __device__ __forceinline__ T ld_nt(const void *p) {
    return __builtin_nontemporal_load(as_global(reinterpret_cast<const T *>(p)));
}
template <class T> __device__ __forceinline__ void st_nt(void *p, T v) {
    __builtin_nontemporal_store(v, as_global(reinterpret_cast<T *>(p)));
}

// Stage 1, rows > cols: X = N^T.  64 x 64 tiles of W transposed through LDS so
// both the W-side and the X-side accesses are coalesced.  VEC (16-byte
// aligned G and M, cols a multiple of 4): in a tile wholly inside the matrix
// each thread moves four consecutive elements per access, on the W side four
// columns of one row (G, M read, M written), on the X side four consecutive
// W rows of one column, encoded into the pair together; tiles at the edge
// take the element path.  The LDS row stride of 65 floats keeps the row
// writes and the column reads free of bank conflicts.
template <typename GradT, bool VEC>
__global__ __launch_bounds__(256) void nesterov_tile_kernel(const MatDesc *__restrict__ descs,
                                                            Geom g, Work w, float mu,
                                                            int nesterov, int tiles_c,
                                                            int blocks_per_mat) {
    __shared__ float tile[64][65];
    __shared__ double sh[4];
    const int64_t e = blockIdx.x / blocks_per_mat;
    const int64_t t = blockIdx.x % blocks_per_mat;
    const int64_t i0 = (t / tiles_c) * 64;  // W row
    const int64_t j0 = (t % tiles_c) * 64;  // W col
    const MatDesc d = descs[e];
    const GradT *__restrict__ gp = static_cast<const GradT *>(d.grad);
    float *__restrict__ mp = d.mom;
    float *__restrict__ xf = w.xf ? w.xf + e * w.x_stride : nullptr;  // fp32 path
    uint16_t *__restrict__ xh = static_cast<uint16_t *>(w.xb) + e * w.x_stride;  // bf16 path
    uint8_t *__restrict__ xl = static_cast<uint8_t *>(w.xl) + e * w.x_stride;
    double acc = 0.0;
    if (VEC && i0 + 64 <= g.rows && j0 + 64 <= g.cols) {
        // all four rows' G and M are requested before any is used; every
        // global access is a non-temporal stream
        const int q4 = 4 * (threadIdx.x & 15), r16 = threadIdx.x >> 4;
        floatx4 gv[4], m[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t src = (i0 + 16 * r + r16) * g.cols + j0 + q4;
            gv[r] = load4_nt<GradT>(gp + src);
            m[r] = __builtin_nontemporal_load(as_global(reinterpret_cast<const floatx4 *>(mp + src)));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ii = 16 * r + r16;
            const int64_t src = (i0 + ii) * g.cols + j0 + q4;
            floatx4 m1;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                m1[q] = mu * m[r][q] + gv[r][q];
                const float n = nesterov ? (mu * m1[q] + gv[r][q]) : m1[q];
                acc += static_cast<double>(n) * static_cast<double>(n);
                tile[ii][q4 + q] = n;
            }
            __builtin_nontemporal_store(m1, as_global(reinterpret_cast<floatx4 *>(mp + src)));
        }
        __syncthreads();
        // X[j][i] = N[i][j]: lane (jj, c4) takes X row j0 + jj, columns i0 + c4 .. +3
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jj = 16 * r + r16;
            floatx4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = tile[q4 + q][jj];
            const int64_t off = (j0 + jj) * g.lp + i0 + q4;
            if (xf) {
                __builtin_nontemporal_store(v, as_global(reinterpret_cast<floatx4 *>(xf + off)));
            } else {
                u32x2 h;
                uint32_t l;
                split_bf16x4(v, &h, &l);
                __builtin_nontemporal_store(h, as_global(reinterpret_cast<u32x2 *>(xh + off)));
                __builtin_nontemporal_store(l, as_global(reinterpret_cast<uint32_t *>(xl + off)));
            }
        }
    } else {
        const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
        for (int r = 0; r < 16; ++r) {
            const int ii = ty + 4 * r;
            const int64_t i = i0 + ii, j = j0 + tx;
            float n = 0.0f;
            if (i < g.rows && j < g.cols) {
                const int64_t src = i * g.cols + j;
                const float gv = load_val<GradT>(gp, src);
                const float m1 = mu * mp[src] + gv;
                n = nesterov ? (mu * m1 + gv) : m1;
                mp[src] = m1;
                acc += static_cast<double>(n) * static_cast<double>(n);
            }
            tile[ii][tx] = n;
        }
        __syncthreads();
        // X[j][i] = N[i][j]: X row = W col (j0 + jj), X col = W row (i0 + tx)
        for (int r = 0; r < 16; ++r) {
            const int jj = ty + 4 * r;
            const int64_t xr = j0 + jj, xc = i0 + tx;
            if (xr < g.cols && xc < g.rows) {
                if (xf)
                    xf[xr * g.lp + xc] = tile[tx][jj];
                else
                    split_bf16(tile[tx][jj], xh + xr * g.lp + xc, xl + xr * g.lp + xc);
            }
        }
    }
    const double s = block_sum<256>(acc, sh);
    if (threadIdx.x == 0) w.partials[blockIdx.x] = s;
}

// ||N||^2 per matrix from its blocks' partial sums, in a fixed order.
__global__ __launch_bounds__(256) void norm_finalize_kernel(const MatDesc *__restrict__ descs,
                                                            Work w, int blocks_per_mat) {
    __shared__ double sh[4];
    const int64_t e = blockIdx.x;
    double acc = 0.0;
    for (int b = threadIdx.x; b < blocks_per_mat; b += 256) acc += w.partials[e * blocks_per_mat + b];
    const double s = block_sum<256>(acc, sh);
    if (threadIdx.x == 0) {
        w.nrm2[e] = s;
        w.call_nrm2[descs[e].call_index] = s;
        // The first step's fold factor.  An all-zero N gives 0, so X = 0 and
        // the update is decay only; a non-finite norm gives NaN everywhere
        // (IEEE propagation of an Inf or NaN in N); a norm outside the fold
        // range is applied by normalize_kernel instead.
        float f;
        if (s == 0.0)
            f = 0.0f;
        else if (!(s <= 1.7976931348623157e308))
            f = __builtin_nanf("");
        else if (prenormalize(s))
            f = 1.0f;
        else
            f = static_cast<float>(1.0 / sqrt(s));
        w.inv_norm[e] = f;
    }
}

// X_0 = N / ||N||_F over the padded sp x lp extent (zeros outside s x l), in
// place: fp32 in xf, or the pair (bf16 hi in xb, 8-bit residual in xl).  The
// factor 1/||N|| is formed in double and each element rounded once, so any
// finite nonzero norm is applied exactly (in fp32 it could over- or
// underflow); ||N|| = 0 gives X = 0 and a non-finite norm NaN.  The fp32 path
// (and the bf16 path with an empty schedule) runs it on every matrix;
// otherwise the bf16 path folds 1/||N|| into its first step and runs it only
// on the matrices prenormalize() selects (prenorm_only: the blocks of the
// others return at once).  Block (e, b) handles padded rows b, b + bpm, ...
__global__ __launch_bounds__(256) void normalize_kernel(Geom g, Work w, int blocks_per_mat, int prenorm_only) {
    const int64_t e = blockIdx.x / blocks_per_mat;
    const int64_t rb = blockIdx.x % blocks_per_mat;
    const double s = w.nrm2[e];
    if (prenorm_only && !prenormalize(s)) return;
    const double inv = s == 0.0 ? 0.0 : (s <= 1.7976931348623157e308 ? 1.0 / sqrt(s) : __builtin_nan(""));
    const bool split = w.xf == nullptr;
    float *__restrict__ xf = split ? nullptr : w.xf + e * w.x_stride;
    uint16_t *__restrict__ xh = static_cast<uint16_t *>(w.xb) + e * w.x_stride;
    uint8_t *__restrict__ xl = static_cast<uint8_t *>(w.xl) + e * w.x_stride;
    for (int64_t i = rb; i < g.sp; i += blocks_per_mat) {
        for (int64_t j = 4 * static_cast<int64_t>(threadIdx.x); j < g.lp; j += 4 * 256) {
            const int64_t off = i * g.lp + j;
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            if (i < g.s) {
                floatx4 n;
                if (split) {
                    // entries past column l of the N pair are never written: mask them
                    n = join_bf16x4(*reinterpret_cast<const u32x2 *>(xh + off),
                                    *reinterpret_cast<const uint32_t *>(xl + off));
                } else {
                    n = *reinterpret_cast<const floatx4 *>(xf + off);
                }
                for (int q = 0; q < 4; ++q)
                    v[q] = (j + q < g.l) ? static_cast<float>(static_cast<double>(n[q]) * inv) : 0.0f;
            }
            if (split) {
                u32x2 h;
                uint32_t l;
                split_bf16x4(v, &h, &l);
                *reinterpret_cast<u32x2 *>(xh + off) = h;
                *reinterpret_cast<uint32_t *>(xl + off) = l;
            } else {
                *reinterpret_cast<floatx4 *>(xf + off) = v;
            }
        }
    }
}

// Zeros the padding (outside s x l, inside sp x lp) of the pair (xb, xl)
// that the momentum pass leaves untouched.  Block (e, r) handles padded row
// row0 + r of matrix e: rows below s only hold padding when l < lp, so the
// launch covers them only then.  A row at or beyond s is padding whole and
// is cleared with 16-byte stores (rows start 256 elements apart from an
// aligned base).
__global__ __launch_bounds__(256) void pad_zero_kernel(Geom g, Work w, int64_t rows_per_mat, int64_t row0) {
    const int64_t e = blockIdx.x / rows_per_mat;
    const int64_t i = row0 + blockIdx.x % rows_per_mat;
    uint16_t *xh = static_cast<uint16_t *>(w.xb) + e * w.x_stride + i * g.lp;
    uint8_t *xl = static_cast<uint8_t *>(w.xl) + e * w.x_stride + i * g.lp;
    if (i >= g.s) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int64_t j = threadIdx.x; j < g.lp / 8; j += 256) reinterpret_cast<u32x4 *>(xh)[j] = z;
        for (int64_t j = threadIdx.x; j < g.lp / 16; j += 256) reinterpret_cast<u32x4 *>(xl)[j] = z;
        return;
    }
    for (int64_t j = g.l + threadIdx.x; j < g.lp; j += 256) {
        xh[j] = 0;
        xl[j] = 0;
    }
}

// ---------------------------------------------------------------------------
// Decay + update from a plain rows x cols fp32 X (the test hook's form).
template <typename ParamT>
__global__ __launch_bounds__(256) void update_plain_kernel(ParamT *__restrict__ p,
                                                           const float *__restrict__ x, int64_t n,
                                                           float dscale, float sscale,
                                                           const float *__restrict__ s_dev) {
    if (s_dev) sscale = *s_dev;
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
        const float wv = load_val<ParamT>(p, i);
        const float r = dscale * wv - sscale * x[i];
        store_val<ParamT>(p, i, r);
    }
}

// Decay + update from the workspace X (s x l, pitch lp, transposed when
// rows > cols), plus the optional ns_out copy in W's orientation.
template <typename ParamT>
__global__ __launch_bounds__(256) void update_from_work_kernel(const MatDesc *__restrict__ descs,
                                                               Geom g, Work w, float dscale,
                                                               float sscale, int tiles_c,
                                                               int blocks_per_mat) {
    __shared__ float tile[64][65];
    const int64_t e = blockIdx.x / blocks_per_mat;
    const int64_t t = blockIdx.x % blocks_per_mat;
    const int64_t i0 = (t / tiles_c) * 64;  // W row
    const int64_t j0 = (t % tiles_c) * 64;  // W col
    const MatDesc d = descs[e];
    ParamT *__restrict__ pp = static_cast<ParamT *>(d.param);
    const XView xv_{w.xf ? w.xf + e * w.x_stride : nullptr, static_cast<const uint16_t *>(w.xb) + e * w.x_stride,
                    static_cast<const uint8_t *>(w.xl) + e * w.x_stride};
    if (w.uscale) sscale = w.uscale[e];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    if (g.transposed) {
        // X row = W col
        for (int r = 0; r < 16; ++r) {
            const int jj = ty + 4 * r;
            const int64_t xr = j0 + jj, xc = i0 + tx;
            tile[jj][tx] = (xr < g.cols && xc < g.rows) ? xv_.at(xr * g.lp + xc) : 0.0f;
        }
        __syncthreads();
    }
    for (int r = 0; r < 16; ++r) {
        const int ii = ty + 4 * r;
        const int64_t i = i0 + ii, j = j0 + tx;
        if (i < g.rows && j < g.cols) {
            const float xv = g.transposed ? tile[tx][ii] : xv_.at(i * g.lp + j);
            const int64_t dst = i * g.cols + j;
            const float wv = load_val<ParamT>(pp, dst);
            store_val<ParamT>(pp, dst, dscale * wv - sscale * xv);
            if (d.ns_out) d.ns_out[dst] = xv;
        }
    }
}

// Decay + update from the bf16 workspace X when X has W's row layout (not
// transposed, l a multiple of 8, 16-byte aligned W and ns_out): 8 consecutive
// elements per lane, 16 + 8 bytes of X and 16 (bf16) or 32 (fp32) bytes of W
// in one load each, every access a non-temporal stream.  Same arithmetic as
// update_from_work_kernel.
template <typename ParamT>
__global__ __launch_bounds__(256) void update_from_work_vec_kernel(const MatDesc *__restrict__ descs, Geom g,
                                                                   Work w, float dscale, float sscale,
                                                                   int blocks_per_mat) {
    const int64_t e = blockIdx.x / blocks_per_mat;
    const int64_t q = static_cast<int64_t>(blockIdx.x % blocks_per_mat) * 256 + threadIdx.x;
    const int64_t gpr = g.l / 8;
    if (q >= g.s * gpr) return;
    const int64_t r = q / gpr, c = (q - r * gpr) * 8;
    if (w.uscale) sscale = w.uscale[e];
    const MatDesc d = descs[e];
    const int64_t xo = e * w.x_stride + r * g.lp + c;
    const u32x4 h = ld_nt<u32x4>(static_cast<const uint16_t *>(w.xb) + xo);
    const u32x2 l = ld_nt<u32x2>(static_cast<const uint8_t *>(w.xl) + xo);
    const uint32_t hw[4] = {h[0], h[1], h[2], h[3]};
    const uint32_t lw[2] = {l[0], l[1]};
    float xv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        xv[k] = join_bf16(static_cast<uint16_t>(hw[k >> 1] >> (16 * (k & 1))),
                          static_cast<uint8_t>(lw[k >> 2] >> (8 * (k & 3))));
    const int64_t dst = r * g.cols + c;
    if constexpr (sizeof(ParamT) == 2) {
        uint16_t *pw = static_cast<uint16_t *>(d.param) + dst;
        const u32x4 wv = ld_nt<u32x4>(pw);
        const uint32_t ww[4] = {wv[0], wv[1], wv[2], wv[3]};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float r0 = dscale * bf16_bits_to_float(static_cast<uint16_t>(ww[k])) - sscale * xv[2 * k];
            const float r1 = dscale * bf16_bits_to_float(static_cast<uint16_t>(ww[k] >> 16)) - sscale * xv[2 * k + 1];
            o[k] = static_cast<uint32_t>(float_to_bf16_bits(r0)) | (static_cast<uint32_t>(float_to_bf16_bits(r1)) << 16);
        }
        st_nt<u32x4>(pw, u32x4{o[0], o[1], o[2], o[3]});
    } else {
        float *pw = static_cast<float *>(d.param) + dst;
        const floatx4 a = ld_nt<floatx4>(pw), b = ld_nt<floatx4>(pw + 4);
        st_nt<floatx4>(pw, floatx4{dscale * a[0] - sscale * xv[0], dscale * a[1] - sscale * xv[1],
                                     dscale * a[2] - sscale * xv[2], dscale * a[3] - sscale * xv[3]});
        st_nt<floatx4>(pw + 4, floatx4{dscale * b[0] - sscale * xv[4], dscale * b[1] - sscale * xv[5],
                                         dscale * b[2] - sscale * xv[6], dscale * b[3] - sscale * xv[7]});
    }
    if (d.ns_out) {
        st_nt<floatx4>(d.ns_out + dst, floatx4{xv[0], xv[1], xv[2], xv[3]});
        st_nt<floatx4>(d.ns_out + dst + 4, floatx4{xv[4], xv[5], xv[6], xv[7]});
    }
}

// The same for a transposed matrix (X = W^T, so W row i is X column i): one
// 64 x 64 tile per block.  X rows j0 .. j0+63, columns i0 .. i0+63 are read
// 8 columns per load (16 + 8 bytes) into LDS, always inside the padded
// workspace (sp and lp are multiples of 256); W rows i0 .. i0+63 are then
// written 8 columns (W cols = X rows) per lane, with non-temporal global
// accesses.  Needs cols % 8 == 0 so that every 8-wide group of a W row is
// inside the matrix or wholly outside it.
template <typename ParamT>
__global__ __launch_bounds__(256) void update_from_work_tvec_kernel(const MatDesc *__restrict__ descs, Geom g,
                                                                    Work w, float dscale, float sscale,
                                                                    int tiles_c, int blocks_per_mat) {
    __shared__ float tile[64][65];
    const int64_t e = blockIdx.x / blocks_per_mat;
    const int64_t t = blockIdx.x % blocks_per_mat;
    const int64_t i0 = (t / tiles_c) * 64;  // W row = X column
    const int64_t j0 = (t % tiles_c) * 64;  // W column = X row
    if (w.uscale) sscale = w.uscale[e];
    const uint16_t *xh = static_cast<const uint16_t *>(w.xb) + e * w.x_stride;
    const uint8_t *xl = static_cast<const uint8_t *>(w.xl) + e * w.x_stride;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int q = threadIdx.x + 256 * half;
        const int row = q >> 3, cg = (q & 7) * 8;
        const int64_t xo = (j0 + row) * g.lp + i0 + cg;
        const u32x4 h = ld_nt<u32x4>(xh + xo);
        const u32x2 l = ld_nt<u32x2>(xl + xo);
        const uint32_t hw[4] = {h[0], h[1], h[2], h[3]};
        const uint32_t lw[2] = {l[0], l[1]};
#pragma unroll
        for (int k = 0; k < 8; ++k)
            tile[row][cg + k] = join_bf16(static_cast<uint16_t>(hw[k >> 1] >> (16 * (k & 1))),
                                          static_cast<uint8_t>(lw[k >> 2] >> (8 * (k & 3))));
    }
    __syncthreads();
    const MatDesc d = descs[e];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int q = threadIdx.x + 256 * half;
        const int wr = q >> 3, wc = (q & 7) * 8;
        const int64_t i = i0 + wr, j = j0 + wc;
        if (i >= g.rows || j >= g.cols) continue;
        float xv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) xv[k] = tile[wc + k][wr];
        const int64_t dst = i * g.cols + j;
        if constexpr (sizeof(ParamT) == 2) {
            uint16_t *pw = static_cast<uint16_t *>(d.param) + dst;
            const u32x4 wv = ld_nt<u32x4>(pw);
            const uint32_t ww[4] = {wv[0], wv[1], wv[2], wv[3]};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float r0 = dscale * bf16_bits_to_float(static_cast<uint16_t>(ww[k])) - sscale * xv[2 * k];
                const float r1 =
                    dscale * bf16_bits_to_float(static_cast<uint16_t>(ww[k] >> 16)) - sscale * xv[2 * k + 1];
                o[k] = static_cast<uint32_t>(float_to_bf16_bits(r0)) |
                       (static_cast<uint32_t>(float_to_bf16_bits(r1)) << 16);
            }
            st_nt<u32x4>(pw, u32x4{o[0], o[1], o[2], o[3]});
        } else {
            float *pw = static_cast<float *>(d.param) + dst;
            const floatx4 a = ld_nt<floatx4>(pw), b = ld_nt<floatx4>(pw + 4);
            st_nt<floatx4>(pw, floatx4{dscale * a[0] - sscale * xv[0], dscale * a[1] - sscale * xv[1],
                                         dscale * a[2] - sscale * xv[2], dscale * a[3] - sscale * xv[3]});
            st_nt<floatx4>(pw + 4, floatx4{dscale * b[0] - sscale * xv[4], dscale * b[1] - sscale * xv[5],
                                             dscale * b[2] - sscale * xv[6], dscale * b[3] - sscale * xv[7]});
        }
        if (d.ns_out) {
            st_nt<floatx4>(d.ns_out + dst, floatx4{xv[0], xv[1], xv[2], xv[3]});
            st_nt<floatx4>(d.ns_out + dst + 4, floatx4{xv[4], xv[5], xv[6], xv[7]});
        }
    }
}

// Unit-RMS mode, first pass: per-block fp64 sums of X^2 over the valid s x l
// region of each matrix (rows b, b + blocks_per_mat, ...).  The square of an
// fp32 value is exact in fp64, so only the order of the additions differs
// from a serial sum.  The bf16 pair (hi, residual) is read 8 columns at a
// time (16 + 8 bytes) when the row length allows it.
__global__ __launch_bounds__(256) void x_sumsq_kernel(Geom g, Work w, const float *__restrict__ x_override,
                                                      int blocks_per_mat) {
    __shared__ double sh[4];
    const int64_t e = blockIdx.x / blocks_per_mat;
    const int b = static_cast<int>(blockIdx.x % blocks_per_mat);
    double acc = 0.0;
    const float *xf = x_override ? x_override : (w.xf ? w.xf + e * w.x_stride : nullptr);
    if (xf) {
        for (int64_t r = b; r < g.s; r += blocks_per_mat)
            for (int64_t c = threadIdx.x; c < g.l; c += 256) {
                const double v = xf[r * g.lp + c];
                acc += v * v;
            }
    } else {
        const uint16_t *xh = static_cast<const uint16_t *>(w.xb) + e * w.x_stride;
        const uint8_t *xl = static_cast<const uint8_t *>(w.xl) + e * w.x_stride;
        const bool vec = (g.l % 8 == 0) && (g.lp % 8 == 0) && (w.x_stride % 8 == 0);
        for (int64_t r = b; r < g.s; r += blocks_per_mat) {
            const int64_t row = r * g.lp;
            if (vec) {
                for (int64_t c = 8 * threadIdx.x; c < g.l; c += 8 * 256) {
                    const uint4 h = *reinterpret_cast<const uint4 *>(xh + row + c);
                    const uint2 l = *reinterpret_cast<const uint2 *>(xl + row + c);
                    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
                    const uint32_t lw[2] = {l.x, l.y};
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const uint16_t hk = static_cast<uint16_t>(hw[k >> 1] >> (16 * (k & 1)));
                        const uint8_t lk = static_cast<uint8_t>(lw[k >> 2] >> (8 * (k & 3)));
                        const double v = join_bf16(hk, lk);
                        acc += v * v;
                    }
                }
            } else {
                for (int64_t c = threadIdx.x; c < g.l; c += 256) {
                    const double v = join_bf16(xh[row + c], xl[row + c]);
                    acc += v * v;
                }
            }
        }
    }
    const double t = block_sum<256>(acc, sh);
    if (threadIdx.x == 0) w.partials[e * blocks_per_mat + b] = t;
}

// Unit-RMS mode, second pass: s_e = fl32(lr * (gsq / sqrt(sum X^2))),
// gsq = gamma * sqrt(rows * cols); a zero X gives s_e = 0.
__global__ __launch_bounds__(256) void unit_rms_finalize_kernel(Work w, int blocks_per_mat, double lr, double gsq,
                                                                float *__restrict__ out) {
    __shared__ double sh[4];
    const int64_t e = blockIdx.x;
    double acc = 0.0;
    for (int b = threadIdx.x; b < blocks_per_mat; b += 256) acc += w.partials[e * blocks_per_mat + b];
    const double ss = block_sum<256>(acc, sh);
    if (threadIdx.x == 0) out[e] = (ss == 0.0) ? 0.0f : static_cast<float>(lr * (gsq / sqrt(ss)));
}

// Copy of the workspace X into a plain rows x cols output (muon_ns_only).
__global__ __launch_bounds__(256) void export_x_kernel(Geom g, XView x, float *__restrict__ out, int tiles_c) {
    __shared__ float tile[64][65];
    const int64_t i0 = (blockIdx.x / tiles_c) * 64;
    const int64_t j0 = (blockIdx.x % tiles_c) * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    if (g.transposed) {
        for (int r = 0; r < 16; ++r) {
            const int jj = ty + 4 * r;
            const int64_t xr = j0 + jj, xc = i0 + tx;
            tile[jj][tx] = (xr < g.cols && xc < g.rows) ? x.at(xr * g.lp + xc) : 0.0f;
        }
        __syncthreads();
    }
    for (int r = 0; r < 16; ++r) {
        const int ii = ty + 4 * r;
        const int64_t i = i0 + ii, j = j0 + tx;
        if (i < g.rows && j < g.cols) out[i * g.cols + j] = g.transposed ? tile[tx][ii] : x.at(i * g.lp + j);
    }
}

// Copy of a plain fp32 N into the momentum-free first stage (muon_ns_only):
// X = N in s x l orientation plus the per-block sums of N^2.
__global__ __launch_bounds__(256) void import_n_kernel(Geom g, const float *__restrict__ n_in, Work w,
                                                       int tiles_c) {
    __shared__ float tile[64][65];
    __shared__ double sh[4];
    const int64_t i0 = (blockIdx.x / tiles_c) * 64;
    const int64_t j0 = (blockIdx.x % tiles_c) * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    double acc = 0.0;
    for (int r = 0; r < 16; ++r) {
        const int ii = ty + 4 * r;
        const int64_t i = i0 + ii, j = j0 + tx;
        float v = 0.0f;
        if (i < g.rows && j < g.cols) {
            v = n_in[i * g.cols + j];
            acc += static_cast<double>(v) * static_cast<double>(v);
            if (!g.transposed) store_n(w, i * g.lp + j, v);
        }
        tile[ii][tx] = v;
    }
    if (g.transposed) {
        __syncthreads();
        for (int r = 0; r < 16; ++r) {
            const int jj = ty + 4 * r;
            const int64_t xr = j0 + jj, xc = i0 + tx;
            if (xr < g.cols && xc < g.rows) store_n(w, xr * g.lp + xc, tile[tx][jj]);
        }
    }
    const double s = block_sum<256>(acc, sh);
    if (threadIdx.x == 0) w.partials[blockIdx.x] = s;
}

// Operands of a single product stage (muon_ns_stage): a plain fp32 s x l X
// into the workspace pair (hi, residual) over the padded sp x lp extent
// (zeros outside s x l), and a plain fp32 s x s matrix into a bf16 sp x sp
// operand (zeros outside), and a bf16 sp x sp operand back out as fp32.
__global__ __launch_bounds__(256) void import_pair_kernel(Geom g, const float *__restrict__ x, Work w) {
    const int64_t i = blockIdx.x;  // padded row
    uint16_t *xh = static_cast<uint16_t *>(w.xb) + i * g.lp;
    uint8_t *xl = static_cast<uint8_t *>(w.xl) + i * g.lp;
    for (int64_t j = threadIdx.x; j < g.lp; j += 256) {
        const float v = (i < g.s && j < g.l) ? x[i * g.l + j] : 0.0f;
        split_bf16(__builtin_canonicalizef(v), xh + j, xl + j);
    }
}

__global__ __launch_bounds__(256) void import_bf16_square_kernel(int64_t s, int64_t sp, const float *__restrict__ m,
                                                                 uint16_t *__restrict__ dst) {
    const int64_t i = blockIdx.x;
    for (int64_t j = threadIdx.x; j < sp; j += 256)
        dst[i * sp + j] = float_to_bf16_bits((i < s && j < s) ? m[i * s + j] : 0.0f);
}

__global__ __launch_bounds__(256) void export_bf16_square_kernel(int64_t s, int64_t sp, const uint16_t *__restrict__ src,
                                                                 float *__restrict__ out) {
    const int64_t i = blockIdx.x;
    for (int64_t j = threadIdx.x; j < s; j += 256) out[i * s + j] = bf16_bits_to_float(src[i * sp + j]);
}

// ---------------------------------------------------------------------------
// AdamW over a table of tensors.  Block b processes elements
// [(b - first_block[k]) * 1024, ...) of tensor k, k found by binary search.
struct AdamwDesc {
    float *param;
    const float *grad;
    float *m;
    float *v;
    int64_t numel;
    int64_t first_block;
};

__global__ __launch_bounds__(256) void adamw_kernel(const AdamwDesc *__restrict__ descs, int count,
                                                    AdamwScalars k) {
    const int64_t b = blockIdx.x;
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (descs[mid].first_block <= b) lo = mid; else hi = mid - 1;
    }
    const AdamwDesc d = descs[lo];
    const int64_t base = (b - d.first_block) * 1024;
    const bool vec = ((reinterpret_cast<uintptr_t>(d.param) | reinterpret_cast<uintptr_t>(d.grad) |
                       reinterpret_cast<uintptr_t>(d.m) | reinterpret_cast<uintptr_t>(d.v)) & 15) == 0;
    const int64_t i = base + threadIdx.x * 4;
    if (vec && i + 4 <= d.numel) {
        // every vector is read and written once: non-temporal streams
        floatx4 p = __builtin_nontemporal_load(as_global(reinterpret_cast<const floatx4 *>(d.param + i)));
        const floatx4 gg = __builtin_nontemporal_load(as_global(reinterpret_cast<const floatx4 *>(d.grad + i)));
        floatx4 m = __builtin_nontemporal_load(as_global(reinterpret_cast<const floatx4 *>(d.m + i)));
        floatx4 v = __builtin_nontemporal_load(as_global(reinterpret_cast<const floatx4 *>(d.v + i)));
        for (int q = 0; q < 4; ++q) {
            const float p1 = k.decay * p[q];
            const float m1 = k.beta1 * m[q] + k.one_minus_beta1 * gg[q];
            const float v1 = k.beta2 * v[q] + (k.one_minus_beta2 * gg[q]) * gg[q];
            const float mh = __fdiv_rn(m1, k.bias_corr1);
            const float vh = __fdiv_rn(v1, k.bias_corr2);
            const float den = sqrt_rn(vh) + k.eps;
            p[q] = p1 - k.lr * __fdiv_rn(mh, den);
            m[q] = m1;
            v[q] = v1;
        }
        __builtin_nontemporal_store(p, as_global(reinterpret_cast<floatx4 *>(d.param + i)));
        __builtin_nontemporal_store(m, as_global(reinterpret_cast<floatx4 *>(d.m + i)));
        __builtin_nontemporal_store(v, as_global(reinterpret_cast<floatx4 *>(d.v + i)));
    } else {
        for (int q = 0; q < 4; ++q) {
            const int64_t ii = i + q;
            if (ii >= d.numel) break;
            const float p1 = k.decay * d.param[ii];
            const float m1 = k.beta1 * d.m[ii] + k.one_minus_beta1 * d.grad[ii];
            const float gv = d.grad[ii];
            const float v1 = k.beta2 * d.v[ii] + (k.one_minus_beta2 * gv) * gv;
            const float mh = __fdiv_rn(m1, k.bias_corr1);
            const float vh = __fdiv_rn(v1, k.bias_corr2);
            const float den = sqrt_rn(vh) + k.eps;
            d.param[ii] = p1 - k.lr * __fdiv_rn(mh, den);
            d.m[ii] = m1;
            d.v[ii] = v1;
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming probe (a measurement aid, no step of the method): `reads` source
// streams and `writes` destination streams of nvec 16-byte vectors each,
// stream k starting k * pitch vectors into its buffer, every vector read and
// written once, coalesced and non-temporal, one vector per lane and stream
// (a workgroup per 256 vectors); each written vector depends on all the
// vectors read by its lane, so no read can be dropped.  Its rate is the HBM
// ceiling for a kernel with the same read : write mix.
template <int R, int W>
__global__ __launch_bounds__(256) void stream_probe_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                           int64_t nvec, int64_t pitch) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < nvec;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        u32x4 v[R];
#pragma unroll
        for (int r = 0; r < R; ++r) v[r] = __builtin_nontemporal_load(as_global(src + i + r * pitch));
        u32x4 x = v[0];
#pragma unroll
        for (int r = 1; r < R; ++r) x ^= v[r];
#pragma unroll
        for (int k = 0; k < W; ++k) {
            __builtin_nontemporal_store(x, as_global(dst + i + k * pitch));
            x[0] += 1u;
        }
    }
}

template <int R, int W>
static hipError_t launch_probe_rw(const void *src, void *dst, int64_t nvec, int64_t pitch, hipStream_t st) {
    const int64_t blocks = std::min<int64_t>((nvec + 255) / 256, 0x7fffffff);
    hipLaunchKernelGGL((stream_probe_kernel<R, W>), dim3(static_cast<unsigned>(std::max<int64_t>(blocks, 1))),
                       dim3(256), 0, st, static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), nvec, pitch);
    return hipGetLastError();
}

hipError_t launch_stream_probe(const void *src, void *dst, int64_t nvec, int64_t pitch, int reads, int writes,
                               hipStream_t st) {
    // the mixes of the elementwise kernels: momentum 6 : 7, AdamW 4 : 3, update 5 : 2, copy 1 : 1
    if (reads == 6 && writes == 7) return launch_probe_rw<6, 7>(src, dst, nvec, pitch, st);
    if (reads == 4 && writes == 3) return launch_probe_rw<4, 3>(src, dst, nvec, pitch, st);
    if (reads == 5 && writes == 2) return launch_probe_rw<5, 2>(src, dst, nvec, pitch, st);
    if (reads == 1 && writes == 1) return launch_probe_rw<1, 1>(src, dst, nvec, pitch, st);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Host launchers.

int nesterov_blocks_per_mat(const Geom &g, int *tiles_c) {
    if (g.transposed) {
        *tiles_c = static_cast<int>((g.cols + 63) / 64);
        return static_cast<int>(((g.rows + 63) / 64) * *tiles_c);
    }
    // kMomElems consecutive elements per block (64 x 64 = one tile's worth)
    *tiles_c = 0;
    return static_cast<int>((g.rows * g.cols + kMomElems - 1) / kMomElems);
}

hipError_t launch_nesterov(const MatDesc *descs, int nmat, const Geom &g, const Work &w, float mu,
                           int nesterov, int grad_bf16, bool vec_ok, hipStream_t st) {
    int tc = 0;
    const int bpm = nesterov_blocks_per_mat(g, &tc);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(bpm) * nmat)), block(256);
    const bool vec = vec_ok && (g.cols % 4 == 0) && (g.lp % 4 == 0);
    if (g.transposed && vec) {
        if (grad_bf16)
            hipLaunchKernelGGL((nesterov_tile_kernel<uint16_t, true>), grid, block, 0, st, descs, g, w, mu, nesterov, tc, bpm);
        else
            hipLaunchKernelGGL((nesterov_tile_kernel<float, true>), grid, block, 0, st, descs, g, w, mu, nesterov, tc, bpm);
    } else if (g.transposed) {
        if (grad_bf16)
            hipLaunchKernelGGL((nesterov_tile_kernel<uint16_t, false>), grid, block, 0, st, descs, g, w, mu, nesterov, tc, bpm);
        else
            hipLaunchKernelGGL((nesterov_tile_kernel<float, false>), grid, block, 0, st, descs, g, w, mu, nesterov, tc, bpm);
    } else if (vec) {
        if (grad_bf16)
            hipLaunchKernelGGL((nesterov_rows_kernel<uint16_t, true>), grid, block, 0, st, descs, g, w, mu, nesterov, bpm);
        else
            hipLaunchKernelGGL((nesterov_rows_kernel<float, true>), grid, block, 0, st, descs, g, w, mu, nesterov, bpm);
    } else {
        if (grad_bf16)
            hipLaunchKernelGGL((nesterov_rows_kernel<uint16_t, false>), grid, block, 0, st, descs, g, w, mu, nesterov, bpm);
        else
            hipLaunchKernelGGL((nesterov_rows_kernel<float, false>), grid, block, 0, st, descs, g, w, mu, nesterov, bpm);
    }
    return hipGetLastError();
}

hipError_t launch_norm_finalize(const MatDesc *descs, int nmat, const Work &w, int blocks_per_mat,
                                hipStream_t st) {
    hipLaunchKernelGGL(norm_finalize_kernel, dim3(nmat), dim3(256), 0, st, descs, w, blocks_per_mat);
    return hipGetLastError();
}

int import_n_blocks(const Geom &g) {
    const int tc = static_cast<int>((g.cols + 63) / 64);
    return static_cast<int>(((g.rows + 63) / 64) * tc);
}

hipError_t launch_import_n(const float *n_in, const Geom &g, const Work &w, hipStream_t st) {
    const int tc = static_cast<int>((g.cols + 63) / 64);
    hipLaunchKernelGGL(import_n_kernel, dim3(import_n_blocks(g)), dim3(256), 0, st, g, n_in, w, tc);
    return hipGetLastError();
}

hipError_t launch_normalize(int nmat, const Geom &g, const Work &w, int prenorm_only, hipStream_t st) {
    // about 16k blocks in all (at least one per matrix, at most one per row)
    const int bpm = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(g.sp, 16384 / std::max(nmat, 1))));
    hipLaunchKernelGGL(normalize_kernel, dim3(static_cast<unsigned>(static_cast<int64_t>(bpm) * nmat)), dim3(256), 0,
                       st, g, w, bpm, prenorm_only);
    return hipGetLastError();
}

hipError_t launch_pad_zero(int nmat, const Geom &g, const Work &w, hipStream_t st) {
    const int64_t row0 = g.l < g.lp ? 0 : g.s;  // rows below s hold padding only when l < lp
    const int64_t rows = g.sp - row0;
    if (rows <= 0 || nmat <= 0) return hipSuccess;
    hipLaunchKernelGGL(pad_zero_kernel, dim3(static_cast<unsigned>(rows * nmat)), dim3(256), 0, st, g, w, rows, row0);
    return hipGetLastError();
}
hipError_t launch_update_plain(void *param, int param_bf16, const float *x, int64_t n, float d,
                               float s, const float *s_dev, hipStream_t st) {
    int64_t nb = (n + 255) / 256;
    if (nb > 65536) nb = 65536;
    if (nb < 1) nb = 1;
    if (param_bf16)
        hipLaunchKernelGGL(update_plain_kernel<uint16_t>, dim3(static_cast<unsigned>(nb)), dim3(256), 0, st,
                           static_cast<uint16_t *>(param), x, n, d, s, s_dev);
    else
        hipLaunchKernelGGL(update_plain_kernel<float>, dim3(static_cast<unsigned>(nb)), dim3(256), 0, st,
                           static_cast<float *>(param), x, n, d, s, s_dev);
    return hipGetLastError();
}

hipError_t launch_unit_rms_scale(int nmat, const Geom &g, const Work &w, const float *x_override,
                                 int blocks_per_mat, double lr, double gsq, float *out, hipStream_t st) {
    hipLaunchKernelGGL(x_sumsq_kernel, dim3(static_cast<unsigned>(static_cast<int64_t>(blocks_per_mat) * nmat)),
                       dim3(256), 0, st, g, w, x_override, blocks_per_mat);
    hipLaunchKernelGGL(unit_rms_finalize_kernel, dim3(static_cast<unsigned>(nmat)), dim3(256), 0, st, w,
                       blocks_per_mat, lr, gsq, out);
    return hipGetLastError();
}

hipError_t launch_update_from_work(const MatDesc *descs, int nmat, const Geom &g, const Work &w,
                                   int param_bf16, float d, float s, bool aligned16, hipStream_t st) {
    const int64_t vbpm = (g.s * (g.l / 8) + 255) / 256;
    if (aligned16 && !w.xf && !g.transposed && g.l % 8 == 0 && g.lp % 8 == 0 && w.x_stride % 8 == 0 &&
        vbpm * nmat <= 0x7fffffff) {
        const int bpm = static_cast<int>(vbpm);
        const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(bpm) * nmat));
        if (param_bf16)
            hipLaunchKernelGGL(update_from_work_vec_kernel<uint16_t>, grid, dim3(256), 0, st, descs, g, w, d, s, bpm);
        else
            hipLaunchKernelGGL(update_from_work_vec_kernel<float>, grid, dim3(256), 0, st, descs, g, w, d, s, bpm);
        return hipGetLastError();
    }
    const int tc = static_cast<int>((g.cols + 63) / 64);
    if (aligned16 && !w.xf && g.transposed && g.cols % 8 == 0) {
        const int bpm = static_cast<int>(((g.rows + 63) / 64) * tc);
        const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(bpm) * nmat));
        if (param_bf16)
            hipLaunchKernelGGL(update_from_work_tvec_kernel<uint16_t>, grid, dim3(256), 0, st, descs, g, w, d, s, tc,
                               bpm);
        else
            hipLaunchKernelGGL(update_from_work_tvec_kernel<float>, grid, dim3(256), 0, st, descs, g, w, d, s, tc,
                               bpm);
        return hipGetLastError();
    }
    const int bpm = static_cast<int>(((g.rows + 63) / 64) * tc);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(bpm) * nmat));
    if (param_bf16)
        hipLaunchKernelGGL(update_from_work_kernel<uint16_t>, grid, dim3(256), 0, st, descs, g, w, d, s, tc, bpm);
    else
        hipLaunchKernelGGL(update_from_work_kernel<float>, grid, dim3(256), 0, st, descs, g, w, d, s, tc, bpm);
    return hipGetLastError();
}

hipError_t launch_import_pair(const Geom &g, const float *x, const Work &w, hipStream_t st) {
    hipLaunchKernelGGL(import_pair_kernel, dim3(static_cast<unsigned>(g.sp)), dim3(256), 0, st, g, x, w);
    return hipGetLastError();
}

hipError_t launch_import_bf16_square(int64_t s, int64_t sp, const float *m, void *dst, hipStream_t st) {
    hipLaunchKernelGGL(import_bf16_square_kernel, dim3(static_cast<unsigned>(sp)), dim3(256), 0, st, s, sp, m,
                       static_cast<uint16_t *>(dst));
    return hipGetLastError();
}

hipError_t launch_export_bf16_square(int64_t s, int64_t sp, const void *src, float *out, hipStream_t st) {
    hipLaunchKernelGGL(export_bf16_square_kernel, dim3(static_cast<unsigned>(s)), dim3(256), 0, st, s, sp,
                       static_cast<const uint16_t *>(src), out);
    return hipGetLastError();
}

hipError_t launch_export_x(const Geom &g, const Work &w, float *out, hipStream_t st) {
    const int tc = static_cast<int>((g.cols + 63) / 64);
    const int nb = static_cast<int>(((g.rows + 63) / 64) * tc);
    const XView x{w.xf, static_cast<const uint16_t *>(w.xb), static_cast<const uint8_t *>(w.xl)};
    hipLaunchKernelGGL(export_x_kernel, dim3(nb), dim3(256), 0, st, g, x, out, tc);
    return hipGetLastError();
}

int64_t adamw_blocks(int64_t numel) { return (numel + 1023) / 1024; }

hipError_t launch_adamw(const void *descs_dev, int count, int64_t total_blocks, const AdamwScalars &k,
                        hipStream_t st) {
    // Grid y-splitting is not needed: 2^31-1 blocks cover 2.2e12 elements.
    hipLaunchKernelGGL(adamw_kernel, dim3(static_cast<unsigned>(total_blocks)), dim3(256), 0, st,
                       static_cast<const AdamwDesc *>(descs_dev), count, k);
    return hipGetLastError();
}

size_t adamw_desc_size() { return sizeof(AdamwDesc); }

void adamw_fill_desc(void *dst, float *param, const float *grad, float *m, float *v, int64_t numel,
                     int64_t first_block) {
    AdamwDesc d{param, grad, m, v, numel, first_block};
    *static_cast<AdamwDesc *>(dst) = d;
}

}  // namespace muon
