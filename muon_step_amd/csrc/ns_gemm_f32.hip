// Grouped Newton-Schulz products with fp32 operands (the MUON_NS_F32 path and
// thin matrices) on gfx950 matrix cores (v_mfma_f32_32x32x2_f32).  The bf16
// path lives in ns_gemm_bf16.hip.
//
// One Newton-Schulz step X <- a X + b (X X^T) X + c (X X^T)^2 X (DeepSeek-V4
// book ch. 6 §3; the deep-dive page, "Newton-Schulz 迭代") is evaluated as
// three dense contractions over every matrix of a same-shape group, one
// launch each:
//
//   GRAM  : A = X X^T         s x s, K = l.  Only lower-triangle tiles are
//                             computed (A is symmetric); each is written to
//                             A (fp32) and, mirrored, to the operand copy.
//   POLY  : B = b A + c A A   s x s, K = s.  A A is symmetric too: lower tiles
//                             only, written mirrored.  Row i of A serves as
//                             column i, so both operands are K-contiguous.
//   APPLY : X' = a X + B X    s x l, K = s.  The aX term is added in fp32 from
//                             the fp32 master X.  The last step instead
//                             writes W <- d W - s_scale X' (and O'_t).
//
// Tiles are 256 x 256 with a K-step of 128 bytes per row (64 bf16 or 32
// fp32), staged global -> registers -> LDS (double-buffered, XOR-swizzled in
// 16-byte chunks so MFMA fragment reads are bank-conflict free), 8 waves of
// 128 x 64.  The B X product needs X with K (= the row index) contiguous; the
// transposition happens in registers while staging.  bf16 operands use
// v_mfma_f32_32x32x16_bf16, fp32 operands v_mfma_f32_32x32x2_f32; both
// accumulate in fp32.  Block ids are renumbered so one matrix's tiles share
// an XCD (and its L2).
#include "common.hpp"
#include "kernels.hpp"

namespace muon {
namespace f32path {

enum Kind { GRAM = 0, POLY = 1, APPLY = 2 };

constexpr int BM = 256, BN = 256, NT = 512;
constexpr int WAVES_N = 4, WM = 128, WN = 64;
constexpr int MI = WM / 32, NI = WN / 32;
constexpr int TILE_BYTES = 256 * 128;           // 256 rows x 128-byte K slab
constexpr int SMEM_BYTES = 4 * TILE_BYTES;      // 2 stages x (P, Q)

// 16-byte chunk index of (row, chunk) inside a 256 x 8-chunk tile.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

template <bool BF16> struct ElemT;
template <> struct ElemT<true> { using T = uint16_t; static constexpr int BK = 64; };
template <> struct ElemT<false> { using T = float; static constexpr int BK = 32; };

template <bool BF16>
__device__ __forceinline__ void store_operand(void *base, int64_t idx, float v);
template <> __device__ __forceinline__ void store_operand<true>(void *base, int64_t idx, float v) {
    static_cast<uint16_t *>(base)[idx] = float_to_bf16_bits(v);
}
template <> __device__ __forceinline__ void store_operand<false>(void *base, int64_t idx, float v) {
    static_cast<float *>(base)[idx] = v;
}

// Rows [row0, row0+256) x one 128-byte K slab of a row-major matrix whose row
// pitch is ld_bytes, into 4 chunks per thread.
__device__ __forceinline__ void load_rows(u32x4 (&r)[4], const char *base, int64_t ld_bytes, int tid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = tid + NT * q;
        const int row = c >> 3, ch = c & 7;
        r[q] = *reinterpret_cast<const u32x4 *>(base + row * ld_bytes + ch * 16);
    }
}

__device__ __forceinline__ void store_rows(char *lds, const u32x4 (&r)[4], int tid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = tid + NT * q;
        reinterpret_cast<u32x4 *>(lds)[swz(c >> 3, c & 7)] = r[q];
    }
}

// K rows x 256 columns of a row-major matrix (the X operand of B X), to be
// stored with K contiguous.  bf16: each thread owns 8 K-rows x 4 columns;
// fp32: 4 K-rows x 4 columns.
template <bool BF16> struct TransStage;

template <> struct TransStage<true> {
    u32x2 in[8];
    __device__ __forceinline__ void load(const char *base, int64_t ld_bytes, int tid) {
        const int kb = tid >> 6, nb = tid & 63;
#pragma unroll
        for (int r = 0; r < 8; ++r)
            in[r] = *reinterpret_cast<const u32x2 *>(base + (kb * 8 + r) * ld_bytes + nb * 8);
    }
    __device__ __forceinline__ void store(char *lds, int tid) const {
        const int kb = tid >> 6, nb = tid & 63;
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
            u32x4 o;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo = in[2 * p][nn >> 1], hi = in[2 * p + 1][nn >> 1];
                o[p] = (nn & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            reinterpret_cast<u32x4 *>(lds)[swz(nb * 4 + nn, kb)] = o;
        }
    }
};

template <> struct TransStage<false> {
    u32x4 in[4];
    __device__ __forceinline__ void load(const char *base, int64_t ld_bytes, int tid) {
        const int kb = tid >> 6, nb = tid & 63;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            in[r] = *reinterpret_cast<const u32x4 *>(base + (kb * 4 + r) * ld_bytes + nb * 16);
    }
    __device__ __forceinline__ void store(char *lds, int tid) const {
        const int kb = tid >> 6, nb = tid & 63;
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
            u32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = in[r][nn];
            reinterpret_cast<u32x4 *>(lds)[swz(nb * 4 + nn, kb)] = o;
        }
    }
};

template <bool BF16>
__device__ __forceinline__ void mma_slab(floatx16 (&acc)[MI][NI], const char *pl, const char *ql, int wm,
                                         int wn, int lane) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int ch = 2 * ks + (lane >> 5);
        u32x4 a[MI], b[NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            a[mi] = reinterpret_cast<const u32x4 *>(pl)[swz(wm * WM + mi * 32 + (lane & 31), ch)];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
            b[ni] = reinterpret_cast<const u32x4 *>(ql)[swz(wn * WN + ni * 32 + (lane & 31), ch)];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                if constexpr (BF16) {
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a[mi]), __builtin_bit_cast(bf16x8, b[ni]), acc[mi][ni], 0, 0, 0);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            __uint_as_float(a[mi][q]), __uint_as_float(b[ni][q]), acc[mi][ni], 0, 0, 0);
                }
            }
    }
}

__device__ __forceinline__ void tri_decode(int64_t t, int *ti, int *tj) {
    int i = static_cast<int>((sqrt(8.0 * static_cast<double>(t) + 1.0) - 1.0) * 0.5);
    while (static_cast<int64_t>(i + 1) * (i + 2) / 2 <= t) ++i;
    while (static_cast<int64_t>(i) * (i + 1) / 2 > t) --i;
    *ti = i;
    *tj = static_cast<int>(t - static_cast<int64_t>(i) * (i + 1) / 2);
}

template <int KIND, bool BF16, int PARAM_BF16>
__global__ __launch_bounds__(NT, 2) void ns_gemm_kernel(const MatDesc *__restrict__ descs, Geom g, Work w,
                                                        NsStep p, int64_t tiles_per_mat, int64_t nblocks) {
    using T = typename ElemT<BF16>::T;
    constexpr int BK = ElemT<BF16>::BK;
    constexpr int ES = static_cast<int>(sizeof(T));
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int64_t L = xcd_swizzle(blockIdx.x, nblocks);
    const int64_t e = L / tiles_per_mat;
    const int64_t t = L % tiles_per_mat;
    int ti, tj;
    if (KIND == APPLY) {
        const int nti = static_cast<int>(g.sp / BM);
        tj = static_cast<int>(t / nti);
        ti = static_cast<int>(t % nti);
    } else {
        tri_decode(t, &ti, &tj);
    }

    // Operand sources.  P supplies output rows, Q output columns.
    const char *psrc;
    const char *qsrc;
    int64_t ld_p, ld_q, kdim;
    if (KIND == GRAM) {
        const char *x = static_cast<const char *>(BF16 ? w.xb : static_cast<void *>(w.xf)) + e * w.x_stride * ES;
        ld_p = ld_q = g.lp * ES;
        psrc = x + static_cast<int64_t>(ti) * BM * ld_p;
        qsrc = x + static_cast<int64_t>(tj) * BN * ld_q;
        kdim = g.lp;
    } else if (KIND == POLY) {
        const char *a = static_cast<const char *>(w.ab) + e * w.a_stride * ES;
        ld_p = ld_q = g.sp * ES;
        psrc = a + static_cast<int64_t>(ti) * BM * ld_p;
        qsrc = a + static_cast<int64_t>(tj) * BN * ld_q;
        kdim = g.sp;
    } else {
        const char *b = static_cast<const char *>(w.bb) + e * w.a_stride * ES;
        const char *x = static_cast<const char *>(BF16 ? w.xb : static_cast<void *>(w.xf)) + e * w.x_stride * ES;
        ld_p = g.sp * ES;
        ld_q = g.lp * ES;
        psrc = b + static_cast<int64_t>(ti) * BM * ld_p;
        qsrc = x + static_cast<int64_t>(tj) * BN * ES;  // column offset; K rows advance below
        kdim = g.sp;
    }

    floatx16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    u32x4 pr[4], qr[4];
    TransStage<BF16> qt;
    const int nk = static_cast<int>(kdim / BK);
    auto load_stage = [&](int kt) {
        load_rows(pr, psrc + static_cast<int64_t>(kt) * 128, ld_p, tid);
        if (KIND == APPLY)
            qt.load(qsrc + static_cast<int64_t>(kt) * BK * ld_q, ld_q, tid);
        else
            load_rows(qr, qsrc + static_cast<int64_t>(kt) * 128, ld_q, tid);
    };
    auto store_stage = [&](int buf) {
        char *pl = smem + buf * 2 * TILE_BYTES;
        store_rows(pl, pr, tid);
        if (KIND == APPLY)
            qt.store(pl + TILE_BYTES, tid);
        else
            store_rows(pl + TILE_BYTES, qr, tid);
    };

    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_stage(kt + 1);
        const char *pl = smem + cur * 2 * TILE_BYTES;
        mma_slab<BF16>(acc, pl, pl + TILE_BYTES, wm, wn, lane);
        if (kt + 1 < nk) store_stage(cur ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    // acc[mi][ni][r] holds output (row, col) of the tile:
    //   row = wm*WM + mi*32 + 8*(r/4) + 4*(lane/32) + r%4,  col = wn*WN + ni*32 + lane%32
    const int64_t row_base = static_cast<int64_t>(ti) * BM + wm * WM + 4 * (lane >> 5);
    const int64_t col_base = static_cast<int64_t>(tj) * BN + wn * WN + (lane & 31);
    if (KIND == GRAM || KIND == POLY) {
        float *af = w.af + e * w.a_stride;
        void *dst = (KIND == GRAM) ? w.ab : w.bb;
        const int64_t off = e * w.a_stride;
        const bool mirror = ti != tj;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t gi = row_base + mi * 32 + 8 * (r >> 2) + (r & 3);
                    const int64_t gj = col_base + ni * 32;
                    float v = acc[mi][ni][r];
                    if (KIND == GRAM) {
                        af[gi * g.sp + gj] = v;
                    } else {
                        v = p.b * af[gi * g.sp + gj] + p.c * v;
                    }
                    store_operand<BF16>(dst, off + gi * g.sp + gj, v);
                    if (mirror) store_operand<BF16>(dst, off + gj * g.sp + gi, v);
                }
    } else {
        const float *xin = w.xf + e * w.x_stride;
        if (!p.final_update) {
            float *xout = w.xf_next + e * w.x_stride;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t gi = row_base + mi * 32 + 8 * (r >> 2) + (r & 3);
                        const int64_t gj = col_base + ni * 32;
                        const int64_t idx = gi * g.lp + gj;
                        float v = p.a * xin[idx] + acc[mi][ni][r];
                        if (gi >= g.s || gj >= g.l) v = 0.0f;
                        xout[idx] = v;
                        if (BF16) store_operand<true>(w.xb_next, e * w.x_stride + idx, v);
                    }
        } else {
            const MatDesc d = descs[e];
            T *unused = nullptr;
            (void)unused;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t gi = row_base + mi * 32 + 8 * (r >> 2) + (r & 3);
                        const int64_t gj = col_base + ni * 32;
                        if (gi < g.s && gj < g.l) {
                            const float v = p.a * xin[gi * g.lp + gj] + acc[mi][ni][r];
                            const int64_t widx = g.transposed ? (gj * g.cols + gi) : (gi * g.cols + gj);
                            if (PARAM_BF16) {
                                uint16_t *pp = static_cast<uint16_t *>(d.param);
                                const float wv = bf16_bits_to_float(pp[widx]);
                                pp[widx] = float_to_bf16_bits(p.dscale * wv - p.sscale * v);
                            } else {
                                float *pp = static_cast<float *>(d.param);
                                pp[widx] = p.dscale * pp[widx] - p.sscale * v;
                            }
                            if (d.ns_out) d.ns_out[widx] = v;
                        }
                    }
        }
    }
}

template <int KIND, bool BF16, int PB>
static hipError_t launch_one(const MatDesc *descs, int nmat, const Geom &g, const Work &w, const NsStep &p,
                             hipStream_t st) {
    static bool attr_set = false;
    auto kern = ns_gemm_kernel<KIND, BF16, PB>;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, SMEM_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    int64_t tiles;
    if (KIND == APPLY) {
        tiles = (g.sp / BM) * (g.lp / BN);
    } else {
        const int64_t nt = g.sp / BM;
        tiles = nt * (nt + 1) / 2;
    }
    const int64_t nblocks = tiles * nmat;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nblocks)), dim3(NT), SMEM_BYTES, st, descs, g, w, p,
                       tiles, nblocks);
    return hipGetLastError();
}

}  // namespace f32path

hipError_t launch_ns_stage_f32(int kind, const MatDesc *descs, int nmat, const Geom &g, const Work &w,
                               const NsStep &p, hipStream_t st) {
    using namespace f32path;
    if (kind == GRAM) return launch_one<GRAM, false, 0>(descs, nmat, g, w, p, st);
    if (kind == POLY) return launch_one<POLY, false, 0>(descs, nmat, g, w, p, st);
    if (p.final_update && p.param_bf16) return launch_one<APPLY, false, 1>(descs, nmat, g, w, p, st);
    return launch_one<APPLY, false, 0>(descs, nmat, g, w, p, st);
}

}  // namespace muon
