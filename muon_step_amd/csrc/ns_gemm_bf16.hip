// Grouped Newton-Schulz products with bf16 operands on gfx950 matrix cores.
//
// One Newton-Schulz step X <- a X + b (X X^T) X + c (X X^T)^2 X (DeepSeek-V4
// book ch. 6 §3; the deep-dive page, "Newton-Schulz 迭代") is evaluated as
// three dense contractions over every matrix of a same-shape group, one
// launch each:
//
//   GRAM  : A = X X^T         s x s, K = l.  Only lower-triangle tiles are
//                             computed (A is symmetric); each is written to
//                             A (fp32) and, mirrored, to the bf16 operand copy.
//   POLY  : B = b A + c A A   s x s, K = s.  A A is symmetric too: lower tiles
//                             only, written mirrored.  Row i of A serves as
//                             column i, so both operands are K-contiguous.
//   APPLY : X' = a X + B X    s x l, K = s.  The aX term is added in fp32 from
//                             the fp32 master X.  The last step instead
//                             writes W <- d W - s_scale X' (and O'_t).
//
// Data movement: 256 x 256 output tiles, 8 waves (two per SIMD) of 128 x 64,
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  Operand slabs of 32 k are
// copied global -> LDS by the direct 16-byte-per-lane DMA
// (global_load_lds_dwordx4) into a 4-stage ring of LDS tiles, three stages in
// flight while one is consumed; each wave waits on its own outstanding-load
// counter, then one barrier per stage.
// The LDS layouts are XOR-swizzled so that every 16-lane phase of a fragment
// read touches all 64 banks once.  The X operand of B X is stored as it lies
// in memory (k rows, n contiguous) and read with ds_read_b64_tr_b16, which
// hands each lane four consecutive k of one column.  Block ids are renumbered
// so one matrix's tiles share an XCD (and its L2).
#include "common.hpp"
#include "kernels.hpp"

namespace muon {
namespace bf16path {

enum Kind { GRAM = 0, POLY = 1, APPLY = 2 };

constexpr int BM = 256, BN = 256, NT = 512;
constexpr int NWAVES = NT / 64, WAVES_N = 4, WM = 128, WN = 64;
constexpr int MI = WM / 32, NI = WN / 32;
constexpr int BK = 32;                  // k per pipeline stage
constexpr int TILE_BYTES = 16384;       // 256 rows x 32 bf16, or 32 k-rows x 256 bf16
constexpr int BLOCKS_PER_WAVE = TILE_BYTES / 1024 / NWAVES;  // 1 KB DMA blocks per wave per operand
constexpr int LOADS_PER_STAGE = 2 * BLOCKS_PER_WAVE;         // DMA instructions per wave per stage

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_tr;
typedef __attribute__((address_space(3))) bf16x4_tr lds_bf16x4_t;

// One LDS object per stage and operand: the compiler tracks DMA writes per
// object, so reading one stage never waits on the DMA filling another.
__shared__ __attribute__((aligned(1024))) char lds_p0[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char lds_p1[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char lds_p2[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char lds_p3[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char lds_q0[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char lds_q1[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char lds_q2[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char lds_q3[TILE_BYTES];

template <int S> __device__ __forceinline__ char *lds_p() {
    if constexpr (S == 0) return lds_p0;
    else if constexpr (S == 1) return lds_p1;
    else if constexpr (S == 2) return lds_p2;
    else return lds_p3;
}
template <int S> __device__ __forceinline__ char *lds_q() {
    if constexpr (S == 0) return lds_q0;
    else if constexpr (S == 1) return lds_q1;
    else if constexpr (S == 2) return lds_q2;
    else return lds_q3;
}

// s_waitcnt with vmcnt = N and the LDS/export counters left alone.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt at their maxima: no wait).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Same, and also wait for all of this wave's outstanding LDS reads.
template <int N> __device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// K-contiguous tile (256 rows x 64 bytes): 16-byte chunk c of row r lives at
// chunk c ^ ((r >> 2) & 3), so 16 consecutive rows reading one chunk cover
// 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kc_offset(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

// N-contiguous tile (32 k-rows x 512 bytes): 64-byte block b of k-row r lives
// at block b ^ (r & 3), so four consecutive k-rows of one block cover 256 B.
__device__ __forceinline__ int nc_offset(int krow, int byte) {
    return krow * 512 + ((((byte >> 6) ^ (krow & 3))) << 6) + (byte & 63);
}

// DMA of one stage: rows [0, 256) x bytes [kt*64, kt*64 + 64) of a
// K-contiguous source into `dst`.  Wave w fills BLOCKS_PER_WAVE consecutive
// 1 KB blocks (16 rows each); lane i lands at block byte 16 i, i.e. row i/4,
// swizzled chunk i%4.
__device__ __forceinline__ void dma_kc(char *dst, const char *src, int64_t ld, int kt, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < BLOCKS_PER_WAVE; ++j) {
        const int blk = wave * BLOCKS_PER_WAVE + j;
        const int row = blk * 16 + (lane >> 2);
        const int chunk = (lane & 3) ^ ((row >> 2) & 3);
        const char *g = src + row * ld + kt * 64 + chunk * 16;
        __builtin_amdgcn_global_load_lds(g, (lds_void_t *)(dst + blk * 1024), 16, 0, 0);
    }
}

// DMA of one stage of the B X operand: k-rows [kt*32, kt*32 + 32) x 512 bytes
// (256 columns) of row-major X into `dst`.  1 KB block b holds k-rows 2b and
// 2b+1; lane i lands at byte 16 i.
__device__ __forceinline__ void dma_nc(char *dst, const char *src, int64_t ld, int kt, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < BLOCKS_PER_WAVE; ++j) {
        const int blk = wave * BLOCKS_PER_WAVE + j;
        const int krow = blk * 2 + (lane >> 5);
        const int u = lane & 31;
        const int byte = ((((u >> 2) ^ (krow & 3))) << 6) + ((u & 3) << 4);
        const char *g = src + (static_cast<int64_t>(kt) * BK + krow) * ld + byte;
        __builtin_amdgcn_global_load_lds(g, (lds_void_t *)(dst + blk * 1024), 16, 0, 0);
    }
}

// The epilogue of the B X product reuses the LDS ring: wave w owns one 16 KB
// array (64 rows x 64 fp32 of its 128 x 64 output block at a time).
__device__ __forceinline__ char *epi_region(int wave) {
    switch (wave) {
        case 0: return lds_p0;
        case 1: return lds_p1;
        case 2: return lds_p2;
        case 3: return lds_p3;
        case 4: return lds_q0;
        case 5: return lds_q1;
        case 6: return lds_q2;
        default: return lds_q3;
    }
}

// 16-byte chunk c of row r (256-byte rows) lives at chunk c ^ (r & 15), so
// sixteen consecutive rows reading one chunk cover all 64 banks.
__device__ __forceinline__ int epi_offset(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

// DMA of 64 rows x 64 fp32 (256 bytes per row) starting at `src` (row pitch
// ld bytes) into the wave's region: 16 instructions of 4 rows each; lane i
// lands at byte 16 i of its 1 KB block, i.e. row i/16, swizzled chunk i%16.
__device__ __forceinline__ void dma_epi(char *dst, const char *src, int64_t ld, int lane) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int row = 4 * t + (lane >> 4);
        const int chunk = (lane & 15) ^ (row & 15);
        __builtin_amdgcn_global_load_lds(src + row * ld + chunk * 16, (lds_void_t *)(dst + t * 1024), 16, 0, 0);
    }
}

template <int KIND, int S>
__device__ __forceinline__ void issue_stage(const char *psrc, int64_t ld_p, const char *qsrc, int64_t ld_q, int kt,
                                            int wave, int lane) {
    dma_kc(lds_p<S>(), psrc, ld_p, kt, wave, lane);
    if constexpr (KIND == APPLY)
        dma_nc(lds_q<S>(), qsrc, ld_q, kt, wave, lane);
    else
        dma_kc(lds_q<S>(), qsrc, ld_q, kt, wave, lane);
}

// Fragments of one 16-k substep: MI A-fragments and NI B-fragments (8 bf16 =
// 16 bytes each per lane).
struct Frags {
    u32x4 a[MI];
    u32x4 b[NI];
};

// Reads substep ks (0 or 1) of the stage in slot S.
template <int KIND, int S>
__device__ __forceinline__ void read_frags(Frags &f, int ks, int wm, int wn, int lane) {
    const char *pl = lds_p<S>();
    const char *ql = lds_q<S>();
    const int chunk = 2 * ks + (lane >> 5);  // k = 8*chunk .. 8*chunk+7 of this stage
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int row = wm * WM + mi * 32 + (lane & 31);
        f.a[mi] = *reinterpret_cast<const u32x4 *>(pl + kc_offset(row, chunk));
    }
    if constexpr (KIND == APPLY) {
        // Lane j of each 16-lane group supplies k-row kbase + j/4, columns
        // n0 + 4(j%4) .. +3; lane i then holds X[kbase .. kbase+3][n0 + i].
        const int grp = lane >> 4, j = lane & 15;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int n0 = wn * WN + ni * 32 + 16 * (grp & 1);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int krow = 16 * ks + 8 * (grp >> 1) + 4 * r + (j >> 2);
                const int byte = (n0 + 4 * (j & 3)) * 2;
                const bf16x4_tr t =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(ql + nc_offset(krow, byte)));
                const u32x2 tt = __builtin_bit_cast(u32x2, t);
                f.b[ni][2 * r] = tt[0];
                f.b[ni][2 * r + 1] = tt[1];
            }
        }
    } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int row = wn * WN + ni * 32 + (lane & 31);
            f.b[ni] = *reinterpret_cast<const u32x4 *>(ql + kc_offset(row, chunk));
        }
    }
}

// acc[mi][ni] += A-fragment x B-fragment.  SWAP multiplies the operands the
// other way round (the Q fragment as the MFMA's first operand), which leaves
// the transposed 32 x 32 block in the accumulator: each lane then holds four
// consecutive output columns of one output row, so the epilogue can move
// 16 bytes per access.
template <bool SWAP>
__device__ __forceinline__ void mma_frags(floatx16 (&acc)[MI][NI], const Frags &f) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            if constexpr (SWAP)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.b[ni]),
                                                                      __builtin_bit_cast(bf16x8, f.a[mi]),
                                                                      acc[mi][ni], 0, 0, 0);
            else
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[mi]),
                                                                      __builtin_bit_cast(bf16x8, f.b[ni]),
                                                                      acc[mi][ni], 0, 0, 0);
        }
}

// One pipeline step: stage kt (slot S) is consumed while up to WAIT/LPS later
// stages may still be in flight; with ISSUE the DMA of stage kt+3 refills the
// slot that stage kt-1 used, which every wave finished before this barrier.
template <int KIND, int S, int WAIT, bool ISSUE>
__device__ __forceinline__ void pipeline_step(floatx16 (&acc)[MI][NI], const char *psrc, int64_t ld_p,
                                              const char *qsrc, int64_t ld_q, int kt, int wave, int wm, int wn,
                                              int lane) {
    wait_vmcnt<WAIT>();
    stage_barrier();
    if constexpr (ISSUE) issue_stage<KIND, (S + 3) & 3>(psrc, ld_p, qsrc, ld_q, kt + 3, wave, lane);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        Frags f;
        read_frags<KIND, S>(f, ks, wm, wn, lane);
        mma_frags<KIND == APPLY>(acc, f);
    }
}

template <int KIND>
__device__ __forceinline__ void main_loop(floatx16 (&acc)[MI][NI], const char *psrc, int64_t ld_p, const char *qsrc,
                                          int64_t ld_q, int nk, int wave, int wm, int wn, int lane) {
    // Before step kt, stages kt, kt+1, kt+2 may be outstanding (2 x LPS newer
    // loads allowed); the last four steps drain the ring.
    constexpr int W2 = 2 * LOADS_PER_STAGE, W1 = LOADS_PER_STAGE;
    issue_stage<KIND, 0>(psrc, ld_p, qsrc, ld_q, 0, wave, lane);
    issue_stage<KIND, 1>(psrc, ld_p, qsrc, ld_q, 1, wave, lane);
    issue_stage<KIND, 2>(psrc, ld_p, qsrc, ld_q, 2, wave, lane);
    int kt = 0;
    for (; kt < nk - 4; kt += 4) {
        pipeline_step<KIND, 0, W2, true>(acc, psrc, ld_p, qsrc, ld_q, kt, wave, wm, wn, lane);
        pipeline_step<KIND, 1, W2, true>(acc, psrc, ld_p, qsrc, ld_q, kt + 1, wave, wm, wn, lane);
        pipeline_step<KIND, 2, W2, true>(acc, psrc, ld_p, qsrc, ld_q, kt + 2, wave, wm, wn, lane);
        pipeline_step<KIND, 3, W2, true>(acc, psrc, ld_p, qsrc, ld_q, kt + 3, wave, wm, wn, lane);
    }
    pipeline_step<KIND, 0, W2, true>(acc, psrc, ld_p, qsrc, ld_q, kt, wave, wm, wn, lane);
    pipeline_step<KIND, 1, W2, false>(acc, psrc, ld_p, qsrc, ld_q, kt + 1, wave, wm, wn, lane);
    pipeline_step<KIND, 2, W1, false>(acc, psrc, ld_p, qsrc, ld_q, kt + 2, wave, wm, wn, lane);
    pipeline_step<KIND, 3, 0, false>(acc, psrc, ld_p, qsrc, ld_q, kt + 3, wave, wm, wn, lane);
}

__device__ __forceinline__ void tri_decode(int64_t t, int *ti, int *tj) {
    int i = static_cast<int>((sqrt(8.0 * static_cast<double>(t) + 1.0) - 1.0) * 0.5);
    while (static_cast<int64_t>(i + 1) * (i + 2) / 2 <= t) ++i;
    while (static_cast<int64_t>(i) * (i + 1) / 2 > t) --i;
    *ti = i;
    *tj = static_cast<int>(t - static_cast<int64_t>(i) * (i + 1) / 2);
}

template <int KIND, int PARAM_BF16>
__global__ __launch_bounds__(NT, 2) void ns_gemm_bf16_kernel(const MatDesc *__restrict__ descs, Geom g, Work w,
                                                             NsStep p, int64_t tiles_per_mat, int64_t nblocks) {
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
        const char *x = static_cast<const char *>(w.xb) + e * w.x_stride * 2;
        ld_p = ld_q = g.lp * 2;
        psrc = x + static_cast<int64_t>(ti) * BM * ld_p;
        qsrc = x + static_cast<int64_t>(tj) * BN * ld_q;
        kdim = g.lp;
    } else if (KIND == POLY) {
        const char *a = static_cast<const char *>(w.ab) + e * w.a_stride * 2;
        ld_p = ld_q = g.sp * 2;
        psrc = a + static_cast<int64_t>(ti) * BM * ld_p;
        qsrc = a + static_cast<int64_t>(tj) * BN * ld_q;
        kdim = g.sp;
    } else {
        const char *b = static_cast<const char *>(w.bb) + e * w.a_stride * 2;
        const char *x = static_cast<const char *>(w.xb) + e * w.x_stride * 2;
        ld_p = g.sp * 2;
        ld_q = g.lp * 2;
        psrc = b + static_cast<int64_t>(ti) * BM * ld_p;
        qsrc = x + static_cast<int64_t>(tj) * BN * 2;  // column offset; k rows advance per stage
        kdim = g.sp;
    }

    floatx16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    // kdim is a multiple of 256, so nk is a multiple of 8 (>= 8).
    const int nk = static_cast<int>(kdim / BK);
    main_loop<KIND>(acc, psrc, ld_p, qsrc, ld_q, nk, wave, wm, wn, lane);

    // ---------------------------------------------------------------- epilogue
    // GRAM / POLY: acc[mi][ni][r] holds output (row, col) of the tile:
    //   row = wm*WM + mi*32 + 8*(r/4) + 4*(lane/32) + r%4,  col = wn*WN + ni*32 + lane%32
    const int64_t row_base = static_cast<int64_t>(ti) * BM + wm * WM + 4 * (lane >> 5);
    const int64_t col_base = static_cast<int64_t>(tj) * BN + wn * WN + (lane & 31);
    if (KIND == GRAM || KIND == POLY) {
        float *af = w.af + e * w.a_stride;
        uint16_t *dst = static_cast<uint16_t *>(KIND == GRAM ? w.ab : w.bb) + e * w.a_stride;
        const bool mirror = ti != tj;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int64_t gi0 = row_base + mi * 32 + 8 * r4;
                    const int64_t gj = col_base + ni * 32;
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t gi = gi0 + q;
                        v[q] = acc[mi][ni][4 * r4 + q];
                        if (KIND == GRAM)
                            af[gi * g.sp + gj] = v[q];
                        else
                            v[q] = p.b * af[gi * g.sp + gj] + p.c * v[q];
                        dst[gi * g.sp + gj] = float_to_bf16_bits(v[q]);
                    }
                    if (mirror) {
                        // rows gi0..gi0+3 of column gj become 4 consecutive columns of row gj
                        u32x2 pk;
                        pk[0] = pack_bf16x2(v[0], v[1]);
                        pk[1] = pack_bf16x2(v[2], v[3]);
                        *reinterpret_cast<u32x2 *>(dst + gj * g.sp + gi0) = pk;
                    }
                }
    } else {
        // Swapped product: acc[mi][ni][4*c4 + q] holds output row
        //   m = wm*WM + mi*32 + lane%32,  columns n = wn*WN + ni*32 + 8*c4 + 4*(lane/32) + q, q = 0..3
        // The fp32 X the aX term needs is staged through LDS in two halves of
        // 64 rows, each wave loading its own 64 x 64 slice with the DMA (all
        // of it in flight at once), then read back in the accumulator layout.
        const float *xin = w.xf + e * w.x_stride;
        const int64_t row0 = static_cast<int64_t>(ti) * BM + wm * WM;  // first output row of this wave
        const int64_t col0 = static_cast<int64_t>(tj) * BN + wn * WN;  // first output column
        char *reg = epi_region(wave);
        wait_lgkm0();
        stage_barrier();  // every wave is done with the operand ring
        // The descriptor (param, ns_out) is needed only by the fused update.
        MatDesc d{};
        if (p.final_update) d = descs[e];
        const bool vec_w = !g.transposed && (g.cols % 4 == 0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            dma_epi(reg, reinterpret_cast<const char *>(xin + (row0 + 64 * h) * g.lp + col0), g.lp * 4, lane);
            wait_vmcnt<0>();
#pragma unroll
            for (int mh = 0; mh < 2; ++mh) {
                const int mi = 2 * h + mh;
                const int lrow = mh * 32 + (lane & 31);
                const int64_t gi = row0 + 64 * h + lrow;
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4) {
                        const int lcol = ni * 32 + 8 * c4 + 4 * (lane >> 5);
                        const int64_t gj = col0 + lcol;
                        const floatx4 x = *reinterpret_cast<const floatx4 *>(reg + epi_offset(lrow, lcol >> 2));
                        floatx4 v;
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = p.a * x[q] + acc[mi][ni][4 * c4 + q];
                        if (!p.final_update) {
                            const int64_t idx = gi * g.lp + gj;
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (gi >= g.s || gj + q >= g.l) v[q] = 0.0f;
                            *reinterpret_cast<floatx4 *>(w.xf_next + e * w.x_stride + idx) = v;
                            u32x2 pk;
                            pk[0] = pack_bf16x2(v[0], v[1]);
                            pk[1] = pack_bf16x2(v[2], v[3]);
                            *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(w.xb_next) + e * w.x_stride + idx) = pk;
                        } else if (gi < g.s) {
                            if (vec_w && gj + 3 < g.l) {
                                // W row gi, columns gj .. gj+3
                                const int64_t widx = gi * g.cols + gj;
                                if (PARAM_BF16) {
                                    uint16_t *pp = static_cast<uint16_t *>(d.param) + widx;
                                    const u32x2 wv = *reinterpret_cast<const u32x2 *>(pp);
                                    u32x2 o;
                                    o[0] = pack_bf16x2(p.dscale * __uint_as_float(wv[0] << 16) - p.sscale * v[0],
                                                       p.dscale * __uint_as_float(wv[0] & 0xffff0000u) - p.sscale * v[1]);
                                    o[1] = pack_bf16x2(p.dscale * __uint_as_float(wv[1] << 16) - p.sscale * v[2],
                                                       p.dscale * __uint_as_float(wv[1] & 0xffff0000u) - p.sscale * v[3]);
                                    *reinterpret_cast<u32x2 *>(pp) = o;
                                } else {
                                    float *pp = static_cast<float *>(d.param) + widx;
                                    const floatx4 wv = *reinterpret_cast<const floatx4 *>(pp);
                                    floatx4 o;
#pragma unroll
                                    for (int q = 0; q < 4; ++q) o[q] = p.dscale * wv[q] - p.sscale * v[q];
                                    *reinterpret_cast<floatx4 *>(pp) = o;
                                }
                                if (d.ns_out) *reinterpret_cast<floatx4 *>(d.ns_out + widx) = v;
                            } else {
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    if (gj + q >= g.l) continue;
                                    const int64_t widx = g.transposed ? ((gj + q) * g.cols + gi) : (gi * g.cols + gj + q);
                                    if (PARAM_BF16) {
                                        uint16_t *pp = static_cast<uint16_t *>(d.param);
                                        const float wv = bf16_bits_to_float(pp[widx]);
                                        pp[widx] = float_to_bf16_bits(p.dscale * wv - p.sscale * v[q]);
                                    } else {
                                        float *pp = static_cast<float *>(d.param);
                                        pp[widx] = p.dscale * pp[widx] - p.sscale * v[q];
                                    }
                                    if (d.ns_out) d.ns_out[widx] = v[q];
                                }
                            }
                        }
                    }
            }
            if (h == 0) wait_lgkm0();  // the slice's LDS reads are done before the next DMA overwrites it
        }
    }
}

template <int KIND, int PB>
static hipError_t launch_one(const MatDesc *descs, int nmat, const Geom &g, const Work &w, const NsStep &p,
                             hipStream_t st) {
    int64_t tiles;
    if (KIND == APPLY) {
        tiles = (g.sp / BM) * (g.lp / BN);
    } else {
        const int64_t nt = g.sp / BM;
        tiles = nt * (nt + 1) / 2;
    }
    const int64_t nblocks = tiles * nmat;
    hipLaunchKernelGGL((ns_gemm_bf16_kernel<KIND, PB>), dim3(static_cast<unsigned>(nblocks)), dim3(NT), 0, st,
                       descs, g, w, p, tiles, nblocks);
    return hipGetLastError();
}

}  // namespace bf16path

hipError_t launch_ns_stage_bf16(int kind, const MatDesc *descs, int nmat, const Geom &g, const Work &w,
                                const NsStep &p, hipStream_t st) {
    using namespace bf16path;
    if (kind == GRAM) return launch_one<GRAM, 0>(descs, nmat, g, w, p, st);
    if (kind == POLY) return launch_one<POLY, 0>(descs, nmat, g, w, p, st);
    if (p.final_update && p.param_bf16) return launch_one<APPLY, 1>(descs, nmat, g, w, p, st);
    return launch_one<APPLY, 0>(descs, nmat, g, w, p, st);
}

}  // namespace muon
