// Grouped Newton-Schulz products with bf16 operands on gfx950 matrix cores.
//
// One Newton-Schulz step X <- a X + b (X X^T) X + c (X X^T)^2 X (DeepSeek-V4
// book ch. 6 §3; the deep-dive page, "Newton-Schulz 迭代") is evaluated as
// three dense contractions over every matrix of a same-shape group, one
// launch each:
//
//   GRAM  : A = X X^T         s x s, K = l.  Only lower-triangle tiles are
//                             computed (A is symmetric), and of a diagonal
//                             tile only the blocks on and below its diagonal;
//                             A is written in bf16, with the mirror.
//   POLY  : B = b A + c A A   s x s, K = s.  A A is symmetric too: the same
//                             triangle, written mirrored.  Row i of A serves
//                             as column i, so both operands are K-contiguous.
//   APPLY : X' = a X + B X    s x l, K = s.  The aX term is added in fp32 from
//                             X = X_hi + X_lo.  The last step instead
//                             writes W <- d W - s_scale X' (and O'_t).
//
// Data movement.  All three products use 256 x 256 tiles, one workgroup of 8
// waves per CU (two per SIMD), each wave owning a 128 x 64 block computed with
// v_mfma_f32_32x32x16_bf16 into fp32 accumulators.  Operand slabs of 64 k (one
// 128-byte line per row) are copied global -> LDS by the 16-byte-per-lane DMA
// (global_load_lds_dwordx4) into a ring of two stages (128 KB); a diagonal tile
// of GRAM or POLY, whose output rows and columns are the same rows of the
// operand, fills a slot with 128 k of those rows instead of the same 64 k twice
// (CfgDiag).  Every product is followed by at most one fragment read for the
// next 16-k substep; the last of a stage's substeps also refills the slot just
// read with the stage after next, so LDS reads and copies run under the MFMAs;
// one barrier per stage, before its last substep.  The LDS layouts are
// XOR-swizzled so that every 16-lane phase of a fragment read touches all 64
// banks once.  The X operand of B X is stored as it lies in memory (k rows, n
// contiguous) and read with ds_read_b64_tr_b16, which hands each lane four
// consecutive k of one column.  The products are issued with the operands
// swapped, so each lane's accumulators hold four consecutive columns of one
// output row; every epilogue stages its block through LDS in rounds of 32 rows
// and stores whole rows (GRAM/POLY also store the block's columns as rows of
// the mirrored tile; APPLY moves 6 bytes per output element: X_hi and its 8-bit
// residual X_lo in and out; the fused update of a bf16 W brings W's rows by DMA
// too).  K loops stop at the true length rounded to 128 (the padding is zero).
// Block ids are renumbered so one matrix's tiles share an XCD (and its L2).
// Tiles that would run as a launch's last, partial wave (every tile, for a Gram
// or A^2 of a group too small to fill half a wave) may instead run split over K
// ranges whose fp32 partial tiles a reduce sums in a fixed order and finishes
// as the epilogue would (sym_reduce_kernel, apply_reduce_kernel).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace muon {
namespace bf16path {

enum Kind { GRAM = 0, POLY = 1, APPLY = 2 };

// Tile geometry shared by the three products: 256 x 256 output tiles, 8
// waves (two per SIMD, one workgroup per CU), each owning a 128 x 64 block,
// and a ring of two 64-k stages (128 KB of LDS).  64 k of bf16 is one 128-byte
// line per row, so every DMA instruction moves whole lines: DMA that moves
// half lines (32-k stages) runs at half the rate through the L1 path.
struct Cfg {
    static constexpr int NT = 512, NWAVES = NT / 64;
    static constexpr int BM = 256, BN = 256;
    static constexpr int WM = 128, WN = 64, MI = WM / 32, NI = WN / 32;
    static constexpr int WAVES_N = BN / WN, WAVES_M = BM / WM;
    static_assert(WAVES_N * WAVES_M == NWAVES, "wave grid");
    static constexpr int STAGES = 2;
    static constexpr int BK = 64;                      // k per stage
    static constexpr int SUBSTEPS = BK / 16;           // 16-k MFMA substeps per stage
    static constexpr int ROWB = BK * 2;                // bytes of one K-contiguous row per slab
    static constexpr int KT_BYTES = ROWB;              // bytes a K-contiguous operand advances per stage
    static constexpr int P_BYTES = BM * ROWB;          // 256 rows x 64 bf16
    static constexpr int Q_BYTES = BN * ROWB;          // BN rows x 64 bf16, or 64 k-rows x BN bf16
    static constexpr int SLOT_BYTES = P_BYTES + Q_BYTES;
    static constexpr int QROW = BN * 2;                // bytes of one k-row of an N-contiguous Q tile
    static constexpr int P_BLOCKS = P_BYTES / 1024 / NWAVES;  // 1 KB DMA blocks per wave and stage
    static constexpr int Q_BLOCKS = Q_BYTES / 1024 / NWAVES;
    static constexpr int LPS = P_BLOCKS + Q_BLOCKS;    // DMA instructions per wave per stage
    static constexpr int EPI_BYTES = 8192;             // epilogue staging per wave and round
    static constexpr int EPI_ROWS = EPI_BYTES / 256;   // rows of 64 fp32 per staging round
    static constexpr int NM = MI * NI;                 // MFMAs per wave and 16-k substep
    static constexpr int NF = MI + NI;                 // fragments per wave and substep
    static constexpr bool MFMA = true;                 // the wave's products are issued
    static constexpr bool DIAG = false;                // products selected by Src::mmask
    static constexpr bool PACKED = false;              // a slot holds 128 k of one operand (CfgDiag)
};

// The K loop of a GRAM or POLY wave whose 128 output rows all lie in the zero
// padding beyond s (last tile row when s is not a multiple of 256): it keeps its
// share of the copies, reads and barriers but issues no products (its
// accumulators stay zero, which is their value), so the other wave on its
// SIMD has the matrix core to itself.
struct CfgIdle : Cfg {
    static constexpr bool MFMA = false;
};

// The K loop of a diagonal tile of GRAM or POLY: only the 32 x 32 blocks on
// and below the diagonal (36 of 64) are needed, the rest is their mirror.  The
// waves take their 128 x 64 blocks in a permuted order and issue only the
// needed products (Src::mmask), so that the two waves sharing a SIMD (w and
// w + 4) hold 8 + 0, 8 + 0, 7 + 3 and 7 + 3 products per substep instead of
// 8 + 8.  Output rows and columns are the same 256 rows of the operand, so a
// slot holds 128 k of them, k .. k+63 in its P slab and k+64 .. k+127 in its
// Q slab, and a stage runs eight substeps whose two fragments both come from
// the P slab (substeps 0-3), then from the Q slab (4-7).  A stage of half
// the products is no shorter than a full one (its length is set by the
// copies' latency and the barrier), so a stage of twice the K with the same
// bytes lets the diagonal tile finish in about half a tile's time; the sums
// run over k in the same order as with 64-k stages.
struct CfgDiag : Cfg {
    static constexpr bool DIAG = true;
    static constexpr bool PACKED = true;
    static constexpr int SUBSTEPS = 8;
    static constexpr int KT_BYTES = 2 * ROWB;
    // wave w -> (wm, wn): (1,0) (1,1) (0,0) (1,2) (0,2) (0,3) (0,1) (1,3)
    static constexpr uint32_t WM_OF = 0x8Bu;    // bit w
    static constexpr uint32_t WN_OF = 0xDE84u;  // bits 2w, 2w+1
};

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_tr;
typedef __attribute__((address_space(3))) bf16x4_tr lds_bf16x4_t;

// The operand ring: slot S holds the P slab, then the Q slab.  After the main
// loop the epilogues reuse it as staging areas.
__shared__ __attribute__((aligned(1024))) char lds_ring[Cfg::STAGES * Cfg::SLOT_BYTES];
// The fused update's W rows, two halves of a round per wave (bf16 parameters).
__shared__ __attribute__((aligned(1024))) char lds_wbuf[Cfg::NWAVES * 4096];

template <int S> __device__ __forceinline__ char *slot_p() { return lds_ring + S * Cfg::SLOT_BYTES; }
template <int S> __device__ __forceinline__ char *slot_q() { return lds_ring + S * Cfg::SLOT_BYTES + Cfg::P_BYTES; }

// Epilogue staging areas: two of 8 KB per wave, area WHICH of every wave in
// slot WHICH of the ring.  Slot 0 is free once the last stage (slot 1) has
// begun, so the first round of an epilogue can be loaded under the last
// stage's MFMAs; slot 1 once every wave has left the main loop.
template <int WHICH> __device__ __forceinline__ char *epi_area(int wave) {
    static_assert(Cfg::NWAVES * Cfg::EPI_BYTES == Cfg::SLOT_BYTES, "one slot per staging area");
    return lds_ring + WHICH * Cfg::SLOT_BYTES + wave * Cfg::EPI_BYTES;
}

// s_waitcnt with vmcnt = N and the LDS/export counters left alone.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt at their maxima: no wait).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// s_waitcnt vmcnt(N) that no memory access is moved across.
template <int N> __device__ __forceinline__ void fenced_wait_vmcnt() {
    asm volatile("" ::: "memory");
    wait_vmcnt<N>();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One global -> LDS DMA of 16 bytes per lane (global_load_lds_dwordx4): lane
// i's 16 bytes at g land at LDS byte l + 16 i (l wave-uniform, passed in M0,
// which is set in the same statement).  The instruction has no register
// results.  It is issued from asm because the compiler, when it sees an
// LDS-writing load, makes every later wait for an LDS read a wait for all of
// them (lgkmcnt 0), which stalls the fragment pipeline; the kernels count
// these loads themselves (wait_vmcnt) and fence LDS reads with barriers that
// carry a memory clobber.
template <bool NT = false> __device__ __forceinline__ void dma16(const char *g, const char *l) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(reinterpret_cast<uintptr_t>(l)));
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(m0)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}

// K-contiguous tile (rows x 128 bytes): 16-byte chunk c of row r lives at
// chunk c ^ ((r >> 1) & 7), so 16 consecutive rows reading one chunk cover 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int kc_offset(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// N-contiguous tile (64 k-rows x QROW bytes): 64-byte block b of k-row r lives
// at block b ^ (r & 3), so four consecutive k-rows of one block cover 256 B.
template <class C> __device__ __forceinline__ int nc_offset(int krow, int byte) {
    return krow * C::QROW + ((((byte >> 6) ^ (krow & 3))) << 6) + (byte & 63);
}

// Epilogue staging rows of 64 fp32 (256 bytes): chunk c of row r lives at
// chunk c ^ (r & 15), so sixteen consecutive rows reading one chunk cover all
// 64 banks.
__device__ __forceinline__ int epi_offset(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

// Length of a K loop over a padded dimension of true length n: the padding
// beyond n is zero and adds nothing, so the loop stops at the first multiple
// of two 64-k stages (the loop runs stages in pairs) at or after n.
__device__ __forceinline__ int64_t k_extent(int64_t n, int64_t padded) {
    return min(padded, (n + 2 * Cfg::BK - 1) / (2 * Cfg::BK) * (2 * Cfg::BK));
}

struct Src {
    const char *p;  // P operand (output rows): K-contiguous rows of X, A or B
    int64_t ld_p;
    const char *q;  // Q operand (output columns): K-contiguous rows, or X itself for APPLY
    int64_t ld_q;
    uint32_t mmask;  // C::DIAG: bit i set = product i of each substep is needed (wave-uniform)
    uint32_t fmask;  // C::DIAG: bit j set = fragment j (read_frag's order) feeds a needed product
};

// DMA block j (0 <= j < LPS) of this wave for stage kt into slot S.  Blocks
// [0, P_BLOCKS) fill the P slab: 1 KB block `blk` holds rows 8 blk .. +7 x
// bytes [kt*128, kt*128 + 128); lane i lands at block byte 16 i, i.e. row
// i/8, swizzled chunk i%8.  The rest fill the Q slab the same way, except for
// APPLY, whose Q slab is k-rows [kt*64, kt*64 + 64) x QROW bytes of row-major
// X: a block holds 1024/QROW consecutive k-rows.  Every instruction moves
// whole 128-byte lines.
template <class C, int KIND, int S>
__device__ __forceinline__ void dma_block(const Src &src, int kt, int j, int wave, int lane) {
    if (j < C::P_BLOCKS) {
        const int blk = wave * C::P_BLOCKS + j;
        const int row = blk * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        dma16(src.p + row * src.ld_p + kt * C::KT_BYTES + chunk * 16, slot_p<S>() + blk * 1024);
    } else if constexpr (KIND == APPLY) {
        constexpr int UNITS = C::QROW / 16;  // 16-byte units per k-row
        const int blk = wave * C::Q_BLOCKS + (j - C::P_BLOCKS);
        const int krow = blk * (1024 / C::QROW) + lane / UNITS;
        const int u = lane % UNITS;
        const int byte = ((((u >> 2) ^ (krow & 3))) << 6) + ((u & 3) << 4);
        dma16(src.q + (static_cast<int64_t>(kt) * C::BK + krow) * src.ld_q + byte, slot_q<S>() + blk * 1024);
    } else {
        const int blk = wave * C::Q_BLOCKS + (j - C::P_BLOCKS);
        const int row = blk * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        dma16(src.q + row * src.ld_q + kt * C::KT_BYTES + chunk * 16, slot_q<S>() + blk * 1024);
    }
}

// Fragments of one 16-k substep: MI P-fragments and NI Q-fragments (8 bf16 =
// 16 bytes each per lane).
struct Frags {
    u32x4 a[Cfg::MI];
    u32x4 b[Cfg::NI];
};

// Reads fragment j of substep ks (0 .. SUBSTEPS-1) of the stage in slot S, in the order
// the products consume them: a0, b0 .. b(NI-1), a1 .. a(MI-1).
template <class C, int KIND, int S>
__device__ __forceinline__ void read_frag(Frags &f, int j, int ks, int wm, int wn, int lane) {
    const bool is_a = j == 0 || j > C::NI;
    const int idx = j == 0 ? 0 : (j <= C::NI ? j - 1 : j - C::NI);
    if constexpr (C::PACKED) {
        // both fragments are rows of the one operand: substeps 0-3 read the P
        // slab, 4-7 the Q slab (the stage's second 64 k)
        const char *slab = ks < 4 ? slot_p<S>() : slot_q<S>();
        const int chunk = 2 * (ks & 3) + (lane >> 5);
        const int row = (is_a ? wm * C::WM : wn * C::WN) + idx * 32 + (lane & 31);
        const u32x4 v = *reinterpret_cast<const u32x4 *>(slab + kc_offset(row, chunk));
        if (is_a)
            f.a[idx] = v;
        else
            f.b[idx] = v;
        return;
    }
    const int chunk = 2 * ks + (lane >> 5);  // k = 8*chunk .. 8*chunk+7 of this stage
    if (is_a) {
        const int row = wm * C::WM + idx * 32 + (lane & 31);
        f.a[idx] = *reinterpret_cast<const u32x4 *>(slot_p<S>() + kc_offset(row, chunk));
    } else if constexpr (KIND == APPLY) {
        // Lane jj of each 16-lane group supplies k-row kbase + jj/4, columns
        // n0 + 4(jj%4) .. +3; lane i then holds X[kbase .. kbase+3][n0 + i].
        const int grp = lane >> 4, jj = lane & 15;
        const int n0 = wn * C::WN + idx * 32 + 16 * (grp & 1);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int krow = 16 * ks + 8 * (grp >> 1) + 4 * r + (jj >> 2);
            const int byte = (n0 + 4 * (jj & 3)) * 2;
            const bf16x4_tr t =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(slot_q<S>() + nc_offset<C>(krow, byte)));
            const u32x2 tt = __builtin_bit_cast(u32x2, t);
            f.b[idx][2 * r] = tt[0];
            f.b[idx][2 * r + 1] = tt[1];
        }
    } else {
        const int row = wn * C::WN + idx * 32 + (lane & 31);
        f.b[idx] = *reinterpret_cast<const u32x4 *>(slot_q<S>() + kc_offset(row, chunk));
    }
}

// Product i of a substep: acc[mi][ni] += with mi = i / NI, ni = i % NI.  The
// operands are swapped (the Q fragment is the MFMA's first operand), which
// leaves the transposed 32 x 32 block in the accumulator: each lane then holds
// four consecutive output columns of one output row, so the epilogues move 16
// bytes per access.
template <class C>
__device__ __forceinline__ void mma_one(floatx16 (&acc)[C::MI][C::NI], const Frags &f, int i) {
    const int mi = i / C::NI, ni = i % C::NI;
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.b[ni]),
                                                          __builtin_bit_cast(bf16x8, f.a[mi]), acc[mi][ni], 0, 0, 0);
}

// Products of one substep (fragments f) with the reads of the next
// substep's fragments (into g, from slot S, substep ks_next) interleaved one
// per product; ISSUE_DMA spreads the LPS DMA blocks of stage kt_dma (into
// slot S_DMA) over the products.  A scheduling fence after each product keeps
// that order, so LDS reads and copies run under the MFMAs.
template <class C, int KIND, int S_READ, bool READ, int S_DMA, bool ISSUE_DMA>
__device__ __forceinline__ void substep(floatx16 (&acc)[C::MI][C::NI], const Frags &f, Frags &g, int ks_next,
                                        const Src &src, int kt_dma, int wave, int wm, int wn, int lane) {
    constexpr int EVERY = C::NM / C::LPS;
    static_assert(EVERY >= 1 && C::NM % C::LPS == 0, "one DMA block per product slot");
#pragma unroll
    for (int i = 0; i < C::NM; ++i) {
        if constexpr (C::DIAG) {
            if (src.mmask & (1u << i)) mma_one<C>(acc, f, i);
        } else if constexpr (C::MFMA) {
            mma_one<C>(acc, f, i);
        }
        if constexpr (C::DIAG) {
            if (READ && i < C::NF && (src.fmask & (1u << i))) read_frag<C, KIND, S_READ>(g, i, ks_next, wm, wn, lane);
        } else {
            if (READ && i < C::NF) read_frag<C, KIND, S_READ>(g, i, ks_next, wm, wn, lane);
        }
        if (ISSUE_DMA && i % EVERY == 0) dma_block<C, KIND, S_DMA>(src, kt_dma, i / EVERY, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Substeps I .. SUBSTEPS-2 of a stage in slot S: substep i computes with the
// fragments in fa (i even) or fb (i odd) and reads substep i+1's into the other.
template <class C, int KIND, int S, int I>
__device__ __forceinline__ void early_substeps(floatx16 (&acc)[C::MI][C::NI], const Src &src, int wave, int wm,
                                               int wn, int lane, Frags &fa, Frags &fb) {
    if constexpr (I < C::SUBSTEPS - 1) {
        if constexpr (I % 2 == 0)
            substep<C, KIND, S, true, S, false>(acc, fa, fb, I + 1, src, 0, wave, wm, wn, lane);
        else
            substep<C, KIND, S, true, S, false>(acc, fb, fa, I + 1, src, 0, wave, wm, wn, lane);
        early_substeps<C, KIND, S, I + 1>(acc, src, wave, wm, wn, lane, fa, fb);
    }
}

// Stage kt, held in slot S, of SUBSTEPS 16-k substeps; fa holds the first
// substep's fragments on entry.  Before the last substep each wave waits for
// its own DMA of stage kt+1 (the only loads in flight) and for its LDS reads,
// then the barrier: stage kt+1 has landed everywhere and no wave reads slot S
// any more, so the last substep refills it with stage kt+2 while reading
// stage kt+1's first fragments from the other slot.  That substep runs at a
// raised wave priority (Gram and A^2 1-2% faster, apply unchanged).
template <class C, int KIND, int S, bool ISSUE, bool LAST>
__device__ __forceinline__ void ring_stage(floatx16 (&acc)[C::MI][C::NI], const Src &src, int kt, int wave, int wm,
                                           int wn, int lane, Frags &fa, Frags &fb) {
    static_assert(C::SUBSTEPS % 2 == 0, "the last substep computes with fb");
    early_substeps<C, KIND, S, 0>(acc, src, wave, wm, wn, lane, fa, fb);
    if constexpr (LAST) {
        substep<C, KIND, S, false, S, false>(acc, fb, fa, 0, src, 0, wave, wm, wn, lane);
    } else {
        wait_lgkm0();
        wait_vmcnt<0>();
        stage_barrier();
        // the substep that issues the copies of stage kt+2 goes first on its
        // SIMD, so that they leave as early as possible
        __builtin_amdgcn_s_setprio(3);
        substep<C, KIND, 1 - S, true, S, ISSUE>(acc, fb, fa, 0, src, kt + 2, wave, wm, wn, lane);
        __builtin_amdgcn_s_setprio(0);
    }
}

// The K loop over nk stages (nk even, at least 2; any nk >= 1 for C::PACKED):
// stages 0 and 1 are loaded up front (loads retire in issue order, so
// vmcnt(LPS) leaves exactly stage 1's in flight once stage 0 has landed).
// The last stage runs in slot 1 (an odd count starts in slot 1), and
// pre_last() runs before it, when no wave reads slot 0 any more (every wave
// has passed the barrier of the stage before): it may start loads into slot 0.
template <class C, int KIND, class PreLast>
__device__ __forceinline__ void main_loop(floatx16 (&acc)[C::MI][C::NI], const Src &src, int nk, int wave, int wm,
                                          int wn, int lane, const PreLast &pre_last) {
    static_assert(C::STAGES == 2 && C::NF <= C::NM, "ring");
    constexpr int L = C::LPS;
    Frags fa, fb;
    int kt = 0;
    bool odd = false;
    if constexpr (C::PACKED) odd = nk & 1;
    if (odd) {
        // an odd count starts in slot 1 (stage 0 runs on its own), so that
        // the last stage still runs in slot 1
#pragma unroll
        for (int j = 0; j < L; ++j) dma_block<C, KIND, 1>(src, 0, j, wave, lane);
        if (nk > 1) {
#pragma unroll
            for (int j = 0; j < L; ++j) dma_block<C, KIND, 0>(src, 1, j, wave, lane);
            wait_vmcnt<L>();
        } else {
            wait_vmcnt<0>();
        }
        stage_barrier();
#pragma unroll
        for (int j = 0; j < C::NF; ++j) read_frag<C, KIND, 1>(fa, j, 0, wm, wn, lane);
        if (nk > 1) ring_stage<C, KIND, 1, true, false>(acc, src, 0, wave, wm, wn, lane, fa, fb);
        kt = 1;
    } else {
#pragma unroll
        for (int j = 0; j < L; ++j) dma_block<C, KIND, 0>(src, 0, j, wave, lane);
#pragma unroll
        for (int j = 0; j < L; ++j) dma_block<C, KIND, 1>(src, 1, j, wave, lane);
        wait_vmcnt<L>();
        stage_barrier();
#pragma unroll
        for (int j = 0; j < C::NF; ++j) read_frag<C, KIND, 0>(fa, j, 0, wm, wn, lane);
    }
    for (; kt < nk - 2; kt += 2) {
        ring_stage<C, KIND, 0, true, false>(acc, src, kt, wave, wm, wn, lane, fa, fb);
        ring_stage<C, KIND, 1, true, false>(acc, src, kt + 1, wave, wm, wn, lane, fa, fb);
    }
    // (a count of one has only the stage in slot 1)
    if (!C::PACKED || nk > 1) ring_stage<C, KIND, 0, false, false>(acc, src, kt, wave, wm, wn, lane, fa, fb);
    pre_last();
    ring_stage<C, KIND, 1, false, true>(acc, src, kt + 1, wave, wm, wn, lane, fa, fb);
}

// DMA of EPI_ROWS rows x 64 bf16 (128 bytes per row: X_hi, or A) starting
// at `src` (row pitch ld bytes) into a staging area: instructions of 8 rows
// each; lane i carries row i/8, chunk i%8 stored at chunk (i%8) ^ ((row/2)%8),
// so 16 consecutive rows reading one chunk touch 16 distinct bank groups.
template <class C, bool NT = false>
__device__ __forceinline__ void dma_bf16_rows(char *dst, const char *src, int64_t ld, int lane) {
#pragma unroll
    for (int t = 0; t < C::EPI_ROWS / 8; ++t) {
        const int row = 8 * t + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        dma16<NT>(src + row * ld + chunk * 16, dst + t * 1024);
    }
}
__device__ __forceinline__ int pair_offset(int row, int col) {
    return row * 128 + ((((col >> 3) ^ ((row >> 1) & 7))) << 4) + ((col & 7) << 1);
}

// DMA of EPI_ROWS rows x 64 residual bytes (64 bytes per row, X_lo) starting
// at `src` (row pitch ld bytes) into a staging area: instructions of 16 rows
// each; lane i carries row i/4, chunk i%4 stored at chunk (i%4) ^ ((row/4)%4),
// so 16 consecutive rows reading one 4-byte word touch 16 distinct banks.
template <class C, bool NT = false>
__device__ __forceinline__ void dma_lo8_rows(char *dst, const char *src, int64_t ld, int lane) {
#pragma unroll
    for (int t = 0; t < C::EPI_ROWS / 16; ++t) {
        const int row = 16 * t + (lane >> 2);
        const int chunk = (lane & 3) ^ ((row >> 2) & 3);
        dma16<NT>(src + row * ld + chunk * 16, dst + t * 1024);
    }
}
__device__ __forceinline__ int lo8_offset(int row, int col) {
    return row * 64 + ((((col >> 4) ^ ((row >> 2) & 3))) << 4) + (col & 15);
}

__device__ __forceinline__ void tri_decode(int64_t t, int *ti, int *tj) {
    int i = static_cast<int>((sqrt(8.0 * static_cast<double>(t) + 1.0) - 1.0) * 0.5);
    while (static_cast<int64_t>(i + 1) * (i + 2) / 2 <= t) ++i;
    while (static_cast<int64_t>(i) * (i + 1) / 2 > t) --i;
    *ti = i;
    *tj = static_cast<int>(t - static_cast<int64_t>(i) * (i + 1) / 2);
}

// ------------------------------------------------------------------------ A, B

// Rows of A that POLY's epilogue combines with the wave's block: the block
// itself, bf16, row pitch sp.
__device__ __forceinline__ const char *poly_a_rows(const Geom &g, const Work &w, int64_t e, int64_t row0,
                                                   int64_t col0) {
    return reinterpret_cast<const char *>(static_cast<const uint16_t *>(w.ab) + e * w.a_stride + row0 * g.sp + col0);
}

// Epilogue of GRAM and POLY.  The wave's 128 x 64 block is finished in four
// rounds of 32 rows staged in LDS.  POLY brings the matching rows of the bf16
// A by DMA (two areas, the next round in flight; round 0 was issued into
// area 0 under the last stage of the main loop).  The values (GRAM:
// A, times inv_norm^2 on the bf16 path's first step; POLY: b A + c A A, times
// inv_norm on that step, so that B X applies the normalisation of X) are
// formed in the accumulator layout and written in place as fp32 rows; the
// rows are stored whole as bf16 (GRAM: A; POLY: B), and for an off-diagonal
// tile each column of the block is stored as 32 consecutive bf16 of a row of
// the mirrored tile.  A exists only in bf16: the b A term of B taken from it
// instead of an fp32 copy changes nothing measurable once B itself is rounded
// to bf16.  Vector-memory instructions retire in issue order; the wait before
// POLY's round h allows what was issued after round h's DMA: round h-1's
// stores (at least ROW_STORES) and round h+1's DMA.
// POLY: A's rows of the four rounds are staged so that they arrive early:
// rounds 0 and 1 under the last K stage (round 0 in the slot-0 area, round 1
// in the wave's 4 KB of lds_wbuf, which the K loop does not use), round 2 in
// the slot-1 area on entry, round 3 in lds_wbuf once round 1 has read it.  A
// round's fp32 values go over its own A rows in a ring area, or, for rounds
// 1 and 3, into the slot-0 area once the previous round's stores have read it.
template <class C, int KIND>
__device__ __forceinline__ void sym_epilogue(const floatx16 (&acc)[C::MI][C::NI], const Geom &g, const Work &w,
                                             const NsStep &p, int64_t e, int ti, int tj, int wm, int wn,
                                             char *const (&area)[2], char *wb, int lane) {
    constexpr int ROUNDS = C::WM / C::EPI_ROWS;
    constexpr int DMA_PER_ROUND = C::EPI_ROWS / 8;
    constexpr int ROW_STORES = C::EPI_ROWS / 4;
    constexpr int STORES = ROW_STORES + C::WN / 16;  // row and mirror stores of a round off the diagonal
    static_assert(ROUNDS == C::MI && C::EPI_ROWS == 32 && C::WN == 64, "one 32 x 64 accumulator block per round");
    const int64_t ld = g.sp;
    const int64_t row0 = static_cast<int64_t>(ti) * C::BM + wm * C::WM;
    const int64_t col0 = static_cast<int64_t>(tj) * C::BN + wn * C::WN;
    uint16_t *dst = static_cast<uint16_t *>(KIND == GRAM ? w.ab : w.bb) + e * w.a_stride;
    // Off-diagonal tiles store every block and its mirror.  Diagonal tiles
    // computed only the 32 x 32 blocks on and below the diagonal (block row >=
    // block column): they store those and mirror the ones strictly below it.
    const bool diag = ti == tj;
    // first step on the bf16 path: X holds N, so A = inv^2 (N N^T) and the
    // product B X is taken with B inv (X' = a inv N + (B inv) N)
    const float inv = p.unnormalized ? w.inv_norm[e] : 1.0f;
    const float gscale = inv * inv;
    const float pb = p.b * inv, pc = p.c * inv;
    const char *a_in = poly_a_rows(g, w, e, row0, col0);
    static_assert(ROUNDS == 4 && C::EPI_ROWS * 128 <= 4096, "a round's A rows fit the wave's lds_wbuf");
    static_assert(2 * STORES + DMA_PER_ROUND + STORES < 64, "vmcnt range");
    const char *const a_src[ROUNDS] = {area[0], wb, area[1], wb};
    char *const f_area[ROUNDS] = {area[0], area[0], area[1], area[0]};
    if constexpr (KIND == POLY) dma_bf16_rows<C>(area[1], a_in + 2 * C::EPI_ROWS * ld * 2, ld * 2, lane);
    const int lrow = lane & 31;
#pragma unroll
    for (int h = 0; h < ROUNDS; ++h) {
        char *reg = KIND == POLY ? f_area[h] : area[h & 1];
        if constexpr (KIND == POLY) {
            // Retirement is in issue order; each wait allows what was issued
            // after round h's rows.  A diagonal tile's rounds may issue fewer
            // stores, so there the waits count none of them.
            if (h == 0)
                fenced_wait_vmcnt<2 * DMA_PER_ROUND>();  // rounds 1 and 2
            else if (h == 1 && diag)
                fenced_wait_vmcnt<DMA_PER_ROUND>();
            else if (h == 1)
                fenced_wait_vmcnt<DMA_PER_ROUND + STORES>();  // round 2, round 0's stores
            else if (h == 2 && diag)
                fenced_wait_vmcnt<DMA_PER_ROUND>();
            else if (h == 2)
                fenced_wait_vmcnt<STORES + STORES + DMA_PER_ROUND>();  // stores 0 and 1, round 3
            else if (diag)
                fenced_wait_vmcnt<0>();
            else
                fenced_wait_vmcnt<STORES>();  // round 2's stores (round 3 followed round 1's)
        }
        const int brow = wm * C::MI + h;  // block row of this round (32-row blocks of the tile)
        floatx4 v[C::NI][4];
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const int lcol = ni * 32 + 8 * c4 + 4 * (lane >> 5);
                if constexpr (KIND == GRAM) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[ni][c4][q] = acc[h][ni][4 * c4 + q] * gscale;
                } else {
                    const u32x2 a2 = *reinterpret_cast<const u32x2 *>(a_src[h] + pair_offset(lrow, lcol));
                    const float a4[4] = {__uint_as_float(a2[0] << 16), __uint_as_float(a2[0] & 0xffff0000u),
                                         __uint_as_float(a2[1] << 16), __uint_as_float(a2[1] & 0xffff0000u)};
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[ni][c4][q] = __builtin_fmaf(pb, a4[q], pc * acc[h][ni][4 * c4 + q]);
                }
            }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const int lcol = ni * 32 + 8 * c4 + 4 * (lane >> 5);
                *reinterpret_cast<floatx4 *>(reg + epi_offset(lrow, lcol >> 2)) = v[ni][c4];
            }
        wait_lgkm0();  // the wave's writes land before its row and column reads
        asm volatile("" ::: "memory");
        const int64_t rbase = row0 + C::EPI_ROWS * h;
#pragma unroll
        for (int r4 = 0; r4 < C::EPI_ROWS / 4; ++r4) {
            const int rrow = 4 * r4 + (lane >> 4), chunk = lane & 15;
            const floatx4 x = *reinterpret_cast<const floatx4 *>(reg + epi_offset(rrow, chunk));
            const int64_t idx = (rbase + rrow) * ld + col0 + 4 * chunk;
            u32x2 pk;
            pk[0] = pack_bf16x2(x[0], x[1]);
            pk[1] = pack_bf16x2(x[2], x[3]);
            if (!diag || brow >= wn * C::NI + (chunk >> 3))
                __builtin_nontemporal_store(pk, as_global(reinterpret_cast<u32x2 *>(dst + idx)));
        }
        {
            // column c of the block -> row col0 + c of the mirrored tile; lane
            // (c, part) moves rows 8*part .. 8*part+7 of the round
#pragma unroll
            for (int t = 0; t < C::WN / 16; ++t) {
                if (diag && brow <= wn * C::NI + t / 2) continue;  // columns 16t.. lie in block wn*NI + t/2
                const int c = 16 * t + (lane >> 2), part = lane & 3;
                float f[8];
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    f[k] = *reinterpret_cast<const float *>(reg + epi_offset(8 * part + k, c >> 2) + (c & 3) * 4);
                u32x4 pk;
#pragma unroll
                for (int k = 0; k < 4; ++k) pk[k] = pack_bf16x2(f[2 * k], f[2 * k + 1]);
                __builtin_nontemporal_store(pk, as_global(reinterpret_cast<u32x4 *>(dst + (col0 + c) * ld + rbase + 8 * part)));
            }
        }
        if constexpr (KIND == POLY) {
            if (h == 1) {
                wait_lgkm0();  // round 1's reads of its A rows are done before the DMA refills lds_wbuf
                asm volatile("" ::: "memory");
                dma_bf16_rows<C>(wb, a_in + 3 * C::EPI_ROWS * ld * 2, ld * 2, lane);
            }
        }
    }
}

// The 128 x 64 output block (block row wm, block column wn of the tile) that
// wave `wave` owns: row-major over the wave grid, or on a diagonal tile the
// permuted order of CfgDiag.
template <class C> __device__ __forceinline__ void wave_block(bool diag, int wave, int *wm, int *wn) {
    *wm = diag ? static_cast<int>((CfgDiag::WM_OF >> wave) & 1) : wave / C::WAVES_N;
    *wn = diag ? static_cast<int>((CfgDiag::WN_OF >> (2 * wave)) & 3) : wave % C::WAVES_N;
}

// Split-K partial of one (matrix, tile, K range): 256 x 256 fp32, stored as
// the accumulators lie, wave by wave, then accumulator group j = (mi NI + ni)
// 4 + c4 (four values), then lane: every store moves 1 KB of consecutive
// bytes.  sym_reduce_kernel reads the same order back.
constexpr int KPART_VALUES = 256 * 256;
template <class C>
__device__ __forceinline__ void store_kpart(const floatx16 (&acc)[C::MI][C::NI], float *dst, int wave, int lane) {
    floatx4 *base = reinterpret_cast<floatx4 *>(dst) + wave * (C::MI * C::NI * 4 * 64) + lane;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                floatx4 v;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = acc[mi][ni][4 * c4 + q];
                *as_global(base + ((mi * C::NI + ni) * 4 + c4) * 64) = v;
            }
}

// One launch covers the chunk's lower-triangle tiles [tile_base, tile_base +
// tile_count) in the order (matrix, tile of the matrix); with splits > 1 each
// of them runs as `splits` workgroups over K ranges of `units` x 128 that store
// fp32 partial tiles (slot (tile - tile_base) * splits + range of w.kpart),
// finished by sym_reduce_kernel.  Workgroups of one K range are consecutive:
// tiles of one matrix then read the same K slab of the operand.
template <class C, int KIND>
__global__ __launch_bounds__(C::NT, 1) void ns_sym_kernel(Geom g, Work w, NsStep p, int64_t tiles_per_mat,
                                                           int64_t nblocks, int64_t tile_base, int64_t tile_count,
                                                           int splits, int units) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t L = xcd_swizzle(blockIdx.x, nblocks);
    const int ks = static_cast<int>(L / tile_count);
    const int64_t tl = L % tile_count;  // tile of the launch
    const int64_t f = tile_base + tl;   // tile of the chunk
    const int64_t e = f / tiles_per_mat;
    const int64_t t = f % tiles_per_mat;
    int ti, tj;
    tri_decode(t, &ti, &tj);
    const bool diag = ti == tj;
    int wm, wn;
    wave_block<C>(diag, wave, &wm, &wn);

    // P supplies output rows (tile ti), Q output columns (tile tj); both are
    // rows of X (GRAM) or of the symmetric A (POLY), K-contiguous.
    Src src;
    {
        // product i = (mi, ni) covers block row wm*MI + mi, block column wn*NI + ni
        // and takes fragments a[mi] (read first for mi = 0, else after the
        // b's) and b[ni]
        uint32_t m = 0, fm = 0;
#pragma unroll
        for (int i = 0; i < C::NM; ++i)
            if (wm * C::MI + i / C::NI >= wn * C::NI + i % C::NI) {
                m |= 1u << i;
                const int mi = i / C::NI, ni = i % C::NI;
                fm |= (1u << (mi == 0 ? 0 : C::NI + mi)) | (1u << (1 + ni));
            }
        src.mmask = __builtin_amdgcn_readfirstlane(m);
        src.fmask = __builtin_amdgcn_readfirstlane(fm);
    }
    int64_t kdim;
    if (KIND == GRAM) {
        const char *x = static_cast<const char *>(w.xb) + e * w.x_stride * 2;
        src.ld_p = src.ld_q = g.lp * 2;
        kdim = k_extent(g.l, g.lp);
        src.p = x + static_cast<int64_t>(ti) * C::BM * src.ld_p;
        src.q = x + static_cast<int64_t>(tj) * C::BN * src.ld_q;
    } else {
        const char *a = static_cast<const char *>(w.ab) + e * w.a_stride * 2;
        src.ld_p = src.ld_q = g.sp * 2;
        kdim = k_extent(g.s, g.sp);
        src.p = a + static_cast<int64_t>(ti) * C::BM * src.ld_p;
        src.q = a + static_cast<int64_t>(tj) * C::BN * src.ld_q;
    }
    // this workgroup's K range (the whole extent when the product is not split;
    // ranges are multiples of 128, as the loop runs stages in pairs)
    const int64_t k0 = static_cast<int64_t>(ks) * units * 2 * C::BK;
    const int64_t k1 = splits > 1 ? min(kdim, k0 + static_cast<int64_t>(units) * 2 * C::BK) : kdim;
    src.p += k0 * 2;
    src.q += k0 * 2;

    floatx16 acc[C::MI][C::NI];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
    // POLY's epilogue rows of A are requested under the last K stage; a split
    // product has no epilogue of its own (sym_reduce_kernel forms B)
    auto pre_last = [&] {
        if constexpr (KIND == POLY)
            if (splits == 1) {
                const char *a_rows = poly_a_rows(g, w, e, static_cast<int64_t>(ti) * C::BM + wm * C::WM,
                                                 static_cast<int64_t>(tj) * C::BN + wn * C::WN);
                dma_bf16_rows<C>(epi_area<0>(wave), a_rows, g.sp * 2, lane);
                dma_bf16_rows<C>(lds_wbuf + wave * 4096, a_rows + C::EPI_ROWS * g.sp * 2, g.sp * 2, lane);
            }
    };
    const int nk = static_cast<int>((k1 - k0) / C::BK);
    if (diag) {
        // P and Q are the same rows: a slot holds 128 k of them (CfgDiag)
        Src one = src;
        one.q = src.p + C::ROWB;
        main_loop<CfgDiag, KIND>(acc, one, nk / 2, wave, wm, wn, lane, pre_last);
    } else if (__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<int64_t>(ti) * C::BM + wm * C::WM >= g.s)))
        main_loop<CfgIdle, KIND>(acc, src, nk, wave, wm, wn, lane, pre_last);
    else
        main_loop<C, KIND>(acc, src, nk, wave, wm, wn, lane, pre_last);

    if (splits > 1) {
        store_kpart<C>(acc, w.kpart + (tl * splits + ks) * KPART_VALUES, wave, lane);
        return;
    }

    // acc[mi][ni][4*c4 + q] holds output row wm*WM + mi*32 + lane%32, column
    // wn*WN + ni*32 + 8*c4 + 4*(lane/32) + q of the tile.
    wait_lgkm0();
    stage_barrier();  // every wave is done with the operand ring
    char *const area[2] = {epi_area<0>(wave), epi_area<1>(wave)};
    sym_epilogue<C, KIND>(acc, g, w, p, e, ti, tj, wm, wn, area, lds_wbuf + wave * 4096, lane);
}

// Split-K Gram / A^2: sums the K ranges' partials of one (matrix, tile) in
// range order (fixed, so the result is deterministic) and finishes them as
// sym_epilogue does: GRAM writes A = sum (times inv_norm^2 on the bf16 path's
// first step), POLY writes B = b A + c sum (b and c times inv_norm on that
// step) with A read back in bf16; both in bf16, with the mirrored element
// for off-diagonal blocks.  Blocks of a diagonal tile above its diagonal were
// not computed and are skipped.  Thread (item) = one partial float4: wave,
// accumulator group and lane, as store_kpart laid them out; 64 blocks of 256
// threads per tile.
template <int KIND>
__global__ __launch_bounds__(256) void sym_reduce_kernel(Geom g, Work w, NsStep p, int64_t tiles_per_mat,
                                                         int64_t tile_base, int splits) {
    using C = Cfg;
    const int64_t tl = blockIdx.x / 64;  // tile of the split launch
    const int64_t tile = tile_base + tl; // matrix * tiles_per_mat + tile of the matrix
    const int item = static_cast<int>(blockIdx.x % 64) * 256 + threadIdx.x;
    const int64_t e = tile / tiles_per_mat;
    int ti, tj;
    tri_decode(tile % tiles_per_mat, &ti, &tj);
    const floatx4 *src = reinterpret_cast<const floatx4 *>(w.kpart) + tl * splits * (KPART_VALUES / 4) + item;
    floatx4 sum = src[0];
    for (int k = 1; k < splits; ++k) {
        const floatx4 v = src[static_cast<int64_t>(k) * (KPART_VALUES / 4)];
#pragma unroll
        for (int q = 0; q < 4; ++q) sum[q] += v[q];
    }
    const int wave = item >> 11, j = (item >> 6) & 31, lane = item & 63;
    const int mi = j / (C::NI * 4), ni = (j / 4) % C::NI, c4 = j % 4;
    const bool diag = ti == tj;
    int wm, wn;
    wave_block<C>(diag, wave, &wm, &wn);
    const int brow = wm * C::MI + mi, bcol = wn * C::NI + ni;  // 32 x 32 blocks of the tile
    if (diag && brow < bcol) return;
    const int64_t row = static_cast<int64_t>(ti) * C::BM + wm * C::WM + mi * 32 + (lane & 31);
    const int64_t col = static_cast<int64_t>(tj) * C::BN + wn * C::WN + ni * 32 + 8 * c4 + 4 * (lane >> 5);
    const int64_t ld = g.sp;
    const float inv = p.unnormalized ? w.inv_norm[e] : 1.0f;
    float v[4];
    if constexpr (KIND == GRAM) {
        const float gscale = inv * inv;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = sum[q] * gscale;
    } else {
        const float pb = p.b * inv, pc = p.c * inv;
        const u32x2 a2 = *as_global(reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(w.ab) +
                                                                   e * w.a_stride + row * ld + col));
        const float a4[4] = {__uint_as_float(a2[0] << 16), __uint_as_float(a2[0] & 0xffff0000u),
                             __uint_as_float(a2[1] << 16), __uint_as_float(a2[1] & 0xffff0000u)};
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(pb, a4[q], pc * sum[q]);
    }
    uint16_t *dst = static_cast<uint16_t *>(KIND == GRAM ? w.ab : w.bb) + e * w.a_stride;
    u32x2 pk;
    pk[0] = pack_bf16x2(v[0], v[1]);
    pk[1] = pack_bf16x2(v[2], v[3]);
    *as_global(reinterpret_cast<u32x2 *>(dst + row * ld + col)) = pk;
    // the mirror: every block of an off-diagonal tile and the blocks strictly
    // below the diagonal of a diagonal tile (a diagonal block holds both halves)
    if (!diag || brow > bcol) {
#pragma unroll
        for (int q = 0; q < 4; ++q) as_global(dst)[(col + q) * ld + row] = float_to_bf16_bits(v[q]);
    }
}

// --------------------------------------------------------------------- a X + B X

// A wave-uniform value (the wave's own tile coordinates), moved to scalar
// registers so that addresses built from it are too.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Global stores addressed as a scalar base plus a 32-bit per-lane offset
// (the compiler builds a 64-bit vector address per store otherwise).  Plain
// vector stores: they count in vmcnt like any other.  In the apply epilogue
// the 8-byte form carries X'_hi, whole 128-byte lines, and goes out
// non-temporal; the 4-byte form carries X'_lo, whose rows are 64-byte halves
// of a line (the other half is another wave's), and stays temporal so that
// L2 merges the halves before write-back.
__device__ __forceinline__ void store_saddr(char *base, uint32_t off, const u32x2 &v) {
    asm volatile("global_store_dwordx2 %0, %1, %2 nt" ::"v"(off), "v"(v), "s"(base) : "memory");
}
__device__ __forceinline__ void store_saddr(char *base, uint32_t off, uint32_t v) {
    asm volatile("global_store_dword %0, %1, %2" ::"v"(off), "v"(v), "s"(base) : "memory");
}

// Output block of one wave in the apply epilogue.
struct ApplyTile {
    int64_t e;     // matrix
    int64_t row0;  // first output row
    int64_t col0;  // first output column
};

// First rows of X_hi (row pitch 2 lp bytes) and X_lo (pitch lp) of a wave's
// output block, and the DMA of one round (EPI_ROWS rows of each) into a
// staging area: X_hi rows in its first PAIR_HALF bytes, X_lo rows after.
constexpr int PAIR_HALF = 4096;
struct XRows {
    const char *hi, *lo;
    int64_t ld_hi, ld_lo;
};
__device__ __forceinline__ XRows x_rows(const Geom &g, const Work &w, const ApplyTile &t) {
    const int64_t first = t.row0 * g.lp + t.col0;
    return {reinterpret_cast<const char *>(static_cast<const uint16_t *>(w.xb) + t.e * w.x_stride + first),
            reinterpret_cast<const char *>(static_cast<const uint8_t *>(w.xl) + t.e * w.x_stride + first), g.lp * 2,
            g.lp};
}
__device__ __forceinline__ void dma_x_round(char *dst, const XRows &x, int h, int lane) {
    dma_bf16_rows<Cfg, true>(dst, x.hi + Cfg::EPI_ROWS * h * x.ld_hi, x.ld_hi, lane);
    dma_lo8_rows<Cfg, true>(dst + PAIR_HALF, x.lo + Cfg::EPI_ROWS * h * x.ld_lo, x.ld_lo, lane);
}

// Row lrow's four columns lcol .. lcol+3 of a X + B X, with X = X_hi + X_lo
// staged in `reg` (X_hi rows, 128 bytes each, in the first PAIR_HALF bytes;
// X_lo rows, 64 bytes each, after).  While X still holds N, `a` is a inv_norm
// (and B was scaled by inv_norm when it was formed).
__device__ __forceinline__ floatx4 apply_value(const floatx16 &acc, const char *reg, int lrow, int lcol, int c4,
                                               float a) {
    const u32x2 h = *reinterpret_cast<const u32x2 *>(reg + pair_offset(lrow, lcol));
    const uint32_t l = *reinterpret_cast<const uint32_t *>(reg + PAIR_HALF + lo8_offset(lrow, lcol));
    const floatx4 x = join_bf16x4(h, l);
    floatx4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(a, x[q], acc[4 * c4 + q]);
    return v;
}

// The wave's 32 x 64 block of values, computed in the accumulator layout from
// the X pair staged in `reg`, rewritten in place as fp32 rows (256 bytes each)
// for the row-contiguous pass.  All of the lane's reads precede its writes, and
// one wave's LDS accesses execute in order, so no value is overwritten before
// it is read.
template <class C>
__device__ __forceinline__ void stage_values(const floatx16 (&accm)[C::NI], char *reg, float a, int lane) {
    const int lrow = lane & 31;
    floatx4 v[C::NI][4];
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            v[ni][c4] = apply_value(accm[ni], reg, lrow, ni * 32 + 8 * c4 + 4 * (lane >> 5), c4, a);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const int lcol = ni * 32 + 8 * c4 + 4 * (lane >> 5);
            *reinterpret_cast<floatx4 *>(reg + epi_offset(lrow, lcol >> 2)) = v[ni][c4];
        }
    wait_lgkm0();  // the wave's writes land before its row-contiguous reads
    asm volatile("" ::: "memory");
}


// DMA of round h's X_hi rows to hi and X_lo rows to lo (two staging places).
__device__ __forceinline__ void dma_x_round_to(char *hi, char *lo, const XRows &x, int h, int lane) {
    dma_bf16_rows<Cfg, true>(hi, x.hi + Cfg::EPI_ROWS * h * x.ld_hi, x.ld_hi, lane);
    dma_lo8_rows<Cfg, true>(lo, x.lo + Cfg::EPI_ROWS * h * x.ld_lo, x.ld_lo, lane);
}

// The wave's 32 x 64 block of X' = a X + acc, X read from the pair staged at
// (hi rows, lo rows) in the accumulator layout, encoded there and written
// back over the very bytes each lane read (so no lane's write can meet
// another lane's read); the lane's eight reads precede its writes.
template <class C>
__device__ __forceinline__ void stage_pair(const floatx16 (&accm)[C::NI], char *hi, char *lo, float a, int lane) {
    const int lrow = lane & 31;
    u32x2 h[C::NI][4];
    uint32_t l[C::NI][4];
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const int lcol = ni * 32 + 8 * c4 + 4 * (lane >> 5);
            h[ni][c4] = *reinterpret_cast<const u32x2 *>(hi + pair_offset(lrow, lcol));
            l[ni][c4] = *reinterpret_cast<const uint32_t *>(lo + lo8_offset(lrow, lcol));
        }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const floatx4 x = join_bf16x4(h[ni][c4], l[ni][c4]);
            floatx4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(a, x[q], accm[ni][4 * c4 + q]);
            split_bf16x4(v, &h[ni][c4], &l[ni][c4]);
        }
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const int lcol = ni * 32 + 8 * c4 + 4 * (lane >> 5);
            *reinterpret_cast<u32x2 *>(hi + pair_offset(lrow, lcol)) = h[ni][c4];
            *reinterpret_cast<uint32_t *>(lo + lo8_offset(lrow, lcol)) = l[ni][c4];
        }
    wait_lgkm0();  // the wave's writes land before its row-contiguous reads
    asm volatile("" ::: "memory");
}

// Epilogue of an intermediate step: X' = a X + B X is written as the bf16 pair
// (X'_hi to xb_next, X'_lo to xl in place).  Outside s x l it is zero without
// a mask: X is zero there, so are the padded rows and columns of A and B, and
// with them every term of X'.  Per round of EPI_ROWS rows the wave's X_hi and
// X_lo rows arrive by DMA in a staging place, the encoded X' pair replaces
// them there (stage_pair) and is read back row-contiguously (16 lanes per
// row) so the stores move whole rows.  A round takes 6 KB of the wave's 20 KB
// (8 KB of each ring slot and 4 KB of lds_wbuf): rounds 0 and 1 were loaded
// under the last stage of the main loop (slot 0, whose 2 KB tail holds round
// 1's X_lo, and lds_wbuf, which the K loop does not use), round 2 is loaded
// into slot 1 on entry and round 3 into round 0's place once round 0's rows
// are read.  Every vector-memory instruction retires in issue order, so each
// wait allows exactly what was issued after that round's DMA.
__device__ __forceinline__ void apply_epilogue_next(const floatx16 (&acc)[Cfg::MI][Cfg::NI], const Geom &g,
                                                    const Work &w, const NsStep &p, const ApplyTile &t,
                                                    char *slot0, char *slot1, char *wb, int lane) {
    using C = Cfg;
    constexpr int ROUNDS = C::WM / C::EPI_ROWS;
    constexpr int DMA = C::EPI_ROWS / 8 + C::EPI_ROWS / 16;  // X_hi, X_lo instructions per round
    constexpr int STORES = 2 * (C::EPI_ROWS / 4);
    static_assert(ROUNDS == 4 && C::EPI_ROWS == 32 && C::WN == 64, "one 32 x 64 accumulator block per round");
    static_assert(C::EPI_ROWS * 128 == PAIR_HALF && C::EPI_BYTES == 8192, "a round's pair takes 6 KB");
    static_assert(DMA + STORES + DMA + STORES + DMA < 64, "vmcnt range");
    char *const hi[ROUNDS] = {slot0, wb, slot1, slot0};
    char *const lo[ROUNDS] = {slot0 + PAIR_HALF, slot0 + PAIR_HALF + 2048, slot1 + PAIR_HALF, slot0 + PAIR_HALF};
    uint8_t *xl = static_cast<uint8_t *>(w.xl) + t.e * w.x_stride;
    uint16_t *xh_out = static_cast<uint16_t *>(w.xb_next) + t.e * w.x_stride;
    const XRows x = x_rows(g, w, t);
    const float a = p.unnormalized ? p.a * w.inv_norm[t.e] : p.a;
    // Stores: a wave-uniform row base plus a per-lane 32-bit offset (lane
    // (rr, chunk) owns columns 4 chunk .. +3 of row rr of each group of four).
    const int rr = lane >> 4, chunk = lane & 15;
    const uint32_t off_lo = static_cast<uint32_t>(rr * g.lp + 4 * chunk);
    const uint32_t off_hi = 2 * off_lo;
    const int64_t row0 = uniform64(t.row0), col0 = uniform64(t.col0);
    dma_x_round_to(hi[2], lo[2], x, 2, lane);
#pragma unroll
    for (int h = 0; h < ROUNDS; ++h) {
        if (h == 0)
            fenced_wait_vmcnt<2 * DMA>();  // rounds 1 and 2 may be in flight
        else if (h == 1)
            fenced_wait_vmcnt<DMA + STORES + DMA>();  // round 2, round 0's stores, round 3
        else if (h == 2)
            fenced_wait_vmcnt<STORES + DMA + STORES>();  // round 0's stores, round 3, round 1's stores
        else
            fenced_wait_vmcnt<2 * STORES>();  // rounds 1 and 2's stores
        stage_pair<C>(acc[h], hi[h], lo[h], a, lane);
#pragma unroll
        for (int r4 = 0; r4 < C::EPI_ROWS / 4; ++r4) {
            const int row = 4 * r4 + rr;
            const u32x2 hv = *reinterpret_cast<const u32x2 *>(hi[h] + pair_offset(row, 4 * chunk));
            const uint32_t lv = *reinterpret_cast<const uint32_t *>(lo[h] + lo8_offset(row, 4 * chunk));
            const int64_t base = (row0 + C::EPI_ROWS * h + 4 * r4) * g.lp + col0;
            store_saddr(reinterpret_cast<char *>(xh_out + base), off_hi, hv);
            store_saddr(reinterpret_cast<char *>(xl + base), off_lo, lv);
        }
        if (h == 0) {
            wait_lgkm0();  // round 0's LDS reads are done before the DMA refills its place
            asm volatile("" ::: "memory");
            dma_x_round_to(hi[3], lo[3], x, 3, lane);
        }
    }
}

// W <- d W - s_scale X' for X' row gi, columns gj .. gj+3 (W row-major with
// the orientation of X'), and O' = X' when asked.  The four elements move as
// one 8- or 16-byte access when they are consecutive in W, inside the matrix
// and aligned (rows of a multiple of 4 elements, 16-byte aligned parameter and
// ns_out: NsStep::vec_ok); one by one otherwise.
template <int PARAM_BF16>
__device__ __forceinline__ void update_row4(const MatDesc &d, const Geom &g, const NsStep &p, int64_t gi, int64_t gj,
                                            const floatx4 &v) {
    if (p.vec_ok && !g.transposed && (g.cols % 4 == 0) && gj + 3 < g.l) {
        const int64_t widx = gi * g.cols + gj;
        if (PARAM_BF16) {
            auto *pp = as_global(reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(d.param) + widx));
            const u32x2 wv = *pp;
            u32x2 o;
            o[0] = pack_bf16x2(p.dscale * __uint_as_float(wv[0] << 16) - p.sscale * v[0],
                               p.dscale * __uint_as_float(wv[0] & 0xffff0000u) - p.sscale * v[1]);
            o[1] = pack_bf16x2(p.dscale * __uint_as_float(wv[1] << 16) - p.sscale * v[2],
                               p.dscale * __uint_as_float(wv[1] & 0xffff0000u) - p.sscale * v[3]);
            *pp = o;
        } else {
            auto *pp = as_global(reinterpret_cast<floatx4 *>(static_cast<float *>(d.param) + widx));
            const floatx4 wv = *pp;
            floatx4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = p.dscale * wv[q] - p.sscale * v[q];
            *pp = o;
        }
        if (d.ns_out) *as_global(reinterpret_cast<floatx4 *>(d.ns_out + widx)) = v;
        return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (gj + q >= g.l) continue;
        const int64_t widx = g.transposed ? ((gj + q) * g.cols + gi) : (gi * g.cols + gj + q);
        if (PARAM_BF16) {
            auto *pp = as_global(static_cast<uint16_t *>(d.param));
            const float wv = bf16_bits_to_float(pp[widx]);
            pp[widx] = float_to_bf16_bits(p.dscale * wv - p.sscale * v[q]);
        } else {
            auto *pp = as_global(static_cast<float *>(d.param));
            pp[widx] = p.dscale * pp[widx] - p.sscale * v[q];
        }
        if (d.ns_out) as_global(d.ns_out)[widx] = v[q];
    }
}

// Epilogue of the last step: W <- d W - s_scale X' (and O' = X' when asked),
// orientation-aware.  Two staging areas: round 0's X rows were requested under
// the last stage of the main loop; round h+1's are requested as soon as round
// h's have landed, so they arrive while round h is computed.  For W in the
// orientation of X' the values are rewritten as fp32 rows and the update
// walks whole rows (16 lanes per 64-column row); for transposed W the
// accumulator layout already puts 32 consecutive X' rows, i.e. 32 consecutive
// elements of a W row, in consecutive lanes.
template <int PARAM_BF16>
__device__ __forceinline__ void apply_epilogue_update(const floatx16 (&acc)[Cfg::MI][Cfg::NI], const MatDesc &d,
                                                      const Geom &g, const Work &w, const NsStep &p,
                                                      const ApplyTile &t, char *const (&area)[2], int lane) {
    using C = Cfg;
    constexpr int ROUNDS = C::WM / C::EPI_ROWS;
    static_assert(C::EPI_ROWS == 32 && C::WN == 64, "one 32 x 64 accumulator block per round");
    const XRows x = x_rows(g, w, t);
    const float a = p.unnormalized ? p.a * w.inv_norm[t.e] : p.a;
#pragma unroll
    for (int h = 0; h < ROUNDS; ++h) {
        char *reg = area[h & 1];
        fenced_wait_vmcnt<0>();  // round h's rows (and round h-1's stores)
        if (h + 1 < ROUNDS) {
            // area (h+1)&1 was last read in round h-1, whose reads ended with it
            dma_x_round(area[(h + 1) & 1], x, h + 1, lane);
            asm volatile("" ::: "memory");
        }
        const int lrow = lane & 31;
        if (g.transposed) {
            const int64_t gi = t.row0 + C::EPI_ROWS * h + lrow;
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    const int lcol = ni * 32 + 8 * c4 + 4 * (lane >> 5);
                    const floatx4 v = apply_value(acc[h][ni], reg, lrow, lcol, c4, a);
                    if (gi < g.s) update_row4<PARAM_BF16>(d, g, p, gi, t.col0 + lcol, v);
                }
        } else {
            stage_values<C>(acc[h], reg, a, lane);
#pragma unroll 4
            for (int r4 = 0; r4 < C::EPI_ROWS / 4; ++r4) {
                const int rrow = 4 * r4 + (lane >> 4), chunk = lane & 15;
                const floatx4 xv = *reinterpret_cast<const floatx4 *>(reg + epi_offset(rrow, chunk));
                const int64_t gi = t.row0 + C::EPI_ROWS * h + rrow;
                if (gi < g.s) update_row4<PARAM_BF16>(d, g, p, gi, t.col0 + 4 * chunk, xv);
            }
        }
        wait_lgkm0();  // this round's LDS reads finish before a later DMA refills the area
        asm volatile("" ::: "memory");
    }
}

// DMA of 16 rows x 64 bf16 of W (row pitch ld bytes) into 2 KB of LDS, plain
// rows of 128 bytes: lane i of instruction t carries row 8t + i/8, chunk i%8.
__device__ __forceinline__ void dma_w_half(char *dst, const char *src, int64_t ld, int lane) {
#pragma unroll
    for (int t = 0; t < 2; ++t) dma16<true>(src + (8 * t + (lane >> 3)) * ld + (lane & 7) * 16, dst + t * 1024);
}

// The fused update for a bf16 W in the orientation of X', on a wave block that
// lies wholly inside W with 16-byte aligned rows (every block, by the launch
// condition), after the first step (X is a bounded iterate).  W is read once, straight
// from HBM, so its rows are brought by DMA into the wave's 4 KB of lds_wbuf a
// half round ahead (16 rows each): W(0) on entry, W(h+1)'s first half once
// round h's first half has used its buffer, its second half likewise.  The
// X rows come through the staging areas as in the other epilogues (round 0
// requested under the last K stage).  Per round the vector-memory stream is
// X(h+1) [6], the first half's stores [4, or 8 with O'], W(h+1) first half
// [2], the second half's stores, W(h+1) second half [2]; since they retire in
// issue order the waits below allow exactly the instructions issued after the
// one awaited (more when O' is stored, which only waits longer).
__device__ __forceinline__ void apply_epilogue_update_staged(const floatx16 (&acc)[Cfg::MI][Cfg::NI],
                                                             const MatDesc &d, const Geom &g, const Work &w,
                                                             const NsStep &p, const ApplyTile &t,
                                                             char *const (&area)[2], char *wb, int lane) {
    using C = Cfg;
    constexpr int ROUNDS = C::WM / C::EPI_ROWS;
    static_assert(ROUNDS == 4 && C::EPI_ROWS == 32 && C::WN == 64, "one 32 x 64 accumulator block per round");
    const XRows x = x_rows(g, w, t);
    const float a = p.unnormalized ? p.a * w.inv_norm[t.e] : p.a;
    uint16_t *const wrow0 = static_cast<uint16_t *>(d.param) + t.row0 * g.cols + t.col0;
    const char *const wsrc = reinterpret_cast<const char *>(wrow0);
    const int64_t wld = g.cols * 2;
    dma_w_half(wb, wsrc, wld, lane);
    dma_w_half(wb + 2048, wsrc + 16 * wld, wld, lane);
    const int rr = lane >> 4, chunk = lane & 15;
#pragma unroll
    for (int h = 0; h < ROUNDS; ++h) {
        char *reg = area[h & 1];
        if (h == 0)
            fenced_wait_vmcnt<2>();  // X(0), W(0) first half
        else
            fenced_wait_vmcnt<6>();  // X(h), W(h) first half
        if (h + 1 < ROUNDS) {
            dma_x_round(area[(h + 1) & 1], x, h + 1, lane);  // its area was last read in round h-1
            asm volatile("" ::: "memory");
        }
        stage_values<C>(acc[h], reg, a, lane);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (half == 1) {
                if (h + 1 < ROUNDS)
                    fenced_wait_vmcnt<12>();  // W(h) second half
                else
                    fenced_wait_vmcnt<4>();
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int rrow = 16 * half + 4 * k + rr;
                const floatx4 xv = *reinterpret_cast<const floatx4 *>(reg + epi_offset(rrow, chunk));
                const u32x2 w2 = *reinterpret_cast<const u32x2 *>(wb + half * 2048 + (rrow - 16 * half) * 128 + chunk * 8);
                u32x2 o;
                o[0] = pack_bf16x2(p.dscale * __uint_as_float(w2[0] << 16) - p.sscale * xv[0],
                                   p.dscale * __uint_as_float(w2[0] & 0xffff0000u) - p.sscale * xv[1]);
                o[1] = pack_bf16x2(p.dscale * __uint_as_float(w2[1] << 16) - p.sscale * xv[2],
                                   p.dscale * __uint_as_float(w2[1] & 0xffff0000u) - p.sscale * xv[3]);
                const int64_t widx = (C::EPI_ROWS * h + rrow) * g.cols + 4 * chunk;
                *as_global(reinterpret_cast<u32x2 *>(wrow0 + widx)) = o;
                if (d.ns_out)
                    *as_global(reinterpret_cast<floatx4 *>(d.ns_out + (t.row0 * g.cols + t.col0) + widx)) = xv;
            }
            wait_lgkm0();  // this half's LDS reads are done before its buffer is refilled
            asm volatile("" ::: "memory");
            if (h + 1 < ROUNDS) {
                dma_w_half(wb + half * 2048, wsrc + (C::EPI_ROWS * (h + 1) + 16 * half) * wld, wld, lane);
                asm volatile("" ::: "memory");
            }
        }
    }
}

// MODE 0: intermediate step (X' to the workspace); 1 / 2: last step with the
// fused update of an fp32 / bf16 parameter; 3: the same for a bf16 parameter
// through apply_epilogue_update_staged after the first step (NsStep::w_staged:
// no transpose, s and l multiples of 256, 16-byte aligned parameters).  One epilogue per
// instantiation keeps each within the register file.
template <int MODE>
__global__ __launch_bounds__(Cfg::NT, 1) void ns_apply_kernel(const MatDesc *__restrict__ descs, Geom g, Work w,
                                                               NsStep p, int64_t tiles_per_mat, int64_t nblocks) {
    using C = Cfg;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t L = xcd_swizzle(blockIdx.x, nblocks);
    const int64_t e = L / tiles_per_mat;
    const int64_t t = L % tiles_per_mat;
    // Consecutive tiles share a column panel of X (tile tj), walking down B.
    const int nti = static_cast<int>(g.sp / C::BM);
    const int tj = static_cast<int>(t / nti);
    const int ti = static_cast<int>(t % nti);

    Src src;
    src.ld_p = g.sp * 2;
    src.ld_q = g.lp * 2;
    src.p = static_cast<const char *>(w.bb) + e * w.a_stride * 2 + static_cast<int64_t>(ti) * C::BM * src.ld_p;
    src.q = static_cast<const char *>(w.xb) + e * w.x_stride * 2 + static_cast<int64_t>(tj) * C::BN * 2;

    floatx16 acc[C::MI][C::NI];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
    auto tile_of = [&] {
        return ApplyTile{e, static_cast<int64_t>(ti) * C::BM + wm * C::WM,
                         static_cast<int64_t>(tj) * C::BN + wn * C::WN};
    };
    // Before the last stage (slot 0 free): the first epilogue round into slot 0,
    // and for MODE 0 the second too (its X_hi into lds_wbuf, its X_lo into the
    // last 2 KB of the wave's part of slot 0).
    auto pre_last = [&] {
        const XRows xr = x_rows(g, w, tile_of());
        dma_x_round(epi_area<0>(wave), xr, 0, lane);
        if constexpr (MODE == 0)
            dma_x_round_to(lds_wbuf + wave * 4096, epi_area<0>(wave) + PAIR_HALF + 2048, xr, 1, lane);
    };
    main_loop<C, APPLY>(acc, src, static_cast<int>(k_extent(g.s, g.sp) / C::BK), wave, wm, wn, lane, pre_last);
    const ApplyTile t_ = tile_of();

    // Swapped product: acc[mi][ni][4*c4 + q] holds output row
    //   m = wm*WM + mi*32 + lane%32,  columns n = wn*WN + ni*32 + 8*c4 + 4*(lane/32) + q, q = 0..3
    // X_hi and X_lo of the aX term are staged through LDS in rounds of
    // EPI_ROWS rows, each wave loading its own slice with the DMA, then read
    // back in the accumulator layout.
    char *const area[2] = {epi_area<0>(wave), epi_area<1>(wave)};
    wait_lgkm0();
    stage_barrier();  // every wave is done with the operand ring
    if constexpr (MODE == 0)
        apply_epilogue_next(acc, g, w, p, t_, area[0], area[1], lds_wbuf + wave * 4096, lane);
    else if constexpr (MODE == 3)
        apply_epilogue_update_staged(acc, descs[e], g, w, p, t_, area, lds_wbuf + wave * 4096, lane);
    else
        apply_epilogue_update<MODE == 2>(acc, descs[e], g, w, p, t_, area, lane);
}

// The K range ks of tile tl of a split a X + B X launch (tiles [tile_base,
// tile_base + tile_count) of the chunk, in the order of ns_apply_kernel):
// the product only, stored as an fp32 partial tile (slot tl * splits + ks of
// w.kpart) for apply_reduce_kernel.  Workgroups of one K range are
// consecutive, so the tiles of one matrix read the same K slab of X.
__global__ __launch_bounds__(Cfg::NT, 1) void ns_apply_split_kernel(Geom g, Work w, int64_t tiles_per_mat,
                                                                     int64_t nblocks, int64_t tile_base,
                                                                     int64_t tile_count, int splits, int units) {
    using C = Cfg;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t L = xcd_swizzle(blockIdx.x, nblocks);
    const int ks = static_cast<int>(L / tile_count);
    const int64_t tl = L % tile_count;
    const int64_t f = tile_base + tl;
    const int64_t e = f / tiles_per_mat;
    const int64_t t = f % tiles_per_mat;
    const int nti = static_cast<int>(g.sp / C::BM);
    const int tj = static_cast<int>(t / nti);
    const int ti = static_cast<int>(t % nti);
    const int64_t kdim = k_extent(g.s, g.sp);
    const int64_t k0 = static_cast<int64_t>(ks) * units * 2 * C::BK;
    const int64_t k1 = min(kdim, k0 + static_cast<int64_t>(units) * 2 * C::BK);
    Src src;
    src.ld_p = g.sp * 2;
    src.ld_q = g.lp * 2;
    src.p = static_cast<const char *>(w.bb) + e * w.a_stride * 2 + static_cast<int64_t>(ti) * C::BM * src.ld_p + k0 * 2;
    src.q = static_cast<const char *>(w.xb) + e * w.x_stride * 2 + static_cast<int64_t>(tj) * C::BN * 2 + k0 * src.ld_q;
    floatx16 acc[C::MI][C::NI];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
    main_loop<C, APPLY>(acc, src, static_cast<int>((k1 - k0) / C::BK), wave, wm, wn, lane, [] {});
    store_kpart<C>(acc, w.kpart + (tl * splits + ks) * KPART_VALUES, wave, lane);
}

// Finishes the split tiles of a X + B X: the partials of each element summed
// in range order, then X' = a X + sum formed from the X pair and written as
// the pair (X'_hi to xb_next, X'_lo to xl in place), as the unsplit epilogue
// does.  Thread (item) = one partial float4 (wave, accumulator group, lane, as
// store_kpart laid them out): four consecutive columns of one row; 64 blocks
// of 256 threads per tile.
__global__ __launch_bounds__(256) void apply_reduce_kernel(Geom g, Work w, NsStep p, int64_t tiles_per_mat,
                                                           int64_t tile_base, int splits) {
    using C = Cfg;
    const int64_t tl = blockIdx.x / 64;
    const int64_t tile = tile_base + tl;
    const int item = static_cast<int>(blockIdx.x % 64) * 256 + threadIdx.x;
    const int64_t e = tile / tiles_per_mat;
    const int64_t t = tile % tiles_per_mat;
    const int nti = static_cast<int>(g.sp / C::BM);
    const int tj = static_cast<int>(t / nti), ti = static_cast<int>(t % nti);
    const floatx4 *src = reinterpret_cast<const floatx4 *>(w.kpart) + tl * splits * (KPART_VALUES / 4) + item;
    floatx4 sum = src[0];
    for (int k = 1; k < splits; ++k) {
        const floatx4 v = src[static_cast<int64_t>(k) * (KPART_VALUES / 4)];
#pragma unroll
        for (int q = 0; q < 4; ++q) sum[q] += v[q];
    }
    const int wave = item >> 11, j = (item >> 6) & 31, lane = item & 63;
    const int mi = j / (C::NI * 4), ni = (j / 4) % C::NI, c4 = j % 4;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t row = static_cast<int64_t>(ti) * C::BM + wm * C::WM + mi * 32 + (lane & 31);
    const int64_t col = static_cast<int64_t>(tj) * C::BN + wn * C::WN + ni * 32 + 8 * c4 + 4 * (lane >> 5);
    const int64_t off = e * w.x_stride + row * g.lp + col;
    const float a = p.unnormalized ? p.a * w.inv_norm[e] : p.a;
    const u32x2 hv = *as_global(reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(w.xb) + off));
    const uint32_t lv = *as_global(reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(w.xl) + off));
    const floatx4 x = join_bf16x4(hv, lv);
    floatx4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = __builtin_fmaf(a, x[q], sum[q]);
    u32x2 h;
    uint32_t l;
    split_bf16x4(v, &h, &l);
    *as_global(reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(w.xb_next) + off)) = h;
    *as_global(reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(w.xl) + off)) = l;
}

}  // namespace bf16path

hipError_t launch_ns_stage_bf16(int kind, const MatDesc *descs, int nmat, const Geom &g, const Work &w,
                                const NsStep &p, hipStream_t st) {
    using namespace bf16path;
    if (kind == GRAM || kind == POLY) {
        using C = Cfg;
        const int64_t nt = g.sp / C::BM;
        const int64_t tiles = nt * (nt + 1) / 2;
        const int64_t all = tiles * nmat;
        const int splits = kind == GRAM ? p.gram_splits : p.poly_splits;
        const int units = kind == GRAM ? p.gram_units : p.poly_units;
        // tiles [0, from) whole, [from, all) split over K (none when splits == 1)
        const int64_t from = splits > 1 ? std::min<int64_t>(std::max<int64_t>(p.split_from, 0), all) : all;
        auto launch = [&](int64_t base, int64_t count, int sp) {
            const int64_t nblocks = count * sp;
            const dim3 grid(static_cast<unsigned>(nblocks)), block(C::NT);
            if (kind == GRAM)
                ns_sym_kernel<C, GRAM><<<grid, block, 0, st>>>(g, w, p, tiles, nblocks, base, count, sp, units);
            else
                ns_sym_kernel<C, POLY><<<grid, block, 0, st>>>(g, w, p, tiles, nblocks, base, count, sp, units);
        };
        if (from > 0) launch(0, from, 1);
        if (from < all) {
            launch(from, all - from, splits);
            const dim3 rgrid(static_cast<unsigned>((all - from) * 64));
            if (kind == GRAM)
                sym_reduce_kernel<GRAM><<<rgrid, dim3(256), 0, st>>>(g, w, p, tiles, from, splits);
            else
                sym_reduce_kernel<POLY><<<rgrid, dim3(256), 0, st>>>(g, w, p, tiles, from, splits);
        }
        return hipGetLastError();
    }
    const int64_t tiles = (g.sp / Cfg::BM) * (g.lp / Cfg::BN);
    const int64_t nblocks = tiles * nmat;
    const dim3 block(Cfg::NT);
    if (!p.final_update) {
        // tiles [0, from) whole, [from, all) split over K (none when apply_splits == 1)
        const int64_t all = nblocks;
        const int64_t from =
            p.apply_splits > 1 ? std::min<int64_t>(std::max<int64_t>(p.apply_split_from, 0), all) : all;
        if (from > 0)
            ns_apply_kernel<0><<<dim3(static_cast<unsigned>(from)), block, 0, st>>>(descs, g, w, p, tiles, from);
        if (from < all) {
            const int64_t count = all - from, sblocks = count * p.apply_splits;
            ns_apply_split_kernel<<<dim3(static_cast<unsigned>(sblocks)), block, 0, st>>>(
                g, w, tiles, sblocks, from, count, p.apply_splits, p.apply_units);
            apply_reduce_kernel<<<dim3(static_cast<unsigned>(count * 64)), dim3(256), 0, st>>>(g, w, p, tiles, from,
                                                                                             p.apply_splits);
        }
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>(nblocks));
    if (p.param_bf16 && p.w_staged && !p.unnormalized)
        ns_apply_kernel<3><<<grid, block, 0, st>>>(descs, g, w, p, tiles, nblocks);
    else if (p.param_bf16)
        ns_apply_kernel<2><<<grid, block, 0, st>>>(descs, g, w, p, tiles, nblocks);
    else
        ns_apply_kernel<1><<<grid, block, 0, st>>>(descs, g, w, p, tiles, nblocks);
    return hipGetLastError();
}

}  // namespace muon
