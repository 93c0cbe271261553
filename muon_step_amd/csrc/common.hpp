// Shared device-side types and helpers of the Muon step library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Per-matrix pointers of one grouped launch (device table, one entry per
// matrix of the chunk being processed).
struct MatDesc {
    void *param;        // W, param dtype, rows x cols
    const void *grad;   // G, grad dtype, rows x cols
    float *mom;         // M, fp32, rows x cols
    float *ns_out;      // optional O'_t, fp32, rows x cols (nullptr = skip)
    int64_t call_index; // position of the matrix in the caller's list
    int64_t pad_;
};

// Geometry of one group of same-shape matrices.  The Newton-Schulz iterate is
// held as X (s x l, row-major, row pitch lp) with s = min(rows, cols),
// l = max(rows, cols); transposed != 0 when rows > cols (X = N^T).
struct Geom {
    int64_t rows, cols;   // W shape
    int64_t s, l;         // X shape
    int64_t sp, lp;       // padded X shape (multiples of the GEMM tiles)
    int32_t transposed;
    int32_t pad_;
};

// Workspace of one chunk: matrix e of the chunk owns
//   xf      + e*x_stride  fp32 X (sp x lp), read by the current step (fp32 path)
//   xf_next + e*x_stride  where the current step writes X (fp32 path)
//   xb      + e*x_stride  X_hi, X rounded to bf16 by the pair codec below: the
//                         MFMA operand (bf16 path)
//   xb_next + e*x_stride  where the current step writes X_hi: the product B X
//                         reads whole column panels of X, so X_hi is
//                         double-buffered
//   xl      + e*x_stride  X_lo, the 8-bit residual of X - X_hi (one byte per
//                         element), rewritten in place by the tile that owns
//                         the elements (bf16 path)
//   af + e*a_stride       fp32 A = X X^T (sp x sp, lower-triangle tiles; fp32
//                         path only, nullptr on the bf16 path)
//   ab + e*a_stride       A as MFMA operand (bf16 or fp32, both triangles)
//   bb + e*a_stride       B = bA + cA^2 as MFMA operand (both triangles)
// Newton-Schulz workspace of one chunk of same-shape matrices.  fp32 path: X
// in xf / xf_next (fp32).  bf16 path: X as hi (bf16) in xb / xb_next
// (ping-pong: it is the operand every tile of the B X product reads) and the
// 8-bit residual lo in xl (updated in place), xf == xf_next == nullptr.
struct Work {
    float *xf;
    float *xf_next;
    void *xb;
    void *xb_next;
    void *xl;
    float *af;
    void *ab;
    void *bb;
    int64_t x_stride;
    int64_t a_stride;
    double *partials;     // per-block sums of N^2
    double *nrm2;         // per chunk matrix: ||N||_F^2
    // per chunk matrix: the factor the bf16 path's first Newton-Schulz step
    // folds into its epilogues (X_0 = N inv_norm): fl32(1/||N||_F); 1 for a
    // matrix that the pre-normalisation pass already scaled (prenormalize());
    // 0 when ||N|| == 0; NaN when ||N||^2 is not finite.
    float *inv_norm;
    double *call_nrm2;    // per call matrix (indexed by MatDesc::call_index)
    const float *uscale;  // per chunk matrix update scale s (unit-RMS mode), else nullptr
    // split-K Gram / A^2 (bf16 path): the fp32 partial product of every
    // (matrix, tile, K range), 256 x 256 values each, in the lane-major order
    // the product kernel stores them; nullptr when the chunk splits no product
    float *kpart;
};

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bfloat16 bits.  gfx950 does this in one
// instruction (v_cvt_pk_bf16_f32) when the compiler lowers the cast.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 p;
    p[0] = static_cast<__bf16>(lo);
    p[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, p);
}

// A float kept as a bf16 hi and an 8-bit residual lo, by integer arithmetic
// on its bit pattern b (monotonic in |x|, sign bit apart):
//   hi = bits 16..31 of b + 0x8080,   lo = bits 8..15 of b + 0x80,
//   decoded b' = (hi << 16) + (int8(lo) << 8),   |b' - b| <= 0x80.
// lo is the next byte of b rounded to 24 bits (to nearest on the pattern,
// halves up), read as a signed offset from hi, so x is carried to 2^-16 of
// its magnitude at every finite value, subnormals included: 0x80 units of the
// last place of an fp32 significand.  hi is x rounded to the nearest bf16,
// except that low halves in [0x7f80, 0x8000] round up: at most 0.502 ulp from
// x.  All-zero bytes decode to +0, and a residual of 0 to hi itself.  Before
// the addition b is capped at 0x7fff7f7f as a signed integer and the sum
// saturates as an unsigned one, so the carry never reaches the sign bit and
// every quiet NaN stays a NaN; finite values within 0x80 units of the largest
// float get an infinite hi and still decode to themselves.  Signalling NaNs
// with a payload below 0x7f80 (never the result of arithmetic) would decode
// as infinities; data read from memory passes __builtin_canonicalizef first.
__device__ __forceinline__ uint32_t pair_sum(float x) {
    const int32_t b = __builtin_elementwise_min(__float_as_int(x), 0x7fff7f7f);
    return __builtin_elementwise_add_sat(static_cast<uint32_t>(b), 0x8080u);
}
__device__ __forceinline__ void split_bf16(float x, uint16_t *hi, uint8_t *lo) {
    const uint32_t y = pair_sum(x);
    *hi = static_cast<uint16_t>(y >> 16);
    *lo = static_cast<uint8_t>(((y >> 8) & 0xffu) ^ 0x80u);
}
// b' from the bytes P = hi << 16 | lo << 8: (P ^ 0x8000) - 0x8000 in one
// v_xad_u32 (a VOP3 operation reads at most one scalar or constant operand, so
// the compiler would otherwise split it; -0x8000 is given in a VGPR).
__device__ __forceinline__ float join_bits(uint32_t p) {
    uint32_t r;
    asm("v_xad_u32 %0, %1, %2, %3" : "=v"(r) : "v"(p), "s"(0x8000u), "v"(0xffff8000u));
    return __uint_as_float(r);
}
__device__ __forceinline__ float join_bf16(uint16_t hi, uint8_t lo) {
    return join_bits((static_cast<uint32_t>(hi) << 16) | (static_cast<uint32_t>(lo) << 8));
}
// Four consecutive values: hi as packed bf16 pairs (value 2k in the low half
// of word k), the residuals as the four bytes of one word (value k in byte k).
__device__ __forceinline__ void split_bf16x4(const floatx4 &v, u32x2 *hi, uint32_t *lo) {
    uint32_t y[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = pair_sum(v[k]);
    // v_perm_b32 picks bytes of {src0, src1} (src1 = bytes 0..3, src0 = 4..7)
    (*hi)[0] = __builtin_amdgcn_perm(y[1], y[0], 0x07060302u);
    (*hi)[1] = __builtin_amdgcn_perm(y[3], y[2], 0x07060302u);
    const uint32_t l01 = __builtin_amdgcn_perm(y[1], y[0], 0x07060501u);  // bytes 1 of y0, y1
    const uint32_t l23 = __builtin_amdgcn_perm(y[3], y[2], 0x07060501u);
    *lo = __builtin_amdgcn_perm(l23, l01, 0x05040100u) ^ 0x80808080u;
}
__device__ __forceinline__ floatx4 join_bf16x4(const u32x2 &h, uint32_t l) {
    floatx4 v;
    // bytes [0, l.k, h.lo16 of value k] with 0x0c selecting a zero byte
    v[0] = join_bits(__builtin_amdgcn_perm(h[0], l, 0x0504000cu));
    v[1] = join_bits(__builtin_amdgcn_perm(h[0], l, 0x0706010cu));
    v[2] = join_bits(__builtin_amdgcn_perm(h[1], l, 0x0504020cu));
    v[3] = join_bits(__builtin_amdgcn_perm(h[1], l, 0x0706030cu));
    return v;
}

// Pointers read from descriptor tables are generic to the compiler, which
// then addresses them with flat instructions (which also count as LDS
// accesses in lgkmcnt).  Every such pointer here points to device memory.
template <class T> __device__ __forceinline__ __attribute__((address_space(1))) T *as_global(T *p) {
    return (__attribute__((address_space(1))) T *)p;
}

// Range of ||N||_F^2 inside which the bf16 path keeps X = N through its first
// Gram and folds 1/||N|| into the epilogues.  Inside it the products of N's
// entries that make up N N^T stay far inside fp32's normal range for any
// matrix of up to 2^40 elements (mean square entry >= 2^-80), and the sums
// far below its maximum.  A matrix outside it (a vanishing momentum, e.g. an
// expert that received no tokens for hundreds of steps, or a huge one) is
// normalised first: X = N / ||N||_F computed in double, so the step does not
// depend on the scale of N (the Frobenius normalisation line of the expanded
// Algorithm 1, DeepSeek-V4 book ch. 6 section 5).  A non-finite norm is not
// normalised: it makes the whole output NaN.
__host__ __device__ inline bool prenormalize(double nrm2) {
    return (nrm2 > 0.0 && nrm2 < 0x1p-40) || (nrm2 > 0x1p40 && nrm2 <= 1.7976931348623157e308);
}

// Blocks whose ids the hardware spreads round-robin over the 8 XCDs are
// renumbered so that consecutive logical ids run on the same XCD (and share
// its L2).  Bijective on [0, nblocks).
__device__ __forceinline__ int64_t xcd_swizzle(int64_t b, int64_t nblocks) {
    const int64_t n_xcd = 8;
    int64_t q = nblocks / n_xcd;
    if (b >= q * n_xcd) return b;
    return (b % n_xcd) * q + b / n_xcd;
}

}  // namespace muon
