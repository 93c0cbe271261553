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
//   xb      + e*x_stride  X_hi = bf16(X), the MFMA operand (bf16 path)
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

// A float kept as hi = bf16(x) and a signed 8-bit residual q:
//   x ~= hi + q * 2^(e - 15),  e the exponent of hi,  q = rne((x - hi) 2^(15 - e))
// clamped to [-128, 127].  x - hi is exact in fp32 and at most half a bf16
// ulp (2^(e - 8)), so |q| <= 128 and the residual's rounding error is at most
// 2^(e - 16), or 2^(e - 15) where q clamps: x is carried to 2^-15 relative
// (2^-16 but for that clamp).  hi + q 2^(e - 15) spans at most 17 bits and is
// exact in fp32.
//
// The unit 2^(e - 15) is never formed.  The codec works against a reference
// float m whose exponent is e + 8 and whose mantissa is 0.5 (plus, in the
// paired form, a few low bits that change nothing): m sits mid-binade with
// ulp 2^(e - 15), so the single rounding of m + (x - hi) rounds x - hi to a
// multiple of the unit (to nearest, ties to even q) and leaves q as the
// difference of the two bit patterns; decoding adds q to m's bits and
// subtracts m, both exact.  e is capped at 119 (|hi| < 2^120; above that only
// hi's precision is kept, and infinite or NaN hi absorbs any residual); below
// 2^-126 the unit is still consistent, with hi's precision the limit.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t s16x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t LO8_REF_ADD = 0x04400000u;  // exponent + 8, mantissa 0.5
constexpr uint32_t LO8_EXP_CAP = 246u << 23;    // exponent field 246 (e = 119)

// Reference bits for one hi given as fp32 bits.
__device__ __forceinline__ uint32_t lo8_ref(uint32_t hf_bits) {
    return min(hf_bits & 0x7f800000u, LO8_EXP_CAP) + LO8_REF_ADD;
}
// Reference bits for the two bf16 of one packed pair (element 0 in the low
// half).  m1 keeps element 0's capped exponent in its bits 14..7: mantissa
// bits far below m's top bit that leave its binade, its ulp and its last bit
// (hence ties) unchanged.
__device__ __forceinline__ void lo8_ref2(uint32_t h2, uint32_t *m0, uint32_t *m1) {
    const u16x2 cap = {static_cast<uint16_t>(LO8_EXP_CAP >> 16), static_cast<uint16_t>(LO8_EXP_CAP >> 16)};
    const uint32_t eb = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, h2 & 0x7f807f80u), cap));
    *m0 = (eb << 16) + LO8_REF_ADD;
    *m1 = eb + LO8_REF_ADD;
}
// q of x against hi (as a float) and its reference bits.
__device__ __forceinline__ int lo8_q(float x, float hf, uint32_t mb) {
    const float t = (x - hf) + __uint_as_float(mb);  // x - hf exact; one rounding to the unit
    return min(max(static_cast<int>(__float_as_uint(t) - mb), -128), 127);
}
// The residual q * 2^(e - 15) from q and the reference bits.
__device__ __forceinline__ float lo8_value(int q, uint32_t mb) {
    return __uint_as_float(mb + static_cast<uint32_t>(q)) - __uint_as_float(mb);
}
__device__ __forceinline__ void split_bf16(float x, uint16_t *hi, uint8_t *lo) {
    const uint16_t h = float_to_bf16_bits(x);
    const uint32_t hb = static_cast<uint32_t>(h) << 16;
    *hi = h;
    *lo = static_cast<uint8_t>(lo8_q(x, __uint_as_float(hb), lo8_ref(hb)) & 0xff);
}
__device__ __forceinline__ float join_bf16(uint16_t hi, uint8_t lo) {
    const uint32_t hb = static_cast<uint32_t>(hi) << 16;
    return __uint_as_float(hb) + lo8_value(static_cast<int8_t>(lo), lo8_ref(hb));
}
// Four consecutive values: hi as packed bf16 pairs, the residuals as four
// bytes of one word (value k in byte k).  BOUNDED: the caller guarantees
// |x| < 2^120 or a non-finite hi (a Newton-Schulz iterate of a normalised
// matrix), so the exponent cap is not needed: for infinite or NaN hi the
// reference overflows, q is meaningless and the decode (which caps) adds a
// finite residual to a non-finite hi.
template <bool BOUNDED = false>
__device__ __forceinline__ void split_bf16x4(const floatx4 &v, u32x2 *hi, uint32_t *lo) {
    u32x2 h;
    h[0] = pack_bf16x2(v[0], v[1]);
    h[1] = pack_bf16x2(v[2], v[3]);
    // opaque to the optimiser, which would otherwise convert each value to
    // bf16 a second time to get its float hi
    asm volatile("" : "+v"(h[0]), "+v"(h[1]));
    *hi = h;
    if (BOUNDED) {
        // References with clear low halves: the low 16 bits of the rounded
        // sum are then q itself (|q| <= 128 never borrows across bit 16), two
        // of them gather into one register and one packed min clamps both
        // (q >= -128 always holds).
        u32x2 qq;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint32_t m0 = ((h[k] & 0x7f80u) << 16) + LO8_REF_ADD;
            const uint32_t m1 = (h[k] & 0x7f800000u) + LO8_REF_ADD;
            const float t0 = (v[2 * k] - __uint_as_float(h[k] << 16)) + __uint_as_float(m0);
            const float t1 = (v[2 * k + 1] - __uint_as_float(h[k] & 0xffff0000u)) + __uint_as_float(m1);
            // v_perm_b32 picks bytes of {src0, src1} (src1 = bytes 0..3)
            const uint32_t g = __builtin_amdgcn_perm(__float_as_uint(t1), __float_as_uint(t0), 0x05040100u);
            const s16x2 c = {127, 127};
            qq[k] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(s16x2, g), c));
        }
        *lo = __builtin_amdgcn_perm(qq[1], qq[0], 0x06040200u);
        return;
    }
    int q[4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        uint32_t m0, m1;
        lo8_ref2(h[k], &m0, &m1);
        q[2 * k] = lo8_q(v[2 * k], __uint_as_float(h[k] << 16), m0);
        q[2 * k + 1] = lo8_q(v[2 * k + 1], __uint_as_float(h[k] & 0xffff0000u), m1);
    }
    // v_perm_b32 picks bytes of {src0, src1} (src1 = bytes 0..3; 0x0c = zero)
    const uint32_t p01 = __builtin_amdgcn_perm(static_cast<uint32_t>(q[1]), static_cast<uint32_t>(q[0]), 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm(static_cast<uint32_t>(q[3]), static_cast<uint32_t>(q[2]), 0x0c0c0400u);
    *lo = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}
// BOUNDED: the values were written by split_bf16x4<true> (|x| < 2^120 or a
// non-finite hi), so the exponent cap is not needed either.
template <bool BOUNDED = false>
__device__ __forceinline__ floatx4 join_bf16x4(const u32x2 &h, uint32_t l) {
    floatx4 v;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        uint32_t m0, m1;
        if (BOUNDED) {
            const uint32_t eb = h[k] & 0x7f807f80u;
            m0 = (eb << 16) + LO8_REF_ADD;
            m1 = eb + LO8_REF_ADD;
        } else {
            lo8_ref2(h[k], &m0, &m1);
        }
        const int q0 = static_cast<int8_t>((l >> (16 * k)) & 0xffu);
        const int q1 = static_cast<int8_t>((l >> (16 * k + 8)) & 0xffu);
        v[2 * k] = __uint_as_float(h[k] << 16) + lo8_value(q0, m0);
        v[2 * k + 1] = __uint_as_float(h[k] & 0xffff0000u) + lo8_value(q1, m1);
    }
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
