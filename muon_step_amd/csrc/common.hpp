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
//   af + e*a_stride       fp32 A = X X^T (sp x sp, lower-triangle tiles)
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
    double *nrm2;         // per chunk matrix
    float *inv_norm;      // per chunk matrix: 1/||N||_F (0 when ||N|| == 0)
    double *call_nrm2;    // per call matrix (indexed by MatDesc::call_index)
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
// exact in fp32.  Below 2^-111 (exponent field < 16) only hi's precision is
// kept; infinite and NaN values are carried by hi alone.
__device__ __forceinline__ uint32_t lo8_encode(float x, uint32_t hbits) {
    // 2^(15 - e) from the exponent field, clamped to 16 .. 254: below 2^-111
    // the residual is far under one step and rounds to 0; for infinite or NaN
    // hi the residual is NaN, which converts to 0.
    const uint32_t ex = min(max((hbits >> 7) & 0xffu, 16u), 254u);
    const float t = (x - __uint_as_float(hbits << 16)) * __uint_as_float((269u - ex) << 23);  // exact
    const int q = min(max(static_cast<int>(rintf(t)), -128), 127);
    return static_cast<uint32_t>(q) & 0xffu;
}
// The residual of hi (hi's bits in the low 16 of hbits): q * 2^(e - 15), with
// the exponent taken from hi's bits and capped at 2^127 so that infinite or
// NaN hi (whose q is 0) gives 0.
__device__ __forceinline__ float lo8_decode(uint32_t qbyte, uint32_t hbits) {
    const float pow2e = __uint_as_float(min((hbits << 16) & 0x7f800000u, 0x7f000000u));
    return static_cast<float>(static_cast<int8_t>(qbyte & 0xffu)) * 0x1p-15f * pow2e;
}
__device__ __forceinline__ void split_bf16(float x, uint16_t *hi, uint8_t *lo) {
    const uint16_t h = float_to_bf16_bits(x);
    *hi = h;
    *lo = static_cast<uint8_t>(lo8_encode(x, h));
}
__device__ __forceinline__ float join_bf16(uint16_t hi, uint8_t lo) {
    return bf16_bits_to_float(hi) + lo8_decode(lo, hi);
}
// Four consecutive values: hi as packed bf16 pairs, the residuals as four
// bytes of one word (value k in byte k).
__device__ __forceinline__ void split_bf16x4(const floatx4 &v, u32x2 *hi, uint32_t *lo) {
    u32x2 h;
    h[0] = pack_bf16x2(v[0], v[1]);
    h[1] = pack_bf16x2(v[2], v[3]);
    *hi = h;
    *lo = lo8_encode(v[0], h[0] & 0xffffu) | (lo8_encode(v[1], h[0] >> 16) << 8) |
          (lo8_encode(v[2], h[1] & 0xffffu) << 16) | (lo8_encode(v[3], h[1] >> 16) << 24);
}
__device__ __forceinline__ floatx4 join_bf16x4(const u32x2 &h, uint32_t l) {
    floatx4 v;
    v[0] = __uint_as_float(h[0] << 16) + lo8_decode(l, h[0]);
    v[1] = __uint_as_float(h[0] & 0xffff0000u) + lo8_decode(l >> 8, h[0] >> 16);
    v[2] = __uint_as_float(h[1] << 16) + lo8_decode(l >> 16, h[1]);
    v[3] = __uint_as_float(h[1] & 0xffff0000u) + lo8_decode(l >> 24, h[1] >> 16);
    return v;
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
