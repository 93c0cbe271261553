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
//   xl      + e*x_stride  X_lo = bf16(X - X_hi), rewritten in place by the
//                         tile that owns the elements (bf16 path)
//   af + e*a_stride       fp32 A = X X^T (sp x sp, lower-triangle tiles)
//   ab + e*a_stride       A as MFMA operand (bf16 or fp32, both triangles)
//   bb + e*a_stride       B = bA + cA^2 as MFMA operand (both triangles)
// Newton-Schulz workspace of one chunk of same-shape matrices.  fp32 path: X
// in xf / xf_next (fp32).  bf16 path: X as a pair of bf16 arrays, hi in
// xb / xb_next (ping-pong: it is the operand every tile of the B X product
// reads) and lo in xl (updated in place), xf == xf_next == nullptr.
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

// A float kept as two bfloat16: hi = bf16(x), lo = bf16(x - hi).  x - hi is
// exact in fp32 (hi is within half a bf16 ulp of x), so hi + lo carries x to
// about 2^-17 relative, and hi + lo is exact in fp32.
__device__ __forceinline__ void split_bf16(float x, uint16_t *hi, uint16_t *lo) {
    const uint16_t h = float_to_bf16_bits(x);
    *hi = h;
    *lo = float_to_bf16_bits(x - bf16_bits_to_float(h));
}
__device__ __forceinline__ float join_bf16(uint16_t hi, uint16_t lo) {
    return bf16_bits_to_float(hi) + bf16_bits_to_float(lo);
}
// Four consecutive values: hi and lo as packed bf16 pairs.
__device__ __forceinline__ void split_bf16x4(const floatx4 &v, u32x2 *hi, u32x2 *lo) {
    u32x2 h, l;
    h[0] = pack_bf16x2(v[0], v[1]);
    h[1] = pack_bf16x2(v[2], v[3]);
    l[0] = pack_bf16x2(v[0] - __uint_as_float(h[0] << 16), v[1] - __uint_as_float(h[0] & 0xffff0000u));
    l[1] = pack_bf16x2(v[2] - __uint_as_float(h[1] << 16), v[3] - __uint_as_float(h[1] & 0xffff0000u));
    *hi = h;
    *lo = l;
}
__device__ __forceinline__ floatx4 join_bf16x4(const u32x2 &h, const u32x2 &l) {
    floatx4 v;
    v[0] = __uint_as_float(h[0] << 16) + __uint_as_float(l[0] << 16);
    v[1] = __uint_as_float(h[0] & 0xffff0000u) + __uint_as_float(l[0] & 0xffff0000u);
    v[2] = __uint_as_float(h[1] << 16) + __uint_as_float(l[1] << 16);
    v[3] = __uint_as_float(h[1] & 0xffff0000u) + __uint_as_float(l[1] & 0xffff0000u);
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
