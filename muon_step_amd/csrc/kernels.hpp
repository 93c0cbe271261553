// Internal launchers of the Muon step library (host side of the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace muon {

struct AdamwScalars {
    float decay, beta1, beta2, one_minus_beta1, one_minus_beta2, bias_corr1, bias_corr2, lr, eps;
};

// Newton-Schulz GEMM tile: every padded X dimension is a multiple of this.
constexpr int kTile = 256;

// ---- fixed scratch of the allocation-free step (noalloc.hip)
// Size of the static device array; equal to MUON_NOALLOC_SCRATCH_BYTES.
constexpr size_t kScratchBytes = size_t(128) << 20;
// Device address of the current device's copy of the array.
hipError_t scratch_address(void **out);

// ---- elementwise (elementwise.hip)
// Workgroups per matrix of the momentum pass, and so its ||N||^2 partial sums
// per matrix: one per 4096 consecutive elements (rows <= cols), or one per
// 64 x 64 tile of W when X is W transposed (*tiles_c: tiles per tile row).
int nesterov_blocks_per_mat(const Geom &g, int *tiles_c);
hipError_t launch_nesterov(const MatDesc *descs, int nmat, const Geom &g, const Work &w, float mu,
                           int nesterov, int grad_bf16, bool vec_ok, hipStream_t st);
hipError_t launch_norm_finalize(const MatDesc *descs, int nmat, const Work &w, int blocks_per_mat,
                                hipStream_t st);
hipError_t launch_import_n(const float *n_in, const Geom &g, const Work &w, hipStream_t st);
int import_n_blocks(const Geom &g);
// X_0 = N / ||N||_F per matrix; prenorm_only: only the matrices whose norm
// lies outside the bf16 fold range (prenormalize()).
hipError_t launch_normalize(int nmat, const Geom &g, const Work &w, int prenorm_only, hipStream_t st);
hipError_t launch_pad_zero(int nmat, const Geom &g, const Work &w, hipStream_t st);
// s_dev, when non-null, is a device float read in place of s.
hipError_t launch_update_plain(void *param, int param_bf16, const float *x, int64_t n, float d,
                               float s, const float *s_dev, hipStream_t st);
// Unit-RMS scale: out[e] = fl32(lr * (gsq / ||X_e||_F)), gsq = gamma * sqrt(rows * cols),
// 0 when X_e = 0; ||X_e||^2 summed in fp64 over the valid s x l region of
// workspace X (x_override, when non-null, is one plain fp32 s x l matrix with
// pitch g.lp instead).  Uses w.partials[0 .. nmat * blocks_per_mat).
hipError_t launch_unit_rms_scale(int nmat, const Geom &g, const Work &w, const float *x_override,
                                 int blocks_per_mat, double lr, double gsq, float *out, hipStream_t st);
// Decay + update from workspace X (per-matrix scale w.uscale when set).
// aligned16: every param and ns_out of the chunk is 16-byte aligned, which
// lets the untransposed bf16-workspace case take 8 elements per lane.
hipError_t launch_update_from_work(const MatDesc *descs, int nmat, const Geom &g, const Work &w,
                                   int param_bf16, float d, float s, bool aligned16, hipStream_t st);
hipError_t launch_export_x(const Geom &g, const Work &w, float *out, hipStream_t st);
// Operands of a single product stage: fp32 s x l X into the pair (w.xb, w.xl),
// fp32 s x s into a bf16 sp x sp operand, and such an operand back to fp32.
hipError_t launch_import_pair(const Geom &g, const float *x, const Work &w, hipStream_t st);
hipError_t launch_import_bf16_square(int64_t s, int64_t sp, const float *m, void *dst, hipStream_t st);
hipError_t launch_export_bf16_square(int64_t s, int64_t sp, const void *src, float *out, hipStream_t st);
int64_t adamw_blocks(int64_t numel);
hipError_t launch_adamw(const void *descs_dev, int count, int64_t total_blocks, const AdamwScalars &k,
                        hipStream_t st);
size_t adamw_desc_size();
// Streaming probe: `reads` source and `writes` destination streams of nvec
// 16-byte vectors each, `pitch` vectors apart ((reads, writes) in {(6,7),
// (4,3), (5,2), (1,1)}).
hipError_t launch_stream_probe(const void *src, void *dst, int64_t nvec, int64_t pitch, int reads, int writes,
                               hipStream_t st);
void adamw_fill_desc(void *dst, float *param, const float *grad, float *m, float *v, int64_t numel,
                     int64_t first_block);

// ---- Newton-Schulz products (ns_bf16.hip, ns_f32.hip)
// One Newton-Schulz step on every matrix of the chunk:
//   A = X X^T (lower-triangle tiles, mirrored), B = b A + c A A (lower-triangle
//   tiles, mirrored), X <- a X + B X.
// When `final_update` is set, the last product writes W_t (and ns_out) instead
// of X:  W <- d W - s (a X + B X).
struct NsStep {
    float a, b, c;
    int final_update;
    int param_bf16;
    float dscale, sscale;
    // bf16 path, first step: the workspace X holds N itself; the Gram is
    // scaled by inv_norm^2 and a X + B X by inv_norm (X_0 = N inv_norm).
    int unnormalized;
    // bf16 path, last step: W rows may be staged through LDS (no transpose,
    // s and l multiples of 256, every parameter and ns_out 16-byte aligned).
    int w_staged;
    // last step: every parameter and ns_out of the chunk is 16-byte aligned,
    // so the per-element fused update may move four elements per access.
    int vec_ok;
    // bf16 Gram and A^2 products: the chunk's lower-triangle tiles from
    // split_from on (in the order (matrix, tile of the matrix); 0: all of them)
    // run with K split into `splits` ranges of `units` x 128 (the last may be
    // shorter) whose fp32 partial tiles a reduce finishes; splits == 1: no
    // tile is split.
    int gram_splits, gram_units;
    int poly_splits, poly_units;
    int64_t split_from;
    // bf16 a X + B X of an intermediate step, likewise: the chunk's tiles
    // (matrix, tile row within the column panel) from apply_split_from on run
    // with K (= s) split into apply_splits ranges of apply_units x 128; a
    // reduce adds a X and writes the X' pair.  The last step is never split.
    int apply_splits, apply_units;
    int64_t apply_split_from;
};

// kind: 0 = A = X X^T, 1 = B = bA + cA^2, 2 = X <- aX + BX (or the fused update).
hipError_t launch_ns_stage_bf16(int kind, const MatDesc *descs, int nmat, const Geom &g, const Work &w,
                                const NsStep &p, hipStream_t st);
hipError_t launch_ns_stage_f32(int kind, const MatDesc *descs, int nmat, const Geom &g, const Work &w,
                               const NsStep &p, hipStream_t st);
inline hipError_t launch_ns_stage(int kind, bool bf16, const MatDesc *descs, int nmat, const Geom &g,
                                  const Work &w, const NsStep &p, hipStream_t st) {
    return bf16 ? launch_ns_stage_bf16(kind, descs, nmat, g, w, p, st)
                : launch_ns_stage_f32(kind, descs, nmat, g, w, p, st);
}

}  // namespace muon
