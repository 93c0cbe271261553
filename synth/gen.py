"""Seeded synthetic inputs (numpy PCG64; an optional torch path for bench scale).

Gradient law for the spectral workloads ("low rank plus noise"): for an
n x m matrix with s = min(n, m),

    G = bf16( U diag(sigma) V^T + E ),
    sigma_j = exp(Uniform(ln 1e-4, ln 1e-1)),  j < s
    U (n x s), V (m x s) Haar-distributed with orthonormal columns
    E_ij ~ Normal(0, std 1e-5)

which reproduces the gradient spectrum the DeepSeek-V4 book (ch. 6, §1)
describes for LLM training: top singular value ~1e-1, weakest ~1e-4..1e-3.
Parameters are Normal(0, std 0.02); the momentum buffer is zero unless a
workload asks for it to be pre-filled with a prior-step gradient drawn from
the same law.

Every matrix i of a workload draws from its own child of
SeedSequence(base_seed), with separate grandchildren for sigma, U, V, noise,
W and the prior gradient, so any subset of matrices can be regenerated alone.
"""

from dataclasses import dataclass, field
import math

import numpy as np

SIGMA_LO = 1e-4
SIGMA_HI = 1e-1
NOISE_STD = 1e-5
PARAM_STD = 0.02

# Streams of one matrix's SeedSequence children.
_S_SIGMA, _S_U, _S_V, _S_NOISE, _S_W, _S_GPREV, _S_GAUSS = range(7)


@dataclass(frozen=True)
class MatrixSpec:
    rows: int
    cols: int
    param_dtype: str = "bf16"    # "bf16" | "f32"
    grad_dtype: str = "bf16"     # "bf16" | "f32"
    law: str = "spectral"        # "spectral" | "gauss"
    prefill_momentum: bool = False
    name: str = ""


@dataclass(frozen=True)
class Workload:
    name: str
    base_seed: int
    matrices: tuple
    adamw: tuple = field(default_factory=tuple)   # tuple of (name, numel)
    description: str = ""

    @property
    def muon_elems(self):
        return sum(mm.rows * mm.cols for mm in self.matrices)


def _c5_matrices():
    mats = []
    for layer in range(27):
        for k in range(4):
            mats.append(MatrixSpec(2048, 2048, name=f"l{layer}.attn{k}"))
        for e in range(64):
            mats.append(MatrixSpec(2048, 1408, name=f"l{layer}.e{e}.up"))
            mats.append(MatrixSpec(2048, 1408, name=f"l{layer}.e{e}.gate"))
            mats.append(MatrixSpec(1408, 2048, name=f"l{layer}.e{e}.down"))
    return tuple(mats)


WORKLOADS = {
    "single_f32_64x128": Workload(
        "single_f32_64x128", 0,
        (MatrixSpec(64, 128, "f32", "f32", law="gauss", name="w"),),
        description="one fp32 64x128 matrix, N(0,1) gradient, zero momentum"),
    "dense_block_bf16": Workload(
        "dense_block_bf16", 2,
        tuple([MatrixSpec(4096, 4096, name=f"attn{k}") for k in range(4)]
              + [MatrixSpec(4096, 14336, name="ffn_up"), MatrixSpec(4096, 14336, name="ffn_gate"),
                 MatrixSpec(14336, 4096, name="ffn_down")]),
        description="4 x 4096^2 attention, 2 x 4096x14336 and 1 x 14336x4096 FFN, bf16"),
    "aspect_stress_bf16": Workload(
        "aspect_stress_bf16", 3,
        (MatrixSpec(1024, 16384, prefill_momentum=True, name="wide"),
         MatrixSpec(16384, 1024, prefill_momentum=True, name="tall"),
         MatrixSpec(7168, 7168, prefill_momentum=True, name="square"),
         MatrixSpec(512, 32768, prefill_momentum=True, name="very_wide")),
        description="1024x16384, 16384x1024, 7168^2, 512x32768 bf16, momentum pre-filled"),
    "moe_256x2048x7168_bf16": Workload(
        "moe_256x2048x7168_bf16", 4,
        tuple(MatrixSpec(2048, 7168, name=f"expert{e}") for e in range(256)),
        description="256 MoE expert matrices 2048x7168 bf16, batched"),
    "moe16b_full_step": Workload(
        "moe16b_full_step", 5, _c5_matrices(),
        adamw=(("embedding", 102400 * 2048), ("head", 102400 * 2048)),
        description="27 layers x (4 x 2048^2 + 64 x (2048x1408 up, gate; 1408x2048 down)) bf16 "
                    "+ AdamW on 2 x 102400x2048 fp32"),
}


def bf16_bits_round(x):
    """float array -> uint16 bfloat16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    r = r.astype(np.uint32)
    nan = np.isnan(x)
    r = np.where(nan, (u >> np.uint64(16)).astype(np.uint32) | np.uint32(0x40), r)
    return (r & np.uint32(0xFFFF)).astype(np.uint16)


def _bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _children(base_seed, index):
    top = np.random.SeedSequence(base_seed)
    # spawn() is deterministic in the index: child i of SeedSequence(base) has
    # spawn_key (i,), so one matrix can be regenerated without the others.
    mat = np.random.SeedSequence(top.entropy, spawn_key=(index,))
    return mat.spawn(7)


def gaussian_f32(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


def _haar_columns(rng, rows, cols):
    """rows x cols matrix with Haar-distributed orthonormal columns (cols <= rows)."""
    z = rng.standard_normal((rows, cols))
    q, r = np.linalg.qr(z)
    d = np.sign(np.diag(r))
    d[d == 0] = 1.0
    return q * d


def spectral_grad(rows, cols, seeds):
    """Low-rank-plus-noise gradient (float64, before any rounding)."""
    s = min(rows, cols)
    rs = np.random.Generator(np.random.PCG64(seeds[_S_SIGMA]))
    sigma = np.exp(rs.uniform(math.log(SIGMA_LO), math.log(SIGMA_HI), size=s))
    u = _haar_columns(np.random.Generator(np.random.PCG64(seeds[_S_U])), rows, s)
    v = _haar_columns(np.random.Generator(np.random.PCG64(seeds[_S_V])), cols, s)
    rn = np.random.Generator(np.random.PCG64(seeds[_S_NOISE]))
    return (u * sigma) @ v.T + rn.standard_normal((rows, cols)) * NOISE_STD


def _cast(x, dtype):
    """Returns (float32 values, raw array in the storage dtype)."""
    if dtype == "bf16":
        bits = bf16_bits_round(np.asarray(x, dtype=np.float32))
        return _bits_to_f32(bits), bits
    x32 = np.asarray(x, dtype=np.float32)
    return x32, x32


def matrix_inputs(workload, index):
    """Inputs of matrix `index` of `workload`.

    Returns a dict with float32 views ("w", "g", "m") holding the exact values
    and raw storage arrays ("w_raw", "g_raw": uint16 bfloat16 bits or float32).
    """
    spec = workload.matrices[index]
    seeds = _children(workload.base_seed, index)
    shape = (spec.rows, spec.cols)
    if spec.law == "gauss":
        g = np.random.Generator(np.random.PCG64(seeds[_S_GAUSS])).standard_normal(shape)
    else:
        g = spectral_grad(spec.rows, spec.cols, seeds)
    g32, g_raw = _cast(g, spec.grad_dtype)
    w = np.random.Generator(np.random.PCG64(seeds[_S_W])).standard_normal(shape) * PARAM_STD
    w32, w_raw = _cast(w, spec.param_dtype)
    if spec.prefill_momentum:
        prev = spectral_grad(spec.rows, spec.cols, seeds[_S_GPREV].spawn(7))
        m32, _ = _cast(prev, spec.grad_dtype)
        m32 = np.array(m32, dtype=np.float32)
    else:
        m32 = np.zeros(shape, dtype=np.float32)
    return {"w": w32, "g": g32, "m": m32, "w_raw": w_raw, "g_raw": g_raw, "spec": spec}


def adamw_inputs(numel, seed, step=1):
    """fp32 AdamW inputs: p ~ N(0, 0.02), g ~ N(0, 1); zero state at step 1,
    and a prefilled state (m ~ N(0, 0.1), v = |N(0, 1)| * 1e-2) otherwise."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    p = (rng.standard_normal(numel) * PARAM_STD).astype(np.float32)
    g = rng.standard_normal(numel).astype(np.float32)
    if step == 1:
        m = np.zeros(numel, np.float32)
        v = np.zeros(numel, np.float32)
    else:
        m = (rng.standard_normal(numel) * 0.1).astype(np.float32)
        v = (np.abs(rng.standard_normal(numel)) * 1e-2).astype(np.float32)
    return p, g, m, v


def spectral_grad_torch(rows, cols, count, generator, device):
    """Bench-scale version of the same law on the device (torch, float32).

    One Haar pair (U, V) per shape, then for every matrix independent sigma,
    independent signed row/column permutations of U and V (which keep the
    columns orthonormal and Haar-distributed up to the shared draw), and
    independent noise.  Returns a bf16 tensor of shape (count, rows, cols).
    """
    import torch

    s = min(rows, cols)
    u, _ = torch.linalg.qr(torch.randn(rows, s, generator=generator, device=device))
    v, _ = torch.linalg.qr(torch.randn(cols, s, generator=generator, device=device))
    out = torch.empty(count, rows, cols, dtype=torch.bfloat16, device=device)
    lo, hi = math.log(SIGMA_LO), math.log(SIGMA_HI)
    for e in range(count):
        sigma = torch.exp(torch.rand(s, generator=generator, device=device) * (hi - lo) + lo)
        pr = torch.randperm(rows, generator=generator, device=device)
        pc = torch.randperm(cols, generator=generator, device=device)
        sr = torch.randint(0, 2, (rows, 1), generator=generator, device=device) * 2.0 - 1.0
        sc = torch.randint(0, 2, (cols, 1), generator=generator, device=device) * 2.0 - 1.0
        ue = (u[pr] * sr) * sigma
        ve = v[pc] * sc
        g = ue @ ve.T
        g += torch.randn(rows, cols, generator=generator, device=device) * NOISE_STD
        out[e].copy_(g)
    return out
