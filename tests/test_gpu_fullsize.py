"""GPU parity at the workloads' full sizes.

The 256 x 2048x7168 expert batch runs exactly as bench.py times it (one call
over all matrices, inputs from the same seeded device generator); sampled
experts are checked against the oracle one by one and every expert against
properties that hold at any size.  The dense-block, aspect-ratio and 16B-MoE
workloads run at their real shapes, every dense-block and aspect-ratio matrix
against the oracle, one 16B-MoE matrix per shape.  AdamW on the
102400x2048 tensors is compared bit for bit on sampled elements.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import BF16_TOL, assert_bitexact, rel_fro, say, scale_of, to_np

pytestmark = pytest.mark.gpu

LR, MU, WD, GAMMA = 0.02, 0.95, 0.1, 0.2


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    assert torch.cuda.is_available()
    return torch


def _ms():
    import muon_step_amd as ms
    return ms


def _ns_norm_band(torch, w0, w1, rows, cols):
    """||O'_t||_F / sqrt(min(n, m)) recovered from the update W1 = fl(d W0) - fl(s X).

    The ratio is the root-mean-square singular value of O'_t.  The two
    refining steps leave every singular value close to 1, so the ratio must
    sit inside [0.95, 1.05]; a matrix that was skipped, zeroed or mixed up
    with another lands far outside."""
    d, s = oracle.muon_scalars_f32(LR, WD, GAMMA, rows, cols)
    x = (float(d) * w0.float() - w1.float()) / float(s)
    return float(torch.linalg.vector_norm(x.double())) / math.sqrt(min(rows, cols))


def _check_sampled(mats_dev, idx, w0_host, g_host, m0_host, rows, cols):
    """Oracle step for one matrix; compares momentum, ||N||^2, O_t and W_t."""
    p, g, m, o = mats_dev
    ref = oracle.muon_step(w0_host, g_host, m0_host, lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA,
                           param_bf16=True)
    assert_bitexact(to_np(m), ref["m_new"], f"momentum of matrix {idx}")
    x_gpu = to_np(o)
    err = rel_fro(x_gpu * scale_of(rows, cols, GAMMA), ref["o"])
    say(f"  matrix {idx} {rows}x{cols}: O rel err {err:.3e}")
    assert err <= BF16_TOL
    w_ref = oracle.apply_update_f32(w0_host, x_gpu, LR, WD, GAMMA, True)
    assert_bitexact(to_np(p), w_ref, f"param of matrix {idx}")
    return ref


def test_moe_expert_batch_full_size(torch_mod):
    """256 x 2048x7168 bf16 in one call, as timed by bench.py; experts 0, 97, 160 and
    255 against the oracle, all 256 against the norm band."""
    torch = torch_mod
    ms = _ms()
    rows, cols, count = 2048, 7168, 256
    say("moe 256 x 2048x7168: generating inputs on the device")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    grads = synth.spectral_grad_torch(rows, cols, count, gen, "cuda")
    params = (torch.randn(count, rows, cols, generator=gen, device="cuda") * synth.gen.PARAM_STD).to(torch.bfloat16)
    moms = torch.zeros(count, rows, cols, dtype=torch.float32, device="cuda")
    w0 = params.clone()
    sampled = (0, 97, 160, 255)
    outs = {e: torch.empty(rows, cols, dtype=torch.float32, device="cuda") for e in sampled}
    mats = [ms.matrix(params[e], grads[e], moms[e], outs.get(e)) for e in range(count)]
    ctx = ms.Context(0)
    try:
        say("moe 256 x 2048x7168: one Muon step")
        ctx.muon_step(mats, ms.make_hparams(lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA))
        torch.cuda.synchronize()
        norms = ctx.muon_last_norms(count)
    finally:
        ctx.close()
    for e in sampled:
        say(f"moe expert {e}: oracle")
        g_host = to_np(grads[e])
        m0 = np.zeros((rows, cols), np.float32)
        ref = _check_sampled((params[e], grads[e], moms[e], outs[e]), e, to_np(w0[e]), g_host, m0, rows, cols)
        nrm2 = float(np.sum(ref["n"].astype(np.float64) ** 2))
        assert abs(norms[e] - nrm2) <= 1e-12 * nrm2
    bands = [_ns_norm_band(torch, w0[e], params[e], rows, cols) for e in range(count)]
    say(f"moe norm band over 256 experts: [{min(bands):.4f}, {max(bands):.4f}]")
    assert all(0.95 < b < 1.05 for b in bands)
    assert bool(torch.isfinite(params.float()).all())
    # every expert's momentum is exactly (1 + 0) * G: zero prior momentum
    assert bool((moms == grads.float()).all())


def test_moe_expert_batch_full_size_unit_rms(torch_mod):
    """The same batch in the unit-RMS scale mode (X written by the last step, ||X|| reduced
    per matrix, a separate update pass): expert 97 against the oracle, and every expert's
    applied update (d W0 - W1) / lr against RMS = gamma, which that mode fixes whatever the
    singular values are (bf16 rounding of W1 perturbs it by about 1e-4)."""
    torch = torch_mod
    ms = _ms()
    rows, cols, count = 2048, 7168, 256
    say("moe 256 x 2048x7168 unit-RMS: generating inputs on the device")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    grads = synth.spectral_grad_torch(rows, cols, count, gen, "cuda")
    params = (torch.randn(count, rows, cols, generator=gen, device="cuda") * synth.gen.PARAM_STD).to(torch.bfloat16)
    moms = torch.zeros(count, rows, cols, dtype=torch.float32, device="cuda")
    w0 = params.clone()
    e = 97
    out = torch.empty(rows, cols, dtype=torch.float32, device="cuda")
    mats = [ms.matrix(params[i], grads[i], moms[i], out if i == e else None) for i in range(count)]
    ctx = ms.Context(0)
    try:
        say("moe 256 x 2048x7168 unit-RMS: one Muon step")
        ctx.muon_step(mats, ms.make_hparams(lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA,
                                            scale_mode=ms.MUON_SCALE_UNIT_RMS))
        torch.cuda.synchronize()
    finally:
        ctx.close()
    say(f"moe expert {e} unit-RMS: oracle")
    w0_host = to_np(w0[e])
    ref = oracle.muon_step(w0_host, to_np(grads[e]), np.zeros((rows, cols), np.float32), lr=LR, momentum=MU,
                           weight_decay=WD, gamma=GAMMA, param_bf16=True, scale_mode="unit_rms")
    x_gpu = to_np(out)
    err = rel_fro(x_gpu * oracle.update_scale(x_gpu, GAMMA, "unit_rms"), ref["o"])
    say(f"  matrix {e} {rows}x{cols}: O rel err {err:.3e}")
    assert err <= BF16_TOL
    w_ref = oracle.apply_update_f32(w0_host, x_gpu, LR, WD, GAMMA, True, "unit_rms")
    assert_bitexact(to_np(params[e]), w_ref, f"param of matrix {e}")
    d = float(np.float32(1.0 - LR * WD))
    rms = [float(torch.linalg.vector_norm(((d * w0[i].double() - params[i].double()) / LR))) /
           math.sqrt(rows * cols) / GAMMA for i in range(count)]
    say(f"moe unit-RMS: RMS(O)/gamma over 256 experts in [{min(rms):.5f}, {max(rms):.5f}]")
    assert all(abs(r - 1.0) < 1e-3 for r in rms)


def _run_workload(torch, specs, seed, cap_bytes=0):
    """One muon_step call over a workload's matrices (device-generated spectral grads,
    params N(0, 0.02), momentum pre-filled with a prior-step gradient where the spec
    says so).  Returns, per matrix name, host copies of W0, G, M0, M, W and O' (every
    matrix's ns_out requested)."""
    ms = _ms()
    by_shape = {}
    for i, sp in enumerate(specs):
        by_shape.setdefault((sp.rows, sp.cols), []).append(i)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    grads, prior = [None] * len(specs), [None] * len(specs)
    for (rows, cols), ids in by_shape.items():
        g = synth.spectral_grad_torch(rows, cols, len(ids), gen, "cuda")
        pf = [i for i in ids if specs[i].prefill_momentum]
        gp = synth.spectral_grad_torch(rows, cols, len(pf), gen, "cuda") if pf else None
        for k, i in enumerate(ids):
            grads[i] = g[k]
        for k, i in enumerate(pf):
            prior[i] = gp[k]
    params, moms, outs, w0, m0 = [], [], [], [], []
    for i, sp in enumerate(specs):
        p = (torch.randn(sp.rows, sp.cols, generator=gen, device="cuda") * synth.gen.PARAM_STD).to(torch.bfloat16)
        m = prior[i].float() if prior[i] is not None else torch.zeros(sp.rows, sp.cols, device="cuda")
        params.append(p)
        w0.append(to_np(p))
        m0.append(to_np(m))
        moms.append(m)
        outs.append(torch.empty(sp.rows, sp.cols, dtype=torch.float32, device="cuda"))
    mats = [ms.matrix(params[i], grads[i], moms[i], outs[i]) for i in range(len(specs))]
    ctx = ms.Context(0, cap_bytes)
    try:
        ctx.muon_step(mats, ms.make_hparams(lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA))
        torch.cuda.synchronize()
    finally:
        ctx.close()
    res = {}
    for i, sp in enumerate(specs):
        res[sp.name] = {"w0": w0[i], "g": to_np(grads[i]), "m0": m0[i], "m": to_np(moms[i]), "w": to_np(params[i]),
                        "o": to_np(outs[i]), "rows": sp.rows, "cols": sp.cols}
    del grads, prior, params, moms, outs, mats
    torch.cuda.empty_cache()
    return res


def _check_against_oracle(r, name):
    """Momentum bit-exact, O within the bf16 tolerance of the oracle, W bit-exact given
    the GPU's O', and the RMS singular value of O' inside [0.95, 1.05]."""
    rows, cols = r["rows"], r["cols"]
    ref = oracle.muon_step(r["w0"], r["g"], r["m0"], lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA,
                           param_bf16=True)
    assert_bitexact(r["m"], ref["m_new"], f"momentum of {name}")
    err = rel_fro(r["o"] * scale_of(rows, cols, GAMMA), ref["o"])
    band = float(np.linalg.norm(r["o"].astype(np.float64))) / math.sqrt(min(rows, cols))
    say(f"  {name} {rows}x{cols}: O rel err {err:.3e}, RMS singular value {band:.4f}")
    assert err <= BF16_TOL
    assert 0.95 < band < 1.05
    w_ref = oracle.apply_update_f32(r["w0"], r["o"], LR, WD, GAMMA, True)
    assert_bitexact(r["w"], w_ref, f"param of {name}")


@pytest.fixture(scope="module")
def aspect_run(torch_mod):
    wl = synth.WORKLOADS["aspect_stress_bf16"]
    say("aspect-ratio set: one call over its four matrices")
    return _run_workload(torch_mod, list(wl.matrices), wl.base_seed)


@pytest.fixture(scope="module")
def dense_run(torch_mod):
    wl = synth.WORKLOADS["dense_block_bf16"]
    say("dense block: one call over its seven matrices")
    return _run_workload(torch_mod, list(wl.matrices), wl.base_seed)


@pytest.mark.parametrize("name", [sp.name for sp in synth.WORKLOADS["aspect_stress_bf16"].matrices])
def test_aspect_ratio_set_full_size(aspect_run, name):
    """1024x16384, 16384x1024, 7168^2 and 512x32768 (momentum pre-filled), run in one
    call; each matrix against the oracle."""
    _check_against_oracle(aspect_run[name], name)


@pytest.mark.parametrize("name", [sp.name for sp in synth.WORKLOADS["dense_block_bf16"].matrices])
def test_dense_block_full_size(dense_run, name):
    """Four 4096^2, two 4096x14336 and one 14336x4096, run in one call; each matrix
    against the oracle."""
    _check_against_oracle(dense_run[name], name)


def test_moe16b_full_step(torch_mod):
    """The full 16B-MoE optimizer step in two calls: Muon over all 27 x (4 + 192)
    matrices (workspace capped at 24 GiB, so each shape group runs in chunks) and
    AdamW over the 102400x2048 embedding and head.  Against the oracle: layers 0
    and 26 (their four attention matrices and experts 0 and 63, up, gate and
    down) and the middle matrix of each shape; 96 spread over the list against
    the norm band; AdamW bit-exact on 8192 sampled elements of each tensor
    (first, last and random positions)."""
    torch = torch_mod
    ms = _ms()
    wl = synth.WORKLOADS["moe16b_full_step"]
    specs = list(wl.matrices)
    say(f"16B-MoE step: {len(specs)} Muon matrices, generating inputs on the device")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.base_seed)
    by_shape = {}
    for i, sp in enumerate(specs):
        by_shape.setdefault((sp.rows, sp.cols), []).append(i)
    grads = [None] * len(specs)
    for (rows, cols), ids in by_shape.items():
        g = synth.spectral_grad_torch(rows, cols, len(ids), gen, "cuda")
        for k, i in enumerate(ids):
            grads[i] = g[k]
    params = [(torch.randn(sp.rows, sp.cols, generator=gen, device="cuda") * synth.gen.PARAM_STD).to(torch.bfloat16)
              for sp in specs]
    moms = [torch.zeros(sp.rows, sp.cols, device="cuda") for sp in specs]
    per_layer = 4 + 3 * 64
    checked = {ids[len(ids) // 2] for ids in by_shape.values()}
    for layer in (0, 26):
        base = layer * per_layer
        checked |= set(range(base, base + 4))                              # attention
        checked |= {base + 4 + 3 * e + k for e in (0, 63) for k in range(3)}  # experts 0, 63
    assert len(specs) == 27 * per_layer and specs[26 * per_layer + 4 + 3 * 63 + 2].name == "l26.e63.down"
    banded = set(range(0, len(specs), len(specs) // 96)) | checked
    w0 = {i: params[i].clone() for i in banded}
    outs = {i: torch.empty(specs[i].rows, specs[i].cols, device="cuda") for i in checked}
    mats = [ms.matrix(params[i], grads[i], moms[i], outs.get(i)) for i in range(len(specs))]
    numel = 102400 * 2048
    ad = []
    for name, n in wl.adamw:
        assert n == numel
        p = torch.randn(n, generator=gen, device="cuda") * synth.gen.PARAM_STD
        g = torch.randn(n, generator=gen, device="cuda")
        ad.append((name, p, g, torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")))
    rs = np.random.default_rng(wl.base_seed)
    pick = np.unique(np.concatenate([np.arange(2048), np.arange(numel - 2048, numel),
                                     rs.integers(0, numel, 4096)]))
    pick_t = torch.from_numpy(pick).cuda()
    ad_before = [(name, to_np(p[pick_t]), to_np(g[pick_t])) for name, p, g, _, _ in ad]
    ahp = ms.adamw_hparams(lr=LR, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=WD, step=1)
    ctx = ms.Context(0, 24 << 30)
    try:
        say("16B-MoE step: Muon over every matrix, then AdamW")
        ctx.muon_step(mats, ms.make_hparams(lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA))
        ctx.muon_adamw_step([ms.adamw_tensor(p, g, m, v) for _, p, g, m, v in ad], ahp)
        torch.cuda.synchronize()
    finally:
        ctx.close()
    say(f"16B-MoE step: {len(checked)} matrices against the oracle")
    for i in sorted(checked):
        sp = specs[i]
        _check_sampled((params[i], grads[i], moms[i], outs[i]), sp.name, to_np(w0[i]), to_np(grads[i]),
                       np.zeros((sp.rows, sp.cols), np.float32), sp.rows, sp.cols)
    bands = [_ns_norm_band(torch, w0[i], params[i], specs[i].rows, specs[i].cols) for i in sorted(banded)]
    say(f"16B-MoE norm band over {len(bands)} matrices: [{min(bands):.4f}, {max(bands):.4f}]")
    assert all(0.95 < b < 1.05 for b in bands)
    for (name, p0, g0), (_, p, _, m, v) in zip(ad_before, ad):
        z = np.zeros_like(p0)
        p_ref, m_ref, v_ref = oracle.adamw_step_f32(p0, g0, z, z, LR, 0.9, 0.95, 1e-8, WD, 1)
        assert_bitexact(to_np(p[pick_t]), p_ref, f"AdamW {name} param")
        assert_bitexact(to_np(m[pick_t]), m_ref, f"AdamW {name} exp_avg")
        assert_bitexact(to_np(v[pick_t]), v_ref, f"AdamW {name} exp_avg_sq")
        say(f"  AdamW {name}: {len(pick)} sampled elements bit-exact")
