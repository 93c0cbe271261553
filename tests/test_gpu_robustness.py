"""GPU parity where the input is extreme or awkward: the scale of N (the step must
not depend on it: the Frobenius normalisation of the expanded Algorithm 1,
DeepSeek-V4 book ch. 6 section 5), non-finite gradients (IEEE propagation),
parameters and state at unaligned addresses, and V4's own gamma = 0.18 (the
deep-dive page's update-scale section).  Every call goes through the C ABI."""

import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import BF16_TOL, F32_TOL, assert_bitexact, rel_fro, say, to_dev, to_np

pytestmark = pytest.mark.gpu

LR, MU, WD, GAMMA = 0.02, 0.95, 0.1, 0.2


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    assert torch.cuda.is_available()
    return torch


@pytest.fixture(scope="module")
def ctx(torch_mod):
    import muon_step_amd as ms
    c = ms.Context(0)
    yield c
    torch_mod.cuda.synchronize()
    c.close()


def _ms():
    import muon_step_amd as ms
    return ms


def _prec(ms, precision):
    return ms.MUON_NS_BF16 if precision == "bf16" else ms.MUON_NS_F32


def _tol(precision):
    return BF16_TOL if precision == "bf16" else F32_TOL


# 2^-80 and 2^-40 put ||N||^2 far below the range in which the bf16 path folds
# 1/||N|| into its first products, 2^40 far above it, 2^-18 inside it near its
# lower end.
SCALES = (-80, -40, -18, 40)


@pytest.mark.parametrize("precision", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 520), (520, 300)])
def test_ns_only_scale_invariant(ctx, torch_mod, shape, precision):
    """NS(2^k N) against the oracle's NS(2^k N) (= NS(N) in exact arithmetic; the oracle
    pins that invariance) for N with the workloads' log-uniform spectrum."""
    ms = _ms()
    w = synth.Workload("t", 51, (synth.MatrixSpec(*shape),))
    inp = synth.matrix_inputs(w, 0)
    _, n = oracle.nesterov_momentum_f32(inp["m"], inp["g"], MU)
    hp = ms.make_hparams(ns_precision=_prec(ms, precision))
    x = torch_mod.empty(shape, dtype=torch_mod.float32, device="cuda")
    for k in SCALES:
        ns = (n.astype(np.float64) * 2.0 ** k).astype(np.float32)
        assert np.array_equal(ns.astype(np.float64), n.astype(np.float64) * 2.0 ** k)  # exact scaling
        ctx.muon_ns_only(to_dev(ns, torch_mod.float32), x, hp)
        torch_mod.cuda.synchronize()
        err = rel_fro(to_np(x), oracle.newton_schulz(ns))
        say(f"ns_only {shape} {precision} N x 2^{k}: rel err {err:.3e}")
        assert err <= _tol(precision)


def _step(ctx, torch_mod, ms, hosts, precision, coeffs=None, gamma=GAMMA):
    """One muon_step over matrices given as host dicts (w, g, m, dtypes); returns the
    device tensors (p, g, m, o) after the step and the norms."""
    dev, mats = [], []
    dt = {"bf16": torch_mod.bfloat16, "f32": torch_mod.float32}
    for h in hosts:
        p = to_dev(h["w"], dt[h["pd"]])
        g = to_dev(h["g"], dt[h["gd"]])
        m = to_dev(h["m"], torch_mod.float32)
        o = torch_mod.empty(h["w"].shape, dtype=torch_mod.float32, device="cuda")
        dev.append((p, g, m, o))
        mats.append(ms.matrix(p, g, m, o))
    ctx.muon_step(mats, ms.make_hparams(lr=LR, momentum=MU, weight_decay=WD, gamma=gamma, coeffs=coeffs,
                                        ns_precision=_prec(ms, precision)))
    torch_mod.cuda.synchronize()
    return dev, ctx.muon_last_norms(len(hosts))


def _scaled_hosts(shapes, seed, scales):
    hosts = []
    for i, ((rows, cols), k) in enumerate(zip(shapes, scales)):
        wl = synth.Workload("t", seed + i, (synth.MatrixSpec(rows, cols, prefill_momentum=True),))
        inp = synth.matrix_inputs(wl, 0)
        f = np.float32(2.0 ** k)
        # bf16 gradient and fp32 momentum times a power of two: exact (no subnormals)
        hosts.append({"w": inp["w"], "g": inp["g"] * f, "m": inp["m"] * f, "pd": "bf16", "gd": "bf16", "k": k})
    return hosts


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_step_scale_invariant(ctx, torch_mod, precision):
    """muon_step with gradient and momentum scaled by 2^k (one group of four same-shape
    matrices at four scales, and a transposed pair): momentum bit-exact, ||N||^2 to
    1e-12, O within the tolerance of the oracle, W bit-exact given the GPU's O'."""
    ms = _ms()
    shapes = [(256, 640)] * 4 + [(640, 256)] * 2
    hosts = _scaled_hosts(shapes, 61, list(SCALES) + [-80, 40])
    dev, norms = _step(ctx, torch_mod, ms, hosts, precision)
    for i, (h, (p, g, m, o)) in enumerate(zip(hosts, dev)):
        ref = oracle.muon_step(h["w"], h["g"], h["m"], lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA,
                               param_bf16=True)
        assert_bitexact(to_np(m), ref["m_new"], f"momentum of matrix {i}")
        nrm2 = float(np.sum(ref["n"].astype(np.float64) ** 2))
        assert abs(norms[i] - nrm2) <= 1e-12 * nrm2
        x = to_np(o)
        err = rel_fro(x * math.sqrt(max(h["w"].shape)) * GAMMA, ref["o"])
        say(f"step {h['w'].shape} {precision} scale 2^{h['k']} (||N||^2 = {nrm2:.3e}): O rel err {err:.3e}")
        assert err <= _tol(precision)
        assert_bitexact(to_np(p), oracle.apply_update_f32(h["w"], x, LR, WD, GAMMA, True), f"param {i}")


def test_step_scale_invariant_full_size_expert(ctx, torch_mod):
    """Two 2048x7168 experts of the MoE batch in one call, one with its gradient scaled by
    2^-40 (||N|| near 1e-12, an expert that saw no tokens for ~500 steps), both against
    the oracle."""
    ms = _ms()
    hosts = _scaled_hosts([(2048, 7168)] * 2, 71, [0, -40])
    for h in hosts:
        h["m"] = np.zeros_like(h["m"])
    dev, _ = _step(ctx, torch_mod, ms, hosts, "bf16")
    for i, (h, (p, g, m, o)) in enumerate(zip(hosts, dev)):
        say(f"full-size expert x 2^{h['k']}: oracle")
        ref = oracle.muon_step(h["w"], h["g"], h["m"], lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA,
                               param_bf16=True)
        assert_bitexact(to_np(m), ref["m_new"], f"momentum of expert {i}")
        x = to_np(o)
        err = rel_fro(x * math.sqrt(7168) * GAMMA, ref["o"])
        say(f"  O rel err {err:.3e}")
        assert err <= BF16_TOL
        assert_bitexact(to_np(p), oracle.apply_update_f32(h["w"], x, LR, WD, GAMMA, True), f"param {i}")


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_step_nonfinite_gradient_propagates(ctx, torch_mod, precision):
    """An Inf or a NaN in G makes ||N||^2 non-finite and, as in the exact algorithm
    (X = N / ||N|| is NaN where N is infinite, and the products spread it), every
    element of O' and of W NaN; the other matrices of the same group are untouched
    by it (against the oracle)."""
    ms = _ms()
    shapes = [(256, 640)] * 3 + [(640, 256)] * 2
    hosts = _scaled_hosts(shapes, 81, [0] * 5)
    hosts[0]["g"] = hosts[0]["g"].copy()
    hosts[0]["g"][3, 17] = np.inf
    hosts[2]["g"] = hosts[2]["g"].copy()
    hosts[2]["g"][100, 600] = np.nan
    hosts[3]["g"] = hosts[3]["g"].copy()
    hosts[3]["g"][500, 7] = -np.inf
    dev, norms = _step(ctx, torch_mod, ms, hosts, precision)
    for i, (h, (p, g, m, o)) in enumerate(zip(hosts, dev)):
        ref = oracle.muon_step(h["w"], h["g"], h["m"], lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA,
                               param_bf16=True)
        assert_bitexact(to_np(m), ref["m_new"], f"momentum of matrix {i}")
        x, w = to_np(o), to_np(p)
        if i in (0, 2, 3):
            assert np.all(np.isnan(ref["o"])), "oracle: a non-finite N gives an all-NaN O"
            assert not math.isfinite(norms[i])
            assert (norms[i] == math.inf) if i in (0, 3) else math.isnan(norms[i])
            assert np.all(np.isnan(x)), f"O' of matrix {i}: {int(np.sum(~np.isnan(x)))} non-NaN"
            assert np.all(np.isnan(w)), f"W of matrix {i}: {int(np.sum(~np.isnan(w)))} non-NaN"
            say(f"non-finite G, matrix {i} {precision}: O' and W all NaN, ||N||^2 = {norms[i]}")
        else:
            err = rel_fro(x * math.sqrt(640) * GAMMA, ref["o"])
            say(f"finite G, matrix {i} {precision}: O rel err {err:.3e}")
            assert err <= _tol(precision)
            assert_bitexact(w, oracle.apply_update_f32(h["w"], x, LR, WD, GAMMA, True), f"param {i}")


def _offset_view(torch_mod, a, dtype, offset):
    """A contiguous view of `a`'s values that starts `offset` elements into a larger
    allocation (so its address is not 16-byte aligned for offset % 4 != 0)."""
    n = a.size
    base = torch_mod.zeros(n + offset, dtype=dtype, device="cuda")
    v = base[offset:].view(a.shape)
    v.copy_(torch_mod.from_numpy(np.ascontiguousarray(a, np.float32)).to(dtype))
    return v


@pytest.mark.parametrize("param_dtype", ["bf16", "f32"])
def test_step_unaligned_views(ctx, torch_mod, param_dtype):
    """param, grad, momentum and ns_out at odd element offsets (unaligned for every
    vector access), on shapes whose last step takes the per-element fused update:
    momentum and W bit-exact against the oracle, O within tolerance; the same shapes
    again at aligned addresses in the same call."""
    ms = _ms()
    shapes = [(256, 512), (256, 512), (512, 256), (96, 300), (300, 96)]
    dt = {"bf16": torch_mod.bfloat16, "f32": torch_mod.float32}
    hosts, dev, mats = [], [], []
    for i, (rows, cols) in enumerate(shapes * 2):
        wl = synth.Workload("t", 91 + i, (synth.MatrixSpec(rows, cols, param_dtype, "bf16", prefill_momentum=True),))
        inp = synth.matrix_inputs(wl, 0)
        off = (1 + i % 3) if i < len(shapes) else 0
        p = _offset_view(torch_mod, inp["w"], dt[param_dtype], off)
        g = _offset_view(torch_mod, inp["g"], torch_mod.bfloat16, off + 2)
        m = _offset_view(torch_mod, inp["m"], torch_mod.float32, off + 1)
        o = _offset_view(torch_mod, np.zeros((rows, cols), np.float32), torch_mod.float32, off)
        hosts.append(inp)
        dev.append((p, g, m, o))
        mats.append(ms.matrix(p, g, m, o))
    ctx.muon_step(mats, ms.make_hparams(lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA))
    torch_mod.cuda.synchronize()
    for i, (h, (p, g, m, o)) in enumerate(zip(hosts, dev)):
        ref = oracle.muon_step(h["w"], h["g"], h["m"], lr=LR, momentum=MU, weight_decay=WD, gamma=GAMMA,
                               param_bf16=param_dtype == "bf16")
        assert_bitexact(to_np(m), ref["m_new"], f"momentum of matrix {i}")
        x = to_np(o)
        err = rel_fro(x * math.sqrt(max(h["w"].shape)) * GAMMA, ref["o"])
        say(f"{'unaligned' if i < len(shapes) else 'aligned'} {h['w'].shape} {param_dtype}: O rel err {err:.3e}")
        assert err <= BF16_TOL
        assert_bitexact(to_np(p), oracle.apply_update_f32(h["w"], x, LR, WD, GAMMA, param_dtype == "bf16"),
                        f"param of matrix {i}")


def test_step_gamma_v4(ctx, torch_mod):
    """DeepSeek-V4's own update scale gamma = 0.18 (the deep-dive page, update-scale
    section), hybrid schedule, both orientations and a ragged shape."""
    ms = _ms()
    shapes = [(256, 640), (640, 256), (200, 330)]
    hosts = _scaled_hosts(shapes, 101, [0, 0, 0])
    gamma = 0.18
    dev, _ = _step(ctx, torch_mod, ms, hosts, "bf16", gamma=gamma)
    for i, (h, (p, g, m, o)) in enumerate(zip(hosts, dev)):
        ref = oracle.muon_step(h["w"], h["g"], h["m"], lr=LR, momentum=MU, weight_decay=WD, gamma=gamma,
                               param_bf16=True)
        x = to_np(o)
        err = rel_fro(x * math.sqrt(max(h["w"].shape)) * gamma, ref["o"])
        say(f"gamma 0.18 {h['w'].shape}: O rel err {err:.3e}")
        assert err <= BF16_TOL
        assert_bitexact(to_np(p), oracle.apply_update_f32(h["w"], x, LR, WD, gamma, True), f"param {i}")
