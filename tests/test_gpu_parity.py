"""GPU parity of the HIP path against the oracle (sizes the oracle finishes in
seconds: several 256-wide tiles, ragged tails, transposed shapes, degenerate
cases).  Every call goes through the C ABI (libmuon_step.so via ctypes)."""

import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (BF16_TOL, F32_TOL, assert_bitexact, rel_fro, say, to_dev, to_np)

pytestmark = pytest.mark.gpu


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


def _spectral_n(rows, cols, seed, prefill=False):
    w = synth.Workload("t", seed, (synth.MatrixSpec(rows, cols, prefill_momentum=prefill),))
    inp = synth.matrix_inputs(w, 0)
    _, n = oracle.nesterov_momentum_f32(inp["m"], inp["g"], 0.95)
    return n


SHAPES = [(64, 128), (128, 64), (33, 65), (65, 33), (1, 7), (7, 1), (1, 1), (300, 520), (520, 300),
          (257, 513), (256, 256), (512, 1024), (700, 260)]


@pytest.mark.parametrize("precision", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES)
def test_ns_only_gaussian(ctx, torch_mod, shape, precision):
    ms = _ms()
    rows, cols = shape
    say(f"ns_only gaussian {shape} {precision}")
    n = np.random.default_rng(rows * 1000 + cols).standard_normal(shape).astype(np.float32)
    hp = ms.make_hparams(ns_precision=ms.MUON_NS_BF16 if precision == "bf16" else ms.MUON_NS_F32)
    x = torch_mod.empty(shape, dtype=torch_mod.float32, device="cuda")
    ctx.muon_ns_only(to_dev(n, torch_mod.float32), x, hp)
    torch_mod.cuda.synchronize()
    ref = oracle.newton_schulz(n)
    err = rel_fro(to_np(x), ref)
    say(f"  rel err {err:.3e}")
    assert err <= (BF16_TOL if precision == "bf16" else F32_TOL)


@pytest.mark.parametrize("precision", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(256, 896), (896, 256), (300, 1100), (128, 2048)])
def test_ns_only_spectral(ctx, torch_mod, shape, precision):
    """The configs' log-uniform [1e-4, 1e-1] spectrum, where the bf16 error budget is tightest."""
    ms = _ms()
    say(f"ns_only spectral {shape} {precision}")
    n = _spectral_n(*shape, seed=17)
    hp = ms.make_hparams(ns_precision=ms.MUON_NS_BF16 if precision == "bf16" else ms.MUON_NS_F32)
    x = torch_mod.empty(shape, dtype=torch_mod.float32, device="cuda")
    ctx.muon_ns_only(to_dev(n, torch_mod.float32), x, hp)
    torch_mod.cuda.synchronize()
    err = rel_fro(to_np(x), oracle.newton_schulz(n))
    say(f"  rel err {err:.3e}")
    assert err <= (BF16_TOL if precision == "bf16" else F32_TOL)


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_ns_only_zero_steps_is_normalisation(ctx, torch_mod, precision):
    """With an empty schedule the output is X_0 = N / ||N||_F.  The fp32 path keeps X
    in fp32 (error ~1e-7); the bf16 path keeps values as a bf16 hi plus an 8-bit
    residual that together hold the fp32 bit pattern rounded to its top 24 bits,
    within 0x80 units of the last place (2^-16 of the element).  N is stored so by
    the momentum pass and X = N / ||N|| again by the normalisation: at most 2^-15
    per element, and 2^-16 in Frobenius norm (the two roundings are independent)."""
    ms = _ms()
    n = np.random.default_rng(5).standard_normal((40, 90)).astype(np.float32)
    hp = ms.make_hparams(coeffs=[], ns_precision=ms.MUON_NS_BF16 if precision == "bf16" else ms.MUON_NS_F32)
    x = torch_mod.empty((40, 90), dtype=torch_mod.float32, device="cuda")
    ctx.muon_ns_only(to_dev(n, torch_mod.float32), x, hp)
    torch_mod.cuda.synchronize()
    ref = n.astype(np.float64) / np.linalg.norm(n.astype(np.float64))
    got = to_np(x)
    bound = 2.0 ** -16 if precision == "bf16" else 1e-6
    elem_bound = 2.0 ** -15 if precision == "bf16" else 1e-6
    assert rel_fro(got, ref) < bound
    assert np.all(np.abs(got - ref) <= 1.05 * elem_bound * np.abs(ref) + 1e-12)


def _run_step(ctx, torch_mod, specs, precision, seed, lr=0.02, wd=0.1, gamma=0.2, mu=0.95, nesterov=True,
              coeffs=None, zero_grad=False, scale_mode="sqrt_max"):
    """Runs muon_step on freshly generated matrices and checks every matrix against the oracle."""
    ms = _ms()
    wl = synth.Workload("t", seed, tuple(specs))
    dt = {"bf16": torch_mod.bfloat16, "f32": torch_mod.float32}
    host, dev, mats = [], [], []
    for i, sp in enumerate(specs):
        inp = synth.matrix_inputs(wl, i)
        if zero_grad:
            inp["g"] = np.zeros_like(inp["g"])
            inp["m"] = np.zeros_like(inp["m"])
        p = to_dev(inp["w"], dt[sp.param_dtype])
        g = to_dev(inp["g"], dt[sp.grad_dtype])
        m = to_dev(inp["m"], torch_mod.float32)
        o = torch_mod.empty((sp.rows, sp.cols), dtype=torch_mod.float32, device="cuda")
        host.append(inp)
        dev.append((p, g, m, o))
        mats.append(ms.matrix(p, g, m, o))
    hp = ms.make_hparams(lr=lr, momentum=mu, weight_decay=wd, gamma=gamma, nesterov=nesterov, coeffs=coeffs,
                         ns_precision=ms.MUON_NS_BF16 if precision == "bf16" else ms.MUON_NS_F32,
                         scale_mode=ms.MUON_SCALE_UNIT_RMS if scale_mode == "unit_rms" else ms.MUON_SCALE_SQRT_MAX)
    ctx.muon_step(mats, hp)
    torch_mod.cuda.synchronize()
    sched = tuple(tuple(c) for c in (coeffs if coeffs is not None else ms.schedule("deepseekv4")))
    tol = BF16_TOL if precision == "bf16" else F32_TOL
    norms = ctx.muon_last_norms(len(specs))
    for i, sp in enumerate(specs):
        inp = host[i]
        p, g, m, o = dev[i]
        m_ref, n_ref = oracle.nesterov_momentum_f32(inp["m"], inp["g"], mu, nesterov)
        assert_bitexact(to_np(m), m_ref, f"momentum of matrix {i} {sp.rows}x{sp.cols}")
        nrm2 = float(np.sum(n_ref.astype(np.float64) ** 2))
        assert abs(norms[i] - nrm2) <= 1e-12 * max(nrm2, 1e-300), (norms[i], nrm2)
        x_gpu = to_np(o)
        x_ref = oracle.newton_schulz(n_ref, sched)
        if zero_grad:
            assert not np.any(x_gpu)
        else:
            err = rel_fro(x_gpu * oracle.update_scale(x_gpu, gamma, scale_mode),
                          x_ref * oracle.update_scale(x_ref, gamma, scale_mode))
            say(f"  matrix {i} {sp.rows}x{sp.cols} p={sp.param_dtype} g={sp.grad_dtype}: O rel err {err:.3e}")
            assert err <= tol
        # unit-RMS mode: s from ||fl32 X||, summed in fp64 in another order on the device
        w_ref = oracle.apply_update_f32(inp["w"], x_gpu, lr, wd, gamma, sp.param_dtype == "bf16", scale_mode)
        assert_bitexact(to_np(p), w_ref, f"param of matrix {i}")
    return host, dev


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_step_mixed_group(ctx, torch_mod, precision):
    """Several shapes and dtype combinations in one call: grouped launches, ragged tiles,
    transposed matrices, bf16/fp32 params and grads; a shape and its transpose share one
    group (96 x 300 with 300 x 96, 256 x 512 with 512 x 256: one launch per product stage,
    momentum and update per orientation); the 512 x 768 bf16 pair, all of one
    orientation, stages W through LDS in the fused update."""
    S = synth.MatrixSpec
    specs = [S(96, 300, "bf16", "bf16"), S(96, 300, "bf16", "bf16"), S(300, 96, "bf16", "bf16"),
             S(260, 260, "f32", "f32", law="gauss"), S(64, 128, "f32", "bf16"), S(128, 64, "bf16", "f32"),
             S(96, 300, "bf16", "bf16", prefill_momentum=True), S(5, 3, "f32", "f32", law="gauss"),
             S(256, 512, "bf16", "bf16"), S(256, 512, "bf16", "bf16"), S(512, 256, "bf16", "bf16"),
             S(512, 768, "bf16", "bf16"), S(512, 768, "bf16", "bf16")]
    say(f"step mixed group {precision}")
    _run_step(ctx, torch_mod, specs, precision, seed=21)


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_step_unit_rms_mode(ctx, torch_mod, precision):
    """The unit-RMS scale mode (Megatron-Bridge recipe): the last step writes X, ||X|| is
    reduced per matrix, and the update runs as a separate pass with a per-matrix scale.
    Grouped, ragged and transposed shapes, both parameter dtypes, the gamma = 0.2 extra
    factor."""
    S = synth.MatrixSpec
    specs = [S(96, 300, "bf16", "bf16"), S(96, 300, "bf16", "bf16"), S(300, 96, "bf16", "bf16"),
             S(260, 260, "f32", "f32", law="gauss"), S(64, 128, "f32", "bf16"), S(5, 3, "f32", "f32", law="gauss"),
             S(256, 512, "bf16", "bf16"), S(512, 256, "bf16", "bf16"), S(1, 9, "f32", "f32")]
    say(f"step unit-RMS {precision}")
    _run_step(ctx, torch_mod, specs, precision, seed=27, scale_mode="unit_rms")


def test_step_unit_rms_degenerate(ctx, torch_mod):
    """Unit-RMS mode with the zero-step schedule (X = N / ||N||, so O = N * gamma / RMS(N))
    and with a zero gradient (X = 0: a zero scale, decay only)."""
    S = synth.MatrixSpec
    specs = [S(70, 130), S(130, 70, "f32", "f32"), S(40, 136), S(24, 64, "f32", "bf16"), S(200, 72),
             S(136, 40, "f32", "f32")]
    say("step unit-RMS zero schedule")
    _run_step(ctx, torch_mod, specs, "bf16", seed=28, coeffs=[], scale_mode="unit_rms")
    say("step zero schedule, bf16 workspace")
    _run_step(ctx, torch_mod, specs, "bf16", seed=30, coeffs=[])
    say("step unit-RMS zero gradient")
    _run_step(ctx, torch_mod, specs, "bf16", seed=29, zero_grad=True, scale_mode="unit_rms")


def test_step_single_f32_64x128_workload(ctx, torch_mod):
    """The single fp32 64x128 workload: N(0,1) gradient, zero momentum, both precisions."""
    wl = synth.WORKLOADS["single_f32_64x128"]
    for precision in ("bf16", "f32"):
        say(f"single_f32_64x128 {precision}")
        _run_step(ctx, torch_mod, list(wl.matrices), precision, seed=wl.base_seed)


def test_step_plain_momentum_and_quintic(ctx, torch_mod):
    ms = _ms()
    S = synth.MatrixSpec
    specs = [S(200, 330), S(330, 200)]
    say("step nesterov=0 quintic")
    _run_step(ctx, torch_mod, specs, "bf16", seed=23, nesterov=False, coeffs=ms.schedule("quintic"))
    say("step zero schedule")
    _run_step(ctx, torch_mod, specs, "f32", seed=24, coeffs=[])


def test_step_zero_gradient_is_decay_only(ctx, torch_mod):
    S = synth.MatrixSpec
    say("step zero gradient")
    _run_step(ctx, torch_mod, [S(70, 130), S(130, 70, "f32", "f32")], "bf16", seed=25, zero_grad=True)


def test_step_split_k_products(ctx, torch_mod):
    """Groups with few Gram / A^2 tiles and a long K split the products' K loop over
    several workgroups and sum the partial tiles in a fixed order: a (2048, 4096) group
    of both orientations (Gram in 3 ranges), a 128 x 4096 matrix (Gram in 8),
    a ragged 300 x 3000 one (Gram in 5), against the oracle; the whole call twice,
    bit for bit."""
    S = synth.MatrixSpec
    specs = [S(2048, 4096), S(4096, 2048), S(128, 4096), S(300, 3000)]
    say("step split-K products")
    _, dev1 = _run_step(ctx, torch_mod, specs, "bf16", seed=35)
    _, dev2 = _run_step(ctx, torch_mod, specs, "bf16", seed=35)
    for (p1, _, m1, o1), (p2, _, m2, o2) in zip(dev1, dev2):
        for a, b in ((p1, p2), (o1, o2)):
            assert np.array_equal(to_np(a).view(np.uint32), to_np(b).view(np.uint32))


def test_step_split_k_apply(ctx, torch_mod):
    """A single 4352^2 matrix: its a X + B X has 17 x 17 = 289 tiles, one wave of 256
    and 33 more, and those 33 run split over K (7 ranges of 640, their partials reduced
    in order before a X is added) in every step but the last; against the oracle, and
    the call repeated bit for bit."""
    S = synth.MatrixSpec
    specs = [S(4352, 4352)]
    say("step split-K apply (4352^2)")
    _, dev1 = _run_step(ctx, torch_mod, specs, "bf16", seed=41)
    _, dev2 = _run_step(ctx, torch_mod, specs, "bf16", seed=41)
    for (p1, _, m1, o1), (p2, _, m2, o2) in zip(dev1, dev2):
        for a, b in ((p1, p2), (o1, o2)):
            assert np.array_equal(to_np(a).view(np.uint32), to_np(b).view(np.uint32))


def test_step_split_k_apply_chunked(torch_mod):
    """Three 4352^2 matrices: the group's apply tiles past its last full wave (99 of
    867, all in the third matrix) split over K.  The step runs once in one chunk and
    once under a workspace cap that forces chunks of one matrix, where only the last
    chunk holds split tiles: the same bits either way (the split depends on the group,
    never on the chunking)."""
    import ctypes
    ms = _ms()
    rows = cols = 4352
    wl = synth.Workload("t", 43, tuple(synth.MatrixSpec(rows, cols) for _ in range(3)))
    inputs = [synth.matrix_inputs(wl, i) for i in range(3)]
    hp = ms.make_hparams()

    def tensors():
        dev, mats = [], []
        for inp in inputs:
            p = to_dev(inp["w"], torch_mod.bfloat16)
            g = to_dev(inp["g"], torch_mod.bfloat16)
            m = to_dev(inp["m"], torch_mod.float32)
            o = torch_mod.empty((rows, cols), dtype=torch_mod.float32, device="cuda")
            dev.append((p, g, m, o))
            mats.append(ms.matrix(p, g, m, o))
        return dev, mats

    dev, mats = tensors()
    need = ctypes.c_size_t()
    arr = (ms.muon_matrix * 3)(*mats)
    assert ms.load().muon_workspace_bytes(arr, 3, ctypes.byref(hp), ctypes.byref(need)) == ms.MUON_OK
    outs = []
    for cap in (0, int(need.value * 0.45)):
        say(f"3 x 4352^2, workspace cap {cap}")
        if cap:
            dev, mats = tensors()
        c = ms.Context(0, cap)
        try:
            c.muon_step(mats, hp)
            torch_mod.cuda.synchronize()
        finally:
            c.close()
        outs.append([(to_np(p), to_np(o), to_np(m)) for p, _, m, o in dev])
    for (p1, o1, m1), (p2, o2, m2) in zip(*outs):
        for a, b in ((p1, p2), (o1, o2), (m1, m2)):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_step_split_k_tail(ctx, torch_mod):
    """A group whose Gram tiles fill one wave of 256 workgroups and two tiles of a
    second (43 x 768x8192: 258 tiles) splits only those last two tiles over K (16
    ranges each, their partials reduced in order).  The first matrix (whole tiles only)
    and the last one (holding the split tiles) against the oracle; the call repeated
    bit for bit."""
    ms = _ms()
    rows, cols, count = 768, 8192, 43
    wl = synth.Workload("t", 36, tuple(synth.MatrixSpec(rows, cols) for _ in range(count)))
    hp = ms.make_hparams()
    results = []
    for rep in range(2):
        host, dev, mats = {}, [], []
        for i in range(count):
            inp = synth.matrix_inputs(wl, i)
            if i in (0, count - 1):
                host[i] = inp
            p = to_dev(inp["w"], torch_mod.bfloat16)
            g = to_dev(inp["g"], torch_mod.bfloat16)
            m = to_dev(inp["m"], torch_mod.float32)
            o = torch_mod.empty((rows, cols), dtype=torch_mod.float32, device="cuda")
            dev.append((p, g, m, o))
            mats.append(ms.matrix(p, g, m, o))
        ctx.muon_step(mats, hp)
        torch_mod.cuda.synchronize()
        results.append([(to_np(p), to_np(o)) for p, g, m, o in dev])
        if rep == 0:
            for i, inp in host.items():
                ref = oracle.muon_step(inp["w"], inp["g"], inp["m"], param_bf16=True)
                x = results[0][i][1]
                err = rel_fro(x * math.sqrt(cols) * 0.2, ref["o"])
                say(f"split-K tail: matrix {i} {rows}x{cols}: O rel err {err:.3e}")
                assert err <= BF16_TOL
                assert_bitexact(results[0][i][0], oracle.apply_update_f32(inp["w"], x, 0.02, 0.1, 0.2, True),
                                f"param of matrix {i}")
    for (p1, o1), (p2, o2) in zip(*results):
        assert np.array_equal(p1.view(np.uint32), p2.view(np.uint32))
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


def test_step_is_deterministic(ctx, torch_mod):
    ms = _ms()
    S = synth.MatrixSpec
    specs = [S(300, 700), S(700, 300), S(256, 2048), S(2048, 256)]
    wl = synth.Workload("t", 26, tuple(specs))
    outs = []
    for rep in range(2):
        tensors, mats = [], []
        for i, sp in enumerate(specs):
            inp = synth.matrix_inputs(wl, i)
            p = to_dev(inp["w"], torch_mod.bfloat16)
            g = to_dev(inp["g"], torch_mod.bfloat16)
            m = to_dev(inp["m"], torch_mod.float32)
            o = torch_mod.empty((sp.rows, sp.cols), dtype=torch_mod.float32, device="cuda")
            tensors.append((p, g, m, o))
            mats.append(ms.matrix(p, g, m, o))
        ctx.muon_step(mats, ms.make_hparams())
        torch_mod.cuda.synchronize()
        outs.append([to_np(t) for tt in tensors for t in (tt[0], tt[3])])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_concurrent_groups_match_sequential(torch_mod, precision):
    """Groups of different shapes run concurrently on side streams by default: two
    consecutive steps (no synchronisation between them) over six groups, among them
    (bf16 products) a split-K Gram / A^2 group and a split-K apply tail, both
    orientations and fp32 params, are bit-identical to the same two steps with every
    group in turn on the caller's stream; the per-matrix norms too."""
    ms = _ms()
    S = synth.MatrixSpec
    specs = [S(256, 4352), S(512, 768), S(768, 512), S(96, 300), S(300, 96), S(260, 260, "f32", "f32"),
             S(4352, 256), S(2304, 2304), S(512, 768, "f32", "bf16")]
    wl = synth.Workload("t", 29, tuple(specs))
    inputs = [synth.matrix_inputs(wl, i) for i in range(len(specs))]
    g2 = [synth.matrix_inputs(synth.Workload("t", 30, tuple(specs)), i)["g"] for i in range(len(specs))]
    dt = {"bf16": torch_mod.bfloat16, "f32": torch_mod.float32}
    results = []
    for concurrent in (True, False):
        c = ms.Context(0)
        try:
            c.muon_set_concurrent_groups(concurrent)
            tensors, first, second = [], [], []
            for i, sp in enumerate(specs):
                p = to_dev(inputs[i]["w"], dt[sp.param_dtype])
                ga, gb = to_dev(inputs[i]["g"], dt[sp.grad_dtype]), to_dev(g2[i], dt[sp.grad_dtype])
                m = to_dev(inputs[i]["m"], torch_mod.float32)
                o = torch_mod.empty((sp.rows, sp.cols), dtype=torch_mod.float32, device="cuda")
                tensors.append((p, m, o, ga, gb))
                first.append(ms.matrix(p, ga, m, o))
                second.append(ms.matrix(p, gb, m, o))
            say(f"  two steps over {len(specs)} matrices, {precision} products, concurrent groups {concurrent}")
            hp = ms.make_hparams(ns_precision=ms.MUON_NS_BF16 if precision == "bf16" else ms.MUON_NS_F32)
            c.muon_step(first, hp)
            c.muon_step(second, hp)
            torch_mod.cuda.synchronize()
            norms = c.muon_last_norms(len(specs))
            results.append(([to_np(t) for tt in tensors for t in tt[:3]], np.asarray(norms)))
        finally:
            c.close()
    (a, na), (b, nb) = results
    for i, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), f"tensor {i}"
    assert np.array_equal(na.view(np.uint64), nb.view(np.uint64))


def test_two_steps_equal_resume(ctx, torch_mod):
    """Step 2 from saved state equals two consecutive steps (all state is caller-owned)."""
    ms = _ms()
    S = synth.MatrixSpec
    sp = S(160, 400)
    wl = synth.Workload("t", 27, (sp,))
    inp = synth.matrix_inputs(wl, 0)
    g2 = synth.matrix_inputs(synth.Workload("t", 28, (sp,)), 0)["g"]
    hp = ms.make_hparams()

    def fresh():
        return (to_dev(inp["w"], torch_mod.bfloat16), to_dev(inp["m"], torch_mod.float32))

    p, m = fresh()
    ga, gb = to_dev(inp["g"], torch_mod.bfloat16), to_dev(g2, torch_mod.bfloat16)
    ctx.muon_step([ms.matrix(p, ga, m)], hp)
    ctx.muon_step([ms.matrix(p, gb, m)], hp)
    torch_mod.cuda.synchronize()
    p_direct, m_direct = to_np(p), to_np(m)
    p2, m2 = fresh()
    ctx.muon_step([ms.matrix(p2, ga, m2)], hp)
    torch_mod.cuda.synchronize()
    saved_p, saved_m = p2.clone().cpu(), m2.clone().cpu()
    p3, m3 = saved_p.cuda(), saved_m.cuda()
    ctx.muon_step([ms.matrix(p3, gb, m3)], hp)
    torch_mod.cuda.synchronize()
    assert np.array_equal(to_np(p3).view(np.uint32), p_direct.view(np.uint32))
    assert np.array_equal(to_np(m3).view(np.uint32), m_direct.view(np.uint32))


# ------------------------------------------------------------------ elementwise bit-exactness


@pytest.mark.parametrize("param_dtype", ["bf16", "f32"])
def test_apply_update_bitexact(ctx, torch_mod, param_dtype):
    ms = _ms()
    rows, cols = 333, 517
    r = np.random.default_rng(31)
    w = (r.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    x = r.standard_normal((rows, cols)).astype(np.float32)
    # special values: zeros of both signs, infinities, NaN, subnormals, huge
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-40, -3e-39, 3e38, -3e38, 1.0], np.float32)
    w.flat[:10] = specials
    x.flat[10:20] = specials
    if param_dtype == "bf16":
        w = oracle.bf16_round_f32(w)
    # bf16 rounding ties: d*w - s*x landing exactly half-way
    hp = ms.make_hparams(lr=0.5, weight_decay=0.5, gamma=0.25)   # d = 0.75, s = 0.5*0.25*sqrt(517)
    p = to_dev(w, torch_mod.bfloat16 if param_dtype == "bf16" else torch_mod.float32)
    ctx.muon_apply_update(p, to_dev(x, torch_mod.float32), hp)
    torch_mod.cuda.synchronize()
    ref = oracle.apply_update_f32(w, x, 0.5, 0.5, 0.25, param_dtype == "bf16")
    assert_bitexact(to_np(p), ref, "apply_update")


@pytest.mark.parametrize("param_dtype", ["bf16", "f32"])
def test_apply_update_unit_rms_bitexact(ctx, torch_mod, param_dtype):
    """The update hook in the unit-RMS mode: s = fl32(lr * gamma * sqrt(n m) / ||x||) with
    ||x||^2 reduced on the device; finite x with zeros, subnormals and a wide range; x = 0
    gives s = 0 (decay only)."""
    ms = _ms()
    rows, cols = 1100, 77
    r = np.random.default_rng(33)
    w = oracle.bf16_round_f32((r.standard_normal((rows, cols)) * 0.02).astype(np.float32))
    x = r.standard_normal((rows, cols)).astype(np.float32)
    x.flat[:6] = np.array([0.0, -0.0, 1e-40, -3e-39, 3e4, -1e-20], np.float32)
    hp = ms.make_hparams(lr=0.5, weight_decay=0.5, gamma=0.25, scale_mode=ms.MUON_SCALE_UNIT_RMS)
    pt = torch_mod.bfloat16 if param_dtype == "bf16" else torch_mod.float32
    for xx in (x, np.zeros_like(x)):
        p = to_dev(w, pt)
        ctx.muon_apply_update(p, to_dev(xx, torch_mod.float32), hp)
        torch_mod.cuda.synchronize()
        ref = oracle.apply_update_f32(w, xx, 0.5, 0.5, 0.25, param_dtype == "bf16", "unit_rms")
        assert_bitexact(to_np(p), ref, "apply_update unit-RMS")


def test_bf16_rounding_ties_bitexact(ctx, torch_mod):
    """fp32 results exactly half-way between bf16 neighbours, both parities, through the
    bf16 parameter store (d = 1, s = 1 so W' = W - X)."""
    ms = _ms()
    base = np.arange(0x3F800000, 0x3F800000 + 1024 * 0x10000, 0x10000, dtype=np.uint32)
    target = (base | np.uint32(0x8000)).view(np.float32)       # exact ties, both parities
    n = target.size                                           # 1024: sqrt(n) * (1/32) == 1
    w = np.zeros((1, n), np.float32)
    x = -target.reshape(1, n)
    hp = ms.make_hparams(lr=1.0, weight_decay=0.0, gamma=1.0 / 32.0)
    d, s = oracle.muon_scalars_f32(1.0, 0.0, 1.0 / 32.0, 1, n)
    assert d == 1.0 and s == 1.0
    p = to_dev(w, torch_mod.bfloat16)
    ctx.muon_apply_update(p, to_dev(x, torch_mod.float32), hp)
    torch_mod.cuda.synchronize()
    ref = oracle.apply_update_f32(w, x, 1.0, 0.0, 1.0 / 32.0, True)
    assert_bitexact(to_np(p), ref, "bf16 ties")


@pytest.mark.parametrize("step", [1, 2, 7])
def test_adamw_bitexact(ctx, torch_mod, step):
    ms = _ms()
    sizes = [1, 3, 1024, 1025, 4099, 70001]
    tensors, host, dev = [], [], []
    for k, n in enumerate(sizes):
        p, g, m, v = synth.adamw_inputs(n, seed=100 + k, step=step)
        if k == 2:
            g[:6] = np.array([0.0, -0.0, 1e-40, 3e30, -3e30, 1e-20], np.float32)
        tp, tg, tm, tv = (to_dev(a, torch_mod.float32) for a in (p, g, m, v))
        if k == 4:   # an unaligned view (scalar path)
            big = [torch_mod.zeros(n + 1, dtype=torch_mod.float32, device="cuda") for _ in range(4)]
            for b, src in zip(big, (tp, tg, tm, tv)):
                b[1:].copy_(src)
            tp, tg, tm, tv = (b[1:] for b in big)
        host.append((p, g, m, v))
        dev.append((tp, tg, tm, tv))
        tensors.append(ms.adamw_tensor(tp, tg, tm, tv))
    hp = ms.adamw_hparams(lr=0.02, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=step)
    ctx.muon_adamw_step(tensors, hp)
    torch_mod.cuda.synchronize()
    for (p, g, m, v), (tp, tg, tm, tv) in zip(host, dev):
        rp, rm, rv = oracle.adamw_step_f32(p, g, m, v, 0.02, 0.9, 0.95, 1e-8, 0.1, step)
        assert_bitexact(to_np(tp), rp, "adamw param")
        assert_bitexact(to_np(tm), rm, "adamw m")
        assert_bitexact(to_np(tv), rv, "adamw v")


def test_momentum_special_values_bitexact(ctx, torch_mod):
    """Nesterov bookkeeping on edge values (NaN propagates into O and W; checked for M only)."""
    ms = _ms()
    rows, cols = 8, 64
    r = np.random.default_rng(41)
    g = r.standard_normal((rows, cols)).astype(np.float32)
    m0 = r.standard_normal((rows, cols)).astype(np.float32)
    g[0, :8] = [0.0, -0.0, 1e-40, -1e-41, 3e38, -3e38, 1e-30, 5.0]
    m0[0, :8] = [-0.0, 0.0, 1e-40, 2e-41, 3e38, -3e38, -1e-30, -5.263158]
    p = to_dev(np.zeros((rows, cols), np.float32), torch_mod.float32)
    tg, tm = to_dev(g, torch_mod.float32), to_dev(m0, torch_mod.float32)
    ctx.muon_step([ms.matrix(p, tg, tm)], ms.make_hparams())
    torch_mod.cuda.synchronize()
    m_ref, _ = oracle.nesterov_momentum_f32(m0, g, 0.95)
    assert_bitexact(to_np(tm), m_ref, "momentum specials")


def test_stream_probe_moves_every_vector(ctx, torch_mod):
    """The HBM probe behind the elementwise ceilings reads every source vector and
    writes every destination vector: destination stream k holds the xor of the
    thread's source vectors plus k in its first word."""
    torch = torch_mod
    nvec, pitch = 3000, 3011
    for r, w in ((6, 7), (4, 3), (5, 2), (1, 1)):
        src = torch.randint(0, 2 ** 31 - 1, (r * pitch * 4,), dtype=torch.int32, device="cuda")
        dst = torch.zeros(w * pitch * 4, dtype=torch.int32, device="cuda")
        ctx.muon_stream_probe(src, dst, nvec * 16, r, w, pitch * 16)
        torch.cuda.synchronize()
        a = src.cpu().numpy().view(np.uint32).reshape(r, pitch, 4)[:, :nvec]
        x = np.bitwise_xor.reduce(a, axis=0)
        d = dst.cpu().numpy().view(np.uint32).reshape(w, pitch, 4)[:, :nvec]
        for k in range(w):
            want = x.copy()
            want[:, 0] = want[:, 0] + np.uint32(k)
            assert np.array_equal(d[k], want), (r, w, k)
