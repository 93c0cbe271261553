"""The allocation-free step muon_step_noalloc (for callers that cannot allocate
device memory) against muon_step on the same inputs, through the C ABI: calls
in a row, the second with a smaller input, every output bit for bit (both
entry points run the same kernels on every matrix; only the chunking of a
group differs, and no result depends on it, split-K tiles included); then a
call that cannot fit the fixed scratch, which must be refused before anything
is enqueued."""

import numpy as np
import pytest

import synth
from gpu_util import say, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    assert torch.cuda.is_available()
    return torch


def _hosts(specs, seed):
    wl = synth.Workload("noalloc", seed, tuple(specs))
    return [synth.matrix_inputs(wl, i) for i in range(len(specs))]


def _run(torch, ms, ctx, entry, hosts, hp):
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}
    dev, mats = [], []
    for h in hosts:
        sp = h["spec"]
        p = to_dev(h["w"], dt[sp.param_dtype])
        g = to_dev(h["g"], dt[sp.grad_dtype])
        m = to_dev(h["m"], torch.float32)
        o = torch.empty(sp.rows, sp.cols, dtype=torch.float32, device="cuda")
        dev.append((p, g, m, o))
        mats.append(ms.matrix(p, g, m, o))
    getattr(ctx, entry)(mats, hp)
    torch.cuda.synchronize()
    norms = ctx.muon_last_norms(len(hosts))
    return [tuple(to_np(t) for t in (p, m, o)) for p, g, m, o in dev], norms


def _same(a, b, what):
    assert a.shape == b.shape, what
    same = (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
    assert bool(same.all()), f"{what}: {int((~same).sum())} elements differ"


def test_noalloc_matches_muon_step(torch_mod):
    import muon_step_amd as ms
    S = synth.MatrixSpec
    first = [S(1024, 2048), S(1024, 2048), S(1024, 2048), S(2048, 1024), S(2048, 1024), S(300, 520, "f32", "bf16"),
             S(520, 300, prefill_momentum=True), S(2048, 7168), S(5, 3, "f32", "f32", law="gauss")]
    second = [S(300, 520), S(64, 128, "f32", "f32", law="gauss")]
    # 43 x 768x8192: the group's last two Gram tiles run split over K; in the fixed
    # scratch the group runs in chunks of three matrices, whose last chunk holds them
    tail = [S(768, 8192)] * 43
    # 21 x 1792x1792: the last five a X + B X tiles run split over K, three
    # ranges each; they lie in the last matrix, which the fixed scratch runs
    # as a chunk of its own
    apply_tail = [S(1792, 1792)] * 21
    ctx = ms.Context(0)
    try:
        for k, (specs, seed, prec) in enumerate(((first, 201, ms.MUON_NS_BF16), (second, 202, ms.MUON_NS_BF16),
                                                 (second, 203, ms.MUON_NS_F32), (tail, 205, ms.MUON_NS_BF16),
                                                 (apply_tail, 206, ms.MUON_NS_BF16))):
            hosts = _hosts(specs, seed)
            hp = ms.make_hparams(ns_precision=prec)
            say(f"call {k + 1}: {len(specs)} matrices, muon_step_noalloc then muon_step")
            got, n_got = _run(torch_mod, ms, ctx, "muon_step_noalloc", hosts, hp)
            ref, n_ref = _run(torch_mod, ms, ctx, "muon_step", hosts, hp)
            for i, (sp, a, b) in enumerate(zip(specs, got, ref)):
                for name, x, y in zip(("param", "momentum", "ns_out"), a, b):
                    _same(x, y, f"call {k + 1} matrix {i} {sp.rows}x{sp.cols} {name}")
            assert n_got == n_ref
            say(f"call {k + 1}: identical")
        # a 4096 x 4096 bf16 matrix needs 151 MB of workspace: refused, nothing enqueued
        h = _hosts([S(4096, 4096)], 204)[0]
        p = to_dev(h["w"], torch_mod.bfloat16)
        g = to_dev(h["g"], torch_mod.bfloat16)
        m = to_dev(h["m"], torch_mod.float32)
        p0 = to_np(p)
        with pytest.raises(ms.MuonError) as ei:
            ctx.muon_step_noalloc([ms.matrix(p, g, m)], ms.make_hparams())
        assert ei.value.status == ms.MUON_ERR_OUT_OF_MEMORY
        assert "fixed scratch" in str(ei.value)
        torch_mod.cuda.synchronize()
        _same(to_np(p), p0, "param of the refused call")
        assert not bool(m.any())
        say(f"oversize call refused: {ei.value}")
    finally:
        torch_mod.cuda.synchronize()
        ctx.close()
