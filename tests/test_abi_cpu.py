"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, its struct layouts match the header (compiled with gcc), and
host-side validation returns the documented status without touching a device."""

import ctypes
import math
import os
import re
import subprocess
import tempfile

import pytest

import muon_step_amd as ms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_step.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ms.LIB_PATH):
        pytest.fail("libmuon_step.so is not built (run __graft_entry__.build())")
    return ms.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(muon_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(lib):
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert sorted(ms.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ms.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(muon_\w+)", out))
    assert set(declared) <= exported


def test_abi_version(lib):
    m = re.search(r"#define MUON_STEP_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.muon_abi_version() == int(m.group(1))


def test_struct_layouts_match_header():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "muon_step.h"
#define F(T, f) printf(#T "." #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("muon_matrix %zu\n", sizeof(muon_matrix));
  printf("muon_hparams %zu\n", sizeof(muon_hparams));
  printf("muon_adamw_tensor %zu\n", sizeof(muon_adamw_tensor));
  printf("muon_adamw_hparams %zu\n", sizeof(muon_adamw_hparams));
  printf("muon_ns_coeff %zu\n", sizeof(muon_ns_coeff));
  F(muon_matrix, rows) F(muon_matrix, param_dtype) F(muon_matrix, grad_dtype) F(muon_matrix, ns_out)
  F(muon_hparams, schedule) F(muon_hparams, num_ns_steps) F(muon_hparams, ns_precision)
  F(muon_hparams, scale_mode) F(muon_adamw_tensor, numel) F(muon_adamw_tensor, grad_dtype)
  F(muon_adamw_hparams, step)
  printf("muon_stage_stats %zu\n", sizeof(muon_stage_stats));
  F(muon_stage_stats, launches) F(muon_stage_stats, total_ms) F(muon_stage_stats, bytes)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), c,
                        "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(line.rsplit(" ", 1) for line in lines if line)
    py = {
        "muon_matrix": ctypes.sizeof(ms.muon_matrix), "muon_hparams": ctypes.sizeof(ms.muon_hparams),
        "muon_adamw_tensor": ctypes.sizeof(ms.muon_adamw_tensor),
        "muon_adamw_hparams": ctypes.sizeof(ms.muon_adamw_hparams),
        "muon_ns_coeff": ctypes.sizeof(ms.muon_ns_coeff),
        "muon_stage_stats": ctypes.sizeof(ms.muon_stage_stats),
    }
    for k, v in py.items():
        assert int(got[k]) == v, k
    for key, val in got.items():
        if "." in key:
            struct, field = key.split(".")
            assert getattr(getattr(ms, struct), field).offset == int(val), key


def test_schedules(lib):
    assert ms.schedule("deepseekv4") == [(3.4445, -4.775, 2.0315)] * 8 + [(2.0, -1.5, 0.5)] * 2
    assert ms.schedule("quintic") == [(3.4445, -4.775, 2.0315)] * 5
    assert lib.muon_schedule(b"nope", None, 0) == -1
    assert lib.muon_schedule(None, None, 0) == -1


def test_status_strings(lib):
    for s in range(5):
        assert lib.muon_status_string(s)
    assert lib.muon_status_string(99) == b"unknown status"


# ------------------------------------------------------------------ host validation

BASE = 1 << 40   # fake device addresses: validation never dereferences them


def _mat(i, rows=64, cols=128, pd=ms.MUON_BF16, gd=ms.MUON_BF16, ns_out=False):
    off = BASE + i * (1 << 32)
    return ms.muon_matrix(off, off + (1 << 30), off + (2 << 30), off + (3 << 30) if ns_out else None,
                          rows, cols, pd, gd)


def _check(lib, mats, hp):
    arr = (ms.muon_matrix * max(1, len(mats)))(*mats)
    buf = ctypes.create_string_buffer(512)
    st = lib.muon_check_step_args(arr if mats else None, len(mats), ctypes.byref(hp) if hp else None,
                                  buf, 512)
    return st, buf.value.decode()


def test_valid_step_args(lib):
    hp = ms.make_hparams()
    assert _check(lib, [_mat(0), _mat(1, 7168, 2048, ns_out=True)], hp) == (ms.MUON_OK, "")
    hp_rms = ms.make_hparams(scale_mode=ms.MUON_SCALE_UNIT_RMS)
    assert _check(lib, [_mat(0), _mat(1, 7168, 2048, ns_out=True)], hp_rms) == (ms.MUON_OK, "")
    assert _check(lib, [], hp)[0] == ms.MUON_OK


@pytest.mark.parametrize("case", [
    "null_param", "null_grad", "null_mom", "rows0", "cols_neg", "dtype", "steps_neg", "steps_big",
    "sched_null", "lr_nan", "gamma_inf", "nesterov2", "precision", "scale_mode", "coeff_nan",
    "grad_aliases_param", "mom_aliases_param", "two_mats_share_param", "ns_out_aliases_grad",
    "null_hparams",
])
def test_invalid_step_args(lib, case):
    hp = ms.make_hparams()
    mats = [_mat(0), _mat(1)]
    m = mats[0]
    if case == "null_param": m.param = None
    elif case == "null_grad": m.grad = None
    elif case == "null_mom": m.momentum = None
    elif case == "rows0": m.rows = 0
    elif case == "cols_neg": m.cols = -3
    elif case == "dtype": m.grad_dtype = 7
    elif case == "steps_neg": hp.num_ns_steps = -1
    elif case == "steps_big": hp.num_ns_steps = 65
    elif case == "sched_null": hp.schedule = None
    elif case == "lr_nan": hp.lr = math.nan
    elif case == "gamma_inf": hp.gamma = math.inf
    elif case == "nesterov2": hp.nesterov = 2
    elif case == "precision": hp.ns_precision = 5
    elif case == "scale_mode": hp.scale_mode = 2
    elif case == "coeff_nan": hp._keep[3].b = math.nan
    elif case == "grad_aliases_param": m.grad = m.param + 16
    elif case == "mom_aliases_param": m.momentum = m.param + 64 * 128 * 2 - 4
    elif case == "two_mats_share_param": mats[1].param = m.param
    elif case == "ns_out_aliases_grad": m.ns_out = m.grad
    st, msg = _check(lib, mats, None if case == "null_hparams" else hp)
    assert st == ms.MUON_ERR_INVALID_ARGUMENT
    assert msg


def test_adjacent_buffers_are_not_aliasing(lib):
    hp = ms.make_hparams()
    m = _mat(0)
    m.grad = m.param + 64 * 128 * 2          # starts right where param ends
    assert _check(lib, [m], hp)[0] == ms.MUON_OK


def test_shared_grad_between_matrices_is_allowed(lib):
    hp = ms.make_hparams()
    a, b = _mat(0), _mat(1)
    b.grad = a.grad                          # read-only memory may be shared
    assert _check(lib, [a, b], hp)[0] == ms.MUON_OK


def _adamw(lib, ts, hp):
    arr = (ms.muon_adamw_tensor * max(1, len(ts)))(*ts)
    buf = ctypes.create_string_buffer(512)
    return lib.muon_check_adamw_args(arr, len(ts), ctypes.byref(hp) if hp else None, buf, 512)


def _t(i, n=1000):
    off = BASE + i * (1 << 34)
    return ms.muon_adamw_tensor(off, off + (1 << 32), off + (2 << 32), off + (3 << 32), n,
                                ms.MUON_F32, ms.MUON_F32)


def test_adamw_validation(lib):
    hp = ms.adamw_hparams()
    assert _adamw(lib, [_t(0), _t(1)], hp) == ms.MUON_OK
    assert _adamw(lib, [_t(0, 0)], hp) == ms.MUON_OK
    t = _t(0); t.param_dtype = ms.MUON_BF16
    assert _adamw(lib, [t], hp) == ms.MUON_ERR_UNSUPPORTED
    t = _t(0); t.grad = t.exp_avg
    assert _adamw(lib, [t], hp) == ms.MUON_ERR_INVALID_ARGUMENT
    t = _t(0); t.numel = -1
    assert _adamw(lib, [t], hp) == ms.MUON_ERR_INVALID_ARGUMENT
    assert _adamw(lib, [_t(0)], ms.adamw_hparams(step=0)) == ms.MUON_ERR_INVALID_ARGUMENT
    assert _adamw(lib, [_t(0)], ms.adamw_hparams(eps=math.nan)) == ms.MUON_ERR_INVALID_ARGUMENT
    assert _adamw(lib, [_t(0)], None) == ms.MUON_ERR_INVALID_ARGUMENT


def test_workspace_bytes_moe_batch(lib):
    hp = ms.make_hparams()
    mats = [_mat(i, 2048, 7168) for i in range(256)]
    arr = (ms.muon_matrix * 256)(*mats)
    out = ctypes.c_size_t()
    assert lib.muon_workspace_bytes(arr, 256, ctypes.byref(hp), ctypes.byref(out)) == ms.MUON_OK
    x, a = 2048 * 7168, 2048 * 2048
    # bf16 path: X as hi (two ping-pong bf16 copies) + its 8-bit residual lo; A bf16; B bf16
    ns = 256 * (x * (2 + 2 + 1) + a * (2 + 2))
    assert ns <= out.value <= ns + 64 * 1024 * 1024


def test_workspace_bytes_concurrent_groups(lib):
    """Groups of different shapes run on concurrent lanes, each lane in its own workspace
    slice: a call of two groups needs about the sum of what each needs alone."""
    hp = ms.make_hparams()

    def need(shapes):
        arr = (ms.muon_matrix * len(shapes))(*[_mat(i, r, c) for i, (r, c) in enumerate(shapes)])
        out = ctypes.c_size_t()
        assert lib.muon_workspace_bytes(arr, len(shapes), ctypes.byref(hp), ctypes.byref(out)) == ms.MUON_OK
        return out.value

    a, b = [(1024, 4096)] * 3, [(512, 2048), (2048, 512)]
    both, one, two = need(a + b), need(a), need(b)
    assert max(one, two) < both
    assert abs(both - (one + two)) <= 4 * 1024 * 1024


def test_workspace_bytes_large_groups_in_turn(lib):
    """Groups whose apply launch fills the chip 8 times or more run in turn in one
    workspace slice: two such groups need about what the larger one needs alone."""
    hp = ms.make_hparams()

    def need(shapes):
        arr = (ms.muon_matrix * len(shapes))(*[_mat(i, r, c) for i, (r, c) in enumerate(shapes)])
        out = ctypes.c_size_t()
        assert lib.muon_workspace_bytes(arr, len(shapes), ctypes.byref(hp), ctypes.byref(out)) == ms.MUON_OK
        return out.value

    a, b = [(2048, 7168)] * 16, [(1024, 4096)] * 40   # 3584 and 2560 apply tiles
    both, one, two = need(a + b), need(a), need(b)
    assert abs(both - max(one, two)) <= 4 * 1024 * 1024


def test_set_concurrent_groups_validates(lib):
    assert lib.muon_set_concurrent_groups(None, 1) == ms.MUON_ERR_INVALID_ARGUMENT


def test_create_without_gpu_reports_device_error(lib):
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is visible")
    except ImportError:
        pass
    h = ctypes.c_void_p()
    assert lib.muon_create(ctypes.byref(h), 0, 0) == ms.MUON_ERR_DEVICE
    assert not h.value
    assert lib.muon_destroy(None) == ms.MUON_OK


# ------------------------------------------------------------- binding argument checks


def test_binding_rejects_wrong_dtypes_before_any_launch():
    """The C ABI has no dtype field for momentum, ns_out, exp_avg or exp_avg_sq: a
    tensor of another dtype must be refused by the binding (a bf16 buffer would be
    read and written over twice its allocation)."""
    import torch
    p = torch.zeros(4, 8, dtype=torch.bfloat16)
    g = torch.zeros(4, 8, dtype=torch.bfloat16)
    for bad in (torch.bfloat16, torch.float16, torch.float64):
        with pytest.raises(TypeError, match="momentum must be float32"):
            ms.matrix(p, g, torch.zeros(4, 8, dtype=bad))
        with pytest.raises(TypeError, match="ns_out must be float32"):
            ms.matrix(p, g, torch.zeros(4, 8), torch.zeros(4, 8, dtype=bad))
        f = torch.zeros(32)
        with pytest.raises(TypeError, match="exp_avg must be float32"):
            ms.adamw_tensor(f, f.clone(), torch.zeros(32, dtype=bad), f.clone())
        with pytest.raises(TypeError, match="exp_avg_sq must be float32"):
            ms.adamw_tensor(f, f.clone(), f.clone(), torch.zeros(32, dtype=bad))
    with pytest.raises(TypeError, match="unsupported dtype"):
        ms.matrix(torch.zeros(4, 8, dtype=torch.float16), g, torch.zeros(4, 8))


def test_binding_rejects_host_tensors_before_any_launch():
    """A host tensor's data_ptr is a host address: every entry point's tensors must be
    GPU tensors of the context's device, checked before the library is called."""
    import torch
    p = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        ms.matrix(p, p.clone(), torch.zeros(4, 8))
    f = torch.zeros(32)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        ms.adamw_tensor(f, f.clone(), f.clone(), f.clone())
    ctx = ms.Context.__new__(ms.Context)   # no device context: the checks come first
    ctx.lib, ctx.device, ctx.handle = ms.load(), 0, None
    hp = ms.make_hparams()
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        ctx.muon_ns_only(torch.zeros(4, 8), torch.zeros(4, 8), hp)
    with pytest.raises(TypeError, match="x_out must be float32"):
        ctx.muon_ns_only(torch.zeros(4, 8), torch.zeros(4, 8, dtype=torch.bfloat16), hp)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        ctx.muon_apply_update(p, torch.zeros(4, 8), hp)
    with pytest.raises(ValueError, match="one shape"):
        ctx.muon_apply_update(p, torch.zeros(8, 4), hp)
    # a descriptor built on another GPU than the context's
    m = ms.muon_matrix()
    m._device = 3
    with pytest.raises(ValueError, match="cuda:3"):
        ctx.muon_step([m], hp)
