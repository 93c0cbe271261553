"""Python binding of the MI355X Muon step library (libmuon_step.so).

Argument marshalling only: every step of the optimizer runs in the library's
HIP kernels.  torch tensors are accepted for convenience (their device
pointers, shapes and the current HIP stream are passed through); the C ABI
itself takes plain pointers and sizes (include/muon_step.h).

The library is loaded from this directory; when it is missing, loading fails
with an error that says how to build it (there is no fallback path).
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuon_step.so")

MUON_OK = 0
MUON_ERR_INVALID_ARGUMENT = 1
MUON_ERR_UNSUPPORTED = 2
MUON_ERR_OUT_OF_MEMORY = 3
MUON_ERR_DEVICE = 4

MUON_F32 = 0
MUON_BF16 = 1
MUON_NS_BF16 = 0
MUON_NS_F32 = 1
MUON_SCALE_SQRT_MAX = 0
MUON_SCALE_UNIT_RMS = 1

# Names every build of the library exports (the functions include/muon_step.h declares).
EXPORTS = (
    "muon_abi_version", "muon_status_string", "muon_schedule", "muon_check_step_args",
    "muon_check_adamw_args", "muon_workspace_bytes", "muon_create", "muon_destroy",
    "muon_last_error", "muon_step", "muon_adamw_step", "muon_ns_only", "muon_apply_update",
    "muon_last_norms", "muon_profile_enable", "muon_profile_read", "muon_step_noalloc",
    "muon_stream_probe", "muon_ns_stage", "muon_set_concurrent_groups",
)

MUON_STAGE_GRAM = 0
MUON_STAGE_POLY = 1
MUON_STAGE_APPLY = 2


class MuonError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class muon_ns_coeff(ctypes.Structure):
    _fields_ = [("a", ctypes.c_double), ("b", ctypes.c_double), ("c", ctypes.c_double)]


class muon_matrix(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p),
                ("ns_out", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("param_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32)]


class muon_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("momentum", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("gamma", ctypes.c_double),
                ("schedule", ctypes.POINTER(muon_ns_coeff)), ("num_ns_steps", ctypes.c_int32),
                ("nesterov", ctypes.c_int32), ("ns_precision", ctypes.c_int32),
                ("scale_mode", ctypes.c_int32)]


class muon_adamw_tensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("numel", ctypes.c_int64),
                ("param_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32)]


class muon_adamw_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64)]


class muon_stage_stats(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


_lib = None


def load(path=LIB_PATH):
    """Loads libmuon_step.so and declares its signatures.  Raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m muon_step_amd.build` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    c = ctypes
    vp, i32, i64, sz = c.c_void_p, c.c_int32, c.c_int64, c.c_size_t
    sig = {
        "muon_abi_version": (i32, []),
        "muon_status_string": (c.c_char_p, [i32]),
        "muon_schedule": (i64, [c.c_char_p, c.POINTER(muon_ns_coeff), i64]),
        "muon_check_step_args": (i32, [c.POINTER(muon_matrix), i64, c.POINTER(muon_hparams),
                                       c.c_char_p, sz]),
        "muon_check_adamw_args": (i32, [c.POINTER(muon_adamw_tensor), i64,
                                        c.POINTER(muon_adamw_hparams), c.c_char_p, sz]),
        "muon_workspace_bytes": (i32, [c.POINTER(muon_matrix), i64, c.POINTER(muon_hparams),
                                       c.POINTER(sz)]),
        "muon_create": (i32, [c.POINTER(vp), i32, sz]),
        "muon_destroy": (i32, [vp]),
        "muon_last_error": (c.c_char_p, [vp]),
        "muon_step": (i32, [vp, c.POINTER(muon_matrix), i64, c.POINTER(muon_hparams), vp]),
        "muon_step_noalloc": (i32, [vp, c.POINTER(muon_matrix), i64, c.POINTER(muon_hparams), vp]),
        "muon_adamw_step": (i32, [vp, c.POINTER(muon_adamw_tensor), i64,
                                  c.POINTER(muon_adamw_hparams), vp]),
        "muon_ns_only": (i32, [vp, vp, vp, i64, i64, c.POINTER(muon_hparams), vp]),
        "muon_apply_update": (i32, [vp, vp, i32, vp, i64, i64, c.POINTER(muon_hparams), vp]),
        "muon_last_norms": (i32, [vp, c.POINTER(c.c_double), i64, c.POINTER(i64)]),
        "muon_stream_probe": (i32, [vp, vp, vp, i64, i64, i32, i32, vp]),
        "muon_ns_stage": (i32, [vp, i32, vp, vp, vp, i64, i64, c.c_double, c.c_double, c.c_double, vp]),
        "muon_profile_enable": (i32, [vp, i32]),
        "muon_set_concurrent_groups": (i32, [vp, i32]),
        "muon_profile_read": (i32, [vp, c.POINTER(muon_stage_stats), i32, c.POINTER(i32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ------------------------------------------------------------------ marshalling helpers

def schedule(name="deepseekv4"):
    """Coefficient triples of a named schedule, from the library."""
    lib = load()
    n = lib.muon_schedule(name.encode(), None, 0)
    if n < 0:
        raise ValueError(f"unknown schedule {name!r}")
    arr = (muon_ns_coeff * n)()
    lib.muon_schedule(name.encode(), arr, n)
    return [(x.a, x.b, x.c) for x in arr]


def make_hparams(lr=0.02, momentum=0.95, weight_decay=0.1, gamma=0.2, nesterov=True,
                 coeffs=None, ns_precision=MUON_NS_BF16, scale_mode=MUON_SCALE_SQRT_MAX):
    """Builds a muon_hparams; `coeffs` defaults to the DeepSeek-V4 hybrid schedule.
    The returned object keeps its schedule array alive."""
    if coeffs is None:
        coeffs = schedule("deepseekv4")
    arr = (muon_ns_coeff * max(1, len(coeffs)))(*[muon_ns_coeff(*c) for c in coeffs])
    hp = muon_hparams(lr, momentum, weight_decay, gamma,
                      ctypes.cast(arr, ctypes.POINTER(muon_ns_coeff)) if coeffs else None,
                      len(coeffs), 1 if nesterov else 0, ns_precision, scale_mode)
    hp._keep = arr
    return hp


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return MUON_F32
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _on_one_gpu(named):
    """Raises unless every (name, tensor) is a GPU tensor and all share one device;
    returns that device's index.  The C ABI takes raw pointers: a host tensor would
    hand a kernel a host address."""
    dev = None
    for name, t in named:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    return dev.index


def _require_f32(named):
    """Raises unless every (name, tensor) is float32: the C ABI has no dtype field
    for these buffers, so another dtype would be read and written past its end."""
    import torch
    for name, t in named:
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")


def matrix(param, grad, momentum, ns_out=None):
    """muon_matrix for torch tensors (row-major contiguous, same shape, one GPU;
    momentum and ns_out float32, param and grad float32 or bfloat16)."""
    named = [("param", param), ("grad", grad), ("momentum", momentum)]
    if ns_out is not None:
        named.append(("ns_out", ns_out))
    for name, t in named:
        if not t.is_contiguous() or t.dim() != 2 or t.shape != param.shape:
            raise ValueError("param, grad, momentum and ns_out must be contiguous 2-D of one shape")
    _require_f32(named[2:])
    pd, gd = _dtype_code(param), _dtype_code(grad)
    dev = _on_one_gpu(named)
    m = muon_matrix(param.data_ptr(), grad.data_ptr(), momentum.data_ptr(),
                    ns_out.data_ptr() if ns_out is not None else None,
                    param.shape[0], param.shape[1], pd, gd)
    m._device = dev
    return m


def _check(lib, ctx, status, what):
    if status != MUON_OK:
        msg = lib.muon_last_error(ctx).decode() if ctx else ""
        raise MuonError(status, f"{what}: {lib.muon_status_string(status).decode()}: {msg}")


class Context:
    """Owns one muon_context (device workspace and descriptor tables)."""

    def __init__(self, device=0, workspace_cap_bytes=0):
        self.lib = load()
        self.device = device
        h = ctypes.c_void_p()
        st = self.lib.muon_create(ctypes.byref(h), device, workspace_cap_bytes)
        if st != MUON_OK:
            raise MuonError(st, f"muon_create: {self.lib.muon_status_string(st).decode()}")
        self.handle = h

    def close(self):
        if self.handle:
            self.lib.muon_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check_device(self, items, what):
        for k, it in enumerate(items):
            dev = getattr(it, "_device", None)
            if dev is not None and dev != self.device:
                raise ValueError(f"{what} {k} lives on cuda:{dev}, the context on cuda:{self.device}")

    def _check_tensors(self, named):
        if _on_one_gpu(named) != self.device:
            raise ValueError(f"tensors live on another GPU than the context (cuda:{self.device})")

    # The methods below keep the C ABI's names.
    def muon_step(self, mats, hp, stream=None):
        self._check_device(mats, "matrix")
        arr = (muon_matrix * len(mats))(*mats)
        st = self.lib.muon_step(self.handle, arr, len(mats), ctypes.byref(hp), _stream_handle(stream))
        _check(self.lib, self.handle, st, "muon_step")

    def muon_step_noalloc(self, mats, hp, stream=None):
        self._check_device(mats, "matrix")
        arr = (muon_matrix * len(mats))(*mats)
        st = self.lib.muon_step_noalloc(self.handle, arr, len(mats), ctypes.byref(hp), _stream_handle(stream))
        _check(self.lib, self.handle, st, "muon_step_noalloc")

    def muon_adamw_step(self, tensors, hp, stream=None):
        self._check_device(tensors, "tensor")
        arr = (muon_adamw_tensor * len(tensors))(*tensors)
        st = self.lib.muon_adamw_step(self.handle, arr, len(tensors), ctypes.byref(hp),
                                      _stream_handle(stream))
        _check(self.lib, self.handle, st, "muon_adamw_step")

    def muon_ns_only(self, n_in, x_out, hp, stream=None):
        named = [("n_in", n_in), ("x_out", x_out)]
        for name, t in named:
            if not t.is_contiguous() or t.dim() != 2 or t.shape != n_in.shape:
                raise ValueError("n_in and x_out must be contiguous 2-D of one shape")
        _require_f32(named)
        self._check_tensors(named)
        st = self.lib.muon_ns_only(self.handle, n_in.data_ptr(), x_out.data_ptr(), n_in.shape[0],
                                   n_in.shape[1], ctypes.byref(hp), _stream_handle(stream))
        _check(self.lib, self.handle, st, "muon_ns_only")

    def muon_apply_update(self, param, x, hp, stream=None):
        named = [("param", param), ("x", x)]
        for name, t in named:
            if not t.is_contiguous() or t.dim() != 2 or t.shape != param.shape:
                raise ValueError("param and x must be contiguous 2-D of one shape")
        _require_f32(named[1:])
        _dtype_code(param)
        self._check_tensors(named)
        st = self.lib.muon_apply_update(self.handle, param.data_ptr(), _dtype_code(param), x.data_ptr(),
                                        param.shape[0], param.shape[1], ctypes.byref(hp),
                                        _stream_handle(stream))
        _check(self.lib, self.handle, st, "muon_apply_update")

    def muon_last_norms(self, capacity):
        out = (ctypes.c_double * max(1, capacity))()
        n = ctypes.c_int64()
        st = self.lib.muon_last_norms(self.handle, out, capacity, ctypes.byref(n))
        _check(self.lib, self.handle, st, "muon_last_norms")
        return list(out[:min(capacity, n.value)])


    def muon_ns_stage(self, stage, out, x=None, m=None, a=0.0, b=0.0, c=0.0, stream=None):
        """One bf16 product stage; x (s x l), m (s x s), out: fp32 GPU tensors."""
        named = [("out", out)] + [(n, t) for n, t in (("x", x), ("m", m)) if t is not None]
        for name, t in named:
            if not t.is_contiguous() or t.dim() != 2:
                raise ValueError(f"{name} must be a contiguous 2-D tensor")
        _require_f32(named)
        self._check_tensors(named)
        s, l = (x.shape if x is not None else (m.shape[0], m.shape[0]))
        st = self.lib.muon_ns_stage(self.handle, stage, x.data_ptr() if x is not None else None,
                                    m.data_ptr() if m is not None else None, out.data_ptr(), s, l, a, b, c,
                                    _stream_handle(stream))
        _check(self.lib, self.handle, st, "muon_ns_stage")

    def muon_stream_probe(self, src, dst, stream_bytes, reads, writes, pitch_bytes=None, stream=None):
        """src, dst: GPU tensors holding `reads` / `writes` streams of stream_bytes each,
        pitch_bytes (default stream_bytes) apart."""
        pitch = stream_bytes if pitch_bytes is None else pitch_bytes
        for name, t, k in (("src", src, reads), ("dst", dst, writes)):
            if not t.is_contiguous() or t.numel() * t.element_size() < (k - 1) * pitch + stream_bytes:
                raise ValueError(f"{name} must be contiguous and hold {k} streams of {stream_bytes} bytes "
                                 f"{pitch} bytes apart")
        self._check_tensors([("src", src), ("dst", dst)])
        st = self.lib.muon_stream_probe(self.handle, src.data_ptr(), dst.data_ptr(), stream_bytes, pitch, reads,
                                        writes, _stream_handle(stream))
        _check(self.lib, self.handle, st, "muon_stream_probe")

    def muon_set_concurrent_groups(self, enable=True):
        _check(self.lib, self.handle, self.lib.muon_set_concurrent_groups(self.handle, 1 if enable else 0),
               "muon_set_concurrent_groups")

    def muon_profile_enable(self, enable=True):
        _check(self.lib, self.handle, self.lib.muon_profile_enable(self.handle, 1 if enable else 0),
               "muon_profile_enable")

    def muon_profile_read(self):
        """Per-stage {name: dict(launches, total_ms, flops, bytes)} since the last enable/read."""
        cap = 32
        out = (muon_stage_stats * cap)()
        n = ctypes.c_int32()
        _check(self.lib, self.handle, self.lib.muon_profile_read(self.handle, out, cap, ctypes.byref(n)),
               "muon_profile_read")
        return {out[i].name.decode(): {"launches": out[i].launches, "total_ms": out[i].total_ms,
                                       "flops": out[i].flops, "bytes": out[i].bytes}
                for i in range(min(cap, n.value))}


def adamw_tensor(param, grad, exp_avg, exp_avg_sq):
    """muon_adamw_tensor for torch tensors (contiguous, equal numel, one GPU;
    exp_avg and exp_avg_sq float32)."""
    named = [("param", param), ("grad", grad), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)]
    for _, t in named:
        if not t.is_contiguous() or t.numel() != param.numel():
            raise ValueError("AdamW tensors must be contiguous with equal numel")
    _require_f32(named[2:])
    pd, gd = _dtype_code(param), _dtype_code(grad)
    dev = _on_one_gpu(named)
    t = muon_adamw_tensor(param.data_ptr(), grad.data_ptr(), exp_avg.data_ptr(),
                          exp_avg_sq.data_ptr(), param.numel(), pd, gd)
    t._device = dev
    return t


def adamw_hparams(lr=0.02, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1):
    return muon_adamw_hparams(lr, beta1, beta2, eps, weight_decay, step)
