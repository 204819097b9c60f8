"""Python binding of libep.so, the fused GEMM + epilogue library for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the library's HIP
kernels; PyTorch provides device memory and streams.  The API mirrors the stateful
plan / execute / free sequence of the pages (nvmath-python's Matmul as described in
"Fusing Matmul Epilogs with nvmath-python" and in the hotdry.top cuBLASLt post):

    p = Plan(x, w, epilog="RELU_AUX_BIAS", epilog_inputs={"bias": b}, b_layout="KN")
    y, aux = p.execute()          # aux["relu_aux"]: int32 tensor holding the uint32 mask words
    dp = Plan(dy, w, epilog="DRELU_BGRAD", epilog_inputs={"relu_aux": aux["relu_aux"]},
              b_layout="NK")
    dx, aux = dp.execute()        # aux["drelu_bgrad"]: float32 bias gradient
    p.free(); dp.free()

The library is loaded from this package directory; if it has not been built the import
of the library fails loudly (there is no fallback).
"""
import ctypes
import os

import torch

__all__ = ["Plan", "EPError", "EPILOGS", "lib", "library_path", "abi_version", "num_tile_cfgs", "validate_operands",
           "describe_plan"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# EP_LIBRARY names another build of the same library (the host-sanitizer build the CPU tests use)
library_path = os.environ.get("EP_LIBRARY") or os.path.join(_HERE, "libep.so")

EPILOGS = {
    "DEFAULT": 0, "BIAS": 1, "RELU_BIAS": 2, "RELU_AUX_BIAS": 3,
    "DRELU_BGRAD": 4, "SWIGLU": 5, "DSWIGLU": 6,
    "GELU_BIAS": 7, "GELU_AUX_BIAS": 8, "DGELU_BGRAD": 9, "SWIGLU_AUX": 10,
}
_LAYOUTS = {"KN": 0, "NK": 1}
_DTYPES = {torch.float16: 0, torch.bfloat16: 1}
_PATHS = {"fused": 0, "unfused": 1}
_BGRAD = {"two_pass": 0, "atomic": 1}
STATUS = {0: "EP_OK", 1: "EP_ERR_INVALID_ARG", 2: "EP_ERR_UNSUPPORTED", 3: "EP_ERR_OUT_OF_MEMORY",
          4: "EP_ERR_HIP", 5: "EP_ERR_INTERNAL"}


class ep_shape(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("b_layout", ctypes.c_int), ("a", ctypes.c_void_p), ("lda", ctypes.c_int64),
                ("b", ctypes.c_void_p), ("ldb", ctypes.c_int64), ("d", ctypes.c_void_p),
                ("ldd", ctypes.c_int64), ("a_layout", ctypes.c_int)]


class ep_epilog_io(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("relu_aux", ctypes.c_void_p),
                ("relu_aux_in", ctypes.c_void_p), ("ld_aux", ctypes.c_int64),
                ("bgrad", ctypes.c_void_p), ("b2", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("up", ctypes.c_void_p), ("ld_gu", ctypes.c_int64), ("d2", ctypes.c_void_p),
                ("ldd2", ctypes.c_int64), ("gelu_aux", ctypes.c_void_p), ("ld_gelu_aux", ctypes.c_int64)]


class ep_options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("bgrad_mode", ctypes.c_int), ("tile_cfg", ctypes.c_int),
                ("split_k", ctypes.c_int), ("split_tail", ctypes.c_int), ("autotune", ctypes.c_int)]


class EPError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {message}")


_lib = None


def lib():
    """The loaded libep.so (raises if it is missing: build it first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is not built; run `python -m dense_gemm_epilogues_amd.build`")
        L = ctypes.CDLL(library_path)
        L.ep_plan_ex.argtypes = [ctypes.POINTER(ep_shape), ctypes.c_int, ctypes.c_int,
                                 ctypes.POINTER(ep_epilog_io), ctypes.POINTER(ep_options),
                                 ctypes.POINTER(ctypes.c_void_p)]
        L.ep_plan_ex.restype = ctypes.c_int
        L.ep_plan.argtypes = [ctypes.POINTER(ep_shape), ctypes.c_int, ctypes.c_int,
                              ctypes.POINTER(ep_epilog_io), ctypes.POINTER(ctypes.c_void_p)]
        L.ep_plan.restype = ctypes.c_int
        L.ep_execute.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.ep_execute.restype = ctypes.c_int
        L.ep_free.argtypes = [ctypes.c_void_p]
        L.ep_free.restype = ctypes.c_int
        L.ep_status_string.argtypes = [ctypes.c_int]
        L.ep_status_string.restype = ctypes.c_char_p
        L.ep_last_error.argtypes = []
        L.ep_last_error.restype = ctypes.c_char_p
        L.ep_plan_info.argtypes = [ctypes.c_void_p, ctypes.c_char_p, ctypes.c_size_t]
        L.ep_plan_info.restype = ctypes.c_int
        L.ep_abi_version.argtypes = []
        L.ep_abi_version.restype = ctypes.c_int
        L.ep_num_tile_cfgs.argtypes = []
        L.ep_num_tile_cfgs.restype = ctypes.c_int
        L.ep_plan_describe.argtypes = [ctypes.POINTER(ep_shape), ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(ep_epilog_io), ctypes.POINTER(ep_options), ctypes.c_int,
                                       ctypes.c_char_p, ctypes.c_size_t]
        L.ep_plan_describe.restype = ctypes.c_int
        _lib = L
    return _lib


def abi_version():
    return lib().ep_abi_version()


def num_tile_cfgs():
    return lib().ep_num_tile_cfgs()


def describe_plan(m, n, k, epilog="DEFAULT", dtype=torch.float16, b_layout="KN", a_layout="MK", cus=256,
                  path="fused", bgrad_mode="two_pass", tile_cfg=-1, split_k=0, split_tail=False):
    """The plan ep_plan_ex would make for an m x n x k GEMM with this epilog on a device with
    `cus` compute units, as the string Plan.info() returns (ep_plan_describe: no device is
    touched, nothing is allocated).  The operands are described by their sizes only, with
    dense leading dimensions; the library checks the pointers it is given for alignment but
    never reads them, so placeholder addresses stand in for them."""
    fake = ctypes.c_void_p(1 << 20)  # non-null, 16-byte aligned, never dereferenced
    dual = epilog in ("SWIGLU", "SWIGLU_AUX")
    shape = ep_shape(m=m, n=n, k=k, b_layout=_LAYOUTS[b_layout], a=fake, lda=k if a_layout == "MK" else m,
                     b=fake, ldb=n if b_layout == "KN" else k, d=fake, ldd=n, a_layout=0 if a_layout == "MK" else 1)
    io = ep_epilog_io()
    if epilog in ("BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "GELU_BIAS", "GELU_AUX_BIAS"):
        io.bias = fake
    if epilog == "RELU_AUX_BIAS":
        io.relu_aux = fake
    if epilog in ("DRELU_BGRAD", "DGELU_BGRAD"):
        io.bgrad = fake
    if epilog == "DRELU_BGRAD":
        io.relu_aux_in = fake
    if epilog in ("GELU_AUX_BIAS", "DGELU_BGRAD"):
        io.gelu_aux = fake
    if dual:
        io.b2 = fake
    if epilog in ("DSWIGLU", "SWIGLU_AUX"):
        io.d2 = fake
    if epilog == "DSWIGLU":
        io.gate, io.up = fake, fake
    opt = ep_options(path=_PATHS[path], bgrad_mode=_BGRAD[bgrad_mode], tile_cfg=tile_cfg, split_k=split_k,
                     split_tail=int(bool(split_tail)), autotune=0)
    buf = ctypes.create_string_buffer(1024)
    _check(lib().ep_plan_describe(ctypes.byref(shape), _DTYPES[dtype], EPILOGS[epilog], ctypes.byref(io),
                                  ctypes.byref(opt), cus, buf, len(buf)))
    return buf.value.decode()


def _check(status):
    if status != 0:
        raise EPError(status, lib().ep_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("operands must be 2-D with unit column stride")
    return t.stride(0)


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensor(name, t, rows, cols, dtype, device, min_cols=False):
    """Raise ValueError unless `t` is a tensor of `dtype` on `device` laid out as the C ABI
    reads it: 2-D (rows x cols, or at least `cols` columns when min_cols) with unit column
    stride, or 1-D of length cols (rows None) with unit stride.  The library receives only a
    pointer and leading dimensions, so these checks stand between a wrong tensor and kernels
    that would read or write past its storage."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if rows is None:
        if t.dim() != 1 or t.shape[0] != cols or (cols > 1 and t.stride(0) != 1):
            raise ValueError(f"{name} must be a contiguous ({cols},) vector, got shape {tuple(t.shape)} "
                             f"stride {t.stride()}")
    else:
        ok_cols = t.dim() == 2 and (t.shape[1] >= cols if min_cols else t.shape[1] == cols)
        if t.dim() != 2 or t.shape[0] != rows or not ok_cols:
            want = f"({rows}, >= {cols})" if min_cols else f"({rows}, {cols})"
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
        if t.stride(1) != 1 and t.shape[1] > 1:
            raise ValueError(f"{name} must have unit column stride, got stride {t.stride()}")
        if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
            raise ValueError(f"{name}: row stride {t.stride(0)} is below the row length {t.shape[1]}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the operands are on {device}")


def validate_operands(a, b, epilog, epilog_inputs, b_layout, a_layout, out, aux_out):
    """Check every tensor a Plan would hand to the C ABI against the problem a and b define
    (raises ValueError; returns (m, n, k)).  All tensors must be on a.device, which must be a
    CUDA (HIP) device; b, b2, out, bias, gate, up, gelu_aux, gu and d_up have a's dtype;
    relu_aux holds int32 words; bias gradients are float32."""
    if not isinstance(a, torch.Tensor) or not isinstance(b, torch.Tensor):
        raise ValueError("a and b must be torch tensors")
    if a.dtype not in _DTYPES:
        raise ValueError(f"a must be float16 or bfloat16, got {a.dtype}")
    if b_layout not in _LAYOUTS:
        raise ValueError(f"unknown b_layout {b_layout!r}")
    if a_layout not in ("MK", "KM"):
        raise ValueError(f"unknown a_layout {a_layout!r}")
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    dt, dev = a.dtype, a.device
    m, k = (a.shape[0], a.shape[1]) if a_layout == "MK" else (a.shape[1], a.shape[0])
    n = b.shape[1] if b_layout == "KN" else b.shape[0]
    _check_tensor("a", a, a.shape[0], a.shape[1], dt, dev)
    _check_tensor("b", b, k if b_layout == "KN" else n, k if b_layout == "NK" else n, dt, dev)
    if out is not None:
        _check_tensor("out", out, m, n, dt, dev)
    ins = epilog_inputs
    nw = (n + 31) // 32
    need = {
        "BIAS": ("bias",), "RELU_BIAS": ("bias",), "RELU_AUX_BIAS": ("bias",), "GELU_BIAS": ("bias",),
        "GELU_AUX_BIAS": ("bias",), "DRELU_BGRAD": ("relu_aux",), "SWIGLU": ("b2",), "SWIGLU_AUX": ("b2",),
        "DSWIGLU": ("gate", "up"), "DGELU_BGRAD": ("gelu_aux",),
    }.get(epilog, ())
    for key in need:
        if key not in ins:
            raise ValueError(f"epilog {epilog} needs epilog_inputs[{key!r}]")
    for key in ins:
        if key not in need:
            raise ValueError(f"epilog {epilog} takes no epilog_inputs[{key!r}]")
    if "bias" in ins:
        _check_tensor("bias", ins["bias"], None, n, dt, dev)
    if "relu_aux" in ins:
        _check_tensor("relu_aux", ins["relu_aux"], m, nw, torch.int32, dev, min_cols=True)
    if "b2" in ins:
        _check_tensor("b2", ins["b2"], b.shape[0], b.shape[1], dt, dev)
        if ins["b2"].stride(0) != b.stride(0):
            raise ValueError("b2 must have the same row stride as b")
    if "gate" in ins:
        _check_tensor("gate", ins["gate"], m, n, dt, dev)
        _check_tensor("up", ins["up"], m, n, dt, dev)
        if ins["gate"].stride(0) != ins["up"].stride(0):
            raise ValueError("gate and up must share a row stride")
    if "gelu_aux" in ins:
        _check_tensor("gelu_aux", ins["gelu_aux"], m, n, dt, dev)
    aux_shapes = {"relu_aux": (m, nw, torch.int32, True), "drelu_bgrad": (None, n, torch.float32, False),
                  "dgelu_bgrad": (None, n, torch.float32, False), "gelu_aux": (m, n, dt, False),
                  "d_up": (m, n, dt, False), "gu": (m, 2 * n, dt, False)}
    for key, t in aux_out.items():
        if key not in aux_shapes:
            raise ValueError(f"unknown aux_out {key!r}")
        rows, cols, adt, mc = aux_shapes[key]
        _check_tensor(f"aux_out[{key!r}]", t, rows, cols, adt, dev, min_cols=mc)
    if dev.type != "cuda":
        raise ValueError(f"operands must be on a CUDA (HIP) device, got {dev}")
    return m, n, k


class Plan:
    """A planned fused GEMM + epilog (the C library's ep_handle).

    a: M x K (a_layout "MK"), or K x M ("KM": the GEMM uses a's transpose; DEFAULT epilog only,
    as in a weight gradient X^T dY).  b: K x N (b_layout "KN") or N x K ("NK").  epilog_inputs:
      BIAS / RELU_BIAS / RELU_AUX_BIAS: {"bias": (N,)}
      DRELU_BGRAD: {"relu_aux": (M, >= ceil(N/32)) int32 mask words}
      SWIGLU / SWIGLU_AUX: {"b2": up weight, same layout as b}; SWIGLU_AUX also returns "gu", the
        (M, 2N) pre-activations [gate | up] that DSWIGLU can take as its gate and up
      DSWIGLU: {"gate": (M, N), "up": (M, N)}
      GELU_BIAS / GELU_AUX_BIAS: {"bias": (N,)}
      DGELU_BGRAD: {"gelu_aux": (M, N) pre-activation saved by GELU_AUX_BIAS}
    aux outputs (execute()'s second value): relu_aux, drelu_bgrad, d_up, gelu_aux, dgelu_bgrad, gu.
    Outputs are allocated here with torch.empty unless `out` / `aux_out` are given and are
    reused by every execute().  Tensors are kept alive for the plan's lifetime.
    path "fused" | "unfused"; bgrad_mode "two_pass" | "atomic"; tile_cfg -1 (by shape) or an
    index < num_tile_cfgs(); split_k 0 (by shape), 1 (never) or 2..8 K ranges per tile;
    split_tail=True (with split_k >= 2) splits only the tiles of the last, partly filled round
    of workgroups and runs the others whole;
    autotune=True times every (tile configuration, split) on these buffers at plan time
    (overwriting the outputs) and keeps the fastest, cached per problem for the process.
    """

    def __init__(self, a, b, epilog="DEFAULT", epilog_inputs=None, b_layout="KN", out=None,
                 aux_out=None, path="fused", bgrad_mode="two_pass", tile_cfg=-1, split_k=0, autotune=False,
                 a_layout="MK", split_tail=False):
        L = lib()
        epilog_inputs = dict(epilog_inputs or {})
        aux_out = dict(aux_out or {})
        if epilog not in EPILOGS:
            raise ValueError(f"unknown epilog {epilog!r}")
        m, n, k = validate_operands(a, b, epilog, epilog_inputs, b_layout, a_layout, out, aux_out)
        if out is None:
            out = torch.empty((m, n), dtype=a.dtype, device=a.device)
        self.epilog = epilog
        self.out = out
        self.aux = {}
        io = ep_epilog_io()
        if epilog in ("BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "GELU_BIAS", "GELU_AUX_BIAS"):
            io.bias = _ptr(epilog_inputs["bias"])
        if epilog == "GELU_AUX_BIAS":
            ga = aux_out.get("gelu_aux")
            if ga is None:
                ga = torch.empty((m, n), dtype=a.dtype, device=a.device)
            io.gelu_aux, io.ld_gelu_aux = _ptr(ga), ga.stride(0)
            self.aux["gelu_aux"] = ga
        if epilog == "DGELU_BGRAD":
            gi = epilog_inputs["gelu_aux"]
            io.gelu_aux, io.ld_gelu_aux = _ptr(gi), gi.stride(0)
            bg = aux_out.get("dgelu_bgrad")
            if bg is None:
                bg = torch.empty((n,), dtype=torch.float32, device=a.device)
            io.bgrad = _ptr(bg)
            self.aux["dgelu_bgrad"] = bg
        if epilog == "RELU_AUX_BIAS":
            ra = aux_out.get("relu_aux")
            if ra is None:
                ra = torch.empty((m, (n + 31) // 32), dtype=torch.int32, device=a.device)
            io.relu_aux = _ptr(ra)
            io.ld_aux = ra.stride(0)
            self.aux["relu_aux"] = ra
        if epilog == "DRELU_BGRAD":
            ri = epilog_inputs["relu_aux"]
            io.relu_aux_in = _ptr(ri)
            io.ld_aux = ri.stride(0)
            bg = aux_out.get("drelu_bgrad")
            if bg is None:
                bg = torch.empty((n,), dtype=torch.float32, device=a.device)
            io.bgrad = _ptr(bg)
            self.aux["drelu_bgrad"] = bg
        if epilog in ("SWIGLU", "SWIGLU_AUX"):
            io.b2 = _ptr(epilog_inputs["b2"])
        if epilog == "SWIGLU_AUX":
            gu = aux_out.get("gu")
            if gu is None:
                gu = torch.empty((m, 2 * n), dtype=a.dtype, device=a.device)
            io.d2, io.ldd2 = _ptr(gu), gu.stride(0)
            self.aux["gu"] = gu
        if epilog == "DSWIGLU":
            g, u = epilog_inputs["gate"], epilog_inputs["up"]
            io.gate, io.up, io.ld_gu = _ptr(g), _ptr(u), g.stride(0)
            d2 = aux_out.get("d_up")
            if d2 is None:
                d2 = torch.empty_like(out)
            io.d2, io.ldd2 = _ptr(d2), d2.stride(0)
            self.aux["d_up"] = d2
        shape = ep_shape(m=m, n=n, k=k, b_layout=_LAYOUTS[b_layout], a=_ptr(a), lda=_ld(a),
                         b=_ptr(b), ldb=_ld(b), d=_ptr(out), ldd=_ld(out), a_layout=0 if a_layout == "MK" else 1)
        opt = ep_options(path=_PATHS[path], bgrad_mode=_BGRAD[bgrad_mode], tile_cfg=tile_cfg, split_k=split_k,
                         split_tail=int(bool(split_tail)), autotune=int(bool(autotune)))
        handle = ctypes.c_void_p()
        self._keep = (a, b, out, epilog_inputs, dict(self.aux))
        _check(L.ep_plan_ex(ctypes.byref(shape), _DTYPES[a.dtype], EPILOGS[epilog], ctypes.byref(io),
                            ctypes.byref(opt), ctypes.byref(handle)))
        self._h = handle

    def execute(self, stream=None):
        """Enqueue on `stream` (default: torch's current stream); returns (out, aux)."""
        if self._h is None:
            raise RuntimeError("plan has been freed")
        _check(lib().ep_execute(self._h, _stream_handle(stream)))
        return self.out, self.aux

    def info(self):
        buf = ctypes.create_string_buffer(1024)
        _check(lib().ep_plan_info(self._h, buf, len(buf)))
        return buf.value.decode()

    def free(self):
        if getattr(self, "_h", None) is not None:
            _check(lib().ep_free(self._h))
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
