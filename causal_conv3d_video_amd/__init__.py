"""Cached causal Conv3D on AMD Instinct MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI of ``libcc3d.so`` (declared in
``include/cc3d.h``), with the same entry-point names.  It only marshals
arguments: every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory and streams.  There is no fallback: if the
library is missing, importing this package raises.

The operation ("Cache-Aware Conv3D Lowering Across Embedded World-Model
Decoders", lowering section): with Z = [C; X] along time and
p_l = p_base - |C|, output frame o is the bias plus the sum over active
temporal taps k of the spatial Conv2D of Z[o + k*d_t - p_l] with W[:, :, k].

Tensor layouts (physical, channels last): activations [N][T][H][W][C];
weights [Cout][Kt][Kh][Kw][Cin]; bias [Cout].  A tensor may be passed either
as a contiguous tensor of that physical shape, or as the PyTorch-convention
NCDHW / OIDHW tensor in ``torch.channels_last_3d`` memory format.
"""
import ctypes
import os

import torch

__all__ = [
    "CC3DError", "Plan", "make_desc",
    "causal_conv3d_plan", "causal_conv3d_plan_variant", "causal_conv3d_plan_autotune", "causal_conv3d_plan_info",
    "causal_conv3d_plan_destroy",
    "causal_conv3d_forward", "causal_conv3d_pack_weights", "causal_conv3d_forward_packed",
    "causal_conv3d_forward_packed_noalloc",
    "causal_conv3d_forward_u8", "causal_conv3d_status_string", "causal_conv3d_counters", "library_path",
    "EXPORTED_SYMBOLS", "VARIANTS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libcc3d.so")

EXPORTED_SYMBOLS = (
    "causal_conv3d_plan", "causal_conv3d_plan_variant", "causal_conv3d_plan_autotune", "causal_conv3d_plan_info",
    "causal_conv3d_plan_destroy",
    "causal_conv3d_forward", "causal_conv3d_pack_weights", "causal_conv3d_forward_packed",
    "causal_conv3d_forward_packed_noalloc",
    "causal_conv3d_forward_u8", "causal_conv3d_status_string", "causal_conv3d_counters",
)

# Every kernel variant name causal_conv3d_plan_variant accepts (include/cc3d.h).
VARIANTS = (("bf16_s3_n64_p24x32_g32", "bf16_s3_n96_p16x32_g32", "bf16_s3_n96_p8x32_x2", "bf16_s3_n32_p8x32")
            + tuple("bf16_s3_few_p%dx128" % r for r in range(4, 17))
            + ("bf16_s1_n192_p8x32", "bf16_s1_n192_p256_rd", "bf16_s1_n32_p8x32", "bf16_gen_n64_p8x32", "bf16_gen_n96_p8x32",
               "bf16_s3d2_n64_p16x32_g32", "bf16_s3s2_n96_p4x32_g32", "bf16_s3s2_n64_p4x32_g32", "f32_direct"))

CC3D_OK, CC3D_ERR_INVALID_ARG, CC3D_ERR_UNSUPPORTED, CC3D_ERR_DEVICE, CC3D_ERR_NO_MEMORY = range(5)
CC3D_F32, CC3D_BF16 = 0, 1
CC3D_MAX_KT = 8

_i32 = ctypes.c_int32


class Desc(ctypes.Structure):
    _fields_ = [(name, _i32) for name in (
        "n", "c_in", "c_out", "h", "w", "t_x", "t_cache", "k_t", "k_h", "k_w",
        "s_t", "s_h", "s_w", "d_t", "d_h", "d_w", "p_h", "p_w", "p_base",
        "groups", "has_bias", "dtype")]


class Tap(ctypes.Structure):
    _fields_ = [(name, _i32) for name in ("delta", "o_lo", "o_hi", "src_lo", "src_hi", "active")]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("t_z", _i32), ("p_l", _i32), ("t_out", _i32), ("h_out", _i32), ("w_out", _i32),
        ("t_cache_out", _i32), ("n_active_taps", _i32), ("taps", Tap * CC3D_MAX_KT),
        ("flops_nominal", ctypes.c_double), ("flops_active", ctypes.c_double),
        ("bytes_conv", ctypes.c_double), ("bytes_cache_out", ctypes.c_double),
        ("kernel_id", _i32), ("block_m", _i32), ("block_n", _i32), ("tiles", ctypes.c_int64),
        ("packed_weight_bytes", ctypes.c_int64), ("weight_layout", ctypes.c_uint64),
        ("workspace_bytes", ctypes.c_int64), ("splits", _i32),
        ("kernel_name", ctypes.c_char * 64),
    ]


class Counters(ctypes.Structure):
    _fields_ = [(name, ctypes.c_uint64) for name in ("fast_path", "unsupported", "invalid", "device_error")]


def _load():
    if not os.path.exists(library_path):
        raise ImportError(
            "libcc3d.so is not built (%s); run `python causal_conv3d_video_amd/build.py`" % library_path)
    lib = ctypes.CDLL(library_path)
    vp = ctypes.c_void_p
    lib.causal_conv3d_plan.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(vp)]
    lib.causal_conv3d_plan.restype = ctypes.c_int
    lib.causal_conv3d_plan_variant.argtypes = [ctypes.POINTER(Desc), ctypes.c_char_p, ctypes.POINTER(vp)]
    lib.causal_conv3d_plan_variant.restype = ctypes.c_int
    lib.causal_conv3d_plan_autotune.argtypes = [ctypes.POINTER(Desc)] + [vp] * 5 + [
        ctypes.c_int, vp, ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_float)]
    lib.causal_conv3d_plan_autotune.restype = ctypes.c_int
    lib.causal_conv3d_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.causal_conv3d_plan_info.restype = ctypes.c_int
    lib.causal_conv3d_plan_destroy.argtypes = [vp]
    lib.causal_conv3d_plan_destroy.restype = None
    lib.causal_conv3d_forward.argtypes = [vp] * 8
    lib.causal_conv3d_forward.restype = ctypes.c_int
    lib.causal_conv3d_pack_weights.argtypes = [vp] * 4
    lib.causal_conv3d_pack_weights.restype = ctypes.c_int
    lib.causal_conv3d_forward_packed.argtypes = [vp] * 8 + [ctypes.c_int64, vp]
    lib.causal_conv3d_forward_packed.restype = ctypes.c_int
    lib.causal_conv3d_forward_packed_noalloc.argtypes = [vp] * 8
    lib.causal_conv3d_forward_packed_noalloc.restype = ctypes.c_int
    lib.causal_conv3d_forward_u8.argtypes = [vp] * 7 + [ctypes.c_float, ctypes.c_float, vp]
    lib.causal_conv3d_forward_u8.restype = ctypes.c_int
    lib.causal_conv3d_status_string.argtypes = [ctypes.c_int]
    lib.causal_conv3d_status_string.restype = ctypes.c_char_p
    lib.causal_conv3d_counters.argtypes = [ctypes.POINTER(Counters), ctypes.c_int]
    lib.causal_conv3d_counters.restype = None
    return lib


_lib = _load()


class CC3DError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, causal_conv3d_status_string(status), status))


def causal_conv3d_status_string(status):
    return _lib.causal_conv3d_status_string(int(status)).decode()


def make_desc(n, c_in, c_out, h, w, t_x, t_cache, k=(3, 3, 3), stride=(1, 1, 1),
              dilation=(1, 1, 1), padding=(1, 1), p_base=2, groups=1, has_bias=True,
              dtype=torch.bfloat16):
    """Descriptor of one call.  dtype: torch.bfloat16 or torch.float32."""
    if dtype == torch.bfloat16:
        code = CC3D_BF16
    elif dtype == torch.float32:
        code = CC3D_F32
    else:
        raise TypeError("dtype must be torch.bfloat16 or torch.float32")
    return Desc(n, c_in, c_out, h, w, t_x, t_cache, k[0], k[1], k[2], stride[0], stride[1],
                stride[2], dilation[0], dilation[1], dilation[2], padding[0], padding[1],
                p_base, groups, int(bool(has_bias)), code)


class Plan:
    """Owns a plan handle (host metadata only: a plan holds no device memory)."""

    def __init__(self, handle, desc):
        self.handle = handle
        self.desc = desc
        self.info = causal_conv3d_plan_info(self)

    @property
    def dtype(self):
        return torch.bfloat16 if self.desc.dtype == CC3D_BF16 else torch.float32

    def shapes(self):
        """Physical shapes of x, cache_in, w, b, out, cache_out."""
        d, i = self.desc, self.info
        return {
            "x": (d.n, d.t_x, d.h, d.w, d.c_in),
            "cache_in": (d.n, d.t_cache, d.h, d.w, d.c_in),
            "w": (d.c_out, d.k_t, d.k_h, d.k_w, d.c_in),
            "b": (d.c_out,),
            "out": (d.n, i["t_out"], i["h_out"], i["w_out"], d.c_out),
            "cache_out": (d.n, i["t_cache_out"], d.h, d.w, d.c_in),
        }

    def close(self):
        if self.handle:
            _lib.causal_conv3d_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def causal_conv3d_plan(desc):
    """Validate ``desc`` and build its plan; raises CC3DError on refusal."""
    h = ctypes.c_void_p()
    st = _lib.causal_conv3d_plan(ctypes.byref(desc), ctypes.byref(h))
    if st != CC3D_OK:
        raise CC3DError(st, "causal_conv3d_plan")
    return Plan(h.value, desc)


def causal_conv3d_plan_variant(desc, kernel_name):
    """Plan ``desc`` on the named kernel variant; raises CC3DError if that
    variant cannot run the call."""
    h = ctypes.c_void_p()
    st = _lib.causal_conv3d_plan_variant(ctypes.byref(desc), kernel_name.encode(), ctypes.byref(h))
    if st != CC3D_OK:
        raise CC3DError(st, "causal_conv3d_plan_variant")
    return Plan(h.value, desc)


def causal_conv3d_plan_autotune(desc, x, cache_in, w, b, out, launches=5, stream=None):
    """Time every bf16 variant that can run ``desc`` on these buffers (each
    from its packed weight image) and return (plan of the fastest, its ms per
    call).  Blocking; overwrites ``out``."""
    probe = causal_conv3d_plan(desc)  # validates desc and gives the buffer shapes
    try:
        p = _marshal(probe, {"x": x, "cache_in": cache_in if desc.t_cache > 0 else None, "w": w,
                             "b": b if desc.has_bias else None, "out": out})
    finally:
        probe.close()
    h = ctypes.c_void_p()
    ms = ctypes.c_float()
    st = _lib.causal_conv3d_plan_autotune(ctypes.byref(desc), p["x"], p["cache_in"], p["w"], p["b"], p["out"],
                                          int(launches), _stream_handle(stream, x), ctypes.byref(h),
                                          ctypes.byref(ms))
    if st != CC3D_OK:
        raise CC3DError(st, "causal_conv3d_plan_autotune")
    return Plan(h.value, desc), ms.value


def causal_conv3d_plan_info(plan):
    info = PlanInfo()
    st = _lib.causal_conv3d_plan_info(plan.handle, ctypes.byref(info))
    if st != CC3D_OK:
        raise CC3DError(st, "causal_conv3d_plan_info")
    out = {name: getattr(info, name) for name, _ in PlanInfo._fields_ if name not in ("taps", "kernel_name")}
    out["kernel_name"] = info.kernel_name.decode()
    out["taps"] = [{name: getattr(info.taps[k], name) for name, _ in Tap._fields_} for k in range(plan.desc.k_t)]
    return out


def causal_conv3d_plan_destroy(plan):
    plan.close()


def _physical(t, shape, name):
    """Check that ``t`` stores exactly ``shape`` densely in that order."""
    if t is None:
        return None
    if tuple(t.shape) == tuple(shape) and t.is_contiguous():
        return t
    if t.dim() == len(shape) == 5:
        v = t.permute(0, 2, 3, 4, 1)
        if tuple(v.shape) == tuple(shape) and v.is_contiguous():
            return v
    raise ValueError("%s: expected a dense %s channels-last tensor, got shape %s strides %s"
                     % (name, tuple(shape), tuple(t.shape), tuple(t.stride())))


def _marshal(plan, tensors):
    shapes = plan.shapes()
    ptrs = {}
    for name, t in tensors.items():
        if t is None:
            ptrs[name] = None
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("%s must be a CUDA (HIP) tensor" % name)
        if t.dtype != plan.dtype:
            raise TypeError("%s has dtype %s, the plan expects %s" % (name, t.dtype, plan.dtype))
        _physical(t, shapes[name], name)
        ptrs[name] = t.data_ptr()
    return ptrs


def _stream_handle(stream, like):
    if stream is None:
        stream = torch.cuda.current_stream(like.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def causal_conv3d_forward(plan, x, cache_in, w, b, out, cache_out=None, stream=None):
    """Launch the plan's cached causal Conv3D on ``stream`` (default: the
    current torch stream of x's device).  Asynchronous; raises CC3DError if
    the library refuses the call."""
    p = _marshal(plan, {"x": x, "cache_in": cache_in if plan.desc.t_cache > 0 else None, "w": w,
                        "b": b if plan.desc.has_bias else None, "out": out, "cache_out": cache_out})
    st = _lib.causal_conv3d_forward(plan.handle, p["x"], p["cache_in"], p["w"], p["b"], p["out"],
                                    p["cache_out"], _stream_handle(stream, x))
    if st != CC3D_OK:
        raise CC3DError(st, "causal_conv3d_forward")


def _device_bytes(t, nbytes, name, like):
    """Pointer of a caller-owned device buffer of at least ``nbytes`` bytes."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise TypeError("%s must be a contiguous CUDA (HIP) tensor" % name)
    if t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes, the plan needs %d" % (name, t.numel() * t.element_size(), nbytes))
    if like is not None and t.device != like.device:
        raise ValueError("%s is on %s, the other buffers on %s" % (name, t.device, like.device))
    return t.data_ptr()


def causal_conv3d_pack_weights(plan, w, w_packed=None, stream=None):
    """Write the plan's packed weight image of ``w`` (bf16 plans) into
    ``w_packed`` (a caller-owned CUDA tensor of at least
    plan.info["packed_weight_bytes"] bytes; allocated here as a uint8 tensor
    when None) and return it.  Plans with the same info["weight_layout"]
    read the same image."""
    p = _marshal(plan, {"w": w})
    nbytes = plan.info["packed_weight_bytes"]
    if w_packed is None:
        w_packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)
    dst = _device_bytes(w_packed, nbytes, "w_packed", w)
    st = _lib.causal_conv3d_pack_weights(plan.handle, p["w"], dst, _stream_handle(stream, w))
    if st != CC3D_OK:
        raise CC3DError(st, "causal_conv3d_pack_weights")
    return w_packed


def causal_conv3d_forward_packed(plan, x, cache_in, w_packed, b, out, cache_out=None, workspace=None, stream=None):
    """The convolution from a packed weight image (causal_conv3d_pack_weights).
    ``workspace``: a CUDA tensor of at least plan.info["workspace_bytes"]
    bytes, zero-filled before its first use (None when that is 0)."""
    p = _marshal(plan, {"x": x, "cache_in": cache_in if plan.desc.t_cache > 0 else None,
                        "b": b if plan.desc.has_bias else None, "out": out, "cache_out": cache_out})
    wp = _device_bytes(w_packed, plan.info["packed_weight_bytes"], "w_packed", x)
    ws_bytes = plan.info["workspace_bytes"]
    ws = None
    if workspace is not None:
        ws = _device_bytes(workspace, ws_bytes, "workspace", x)
        ws_bytes = workspace.numel() * workspace.element_size()
    elif ws_bytes > 0:
        raise ValueError("this plan needs a workspace of %d bytes" % ws_bytes)
    st = _lib.causal_conv3d_forward_packed(plan.handle, p["x"], p["cache_in"], wp, p["b"], p["out"],
                                           p["cache_out"], ws, int(ws_bytes if ws else 0), _stream_handle(stream, x))
    if st != CC3D_OK:
        raise CC3DError(st, "causal_conv3d_forward_packed")


NOALLOC_SCRATCH_BYTES = 64 << 20   # CC3D_NOALLOC_SCRATCH_BYTES


def causal_conv3d_forward_packed_noalloc(plan, x, cache_in, w_packed, b, out, cache_out=None, stream=None):
    """causal_conv3d_forward_packed with the split workspace in the
    library's static per-device array: allocates no device memory.  Calls
    that overlap on one device race."""
    p = _marshal(plan, {"x": x, "cache_in": cache_in if plan.desc.t_cache > 0 else None,
                        "b": b if plan.desc.has_bias else None, "out": out, "cache_out": cache_out})
    wp = _device_bytes(w_packed, plan.info["packed_weight_bytes"], "w_packed", x)
    st = _lib.causal_conv3d_forward_packed_noalloc(plan.handle, p["x"], p["cache_in"], wp, p["b"], p["out"],
                                                   p["cache_out"], _stream_handle(stream, x))
    if st != CC3D_OK:
        raise CC3DError(st, "causal_conv3d_forward_packed_noalloc")


def causal_conv3d_forward_u8(plan, x, cache_in, w, b, out, cache_out=None, scale=0.5, offset=0.5, stream=None):
    """The RGB head with 8-bit pixel output: ``out`` is a uint8 CUDA tensor of
    the plan's output shape, code = trunc(clamp(fma(y, scale, offset) * 255,
    0, 255)) in fp32."""
    if not isinstance(out, torch.Tensor) or not out.is_cuda or out.dtype != torch.uint8:
        raise TypeError("out must be a uint8 CUDA (HIP) tensor")
    _physical(out, plan.shapes()["out"], "out")
    p = _marshal(plan, {"x": x, "cache_in": cache_in if plan.desc.t_cache > 0 else None, "w": w,
                        "b": b if plan.desc.has_bias else None, "cache_out": cache_out})
    st = _lib.causal_conv3d_forward_u8(plan.handle, p["x"], p["cache_in"], p["w"], p["b"], out.data_ptr(),
                                       p["cache_out"], float(scale), float(offset), _stream_handle(stream, x))
    if st != CC3D_OK:
        raise CC3DError(st, "causal_conv3d_forward_u8")


def causal_conv3d_counters(reset=False):
    c = Counters()
    _lib.causal_conv3d_counters(ctypes.byref(c), int(bool(reset)))
    return {name: getattr(c, name) for name, _ in Counters._fields_}
