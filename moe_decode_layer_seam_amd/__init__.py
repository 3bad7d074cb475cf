"""MI355X (gfx950) small-batch decode MoE FFN: Python binding of the C ABI.

Argument marshalling only -- every step of the layer runs in the HIP kernels
of ``libmoe_decode.so`` (declared in ``include/moe_decode.h``).  The functions
keep the C names without the ``moe_decode_`` prefix: ``plan``,
``scratch_bytes``, ``run``, ``run_noalloc``, ``inspect``, ``status``,
``timing``, ``timing_read``, ``timeline``, ``timeline_read``, ``destroy``,
``quantize_weight``, ``quantize_weight_fp4``, ``hc_fold``, ``attn_x8``,
``read_probe``, ``strerror``, ``last_hip_error`` (``run_ptrs`` and
``inspect_tensor`` are thin variants of ``run`` and ``inspect``).  Tensors are
torch tensors on the GPU (torch supplies device memory and streams); shapes,
dtypes and contiguity are checked here before the pointers cross the
boundary, because the kernels' loads are unchecked.

There is no fallback: if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime first, so the library shares it

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree library; MOE_DECODE_LIBRARY names another build of it instead
LIB_PATH = os.environ.get("MOE_DECODE_LIBRARY") or os.path.join(_PKG, "libmoe_decode.so")

OK, EINVAL, ENOMEM, EHIP, ECAPTURE = 0, -1, -2, -3, -4
MAX_TOKENS = 48

TAPS = {"normed": 0, "x8": 1, "x8s": 2, "logits": 3, "topk_ids": 4, "topk_w": 5,
        "counts": 6, "pair_row": 7, "row_tok": 8, "a8": 9, "a8s": 10, "status": 11}
KERNELS = {"seam": 0, "logits": 1, "route": 2, "w13": 3, "act": 4, "w2": 5, "combine": 6,
           "persistent": 7}


# routed expert weight formats (moe_decode.h MOE_DECODE_ROUTED_*)
ROUTED = {"e4m3": 0, "mxfp4": 1}
# schedules (MOE_DECODE_SCHEDULE_*): the fastest (today the short launches),
# the short launches always, or the persistent launch where it covers a step
SCHEDULES = {"auto": 0, "launches": 1, "persistent": 2}


class Dims(ctypes.Structure):
    """moe_decode_dims."""
    _fields_ = [("hidden", ctypes.c_int32), ("experts", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("routed_scale", ctypes.c_float),
                ("routed_format", ctypes.c_int32), ("schedule", ctypes.c_int32)]


class MoeDecodeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first "
                "(python -m moe_decode_layer_seam_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_decode_plan.argtypes = [ctypes.POINTER(Dims), _P, ctypes.POINTER(_P)]
        L.moe_decode_plan.restype = ctypes.c_int
        L.moe_decode_scratch_bytes.argtypes = [_P]
        L.moe_decode_scratch_bytes.restype = ctypes.c_size_t
        L.moe_decode_run.argtypes = [_P, ctypes.c_int32] + [_P] * 14
        L.moe_decode_run.restype = ctypes.c_int
        L.moe_decode_run_noalloc.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32] + [_P] * 15
        L.moe_decode_run_noalloc.restype = ctypes.c_int
        L.moe_decode_inspect.argtypes = [_P, ctypes.c_int32, ctypes.POINTER(_P),
                                         ctypes.POINTER(ctypes.c_size_t)]
        L.moe_decode_inspect.restype = ctypes.c_int
        L.moe_decode_status.argtypes = [_P, _P, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32]
        L.moe_decode_status.restype = ctypes.c_int
        L.moe_decode_timing.argtypes = [_P, ctypes.c_int32]
        L.moe_decode_timing.restype = ctypes.c_int
        L.moe_decode_timing_read.argtypes = [_P, ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                                             ctypes.POINTER(ctypes.c_int32)]
        L.moe_decode_timing_read.restype = ctypes.c_int
        L.moe_decode_timeline.argtypes = [_P, ctypes.c_int32]
        L.moe_decode_timeline.restype = ctypes.c_int
        L.moe_decode_timeline_read.argtypes = [_P, ctypes.c_int32, _P, ctypes.c_size_t,
                                               ctypes.POINTER(ctypes.c_int32)]
        L.moe_decode_timeline_read.restype = ctypes.c_int
        L.moe_decode_destroy.argtypes = [_P]
        L.moe_decode_destroy.restype = None
        L.moe_decode_quantize_weight.argtypes = [_P, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, _P, _P, _P]
        L.moe_decode_quantize_weight.restype = ctypes.c_int
        L.moe_decode_quantize_weight_fp4.argtypes = [_P, ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int32, _P, _P, _P]
        L.moe_decode_quantize_weight_fp4.restype = ctypes.c_int
        L.moe_decode_hc_fold.argtypes = [ctypes.c_int32, ctypes.c_int32] + [_P] * 8
        L.moe_decode_hc_fold.restype = ctypes.c_int
        L.moe_decode_attn_x8.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_float, _P, _P, _P]
        L.moe_decode_attn_x8.restype = ctypes.c_int
        L.moe_decode_read_probe.argtypes = [_P, ctypes.c_size_t, _P, _P]
        L.moe_decode_read_probe.restype = ctypes.c_int
        L.moe_decode_strerror.argtypes = [ctypes.c_int]
        L.moe_decode_strerror.restype = ctypes.c_char_p
        L.moe_decode_last_hip_error.argtypes = [_P]
        L.moe_decode_last_hip_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


EXPORTS = ("moe_decode_plan", "moe_decode_scratch_bytes", "moe_decode_run", "moe_decode_run_noalloc",
           "moe_decode_inspect", "moe_decode_status", "moe_decode_timing", "moe_decode_timing_read",
           "moe_decode_timeline", "moe_decode_timeline_read",
           "moe_decode_destroy", "moe_decode_quantize_weight",
           "moe_decode_quantize_weight_fp4", "moe_decode_hc_fold", "moe_decode_attn_x8",
           "moe_decode_read_probe", "moe_decode_strerror", "moe_decode_last_hip_error")

PROBE_BLOCKS = 4096  # MOE_DECODE_PROBE_BLOCKS


def strerror(code: int) -> str:
    return lib().moe_decode_strerror(code).decode()


def last_hip_error(handle=None) -> str:
    return lib().moe_decode_last_hip_error(handle).decode()


def _stream_ptr(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int, what: str, handle=None) -> None:
    if rc != OK:
        detail = last_hip_error(handle)
        raise MoeDecodeError(rc, f"{what} [{detail}]")


# ---- the C ABI, marshalled -------------------------------------------------

def plan(hidden: int, experts: int, topk: int, inter: int, shared_inter: int,
         max_tokens: int = MAX_TOKENS, rms_eps: float = 1e-6,
         routed_scale: float = 1.0, stream=None, routed: str = "e4m3",
         schedule: str = "auto") -> int:
    """moe_decode_plan: returns an opaque handle (int).  routed: the routed
    experts' weight format, "e4m3" or "mxfp4"; schedule: "auto" (the
    fastest: today the short launches), "launches" (the short launches) or
    "persistent" (the persistent launch for the small steps it covers, the
    short launches otherwise)."""
    d = Dims(hidden, experts, topk, inter, shared_inter, max_tokens, rms_eps, routed_scale,
             ROUTED[routed], SCHEDULES[schedule])
    h = _P()
    _check(lib().moe_decode_plan(ctypes.byref(d), _stream_ptr(stream), ctypes.byref(h)),
           "moe_decode_plan")
    return h.value


def scratch_bytes(handle: int) -> int:
    return lib().moe_decode_scratch_bytes(handle)


def _tensor(t: torch.Tensor, name: str, shape, dtype) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: {tuple(t.shape)} {t.dtype} contiguous={t.is_contiguous()} "
                         f"cuda={t.is_cuda}, want {tuple(shape)} {dtype} contiguous on the GPU")
    return t.data_ptr()


def run(handle: int, dims: dict, x, norm_w, gate_w, bias, w13, w13_s, w2, w2_s,
        sgu, sgu_s, sw2, sw2_s, out, stream=None) -> None:
    """moe_decode_run on torch tensors.  dims: hidden, experts, topk, inter,
    shared_inter and routed ("e4m3", the default, or "mxfp4") -- the plan's.
    E4M3 tensors may be torch.float8_e4m3fn or uint8; E2M1 pairs and scales
    uint8."""
    H, E, I, Is = dims["hidden"], dims["experts"], dims["inter"], dims["shared_inter"]
    fp4 = dims.get("routed", "e4m3") == "mxfp4"
    m = x.shape[0]

    def q(t, name, shape):
        dt = torch.float8_e4m3fn if t.dtype == torch.float8_e4m3fn else torch.uint8
        return _tensor(t, name, shape, dt)

    ptrs = [
        _tensor(x, "x", (m, H), torch.bfloat16),
        _tensor(norm_w, "norm_w", (H,), torch.bfloat16),
        _tensor(gate_w, "gate_w", (E, H), torch.bfloat16),
        _tensor(bias, "bias", (E,), torch.float32),
        *((_tensor(w13, "w13", (E, 2 * I, H // 2), torch.uint8),
           _tensor(w13_s, "w13_s", (E,) + fp4_codes_shape(2 * I, H), torch.uint8),
           _tensor(w2, "w2", (E, H, I // 2), torch.uint8),
           _tensor(w2_s, "w2_s", (E,) + fp4_codes_shape(H, I), torch.uint8)) if fp4 else
          (q(w13, "w13", (E, 2 * I, H)), _tensor(w13_s, "w13_s", (E, 2 * I // 32, H // 32), torch.uint8),
           q(w2, "w2", (E, H, I)), _tensor(w2_s, "w2_s", (E, H // 32, I // 32), torch.uint8))),
        q(sgu, "sgu", (2 * Is, H)), _tensor(sgu_s, "sgu_s", (2 * Is // 32, H // 32), torch.uint8),
        q(sw2, "sw2", (H, Is)), _tensor(sw2_s, "sw2_s", (H // 32, Is // 32), torch.uint8),
        _tensor(out, "out", (m, H), torch.bfloat16),
    ]
    rc = lib().moe_decode_run(handle, m, *ptrs, _stream_ptr(stream))
    _check(rc, "moe_decode_run", handle)


def run_noalloc(dims: dict, x, norm_w, gate_w, bias, w13, w13_s, w2, w2_s, sgu, sgu_s, sw2, sw2_s,
                out, status, max_tokens: int = MAX_TOKENS, rms_eps: float = 1e-6,
                routed_scale: float = 1.0, schedule: str = "auto", stream=None) -> None:
    """moe_decode_run_noalloc: the step without a plan or any allocation.
    dims as for `run` (plus the layer's hidden..shared_inter); status an
    int32 (or uint32) tensor of one element on the GPU, which the kernels'
    status bits are ORed into (the caller zeroes it)."""
    H, E, K, I, Is = dims["hidden"], dims["experts"], dims["topk"], dims["inter"], dims["shared_inter"]
    routed = dims.get("routed", "e4m3")
    fp4 = routed == "mxfp4"
    m = x.shape[0]
    d = Dims(H, E, K, I, Is, max_tokens, rms_eps, routed_scale, ROUTED[routed], SCHEDULES[schedule])

    def q(t, name, shape):
        dt = torch.float8_e4m3fn if t.dtype == torch.float8_e4m3fn else torch.uint8
        return _tensor(t, name, shape, dt)

    ptrs = [
        _tensor(x, "x", (m, H), torch.bfloat16),
        _tensor(norm_w, "norm_w", (H,), torch.bfloat16),
        _tensor(gate_w, "gate_w", (E, H), torch.bfloat16),
        _tensor(bias, "bias", (E,), torch.float32),
        *((_tensor(w13, "w13", (E, 2 * I, H // 2), torch.uint8),
           _tensor(w13_s, "w13_s", (E,) + fp4_codes_shape(2 * I, H), torch.uint8),
           _tensor(w2, "w2", (E, H, I // 2), torch.uint8),
           _tensor(w2_s, "w2_s", (E,) + fp4_codes_shape(H, I), torch.uint8)) if fp4 else
          (q(w13, "w13", (E, 2 * I, H)), _tensor(w13_s, "w13_s", (E, 2 * I // 32, H // 32), torch.uint8),
           q(w2, "w2", (E, H, I)), _tensor(w2_s, "w2_s", (E, H // 32, I // 32), torch.uint8))),
        q(sgu, "sgu", (2 * Is, H)), _tensor(sgu_s, "sgu_s", (2 * Is // 32, H // 32), torch.uint8),
        q(sw2, "sw2", (H, Is)), _tensor(sw2_s, "sw2_s", (H // 32, Is // 32), torch.uint8),
        _tensor(out, "out", (m, H), torch.bfloat16),
    ]
    st = _tensor(status, "status", (1,), status.dtype)
    rc = lib().moe_decode_run_noalloc(ctypes.byref(d), m, *ptrs, st, _stream_ptr(stream))
    _check(rc, "moe_decode_run_noalloc")


def run_ptrs(handle: int, m: int, ptrs, stream=None) -> int:
    """moe_decode_run on raw device pointers (13 of them, in C order); returns
    the C return code without raising (for boundary tests)."""
    return lib().moe_decode_run(handle, m, *ptrs, _stream_ptr(stream))


def inspect(handle: int, tap: str):
    """moe_decode_inspect: (device pointer, bytes) of an intermediate."""
    p = _P()
    n = ctypes.c_size_t()
    _check(lib().moe_decode_inspect(handle, TAPS[tap], ctypes.byref(p), ctypes.byref(n)),
           "moe_decode_inspect", handle)
    return p.value, n.value


def status(handle: int, clear: bool = True, stream=None) -> int:
    """moe_decode_status: the plan's sticky status word (0: every run since
    the last clear was valid); synchronises the stream, and by default
    clears the word."""
    v = ctypes.c_uint32()
    _check(lib().moe_decode_status(handle, _stream_ptr(stream), ctypes.byref(v), 1 if clear else 0),
           "moe_decode_status", handle)
    return v.value


def inspect_tensor(handle: int, tap: str, dtype=torch.uint8) -> torch.Tensor:
    """A copy of an intermediate as a flat torch tensor of ``dtype`` on the
    current device (after the run's stream has been synchronised)."""
    ptr, nbytes = inspect(handle, tap)
    out = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    err = _hip().hipMemcpy(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ptr),
                           ctypes.c_size_t(nbytes), 3)  # hipMemcpyDeviceToDevice
    if err != 0:
        raise RuntimeError(f"device copy of {tap} failed ({err})")
    return out.view(dtype)


_hip_rt = None


def _hip() -> ctypes.CDLL:
    """The HIP runtime torch already loaded (same soname, same instance)."""
    global _hip_rt
    if _hip_rt is None:
        _hip_rt = ctypes.CDLL("libamdhip64.so.7")
        _hip_rt.hipMemcpy.restype = ctypes.c_int
    return _hip_rt


def timing(handle: int, on: bool) -> None:
    _check(lib().moe_decode_timing(handle, 1 if on else 0), "moe_decode_timing", handle)


def timing_read(handle: int, kernel: str) -> tuple[float, int]:
    ms = ctypes.c_double()
    runs = ctypes.c_int32()
    _check(lib().moe_decode_timing_read(handle, KERNELS[kernel], ctypes.byref(ms), ctypes.byref(runs)),
           "moe_decode_timing_read", handle)
    return ms.value, runs.value


def timeline(handle: int, on: bool) -> None:
    _check(lib().moe_decode_timeline(handle, 1 if on else 0), "moe_decode_timeline", handle)


def timeline_read(handle: int, kernel: str):
    """The last run's stamps of one kernel: uint64 [blocks, 8] (100 MHz clock)."""
    import numpy as np
    buf = np.zeros(1024 * 8, np.uint64)
    nb = ctypes.c_int32()
    _check(lib().moe_decode_timeline_read(handle, KERNELS[kernel], buf.ctypes.data, buf.size,
                                          ctypes.byref(nb)), "moe_decode_timeline_read", handle)
    return buf[: nb.value * 8].reshape(nb.value, 8)


def destroy(handle: int) -> None:
    lib().moe_decode_destroy(handle)


def hc_fold(part: torch.Tensor, residual: torch.Tensor, post: torch.Tensor, res: torch.Tensor,
            pre: torch.Tensor, residual_out: torch.Tensor = None, x: torch.Tensor = None, stream=None):
    """moe_decode_hc_fold: part bf16 [m, H], residual bf16 [m, 4, H], post f32
    [m, 4] (or [m, 4, 1]), res f32 [m, 4, 4], pre f32 [m, 4] -> (residual_out
    [m, 4, H], x [m, H]) bf16.  residual_out may be residual (in place)."""
    m, H = part.shape
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    if x is None:
        x = torch.empty_like(part)
    ptrs = [_tensor(part, "part", (m, H), torch.bfloat16),
            _tensor(residual, "residual", (m, 4, H), torch.bfloat16),
            _tensor(post.reshape(m, 4) if post.dim() == 3 else post, "post", (m, 4), torch.float32),
            _tensor(res, "res", (m, 4, 4), torch.float32),
            _tensor(pre, "pre", (m, 4), torch.float32),
            _tensor(residual_out, "residual_out", (m, 4, H), torch.bfloat16),
            _tensor(x, "x", (m, H), torch.bfloat16)]
    _check(lib().moe_decode_hc_fold(m, H, *ptrs, _stream_ptr(stream)), "moe_decode_hc_fold")
    return residual_out, x


def attn_x8(x: torch.Tensor, norm_w: torch.Tensor, rms_eps: float = 1e-6, x8: torch.Tensor = None,
            x8s: torch.Tensor = None, stream=None):
    """moe_decode_attn_x8: x bf16 [m, H], norm_w bf16 [H] -> (x8 uint8 [m, H]
    E4M3, x8s uint8 [m, H/32] E8M0)."""
    m, H = x.shape
    if x8 is None:
        x8 = torch.empty((m, H), dtype=torch.uint8, device=x.device)
    if x8s is None:
        x8s = torch.empty((m, H // 32), dtype=torch.uint8, device=x.device)
    ptrs = [_tensor(x, "x", (m, H), torch.bfloat16), _tensor(norm_w, "norm_w", (H,), torch.bfloat16)]
    _check(lib().moe_decode_attn_x8(m, H, *ptrs, rms_eps,
                                    _tensor(x8, "x8", (m, H), torch.uint8),
                                    _tensor(x8s, "x8s", (m, H // 32), torch.uint8), _stream_ptr(stream)),
           "moe_decode_attn_x8")
    return x8, x8s


def read_probe(buf: torch.Tensor, sink: torch.Tensor = None, stream=None) -> torch.Tensor:
    """moe_decode_read_probe: one streaming read of the bytes of buf (uint8,
    contiguous, a multiple of 16 bytes).  Returns sink, int32 [PROBE_BLOCKS]:
    the XOR of the 32-bit words each block read."""
    if sink is None:
        sink = torch.empty(PROBE_BLOCKS, dtype=torch.int32, device=buf.device)
    n = buf.numel()
    _check(lib().moe_decode_read_probe(_tensor(buf, "buf", (n,), torch.uint8), n,
                                       _tensor(sink, "sink", (PROBE_BLOCKS,), torch.int32),
                                       _stream_ptr(stream)), "moe_decode_read_probe")
    return sink


def fp4_codes_shape(rows: int, cols: int) -> tuple:
    """Shape of the E8M0 code array of one MXFP4 [rows, cols] matrix: blocked
    [rows/16, ceil(cols/512), 16, 16] (16-row tile, 512-column segment, row,
    32-column block)."""
    return (rows // 16, (cols + 511) // 512, 16, 16)


def quantize_weight_fp4(w: torch.Tensor, q: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """moe_decode_quantize_weight_fp4: fp32 [..., rows, cols] -> E2M1 pairs q
    (uint8 [..., rows, cols/2]) and blocked E8M0 codes (uint8 [...,
    *fp4_codes_shape(rows, cols)])."""
    rows, cols = w.shape[-2], w.shape[-1]
    count = w.numel() // (rows * cols)
    if w.dtype != torch.float32 or not w.is_contiguous() or not w.is_cuda:
        raise ValueError("w: contiguous float32 on the GPU required")
    if tuple(q.shape) != tuple(w.shape[:-1]) + (cols // 2,) or q.dtype != torch.uint8 or not q.is_contiguous():
        raise ValueError("q: uint8 [..., rows, cols/2]")
    if (tuple(scales.shape) != tuple(w.shape[:-2]) + fp4_codes_shape(rows, cols) or scales.dtype != torch.uint8
            or not scales.is_contiguous()):
        raise ValueError("scales: uint8 [..., rows/16, ceil(cols/512), 16, 16]")
    rc = lib().moe_decode_quantize_weight_fp4(w.data_ptr(), count, rows, cols, q.data_ptr(),
                                              scales.data_ptr(), _stream_ptr(stream))
    _check(rc, "moe_decode_quantize_weight_fp4")


def quantize_weight(w: torch.Tensor, q: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """moe_decode_quantize_weight: fp32 [..., rows, cols] -> E4M3 bytes q (same
    shape, uint8 or float8_e4m3fn) and E8M0 scales [..., rows/32, cols/32]."""
    rows, cols = w.shape[-2], w.shape[-1]
    count = w.numel() // (rows * cols)
    if w.dtype != torch.float32 or not w.is_contiguous() or not w.is_cuda:
        raise ValueError("w: contiguous float32 on the GPU required")
    if q.shape != w.shape or q.element_size() != 1 or not q.is_contiguous():
        raise ValueError("q: one byte per element, same shape as w")
    if tuple(scales.shape) != tuple(w.shape[:-2]) + (rows // 32, cols // 32) or scales.dtype != torch.uint8:
        raise ValueError("scales: uint8 [..., rows/32, cols/32]")
    rc = lib().moe_decode_quantize_weight(w.data_ptr(), count, rows, cols, q.data_ptr(),
                                          scales.data_ptr(), _stream_ptr(stream))
    _check(rc, "moe_decode_quantize_weight")
