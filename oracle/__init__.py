"""ctypes binding of the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the checker of the HIP path.  Only the tests, the
package smoke check and the benchmark's CPU-baseline leg may import this
module.  It never receives anything the HIP path computed.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

_P = ctypes.c_void_p
_I = ctypes.c_int32


# routed expert weight formats (the shared expert is always E4M3)
FMT_E4M3, FMT_MXFP4 = 0, 1
FORMATS = {"e4m3": FMT_E4M3, "mxfp4": FMT_MXFP4}


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("experts", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("routed_scale", ctypes.c_float), ("routed_format", ctypes.c_int32)]


def build() -> str:
    """Compile the oracle with gcc (no fused multiply-adds); returns the path."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-o", _SO, os.path.join(_HERE, "moe_oracle.c"), "-lm"]
    subprocess.check_call(cmd)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_rne.argtypes = [ctypes.c_double]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_rne.argtypes = [ctypes.c_double]
        L.orc_e4m3_rne.restype = ctypes.c_uint8
        L.orc_mx_code.argtypes = [ctypes.c_double]
        L.orc_mx_code.restype = _I
        L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_rne.argtypes = [ctypes.c_double]
        L.orc_e2m1_rne.restype = ctypes.c_uint8
        L.orc_fp4_code.argtypes = [ctypes.c_double]
        L.orc_fp4_code.restype = _I
        for f in ("orc_e4m3_rne_array", "orc_mx_code_array", "orc_bf16_rne_array",
                  "orc_e2m1_rne_array"):
            getattr(L, f).argtypes = [ctypes.c_int64, _P, _P]
            getattr(L, f).restype = None
        L.orc_mx_quant_row.argtypes = [_I, _P, _P, _P]
        L.orc_quant_weight.argtypes = [_I, _I, _P, _P, _P]
        L.orc_quant_weight_fp4.argtypes = [_I, _I, _P, _P, _P]
        L.orc_fp4_code_index.argtypes = [_I, _I, _I]
        L.orc_fp4_code_index.restype = ctypes.c_size_t
        L.orc_expert_fmt.argtypes = [_I, _I, _I] + [_P] * 9
        L.orc_expert_up.argtypes = [_I, _I, _I] + [_P] * 9
        L.orc_expert_down.argtypes = [_I, _I, _I] + [_P] * 5
        L.orc_combine.argtypes = [_I, _I] + [_P] * 5
        L.orc_rmsnorm.argtypes = [_I, _I, _P, _P, ctypes.c_float, _P]
        L.orc_hc_fold.argtypes = [_I, _I] + [_P] * 7
        L.orc_vllm_mx_code.argtypes = [ctypes.c_double]
        L.orc_vllm_mx_code.restype = _I
        L.orc_attn_x8.argtypes = [_I, _I, _P, _P, ctypes.c_float, _P, _P]
        L.orc_router.argtypes = [_I, _I, _I, _I, _P, _P, _P, ctypes.c_float,
                                 _P, _P, _P, _P]
        L.orc_plan.argtypes = [_I, _I, _I, _P, _P, _P]
        L.orc_expert.argtypes = [_I, _I] + [_P] * 9
        L.orc_layer.argtypes = [ctypes.POINTER(Dims), _I] + [_P] * 20
        L.orc_layer.restype = _I
        for f in ("orc_mx_quant_row", "orc_quant_weight", "orc_quant_weight_fp4",
                  "orc_rmsnorm", "orc_router", "orc_plan", "orc_expert", "orc_expert_fmt",
                  "orc_expert_up", "orc_expert_down", "orc_combine",
                  "orc_hc_fold", "orc_attn_x8"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- scalar formats ------------------------------------------------------

def bf16_value(b: int) -> float:
    return lib().orc_bf16_value(b)


def e4m3_value(b: int) -> float:
    return lib().orc_e4m3_value(b)


def e4m3_rne(v: float) -> int:
    return lib().orc_e4m3_rne(v)


def mx_code(amax: float) -> int:
    return lib().orc_mx_code(amax)


def e2m1_value(nibble: int) -> float:
    return lib().orc_e2m1_value(nibble)


def e2m1_rne(v: float) -> int:
    return lib().orc_e2m1_rne(v)


def fp4_code(amax: float) -> int:
    return lib().orc_fp4_code(amax)


def e2m1_rne_array(v) -> np.ndarray:
    v = _c(v, np.float64).ravel()
    out = np.empty(v.size, np.uint8)
    lib().orc_e2m1_rne_array(v.size, _p(v), _p(out))
    return out


def e4m3_rne_array(v) -> np.ndarray:
    v = _c(v, np.float64).ravel()
    out = np.empty(v.size, np.uint8)
    lib().orc_e4m3_rne_array(v.size, _p(v), _p(out))
    return out


def mx_code_array(amax) -> np.ndarray:
    a = _c(amax, np.float64).ravel()
    out = np.empty(a.size, np.int32)
    lib().orc_mx_code_array(a.size, _p(a), _p(out))
    return out


def bf16_rne_array(v) -> np.ndarray:
    v = _c(v, np.float64).ravel()
    out = np.empty(v.size, np.uint16)
    lib().orc_bf16_rne_array(v.size, _p(v), _p(out))
    return out


# ---- quantisers ----------------------------------------------------------

def mx_quant_row(v) -> tuple[np.ndarray, np.ndarray]:
    v = _c(v, np.float64).ravel()
    q = np.empty(v.size, np.uint8)
    c = np.empty(v.size // 32, np.uint8)
    lib().orc_mx_quant_row(v.size, _p(v), _p(q), _p(c))
    return q, c


def quant_weight(w) -> tuple[np.ndarray, np.ndarray]:
    """fp32 [rows, cols] -> (E4M3 [rows, cols] u8, E8M0 [rows/32, cols/32] u8)."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows // 32, cols // 32), np.uint8)
    lib().orc_quant_weight(rows, cols, _p(w), _p(q), _p(s))
    return q, s


def quant_weight_into(w, q_out: np.ndarray, s_out: np.ndarray) -> None:
    """Same as quant_weight, writing into caller-owned contiguous views."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    assert q_out.flags.c_contiguous and s_out.flags.c_contiguous
    assert q_out.shape == (rows, cols) and s_out.shape == (rows // 32, cols // 32)
    lib().orc_quant_weight(rows, cols, _p(w), _p(q_out), _p(s_out))


def fp4_codes_shape(rows: int, cols: int) -> tuple:
    """Shape of an MXFP4 matrix's blocked code array."""
    return (rows // 16, (cols + 511) // 512, 16, 16)


def fp4_code_index(cols: int, r: int, b: int) -> int:
    return lib().orc_fp4_code_index(cols, r, b)


def quant_weight_fp4(w) -> tuple[np.ndarray, np.ndarray]:
    """fp32 [rows, cols] -> (E2M1 pairs [rows, cols/2] u8, blocked E8M0 codes
    [rows/16, ceil(cols/512), 16, 16] u8)."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols // 2), np.uint8)
    s = np.empty(fp4_codes_shape(rows, cols), np.uint8)
    lib().orc_quant_weight_fp4(rows, cols, _p(w), _p(q), _p(s))
    return q, s


def quant_weight_fp4_into(w, q_out: np.ndarray, s_out: np.ndarray) -> None:
    w = _c(w, np.float32)
    rows, cols = w.shape
    assert q_out.flags.c_contiguous and s_out.flags.c_contiguous
    assert q_out.shape == (rows, cols // 2) and s_out.shape == fp4_codes_shape(rows, cols)
    lib().orc_quant_weight_fp4(rows, cols, _p(w), _p(q_out), _p(s_out))


# ---- layer steps ---------------------------------------------------------

def hc_fold(part, residual, post, res, pre) -> tuple[np.ndarray, np.ndarray]:
    """The hyper-connection residual fold: part bf16 bits [m, H], residual
    [m, 4, H], post [m, 4], res [m, 4, 4], pre [m, 4] -> (residual_out
    [m, 4, H], x [m, H]) bf16 bits."""
    part = _c(part, np.uint16)
    residual = _c(residual, np.uint16)
    post, res, pre = _c(post, np.float32), _c(res, np.float32), _c(pre, np.float32)
    m, h = part.shape
    assert residual.shape == (m, 4, h) and post.shape == (m, 4) and res.shape == (m, 4, 4) and pre.shape == (m, 4)
    ro = np.empty((m, 4, h), np.uint16)
    x = np.empty((m, h), np.uint16)
    lib().orc_hc_fold(m, h, _p(part), _p(residual), _p(post), _p(res), _p(pre), _p(ro), _p(x))
    return ro, x


def vllm_mx_code(amax: float) -> int:
    return lib().orc_vllm_mx_code(amax)


def attn_x8(x, w, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """The attention seam's norm + MXFP8: x bf16 bits [m, H], w [H] ->
    (x8 [m, H], x8s [m, H/32])."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    m, h = x.shape
    x8 = np.empty((m, h), np.uint8)
    x8s = np.empty((m, h // 32), np.uint8)
    lib().orc_attn_x8(m, h, _p(x), _p(w), eps, _p(x8), _p(x8s))
    return x8, x8s


def rmsnorm(x, w, eps: float) -> np.ndarray:
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    m, h = x.shape
    y = np.empty((m, h), np.uint16)
    lib().orc_rmsnorm(m, h, _p(x), _p(w), eps, _p(y))
    return y


def router(y, gate_w, bias, k: int, routed_scale: float = 1.0) -> dict:
    y = _c(y, np.uint16)
    g = _c(gate_w, np.uint16)
    b = _c(bias, np.float32)
    m, h = y.shape
    e = g.shape[0]
    logits = np.empty((m, e), np.float64)
    ids = np.empty((m, k), np.int32)
    wts = np.empty((m, k), np.float64)
    margin = np.empty(m, np.float64)
    lib().orc_router(m, h, e, k, _p(y), _p(g), _p(b), routed_scale,
                     _p(logits), _p(ids), _p(wts), _p(margin))
    return {"logits": logits, "ids": ids, "wts": wts, "margin": margin}


def plan(ids, experts: int) -> tuple[np.ndarray, np.ndarray]:
    ids = _c(ids, np.int32)
    m, k = ids.shape
    counts = np.empty(experts, np.int32)
    row = np.empty((m, k), np.int32)
    lib().orc_plan(m, experts, k, _p(ids), _p(counts), _p(row))
    return counts, row


def expert(x8, x8s, w13, w13_s, w2, w2_s, fmt: str = "e4m3") -> dict:
    """One token through one expert whose weights are in format fmt ("e4m3"
    or "mxfp4"): returns y [H] (f64), a8 [I], a8s [I/32]."""
    x8 = _c(x8, np.uint8).ravel()
    x8s = _c(x8s, np.uint8).ravel()
    w13 = _c(w13, np.uint8)
    w13_s = _c(w13_s, np.uint8)
    w2 = _c(w2, np.uint8)
    w2_s = _c(w2_s, np.uint8)
    h = x8.size
    inter = w13.shape[0] // 2
    y = np.empty(h, np.float64)
    a8 = np.empty(inter, np.uint8)
    a8s = np.empty(inter // 32, np.uint8)
    lib().orc_expert_fmt(h, inter, FORMATS[fmt], _p(x8), _p(x8s), _p(w13), _p(w13_s),
                         _p(w2), _p(w2_s), _p(y), _p(a8), _p(a8s))
    return {"y": y, "a8": a8, "a8s": a8s}


def expert_up(x8, x8s, w13, w13_s, fmt: str = "e4m3") -> dict:
    """The up half of one expert for one token: h [2I] (double), habs [2I]
    (sums of |x_k w_nk|), a [I] (fp32 SiLU(g) u, as double), a8 [I], a8s
    [I/32]."""
    x8 = _c(x8, np.uint8).ravel()
    x8s = _c(x8s, np.uint8).ravel()
    w13 = _c(w13, np.uint8)
    w13_s = _c(w13_s, np.uint8)
    h = x8.size
    inter = w13.shape[0] // 2
    hv = np.empty(2 * inter, np.float64)
    habs = np.empty(2 * inter, np.float64)
    av = np.empty(inter, np.float64)
    a8 = np.empty(inter, np.uint8)
    a8s = np.empty(inter // 32, np.uint8)
    lib().orc_expert_up(h, inter, FORMATS[fmt], _p(x8), _p(x8s), _p(w13), _p(w13_s),
                        _p(hv), _p(habs), _p(av), _p(a8), _p(a8s))
    return {"h": hv, "habs": habs, "a": av, "a8": a8, "a8s": a8s}


def expert_down(a8, a8s, w2, w2_s, fmt: str = "e4m3") -> np.ndarray:
    """The down half: y [H] = a8 . W2^T in double."""
    a8 = _c(a8, np.uint8).ravel()
    a8s = _c(a8s, np.uint8).ravel()
    w2 = _c(w2, np.uint8)
    w2_s = _c(w2_s, np.uint8)
    inter = a8.size
    h = w2.shape[0]
    y = np.empty(h, np.float64)
    lib().orc_expert_down(h, inter, FORMATS[fmt], _p(a8), _p(a8s), _p(w2), _p(w2_s), _p(y))
    return y


def combine(wts, y_routed, y_shared) -> np.ndarray:
    """One token's output sum in double: wts [k], y_routed [k, H], y_shared
    [H] -> out_f64 [H]."""
    wts = _c(wts, np.float64).ravel()
    y_routed = _c(y_routed, np.float64)
    y_shared = _c(y_shared, np.float64).ravel()
    k, h = y_routed.shape
    out = np.empty(h, np.float64)
    lib().orc_combine(k, h, _p(wts), _p(y_routed), _p(y_shared), _p(out), None)
    return out


def layer(dims: dict, inp: dict, w: dict, rows=None) -> dict:
    """The whole layer on token rows ``rows`` of inp["x"] (default: all).

    dims: hidden, experts, topk, inter, shared_inter, rms_eps, routed_scale,
          routed ("e4m3", the default, or "mxfp4": the routed experts' format).
    inp:  x [M,H] u16 (bf16 bits), norm_w [H] u16, gate_w [E,H] u16, bias [E] f32.
    w:    w13, w13_s, w2, w2_s, sgu, sgu_s, sw2, sw2_s (uint8 arrays)."""
    x = _c(inp["x"], np.uint16)
    if rows is not None:
        x = np.ascontiguousarray(x[np.asarray(rows)])
    m, H = x.shape
    E, K = dims["experts"], dims["topk"]
    d = Dims(H, E, K, dims["inter"], dims["shared_inter"],
             dims.get("rms_eps", 1e-6), dims.get("routed_scale", 1.0),
             FORMATS[dims.get("routed", "e4m3")])
    out = {
        "normed": np.empty((m, H), np.uint16),
        "x8": np.empty((m, H), np.uint8),
        "x8s": np.empty((m, H // 32), np.uint8),
        "logits": np.empty((m, E), np.float64),
        "ids": np.empty((m, K), np.int32),
        "wts": np.empty((m, K), np.float64),
        "out_f64": np.empty((m, H), np.float64),
        "out": np.empty((m, H), np.uint16),
    }
    args = [x, _c(inp["norm_w"], np.uint16), _c(inp["gate_w"], np.uint16),
            _c(inp["bias"], np.float32)]
    wl = [w[n] for n in ("w13", "w13_s", "w2", "w2_s", "sgu", "sgu_s", "sw2", "sw2_s")]
    for a in wl:
        assert a.dtype == np.uint8 and a.flags.c_contiguous
    rc = lib().orc_layer(ctypes.byref(d), m, *[_p(a) for a in args],
                         *[_p(a) for a in wl],
                         *[_p(out[n]) for n in ("normed", "x8", "x8s", "logits",
                                                "ids", "wts", "out_f64", "out")])
    if rc != 0:
        raise ValueError(f"oracle rejected the layer dimensions ({rc})")
    return out


def layer_parallel(dims: dict, inp: dict, w: dict, rows, workers: int = 8) -> dict:
    """``layer`` on each token row in ``rows`` in a thread pool (token rows are
    independent), results stacked in the order of ``rows``."""
    rows = list(rows)
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        parts = list(ex.map(lambda r: layer(dims, inp, w, rows=[r]), rows))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
