"""Python binding of the MI355X sparse MoE FFN library (libmoe_gfx950.so).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the layer runs in the library's gfx950
kernels behind the C ABI declared in include/moe.h.  The library is loaded on
first use and a missing library is an error (there is no fallback path).

Entry points mirror the C ABI: route, permute, quant_e4m3_1x128,
quant_mxfp8, grouped_ffn, combine, layer, layer_noalloc (plus
workspace-size queries).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_GFX950_LIB names another build of the same library (the host-sanitizer
# build the CPU tests run the boundary's argument checks under)
LIB_PATH = os.environ.get("MOE_GFX950_LIB") or os.path.join(HERE, "libmoe_gfx950.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
F32, BF16, E4M3, MXFP4, MXFP8 = 0, 1, 2, 3, 4
SOFTMAX, SIGMOID = 0, 1

DT = {"f32": F32, "bf16": BF16, "e4m3": E4M3, "mxfp4": MXFP4, "mxfp8": MXFP8}
SCORE = {"softmax": SOFTMAX, "sigmoid": SIGMOID}

EXPORTS = [
    "moe_route", "moe_route_workspace_size", "moe_permute", "moe_permute_workspace_size",
    "moe_quant_e4m3_1x128", "moe_quant_mxfp8", "moe_grouped_ffn", "moe_grouped_ffn_workspace_size",
    "moe_combine", "moe_layer", "moe_layer_workspace_size", "moe_layer_noalloc", "moe_mx_pack_scales",
    "moe_status_string", "moe_last_error",
]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_string(status)}: {msg}")
        self.status = status


class ExpertsT(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("dt", ctypes.c_int32),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("s_gate_up_packed", ctypes.c_void_p), ("s_down_packed", ctypes.c_void_p)]


_lib = None
_P, _I32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libmoe_gfx950.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m routed_expert_ffn_04_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "moe_route": ([_P, _I32, _I32, _I32, _P, _P, _I32, _I32, _I32, _P, _P, _P, _SZ, _P], _I32),
            "moe_route_workspace_size": ([_I32, _I32], _SZ),
            "moe_permute": ([_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P], _I32),
            "moe_permute_workspace_size": ([_I32, _I32, _I32], _SZ),
            "moe_quant_e4m3_1x128": ([_P, _I32, _I32, _I32, _P, _P, _P], _I32),
            "moe_quant_mxfp8": ([_P, _I32, _I32, _I32, _P, _P, _P], _I32),
            "moe_grouped_ffn": ([_P, _I32, _P, _P, _I32, _P, _I32, _I32, ctypes.POINTER(ExpertsT),
                                 _P, _P, _I32, ctypes.POINTER(ExpertsT), _P, _I32, _P, _P, _I32, _P, _SZ, _P], _I32),
            "moe_grouped_ffn_workspace_size": ([_I32, _I32, _I32, _I32, _I32, _I32], _SZ),
            "moe_combine": ([_P, _I32, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _P, _I32, _P], _I32),
            "moe_layer": ([_P, _I32, _I32, _I32, _P, _P, _I32, _I32, _I32, ctypes.POINTER(ExpertsT),
                           ctypes.POINTER(ExpertsT), _P, _I32, _I32, _P, _P, _P, _P, _SZ, _P], _I32),
            "moe_layer_workspace_size": ([_I32] * 10, _SZ),
            "moe_layer_noalloc": ([_P, _I32, _I32, _I32, _P, _P, _I32, _I32, _I32, ctypes.POINTER(ExpertsT),
                                   ctypes.POINTER(ExpertsT), _P, _I32, _I32, _P, _P, _P, _P], _I32),
            "moe_mx_pack_scales": ([ctypes.POINTER(ExpertsT), _P, _P, _P], _I32),
            "moe_status_string": ([_I32], ctypes.c_char_p),
            "moe_last_error": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def status_string(st: int) -> str:
    return lib().moe_status_string(st).decode()


def _check(st: int):
    if st != MOE_OK:
        raise MoeError(st, lib().moe_last_error().decode())


# ---------------------------------------------------------------- helpers

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dt_of(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _workspace(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


@dataclass
class Experts:
    """Device tensors of an expert bank (output-major weights; see moe.h).
    dt: the weight type (default: from the tensor dtype; MXFP4 banks, packed
    uint8 [n][I][H/2] with uint8 E8M0 scales, must say MXFP4)."""
    w_gate: object
    w_up: object
    w_down: object
    s_gate: object = None
    s_up: object = None
    s_down: object = None
    dt: Optional[int] = None
    s_gate_up_packed: object = None    # MXFP4: exponents in the 16-row tiles' order (pack_mx_scales)
    s_down_packed: object = None

    def struct(self) -> ExpertsT:
        n, I, H = self.w_gate.shape
        dt = _dt_of(self.w_gate) if self.dt is None else self.dt
        if dt == MXFP4:
            H *= 2
        for t in (self.w_gate, self.w_up, self.w_down):
            assert t.is_contiguous() and t.is_cuda
        return ExpertsT(n, H, I, dt, _ptr(self.w_gate), _ptr(self.w_up), _ptr(self.w_down),
                        _ptr(self.s_gate), _ptr(self.s_up), _ptr(self.s_down),
                        _ptr(self.s_gate_up_packed), _ptr(self.s_down_packed))

    def pack_mx_scales(self, stream=None) -> "Experts":
        """A copy of this MXFP4 bank that also carries its exponents in the
        16-row tiles' order (moe_mx_pack_scales): a weight-load-time step.
        Returns the bank unchanged where the shape does not allow it
        (H % 1024 or I % 512 nonzero) or the weights are not MXFP4."""
        import dataclasses
        import torch
        st = self.struct()
        if st.dt != MXFP4 or st.H % 1024 or st.I % 512:
            return self
        dev = self.w_gate.device
        gu = torch.empty(2 * st.n * st.I * (st.H // 32), dtype=torch.uint8, device=dev)
        dn = torch.empty(st.n * st.H * (st.I // 32), dtype=torch.uint8, device=dev)
        _check(lib().moe_mx_pack_scales(ctypes.byref(st), _ptr(gu), _ptr(dn), _stream(stream)))
        return dataclasses.replace(self, s_gate_up_packed=gu, s_down_packed=dn)

    @staticmethod
    def from_bank(bank, pack: bool = True) -> "Experts":
        """Device bank of a synthetic bank; MXFP4 banks also get their packed
        exponents unless pack is False."""
        e = Experts(bank.w_gate, bank.w_up, bank.w_down, bank.s_gate, bank.s_up, bank.s_down,
                    MXFP4 if bank.dt == "mxfp4" else None)
        return e.pack_mx_scales() if pack and bank.dt == "mxfp4" else e


# ---------------------------------------------------------------- entry points

def route(x, w_router, bias, k: int, score: str, stream=None, ws=None, out=None):
    """topk_ids [T][k] int32, topk_w [T][k] fp32 (moe_route)."""
    import torch
    T, H = x.shape
    E = w_router.shape[1]
    if out is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    else:
        ids, w = out
    need = lib().moe_route_workspace_size(T, E)
    ws = ws if ws is not None else _workspace(need, x.device)
    _check(lib().moe_route(_ptr(x), _dt_of(x), T, H, _ptr(w_router), _ptr(bias), E, k, SCORE[score],
                           _ptr(ids), _ptr(w), _ptr(ws), ws.numel(), _stream(stream)))
    return ids, w


def permute(topk_ids, E: int, stream=None, ws=None, out=None):
    """counts [E], offsets [E+1], src [T*k], dest [T*k] (moe_permute)."""
    import torch
    T, k = topk_ids.shape
    dev = topk_ids.device
    if out is None:
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        src = torch.empty(T * k, dtype=torch.int32, device=dev)
        dest = torch.empty(T * k, dtype=torch.int32, device=dev)
    else:
        counts, offsets, src, dest = out
    need = lib().moe_permute_workspace_size(T, k, E)
    ws = ws if ws is not None else _workspace(need, dev)
    _check(lib().moe_permute(_ptr(topk_ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(src), _ptr(dest),
                             _ptr(ws), ws.numel(), _stream(stream)))
    return counts, offsets, src, dest


def quant_e4m3_1x128(x, stream=None, out=None):
    """codes [rows][cols] uint8, scales [rows][cols/128] fp32."""
    import torch
    rows, cols = x.shape
    if out is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        s = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device)
    else:
        q, s = out
    _check(lib().moe_quant_e4m3_1x128(_ptr(x), _dt_of(x), rows, cols, _ptr(q), _ptr(s), _stream(stream)))
    return q, s


def quant_mxfp8(x, stream=None, out=None):
    """MXFP8: E4M3 codes [rows][cols] uint8, E8M0 exponents [rows][cols/32] uint8."""
    import torch
    rows, cols = x.shape
    if out is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        e = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    else:
        q, e = out
    _check(lib().moe_quant_mxfp8(_ptr(x), _dt_of(x), rows, cols, _ptr(q), _ptr(e), _stream(stream)))
    return q, e


def _act_dt(a, a_scale) -> int:
    """E4M3 codes with fp32 1x128 scales, or MXFP8 codes with uint8 E8M0 exponents."""
    import torch
    if a_scale is not None and a_scale.dtype == torch.uint8:
        return MXFP8
    return _dt_of(a)


def _is_fp8(dtype) -> bool:
    import torch
    return dtype in (torch.uint8, torch.float8_e4m3fn)


def grouped_ffn(a, offsets, routed: Experts, *, a_scale=None, src=None, src_div: int = 1, R_max=None,
                a_sh=None, a_sh_scale=None, shared: Optional[Experts] = None, y_dtype=None,
                y=None, y_scale=None, y_sh=None, y_sh_dtype=None, stream=None, ws=None):
    """moe_grouped_ffn.  Returns (y [R_max][H], y_sh [S][H]); with an fp8 y_dtype
    (torch.uint8 codes) y is the pair (codes, scales [R_max][H/128])."""
    import torch
    rs = routed.struct()
    G, H = rs.n, rs.H
    R_max = (src.numel() if src is not None else a.shape[0]) if R_max is None else R_max
    S = 0 if a_sh is None else a_sh.shape[0]
    ss = shared.struct() if shared is not None else None
    y_dtype = y.dtype if y is not None else (y_dtype or torch.float32)
    fp8_y = _is_fp8(y_dtype)
    y_sh_dtype = y_sh_dtype or (torch.bfloat16 if fp8_y else y_dtype)
    dev = a.device
    if y is None:
        y = torch.empty((R_max, H), dtype=torch.uint8 if fp8_y else y_dtype, device=dev)
    if fp8_y and y_scale is None:
        y_scale = torch.empty((R_max, H // 128), dtype=torch.float32, device=dev)
    if y_sh is None and shared is not None and S > 0:
        y_sh = torch.empty((S, H), dtype=y_sh_dtype, device=dev)
    need = lib().moe_grouped_ffn_workspace_size(R_max, G, S if shared is not None else 0, H, rs.I, rs.dt)
    ws = ws if ws is not None else _workspace(need, dev)
    _check(lib().moe_grouped_ffn(_ptr(a), _act_dt(a, a_scale), _ptr(a_scale), _ptr(src), src_div, _ptr(offsets), G, R_max,
                                 ctypes.byref(rs), _ptr(a_sh), _ptr(a_sh_scale), S,
                                 ctypes.byref(ss) if ss is not None else None,
                                 _ptr(y), _dt_of(y), _ptr(y_scale) if fp8_y else None, _ptr(y_sh),
                                 _dt_of(y_sh) if y_sh is not None else F32, _ptr(ws), ws.numel(), _stream(stream)))
    return ((y, y_scale) if fp8_y else y), y_sh


def combine(y_perm, y_sh, dest, topk_w, out_dtype=None, out=None, stream=None, y_scale=None):
    """moe_combine.  y_perm fp32/bf16, or e4m3 codes (torch.uint8) with
    y_scale [rows][H/128]."""
    import torch
    T, k = topk_w.shape
    H = y_perm.shape[1]
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y_perm.device)
    _check(lib().moe_combine(_ptr(y_perm), _dt_of(y_perm), _ptr(y_scale), _ptr(y_sh),
                             _dt_of(y_sh) if y_sh is not None else F32, _ptr(dest), _ptr(topk_w), T, k, H,
                             _ptr(out), _dt_of(out), _stream(stream)))
    return out


def layer_workspace_size(T, H, E, k, I, x_dt, w_dt, has_shared, out_dt, y_dt=None) -> int:
    return lib().moe_layer_workspace_size(T, H, E, k, I, x_dt, w_dt, int(has_shared), out_dt,
                                          out_dt if y_dt is None else y_dt)


def layer(x, w_router, bias, k: int, score: str, routed: Experts, shared: Optional[Experts] = None,
          out_dtype=None, out=None, want_routing: bool = False, ws=None, stream=None, y_dtype=None):
    """The fused layer (moe_layer).  Returns out, or (out, ids, w, counts).
    y_dtype: dtype of the routed expert outputs before the combine (default:
    out_dtype; torch.uint8 = e4m3, the FP8 combine)."""
    import torch
    T, H = x.shape
    E = w_router.shape[1]
    rs = routed.struct()
    ss = shared.struct() if shared is not None else None
    out_dtype = out_dtype or torch.float32
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    ids = w = counts = None
    if want_routing:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    y_dt = _dt_of(out) if y_dtype is None else (E4M3 if _is_fp8(y_dtype) else _dt_of(torch.empty(0, dtype=y_dtype)))
    need = layer_workspace_size(T, H, E, k, rs.I, _dt_of(x), rs.dt, ss is not None, _dt_of(out), y_dt)
    ws = ws if ws is not None else _workspace(need, dev)
    _check(lib().moe_layer(_ptr(x), _dt_of(x), T, H, _ptr(w_router), _ptr(bias), E, k, SCORE[score],
                           ctypes.byref(rs), ctypes.byref(ss) if ss is not None else None,
                           _ptr(out), _dt_of(out), y_dt, _ptr(ids), _ptr(w), _ptr(counts),
                           _ptr(ws), ws.numel(), _stream(stream)))
    return (out, ids, w, counts) if want_routing else out


def layer_noalloc(x, w_router, bias, k: int, score: str, routed: Experts, shared: Optional[Experts] = None,
                  out_dtype=None, out=None, want_routing: bool = False, stream=None, y_dtype=None):
    """moe_layer_noalloc: the fused layer with the library's own static
    scratch (no workspace argument, no device allocation by the library).
    Outputs are allocated here unless `out` (and, with want_routing, the
    routing buffers) are passed in."""
    import torch
    T, H = x.shape
    E = w_router.shape[1]
    rs = routed.struct()
    ss = shared.struct() if shared is not None else None
    out_dtype = out_dtype or torch.float32
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    ids = w = counts = None
    if want_routing:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    y_dt = _dt_of(out) if y_dtype is None else (E4M3 if _is_fp8(y_dtype) else _dt_of(torch.empty(0, dtype=y_dtype)))
    _check(lib().moe_layer_noalloc(_ptr(x), _dt_of(x), T, H, _ptr(w_router), _ptr(bias), E, k, SCORE[score],
                                   ctypes.byref(rs), ctypes.byref(ss) if ss is not None else None,
                                   _ptr(out), _dt_of(out), y_dt, _ptr(ids), _ptr(w), _ptr(counts), _stream(stream)))
    return (out, ids, w, counts) if want_routing else out
