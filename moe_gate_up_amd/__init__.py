"""Python binding of the warp-decode MoE decode layer's C ABI (include/moe_decode.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe_decode.so``.  PyTorch supplies device memory and streams.  There is no
fallback: if the library is missing, or a tensor is not on the GPU, the calls
raise.

The functions keep the C names and argument order; tensor shapes are checked
against the declared sizes before anything is launched, so a mis-sized tensor
raises here instead of being read out of bounds on the device.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_decode.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_ALIGN = -3
MOE_ERR_LAUNCH = -4
MOE_ERR_ALIAS = -5
MOE_ERR_ARG = -6
MOE_ERR_SCRATCH = -7
MOE_GATE_UP_PER_SLOT = 1
MOE_GATE_UP_EXPERT_GROUPED = 2
MOE_GATE_UP_EXPERT_GROUPED_MFMA = 3
MOE_DOWN_PER_TOKEN = 1
MOE_DOWN_EXPERT_GROUPED = 2
MOE_DOWN_EXPERT_GROUPED_MFMA = 3

EXPORTS = (
    "moe_decode_gate_up", "moe_decode_down", "moe_decode_gate_up_ex", "moe_decode_down_ex",
    "moe_decode_gate_up_plan", "moe_decode_down_plan", "moe_decode_conventional_workspace",
    "moe_decode_conventional", "moe_decode_conventional_noalloc", "moe_decode_route", "moe_decode_gate_up_routed", "moe_decode_gate_up_routed_ex",
    "moe_decode_copy_peak", "moe_decode_read_peak",
    "moe_decode_strerror",
)

_lock = threading.Lock()
_lib = None


class MoeDecodeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def lib() -> ctypes.CDLL:
    """Load libmoe_decode.so (built by __graft_entry__.build() / moe_gate_up_amd.build)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
            L = ctypes.CDLL(LIB_PATH)
            P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
            IP = ctypes.POINTER(ctypes.c_int)
            L.moe_decode_gate_up.argtypes = [P] * 7 + [I] * 5 + [P]
            L.moe_decode_down.argtypes = [P] * 6 + [I] * 5 + [P]
            L.moe_decode_gate_up_ex.argtypes = [P] * 7 + [I] * 7 + [P]
            L.moe_decode_down_ex.argtypes = [P] * 6 + [I] * 7 + [P]
            L.moe_decode_gate_up_plan.argtypes = [I] * 5 + [IP, IP, IP]
            L.moe_decode_down_plan.argtypes = [I] * 5 + [IP, IP, IP]
            L.moe_decode_conventional_workspace.argtypes = [I] * 5 + [ctypes.POINTER(ctypes.c_size_t)]
            L.moe_decode_conventional.argtypes = [P] * 11 + [S] + [I] * 5 + [P]
            L.moe_decode_conventional_noalloc.argtypes = [P] * 10 + [I] * 5 + [P]
            L.moe_decode_route.argtypes = [P] * 3 + [I] * 3 + [P]
            L.moe_decode_gate_up_routed.argtypes = [P] * 9 + [I] * 5 + [P]
            L.moe_decode_gate_up_routed_ex.argtypes = [P] * 9 + [I] * 7 + [P]
            L.moe_decode_copy_peak.argtypes = [P, P, S, P]
            L.moe_decode_read_peak.argtypes = [P, S, P, P]
            L.moe_decode_strerror.argtypes = [I]
            L.moe_decode_strerror.restype = ctypes.c_char_p
            for n in EXPORTS[:-1]:
                getattr(L, n).restype = I
            _lib = L
        return _lib


def strerror(code: int) -> str:
    return lib().moe_decode_strerror(int(code)).decode()


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, numel=None, dtypes=None):
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _types():
    import torch
    return dict(bf16=(torch.bfloat16, torch.int16, torch.uint16), i32=(torch.int32,), f32=(torch.float32,),
                u8=(torch.uint8,))


def moe_decode_gate_up(x, topk_ids, w_gate, s_gate, w_up, s_up, h_out, B=None, H=None, I=None, E=None, k=None,
                       stream=None, rows_per_wave=None, variant=None):
    """h_out[b,j,n] = bf16(SiLU(gate) * up) for expert topk_ids[b,j] (see include/moe_decode.h)."""
    T = _types()
    B = x.shape[0] if B is None else B
    H = x.shape[-1] if H is None else H
    k = topk_ids.shape[-1] if k is None else k
    E = w_gate.shape[0] if E is None else E
    I = w_gate.shape[1] if I is None else I
    args = [
        _dev(x, "x", B * H, T["bf16"]), _dev(topk_ids, "topk_ids", B * k, T["i32"]),
        _dev(w_gate, "w_gate", E * I * H, T["u8"]), _dev(s_gate, "s_gate", E * I * (H // 32), T["u8"]),
        _dev(w_up, "w_up", E * I * H, T["u8"]), _dev(s_up, "s_up", E * I * (H // 32), T["u8"]),
        _dev(h_out, "h_out", B * k * I, T["bf16"]), B, H, I, E, k,
    ]
    if rows_per_wave is None and variant is None:
        rc = lib().moe_decode_gate_up(*args, _stream(stream))
    else:
        rc = lib().moe_decode_gate_up_ex(*args, int(variant or 0), int(rows_per_wave or 0), _stream(stream))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_gate_up")
    return h_out


def moe_decode_route(logits, topk_ids, topk_weights, B=None, E=None, k=None, stream=None):
    """Top-k router: topk_ids / topk_weights [B,k] from logits fp32 [B,E] (see include/moe_decode.h)."""
    T = _types()
    B = logits.shape[0] if B is None else B
    E = logits.shape[-1] if E is None else E
    k = topk_ids.shape[-1] if k is None else k
    rc = lib().moe_decode_route(
        _dev(logits, "logits", B * E, T["f32"]), _dev(topk_ids, "topk_ids", B * k, T["i32"]),
        _dev(topk_weights, "topk_weights", B * k, T["f32"]), B, E, k, _stream(stream))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_route")
    return topk_ids, topk_weights


def moe_decode_gate_up_routed(x, logits, w_gate, s_gate, w_up, s_up, h_out, topk_ids_out, topk_weights_out,
                              B=None, H=None, I=None, E=None, k=None, stream=None, rows_per_wave=None, variant=None):
    """gate/up with the top-k router step fused in: h_out, topk_ids_out and topk_weights_out
    from x and the router logits (see include/moe_decode.h)."""
    T = _types()
    B = x.shape[0] if B is None else B
    H = x.shape[-1] if H is None else H
    k = topk_ids_out.shape[-1] if k is None else k
    E = w_gate.shape[0] if E is None else E
    I = w_gate.shape[1] if I is None else I
    args = [
        _dev(x, "x", B * H, T["bf16"]), _dev(logits, "logits", B * E, T["f32"]),
        _dev(w_gate, "w_gate", E * I * H, T["u8"]), _dev(s_gate, "s_gate", E * I * (H // 32), T["u8"]),
        _dev(w_up, "w_up", E * I * H, T["u8"]), _dev(s_up, "s_up", E * I * (H // 32), T["u8"]),
        _dev(h_out, "h_out", B * k * I, T["bf16"]), _dev(topk_ids_out, "topk_ids_out", B * k, T["i32"]),
        _dev(topk_weights_out, "topk_weights_out", B * k, T["f32"]), B, H, I, E, k,
    ]
    if rows_per_wave is None and variant is None:
        rc = lib().moe_decode_gate_up_routed(*args, _stream(stream))
    else:
        rc = lib().moe_decode_gate_up_routed_ex(*args, int(variant or 0), int(rows_per_wave or 0), _stream(stream))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_gate_up_routed")
    return h_out, topk_ids_out, topk_weights_out


def moe_decode_down(h, topk_ids, topk_weights, w_down, s_down, y_out, B=None, H=None, I=None, E=None, k=None,
                    stream=None, rows_per_wave=None, variant=None):
    """y_out[b,o] = bf16(sum_j w[b,j] * down row . h[b,j,:]) (see include/moe_decode.h)."""
    T = _types()
    B = h.shape[0] if B is None else B
    k = topk_ids.shape[-1] if k is None else k
    E = w_down.shape[0] if E is None else E
    H = w_down.shape[1] if H is None else H
    I = w_down.shape[2] if I is None else I
    args = [
        _dev(h, "h", B * k * I, T["bf16"]), _dev(topk_ids, "topk_ids", B * k, T["i32"]),
        _dev(topk_weights, "topk_weights", B * k, T["f32"]),
        _dev(w_down, "w_down", E * H * I, T["u8"]), _dev(s_down, "s_down", E * H * (I // 32), T["u8"]),
        _dev(y_out, "y_out", B * H, T["bf16"]), B, H, I, E, k,
    ]
    if rows_per_wave is None and variant is None:
        rc = lib().moe_decode_down(*args, _stream(stream))
    else:
        rc = lib().moe_decode_down_ex(*args, int(variant or 0), int(rows_per_wave or 0), _stream(stream))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_down")
    return y_out


def moe_decode_gate_up_plan(B, H, I, E, k):
    """(variant, rows_per_wave, workgroups) the built-in table picks."""
    v, r, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rc = lib().moe_decode_gate_up_plan(B, H, I, E, k, ctypes.byref(v), ctypes.byref(r), ctypes.byref(g))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_gate_up_plan")
    return v.value, r.value, g.value


def moe_decode_down_plan(B, H, I, E, k):
    """(variant, rows_per_wave, workgroups) the built-in table picks."""
    v, r, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rc = lib().moe_decode_down_plan(B, H, I, E, k, ctypes.byref(v), ctypes.byref(r), ctypes.byref(g))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_down_plan")
    return v.value, r.value, g.value


def moe_decode_conventional_workspace(B, H, I, E, k):
    """Bytes of device workspace moe_decode_conventional needs."""
    n = ctypes.c_size_t()
    rc = lib().moe_decode_conventional_workspace(B, H, I, E, k, ctypes.byref(n))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_conventional_workspace")
    return n.value


def moe_decode_conventional(x, topk_ids, topk_weights, w_gate, s_gate, w_up, s_up, w_down, s_down, y_out, workspace,
                            stream=None):
    """The expert-centric path (see include/moe_decode.h); workspace: a uint8 GPU tensor."""
    T = _types()
    B, H = x.shape
    k = topk_ids.shape[-1]
    E, I = w_gate.shape[0], w_gate.shape[1]
    wb = E * I * H
    args = [
        _dev(x, "x", B * H, T["bf16"]), _dev(topk_ids, "topk_ids", B * k, T["i32"]),
        _dev(topk_weights, "topk_weights", B * k, T["f32"]),
        _dev(w_gate, "w_gate", wb, T["u8"]), _dev(s_gate, "s_gate", wb // 32, T["u8"]),
        _dev(w_up, "w_up", wb, T["u8"]), _dev(s_up, "s_up", wb // 32, T["u8"]),
        _dev(w_down, "w_down", wb, T["u8"]), _dev(s_down, "s_down", wb // 32, T["u8"]),
        _dev(y_out, "y_out", B * H, T["bf16"]), _dev(workspace, "workspace", None, T["u8"]),
        workspace.numel(), B, H, I, E, k,
    ]
    rc = lib().moe_decode_conventional(*args, _stream(stream))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_conventional")
    return y_out


def moe_decode_conventional_noalloc(x, topk_ids, topk_weights, w_gate, s_gate, w_up, s_up, w_down, s_down, y_out,
                                    stream=None):
    """The expert-centric path on the library's fixed scratch buffer, with no
    workspace and no allocation (see include/moe_decode.h)."""
    T = _types()
    B, H = x.shape
    k = topk_ids.shape[-1]
    E, I = w_gate.shape[0], w_gate.shape[1]
    wb = E * I * H
    args = [
        _dev(x, "x", B * H, T["bf16"]), _dev(topk_ids, "topk_ids", B * k, T["i32"]),
        _dev(topk_weights, "topk_weights", B * k, T["f32"]),
        _dev(w_gate, "w_gate", wb, T["u8"]), _dev(s_gate, "s_gate", wb // 32, T["u8"]),
        _dev(w_up, "w_up", wb, T["u8"]), _dev(s_up, "s_up", wb // 32, T["u8"]),
        _dev(w_down, "w_down", wb, T["u8"]), _dev(s_down, "s_down", wb // 32, T["u8"]),
        _dev(y_out, "y_out", B * H, T["bf16"]), B, H, I, E, k,
    ]
    rc = lib().moe_decode_conventional_noalloc(*args, _stream(stream))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_conventional_noalloc")
    return y_out


def moe_decode_copy_peak(src, dst, stream=None):
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    rc = lib().moe_decode_copy_peak(_dev(src, "src"), _dev(dst, "dst"), n, _stream(stream))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_copy_peak")


def moe_decode_read_peak(src, sink, stream=None):
    n = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink needs 4 bytes")
    rc = lib().moe_decode_read_peak(_dev(src, "src"), n, _dev(sink, "sink"), _stream(stream))
    if rc:
        raise MoeDecodeError(rc, "moe_decode_read_peak")
