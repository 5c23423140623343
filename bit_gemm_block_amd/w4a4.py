"""Python binding of libw4a4.so: argument marshalling only.

Every function takes torch tensors that live on a ROCm device, checks dtype,
shape and contiguity, and calls the C entry point of the same name on the
current HIP stream of that device.  No arithmetic of the layer happens here;
outputs that the caller does not pass are allocated with torch (device memory
plumbing only).  When the shared library is missing every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libw4a4.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "w4a4.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_WORKSPACE, ERR_HIP = range(6)
F32, F16 = 0, 1
(CODES_PACKED, CODES_I8, CODES_I8_TILED, CODES_PACKED_TILED, CODES_PACKED_TILED_OB,
 CODES_F6_TILED) = range(6)
WEIGHTS_ROWMAJOR, WEIGHTS_TILED, WEIGHTS_TILED_OB, WEIGHTS_TILED_F6 = 0, 1, 2, 3
_LAYOUTS = {"packed": CODES_PACKED, "i8": CODES_I8, "i8_tiled": CODES_I8_TILED,
            "packed_tiled": CODES_PACKED_TILED, "packed_tiled_ob": CODES_PACKED_TILED_OB,
            "f6_tiled": CODES_F6_TILED}
_TILED_CODES = (CODES_I8_TILED, CODES_PACKED_TILED, CODES_F6_TILED)
_PACKED_CODES = (CODES_PACKED, CODES_PACKED_TILED)
_WLAYOUTS = {"rowmajor": WEIGHTS_ROWMAJOR, "tiled": WEIGHTS_TILED, "tiled_ob": WEIGHTS_TILED_OB,
             "tiled_f6": WEIGHTS_TILED_F6}

_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SIGS = {
    "w4a4_abi_version": (_INT, []),
    "w4a4_status_string": (ctypes.c_char_p, [_INT]),
    "w4a4_last_hip_error": (_INT, []),
    "w4a4_hadamard_rotate": (_INT, [_P, _INT, _P, _I64, _I64, _I64, _P]),
    "w4a4_quantize_act_int4": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _INT, _P, _P]),
    "w4a4_quantize_act_int8": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _INT, _P, _P]),
    "w4a4_quantize_weight_int4": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _P, _INT, _P, _INT,
                                         _P]),
    "w4a4_lowrank_project": (_INT, [_P, _INT, _P, _I64, _I64, _I64, _P, _P]),
    "w4a4_qgemm_w4a4": (_INT, [_P, _INT, _P, _P, _INT, _P, _INT, _I64, _I64, _I64, _I64, _P, _P,
                               _P]),
    "w4a4_qlinear_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64, _I64]),
    "w4a4_qlinear_workspace_layout": (_INT, [_I64, _I64, _I64, _I64, _INT, _I64, _INT,
                                             ctypes.POINTER(ctypes.c_size_t),
                                             ctypes.POINTER(_INT),
                                             ctypes.POINTER(ctypes.c_size_t)]),
    "w4a4_qlinear_forward": (_INT, [_P, _INT, _P, _INT, _P, _INT, _I64, _I64, _I64, _I64, _I64,
                                    _P, _P, _I64, _P, _P, ctypes.c_size_t, _P]),
    "w4a8_qlinear_forward": (_INT, [_P, _INT, _P, _INT, _P, _INT, _I64, _I64, _I64, _I64, _I64,
                                    _P, _P, _I64, _P, _P, ctypes.c_size_t, _P]),
    "w4a4_qlinear_forward_noalloc": (_INT, [_P, _INT, _P, _INT, _P, _INT, _I64, _I64, _I64, _I64,
                                            _I64, _P, _P, _I64, _P, _P]),
    "w4a4_quantize_act_asym_int4": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _P, _INT, _P, _P,
                                           _P]),
    "w4a4_quantize_weight_residual_int4": (_INT, [_P, _INT, _I64, _I64, _I64, _I64, _P, _P, _INT,
                                                  _P]),
    "w4a4_qgemm_residual": (_INT, [_P, _P, _P, _P, _INT, _I64, _I64, _I64, _I64, _P, _P, _P]),
    "w4a4_quantize_mxfp4": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _INT, _P, _P]),
    "w4a4_qgemm_mxfp4": (_INT, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "w4a4_weights_tiled_to_ob": (_INT, [_P, _I64, _I64, _P, _P]),
    "w4a4_qlinear_forward_mxfp4": (_INT, [_P, _INT, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _I64,
                                          _P, _P, ctypes.c_size_t, _P]),
    "w4a4_qlinear_forward_residual": (_INT, [_P, _INT, _P, _P, _INT, _I64, _I64, _I64, _I64, _I64,
                                             _P, _P, ctypes.c_size_t, _P]),
    "w4a4_weight_group_sums": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P]),
    "w4a4_qgemm_asym": (_INT, [_P, _P, _P, _I64, _P, _P, _INT, _P, _I64, _I64, _I64, _P, _P]),
    "w4a4_qlinear_forward_asym": (_INT, [_P, _INT, _P, _P, _INT, _P, _I64, _I64, _I64, _I64, _P,
                                         _P, _I64, _P, _P, ctypes.c_size_t, _P]),
}


class W4A4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().w4a4_status_string(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError {lib().w4a4_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [status {status}]")


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_gemm_block_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/w4a4.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(w4a[48]_\w+)\s*\(", text, re.M)))


def pad16(n: int) -> int:
    """Rows of a tiled layout: n rounded up to a multiple of 16."""
    return (n + 15) // 16 * 16


def code_bytes_per_row(layout: str, K: int) -> int:
    """Bytes per (padded) row of codes of K channels in a codes or weight
    layout: K/2 packed nibbles, K int8 codes, or 3K/4 for the FP6 tiles."""
    if layout in ("f6_tiled", "tiled_f6"):
        return 3 * K // 4
    if layout in ("i8", "i8_tiled"):
        return K
    return K // 2


def ob_bytes(rows: int, K: int) -> int:
    """Bytes of an offset-binary tiled buffer (flat uint8): the tiles of
    pad16(rows) rows, then one int32 sum per padded row."""
    return pad16(rows) * (K // 2 + 4)


def ob_sums(buf: torch.Tensor, rows: int, K: int) -> torch.Tensor:
    """The int32 row sums that follow the tiles of an offset-binary buffer."""
    off = pad16(rows) * (K // 2)
    return buf[off:off + 4 * pad16(rows)].view(torch.int32)[:rows]


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise W4A4Error(fn, status)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def hadamard_rotate(x: torch.Tensor, had_block: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _dev(x, "x")
    M, K = x.shape
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=x.device)
    _dev(out, "out")
    _check("hadamard_rotate", lib().w4a4_hadamard_rotate(
        _ptr(x), _dt(x), _ptr(out), M, K, had_block, _stream(x)))
    return out


def quantize_act_int4(x: torch.Tensor, had_block: int, xq: Optional[torch.Tensor] = None,
                      x_scale: Optional[torch.Tensor] = None,
                      layout: str = "packed") -> Tuple[torch.Tensor, torch.Tensor]:
    """Codes in layout "packed" ([M, K/2] nibbles), "i8" ([M, K] int8 in
    the GEMM's K order), "i8_tiled" ([pad16(M), K] in 2 KB tiles) or
    "packed_tiled" ([pad16(M), K/2] in the weights' 1 KB tiles) or
    "packed_tiled_ob" (flat, ob_bytes(M, K): offset-binary tiles and the row
    sums of the odd channels' codes) or "f6_tiled" ([pad16(M), 3K/4]: FP6
    E2M3 tiles of 1536 bytes), and one float32 scale per row."""
    _dev(x, "x")
    M, K = x.shape
    lay = _LAYOUTS[layout]
    if xq is None and lay == CODES_PACKED_TILED_OB:
        xq = torch.empty((ob_bytes(M, K),), dtype=torch.uint8, device=x.device)
    elif xq is None:
        rows = pad16(M) if lay in _TILED_CODES else M
        xq = torch.empty((rows, code_bytes_per_row(layout, K)), dtype=torch.uint8,
                         device=x.device)
    if x_scale is None:
        x_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check("quantize_act_int4", lib().w4a4_quantize_act_int4(
        _ptr(x), _dt(x), M, K, had_block, _ptr(xq), lay, _ptr(x_scale), _stream(x)))
    return xq, x_scale


def quantize_act_int8(x: torch.Tensor, had_block: int, xq: Optional[torch.Tensor] = None,
                      x_scale: Optional[torch.Tensor] = None,
                      layout: str = "i8") -> Tuple[torch.Tensor, torch.Tensor]:
    """8-bit activation codes (|q| <= 127) of a W4A8 layer, in layout "i8"
    ([M, K]) or "i8_tiled" ([pad16(M), K]), and one float32 scale per row."""
    _dev(x, "x")
    M, K = x.shape
    lay = _LAYOUTS[layout]
    if xq is None:
        xq = torch.empty((pad16(M) if lay in _TILED_CODES else M, K), dtype=torch.uint8,
                         device=x.device)
    if x_scale is None:
        x_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check("quantize_act_int8", lib().w4a4_quantize_act_int8(
        _ptr(x), _dt(x), M, K, had_block, _ptr(xq), lay, _ptr(x_scale), _stream(x)))
    return xq, x_scale


def quantize_weight_int4(w: torch.Tensor, had_block: int, w_group: int,
                         scale_dtype: torch.dtype = torch.float16,
                         layout: str = "rowmajor") -> Tuple[torch.Tensor, torch.Tensor]:
    """Packed codes in layout "rowmajor" ([N, K/2]) or "tiled" ([pad16(N),
    K/2] in 1 KB tiles), or FP6 E2M3 codes in layout "tiled_f6" ([pad16(N),
    3K/4] in 1536-byte tiles), and the scales [N] or [N, K/w_group]."""
    _dev(w, "w")
    N, K = w.shape
    wl = _WLAYOUTS[layout]
    wq = torch.empty((N if wl == WEIGHTS_ROWMAJOR else pad16(N), code_bytes_per_row(layout, K)),
                     dtype=torch.uint8, device=w.device)
    shape = (N,) if w_group == 0 else (N, K // w_group)
    ws = torch.empty(shape, dtype=scale_dtype, device=w.device)
    _check("quantize_weight_int4", lib().w4a4_quantize_weight_int4(
        _ptr(w), _dt(w), N, K, had_block, w_group, _ptr(wq), wl, _ptr(ws), _dt(ws),
        _stream(w)))
    return wq, ws


def lowrank_project(x: torch.Tensor, At: torch.Tensor, t: Optional[torch.Tensor] = None) -> torch.Tensor:
    """t = x . A with A given transposed, At [rank, K]."""
    _dev(x, "x")
    _dev(At, "At")
    M, K = x.shape
    if At.dtype != x.dtype or At.shape[1] != K:
        raise ValueError("At must be [rank, K] in x's dtype")
    rank = At.shape[0]
    if t is None:
        t = torch.empty((M, rank), dtype=torch.float32, device=x.device)
    _check("lowrank_project", lib().w4a4_lowrank_project(
        _ptr(x), _dt(x), _ptr(At), M, K, rank, _ptr(t), _stream(x)))
    return t


def qgemm_w4a4(xq: torch.Tensor, x_scale: Optional[torch.Tensor], wq: torch.Tensor,
               w_scale: Optional[torch.Tensor], w_group: int, want_y: bool = True,
               want_acc: bool = False, y: Optional[torch.Tensor] = None,
               acc: Optional[torch.Tensor] = None, layout: str = "packed",
               w_layout: str = "rowmajor", M: Optional[int] = None, N: Optional[int] = None):
    """M and N default to x_scale's and w_scale's lengths (else xq's and wq's
    rows, which tiled layouts pad to a multiple of 16)."""
    _dev(xq, "xq")
    _dev(wq, "wq")
    lay = _LAYOUTS[layout]
    wl = _WLAYOUTS[w_layout]
    if M is None:
        M = x_scale.shape[0] if x_scale is not None else xq.shape[0]
    if N is None:
        N = w_scale.shape[0] if w_scale is not None else wq.shape[0]
    if wl == WEIGHTS_TILED_OB:  # flat buffers: K from the weights' size
        K = 2 * (wq.numel() // pad16(N) - 4)
        if wq.numel() != ob_bytes(N, K):
            raise ValueError("wq is not an offset-binary buffer of N rows")
    elif wl == WEIGHTS_TILED_F6:
        K = 4 * wq.shape[1] // 3
        if wq.shape[0] < pad16(N) or wq.shape[1] != 3 * K // 4:
            raise ValueError("wq is not an FP6 tiled buffer of N rows")
    else:
        K = 2 * wq.shape[1]
        if wq.shape[0] < (pad16(N) if wl == WEIGHTS_TILED else N):
            raise ValueError("wq has too few rows")
    if lay == CODES_PACKED_TILED_OB:
        if xq.numel() != ob_bytes(M, K):
            raise ValueError("xq is not an offset-binary buffer of M rows and K channels")
    else:
        if xq.shape[1] != code_bytes_per_row(layout, K):
            raise ValueError("xq and wq disagree on K")
        if xq.shape[0] < (pad16(M) if lay in _TILED_CODES else M):
            raise ValueError("xq has too few rows")
    if want_y and y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    if want_acc and acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    wst = _dt(w_scale) if w_scale is not None else F32
    _check("qgemm_w4a4", lib().w4a4_qgemm_w4a4(
        _ptr(xq), lay, _ptr(x_scale), _ptr(wq), wl, _ptr(w_scale), wst, w_group, M, N, K,
        _ptr(y), _ptr(acc), _stream(xq)))
    return y, acc


def weights_tiled_to_ob(wq: torch.Tensor, N: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Offset-binary form (flat, ob_bytes(N, K)) of tiled weights [pad16(N), K/2]."""
    _dev(wq, "wq")
    K = 2 * wq.shape[1]
    if wq.shape[0] != pad16(N):
        raise ValueError("wq must be tiled weights of pad16(N) rows")
    if out is None:
        out = torch.empty((ob_bytes(N, K),), dtype=torch.uint8, device=wq.device)
    if out.numel() != ob_bytes(N, K):
        raise ValueError("out must hold ob_bytes(N, K) bytes")
    _check("weights_tiled_to_ob", lib().w4a4_weights_tiled_to_ob(
        _ptr(wq), N, K, _ptr(out), _stream(wq)))
    return out


def qlinear_workspace_size(M: int, N: int, K: int, rank: int) -> int:
    return int(lib().w4a4_qlinear_workspace_size(M, N, K, rank))


def qlinear_workspace(M: int, N: int, K: int, rank: int, device) -> torch.Tensor:
    """A workspace for qlinear_forward calls up to these sizes (device memory,
    contents unspecified)."""
    return torch.empty((max(qlinear_workspace_size(M, N, K, rank), 1),), dtype=torch.uint8,
                       device=device)


def qlinear_workspace_layout(M: int, N: int, K: int, rank: int, w_layout: str = "rowmajor",
                             w_group: int = 0, act_bits: int = 4) -> Tuple[int, str, int]:
    """(codes byte offset, codes layout name, scales byte offset) of what
    qlinear_forward leaves in its workspace for a call of these sizes."""
    co, so = ctypes.c_size_t(0), ctypes.c_size_t(0)
    cl = _INT(0)
    _check("qlinear_workspace_layout", lib().w4a4_qlinear_workspace_layout(
        M, N, K, rank, _WLAYOUTS[w_layout], w_group, act_bits, ctypes.byref(co),
        ctypes.byref(cl), ctypes.byref(so)))
    name = {v: k for k, v in _LAYOUTS.items()}[cl.value]
    return int(co.value), name, int(so.value)


def qlinear_forward(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor, had_block: int,
                    w_group: int, At: Optional[torch.Tensor] = None,
                    Bt: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    w_layout: str = "rowmajor", act_bits: int = 4) -> torch.Tensor:
    """Y = dequant(int4 GEMM(rotate+quantize(x), wq)) + x . A . B, with the
    low-rank factors given transposed: At [rank, K], Bt [N, rank].  N is
    w_scale's length.  act_bits 8 runs the W4A8 layer."""
    if act_bits not in (4, 8):
        raise ValueError("act_bits must be 4 or 8")
    _dev(x, "x")
    _dev(wq, "wq")
    _dev(w_scale, "w_scale")
    wl = _WLAYOUTS[w_layout]
    M, K = x.shape
    N = w_scale.shape[0]
    if wl == WEIGHTS_TILED_OB:
        if wq.numel() != ob_bytes(N, K):
            raise ValueError("wq is not an offset-binary buffer matching w_scale and x")
    elif (wq.shape[0] < (N if wl == WEIGHTS_ROWMAJOR else pad16(N)) or
          wq.shape[1] != code_bytes_per_row(w_layout, K)):
        raise ValueError("wq does not match w_scale and x")
    rank = 0 if At is None else At.shape[0]
    if rank:
        if Bt is None or At.dtype != x.dtype or Bt.dtype != x.dtype:
            raise ValueError("At and Bt must both be given in x's dtype")
        if tuple(At.shape) != (rank, K) or tuple(Bt.shape) != (N, rank):
            raise ValueError("At must be [rank, K] and Bt [N, rank]")
        _dev(At, "At")
        _dev(Bt, "Bt")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = qlinear_workspace(M, N, K, rank, x.device)
    fwd = lib().w4a4_qlinear_forward if act_bits == 4 else lib().w4a8_qlinear_forward
    _check("qlinear_forward", fwd(
        _ptr(x), _dt(x), _ptr(wq), wl, _ptr(w_scale), _dt(w_scale), M, N, K, had_block, w_group,
        _ptr(At), _ptr(Bt), rank, _ptr(y), _ptr(workspace), workspace.numel(), _stream(x)))
    return y


# ---- asymmetric group-wise activations -------------------------------------
NOALLOC_SCRATCH_BYTES = 32 << 20   # W4A4_NOALLOC_SCRATCH_BYTES of include/w4a4.h


def qlinear_forward_noalloc(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                            had_block: int, w_group: int, At: Optional[torch.Tensor] = None,
                            Bt: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                            w_layout: str = "rowmajor") -> torch.Tensor:
    """qlinear_forward with its scratch in the library's fixed per-device
    array instead of a workspace (the C call allocates nothing; y is
    allocated here when not given)."""
    _dev(x, "x")
    _dev(wq, "wq")
    _dev(w_scale, "w_scale")
    wl = _WLAYOUTS[w_layout]
    M, K = x.shape
    N = w_scale.shape[0]
    rank = 0 if At is None else At.shape[0]
    if rank:
        if Bt is None or tuple(At.shape) != (rank, K) or tuple(Bt.shape) != (N, rank):
            raise ValueError("At must be [rank, K] and Bt [N, rank]")
        _dev(At, "At")
        _dev(Bt, "Bt")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check("qlinear_forward_noalloc", lib().w4a4_qlinear_forward_noalloc(
        _ptr(x), _dt(x), _ptr(wq), wl, _ptr(w_scale), _dt(w_scale), M, N, K, had_block, w_group,
        _ptr(At), _ptr(Bt), rank, _ptr(y), _stream(x)))
    return y


def quantize_act_asym_int4(x: torch.Tensor, had_block: int, group: Optional[int] = None,
                           layout: str = "packed", xq: Optional[torch.Tensor] = None,
                           sx: Optional[torch.Tensor] = None, zx: Optional[torch.Tensor] = None):
    """uint4 codes with one float32 scale and one int32 zero point per token
    and group (default: the Hadamard block).  The nibbles hold q - 8; layout
    "packed" ([M, K/2]) or "packed_tiled" ([pad16(M), K/2]).  Returns
    (xq, x_scale [M, K/group], x_zero [M, K/group])."""
    _dev(x, "x")
    M, K = x.shape
    group = had_block if group is None else group
    lay = _LAYOUTS[layout]
    if xq is None:
        xq = torch.empty((pad16(M) if lay in _TILED_CODES else M, K // 2), dtype=torch.uint8,
                         device=x.device)
    G = K // group if group > 0 else 0
    if sx is None:
        sx = torch.empty((M, G), dtype=torch.float32, device=x.device)
    if zx is None:
        zx = torch.empty((M, G), dtype=torch.int32, device=x.device)
    for t, n in ((xq, "xq"), (sx, "x_scale"), (zx, "x_zero")):
        _dev(t, n)
    _check("quantize_act_asym_int4", lib().w4a4_quantize_act_asym_int4(
        _ptr(x), _dt(x), M, K, had_block, group, _ptr(xq), lay, _ptr(sx), _ptr(zx), _stream(x)))
    return xq, sx, zx


def weight_group_sums(wq: torch.Tensor, group: int, N: Optional[int] = None,
                      w_layout: str = "rowmajor") -> torch.Tensor:
    """int32 [N, K/group]: the signed weight codes summed over each group."""
    _dev(wq, "wq")
    wl = _WLAYOUTS[w_layout]
    K = 2 * wq.shape[1]
    N = wq.shape[0] if N is None else N
    if wq.shape[0] < (pad16(N) if wl == WEIGHTS_TILED else N):
        raise ValueError("wq has too few rows")
    out = torch.empty((N, K // group if group > 0 else 0), dtype=torch.int32, device=wq.device)
    _check("weight_group_sums", lib().w4a4_weight_group_sums(
        _ptr(wq), wl, N, K, group, _ptr(out), _stream(wq)))
    return out


def qgemm_asym(xq: torch.Tensor, x_scale: torch.Tensor, x_zero: torch.Tensor, group: int,
               wq: torch.Tensor, w_scale: torch.Tensor, w_gsum: torch.Tensor,
               y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Asymmetric activation codes (packed tiled) times tiled int4 weights
    with per-channel scales; M from x_scale, N from w_scale."""
    for t, n in ((xq, "xq"), (x_scale, "x_scale"), (x_zero, "x_zero"), (wq, "wq"),
                 (w_scale, "w_scale"), (w_gsum, "w_gsum")):
        _dev(t, n)
    M, N, K = x_scale.shape[0], w_scale.shape[0], 2 * wq.shape[1]
    G = K // group if group > 0 else 0
    if xq.shape[1] != K // 2 or xq.shape[0] < pad16(M) or wq.shape[0] < pad16(N):
        raise ValueError("xq / wq do not match the tiled layouts of M, N, K")
    if tuple(x_scale.shape) != (M, G) or tuple(x_zero.shape) != (M, G) or \
            tuple(w_gsum.shape) != (N, G):
        raise ValueError("scales, zero points and weight sums must be [rows, K/group]")
    if x_zero.dtype != torch.int32 or w_gsum.dtype != torch.int32:
        raise TypeError("zero points and weight sums are int32")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    _check("qgemm_asym", lib().w4a4_qgemm_asym(
        _ptr(xq), _ptr(x_scale), _ptr(x_zero), group, _ptr(wq), _ptr(w_scale), _dt(w_scale),
        _ptr(w_gsum), M, N, K, _ptr(y), _stream(xq)))
    return y


def qlinear_forward_asym(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                         w_gsum: torch.Tensor, had_block: int,
                         At: Optional[torch.Tensor] = None, Bt: Optional[torch.Tensor] = None,
                         y: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer with asymmetric group-wise activations (group = had_block)
    on tiled weights with per-channel scales."""
    _dev(x, "x")
    _dev(wq, "wq")
    _dev(w_scale, "w_scale")
    _dev(w_gsum, "w_gsum")
    M, K = x.shape
    N = w_scale.shape[0]
    if wq.shape[0] < pad16(N) or wq.shape[1] != K // 2:
        raise ValueError("wq does not match w_scale and x")
    rank = 0 if At is None else At.shape[0]
    if rank:
        if Bt is None or At.dtype != x.dtype or Bt.dtype != x.dtype:
            raise ValueError("At and Bt must both be given in x's dtype")
        if tuple(At.shape) != (rank, K) or tuple(Bt.shape) != (N, rank):
            raise ValueError("At must be [rank, K] and Bt [N, rank]")
        _dev(At, "At")
        _dev(Bt, "Bt")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = qlinear_workspace(M, N, K, rank, x.device)
    _check("qlinear_forward_asym", lib().w4a4_qlinear_forward_asym(
        _ptr(x), _dt(x), _ptr(wq), _ptr(w_scale), _dt(w_scale), _ptr(w_gsum), M, N, K,
        had_block, _ptr(At), _ptr(Bt), rank, _ptr(y), _ptr(workspace), workspace.numel(),
        _stream(x)))
    return y


# ---- in-GEMM residual of salient channels ----------------------------------
def res_pad(r: int) -> int:
    """Residual rank rounded up to whole 128-channel tiles."""
    return (r + 127) // 128 * 128


def quantize_weight_residual_int4(w: torch.Tensor, had_block: int, res_rank: int,
                                  scale_dtype: torch.dtype = torch.float16):
    """Tiled packed codes with the residual tiles of channels [0, res_rank)
    after each row block's code tiles ([pad16(N), (K + res_pad)/2]), and the
    per-channel scales [N]."""
    _dev(w, "w")
    N, K = w.shape
    wq = torch.empty((pad16(N), (K + res_pad(res_rank)) // 2), dtype=torch.uint8, device=w.device)
    ws = torch.empty((N,), dtype=scale_dtype, device=w.device)
    _check("quantize_weight_residual_int4", lib().w4a4_quantize_weight_residual_int4(
        _ptr(w), _dt(w), N, K, had_block, res_rank, _ptr(wq), _ptr(ws), _dt(ws), _stream(w)))
    return wq, ws


def qgemm_residual(xq: torch.Tensor, x_scale: Optional[torch.Tensor], wq: torch.Tensor,
                   w_scale: Optional[torch.Tensor], res_rank: int, M: int, N: int, K: int,
                   want_y: bool = True, want_acc: bool = False,
                   y: Optional[torch.Tensor] = None, acc: Optional[torch.Tensor] = None):
    """Packed tiled codes times residual-extended tiled weights."""
    _dev(xq, "xq")
    _dev(wq, "wq")
    if xq.shape[1] != K // 2 or xq.shape[0] < pad16(M):
        raise ValueError("xq does not match M and K")
    if wq.shape[1] != (K + res_pad(res_rank)) // 2 or wq.shape[0] < pad16(N):
        raise ValueError("wq does not match N, K and the residual rank")
    if want_y and y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    if want_acc and acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    wst = _dt(w_scale) if w_scale is not None else F32
    _check("qgemm_residual", lib().w4a4_qgemm_residual(
        _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), wst, res_rank, M, N, K, _ptr(y),
        _ptr(acc), _stream(xq)))
    return y, acc


def qlinear_forward_residual(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                             res_rank: int, had_block: int, y: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer with the in-GEMM residual of the first res_rank channels."""
    _dev(x, "x")
    _dev(wq, "wq")
    _dev(w_scale, "w_scale")
    M, K = x.shape
    N = w_scale.shape[0]
    if wq.shape[0] < pad16(N) or wq.shape[1] != (K + res_pad(res_rank)) // 2:
        raise ValueError("wq does not match w_scale, x and the residual rank")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = qlinear_workspace(M, N, K, 0, x.device)
    _check("qlinear_forward_residual", lib().w4a4_qlinear_forward_residual(
        _ptr(x), _dt(x), _ptr(wq), _ptr(w_scale), _dt(w_scale), res_rank, M, N, K, had_block,
        _ptr(y), _ptr(workspace), workspace.numel(), _stream(x)))
    return y


# ---- MXFP4 ------------------------------------------------------------------
def mx_scale_bytes(rows: int, K: int, layout: str) -> int:
    """Bytes of the E8M0 scales of [rows, K] MXFP4 codes in a layout."""
    return pad16(rows) * K // 32 if layout == "packed_tiled" else rows * K // 32


def quantize_mxfp4(x: torch.Tensor, had_block: int, layout: str = "packed",
                   xq: Optional[torch.Tensor] = None, xs: Optional[torch.Tensor] = None):
    """E2M1 codes (packed, [M, K/2] or tiled [pad16(M), K/2]) and E8M0 scale
    bytes ([M, K/32], or the tiled scale array of w4a4_quantize_mxfp4)."""
    _dev(x, "x")
    M, K = x.shape
    lay = _LAYOUTS[layout]
    if lay not in _PACKED_CODES:
        raise ValueError("MXFP4 codes are packed")
    if xq is None:
        xq = torch.empty((pad16(M) if lay in _TILED_CODES else M, K // 2), dtype=torch.uint8,
                         device=x.device)
    if xs is None:
        xs = (torch.empty((M, K // 32), dtype=torch.uint8, device=x.device) if layout == "packed"
              else torch.empty((mx_scale_bytes(M, K, layout),), dtype=torch.uint8, device=x.device))
    _dev(xq, "xq")
    _dev(xs, "xs")
    _check("quantize_mxfp4", lib().w4a4_quantize_mxfp4(
        _ptr(x), _dt(x), M, K, had_block, _ptr(xq), lay, _ptr(xs), _stream(x)))
    return xq, xs


def qgemm_mxfp4(xq: torch.Tensor, xs: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor,
                M: int, N: int, K: int, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MXFP4 GEMM on tiled codes and scales."""
    for t, n in ((xq, "xq"), (xs, "xs"), (wq, "wq"), (ws, "ws")):
        _dev(t, n)
    if xq.shape[1] != K // 2 or wq.shape[1] != K // 2 or xq.shape[0] < pad16(M) or \
            wq.shape[0] < pad16(N):
        raise ValueError("codes do not match the tiled layouts of M, N, K")
    if xs.numel() < mx_scale_bytes(M, K, "packed_tiled") or ws.numel() < mx_scale_bytes(N, K, "packed_tiled"):
        raise ValueError("scale arrays too small")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    _check("qgemm_mxfp4", lib().w4a4_qgemm_mxfp4(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _stream(xq)))
    return y


def qlinear_forward_mxfp4(x: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor, N: int,
                          had_block: int, At: Optional[torch.Tensor] = None,
                          Bt: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The MXFP4 layer on tiled MXFP4 weights (codes wq, scales ws)."""
    _dev(x, "x")
    _dev(wq, "wq")
    _dev(ws, "ws")
    M, K = x.shape
    if wq.shape[0] < pad16(N) or wq.shape[1] != K // 2 or ws.numel() < mx_scale_bytes(N, K, "packed_tiled"):
        raise ValueError("wq / ws do not match N and K")
    rank = 0 if At is None else At.shape[0]
    if rank:
        if Bt is None or At.dtype != x.dtype or Bt.dtype != x.dtype:
            raise ValueError("At and Bt must both be given in x's dtype")
        if tuple(At.shape) != (rank, K) or tuple(Bt.shape) != (N, rank):
            raise ValueError("At must be [rank, K] and Bt [N, rank]")
        _dev(At, "At")
        _dev(Bt, "Bt")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = qlinear_workspace(M, N, K, rank, x.device)
    _check("qlinear_forward_mxfp4", lib().w4a4_qlinear_forward_mxfp4(
        _ptr(x), _dt(x), _ptr(wq), _ptr(ws), M, N, K, had_block, _ptr(At), _ptr(Bt), rank,
        _ptr(y), _ptr(workspace), workspace.numel(), _stream(x)))
    return y
