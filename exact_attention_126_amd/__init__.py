"""MI355X exact attention: Python binding of the C ABI in include/fa.h.

The functions below only marshal arguments (torch tensors -> device pointers, sizes, the
current HIP stream) and call libfa.so; every step of the computation runs in the library's
HIP kernels.  There is no fallback: if the library is missing, calls raise.

torch is imported before libfa.so is loaded so that the process maps a single HIP runtime
(torch's) and torch's streams are valid inside the library.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_DTYPE_BF16 = 0
FA_DTYPE_F32 = 1
FA_MASK_NONE = 0
FA_MASK_CAUSAL = 1
FA_MASK_CAUSAL_BOTTOM_RIGHT = 2
MASKS = {"none": FA_MASK_NONE, "causal": FA_MASK_CAUSAL, "causal_bottom_right": FA_MASK_CAUSAL_BOTTOM_RIGHT}
FA_OK = 0
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_ALIGN", 3: "FA_ERR_SHAPE", 4: "FA_ERR_UNSUPPORTED",
                5: "FA_ERR_WORKSPACE", 6: "FA_ERR_HIP", 7: "FA_ERR_ARG", 8: "FA_ERR_SCRATCH"}
# Size of the fixed device scratch behind fa_decode_noalloc (FA_DECODE_NOALLOC_SCRATCH_BYTES)
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20
EXPORTED = ["fa_fwd", "fa_fwd_ex", "fa_fwd_fp8", "fa_fwd_masked_workspace_bytes", "fa_fwd_masked", "fa_decode_workspace_bytes", "fa_decode_split", "fa_decode_split_ex",
            "fa_decode_split_fp8kv", "fa_decode_combine", "fa_decode_noalloc", "fa_bwd_workspace_bytes", "fa_bwd",
            "fa_status_string"]

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({fa_status_string(status)})")


def lib() -> ctypes.CDLL:
    """Load libfa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Opens a build of the library at `path` and declares its entry points (the functions of this
    module call whichever library lib() returns).  Raises if the file does not exist."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m exact_attention_126_amd.build`")
    L = ctypes.CDLL(path)
    i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, f32, i32, vp]
    L.fa_fwd.restype = i32
    L.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, f32, i32, vp]
    L.fa_fwd_ex.restype = i32
    L.fa_decode_split_ex.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_decode_split_ex.restype = i32
    L.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, f32, vp]
    L.fa_fwd_fp8.restype = i32
    L.fa_decode_split_fp8kv.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, i64, i64, f32, i32,
                                        vp]
    L.fa_decode_split_fp8kv.restype = i32
    L.fa_decode_workspace_bytes.argtypes = [i64, i64, i64, i32]
    L.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.fa_decode_split.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_decode_split.restype = i32
    L.fa_decode_combine.argtypes = [vp, ctypes.c_size_t, vp, vp, i64, i64, i64, i32, i32, vp]
    L.fa_decode_combine.restype = i32
    L.fa_fwd_masked_workspace_bytes.argtypes = [i64, i64]
    L.fa_fwd_masked_workspace_bytes.restype = ctypes.c_size_t
    L.fa_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp, ctypes.c_size_t, f32,
                                i32, vp]
    L.fa_fwd_masked.restype = i32
    L.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32, vp]
    L.fa_decode_noalloc.restype = i32
    L.fa_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, i64, i64, i64, i32,
                         f32, i32, vp]
    L.fa_bwd.restype = i32
    L.fa_status_string.argtypes = [i32]
    L.fa_status_string.restype = ctypes.c_char_p
    return L


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_shapes(q, k, v, o=None, lse=None, same_heads: bool = True):
    """The library sees only pointers and sizes, so the sizes it is given must describe the tensors."""
    if q.dim() != 4 or k.dim() != 4 or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}: need [B,H,N,d] and v like k")
    if k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3] or (same_heads and k.shape[1] != q.shape[1]):
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree on batch, heads or head dim")
    if o is not None and tuple(o.shape) != tuple(q.shape):
        raise ValueError(f"o {tuple(o.shape)} must have the shape of q {tuple(q.shape)}")
    if lse is not None and tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError(f"lse {tuple(lse.shape)} must be {tuple(q.shape[:3])}")


def _raise(status: int, where: str):
    if status != FA_OK:
        raise FAError(status, where)


def fa_fwd(q, k, v, o, lse, causal: bool = False, scale: float | None = None, stream=None) -> None:
    """Fused attention forward into caller-provided o [B,H,Nq,d] and lse [B,H,Nq] (float32)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(t, n, q.dtype)
    _check(lse, "lse", torch.float32)
    _check_shapes(q, k, v, o, lse)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, int(bool(causal)),
                      float(scale), _dtype_code(q), _stream(stream))
    _raise(st, "fa_fwd")


def fa_fwd_ex(q, k, v, o, lse, mask=FA_MASK_NONE, scale: float | None = None, stream=None) -> None:
    """Forward with grouped K/V heads (k, v [B,H_kv,Nk,d], H_kv dividing H) and a causal alignment
    (FA_MASK_NONE, FA_MASK_CAUSAL top-left, FA_MASK_CAUSAL_BOTTOM_RIGHT; or their MASKS names)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(t, n, q.dtype)
    _check(lse, "lse", torch.float32)
    _check_shapes(q, k, v, o, lse, same_heads=False)
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    m = MASKS[mask] if isinstance(mask, str) else int(mask)
    st = lib().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, H_kv, Nq, Nk, d, m, float(scale),
                         _dtype_code(q), _stream(stream))
    _raise(st, "fa_fwd_ex")


def fa_fwd_masked_workspace_bytes(Nq: int, Nk: int) -> int:
    return int(lib().fa_fwd_masked_workspace_bytes(Nq, Nk))


def fa_fwd_masked(q, k, v, o, lse, mask, workspace, scale: float | None = None, stream=None) -> None:
    """Forward with an element mask: mask [Nq, ceil(Nk/64)] 64-bit words (int64 or uint64 device
    tensor; bit j % 64 of word [i][j // 64] set iff key j is visible to query row i), shared by every
    batch and head; workspace of fa_fwd_masked_workspace_bytes(Nq, Nk) bytes.  k, v may have fewer
    heads than q (grouped heads, as fa_fwd_ex)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(t, n, q.dtype)
    _check(lse, "lse", torch.float32)
    _check(workspace, "workspace")
    _check_shapes(q, k, v, o, lse, same_heads=False)
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    _check(mask, "mask")
    if mask.dtype not in (torch.int64, torch.uint64) or tuple(mask.shape) != (Nq, (Nk + 63) // 64):
        raise ValueError(f"mask must be [Nq, ceil(Nk/64)] = {(Nq, (Nk + 63) // 64)} 64-bit words, got "
                         f"{tuple(mask.shape)} {mask.dtype}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, H_kv, Nq, Nk, d, _ptr(mask),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), float(scale),
                             _dtype_code(q), _stream(stream))
    _raise(st, "fa_fwd_masked")


def _check_codes(t, name):
    _check(t, name)
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn), got {t.dtype}")


def fa_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, mask=FA_MASK_NONE, scale: float | None = None,
               stream=None) -> None:
    """Forward with FP8 inputs: q [B,H,Nq,d], k/v [B,H_kv,Nk,d] E4M3 codes; q_scale [B,H] and
    k_scale/v_scale [B,H_kv] float32; o [B,H,Nq,d] bf16 and lse [B,H,Nq] float32 out."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_codes(t, n)
    _check(o, "o", torch.bfloat16)
    _check(lse, "lse", torch.float32)
    _check_shapes(q, k, v, o, lse, same_heads=False)
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    for t, n, cnt in ((q_scale, "q_scale", B * H), (k_scale, "k_scale", B * H_kv), (v_scale, "v_scale", B * H_kv)):
        _check(t, n, torch.float32)
        if t.numel() != cnt:
            raise ValueError(f"{n} must hold {cnt} scales, has {t.numel()}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    m = MASKS[mask] if isinstance(mask, str) else int(mask)
    st = lib().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(o), _ptr(lse),
                          B, H, H_kv, Nq, Nk, d, m, float(scale), _stream(stream))
    _raise(st, "fa_fwd_fp8")


def fa_decode_workspace_bytes(B: int, H: int, d: int, num_splits: int) -> int:
    return int(lib().fa_decode_workspace_bytes(B, H, d, num_splits))


def fa_decode_split(q, k, v, workspace, num_splits: int, scale: float | None = None, stream=None) -> None:
    """Per-split partials of one-token decode; q [B,H,1,d], k/v [B,H,Nk,d], workspace uint8/float32."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype)
    _check(workspace, "workspace")
    _check_shapes(q, k, v)
    if q.shape[2] != 1:
        raise ValueError(f"decode takes one query token per head, q is {tuple(q.shape)}")
    B, H, _, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_decode_split(_ptr(q), _ptr(k), _ptr(v), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               B, H, Nk, d, float(scale), int(num_splits), _dtype_code(q), _stream(stream))
    _raise(st, "fa_decode_split")


def fa_decode_split_ex(q, k, v, workspace, num_splits: int, scale: float | None = None, stream=None) -> None:
    """Per-split decode partials with grouped K/V heads: q [B,H,1,d], k/v [B,H_kv,Nk,d]."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype)
    _check(workspace, "workspace")
    _check_shapes(q, k, v, same_heads=False)
    if q.shape[2] != 1:
        raise ValueError(f"decode takes one query token per head, q is {tuple(q.shape)}")
    B, H, _, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_decode_split_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), B, H, H_kv, Nk, d, float(scale),
                                  int(num_splits), _dtype_code(q), _stream(stream))
    _raise(st, "fa_decode_split_ex")


def fa_decode_split_fp8kv(q, k, v, k_scale, v_scale, workspace, num_splits: int, scale: float | None = None,
                          stream=None) -> None:
    """Per-split decode partials over an FP8 KV cache: q [B,H,1,d] bf16, k/v [B,H_kv,Nk,d] E4M3
    codes (uint8 or float8_e4m3fn), k_scale/v_scale [B,H_kv] float32 (a code's value times its
    head's scale)."""
    _check(q, "q", torch.bfloat16)
    for t, n in ((k, "k"), (v, "v")):
        _check_codes(t, n)
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _check(t, n, torch.float32)
    _check(workspace, "workspace")
    _check_shapes(q, k, v, same_heads=False)
    if q.shape[2] != 1:
        raise ValueError(f"decode takes one query token per head, q is {tuple(q.shape)}")
    B, H, _, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t.numel() != B * H_kv:
            raise ValueError(f"{n} must hold B*H_kv = {B * H_kv} scales, has {t.numel()}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_decode_split_fp8kv(_ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), B, H, H_kv, Nk, d, float(scale),
                                     int(num_splits), _stream(stream))
    _raise(st, "fa_decode_split_fp8kv")


def fa_decode_combine(workspace, o, lse, num_splits: int, stream=None) -> None:
    """Merge the split partials into o [B,H,1,d] and lse [B,H,1]."""
    if o.dim() != 4 or o.shape[2] != 1:
        raise ValueError(f"o {tuple(o.shape)} must be [B,H,1,d]")
    B, H, _, d = o.shape
    if tuple(lse.shape) != (B, H, 1):
        raise ValueError(f"lse {tuple(lse.shape)} must be {(B, H, 1)}")
    _check(workspace, "workspace")
    _check(o, "o")
    _check(lse, "lse", torch.float32)
    st = lib().fa_decode_combine(_ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(o), _ptr(lse),
                                 B, H, d, int(num_splits), _dtype_code(o), _stream(stream))
    _raise(st, "fa_decode_combine")


def fa_decode_noalloc(q, k, v, o, lse, num_splits: int, scale: float | None = None, stream=None) -> None:
    """One-token decode, split and combine, with the partials in the library's fixed device scratch
    instead of a workspace (nothing is allocated): q [B,H,1,d], k/v [B,H_kv,Nk,d], o [B,H,1,d],
    lse [B,H,1] float32.  Calls that overlap on one GPU share the scratch and race."""
    if o.dim() != 4 or tuple(o.shape) != tuple(q.shape):
        raise ValueError(f"o {tuple(o.shape)} must have the shape of q {tuple(q.shape)}")
    if q.dim() != 4 or tuple(lse.shape) != (q.shape[0], q.shape[1], 1):
        raise ValueError(f"lse {tuple(lse.shape)} must be [B,H,1] for q {tuple(q.shape)}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(t, n, q.dtype)
    _check(lse, "lse", torch.float32)
    _check_shapes(q, k, v, same_heads=False)
    if q.shape[2] != 1:
        raise ValueError(f"decode takes one query token per head, q is {tuple(q.shape)}")
    B, H, _, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, H_kv, Nk, d, float(scale),
                                 int(num_splits), _dtype_code(q), _stream(stream))
    _raise(st, "fa_decode_noalloc")


def fa_bwd_workspace_bytes(B: int, H: int, Nq: int) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, Nq))


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, workspace, mask=FA_MASK_NONE, scale: float | None = None,
           stream=None) -> None:
    """Gradients dq [B,H,Nq,d], dk and dv [B,H_kv,Nk,d] (bf16) of a loss with gradient do w.r.t. the
    forward's o, recomputing P from q, k and the forward's lse; workspace of fa_bwd_workspace_bytes."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, q.dtype)
    _check(lse, "lse", torch.float32)
    _check(workspace, "workspace")
    _check_shapes(q, k, v, o, lse, same_heads=False)
    if tuple(do.shape) != tuple(q.shape) or tuple(dq.shape) != tuple(q.shape) or tuple(dk.shape) != tuple(k.shape) \
            or tuple(dv.shape) != tuple(k.shape):
        raise ValueError("do and dq must have the shape of q, dk and dv the shape of k")
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    m = MASKS[mask] if isinstance(mask, str) else int(mask)
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                      _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, H_kv, Nq, Nk, d, m,
                      float(scale), _dtype_code(q), _stream(stream))
    _raise(st, "fa_bwd")


# ---- conveniences that allocate the outputs with torch and call the entry points above
def attention(q, k, v, causal: bool = False, scale: float | None = None, stream=None, mask=None):
    """(o, lse) = attention(q, k, v): allocates the outputs and calls fa_fwd, or fa_fwd_ex when
    k/v have fewer heads than q or a mask (fa_mask_t value or MASKS name) is given."""
    B, H, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if mask is None and k.shape[1] == H:
        fa_fwd(q, k, v, o, lse, causal, scale, stream)
    else:
        fa_fwd_ex(q, k, v, o, lse, (FA_MASK_CAUSAL if causal else FA_MASK_NONE) if mask is None else mask, scale,
                  stream)
    return o, lse


def attention_masked(q, k, v, mask, scale: float | None = None, stream=None):
    """(o, lse) = fa_fwd_masked with freshly allocated outputs and workspace."""
    B, H, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(16, fa_fwd_masked_workspace_bytes(Nq, k.shape[2])), dtype=torch.uint8, device=q.device)
    fa_fwd_masked(q, k, v, o, lse, mask, ws, scale, stream)
    return o, lse


def attention_fp8(q, k, v, q_scale, k_scale, v_scale, mask=FA_MASK_NONE, scale: float | None = None, stream=None):
    """(o, lse) = fa_fwd_fp8 on E4M3 codes with their per-head scales; o is bf16."""
    B, H, Nq, d = q.shape
    o = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, mask, scale, stream)
    return o, lse


def decode_workspace(q, num_splits: int):
    B, H, _, d = q.shape
    return torch.empty(fa_decode_workspace_bytes(B, H, d, num_splits) // 4, dtype=torch.float32, device=q.device)


def decode(q, k, v, num_splits: int, scale: float | None = None, workspace=None, stream=None):
    """(o, lse) of one-token decode: fa_decode_split (fa_decode_split_ex when k/v have fewer heads
    than q) then fa_decode_combine on the same stream."""
    B, H, _, d = q.shape
    if workspace is None:
        workspace = decode_workspace(q, num_splits)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, 1), dtype=torch.float32, device=q.device)
    if k.shape[1] == H:
        fa_decode_split(q, k, v, workspace, num_splits, scale, stream)
    else:
        fa_decode_split_ex(q, k, v, workspace, num_splits, scale, stream)
    fa_decode_combine(workspace, o, lse, num_splits, stream)
    return o, lse


def decode_fp8kv(q, k, v, k_scale, v_scale, num_splits: int, scale: float | None = None, workspace=None,
                 stream=None):
    """(o, lse) of one-token decode over an FP8 KV cache: fa_decode_split_fp8kv then
    fa_decode_combine (bf16 o) on the same stream."""
    B, H, _, d = q.shape
    if workspace is None:
        workspace = decode_workspace(q, num_splits)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, 1), dtype=torch.float32, device=q.device)
    fa_decode_split_fp8kv(q, k, v, k_scale, v_scale, workspace, num_splits, scale, stream)
    fa_decode_combine(workspace, o, lse, num_splits, stream)
    return o, lse


def attention_backward(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, stream=None, mask=None):
    """(dq, dk, dv) for the forward (o, lse) = attention(q, k, v, causal / mask, scale): allocates the
    gradients and the workspace and calls fa_bwd."""
    B, H, Nq, _ = q.shape
    ws = torch.empty(fa_bwd_workspace_bytes(B, H, Nq) // 4, dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, (FA_MASK_CAUSAL if causal else FA_MASK_NONE) if mask is None else mask,
           scale, stream)
    return dq, dk, dv
