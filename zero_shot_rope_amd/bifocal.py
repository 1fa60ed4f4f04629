"""ctypes binding of the bifocal attention C ABI (include/bifocal.h).

Argument marshalling only: tensors become device pointers and sizes, the current torch
stream becomes the hipStream_t, a negative status becomes a BifocalError. Every step of
the attention runs in the HIP kernels of libbifocal.so. The library is required: when it
is missing the entry points raise instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libbifocal.so"
_lock = threading.Lock()
_lib = None

EXPORTED_SYMBOLS = (
    "bifocal_group_size",
    "bifocal_prefill_workspace_bytes",
    "bifocal_prefill",
    "bifocal_prefill_chunk",
    "bifocal_decode_workspace_bytes",
    "bifocal_decode",
    "bifocal_decode_noalloc",
    "bifocal_decode_step",
    "bifocal_decode_varlen_workspace_bytes",
    "bifocal_decode_varlen",
    "bifocal_prefill_unfused_workspace_bytes",
    "bifocal_prefill_unfused",
    "bifocal_decode_unfused_workspace_bytes",
    "bifocal_decode_unfused",
    "bifocal_positions",
    "bifocal_status_string",
)


class BifocalError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {bifocal_status_string(status)} (status {status})")


def library_path() -> str:
    return os.environ.get("BIFOCAL_LIBRARY", os.path.join(HERE, _LIB_NAME))


def load_library():
    """dlopen libbifocal.so (once) and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library {path} is not built; run `python -m zero_shot_rope_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(path)
        c_i64, c_int, c_vp, c_dbl, c_sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double, ctypes.c_size_t
        fp = ctypes.POINTER(ctypes.c_float)
        lib.bifocal_group_size.argtypes = [c_i64, c_i64]
        lib.bifocal_group_size.restype = c_i64
        lib.bifocal_prefill_workspace_bytes.argtypes = [c_int, c_int, c_int, c_i64]
        lib.bifocal_prefill_workspace_bytes.restype = c_sz
        lib.bifocal_prefill.argtypes = [c_vp, c_vp, c_vp, c_vp, fp, c_int, c_int, c_int, c_int,
                                        c_i64, c_i64, c_i64, c_dbl, c_vp, c_sz, c_vp]
        lib.bifocal_prefill.restype = c_int
        lib.bifocal_prefill_chunk.argtypes = [c_vp, c_vp, c_vp, c_vp, fp, c_int, c_int, c_int, c_int,
                                              c_i64, c_i64, c_i64, c_i64, c_i64, c_dbl, c_vp, c_sz, c_vp]
        lib.bifocal_prefill_chunk.restype = c_int
        lib.bifocal_decode_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_i64]
        lib.bifocal_decode_workspace_bytes.restype = c_sz
        lib.bifocal_decode.argtypes = [c_vp, c_vp, c_vp, c_vp, fp, c_int, c_int, c_int, c_int,
                                       c_i64, c_i64, c_i64, c_i64, c_dbl, c_vp, c_sz, c_vp]
        lib.bifocal_decode.restype = c_int
        lib.bifocal_decode_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, fp, c_int, c_int, c_int, c_int,
                                               c_i64, c_i64, c_i64, c_i64, c_dbl, c_vp]
        lib.bifocal_decode_noalloc.restype = c_int
        lib.bifocal_decode_step.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, fp, c_int, c_int, c_int, c_int,
                                            c_i64, c_i64, c_i64, c_i64, c_dbl, c_vp, c_sz, c_vp]
        lib.bifocal_decode_step.restype = c_int
        lib.bifocal_decode_varlen_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_i64]
        lib.bifocal_decode_varlen_workspace_bytes.restype = c_sz
        lib.bifocal_decode_varlen.argtypes = [c_vp, c_vp, c_vp, c_vp, fp, c_int, c_int, c_int, c_int,
                                              c_vp, c_i64, c_i64, c_i64, c_i64, c_dbl, c_vp, c_sz, c_vp]
        lib.bifocal_decode_varlen.restype = c_int
        lib.bifocal_prefill_unfused_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_i64]
        lib.bifocal_prefill_unfused_workspace_bytes.restype = c_sz
        lib.bifocal_prefill_unfused.argtypes = [c_vp, c_vp, c_vp, c_vp, fp, c_int, c_int, c_int, c_int,
                                                c_i64, c_i64, c_i64, c_dbl, c_vp, c_sz, c_vp]
        lib.bifocal_prefill_unfused.restype = c_int
        lib.bifocal_decode_unfused_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_i64]
        lib.bifocal_decode_unfused_workspace_bytes.restype = c_sz
        lib.bifocal_decode_unfused.argtypes = [c_vp, c_vp, c_vp, c_vp, fp, c_int, c_int, c_int, c_int,
                                               c_i64, c_i64, c_i64, c_i64, c_dbl, c_vp, c_sz, c_vp]
        lib.bifocal_decode_unfused.restype = c_int
        lib.bifocal_positions.argtypes = [c_i64, c_i64, ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int32), c_vp]
        lib.bifocal_positions.restype = c_int
        lib.bifocal_status_string.argtypes = [c_int]
        lib.bifocal_status_string.restype = ctypes.c_char_p
        _lib = lib
        return lib


# ---------------------------------------------------------------------------------------
# Raw entry points (same names and argument order as the C ABI; pointers may be ints)
# ---------------------------------------------------------------------------------------
def bifocal_status_string(status: int) -> str:
    return load_library().bifocal_status_string(int(status)).decode()


def bifocal_group_size(L: int, w_pretrained: int) -> int:
    return int(load_library().bifocal_group_size(int(L), int(w_pretrained)))


def bifocal_prefill_workspace_bytes(batch: int, n_kv_heads: int, head_dim: int, L: int) -> int:
    return int(load_library().bifocal_prefill_workspace_bytes(batch, n_kv_heads, head_dim, int(L)))


def bifocal_decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, max_L: int) -> int:
    return int(load_library().bifocal_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, int(max_L)))


def bifocal_decode_varlen_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                                          max_len: int) -> int:
    return int(load_library().bifocal_decode_varlen_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim,
                                                                    int(max_len)))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _fptr(t):
    p = _ptr(t)
    return None if p is None else ctypes.cast(ctypes.c_void_p(p), ctypes.POINTER(ctypes.c_float))


def _stream(stream, device=None) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def bifocal_prefill(q, k, v, o, lse, batch, n_q_heads, n_kv_heads, head_dim, L, w0, w_pretrained,
                    rope_theta, workspace=None, workspace_bytes=0, stream=None) -> None:
    lib = load_library()
    st = lib.bifocal_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse), batch, n_q_heads, n_kv_heads,
                             head_dim, int(L), int(w0), int(w_pretrained), float(rope_theta), _ptr(workspace),
                             int(workspace_bytes), _stream(stream))
    if st != 0:
        raise BifocalError(st, "bifocal_prefill")


def bifocal_prefill_chunk(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, q_len, q_offset,
                          cache_capacity, w0, w_pretrained, rope_theta, workspace=None, workspace_bytes=0,
                          stream=None) -> None:
    lib = load_library()
    st = lib.bifocal_prefill_chunk(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _fptr(lse), batch, n_q_heads,
                                   n_kv_heads, head_dim, int(q_len), int(q_offset), int(cache_capacity), int(w0),
                                   int(w_pretrained), float(rope_theta), _ptr(workspace), int(workspace_bytes),
                                   _stream(stream))
    if st != 0:
        raise BifocalError(st, "bifocal_prefill_chunk")


def bifocal_decode(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, L, cache_capacity,
                   w0, w_pretrained, rope_theta, workspace, workspace_bytes, stream=None) -> None:
    lib = load_library()
    st = lib.bifocal_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _fptr(lse), batch, n_q_heads,
                            n_kv_heads, head_dim, int(L), int(cache_capacity), int(w0), int(w_pretrained),
                            float(rope_theta), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if st != 0:
        raise BifocalError(st, "bifocal_decode")


def bifocal_decode_noalloc(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, L, cache_capacity,
                           w0, w_pretrained, rope_theta, stream=None) -> None:
    lib = load_library()
    st = lib.bifocal_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _fptr(lse), batch, n_q_heads,
                                    n_kv_heads, head_dim, int(L), int(cache_capacity), int(w0), int(w_pretrained),
                                    float(rope_theta), _stream(stream))
    if st != 0:
        raise BifocalError(st, "bifocal_decode_noalloc")


def bifocal_decode_step(q_raw, k_raw, v_new, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, L,
                        cache_capacity, w0, w_pretrained, rope_theta, workspace, workspace_bytes,
                        stream=None) -> None:
    lib = load_library()
    st = lib.bifocal_decode_step(_ptr(q_raw), _ptr(k_raw), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(o),
                                 _fptr(lse), batch, n_q_heads, n_kv_heads, head_dim, int(L), int(cache_capacity),
                                 int(w0), int(w_pretrained), float(rope_theta), _ptr(workspace), int(workspace_bytes),
                                 _stream(stream))
    if st != 0:
        raise BifocalError(st, "bifocal_decode_step")


def bifocal_decode_varlen(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, seq_lens, max_len,
                          cache_capacity, w0, w_pretrained, rope_theta, workspace, workspace_bytes,
                          stream=None) -> None:
    lib = load_library()
    st = lib.bifocal_decode_varlen(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _fptr(lse), batch, n_q_heads,
                                   n_kv_heads, head_dim, _ptr(seq_lens), int(max_len), int(cache_capacity), int(w0),
                                   int(w_pretrained), float(rope_theta), _ptr(workspace), int(workspace_bytes),
                                   _stream(stream))
    if st != 0:
        raise BifocalError(st, "bifocal_decode_varlen")


def bifocal_prefill_unfused_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                                            L: int) -> int:
    return int(load_library().bifocal_prefill_unfused_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim,
                                                                      int(L)))


def bifocal_prefill_unfused(q, k, v, o, lse, batch, n_q_heads, n_kv_heads, head_dim, L, w0, w_pretrained,
                            rope_theta, workspace, workspace_bytes, stream=None) -> None:
    lib = load_library()
    st = lib.bifocal_prefill_unfused(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _fptr(lse), batch, n_q_heads, n_kv_heads,
                                     head_dim, int(L), int(w0), int(w_pretrained), float(rope_theta), _ptr(workspace),
                                     int(workspace_bytes), _stream(stream))
    if st != 0:
        raise BifocalError(st, "bifocal_prefill_unfused")


def bifocal_decode_unfused_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                                           cache_capacity: int) -> int:
    return int(load_library().bifocal_decode_unfused_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim,
                                                                     int(cache_capacity)))


def bifocal_decode_unfused(q, k_cache, v_cache, o, lse, batch, n_q_heads, n_kv_heads, head_dim, L, cache_capacity,
                           w0, w_pretrained, rope_theta, workspace, workspace_bytes, stream=None) -> None:
    lib = load_library()
    st = lib.bifocal_decode_unfused(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _fptr(lse), batch, n_q_heads,
                                    n_kv_heads, head_dim, int(L), int(cache_capacity), int(w0), int(w_pretrained),
                                    float(rope_theta), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if st != 0:
        raise BifocalError(st, "bifocal_decode_unfused")


def bifocal_positions(L, w_pretrained, f_out, G_out, stream=None) -> None:
    lib = load_library()
    i32p = ctypes.POINTER(ctypes.c_int32)
    fo = None if f_out is None else ctypes.cast(ctypes.c_void_p(_ptr(f_out)), i32p)
    go = None if G_out is None else ctypes.cast(ctypes.c_void_p(_ptr(G_out)), i32p)
    st = lib.bifocal_positions(int(L), int(w_pretrained), fo, go, _stream(stream))
    if st != 0:
        raise BifocalError(st, "bifocal_positions")


# ---------------------------------------------------------------------------------------
# Tensor conveniences: shapes from the tensors, outputs allocated when not given
# ---------------------------------------------------------------------------------------
def _check(t, name, ndim, device=None):
    import torch

    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 CUDA/HIP tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _outputs(out, lse, want_lse, out_shape, lse_shape, device):
    """Allocate the outputs, or check the caller's: the kernels write exactly these shapes."""
    import torch

    if out is None:
        out = torch.empty(out_shape, dtype=torch.bfloat16, device=device)
    elif (not isinstance(out, torch.Tensor) or out.dtype != torch.bfloat16 or out.device != device
          or not out.is_contiguous() or tuple(out.shape) != tuple(out_shape)):
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape {tuple(out_shape)} on {device}")
    if lse is None and want_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=device)
    elif lse is not None and (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32
                              or lse.device != device or not lse.is_contiguous()
                              or tuple(lse.shape) != tuple(lse_shape)):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {tuple(lse_shape)} on {device}")
    return out, lse


def _workspace(ws, need, device):
    """The caller's workspace (any dtype; its size is checked by the library), or a new one."""
    import torch

    if ws is None:
        return torch.empty(max(need, 4), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return ws


def prefill(q, k, v, *, w0: int, w_pretrained: int, rope_theta: float, out=None, lse=None,
            want_lse: bool = False, workspace=None, stream=None):
    """q [B, L, Hq, D], k/v [B, L, Hkv, D] (bf16, post-base-RoPE) -> o (and lse [B, Hq, L]).

    `workspace`: None runs the single-launch fused mode; a tensor (>= the workspace query)
    runs the mode that rotates the keys once into it first; "auto" allocates one.
    """
    import torch

    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, 4, q.device)
    B, L, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != L or k.shape[3] != D:
        raise ValueError("k/v shapes do not match q")
    out, lse = _outputs(out, lse, want_lse, q.shape, (B, Hq, L), q.device)
    if isinstance(workspace, str) and workspace == "auto":
        workspace = torch.empty(bifocal_prefill_workspace_bytes(B, k.shape[2], D, L), dtype=torch.uint8,
                                device=q.device)
    elif workspace is not None:
        workspace = _workspace(workspace, 0, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    bifocal_prefill(q, k, v, out, lse, B, Hq, k.shape[2], D, L, w0, w_pretrained, rope_theta, workspace, ws_bytes,
                    _stream(stream, q.device))
    return (out, lse) if (want_lse or lse is not None) else out


def prefill_chunk(q, k_cache, v_cache, *, q_offset: int, w0: int, w_pretrained: int, rope_theta: float, out=None,
                  lse=None, want_lse: bool = False, workspace=None, stream=None):
    """q [B, Lq, Hq, D] at positions q_offset .. q_offset + Lq - 1 against caches [B, cap, Hkv, D]
    holding positions 0 .. q_offset + Lq - 1 -> o [B, Lq, Hq, D] (and lse [B, Hq, Lq]).

    `workspace`: None (single launch), a tensor (>= the workspace query for L = q_offset + Lq)
    or "auto", as for prefill.
    """
    import torch

    _check(q, "q", 4)
    _check(k_cache, "k_cache", 4, q.device)
    _check(v_cache, "v_cache", 4, q.device)
    B, Lq, Hq, D = q.shape
    cap, Hkv = k_cache.shape[1], k_cache.shape[2]
    if v_cache.shape != k_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shapes do not match q")
    L = int(q_offset) + Lq
    out, lse = _outputs(out, lse, want_lse, q.shape, (B, Hq, Lq), q.device)
    if isinstance(workspace, str) and workspace == "auto":
        workspace = torch.empty(bifocal_prefill_workspace_bytes(B, Hkv, D, L), dtype=torch.uint8, device=q.device)
    elif workspace is not None:
        workspace = _workspace(workspace, 0, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    bifocal_prefill_chunk(q, k_cache, v_cache, out, lse, B, Hq, Hkv, D, Lq, q_offset, cap, w0, w_pretrained,
                          rope_theta, workspace, ws_bytes, _stream(stream, q.device))
    return (out, lse) if (want_lse or lse is not None) else out


def decode(q, k_cache, v_cache, *, L: int, w0: int, w_pretrained: int, rope_theta: float, workspace=None,
           out=None, lse=None, want_lse: bool = False, stream=None):
    """q [B, Hq, D]; caches [B, Lcap, Hkv, D] (bf16) -> o [B, Hq, D] (and lse [B, Hq])."""
    import torch

    _check(q, "q", 3)
    _check(k_cache, "k_cache", 4, q.device)
    _check(v_cache, "v_cache", 4, q.device)
    B, Hq, D = q.shape
    cap, Hkv = k_cache.shape[1], k_cache.shape[2]
    if v_cache.shape != k_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shapes do not match q")
    workspace = _workspace(workspace, bifocal_decode_workspace_bytes(B, Hq, Hkv, D, L), q.device)
    out, lse = _outputs(out, lse, want_lse, q.shape, (B, Hq), q.device)
    bifocal_decode(q, k_cache, v_cache, out, lse, B, Hq, Hkv, D, L, cap, w0, w_pretrained, rope_theta,
                   workspace, workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    return (out, lse) if (want_lse or lse is not None) else out


def decode_noalloc(q, k_cache, v_cache, *, L: int, w0: int, w_pretrained: int, rope_theta: float, out=None,
                   lse=None, want_lse: bool = False, stream=None):
    """`decode` through the entry point that allocates nothing: the split partials live in the
    library's static scratch of the inputs' device (outputs are still allocated here when not
    given). Calls that overlap on one device race on that scratch."""
    import torch

    _check(q, "q", 3)
    _check(k_cache, "k_cache", 4, q.device)
    _check(v_cache, "v_cache", 4, q.device)
    B, Hq, D = q.shape
    cap, Hkv = k_cache.shape[1], k_cache.shape[2]
    if v_cache.shape != k_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shapes do not match q")
    out, lse = _outputs(out, lse, want_lse, q.shape, (B, Hq), q.device)
    with torch.cuda.device(q.device):  # the library uses the current device's scratch
        bifocal_decode_noalloc(q, k_cache, v_cache, out, lse, B, Hq, Hkv, D, L, cap, w0, w_pretrained, rope_theta,
                               _stream(stream, q.device))
    return (out, lse) if (want_lse or lse is not None) else out


def decode_step(q_raw, k_raw, v_new, k_cache, v_cache, *, L: int, w0: int, w_pretrained: int, rope_theta: float,
                workspace=None, out=None, lse=None, want_lse: bool = False, stream=None):
    """The new token at p = L - 1 from raw (pre-RoPE) vectors: q_raw [B, Hq, D], k_raw and v_new
    [B, Hkv, D]. Writes its rotated key and its value into cache row p (in place), then decodes
    -> o [B, Hq, D] (and lse [B, Hq])."""
    import torch

    _check(q_raw, "q_raw", 3)
    _check(k_raw, "k_raw", 3, q_raw.device)
    _check(v_new, "v_new", 3, q_raw.device)
    _check(k_cache, "k_cache", 4, q_raw.device)
    _check(v_cache, "v_cache", 4, q_raw.device)
    B, Hq, D = q_raw.shape
    cap, Hkv = k_cache.shape[1], k_cache.shape[2]
    if v_cache.shape != k_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shapes do not match q_raw")
    if k_raw.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D):
        raise ValueError("k_raw / v_new must be [batch, n_kv_heads, head_dim]")
    workspace = _workspace(workspace, bifocal_decode_workspace_bytes(B, Hq, Hkv, D, L), q_raw.device)
    out, lse = _outputs(out, lse, want_lse, q_raw.shape, (B, Hq), q_raw.device)
    bifocal_decode_step(q_raw, k_raw, v_new, k_cache, v_cache, out, lse, B, Hq, Hkv, D, L, cap, w0, w_pretrained,
                        rope_theta, workspace, workspace.numel() * workspace.element_size(),
                        _stream(stream, q_raw.device))
    return (out, lse) if (want_lse or lse is not None) else out


def decode_varlen(q, k_cache, v_cache, seq_lens, *, max_len: int, w0: int, w_pretrained: int, rope_theta: float,
                  workspace=None, out=None, lse=None, want_lse: bool = False, stream=None):
    """q [B, Hq, D]; caches [B, Lcap, Hkv, D]; seq_lens int32 [B] on the device (each <= max_len)
    -> o [B, Hq, D] (and lse [B, Hq]); sequence b decodes at its own length seq_lens[b]."""
    import torch

    _check(q, "q", 3)
    _check(k_cache, "k_cache", 4, q.device)
    _check(v_cache, "v_cache", 4, q.device)
    if not isinstance(seq_lens, torch.Tensor) or seq_lens.dtype != torch.int32 or seq_lens.device != q.device \
            or not seq_lens.is_contiguous() or seq_lens.shape != (q.shape[0],):
        raise ValueError("seq_lens must be a contiguous int32 tensor of shape [batch] on the inputs' device")
    B, Hq, D = q.shape
    cap, Hkv = k_cache.shape[1], k_cache.shape[2]
    if v_cache.shape != k_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shapes do not match q")
    workspace = _workspace(workspace, bifocal_decode_varlen_workspace_bytes(B, Hq, Hkv, D, max_len), q.device)
    out, lse = _outputs(out, lse, want_lse, q.shape, (B, Hq), q.device)
    bifocal_decode_varlen(q, k_cache, v_cache, out, lse, B, Hq, Hkv, D, seq_lens, max_len, cap, w0, w_pretrained,
                          rope_theta, workspace, workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    return (out, lse) if (want_lse or lse is not None) else out


def prefill_unfused(q, k, v, *, w0: int, w_pretrained: int, rope_theta: float, out=None, lse=None,
                    want_lse: bool = False, workspace=None, stream=None):
    """The three-pass form of `prefill` (same shapes and result); allocates its workspace when
    none is given."""
    import torch

    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, 4, q.device)
    B, L, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != L or k.shape[3] != D:
        raise ValueError("k/v shapes do not match q")
    out, lse = _outputs(out, lse, want_lse, q.shape, (B, Hq, L), q.device)
    workspace = _workspace(workspace, bifocal_prefill_unfused_workspace_bytes(B, Hq, k.shape[2], D, L), q.device)
    bifocal_prefill_unfused(q, k, v, out, lse, B, Hq, k.shape[2], D, L, w0, w_pretrained, rope_theta, workspace,
                            workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    return (out, lse) if (want_lse or lse is not None) else out


def decode_unfused(q, k_cache, v_cache, *, L: int, w0: int, w_pretrained: int, rope_theta: float, workspace=None,
                   out=None, lse=None, want_lse: bool = False, stream=None):
    """The three-pass form of `decode` (same shapes and result)."""
    import torch

    _check(q, "q", 3)
    _check(k_cache, "k_cache", 4, q.device)
    _check(v_cache, "v_cache", 4, q.device)
    B, Hq, D = q.shape
    cap, Hkv = k_cache.shape[1], k_cache.shape[2]
    if v_cache.shape != k_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shapes do not match q")
    workspace = _workspace(workspace, bifocal_decode_unfused_workspace_bytes(B, Hq, Hkv, D, cap), q.device)
    out, lse = _outputs(out, lse, want_lse, q.shape, (B, Hq), q.device)
    bifocal_decode_unfused(q, k_cache, v_cache, out, lse, B, Hq, Hkv, D, L, cap, w0, w_pretrained, rope_theta,
                           workspace, workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    return (out, lse) if (want_lse or lse is not None) else out


def positions(L: int, w_pretrained: int, device="cuda", stream=None):
    """Run the device position arithmetic: returns (f int32 [L], G int)."""
    import torch

    f = torch.empty(L, dtype=torch.int32, device=device)
    g = torch.empty(1, dtype=torch.int32, device=device)
    bifocal_positions(L, w_pretrained, f, g, _stream(stream, f.device))
    return f, int(g.item())
