"""Python binding of libdetattn.so: argument marshalling only.

The functions named like the C entry points (``attn_prefill_fwd``,
``attn_decode_split_fwd``, ``attn_paged_extend_fwd``, ``attn_chunk_merge``,
``attn_partials_bytes``, ``attn_extend_workspace_bytes``, ``attn_num_chunks``,
``attn_status_str``, and the GEMM's
``det_gemm_fwd``, ``det_gemm_workspace_bytes``, ``det_gemm_num_chunks``,
``det_gemm_num_configs``, ``det_gemm_config_tile``) take torch
tensors that already live on the GPU, pass their device pointers and sizes to
the C ABI and raise ``DetAttnError`` on a non-zero status.  ``prefill``,
``decode``, ``paged_extend`` and ``gemm`` additionally
allocate the outputs (and the partials of the split schedule) with torch and
chain the split and merge launches on the current stream.  Every step of the
computation runs in the HIP kernels of the library; there is no fallback: if the
library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "DetAttnError", "BF16", "FP8_E4M3", "MONOLITHIC", "SPLIT", "BLOCK_KEYS", "CHUNK_KEYS",
    "PAGE_SIZE", "library_path", "load_library", "attn_status_str", "attn_num_chunks",
    "attn_partials_bytes", "attn_extend_workspace_bytes", "attn_prefill_fwd", "attn_decode_split_fwd", "attn_paged_extend_fwd",
    "attn_chunk_merge", "attn_decode_fwd_noalloc", "DECODE_SCRATCH_BYTES", "prefill", "decode",
    "paged_extend", "WEIGHT_NK", "WEIGHT_KN",
    "GEMM_BLOCK_K", "GEMM_CHUNK_K", "det_gemm_num_chunks", "det_gemm_workspace_bytes",
    "det_gemm_num_configs", "det_gemm_config_tile", "det_gemm_fwd", "gemm",
]

BF16, FP8_E4M3 = 0, 1
MONOLITHIC, SPLIT = 0, 1
BLOCK_KEYS, CHUNK_KEYS, PAGE_SIZE = 64, 512, 16
WEIGHT_NK, WEIGHT_KN = 0, 1
GEMM_BLOCK_K, GEMM_CHUNK_K = 64, 1024
DECODE_SCRATCH_BYTES = 128 << 20  # static partials of attn_decode_fwd_noalloc, per GPU

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None


class DetAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {attn_status_str(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libdetattn.so")


def load_library() -> ctypes.CDLL:
    """Load the in-tree HIP library; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m deterministic_flash_attention_amd.build`")
    lib = ctypes.CDLL(path)
    c_i32, c_i64, c_f32, c_sz, c_p = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                      ctypes.c_size_t, ctypes.c_void_p)
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_num_chunks.argtypes = [c_i32]
    lib.attn_num_chunks.restype = c_i32
    lib.attn_partials_bytes.argtypes = [c_i64, c_i32, c_i32, c_i32]
    lib.attn_partials_bytes.restype = c_sz
    lib.attn_extend_workspace_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32]
    lib.attn_extend_workspace_bytes.restype = c_sz
    lib.attn_prefill_fwd.argtypes = [c_i32, c_p, c_p, c_p, c_p, c_p, c_i32, c_i32, c_i32, c_i64,
                                     c_i64, c_i32, c_i32, c_i32, c_f32, c_i32, c_i32, c_i32,
                                     c_f32, c_f32, c_f32, c_i32, c_p, c_p, c_p, c_sz, c_p]
    lib.attn_prefill_fwd.restype = ctypes.c_int
    lib.attn_decode_split_fwd.argtypes = [c_i32, c_p, c_p, c_p, c_i64, c_i64, c_i64, c_i64, c_p,
                                          c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                          c_i32, c_f32, c_f32, c_f32, c_f32, c_i32, c_p, c_sz,
                                          c_p, c_p, c_p]
    lib.attn_decode_split_fwd.restype = ctypes.c_int
    lib.attn_paged_extend_fwd.argtypes = [c_i32, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i64, c_i64,
                                          c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i64, c_i32,
                                          c_i32, c_i32, c_i32, c_f32, c_i32, c_i32, c_i32, c_f32,
                                          c_f32, c_f32, c_i32, c_p, c_p, c_p, c_sz, c_p]
    lib.attn_paged_extend_fwd.restype = ctypes.c_int
    lib.attn_chunk_merge.argtypes = [c_p, c_sz, c_i64, c_i32, c_i32, c_i32, c_f32, c_p, c_p, c_p]
    lib.attn_chunk_merge.restype = ctypes.c_int
    lib.attn_decode_fwd_noalloc.argtypes = [c_i32, c_p, c_p, c_p, c_i64, c_i64, c_i64, c_i64,
                                            c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                            c_i32, c_i32, c_f32, c_f32, c_f32, c_f32, c_p, c_p,
                                            c_p]
    lib.attn_decode_fwd_noalloc.restype = ctypes.c_int
    lib.det_gemm_num_chunks.argtypes = [c_i64]
    lib.det_gemm_num_chunks.restype = c_i32
    lib.det_gemm_workspace_bytes.argtypes = [c_i64, c_i64, c_i64]
    lib.det_gemm_workspace_bytes.restype = c_sz
    lib.det_gemm_num_configs.argtypes = []
    lib.det_gemm_num_configs.restype = c_i32
    lib.det_gemm_config_tile.argtypes = [c_i32, ctypes.POINTER(c_i32), ctypes.POINTER(c_i32)]
    lib.det_gemm_config_tile.restype = ctypes.c_int
    lib.det_gemm_fwd.argtypes = [c_p, c_i64, c_p, c_i64, c_i32, c_p, c_i64, c_i64, c_i64, c_i64,
                                 c_i32, c_i32, c_p, c_sz, c_p]
    lib.det_gemm_fwd.restype = ctypes.c_int
    _LIB = lib
    return lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the C ABI must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DetAttnError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported input dtype {t.dtype}")


# ---------------------------------------------------------------- C-ABI mirrors
def attn_status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def attn_num_chunks(max_seqlen_k: int) -> int:
    return int(load_library().attn_num_chunks(int(max_seqlen_k)))


def attn_partials_bytes(rows: int, num_heads_q: int, max_chunks: int, head_dim: int) -> int:
    return int(load_library().attn_partials_bytes(int(rows), int(num_heads_q), int(max_chunks),
                                                  int(head_dim)))


def attn_extend_workspace_bytes(batch: int, num_heads_q: int, num_heads_kv: int,
                                max_chunks: int, head_dim: int) -> int:
    return int(load_library().attn_extend_workspace_bytes(int(batch), int(num_heads_q),
                                                          int(num_heads_kv), int(max_chunks),
                                                          int(head_dim)))


def attn_prefill_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                     softmax_scale: float, causal: bool, schedule: int = MONOLITHIC,
                     o=None, lse=None, partials=None, descales=(1.0, 1.0, 1.0),
                     window=(-1, -1), stream=None) -> None:
    """Mirror of the C ``attn_prefill_fwd``; outputs are caller-provided tensors."""
    lib = load_library()
    st = lib.attn_prefill_fwd(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        int(cu_seqlens_q.numel() - 1), int(max_seqlen_q), int(max_seqlen_k), int(q.shape[0]),
        int(k.shape[0]), int(q.shape[1]), int(k.shape[1]), int(q.shape[2]), float(softmax_scale),
        int(bool(causal)), int(window[0]), int(window[1]), float(descales[0]), float(descales[1]),
        float(descales[2]), int(schedule), _ptr(o), _ptr(lse), _ptr(partials),
        0 if partials is None else partials.numel() * partials.element_size(), _stream(stream))
    _check("attn_prefill_fwd", st)


def _cache_geometry(k_cache, kv_layout: str):
    """(num_pages, page_size, Hkv, D) and the (page, token, head) element strides of a
    contiguous paged cache: "NHD" is [num_pages, 16, Hkv, D] (tokens outer), "HND" is
    [num_pages, Hkv, 16, D] (heads outer, each head's page rows contiguous)."""
    if kv_layout == "NHD":
        npages, psize, hkv, d = k_cache.shape
        return npages, psize, hkv, d, psize * hkv * d, hkv * d, d
    if kv_layout == "HND":
        npages, hkv, psize, d = k_cache.shape
        return npages, psize, hkv, d, hkv * psize * d, d, psize * d
    raise ValueError(f"kv_layout must be 'NHD' or 'HND', not {kv_layout!r}")


def attn_decode_split_fwd(q, k_cache, v_cache, page_table, context_lens, max_context_len: int,
                          softmax_scale: float, schedule: int = SPLIT, partials=None, o=None,
                          lse=None, descales=(1.0, 1.0, 1.0), window_left: int = -1,
                          stream=None, kv_layout: str = "NHD") -> None:
    """Mirror of the C ``attn_decode_split_fwd`` for contiguous caches in the
    "NHD" [num_pages, 16, Hkv, D] or "HND" [num_pages, Hkv, 16, D] layout."""
    lib = load_library()
    npages, psize, hkv, d, s_page, s_tok, s_head = _cache_geometry(k_cache, kv_layout)
    st = lib.attn_decode_split_fwd(
        _dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), int(npages),
        int(s_page), int(s_tok), int(s_head), _ptr(page_table), int(page_table.shape[1]),
        _ptr(context_lens), int(max_context_len), int(window_left), int(q.shape[0]), int(psize),
        int(q.shape[1]), int(hkv), int(d), float(softmax_scale), float(descales[0]),
        float(descales[1]),
        float(descales[2]), int(schedule), _ptr(partials),
        0 if partials is None else partials.numel() * partials.element_size(), _ptr(o),
        _ptr(lse), _stream(stream))
    _check("attn_decode_split_fwd", st)


def attn_paged_extend_fwd(q, cu_seqlens_q, k_cache, v_cache, page_table, context_lens,
                          max_seqlen_q: int, max_context_len: int, softmax_scale: float,
                          causal: bool, schedule: int = MONOLITHIC, o=None, lse=None,
                          partials=None, descales=(1.0, 1.0, 1.0), window=(-1, -1),
                          stream=None, kv_layout: str = "NHD") -> None:
    """Mirror of the C ``attn_paged_extend_fwd`` for contiguous caches in the
    "NHD" [num_pages, 16, Hkv, D] or "HND" [num_pages, Hkv, 16, D] layout.
    ``partials``: the split schedule's chunk partials, or for the monolithic
    schedule an optional workspace of ``attn_extend_workspace_bytes`` bytes
    whose counters start at zero (a ``torch.zeros`` buffer)."""
    lib = load_library()
    npages, psize, hkv, d, s_page, s_tok, s_head = _cache_geometry(k_cache, kv_layout)
    st = lib.attn_paged_extend_fwd(
        _dtype_code(q), _ptr(q), _ptr(cu_seqlens_q), _ptr(k_cache), _ptr(v_cache), int(npages),
        int(s_page), int(s_tok), int(s_head), _ptr(page_table), int(page_table.shape[1]),
        _ptr(context_lens), int(cu_seqlens_q.numel() - 1), int(max_seqlen_q),
        int(max_context_len), int(q.shape[0]), int(psize), int(q.shape[1]), int(hkv), int(d),
        float(softmax_scale), int(bool(causal)), int(window[0]), int(window[1]),
        float(descales[0]), float(descales[1]), float(descales[2]), int(schedule), _ptr(o),
        _ptr(lse), _ptr(partials),
        0 if partials is None else partials.numel() * partials.element_size(), _stream(stream))
    _check("attn_paged_extend_fwd", st)


def attn_chunk_merge(partials, rows: int, num_heads_q: int, max_chunks: int, head_dim: int,
                     o, lse=None, v_descale: float = 1.0, stream=None) -> None:
    """Mirror of the C ``attn_chunk_merge``."""
    lib = load_library()
    st = lib.attn_chunk_merge(_ptr(partials),
                              0 if partials is None else partials.numel() * partials.element_size(),
                              int(rows), int(num_heads_q), int(max_chunks), int(head_dim),
                              float(v_descale), _ptr(o), _ptr(lse), _stream(stream))
    _check("attn_chunk_merge", st)


def attn_decode_fwd_noalloc(q, k_cache, v_cache, page_table, context_lens,
                            max_context_len: int, softmax_scale: float, o, lse=None,
                            descales=(1.0, 1.0, 1.0), window_left: int = -1, stream=None,
                            kv_layout: str = "NHD") -> None:
    """Mirror of the C ``attn_decode_fwd_noalloc``: split decode plus merge
    with the partials in the library's static device scratch; ``o`` (and
    ``lse``) are caller-provided, nothing is allocated."""
    lib = load_library()
    npages, psize, hkv, d, s_page, s_tok, s_head = _cache_geometry(k_cache, kv_layout)
    st = lib.attn_decode_fwd_noalloc(
        _dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), int(npages), int(s_page),
        int(s_tok), int(s_head), _ptr(page_table), int(page_table.shape[1]), _ptr(context_lens),
        int(max_context_len), int(window_left), int(q.shape[0]), int(psize), int(q.shape[1]),
        int(hkv), int(d), float(softmax_scale), float(descales[0]), float(descales[1]),
        float(descales[2]), _ptr(o), _ptr(lse), _stream(stream))
    _check("attn_decode_fwd_noalloc", st)


def _rows_ptr(t: Optional[torch.Tensor]) -> Tuple[Optional[int], int]:
    """Pointer and row stride (elements) of a 2-D tensor with unit column stride."""
    if t is None:
        return None, 0
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("GEMM operands must be 2-D with contiguous rows")
    return t.data_ptr(), int(t.stride(0)) if t.shape[0] > 1 else int(max(t.stride(0), t.shape[1]))


def det_gemm_num_chunks(k: int) -> int:
    return int(load_library().det_gemm_num_chunks(int(k)))


def det_gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(load_library().det_gemm_workspace_bytes(int(m), int(n), int(k)))


def det_gemm_num_configs() -> int:
    return int(load_library().det_gemm_num_configs())


def det_gemm_config_tile(config: int) -> Tuple[int, int]:
    bm, bn = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("det_gemm_config_tile",
           load_library().det_gemm_config_tile(int(config), ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def det_gemm_fwd(a, w, c, weight_layout: int = WEIGHT_NK, schedule: int = MONOLITHIC,
                 config: int = -1, workspace=None, stream=None) -> None:
    """Mirror of the C ``det_gemm_fwd``: C = A W^T (W [N, K]) or A W (W [K, N]).
    Row strides are taken from the tensors (rows must be contiguous)."""
    m, k = a.shape
    n = w.shape[0] if weight_layout == WEIGHT_NK else w.shape[1]
    if c.shape[0] != m or c.shape[1] != n:
        raise ValueError("C must be [M, N]")
    pa, lda = _rows_ptr(a)
    pw, ldw = _rows_ptr(w)
    pc, ldc = _rows_ptr(c)
    st = load_library().det_gemm_fwd(
        pa, lda, pw, ldw, int(weight_layout), pc, ldc, int(m), int(n), int(k), int(schedule),
        int(config), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check("det_gemm_fwd", st)


# ------------------------------------------------------------- conveniences
def gemm(a, w, weight_layout: int = WEIGHT_NK, schedule: Optional[int] = None, config: int = -1,
         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
         stream=None) -> torch.Tensor:
    """Batch-invariant C = A W^T ([N, K] weight) or A W ([K, N] weight) in bf16.
    schedule None picks SPLIT when M is at most 64 (decode-sized), else
    MONOLITHIC; both give the same bits."""
    m = a.shape[0]
    n = w.shape[0] if weight_layout == WEIGHT_NK else w.shape[1]
    if schedule is None:
        schedule = SPLIT if m <= 64 else MONOLITHIC
    c = out if out is not None else torch.empty(m, n, dtype=torch.bfloat16, device=a.device)
    if schedule == SPLIT and workspace is None:
        nbytes = det_gemm_workspace_bytes(m, n, a.shape[1])
        workspace = torch.empty(max(nbytes // 4, 4), dtype=torch.float32, device=a.device)
    det_gemm_fwd(a, w, c, weight_layout, schedule, config, workspace, stream)
    return c
def _new_partials(rows: int, hq: int, cmax: int, d: int, device) -> torch.Tensor:
    nbytes = attn_partials_bytes(rows, hq, cmax, d)
    return torch.empty(max(nbytes // 4, 4), dtype=torch.float32, device=device)


def prefill(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
            causal: bool, softmax_scale: Optional[float] = None, schedule: int = MONOLITHIC,
            descales=(1.0, 1.0, 1.0), out: Optional[torch.Tensor] = None,
            return_lse: bool = False, window=(-1, -1), stream=None):
    """Packed-varlen attention forward; returns O (bf16) and optionally lse.

    With ``schedule=SPLIT`` the chunk partials go to a workspace and
    ``attn_chunk_merge`` folds them on the same stream."""
    tq, hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty(tq, hq, d, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(tq, hq, dtype=torch.float32, device=q.device) if return_lse else None
    if schedule == SPLIT:
        cmax = attn_num_chunks(max_seqlen_k)
        part = _new_partials(tq, hq, cmax, d, q.device)
        attn_prefill_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                         softmax_scale, causal, SPLIT, partials=part, descales=descales,
                         window=window, stream=stream)
        attn_chunk_merge(part, tq, hq, cmax, d, o, lse, v_descale=descales[2], stream=stream)
    else:
        attn_prefill_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                         softmax_scale, causal, MONOLITHIC, o=o, lse=lse, descales=descales,
                         window=window, stream=stream)
    return (o, lse) if return_lse else o


def decode(q, k_cache, v_cache, page_table, context_lens, max_context_len: int,
           softmax_scale: Optional[float] = None, schedule: int = SPLIT,
           descales=(1.0, 1.0, 1.0), out: Optional[torch.Tensor] = None,
           return_lse: bool = False, partials: Optional[torch.Tensor] = None,
           window_left: int = -1, stream=None, kv_layout: str = "NHD"):
    """Single-token paged decode; returns O (bf16) and optionally lse.  kv_layout
    "NHD" ([num_pages, 16, Hkv, D]) or "HND" ([num_pages, Hkv, 16, D]): the same bits."""
    b, hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty(b, hq, d, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(b, hq, dtype=torch.float32, device=q.device) if return_lse else None
    if schedule == SPLIT:
        cmax = attn_num_chunks(max_context_len)
        part = partials if partials is not None else _new_partials(b, hq, cmax, d, q.device)
        attn_decode_split_fwd(q, k_cache, v_cache, page_table, context_lens, max_context_len,
                              softmax_scale, SPLIT, partials=part, descales=descales,
                              window_left=window_left, stream=stream, kv_layout=kv_layout)
        attn_chunk_merge(part, b, hq, cmax, d, o, lse, v_descale=descales[2], stream=stream)
    else:
        attn_decode_split_fwd(q, k_cache, v_cache, page_table, context_lens, max_context_len,
                              softmax_scale, MONOLITHIC, o=o, lse=lse, descales=descales,
                              window_left=window_left, stream=stream, kv_layout=kv_layout)
    return (o, lse) if return_lse else o


def paged_extend(q, cu_seqlens_q, k_cache, v_cache, page_table, context_lens, max_seqlen_q: int,
                 max_context_len: int, causal: bool, softmax_scale: Optional[float] = None,
                 schedule: int = MONOLITHIC, descales=(1.0, 1.0, 1.0),
                 out: Optional[torch.Tensor] = None, return_lse: bool = False, window=(-1, -1),
                 stream=None, kv_layout: str = "NHD", workspace: Optional[torch.Tensor] = None):
    """Mixed prefill / extend / decode batch over a paged KV cache; returns O
    (bf16) and optionally lse.  Sequence b's rows are its last
    cu_seqlens_q[b+1] - cu_seqlens_q[b] tokens of context_lens[b].  ``workspace``
    (monolithic schedule): see ``attn_paged_extend_fwd``."""
    tq, hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    o = out if out is not None else torch.empty(tq, hq, d, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(tq, hq, dtype=torch.float32, device=q.device) if return_lse else None
    if schedule == SPLIT:
        cmax = attn_num_chunks(max_context_len)
        part = _new_partials(tq, hq, cmax, d, q.device)
        attn_paged_extend_fwd(q, cu_seqlens_q, k_cache, v_cache, page_table, context_lens,
                              max_seqlen_q, max_context_len, softmax_scale, causal, SPLIT,
                              partials=part, descales=descales, window=window, stream=stream,
                              kv_layout=kv_layout)
        attn_chunk_merge(part, tq, hq, cmax, d, o, lse, v_descale=descales[2], stream=stream)
    else:
        attn_paged_extend_fwd(q, cu_seqlens_q, k_cache, v_cache, page_table, context_lens,
                              max_seqlen_q, max_context_len, softmax_scale, causal, MONOLITHIC,
                              o=o, lse=lse, partials=workspace, descales=descales, window=window,
                              stream=stream, kv_layout=kv_layout)
    return (o, lse) if return_lse else o
