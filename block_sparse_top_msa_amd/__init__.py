"""Python binding of libmsa.so, the MI355X MiniMax Sparse Attention library.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in include/msa.h.  PyTorch provides device memory and the
current stream.  There is no fallback: if libmsa.so is missing or fails to
load, importing this package raises.

    proxy_score(q, k, cu_seqlens_q, ...)          msa_proxy_score page
    topk_select(max_score, topk, num_kv_heads)    the top-K block select
    sparse_attention(q, k, v, q2k_indices, ...)   msa_sparse_attention page
    validate_attention(q, k, v, q2k_indices, ...) its device-side caller contracts
    prepare_msa_nvfp4_sparse_decode(q, k, v, ...) a bound E2M1 paged decode runner
    tile_union(q2k, cu_seqlens_q, lengths_k, ...) the per-tile union builder
    qsa_indexed_forward(q, k, v, indices, ...)    qsa page, indexed API
    qsa_bitmap_forward(q, k, v, bitmap, ...)      qsa page, bitmap API
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "attention_plan", "sparse_attention_noalloc", "proxy_topk", "proxy_topk_workspace_size",
    "MsaError", "lib", "library_path", "sparse_attention", "validate_attention",
    "prepare_msa_nvfp4_sparse_decode", "MSANvfp4DecodeRunner", "proxy_score",
    "topk_select",
    "tile_union", "qsa_indexed_forward", "qsa_bitmap_forward", "workspace_size", "Workspace", "KV_BF16", "KV_FP8_E4M3",
    "KV_E2M1X2", "KV_F16",
    "REDUCE_NONE", "REDUCE_ALL", "REDUCE_GROUP", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libmsa.so")

KV_BF16, KV_FP8_E4M3, KV_E2M1X2, KV_F16 = 0, 1, 2, 3
REDUCE_NONE, REDUCE_ALL, REDUCE_GROUP = 0, 1, 2
BLOCK = 128

EXPORTED_SYMBOLS = (
    "msa_sparse_attention_workspace_size", "msa_sparse_attention", "msa_proxy_score",
    "msa_topk_select", "msa_tile_union", "msa_qsa_indexed_forward", "msa_qsa_bitmap_forward",
    "msa_validate_attention", "msa_sparse_attention_plan", "msa_sparse_attention_noalloc",
    "msa_proxy_topk_workspace_size", "msa_proxy_topk", "msa_status_string", "msa_last_error",
    "msa_version",
)

_STATUS = {0: "MSA_OK", 1: "MSA_ERR_NULL", 2: "MSA_ERR_SHAPE", 3: "MSA_ERR_DTYPE",
           4: "MSA_ERR_CONFLICT", 5: "MSA_ERR_UNSUPPORTED", 6: "MSA_ERR_WORKSPACE",
           7: "MSA_ERR_HIP", 8: "MSA_ERR_CONTRACT"}


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = _STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


class Strides(ctypes.Structure):
    _fields_ = [("page", ctypes.c_int64), ("head", ctypes.c_int64), ("token", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32P = ctypes.c_void_p


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("total_q", ctypes.c_int32),
        ("num_qo_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32), ("max_k_tiles", ctypes.c_int32),
        ("page_table_width", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("k_global_scale", ctypes.c_float),
        ("v_global_scale", ctypes.c_float), ("kv_dtype", ctypes.c_int32),
        ("splits", ctypes.c_int32),
        ("q", _P), ("k", _P), ("v", _P), ("k_scale", _P), ("v_scale", _P),
        ("k_strides", Strides), ("v_strides", Strides),
        ("k_scale_strides", Strides), ("v_scale_strides", Strides),
        ("q2k", _I32P), ("cu_seqlens_q", _I32P), ("cu_seqlens_k", _I32P),
        ("page_table", _I32P), ("seqused_k", _I32P),
        ("out", _P), ("lse", _P),
        ("lse_t", _P), ("lse_temperature_scale", ctypes.c_float),
        ("q_offset_mode", ctypes.c_int32), ("q_offset_value", ctypes.c_int32),
        ("q_offset", _I32P),
    ]


class ProxyArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("total_q", ctypes.c_int32),
        ("num_qo_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("max_seqlen_q", ctypes.c_int32),
        ("max_k_tiles", ctypes.c_int32), ("page_table_width", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("reduce_heads", ctypes.c_int32),
        ("q", _P), ("k", _P), ("k_strides", Strides),
        ("cu_seqlens_q", _I32P), ("cu_seqlens_k", _I32P), ("page_table", _I32P),
        ("seqused_k", _I32P), ("out", _P),
        ("q_offset_mode", ctypes.c_int32), ("q_offset_value", ctypes.c_int32),
        ("q_offset", _I32P),
    ]


class QsaArgs(ctypes.Structure):
    _fields_ = [
        ("total_q", ctypes.c_int32), ("num_qo_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("width", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("q", _P), ("k", _P), ("v", _P), ("k_strides", Strides), ("v_strides", Strides),
        ("indices", _I32P), ("out", _P), ("out_f32", _P), ("lse", _P),
        ("bitmap", _P), ("num_kv_tokens", ctypes.c_int32),
    ]


def _load():
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build it with `python block_sparse_top_msa_amd/build.py` "
            "(the MSA path runs only in its HIP kernels; there is no fallback)")
    L = ctypes.CDLL(library_path)
    L.msa_sparse_attention_workspace_size.argtypes = [ctypes.POINTER(AttnArgs),
                                                      ctypes.POINTER(ctypes.c_size_t)]
    L.msa_sparse_attention.argtypes = [ctypes.POINTER(AttnArgs), _P, ctypes.c_size_t, _P]
    L.msa_sparse_attention_noalloc.argtypes = [ctypes.POINTER(AttnArgs), _P]
    L.msa_proxy_score.argtypes = [ctypes.POINTER(ProxyArgs), _P]
    L.msa_proxy_topk_workspace_size.argtypes = [ctypes.POINTER(ProxyArgs), ctypes.c_int32,
                                                ctypes.POINTER(ctypes.c_size_t)]
    L.msa_proxy_topk.argtypes = [ctypes.POINTER(ProxyArgs), ctypes.c_int32, _P, _P,
                                 ctypes.c_size_t, _P]
    L.msa_topk_select.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]
    L.msa_tile_union.argtypes = [_P, _P, _P] + [ctypes.c_int32] * 8 + [_P, _P, _P, _P]
    L.msa_qsa_indexed_forward.argtypes = [ctypes.POINTER(QsaArgs), _P]
    L.msa_qsa_bitmap_forward.argtypes = [ctypes.POINTER(QsaArgs), _P]
    L.msa_validate_attention.argtypes = [ctypes.POINTER(AttnArgs), _P]
    L.msa_sparse_attention_plan.argtypes = [ctypes.POINTER(AttnArgs),
                                            ctypes.POINTER(ctypes.c_int32),
                                            ctypes.POINTER(ctypes.c_int32)]
    for fn in ("msa_sparse_attention_workspace_size", "msa_sparse_attention", "msa_proxy_score",
               "msa_topk_select", "msa_tile_union", "msa_qsa_indexed_forward",
               "msa_qsa_bitmap_forward", "msa_validate_attention",
               "msa_sparse_attention_plan", "msa_sparse_attention_noalloc",
               "msa_proxy_topk_workspace_size", "msa_proxy_topk"):
        getattr(L, fn).restype = ctypes.c_int
    L.msa_status_string.argtypes = [ctypes.c_int]
    L.msa_status_string.restype = ctypes.c_char_p
    L.msa_last_error.argtypes = []
    L.msa_last_error.restype = ctypes.c_char_p
    L.msa_version.argtypes = []
    L.msa_version.restype = ctypes.c_char_p
    return L


lib = _load()


def _check(status: int):
    if status != 0:
        raise MsaError(status, lib.msa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _kv_format(k: torch.Tensor, k_scale) -> int:
    if k.dtype == torch.bfloat16:
        return KV_BF16
    if k.dtype == torch.float16:
        return KV_F16
    if k.dtype == torch.float8_e4m3fn:
        return KV_FP8_E4M3
    if k.dtype == torch.uint8:
        if k_scale is None:
            raise ValueError("uint8 K/V is packed E2M1 and needs k_scale / v_scale")
        return KV_E2M1X2
    raise ValueError(f"unsupported K/V dtype {k.dtype} (bf16, float8_e4m3fn, or uint8 packed E2M1)")


def _strides(t: Optional[torch.Tensor], paged: bool) -> Strides:
    if t is None:
        return Strides(0, 0, 0)
    es = t.element_size()
    if t.stride(-1) != 1:
        raise MsaError(5, "the last dimension must be contiguous (views are never copied)")
    if paged:
        if t.dim() != 4 or t.shape[2] != BLOCK:
            raise ValueError(f"paged K/V must be (num_pages, num_kv_heads, 128, d'), got {tuple(t.shape)}")
        return Strides(t.stride(0) * es, t.stride(1) * es, t.stride(2) * es)
    if t.dim() != 3:
        raise ValueError(f"flat K/V must be (total_k, num_kv_heads, d'), got {tuple(t.shape)}")
    return Strides(0, t.stride(1) * es, t.stride(0) * es)


# Convenience bounds for calls that omit max_seqlen_q / max_k_tiles: these read
# device lengths on the host, which synchronises the stream.  Callers on the
# launch path (graphs, serving loops) pass both bounds instead.
def _host_max_seqlen(cu: torch.Tensor) -> int:
    c = cu.to("cpu", torch.int64)
    return int((c[1:] - c[:-1]).max()) if c.numel() > 1 else 0


def _host_max_tiles(cu_k, seqused_k) -> int:
    if seqused_k is not None:
        L = int(seqused_k.max().item()) if seqused_k.numel() else 0
    else:
        L = _host_max_seqlen(cu_k)
    return (L + BLOCK - 1) // BLOCK


class Workspace:
    """Caller-owned workspace of sparse_attention (the fp32 partials of every
    split and their LSE, or staged bf16 pages) and of proxy_topk.  Created
    zero-filled: its last 64 KiB hold the split-KV arrival counters, which
    the library keeps at zero between launches.  Launches that may overlap
    need separate workspaces."""

    def __init__(self, nbytes: int, device):
        self.nbytes = int(nbytes)
        self.buffer = torch.zeros(max(self.nbytes, 256) + 256, dtype=torch.uint8, device=device)
        off = (-self.buffer.data_ptr()) % 256
        self.view = self.buffer[off:off + max(self.nbytes, 256)]

    def ensure(self, nbytes: int) -> "Workspace":
        return self if nbytes <= self.nbytes else Workspace(nbytes, self.buffer.device)


_ws_cache: dict = {}


def _attn_args(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k, causal, softmax_scale,
               page_table, seqused_k, k_scale, v_scale, k_global_scale, v_global_scale,
               max_seqlen_q, max_k_tiles, out, lse, splits):
    paged = page_table is not None
    fmt = _kv_format(k, k_scale)
    a = AttnArgs()
    a.batch = cu_seqlens_q.numel() - 1
    a.total_q = q.shape[0]
    a.num_qo_heads = q.shape[1]
    a.num_kv_heads = k.shape[1]
    a.head_dim = q.shape[2]
    a.topk = q2k_indices.shape[2]
    a.max_seqlen_q = _host_max_seqlen(cu_seqlens_q) if max_seqlen_q is None else int(max_seqlen_q)
    a.max_k_tiles = _host_max_tiles(cu_seqlens_k, seqused_k) if max_k_tiles is None else int(max_k_tiles)
    a.page_table_width = page_table.shape[1] if paged else 0
    a.causal = 1 if causal else 0
    a.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    a.k_global_scale = 0.0 if k_global_scale is None else float(k_global_scale)
    a.v_global_scale = 0.0 if v_global_scale is None else float(v_global_scale)
    a.kv_dtype = fmt
    a.splits = int(splits)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.k_strides = _strides(k, paged)
    a.v_strides = _strides(v, paged)
    a.k_scale_strides = _strides(k_scale, paged) if k_scale is not None else Strides(0, 0, 0)
    a.v_scale_strides = _strides(v_scale, paged) if v_scale is not None else Strides(0, 0, 0)
    a.q2k = _ptr(q2k_indices)
    a.cu_seqlens_q = _ptr(cu_seqlens_q)
    a.cu_seqlens_k = _ptr(cu_seqlens_k)
    a.page_table = _ptr(page_table)
    a.seqused_k = _ptr(seqused_k)
    a.out = _ptr(out)
    a.lse = _ptr(lse)
    return a


def _set_q_offset(a, q_offset, total_q):
    """q_offset: None (right-aligned causal positions), an int o (query iq of
    every request at KV position o + iq) or a device int32 tensor [total_q]
    (each query row's own position)."""
    if q_offset is None:
        a.q_offset_mode = 0
    elif isinstance(q_offset, int):
        a.q_offset_mode, a.q_offset_value = 1, int(q_offset)
    else:
        if (q_offset.dtype != torch.int32 or not q_offset.is_contiguous()
                or q_offset.numel() != total_q):
            raise ValueError(f"q_offset must be an int or a contiguous int32 tensor of "
                             f"{total_q} query positions")
        a.q_offset_mode, a.q_offset = 2, _ptr(q_offset)


def _check_i32(name, t):
    if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous int32 tensor")


def workspace_size(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k=None, *, page_table=None,
                   seqused_k=None, k_scale=None, v_scale=None, max_seqlen_q=None,
                   max_k_tiles=None, splits=0) -> int:
    a = _attn_args(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k, False, None, page_table,
                   seqused_k, k_scale, v_scale, None, None, max_seqlen_q, max_k_tiles, None,
                   None, splits)
    n = ctypes.c_size_t(0)
    _check(lib.msa_sparse_attention_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return int(n.value)


def attention_plan(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k=None, *, page_table=None,
                   seqused_k=None, k_scale=None, v_scale=None, max_seqlen_q=None,
                   max_k_tiles=None, splits=0, return_temperature_lse=False):
    """(decode_route, splits) that sparse_attention takes for these arguments:
    decode_route 1 is the paged/flat decode kernel (split-KV partials merged
    by LSE when splits > 1), 0 the prefill tiles."""
    a = _attn_args(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k, False, None, page_table,
                   seqused_k, k_scale, v_scale, None, None, max_seqlen_q, max_k_tiles, None,
                   None, splits)
    if return_temperature_lse:
        a.lse_t, a.lse_temperature_scale = a.q, 1.0   # only tested for non-NULL
    route, nsplit = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.msa_sparse_attention_plan(ctypes.byref(a), ctypes.byref(route),
                                         ctypes.byref(nsplit)))
    return int(route.value), int(nsplit.value)


def validate_attention(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k=None, causal=False,
                       page_table=None, seqused_k=None, k_scale=None, v_scale=None, *,
                       max_seqlen_q=None, max_k_tiles=None, out=None):
    """Debug check of the device-side caller contracts of sparse_attention
    with these arguments (cu_seqlens, KV lengths, page ids, q2k row order and
    padding).  Synchronises the stream; raises MsaError (MSA_ERR_CONTRACT)
    naming the first violation.  Never runs the attention.  Setting
    MSA_VALIDATE=1 in the environment makes every sparse_attention call run
    this check first."""
    for name, t in (("q2k_indices", q2k_indices), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k), ("page_table", page_table),
                    ("seqused_k", seqused_k)):
        _check_i32(name, t)
    a = _attn_args(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k, causal, None, page_table,
                   seqused_k, k_scale, v_scale, None, None, max_seqlen_q, max_k_tiles,
                   torch.empty_like(q) if out is None else out, None, 0)
    _check(lib.msa_validate_attention(ctypes.byref(a), _stream()))


def sparse_attention(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k=None, causal=False,
                     softmax_scale=None, page_table=None, seqused_k=None,
                     return_softmax_lse=False, k_scale=None, v_scale=None,
                     k_global_scale=None, v_global_scale=None, *, max_seqlen_q=None,
                     max_k_tiles=None, workspace: Optional[Workspace] = None, out=None,
                     lse=None, splits=0, return_temperature_lse=False,
                     lse_temperature_scale=1.0, lse_t=None, q_offset=None):
    """MSA forward (msa_sparse_attention page).  Returns out, or (out, lse),
    or with return_temperature_lse (out, lse, lse_t), lse_t = ln sum_j
    exp(lse_temperature_scale * z_j) over the attended keys.  q_offset: the
    queries' causal positions, None (right-aligned), an int o (query iq of
    every request at o + iq) or an int32 tensor [total_q] of per-row
    positions."""
    want = torch.float16 if k.dtype == torch.float16 else torch.bfloat16
    if q.dtype != want or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous {want} tensor (total_q, num_qo_heads, 128) "
                         "(fp16 q goes with fp16 k / v, bf16 q with every other K/V format)")
    for name, t in (("q2k_indices", q2k_indices), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k), ("page_table", page_table),
                    ("seqused_k", seqused_k)):
        _check_i32(name, t)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and (return_softmax_lse or return_temperature_lse):
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    if return_temperature_lse and lse_t is None:
        lse_t = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    a = _attn_args(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k, causal, softmax_scale,
                   page_table, seqused_k, k_scale, v_scale, k_global_scale, v_global_scale,
                   max_seqlen_q, max_k_tiles, out, lse, splits)
    if return_temperature_lse:
        a.lse_t = _ptr(lse_t)
        a.lse_temperature_scale = float(lse_temperature_scale)
    _set_q_offset(a, q_offset, q.shape[0])
    need = ctypes.c_size_t(0)
    _check(lib.msa_sparse_attention_workspace_size(ctypes.byref(a), ctypes.byref(need)))
    ws_ptr, ws_bytes = None, 0
    if need.value:
        if workspace is None:
            key = (q.device, torch.cuda.current_stream().cuda_stream)
            ws = _ws_cache.get(key)
            ws = Workspace(need.value, q.device) if ws is None else ws.ensure(need.value)
            _ws_cache[key] = ws
            workspace = ws
        elif workspace.nbytes < need.value:
            raise MsaError(6, f"workspace of {need.value} bytes needed, got {workspace.nbytes}")
        ws_ptr, ws_bytes = _ptr(workspace.view), workspace.nbytes
    _check(lib.msa_sparse_attention(ctypes.byref(a), ws_ptr, ws_bytes, _stream()))
    if return_temperature_lse:
        return out, lse, lse_t
    return (out, lse) if return_softmax_lse else out


def sparse_attention_noalloc(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k=None,
                             causal=False, softmax_scale=None, page_table=None, seqused_k=None,
                             k_scale=None, v_scale=None, k_global_scale=None,
                             v_global_scale=None, *, max_seqlen_q, max_k_tiles, out, lse=None,
                             splits=0, q_offset=None):
    """sparse_attention through msa_sparse_attention_noalloc: the library's
    own per-GPU scratch serves as the workspace, and the caller passes every
    output, so nothing is allocated (on the host side nothing is read from
    the device either).  Calls that may overlap on one GPU race on the
    scratch.  Returns out (and lse when given)."""
    for name, t in (("q2k_indices", q2k_indices), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k), ("page_table", page_table),
                    ("seqused_k", seqused_k)):
        _check_i32(name, t)
    a = _attn_args(q, k, v, q2k_indices, cu_seqlens_q, cu_seqlens_k, causal, softmax_scale,
                   page_table, seqused_k, k_scale, v_scale, k_global_scale, v_global_scale,
                   max_seqlen_q, max_k_tiles, out, lse, splits)
    _set_q_offset(a, q_offset, q.shape[0])
    _check(lib.msa_sparse_attention_noalloc(ctypes.byref(a), _stream()))
    return out if lse is None else (out, lse)


class MSANvfp4DecodeRunner:
    """Bound packed-E2M1 paged decode (prepare_msa_nvfp4_sparse_decode page):
    every tensor, the output, the LSE and the split-KV workspace are fixed
    at preparation; calling the runner launches the decode on the current
    stream with no allocation and no host synchronisation (so it can be
    captured in a HIP graph) and returns out.  `splits` is the split-KV
    factor the launch uses; `decode_route` is 1 when the call takes the
    decode kernel (the E2M1 pages dequantised in registers)."""

    decode_route = 1

    def __init__(self, args: "AttnArgs", keep: tuple, out, lse, workspace, splits: int):
        self._args, self._keep = args, keep
        self.out, self.lse, self.workspace, self.splits = out, lse, workspace, splits
        self._ws = (None, 0) if workspace is None else (_ptr(workspace.view), workspace.nbytes)

    def __call__(self):
        _check(lib.msa_sparse_attention(ctypes.byref(self._args), self._ws[0], self._ws[1],
                                        _stream()))
        return self.out


def prepare_msa_nvfp4_sparse_decode(q, k, v, q2k_indices, *, k_scale, v_scale, page_table,
                                    seqused_k, k_global_scale, v_global_scale,
                                    workspace_buffer=None, seqlen_q=1, softmax_scale=None,
                                    out=None, lse=None, backend="hip"):
    """Validate and bind a packed-E2M1 (NVFP4-layout) paged decode
    (prepare_msa_nvfp4_sparse_decode page): q bf16 [batch * seqlen_q, Hq,
    128], request b owning rows [b * seqlen_q, (b + 1) * seqlen_q); k, v
    uint8 [num_pages, Hkv, 128, 64]; q2k [Hkv, batch * seqlen_q, 16];
    k_scale, v_scale [num_pages, Hkv, 128, 8] E4M3 bytes (uint8 or
    float8_e4m3fn views, both stored linearly); page_table [batch,
    max_pages]; seqused_k [batch] including the new tokens; positive global
    scales.  Causal, right-aligned: token i of request b sits at KV position
    seqused_k[b] - seqlen_q + i.  workspace_buffer: optional caller-owned
    uint8 bytes for the split-KV partials (otherwise allocated here, once).
    Returns an MSANvfp4DecodeRunner."""
    if backend not in ("hip", "cake"):
        raise ValueError(f"unknown backend {backend!r}")
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != 128 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [batch * seqlen_q, num_q_heads, 128] tensor")
    if not 1 <= int(seqlen_q) <= 32:
        raise ValueError(f"seqlen_q must be in [1, 32], got {seqlen_q}")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != torch.uint8 or t.dim() != 4 or t.shape[2] != BLOCK or t.shape[3] != 64:
            raise ValueError(f"{name} must be uint8 [num_pages, num_kv_heads, 128, 64]")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn) or t.dim() != 4 or t.shape[3] != 8:
            raise ValueError(f"{name} must be uint8 or float8_e4m3fn [num_pages, num_kv_heads, 128, 8]")
    k_scale, v_scale = k_scale.view(torch.uint8), v_scale.view(torch.uint8)
    hkv = k.shape[1]
    if q2k_indices.dim() != 3 or q2k_indices.shape[0] != hkv or q2k_indices.shape[2] != 16 \
            or q2k_indices.shape[1] != q.shape[0]:
        raise ValueError("q2k_indices must be int32 [num_kv_heads, batch * seqlen_q, 16]")
    if q.shape[1] % hkv or q.shape[1] // hkv > 16:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads, at most 16 per KV head")
    if not (k_global_scale > 0 and v_global_scale > 0):
        raise ValueError("k_global_scale and v_global_scale must be positive")
    for name, t in (("q2k_indices", q2k_indices), ("page_table", page_table),
                    ("seqused_k", seqused_k)):
        _check_i32(name, t)
    batch = seqused_k.numel()
    if q.shape[0] != batch * int(seqlen_q):
        raise ValueError(f"q has {q.shape[0]} rows, expected batch * seqlen_q = {batch * seqlen_q}")
    cu_q = torch.arange(0, batch + 1, dtype=torch.int32, device=q.device) * int(seqlen_q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    a = _attn_args(q, k, v, q2k_indices, cu_q, None, True, softmax_scale, page_table, seqused_k,
                   k_scale, v_scale, k_global_scale, v_global_scale, int(seqlen_q),
                   page_table.shape[1], out, lse, 0)
    need = ctypes.c_size_t(0)
    _check(lib.msa_sparse_attention_workspace_size(ctypes.byref(a), ctypes.byref(need)))
    route, splits = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.msa_sparse_attention_plan(ctypes.byref(a), ctypes.byref(route), ctypes.byref(splits)))
    ws = None
    if need.value:
        if workspace_buffer is None:
            ws = Workspace(need.value, q.device)
        else:
            if workspace_buffer.dtype != torch.uint8 or not workspace_buffer.is_contiguous():
                raise ValueError("workspace_buffer must be contiguous uint8 bytes")
            off = (-workspace_buffer.data_ptr()) % 256
            if workspace_buffer.numel() - off < need.value:
                raise MsaError(6, f"workspace_buffer needs {need.value} bytes past 256-byte "
                                  f"alignment, got {workspace_buffer.numel() - off}")
            ws = Workspace.__new__(Workspace)
            ws.nbytes = workspace_buffer.numel() - off
            ws.buffer = workspace_buffer
            ws.view = workspace_buffer[off:]
            ws.view.zero_()   # the split counters start at zero (preparation, not the runner)
    keep = (q, k, v, q2k_indices, k_scale, v_scale, page_table, seqused_k, cu_q)
    run = MSANvfp4DecodeRunner(a, keep, out, lse, ws, int(splits.value))
    run.decode_route = int(route.value)
    return run


def _proxy_args(q, k, cu_seqlens_q, cu_seqlens_k, page_table, seqused_k, causal, max_seqlen_q,
                max_k_tiles, reduce_heads, q_offset):
    """ProxyArgs for these tensors, and (score heads, max_k_tiles)."""
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k),
                    ("page_table", page_table), ("seqused_k", seqused_k)):
        _check_i32(name, t)
    paged = page_table is not None
    if k.dtype == torch.bfloat16:
        fmt = KV_BF16
    elif k.dtype == torch.float16:
        fmt = KV_F16
    elif k.dtype == torch.float8_e4m3fn:
        fmt = KV_FP8_E4M3
    else:
        raise ValueError(f"proxy K must be bf16, float16 or float8_e4m3fn, got {k.dtype}")
    want = torch.float16 if fmt == KV_F16 else torch.bfloat16
    if q.dtype != want or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous {want} tensor (total_q, num_qo_heads, 128) "
                         "(fp16 q goes with fp16 k, bf16 q with bf16 or fp8 k)")
    T = _host_max_tiles(cu_seqlens_k, seqused_k) if max_k_tiles is None else int(max_k_tiles)
    if reduce_heads == "group":
        rmode, H = REDUCE_GROUP, k.shape[1]
    elif reduce_heads in (False, True, 0, 1):
        rmode = REDUCE_ALL if reduce_heads else REDUCE_NONE
        H = 1 if reduce_heads else q.shape[1]
    else:
        raise ValueError(f"reduce_heads must be False, True or 'group', got {reduce_heads!r}")
    a = ProxyArgs()
    a.batch = cu_seqlens_q.numel() - 1
    a.total_q = q.shape[0]
    a.num_qo_heads = q.shape[1]
    a.num_kv_heads = k.shape[1]
    a.head_dim = q.shape[2]
    a.max_seqlen_q = _host_max_seqlen(cu_seqlens_q) if max_seqlen_q is None else int(max_seqlen_q)
    a.max_k_tiles = T
    a.page_table_width = page_table.shape[1] if paged else 0
    a.causal = 1 if causal else 0
    a.kv_dtype = fmt
    a.reduce_heads = rmode
    a.q, a.k = _ptr(q), _ptr(k)
    a.k_strides = _strides(k, paged)
    a.cu_seqlens_q = _ptr(cu_seqlens_q)
    a.cu_seqlens_k = _ptr(cu_seqlens_k)
    a.page_table = _ptr(page_table)
    a.seqused_k = _ptr(seqused_k)
    _set_q_offset(a, q_offset, q.shape[0])
    return a, H, T


def proxy_score(q, k, cu_seqlens_q, cu_seqlens_k=None, *, page_table=None, seqused_k=None,
                causal=True, max_seqlen_q=None, max_k_tiles=None, output=None,
                reduce_heads=False, q_offset=None):
    """Stage-1 block max of unscaled masked QK^T (msa_proxy_score page).
    reduce_heads: False (per query head), True (max over all heads) or
    "group" (max over each KV head's query heads).  q_offset: None
    (right-aligned), an int o (query iq at o + iq) or an int32 tensor of
    per-row positions.  Returns fp32 (num_qo_heads | 1 | num_kv_heads,
    max_k_tiles, total_q)."""
    a, H, T = _proxy_args(q, k, cu_seqlens_q, cu_seqlens_k, page_table, seqused_k, causal,
                          max_seqlen_q, max_k_tiles, reduce_heads, q_offset)
    if output is None:
        output = torch.empty(H, T, q.shape[0], dtype=torch.float32, device=q.device)
    elif (output.shape != (H, T, q.shape[0]) or output.dtype != torch.float32
          or not output.is_contiguous()):
        raise ValueError(f"output must be contiguous fp32 {(H, T, q.shape[0])}")
    a.out = _ptr(output)
    _check(lib.msa_proxy_score(ctypes.byref(a), _stream()))
    return output


def proxy_topk(q, k, cu_seqlens_q, cu_seqlens_k=None, *, topk, page_table=None, seqused_k=None,
               causal=True, max_seqlen_q=None, max_k_tiles=None, reduce_heads=False,
               q_offset=None, out=None, workspace=None):
    """Proxy score -> head reduction -> top-K select in one call
    (msa_proxy_topk): q2k int32 (num_kv_heads, total_q, topk), equal to
    topk_select(proxy_score(...), topk, num_kv_heads).  On decode shapes the
    selection runs inside the proxy pass and no score buffer exists.
    workspace: a Workspace of at least proxy_topk_workspace_size bytes, or
    None (one is allocated)."""
    a, _, _ = _proxy_args(q, k, cu_seqlens_q, cu_seqlens_k, page_table, seqused_k, causal,
                          max_seqlen_q, max_k_tiles, reduce_heads, q_offset)
    if out is None:
        out = torch.empty(k.shape[1], q.shape[0], int(topk), dtype=torch.int32, device=q.device)
    elif (out.shape != (k.shape[1], q.shape[0], int(topk)) or out.dtype != torch.int32
          or not out.is_contiguous()):
        raise ValueError(f"out must be contiguous int32 {(k.shape[1], q.shape[0], int(topk))}")
    need = ctypes.c_size_t(0)
    _check(lib.msa_proxy_topk_workspace_size(ctypes.byref(a), int(topk), ctypes.byref(need)))
    if workspace is None:
        workspace = Workspace(max(1, need.value), q.device)
    elif workspace.nbytes < need.value:
        raise MsaError(6, f"workspace of {need.value} bytes needed, got {workspace.nbytes}")
    _check(lib.msa_proxy_topk(ctypes.byref(a), int(topk), _ptr(out), _ptr(workspace.view),
                              workspace.nbytes, _stream()))
    return out


def proxy_topk_workspace_size(q, k, cu_seqlens_q, cu_seqlens_k=None, *, topk, page_table=None,
                              seqused_k=None, causal=True, max_seqlen_q=None, max_k_tiles=None,
                              reduce_heads=False) -> int:
    a, _, _ = _proxy_args(q, k, cu_seqlens_q, cu_seqlens_k, page_table, seqused_k, causal,
                          max_seqlen_q, max_k_tiles, reduce_heads, None)
    need = ctypes.c_size_t(0)
    _check(lib.msa_proxy_topk_workspace_size(ctypes.byref(a), int(topk), ctypes.byref(need)))
    return int(need.value)


def topk_select(max_score, topk, num_kv_heads, mode=None, out=None):
    """Top-K block select: fp32 (H_s, T, total_q) -> int32 q2k (Hkv, total_q, topk).
    mode None picks ALL for H_s == 1 and NONE for H_s == num_kv_heads."""
    if max_score.dtype != torch.float32 or not max_score.is_contiguous():
        raise ValueError("max_score must be a contiguous fp32 tensor")
    hs, T, total_q = max_score.shape
    if mode is None:
        mode = REDUCE_ALL if hs == 1 else (REDUCE_NONE if hs == num_kv_heads else REDUCE_GROUP)
    if out is None:
        out = torch.empty(num_kv_heads, total_q, topk, dtype=torch.int32, device=max_score.device)
    _check(lib.msa_topk_select(_ptr(max_score), hs, T, total_q, int(topk), int(num_kv_heads),
                               int(mode), _ptr(out), _stream()))
    return out


def tile_union(q2k, cu_seqlens_q, lengths_k, tile_tokens, max_k_tiles, max_seqlen_q=None,
               max_union=None):
    """The attention kernel's per-tile union, exported for checking.  Returns
    (blocks int32, masks uint64-as-int64, counts int32) shaped
    (Hkv, B, tiles_per_req, max_union) / (Hkv, B, tiles_per_req)."""
    _check_i32("q2k", q2k)
    _check_i32("cu_seqlens_q", cu_seqlens_q)
    _check_i32("lengths_k", lengths_k)
    hkv, total_q, topk = q2k.shape
    B = cu_seqlens_q.numel() - 1
    mq = _host_max_seqlen(cu_seqlens_q) if max_seqlen_q is None else int(max_seqlen_q)
    tiles = (mq + tile_tokens - 1) // tile_tokens
    mu = min(tile_tokens * topk, max_k_tiles) if max_union is None else int(max_union)
    mu = max(mu, 1)
    blocks = torch.empty(hkv, B, tiles, mu, dtype=torch.int32, device=q2k.device)
    masks = torch.empty(hkv, B, tiles, mu, dtype=torch.int64, device=q2k.device)
    counts = torch.empty(hkv, B, tiles, dtype=torch.int32, device=q2k.device)
    _check(lib.msa_tile_union(_ptr(q2k), _ptr(cu_seqlens_q), _ptr(lengths_k), B, total_q, hkv,
                              topk, mq, int(max_k_tiles), int(tile_tokens), mu, _ptr(blocks),
                              _ptr(masks), _ptr(counts), _stream()))
    return blocks, masks, counts


def _qsa_args(q, k, v, softmax_scale, out, out_f32, lse, return_f32, return_lse):
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or q.dim() != 3:
        raise ValueError("q must be a contiguous bf16 tensor (T, Hq, 256)")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{name} must be bf16 (Tk, Hkv, 256) with a contiguous last dim")
    T, hq, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if return_f32 and out_f32 is None:
        out_f32 = torch.empty(T, hq, d, dtype=torch.float32, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty(hq, T, dtype=torch.float32, device=q.device)
    a = QsaArgs()
    a.total_q, a.num_qo_heads, a.num_kv_heads, a.head_dim = T, hq, k.shape[1], d
    a.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.k_strides = Strides(0, k.stride(1) * 2, k.stride(0) * 2)
    a.v_strides = Strides(0, v.stride(1) * 2, v.stride(0) * 2)
    a.out, a.out_f32, a.lse = _ptr(out), _ptr(out_f32), _ptr(lse)
    return a, out, out_f32, lse


def qsa_indexed_forward(q, k, v, indices, softmax_scale=None, out=None, out_f32=None, lse=None,
                        return_f32=True, return_lse=True):
    """Packed query sparse attention over caller-selected tokens (qsa page,
    indexed API): q bf16 (T, Hq, 256); k, v bf16 (Tk, Hkv, 256), last dim
    contiguous; indices int32 (T, W), absolute token ids in groups of four,
    -1 padded.  Returns (out bf16, out_f32, lse (Hq, T)); out_f32 / lse are
    None when not requested."""
    if indices.dtype != torch.int32 or not indices.is_contiguous() or indices.dim() != 2:
        raise ValueError("indices must be a contiguous int32 (T, W) tensor")
    a, out, out_f32, lse = _qsa_args(q, k, v, softmax_scale, out, out_f32, lse, return_f32,
                                     return_lse)
    a.width = indices.shape[1]
    a.indices = _ptr(indices)
    _check(lib.msa_qsa_indexed_forward(ctypes.byref(a), _stream()))
    return out, out_f32, lse


def qsa_bitmap_forward(q, k, v, bitmap, softmax_scale=None, out=None, out_f32=None, lse=None,
                       return_f32=True, return_lse=True):
    """Packed query sparse attention with each query's keys given by a
    4-token block bitmap (qsa page, bitmap API): bitmap uint8 or bool
    (T, ceil(Tk / 4)), a non-zero entry selecting the block's tokens (< Tk);
    q, k, v and the outputs as in qsa_indexed_forward."""
    if bitmap.dtype == torch.bool:
        bitmap = bitmap.view(torch.uint8)
    if bitmap.dtype != torch.uint8 or not bitmap.is_contiguous() or bitmap.dim() != 2:
        raise ValueError("bitmap must be a contiguous uint8 or bool (T, ceil(Tk / 4)) tensor")
    tk = k.shape[0]
    if bitmap.shape != (q.shape[0], (tk + 3) // 4):
        raise ValueError(f"bitmap must be ({q.shape[0]}, {(tk + 3) // 4}), got {tuple(bitmap.shape)}")
    a, out, out_f32, lse = _qsa_args(q, k, v, softmax_scale, out, out_f32, lse, return_f32,
                                     return_lse)
    a.bitmap = _ptr(bitmap)
    a.num_kv_tokens = tk
    _check(lib.msa_qsa_bitmap_forward(ctypes.byref(a), _stream()))
    return out, out_f32, lse

