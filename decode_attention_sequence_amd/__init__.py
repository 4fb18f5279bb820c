"""Python binding of libdcp: sharded paged decode attention on AMD MI355X (gfx950).

Argument marshalling only. Every computation runs in the HIP kernels of
``libdcp.so`` (C ABI in ``include/dcp.h``); PyTorch provides device memory and
the current HIP stream. If the library is not built, importing works but every
call raises ``LibraryMissing`` -- there is no fallback implementation.

Entry points (same names as the C ABI, without the ``dcp_`` prefix):
  block_remap        global block table -> per-shard local tables (block j on shard j % D,
                     or contiguous runs of ceil(nb / D) blocks with ownership="contiguous")
  block_remap_update the same tables after sequences grew or shrank, remapping only changed blocks
  kv_append          a decode step's KV write into the owning block (fp8: quantised on write)
  workspace_size     device workspace bytes for a descriptor
  decode_partial     one shard's partial output and log-sum-exp
  decode_partial_mtp the same for q_len query tokens per sequence (causal by global position)
  lse_merge          merge of D partials: O = sum_i exp(LSE_i) / sum_j exp(LSE_j) * O_i
  decode_all_shards  all D shards of one layer plus the merge, fused
"""
from __future__ import annotations

import ctypes
import math
import os
from pathlib import Path
from typing import Optional

import torch

__all__ = [
    "AttnDesc", "DcpError", "LibraryMissing", "F32", "BF16", "FP8_E4M3", "KV_SEPARATE",
    "KV_LATENT", "OWN_INTERLEAVED", "OWN_CONTIGUOUS", "library_path", "lib", "make_desc", "block_remap", "block_remap_update", "kv_append", "workspace_size",
    "decode_partial", "decode_partial_mtp", "decode_partial_token", "decode_partial_plan",
    "decode_partial_run", "lse_merge", "decode_all_shards", "decode_all_shards_plan",
    "decode_all_shards_run", "decode_all_shards_noalloc", "status_str", "version",
]

# The library the binding loads: the in-tree build, or the file named by the
# DCP_LIBRARY environment variable (e.g. a build with host-side sanitizers).
_LIB_PATH = (Path(os.environ["DCP_LIBRARY"]).resolve() if os.environ.get("DCP_LIBRARY")
             else Path(__file__).resolve().with_name("libdcp.so"))

F32, BF16, FP8_E4M3 = 0, 1, 2
KV_SEPARATE, KV_LATENT = 0, 1
OWN_INTERLEAVED, OWN_CONTIGUOUS = 0, 1
_OWNERSHIP = {"interleaved": OWN_INTERLEAVED, "contiguous": OWN_CONTIGUOUS}
DCP_OK, DCP_ERR_INVALID_ARG, DCP_ERR_UNSUPPORTED, DCP_ERR_WORKSPACE, DCP_ERR_HIP = range(5)


class LibraryMissing(ImportError):
    pass


class DcpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libdcp error {status}: {message}")
        self.status = status


class DcpValueError(DcpError, ValueError):
    """Invalid or unsupported arguments (the library enqueued nothing)."""


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("qk_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_shards", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("num_cache_blocks", ctypes.c_int32),
        ("kv_kind", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("kv_block_stride", ctypes.c_int64),
        ("kv_token_stride", ctypes.c_int64),
        ("kv_head_stride", ctypes.c_int64),
        ("q_len", ctypes.c_int32),
    ]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def library_path() -> Path:
    return _LIB_PATH


def lib():
    """The loaded libdcp (raises LibraryMissing if it has not been built)."""
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            raise LibraryMissing(
                f"{_LIB_PATH} is not built; run `python -m decode_attention_sequence_amd.build`")
        L = ctypes.CDLL(str(_LIB_PATH))
        L.dcp_block_remap.argtypes = [_P, _P, _I, _I, _I, _I, _P, _P, _P]
        L.dcp_block_remap.restype = _I
        L.dcp_block_remap_ex.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P]
        L.dcp_block_remap_ex.restype = _I
        L.dcp_block_remap_update.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P]
        L.dcp_block_remap_update.restype = _I
        L.dcp_kv_append.argtypes = [ctypes.POINTER(AttnDesc), _I, _P, _P, _P, _P, _I, _I, _P,
                                    _P, _P, _P, _P]
        L.dcp_kv_append.restype = _I
        L.dcp_workspace_size.argtypes = [ctypes.POINTER(AttnDesc)]
        L.dcp_workspace_size.restype = ctypes.c_size_t
        L.dcp_decode_partial.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, _P,
                                         _P, ctypes.c_size_t, _P]
        L.dcp_decode_partial.restype = _I
        L.dcp_decode_partial_mtp.argtypes = [ctypes.POINTER(AttnDesc), _I, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.dcp_decode_partial_mtp.restype = _I
        L.dcp_decode_partial_token.argtypes = [ctypes.POINTER(AttnDesc), _I, _P, _P, _P, _P, _P,
                                               _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.dcp_decode_partial_token.restype = _I
        L.dcp_lse_merge.argtypes = [_P, _P, _I, _I, _I, _I, _P, _I, _P, _P]
        L.dcp_lse_merge.restype = _I
        L.dcp_decode_all_shards.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P,
                                            _P, _P, ctypes.c_size_t, _P]
        L.dcp_decode_all_shards.restype = _I
        L.dcp_decode_all_shards_timed.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P,
                                                  _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P]
        L.dcp_decode_all_shards_timed.restype = _I
        L.dcp_decode_all_shards_noalloc.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P,
                                                    _P, _P, _P, _P]
        L.dcp_decode_all_shards_noalloc.restype = _I
        L.dcp_decode_partial_plan.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, ctypes.c_size_t, _P]
        L.dcp_decode_partial_plan.restype = _I
        L.dcp_decode_partial_run.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P,
                                             _P, ctypes.c_size_t, _P]
        L.dcp_decode_partial_run.restype = _I
        L.dcp_decode_all_shards_plan.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, ctypes.c_size_t,
                                                 _P]
        L.dcp_decode_all_shards_plan.restype = _I
        L.dcp_decode_all_shards_run.argtypes = [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P,
                                                _P, _P, ctypes.c_size_t, _P]
        L.dcp_decode_all_shards_run.restype = _I
        L.dcp_status_str.argtypes = [_I]
        L.dcp_status_str.restype = ctypes.c_char_p
        L.dcp_version.argtypes = []
        L.dcp_version.restype = _I
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().dcp_status_str(status).decode()


def version() -> int:
    return int(lib().dcp_version())


def _check(status: int):
    if status == DCP_OK:
        return
    msg = status_str(status)
    if status in (DCP_ERR_INVALID_ARG, DCP_ERR_UNSUPPORTED, DCP_ERR_WORKSPACE):
        raise DcpValueError(status, msg)
    raise DcpError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], dtype, numel: int):
    """Host-side size check of a buffer the library will index on the device."""
    if t is None or not t.is_contiguous() or t.numel() != numel or (dtype and t.dtype != dtype):
        got = None if t is None else (tuple(t.shape), t.dtype, t.is_contiguous())
        raise DcpValueError(DCP_ERR_INVALID_ARG,
                            f"expected a contiguous {dtype or ''} tensor of {numel} elements, got {got}")


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_DTYPE_CODE = {
    torch.float32: F32,
    torch.bfloat16: BF16,
    torch.float8_e4m3fn: FP8_E4M3,
    torch.uint8: FP8_E4M3,  # raw e4m3 codes
}


def _code(t: torch.Tensor) -> int:
    try:
        return _DTYPE_CODE[t.dtype]
    except KeyError:
        raise DcpValueError(DCP_ERR_UNSUPPORTED, f"unsupported dtype {t.dtype}") from None


def make_desc(kind: int, q: torch.Tensor, k_cache: torch.Tensor, block_table: torch.Tensor, *,
              num_shards: int, v_dim: Optional[int] = None, softmax_scale: Optional[float] = None,
              max_seq_len: Optional[int] = None, out_dtype: int = F32,
              q_len: int = 1) -> AttnDesc:
    """Descriptor for q [B, q_len * Hq, qk_dim] (or [B, q_len, Hq, qk_dim]) and a cache laid
    out as [num_blocks, block_size, Hkv, dim] (KV_SEPARATE) or [num_blocks, block_size, qk_dim]
    (KV_LATENT); strides are taken from ``k_cache``."""
    d = AttnDesc()
    d.struct_size = ctypes.sizeof(AttnDesc)
    if q.dim() == 4:
        d.batch, q_len, d.num_q_heads, d.qk_dim = (int(x) for x in q.shape)
    else:
        d.batch, rows, d.qk_dim = (int(x) for x in q.shape)
        if rows % q_len:
            raise DcpValueError(DCP_ERR_INVALID_ARG, f"{rows} query rows are not {q_len} tokens")
        d.num_q_heads = rows // q_len
    d.q_len = int(q_len)
    if k_cache.numel() == 0:  # an empty pool reports zero strides; use contiguous ones
        strides, acc = [], 1
        for n in reversed(k_cache.shape):
            strides.append(acc)
            acc *= max(int(n), 1)
        stride = tuple(reversed(strides))
    else:
        stride = tuple(int(x) for x in k_cache.stride())
    d.kv_kind = kind
    if kind == KV_LATENT:
        d.num_kv_heads = 1
        d.v_dim = int(v_dim if v_dim is not None else d.qk_dim)
        d.kv_head_stride = 0
    else:
        d.num_kv_heads = int(k_cache.shape[2])
        d.v_dim = int(v_dim if v_dim is not None else k_cache.shape[3])
        d.kv_head_stride = stride[2]
    d.block_size = int(k_cache.shape[1])
    d.kv_block_stride = stride[0]
    d.kv_token_stride = stride[1]
    d.num_cache_blocks = int(k_cache.shape[0])
    d.max_blocks_per_seq = int(block_table.shape[1])
    d.num_shards = int(num_shards)
    d.max_seq_len = int(max_seq_len if max_seq_len is not None
                        else d.max_blocks_per_seq * d.block_size)
    d.q_dtype = _code(q)
    d.kv_dtype = _code(k_cache)
    d.out_dtype = out_dtype
    d.softmax_scale = float(softmax_scale if softmax_scale is not None
                            else 1.0 / math.sqrt(d.qk_dim))
    return d


def workspace_size(desc: AttnDesc) -> int:
    n = int(lib().dcp_workspace_size(ctypes.byref(desc)))
    if n == 0:
        raise DcpValueError(DCP_ERR_INVALID_ARG, "descriptor is invalid or unsupported")
    return n


def alloc_workspace(desc: AttnDesc, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte aligned blocks (checked by the library).
    return torch.empty(workspace_size(desc), dtype=torch.uint8, device=device)


def block_remap(block_table: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
                num_shards: int, local_table: Optional[torch.Tensor] = None,
                local_lens: Optional[torch.Tensor] = None, ownership: str = "interleaved"):
    """-> (local_table int32 [D, B, ceil(max_blocks / D)], local_lens int32 [D, B]).

    ``ownership`` is "interleaved" (block j on shard j % D) or "contiguous"
    (runs of ceil(nb / D) blocks per shard)."""
    if ownership not in _OWNERSHIP:
        raise DcpValueError(DCP_ERR_INVALID_ARG, f"unknown ownership {ownership!r}")
    B, mb = block_table.shape
    width = -(-mb // num_shards)
    dev = block_table.device
    if local_table is None:
        local_table = torch.empty((num_shards, B, width), dtype=torch.int32, device=dev)
    if local_lens is None:
        local_lens = torch.empty((num_shards, B), dtype=torch.int32, device=dev)
    _need(block_table, torch.int32, B * mb)
    _need(seq_lens, torch.int32, B)
    _need(local_table, torch.int32, num_shards * B * width)
    _need(local_lens, torch.int32, num_shards * B)
    _check(lib().dcp_block_remap_ex(_ptr(block_table), _ptr(seq_lens), B, mb, block_size,
                                    num_shards, _OWNERSHIP[ownership], _ptr(local_table),
                                    _ptr(local_lens), _stream(dev)))
    return local_table, local_lens


def block_remap_update(block_table: torch.Tensor, old_seq_lens: torch.Tensor,
                       seq_lens: torch.Tensor, block_size: int, num_shards: int,
                       local_table: torch.Tensor, local_lens: torch.Tensor):
    """Update (local_table, local_lens), the interleaved remap for ``old_seq_lens``, in place
    to the remap for ``seq_lens``; only blocks that were added or dropped are touched."""
    B, mb = block_table.shape
    width = -(-mb // num_shards)
    _need(block_table, torch.int32, B * mb)
    _need(old_seq_lens, torch.int32, B)
    _need(seq_lens, torch.int32, B)
    _need(local_table, torch.int32, num_shards * B * width)
    _need(local_lens, torch.int32, num_shards * B)
    _check(lib().dcp_block_remap_update(_ptr(block_table), _ptr(old_seq_lens), _ptr(seq_lens), B,
                                        mb, block_size, num_shards, _ptr(local_table),
                                        _ptr(local_lens), _stream(block_table.device)))
    return local_table, local_lens


def kv_append(desc: AttnDesc, positions: torch.Tensor, k_new: torch.Tensor,
              v_new: Optional[torch.Tensor], block_table: torch.Tensor, k_cache: torch.Tensor,
              v_cache: Optional[torch.Tensor], kv_scale: Optional[torch.Tensor], shard: int = -1,
              token_seq: Optional[torch.Tensor] = None):
    """Write each new token's row(s) (k_new [T, Hkv, qk_dim] or latent [T, qk_dim]; v_new
    [T, Hkv, v_dim]) into the cache slot of its position. shard=-1 takes the global block
    table; shard=r takes shard r's local table and writes only the tokens r owns."""
    n = int(positions.shape[0])
    rows = desc.num_kv_heads if desc.kv_kind == KV_SEPARATE else 1
    width = desc.max_blocks_per_seq if shard < 0 else -(-desc.max_blocks_per_seq // desc.num_shards)
    _need(positions, torch.int32, n)
    _need(k_new, None, n * rows * desc.qk_dim)
    if desc.kv_kind == KV_SEPARATE:
        _need(v_new, k_new.dtype, n * rows * desc.v_dim)
    if token_seq is not None:
        _need(token_seq, torch.int32, n)
    _need(block_table, torch.int32, desc.batch * width)
    if desc.kv_dtype == FP8_E4M3:
        _need(kv_scale, torch.float32, desc.num_cache_blocks * desc.block_size)
    _check(lib().dcp_kv_append(ctypes.byref(desc), n, _ptr(token_seq), _ptr(positions),
                               _ptr(k_new), _ptr(v_new), _code(k_new), int(shard),
                               _ptr(block_table), _ptr(k_cache), _ptr(v_cache), _ptr(kv_scale),
                               _stream(k_cache.device)))


def decode_partial(desc: AttnDesc, q, k_cache, v_cache, kv_scale, local_block_table,
                   local_seq_lens, workspace: Optional[torch.Tensor] = None,
                   o_partial: Optional[torch.Tensor] = None,
                   lse_partial: Optional[torch.Tensor] = None):
    """One shard's (O_r [B, Hq, v_dim] fp32, LSE_r [B, Hq] fp32)."""
    dev = q.device
    if workspace is None:
        workspace = alloc_workspace(desc, dev)
    rows = _rows(desc)
    if o_partial is None:
        o_partial = torch.empty((desc.batch, rows, desc.v_dim), dtype=torch.float32, device=dev)
    if lse_partial is None:
        lse_partial = torch.empty((desc.batch, rows), dtype=torch.float32, device=dev)
    _check(lib().dcp_decode_partial(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(kv_scale), _ptr(local_block_table),
                                    _ptr(local_seq_lens), _ptr(o_partial), _ptr(lse_partial),
                                    _ptr(workspace), workspace.numel(), _stream(dev)))
    return o_partial, lse_partial


def decode_partial_mtp(desc: AttnDesc, shard: int, q_pos: torch.Tensor, q, k_cache, v_cache,
                       kv_scale, local_block_table, local_seq_lens,
                       workspace: Optional[torch.Tensor] = None,
                       o_partial: Optional[torch.Tensor] = None,
                       lse_partial: Optional[torch.Tensor] = None):
    """One shard's multi-token partial: query t of sequence b at global position
    q_pos[b] + t sees that shard's positions up to its own. Returns
    (O_r [B, q_len * Hq, v_dim] fp32, LSE_r [B, q_len * Hq] fp32)."""
    dev = q.device
    if workspace is None:
        workspace = alloc_workspace(desc, dev)
    rows = _rows(desc)
    if o_partial is None:
        o_partial = torch.empty((desc.batch, rows, desc.v_dim), dtype=torch.float32, device=dev)
    if lse_partial is None:
        lse_partial = torch.empty((desc.batch, rows), dtype=torch.float32, device=dev)
    _need(q_pos, torch.int32, desc.batch)
    _check(lib().dcp_decode_partial_mtp(ctypes.byref(desc), int(shard), _ptr(q_pos), _ptr(q),
                                        _ptr(k_cache), _ptr(v_cache), _ptr(kv_scale),
                                        _ptr(local_block_table), _ptr(local_seq_lens),
                                        _ptr(o_partial), _ptr(lse_partial), _ptr(workspace),
                                        workspace.numel(), _stream(dev)))
    return o_partial, lse_partial


def decode_partial_token(desc: AttnDesc, shard: int, q, k_cache, v_cache, kv_scale, block_table,
                         seq_lens, workspace: Optional[torch.Tensor] = None,
                         o_partial: Optional[torch.Tensor] = None,
                         lse_partial: Optional[torch.Tensor] = None):
    """One shard's partial under token-level interleave (position t on shard
    t % D), over the global table and lengths: (O_r [B, Hq, v_dim], LSE_r [B, Hq])."""
    dev = q.device
    if workspace is None:
        workspace = alloc_workspace(desc, dev)
    rows = _rows(desc)
    if o_partial is None:
        o_partial = torch.empty((desc.batch, rows, desc.v_dim), dtype=torch.float32, device=dev)
    if lse_partial is None:
        lse_partial = torch.empty((desc.batch, rows), dtype=torch.float32, device=dev)
    _check(lib().dcp_decode_partial_token(ctypes.byref(desc), int(shard), _ptr(q), _ptr(k_cache),
                                          _ptr(v_cache), _ptr(kv_scale), _ptr(block_table),
                                          _ptr(seq_lens), _ptr(o_partial), _ptr(lse_partial),
                                          _ptr(workspace), workspace.numel(), _stream(dev)))
    return o_partial, lse_partial


def _rows(desc: AttnDesc) -> int:
    return max(1, int(desc.q_len)) * int(desc.num_q_heads)


def lse_merge(o_partials: torch.Tensor, lse_partials: torch.Tensor,
              out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
              lse_out: Optional[torch.Tensor] = None, want_lse: bool = True):
    """Merge [P, B, H, Dv] partials -> (O [B, H, Dv], LSE [B, H] or None)."""
    P, B, H, Dv = (int(x) for x in o_partials.shape)
    dev = o_partials.device
    if out is None:
        out = torch.empty((B, H, Dv), dtype=out_dtype, device=dev)
    if lse_out is None and want_lse:
        lse_out = torch.empty((B, H), dtype=torch.float32, device=dev)
    _check(lib().dcp_lse_merge(_ptr(o_partials), _ptr(lse_partials), P, B, H, Dv, _ptr(out),
                               _code(out), _ptr(lse_out), _stream(dev)))
    return out, lse_out


def decode_all_shards(desc: AttnDesc, q, k_cache, v_cache, kv_scale, block_table, seq_lens,
                      workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                      lse_out: Optional[torch.Tensor] = None, want_lse: bool = True,
                      attn_events=None):
    """All shards plus the merge: (O [B, Hq, v_dim] of desc.out_dtype, LSE [B, Hq] or None).

    ``attn_events`` = (begin, end) HIP event handles (see HipEvent) recorded
    around the attention kernel."""
    dev = q.device
    if workspace is None:
        workspace = alloc_workspace(desc, dev)
    rows = _rows(desc)
    if out is None:
        dt = torch.float32 if desc.out_dtype == F32 else torch.bfloat16
        out = torch.empty((desc.batch, rows, desc.v_dim), dtype=dt, device=dev)
    if lse_out is None and want_lse:
        lse_out = torch.empty((desc.batch, rows), dtype=torch.float32, device=dev)
    if attn_events is None:
        _check(lib().dcp_decode_all_shards(ctypes.byref(desc), _ptr(q), _ptr(k_cache),
                                           _ptr(v_cache), _ptr(kv_scale), _ptr(block_table),
                                           _ptr(seq_lens), _ptr(out), _ptr(lse_out),
                                           _ptr(workspace), workspace.numel(), _stream(dev)))
    else:
        ev0, ev1 = attn_events
        _check(lib().dcp_decode_all_shards_timed(
            ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_scale),
            _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse_out), _ptr(workspace),
            workspace.numel(), _stream(dev), ev0.handle, ev1.handle))
    return out, lse_out


def decode_partial_plan(desc: AttnDesc, local_seq_lens, workspace: torch.Tensor):
    """Plan one shard's partial for these local lengths into ``workspace``
    (reused by decode_partial_run until the next plan on it)."""
    _need(local_seq_lens, torch.int32, desc.batch)
    _check(lib().dcp_decode_partial_plan(ctypes.byref(desc), _ptr(local_seq_lens), _ptr(workspace),
                                         workspace.numel(), _stream(workspace.device)))
    return workspace


def decode_partial_run(desc: AttnDesc, q, k_cache, v_cache, kv_scale, local_block_table,
                       workspace: torch.Tensor, o_partial: Optional[torch.Tensor] = None,
                       lse_partial: Optional[torch.Tensor] = None):
    """decode_partial on the plan in ``workspace`` (decode_partial_plan): the
    lengths are the planned ones. Returns (O_r, LSE_r)."""
    dev = q.device
    rows = _rows(desc)
    if o_partial is None:
        o_partial = torch.empty((desc.batch, rows, desc.v_dim), dtype=torch.float32, device=dev)
    if lse_partial is None:
        lse_partial = torch.empty((desc.batch, rows), dtype=torch.float32, device=dev)
    _check(lib().dcp_decode_partial_run(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(kv_scale), _ptr(local_block_table), _ptr(o_partial),
                                        _ptr(lse_partial), _ptr(workspace), workspace.numel(),
                                        _stream(dev)))
    return o_partial, lse_partial


def decode_all_shards_plan(desc: AttnDesc, seq_lens, workspace: torch.Tensor):
    """Plan the fused all-shards call for these global lengths into ``workspace``."""
    _need(seq_lens, torch.int32, desc.batch)
    _check(lib().dcp_decode_all_shards_plan(ctypes.byref(desc), _ptr(seq_lens), _ptr(workspace),
                                            workspace.numel(), _stream(workspace.device)))
    return workspace


def decode_all_shards_run(desc: AttnDesc, q, k_cache, v_cache, kv_scale, block_table,
                          workspace: torch.Tensor, out: Optional[torch.Tensor] = None,
                          lse_out: Optional[torch.Tensor] = None, want_lse: bool = True):
    """decode_all_shards on the plan in ``workspace`` (decode_all_shards_plan)."""
    dev = q.device
    rows = _rows(desc)
    if out is None:
        dt = torch.float32 if desc.out_dtype == F32 else torch.bfloat16
        out = torch.empty((desc.batch, rows, desc.v_dim), dtype=dt, device=dev)
    if lse_out is None and want_lse:
        lse_out = torch.empty((desc.batch, rows), dtype=torch.float32, device=dev)
    _check(lib().dcp_decode_all_shards_run(ctypes.byref(desc), _ptr(q), _ptr(k_cache),
                                           _ptr(v_cache), _ptr(kv_scale), _ptr(block_table),
                                           _ptr(out), _ptr(lse_out), _ptr(workspace),
                                           workspace.numel(), _stream(dev)))
    return out, lse_out


def decode_all_shards_noalloc(desc: AttnDesc, q, k_cache, v_cache, kv_scale, block_table,
                              seq_lens, out: torch.Tensor, lse_out: Optional[torch.Tensor] = None):
    """decode_all_shards without a workspace: the library's static device scratch
    holds the plan and partials. ``out`` (and ``lse_out``) are the caller's buffers;
    the call allocates nothing."""
    _check(lib().dcp_decode_all_shards_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache),
                                               _ptr(v_cache), _ptr(kv_scale), _ptr(block_table),
                                               _ptr(seq_lens), _ptr(out), _ptr(lse_out),
                                               _stream(q.device)))
    return out, lse_out


class HipEvent:
    """A raw HIP event (hipEventCreate / hipEventElapsedTime through ctypes)."""

    _hip = None

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            h.hipEventCreate.restype = ctypes.c_int
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            h.hipEventDestroy.restype = ctypes.c_int
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventElapsedTime.restype = ctypes.c_int
            cls._hip = h
        return cls._hip

    def __init__(self):
        self.handle = ctypes.c_void_p()
        rc = self._rt().hipEventCreate(ctypes.byref(self.handle))
        if rc != 0:
            raise DcpError(DCP_ERR_HIP, f"hipEventCreate failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = self._rt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise DcpError(DCP_ERR_HIP, f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and self.handle:
            self._hip.hipEventDestroy(self.handle)
