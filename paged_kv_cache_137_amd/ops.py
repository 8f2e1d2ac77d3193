"""Python entry points of the paged-attention hot path, over torch device tensors.

Each function checks shapes and dtypes, then hands raw device pointers, sizes and
the current HIP stream to the matching C call in libpkv.so.  torch only provides
memory and the stream.  The computation is entirely in the library's kernels.
"""

from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import CacheDesc, check, lib

BLOCK_SIZE = 16           # the default block size (tokens per block)
BLOCK_SIZES = (8, 16, 32)  # block sizes the library is built for
PARTITION_AUTO = _lib.PKV_PARTITION_AUTO  # the library picks the partition from the batch shape
DEFAULT_PARTITION = PARTITION_AUTO

_DT = {torch.float32: _lib.PKV_F32, torch.float16: _lib.PKV_F16, torch.bfloat16: _lib.PKV_BF16}


def pkv_dtype(dt: torch.dtype) -> int:
    try:
        return _DT[dt]
    except KeyError:
        raise ValueError(f"unsupported dtype {dt}; use float32, float16 or bfloat16") from None


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, dim=None, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def cache_desc(k_cache: torch.Tensor) -> CacheDesc:
    nb, H, B, D = k_cache.shape
    return CacheDesc(nb, H, D, B, pkv_dtype(k_cache.dtype))


def kv_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Write new tokens' K/V [T][H][D] into the slots slot_mapping (int64 [T]) names."""
    _need(k_cache, "k_cache", dim=4)
    dev = k_cache.device
    _need(v_cache, "v_cache", dtype=k_cache.dtype, device=dev)
    _need(k, "k", dtype=k_cache.dtype, dim=3, device=dev)
    _need(v, "v", dtype=k_cache.dtype, dim=3, device=dev)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, dim=1, device=dev)
    if v_cache.shape != k_cache.shape or v.shape != k.shape:
        raise ValueError("k/v and k_cache/v_cache shapes must match")
    T, H, D = k.shape
    if (H, D) != (k_cache.shape[1], k_cache.shape[3]) or slot_mapping.shape[0] != T:
        raise ValueError("k [T][H][D] does not match the cache or slot_mapping")
    desc = cache_desc(k_cache)
    with torch.cuda.device(dev):
        check("pkv_kv_cache_write", lib().pkv_kv_cache_write(
            _ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _stream(dev)))


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_pairs: torch.Tensor) -> None:
    """Copy whole blocks, (src, dst) rows of int64 block_pairs [n][2], keys and values, in one launch."""
    _need(k_cache, "k_cache", dim=4)
    dev = k_cache.device
    _need(v_cache, "v_cache", dtype=k_cache.dtype, device=dev)
    _need(block_pairs, "block_pairs", dtype=torch.int64, dim=2, device=dev)
    if v_cache.shape != k_cache.shape or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n][2]; k_cache and v_cache must match")
    desc = cache_desc(k_cache)
    with torch.cuda.device(dev):
        check("pkv_copy_blocks", lib().pkv_copy_blocks(
            _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(block_pairs), block_pairs.shape[0], _stream(dev)))


def decode_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                           partition_size: int = DEFAULT_PARTITION) -> int:
    return int(lib().pkv_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, partition_size))


def decode_shared_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                                  partition_size: int = DEFAULT_PARTITION) -> int:
    return int(lib().pkv_decode_shared_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len,
                                                       partition_size))


def decode_partition(num_seqs: int, num_heads: int, max_context_len: int,
                     partition_size: int = DEFAULT_PARTITION, shared: bool = False) -> int:
    """The partition size (0 = no split) a decode call uses for these arguments.

    Raises ValueError for an invalid shape (num_seqs < 0, num_heads <= 0,
    max_context_len <= 0, partition_size below PARTITION_AUTO)."""
    res = ctypes.c_int32(0)
    st = lib().pkv_decode_partition(num_seqs, num_heads, max_context_len, partition_size, int(shared),
                                    ctypes.byref(res))
    if st != _lib.PKV_OK:
        raise ValueError(f"decode_partition: invalid shape ({lib().pkv_status_str(st).decode()})")
    return int(res.value)


def decode_partition_for_lengths(context_lens, num_heads: int) -> int:
    """A partition size chosen from the context lengths themselves (host values:
    a sequence of ints or a CPU array), for callers that know them; 0 = no split.

    Raises ValueError when a length is below 1 or num_heads <= 0: an invalid
    batch never becomes a partition size (in particular not PARTITION_AUTO)."""
    import numpy as np

    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if lens.ndim != 1:
        raise ValueError("context_lens must be one-dimensional")
    res = ctypes.c_int32(0)
    st = lib().pkv_decode_partition_for_lengths(lens.ctypes.data if lens.size else None, int(lens.size),
                                                int(num_heads), ctypes.byref(res))
    if st != _lib.PKV_OK:
        raise ValueError(f"decode_partition_for_lengths: invalid batch ({lib().pkv_status_str(st).decode()})")
    return int(res.value)


def _decode_call(fn_name, q, k_cache, v_cache, block_tables, context_lens, scale, out,
                 max_context_len, partition_size, workspace):
    _need(k_cache, "k_cache", dim=4)
    dev = k_cache.device
    _need(v_cache, "v_cache", dtype=k_cache.dtype, device=dev)
    _need(q, "q", dtype=k_cache.dtype, dim=3, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    _need(out, "out", dim=3, device=dev)
    S, H, D = q.shape
    if v_cache.shape != k_cache.shape or (H, D) != (k_cache.shape[1], k_cache.shape[3]):
        raise ValueError("q [S][H][D] does not match the cache")
    if out.shape != q.shape or out.dtype not in (torch.float32, q.dtype):
        raise ValueError("out must be [S][H][D] of float32 or q's dtype")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables/context_lens must have one row per sequence")
    mbps = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = mbps * k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    sizer = decode_shared_workspace_bytes if fn_name == "pkv_paged_attn_decode_shared" else decode_workspace_bytes
    need = sizer(S, H, D, max_context_len, partition_size) if S else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    desc = cache_desc(k_cache)
    with torch.cuda.device(dev):
        check(fn_name, getattr(lib(), fn_name)(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(block_tables), mbps,
            _ptr(context_lens), S, int(max_context_len), float(scale), _ptr(out), pkv_dtype(out.dtype),
            int(partition_size), _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, *,
                      max_context_len: int | None = None, partition_size: int = DEFAULT_PARTITION,
                      workspace: torch.Tensor | None = None):
    """Decode attention of q [S][H][D] over each sequence's paged context; fills out.

    max_context_len bounds every context_lens entry.  By default it is the table
    capacity (max_blocks_per_seq * block_size).  partition_size = 0 disables the
    split-context path; PARTITION_AUTO (the default) lets the library choose from
    the batch shape: no split when num_seqs * ceil(num_heads / 4) >= 1024 and
    max_context_len is at most 4096 tokens, else partitions of 256 to 2048 tokens
    that give about that many units (decode_partition reports the choice).  The
    rule reads max_context_len, not the lengths on the device: with the default
    (the table capacity), tables padded past 4096 tokens make a large batch
    split even when every real context is short; pass the real maximum when it
    is known.  Without a workspace, one is allocated through torch.

    Leading blocks that neighbouring sequences share (parallel samples, a
    common prefix: the same physical ids at the start of their tables, within
    windows of four consecutive sequences) are found on the device and read
    once for all of them.
    """
    return _decode_call("pkv_paged_attn_decode", q, k_cache, v_cache, block_tables, context_lens, scale, out,
                        max_context_len, partition_size, workspace)


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out, *,
                              max_context_len: int | None = None, partition_size: int = DEFAULT_PARTITION):
    """paged_attn_decode without a workspace, for callers that cannot allocate
    (graph capture, tight serving loops): the library's fixed per-GPU scratch
    (PKV_NOALLOC_SCRATCH_BYTES) serves instead, and nothing is allocated.  Calls
    that may overlap on one GPU race on that scratch.  Raises PKVError with
    PKV_EWORKSPACE when the batch needs more scratch than that."""
    _need(k_cache, "k_cache", dim=4)
    dev = k_cache.device
    _need(v_cache, "v_cache", dtype=k_cache.dtype, device=dev)
    _need(q, "q", dtype=k_cache.dtype, dim=3, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    _need(out, "out", dim=3, device=dev)
    S, H, D = q.shape
    if v_cache.shape != k_cache.shape or (H, D) != (k_cache.shape[1], k_cache.shape[3]):
        raise ValueError("q [S][H][D] does not match the cache")
    if out.shape != q.shape or out.dtype not in (torch.float32, q.dtype):
        raise ValueError("out must be [S][H][D] of float32 or q's dtype")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables/context_lens must have one row per sequence")
    mbps = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = mbps * k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    desc = cache_desc(k_cache)
    with torch.cuda.device(dev):
        check("pkv_paged_attn_decode_noalloc", lib().pkv_paged_attn_decode_noalloc(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(block_tables), mbps,
            _ptr(context_lens), S, int(max_context_len), float(scale), _ptr(out), pkv_dtype(out.dtype),
            int(partition_size), _stream(dev)))
    return out


def paged_attn_decode_shared(q, k_cache, v_cache, block_tables, context_lens, scale, out, *,
                             max_context_len=None, partition_size=DEFAULT_PARTITION, workspace=None):
    """paged_attn_decode under the shared-prefix decode's name: the one-call
    decode reads shared leading blocks once itself.  Same arguments and result."""
    return _decode_call("pkv_paged_attn_decode_shared", q, k_cache, v_cache, block_tables, context_lens, scale,
                        out, max_context_len, partition_size, workspace)


def paged_attn_decode_partial(q, k_cache, v_cache, block_tables, context_lens, scale, out, *,
                              max_context_len=None, partition_size=DEFAULT_PARTITION, workspace=None):
    """First stage of the two-stage decode (plan and per-partition kernels).  The
    two-stage form does not look for shared blocks; with the second stage it
    equals paged_attn_decode bit for bit on batches without sharing."""
    return _decode_call("pkv_paged_attn_decode_partial", q, k_cache, v_cache, block_tables, context_lens, scale,
                        out, max_context_len, partition_size, workspace)


def paged_attn_decode_reduce(q, k_cache, v_cache, block_tables, context_lens, scale, out, *,
                             max_context_len=None, partition_size=DEFAULT_PARTITION, workspace=None):
    """Second stage of the two-stage decode (the split-context reduce; nothing
    runs when no context is split)."""
    return _decode_call("pkv_paged_attn_decode_reduce", q, k_cache, v_cache, block_tables, context_lens, scale,
                        out, max_context_len, partition_size, workspace)


def kv_read_probe(k_cache, v_cache, block_tables, context_lens, out=None, *, max_context_len: int | None = None,
                  partition_size: int = DEFAULT_PARTITION, workspace: torch.Tensor | None = None):
    """The decode's K/V tile reads without its arithmetic (a measurement aid).

    Returns out, uint32 [S][H] as int32 storage: the XOR of every 32-bit word of
    each sequence's K and V tiles for that head, over blocks 0 .. ceil(ctx/B)-1.
    """
    _need(k_cache, "k_cache", dim=4)
    dev = k_cache.device
    _need(v_cache, "v_cache", dtype=k_cache.dtype, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, dim=1, device=dev)
    S, H = context_lens.shape[0], k_cache.shape[1]
    if out is None:
        out = torch.zeros((S, H), dtype=torch.int32, device=dev)
    else:
        _need(out, "out", dtype=torch.int32, dim=2, device=dev)
        out.zero_()
    mbps = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = mbps * k_cache.shape[2]
    need = decode_workspace_bytes(S, H, k_cache.shape[3], max_context_len, partition_size) if S else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    desc = cache_desc(k_cache)
    with torch.cuda.device(dev):
        check("pkv_kv_read_probe", lib().pkv_kv_read_probe(
            _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(block_tables), mbps, _ptr(context_lens), S,
            int(max_context_len), int(partition_size), _ptr(out), _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def paged_attn_prefill(q, k, v, block_tables, prompt_lens, out, *, scale: float | None = None,
                       max_prompt_len: int | None = None):
    """Causal attention of packed prompts q/k/v [T][H][D] (f16 or bf16); fills out.

    prompt_lens is an int32 device tensor.  max_prompt_len bounds its entries;
    by default it is T.  block_tables may be None.  It is reserved, because the
    prompt's contiguous k/v hold the same bytes as its blocks once written.
    """
    _need(q, "q", dim=3)
    dev = q.device
    _need(k, "k", dtype=q.dtype, device=dev)
    _need(v, "v", dtype=q.dtype, device=dev)
    _need(prompt_lens, "prompt_lens", dtype=torch.int32, dim=1, device=dev)
    _need(out, "out", dim=3, device=dev)
    if k.shape != q.shape or v.shape != q.shape or out.shape != q.shape:
        raise ValueError("q, k, v and out must all be [T][H][D]")
    if out.dtype not in (torch.float32, q.dtype):
        raise ValueError("out must be float32 or q's dtype")
    T, H, D = q.shape
    mbps = 0
    if block_tables is not None:
        _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
        mbps = block_tables.shape[1]
    if max_prompt_len is None:
        max_prompt_len = T
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with torch.cuda.device(dev):
        check("pkv_paged_attn_prefill", lib().pkv_paged_attn_prefill(
            _ptr(q), _ptr(k), _ptr(v), H, D, pkv_dtype(q.dtype), _ptr(block_tables), mbps, _ptr(prompt_lens),
            prompt_lens.shape[0], T, int(max_prompt_len), float(scale), _ptr(out), pkv_dtype(out.dtype),
            _stream(dev)))
    return out


def paged_attn_prefill_cached(q, k_cache, v_cache, block_tables, prefix_lens, prompt_lens, out, *,
                              scale: float | None = None, max_prompt_len: int | None = None,
                              max_prefix_len: int | None = None):
    """Prompt phase of new tokens q [T][H][D] over cached prefixes plus themselves; fills out.

    Prompt p's first prefix_lens[p] positions are already cached, and its new
    tokens' K/V have been written after them.  Everything is read through
    block_tables.  prefix_lens may be None (no prefix).  max_prompt_len and
    max_prefix_len bound the entries; by default they are T and the table
    capacity minus max_prompt_len.
    """
    _need(k_cache, "k_cache", dim=4)
    dev = k_cache.device
    _need(v_cache, "v_cache", dtype=k_cache.dtype, device=dev)
    _need(q, "q", dtype=k_cache.dtype, dim=3, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, dim=2, device=dev)
    _need(prompt_lens, "prompt_lens", dtype=torch.int32, dim=1, device=dev)
    if prefix_lens is not None:
        _need(prefix_lens, "prefix_lens", dtype=torch.int32, dim=1, device=dev)
    _need(out, "out", dim=3, device=dev)
    T, H, D = q.shape
    if out.shape != q.shape or out.dtype not in (torch.float32, q.dtype):
        raise ValueError("out must be [T][H][D] of float32 or q's dtype")
    if v_cache.shape != k_cache.shape or (H, D) != (k_cache.shape[1], k_cache.shape[3]):
        raise ValueError("q [T][H][D] does not match the cache")
    P = prompt_lens.shape[0]
    if block_tables.shape[0] != P or (prefix_lens is not None and prefix_lens.shape[0] != P):
        raise ValueError("one block table row and one prefix length per prompt")
    mbps = block_tables.shape[1]
    if max_prompt_len is None:
        max_prompt_len = T
    if max_prefix_len is None:
        max_prefix_len = max(0, mbps * k_cache.shape[2] - max_prompt_len)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    desc = cache_desc(k_cache)
    with torch.cuda.device(dev):
        check("pkv_paged_attn_prefill_cached", lib().pkv_paged_attn_prefill_cached(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(block_tables), mbps,
            _ptr(prefix_lens), _ptr(prompt_lens), P, T, int(max_prompt_len), int(max_prefix_len), float(scale),
            _ptr(out), pkv_dtype(out.dtype), _stream(dev)))
    return out


def swap_blocks(src_k: torch.Tensor, src_v: torch.Tensor, dst_k: torch.Tensor, dst_v: torch.Tensor,
                block_pairs: torch.Tensor, device=None) -> None:
    """Copy (src block, dst block) pairs from one pool to another, in one launch.

    Either pool may live on the GPU or in pinned host memory
    (torch.empty(..., pin_memory=True)); block_pairs (int64 [n][2]) likewise.
    The copy runs on `device`'s current stream (by default, the GPU pool's
    device).  This is the swap-out / swap-in of a preempted sequence's blocks.
    """
    for name, t in (("src_k", src_k), ("src_v", src_v), ("dst_k", dst_k), ("dst_v", dst_v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [blocks][H][B][D] tensor")
        if not t.is_cuda and not t.is_pinned():
            raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    if src_k.shape != src_v.shape or dst_k.shape != dst_v.shape or src_k.shape[1:] != dst_k.shape[1:]:
        raise ValueError("pools must agree in [H][B][D]")
    if len({src_k.dtype, src_v.dtype, dst_k.dtype, dst_v.dtype}) != 1:
        raise ValueError("pools must share one dtype")
    if block_pairs.dtype != torch.int64 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be int64 [n][2]")
    if not block_pairs.is_cuda and not block_pairs.is_pinned():
        raise ValueError("block_pairs must be on the GPU or in pinned host memory")
    if device is None:
        device = next((t.device for t in (src_k, dst_k, block_pairs) if t.is_cuda), torch.device("cuda", 0))
    desc = cache_desc(src_k)
    with torch.cuda.device(device):
        check("pkv_swap_blocks", lib().pkv_swap_blocks(
            _ptr(src_k), _ptr(src_v), src_k.shape[0], _ptr(dst_k), _ptr(dst_v), dst_k.shape[0], ctypes.byref(desc),
            _ptr(block_pairs), block_pairs.shape[0], _stream(device)))
