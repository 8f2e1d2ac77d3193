"""Helpers for the GPU tests: host numpy storage <-> torch device tensors, tolerances."""

import numpy as np
import torch

# Attention tolerance on float32 outputs, per input dtype: 1e-5 for fp32 inputs,
# 5e-3 for fp16/bf16 inputs with fp32 accumulation.
TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 5e-3}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def up(a: np.ndarray, dt: str | None = None, dev="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def down(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy storage array (bf16 as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    """Raw bit pattern view (NaN-safe equality)."""
    return a.view({2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def rne_to(x32: np.ndarray, dt: str) -> np.ndarray:
    """float32 -> storage dtype, round to nearest even (the expected rounding of a dtype output)."""
    if dt == "f32":
        return x32
    if dt == "f16":
        return x32.astype(np.float16)
    u = x32.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def upload_decode(d, dev="cuda"):
    return dict(
        q=up(d.q, d.dtype, dev), k_cache=up(d.k_cache, d.dtype, dev), v_cache=up(d.v_cache, d.dtype, dev),
        block_tables=up(d.block_tables, None, dev), context_lens=up(d.context_lens, None, dev),
    )


def run_decode(ops, t, d, out_dtype="f32", partition_size=512, fn=None, fill=float("nan")):
    out = nan_out(d.q.shape, out_dtype, dev=t["q"].device, fill=fill)
    (fn or ops.paged_attn_decode)(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                  d.scale, out, max_context_len=d.max_context_len, partition_size=partition_size)
    return out


def nan_out(shape, out_dtype: str | torch.dtype = "f32", dev="cuda", fill=float("nan")) -> torch.Tensor:
    """An output buffer filled with NaN before the launch, so that any element a
    kernel fails to write fails the comparison instead of passing on stale data.
    Tests that expect NaN outputs pass a finite `fill` instead."""
    dt = TORCH_DT[out_dtype] if isinstance(out_dtype, str) else out_dtype
    return torch.full(tuple(shape), fill, dtype=dt, device=dev)


def timed(fn, *args, **kw):
    """(fn(*args, **kw), seconds it took)."""
    import time

    t0 = time.perf_counter()
    r = fn(*args, **kw)
    return r, time.perf_counter() - t0
