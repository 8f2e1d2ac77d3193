"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one decode step of the Llama-2-7B-shaped workload: 256 sequences,
32 heads x 128, bf16, 16-token blocks, context lengths lognormal (median 600,
sigma 0.8) clipped to [16, 4096], in shuffled physical blocks.  The step
  1. writes the 256 current tokens' K/V into their slots (kv_cache_write),
  2. runs paged_attn_decode, the one-call decode: the plan kernel and the
     persistent decode kernel, with the library's automatic context partition
     (for 256 sequences x 8 head groups: no split, so no reduce runs;
     --partition 512 times the split path and its reduce instead).
Inputs are resident in HBM before the timed region starts.  One JSON line is
printed.  value = KV bytes attended per step (sum of context lengths x 2 x heads
x head_dim x 2 B) / wall time per step.

The same line also carries:
  roofline      the decode kernel alone.  Algorithmic bytes per launch / its
                mean duration from HIP events on the launch stream, against
                MI355X's 8 TB/s.  traffic comes from the committed rocprofv3
                counter summary, if it was taken on this kernel source.
  cpu_baseline  the float64 CPU oracle as it stands, on the host's cores (one
                process per core) and on one thread, over a time-boxed sample
                of the same step's sequences; and its prefill on the mixed
                step's 8 prompts.
  mixed_step    the mixed prefill+decode step (8 prompts prefilled while 192
                sequences decode), per kernel, with prefill's MFMA rate; and
                the same step with the prefill on a second stream beside the
                write and the decode.
  opt13b_decode the OPT-13B-shape decode step (fp16, 64 sequences, 40 heads).
  sharing_step  parallel sampling over shared prompt blocks: the batched
                copy-on-write copy, then decode (logical and unique KV GB/s),
                through paged_attn_decode (which reads shared blocks once) and
                through the two-stage form (which does not).
  cached_prefix_prefill  requests prefilling over one cached shared prefix.
  prefill_prompt_count  the fresh prefill alone on the mixed step's 8 prompts and on
                256 prompts of the same length distribution.
  headline_sustained_1s  the headline step back to back for about a second,
                with the GPU's shader clock sampled meanwhile (rocm-smi); the
                8-prompt prefill gets the same sustained run and clock sample.
  block_size_sweep  the same decode at 8-, 16- and 32-token blocks (the pool's
                bytes re-tiled, fresh shuffled tables).
  decode_launch_shape  the headline decode at 1, 2 and 4 workgroups per CU.
  config3_as_written  the headline batch with 512-token partitions and the
                reduce, in the two-stage form.
  read_probe    the decode's tile reads without its arithmetic, in table order
                and in address order: the ceiling of the access pattern.
  hbm_reference a contiguous PyTorch sum and copy over the same K pool, for
                context (the decode's gathered reads outrun both).
  swap          swap-out/swap-in of 2048 blocks between the device pool and a
                pinned host pool (pkv_swap_blocks), beside a plain contiguous
                device<->host copy of the same bytes.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV HBM GB/s (% of peak) + tokens attended/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
PMC_SUMMARY = os.path.join(ROOT, "profiles", "paged_decode_pmc.txt")
# The decode kernel's source and the headers it includes: the counter-derived
# traffic is reported only while these are unchanged.
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_137_amd", "csrc", f)
                  for f in ("paged_decode.hip", "pkv_device.h", "pkv_internal.h")]


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--partition", type=int, default=-1,
                    help="decode partition in tokens; -1 (default) = the library's automatic choice, 0 = no split")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the sharing and cached-prefix measurements")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU oracle sample: about a quarter of this per leg (decode / prefill, 1 thread / all cores)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of a known size (for counter calibration) and exit")
    return ap.parse_args()


def source_digest(paths=DECODE_SOURCES) -> str:
    h = hashlib.sha1()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:12]


def read_pmc_summary():
    """Counter-derived HBM bytes per decode launch, if taken on the current kernel source."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    kv = {}
    for line in open(PMC_SUMMARY):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("decode_source_sha1") != source_digest():
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main() -> int:
    a = _args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the library runs on one GPU and has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from paged_kv_cache_137_amd import ops
    from paged_kv_cache_137_amd import workloads as W
    from paged_kv_cache_137_amd.blocks import slot_mapping

    dev = torch.device("cuda:0")

    def up(x, dt=None):
        x = np.ascontiguousarray(x)
        if dt == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    if a.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n}))
        return 0

    # ---------------- decode step (the headline) ----------------
    d = W.decode_config(3, poison=False, with_new_tokens=True)
    # The CPU oracle baseline runs first: its process pool is forked before this
    # process initialises the GPU.
    cpu_line = None
    if not a.no_cpu_baseline:
        cpu_line = cpu_baseline(d, W.mixed_prefill(), a.cpu_seconds)
    torch.cuda.set_device(dev)
    S, H, D = d.q.shape
    sum_ctx = int(d.context_lens.sum())
    kv_bytes = sum_ctx * 2 * H * D * 2
    t = dict(q=up(d.q, "bf16"), kc=up(d.k_cache, "bf16"), vc=up(d.v_cache, "bf16"),
             bt=up(d.block_tables), cl=up(d.context_lens), kn=up(d.k_new, "bf16"), vn=up(d.v_new, "bf16"))
    t["sm"] = up(slot_mapping(d.block_tables, np.arange(S), d.context_lens - 1))
    out = torch.empty((S, H, D), dtype=torch.bfloat16, device=dev)
    mcl = d.max_context_len
    part_used = ops.decode_partition(S, H, mcl, a.partition)
    ws = torch.empty(max(1, ops.decode_workspace_bytes(S, H, D, mcl, a.partition)), dtype=torch.uint8, device=dev)
    dargs = (t["q"], t["kc"], t["vc"], t["bt"], t["cl"], d.scale, out)
    dkw = dict(max_context_len=mcl, partition_size=a.partition, workspace=ws)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ops.kv_cache_write(t["kn"], t["vn"], t["sm"], t["kc"], t["vc"])
        if ev is not None:
            ev[1].record()
        ops.paged_attn_decode(*dargs, **dkw)
        if ev is not None:
            ev[2].record()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / a.steps

    # per-kernel durations from HIP events on the launch stream (a separate, equal pass)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    t_write = [e[0].elapsed_time(e[1]) for e in evs]
    t_dec = [e[1].elapsed_time(e[2]) for e in evs]
    k_write, k_dec = (sum(x) / a.steps for x in (t_write, t_dec))

    def pct(x):
        q = np.percentile(np.asarray(x), [10, 50, 90])
        return [round(float(v), 5) for v in q]

    value = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = kv_bytes / (k_dec * 1e-3) / 1e9
    traffic = read_pmc_summary()
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-2-7B-shape paged decode step: 256 seqs, 32 heads x 128, bf16, 16-token blocks, "
                        "ctx lognormal(600, 0.8) in [16, 4096], shuffled blocks, "
                        + ("automatic partition" if a.partition == ops.PARTITION_AUTO else f"partition {a.partition}")
                        + f" (resolved: {part_used or 'no split'})",
            "num_seqs": S, "num_heads": H, "head_dim": D, "block_size": 16, "partition_size": a.partition,
            "partition_resolved": part_used,
            "sum_context_len": sum_ctx, "max_context_len": mcl, "num_blocks": d.num_blocks,
            "seed": W.config_seed(3),
        },
        "pct_of_peak_hbm": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_attended_per_s": round(sum_ctx / (ms_step * 1e-3), 1),
        "head_tokens_attended_per_s": round(sum_ctx * H / (ms_step * 1e-3), 1),
        "kernels_ms": {"kv_cache_write": round(k_write, 5), "paged_attn_decode": round(k_dec, 5)},
        "kernels_ms_p10_p50_p90": {"kv_cache_write": pct(t_write), "paged_attn_decode": pct(t_dec)},
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_plan_kernel + decode_kernel<bf16,bf16,128,16> (one pkv_paged_attn_decode call, "
                      "bracketed by HIP events; this batch is not split, so no reduce runs)",
            "launch_ms": round(k_dec, 5),
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": kv_bytes,
            "traffic": None if traffic is None else int(traffic),
        },
    }
    # The same step back to back for about a second, the shader clock sampled
    # meanwhile (context for the prefill's clock under its matrix work).
    with _ClockSampler() as clk:
        t_end, n_sus = time.perf_counter() + 1.0, 0
        t1 = time.perf_counter()
        while time.perf_counter() < t_end:
            for _ in range(5):
                step()
            n_sus += 5
            torch.cuda.synchronize()
        sus_wall = time.perf_counter() - t1
    line["headline_sustained_1s"] = {"steps": n_sus, "ms_per_step": round(sus_wall * 1e3 / n_sus, 4),
                                     "sclk_MHz": clk.summary()}
    line["config3_as_written"] = config3_as_written(a, t, d)
    line["read_probe"] = read_probe(a, t, d, k_dec)
    if not a.no_extras:
        line["block_size_sweep"] = block_size_sweep(a, t, d)
        line["swap"] = swap_step(a, t)
        line["hbm_reference"] = hbm_reference(t)
        line["decode_launch_shape"] = decode_launch_shape(a, t, d, dargs, dkw)
    del t, ws, out
    torch.cuda.empty_cache()

    # ---------------- mixed prefill + decode step ----------------
    if not a.no_mixed:
        line["mixed_step"] = mixed_step(a, dev, up)

    # ---------------- sharing, copy-on-write and cached-prefix prefill ----------------
    if not a.no_extras:
        line["opt13b_decode"] = opt13b_decode(a, dev, up)
        line["sharing_step"] = sharing_step(a, dev, up)
        line["cached_prefix_prefill"] = cached_prefix_prefill(a, dev, up)
        line["prefill_prompt_count"] = prefill_prompt_count(a, dev, up)

    if cpu_line is not None:
        line["cpu_baseline"] = cpu_line
    print(json.dumps(line), flush=True)
    return 0


def config3_as_written(a, t, d):
    """The headline batch exactly as the configuration states it: the split
    into 512-token partitions followed by the reduce, in the two-stage form
    (plan + persistent decode, then the reduce), timed by the wall clock and
    per stage with HIP events."""
    import numpy as np
    import torch

    from paged_kv_cache_137_amd import ops

    S, H, D = d.q.shape
    kv_bytes = int(d.context_lens.sum()) * 2 * H * D * 2
    out = torch.empty((S, H, D), dtype=torch.bfloat16, device=t["q"].device)
    ws = torch.empty(ops.decode_workspace_bytes(S, H, D, d.max_context_len, 512), dtype=torch.uint8,
                     device=t["q"].device)
    args = (t["q"], t["kc"], t["vc"], t["bt"], t["cl"], d.scale, out)
    kw = dict(max_context_len=d.max_context_len, partition_size=512, workspace=ws)

    def run(ev=None):
        if ev is not None:
            ev[0].record()
        ops.paged_attn_decode_partial(*args, **kw)
        if ev is not None:
            ev[1].record()
        ops.paged_attn_decode_reduce(*args, **kw)
        if ev is not None:
            ev[2].record()

    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    p_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    r_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    splits = int((d.context_lens > 512).sum())
    return {"workload": "headline batch, 512-token partitions + reduce (two-stage form)",
            "sequences_split": splits, "ms": round(ms, 4), "GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
            "frac": round(kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernels_ms": {"plan_and_decode": round(p_ms, 5), "reduce": round(r_ms, 5)}}


def read_probe(a, t, d, decode_ms):
    """The decode's K/V tile reads without its arithmetic (pkv_kv_read_probe):
    the same plan, scheduling and nontemporal 16-byte loads over the headline
    batch's blocks, first through its shuffled tables, then with the same
    sequences' blocks laid out in address order.  Its rate is the ceiling of
    this access pattern on this GPU; the decode's time is set beside it."""
    import numpy as np
    import torch

    from paged_kv_cache_137_amd import ops

    S, H, D = d.q.shape
    ctx = d.context_lens.astype(np.int64)
    tiles = int((-(-ctx // 16)).sum())
    tile_bytes = tiles * 16 * 2 * H * D * 2  # whole tiles, keys and values
    ws = torch.empty(ops.decode_workspace_bytes(S, H, D, d.max_context_len, ops.PARTITION_AUTO), dtype=torch.uint8,
                     device=t["q"].device)
    out = torch.zeros((S, H), dtype=torch.int32, device=t["q"].device)
    res = {"workload": "headline batch's K/V tiles, whole 16-token tiles, keys and values",
           "bytes": tile_bytes}
    need = -(-ctx // 16)
    offs = np.concatenate([[0], np.cumsum(need)])
    seq_tables = np.zeros_like(d.block_tables)
    for s_ in range(S):
        seq_tables[s_, : need[s_]] = np.arange(offs[s_], offs[s_ + 1], dtype=np.int32)
        seq_tables[s_, need[s_]:] = offs[s_]
    for name, bt in (("table_order", t["bt"]), ("address_order", torch.from_numpy(seq_tables).to(t["q"].device))):
        ms = _time_events(lambda: ops.kv_read_probe(t["kc"], t["vc"], bt, t["cl"], out,
                                                    max_context_len=d.max_context_len, workspace=ws),
                          a.warmup, a.steps)
        res[name] = {"ms": round(ms, 4), "GBps": round(tile_bytes / (ms * 1e-3) / 1e9, 1),
                     "frac": round(tile_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    res["decode_ms_over_probe_ms"] = round(decode_ms / res["table_order"]["ms"], 4)
    return res


def mixed_step(a, dev, up):
    import numpy as np
    import torch

    from paged_kv_cache_137_amd import ops
    from paged_kv_cache_137_amd import workloads as W
    from paged_kv_cache_137_amd.blocks import slot_mapping

    mx = W.mixed_config(poison=False)
    d, p = mx.decode, mx.prefill
    S, H, D = d.q.shape
    seq_p = np.repeat(np.arange(len(p.prompt_lens)), p.prompt_lens)
    pos_p = np.concatenate([np.arange(L) for L in p.prompt_lens])
    sm = np.concatenate([slot_mapping(p.block_tables, seq_p, pos_p),
                         slot_mapping(d.block_tables, np.arange(S), d.context_lens - 1)])
    k_all = up(np.concatenate([p.k, d.k_new]), "bf16")
    v_all = up(np.concatenate([p.v, d.v_new]), "bf16")
    kc, vc = up(d.k_cache, "bf16"), up(d.v_cache, "bf16")
    pq, pk, pv = up(p.q, "bf16"), up(p.k, "bf16"), up(p.v, "bf16")
    plens, ptab = up(p.prompt_lens), up(p.block_tables)
    q, bt, cl, smd = up(d.q, "bf16"), up(d.block_tables), up(d.context_lens), up(sm)
    pout = torch.empty(pq.shape, dtype=torch.bfloat16, device=dev)
    dout = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    mpl, mcl = int(p.prompt_lens.max()), d.max_context_len
    ws = torch.empty(max(1, ops.decode_workspace_bytes(S, H, D, mcl, ops.PARTITION_AUTO)), dtype=torch.uint8,
                     device=dev)

    def run(ev=None):
        if ev is not None:
            ev[0].record()
        ops.kv_cache_write(k_all, v_all, smd, kc, vc)
        if ev is not None:
            ev[1].record()
        ops.paged_attn_prefill(pq, pk, pv, ptab, plens, pout, max_prompt_len=mpl)
        if ev is not None:
            ev[2].record()
        ops.paged_attn_decode(q, kc, vc, bt, cl, d.scale, dout, max_context_len=mcl,
                              partition_size=ops.PARTITION_AUTO, workspace=ws)
        if ev is not None:
            ev[3].record()

    for _ in range(a.warmup):
        run()
    n = max(5, a.steps // 2)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / n
    w_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / n
    p_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / n
    d_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / n
    # The same step after about a second of back-to-back steps: the GPU's power
    # management settles within tens of milliseconds of sustained matrix work,
    # and the first launches of a burst land in its transient.
    with _ClockSampler() as clk:
        t_end = time.perf_counter() + 1.0
        while time.perf_counter() < t_end:
            for _ in range(5):
                run()
            torch.cuda.synchronize()
        evs2 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        for e in evs2:
            run(e)
        torch.cuda.synchronize()
    sus = {k: sum(e[i].elapsed_time(e[i + 1]) for e in evs2) / n for i, k in
           enumerate(("kv_cache_write", "paged_attn_prefill", "paged_attn_decode"))}
    # The same step with the prefill (matrix cores) on a second stream, running
    # beside the write and the decode (HBM); they share no buffer.  Both
    # streams keep the default priority.
    side = torch.cuda.Stream(device=dev)
    main = torch.cuda.current_stream(dev)

    def run_overlapped():
        side.wait_stream(main)
        with torch.cuda.stream(side):
            ops.paged_attn_prefill(pq, pk, pv, ptab, plens, pout, max_prompt_len=mpl)
        ops.kv_cache_write(k_all, v_all, smd, kc, vc)
        ops.paged_attn_decode(q, kc, vc, bt, cl, d.scale, dout, max_context_len=mcl,
                              partition_size=ops.PARTITION_AUTO, workspace=ws)
        main.wait_stream(side)

    for _ in range(a.warmup):
        run_overlapped()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        run_overlapped()
    torch.cuda.synchronize()
    ovl_ms = (time.perf_counter() - t0) * 1e3 / n
    T = int(k_all.shape[0])
    write_bytes = 2 * T * H * D * 2 * 2
    L = p.prompt_lens.astype(np.int64)
    flops = 4.0 * D * H * float((L * (L + 1) // 2).sum())
    dec_bytes = int(d.context_lens.sum()) * 2 * H * D * 2
    return {
        "workload": "8 prompts U[128,2048] prefilled into fresh shuffled blocks + 192 decodes lognormal(800,0.8), "
                    "32 heads x 128, bf16",
        "ms_per_step": round(wall_ms, 4),
        "ms_per_step_overlapped": round(ovl_ms, 4),
        "kernels_ms": {"kv_cache_write": round(w_ms, 5), "paged_attn_prefill": round(p_ms, 5),
                       "paged_attn_decode": round(d_ms, 5)},
        "write_GBps": round(write_bytes / (w_ms * 1e-3) / 1e9, 1),
        "prefill_tokens": int(L.sum()),
        "prefill_TFLOPs": round(flops / (p_ms * 1e-3) / 1e12, 1),
        "prefill_mfma_frac": round(flops / (p_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "decode_GBps": round(dec_bytes / (d_ms * 1e-3) / 1e9, 1),
        "decode_tokens_attended_per_s": round(float(d.context_lens.sum()) / (d_ms * 1e-3), 1),
        "after_1s_of_steps": {
            "kernels_ms": {k: round(v, 5) for k, v in sus.items()},
            "prefill_TFLOPs": round(flops / (sus["paged_attn_prefill"] * 1e-3) / 1e12, 1),
            "prefill_mfma_frac": round(flops / (sus["paged_attn_prefill"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "decode_GBps": round(dec_bytes / (sus["paged_attn_decode"] * 1e-3) / 1e9, 1),
            "sclk_MHz": clk.summary(),
        },
    }


def _time_events(fn, warmup, steps):
    import torch

    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def opt13b_decode(a, dev, up):
    """OPT-13B-shape decode step (fp16, 40 heads x 128, 64 sequences, context
    lengths U[1, 2048], shuffled blocks): plan + persistent decode + reduce,
    timed with HIP events."""
    import torch

    from paged_kv_cache_137_amd import ops
    from paged_kv_cache_137_amd import workloads as W

    d = W.decode_config(2, poison=False)
    S, H, D = d.q.shape
    t = dict(q=up(d.q), kc=up(d.k_cache), vc=up(d.v_cache), bt=up(d.block_tables), cl=up(d.context_lens))
    out = torch.empty((S, H, D), dtype=torch.float16, device=dev)
    ws = torch.empty(ops.decode_workspace_bytes(S, H, D, d.max_context_len, ops.PARTITION_AUTO), dtype=torch.uint8,
                     device=dev)
    ms = _time_events(lambda: ops.paged_attn_decode(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], d.scale, out,
                                                    max_context_len=d.max_context_len,
                                                    partition_size=ops.PARTITION_AUTO, workspace=ws),
                      a.warmup, a.steps)
    nbytes = int(d.context_lens.sum()) * 2 * H * D * 2
    return {"workload": "OPT-13B-shape decode step: 64 seqs, 40 heads x 128, fp16, ctx U[1, 2048], shuffled blocks, "
                        f"automatic partition ({ops.decode_partition(S, H, d.max_context_len)} tokens)",
            "sum_context_len": int(d.context_lens.sum()), "ms": round(ms, 4),
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def sharing_step(a, dev, up):
    """Block sharing (OPT-13B head shape, fp16): 128 prompts x 4 parallel samples.

    Each group's samples read the prompt's physical blocks; the partly filled
    last prompt block is copied on write (batched pkv_copy_blocks), then every
    sample decodes, once with the plain decode (every sample reads its whole
    context through its table) and once with the shared-prefix decode (blocks
    that a window's samples share are read once for all of them).  KV GB/s is
    reported against both the logical bytes (each sample's whole context) and
    the unique bytes (distinct slots read).
    """
    import numpy as np
    import torch

    from paged_kv_cache_137_amd import ops
    from paged_kv_cache_137_amd import workloads as W

    d = W.decode_config(4, poison=False)
    S, H, D = d.q.shape
    pairs = up(d.info["cow_pairs"].astype(np.int64))
    t = dict(q=up(d.q), kc=up(d.k_cache), vc=up(d.v_cache), bt=up(d.block_tables), cl=up(d.context_lens))
    out = torch.empty((S, H, D), dtype=torch.float16, device=dev)
    copy_ms = _time_events(lambda: ops.copy_blocks(t["kc"], t["vc"], pairs), a.warmup, a.steps)
    # The one-call decode (paged_attn_decode) finds the shared prompt blocks on
    # the device and reads them once per group; automatic partition (no split).
    ws = torch.empty(ops.decode_workspace_bytes(S, H, D, d.max_context_len, ops.PARTITION_AUTO),
                     dtype=torch.uint8, device=dev)
    dec_ms = _time_events(lambda: ops.paged_attn_decode(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], d.scale, out,
                                                        max_context_len=d.max_context_len,
                                                        partition_size=ops.PARTITION_AUTO, workspace=ws),
                          a.warmup, a.steps)
    # For contrast, the two-stage form, which reads every sample's blocks
    # through its own table, at 512-token partitions (its fastest size here).
    ws2 = torch.empty(ops.decode_workspace_bytes(S, H, D, d.max_context_len, 512), dtype=torch.uint8, device=dev)

    def two_stage():
        kw = dict(max_context_len=d.max_context_len, partition_size=512, workspace=ws2)
        ops.paged_attn_decode_partial(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], d.scale, out, **kw)
        ops.paged_attn_decode_reduce(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], d.scale, out, **kw)

    two_ms = _time_events(two_stage, a.warmup, a.steps)
    used = np.zeros((d.num_blocks, 16), dtype=bool)
    for s_ in range(S):
        n = int(d.context_lens[s_])
        nfull, rem = divmod(n, 16)
        used[d.block_tables[s_, :nfull]] = True
        if rem:
            used[d.block_tables[s_, nfull], :rem] = True
    per_tok = 2 * H * D * 2
    logical = int(d.context_lens.sum()) * per_tok
    unique = int(used.sum()) * per_tok
    npairs = int(pairs.shape[0])
    copy_bytes = npairs * H * 16 * D * 2 * 2 * 2
    return {
        "workload": "OPT-13B head shape (40 x 128), fp16, 128 prompts U[64,1024] x 4 samples, own tokens U[1,256]",
        "copy_blocks_pairs": npairs,
        "copy_blocks_ms": round(copy_ms, 5),
        "copy_blocks_GBps": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
        "paged_attn_decode_ms": round(dec_ms, 4),
        "paged_attn_decode_logical_GBps": round(logical / (dec_ms * 1e-3) / 1e9, 1),
        "paged_attn_decode_unique_GBps": round(unique / (dec_ms * 1e-3) / 1e9, 1),
        "paged_attn_decode_unique_frac": round(unique / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "two_stage_ms": round(two_ms, 4),
        "two_stage_logical_GBps": round(logical / (two_ms * 1e-3) / 1e9, 1),
        "two_stage_unique_GBps": round(unique / (two_ms * 1e-3) / 1e9, 1),
        "physical_blocks": d.info["physical_blocks_used"],
        "logical_blocks": d.info["logical_blocks"],
    }


def cached_prefix_prefill(a, dev, up):
    """16 requests share a cached 1024-token prefix; each prefills 256 new tokens (32 x 128, bf16)."""
    import numpy as np
    import torch

    from paged_kv_cache_137_amd import ops
    from paged_kv_cache_137_amd import workloads as W
    from paged_kv_cache_137_amd.blocks import BlockManager

    H, D, B, R, C, L = 32, 128, 16, 16, 1024, 256
    nb = C // B + R * (L // B) + 8
    m = BlockManager(nb, B, free_order=np.random.default_rng(5).permutation(nb))
    m.add_sequence(-1, C)
    for r in range(R):
        m.fork(-1, r)
        for _ in range(L):
            m.append_token(r)
    tables = up(m.block_tables(range(R), pad=0))
    kc = up(W.normal((91, 1), (nb, H, B, D), "bf16"), "bf16")
    vc = up(W.normal((91, 2), (nb, H, B, D), "bf16"), "bf16")
    q = up(W.normal((91, 3), (R * L, H, D), "bf16"), "bf16")
    out = torch.empty((R * L, H, D), dtype=torch.bfloat16, device=dev)
    pre = up(np.full(R, C, np.int32))
    lens = up(np.full(R, L, np.int32))
    ms = _time_events(lambda: ops.paged_attn_prefill_cached(q, kc, vc, tables, pre, lens, out, max_prompt_len=L,
                                                            max_prefix_len=C), a.warmup, a.steps)
    flops = 4.0 * D * H * R * sum(C + i + 1 for i in range(L))
    return {
        "workload": "16 requests x 256 new tokens over one cached 1024-token prefix, 32 heads x 128, bf16",
        "ms": round(ms, 4),
        "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
        "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
    }


class _ClockSampler:
    """Samples the GPU's shader clock (rocm-smi --showclocks, a child process)
    about ten times a second while the with-block runs; None when rocm-smi is
    not there or prints no clock."""

    def __init__(self):
        self.samples, self._stop, self._th = [], False, None

    def _run(self):
        import subprocess

        while not self._stop:
            try:
                r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=5)
                card = json.loads(r.stdout[r.stdout.index("{"):])
                for v in card.values():
                    self.samples.append(int(str(v["sclk clock speed:"]).strip("()Mhz")))
                    break
            except Exception:
                return
            time.sleep(0.05)

    def __enter__(self):
        import threading

        self._th = threading.Thread(target=self._run, daemon=True)
        self._th.start()
        return self

    def __exit__(self, *exc):
        self._stop = True
        self._th.join(timeout=10)
        return False

    def summary(self):
        xs = self.samples
        if not xs:
            return None
        return {"min": min(xs), "mean": round(sum(xs) / len(xs)), "max": max(xs), "samples": len(xs)}


def prefill_prompt_count(a, dev, up):
    """The fresh prefill alone (HIP events, inputs resident and warm): the mixed
    step's 8 prompts, and 256 prompts drawn from the same length distribution
    (U[128, 2048]), which take the enumeration for more than 64 prompts.  Both
    32 heads x 128, bf16.  q/k/v of the 256-prompt batch are drawn on the device
    (seeded); only the timing is used."""
    import numpy as np
    import torch

    from paged_kv_cache_137_amd import ops
    from paged_kv_cache_137_amd import workloads as W

    H, D = 32, 128
    res = {"workload": "fresh causal prefill alone, 32 heads x 128, bf16: the mixed step's 8 prompts, and 256 prompts "
                       "with lengths U[128, 2048]"}
    p5 = W.mixed_config(poison=False).prefill
    g = torch.Generator(device=dev)
    g.manual_seed(137256)
    cases = (("8_prompts", p5.prompt_lens.astype(np.int64), True),
             ("256_prompts", np.random.default_rng(137256).integers(128, 2049, size=256).astype(np.int64), False))
    for name, L, from_workload in cases:
        T = int(L.sum())
        if from_workload:
            q, k, v = up(p5.q, "bf16"), up(p5.k, "bf16"), up(p5.v, "bf16")
        else:
            q, k, v = (torch.randn((T, H, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
                       for _ in range(3))
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
        lens = up(L.astype(np.int32))
        steps = a.steps if T < 20000 else max(3, a.steps // 10)
        def call():
            ops.paged_attn_prefill(q, k, v, None, lens, out, max_prompt_len=int(L.max()))

        ms = _time_events(call, max(1, a.warmup // 2), steps)
        flops = 4.0 * D * H * float((L * (L + 1) // 2).sum())
        res[name] = {"tokens": T, "ms": round(ms, 4), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                     "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        if from_workload:
            # The same launch back to back for about a second, with the shader
            # clock sampled meanwhile: the matrix work runs at the clock the
            # power management grants, below the 2.4 GHz the peak assumes.
            with _ClockSampler() as clk:
                t_end = time.perf_counter() + 1.0
                n_sus, e0, e1 = 0, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                while time.perf_counter() < t_end:
                    for _ in range(20):
                        call()
                    n_sus += 20
                    torch.cuda.synchronize()
                e1.record()
                torch.cuda.synchronize()
            sus_ms = e0.elapsed_time(e1) / n_sus
            res[name]["sustained_1s"] = {"launches": n_sus, "ms": round(sus_ms, 4),
                                         "TFLOPs": round(flops / (sus_ms * 1e-3) / 1e12, 1),
                                         "sclk_MHz": clk.summary()}
        del q, k, v, out
    res["tflops_256_over_8"] = round(res["256_prompts"]["TFLOPs"] / res["8_prompts"]["TFLOPs"], 4)
    return res


def decode_launch_shape(a, t, d, dargs, dkw):
    """The headline decode (paged_attn_decode) with 1, 2 and 4 workgroups per CU
    (the library's default is 1; PKV_DECODE_WG_PER_CU overrides it), timed with
    HIP events."""
    from paged_kv_cache_137_amd import ops

    kv_bytes = int(d.context_lens.sum()) * 2 * d.num_heads * d.head_dim * 2
    old = os.environ.get("PKV_DECODE_WG_PER_CU")
    res = {}
    try:
        for n in (1, 2, 4):
            os.environ["PKV_DECODE_WG_PER_CU"] = str(n)

            ms = _time_events(lambda: ops.paged_attn_decode(*dargs, **dkw), a.warmup, a.steps)
            res[str(n)] = {"ms": round(ms, 4), "GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 1)}
    finally:
        if old is None:
            os.environ.pop("PKV_DECODE_WG_PER_CU", None)
        else:
            os.environ["PKV_DECODE_WG_PER_CU"] = old
    return {"workgroups_per_cu": res}


def hbm_reference(t):
    """Plain PyTorch passes over the same K pool on the same GPU, for context
    (not a ceiling: the decode's gathered reads outrun both; read_probe is the
    ceiling of its access pattern): a contiguous sum (read only, fp32
    accumulation) and a device-to-device copy (read + write).  Timed with HIP
    events, 20 passes each after 3 warm-up passes."""
    import torch
    kc = t["kc"]
    nbytes = kc.numel() * kc.element_size()
    dst = torch.empty_like(kc)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 20

    ms_sum = timed(lambda: kc.sum(dtype=torch.float32))
    ms_copy = timed(lambda: dst.copy_(kc))
    del dst
    return {"bytes": nbytes,
            "torch_sum_ms": round(ms_sum, 4), "torch_sum_read_GBps": round(nbytes / ms_sum / 1e6, 1),
            "torch_copy_ms": round(ms_copy, 4), "torch_copy_read_plus_write_GBps": round(2 * nbytes / ms_copy / 1e6, 1)}


def block_size_sweep(a, t, d):
    """Decode of the headline batch at block sizes 8, 16 and 32.

    The resident pool's bytes are re-tiled as [blocks][heads][B][dim] for each
    B and every sequence gets freshly shuffled physical blocks, so the bytes
    attended are the same and only the block granularity changes.
    """
    import numpy as np
    import torch

    from paged_kv_cache_137_amd import ops

    S, H, D = d.q.shape
    ctx = d.context_lens.astype(np.int64)
    kv_bytes = int(ctx.sum()) * 2 * H * D * 2
    out = torch.empty((S, H, D), dtype=torch.bfloat16, device=t["q"].device)
    res = {}
    for B in (8, 16, 32):
        nb = t["kc"].numel() // (H * B * D)
        need = -(-ctx // B)
        total = int(need.sum())
        if total + 1 > nb:
            res[str(B)] = None
            continue
        perm = np.random.default_rng(1000 + B).permutation(nb).astype(np.int32)
        tables = np.full((S, int(need.max())), perm[total], dtype=np.int32)
        offs = np.concatenate([[0], np.cumsum(need)])
        for s_ in range(S):
            tables[s_, : need[s_]] = perm[offs[s_]: offs[s_ + 1]]
        kc = t["kc"].view(-1)[: nb * H * B * D].view(nb, H, B, D)
        vc = t["vc"].view(-1)[: nb * H * B * D].view(nb, H, B, D)
        bt = torch.from_numpy(tables).to(t["q"].device)
        ws = torch.empty(ops.decode_workspace_bytes(S, H, D, d.max_context_len, a.partition), dtype=torch.uint8,
                         device=t["q"].device)
        ms = _time_events(lambda: ops.paged_attn_decode(t["q"], kc, vc, bt, t["cl"], d.scale, out,
                                                        max_context_len=d.max_context_len,
                                                        partition_size=a.partition, workspace=ws),
                          a.warmup, a.steps)
        res[str(B)] = {"decode_ms": round(ms, 4), "GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
                       "frac": round(kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return {"workload": "headline decode batch (partial + reduce), block sizes 8/16/32", "by_block_size": res}


def swap_step(a, t, n_blocks: int = 2048):
    """Swap-out and swap-in of n_blocks scattered 16-token blocks (keys and values)
    between the device pool and a pinned host pool, beside a contiguous copy of
    the same byte count (torch copy_, one DMA transfer) in each direction."""
    import numpy as np
    import torch

    from paged_kv_cache_137_amd import ops

    kc, vc = t["kc"], t["vc"]
    nb = kc.shape[0]
    dev = kc.device
    ids = np.random.default_rng(7).permutation(nb)[:n_blocks].astype(np.int64)
    hk = torch.empty((n_blocks,) + tuple(kc.shape[1:]), dtype=kc.dtype, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    out_pairs = torch.from_numpy(np.stack([ids, np.arange(n_blocks)], axis=1)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(n_blocks), ids], axis=1)).to(dev)
    nbytes = 2 * hk.numel() * hk.element_size()
    steps, warm = max(3, a.steps // 10), 2
    out_ms = _time_events(lambda: ops.swap_blocks(kc, vc, hk, hv, out_pairs), warm, steps)
    in_ms = _time_events(lambda: ops.swap_blocks(hk, hv, kc, vc, in_pairs, device=dev), warm, steps)
    dk = torch.empty((2,) + tuple(hk.shape), dtype=kc.dtype, device=dev)
    hd = torch.empty(tuple(dk.shape), dtype=kc.dtype, pin_memory=True)
    d2h_ms = _time_events(lambda: hd.copy_(dk, non_blocking=True), warm, steps)
    h2d_ms = _time_events(lambda: dk.copy_(hd, non_blocking=True), warm, steps)
    gbps = lambda ms: round(nbytes / (ms * 1e-3) / 1e9, 1)  # noqa: E731
    return {
        "workload": f"{n_blocks} scattered blocks x (keys + values), 32 heads x 16 x 128 bf16 "
                    f"({nbytes / 2**20:.0f} MiB per direction)",
        "swap_out_ms": round(out_ms, 3), "swap_out_GBps": gbps(out_ms),
        "swap_in_ms": round(in_ms, 3), "swap_in_GBps": gbps(in_ms),
        "contiguous_d2h_GBps": gbps(d2h_ms), "contiguous_h2d_GBps": gbps(h2d_ms),
    }


def _cpu_model() -> str:
    """The host CPU as /proc/cpuinfo describes it: model name, family / model /
    stepping, clock and cache (a virtual machine may report a generic name)."""
    info = {}
    try:
        for ln in open("/proc/cpuinfo"):
            if ":" in ln:
                k, v = ln.split(":", 1)
                info.setdefault(k.strip(), v.strip())
            elif info:
                break  # the first processor's block is enough
    except OSError:
        return "unknown"
    parts = [info.get("model name", "unknown")]
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    if ids:
        parts.append("(" + ", ".join(ids) + ")")
    if "cpu MHz" in info:
        parts.append(f"{float(info['cpu MHz']):.0f} MHz")
    if "cache size" in info:
        parts.append(f"cache {info['cache size']}")
    return " ".join(parts)


# The all-core CPU runs use a process pool forked before this process touches
# the GPU; the workers read these inputs (inherited through fork) and do only
# NumPy work, one BLAS thread each.
_CPU_DECODE = None
_CPU_PREFILL = None


def _cpu_worker_init():
    import threadpoolctl

    global _CPU_LIMIT
    _CPU_LIMIT = threadpoolctl.threadpool_limits(1)


def _cpu_decode_seq(s_):
    import oracle

    d = _CPU_DECODE
    oracle.attention.paged_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, d.scale, d.dtype,
                                  seqs=[s_])
    return int(d.context_lens[s_])


def _prefill_units(p, heads_per_unit=4):
    return [(i, h0) for i in range(len(p.prompt_lens)) for h0 in range(0, p.num_heads, heads_per_unit)]


def _cpu_prefill_unit(unit, p=None):
    """The oracle's causal prefill of one prompt for 4 of its heads; returns the
    unit's causal FLOPs (4 * D * heads * L(L+1)/2)."""
    import numpy as np

    import oracle

    p = _CPU_PREFILL if p is None else p
    i, h0 = unit
    hs = slice(h0, min(h0 + 4, p.num_heads))
    off = int(p.prompt_lens[:i].sum())
    L = int(p.prompt_lens[i])
    sub = [np.ascontiguousarray(x[off:off + L, hs]) for x in (p.q, p.k, p.v)]
    oracle.attention.causal_prefill(*sub, [L], 1.0 / np.sqrt(p.head_dim), p.dtype)
    return 4.0 * p.head_dim * sub[0].shape[1] * L * (L + 1) / 2


def cpu_baseline(d, p, seconds: float, max_workers: int = 16):
    """The float64 oracle, as it stands, on the host cores: one thread, then every
    core of this process's CPU share (at most max_workers; the box gives one GPU
    a share of 16).

    Decode: whole sequences of the headline step (the oracle's paged_decode on
    one sequence), in order, wrapping round.  Prefill: the mixed step's 8 prompts in
    units of (prompt, 4 heads), the oracle's causal_prefill on each.  Each leg
    runs about seconds / 4.  The one-thread legs are time-boxed; the all-core
    legs map a fixed list of units, sized from the one-thread rate, over a
    process pool (one BLAS thread per process).  Must run before this process
    initialises the GPU (the pool is forked)."""
    import multiprocessing as mp

    import threadpoolctl

    global _CPU_DECODE, _CPU_PREFILL
    _CPU_DECODE, _CPU_PREFILL = d, p
    H, D = d.num_heads, d.head_dim
    per_tok = 2 * H * D * 2
    leg = seconds / 4
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(affinity, max_workers))

    with threadpoolctl.threadpool_limits(1):
        done, tokens = 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < leg:
            tokens += _cpu_decode_seq(done % d.num_seqs)
            done += 1
        dec1 = (done, tokens, time.perf_counter() - t0)
        units = _prefill_units(p)
        n1, fl1 = 0, 0.0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < leg:
            fl1 += _cpu_prefill_unit(units[(n1 * 7) % len(units)])
            n1 += 1
        pre1 = (n1, fl1, time.perf_counter() - t0)

    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_cpu_worker_init) as pool:
        nd = max(cores, min(64 * d.num_seqs, int(dec1[0] / dec1[2] * cores * leg)))
        t0 = time.perf_counter()
        tok_all = sum(pool.map(_cpu_decode_seq, [i % d.num_seqs for i in range(nd)], chunksize=1))
        dec_all = time.perf_counter() - t0
        npf = max(cores, min(64 * len(units), int(pre1[0] / pre1[2] * cores * leg)))
        t0 = time.perf_counter()
        fl_all = sum(pool.map(_cpu_prefill_unit, [units[(i * 7) % len(units)] for i in range(npf)], chunksize=1))
        pre_all = time.perf_counter() - t0
    _CPU_DECODE = _CPU_PREFILL = None

    return {
        "value": round(tok_all * per_tok / dec_all / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{nd} whole-sequence decodes of the headline step's {d.num_seqs} sequences, in order and "
                  f"wrapping round ({tok_all} tokens, {dec_all:.1f} s), float64 NumPy, over {cores} processes "
                  f"with one BLAS thread each",
        "tokens_attended_per_s": round(tok_all / dec_all, 1),
        "host_cores_in_affinity": affinity,
        "cpu_model": _cpu_model(),
        "one_thread": {
            "value": round(dec1[1] * per_tok / dec1[2] / 1e9, 4), "unit": "GB/s", "cores": 1,
            "tokens_attended_per_s": round(dec1[1] / dec1[2], 1),
            "sample": f"{dec1[0]} whole-sequence decodes ({dec1[1]} tokens, {dec1[2]:.1f} s), BLAS limited to 1 thread",
        },
        "prefill": {
            "workload": "the mixed step's 8 prompts (32 heads x 128, bf16 inputs), causal, float64 oracle, in units of "
                        "(prompt, 4 heads)",
            "all_cores_GFLOPs": round(fl_all / pre_all / 1e9, 3), "all_cores_units": npf,
            "all_cores_seconds": round(pre_all, 2), "cores": cores,
            "one_thread_GFLOPs": round(pre1[1] / pre1[2] / 1e9, 3), "one_thread_units": pre1[0],
            "one_thread_seconds": round(pre1[2], 2),
            "flops_counted": "causal algorithmic FLOPs, 4 x head_dim x heads x L(L+1)/2 per unit",
        },
    }


if __name__ == "__main__":
    sys.exit(main())
