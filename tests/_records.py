"""Parity records of the GPU tests: one JSON line per (config, kernel).

Each record holds the largest |GPU - oracle| difference, the tolerance it was
held to, how many outputs were compared, the bit-exact checks that passed, how
long the float64 oracle took and on what host.  Records are appended to the file
named by the environment variable PKV_PARITY_RECORDS; nothing is written when
it is unset.
"""

from __future__ import annotations

import json
import os
import platform


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
        return platform.processor() or "unknown"
    parts = [info.get("model name", platform.processor() or "unknown")]
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    if ids:
        parts.append("(" + ", ".join(ids) + ")")
    if "cpu MHz" in info:
        parts.append(f"{float(info['cpu MHz']):.0f} MHz")
    if "cache size" in info:
        parts.append(f"cache {info['cache size']}")
    return " ".join(parts)


def host_info() -> dict:
    try:
        import threadpoolctl

        blas = max((p.get("num_threads", 0) for p in threadpoolctl.threadpool_info()), default=0)
    except Exception:  # pragma: no cover
        blas = None
    return {"host_cores": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(), "blas_threads": blas}


def record(config: str, kernel: str, **fields) -> None:
    path = os.environ.get("PKV_PARITY_RECORDS")
    if not path:
        return
    rec = {"config": config, "kernel": kernel, **fields, **host_info()}
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")
