"""Independent oracle chains spread over the host's cores.

TEST INFRASTRUCTURE ONLY (like the rest of this package): the test suite and the benchmark's
CPU-baseline leg use it to run many (sequence, value head) chains of the fp64 oracle at once. It adds
no arithmetic: each worker calls ``gdn_chain`` on the arguments ``chain_inputs`` cut out in the parent,
so a job carries only its own chain's slices. Workers are started with ``spawn`` (nothing is inherited
from a parent that may hold a GPU context) and run their linear algebra on one thread each.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import sys
from concurrent.futures import ProcessPoolExecutor

from . import gdn_oracle as O

_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "NUMEXPR_NUM_THREADS")


MAX_WORKERS = 16  # a one-GPU host's CPU share, whatever the affinity mask shows


def host_cores() -> int:
    """Cores this process may run on."""
    return len(os.sched_getaffinity(0))


def default_workers() -> int:
    return max(1, min(MAX_WORKERS, host_cores()))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _spawn_possible() -> bool:
    """A spawned worker re-imports the parent's main module; that needs a main module that exists as a
    file or an importable module (not ``python -c`` or a script read from stdin)."""
    m = sys.modules.get("__main__")
    f = getattr(m, "__file__", None)
    return getattr(m, "__spec__", None) is not None or (f is not None and os.path.isfile(f))


def _run(job):
    args, kw = job
    return O.gdn_chain(**args, **kw)


def run_chains(inp, chains, *, workers=None, timeout=3600.0, **kw):
    """Runs ``prefill_chain(inp, n, h, **kw)`` for every (n, h) in ``chains`` over a process pool and
    returns the results in order (``state_in``/``conv_in`` in ``kw`` override those of ``inp``). Runs in
    this process when one worker suffices or workers cannot be spawned; raises TimeoutError after
    ``timeout`` seconds."""
    chains = list(chains)
    st, ci = kw.pop("state_in", None), kw.pop("conv_in", None)
    # chain_inputs upcasts only each chain's slices, so long inputs are never copied whole to fp64
    jobs = [(O.chain_inputs(inp, n, h, state_in=st, conv_in=ci), kw) for n, h in chains]
    workers = min(workers or default_workers(), max(1, len(jobs)))
    if workers <= 1 or not _spawn_possible():
        return [_run(j) for j in jobs]
    saved = {v: os.environ.get(v) for v in _THREAD_VARS}
    for v in _THREAD_VARS:
        os.environ[v] = "1"
    try:
        with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
            return list(ex.map(_run, jobs, chunksize=max(1, len(jobs) // (4 * workers)), timeout=timeout))
    finally:
        for v, val in saved.items():
            if val is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = val
