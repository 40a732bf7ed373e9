"""Run the fp64 oracle on sampled query rows, one query head per worker
process (spawned, so no GPU or BLAS state is inherited).  The arithmetic is
the oracle's own ``attention_rows``; this only distributes heads."""

import multiprocessing as mp
import os
import tempfile

import numpy as np

_NAMES = ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")


def _worker(args):
    d, h, scale, rows = args
    import oracle
    x = {n: np.load(os.path.join(d, n + ".npy"), mmap_mode="r") for n in _NAMES}
    cu = [np.load(os.path.join(d, n + ".npy")) for n in ("cu_q", "cu_prefix", "cu_suffix_real")]
    rph = np.zeros((x["q"].shape[1], rows.size), dtype=np.int64)
    rph[h] = rows
    out, lse = oracle.attention_rows(x["q"], x["k_prefix"], x["v_prefix"], x["k_suffix"],
                                     x["v_suffix"], *cu, scale, rph, heads=[h])
    return h, out[0], lse[0]


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_rows_parallel(x, rows_per_head, workers=None):
    """out [Hq, n, D] and lse [Hq, n] (float64) for rows_per_head [Hq, n]."""
    workers = workers or default_workers()
    hq = x["q"].shape[1]
    n = rows_per_head.shape[1]
    d = x["q"].shape[2]
    out = np.zeros((hq, n, d))
    lse = np.zeros((hq, n))
    env_old = {k: os.environ.get(k) for k in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS")}
    os.environ["OPENBLAS_NUM_THREADS"] = "1"
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        with tempfile.TemporaryDirectory(prefix="jpa_oracle_") as tmp:
            for name in _NAMES + ("cu_q", "cu_prefix", "cu_suffix_real"):
                np.save(os.path.join(tmp, name + ".npy"), np.asarray(x[name]))
            tasks = [(tmp, h, float(x["scale"]), np.asarray(rows_per_head[h])) for h in range(hq)]
            ctx = mp.get_context("spawn")
            with ctx.Pool(workers) as pool:
                for h, o, l in pool.imap_unordered(_worker, tasks):
                    out[h] = o
                    lse[h] = l
    finally:
        for k, v in env_old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return out, lse
