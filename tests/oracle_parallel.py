"""Test helper: the oracle's accept sampler over many independent rows, split
across worker processes. Rows do not interact in the sampler, so the result is
the oracle's own result on the whole array."""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def _accept_chunk(args):
    import oracle
    tl, dl, d, ua, us, T, hz = args
    return oracle.spec_accept(tl, dl, d, ua, us, T, horizons=hz)


def spec_accept_rows(tl, dl, d, ua, us, T=1.0, horizons=None, workers=None):
    n = tl.shape[0]
    workers = workers or max(1, min(8, len(os.sched_getaffinity(0))))
    chunks = [c for c in np.array_split(np.arange(n), workers * 4) if len(c)]
    jobs = [(tl[c], dl[c], d[c], ua[c], us[c], T, None if horizons is None else horizons[c]) for c in chunks]
    with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_accept_chunk, jobs))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])
