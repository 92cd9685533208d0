"""The oracle's bf16 round-to-nearest-even over every one of the 2^32 fp32
bit patterns: equal to torch's CPU fp32 -> bf16 cast for every non-NaN input
(a library routine for the same definition), and for every NaN input a quiet
NaN with the input's sign (the reading for NaN; torch canonicalises NaN
payloads, so only NaN-ness is compared there).  Split over the host's cores."""
import ctypes
import multiprocessing as mp
import os

import numpy as np

CHUNK = 1 << 24
N_CHUNKS = (1 << 32) // CHUNK


def _check_range(first: int, last: int):
    import torch
    import oracle
    torch.set_num_threads(1)
    o = oracle.get()
    base = np.arange(CHUNK, dtype=np.uint32)
    u = np.empty(CHUNK, np.uint32)
    ours = np.empty(CHUNK, np.uint16)
    tb = torch.empty(CHUNK, dtype=torch.bfloat16)
    bad = bad_nan = 0
    for c in range(first, last):
        np.add(base, np.uint32(c * CHUNK), out=u)
        f = u.view(np.float32)
        o.lib.z1o_bf16_rne_array(CHUNK, f.ctypes.data_as(ctypes.c_void_p),
                                 ours.ctypes.data_as(ctypes.c_void_p))
        tb.copy_(torch.from_numpy(f))
        ref = tb.view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        bad += int(np.count_nonzero((ours != ref) & ~nan))
        if nan.any():
            h = ours[nan]
            sign_in = (u[nan] >> 31).astype(np.uint16)
            quiet_nan = ((h & 0x7FC0) == 0x7FC0) & ((h >> 15) == sign_in)
            bad_nan += int(np.count_nonzero(~quiet_nan))
    return bad, bad_nan


def test_bf16_rne_exhaustive_vs_torch():
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    step = -(-N_CHUNKS // workers)
    ranges = [(a, min(a + step, N_CHUNKS)) for a in range(0, N_CHUNKS, step)]
    with mp.get_context("spawn").Pool(len(ranges)) as pool:
        res = pool.starmap(_check_range, ranges)
    bad = sum(r[0] for r in res)
    bad_nan = sum(r[1] for r in res)
    assert bad == 0, f"{bad} non-NaN fp32 patterns round differently from torch"
    assert bad_nan == 0, f"{bad_nan} NaN patterns do not give a quiet NaN of the same sign"
