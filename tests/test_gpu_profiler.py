"""The per-kernel event timer counts every launch when several host threads
launch at once.

The timer is process-wide host state behind a mutex; an event pair joins its
records only once both events are recorded. Two threads, each on its own
stream, issue permutes through the C ABI (ctypes releases the GIL for the
call, so the library is entered concurrently); every launch must be counted
once, with a positive time, and the permuted rows must be what a single
thread produces.
"""
import threading

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

N_CALLS = 200


def test_profiler_counts_launches_from_two_threads():
    import torch
    import token_dispatch_grouped_amd as m
    from token_dispatch_grouped_amd import _lib

    T, d, E, k = 1000, 256, 8, 2
    print(f"[profiler] two threads x {N_CALLS} permutes, T={T} d={d} k={k}", flush=True)
    shape = _lib.make_shape(T, d, E, k, 64, m.MOE_DTYPE_BF16)
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.integers(0, 1 << 16, size=(T, d), dtype=np.uint16).view(np.int16)).cuda()
    perm = torch.from_numpy(rng.permutation(T * k).astype(np.int32).reshape(T, k)).cuda()
    outs = [torch.zeros(T * k, d, dtype=torch.int16, device="cuda") for _ in range(2)]
    ref = torch.zeros_like(outs[0])
    _lib.moe_permute(shape, x, perm, ref)
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def worker(i):
        try:
            h = streams[i].cuda_stream
            for _ in range(N_CALLS):
                _lib.moe_permute(shape, x, perm, outs[i], stream=h)
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    _lib.moe_profiler_reset()
    _lib.moe_profiler_enable(True)
    try:
        threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        rec = _lib.moe_profiler_read_all()
    finally:
        _lib.moe_profiler_enable(False)
        _lib.moe_profiler_reset()
    assert not errors, errors
    assert "permute" in rec, rec
    launches, ms = rec["permute"]
    assert launches == 2 * N_CALLS, rec
    assert ms > 0.0
    for o in outs:
        assert torch.equal(o, ref)
