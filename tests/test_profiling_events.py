"""verify_attn_set_profiling_events: three events per run, two (the caller ends a run with the
next run's `before`), or none; any other combination is rejected. Timing with events must not
change the outputs."""
import ctypes

import numpy as np
import pytest

import workloads as wl
from mla_tree_verify_paged_amd import binding as B
from tests.conftest import gpu_available
from tests.gpu_helpers import run_gpu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


class _Events:
    """hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        import torch  # noqa: F401  (loads the runtime)
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value

    def record(self, e):
        assert self.rt.hipEventRecord(e, None) == 0

    def destroy(self, e):
        self.rt.hipEventDestroy(e)


def test_event_combinations_and_two_event_timing():
    import torch
    from mla_tree_verify_paged_amd import VerifyAttn
    w = wl.build_workload("ev", np.random.default_rng(30), 64, [300], [4], 1024)
    va = VerifyAttn(w.num_heads, max_batch=1, max_q_per_req=w.max_q_per_req,
                    max_q_tokens=w.num_tokens)
    base = run_gpu(w, va=va)
    ev = _Events()
    e = [ev.create() for _ in range(5)]
    try:
        for bad in [(e[0], None, None), (None, e[1], None), (e[0], None, e[2]),
                    (None, e[1], e[2]), (None, None, e[2])]:
            with pytest.raises(B.VerifyAttnError) as err:
                B.verify_attn_set_profiling_events(va.ctx, *bad)
            assert err.value.status == B.VA_ERR_INVALID
        # two events per run: edge, mid; the next run's edge ends this one
        B.verify_attn_set_profiling_events(va.ctx, e[0], e[1], None)
        first = run_gpu(w, va=va)
        B.verify_attn_set_profiling_events(va.ctx, e[2], e[3], None)
        run_gpu(w, va=va)
        ev.record(e[4])
        B.verify_attn_set_profiling_events(va.ctx, None, None, None)
        torch.cuda.synchronize()
        part, comb = ev.elapsed_ms(e[0], e[1]), ev.elapsed_ms(e[1], e[2])
        part2, comb2 = ev.elapsed_ms(e[2], e[3]), ev.elapsed_ms(e[3], e[4])
        assert part > 0 and comb > 0 and part2 > 0 and comb2 > 0
        # the same outputs with and without events
        for x, y in zip(base[:3], first[:3]):
            assert np.array_equal(x, y)
    finally:
        B.verify_attn_set_profiling_events(va.ctx, None, None, None)
        for x in e:
            ev.destroy(x)
