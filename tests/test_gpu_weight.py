"""The device's fixed-point softmax weight (the builder's q = W / Z and the
acceptance walk's p, q and residual all come from it) against the oracle's
tvo_weight, bit for bit, on every fp32 logit x in [-33, 0] of a row whose
maximum is 0, at temperatures 1, 0.7 and 1.6 (inverse temperature rounded to
fp32 as the library does), and in the inv_t == 1 form of the row passes.
Below -33 both clamp to weight 0 (pinned on the CPU side of the oracle)."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_best_amd as tv

pytestmark = pytest.mark.gpu

NEG_ZERO = 0x80000000
NEG_33 = 0xC2040000           # bit pattern of -33.0: negative floats grow with their bits
CHUNK = 1 << 26


def _inv_t(T):
    return float(np.float32(1.0) / np.float32(T))


def _spans():
    yield 0, 1                                  # +0.0
    first = NEG_ZERO
    while first <= NEG_33:
        n = min(CHUNK, NEG_33 - first + 1)
        yield first, n
        first += n


@pytest.mark.parametrize("T,unit", [(1.0, 1), (1.0, 0), (0.7, 0), (1.6, 0)],
                         ids=["T1-unit", "T1", "T0.7", "T1.6"])
def test_weight_every_logit_in_range(T, unit):
    import os
    prev = oracle.set_threads(min(16, len(os.sched_getaffinity(0))))
    L = tv.lib()
    inv_t = _inv_t(T)
    buf = torch.empty(CHUNK, dtype=torch.int64, device="cuda")
    checked = 0
    try:
        for first, n in _spans():
            st = L.tv_debug_weights(first, n, 0.0, inv_t, unit, buf.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
            assert st == tv.TV_OK
            got = buf[:n].cpu().numpy().view(np.uint64)
            want = oracle.weight_range(first, n, 0.0, inv_t)
            if not np.array_equal(got, want):
                bad = np.flatnonzero(got != want)[:5]
                xs = (np.arange(n, dtype=np.uint64)[bad] + first).astype(np.uint32).view(np.float32)
                raise AssertionError(f"T={T} unit={unit}: x={xs.tolist()} gpu={got[bad].tolist()} "
                                     f"oracle={want[bad].tolist()}")
            checked += n
    finally:
        oracle.set_threads(prev)
    assert checked == (NEG_33 - NEG_ZERO + 1) + 1
