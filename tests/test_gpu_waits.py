"""The role-split prefill's slot waits are bounded; a wait that gives up must
never pass for a valid result.

The host forces give-ups with a tiny spin limit (the KDA_WAIT_SPIN_LIMIT
testing knob, read by the library at each launch), so every kernel still runs
to its normal end: waves that give up only read or write an LDS slot early.
Every 16-column group of S_T (one chain wave's columns) must then be either
all NaN (a give-up that may have touched its data) or the oracle's result
within the bf16 tolerance.  Afterwards, with the default limit, the same call
is exact again (no state survives the call).
"""
import os

import numpy as np
import pytest
import torch

from linear_recurrent_attention_chunkwise_amd.inputs import WORKLOADS, make_prefill_inputs
from tests.gpu_helpers import gpu_prefill, host, oracle_prefill, slice_relerr, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import linear_recurrent_attention_chunkwise_amd as m
    assert m.abi_version() == 8
    return m


def test_forced_wait_give_up_poisons_state(kda, gpu_device):
    w = WORKLOADS["k3_prefill_bf16"].with_(H=8)
    inp = make_prefill_inputs(w, T=2048)
    g = to_dev(inp, gpu_device)
    o_ref, S_ref = oracle_prefill(inp)
    os.environ["KDA_WAIT_SPIN_LIMIT"] = "0"
    try:
        print("[waits] spin limit 0", flush=True)
        _, S_T = gpu_prefill(kda, g, 16)
    finally:
        del os.environ["KDA_WAIT_SPIN_LIMIT"]
    S = host(S_T)
    poisoned = 0
    for h in range(w.H):
        for c in range(0, 128, 16):
            blk = S[0, h, :, c:c + 16]
            ref = S_ref[0, h, :, c:c + 16]
            if np.isnan(blk).any():
                assert np.isnan(blk).all(), (h, c)
                poisoned += 1
            else:
                err = np.max(np.abs(blk - ref)) / np.max(np.abs(S_ref[0, h]))
                assert err <= 2e-2, (h, c, err)
    print(f"[waits] {poisoned} of {w.H * 8} column groups poisoned", flush=True)
    assert poisoned > 0
    o, S_T = gpu_prefill(kda, g, 16)
    assert slice_relerr(host(o), o_ref, 2) <= 2e-2
    assert slice_relerr(host(S_T), S_ref, 1) <= 2e-2
