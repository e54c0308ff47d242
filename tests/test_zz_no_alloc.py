"""The allocation-free decode step (static device scratch) against the workspace
entry point it stands for: identical outputs, selections and lse on two calls in a
row, the second on a smaller input, through the C ABI."""
import numpy as np
import pytest
import torch

import block_sparse_attention_06_amd as Q
from synth import generate, workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def _step(batch, lk, seq):
    wl = workload("decode1m", batch=batch, lk=lk)
    inp = generate(wl, device=DEV, seq_lens=seq)
    args = (inp["q"], inp["q_idx"], inp["w"], inp["k_pooled"], inp["k_cache"], inp["v_cache"],
            inp["seq_lens"])
    ref = [t.clone() for t in Q.qsa_decode_forward(*args, budget=wl.budget)]
    got = Q.qsa_decode_forward_noalloc(*args, budget=wl.budget)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_decode_matches_workspace_entry_point():
    # First call: 6 sequences of up to 256K tokens (ragged lengths, a short one); second
    # call: a smaller input in the same scratch (2 sequences of up to 40K tokens).
    for batch, lk, seq in ((6, 262144, [262144, 262144 - 4001, 70000, 2048, 1500, 9]),
                           (2, 40000, [40000, 17]) ):
        _say(f"noalloc decode batch={batch} lk={lk} seq={seq}")
        ref, got = _step(batch, lk, seq)
        for name, a, b in zip(("out", "lse", "sel"), got, ref):
            assert torch.equal(a, b), f"{name} differs (batch {batch}, lk {lk})"
        assert int((got[2] >= 0).sum()) > 0
