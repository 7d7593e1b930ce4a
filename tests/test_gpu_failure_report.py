"""GPU: a split combine that gives up waiting is reported to the host.

The split-T decode combines its splits inside the launch; each combine polls
ready flags with a bounded wait.  A test control (gqa_set_merge_wait) makes
every combine wait for a flag value that no split writes, so each one gives up
after a few polls while every workgroup still exits normally.  The outputs of
that call must be NaN (never a silently wrong finite value), the workspace's
sticky status must turn into GQA_ERR_DEVICE, and after a clear the same
workspace must give correct results again.
"""
import sys

import pytest
import torch

import workloads as W
from harness import Pair, compare_rows

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_gqa_attention_attn_amd  # noqa: F401  (fails loudly if the library is missing)


def test_merge_give_up_is_reported():
    import causal_gqa_attention_attn_amd as lib
    say("case: forced split-combine give-up, Hq=32 Hkv=8 d=128, two 2000-token caches (8 splits each)")
    shape = W.AttnShape(B=2, n=2000, Hq=32, Hkv=8, d=128, dtype=torch.bfloat16, theta=1e4)
    inp = W.prefill_inputs(shape, 901)
    pair = Pair(1, 8, 128, 300, 2, 140, torch.bfloat16, 1e4)
    ids = [0, 1]
    pair.prefill(0, ids, inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    dshape = W.AttnShape(B=2, n=1, Hq=32, Hkv=8, d=128, dtype=torch.bfloat16, theta=1e4)
    o, r = pair.step(0, ids, W.decode_step_inputs(dshape, 902, 0))
    compare_rows(o, r, torch.bfloat16)
    lib.gqa_workspace_status(pair.gpu.handle, pair.ws)          # nothing to report
    q = W.decode_step_inputs(dshape, 903, 0).q
    lib.gqa_set_merge_wait(64, True)
    try:
        bad, _ = pair.decode(0, ids, q, [2001, 2001], oracle=False)
    finally:
        lib.gqa_set_merge_wait(1 << 18, False)
    assert torch.isnan(bad.float()).all(), "a combine that gave up must write NaN, never a finite value"
    with pytest.raises(lib.GqaError) as e:
        lib.gqa_workspace_status(pair.gpu.handle, pair.ws, clear=True)
    assert e.value.name == "DEVICE"
    lib.gqa_workspace_status(pair.gpu.handle, pair.ws)          # cleared
    # the same workspace serves correct decode steps again, fused and unfused
    for t in range(2):
        o, r = pair.step_fused(0, ids, W.decode_step_inputs(dshape, 904, t))
        compare_rows(o, r, torch.bfloat16)
        o, r = pair.step(0, ids, W.decode_step_inputs(dshape, 905, t))
        compare_rows(o, r, torch.bfloat16)
    lib.gqa_workspace_status(pair.gpu.handle, pair.ws)
    pair.check_cache(ids)
