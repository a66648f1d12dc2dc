"""moe_lora_forward_noalloc (the static-scratch entry point) against
moe_lora_forward (the workspace entry point), through the C ABI.

Two calls in a row on the same GPU, the second with a smaller batch, so the
second runs on scratch that still holds the first call's intermediates; each
must agree with the workspace entry point on the same inputs (the oracle's
bars; with the fixed-order combine the two also agree bit for bit, since
they share every kernel). A call that needs more than the static array is
refused before anything is enqueued.
"""
import sys

import numpy as np
import pytest
import torch

from lora_mixture_experts_amd import moe_lora as ml
from lora_mixture_experts_amd import workloads as wl

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL = 1e-2, 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def metrics(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.abs(a - b)
    return err.max() / np.abs(b).max(), err.mean() / np.abs(b).mean()


def _inputs(case, dev, T):
    t = wl.device_tensors(case, dev)
    return t, t["x"][:T].contiguous(), t["logits"][:T].contiguous(), t["adapter_ids"][:T].contiguous()


def _both(case, t, x, lg, ad, T, dev, flags=0):
    d = ml.make_desc(T, case.H, case.I, case.E, case.top_k, case.L, case.r, flags=flags)
    wts = ml.weights_struct(t["w_gate_up"], t["w_down"], t["a_gate_up"], t["b_gate_up"], t["a_down"],
                            t["b_down"])
    ws = torch.empty(ml.workspace_bytes(d), dtype=torch.uint8, device=dev)
    ref = torch.full((T, case.H), float("nan"), dtype=torch.float32, device=dev)
    ml.forward(d, wts, x, lg, ad, ref, ws)
    got = torch.full((T, case.H), float("nan"), dtype=torch.float32, device=dev)
    ml.forward_noalloc(d, wts, x, lg, ad, got)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    dev = torch.device("cuda:0")
    case = wl.make_case("decode")
    t, x, lg, ad = _inputs(case, dev, case.T)
    # first call: the 16-token decode batch; second: a 5-token batch (smaller
    # plan, different block counts) on the scratch the first call left behind
    for flags in (0, ml.FLAG_FUSED_COMBINE):
        for T in (case.T, 5):
            log(f"noalloc decode T={T} flags={flags}")
            got, ref = _both(case, t, x[:T].contiguous(), lg[:T].contiguous(), ad[:T].contiguous(), T, dev,
                             flags)
            assert np.all(np.isfinite(got))
            mx, mean = metrics(got, ref)
            assert mx <= MAX_TOL and mean <= MEAN_TOL, (T, mx, mean)
            if not flags & ml.FLAG_FUSED_COMBINE:
                np.testing.assert_array_equal(got, ref)


def test_noalloc_refuses_a_call_larger_than_the_scratch():
    dev = torch.device("cuda:0")
    c = wl.CONFIGS["prefill"]
    d = ml.make_desc(c["T"], c["H"], c["I"], c["E"], c["top_k"], c["L"], c["r"])
    assert ml.workspace_bytes(d) > ml.SCRATCH_BYTES
    # pointers of the right alignment; nothing is read because the call is
    # refused on the host before any launch
    buf = torch.zeros(4096, dtype=torch.bfloat16, device=dev)
    wts = ml.weights_struct(buf, buf, buf, buf, buf, buf)
    out = torch.full((8,), 3.0, dtype=torch.float32, device=dev)
    lg = torch.zeros(8, dtype=torch.float32, device=dev)
    ad = torch.zeros(8, dtype=torch.int32, device=dev)
    with pytest.raises(ml.MoeLoraError) as ei:
        ml.forward_noalloc(d, wts, buf, lg, ad, out)
    assert ei.value.code == ml.ESCRATCH
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
