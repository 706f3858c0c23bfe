"""KDA_VALIDATE=1: the opt-in device check of g, beta and cu_seqlens.

Inputs at the edges of the preconditions (g = -5 and 0, beta = 0 and 1)
pass and give the same result as an unchecked call; values outside them,
NaN and malformed sequence offsets are reported as KDA_ERR_DOMAIN before
the computation is launched (the output buffer keeps its contents).
"""
import math

import pytest
import torch

from gpu_common import say

pytestmark = pytest.mark.gpu
DEV = "cuda"
DOMAIN = 7


@pytest.fixture(scope="module")
def kda():
    import linear_attention_recurrence_delta_amd as m
    return m


def _prefill_inputs(T=100, H=2, d=128, seed=21):
    from linear_attention_recurrence_delta_amd import synth
    q, k, v, g, beta, _ = synth.token_inputs(T, H, d, d, torch.bfloat16, seed, DEV)
    cu = torch.tensor([0, 37, T], dtype=torch.int32, device=DEV)
    return q, k, v, g, beta, cu


def _expect_domain(kda, fn):
    with pytest.raises(kda.KdaError) as e:
        fn()
    assert e.value.status == DOMAIN


def test_valid_edges_pass_and_match(kda, monkeypatch):
    say("CASE validate: valid edge values")
    q, k, v, g, beta, cu = _prefill_inputs()
    g[:10].fill_(-5.0)
    g[10:20].fill_(0.0)
    beta[:5].fill_(0.0)
    beta[5:9].fill_(1.0)
    ref = kda.kda_prefill(q, k, v, g, beta, None, cu)
    monkeypatch.setenv("KDA_VALIDATE", "1")
    got = kda.kda_prefill(q, k, v, g, beta, None, cu)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])


@pytest.mark.parametrize("where,value", [("g", -5.5), ("g", 0.25), ("g", math.nan),
                                         ("beta", 1.5), ("beta", -0.01), ("beta", math.nan)])
def test_out_of_range_prefill_inputs(kda, monkeypatch, where, value):
    say("CASE validate: prefill %s = %r" % (where, value))
    q, k, v, g, beta, cu = _prefill_inputs()
    t = g if where == "g" else beta
    t.view(-1)[t.numel() - 3] = value  # one element, near the end
    monkeypatch.setenv("KDA_VALIDATE", "1")
    o = torch.full_like(v, 7.0)
    _expect_domain(kda, lambda: kda.kda_prefill(q, k, v, g, beta, None, cu, out=o))
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())  # nothing was launched
    monkeypatch.setenv("KDA_VALIDATE", "0")
    kda.kda_prefill(q, k, v, g, beta, None, cu)  # unchecked: runs (numbers undefined)
    torch.cuda.synchronize()


@pytest.mark.parametrize("cu_list", [[0, 60, 37, 100], [1, 37, 100], [0, 37, 99]])
def test_malformed_cu_seqlens(kda, monkeypatch, cu_list):
    say("CASE validate: cu_seqlens %s" % cu_list)
    q, k, v, g, beta, _ = _prefill_inputs()
    cu = torch.tensor(cu_list, dtype=torch.int32, device=DEV)
    monkeypatch.setenv("KDA_VALIDATE", "1")
    _expect_domain(kda, lambda: kda.kda_prefill(q, k, v, g, beta, None, cu))


def test_decode_inputs(kda, monkeypatch):
    from linear_attention_recurrence_delta_amd import synth
    say("CASE validate: decode")
    N, H, d = 6, 3, 128
    S = synth.decode_state(N, H, d, 0.05, 22, DEV)
    q, k, v, g, beta = synth.decode_inputs(N, H, d, torch.bfloat16, 23, DEV)
    monkeypatch.setenv("KDA_VALIDATE", "1")
    S1 = S.clone()
    kda.kda_decode_step(q, k, v, g, beta, S1)
    g[N - 1, H - 1, d - 1] = 0.5
    S2 = S.clone()
    _expect_domain(kda, lambda: kda.kda_decode_step(q, k, v, g, beta, S2))
    torch.cuda.synchronize()
    assert torch.equal(S2, S)  # the state was not touched


def test_binding_checks_output_shapes(kda):
    """The Python binding refuses caller-supplied outputs of the wrong shape
    or device before the C ABI is called (the kernels size their stores from
    T, H and d, not from the buffers)."""
    say("CASE binding: out= / final_state= shapes")
    q, k, v, g, beta, cu = _prefill_inputs()
    T, H = q.shape[:2]
    bad_o = torch.empty((T - 1, H, 128), dtype=torch.bfloat16, device=DEV)
    bad_s = torch.empty((1, H, 128, 128), dtype=torch.float32, device=DEV)  # 2 sequences
    with pytest.raises(ValueError):
        kda.kda_prefill(q, k, v, g, beta, None, cu, out=bad_o)
    with pytest.raises(ValueError):
        kda.kda_prefill(q, k, v, g, beta, None, cu, final_state=bad_s)
    with pytest.raises(ValueError):
        kda.kda_prefill(q, k, v, g, beta, None, cu.cpu())
    from linear_attention_recurrence_delta_amd import synth
    dq, dk, dv, dg, db = synth.decode_inputs(4, 2, 128, torch.bfloat16, 22, DEV)
    S = torch.zeros((4, 2, 128, 128), device=DEV)
    with pytest.raises(ValueError):
        kda.kda_decode_step(dq, dk, dv, dg, db, S, out=torch.empty((4, 1, 128), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        kda.kda_decode_step(dq, dk, dv, dg, db, S.cpu())
