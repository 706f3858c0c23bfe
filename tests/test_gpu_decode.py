"""GPU parity of kda_decode_step against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from gpu_common import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def kda():
    import linear_attention_recurrence_delta_amd as m
    return m


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_decode_steps_match_oracle(kda, oracle_mod, dtype, d):
    from linear_attention_recurrence_delta_amd import synth
    N, H, steps = 5, 3, 4
    say("CASE decode d=%d dtype=%s N=%d H=%d steps=%d" % (d, dtype, N, H, steps))
    S = synth.decode_state(N, H, d, 0.05, 7, DEV)
    S_ref = f64(S)
    for st in range(steps):
        q, k, v, g, beta = synth.decode_inputs(N, H, d, dtype, 100 * d + st, DEV)
        o = kda.kda_decode_step(q, k, v, g, beta, S, scale=0.9)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle_mod.decode_step(f64(q), f64(k), f64(v), f64(g), f64(beta), S_ref, scale=0.9)
        eo, es = rel_err(f64(o), o_ref), rel_err(f64(S), S_ref)
        say("  step %d rel err o=%.3e S=%.3e" % (st, eo, es))
        assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_equals_prefill_of_one_token(kda):
    from linear_attention_recurrence_delta_amd import synth
    N, H, d = 6, 4, 128
    say("CASE decode vs prefill T=1")
    S = synth.decode_state(N, H, d, 0.05, 8, DEV)
    q, k, v, g, beta = synth.decode_inputs(N, H, d, torch.float32, 9, DEV)
    cu = torch.arange(N + 1, dtype=torch.int32, device=DEV)
    o_p, S_p = kda.kda_prefill(q, k, v, g, beta, S.clone(), cu, chunk_size=16)
    o_d = kda.kda_decode_step(q, k, v, g, beta, S)
    torch.cuda.synchronize()
    assert rel_err(f64(o_d), f64(o_p)) <= 1e-5
    assert rel_err(f64(S), f64(S_p)) <= 1e-5


def test_decode_exact_recall(kda):
    # g = 0, beta = 1, q = k unit: the step returns v exactly (up to rounding).
    from linear_attention_recurrence_delta_amd import synth
    N, H, d = 4, 2, 128
    say("CASE decode exact recall")
    S = synth.decode_state(N, H, d, 0.3, 10, DEV)
    q, k, v, g, beta = synth.decode_inputs(N, H, d, torch.float32, 11, DEV)
    g.zero_()
    beta.fill_(1.0)
    o = kda.kda_decode_step(k, k, v, g, beta, S)
    torch.cuda.synchronize()
    assert rel_err(f64(o), f64(v)) <= 1e-5


def test_decode_deterministic(kda):
    from linear_attention_recurrence_delta_amd import synth
    N, H, d = 16, 8, 128
    S1 = synth.decode_state(N, H, d, 0.05, 12, DEV)
    S2 = S1.clone()
    q, k, v, g, beta = synth.decode_inputs(N, H, d, torch.bfloat16, 13, DEV)
    o1 = kda.kda_decode_step(q, k, v, g, beta, S1)
    o2 = kda.kda_decode_step(q, k, v, g, beta, S2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
