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


# Workgroups per launch of the decode kernel is at most (CUs x 64) / (waves
# per workgroup); 2.5x that many units (+7, ragged) makes each workgroup walk
# two or three units, prefetching the next one while it finishes the current.
_DECODE_THREADS = {16: 64, 32: 64, 64: 256, 128: 1024}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [16, 64, 128])
def test_decode_units_beyond_the_grid(kda, oracle_mod, dtype, d):
    from linear_attention_recurrence_delta_amd import synth
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * 64 // (_DECODE_THREADS[d] // 64)
    H = 8
    N = (5 * blocks // 2 + 7 + H - 1) // H
    say("CASE decode d=%d dtype=%s N=%d H=%d (%d units, grid %d)" % (d, dtype, N, H, N * H, blocks))
    S0 = synth.decode_state(N, H, d, 0.05, 20 + d, DEV)
    q, k, v, g, beta = synth.decode_inputs(N, H, d, dtype, 21 + d, DEV)
    S = S0.clone()
    o = kda.kda_decode_step(q, k, v, g, beta, S, scale=0.8)
    torch.cuda.synchronize()
    # Oracle on sampled units: the first, ones walked second and third by a
    # workgroup, and the last (ragged) ones.
    units = N * H
    picks = sorted({0, 1, blocks - 1, blocks, blocks + 1, 2 * blocks - 1, 2 * blocks, 2 * blocks + 3,
                    units - 2, units - 1} | set(range(0, units, max(1, units // 40))))
    n_idx = torch.tensor([u // H for u in picks], device=DEV)
    h_idx = torch.tensor([u % H for u in picks], device=DEV)
    sel = lambda x: f64(x[n_idx, h_idx].unsqueeze(1))
    o_ref, S_ref = oracle_mod.decode_step(sel(q), sel(k), sel(v), sel(g), sel(beta), sel(S0), scale=0.8)
    eo, es = rel_err(sel(o), o_ref), rel_err(sel(S), S_ref)
    say("  %d sampled units: rel err o=%.3e S=%.3e" % (len(picks), eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    # The same sequences decoded in a launch of their own (fewer units than
    # workgroups: one unit each) give bitwise the same results.
    for lo, hi in ((0, 3), (N // 2, N // 2 + 5), (N - 4, N)):
        S_part = S0[lo:hi].clone()
        o_part = kda.kda_decode_step(q[lo:hi].contiguous(), k[lo:hi].contiguous(), v[lo:hi].contiguous(),
                                     g[lo:hi].contiguous(), beta[lo:hi].contiguous(), S_part, scale=0.8)
        torch.cuda.synchronize()
        assert torch.equal(o_part, o[lo:hi]) and torch.equal(S_part, S[lo:hi])
