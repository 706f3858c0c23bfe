"""kda_prefill_ex_noalloc: the prefill without workspace allocation (for
callers that cannot allocate), checked against kda_prefill_ex with the same
description on two calls in a row, the second smaller, so that the static
buffer's contents left by the first call cannot leak into the second.
Both calls need the buffer: they are dense single sequences long enough for
the library to run the segment scan."""
import pytest
import torch

from gpu_common import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16 = torch.bfloat16


@pytest.fixture(scope="module")
def kda():
    import linear_attention_recurrence_delta_amd as m
    return m


def _case(kda, T, H, seed):
    from linear_attention_recurrence_delta_amd import synth
    q, k, v, g, beta, gen = synth.token_inputs(T, H, 128, 128, BF16, seed, DEV, "mild")
    S0 = synth.initial_state(1, H, 128, 128, 0.05, gen, DEV)
    need = kda.kda_prefill_ex_workspace_bytes(1, T, H, 128, 128, BF16)
    say("CASE noalloc T=%d H=%d: the plan needs %d bytes of workspace (static buffer %d)"
        % (T, H, need, kda.kda_noalloc_scratch_bytes()))
    assert 0 < need <= kda.kda_noalloc_scratch_bytes()
    o_ref, S_ref = kda.kda_prefill(q, k, v, g, beta, S0)
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    kda.kda_prefill(q, k, v, g, beta, S0, noalloc=True, out=o, final_state=S)
    torch.cuda.synchronize()
    e_o, e_s = rel_err(f64(o), f64(o_ref)), rel_err(f64(S), f64(S_ref))
    say("  vs kda_prefill: rel err o=%.3e S=%.3e, bitwise %s" % (e_o, e_s, torch.equal(o, o_ref) and torch.equal(S, S_ref)))
    assert e_o <= TOL[BF16] and e_s <= TOL[BF16]
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)  # same plan, same kernels


def test_two_calls_second_smaller(kda):
    _case(kda, 40000, 2, 3100)   # 2 (sequence, head) units: 32 segments
    _case(kda, 36000, 1, 3101)   # 1 unit: a smaller buffer footprint


def test_no_workspace_calls(kda):
    # a packed batch needs no workspace: the call runs as kda_prefill
    from linear_attention_recurrence_delta_amd import synth
    q, k, v, g, beta, _ = synth.token_inputs(500, 2, 128, 128, BF16, 3102, DEV)
    cu = torch.tensor([0, 123, 500], dtype=torch.int32, device=DEV)
    o_ref, S_ref = kda.kda_prefill(q, k, v, g, beta, None, cu)
    o, S = kda.kda_prefill(q, k, v, g, beta, None, cu, noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
