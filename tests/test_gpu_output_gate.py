"""kda_output_gate: Sigmoid(gate) * RMSNorm(o) * weight per (token, head) row.

Compared with the oracle's fp64 evaluation of the same bf16/fp32 inputs:
every supported d_v in both dtypes, ragged token counts (rows that do not
fill a workgroup), in-place use, zero rows, large-magnitude rows, and the
K3-sized output (32768 tokens x 96 heads x 128).
"""
import numpy as np
import pytest
import torch

from gpu_common import f64, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
# bf16 result: one rounding of y (2^-9 relative) on top of fp32 arithmetic
TOL = {torch.bfloat16: 8e-3, torch.float32: 1e-5}


@pytest.fixture(scope="module")
def kda():
    import linear_attention_recurrence_delta_amd as m
    return m


def _inputs(T, H, dv, dtype, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    o = (torch.randn((T, H, dv), generator=gen, device=DEV) * 0.7).to(dtype)
    gate = (2.0 * torch.randn((T, H, dv), generator=gen, device=DEV)).to(dtype)
    w = 1.0 + 0.25 * torch.randn((dv,), generator=gen, device=DEV)
    return o, gate, w


def _max_rel_row(got, ref):
    """max over rows of |got - ref| / max |ref| in that row (rows of mixed scale)."""
    got, ref = f64(got), np.asarray(ref)
    den = np.max(np.abs(ref), axis=-1, keepdims=True)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_parity(kda, oracle_mod, dtype, dv):
    say("CASE output gate %s d_v=%d" % (dtype, dv))
    o, gate, w = _inputs(333, 3, dv, dtype, 500 + dv)
    y = kda.kda_output_gate(o, gate, w, eps=1e-6)
    torch.cuda.synchronize()
    ref = oracle_mod.output_gate(f64(o), f64(gate), f64(w), 1e-6)
    err = _max_rel_row(y, ref)
    say("  max row-relative error %.3e" % err)
    assert err <= TOL[dtype]


def test_in_place_and_special_rows(kda, oracle_mod):
    say("CASE output gate in place, zero and large rows")
    o, gate, w = _inputs(77, 2, 128, torch.bfloat16, 510)
    o[3, 1].zero_()
    o[10, 0] *= 300.0
    ref = oracle_mod.output_gate(f64(o), f64(gate), f64(w), 1e-5)
    y = kda.kda_output_gate(o, gate, w, eps=1e-5, out=o)   # y is o
    torch.cuda.synchronize()
    assert y.data_ptr() == o.data_ptr()
    assert bool((o[3, 1] == 0).all())
    assert _max_rel_row(o, ref) <= TOL[torch.bfloat16]


def test_k3_sized_output(kda, oracle_mod):
    say("CASE output gate 32768 x 96 x 128 bf16, sampled rows")
    o, gate, w = _inputs(32768, 96, 128, torch.bfloat16, 511)
    y = kda.kda_output_gate(o, gate, w, eps=1e-6)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 4095, 20000, 32767], device=DEV)
    ref = oracle_mod.output_gate(f64(o.index_select(0, rows)), f64(gate.index_select(0, rows)), f64(w), 1e-6)
    assert _max_rel_row(y.index_select(0, rows), ref) <= TOL[torch.bfloat16]
    assert torch.isfinite(y).all()
