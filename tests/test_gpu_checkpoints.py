"""State checkpoints during prefill (kda_prefill_checkpointed).

Checkpoint j of sequence n is the state after its first (j + 1) * interval
tokens; the oracle computes it by definition (the final state of its
token-by-token recurrence over that prefix).  Each checkpoint is compared with
the oracle to the same bar as a final state; the outputs and final states
of the call must be bitwise those of kda_prefill, slots past the last
checkpoint must stay untouched, and both prefill kernels are covered.
"""
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


def _inputs(lengths, H, d, dtype, seed, init_std=None):
    from linear_attention_recurrence_delta_amd import synth
    T = sum(lengths)
    q, k, v, g, beta, gen = synth.token_inputs(T, H, d, d, dtype, seed, DEV)
    S0 = synth.initial_state(len(lengths), H, d, d, init_std, gen, DEV) if init_std else None
    cu_list = [0] + [int(x) for x in np.cumsum(lengths)]
    cu = torch.tensor(cu_list, dtype=torch.int32, device=DEV)
    return q, k, v, g, beta, S0, cu, cu_list


def _check(kda, oracle_mod, lengths, H, d, dtype, interval, chunk, seed, init_std=None, plan=None):
    say("CASE checkpoints lengths=%s H=%d d=%d %s interval=%d chunk=%d plan=%s S0=%s"
        % (lengths, H, d, dtype, interval, chunk, plan, init_std))
    q, k, v, g, beta, S0, cu, cu_list = _inputs(lengths, H, d, dtype, seed, init_std)
    T = sum(lengths)
    cap = T // interval
    ck = torch.full((cap + 2, H, d, d), float("nan"), dtype=torch.float32, device=DEV)  # 2 spare slots
    o, S, ck, first = kda.kda_prefill_checkpointed(q, k, v, g, beta, S0, cu, checkpoint_interval=interval,
                                                   chunk_size=chunk, checkpoints=ck, plan=plan)
    o_ref, S_ref = kda.kda_prefill(q, k, v, g, beta, S0, cu, chunk_size=chunk, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    exp_ck, exp_first = oracle_mod.prefill_checkpoints(f64(q), f64(k), f64(v), f64(g), f64(beta),
                                                       None if S0 is None else f64(S0), np.array(cu_list),
                                                       interval=interval)
    assert first.cpu().tolist() == exp_first.tolist()
    n_ck = int(exp_first[-1])
    got = f64(ck)
    worst = 0.0
    for s in range(n_ck):
        worst = max(worst, rel_err(got[s], exp_ck[s]))
    say("  %d checkpoints, worst rel err %.3e" % (n_ck, worst))
    assert worst <= TOL[dtype], worst
    assert np.isnan(got[n_ck:]).all()  # slots past the last checkpoint are not written
    # a sequence whose length is a multiple of the interval ends on its final state
    for n, L in enumerate(lengths):
        if L and L % interval == 0:
            np.testing.assert_array_equal(got[int(exp_first[n + 1]) - 1], f64(S[n]))


@pytest.mark.parametrize("interval", [16, 32, 64])
def test_bf16_varlen_default_kernel(kda, oracle_mod, interval):
    _check(kda, oracle_mod, [37, 0, 64, 1, 130, 200, 16], 2, 128, torch.bfloat16, interval, 0, 301)


def test_bf16_initial_state_and_many_heads(kda, oracle_mod):
    _check(kda, oracle_mod, [96, 50, 160], 5, 128, torch.bfloat16, 32, 0, 302, init_std=0.05)


@pytest.mark.parametrize("chunk,interval", [(16, 16), (32, 32), (64, 64), (64, 128)])
def test_bf16_chunk_staged_kernel(kda, oracle_mod, chunk, interval):
    _check(kda, oracle_mod, [37, 0, 64, 1, 130, 200], 2, 128, torch.bfloat16, interval, chunk, 303,
           init_std=0.05, plan=dict(kernel=2))  # KDA_KERNEL_CHUNK_STAGED


@pytest.mark.parametrize("cols", [16, 128])
def test_bf16_pipelined_slab_widths(kda, oracle_mod, cols):
    """Checkpoints from the pipeline at the narrowest and the widest slab:
    fp32 row-major states whichever workgroup holds a column."""
    _check(kda, oracle_mod, [37, 0, 64, 1, 130, 200, 16], 2, 128, torch.bfloat16, 16, 0, 305, init_std=0.05,
           plan=dict(kernel=1, slab_columns=cols))


def test_no_segment_scan_with_checkpoints(kda):
    """Checkpoints pin every chunk to one chain: an explicit segment scan is
    refused (KDA_ERR_UNSUPPORTED) and the library never picks one."""
    from linear_attention_recurrence_delta_amd import synth
    q, k, v, g, beta, _ = synth.token_inputs(2048, 1, 128, 128, torch.bfloat16, 307, DEV)
    with pytest.raises(kda.KdaError) as e:
        kda.kda_prefill_checkpointed(q, k, v, g, beta, checkpoint_interval=256, plan=dict(segments=4))
    assert e.value.status == 3
    assert kda.kda_prefill_ex_workspace_bytes(1, 1 << 20, 16, 128, 128, torch.bfloat16,
                                              checkpoint_interval=1024, checkpoint_capacity=1024) == 0


@pytest.mark.parametrize("d,chunk", [(16, 16), (64, 32), (128, 16)])
def test_fp32(kda, oracle_mod, d, chunk):
    _check(kda, oracle_mod, [33, 48, 0, 70], 2, d, torch.float32, 2 * chunk, chunk, 304, init_std=0.3)


def test_dense_batch_layout(kda, oracle_mod):
    """cu_seqlens = None: equal-length sequences, checkpoints by sequence."""
    from linear_attention_recurrence_delta_amd import synth
    say("CASE checkpoints dense B=3 T=80 interval 32")
    B, L, H, d = 3, 80, 2, 128
    q, k, v, g, beta, _ = synth.token_inputs(B * L, H, d, d, torch.bfloat16, 305, DEV)
    o, S, ck, first = kda.kda_prefill_checkpointed(q, k, v, g, beta, None, None, num_seqs=B,
                                                   checkpoint_interval=32)
    torch.cuda.synchronize()
    assert first.cpu().tolist() == [0, 2, 4, 6]
    cu = np.array([0, L, 2 * L, 3 * L])
    exp_ck, _ = oracle_mod.prefill_checkpoints(f64(q), f64(k), f64(v), f64(g), f64(beta), None, cu, interval=32)
    got = f64(ck)
    assert ck.shape[0] == (B * L) // 32 == 7
    for s in range(6):
        assert rel_err(got[s], exp_ck[s]) <= TOL[torch.bfloat16]


def test_interval_longer_than_every_sequence(kda, oracle_mod):
    say("CASE checkpoints interval 512 > every length")
    q, k, v, g, beta, S0, cu, _ = _inputs([100, 200, 300], 2, 128, torch.bfloat16, 306)
    ck = torch.full((1, 2, 128, 128), 7.0, dtype=torch.float32, device=DEV)  # T // 512 = 1 slot
    o, S, ck, first = kda.kda_prefill_checkpointed(q, k, v, g, beta, S0, cu, checkpoint_interval=512,
                                                   checkpoints=ck)
    torch.cuda.synchronize()
    assert first.cpu().tolist() == [0, 0, 0, 0]
    assert bool((ck == 7.0).all())
