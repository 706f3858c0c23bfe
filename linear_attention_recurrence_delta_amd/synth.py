"""Seeded synthetic inputs shaped like the KDA layers the pages describe.

This module holds no step of the method: it only draws random tensors with
the stated distributions.  Both the HIP path and the CPU oracle consume its
output (the oracle gets exact fp64 copies of the very values handed to the
GPU).  Shapes follow "Inside Kimi K3" (flozi.net), section "Sequence
mixing": 96 heads of dimension 128 per KDA layer; the log-decay uses the K3
bound g in (g_min, 0) with g_min = -5 ("Understanding Kimi K3's attention",
g_min equation); q and k are unit-norm (L2Norm sits upstream of the core in
the same page's symbol table).

Recipe (every workload):
  q, k ~ N(0, 1), then divided by their L2 norm over the head dim (fp32), then
         cast to the q/k/v dtype;
  v    ~ N(0, 1), cast;
  g    = -5 * sigmoid(z), z ~ N(0, 1) per channel (fp32), so g in (-5, 0);
  beta = sigmoid(N(0, 1)) (fp32);
  S0   ~ N(0, init_std^2) (fp32) when an initial state is asked for.
Draw order is fixed: q, k, v, z, beta logits, S0.  Draws use a torch
generator on the target device seeded with `seed`.
"""
from __future__ import annotations

import math

import numpy as np
import torch

G_MIN = -5.0


def _gen(device, seed):
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def _unit_rows(x):
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def token_inputs(T, H, dk, dv, dtype, seed, device, g_mode="k3", chunk_rows=1 << 22):
    """q, k, v ([T,H,d] in dtype), g ([T,H,dk] fp32), beta ([T,H] fp32).

    g_mode: "k3" -> g = -5 sigmoid(z); "mild" -> g = -0.05 sigmoid(z);
            "zero" -> g = 0.  Large tensors are drawn in row blocks to bound
    temporary memory; the draw order stays q, k, v, z, beta.
    """
    gen = _gen(device, seed)
    out = {}
    for name, d, unit in (("q", dk, True), ("k", dk, True), ("v", dv, False)):
        t = torch.empty((T, H, d), dtype=dtype, device=device)
        rows = max(1, chunk_rows // max(1, H * d))
        for a in range(0, T, rows):
            b = min(T, a + rows)
            x = torch.randn((b - a, H, d), generator=gen, device=device, dtype=torch.float32)
            t[a:b] = (_unit_rows(x) if unit else x).to(dtype)
        out[name] = t
    g = torch.empty((T, H, dk), dtype=torch.float32, device=device)
    rows = max(1, chunk_rows // max(1, H * dk))
    for a in range(0, T, rows):
        b = min(T, a + rows)
        z = torch.randn((b - a, H, dk), generator=gen, device=device, dtype=torch.float32)
        if g_mode == "k3":
            g[a:b] = G_MIN * torch.sigmoid(z)
        elif g_mode == "mild":
            g[a:b] = -0.05 * torch.sigmoid(z)
        elif g_mode == "zero":
            g[a:b] = 0.0
        else:
            raise ValueError(g_mode)
    beta = torch.sigmoid(torch.randn((T, H), generator=gen, device=device, dtype=torch.float32))
    return out["q"], out["k"], out["v"], g, beta, gen


def fused_inputs(T, H, d, dtype, seed, device, a_log_std=0.3, chunk_rows=1 << 22):
    """Inputs of the fused entry point: raw (unnormalised) q, k with norms that
    vary per token (N(0, 1) rows times e^{N(0, 0.5)}), v ~ N(0, 1), decay
    logits z ~ N(0, 1) (all in dtype), beta = sigmoid(N(0, 1)) and per-head
    a_log ~ N(0, a_log_std^2) (fp32; a_log_std = 0 gives the same g
    distribution as token_inputs).  Draw order: q, k, v, z, beta, a_log."""
    gen = _gen(device, seed)
    out = {}
    rows = max(1, chunk_rows // max(1, H * d))
    for name in ("q", "k", "v", "z"):
        t = torch.empty((T, H, d), dtype=dtype, device=device)
        for a in range(0, T, rows):
            b = min(T, a + rows)
            x = torch.randn((b - a, H, d), generator=gen, device=device, dtype=torch.float32)
            if name in ("q", "k"):
                x = x * torch.exp(0.5 * torch.randn((b - a, H, 1), generator=gen, device=device))
            t[a:b] = x.to(dtype)
        out[name] = t
    beta = torch.sigmoid(torch.randn((T, H), generator=gen, device=device, dtype=torch.float32))
    a_log = a_log_std * torch.randn((H,), generator=gen, device=device, dtype=torch.float32)
    return out["q"], out["k"], out["v"], out["z"], a_log, beta, gen


def initial_state(N, H, dk, dv, std, gen, device):
    return std * torch.randn((N, H, dk, dv), generator=gen, device=device, dtype=torch.float32)


def varlen_lengths(n_seqs=16, total=32768, lo=256, hi=8192, seed=2):
    """Sequence lengths log-uniform in [lo, hi], rescaled to sum to `total`.

    u_i ~ U(0,1) (numpy default_rng(seed)); L_i = lo * (hi/lo)^u_i; rescale
    L_i <- round(L_i * total / sum L); clamp to [lo, hi]; put the remainder on
    the longest length that can take it (repeat until the sum is exact).
    """
    rng = np.random.default_rng(seed)
    u = rng.random(n_seqs)
    L = lo * (hi / lo) ** u
    L = np.round(L * total / L.sum()).astype(np.int64)
    L = np.clip(L, lo, hi)
    for _ in range(4 * n_seqs):
        rem = int(total - L.sum())
        if rem == 0:
            break
        order = np.argsort(-L) if rem > 0 else np.argsort(L)
        for i in order:
            room = (hi - L[i]) if rem > 0 else (L[i] - lo)
            if room > 0:
                step = min(abs(rem), int(room))
                L[i] += step if rem > 0 else -step
                break
    assert int(L.sum()) == total and L.min() >= lo and L.max() <= hi
    return [int(x) for x in L]


def cu_from_lengths(lengths, device):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return torch.from_numpy(cu).to(device)


# ---------------------------------------------------------------------------
# The workloads: small oracle-sized cases and the K3-shaped ones.
# ---------------------------------------------------------------------------
WORKLOADS = {
    # name: (N, T per sequence or lengths, H, d, dtype, chunk, init_std, seed)
    "single_head_fp32": dict(N=1, T=64, H=1, d=16, dtype=torch.float32, chunk=16, init_std=None, seed=0),
    "multi_head_bf16": dict(N=1, T=4096, H=8, d=128, dtype=torch.bfloat16, chunk=64, init_std=0.02, seed=1),
    "k3_varlen_32k": dict(N=16, T=None, H=96, d=128, dtype=torch.bfloat16, chunk=64, init_std=None, seed=2),
    "k3_dense_32k": dict(N=1, T=32768, H=96, d=128, dtype=torch.bfloat16, chunk=64, init_std=None, seed=2),
    "long_1m_h16": dict(N=1, T=1048576, H=16, d=128, dtype=torch.bfloat16, chunk=64, init_std=None, seed=3),
}


def workload_inputs(name, device, g_mode="k3"):
    """Inputs of a named workload: dict with q, k, v, g, beta, S0, cu, lengths."""
    w = WORKLOADS[name]
    if w["T"] is None:
        lengths = varlen_lengths()
        T = sum(lengths)
        cu = cu_from_lengths(lengths, device)
        N = len(lengths)
    else:
        T = w["N"] * w["T"]
        lengths = [w["T"]] * w["N"]
        cu = None
        N = w["N"]
    q, k, v, g, beta, gen = token_inputs(T, w["H"], w["d"], w["d"], w["dtype"], w["seed"], device, g_mode)
    S0 = initial_state(N, w["H"], w["d"], w["d"], w["init_std"], gen, device) if w["init_std"] else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, cu=cu, lengths=lengths, N=N, T=T,
                H=w["H"], d=w["d"], dtype=w["dtype"], chunk=w["chunk"])


def decode_inputs(N, H, d, dtype, seed, device, g_mode="k3"):
    """One decode token per (n, h): q, k unit-norm, v, g in (-5, 0), beta."""
    q, k, v, g, beta, gen = token_inputs(N, H, d, d, dtype, seed, device, g_mode)
    return q, k, v, g, beta


def decode_state(N, H, d, std, seed, device):
    gen = _gen(device, seed)
    return std * torch.randn((N, H, d, d), generator=gen, device=device, dtype=torch.float32)


def log2_ceil(x):
    return int(math.ceil(math.log2(max(1, x))))
