"""Helpers shared by the GPU tests: tolerances, comparison, oracle slices."""
import sys

import numpy as np
import torch

# Tolerances (max |got - ref| / max |ref| per output tensor):
#   fp32 q/k/v path: 1e-4;  bf16 q/k/v with fp32 state: 2e-2.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.max(np.abs(ref))
    if denom == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / denom)


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def unit_slice(x, a, b, h):
    """Tokens [a, b) of head h, keeping a head axis of 1: [b-a, 1, d]."""
    return x[a:b, h:h + 1]


def oracle_units(oracle, inp, units, cu_list, scale=1.0, t_limit=None):
    """Run the oracle on selected (sequence, head) units.

    Returns {(n, h): (o [L,1,dv], S [dk,dv])} where L = sequence length
    (or t_limit tokens if given)."""
    out = {}
    for (n, h) in units:
        a, b = cu_list[n], cu_list[n + 1]
        if t_limit is not None:
            b = min(b, a + t_limit)
        S0 = None
        if inp.get("S0") is not None:
            S0 = f64(inp["S0"][n:n + 1, h:h + 1])
        o, S = oracle.prefill(f64(unit_slice(inp["q"], a, b, h)), f64(unit_slice(inp["k"], a, b, h)),
                              f64(unit_slice(inp["v"], a, b, h)), f64(unit_slice(inp["g"], a, b, h)),
                              f64(inp["beta"][a:b, h:h + 1]), initial_state=S0, scale=scale)
        out[(n, h)] = (o, S[0, 0])
    return out
