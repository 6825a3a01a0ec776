"""Helpers for the GPU parity tests (comparison metrics and device copies)."""
import sys

import numpy as np
import torch

# Tolerances (o: max-abs on the io dtype output; states: relative L2 over the
# whole written-state tensor).  bf16 state storage alone costs ~1.7e-3 rel-L2,
# so bf16 states are held to 5e-3 against the oracle fed the same bf16 input.
O_MAXABS = 2e-2
STATE_REL_F32 = 1e-3
STATE_REL_BF16 = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return None if x is None else x.cuda()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def max_abs(got, ref):
    if np.asarray(ref).size == 0:
        return 0.0
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def host(t):
    return t.detach().float().cpu().numpy()
