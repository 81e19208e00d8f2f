"""Pin of the oracle's clip coefficient against an independent implementation:
torch.nn.utils.clip_grad_norm_ on fp64 gradient tensors.

The pages set global gradient clipping ("gradient_clipping": 1.0 in the
DeepSpeed configuration of the tutorial's §4.2) and name no formula; the
oracle reads it as coef = min(1, max_norm / (norm + 1e-6)) in fp64, rounded
once to fp32.  torch scales every gradient by that same clamped coefficient,
so a gradient element that is a power of two gives the coefficient back
exactly after the call (a power-of-two divide is exact).

The cases put norms where the + 1e-6 decides the fp32 coefficient (norms of
1e-5 .. 1e-2 against comparable max_norm, and norms within 1e-6 below
max_norm, where the clamp alone would give 1), both sides of the clamp, and
norms exactly equal to max_norm.  Exact cases use integer vectors whose sum of
squares is a perfect square, scaled by powers of two, so that both sides see
the same exact norm and the fp64 coefficients must agree bit for bit; random
cases compare the fp32 coefficient exactly and the norm within the summation
error bound.
"""
import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

# integer vectors with an integer norm and at least one power-of-two entry (its index)
PYTHAGOREAN = [((3, 4), 5, 1), ((1, 2, 2), 3, 0), ((2, 3, 6), 7, 0), ((1, 4, 8), 9, 2),
               ((2, 6, 9), 11, 0), ((8, 15), 17, 0), ((4, 4, 7), 9, 0), ((2, 10, 11), 15, 0),
               ((4, 13, 16), 21, 2), ((16, 63), 65, 0)]


def _torch_clip(g: np.ndarray, max_norm: float, probe: int):
    """(total_norm, clamped coefficient) from torch on fp64 gradients."""
    p = torch.nn.Parameter(torch.zeros(g.size, dtype=torch.float64))
    p.grad = torch.from_numpy(g.astype(np.float64).copy())
    total = torch.nn.utils.clip_grad_norm_([p], max_norm, norm_type=2.0, foreach=False)
    coef = float(p.grad[probe]) / float(g[probe])
    return float(total), coef


def _oracle_fin(acc: np.ndarray, k: int, max_norm: float, bf16: bool = False):
    """Oracle finalize for fp32 sums `acc` (multiples of 2^-24) with
    inv = 2^-k, so g = acc * 2^-k exactly."""
    inv64 = 2.0 ** -k
    if bf16:
        return oracle.finalize_bf16(oracle.sq_tree(acc.astype(np.float32)), False, inv64, max_norm)
    return oracle.finalize(oracle.exact_sq_units(acc.astype(np.float32)), False, inv64, max_norm)


def _exact_cases():
    out = []
    for vec, norm_int, probe in PYTHAGOREAN:
        for e in (-14, -10, -7, -4, 0, 3):
            k = 12
            acc = np.array(vec, dtype=np.float64) * 2.0 ** e
            norm = norm_int * 2.0 ** (e - k)
            # max_norm: the norm itself, 5e-7 and 2e-6 above it (the + 1e-6 decides
            # whether it clips), a third and three times it, 1e-7 below it
            for mx in (norm, norm + 5e-7, norm + 2e-6, norm / 3.0, norm * 3.0, norm - 1e-7):
                if mx > 0:
                    out.append((acc, k, mx, probe))
    return out


@pytest.mark.parametrize("bf16", [False, True])
def test_coefficient_equals_torch_on_exact_norms(bf16):
    n_clipped = n_eps_visible = 0
    for acc, k, mx, probe in _exact_cases():
        g = acc * 2.0 ** -k
        t_norm, t_coef = _torch_clip(g, mx, probe)
        fin = _oracle_fin(acc, k, mx, bf16)
        assert fin.norm == t_norm, (acc, k, mx)
        assert fin.coef == np.float32(t_coef), (acc, k, mx, fin.coef, t_coef)
        if t_coef < 1.0:
            n_clipped += 1
            if t_norm <= mx:  # the clamp alone would give 1; only + 1e-6 clips
                n_eps_visible += 1
    # the cases reach the clipped side, and cases where only + 1e-6 makes coef < 1
    assert n_clipped > 50 and n_eps_visible > 10


def test_eps_term_is_observable():
    """Without + 1e-6 these coefficients would differ in fp32: the pin is
    sensitive to the term it pins."""
    seen = 0
    for acc, k, mx, probe in _exact_cases():
        g = acc * 2.0 ** -k
        t_norm, t_coef = _torch_clip(g, mx, probe)
        no_eps = np.float32(min(1.0, mx / t_norm))
        if no_eps != np.float32(t_coef):
            seen += 1
            assert _oracle_fin(acc, k, mx).coef == np.float32(t_coef)
    assert seen > 100


@pytest.mark.parametrize("bf16", [False, True])
def test_coefficient_equals_torch_on_random_sums(bf16):
    """Random fp16-grid sums at norms 1e-5 .. 10: the fp32 coefficient equals
    torch's exactly; the norms agree within the fp64 summation bound (torch
    sums squares in floating point, the oracle exactly or by its tree)."""
    rng = np.random.default_rng(11)
    for trial in range(300):
        n = int(rng.integers(1, 3000))
        scale = 2.0 ** int(rng.integers(-20, 4))
        acc = (rng.standard_normal(n) * scale).astype(np.float16).astype(np.float64)
        acc[0] = 2.0 ** int(rng.integers(-14, 5))  # power-of-two probe element
        k = int(rng.integers(0, 24))
        g = acc * 2.0 ** -k
        exact = math.sqrt(math.fsum(x * x for x in g))
        mx = exact * float(rng.choice([0.25, 0.999999, 1.0, 1.0000005, 4.0]))
        mx = mx if rng.random() < 0.7 else float(rng.choice([1e-5, 1e-4, 1e-3, 1e-2, 1.0]))
        t_norm, t_coef = _torch_clip(g, mx, 0)
        fin = _oracle_fin(acc, k, mx, bf16)
        gamma = (n + 2) * 2.0 ** -53 / (1 - (n + 2) * 2.0 ** -53)
        assert abs(fin.norm - t_norm) <= gamma * exact + 1e-300, trial
        c32 = np.float32(t_coef)
        if fin.coef != c32:
            # only possible when the two norms straddle an fp32 rounding boundary of coef
            lo, hi = sorted((fin.norm, t_norm))
            c_hi, c_lo = mx / (lo + 1e-6), mx / (hi + 1e-6)
            assert np.float32(min(1.0, c_hi)) != np.float32(min(1.0, c_lo)), trial


def test_no_clipping_reading():
    """max_norm <= 0 turns clipping off (the DeepSpeed setting 0.0 disables
    it); torch has no such value, so this reading is stated, not pinned."""
    acc = np.array([3.0, 4.0])
    for mx in (0.0, -1.0):
        assert _oracle_fin(acc, 0, mx).coef == np.float32(1.0)
        assert _oracle_fin(acc, 0, mx, bf16=True).coef == np.float32(1.0)
