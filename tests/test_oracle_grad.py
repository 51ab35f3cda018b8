"""Pins for the oracle's attention gradients (``oracle.attention_grad``).

The gradient formulas are not printed on the pages, so they are checked against
things other than themselves:
  * central finite differences of a scalar loss sum(O * G) through the pinned
    forward oracle, and through the pure-Python scalar forward (no numpy), on
    tiny inputs;
  * closed forms: a single key (dV = dO, dQ = dK = 0); scale 0 (dQ = dK = 0,
    dV_j = sum over the rows that see key j of dO_i / #visible(i));
  * invariants: sum over keys of dK is 0 (softmax rows sum to 1 for every
    logit shift), sum over keys of dV equals sum over queries of dO, a shift of
    every key by the same vector leaves all gradients unchanged, and a joint
    permutation of K/V rows permutes dK/dV and leaves dQ unchanged.
The mutation tests plant plausible mistakes in copies of the gradient and check
that the pins catch each one.
"""
import numpy as np
import pytest

import oracle
from oracle import core as oa
from test_oracle import brute_force, rnd


def loss_grad_fd(forward, q, k, v, g, eps=1e-6):
    """Central differences of L = sum(forward(q, k, v) * g) w.r.t. q, k and v."""
    out = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        grad = np.zeros_like(args[which])
        for idx in np.ndindex(*args[which].shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            grad[idx] = (np.sum(forward(*plus) * g) - np.sum(forward(*minus) * g)) / (2 * eps)
        out.append(grad)
    return out


# Pins parameterised by a head-level gradient function grad(q, k, v, do, causal, s) -> (dQ, dK, dV)

def pin_finite_differences(grad):
    for causal in (False, True):
        for (N, d, seed) in ((1, 2, 0), (4, 3, 1), (6, 2, 2)):
            q, k, v, g = rnd(seed, N, d), rnd(seed + 5, N, d), rnd(seed + 9, N, d), rnd(seed + 13, N, d)
            s = float(np.float32(0.8))
            fwd = lambda a, b, c: oa._head_attention(a, b, c, causal, s)[0]
            fd = loss_grad_fd(fwd, q, k, v, g)
            an = grad(q, k, v, g, causal, s)
            for x, y in zip(an, fd):
                if not np.allclose(x, y, rtol=0, atol=1e-7):
                    return False
    return True


def pin_fd_pure_python(grad):
    """The same check through the scalar pure-Python forward."""
    q, k, v, g = rnd(31, 5, 3), rnd(32, 5, 3), rnd(33, 5, 3), rnd(34, 5, 3)
    for causal in (False, True):
        fwd = lambda a, b, c: brute_force(a, b, c, causal, 0.45)[0]
        fd = loss_grad_fd(fwd, q, k, v, g)
        an = grad(q, k, v, g, causal, float(np.float32(0.45)))
        for x, y in zip(an, fd):
            if not np.allclose(x, y, rtol=0, atol=1e-7):
                return False
    return True


def pin_single_key(grad):
    q, k, v, g = rnd(40, 1, 4), rnd(41, 1, 4), rnd(42, 1, 4), rnd(43, 1, 4)
    dq, dk, dv = grad(q, k, v, g, True, 0.6)
    return np.allclose(dv, g, rtol=0, atol=1e-14) and not np.any(dq) and not np.any(dk)


def pin_scale_zero(grad):
    N, d = 9, 3
    q, k, v, g = rnd(44, N, d), rnd(45, N, d), rnd(46, N, d), rnd(47, N, d)
    for causal in (False, True):
        dq, dk, dv = grad(q, k, v, g, causal, 0.0)
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        w = g / cnt[:, None]                                   # dO_i / #visible(i)
        exp_dv = np.cumsum(w[::-1], axis=0)[::-1] if causal else np.repeat(w.sum(0, keepdims=True), N, 0)
        if np.any(dq) or np.any(dk) or not np.allclose(dv, exp_dv, rtol=0, atol=1e-12):
            return False
    return True


def pin_sums(grad):
    q, k, v, g = rnd(48, 11, 4), rnd(49, 11, 4), rnd(50, 11, 4), rnd(51, 11, 4)
    for causal in (False, True):
        dq, dk, dv = grad(q, k, v, g, causal, 0.7)
        if not (np.allclose(dk.sum(0), 0, rtol=0, atol=1e-12) and np.allclose(dv.sum(0), g.sum(0), rtol=0, atol=1e-12)):
            return False
    return True


def pin_key_shift(grad):
    q, k, v, g = rnd(52, 8, 5), rnd(53, 8, 5), rnd(54, 8, 5), rnd(55, 8, 5)
    u = rnd(56, 5)
    for causal in (False, True):
        a = grad(q, k, v, g, causal, 0.5)
        b = grad(q, k + u[None, :], v, g, causal, 0.5)
        if not all(np.allclose(x, y, rtol=0, atol=1e-11) for x, y in zip(a, b)):
            return False
    return True


def pin_kv_permutation(grad):
    q, k, v, g = rnd(57, 7, 3), rnd(58, 7, 3), rnd(59, 7, 3), rnd(60, 7, 3)
    perm = np.random.default_rng(61).permutation(7)
    dq, dk, dv = grad(q, k, v, g, False, 0.9)
    dq2, dk2, dv2 = grad(q, k[perm], v[perm], g, False, 0.9)
    return (np.allclose(dq, dq2, rtol=0, atol=1e-12) and np.allclose(dk[perm], dk2, rtol=0, atol=1e-12)
            and np.allclose(dv[perm], dv2, rtol=0, atol=1e-12))


PINS = [pin_finite_differences, pin_fd_pure_python, pin_single_key, pin_scale_zero, pin_sums, pin_key_shift,
        pin_kv_permutation]


def _oracle_grad(q, k, v, do, causal, s):
    return oa._head_attention_grad(q, k, v, do, causal, s)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_grad_pins(pin):
    assert pin(_oracle_grad)


def test_batched_matches_head():
    q, k, v, g = (rnd(70 + i, 2, 3, 10, 4) for i in range(4))
    dq, dk, dv = oracle.attention_grad(q, k, v, g, True, 0.3)
    for b in range(2):
        for h in range(3):
            ref = oa._head_attention_grad(q[b, h], k[b, h], v[b, h], g[b, h], True, float(np.float32(0.3)))
            for x, y in zip((dq[b, h], dk[b, h], dv[b, h]), ref):
                assert np.array_equal(x, y)


# ---- mutation tests: plausible mistakes in copies of the gradient ----

def _mutant(kind):
    def grad(q, k, v, do, causal, s):
        _, _, P = oa._head_attention(q, k, v, causal, s)
        dV = P @ do if kind == "dv_untransposed" else P.T @ do
        dP = do @ v.T
        if kind == "d_colsum":
            D = np.sum(dP * P, axis=0, keepdims=True)
        else:
            D = np.sum(dP * P, axis=1, keepdims=True)
        dS = P * dP if kind == "no_d" else P * (dP - D)
        if kind == "ds_sign":
            dS = -dS
        dQ = (dS.T @ k) if kind == "dq_transposed" else (dS @ k)
        dQ = dQ if kind == "dq_no_scale" else s * dQ
        dK = s * (dS.T @ (k if kind == "dk_uses_k" else q))
        if kind == "dk_scale_squared":
            dK = s * dK
        return dQ, dK, dV
    return grad


MUTANTS = ["dv_untransposed", "d_colsum", "no_d", "ds_sign", "dq_transposed", "dq_no_scale", "dk_uses_k",
           "dk_scale_squared"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    caught = [p.__name__ for p in PINS if not p(_mutant(kind))]
    assert len(caught) >= 2, f"fewer than two pins catch the mistake {kind}: {caught}"


def test_unmutated_copy_passes():
    assert all(p(_mutant("none")) for p in PINS)
