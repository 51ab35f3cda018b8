"""CPU model of the bf16 forward kernel's rule for raising its reference maximum.

The online softmax of "Describe Flash Attention at a high level"
(mantramindai.in), section "The two ideas", idea 2, keeps a running maximum per
query row and rescales the running sum and output whenever it rises. The fused
bf16 kernel instead keeps a *reference* maximum that it raises only when
needed: a 32-key sub-tile is accepted against the current reference if, for
every lane of the wave, the sum of the 16 probabilities that lane computed is
at most 256 (and finite); otherwise the wave takes the exact update (reference
raised to the row maximum, sum and output rescaled by exp2(m_old - m_new)) and
recomputes the sub-tile. Mathematically any reference gives the same output and
log-sum-exp, because the same one enters the output and the sum.

This model restates that rule in float64 (no bf16 rounding, whole waves of 32
query rows, the kernel's lane split of a sub-tile's keys) and checks against
the plain definition in ``oracle.attention`` that
  * output and LSE equal the definition to float64 rounding,
  * every probability that enters the sums is at most 256 (the bound the
    kernel relies on for fp32 range and bf16 representability),
  * the exact update fires on every wave's first sub-tile and rarely after.
"""
import math

import numpy as np
import pytest

import oracle

LIMIT = 256.0
LOG2E = 1.0 / math.log(2.0)


def lane_of_key():
    """Half (0 or 1) of the lane pair that holds each of a sub-tile's 32 keys.

    In the 32x32 MFMA accumulator, lane half hf holds the keys
    (r % 4) + 8 * (r // 4) + 4 * hf for r = 0..15.
    """
    half = np.empty(32, dtype=np.int64)
    for hf in range(2):
        for r in range(16):
            half[(r % 4) + 8 * (r // 4) + 4 * hf] = hf
    return half


def lazy_reference_attention(q, k, v, causal, scale):
    """One head, float64. Returns (O, LSE, updates, largest accepted probability, waves)."""
    N, _ = q.shape
    c2 = scale * LOG2E
    if not c2 >= np.finfo(np.float32).tiny:
        c2 = float(np.finfo(np.float32).tiny)
    half = lane_of_key()
    O = np.zeros_like(v[:N])
    lsum = np.zeros(N)
    m_ref = np.full(N, -np.inf)
    updates, pmax, waves = 0, 0.0, 0
    for w0 in range(0, N, 32):
        rows = np.arange(w0, min(w0 + 32, N))
        waves += 1
        n_sub = math.ceil((min(N, w0 + 32) if causal else N) / 32)
        for t in range(n_sub):
            keys = np.arange(32 * t, 32 * t + 32)
            s = q[rows] @ k[np.minimum(keys, N - 1)].T
            vis = keys[None, :] < N
            if causal:
                vis = vis & (keys[None, :] <= rows[:, None])
            s = np.where(vis, s, -np.inf)

            def probs():
                with np.errstate(invalid="ignore", over="ignore"):
                    return np.exp2(s * c2 - m_ref[rows, None] * c2)

            p = probs()
            with np.errstate(invalid="ignore"):
                lane_sums = np.stack([p[:, half == hf].sum(axis=1) for hf in range(2)])
            if not np.all(lane_sums <= LIMIT):  # NaN and inf fail this too
                m_new = np.maximum(m_ref[rows], s.max(axis=1))
                alpha = np.exp2((m_ref[rows] - m_new) * c2)
                lsum[rows] *= alpha
                O[rows] *= alpha[:, None]
                m_ref[rows] = m_new
                p = probs()
                updates += 1
            assert np.all(np.isfinite(p))
            pmax = max(pmax, float(p.max()))
            lsum[rows] += p.sum(axis=1)
            O[rows] += p @ v[np.minimum(keys, N - 1)]  # masked keys have p = 0
    O = O / lsum[:, None]
    lse = m_ref * scale + np.log(lsum)
    return O, lse, updates, pmax, waves


def head(seed, N, d, k_mult=1.0, q_mult=1.0):
    rng = np.random.default_rng([seed, N, d])
    q = rng.standard_normal((N, d)) * q_mult
    k = rng.standard_normal((N, d)) * k_mult
    v = rng.standard_normal((N, d))
    return q, k, v


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N,d,k_mult", [(1, 64, 1.0), (33, 64, 1.0), (300, 64, 1.0), (512, 128, 2.0), (700, 64, 1.0)])
def test_lazy_reference_equals_definition(N, d, k_mult, causal):
    q, k, v = head(11, N, d, k_mult)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    O, lse, updates, pmax, waves = lazy_reference_attention(q, k, v, causal, scale)
    O_ref, L_ref = oracle.attention(q[None, None], k[None, None], v[None, None], causal, scale)
    np.testing.assert_allclose(O, O_ref[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, L_ref[0, 0], rtol=0, atol=1e-12)
    assert pmax <= LIMIT
    assert updates >= waves  # every wave's first sub-tile sets the reference


def test_updates_are_rare_at_the_prefill_shape():
    """K x 2 (logit std 2, the gated workload's sharpening), d = 128, one head of 2048 rows."""
    N, d = 2048, 128
    q, k, v = head(3, N, d, k_mult=2.0)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    O, lse, updates, pmax, waves = lazy_reference_attention(q, k, v, True, scale)
    sub_tiles = sum(math.ceil(min(N, w0 + 32) / 32) for w0 in range(0, N, 32))
    O_ref, L_ref = oracle.attention(q[None, None], k[None, None], v[None, None], True, scale)
    np.testing.assert_allclose(O, O_ref[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, L_ref[0, 0], rtol=0, atol=1e-12)
    assert pmax <= LIMIT
    # beyond the first sub-tile of each wave, at most one sub-tile in ten takes the exact update
    assert updates - waves <= 0.1 * (sub_tiles - waves), (updates, waves, sub_tiles)


@pytest.mark.parametrize("q_mult", [4.0, 16.0])
def test_sharp_rows_take_the_exact_update_and_stay_exact(q_mult):
    """Logit std 4 and 16: the reference must rise often; the result stays the definition."""
    N, d = 256, 64
    q, k, v = head(5, N, d, q_mult=q_mult)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    for causal in (True, False):
        O, lse, updates, pmax, waves = lazy_reference_attention(q, k, v, causal, scale)
        O_ref, L_ref = oracle.attention(q[None, None], k[None, None], v[None, None], causal, scale)
        np.testing.assert_allclose(O, O_ref[0, 0], rtol=0, atol=1e-10)
        np.testing.assert_allclose(lse, L_ref[0, 0], rtol=1e-13, atol=1e-10)
        assert pmax <= LIMIT
        assert updates > waves


def test_scale_zero_gives_uniform_weights():
    """scale 0: the kernel floors the exp2 factor at FLT_MIN, every visible probability is ~1."""
    N, d = 100, 64
    q, k, v = head(7, N, d)
    O, lse, updates, pmax, waves = lazy_reference_attention(q, k, v, True, 0.0)
    expect = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(O, expect, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.log(np.arange(1, N + 1)), rtol=0, atol=1e-12)
    assert updates == waves


def test_a_dropped_rescale_is_caught():
    """The model's checks are sharp: skipping the rescale of the running output in the
    exact update (a plausible slip) moves the result far from the definition."""
    N, d = 256, 64
    q, k, v = head(9, N, d, q_mult=4.0)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    O_ref, _ = oracle.attention(q[None, None], k[None, None], v[None, None], True, scale)
    O, _, _, _, _ = lazy_reference_attention(q, k, v, True, scale)
    assert np.max(np.abs(O - O_ref[0, 0])) < 1e-12
    # the mutant: the same recurrence with O not scaled by alpha
    mutant = _mutant_without_output_rescale(q, k, v, True, scale)
    assert np.max(np.abs(mutant - O_ref[0, 0])) > 1e-3


def _mutant_without_output_rescale(q, k, v, causal, scale):
    N, _ = q.shape
    c2 = scale * LOG2E
    half = lane_of_key()
    O = np.zeros_like(v)
    lsum = np.zeros(N)
    m_ref = np.full(N, -np.inf)
    for w0 in range(0, N, 32):
        rows = np.arange(w0, min(w0 + 32, N))
        for t in range(math.ceil((min(N, w0 + 32) if causal else N) / 32)):
            keys = np.arange(32 * t, 32 * t + 32)
            s = q[rows] @ k[np.minimum(keys, N - 1)].T
            vis = (keys[None, :] < N) & ((keys[None, :] <= rows[:, None]) if causal else True)
            s = np.where(vis, s, -np.inf)
            with np.errstate(invalid="ignore", over="ignore"):
                p = np.exp2(s * c2 - m_ref[rows, None] * c2)
                lane_sums = np.stack([p[:, half == hf].sum(axis=1) for hf in range(2)])
            if not np.all(lane_sums <= LIMIT):
                m_new = np.maximum(m_ref[rows], s.max(axis=1))
                lsum[rows] *= np.exp2((m_ref[rows] - m_new) * c2)
                m_ref[rows] = m_new  # O is left unscaled: the planted mistake
                p = np.exp2(s * c2 - m_ref[rows, None] * c2)
            lsum[rows] += p.sum(axis=1)
            O[rows] += p @ v[np.minimum(keys, N - 1)]
    return O / lsum[:, None]
