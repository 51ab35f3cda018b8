"""Pins for the CPU oracle: it is checked against things other than itself.

Every pin is written from the mathematics or from figures the pages print:
  * brute force: a pure-Python scalar loop (math.exp / math.fsum, no numpy)
    on tiny inputs;
  * softmax rows sum to 1;
  * closed forms: a single key (O = V_0), identical keys (O = mean of the
    visible V rows), scale 0 (prefix means, LSE = ln(#visible));
  * invariances: a per-row logit shift leaves O unchanged and moves LSE by the
    shift; permuting K/V rows jointly leaves O unchanged; permuting Q rows
    permutes the outputs;
  * the streaming recurrence equals the definition over many block sizes,
    and on the worked example a page prints;
  * split-KV decode is independent of the split count and equals the last
    row of a causal prefill.
The mutation tests at the end plant plausible mistakes in copies of the
oracle's head function and check that at least one pin catches each.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import core as oa


def brute_force(q, k, v, causal, scale):
    """Pure-Python scalar attention (no numpy arithmetic)."""
    s = float(np.float32(scale))
    q, k, v = q.tolist(), k.tolist(), v.tolist()
    O, L = [], []
    for i, qi in enumerate(q):
        vis = [j for j in range(len(k)) if not causal or j <= i]
        logits = [s * math.fsum(a * b for a, b in zip(qi, k[j])) for j in vis]
        mx = max(logits)
        ex = [math.exp(x - mx) for x in logits]
        den = math.fsum(ex)
        O.append([math.fsum(e * v[j][c] for e, j in zip(ex, vis)) / den for c in range(len(v[0]))])
        L.append(mx + math.log(den))
    return np.array(O), np.array(L)


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------------------
# Pin suite, parameterised by the head function so the mutation tests can reuse it.
# head(q, k, v, causal, s, rows) -> (O, LSE, P) for one head.
# --------------------------------------------------------------------------------------

def pin_brute_force(head):
    for causal in (False, True):
        for (N, d, seed) in ((1, 1, 0), (3, 2, 1), (6, 3, 2), (8, 4, 3)):
            q, k, v = rnd(seed, N, d), rnd(seed + 10, N, d), rnd(seed + 20, N, d)
            O, L, _ = head(q, k, v, causal, 0.7, None)
            Ob, Lb = brute_force(q, k, v, causal, 0.7)
            if not (np.allclose(O, Ob, rtol=0, atol=1e-12) and np.allclose(L, Lb, rtol=0, atol=1e-12)):
                return False
    return True


def pin_rows_sum_to_one(head):
    for causal in (False, True):
        q, k = rnd(4, 33, 8), rnd(5, 33, 8)
        P = head(q, k, np.zeros((33, 1)), causal, 0.35, None)[2]
        if not np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12):
            return False
        if causal and not np.all(np.triu(P, 1) == 0):
            return False
    return True


def pin_single_key(head):
    q, k, v = rnd(6, 1, 5), rnd(7, 1, 5), rnd(8, 1, 5)
    s = float(np.float32(0.3))
    O, L, _ = head(q, k, v, True, 0.3, None)
    return np.array_equal(O, v) and abs(L[0] - s * float(q[0] @ k[0])) < 1e-12


def pin_identical_keys(head):
    N, d = 9, 4
    q, v = rnd(9, N, d), rnd(10, N, d)
    k = np.repeat(rnd(11, 1, d), N, axis=0)
    s = float(np.float32(0.5))
    for causal in (False, True):
        O, L, _ = head(q, k, v, causal, 0.5, None)
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        mean = np.cumsum(v, axis=0) / cnt[:, None] if causal else np.repeat(v.mean(axis=0, keepdims=True), N, 0)
        lse = s * (q @ k[0]) + np.log(cnt)
        if not (np.allclose(O, mean, rtol=0, atol=1e-12) and np.allclose(L, lse, rtol=0, atol=1e-12)):
            return False
    return True


def pin_scale_zero(head):
    N, d = 12, 3
    q, k, v = rnd(12, N, d), rnd(13, N, d), rnd(14, N, d)
    Oc, Lc, _ = head(q, k, v, True, 0.0, None)
    On, Ln, _ = head(q, k, v, False, 0.0, None)
    idx = np.arange(1, N + 1)
    return (np.allclose(Oc, np.cumsum(v, 0) / idx[:, None], rtol=0, atol=1e-12)
            and np.allclose(Lc, np.log(idx), rtol=0, atol=1e-12)
            and np.allclose(On, np.repeat(v.mean(0, keepdims=True), N, 0), rtol=0, atol=1e-12)
            and np.allclose(Ln, np.log(N), rtol=0, atol=1e-12))


def pin_shift_invariance(head):
    N, d = 10, 4
    q, k, v = rnd(15, N, d), rnd(16, N, d), rnd(17, N, d)
    u = rnd(18, d)
    s = float(np.float32(0.6))
    for causal in (False, True):
        O, L, _ = head(q, k, v, causal, 0.6, None)
        O2, L2, _ = head(q, k + u[None, :], v, causal, 0.6, None)
        if not (np.allclose(O, O2, rtol=0, atol=1e-12) and np.allclose(L2 - L, s * (q @ u), rtol=0, atol=1e-12)):
            return False
    return True


def pin_permutation(head):
    N, d = 11, 4
    q, k, v = rnd(19, N, d), rnd(20, N, d), rnd(21, N, d)
    perm = np.random.default_rng(22).permutation(N)
    O, L, _ = head(q, k, v, False, 0.45, None)
    O2, L2, _ = head(q, k[perm], v[perm], False, 0.45, None)
    O3, L3, _ = head(q[perm], k, v, False, 0.45, None)
    return (np.allclose(O, O2, rtol=0, atol=1e-12) and np.allclose(L, L2, rtol=0, atol=1e-12)
            and np.allclose(O3, O[perm], rtol=0, atol=1e-12) and np.allclose(L3, L[perm], rtol=0, atol=1e-12))


def pin_rows_subset(head):
    N, d = 14, 4
    q, k, v = rnd(23, N, d), rnd(24, N, d), rnd(25, N, d)
    rows = [0, 5, 13]
    for causal in (False, True):
        O, L, _ = head(q, k, v, causal, 0.4, None)
        Or, Lr, _ = head(q, k, v, causal, 0.4, rows)
        if not (np.allclose(Or, O[rows], rtol=0, atol=1e-12) and np.allclose(Lr, L[rows], rtol=0, atol=1e-12)):
            return False
    return True


def _f32_scale(head):
    """The head functions take the float64 multiplier itself; pins state scales as float32 values."""
    return lambda q, k, v, causal, s, rows: head(q, k, v, causal, float(np.float32(s)), rows)


PINS = [pin_brute_force, pin_rows_sum_to_one, pin_single_key, pin_identical_keys, pin_scale_zero,
        pin_shift_invariance, pin_permutation, pin_rows_subset]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_head_pins(pin):
    assert pin(_f32_scale(oa._head_attention))


def test_attention_batched_matches_head():
    B, H, N, d = 2, 3, 7, 4
    q, k, v = rnd(30, B, H, N, d), rnd(31, B, H, N, d), rnd(32, B, H, N, d)
    O, L = oracle.attention(q, k, v, True, 0.25)
    for b in range(B):
        for h in range(H):
            Ob, Lb = brute_force(q[b, h], k[b, h], v[b, h], True, 0.25)
            np.testing.assert_allclose(O[b, h], Ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(L[b, h], Lb, rtol=0, atol=1e-12)
    # head subset leaves the others untouched (NaN)
    O2, _ = oracle.attention(q, k, v, True, 0.25, heads=[(1, 2)])
    np.testing.assert_array_equal(O2[1, 2], O[1, 2])
    assert np.isnan(O2[0, 0]).all()


# --------------------------------------------------------------------------------------
# Streaming recurrence and decode
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 2, 3, 5, 16, 37])
def test_online_recurrence_equals_definition(causal, block):
    N, d = 37, 6
    q, k, v = rnd(40, N, d), rnd(41, N, d) * 2.0, rnd(42, N, d)
    O, L = oracle.online_attention(q, k, v, causal, 0.4, block)
    Ob, Lb = brute_force(q, k, v, causal, 0.4)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


def test_pages_streaming_example(golden_dir):
    """The worked example of the online recurrence that a page prints (8 keys, d=4, blocks of 2)."""
    g = json.load(open(os.path.join(golden_dir, "streaming_example.json")))
    rng = np.random.default_rng(g["seed"])
    T, d = g["T"], g["d"]
    q = rng.normal(size=d)
    K, V = rng.normal(size=(T, d)), rng.normal(size=(T, d))
    scale = 1.0 / math.sqrt(d)             # 0.5, exact in float32
    o_def, lse_def = oracle.decode(q[None, None, :], K[None, None], V[None, None], scale)
    o_str, lse_str = oracle.online_attention(q[None, :], K, V, False, scale, g["block"])
    assert bool(np.allclose(o_def[0, 0], o_str[0])) == g["expected_allclose"]
    assert np.max(np.abs(o_def[0, 0] - o_str[0])) < 1e-14
    ob, lb = brute_force(q[None, :], K, V, False, scale)
    np.testing.assert_allclose(o_def[0, 0], ob[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse_def[0, 0], lb[0], rtol=0, atol=1e-14)


@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 64, 100, 1000])
def test_split_decode_independent_of_nsplit(nsplit):
    L, d = 100, 8
    q, kc, vc = rnd(50, d), rnd(51, L, d) * 2.0, rnd(52, L, d)
    o, lse = oracle.split_decode(q, kc, vc, nsplit)
    od, lsed = oracle.decode(q[None, None], kc[None, None], vc[None, None])
    ob, lb = brute_force(q[None, :], kc, vc, False, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(od[0, 0], ob[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lsed[0, 0], lb[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, od[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lsed[0, 0], rtol=0, atol=1e-12)


def test_decode_equals_last_row_of_causal_prefill():
    N, d = 29, 8
    q, k, v = rnd(60, 1, 1, N, d), rnd(61, 1, 1, N, d), rnd(62, 1, 1, N, d)
    scale = 1.0 / math.sqrt(d)
    O, L = oracle.attention(q, k, v, True, scale)
    o, lse = oracle.decode(q[:, :, N - 1, :], k, v)
    np.testing.assert_allclose(o[0, 0], O[0, 0, N - 1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], L[0, 0, N - 1], rtol=0, atol=1e-12)


def test_decode_permutation_of_cache():
    L, d = 77, 8
    q, kc, vc = rnd(63, d), rnd(64, L, d), rnd(65, L, d)
    perm = np.random.default_rng(66).permutation(L)
    o1, l1 = oracle.split_decode(q, kc, vc, 7)
    o2, l2 = oracle.split_decode(q, kc[perm], vc[perm], 7)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------
# Figures the pages print
# --------------------------------------------------------------------------------------

def test_pages_score_matrix_sizes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "pages_figures.json")))
    for key in ("score_matrix_t8192", "score_matrix_t16384"):
        e = g[key]
        per_head = oracle.naive_workspace_bytes(1, 1, e["T"], e["elem_bytes"])
        all_heads = oracle.naive_workspace_bytes(1, e["heads"], e["T"], e["elem_bytes"])
        # the pages round: 134 MB (decimal) per head at 8K; 512 MB (binary MiB) per head at 16K
        assert round(per_head / 1e6) == e["bytes_per_head_MB"] or round(per_head / 2**20) == e["bytes_per_head_MB"]
        assert abs(all_heads / 1e9 - e["bytes_all_heads_GB"]) / e["bytes_all_heads_GB"] < 0.08 or \
            round(all_heads / 2**30) == e["bytes_all_heads_GB"]
    e = g["score_entries_n4000"]
    assert round(oracle.naive_workspace_bytes(1, 1, e["N"], 1) / 1e6) == e["entries_per_head_million"]


def test_flop_count():
    # 4*d per visible pair: count the visible pairs of the causal mask directly on small sizes
    for N in (1, 2, 7, 64, 65):
        visible = int(np.tril(np.ones((N, N), dtype=bool)).sum())
        assert oracle.attention_flops(2, 3, N, 16, True) == 4 * 16 * 6 * visible
        assert oracle.attention_flops(2, 3, N, 16, False) == 4 * 16 * 6 * N * N
    assert oracle.attention_flops(1, 32, 8192, 128, True) == 549_822_922_752
    assert oracle.attention_flops(1, 1, 256, 64, False) == 16_777_216
    assert oracle.attention_flops(4, 16, 1024, 64, True) == 8_598_323_200


# --------------------------------------------------------------------------------------
# Mutation tests: plausible mistakes planted in copies of the oracle's head function.
# --------------------------------------------------------------------------------------

def _mutant(kind):
    def head(q, k, v, causal, s, rows):
        qi = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        if kind == "transposed_scores":
            S = s * (k @ q.T)[qi] if k.shape[0] == q.shape[0] else s * (q[qi] @ k.T)
        elif kind == "scale_dropped":
            S = q[qi] @ k.T
        elif kind == "scale_squared":
            S = s * s * (q[qi] @ k.T)
        else:
            S = s * (q[qi] @ k.T)
        if causal:
            j = np.arange(k.shape[0])[None, :]
            i = qi[:, None]
            if kind == "mask_flipped":
                S = np.where(j < i, -np.inf, S)
            elif kind == "mask_diag_excluded":
                S = np.where(j >= i, -np.inf, S)
            else:
                S = np.where(j > i, -np.inf, S)
        axis = 0 if kind == "softmax_wrong_axis" else 1
        m = S.max(axis=axis, keepdims=True)
        P = np.exp(S - m)
        l = P.sum(axis=axis, keepdims=True)
        if kind != "not_normalised":
            P = P / l
        O = P @ (k if kind == "multiplies_k" else v)
        if axis == 0:
            m, l = m.T, l.T
        lse = (np.log(l[:, 0]) if kind == "lse_without_max" else m[:, 0] + np.log(l[:, 0]))
        if kind == "lse_log2":
            lse = m[:, 0] + np.log2(l[:, 0])
        return O, lse, P
    return head


MUTANTS = ["transposed_scores", "scale_dropped", "scale_squared", "mask_flipped", "mask_diag_excluded",
           "softmax_wrong_axis", "not_normalised", "multiplies_k", "lse_without_max", "lse_log2"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    head = _f32_scale(_mutant(kind))
    failed = [p.__name__ for p in PINS if not _safe(p, head)]
    assert len(failed) >= 3, f"fewer than three pins caught the planted mistake {kind}: {failed}"


def _safe(pin, head):
    with np.errstate(all="ignore"):
        try:
            return bool(pin(head))
        except Exception:
            return False


def test_unmutated_copy_passes_all_pins():
    head = _f32_scale(_mutant("none"))
    assert all(_safe(p, head) for p in PINS)


def test_online_mutants_caught():
    """A streaming fold whose merge forgets to shrink the old sum (or the old output) when the
    running maximum rises disagrees with brute force; the correct merge agrees."""
    N, d = 20, 4
    q, k, v = rnd(70, N, d), rnd(71, N, d) * 3, rnd(72, N, d)
    Ob, _ = brute_force(q, k, v, False, 0.5)

    def fold(shrink_l, shrink_o):
        m, l, o = np.full(N, -np.inf), np.zeros(N), np.zeros((N, d))
        for st in range(0, N, 3):
            S = 0.5 * (q @ k[st:st + 3].T)
            mb = S.max(axis=1)
            P = np.exp(S - mb[:, None])
            M = np.maximum(m, mb)
            a, b = np.exp(m - M), np.exp(mb - M)           # exp(-inf) = 0 on the first block
            l = (a * l if shrink_l else l) + b * P.sum(axis=1)
            o = (a[:, None] * o if shrink_o else o) + b[:, None] * (P @ v[st:st + 3])
            m = M
        return o / l[:, None]

    assert np.allclose(fold(True, True), Ob, atol=1e-12)
    assert not np.allclose(fold(False, True), Ob, atol=1e-6)
    assert not np.allclose(fold(True, False), Ob, atol=1e-6)


def test_online_block_partial_and_merge_special_cases():
    """A block with no visible key for a row is the empty partial (-inf, 0, 0) and merging it changes
    nothing; merging is symmetric; a single block's partial normalised is that block's softmax."""
    S = np.array([[0.3, -np.inf, 1.2], [-np.inf, -np.inf, -np.inf]])
    v = rnd(80, 3, 2)
    m, l, o = oa._block_partial(S, v)
    assert m[1] == -np.inf and l[1] == 0 and not o[1].any()
    p = np.exp(S[0] - 1.2)
    np.testing.assert_allclose(o[0] / l[0], (p / p.sum()) @ v, rtol=0, atol=1e-15)
    other = oa._block_partial(np.array([[2.0, 0.1], [0.5, -1.0]]), rnd(81, 2, 2))
    ab, ba = oa._merge((m, l, o), other), oa._merge(other, (m, l, o))
    for x, y in zip(ab, ba):
        np.testing.assert_allclose(x, y, rtol=1e-15, atol=0)
    np.testing.assert_array_equal(oa._merge(other, (np.full(2, -np.inf), np.zeros(2), np.zeros((2, 2))))[2],
                                  other[2])
