"""Pins for the oracle's paged decode (``oracle.paged_decode``) and for the
paged-cache generator.

The gather is checked against things other than itself:
  * layout identity: a pool made by reshaping contiguous caches (with the
    identity block table) gives exactly ``decode`` of those caches;
  * truncation: with ragged lengths and NaN in every pool row that holds no
    key, the result equals ``decode`` over the first seq_lens[b] keys of the
    contiguous caches, and stays finite;
  * a shuffled pool (page ids permuted, the table remapped) gives the
    identical result;
  * brute force: a pure-Python loop with explicit page lookups on tiny inputs;
  * closed forms: one key (o = that key's V row, lse = s q.k), length 0
    (o = 0, lse = -inf), page size 1 and a single page per sequence.
The mutation tests plant plausible gather mistakes in copies and check that a
pin catches each.
"""
import math

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from oracle import core as oa


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def identity_pool(c, ps):
    """[B,H,L,d] with L a multiple of ps -> pool [B*L/ps, H, ps, d] and the identity table."""
    B, H, L, d = c.shape
    P = L // ps
    pool = c.reshape(B, H, P, ps, d).transpose(0, 2, 1, 3, 4).reshape(B * P, H, ps, d)
    return pool, np.arange(B * P, dtype=np.int32).reshape(B, P)


def brute_paged(q, kp, vp, table, lens, scale):
    """Pure-Python scalar decode with explicit page lookups (no numpy arithmetic)."""
    s = float(np.float32(scale))
    ps = kp.shape[2]
    B, H, _ = q.shape
    out = np.zeros(q.shape[:2] + (vp.shape[-1],))
    for b in range(B):
        for h in range(H):
            keys = [(int(table[b][j // ps]), j % ps) for j in range(int(lens[b]))]
            if not keys:
                continue
            qv = q[b][h].tolist()
            logits = [s * math.fsum(a * x for a, x in zip(qv, kp[pg][h][r].tolist())) for pg, r in keys]
            mx = max(logits)
            ex = [math.exp(t - mx) for t in logits]
            den = math.fsum(ex)
            for c in range(vp.shape[-1]):
                out[b, h, c] = math.fsum(e * float(vp[pg][h][r][c]) for e, (pg, r) in zip(ex, keys)) / den
    return out


# Pins parameterised by f(q, k_pages, v_pages, block_table, seq_lens, scale) -> (o, lse).

def pin_layout_identity(f):
    for ps in (1, 4, 16):
        c_k, c_v, q = rnd(1, 2, 3, 32, 8), rnd(2, 2, 3, 32, 8), rnd(3, 2, 3, 8)
        kp, table = identity_pool(c_k, ps)
        vp, _ = identity_pool(c_v, ps)
        o, lse = f(q, kp, vp, table, np.full(2, 32), None)
        ro, rl = oracle.decode(q, c_k, c_v)
        if not (np.array_equal(o, ro) and np.array_equal(lse, rl)):
            return False
    return True


def pin_truncation_ignores_unused_rows(f):
    for ps in (1, 3, 8):
        q, k, v = si.random_case(40 + ps, 5, 2, 1, 8, "f32", nk=29)
        lens = si.seq_lengths(ps, 5, 29, ps)
        kp, vp, table, lens = si.page_cache(ps, k, v, lens, ps)
        o, _ = f(q[:, :, 0], kp, vp, table, lens, None)
        if not np.isfinite(o).all():
            return False
        for b in range(5):
            ro, _ = oracle.decode(q[b:b + 1, :, 0], k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]])
            if not np.array_equal(o[b:b + 1], ro):
                return False
    return True


def pin_pool_permutation(f):
    q, k, v = si.random_case(50, 3, 2, 1, 4, "f32", nk=21)
    kp, vp, table, lens = si.page_cache(50, k, v, np.array([21, 5, 13]), 4)
    perm = np.random.default_rng(51).permutation(kp.shape[0])
    inv = np.argsort(perm)
    table2 = np.where(table >= 0, inv[np.maximum(table, 0)], -1)
    a = f(q[:, :, 0], kp, vp, table, lens, None)
    b = f(q[:, :, 0], kp[perm], vp[perm], table2, lens, None)
    return all(np.array_equal(x, y) for x, y in zip(a, b))


def pin_brute_force(f):
    q, k, v = si.random_case(60, 3, 2, 1, 3, "f32", nk=7)
    for ps in (2, 3):
        kp, vp, table, lens = si.page_cache(60 + ps, k, v, np.array([7, 1, 4]), ps)
        o, _ = f(q[:, :, 0], kp, vp, table, lens, 0.6)
        if not np.allclose(o, brute_paged(q[:, :, 0], kp, vp, table, lens, 0.6), rtol=0, atol=1e-12):
            return False
    return True


def pin_single_key_and_empty(f):
    q, k, v = si.random_case(70, 3, 2, 1, 8, "f32", nk=9)
    kp, vp, table, lens = si.page_cache(70, k, v, np.array([1, 0, 9]), 4)
    o, lse = f(q[:, :, 0], kp, vp, table, lens, 0.5)
    s = float(np.float32(0.5))
    qk = np.sum(q[0, :, 0].astype(np.float64) * k[0, :, 0].astype(np.float64), -1)
    ok = np.array_equal(o[0], v[0, :, 0]) and np.allclose(lse[0], s * qk, rtol=0, atol=1e-12)
    return ok and not o[1].any() and np.all(lse[1] == -np.inf) and np.isfinite(o[2]).all()


def pin_single_page(f):
    """Page size >= every length: each sequence is one page, which is its contiguous cache."""
    q, k, v = rnd(80, 2, 2, 4), rnd(81, 2, 2, 16, 4), rnd(82, 2, 2, 16, 4)
    kp, vp = k, v                                              # pool page b = sequence b, [H, 16, d]
    o, _ = f(q, kp, vp, np.array([[1], [0]]), np.array([11, 16]), None)
    r0, _ = oracle.decode(q[:1], k[1:2, :, :11], v[1:2, :, :11])
    r1, _ = oracle.decode(q[1:], k[:1], v[:1])
    return np.array_equal(o[:1], r0) and np.array_equal(o[1:], r1)


PINS = [pin_layout_identity, pin_truncation_ignores_unused_rows, pin_pool_permutation, pin_brute_force,
        pin_single_key_and_empty, pin_single_page]


def _oracle(q, kp, vp, table, lens, scale):
    return oracle.paged_decode(q, kp, vp, table, lens, scale)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_paged_pins(pin):
    assert pin(_oracle)


def test_invalid_tables_rejected():
    kp = np.zeros((4, 1, 2, 3))
    q = np.zeros((1, 1, 3))
    with pytest.raises(ValueError):
        oracle.paged_decode(q, kp, kp, np.array([[0, 9]]), np.array([4]))      # page id outside the pool
    with pytest.raises(ValueError):
        oracle.paged_decode(q, kp, kp, np.array([[0, -1]]), np.array([3]))     # unused-entry marker read
    with pytest.raises(ValueError):
        oracle.paged_decode(q, kp, kp, np.array([[0, 1]]), np.array([5]))      # length beyond the table
    with pytest.raises(ValueError):
        oracle.paged_decode(q, kp, kp, np.array([[0, 1]]), np.array([-1]))


def test_generator_layout():
    """page_cache: every key lands where the table says, nothing else is finite, unused entries are -1."""
    B, H, L, d, ps = 4, 3, 23, 5, 4
    k = np.arange(B * H * L * d, dtype=np.float32).reshape(B, H, L, d)
    lens = si.seq_lengths(9, B, L, ps)
    kp, vp, table, lens2 = si.page_cache(9, k, k + 0.5, lens, ps)
    assert np.array_equal(lens, lens2) and list(lens[:4]) == [1, 3, 4, 5]
    assert kp.shape == (sum(-(-int(n) // ps) for n in lens) + 3, H, ps, d) and table.shape == (B, 6)
    seen = np.zeros(kp.shape[:3], dtype=bool)
    for b in range(B):
        for j in range(lens[b]):
            pg, r = table[b, j // ps], j % ps
            assert np.array_equal(kp[pg, :, r], k[b, :, j]) and np.array_equal(vp[pg, :, r], k[b, :, j] + 0.5)
            seen[pg, :, r] = True
        assert (table[b, -(-int(lens[b]) // ps):] == -1).all()
    assert np.isnan(kp[~seen]).all() and np.isnan(vp[~seen]).all()
    assert sorted(table[table >= 0].tolist()) == sorted(set(table[table >= 0].tolist()))   # no page used twice


def test_generator_bf16_filler_and_determinism():
    q, k, v = si.random_case(3, 2, 2, 1, 8, "bf16", nk=10)
    a = si.page_cache(3, k, v, np.array([10, 3]), 4)
    b = si.page_cache(3, k, v, np.array([10, 3]), 4)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert a[0].dtype == np.uint16 and (a[0] == si.BF16_NAN_BITS).any()
    assert np.isnan(si.as_float64(a[0], "bf16")).any()


# ---- mutation tests: plausible gather mistakes in copies of the oracle ----

def _mutant(kind):
    def gather(pool, row, length):
        num_pages, H, ps, d = pool.shape
        n_used = length // ps if kind == "floor_pages" else -(-length // ps)
        out = np.empty((H, length, d))
        for i in range(n_used):
            page = int(row[i])
            rows = min(ps, length - i * ps)
            src = pool[page].reshape(ps, H, d).transpose(1, 0, 2) if kind == "token_major_pool" else pool[page]
            if kind == "offset_off_by_one":
                src = np.roll(src, -1, axis=1)
            if kind == "tail_from_end" and rows < ps:
                out[:, i * ps:i * ps + rows] = src[:, ps - rows:]
            else:
                out[:, i * ps:i * ps + rows] = src[:, :rows]
        if kind == "floor_pages":
            out[:, n_used * ps:] = 0.0
        return out

    def f(q, kp, vp, table, lens, scale):
        B, H, d = q.shape
        o, lse = np.zeros((B, H, vp.shape[-1])), np.full((B, H), -np.inf)
        tab = np.asarray(table).T.reshape(np.shape(table)) if kind == "table_transposed" else np.asarray(table)
        for b in range(B):
            n = int(lens[b])
            if kind == "ignore_lengths":
                n = -(-n // kp.shape[2]) * kp.shape[2]
            if n == 0:
                continue
            kc, vc = gather(kp, tab[b], n)[None], gather(vp, tab[b], n)[None]
            sc = 1.0 if kind == "no_scale" else scale
            o[b:b + 1], lse[b:b + 1] = oracle.decode(q[b:b + 1], kc, vc, sc)
        return o, lse
    return f


MUTANTS = ["floor_pages", "token_major_pool", "offset_off_by_one", "tail_from_end", "table_transposed",
           "ignore_lengths", "no_scale"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    caught = []
    for p in PINS:
        try:
            ok = p(_mutant(kind))
        except (IndexError, ValueError):
            ok = False
        if not ok:
            caught.append(p.__name__)
    assert len(caught) >= 4, f"fewer than four pins catch the mistake {kind}: {caught}"


def test_unmutated_copy_passes():
    assert all(p(_mutant("none")) for p in PINS)


def test_gather_is_the_oracle_step():
    """The module-level gather is the one paged_decode uses (no second copy)."""
    pool = rnd(90, 3, 2, 4, 5)
    g = oa.gather_pages(pool, np.array([2, 0]), 6)
    assert np.array_equal(g[:, :4], pool[2]) and np.array_equal(g[:, 4:], pool[0, :, :2])
