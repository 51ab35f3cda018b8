"""CPU model of the tiles, sub-tiles and split ranges the kernels visit.

Each model restates one kernel's loop bounds and mask decisions (the integer
logic only, no arithmetic) and checks, over ragged sizes and both causal
settings, that
  * every visible (query, key) pair is computed exactly once,
  * every piece of work the kernel runs without a mask holds only visible
    pairs (so skipping the mask there is safe),
  * every piece of work the kernel scores lies inside the tiles it loaded,
  * the work spent on masked pairs stays small.
The decode split shape is checked against the library's own arithmetic
through fa_decode_workspace_bytes (no GPU needed).
"""
import math

import numpy as np
import pytest

from exact_io_aware_74_amd import binding

SIZES = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 511, 512, 513, 700, 1000]


def visible(N, causal):
    v = np.ones((N, N), dtype=bool)
    return np.tril(v) if causal else v


def check_cover(cover, N, causal):
    np.testing.assert_array_equal(cover, visible(N, causal).astype(np.int64))


def fwd_bf16_model(N, causal, NW=8):
    """fwd_bf16_kernel with NW waves of 32 query rows per workgroup (8: 256-row workgroups; 4: the
    128-row ones taken at d = 64 for small grids), 64-key tiles, 32-key sub-tiles; row block b sits
    on wave b for b < NW/2 and on wave 3NW/2 - 1 - b otherwise; sub-tiles 1 .. 2*j_clean are scored
    in the unmasked loop. Also checks the copy ring: every tile a wave reads during tile iteration j
    (tiles j and j + 1) was published by a barrier before that iteration, and a slot is rewritten
    only after a barrier that follows every read of its previous tile."""
    BR, BC = 32 * NW, 64
    cover = np.zeros((N, N), dtype=np.int64)
    scored = 0
    for qt in range(math.ceil(N / BR)):
        q0 = qt * BR
        kv_end = min(N, q0 + BR) if causal else N
        n_kt = math.ceil(kv_end / BC)
        ring_protocol(n_kt)
        blocks = sorted(w if w < NW // 2 else 3 * NW // 2 - 1 - w for w in range(NW))
        assert blocks == list(range(NW))          # the wave -> row block map is a permutation
        for w in range(NW):
            rb = w if w < NW // 2 else 3 * NW // 2 - 1 - w
            wq0 = q0 + 32 * rb
            wv_end = min(N, wq0 + 32) if causal else N
            n_st = math.ceil(wv_end / 32) if wq0 < N else 0
            assert n_st <= 2 * n_kt
            n_clean = min((wq0 + 1) // 32 if causal else N // 32, N // 32)
            j_clean = max(0, (n_clean - 1) // 2)
            r0, r1 = wq0, min(wq0 + 32, N)
            for t in range(n_st):
                k0, k1 = 32 * t, 32 * t + 32
                needs_mask = (32 * t + 32 > N) or (causal and 32 * t + 31 > wq0)
                if 1 <= t <= 2 * j_clean:
                    assert not needs_mask, (N, qt, w, t)
                vis = visible(N, causal)[r0:r1, k0:min(k1, N)]
                if not needs_mask:
                    assert vis.all() and k1 <= N
                cover[r0:r1, k0:min(k1, N)] += vis
                scored += (r1 - r0) * 32
    return cover, scored


def ring_protocol(n_kt, nbuf=4):
    """The forward's copy ring for one workgroup: tiles 0 and 1 copied and published before the loop,
    tiles 2 and 3 copied right after; end of tile j: if j + 4 < n_kt, wait until tile j + 2 is in,
    barrier, copy tile j + 4 into tile j's slot; at j = max(0, n_kt - 4), wait for every copy and
    barrier; later tiles have no barrier."""
    issued = {}                                    # tile -> slot
    published = set()
    slot_holds = {}                                # slot -> tile
    def issue(t):
        s = t % nbuf
        if s in slot_holds:
            assert slot_holds[s] in done_reading, (n_kt, t)   # previous tile of the slot fully read
        slot_holds[s] = t
        issued[t] = s
    done_reading = set()
    for t in range(min(2, n_kt)):
        issue(t)
    published |= set(issued)
    for t in range(2, min(4, n_kt)):
        issue(t)
    for j in range(n_kt):
        for t in (j, j + 1):                       # tiles read during iteration j
            if t < n_kt:
                assert t in published, (n_kt, j, t)
        done_reading.add(j)                        # nothing reads tile j after iteration j
        if j + 4 < n_kt:
            published |= {t for t in issued if t <= j + 2}
            issue(j + 4)
        elif j == max(0, n_kt - 4):
            published |= set(issued)
    assert set(issued) == set(range(n_kt))


def fwd_fp8_model(N, causal):
    """fwd_fp8_kernel: 256-row workgroups, 128-key tiles, 64-key units; a unit is masked only
    when it holds keys past N or (causal) keys after the wave's first row. Row blocks sit on the
    waves as in the bf16 kernel, and the copy ring follows the same protocol (during tile j a wave
    reads tiles j and j + 1). Tiles j < j_clean run
    the straight-line step, which masks nothing and takes a next unit for granted: units
    1 .. 2*j_clean must need no mask and exist."""
    BR, BC = 256, 128
    cover = np.zeros((N, N), dtype=np.int64)
    for qt in range(math.ceil(N / BR)):
        q0 = qt * BR
        kv_end = min(N, q0 + BR) if causal else N
        n_kt = math.ceil(kv_end / BC)
        ring_protocol(n_kt)
        for w in range(8):
            rb = w if w < 4 else 11 - w
            wq0 = q0 + 32 * rb
            wv_end = min(N, wq0 + 32) if causal else N
            n_u = math.ceil(wv_end / 64) if wq0 < N else 0
            assert n_u <= 2 * n_kt
            n_clean = min((wq0 + 1) // 64 if causal else N // 64, N // 64)
            j_clean = max(0, (n_clean - 1) // 2)
            assert n_u == 0 or j_clean == 0 or 2 * j_clean < n_u   # waves past N return at once
            r0, r1 = wq0, min(wq0 + 32, N)
            for u in range(n_u):
                k0, k1 = 64 * u, 64 * u + 64
                masked = (64 * u + 64 > N) or (causal and 64 * u + 63 > wq0)
                if 1 <= u <= 2 * j_clean:
                    assert not masked, (N, qt, w, u)
                vis = visible(N, causal)[r0:r1, k0:min(k1, N)]
                if not masked:
                    assert vis.all() and k1 <= N
                cover[r0:r1, k0:min(k1, N)] += vis
    return cover


def bwd_dkdv_ring(n_t):
    """The dK/dV kernel's two-slot Q/dO ring: tile 0 is copied and published before the loop,
    tile 1 copied; tile t sits in slot t % 2 and is read during step t; the step ends with a
    full wait (tile t + 1 lands) and a barrier, after which tile t + 2 is copied into slot t % 2."""
    slot, published = {0: 0}, {0}
    if n_t > 1:
        slot[1] = 1
    for t in range(n_t):
        assert slot[t % 2] == t and t in published
        published |= {slot[s] for s in slot}
        if t + 2 < n_t:
            slot[t % 2] = t + 2


def bwd_dkdv_model(N, causal):
    """bwd_dkdv_kernel: 128-key workgroups of eight waves; wave w owns keys k0 + 32 (w % 4) ..
    + 31 and the query block 32 (w // 4) of every 64-row tile from query tile k0 / 64 on (causal).
    A block with no visible pair (before the wave's keys, or past the last row) is skipped; a
    block that needs the mask takes the masked path, which zeroes its hidden probabilities. The
    two waves of a key block cover the two halves of each tile; their sums are added at the end."""
    BT = 64
    cover = np.zeros((N, N), dtype=np.int64)
    n_qt = math.ceil(N / BT)
    for kt in range(math.ceil(N / 128)):
        k0 = kt * 128
        qt0 = k0 // BT if causal else 0
        n_t = max(n_qt - qt0, 0)
        assert n_t >= 1
        bwd_dkdv_ring(n_t)
        for w in range(8):
            kb, par = w % 4, w // 4
            kw0 = k0 + 32 * kb
            c0, c1 = kw0, min(kw0 + 32, N)
            for t in range(n_t):
                qb0 = (qt0 + t) * BT + 32 * par
                active = qb0 < N and not (causal and qb0 + 31 < kw0)
                vis = visible(N, causal)[qb0:min(qb0 + 32, N), c0:c1] if qb0 < N and c0 < N else np.zeros((0, 0), bool)
                need_mask = (qb0 + 32 > N) or (causal and qb0 < kw0 + 31)
                if not active:
                    assert not vis.any()
                    continue
                if not need_mask:
                    assert vis.all()
                if c0 < N:  # the sums of keys past N are not written
                    cover[qb0:min(qb0 + 32, N), c0:c1] += vis
    return cover


def bwd_dq_model(N, causal):
    """bwd_dq_kernel: 256-query workgroups, 32 queries per wave, 32-key sub-tiles of 64-key tiles."""
    BT = 64
    cover = np.zeros((N, N), dtype=np.int64)
    for qt in range(math.ceil(N / 256)):
        q0 = qt * 256
        kv_end = min(N, q0 + 256) if causal else N
        n_kt = math.ceil(kv_end / BT)
        for w in range(8):
            wq0 = q0 + 32 * w
            wv_end = min(N, wq0 + 32) if causal else N
            n_st = math.ceil(wv_end / 32) if wq0 < N else 0
            r0, r1 = wq0, min(wq0 + 32, N)
            for j in range(n_kt):
                for h in range(2):
                    t = 2 * j + h
                    if t >= n_st:
                        continue
                    need_mask = (32 * t + 32 > N) or (causal and 32 * t + 31 > wq0)
                    vis = visible(N, causal)[r0:r1, 32 * t:min(32 * t + 32, N)]
                    if not need_mask:
                        assert vis.all()
                    cover[r0:r1, 32 * t:min(32 * t + 32, N)] += vis
            assert n_st <= 2 * n_kt
    return cover


def fwd_f32_model(N, causal):
    """fwd_f32_kernel: four query rows per workgroup (one per wave), 64-key tiles loaded up to the
    workgroup's last row (causal) or to N; each lane scores one key of the tile, kept iff key < N and
    (non-causal or key <= row); rows past N write nothing."""
    cover = np.zeros((N, N), dtype=np.int64)
    lanes = np.arange(64)
    for qt in range(math.ceil(N / 4)):
        q0 = 4 * qt
        kv_end = min(N, q0 + 4) if causal else N
        n_tiles = math.ceil(kv_end / 64)
        for w in range(4):
            row = q0 + w
            for t in range(n_tiles):
                keys = 64 * t + lanes
                vis = (keys < N) & ((keys <= row) if causal else True)
                if row < N:
                    cover[row, keys[vis]] += 1
            if row < N:                               # every visible key of the row lies in a loaded tile
                assert (row + 1 if causal else N) <= 64 * n_tiles
    return cover


def fwd_f32_split_model(N, causal, W=4):
    """fwd_f32_split_kernel: one query row per workgroup; wave w takes the 64-key tiles w, w + W, ...
    up to the row's last visible key; a lane's key is kept iff key < kv_end, its K row is read at
    that key (else at key 0), and the P V loop runs over the tile's first nk = min(64, kv_end - 64 t)
    keys, which must be exactly the kept ones. Wave 0 always holds tile 0, so the merged maximum is
    finite."""
    cover = np.zeros((N, N), dtype=np.int64)
    lanes = np.arange(64)
    for row in range(N):
        kv_end = row + 1 if causal else N
        n_tiles = math.ceil(kv_end / 64)
        per_wave = [list(range(w, n_tiles, W)) for w in range(W)]
        assert sorted(t for ts in per_wave for t in ts) == list(range(n_tiles))
        assert per_wave[0][:1] == [0]
        for ts in per_wave:
            for t in ts:
                keys = 64 * t + lanes
                vis = keys < kv_end
                assert np.where(vis, keys, 0).max() < N                 # K reads in bounds
                nk = min(64, kv_end - 64 * t)
                assert 1 <= nk <= 64 and np.array_equal(vis, lanes < nk)  # V reads = the kept keys
                cover[row, keys[vis]] += 1
    return cover


@pytest.mark.parametrize("NW", [8, 4])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SIZES)
def test_forward_bf16_tiles(N, causal, NW):
    cover, _ = fwd_bf16_model(N, causal, NW)
    check_cover(cover, N, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SIZES)
def test_forward_f32_tiles(N, causal):
    check_cover(fwd_f32_model(N, causal), N, causal)
    check_cover(fwd_f32_split_model(N, causal), N, causal)


@pytest.mark.parametrize("n_kt", list(range(1, 40)))
def test_forward_copy_ring(n_kt):
    ring_protocol(n_kt)


def test_forward_copy_ring_catches_an_early_rewrite():
    """A ring whose last barrier comes one tile too early (the barrier-free stretch one tile longer)
    reads a tile no barrier published: the model rejects it."""
    def too_early(n_kt, nbuf=4):
        published, issued = set(), set()
        for t in range(min(4, n_kt)):
            issued.add(t)
        published |= {0, 1} & issued
        for j in range(n_kt):
            for t in (j, j + 1):
                if t < n_kt and t not in published:
                    return False
            if j + 5 < n_kt:
                published |= {t for t in issued if t <= j + 2}
                issued.add(j + 4)
            elif j == max(0, n_kt - 5):
                issued |= set(range(n_kt))
                published |= {t for t in issued if t <= j + 2}
        return True
    assert not all(too_early(n) for n in range(1, 40))


def test_forward_bf16_masked_work_is_small():
    """At the 8K causal workload the scored positions exceed the visible pairs only by the
    upper triangles of the diagonal sub-tiles (each wave scores 32 x 32 there, 528 of them
    visible): a ratio of 1 + 31 / (N + 1), 0.38% (the MFMA count measures 0.36%)."""
    N = 8192
    n_vis = N * (N + 1) // 2
    # scored = sum over waves of 32 rows x 32 * n_st keys, with n_st = (wq0 + 32) / 32
    scored = sum(32 * 32 * ((32 * w + 32) // 32) for w in range(N // 32))
    assert scored / n_vis == pytest.approx(1 + 31 / (N + 1), rel=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SIZES)
def test_forward_fp8_tiles(N, causal):
    check_cover(fwd_fp8_model(N, causal), N, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SIZES)
def test_backward_dkdv_tiles(N, causal):
    check_cover(bwd_dkdv_model(N, causal), N, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SIZES)
def test_backward_dq_tiles(N, causal):
    check_cover(bwd_dq_model(N, causal), N, causal)


def decode_splits(L, nsplit):
    """The split shape: chunk = ceil(L / min(nsplit, L)) keys, ceil(L / chunk) splits."""
    n = min(nsplit, L)
    chunk = -(-L // n)
    ns = -(-L // chunk)
    return chunk, ns


@pytest.mark.parametrize("L", [1, 2, 7, 100, 333, 512, 4097, 32768])
@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 64, 999, 5000])
def test_decode_splits_cover_once_and_match_the_library(L, nsplit):
    chunk, ns = decode_splits(L, nsplit)
    covered = np.zeros(L, dtype=np.int64)
    for s in range(ns):
        lo, hi = s * chunk, min(L, (s + 1) * chunk)
        assert hi > lo                                       # no empty split
        covered[lo:hi] += 1
    assert (covered == 1).all()
    lib = binding.load()
    assert lib.fa_decode_workspace_bytes(2, 3, L, 128, nsplit) == 2 * 3 * ns * (128 + 2) * 4


@pytest.mark.parametrize("page_size", [1, 16, 256])
@pytest.mark.parametrize("nsplit", [1, 5, 64])
def test_paged_decode_splits(page_size, nsplit):
    """Paged splits cut Lmax = max_pages * page_size keys like the contiguous decode; a sequence
    of any length 0 .. Lmax has each of its keys in exactly one split, and the page-table index
    of every key it reads stays below max_pages."""
    max_pages = 5
    lmax = max_pages * page_size
    chunk, ns = decode_splits(lmax, nsplit)
    for length in sorted({0, 1, page_size - 1, page_size, lmax - 1, lmax} - {-1}):
        covered = np.zeros(max(length, 1), dtype=np.int64)
        for s in range(ns):
            kbeg, kend = s * chunk, min(length, s * chunk + chunk)
            for key in range(kbeg, kend):
                assert key // page_size < max_pages
                covered[key] += 1
        assert (covered[:length] == 1).all()


def head_group(NW, BH, n_qt):
    """The forward launcher's heads per group of the workgroup order (one group: all heads)."""
    if NW == 8 and ((BH >= 64 and n_qt >= 16) or n_qt >= 128):
        return min(16, BH)
    return BH


def workgroup_item(i, BH, n_qt, GH):
    """fwd_bf16_kernel's workgroup -> (head, rank) map for heads in groups of GH."""
    grp = i // (GH * n_qt)
    gh = min(GH, BH - grp * GH)
    r = i - grp * GH * n_qt
    return grp * GH + r % gh, r // gh


@pytest.mark.parametrize("BH", [1, 3, 8, 16, 24, 32, 64, 72, 128, 256])
@pytest.mark.parametrize("n_qt", [1, 2, 16, 33, 128, 512])
def test_forward_workgroup_order_is_a_permutation(BH, n_qt):
    """Every (head, query tile) is taken by exactly one workgroup; in a group of 16 heads workgroup i
    (which runs on XCD i % 8) takes a head of the group's XCD i % 8 pair, ranks in order."""
    GH = head_group(8, BH, n_qt)
    items = [workgroup_item(i, BH, n_qt, GH) for i in range(BH * n_qt)]
    assert sorted(items) == [(b, r) for b in range(BH) for r in range(n_qt)]
    if GH == 16:
        full = (BH // 16) * 16 * n_qt
        for i in range(full):
            bh, rank = items[i]
            assert (bh - 16 * (i // (16 * n_qt))) % 8 == i % 8
        ranks = [items[i][1] for i in range(16 * n_qt)]
        assert ranks == sorted(ranks)                 # heaviest (lowest rank) first within a group
    else:
        assert items == [(i % BH, i // BH) for i in range(BH * n_qt)]
