"""Parity of the paged-KV decode (fa_decode_paged) with the oracle's paged decode
(gather the pages, then the plain definition), through the C ABI.

Pools come from the seeded page_cache generator: pages handed out in a shuffled
order, every pool row that holds no key set to NaN and block-table entries past
a sequence's last page set to -1, so a read of anything but a sequence's own
keys makes the output non-finite."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from exact_io_aware_74_amd import binding as fa
from helpers import assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu


def to_dev_i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def paged_case(seed, B, H, Lmax, d, page_size, lens=None, std=1.0):
    q, k, v = si.random_case(seed, B, H, 1, d, "bf16", nk=Lmax, std=std)
    lens = si.seq_lengths(seed, B, Lmax, page_size) if lens is None else np.asarray(lens, np.int32)
    kp, vp, table, lens = si.page_cache(seed, k, v, lens, page_size)
    return q[:, :, 0], kp, vp, table, lens


def run_paged(q, kp, vp, table, lens, nsplit):
    o = fa.decode_paged(to_device(q, "bf16"), to_device(kp, "bf16"), to_device(vp, "bf16"), to_dev_i32(table),
                        to_dev_i32(lens), nsplit=nsplit)
    torch.cuda.synchronize()
    return to_f64(o)


def oracle_paged(q, kp, vp, table, lens):
    f = lambda x: si.as_float64(x, "bf16")
    return oracle.paged_decode(f(q), f(kp), f(vp), table, lens)[0]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("page_size", [1, 8, 16, 64, 1024])
def test_ragged_lengths(d, page_size):
    """Seeded ragged lengths: 1, page-1, page, page+1 and Lmax keys, then uniform draws."""
    q, kp, vp, table, lens = paged_case(page_size + d, 7, 3, 1100, d, page_size)
    got = run_paged(q, kp, vp, table, lens, nsplit=16)
    ref = oracle_paged(q, kp, vp, table, lens)
    assert_close(got, ref, "bf16")
    for b in range(len(lens)):  # and each sequence alone: short rows would dominate the whole-tensor norm
        assert_close(got[b], ref[b], "bf16", what=f"sequence {b} ({int(lens[b])} keys)")


@pytest.mark.parametrize("nsplit", [1, 3, 64, 777, 5000])
def test_nsplit_sweep(nsplit):
    q, kp, vp, table, lens = paged_case(31, 5, 2, 777, 128, 16, std=2.0)
    assert_close(run_paged(q, kp, vp, table, lens, nsplit), oracle_paged(q, kp, vp, table, lens), "bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("page_size", [1, 16, 256])
def test_equals_contiguous_decode_bitwise(d, page_size):
    """Full lengths: the paged kernel splits like fa_decode over Lkv = max_pages * page_size and
    visits the keys in the same order, so the outputs are identical bit for bit."""
    B, H, L = 3, 4, 1024
    q, k, v = si.random_case(41 + d, B, H, 1, d, "bf16", nk=L)
    kp, vp, table, lens = si.page_cache(41, k, v, np.full(B, L), page_size)
    qd = to_device(q[:, :, 0], "bf16")
    for ns in (1, 7, 64):
        a = fa.decode(qd, to_device(k, "bf16"), to_device(v, "bf16"), nsplit=ns)
        b = fa.decode_paged(qd, to_device(kp, "bf16"), to_device(vp, "bf16"), to_dev_i32(table), to_dev_i32(lens),
                            nsplit=ns)
        assert torch.equal(a, b), (ns, page_size, d)


def test_single_key_and_empty_sequences():
    q, kp, vp, table, lens = paged_case(51, 4, 3, 40, 128, 8, lens=[1, 0, 40, 0])
    got = run_paged(q, kp, vp, table, lens, nsplit=4)
    ref = oracle_paged(q, kp, vp, table, lens)
    assert not got[1].any() and not got[3].any()               # no keys -> 0
    np.testing.assert_array_equal(got[0], si.as_float64(vp[table[0, 0], :, 0], "bf16"))   # one key -> its V row
    assert_close(got, ref, "bf16")


def test_bad_page_ids_and_lengths_poison_only_their_rows():
    """A page id outside the pool, or a length outside [0, max_pages * page_size], turns that
    sequence's output into NaN; the kernel reads nothing outside the pool and the table."""
    B, H, L, ps = 6, 2, 100, 16
    q, kp, vp, table, lens = paged_case(61, B, H, L, 128, ps, lens=[100, 37, 50, 64, 100, 9])
    table = table.copy()
    lens = lens.copy()
    table[1, 1] = kp.shape[0]          # one past the pool, inside sequence 1's pages
    table[2, 3] = -7                   # negative id, sequence 2's last page
    lens[3] = table.shape[1] * ps + 1  # longer than the table allows
    lens[4] = -1
    got = run_paged(q, kp, vp, table, lens, nsplit=8)
    for b in (1, 2, 3, 4):
        assert np.isnan(got[b]).all(), b
    keep = [0, 5]
    ref = oracle_paged(q[keep], kp, vp, table[keep], lens[keep])
    assert_close(got[keep], ref, "bf16")


def test_deterministic():
    q, kp, vp, table, lens = paged_case(71, 4, 4, 3000, 128, 16)
    a = run_paged(q, kp, vp, table, lens, 64)
    b = run_paged(q, kp, vp, table, lens, 64)
    np.testing.assert_array_equal(a, b)


def test_workload_decode_b16h32_l32768_paged_sampled_heads():
    """The decode workload (B=16, H=32, 32768 keys, d=128, nsplit=64) in 16-key pages of a
    shuffled pool, as the benchmark times it; sampled heads against the oracle."""
    w = si.WORKLOADS["decode_b16h32_l32768_d128"]
    ps = 16
    q = si.tensor_full(w, "q")[:, :, 0, :]
    k, v = si.tensor_full(w, "k"), si.tensor_full(w, "v")
    kp, vp, table, lens = si.page_cache(w.wid, k, v, np.full(w.B, w.Lkv), ps)
    del k, v
    o = fa.decode_paged(to_device(q, "bf16"), to_device(kp, "bf16"), to_device(vp, "bf16"), to_dev_i32(table),
                        to_dev_i32(lens), nsplit=w.nsplit)
    got_all = to_f64(o)
    assert np.isfinite(got_all).all()
    got, ref = [], []
    for b, h in [(0, 0), (3, 5), (7, 31), (8, 16), (12, 1), (15, 31)]:
        pages = table[b, :w.Lkv // ps]
        # the sequence's own pages, compacted (layout only): pool page i = logical page i
        sub_k, sub_v = kp[pages, h:h + 1], vp[pages, h:h + 1]
        r = oracle_paged(q[b:b + 1, h:h + 1], sub_k, sub_v, np.arange(len(pages))[None], lens[b:b + 1])
        got.append(got_all[b, h])
        ref.append(r[0, 0])
    print("paged decode full-size", assert_close(np.stack(got), np.stack(ref), "bf16"))


@pytest.mark.timeout(600)
def test_long_sequences_in_large_pages():
    """Two sequences of 1,048,909 and 300,001 keys (d = 128) in 64-key pages of a shuffled pool,
    64 splits (16,390 keys each, so the shorter sequence's last splits are empty), against the oracle."""
    Lmax = (1 << 20) + 333
    q, kp, vp, table, lens = paged_case(81, 2, 1, Lmax, 128, 64, lens=[Lmax, 300001])
    got = run_paged(q, kp, vp, table, lens, 64)
    print("paged long sequences", assert_close(got, oracle_paged(q, kp, vp, table, lens), "bf16"))


def test_largest_page_size():
    """Pages of 65,536 keys (the largest page size accepted), five sequences of 1, 65,535, 65,536, 65,537 and
    70,000 keys (one or two pages each, the rest of each page NaN)."""
    Lmax, ps = 70000, 65536
    q, kp, vp, table, lens = paged_case(91, 5, 1, Lmax, 128, ps, lens=[1, ps - 1, ps, ps + 1, Lmax])
    got = run_paged(q, kp, vp, table, lens, nsplit=16)
    ref = oracle_paged(q, kp, vp, table, lens)
    for b in range(5):  # each sequence on its own: the one-key row would dominate a whole-tensor norm
        print("largest pages, length", int(lens[b]), assert_close(got[b], ref[b], "bf16"))
