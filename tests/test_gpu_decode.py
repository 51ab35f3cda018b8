"""Parity of split-KV decode (split + combine kernels) with the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from exact_io_aware_74_amd import binding as fa
import oracle_pool
from helpers import WholeTensorCheck, assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu


def _decode_case(B, H, L, d, nsplit, seed, std=1.0):
    q, k, v = si.random_case(seed, B, H, 1, d, "bf16", nk=L, std=std)
    qd = to_device(q[:, :, 0, :], "bf16")
    kd, vd = to_device(k, "bf16"), to_device(v, "bf16")
    o = fa.decode(qd, kd, vd, nsplit=nsplit)
    torch.cuda.synchronize()
    ref, _ = oracle.decode(si.as_float64(q, "bf16"), si.as_float64(k, "bf16"), si.as_float64(v, "bf16"))
    return to_f64(o), ref, (qd, kd, vd)


@pytest.mark.timeout(900)
def test_workload_decode_whole_tensor():
    """The full decode workload (B=16, H=32, Lkv=32768, d=128, 64 splits) against the oracle on
    every head: whole-tensor relative L2 and max abs. The oracle runs in worker processes, each
    regenerating a batch row's heads from the seed."""
    name = "decode_b16h32_l32768_d128"
    w = si.WORKLOADS[name]
    qd = to_device(si.tensor_full(w, "q")[:, :, 0, :], "bf16")
    kd = to_device(si.tensor_full(w, "k"), "bf16")
    vd = to_device(si.tensor_full(w, "v"), "bf16")
    o = to_f64(fa.decode(qd, kd, vd, nsplit=w.nsplit))
    del qd, kd, vd
    chk = WholeTensorCheck("bf16")
    tasks = [(name, b, list(range(h0, h0 + 8))) for b in range(w.B) for h0 in range(0, w.H, 8)]
    for batch in oracle_pool.run(oracle_pool.decode_heads, tasks, oracle_pool.default_workers(0.5)):
        for b, h, ref, _ in batch:
            chk.add((b, h), o[b, h], ref)
    assert chk.heads == w.B * w.H
    print("decode whole tensor", chk.assert_bounds(with_lse=False))


@pytest.mark.parametrize("nsplit", [1, 2, 7, 64, 999, 1000, 5000])
def test_nsplit_sweep(nsplit):
    got, ref, _ = _decode_case(2, 3, 1000, 128, nsplit, seed=11, std=2.0)
    assert_close(got, ref, "bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [1, 2, 17, 333, 4097])
def test_ragged_cache_lengths(d, L):
    got, ref, _ = _decode_case(2, 2, L, d, 64, seed=L + d)
    assert_close(got, ref, "bf16")


def test_single_key_returns_v():
    got, _, (qd, kd, vd) = _decode_case(3, 2, 1, 128, 4, seed=3)
    np.testing.assert_array_equal(got, to_f64(vd[:, :, 0, :]))


def test_decode_equals_last_row_of_causal_prefill():
    B, H, N, d = 2, 4, 515, 128
    q, k, v = si.random_case(21, B, H, N, d, "bf16")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o_fwd, _ = fa.fwd(qd, kd, vd, causal=True)
    o_dec = fa.decode(qd[:, :, N - 1, :].contiguous(), kd, vd, nsplit=8)
    ref, _ = oracle.decode(si.as_float64(q[:, :, N - 1], "bf16"), si.as_float64(k, "bf16"), si.as_float64(v, "bf16"))
    assert_close(to_f64(o_dec), ref, "bf16")
    assert_close(to_f64(o_fwd[:, :, N - 1, :]), ref, "bf16")


def test_cache_permutation_invariance():
    B, H, L, d = 1, 2, 700, 64
    q, k, v = si.random_case(22, B, H, 1, d, "bf16", nk=L)
    perm = np.random.default_rng(5).permutation(L)
    qd = to_device(q[:, :, 0, :], "bf16")
    o1 = to_f64(fa.decode(qd, to_device(k, "bf16"), to_device(v, "bf16"), nsplit=7))
    o2 = to_f64(fa.decode(qd, to_device(np.ascontiguousarray(k[:, :, perm]), "bf16"),
                          to_device(np.ascontiguousarray(v[:, :, perm]), "bf16"), nsplit=7))
    ref, _ = oracle.decode(si.as_float64(q, "bf16"), si.as_float64(k, "bf16"), si.as_float64(v, "bf16"))
    assert_close(o1, ref, "bf16")
    assert_close(o2, ref, "bf16")


def test_workspace_regrows_and_streams():
    """Small, large, small again on one stream, then on a second stream: all correct."""
    for L, ns in ((100, 4), (5000, 64), (300, 3)):
        got, ref, _ = _decode_case(2, 2, L, 128, ns, seed=L)
        assert_close(got, ref, "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got, ref, _ = _decode_case(1, 3, 2000, 64, 16, seed=77)
    s.synchronize()
    assert_close(got, ref, "bf16")


def test_deterministic():
    _, _, (qd, kd, vd) = _decode_case(2, 2, 3000, 128, 64, seed=9)
    a = fa.decode(qd, kd, vd, nsplit=64)
    b = fa.decode(qd, kd, vd, nsplit=64)
    assert torch.equal(a, b)


def test_shutdown_then_decode_again():
    """fa_shutdown frees the library's decode workspaces; the next decode allocates afresh and
    gives the same result, twice over."""
    got, ref, (qd, kd, vd) = _decode_case(2, 3, 900, 128, 16, seed=90)
    assert_close(got, ref, "bf16")
    first = fa.decode(qd, kd, vd, nsplit=16)
    for _ in range(2):
        torch.cuda.synchronize()
        fa.shutdown()
        again = fa.decode(qd, kd, vd, nsplit=16)
        torch.cuda.synchronize()
        assert torch.equal(first, again)


@pytest.mark.timeout(600)
def test_one_long_sequence():
    """One head with a 2,097,929-key cache (d = 128): 64 splits of 32,781 keys (256 batches per workgroup)
    and a single split over every key (one workgroup, 16,391 batches), both against the oracle."""
    L, d = (1 << 21) + 777, 128
    q, k, v = si.random_case(23, 1, 1, 1, d, "bf16", nk=L)
    qd = to_device(q[:, :, 0, :], "bf16")
    kd, vd = to_device(k, "bf16"), to_device(v, "bf16")
    outs = {ns: to_f64(fa.decode(qd, kd, vd, nsplit=ns)) for ns in (64, 1)}
    del kd, vd
    ref, _ = oracle.decode(si.as_float64(q, "bf16"), si.as_float64(k, "bf16"), si.as_float64(v, "bf16"))
    for ns, got in outs.items():
        print("long sequence, nsplit", ns, assert_close(got, ref, "bf16"))


def test_concurrent_host_threads_on_their_own_streams():
    """Four host threads, each with its own stream, decode shapes of growing size at the same time
    (each stream's workspace is created and regrown under the library's lock while the others run);
    every result equals the same call made alone."""
    import threading
    shapes = [(2, 3, 700, 128, 16), (1, 4, 5000, 64, 64), (3, 2, 20000, 128, 128), (2, 2, 333, 128, 5)]
    cases = []
    for i, (B, H, L, d, ns) in enumerate(shapes):
        q, k, v = si.random_case(600 + i, B, H, 1, d, "bf16", nk=L)
        cases.append((to_device(q[:, :, 0, :], "bf16"), to_device(k, "bf16"), to_device(v, "bf16"), ns))
    alone = [fa.decode(qd, kd, vd, nsplit=ns) for qd, kd, vd, ns in cases]
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = []
                for rep in range(3):
                    for j in range(len(cases)):
                        qd, kd, vd, ns = cases[(t + j) % len(cases)]
                        outs.append(((t + j) % len(cases), fa.decode(qd, kd, vd, nsplit=ns)))
            s.synchronize()
            results[t] = outs
        except Exception as e:  # reported below, with the thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for t in range(4):
        for j, o in results[t]:
            assert torch.equal(o, alone[j]), (t, j)
