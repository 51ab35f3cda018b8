"""Every kernel path writes exactly its outputs: each output (and the ablation's
workspace) is a view into a larger buffer whose margins hold a canary value and
whose interior starts as NaN. After the call the margins must be untouched, the
interior fully written, and the result bit-identical to an unguarded call on the
same inputs. Shapes are chosen to reach each launch path: the four-wave (128-row)
and eight-wave (256-row) bf16 forward at d = 64, the d = 128 forward, both fp32
kernels (one row per workgroup up to 512 rows, four rows per workgroup above),
the FP8 forward, the contiguous, no-allocation and paged decodes, and the
three-kernel ablation."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from exact_io_aware_74_amd import binding as fa
from helpers import to_device

pytestmark = pytest.mark.gpu

PAD = 4096        # elements of margin on each side (keeps the 16-byte alignment for every dtype used)
CANARY = 7.0


class Guarded:
    """A contiguous tensor of `shape` inside a buffer with canary margins; the interior starts as NaN."""

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape))
        self.buf = torch.full((self.n + 2 * PAD,), CANARY, dtype=dtype, device="cuda")
        self.t = self.buf[PAD:PAD + self.n].view(shape)
        self.t.fill_(float("nan"))

    def check(self, what):
        torch.cuda.synchronize()
        assert (self.buf[:PAD] == CANARY).all(), f"{what}: write before the buffer"
        assert (self.buf[PAD + self.n:] == CANARY).all(), f"{what}: write past the buffer"
        assert not torch.isnan(self.t).any(), f"{what}: not fully written"


FWD_CASES = [(64, (1, 3, 300)),      # d = 64, few tiles: four-wave workgroups
             (64, (2, 64, 1000)),    # d = 64, 512 256-row tiles: eight-wave workgroups
             (128, (1, 3, 300)),
             (128, (2, 2, 1))]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,shape", FWD_CASES)
def test_fwd_bf16(d, shape, causal):
    B, H, N = shape
    q, k, v = (to_device(x, "bf16") for x in si.random_case(31 + N + d, B, H, N, d, "bf16"))
    o, lse = Guarded((B, H, N, d), torch.bfloat16), Guarded((B, H, N), torch.float32)
    fa.fwd(q, k, v, causal=causal, out=o.t, lse=lse.t)
    o.check("O")
    lse.check("LSE")
    o2, l2 = fa.fwd(q, k, v, causal=causal)
    assert torch.equal(o.t, o2) and torch.equal(lse.t, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,shape", [(64, (1, 1, 300)), (128, (1, 1, 512)), (64, (1, 2, 300)), (128, (2, 1, 700))])
def test_fwd_f32(d, shape, causal):
    B, H, N = shape
    q, k, v = (to_device(x, "f32") for x in si.random_case(41 + N + d, B, H, N, d, "f32"))
    o, lse = Guarded((B, H, N, d), torch.float32), Guarded((B, H, N), torch.float32)
    fa.fwd(q, k, v, causal=causal, out=o.t, lse=lse.t)
    o.check("O")
    lse.check("LSE")
    o2, l2 = fa.fwd(q, k, v, causal=causal)
    assert torch.equal(o.t, o2) and torch.equal(lse.t, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_fp8(d, causal):
    B, H, N = 1, 3, 300
    q8, k8, v8, ds = si.fp8_case(51 + d, B, H, N, d)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q8, k8, v8))
    o, lse = Guarded((B, H, N, d), torch.bfloat16), Guarded((B, H, N), torch.float32)
    fa.fwd_fp8(q, k, v, ds, causal=causal, out=o.t, lse=lse.t)
    o.check("O")
    lse.check("LSE")
    o2, l2 = fa.fwd_fp8(q, k, v, ds, causal=causal)
    assert torch.equal(o.t, o2) and torch.equal(lse.t, l2)


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_decode(d, noalloc):
    B, H, L = 2, 3, 1000
    q, k, v = si.random_case(61 + d, B, H, 1, d, "bf16", nk=L)
    qd, kd, vd = to_device(q[:, :, 0, :], "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    o = Guarded((B, H, d), torch.bfloat16)
    fa.decode(qd, kd, vd, nsplit=7, out=o.t, noalloc=noalloc)
    o.check("o")
    assert torch.equal(o.t, fa.decode(qd, kd, vd, nsplit=7))


@pytest.mark.parametrize("d", [64, 128])
def test_decode_paged(d):
    B, H, Lmax, page = 2, 3, 500, 16
    q, k, v = si.random_case(71 + d, B, H, 1, d, "bf16", nk=Lmax)
    lens = si.seq_lengths(71 + d, B, Lmax, page)
    kp, vp, table, lens = si.page_cache(71 + d, k, v, lens, page)
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    args = (to_device(q[:, :, 0, :], "bf16"), to_device(kp, "bf16"), to_device(vp, "bf16"), i32(table), i32(lens))
    o = Guarded((B, H, d), torch.bfloat16)
    fa.decode_paged(*args, nsplit=5, out=o.t)
    o.check("o")
    assert torch.equal(o.t, fa.decode_paged(*args, nsplit=5))


@pytest.mark.parametrize("causal", [False, True])
def test_naive(causal):
    B, H, N, d = 1, 2, 200, 64
    q, k, v = (to_device(x, "bf16") for x in si.random_case(81, B, H, N, d, "bf16"))
    o, lse = Guarded((B, H, N, d), torch.bfloat16), Guarded((B, H, N), torch.float32)
    ws = Guarded((fa.naive_workspace_bytes(B, H, N) // 4,), torch.float32)
    fa.naive_fwd(q, k, v, causal=causal, workspace=ws.t, out=o.t, lse=lse.t)
    o.check("O")
    lse.check("LSE")
    torch.cuda.synchronize()
    assert (ws.buf[:PAD] == CANARY).all() and (ws.buf[PAD + ws.n:] == CANARY).all(), "workspace margins written"
    o2, l2 = fa.naive_fwd(q, k, v, causal=causal)
    assert torch.equal(o.t, o2) and torch.equal(lse.t, l2)
