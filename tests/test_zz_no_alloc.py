"""The allocation-free accept (vs_accept_noalloc) against vs_accept on the same
inputs: greedy chains, greedy token trees (ancestor masks) and stochastic
chains, two calls in a row, the second with fewer sequences and rows than the
first (the library's fixed statistics array keeps the first call's contents).
Results are integers and must be identical."""
import numpy as np
import pytest
import torch

from synth.workloads import TINY
from tests import gpu_common as G
from verification_verify_step_amd import binding as B

pytestmark = pytest.mark.gpu

CFG = TINY
V = CFG.vocab


@pytest.fixture(scope="module")
def eng():
    e = G.engine(CFG, force_host=True, max_rows=320, max_seqs=40, max_ctx=256)
    yield e
    e.close()


def _inputs(rng, n_seq, k, seed):
    M = n_seq * (k + 1)
    zt = (rng.standard_normal((M, V)) * 2.0).astype(np.float32)
    zd = (zt + rng.standard_normal((M, V)).astype(np.float32) * 0.7).astype(np.float32)
    toks = rng.integers(0, V, M).astype(np.int32)
    for i in range(n_seq):  # the first drafts of each sequence agree with the target's argmax
        for s in range(k):
            r = i * (k + 1) + s
            if s < i % (k + 1):
                toks[r + 1] = int(np.argmax(zt[r]))
    U = np.stack([G.uniforms(seed + i, 1) for i in range(n_seq)])
    return zt, zd, toks, U


def _both(eng, batch, n_seq, mode, zt, zd, toks, U, T=1.0):
    dzt, dzd, dtok, du = (torch.from_numpy(zt).cuda(), torch.from_numpy(zd).cuda(), G.i32(toks),
                          G.f64(U.reshape(-1)))
    r1 = torch.full((n_seq, B.VS_RESULT_INTS), -7, dtype=torch.int32, device="cuda")
    r2 = torch.full((n_seq, B.VS_RESULT_INTS), -9, dtype=torch.int32, device="cuda")
    dz = dzd.data_ptr() if mode == B.VS_SAMPLE else None
    uu = du.data_ptr() if mode == B.VS_SAMPLE else None
    B.vs_accept(eng.model, batch, mode, T, dtok.data_ptr(), dzt.data_ptr(), dz, uu, r1.data_ptr(), eng.stream)
    B.vs_accept_noalloc(V, batch, mode, T, dtok.data_ptr(), dzt.data_ptr(), dz, uu, r2.data_ptr(), eng.stream)
    torch.cuda.synchronize()
    return r1.cpu().numpy(), r2.cpu().numpy()


@pytest.mark.parametrize("mode", [B.VS_GREEDY, B.VS_SAMPLE])
def test_noalloc_accept_equals_accept(eng, mode):
    rng = np.random.default_rng(0x5EED0A11 + mode)
    for n_seq, k in ((32, 8), (5, 3)):  # the second call is smaller than the first
        zt, zd, toks, U = _inputs(rng, n_seq, k, 100 * n_seq)
        batch = B.make_batch(list(range(n_seq)), [k + 1] * n_seq)
        r1, r2 = _both(eng, batch, n_seq, mode, zt, zd, toks, U)
        assert np.array_equal(r1, r2), (n_seq, k)


def test_noalloc_accept_tree_masks(eng):
    """Greedy walks over token trees (each row's parent is a random earlier
    row), two calls in a row, the second smaller."""
    rng = np.random.default_rng(0x5EED0A12)
    for n_seq, R in ((6, 40), (2, 9)):
        M = n_seq * R
        zt = (rng.standard_normal((M, V)) * 2.0).astype(np.float32)
        toks = rng.integers(0, V, M).astype(np.int32)
        depth = np.zeros(M, dtype=np.int32)
        mask = np.zeros(M, dtype=np.uint64)
        for i in range(n_seq):
            base = i * R
            mask[base] = 1
            for r in range(1, R):
                par = int(rng.integers(0, r))
                depth[base + r] = depth[base + par] + 1
                mask[base + r] = mask[base + par] | np.uint64(1 << r)
                if rng.random() < 0.5:  # make some paths match the argmax of their parent
                    toks[base + r] = int(np.argmax(zt[base + par]))
        dd = G.i32(depth)
        dm = torch.tensor(mask.view(np.int64), device="cuda")
        batch = B.make_batch(list(range(n_seq)), [R] * n_seq, dd.data_ptr(), dm.data_ptr())
        r1, r2 = _both(eng, batch, n_seq, B.VS_GREEDY, zt, zt, toks, np.zeros((n_seq, B.VS_N_UNIFORMS)))
        assert np.array_equal(r1, r2), (n_seq, R)
        assert (r1[:, 0] > 0).any()


def test_noalloc_rejects_bad_arguments(eng):
    batch = B.make_batch([0], [3])
    z = torch.zeros((3, V), dtype=torch.float32, device="cuda")
    t = G.i32([0, 1, 2])
    r = torch.zeros((1, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    with pytest.raises(B.VsError):
        B.vs_accept_noalloc(V + 8, batch, B.VS_GREEDY, 1.0, t.data_ptr(), z.data_ptr(), None, None, r.data_ptr(),
                            eng.stream)
    big = B.make_batch(list(range(20)), [60] * 20)  # 1200 rows, beyond the fixed array
    with pytest.raises(B.VsError):
        B.vs_accept_noalloc(V, big, B.VS_GREEDY, 1.0, t.data_ptr(), z.data_ptr(), None, None, r.data_ptr(), eng.stream)
