"""eagle_op_linear_noalloc (the projection with the library's own fixed
device array as workspace) against eagle_op_linear with a caller workspace:
the same kernels, so the same bits, on consecutive calls that reuse the
array with a smaller shape second."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

E = pytest.importorskip("speculative_decoding_draft_amd")

BF16, F32 = 1, 0


def _operands(M, N, K, dtype, seed, epi):
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=gen)
    rows = 2 * N if epi == 2 else N
    w = (torch.randn((rows, K), generator=gen) * 0.02)
    if dtype == BF16:
        hi = x.to(torch.bfloat16)
        lo = (x - hi.float()).to(torch.bfloat16)
        xd = torch.cat([hi.reshape(-1), lo.reshape(-1)]).cuda()
        wb = w.to(torch.bfloat16).cuda()
        wd = torch.empty_like(wb)
        E.op_pack(wb, wd, rows, K)
    else:
        xd, wd = x.cuda(), w.cuda()
    y0 = torch.randn((M, N), generator=gen)
    return xd, wd, y0


def _out(M, N, dtype, epi, y0):
    if epi == 2:
        planes = 2 if dtype == BF16 else 1
        return torch.zeros(planes * M * N, dtype=torch.bfloat16 if dtype == BF16 else torch.float32,
                           device="cuda")
    return (y0.clone() if epi == 1 else torch.zeros_like(y0)).cuda()


# (dtype, epilogue, M, N, K): each pair runs a larger shape, then a smaller one
CASES = [
    [(BF16, 0, 27, 12288, 4096), (BF16, 0, 10, 4096, 4096)],
    [(BF16, 1, 61, 4096, 11008), (BF16, 1, 27, 4096, 4096)],
    [(BF16, 2, 300, 2752, 1024), (BF16, 2, 150, 1376, 1024)],
    [(F32, 0, 33, 1024, 512), (F32, 0, 17, 256, 256)],
]


@pytest.mark.parametrize("pair", CASES, ids=lambda p: f"epi{p[0][1]}_M{p[0][2]}")
def test_noalloc_equals_workspace_call(pair):
    for i, (dtype, epi, M, N, K) in enumerate(pair):
        print(f"noalloc call {i}: dtype={dtype} epi={epi} M={M} N={N} K={K}", flush=True)
        assert E.op_linear_workspace(dtype, epi, M, N, K) <= E.NOALLOC_SCRATCH_BYTES
        xd, wd, y0 = _operands(M, N, K, dtype, seed=M * 7 + N + K + epi, epi=epi)
        ref = _out(M, N, dtype, epi, y0)
        ws = torch.zeros(max(E.op_linear_workspace(dtype, epi, M, N, K), 256), dtype=torch.uint8,
                         device="cuda")
        E.op_linear(dtype, epi, xd, wd, ref, M, N, K, ws)
        got = _out(M, N, dtype, epi, y0)
        E.op_linear_noalloc(dtype, epi, xd, wd, got, M, N, K)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), ref.cpu()), f"call {i} differs"


def test_noalloc_rejects_oversized_shape():
    """A shape whose partial planes exceed the fixed array is refused on the
    host, before any launch (the pointers are never dereferenced)."""
    M, N, K = 512, 32000, 8192
    need = E.op_linear_workspace(BF16, 0, M, N, K)
    assert need > E.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(16, device="cuda")
    with pytest.raises(E.EagleError) as ei:
        E.op_linear_noalloc(BF16, 0, t, t, t, M, N, K)
    assert ei.value.status == E.E_CAPACITY
