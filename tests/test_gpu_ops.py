"""Kernel-level parity of the projection and LM-head kernels (eagle_ops.h)
against fp64 numpy on the same bf16 / fp32 inputs."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

E = pytest.importorskip("speculative_decoding_draft_amd")

BF16, F32 = 1, 0


def _rand(shape, gen, scale, dtype):
    t = torch.randn(shape, generator=gen, dtype=torch.float32) * scale
    return t.to(torch.bfloat16) if dtype == BF16 else t


def _act(shape, gen, dtype):
    """fp32 activations and their device operand (bf16: hi plane then lo plane)."""
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if dtype != BF16:
        return x, x.cuda()
    hi = x.to(torch.bfloat16)
    lo = (x - hi.float()).to(torch.bfloat16)
    return x, torch.cat([hi.reshape(-1), lo.reshape(-1)]).cuda()


def _from_planes(t, shape, dtype):
    t = t.cpu()
    if dtype != BF16:
        return t.double().numpy().reshape(shape)
    n = int(np.prod(shape))
    return (t[:n].double() + t[n:].double()).numpy().reshape(shape)


def _dev_weight(w, dtype):
    """Device copy of a weight in the layout the kernels take: fp32 row-major,
    bf16 fragment-packed by eagle_op_pack."""
    wd = w.cuda()
    if dtype != BF16:
        return wd
    packed = torch.empty_like(wd)
    E.op_pack(wd, packed, w.shape[0], w.shape[1])
    return packed


def _pack_ref(w):
    """The packed layout written out with numpy (rows % 16 == 0 part, then the
    row-major tail), for a bit-exact check of eagle_op_pack."""
    a = w.view(torch.int16).numpy()
    N, K = a.shape
    n16 = N // 16 * 16
    head = a[:n16].reshape(N // 16, 16, K // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    return np.concatenate([head, a[n16:].reshape(-1)])


@pytest.mark.parametrize("N,K", [(16, 32), (48, 96), (4096, 4096), (1000, 1024), (5, 64)])
def test_pack_layout(N, K):
    print(f"pack N={N} K={K}", flush=True)
    gen = torch.Generator().manual_seed(N * 3 + K)
    w = _rand((N, K), gen, 0.02, BF16)
    src = w.cuda()
    dst = torch.empty_like(src)
    E.op_pack(src, dst, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().view(torch.int16).numpy().reshape(-1), _pack_ref(w))


def _ws(nbytes):
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")


def _rel(got, ref):
    """max over rows of |got - ref|_inf / |ref|_inf"""
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1) + 1e-30
    return float((num / den).max())


LINEAR = [  # (dtype, M, N, K): split-K, tails, several M tiles, prefill-sized M
    (BF16, 1, 4096, 4096), (BF16, 10, 4096, 8192), (BF16, 27, 12288, 4096),
    (BF16, 61, 4096, 11008), (BF16, 65, 1000, 1024), (BF16, 100, 256, 512),
    (BF16, 256, 512, 4096), (F32, 17, 256, 256), (F32, 17, 256, 688), (F32, 33, 1024, 512),
    # the six-wave, two-split q|k|v shape at two and four m-tiles
    (BF16, 61, 12288, 4096), (BF16, 54, 12288, 4096),
    # many rows (a batch's verify rows, prefill chunks): the 256-row weight
    # tiles with activations copied straight into LDS, above 128 rows and
    # from 81 rows for wide or deep shapes (128- or 256-row chunks): ragged N
    # (a half block, a partial tile), a second and third row chunk with one
    # row, a single split; 81-128 rows of a 4096 x 4096 shape stay on 64-row
    # passes
    (BF16, 108, 12288, 4096), (BF16, 216, 8200, 1024), (BF16, 300, 8192, 512),
    (BF16, 130, 4096, 1024), (BF16, 257, 4104, 2048), (BF16, 129, 1000, 256),
    (BF16, 512, 4096, 11008), (BF16, 100, 4096, 11008), (BF16, 90, 4096, 4096),
    # the prefill chunk shapes: 256-row m-chunks (MT = 8), two of them, with
    # two K splits (512 rows) and a ragged second chunk (300 rows)
    (BF16, 512, 12288, 4096), (BF16, 300, 12288, 4096),
]


@pytest.mark.parametrize("dtype,M,N,K", LINEAR)
@pytest.mark.parametrize("epi", [0, 1])
def test_linear(dtype, M, N, K, epi):
    print(f"linear dtype={dtype} M={M} N={N} K={K} epi={epi}", flush=True)
    gen = torch.Generator().manual_seed(M * 131 + N * 7 + K + epi)
    x, xd = _act((M, K), gen, dtype)
    w = _rand((N, K), gen, 0.02, dtype)
    y0 = torch.randn((M, N), generator=gen)
    ref = x.double().numpy() @ w.double().numpy().T
    y = (y0.clone() if epi == 1 else torch.zeros(M, N)).cuda()
    ws = _ws(E.op_linear_workspace(dtype, epi, M, N, K))
    wd = _dev_weight(w, dtype)
    E.op_linear(dtype, epi, xd, wd, y, M, N, K, ws)
    torch.cuda.synchronize()
    got = y.cpu().double().numpy()
    if epi == 1:
        got = got - y0.double().numpy()
    assert _rel(got, ref) < 1e-4
    if epi == 0:   # same bits on a second run
        y2 = torch.zeros(M, N, device="cuda")
        E.op_linear(dtype, epi, xd, wd, y2, M, N, K, ws)
        torch.cuda.synchronize()
        assert torch.equal(y2.cpu(), y.cpu())


@pytest.mark.parametrize("dtype,M,N,K", [(BF16, 61, 11008, 4096), (BF16, 10, 1376, 1024),
                                         (BF16, 1, 11008, 4096), (F32, 17, 688, 256),
                                         (BF16, 100, 2720, 1024), (BF16, 200, 1376, 1024),
                                         # wide FFNs: fourteen-wave workgroups
                                         (BF16, 27, 17008, 512), (F32, 17, 17000, 256),
                                         # prefill chunks: gate|up unsplit over two 256-row
                                         # m-chunks plus the SiLU pass (512 rows, 7B FFN),
                                         # a ragged second chunk (300 rows, 8B FFN), one
                                         # chunk with four splits (200 rows)
                                         (BF16, 512, 11008, 4096), (BF16, 300, 14336, 4096),
                                         (BF16, 200, 11008, 4096)])
def test_swiglu(dtype, M, N, K):
    print(f"swiglu dtype={dtype} M={M} N={N} K={K}", flush=True)
    gen = torch.Generator().manual_seed(M + N + K)
    x, xd = _act((M, K), gen, dtype)
    w = _rand((2 * N, K), gen, 0.02, dtype)
    g = x.double().numpy() @ w[:N].double().numpy().T
    u = x.double().numpy() @ w[N:].double().numpy().T
    ref = g / (1 + np.exp(-g)) * u
    planes = 2 if dtype == BF16 else 1
    out = torch.zeros(planes * M * N, dtype=torch.bfloat16 if dtype == BF16 else torch.float32,
                      device="cuda")
    ws = _ws(E.op_linear_workspace(dtype, 2, M, N, K))
    E.op_linear(dtype, 2, xd, _dev_weight(w, dtype), out, M, N, K, ws)
    torch.cuda.synchronize()
    got = _from_planes(out, (M, N), dtype)
    tol = 1e-5 * np.abs(ref) + 1e-4 * np.abs(ref).max()
    assert np.all(np.abs(got - ref) <= tol)


@pytest.mark.parametrize("dtype,M,V,H,k", [(BF16, 1, 32000, 4096, 10), (BF16, 10, 32000, 4096, 10),
                                           (BF16, 8, 5000, 1024, 8), (F32, 4, 1024, 256, 4),
                                           (F32, 1, 1000, 256, 16), (BF16, 40, 32000, 4096, 10),
                                           (F32, 70, 2000, 256, 5), (BF16, 90, 5000, 1024, 16),
                                           (BF16, 4, 3001, 1024, 7), (BF16, 5, 3001, 1024, 7),
                                           (BF16, 20, 32000, 4096, 10), (F32, 12, 1500, 256, 6),
                                           (BF16, 80, 32000, 4096, 10), (BF16, 10, 32000, 8192, 10)])
def test_lmhead_topk(dtype, M, V, H, k):
    print(f"topk dtype={dtype} M={M} V={V} H={H} k={k}", flush=True)
    gen = torch.Generator().manual_seed(M + V + H + k)
    x, xd = _act((M, H), gen, dtype)
    w = _rand((V, H), gen, 0.02, dtype)
    lg = x.double().numpy() @ w.double().numpy().T
    ids = torch.zeros((M, k), dtype=torch.int32, device="cuda")
    lp = torch.zeros((M, k), dtype=torch.float32, device="cuda")
    ws = _ws(E.op_lmhead_workspace(M, V, k))
    E.op_lmhead(dtype, k, xd, _dev_weight(w, dtype), M, V, H, ids, lp, None, ws)
    torch.cuda.synchronize()
    ids, lp = ids.cpu().numpy(), lp.cpu().numpy()
    for r in range(M):
        order = np.lexsort((np.arange(V), -lg[r]))
        srt = lg[r][order]
        if np.min(srt[:k] - srt[1:k + 1]) < 1e-4:
            continue      # near-tie inside the top k+1: the order is not determined
        assert list(ids[r]) == list(order[:k])
        ref_lp = lg[r] - lg[r].max() - np.log(np.exp(lg[r] - lg[r].max()).sum())
        assert np.allclose(lp[r], ref_lp[ids[r]], atol=2e-5)


@pytest.mark.parametrize("dtype,M,V,H", [(BF16, 61, 32000, 4096), (BF16, 100, 3000, 1024),
                                         (F32, 17, 1024, 256), (BF16, 33, 1000, 512),
                                         (F32, 75, 777, 256), (BF16, 27, 32000, 4096),
                                         (BF16, 3, 2000, 512), (F32, 9, 999, 256)])
def test_lmhead_argmax(dtype, M, V, H):
    print(f"argmax dtype={dtype} M={M} V={V} H={H}", flush=True)
    gen = torch.Generator().manual_seed(M * V + H)
    x, xd = _act((M, H), gen, dtype)
    w = _rand((V, H), gen, 0.02, dtype)
    lg = x.double().numpy() @ w.double().numpy().T
    g = torch.zeros(M, dtype=torch.int32, device="cuda")
    mg = torch.zeros(M, dtype=torch.float32, device="cuda")
    logits = torch.zeros((M, V), dtype=torch.float32, device="cuda")
    ws = _ws(E.op_lmhead_workspace(M, V, 0))
    E.op_lmhead(dtype, 0, xd, _dev_weight(w, dtype), M, V, H, g, mg, logits, ws)
    torch.cuda.synchronize()
    g, mg, logits = g.cpu().numpy(), mg.cpu().numpy(), logits.cpu().double().numpy()
    assert _rel(logits, lg) < 1e-4
    srt = np.sort(lg, axis=1)
    ref_margin = srt[:, -1] - srt[:, -2]
    ok = ref_margin > 1e-4
    assert np.array_equal(g[ok], np.argmax(lg, axis=1)[ok])
    assert np.allclose(mg, ref_margin, atol=2e-4)


# residual update + sliced RMSNorm + the projection that applies the rows'
# RMSNorm factors (eagle_op_norm_linear), one case per launch form the
# decoder layers take: (epilogue, M, N, H, planes)
NORM_LINEAR = [
    (0, 27, 12288, 4096, 16),   # 27 verify rows: six-wave q|k|v plan, factors through LDS
    (0, 27, 4096, 4096, 8),     # eight waves, eight splits
    (0, 61, 12288, 4096, 8),    # four m-tiles
    (0, 65, 6144, 4096, 5),     # five m-tiles: factors in registers
    (0, 108, 4096, 4096, 2),    # two 64-row m-chunks
    (0, 216, 12288, 4096, 4),   # many rows: rows_kernel
    (0, 61, 10240, 8192, 3),    # H = 8192: 512-thread slices
    (0, 10, 12288, 4096, 0),    # no planes (the embedding's norm)
    (0, 1, 4096, 4096, 2),      # one row (the draft's first pass)
    (0, 27, 4100, 4096, 8),     # ragged output rows (not a whole 16-row block)
    (2, 27, 11008, 4096, 8),    # SwiGLU, six waves
    (2, 65, 14336, 4096, 8),    # SwiGLU, five m-tiles
    (2, 108, 11008, 4096, 8),   # SwiGLU, two m-chunks of eight waves
    (2, 216, 11008, 4096, 16),  # SwiGLU over planes (rows_kernel + SiLU pass)
    (2, 1, 11008, 4096, 8),     # SwiGLU, one row
]


@pytest.mark.parametrize("epi,M,N,H,S", NORM_LINEAR)
def test_norm_linear(epi, M, N, H, S):
    from oracle.numerics import rmsnorm, silu
    print(f"norm_linear epi={epi} M={M} N={N} H={H} S={S}", flush=True)
    gen = torch.Generator().manual_seed(M * 17 + N + H + S + epi)
    eps = 1e-5
    h0 = torch.randn((M, H), generator=gen)
    part = torch.randn((max(S, 1), M, H), generator=gen) * 0.25
    gain = 1.0 + 0.1 * torch.randn(H, generator=gen)
    rows = 2 * N if epi == 2 else N
    w = _rand((rows, H), gen, 0.02, BF16)
    h_ref = h0.double().numpy() + part[:S].double().numpy().sum(axis=0) if S else h0.double().numpy()
    x = rmsnorm(h_ref, gain.double().numpy(), eps)
    wt = w.double().numpy()
    if epi == 2:
        ref = silu(x @ wt[:N].T) * (x @ wt[N:].T)
    else:
        ref = x @ wt.T
    wd = _dev_weight(w, BF16)
    ws = _ws(E.op_norm_linear_workspace(epi, M, N, H))
    partd, gaind = part.cuda(), gain.cuda()
    outs = []
    for _ in range(2):   # the same bits on a second run
        hd = h0.clone().cuda()
        if epi == 2:
            y = torch.zeros(2 * M * N, dtype=torch.bfloat16, device="cuda")
        else:
            y = torch.zeros(M, N, device="cuda")
        E.op_norm_linear(epi, hd, partd if S else None, S, gaind, eps, wd, y, M, N, H, ws)
        torch.cuda.synchronize()
        outs.append((hd.cpu(), y.cpu()))
    h_got = outs[0][0].double().numpy()
    assert np.abs(h_got - h_ref).max() <= 1e-6 * np.abs(h_ref).max()
    if epi == 2:
        got = _from_planes(outs[0][1], (M, N), BF16)
        tol = 1e-5 * np.abs(ref) + 1e-4 * np.abs(ref).max()
        assert np.all(np.abs(got - ref) <= tol)
    else:
        assert _rel(outs[0][1].double().numpy(), ref) < 1e-4
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][0], outs[1][0])


def test_norm_linear_rejects_bad_shapes():
    assert E.op_norm_linear_workspace(0, 27, 4096, 4000) == 0    # H not a multiple of 1024
    assert E.op_norm_linear_workspace(1, 27, 4096, 4096) == 0    # no EPI_ADD form
    assert E.op_norm_linear_workspace(2, 27, 4090, 4096) == 0    # SwiGLU N not a multiple of 16
    assert E.op_norm_linear_workspace(0, 27, 4096, 4096) > 0
