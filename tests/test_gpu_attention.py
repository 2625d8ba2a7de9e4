"""Kernel-level parity of the attention kernels (eagle_op_attention) with the
oracle's attention at the contexts the workloads reach: the split-KV form
with tree masks (verify rows after 2048 keys with 32 heads; 4096 keys with
GQA 32/8; 1280 keys with GQA 64/8), the one-pass form on a 512-row prefill
chunk after a 3072-key prefix, draft-style rows (keys from slot 1, a few tree
keys), ragged context lengths, and the fp32 kernel.

Inputs are seeded; K/V go through a shuffled page table. The oracle gets the
exact values the kernels see (for bf16 the hi + lo operand planes, summed in
fp64) and computes softmax(q k^T / sqrt(d)) v over each row's visible keys
([E2] "The Mask Preserves Tree Semantics in One Target Pass": each row sees
the context, its ancestors and itself)."""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

E = pytest.importorskip("speculative_decoding_draft_amd")

BF16, F32 = 1, 0
PAGE = 64


def _planes(x, dtype):
    """(device operand planes, exact fp64 value) of an fp32 tensor."""
    if dtype == F32:
        return [x], x.double()
    hi = x.to(torch.bfloat16)
    lo = (x - hi.float()).to(torch.bfloat16)
    return [hi, lo], hi.double() + lo.double()


def _random_tree(n, gen):
    """Parents of n verify rows (row 0 the root, parent[r] < r) and each
    row's ancestor set as a 128-bit mask (bit j = tree row j)."""
    parent = [-1] + [int(torch.randint(0, r, (1,), generator=gen)) for r in range(1, n)]
    masks = np.zeros((n, 2), dtype=np.uint64)
    anc = []
    for r in range(n):
        a, j = [], r
        while j >= 0:
            a.append(j)
            j = parent[j]
        anc.append(a)
        for j in a:
            masks[r, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return parent, anc, masks


def _run(dtype, nq, nkv, d, M, pre_lo, prehi, tree_base, n_tree, masks, key_end, seed):
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn((M, nq, d), generator=gen) * 1.3
    K = torch.randn((key_end, nkv, d), generator=gen) * 1.3
    Vv = torch.randn((key_end, nkv, d), generator=gen)
    qp, q64 = _planes(q, dtype)
    kp, k64 = _planes(K, dtype)
    vp, v64 = _planes(Vv, dtype)
    # paged cache: physical page perm[p] holds logical page p, planes K.., V..
    # (bf16 V planes transposed within the page). Slots no row sees -- below
    # pre_lo, and past key_end in the last page -- hold NaN in bf16 caches:
    # the kernels read whole pages and must keep those slots out of the sums.
    n_pages = (key_end + PAGE - 1) // PAGE
    perm = torch.randperm(n_pages, generator=gen)
    planes = kp + vp
    pad = n_pages * PAGE - key_end
    fill = float("nan") if dtype == BF16 else 0.0
    tiles = []
    for n_pl, pl in enumerate(planes):
        t = torch.cat([pl, torch.full((pad, nkv, d), fill, dtype=pl.dtype)]) if pad else pl.clone()
        if dtype == BF16:
            t[:pre_lo] = fill
        t = t.reshape(n_pages, PAGE, nkv, d)
        if dtype == BF16 and n_pl >= 2:
            tiles.append(t.permute(0, 2, 3, 1))   # V^T: [page, nkv, d, 64]
        else:
            tiles.append(t.permute(0, 2, 1, 3))   # [page, nkv, 64, d]
    logical = torch.stack([t.reshape(n_pages, -1) for t in tiles], dim=1)    # [page, planes, ...]
    phys = torch.empty_like(logical)
    phys[perm] = logical
    kv = phys.contiguous().cuda()
    table = perm.to(torch.int32).cuda()
    qd = torch.cat([p.reshape(-1) for p in qp]).cuda()
    out = torch.zeros(len(qp) * M * nq * d, dtype=qp[0].dtype, device="cuda")
    prehi_d = torch.tensor(prehi, dtype=torch.int32, device="cuda")
    if masks is None:
        masks = np.zeros((M, 2), dtype=np.uint64)
    mask_d = torch.from_numpy(masks.view(np.int64).reshape(-1).copy()).cuda()
    ws = torch.zeros(max(E.op_attention_workspace(dtype, M, nq, d, key_end), 256),
                     dtype=torch.uint8, device="cuda")
    E.op_attention(dtype, qd, kv, table, nkv, nq, d, M, pre_lo, prehi_d, mask_d, tree_base,
                   n_tree, key_end, 1.0 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    o = out.cpu()
    got = o.double() if dtype == F32 else o[:M * nq * d].double() + o[M * nq * d:].double()
    # visibility of each row over the key slots, for the oracle
    vis = np.zeros((M, key_end), dtype=bool)
    for r in range(M):
        vis[r, pre_lo:prehi[r]] = True
        for j in range(n_tree):
            if int(masks[r, j // 64]) >> (j % 64) & 1:
                vis[r, tree_base + j] = True
    from oracle.model import attention
    ref = attention(q64.numpy(), k64.numpy(), v64.numpy(), vis, 1.0 / math.sqrt(d))
    got = got.numpy().reshape(M, nq * d)
    ref = ref.reshape(M, nq * d)
    err = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)
    return float(err.max())


# (name, dtype, nq, nkv, d, context keys, tree rows)
VERIFY = [
    ("c3_ctx2048_m61", BF16, 32, 32, 128, 2048, 61),
    ("c4_ctx4031_m65_gqa4", BF16, 32, 8, 128, 4031, 65),
    ("c5_ctx1280_m61_gqa8", BF16, 64, 8, 128, 1280, 61),
    ("c2_ctx517_m27", BF16, 32, 32, 128, 517, 27),
    ("ragged_ctx70_m5", BF16, 32, 8, 128, 70, 5),
    ("c3_ctx700_m61_from5", BF16, 32, 32, 128, 700, 61),
    ("c1_f32_ctx96_m17", F32, 4, 4, 64, 96, 17),
]


@pytest.mark.parametrize("name,dtype,nq,nkv,d,ctx,M", VERIFY, ids=[v[0] for v in VERIFY])
def test_verify_attention(name, dtype, nq, nkv, d, ctx, M):
    """Verify rows: context [0, ctx) visible to all, tree rows at ctx + j
    under the ancestry mask."""
    print(f"attention {name}", flush=True)
    gen = torch.Generator().manual_seed(ctx + M)
    parent, anc, masks = _random_tree(M, gen)
    pre_lo = 5 if name.endswith("_from5") else 0   # a visible prefix not starting at a page
    err = _run(dtype, nq, nkv, d, M, pre_lo, [ctx] * M, ctx, M, masks, ctx + M, seed=ctx * 3 + M)
    print(f"{name}: rel err {err:.2e}", flush=True)
    assert err < 1e-3


@pytest.mark.parametrize("nq,nkv,pre_lo", [(32, 8, 0), (32, 32, 0), (32, 32, 1)])
def test_prefill_chunk_after_long_prefix(nq, nkv, pre_lo):
    """A 512-row prefill chunk after 3072 cached keys: causal rows, no tree
    keys (the one-pass form). Row r at slot 3072 + r sees slots
    pre_lo..3072 + r (pre_lo = 1: the draft's catch-up over a prompt, whose
    first token never enters the draft)."""
    print(f"flash nq={nq} nkv={nkv} pre_lo={pre_lo}", flush=True)
    P, M = 3072, 512
    err = _run(BF16, nq, nkv, 128, M, pre_lo, [P + r + 1 for r in range(M)], 0, 0, None, P + M,
               seed=nq + nkv)
    print(f"flash 512 rows after {P}: rel err {err:.2e}", flush=True)
    assert err < 1e-3


def test_draft_rows_with_tree_keys():
    """Draft-pass rows: committed draft keys from slot 1 (the first prompt
    token never enters the draft) and a few tree keys after them, each row
    seeing its own ancestors among them."""
    gen = torch.Generator().manual_seed(7)
    ctx, n_tree, M = 1601, 40, 10
    _, _, tmask = _random_tree(n_tree, gen)
    rows = torch.randperm(n_tree, generator=gen)[:M].tolist()   # rows expand these tree nodes
    masks = tmask[rows]
    err = _run(BF16, 32, 32, 128, M, 1, [ctx + 1] * M, ctx + 1, n_tree, masks, ctx + 1 + n_tree,
               seed=11)
    print(f"draft rows: rel err {err:.2e}", flush=True)
    assert err < 1e-3
