"""Pins of the oracle's model arithmetic to independent library routines.

The Llama layer (RMSNorm, rotate-half RoPE, GQA attention, SwiGLU) is checked
against torch's functional ops and against the `transformers` Llama model
loaded with the same synthetic weights; the rounding helpers against torch's
own bf16 conversion.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import numerics as N
from oracle.model import Config, Draft, Target, Weights, argmax_lowest, attention, causal_vis


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(50_000) * np.exp(rng.uniform(-20, 20, 50_000))
    x = np.concatenate([x, [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 65504.0]])
    want = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(N.to_bf16(x), want)


def test_rmsnorm_silu_logsoftmax_match_torch():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((5, 64)) * 3
    g = rng.standard_normal(64)
    want = torch.nn.functional.rms_norm(torch.from_numpy(h), (64,), torch.from_numpy(g), eps=1e-5)
    assert np.allclose(N.rmsnorm(h, g, 1e-5), want.numpy(), rtol=1e-13, atol=0)
    x = rng.standard_normal(1000) * 10
    assert np.allclose(N.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-300)
    z = rng.standard_normal((3, 100)) * 5
    assert np.allclose(N.log_softmax(z), torch.log_softmax(torch.from_numpy(z), -1).numpy(), rtol=1e-12)


def test_rope_preserves_norm_and_depends_on_relative_position():
    rng = np.random.default_rng(2)
    d = 64
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    dots = []
    for p, pk in [(10, 3), (107, 100), (1007, 1000)]:
        cq, sq = N.rope_tables([p], d, 10000.0)
        ck, sk = N.rope_tables([pk], d, 10000.0)
        qr, kr = N.apply_rope(q, cq, sq), N.apply_rope(k, ck, sk)
        assert np.linalg.norm(qr) == pytest.approx(np.linalg.norm(q), rel=1e-6)
        dots.append(float(np.sum(qr * kr)))
    assert dots[0] == pytest.approx(dots[1], rel=1e-5) and dots[0] == pytest.approx(dots[2], rel=1e-5)
    c0, s0 = N.rope_tables([0], d, 10000.0)
    assert np.array_equal(N.apply_rope(q, c0, s0), q)   # position 0 is the identity


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(3)
    M, S, nq, nkv, d = 7, 19, 8, 2, 16
    q = rng.standard_normal((M, nq, d))
    kc = rng.standard_normal((S, nkv, d))
    vc = rng.standard_normal((S, nkv, d))
    vis = rng.random((M, S)) < 0.6
    vis[:, 0] = True
    got = attention(q, kc, vc, vis, 1 / math.sqrt(d))
    G = nq // nkv
    kq = torch.from_numpy(np.repeat(kc, G, axis=1)).permute(1, 0, 2)
    vq = torch.from_numpy(np.repeat(vc, G, axis=1)).permute(1, 0, 2)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), kq, vq, attn_mask=torch.from_numpy(vis))
    assert np.allclose(got, want.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def _hf_llama(w, W):
    from transformers import LlamaConfig, LlamaForCausalLM
    c = Config(w)
    hc = LlamaConfig(vocab_size=c.vocab, hidden_size=c.hidden, intermediate_size=c.ffn,
                     num_hidden_layers=c.n_layers, num_attention_heads=c.n_heads,
                     num_key_value_heads=c.n_kv_heads, rms_norm_eps=c.eps,
                     rope_theta=c.rope_base, max_position_embeddings=4096,
                     tie_word_embeddings=False, attention_bias=False, mlp_bias=False,
                     hidden_act="silu")
    hc._attn_implementation = "eager"
    model = LlamaForCausalLM(hc).to(torch.float64).eval()
    t = lambda kind, grp, l=0: torch.from_numpy(W.get(kind, grp, l).astype(np.float64))
    S = synth
    with torch.no_grad():
        model.model.embed_tokens.weight.copy_(t(S.EMBED, S.GLOBAL))
        model.lm_head.weight.copy_(t(S.LM_HEAD, S.GLOBAL))
        model.model.norm.weight.copy_(t(S.FINAL_NORM, S.GLOBAL))
        for i, L in enumerate(model.model.layers):
            L.input_layernorm.weight.copy_(t(S.ATTN_NORM, S.TARGET, i))
            L.post_attention_layernorm.weight.copy_(t(S.FFN_NORM, S.TARGET, i))
            L.self_attn.q_proj.weight.copy_(t(S.WQ, S.TARGET, i))
            L.self_attn.k_proj.weight.copy_(t(S.WK, S.TARGET, i))
            L.self_attn.v_proj.weight.copy_(t(S.WV, S.TARGET, i))
            L.self_attn.o_proj.weight.copy_(t(S.WO, S.TARGET, i))
            L.mlp.gate_proj.weight.copy_(t(S.WGATE, S.TARGET, i))
            L.mlp.up_proj.weight.copy_(t(S.WUP, S.TARGET, i))
            L.mlp.down_proj.weight.copy_(t(S.WDOWN, S.TARGET, i))
    return model


@pytest.mark.parametrize("name", ["c1", "c4"])
def test_target_matches_transformers_llama(name):
    """Whole target forward (fp32 contract) vs transformers' Llama in fp64."""
    w = synth.workloads.get("c1") if name == "c1" else synth.workloads.mini("c4")
    w["dtype"] = "f32"
    W = Weights(Config(w))
    model = _hf_llama(w, W)
    toks = synth.prompt(5, 20, w["vocab"])
    with torch.no_grad():
        want = model(torch.from_numpy(toks[None].astype(np.int64))).logits[0].numpy()
    tgt = Target(Config(w), W)
    n = len(toks)
    kv = tgt.new_kv(n)
    f, _ = tgt.forward(toks, np.arange(n), np.arange(n), causal_vis(n, 0, n), kv)
    got = tgt.logits(f)
    err = np.abs(got - want).max() / np.abs(want).max()
    assert err < 2e-5
    assert np.array_equal(argmax_lowest(got)[0], np.argmax(want, axis=1))


def test_argmax_ties_go_to_lowest_id():
    g, margin = argmax_lowest(np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]]))
    assert list(g) == [1, 0] and list(margin) == [0.0, 0.0]


def test_draft_topk_order_and_logp():
    w = synth.workloads.mini("c3")
    c = Config(w)
    d = Draft(c, Weights(c))
    rng = np.random.default_rng(4)
    out = rng.standard_normal((3, c.hidden))
    ids, lp, lg = d.topk(out, 10)
    for r in range(3):
        order = sorted(range(c.vocab), key=lambda v: (-lg[r, v], v))[:10]
        assert list(ids[r]) == order
        full = lg[r].astype(np.float64)
        ref = full - np.log(np.sum(np.exp(full)))
        assert np.allclose(lp[r], ref[ids[r]], atol=2e-6)
    assert np.all(np.diff(lp, axis=1) <= 0)
