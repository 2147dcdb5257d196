"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a closed form, a library routine on a
special case, an invariant, brute force or a hand-written case from the pages'
rules.  `test_pins_catch_planted_mistakes` plants plausible mistakes in the
oracle (on the CPU) and checks that the pins notice them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.dflash_oracle as ref
from tests import torch_reference as tref
from workloads import TINY, scaled, synth

HERE = os.path.dirname(os.path.abspath(__file__))

SMALL = scaled(TINY, name="pin-small", n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2,
               head_dim=16, intermediate=96, vocab=257, n_feat_layers=3, target_hidden=32)


def small_model(cfg=SMALL, seed=0):
    # Larger init std than the workloads so that every term moves the logits visibly.
    return synth.drafter_weights(cfg, seed=seed, std=0.2, gain_std=0.2)


def context(cfg, w, T, seed=0):
    feats = synth.target_features(cfg, T, f"ctx{T}", seed=seed)
    return ref.prefill_context(cfg, w, feats)


# ------------------------------------------------------------------------------------------
# Fusion and KV injection
# ------------------------------------------------------------------------------------------

def test_fuse_one_hot_selects_columns():
    """Closed form: fusing the unit vector e_f returns column f of W_fuse."""
    w = synth.normal("fuse-w", (8, 12), dtype="f32")
    X = np.eye(12)[[3, 0, 11]]
    c = ref.fuse_features(X, w)
    np.testing.assert_array_equal(c, w.double().numpy()[:, [3, 0, 11]].T)


def test_injection_equals_projection_of_concatenated_features():
    """Associativity: RoPE(W_k (W_fuse X)) == RoPE((W_k W_fuse) X) with the product
    precomputed, and likewise for V -- injection is a projection of the concatenated
    multi-layer features into each layer's K/V (KV injection, wiki and blog)."""
    cfg = SMALL
    w = small_model()
    T = 9
    X = synth.target_features(cfg, T, "assoc").double().numpy()
    pos = np.arange(T) + 5
    ks, vs = [], []
    c = ref.fuse_features(X, w["w_fuse"])
    for l in range(cfg.n_layers):
        k, v = ref.inject_kv(c, pos, w[f"wk.{l}"], w[f"wv.{l}"], cfg.n_kv_heads, cfg.head_dim,
                             cfg.rope_theta)
        Mk = w[f"wk.{l}"].double().numpy() @ w["w_fuse"].double().numpy()
        Mv = w[f"wv.{l}"].double().numpy() @ w["w_fuse"].double().numpy()
        k2 = tref.rope_complex(torch.from_numpy(X @ Mk.T).view(T, cfg.n_kv_heads, cfg.head_dim),
                               torch.from_numpy(pos), cfg.rope_theta).numpy()
        v2 = (X @ Mv.T).reshape(T, cfg.n_kv_heads, cfg.head_dim)
        np.testing.assert_allclose(k, k2, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(v, v2, rtol=1e-10, atol=1e-10)


# ------------------------------------------------------------------------------------------
# RoPE
# ------------------------------------------------------------------------------------------

def test_rope_closed_form_d4():
    """d = 4, theta = 1e4: pair (0,2) turns by pos * 1, pair (1,3) by pos * 1e-2."""
    z = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    out = ref.rope(z, np.array([2]), 1e4)[0, 0]
    a, b = 2.0, 0.02
    want = [1 * math.cos(a) - 3 * math.sin(a), 2 * math.cos(b) - 4 * math.sin(b),
            3 * math.cos(a) + 1 * math.sin(a), 4 * math.cos(b) + 2 * math.sin(b)]
    np.testing.assert_allclose(out, want, rtol=1e-14, atol=1e-14)


def test_rope_invariants():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((6, 3, 16))
    pos = rng.integers(0, 5000, 6)
    np.testing.assert_array_equal(ref.rope(z, np.zeros(6), 1e6), z)            # pos 0 = identity
    np.testing.assert_allclose(np.linalg.norm(ref.rope(z, pos, 1e6), axis=-1),
                               np.linalg.norm(z, axis=-1), rtol=1e-12)          # norm preserved
    q, k = rng.standard_normal((1, 1, 16)), rng.standard_normal((1, 1, 16))
    dots = []
    for shift in (0, 17, 4096):                                                 # relative position
        qa = ref.rope(q, np.array([30 + shift]), 1e4)
        kb = ref.rope(k, np.array([7 + shift]), 1e4)
        dots.append(float((qa * kb).sum()))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((5, 2, 32))
    pos = np.array([0, 1, 100, 2047, 32783])
    want = tref.rope_complex(torch.from_numpy(z), torch.from_numpy(pos), 1.5e5).numpy()
    np.testing.assert_allclose(ref.rope(z, pos, 1.5e5), want, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------------
# RMSNorm, attention
# ------------------------------------------------------------------------------------------

def test_rms_norm_closed_form_and_library():
    g = np.linspace(0.5, 1.5, 8)
    c = 3.0
    out = ref.rms_norm(np.full((1, 8), c), g, 1e-6)
    np.testing.assert_allclose(out[0], g * c / math.sqrt(c * c + 1e-6), rtol=1e-14)
    z = np.random.default_rng(3).standard_normal((4, 8))
    lib = torch.nn.functional.rms_norm(torch.from_numpy(z), (8,), torch.from_numpy(g), eps=1e-6)
    np.testing.assert_allclose(ref.rms_norm(z, g, 1e-6), lib.numpy(), rtol=1e-13)


def test_attention_against_sdpa_and_special_cases():
    rng = np.random.default_rng(4)
    R, nq, nkv, d, N = 16, 8, 2, 16, 37
    q = rng.standard_normal((R, nq, d))
    k = rng.standard_normal((N, nkv, d))
    v = rng.standard_normal((N, nkv, d))
    o = ref.attention(q, k, v)
    qt = torch.from_numpy(q).transpose(0, 1).contiguous()
    kt = torch.from_numpy(k).repeat_interleave(nq // nkv, 1).transpose(0, 1).contiguous()
    vt = torch.from_numpy(v).repeat_interleave(nq // nkv, 1).transpose(0, 1).contiguous()
    lib = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).transpose(0, 1).numpy()
    np.testing.assert_allclose(o, lib, rtol=1e-11, atol=1e-12)
    # one key -> its value, whatever the query
    o1 = ref.attention(q, k[:1], v[:1])
    np.testing.assert_allclose(o1, np.broadcast_to(v[:1].repeat(nq // nkv, 1), o1.shape),
                               rtol=1e-14)
    # identical keys -> mean of the values
    kk = np.repeat(k[:1], N, axis=0)
    o2 = ref.attention(q, kk, v)
    np.testing.assert_allclose(o2, np.broadcast_to(v.mean(0).repeat(nq // nkv, 0), o2.shape),
                               rtol=1e-12, atol=1e-13)
    # no mask: the output does not depend on the order of the keys
    perm = rng.permutation(N)
    np.testing.assert_allclose(ref.attention(q, k[perm], v[perm]), o, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------------------------
# Whole draft pass
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,nb", [(0, 16), (23, 16), (23, 8), (9, 32), (0, 32)])
def test_draft_pass_matches_independent_torch_model(T, nb):
    """With zero context the step is a plain bidirectional pre-norm transformer over the
    block; with context, the injected K/V are extra keys of every layer.  Compared with an
    independent float64 implementation built from torch library layers, at block sizes 8,
    16 and 32 (reading R22: B - 1 drafts per block)."""
    cfg = scaled(SMALL, block_size=nb) if nb != 16 else SMALL
    w = small_model()
    ks, vs = context(cfg, w, T) if T else ([], [])
    out = ref.draft_block(cfg, w, ks, vs, anchor=17, want_logits=True)
    lib = tref.draft_logits(cfg, w, ks, vs, anchor=17).numpy()
    np.testing.assert_allclose(out["logits"], lib, rtol=1e-9, atol=1e-9)
    np.testing.assert_array_equal(out["ids"], lib.argmax(-1))
    assert out["ids"].shape == (nb - 1,)


def test_block_attention_with_zero_queries_is_the_mean_value():
    """With W_q = 0 every score is 0, so each block row's attention output is the plain
    mean of the values over all T context keys and all B block keys (no mask): a closed
    form that fixes how many block keys the pass attends to, at B = 8, 16 and 32."""
    for nb, T in ((8, 5), (16, 0), (32, 7)):
        cfg = scaled(SMALL, name=f"pin-mean-{nb}", n_layers=1, block_size=nb)
        w = dict(small_model(cfg))
        w["wq.0"] = torch.zeros_like(w["wq.0"])
        assert cfg.q_dim == cfg.hidden
        w["wo.0"] = torch.eye(cfg.hidden, dtype=w["wo.0"].dtype)
        w["w_down.0"] = torch.zeros_like(w["w_down.0"])      # layer output = x + o
        feats = synth.target_features(cfg, T, f"mean{nb}") if T else None
        ks, vs = ref.prefill_context(cfg, w, feats) if T else ([], [])
        out = ref.draft_block(cfg, w, ks, vs, anchor=4, want_hidden=True)
        x0, x1 = out["hidden"][0], out["hidden"][1]
        # The block's own values, from the library: V = W_v RMSNorm(x0)
        u = torch.nn.functional.rms_norm(torch.from_numpy(x0), (cfg.hidden,),
                                         w["attn_norm.0"].double(), eps=cfg.rms_eps)
        vb = (u @ w["wv.0"].double().T).numpy().reshape(nb, cfg.n_kv_heads, cfg.head_dim)
        allv = np.concatenate([vs[0], vb], axis=0) if T else vb
        mean = allv.mean(axis=0)                                  # [n_kv, d]
        grp = cfg.n_q_heads // cfg.n_kv_heads
        o = np.concatenate([mean[h // grp] for h in range(cfg.n_q_heads)])
        np.testing.assert_allclose(x1 - x0, np.broadcast_to(o, x0.shape),
                                   rtol=1e-12, atol=1e-12)


def test_gqa_with_replicated_kv_equals_mha():
    cfg = SMALL
    w = small_model()
    T = 11
    feats = synth.target_features(cfg, T, "gqa")
    mha = scaled(cfg, n_kv_heads=cfg.n_q_heads)
    wm = dict(w)
    rep = cfg.n_q_heads // cfg.n_kv_heads
    for l in range(cfg.n_layers):
        for nm in ("wk", "wv"):
            t = w[f"{nm}.{l}"].view(cfg.n_kv_heads, cfg.head_dim, cfg.hidden)
            wm[f"{nm}.{l}"] = t.repeat_interleave(rep, 0).reshape(-1, cfg.hidden)
    a = ref.draft_block(cfg, w, *ref.prefill_context(cfg, w, feats), anchor=3, want_logits=True)
    b = ref.draft_block(mha, wm, *ref.prefill_context(mha, wm, feats), anchor=3, want_logits=True)
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=1e-11, atol=1e-11)


def test_context_order_is_irrelevant_but_positions_matter():
    """Bidirectional attention without a mask: permuting where injected entries are stored
    (the page table) changes nothing; moving the whole frame by a constant changes nothing
    either (RoPE depends on relative positions only)."""
    cfg = SMALL
    w = small_model()
    T = 20
    feats = synth.target_features(cfg, T, "perm")
    ks, vs = ref.prefill_context(cfg, w, feats)
    base = ref.draft_block(cfg, w, ks, vs, anchor=5, want_logits=True)["logits"]
    perm = np.random.default_rng(5).permutation(T)
    p = ref.draft_block(cfg, w, [k[perm] for k in ks], [v[perm] for v in vs], anchor=5,
                        want_logits=True)["logits"]
    np.testing.assert_allclose(p, base, rtol=1e-11, atol=1e-11)


def test_argmax_planted_row_and_lowest_index_tie():
    cfg = SMALL
    w = small_model()
    ks, vs = context(cfg, w, 7)
    out = ref.draft_block(cfg, w, ks, vs, anchor=9, want_hidden=True)
    y = ref.rms_norm(out["hidden"][-1][1:], w["final_norm"], cfg.rms_eps)   # [15, H]
    lm = w["lm_head"].double().clone()
    r, j = 123, 4
    lm[r] = torch.from_numpy(y[j] / np.linalg.norm(y[j]) * 50.0)
    w2 = dict(w, lm_head=lm)
    o2 = ref.draft_block(cfg, w2, ks, vs, anchor=9)
    assert o2["ids"][j] == r
    lm[40] = lm[r]                      # exact duplicate at a lower index wins the tie
    o3 = ref.draft_block(cfg, dict(w, lm_head=lm), ks, vs, anchor=9)
    assert o3["ids"][j] == 40 and o3["gap"][j] == 0.0


def test_top2_second_value_against_sort():
    """top2's second value (the one every near-tie excusal rests on) equals the second
    entry of a descending library sort, on rows with distinct values, a duplicated
    maximum (gap 0) and a duplicated runner-up; the index is the lowest maximal one."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((300, 97))
    x[5, [3, 70]] = x[5].max() + 1.0                  # duplicated maximum
    srt = np.sort(x[6])[::-1]
    x[6, np.argsort(x[6])[-3]] = srt[1]               # duplicated runner-up
    idx, v1, v2 = ref.top2(x)
    desc = -np.sort(-x, axis=1)
    np.testing.assert_array_equal(v1, desc[:, 0])
    np.testing.assert_array_equal(v2, desc[:, 1])
    np.testing.assert_array_equal(idx, [int(np.nonzero(r == r.max())[0][0]) for r in x])
    assert idx[5] == 3 and v1[5] == v2[5]
    assert v2[6] == srt[1] and v1[6] - v2[6] == srt[0] - srt[1]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_draft_step_equals_draft_block_over_the_grown_context(dtype):
    """draft_step (inject the new positions, then draft, then verify) gives the same ids,
    gaps, accept length and bonus as draft_block over prefill_context of the concatenated
    features followed by verify_greedy -- injection is incremental."""
    cfg = scaled(SMALL, name=f"pin-step-{dtype}", dtype=dtype)
    w = synth.drafter_weights(cfg, seed=3, std=0.2, gain_std=0.2)
    old = synth.target_features(cfg, 11, "step-old")
    new = synth.target_features(cfg, 6, "step-new")
    ks, vs = ref.prefill_context(cfg, w, old)
    whole = ref.prefill_context(cfg, w, torch.cat([old, new], dim=0))
    want = ref.draft_block(cfg, w, *whole, anchor=13)
    t, _ = synth.planted_targets(want["ids"][None], cfg.vocab, f"step-{dtype}", k=np.array([6]))
    got = ref.draft_step(cfg, w, ks, vs, new, anchor=13, target_ids=t[0])
    np.testing.assert_array_equal(got["ids"], want["ids"])
    np.testing.assert_allclose(got["gap"], want["gap"], rtol=1e-12, atol=1e-12)
    acc, bonus, emitted = ref.verify_greedy(want["ids"], t[0])
    assert (got["accept_len"], got["bonus"], got["emitted"]) == (acc, bonus, emitted)
    assert acc == 7


def test_inv_cdf_against_searchsorted_and_fallback():
    """inv_cdf is the first index whose cumulative weight exceeds u * total (the library's
    right-sided searchsorted), never a zero-weight index; u = 1 (no cumulative sum exceeds
    the total) falls back to the last positive weight; the margin is the distance to the
    nearest cell boundary, 0 on a boundary."""
    rng = np.random.default_rng(22)
    for _ in range(200):
        w = rng.random(9) * (rng.random(9) < 0.6)
        if not w.any():
            continue
        c = np.cumsum(w)
        for u in rng.random(20):
            j, mg = ref.inv_cdf(w, float(u))
            assert j == int(np.searchsorted(c, u * c[-1], side="right"))
            assert w[j] > 0
            lo = c[j - 1] if j else 0.0
            assert mg == pytest.approx(min(u * c[-1] - lo, c[j] - u * c[-1]) / c[-1])
    w = np.array([0.0, 0.2, 0.3, 0.5, 0.0, 0.0])
    assert ref.inv_cdf(w, 1.0) == (3, 0.0)
    j, mg = ref.inv_cdf(w, 0.0)
    assert j == 1 and mg == 0.0
    j, mg = ref.inv_cdf(w, 0.5)                           # exactly on the 2|3 boundary
    assert j == 3 and mg == 0.0


# ------------------------------------------------------------------------------------------
# Input-fusion variant (reading R21)
# ------------------------------------------------------------------------------------------

def _fusion_case(dtype="f32", T=21, seed=4):
    cfg = scaled(SMALL, name=f"pin-fusion-{dtype}", dtype=dtype)
    w = synth.drafter_weights(cfg, seed=seed, std=0.2, gain_std=0.2)
    feats = synth.target_features(cfg, T, f"fusion{T}", seed=seed)
    return cfg, w, feats


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_input_fusion_matches_independent_torch_model(dtype):
    """The input-fusion prefill equals an independent float64 torch model (library layers,
    causal scaled_dot_product_attention); in bf16 mode both sides cast the cached K/V and
    attend to the cast values.  Layer 0 is exact; later layers carry the two sides'
    different bf16 casts (the torch side rounds through float32) in rare elements."""
    cfg, w, feats = _fusion_case(dtype)
    ks, vs = ref.prefill_input_fusion(cfg, w, feats)
    tk, tv = tref.input_fusion_kv(cfg, w, feats, bf16=dtype == "bf16")
    for l in range(cfg.n_layers):
        for a, b in ((ks[l], tk[l].numpy()), (vs[l], tv[l].numpy())):
            assert a.shape == (feats.shape[0], cfg.n_kv_heads, cfg.head_dim)
            if dtype == "f32":
                np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)
            else:
                np.testing.assert_array_equal(ref.round_bf16(a), a)
                close = np.isclose(a, b, rtol=2 ** -7, atol=1e-9)
                assert close.all() and (a != b).mean() < 0.01


def test_input_fusion_is_causal():
    """Row t's cache entries depend on context rows 0..t only: the prefill of a prefix is
    the prefix of the prefill (every layer), and changing one row changes the later rows'
    K/V from layer 1 on (through attention) but no earlier row's, and no other row's
    layer-0 K/V (nothing mixes positions before the first attention)."""
    cfg, w, feats = _fusion_case(T=19)
    ks, vs = ref.prefill_input_fusion(cfg, w, feats)
    for t in (1, 7, 16):
        pk, pv = ref.prefill_input_fusion(cfg, w, feats[:t])
        for l in range(cfg.n_layers):
            np.testing.assert_allclose(pk[l], ks[l][:t], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(pv[l], vs[l][:t], rtol=1e-12, atol=1e-12)
    f2 = feats.clone()
    f2[9] = f2[9] + 1.0
    k2, v2 = ref.prefill_input_fusion(cfg, w, f2)
    for l in range(cfg.n_layers):
        np.testing.assert_array_equal(k2[l][:9], ks[l][:9])
        np.testing.assert_array_equal(v2[l][:9], vs[l][:9])
        assert np.abs(k2[l][9] - ks[l][9]).max() > 1e-3
        later = np.abs(v2[l][10:] - vs[l][10:]).max(axis=(1, 2))
        if l == 0:
            assert later.max() == 0.0
        else:
            assert later.min() > 1e-6


def test_input_fusion_one_position_context():
    """A one-position context: attention over a single key returns that key's value
    exactly (its softmax weight is 1), so each layer is the block-free pass
    x += W_o [v of the head's KV group] + MLP, written here with library layers; the
    cached K/V follow from it.  This ties the layer residual structure, the head grouping
    of the value and the norm placement to a closed form."""
    cfg, w, feats = _fusion_case(T=1)
    ks, vs = ref.prefill_input_fusion(cfg, w, feats)
    F_ = torch.nn.functional
    dbl = lambda t: t.detach().to(torch.float64)
    x = F_.linear(dbl(feats), dbl(w["w_fuse"]))
    grp = cfg.n_q_heads // cfg.n_kv_heads
    for l in range(cfg.n_layers):
        u = F_.rms_norm(x, (cfg.hidden,), dbl(w[f"attn_norm.{l}"]), eps=cfg.rms_eps)
        k = F_.linear(u, dbl(w[f"wk.{l}"])).view(1, cfg.n_kv_heads, cfg.head_dim)
        v = F_.linear(u, dbl(w[f"wv.{l}"])).view(1, cfg.n_kv_heads, cfg.head_dim)
        np.testing.assert_allclose(ks[l], k.numpy(), rtol=1e-11, atol=1e-11)   # RoPE(0) = id
        np.testing.assert_allclose(vs[l], v.numpy(), rtol=1e-11, atol=1e-11)
        o = v.repeat_interleave(grp, dim=1).reshape(1, -1)
        x = x + F_.linear(o, dbl(w[f"wo.{l}"]))
        u = F_.rms_norm(x, (cfg.hidden,), dbl(w[f"mlp_norm.{l}"]), eps=cfg.rms_eps)
        x = x + F_.linear(F_.silu(F_.linear(u, dbl(w[f"w_gate.{l}"]))) *
                          F_.linear(u, dbl(w[f"w_up.{l}"])), dbl(w[f"w_down.{l}"]))


def _fusion_error():
    cfg, w, feats = _fusion_case(T=21)
    ks, vs = ref.prefill_input_fusion(cfg, w, feats)
    tk, tv = tref.input_fusion_kv(cfg, w, feats)
    return max(float(np.abs(a - b.numpy()).max()) for a, b in zip(ks + vs, tk + tv))


@pytest.mark.parametrize("mutation", ["no_mask", "mask_excludes_self", "mask_one_ahead",
                                      "scale", "kv_group"])
def test_input_fusion_pins_catch_planted_mistakes(monkeypatch, mutation):
    assert _fusion_error() < 1e-9
    orig = ref.causal_attention

    def masked(allow_fn):
        def attn(q, k, v):
            N, n_q, d = q.shape
            grp = n_q // k.shape[1]
            allowed = allow_fn(N)
            out = np.empty((N, n_q, d))
            for h in range(n_q):
                s = q[:, h] @ k[:, h // grp].T / math.sqrt(d)
                s = np.where(allowed, s, -1e300)
                p = np.where(allowed, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
                p /= np.maximum(p.sum(axis=1, keepdims=True), 1e-300)
                out[:, h] = p @ v[:, h // grp]
            return out
        return attn

    if mutation == "no_mask":
        monkeypatch.setattr(ref, "causal_attention", masked(lambda N: np.ones((N, N), bool)))
    elif mutation == "mask_excludes_self":
        monkeypatch.setattr(ref, "causal_attention",
                            masked(lambda N: np.tril(np.ones((N, N), bool), -1) | (np.eye(N, dtype=bool) & (np.arange(N) == 0)[:, None])))
    elif mutation == "mask_one_ahead":
        monkeypatch.setattr(ref, "causal_attention", masked(lambda N: np.tril(np.ones((N, N), bool), 1)))
    elif mutation == "scale":
        monkeypatch.setattr(ref, "causal_attention", lambda q, k, v: orig(q * 2.0, k, v))
    elif mutation == "kv_group":
        monkeypatch.setattr(ref, "causal_attention",
                            lambda q, k, v: orig(q, k[:, ::-1].copy(), v[:, ::-1].copy()))
    assert _fusion_error() > 1e-4, mutation


# ------------------------------------------------------------------------------------------
# bf16 storage points (reading R19)
# ------------------------------------------------------------------------------------------

def test_round_bf16_matches_library_conversion():
    """Round-to-nearest-even to bf16, checked against torch's float32 -> bfloat16 cast on
    float32 inputs, including exact halfway cases and values across many binades."""
    rng = np.random.default_rng(10)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    expo = (bits >> 7) & 0xFF
    bits = bits[(expo >= 1) & (expo <= 253)]                      # normal, far from overflow
    halfway = ((bits << 16) | 0x8000).view(np.float32)           # exactly between two bf16
    for v in (x, halfway):
        want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
        np.testing.assert_array_equal(ref.round_bf16(v.astype(np.float64)), want)


def test_bf16_model_matches_torch_model_with_the_same_casts():
    """A bf16 drafter (reading R19: bf16 KV cache, full-precision activations) computed by
    the oracle equals an independent torch float64 model that casts its cached K/V to
    bf16; and it stays within bf16 noise of the exact model while differing from it (the
    rounding is really applied)."""
    cfg = scaled(SMALL, name="pin-small-bf16", dtype="bf16")
    w = synth.drafter_weights(cfg, seed=0, std=0.2, gain_std=0.2)
    feats = synth.target_features(cfg, 19, "bf16pin")
    ks, vs = ref.prefill_context(cfg, w, feats)
    tk, tv = tref.context_kv(cfg, w, feats, bf16=True)
    for a, b in zip(ks + vs, tk + tv):
        np.testing.assert_array_equal(a, b.numpy())
        np.testing.assert_array_equal(ref.round_bf16(a), a)
    out = ref.draft_block(cfg, w, ks, vs, anchor=11, want_logits=True)
    lib = tref.draft_logits(cfg, w, tk, tv, anchor=11).numpy()
    np.testing.assert_allclose(out["logits"], lib, rtol=1e-9, atol=1e-9)
    exact = ref.draft_block(cfg, w, *ref.prefill_context(cfg, w, feats, precision="exact"),
                            anchor=11, want_logits=True, precision="exact")["logits"]
    diff = np.abs(exact - out["logits"]).max() / np.abs(exact).max()
    assert 1e-5 < diff < 5e-2


# ------------------------------------------------------------------------------------------
# Greedy verify
# ------------------------------------------------------------------------------------------

def test_verify_greedy_hand_cases():
    with open(os.path.join(HERE, "golden", "verify_greedy_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        acc, bonus, emitted = ref.verify_greedy(c["draft"], c["target"])
        assert (acc, bonus, emitted) == (c["accept_len"], c["bonus"], c["emitted"]), c["why"]


def test_verify_greedy_brute_force_over_all_match_masks():
    """All 2^15 patterns of which drafts equal the target: accept_len = 1 + number of
    trailing ones of the mask = position of the first mismatch + 1, always in [1, 16]."""
    rng = np.random.default_rng(6)
    for mask in range(1 << 15):
        d = rng.integers(0, 1000, 15)
        t = np.append(d.copy(), 7)
        for i in range(15):
            if not (mask >> i) & 1:
                t[i] = d[i] + 1
        acc, bonus, emitted = ref.verify_greedy(d, t)
        first_zero = next((i for i in range(15) if not (mask >> i) & 1), 15)
        assert acc == first_zero + 1 and 1 <= acc <= 16
        assert bonus == t[first_zero] and emitted == list(d[:first_zero]) + [t[first_zero]]


def test_planted_targets_pin_accept_length():
    d = synth.uniform_ints("plant-d", (64, 15), 0, 99)
    t, k = synth.planted_targets(d, 100, "plant")
    for b in range(64):
        assert ref.verify_greedy(d[b], t[b])[0] == k[b] + 1
    t, k = synth.planted_targets(d, 100, "plant-full", k=np.full(64, 15))
    assert all(ref.verify_greedy(d[b], t[b])[0] == 16 for b in range(64))


# ------------------------------------------------------------------------------------------
# Temperature-1 verify
# ------------------------------------------------------------------------------------------

def _cells(w):
    """Cut points of the inverse-CDF partition of [0, 1) for weights w."""
    c = np.cumsum(w) / np.sum(w)
    return np.concatenate([[0.0], c])


def _mid(lo, hi):
    return 0.5 * (lo + hi)


def test_verify_sampled_preserves_target_distribution_exactly():
    """Exact enumeration over the cells of the uniforms for one draft position and a
    4-token vocabulary: P(first emitted token = x) = p(x), the distribution-preservation
    property of the blog's 'How it works' section, for several (q, p) pairs."""
    rng = np.random.default_rng(7)
    for trial in range(12):
        dl = rng.standard_normal((1, 4)) * 2.0
        tl = rng.standard_normal((2, 4)) * 2.0
        q, p = ref.softmax(dl[0]), ref.softmax(tl[0])
        prob = np.zeros(4)
        qc = _cells(q)
        for j in range(4):                                    # draft cell -> d = j
            ud = _mid(qc[j], qc[j + 1])
            ratio = min(1.0, p[j] / q[j])
            for ua, wa in ((ratio * 0.5, ratio), (ratio + (1 - ratio) * 0.5, 1 - ratio)):
                if wa <= 0:
                    continue
                r = np.maximum(p - q, 0)
                rc = _cells(r) if r.sum() > 0 else _cells(p)
                for x in range(4):                            # resample cell -> x
                    wr = rc[x + 1] - rc[x]
                    if wr <= 0:
                        continue
                    o = ref.verify_sampled(dl, tl, [ud], [ua], _mid(rc[x], rc[x + 1]))
                    prob[o["emitted"][0]] += q[j] * wa * wr
        np.testing.assert_allclose(prob, p, rtol=1e-12, atol=1e-14)


def test_verify_sampled_equal_distributions_always_accept():
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((16, 50))
    for s in range(20):
        ud, ua = rng.random(15), rng.random(15)
        o = ref.verify_sampled(logits[:15], logits, ud, ua, rng.random())
        assert o["accept_len"] == 16 and len(o["emitted"]) == 16
        assert o["emitted"][:15] == list(o["draft_ids"])


def test_verify_sampled_monte_carlo_second_position():
    """Two draft positions, 3-token vocabulary, 20000 seeded draws: the second emitted
    token (when there is one) follows p_2 (chi-square at the 1e-4 level)."""
    rng = np.random.default_rng(9)
    dl = rng.standard_normal((2, 3)) * 1.5
    tl = rng.standard_normal((3, 3)) * 1.5
    p2 = ref.softmax(tl[1])
    counts = np.zeros(3)
    for _ in range(20000):
        o = ref.verify_sampled(dl, tl, rng.random(2), rng.random(2), rng.random())
        if len(o["emitted"]) >= 2:
            counts[o["emitted"][1]] += 1
    n = counts.sum()
    chi2 = ((counts - n * p2) ** 2 / (n * p2)).sum()
    assert chi2 < 18.4          # chi-square, 2 dof, p = 1e-4


# ------------------------------------------------------------------------------------------
# The pins notice planted mistakes
# ------------------------------------------------------------------------------------------

def _whole_pass_error(cfg=SMALL, T=23):
    w = small_model()
    ks, vs = context(cfg, w, T)
    a = ref.draft_block(cfg, w, ks, vs, anchor=17, want_logits=True)["logits"]
    b = tref.draft_logits(cfg, w, ks, vs, anchor=17).numpy()
    return float(np.abs(a - b).max())


@pytest.mark.parametrize("mutation", ["rope_sign", "rope_interleaved", "drop_gain",
                                      "causal_mask", "kv_group", "silu_sign", "scale"])
def test_pins_catch_planted_mistakes(monkeypatch, mutation):
    assert _whole_pass_error() < 1e-8
    orig_rope, orig_rms, orig_attn, orig_silu = ref.rope, ref.rms_norm, ref.attention, ref.silu

    if mutation == "rope_sign":
        def bad(z, pos, theta):
            return orig_rope(z, -np.asarray(pos), theta)
        monkeypatch.setattr(ref, "rope", bad)
    elif mutation == "rope_interleaved":
        def bad(z, pos, theta):
            d = z.shape[-1]
            perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
            inv = np.argsort(perm)
            return orig_rope(z[..., perm], pos, theta)[..., inv]
        monkeypatch.setattr(ref, "rope", bad)
    elif mutation == "drop_gain":
        monkeypatch.setattr(ref, "rms_norm", lambda z, g, eps: orig_rms(z, np.ones_like(ref.f64(g)), eps))
    elif mutation == "causal_mask":
        def bad(q, k, v):
            return orig_attn(q, k[: k.shape[0] - 8], v[: v.shape[0] - 8])
        monkeypatch.setattr(ref, "attention", bad)
    elif mutation == "kv_group":
        def bad(q, k, v):
            return orig_attn(q, k[:, ::-1].copy(), v[:, ::-1].copy())
        monkeypatch.setattr(ref, "attention", bad)
    elif mutation == "silu_sign":
        monkeypatch.setattr(ref, "silu", lambda z: z / (1.0 + np.exp(z)))
    elif mutation == "scale":
        monkeypatch.setattr(ref, "attention", lambda q, k, v: orig_attn(q * math.sqrt(2), k, v))
    assert _whole_pass_error() > 1e-4, mutation
