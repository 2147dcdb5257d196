"""Block sizes 8 and 32, and the input-fusion prefill, through the C ABI against the oracle.

Block sizes: the drafted ids, logits and gaps of a block of 8 or 32 tokens against
oracle.draft_block with that block size (tolerances as in test_gpu_parity: fp32 ids exact
except at near-ties and logits within 1e-4 of their range; bf16 over a seeded shared cache
within gpu_setup.LOGIT_MAX), and greedy verification of 8- and 32-token blocks bit-exact.

Input-fusion prefill (the oracle's prefill_input_fusion): the cache each layer writes,
then a draft over it.  fp32: within 1e-5 of RMS.  bf16: each side stores its own bf16
rounding and the context rows attend to the stored values, so a value that one side rounds
the other way moves the next layer's inputs.  Layer 0 (no rounding upstream) takes the
injection bound (the bf16 rounding of a value within 2e-5 (|exact| + RMS), under 1% of the
values off round(exact)); from layer 1 on, an fp32-versus-fp64 evaluation of the same
prefill at the 8B shape moves the unrounded values by at most 8.8e-4 (48 positions) and
1.3e-3 (512 positions) of (|exact| + RMS), with up to 10% of the stored values one bf16
step apart, so the bound there is 5e-3 and 30%.  The draft after a bf16 prefill takes the
injected-context logit bounds of gpu_setup.check_injected_request.
"""
import numpy as np
import pytest
import torch

import oracle.dflash_oracle as ref
from block_diffusion_drafter_hidden_amd import Drafter, binding as B
from tests import gpu_setup as G
from workloads import GPT_OSS_120B, TINY, QWEN3_8B, scaled, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not G.gpu_available(), reason="needs a GPU")]

# Qwen3-8B head layout (GQA 4, d = 128) at a small width.
SMALL_BF16 = scaled(QWEN3_8B, name="variants-bf16", n_layers=2, hidden=512, n_q_heads=8,
                    n_kv_heads=2, head_dim=128, intermediate=1344, vocab=8192,
                    n_feat_layers=3, target_hidden=512)

PF_REL_LATER = 5e-3
PF_FLIPS_LATER = 0.3


# ------------------------------------------------------------------------------------------
# Block sizes 8 and 32
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("nb", [8, 32])
def test_block_sizes_tiny_f32_match_oracle(nb):
    """fp32 tiny model, injected contexts (one empty, one spanning several 32-key steps and
    a ragged tail), a block of nb tokens: nb - 1 ids per request."""
    cfg = scaled(TINY, name=f"tiny-b{nb}", block_size=nb)
    ctx = [128, 0, 45]
    print(f"[block {nb}] tiny f32 ctx {ctx}", flush=True)
    s = G.build(cfg, ctx, tag=f"blk{nb}")
    anchors = synth.anchor_ids(cfg, len(ctx), tag=f"blk{nb}-anchor")
    ids, logits, gap = G.run_draft(s, anchors, want_logits=True, want_gap=True)
    assert ids.shape == (len(ctx), nb - 1)
    for b in range(len(ctx)):
        ks, vs = G.oracle_context(s, b)
        orc = ref.draft_block(cfg, s.w, ks, vs, int(anchors[b]), want_logits=True)
        assert orc["ids"].shape == (nb - 1,)
        bad, _ = G.compare_ids(ids[b], orc, cfg.dtype)
        assert bad == 0, (b, ids[b], orc["ids"])
        err = np.abs(logits[b] - orc["logits"])
        assert err.max() <= 1e-4 * np.abs(orc["logits"]).max(), (b, err.max())
        same = ids[b] == orc["ids"]
        np.testing.assert_allclose(gap[b][same], orc["gap"][same], rtol=0,
                                   atol=2e-4 * np.abs(orc["logits"]).max())


# gpt-oss head layout (GQA 8, d = 64) and GQA 8 at d = 128, at a small width.
SMALL_OSS_BF16 = scaled(GPT_OSS_120B, name="variants-oss-bf16", n_layers=2, hidden=512,
                        n_q_heads=16, n_kv_heads=2, head_dim=64, intermediate=1024,
                        vocab=8192, n_feat_layers=3, target_hidden=512)
SMALL_G8_D128_BF16 = scaled(SMALL_BF16, name="variants-g8d128-bf16", n_q_heads=16,
                            n_kv_heads=2)
LAYOUTS = {"gqa4-d128": SMALL_BF16, "gqa8-d64": SMALL_OSS_BF16,
           "gqa8-d128": SMALL_G8_D128_BF16,
           # groups of one and two heads: fragments loaded straight from the pages
           "gqa1-d128": scaled(SMALL_BF16, name="variants-g1d128-bf16", n_q_heads=2),
           "gqa2-d64": scaled(SMALL_OSS_BF16, name="variants-g2d64-bf16", n_q_heads=4)}


@pytest.mark.parametrize("n_q,n_kv,d", [(8, 2, 64), (16, 2, 64), (4, 2, 128), (8, 2, 128)])
def test_f32_head_groups_match_oracle(n_q, n_kv, d):
    """fp32 models with the other head groups of the fp32 attention kernel (GQA 4 and 8 at
    d = 64, GQA 2 and 4 at d = 128; TINY is GQA 2 at d = 64), injected contexts spanning
    several 32-key steps with a ragged tail and an empty one: ids, logits and gaps against
    the oracle as in the TINY block-size test."""
    cfg = scaled(TINY, name=f"tiny-q{n_q}-kv{n_kv}-d{d}", n_q_heads=n_q, n_kv_heads=n_kv,
                 head_dim=d)
    ctx = [150, 0, 77]
    print(f"[f32 heads] {cfg.name} ctx {ctx}", flush=True)
    s = G.build(cfg, ctx, tag=f"f32-{cfg.name}")
    anchors = synth.anchor_ids(cfg, len(ctx), tag=f"f32-{cfg.name}-anchor")
    ids, logits, gap = G.run_draft(s, anchors, want_logits=True, want_gap=True)
    for b in range(len(ctx)):
        ks, vs = G.oracle_context(s, b)
        orc = ref.draft_block(cfg, s.w, ks, vs, int(anchors[b]), want_logits=True)
        bad, _ = G.compare_ids(ids[b], orc, cfg.dtype)
        assert bad == 0, (b, ids[b], orc["ids"])
        err = np.abs(logits[b] - orc["logits"])
        assert err.max() <= 1e-4 * np.abs(orc["logits"]).max(), (b, err.max())
        same = ids[b] == orc["ids"]
        np.testing.assert_allclose(gap[b][same], orc["gap"][same], rtol=0,
                                   atol=2e-4 * np.abs(orc["logits"]).max())


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("nb", [8, 32])
def test_block_sizes_bf16_shared_cache_match_oracle(nb, layout):
    """bf16 model with the 8B head layout (and the GQA-8 layouts of the gpt-oss shape at
    d = 64 and of d = 128, and groups of one and two heads), seeded shared cache (both sides
    read the same K/V), three requests with ragged contexts; a block of 32 is two query
    tiles per request over the same 32 block keys."""
    cfg = scaled(LAYOUTS[layout], name=f"variants-{layout}-b{nb}", block_size=nb)
    ctx = [200, 17, 0]
    print(f"[block {nb}] bf16 {layout} ctx {ctx}", flush=True)
    tag = f"blkbf{nb}" if layout == "gqa4-d128" else f"blkbf{nb}-{layout}"
    s = G.build(cfg, ctx, tag=tag, inject=False)
    G.fill_cache(s.cache, 7, tag)
    anchors = synth.anchor_ids(cfg, len(ctx), tag=f"{tag}-anchor")
    ids, logits, gap = G.run_draft(s, anchors, want_logits=True, want_gap=True)
    # The same draft without logits (at 32 tokens the 96 rows take the 256-row LM head, which
    # then multiplies the hi piece alone and recomputes the candidate columns exactly).
    a = torch.as_tensor(np.asarray(anchors, dtype=np.int32)).to("cuda")
    ids2 = torch.full((len(ctx), nb - 1), -7, dtype=torch.int32, device="cuda")
    gap2 = torch.full((len(ctx), nb - 1), -1.0, dtype=torch.float32, device="cuda")
    s.dr.draft(s.cache, a, ids2, None, top2_gap=gap2)
    torch.cuda.synchronize()
    ids2, gap2 = ids2.cpu().numpy(), gap2.cpu().numpy()
    for b in range(len(ctx)):
        ks, vs = G.pool_context(s.cache, s.table, b, int(ctx[b]))
        orc = ref.draft_block(cfg, s.w, ks, vs, int(anchors[b]), want_logits=True)
        G.check_request(f"block {nb}", b, ids[b], logits[b], gap[b], orc, cfg.dtype)
        bad, _ = G.compare_ids(ids2[b], orc, cfg.dtype)
        agree = ids2[b] == orc["ids"]
        assert bad == 0 and (np.abs(gap2[b] - orc["gap"])[agree] < G.GAP_TOL).all()


def test_block8_batched_rows_take_the_tall_kernels():
    """Five requests with 8-token blocks: 80 padded rows, so every GEMM runs the 128-row
    kernel and the LM head the 256-row kernel (with logits: both pieces; without: the hi
    piece and the refinement), with 7 drafts per request mapped out of 16-row blocks."""
    nb = 8
    cfg = scaled(SMALL_BF16, name="variants-bf16-b8x5", block_size=nb)
    ctx = [33, 0, 190, 16, 77]
    s = G.build(cfg, ctx, tag="blk8x5", inject=False)
    G.fill_cache(s.cache, 9, "blk8x5")
    anchors = synth.anchor_ids(cfg, len(ctx), tag="blk8x5-anchor")
    ids, logits, gap = G.run_draft(s, anchors, want_logits=True, want_gap=True)
    a = torch.as_tensor(np.asarray(anchors, dtype=np.int32)).to("cuda")
    ids2 = torch.full((len(ctx), nb - 1), -7, dtype=torch.int32, device="cuda")
    gap2 = torch.full((len(ctx), nb - 1), -1.0, dtype=torch.float32, device="cuda")
    s.dr.draft(s.cache, a, ids2, None, top2_gap=gap2)
    torch.cuda.synchronize()
    ids2, gap2 = ids2.cpu().numpy(), gap2.cpu().numpy()
    for b in range(len(ctx)):
        ks, vs = G.pool_context(s.cache, s.table, b, int(ctx[b]))
        orc = ref.draft_block(cfg, s.w, ks, vs, int(anchors[b]), want_logits=True)
        G.check_request("block 8 x 5", b, ids[b], logits[b], gap[b], orc, cfg.dtype)
        bad, _ = G.compare_ids(ids2[b], orc, cfg.dtype)
        agree = ids2[b] == orc["ids"]
        assert bad == 0 and (np.abs(gap2[b] - orc["gap"])[agree] < G.GAP_TOL).all()


@pytest.mark.parametrize("nb", [8, 32])
def test_verify_greedy_block_sizes_bit_exact(nb):
    Bn = 129
    d = synth.uniform_ints(f"gv{nb}-d", (Bn, nb - 1), 0, 50)
    t, k = synth.planted_targets(d, 51, f"gv{nb}")
    t[0, :nb - 1] = d[0]                   # a full match
    acc = torch.empty(Bn, dtype=torch.int32, device="cuda")
    bon = torch.empty_like(acc)
    emi = torch.empty((Bn, nb), dtype=torch.int32, device="cuda")
    B.verify_accept(torch.from_numpy(d).cuda(), torch.from_numpy(t).cuda(), acc, bon, emi)
    torch.cuda.synchronize()
    acc, bon, emi = acc.cpu().numpy(), bon.cpu().numpy(), emi.cpu().numpy()
    for b in range(Bn):
        a, bo, e = ref.verify_greedy(d[b], t[b])
        assert acc[b] == a and bon[b] == bo, b
        assert list(emi[b, :a]) == e and (emi[b, a:] == -1).all()
    assert acc[0] == nb
    np.testing.assert_array_equal(acc[1:], k[1:] + 1)


# ------------------------------------------------------------------------------------------
# Input-fusion prefill
# ------------------------------------------------------------------------------------------

def prefill_setup(cfg, lens, tag, seed=5):
    """A drafter and an empty cache with room for `lens` positions per request; features of
    every request's context."""
    lens = np.asarray(lens, dtype=np.int32)
    w = synth.drafter_weights(cfg, seed=seed)
    wd = {k: v.to("cuda") for k, v in w.items()}
    table, num_pages = synth.page_table(f"{cfg.name}/{tag}", lens + 16, cfg.page_size, seed,
                                        spare_pages=3)
    dr = Drafter(cfg, wd, max_batch=len(lens), max_ctx=table.shape[1] * cfg.page_size,
                 max_inject_rows=16)
    cache = dr.new_cache(table, np.zeros(len(lens), dtype=np.int32), num_pages)
    feats = [synth.target_features(cfg, int(T), f"{tag}/b{b}", seed=seed)
             for b, T in enumerate(lens)]
    return G.Setup(cfg, w, wd, dr, cache, lens, table, feats)


def prefill_calls(s, b, splits):
    """Prefill request b's context in calls ending at each position of `splits`, setting
    ctx_lens[b] to the start of each call (the caller advances it)."""
    start = 0
    for end in splits:
        s.cache.ctx_lens[b] = start
        print(f"[prefill] request {b}: rows {start}..{end - 1}", flush=True)
        s.dr.prefill_input_fusion(s.cache, s.feats[b][start:end].to("cuda").contiguous(), b)
        start = end
    s.cache.ctx_lens[b] = start


def check_prefill_cache(s, b, T, orc_unrounded, tag):
    ku, vu = orc_unrounded
    gk, gv = G.gather_pool(s, b, T, "k"), G.gather_pool(s, b, T, "v")
    for l in range(s.cfg.n_layers):
        for name, g, e in (("k", gk[l], ku[l][:T]), ("v", gv[l], vu[l][:T])):
            if l == 0:
                ok, info = G.cache_matches(g, e, s.cfg.dtype)
            else:
                ok, info = G.cache_matches(g, e, s.cfg.dtype, rel=PF_REL_LATER,
                                           max_flip_frac=PF_FLIPS_LATER)
            print(f"[{tag}] request {b} layer {l} {name}: {info}", flush=True)
            assert ok, (tag, b, l, name, info)


def test_prefill_input_fusion_tiny_f32_matches_oracle():
    """fp32 tiny model: request 0 prefills 2088 positions in one call (two chunks, 2048 +
    40, the second a ragged 16-row group), request 1 prefills 141 positions in two calls
    (100 + 41: the second starts inside a page and a 16-row group).  Cache of every layer,
    then a draft over it, against the oracle."""
    cfg = TINY
    s = prefill_setup(cfg, [2088, 141], "pf-tiny")
    prefill_calls(s, 0, [2088])
    prefill_calls(s, 1, [100, 141])
    anchors = synth.anchor_ids(cfg, 2, tag="pf-tiny-anchor")
    ids, logits, gap = G.run_draft(s, anchors, want_logits=True, want_gap=True)
    for b in range(2):
        T = int(s.ctx_lens[b])
        ks, vs = ref.prefill_input_fusion(cfg, s.w, s.feats[b])
        check_prefill_cache(s, b, T, (ks, vs), "prefill tiny")
        orc = ref.draft_block(cfg, s.w, ks, vs, int(anchors[b]), want_logits=True)
        bad, _ = G.compare_ids(ids[b], orc, cfg.dtype)
        assert bad == 0
        err = np.abs(logits[b] - orc["logits"])
        assert err.max() <= 1e-4 * np.abs(orc["logits"]).max(), err.max()


def test_prefill_input_fusion_edge_lengths_tiny_f32():
    """fp32 tiny model: prefills of 1 position (one group of 1 row and 15 padding rows), 16
    (one whole group) and 17 (a whole group and a 1-row group), each then drafted over;
    cache and draft against the oracle."""
    cfg = TINY
    s = prefill_setup(cfg, [1, 16, 17], "pf-edges")
    for b, T in enumerate([1, 16, 17]):
        prefill_calls(s, b, [T])
    anchors = synth.anchor_ids(cfg, 3, tag="pf-edges-anchor")
    ids, logits, gap = G.run_draft(s, anchors, want_logits=True, want_gap=True)
    for b in range(3):
        ks, vs = ref.prefill_input_fusion(cfg, s.w, s.feats[b])
        check_prefill_cache(s, b, int(s.ctx_lens[b]), (ks, vs), "prefill edges")
        orc = ref.draft_block(cfg, s.w, ks, vs, int(anchors[b]), want_logits=True)
        bad, _ = G.compare_ids(ids[b], orc, cfg.dtype)
        assert bad == 0
        assert np.abs(logits[b] - orc["logits"]).max() <= 1e-4 * np.abs(orc["logits"]).max()


def test_prefill_input_fusion_qwen_shape_bf16_matches_oracle():
    """The Qwen3-8B-shaped bf16 drafter: request 0 prefills 72 positions in one call (four
    16-row groups and a ragged half group), request 1 prefills 73 in two calls (40 + 33).
    Cache of every layer, then a draft over it, against the oracle."""
    cfg = QWEN3_8B
    s = prefill_setup(cfg, [72, 73], "pf-qwen")
    prefill_calls(s, 0, [72])
    prefill_calls(s, 1, [40, 73])
    anchors = synth.anchor_ids(cfg, 2, tag="pf-qwen-anchor")
    ids, logits, gap = G.run_draft(s, anchors, want_logits=True, want_gap=True)
    for b in range(2):
        print(f"[prefill qwen] oracle request {b}", flush=True)
        ks, vs, ku, vu = ref.prefill_input_fusion(cfg, s.w, s.feats[b], want_unrounded=True)
        check_prefill_cache(s, b, int(s.ctx_lens[b]), (ku, vu), "prefill qwen")
        G.check_injected_request("prefill qwen", cfg, s.w, b, int(anchors[b]), ids[b],
                                 logits[b], gap[b], (ks, vs))


@pytest.mark.parametrize("layout", ["gqa8-d64", "gqa8-d128", "gqa2-d64", "gqa1-d128"])
def test_prefill_input_fusion_head_layouts_bf16(layout):
    """The causal prefill with the other head layouts at a small width (GQA 8 at d = 64 and
    128 through LDS, groups of two and one head straight from the pages): request 0
    prefills 72 positions in one call, request 1 73 in two calls (40 + 33).  Cache of every
    layer, then a draft over it, against the oracle."""
    cfg = LAYOUTS[layout]
    s = prefill_setup(cfg, [72, 73], f"pf-{layout}")
    prefill_calls(s, 0, [72])
    prefill_calls(s, 1, [40, 73])
    anchors = synth.anchor_ids(cfg, 2, tag=f"pf-{layout}-anchor")
    ids, logits, gap = G.run_draft(s, anchors, want_logits=True, want_gap=True)
    for b in range(2):
        ks, vs, ku, vu = ref.prefill_input_fusion(cfg, s.w, s.feats[b], want_unrounded=True)
        check_prefill_cache(s, b, int(s.ctx_lens[b]), (ku, vu), f"prefill {layout}")
        G.check_injected_request(f"prefill {layout}", cfg, s.w, b, int(anchors[b]), ids[b],
                                 logits[b], gap[b], (ks, vs))


def test_prefill_input_fusion_2048_positions_prefix():
    """The benchmark's prefill (2048 positions of the Qwen3-8B-shaped drafter, one call):
    the cache of the first 48 positions depends on those rows only (causal attention), so it
    must match the oracle's prefill of those 48 rows; the remaining positions are checked
    for finite values in every layer."""
    cfg = QWEN3_8B
    s = prefill_setup(cfg, [2048], "pf-2048")
    prefill_calls(s, 0, [2048])
    torch.cuda.synchronize()
    print("[prefill 2048] oracle of the first 48 rows", flush=True)
    _, _, ku, vu = ref.prefill_input_fusion(cfg, s.w, s.feats[0][:48], want_unrounded=True)
    check_prefill_cache(s, 0, 48, (ku, vu), "prefill 2048")
    for which in ("k", "v"):
        g = G.gather_pool(s, 0, 2048, which)
        assert np.isfinite(g).all()
        assert (np.abs(g[:, 48:]).max(axis=(1, 2, 3)) > 0).all()
