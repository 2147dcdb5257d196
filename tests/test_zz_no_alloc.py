"""dflash_draft_block_noalloc (the draft step on the library's own scratch array, for
callers that cannot allocate) against dflash_draft_block with a caller workspace: the same
kernels, so ids, top-2 gaps and logits must agree bit for bit, on two calls in a row, the
second with a smaller batch (the array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_hidden_amd import binding as B
from tests import gpu_setup as G
from workloads import WORKLOADS, scaled, synth
from workloads import TINY

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not G.gpu_available(), reason="needs a GPU")]

SMALL_BF16 = scaled(TINY, name="noalloc-small-bf16", dtype="bf16", hidden=256, head_dim=128,
                    n_q_heads=4, n_kv_heads=1, intermediate=512, vocab=4096)


def _draft(s, anchors, noalloc):
    n = len(anchors)
    a = torch.as_tensor(np.asarray(anchors, dtype=np.int32)).cuda()
    ids = torch.full((n, 15), -7, dtype=torch.int32, device="cuda")
    gap = torch.full((n, 15), -1.0, dtype=torch.float32, device="cuda")
    logits = torch.full((n, 15, s.cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        B.draft_block_noalloc(s.dr.ccfg, s.dr.packed, s.dr.embed, s.cache.c(), a, ids,
                              logits_out=logits, top2_gap=gap)
    else:
        s.dr.draft(s.cache, a, ids, logits, top2_gap=gap)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), gap.cpu().numpy(), logits.cpu().numpy()


def _same(a, b):
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("which", ["small", "qwen3_b1"])
def test_noalloc_matches_workspace_call(which):
    if which == "small":
        cfg, ctx = SMALL_BF16, [200, 0, 77, 31, 130]
    else:
        wl = WORKLOADS["qwen3_b1"]
        cfg, ctx = wl.cfg, [int(synth.context_lengths(wl)[0]), 517]
    print(f"[noalloc] {which}: contexts {ctx}", flush=True)
    s = G.build(cfg, ctx, tag=f"noalloc-{which}")
    need = B.workspace_size(s.dr.ccfg, len(ctx), 0, s.cache.max_pages * 16)
    assert need <= B.noalloc_scratch_bytes()
    anchors = synth.anchor_ids(cfg, len(ctx), tag=f"noalloc-{which}")
    want = _draft(s, anchors, noalloc=False)
    got = _draft(s, anchors, noalloc=True)
    _same(got, want)
    # A second call with a smaller batch (the first two requests' page-table rows): the
    # scratch still holds the first call's values.
    s2 = G.Setup(s.cfg, s.w, s.wd, s.dr, B.PagedCache(s.cache.k_pool, s.cache.v_pool,
                                                      s.cache.block_table[:2].contiguous(),
                                                      s.cache.ctx_lens[:2].contiguous(),
                                                      s.cache.num_pages, s.cache.max_pages),
                 s.ctx_lens[:2], s.table[:2], s.feats[:2])
    want2 = _draft(s2, anchors[:2], noalloc=False)
    got2 = _draft(s2, anchors[:2], noalloc=True)
    _same(got2, want2)
    print(f"[noalloc] {which}: ids, gaps and logits bit-identical on both calls", flush=True)
