"""Full-size parity at the batch-32 ragged, LLaMA temperature-1 and gpt-oss long-context
shapes, on sampled requests.

Every request's cache is filled with seeded synthetic K/V (device RNG); a few sampled
requests' contexts are then injected through the library from their target features (the
oracle recomputes the injection), and for the other sampled requests the oracle reads the
same cache contents back from the device.  The whole batch is drafted in one call in the
workspace configuration a caller at that batch would use.  Checks on the sampled requests:
draft ids bit-exact except near-ties, logit error within half the near-tie band, the
top-1/top-2 gap (recomputed from the GPU logits and as the library reports it) within the
band of the oracle's, greedy verify of planted targets bit-exact; on every request: greedy
verify bit-exact against the oracle's prefix matcher.  The LM-head entry point runs alone on
every request's 15 rows of seeded hidden states at the full vocabulary.  The temperature-1 verify runs at its full size (64 x 16 x 128256)
against the oracle on every request.  Tolerances as in test_gpu_parity."""
import numpy as np
import pytest
import torch

import oracle.dflash_oracle as ref
from block_diffusion_drafter_hidden_amd import Drafter, binding as B
from tests import gpu_setup as G
from workloads import WORKLOADS, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not G.gpu_available(), reason="needs a GPU")]


def sampled_requests(wl, n):
    rng = np.random.Generator(np.random.PCG64(synth.stream_seed(wl.seed, wl.name + "/sample")))
    return rng.choice(wl.batch, size=n, replace=False).tolist()


def weights64(w):
    """Host weights widened to float64 once (the embedding stays bf16: two rows are read)."""
    return {k: (v if k == "embed" else ref.f64(v)) for k, v in w.items()}


def build_batch(wl, injected, tag):
    cfg = wl.cfg
    ctx = synth.context_lengths(wl)
    print(f"[{tag}] {wl.name}: batch {wl.batch}, contexts {ctx.min()}..{ctx.max()}, "
          f"injected {injected}", flush=True)
    w = synth.drafter_weights(cfg, seed=wl.seed)
    wd = {k: v.to("cuda") for k, v in w.items()}
    table, num_pages = synth.page_table(f"{wl.name}/{tag}", ctx + 16, cfg.page_size, wl.seed,
                                        spare_pages=3)
    dr = Drafter(cfg, wd, max_batch=wl.batch, max_ctx=table.shape[1] * cfg.page_size,
                 max_inject_rows=256)
    del wd
    cache = dr.new_cache(table, ctx, num_pages)
    G.fill_cache(cache, wl.seed, tag)                 # synthetic K/V of every request
    feats = {}
    for b in injected:
        T = int(ctx[b])
        feats[b] = synth.target_features(cfg, T, f"{tag}/ctx/b{b}", seed=wl.seed)
        dr.inject(cache, feats[b].to("cuda"), torch.full((T,), b, dtype=torch.int32,
                                                         device="cuda"),
                  torch.arange(T, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    return cfg, w, dr, cache, ctx, table, feats


def lm_head_check(tag, cfg, dr, w64, rows, seed):
    """dflash_lm_head_argmax at the full vocabulary on `rows` seeded hidden rows (the
    128/256-row kernels): sampled rows' logits against the oracle's final norm + LM head,
    ids bit-exact except at near-ties."""
    y = synth.normal(f"{tag}/lm-rows", (rows, cfg.hidden), std=1.5, seed=seed)
    ids = torch.empty(rows, dtype=torch.int32, device="cuda")
    logits = torch.empty((rows, cfg.vocab), dtype=torch.float32, device="cuda")
    B.lm_head_argmax(dr.ccfg, dr.packed, y.cuda(), ids, dr.ws, logits)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(synth.stream_seed(seed, tag + "/lm-sample")))
    sample = np.union1d([0, rows - 1], rng.choice(rows, 62, replace=False))
    yn = ref.rms_norm(ref.f64(y)[sample], w64["final_norm"], cfg.rms_eps)
    want = yn @ w64["lm_head"].T
    idx, v1, v2 = ref.top2(want)
    got = logits.cpu().numpy()[sample]
    err = np.abs(got - want)
    tie = (v1 - v2) < 2e-2
    bad = int(((ids.cpu().numpy()[sample] != idx) & ~tie).sum())
    print(f"[{tag}] LM head {rows} rows x {cfg.vocab}: logit error max {err.max():.3e} "
          f"mean {err.mean():.3e}, mismatches {bad}, near-ties {int(tie.sum())}", flush=True)
    assert bad == 0 and err.max() <= G.LOGIT_MAX


def draft_and_check(wl, n_injected, n_pool, tag, lm_rows=None):
    sampled = sampled_requests(wl, n_injected + n_pool)
    injected = sampled[:n_injected]
    cfg, w, dr, cache, ctx, table, feats = build_batch(wl, injected, tag)
    w64 = weights64(w)
    del w
    Bn = wl.batch
    anchors = synth.anchor_ids(cfg, Bn, wl.seed, tag=f"{tag}-anchor")
    ids = torch.full((Bn, 15), -7, dtype=torch.int32, device="cuda")
    gap = torch.full((Bn, 15), -1.0, dtype=torch.float32, device="cuda")
    logits = torch.empty((Bn, 15, cfg.vocab), dtype=torch.float32, device="cuda")
    dr.draft(cache, torch.from_numpy(anchors).cuda(), ids, logits, top2_gap=gap)
    torch.cuda.synchronize()
    ids_h, gap_h = ids.cpu().numpy(), gap.cpu().numpy()
    assert ((ids_h >= 0) & (ids_h < cfg.vocab)).all() and (gap_h >= 0).all()
    orc_ids, orc_gaps = {}, {}
    for b in sorted(sampled):
        how = "injected" if b in injected else "read back"
        print(f"[{tag}] oracle request {b} (context {int(ctx[b])}, {how})", flush=True)
        lg_b = logits[b].cpu().numpy()
        if b in injected:
            own = ref.prefill_context(cfg, w64, feats[b])
            T = int(ctx[b])
            rng = np.random.Generator(np.random.PCG64(b))
            pos = np.union1d(rng.choice(T, min(T, 496), replace=False), np.arange(T - 16, T))
            gk, gv = G.pool_context(cache, table, b, T)
            exact_k, exact_v = ref.prefill_context(cfg, w64, feats[b][pos], positions=pos,
                                                   precision="exact")
            for l in range(cfg.n_layers):
                for gg, e in ((gk[l][pos], exact_k[l]), (gv[l][pos], exact_v[l])):
                    ok, info = G.cache_matches(gg, e, cfg.dtype)
                    assert ok, (b, l, info)
            del gk, gv, exact_k, exact_v
            orc = G.check_injected_request(tag, cfg, w64, b, int(anchors[b]), ids_h[b], lg_b,
                                           gap_h[b], own)
            del own
        else:
            ks, vs = G.pool_context(cache, table, b, int(ctx[b]))
            orc = ref.draft_block(cfg, w64, ks, vs, int(anchors[b]), want_logits=True)
            del ks, vs
            G.check_request(tag, b, ids_h[b], lg_b, gap_h[b], orc, cfg.dtype)
        orc_ids[b] = orc["ids"]
        orc_gaps[b] = (orc["gap"], orc["top1"], orc["top2"])
    del logits
    # The same draft without logits: past 4 requests the LM head then multiplies the hi
    # piece of its input alone and recomputes exactly the columns that can still be among a
    # row's top two.  Ids and gaps against the oracle on the sampled requests, and against
    # the call above (both exact fp32 evaluations, in different orders) on every request.
    ids2 = torch.full((Bn, 15), -7, dtype=torch.int32, device="cuda")
    gap2 = torch.full((Bn, 15), -1.0, dtype=torch.float32, device="cuda")
    dr.draft(cache, torch.from_numpy(anchors).cuda(), ids2, None, top2_gap=gap2)
    torch.cuda.synchronize()
    ids2_h, gap2_h = ids2.cpu().numpy(), gap2.cpu().numpy()
    same = ids2_h == ids_h
    print(f"[{tag}] draft without logits: {int((~same).sum())} ids differ from the logits "
          f"call (gaps there {gap_h[~same]}), gap difference max "
          f"{np.abs(gap2_h - gap_h)[same].max():.3e}", flush=True)
    assert (same | (gap_h < 1e-3)).all()
    assert np.abs(gap2_h - gap_h)[same].max() < 1e-3
    for b in sorted(sampled):
        orc_b = {"ids": orc_ids[b], "gap": orc_gaps[b][0], "top1": orc_gaps[b][1],
                 "top2": orc_gaps[b][2]}
        bad, _ = G.compare_ids(ids2_h[b], orc_b, cfg.dtype)
        agree = ids2_h[b] == orc_ids[b]
        assert bad == 0 and (np.abs(gap2_h[b] - orc_gaps[b][0])[agree] < G.GAP_TOL).all()
    # Greedy verify of the whole batch against planted targets (the sampled requests' targets
    # are planted from the oracle's drafts, the others from the GPU's).
    base = np.stack([orc_ids.get(b, ids_h[b]) for b in range(Bn)])
    t, k = synth.planted_targets(base, cfg.vocab, f"{tag}-plant", wl.seed)
    acc = torch.empty(Bn, dtype=torch.int32, device="cuda")
    bon = torch.empty_like(acc)
    B.verify_accept(ids, torch.from_numpy(t).cuda(), acc, bon)
    torch.cuda.synchronize()
    acc_h, bon_h = acc.cpu().numpy(), bon.cpu().numpy()
    for b in range(Bn):
        want = ref.verify_greedy(ids_h[b], t[b])
        assert (int(acc_h[b]), int(bon_h[b])) == want[:2], b
    for b in sampled:   # and against the oracle's own drafts, unless a near-tie intervenes
        want = ref.verify_greedy(orc_ids[b], t[b])
        first_diff = next((j for j in range(15) if ids_h[b][j] != orc_ids[b][j]), 15)
        if first_diff >= want[0]:
            assert int(acc_h[b]) == want[0] == int(k[b]) + 1
    if lm_rows:
        lm_head_check(tag, cfg, dr, w64, lm_rows, wl.seed)


def test_qwen3_8b_shape_batch32_ragged_paged():
    draft_and_check(WORKLOADS["qwen3_b32"], 2, 6, "b32", lm_rows=480)


def test_qwen3_8b_shape_batch8_deep_ksplits():
    # 128 rows at the Qwen3-8B width: the Q|K|V and O GEMMs split K four ways and the down
    # projection eight ways (few output blocks), so every k-split reduction runs at its
    # largest slice count.
    from workloads import QWEN3_8B, Workload
    wl = Workload("qwen3-8b-shaped-b16-drafter-batch8-ctx256..1024", QWEN3_8B, batch=8,
                  ctx=(256, 1024), seed=5)
    draft_and_check(wl, 2, 1, "b8")


def test_llama_shape_batch64_ctx4096_draft_logits():
    draft_and_check(WORKLOADS["llama_b64"], 1, 3, "b64", lm_rows=960)


def test_gpt_oss_shape_batch128_ctx32768():
    draft_and_check(WORKLOADS["gptoss_b128"], 1, 3, "b128", lm_rows=1920)


def test_temperature1_verify_full_size():
    wl = WORKLOADS["llama_b64"]
    dl, tl, ud, ua, ur = synth.sampled_verify_inputs(wl)
    Bn, V = dl.shape[0], dl.shape[2]
    print(f"[t1] batch {Bn} vocab {V}", flush=True)
    dev = lambda x: torch.as_tensor(x).cuda().contiguous()
    d_ids = torch.empty((Bn, 15), dtype=torch.int32, device="cuda")
    acc = torch.empty(Bn, dtype=torch.int32, device="cuda")
    emi = torch.empty((Bn, 16), dtype=torch.int32, device="cuda")
    ws = torch.empty(B.verify_sampled_workspace_size(Bn, V), dtype=torch.uint8, device="cuda")
    B.verify_accept_sampled(dev(dl), dev(tl), dev(ud), dev(ua), dev(ur), d_ids, acc, emi, ws)
    torch.cuda.synchronize()
    d_h, a_h, e_h = d_ids.cpu().numpy(), acc.cpu().numpy(), emi.cpu().numpy()
    excused = 0
    for b in range(Bn):
        o = ref.verify_sampled(dl[b], tl[b], ud[b], ua[b], float(ur[b]))
        if any(m[2] <= G.SAMPLED_MARGIN for m in o["margins"]):
            excused += 1
            continue
        np.testing.assert_array_equal(d_h[b], o["draft_ids"])
        assert a_h[b] == o["accept_len"], b
        assert list(e_h[b, :a_h[b]]) == o["emitted"] and (e_h[b, a_h[b]:] == -1).all(), b
    print(f"[t1] excused requests {excused}", flush=True)
    assert excused <= Bn // 10
