"""Closed-loop decoding on the host: the synthetic target's planting rule (numpy and device
forms agree) and the oracle's loop pinned against one-shot computations.

The loop's bookkeeping is checked against things other than itself: after any number of
iterations the context equals injecting all accepted slots' features at once (the
associativity of appending), every iteration's draft equals a fresh draft pass over that
one-shot context, and the accept lengths are the planted ones."""
import numpy as np
import torch

import oracle.dflash_oracle as ref
from workloads import TINY, scaled, synth

SMALL = scaled(TINY, name="loop-small", n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2,
               head_dim=16, intermediate=96, vocab=257, n_feat_layers=3, target_hidden=32)


def test_plant_device_matches_plant():
    V = 1000
    rng = np.random.default_rng(0)
    for trial in range(20):
        B = 7
        d = rng.integers(0, V, size=(B, 15))
        k, fill, r = synth.plant_draws(f"p{trial}", B, V, k=rng.integers(0, 16, size=B))
        k[0], k[1] = 0, 15
        t = synth.plant(d, k, fill, r, V)
        td = synth.plant_device(torch.from_numpy(d).int(), torch.from_numpy(k),
                                torch.from_numpy(fill), torch.from_numpy(r), V)
        assert np.array_equal(t, td.numpy())
        for b in range(B):
            assert ref.verify_greedy(d[b], t[b])[0] == k[b] + 1


def _loop(cfg, w, T0, iters, seed=0):
    feats0 = synth.target_features(cfg, T0, "loop/ctx", seed=seed)
    ks, vs = ref.prefill_context(cfg, w, feats0) if T0 else ([], [])
    block_feats = [synth.target_features(cfg, 16, f"loop/it{i}", seed=seed)
                   for i in range(iters)]
    draws = [synth.plant_draws(f"loop/it{i}", 1, cfg.vocab, seed) for i in range(iters)]

    def targets(i, ids):
        k, fill, r = draws[i]
        return synth.plant(ids[None], k, fill, r, cfg.vocab)[0]

    out = ref.decode_loop(cfg, w, ks, vs, 5, block_feats, targets)
    return out, feats0, block_feats, draws


def test_loop_context_equals_one_shot_injection():
    w = synth.drafter_weights(SMALL, seed=1, std=0.2, gain_std=0.2)
    for T0 in (0, 9):
        out, feats0, block_feats, draws = _loop(SMALL, w, T0, iters=4)
        acc = [rec["accept_len"] for rec in out["iterations"]]
        assert acc == [int(d[0][0]) + 1 for d in draws]            # planted lengths
        assert [rec["ctx_len"] for rec in out["iterations"]] == list(T0 + np.cumsum([0] + acc[:-1]))
        rows = [feats0] if T0 else []
        rows += [bf[:a] for bf, a in zip(block_feats, acc)]
        all_feats = torch.cat(rows)
        ks, vs = ref.prefill_context(SMALL, w, all_feats)
        assert out["ctx_len"] == all_feats.shape[0]
        for l in range(SMALL.n_layers):
            np.testing.assert_allclose(out["k_ctx"][l], ks[l], rtol=0, atol=1e-12)
            np.testing.assert_allclose(out["v_ctx"][l], vs[l], rtol=0, atol=1e-12)
        # iteration i drafts from the context of everything accepted before it
        for i, rec in enumerate(out["iterations"]):
            T = rec["ctx_len"]
            fresh = ref.draft_block(SMALL, w, [k[:T] for k in ks], [v[:T] for v in vs],
                                    rec["anchor"])
            assert np.array_equal(fresh["ids"], rec["ids"])
            nxt = out["iterations"][i + 1]["anchor"] if i + 1 < len(acc) else out["anchor"]
            assert nxt == rec["bonus"] == rec["target_ids"][rec["accept_len"] - 1]
