"""The seeded input generator (CPU only)."""
import json
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_verify_batches_are_whole_dflash_blocks():
    blk = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["dflash_block_max"]
    for w in synth.WORKLOADS[:4]:
        assert w.T % blk == 0, w.name


def test_generator_is_deterministic_and_per_expert():
    w = synth.workload("tiny")
    a, b = synth.make_activations(w), synth.make_activations(w)
    assert np.array_equal(a["x_bf16"], b["x_bf16"]) and np.array_equal(a["logits"], b["logits"])
    g1 = synth.expert_weights_f32(w, 2)
    g2 = [m for e, *m in synth.all_expert_weights_f32(w) if e == 2][0]
    for x, y in zip(g1, g2):
        assert np.array_equal(x, y)


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-8 + 2**-20], np.float32)
    back = synth.bf16_bits_to_f32(synth.bf16_bits_from_f32(f))
    assert list(back) == [1.0, 1.0, 1.0 + 2**-6, -2.5, 1.0 + 2**-7]


def test_weight_and_activation_statistics():
    w = synth.workload("tiny")
    acts = synth.make_activations(w)
    assert abs(acts["x"].std() - 1.0) < 0.05
    g, u, d = synth.expert_weights_f32(w, 0)
    assert g.shape == (w.f, w.d) and d.shape == (w.d, w.f)
    assert abs(g.std() - 0.02) < 0.001


def test_zipf_bias_makes_top_expert_about_ten_times_median():
    w = synth.workload("share_64seq")
    logits = synth.make_activations(w)["logits"]
    top = np.argsort(-logits, axis=1, kind="stable")[:, :w.k]
    n = np.bincount(top.ravel(), minlength=w.E)
    ratio = n.max() / np.median(n)
    assert 5.0 < ratio < 20.0, ratio


def test_dflash_batches_are_seeded_distributions_with_drafts_in_range():
    a = synth.dflash_batch(3, 4, 1000, seed=7)
    b = synth.dflash_batch(3, 4, 1000, seed=7)
    c = synth.dflash_batch(3, 4, 1000, seed=8)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert not np.array_equal(a["p_target"], c["p_target"])
    assert a["draft"].shape == (3, 4) and a["draft"].dtype == np.int32
    assert a["p_draft"].shape == (3, 4, 1000) and a["p_target"].shape == (3, 5, 1000)
    assert a["u"].shape == (3, 4) and a["r"].shape == (3,)
    assert np.all((a["draft"] >= 0) & (a["draft"] < 1000))
    for p in (a["p_draft"], a["p_target"]):
        assert p.dtype == np.float32 and np.all(p >= 0)
        np.testing.assert_allclose(p.sum(axis=-1, dtype=np.float64), 1.0, atol=1e-5)
    assert np.all((a["u"] >= 0) & (a["u"] < 1)) and np.all((a["r"] >= 0) & (a["r"] < 1))


def test_dflash_drafter_tracks_the_target():
    # the drafter perturbs the target's logits slightly: most of the mass overlaps
    a = synth.dflash_batch(4, 2, 20000, seed=9)
    overlap = np.minimum(a["p_draft"], a["p_target"][:, :2]).sum(axis=-1)
    assert overlap.mean() > 0.9


def test_dflash_recipe_reproduces_the_pages_coding_acceptance_length():
    # the synthetic drafter is calibrated to the pages' coding figure: the
    # oracle's acceptance pass over 512 synthetic sequences accepts about
    # 6.3 of 8 drafted tokens (standard error of the mean ~0.1)
    import oracle
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    d = synth.dflash_batch(512, facts["dflash_block_max"], 8192, seed=4001)
    n, _ = oracle.dflash_accept(d["draft"], d["p_draft"], d["p_target"], d["u"], d["r"])
    assert abs(n.mean() - facts["acceptance_length_coding"]) < 0.5, n.mean()
