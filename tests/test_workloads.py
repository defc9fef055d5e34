"""The synthetic workload recipes reproduce the shapes and byte counts the pages print.

Fixture: tests/golden/page_facts.json (each entry cites its page and section).
"""
import json
import os

from synth import gen

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_decode_step_weight_bytes():
    b = gen.decode_step_weight_bytes()
    assert b == 3_087_138_816
    assert round(b / 1e9, FACTS["decode_weight_bytes_GB"]["digits"]) == FACTS["decode_weight_bytes_GB"]["value"]


def test_lm_head_and_kv_sizes():
    assert [gen.V, gen.H] == FACTS["lm_head_shape"]["value"]
    assert round(gen.V * gen.H * 2 / 1e6) == FACTS["lm_head_MB"]["value"]
    shapes = dict((n, (a, b)) for n, a, b in gen.block_shapes())
    for name in ("wk", "wv"):
        n, k = shapes[name]
        assert round(n * k * 2 / 1e6, 2) == FACTS["kv_projection_MB"]["value"]


def test_gemv_count_heads_and_cache_bytes():
    assert gen.N_LAYERS == FACTS["n_layers"]["value"]
    assert gen.N_LAYERS * len(gen.block_shapes()) + 1 == FACTS["n_gemv_per_step"]["value"]
    assert (gen.NQ, gen.NKV) == (FACTS["heads"]["value"]["q"], FACTS["heads"]["value"]["kv"])
    assert gen.NQ * gen.HEAD_DIM == gen.H
    # K and V, 2 kv heads of head_dim, BF16, every layer: bytes of cache per token
    per_token = gen.N_LAYERS * 2 * gen.NKV * gen.HEAD_DIM * 2
    assert round(per_token / 1024) == FACTS["cache_bytes_per_token_KB"]["value"]


def test_chain_recipe_shape():
    t = gen.make_stage_tensors("ln_gelu_chain_768x72", n_layers=2)
    assert t["layers"][0]["W"].shape == (768, 768)
    assert FACTS["chain_blocks"]["value"] == {"blocks": 72, "width": 768}


def test_generator_is_seeded():
    a = gen.normal((4, 5), 0.02, gen.seed_of(4, 3, 2))
    b = gen.normal((4, 5), 0.02, gen.seed_of(4, 3, 2))
    c = gen.normal((4, 5), 0.02, gen.seed_of(4, 3, 3))
    assert (a.view(-1) == b.view(-1)).all() and not (a.view(-1) == c.view(-1)).all()
