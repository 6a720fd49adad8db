"""The seeded input generator: determinism, shapes, bf16 representability."""
import numpy as np

from workloads import CONFIGS, make_inputs, marker_tokens, small_layer_config, zipf_router_bias


def test_deterministic_and_thread_independent():
    cfg = small_layer_config(CONFIGS["small_bf16"], 3000, d=64, d_ff=32)
    a = make_inputs(cfg, threads=1)
    b = make_inputs(cfg, threads=7)
    for key in ("h", "w_router", "w1", "w2"):
        assert np.array_equal(a[key], b[key])


def test_bf16_values_are_representable():
    cfg = small_layer_config(CONFIGS["mixtral_bf16"], 64, d=128, d_ff=64)
    inp = make_inputs(cfg)
    for key in ("h", "w_router", "w1", "w2"):
        assert not (inp[key].view(np.uint32) & 0xFFFF).any()


def test_shapes_and_local_experts():
    cfg = small_layer_config(CONFIGS["ep_share_bf16"], 16, d=64, d_ff=32)
    inp = make_inputs(cfg)
    assert inp["h"].shape == (16, 64)
    assert inp["w_router"].shape == (64, 256)
    assert inp["w1"].shape == (32, 64, 64) and inp["w2"].shape == (32, 64, 32)
    assert inp["expert_ids"].tolist() == list(range(32))
    allx = make_inputs(cfg, experts="all", with_h=False)
    assert np.array_equal(allx["w1"][:32], inp["w1"])


def test_weight_scale():
    cfg = small_layer_config(CONFIGS["small_bf16"], 8)
    inp = make_inputs(cfg)
    assert abs(inp["w1"].std() * np.sqrt(cfg.d) - 1) < 0.01
    assert abs(inp["w2"].std() * np.sqrt(cfg.d_ff) - 1) < 0.01


def test_zipf_bias_monotone_and_spacing():
    b = zipf_router_bias(128, 1.2, 1.2)
    assert (np.diff(b) < 0).all()
    # 1.2 * ln(w_2 / w_1) = 1.2 * (-1.2 ln 2)
    assert abs((b[1] - b[0]) - (-1.44 * np.log(2))) < 1e-5


def test_markers_distinct():
    h = marker_tokens(64, 32)
    assert len({tuple(r) for r in h.tolist()}) == 64
