"""The seeded input generator: formats and workload structure (no GPU)."""
import numpy as np

import synth
from tests.oracle_pins import _golden_rows


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)  # bf16 spacing at 1.0
    vals = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + np.float32(2.0 ** -20), -2.5,
                     np.float32(3.3895313892515355e38)], np.float32)
    got = synth.bf16_from_f32(vals)
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F7F]
    assert np.array_equal(synth.f32_from_bf16(got)[:2], [1.0, 1.0])


def test_mxfp4_quantizer_rounding_and_saturation():
    # block amax 6 -> shared exponent 0; ties go to the even code; 7 saturates
    row = np.zeros((1, 32))
    row[0, :10] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.3, 0.0]
    q, s = synth.mxfp4_quantize(row)
    codes = np.empty(32, np.uint8)
    codes[0::2], codes[1::2] = q[0] & 15, q[0] >> 4
    assert s[0, 0] == 127
    assert list(codes[:10]) == [7, 0, 2, 2, 4, 4, 6, 6, 9, 0]
    q2, s2 = synth.mxfp4_quantize(np.full((1, 32), 7.0))
    assert s2[0, 0] == 127 and (q2 == 0x77).all()  # 7.0: amax exponent 0, then 7/1 saturates to 6
    q3, s3 = synth.mxfp4_quantize(np.zeros((1, 32)))
    assert s3[0, 0] == 0 and not q3.any()


def test_presets_match_page_shapes():
    """The synthetic layers carry the shapes the pages print (fixture
    tests/golden/gpt_oss_layer_shapes.txt, each value cited there)."""
    g = {k: int(v) for k, v in _golden_rows("gpt_oss_layer_shapes.txt")}
    # the page figures agree with each other
    assert g["experts_20b"] * g["layers_20b"] == g["expert_subnets_20b"]
    assert g["topk"] * g["layers_20b"] == g["subnets_firing_20b"]
    assert g["expert_width"] % 256 == g["width_mod_256"] and g["expert_width"] % 128 == g["width_mod_128"]
    c = synth.CONFIGS
    for name in ("20b_decode", "20b_prefill_zipf", "20b_mxfp4_decode", "20b_mxfp4_prefill"):
        assert (c[name].H, c[name].E, c[name].k, c[name].I) == (g["hidden"], g["experts_20b"], g["topk"],
                                                                g["expert_width"]), name
    assert (c["120b_sweep"].H, c["120b_sweep"].E, c["120b_sweep"].k) == (g["hidden"], g["experts_120b"], g["topk"])
    assert c["20b_mxfp4_prefill"].T == 32768 and c["20b_prefill_zipf"].T == 8192 and c["20b_decode"].T == 16
    assert c["20b_mxfp4_decode"].wfmt == 1 and c["20b_mxfp4_prefill"].wfmt == 1 and c["20b_decode"].wfmt == 0
    assert (c["tiny"].T, c["tiny"].H, c["tiny"].E, c["tiny"].k, c["tiny"].I) == (64, 256, 8, 2, 512)


def test_generation_is_seeded_and_deterministic():
    a = synth.make_layer("tiny")
    b = synth.make_layer("tiny")
    assert np.array_equal(a.x, b.x) and np.array_equal(a.weights.gate_up, b.weights.gate_up)
    xf = synth.f32_from_bf16(a.x)
    assert abs(xf.std() - 1.0) < 0.05
    wf = synth.f32_from_bf16(a.weights.down)
    assert abs(wf.std() - 0.02) < 0.001


def test_zipf_first_choice_share():
    """The constant-channel bias makes each expert's first-choice share track
    Zipf(1.1) on the prefill workload."""
    cfg = synth.CONFIGS["20b_prefill_zipf"]
    x = synth.make_x(cfg, T=4096)
    wr = synth.make_router(cfg)
    lg = synth.f32_from_bf16(x).astype(np.float64) @ synth.f32_from_bf16(wr).astype(np.float64).T
    first = np.bincount(lg.argmax(1), minlength=cfg.E) / lg.shape[0]
    p = synth.zipf_probs(cfg.E, cfg.zipf_s)
    assert np.all(np.abs(first[:6] - p[:6]) < 0.03), (first[:6], p[:6])
    assert first[0] > 5 * first[-1]


def test_sample_tokens():
    s = synth.sample_tokens(8192, 512, 1)
    assert len(set(s.tolist())) == 512 and s.min() >= 0 and s.max() < 8192 and np.all(np.diff(s) > 0)
    assert np.array_equal(s, synth.sample_tokens(8192, 512, 1))
    assert np.array_equal(synth.sample_tokens(16, 512, 1), np.arange(16))
