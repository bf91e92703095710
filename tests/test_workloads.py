"""The seeded input generator: quantisation, distributions and masks."""
import numpy as np
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 0.02,
                        g.standard_normal(1000).astype(np.float32) * 1e4,
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_determinism_and_shapes():
    a = wl.make_inputs(64, 16, 50, wl.DTYPE_BF16, 7, ignore_frac=0.25)
    b = wl.make_inputs(64, 16, 50, wl.DTYPE_BF16, 7, ignore_frac=0.25)
    assert a.H.dtype == np.uint16 and a.H.shape == (64, 16) and a.W.shape == (50, 16)
    assert np.array_equal(a.H, b.H) and np.array_equal(a.W, b.W) and np.array_equal(a.y, b.y)
    c = wl.make_inputs(64, 16, 50, wl.DTYPE_BF16, 8)
    assert not np.array_equal(a.H, c.H)
    ok = a.y[a.y != wl.IGNORE_INDEX]
    assert ok.min() >= 0 and ok.max() < 50


def test_zipf_statistics():
    g = np.random.default_rng(1)
    V = 124160
    y = wl.zipf_targets(g, 400000, V, 1.1)
    assert y.min() >= 0 and y.max() < V
    w = np.arange(1, V + 1, dtype=np.float64) ** -1.1
    p0 = w[0] / w.sum()
    assert abs((y == 0).mean() - p0) < 0.005
    assert abs((y == 1).mean() - w[1] / w.sum()) < 0.004


def test_prompt_masks_match_configs():
    c2, c4 = wl.CONFIGS[2], wl.CONFIGS[4]
    m2 = wl.prefix_mask(c2.T, c2.n_seq, c2.masked_prefix)
    assert m2.sum() == c2.T // 4 == c2.n_ignored
    assert m2[:1024].all() and not m2[1024:4096].any() and m2[4096:5120].all()
    m4 = wl.prefix_mask(c4.T, c4.n_seq, c4.masked_prefix)
    assert m4.sum() == 39321 == int(0.3 * c4.T) and m4[:39321].all() and not m4[39321:].any()


def test_config_table():
    assert [c.T for c in wl.CONFIGS] == [256, 4096, 16384, 65536, 131072]
    assert [c.V for c in wl.CONFIGS] == [1000, 32000, 151936, 124160, 124160]
    assert [c.d for c in wl.CONFIGS] == [128, 2048, 2048, 2048, 4096]
    assert wl.CONFIGS[3].counted_flops() == 8 * 65536 * 2048 * 124160
    assert wl.CONFIGS[1].scales() == (1 / 4096, 1 / 4096)
    assert wl.CONFIGS[2].scales() == (1 / 12288, 1 / 12288)


def test_config0_inputs_small():
    x = wl.config_inputs(0)
    assert x.H.dtype == np.float32 and x.H.shape == (256, 128) and x.W.shape == (1000, 128)
    assert abs(x.W.std() - 0.02) < 0.001
    rows = wl.sample_rows(0, 32)
    assert len(np.unique(rows)) == 32 and np.all(np.diff(rows) > 0)
