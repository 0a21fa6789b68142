"""Seeded input generator: reproducibility, shapes, dtypes and distributions."""
import numpy as np
import torch

from ssm_inputs import configs, generate


def _small(cfg, **kw):
    return cfg.with_shape(**kw)


def test_scan_inputs_reproducible_and_shaped():
    cfg = _small(configs.MAMBA130M_LAYER, Bsz=2, L=33, Dm=40)
    a = generate.scan_inputs(cfg)
    b = generate.scan_inputs(cfg)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    assert a["x"].shape == (2, 33, 40) and a["x"].dtype == torch.bfloat16
    assert a["B"].shape == (2, 33, 16) and a["C"].dtype == torch.bfloat16
    assert a["A"].shape == (40, 16) and a["A"].dtype == torch.float32
    assert a["D"].shape == (40,) and a["D"].dtype == torch.float32
    c = generate.scan_inputs(cfg, seed=cfg.seed + 1)
    assert not torch.equal(a["x"], c["x"])


def test_delta_range_and_positivity():
    cfg = _small(configs.TINY_FP32, L=512)
    inp = generate.scan_inputs(cfg)
    d = inp["delta"]
    assert torch.all(d > 0)
    # softplus(0.5 N(0,1) + inv_softplus(u)), u in [1e-3, 1e-1]: median ~ u
    med = d.median().item()
    assert 1e-3 < med < 1e-1


def test_per_channel_delta_is_constant_in_time():
    cfg = _small(configs.LONG_CONTEXT_1M, L=64, Dm=32)
    d = generate.scan_inputs(cfg)["delta"].float()
    assert torch.equal(d, d[:, :1, :].expand_as(d))
    assert torch.all(d >= 9e-4) and torch.all(d <= 0.101)


def test_s4d_real_and_lognormal_A():
    a = generate.scan_inputs(_small(configs.TINY_FP32, L=4))["A"]
    assert torch.equal(a, -torch.arange(1, 17, dtype=torch.float32).expand(64, 16))
    r = generate.scan_inputs(_small(configs.MAMBA130M_LAYER, Bsz=1, L=4, Dm=256))["A"]
    assert torch.all(r < 0)
    lg = torch.log(-r)
    assert abs(lg.std().item() - 0.5) < 0.05


def test_inv_softplus_roundtrip():
    u = torch.tensor([1e-3, 1e-2, 0.05, 0.1, 1.0], dtype=torch.float32)
    assert torch.allclose(generate.softplus(generate.inv_softplus(u)), u, rtol=1e-5)


def test_bf16_widening_is_exact():
    """The oracle sees bf16 device values exactly: bf16 -> fp64 loses nothing."""
    x = generate.scan_inputs(_small(configs.MAMBA130M_LAYER, Bsz=1, L=8, Dm=64))["x"]
    wide = x.double().numpy()
    back = torch.from_numpy(wide).to(torch.bfloat16)
    assert torch.equal(back, x)
    assert np.array_equal(wide, x.float().numpy().astype(np.float64))


def test_decode_tokens():
    cfg = configs.DECODE_256x8192.with_shape(Bsz=4, Dm=128)
    st = generate.step_state(cfg)
    toks = generate.step_tokens(cfg, st, 3)
    assert st["h"].shape == (4, 128, 16) and st["h"].dtype == torch.float32
    assert abs(st["h"].std().item() - 0.1) < 0.01
    assert len(toks) == 3 and toks[0]["x"].shape == (4, 128) and toks[0]["B"].shape == (4, 16)
    assert not torch.equal(toks[0]["x"], toks[1]["x"])


def test_decode_state_complex():
    cfg = configs.DECODE_256x8192.with_shape(Bsz=4, Dm=128)
    st = generate.step_state_complex(cfg)
    real = generate.step_state(cfg)
    assert st["h"].dtype == torch.complex64 and st["h"].shape == (4, 128, 16)
    assert torch.equal(st["h"].real, real["h"])  # the real part is step_state's draw
    assert abs(st["h"].imag.std().item() - 0.1) < 0.01
    assert st["A"].dtype == torch.complex64 and bool((st["A"].real < 0).all())
    # complex state and A take 8 bytes per value: 2 x 134 MB of state per step at full size
    full = configs.DECODE_256x8192
    extra = 8 * full.Bsz * full.Dm * full.N + 4 * full.Dm * full.N
    assert generate.alg_bytes_step_complex(full) - generate.alg_bytes_step(full) == extra


def test_algorithmic_bytes_match_published_table():
    # inputs read once + outputs written once; the [B,L,D,N] state never counts
    assert abs(generate.alg_bytes_scan(configs.MAMBA2P8B_LAYER) / 1e6 - 2019.1) < 0.5
    assert abs(generate.alg_bytes_scan(configs.LONG_CONTEXT_1M) / 1e6 - 6509.7) < 0.5
    assert abs(generate.alg_bytes_scan(configs.MAMBA130M_LAYER) / 1e6 - 152.9) < 0.5
    assert abs(generate.alg_bytes_step(configs.DECODE_256x8192) / 1e6 - 281.6) < 0.5


def test_packed_lengths_and_offsets():
    lens = generate.packed_lengths(400, 50, seed=3, p_empty=0.1, max_len=200)
    assert len(lens) == 400 and min(lens) == 0 and max(lens) <= 200
    assert 20 <= lens.count(0) <= 70
    assert generate.packed_lengths(400, 50, seed=3, p_empty=0.1, max_len=200) == lens
    cu = generate.cu_seqlens([3, 0, 2])
    assert cu.dtype == torch.int64 and cu.tolist() == [0, 3, 3, 5]


def test_packed_config_sums_to_its_length():
    from ssm_inputs import PACKED_2P8B_LAYER as cfg
    lens = generate.packed_config_lengths(cfg)
    assert sum(lens) == cfg.L and min(lens) >= 0 and len(lens) > 10
    assert max(lens[:-1]) <= cfg.max_len
    small = cfg.__class__(**{**cfg.__dict__, "L": 3000, "Dm": 8, "mean_len": 100, "max_len": 400})
    inp = generate.packed_inputs(small)
    nseq = inp["cu"].numel() - 1
    assert inp["x"].shape == (3000, 8) and inp["B"].shape == (3000, 16)
    assert inp["h_init"].shape == (nseq, 8, 16)
    assert int(inp["cu"][0]) == 0 and int(inp["cu"][-1]) == 3000
    assert bool(torch.all(inp["cu"][1:] >= inp["cu"][:-1]))
