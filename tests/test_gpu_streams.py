"""Calls enqueued on two streams at once (each stream has its own scratch
memory) give the same results as the same calls made one after another."""
import pytest
import torch

from ssm_inputs import configs, generate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ss():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_18_amd import ssmscan
    ssmscan.lib()
    return ssmscan


def test_two_streams_concurrently(ss):
    print("case: two streams", flush=True)
    c1 = configs.ScanConfig("streams_a", 2, 3000, 320, 16, "bf16", "s4d_real", "per_token", 1.0, 61)
    c2 = configs.ScanConfig("streams_b", 3, 1700, 130, 16, "bf16", "lognormal", "per_token", 1.0, 62)
    cs = configs.SSD_LAYER.with_shape(name="streams_ssd", Bsz=2, L=900, Dm=256, N=128, h0_std=0.5, seed=63)
    a, b, d = generate.scan_inputs(c1, DEV), generate.scan_inputs(c2, DEV), generate.ssd_inputs(cs, DEV)
    sa = lambda **k: ss.scan_fwd(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], **k)
    sb = lambda **k: ss.scan_fwd(b["x"], b["delta"], b["A"], b["B"], b["C"], b["D"], **k)
    sd = lambda **k: ss.scan_ssd_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], 64, h_init=d["h_init"], **k)
    ya, ha = sa()
    yb, hb = sb()
    yd, hd = sd()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [(torch.empty_like(ya), torch.empty_like(ha)), (torch.empty_like(yb), torch.empty_like(hb)),
            (torch.empty_like(yd), torch.empty_like(hd))]
    for _ in range(3):
        for o in outs:
            o[0].zero_(), o[1].zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            sa(y=outs[0][0], h_final=outs[0][1])
            sd(y=outs[2][0], h_final=outs[2][1])
        with torch.cuda.stream(s2):
            sb(y=outs[1][0], h_final=outs[1][1])
        torch.cuda.synchronize()
        for (y, h), (ye, he), name in zip(outs, ((ya, ha), (yb, hb), (yd, hd)), ("scan a", "scan b", "ssd")):
            assert torch.equal(y, ye), f"{name}: y differs"
            assert torch.equal(h, he), f"{name}: h_final differs"
