"""HIP graph capture of libssmscan calls: every replay must equal the eager
result, with eager work and synchronisations between replays."""
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


def test_scan_replays_match_eager(ss):
    print("case: scan graph replay", flush=True)
    cfg = configs.ScanConfig("graph_scan", 2, 700, 192, 16, "bf16", "s4d_real", "per_token", 1.0, 31)
    inp = generate.scan_inputs(cfg, DEV)
    y_eager, h_eager = ss.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y = torch.empty_like(y_eager)
    hf = torch.empty_like(h_eager)
    with torch.cuda.stream(s):
        # scratch memory is per (device, stream): size it before capturing
        ss.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], y=y, h_final=hf)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ss.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], y=y, h_final=hf)
    for k in range(4):
        y.zero_()
        hf.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {k}: y differs"
        assert torch.equal(hf, h_eager), f"replay {k}: h_final differs"
        # eager work between replays
        y2, _ = ss.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"])
        torch.cuda.synchronize()
        assert torch.equal(y2, y_eager)


def test_step_replays_match_eager(ss):
    print("case: decode graph replay", flush=True)
    cfg = configs.DECODE_256x8192.with_shape(Bsz=8, Dm=512)
    st = generate.step_state(cfg, DEV)
    toks = generate.step_tokens(cfg, st, 3)
    h0 = st["h"].clone()

    def eager_steps(h, n):
        ys = []
        for i in range(n):
            t = toks[i % 3]
            ys.append(ss.step(t["x"], t["delta"], st["A"], t["B"], t["C"], st["D"], h))
        return ys

    hg = h0.clone()
    ybuf = [torch.empty(8, 512, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(3):
            t = toks[i]
            ss.step(t["x"], t["delta"], st["A"], t["B"], t["C"], st["D"], hg, y=ybuf[i])
    # capture does not execute: hg is still h0
    assert torch.equal(hg, h0)
    he = h0.clone()
    for k in range(4):
        g.replay()
        torch.cuda.synchronize()
        ye = eager_steps(he, 3)
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(ybuf[i], ye[i]), f"replay {k}, step {i}: y differs"
        assert torch.equal(hg, he), f"replay {k}: state differs"


def test_packed_scan_replays_match_eager(ss):
    print("case: packed scan graph replay", flush=True)
    lengths = [100, 0, 333, 1, 250]
    cfg = configs.ScanConfig("graph_packed", 1, sum(lengths), 192, 16, "bf16", "s4d_real", "per_token", 1.0, 41)
    inp = generate.scan_inputs(cfg, DEV)
    x, dl, B, C = (inp[k][0] for k in ("x", "delta", "B", "C"))
    cu = generate.cu_seqlens(lengths, DEV)
    h0 = torch.randn((len(lengths), 192, 16), device=DEV)
    args = (x, dl, inp["A"], B, C, inp["D"], cu)
    y_eager, h_eager = ss.scan_varlen_fwd(*args, h_init=h0)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y = torch.empty_like(y_eager)
    hf = torch.empty_like(h_eager)
    with torch.cuda.stream(s):
        ss.scan_varlen_fwd(*args, h_init=h0, y=y, h_final=hf)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ss.scan_varlen_fwd(*args, h_init=h0, y=y, h_final=hf)
    for k in range(3):
        y.zero_()
        hf.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {k}: y differs"
        assert torch.equal(hf, h_eager), f"replay {k}: h_final differs"
        y2, _ = ss.scan_varlen_fwd(*args, h_init=h0)
        torch.cuda.synchronize()
        assert torch.equal(y2, y_eager)
