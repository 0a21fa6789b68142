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


def _replay_check(ss_call, outs, eager, reps=3):
    """Capture ss_call (writing into outs) on a side stream and compare every
    replay with the eager tensors, with eager work between replays."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ss_call()  # scratch memory is per (device, stream): size it before capturing
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ss_call()
    for k in range(reps):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"replay {k}: output {i} differs"
        ss_call()  # eager work between replays (on the current stream)
        torch.cuda.synchronize()


def test_ssd_replays_match_eager(ss):
    print("case: scalar-decay layer graph replay", flush=True)
    cfg = configs.SSD_LAYER.with_shape(name="graph_ssd", Bsz=2, L=500, Dm=192, N=64, h0_std=0.5, seed=51)
    inp = generate.ssd_inputs(cfg, DEV)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], 64)
    ss.set_option(ss.SSM_OPT_SEGMENT_LEN, 128)
    try:
        y_e, h_e = ss.scan_ssd_fwd(*args, h_init=inp["h_init"])
        torch.cuda.synchronize()
        y, hf = torch.empty_like(y_e), torch.empty_like(h_e)
        _replay_check(lambda: ss.scan_ssd_fwd(*args, h_init=inp["h_init"], y=y, h_final=hf), (y, hf), (y_e, h_e))
    finally:
        ss.set_option(ss.SSM_OPT_SEGMENT_LEN, 0)


def test_complex_scan_replays_match_eager(ss):
    print("case: complex scan graph replay", flush=True)
    cfg = configs.ScanConfig("graph_cplx", 2, 400, 130, 16, "bf16", "s4d_real", "per_token", 1.0, 52)
    inp = generate.scan_inputs(cfg, DEV)
    A = generate.complex_A(130, 16, 53, DEV)
    args = (inp["x"], inp["delta"], A, inp["B"], inp["C"], inp["D"])
    y_e, h_e = ss.scan_complex_fwd(*args)
    torch.cuda.synchronize()
    y, hf = torch.empty_like(y_e), torch.empty_like(h_e)
    _replay_check(lambda: ss.scan_complex_fwd(*args, y=y, h_final=hf), (y, hf), (y_e, h_e))


def test_backward_replays_match_eager(ss):
    print("case: backward graph replay", flush=True)
    cfg = configs.ScanConfig("graph_bwd", 2, 300, 130, 16, "bf16", "lognormal", "per_token", 1.0, 54)
    inp = generate.scan_inputs(cfg, DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(55)
    dy = torch.randn(inp["x"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], dy)
    eager = ss.scan_bwd(*args)
    torch.cuda.synchronize()
    names = sorted(k for k, v in eager.items() if v is not None)
    out = {k: torch.empty_like(eager[k]) for k in names}
    _replay_check(lambda: ss.scan_bwd(*args, out=out), [out[k] for k in names], [eager[k] for k in names])


def test_complex_backward_replays_match_eager(ss):
    print("case: complex backward graph replay", flush=True)
    cfg = configs.ScanConfig("graph_cbwd", 2, 300, 130, 16, "bf16", "s4d_real", "per_token", 1.0, 56)
    inp = generate.scan_inputs(cfg, DEV)
    A = generate.complex_A(130, 16, 57, DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(58)
    dy = torch.randn(inp["x"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    h0 = torch.complex(torch.randn((2, 130, 16), generator=gen, device=DEV),
                       torch.randn((2, 130, 16), generator=gen, device=DEV))
    dhf = torch.complex(torch.randn((2, 130, 16), generator=gen, device=DEV),
                        torch.randn((2, 130, 16), generator=gen, device=DEV))
    args = (inp["x"], inp["delta"], A, inp["B"], inp["C"], inp["D"], dy)
    eager = ss.scan_complex_bwd(*args, h_init=h0, dh_final=dhf)
    torch.cuda.synchronize()
    names = sorted(k for k, v in eager.items() if v is not None)
    out = {k: torch.empty_like(eager[k]) for k in names}
    _replay_check(lambda: ss.scan_complex_bwd(*args, h_init=h0, dh_final=dhf, out=out), [out[k] for k in names],
                  [eager[k] for k in names])


def test_packed_backward_replays_match_eager(ss):
    print("case: packed backward graph replay", flush=True)
    cfg = configs.PackedConfig("graph_pbwd", 1500, 130, 16, "bf16", "s4d_real", "per_token", 1.0, mean_len=200,
                               max_len=600, p_empty=0.1, h0_std=0.5, seed=59)
    inp = generate.packed_inputs(cfg, DEV)
    nseq = inp["cu"].numel() - 1
    gen = torch.Generator(device=DEV)
    gen.manual_seed(60)
    dy = torch.randn(inp["x"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    dhf = torch.randn((nseq, 130, 16), generator=gen, device=DEV)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["cu"], dy)
    eager = ss.scan_varlen_bwd(*args, h_init=inp["h_init"], dh_final=dhf)
    torch.cuda.synchronize()
    names = sorted(k for k, v in eager.items() if v is not None)
    out = {k: torch.empty_like(eager[k]) for k in names}
    _replay_check(lambda: ss.scan_varlen_bwd(*args, h_init=inp["h_init"], dh_final=dhf, out=out),
                  [out[k] for k in names], [eager[k] for k in names])


def test_captured_scratch_survives_a_larger_eager_call(ss):
    """A graph keeps the address of the stream's scratch buffer.  A later,
    larger eager call on the same stream must not free that buffer (it is
    kept until ssm_release_workspaces), so replays stay correct."""
    print("case: capture, larger eager call on the capture stream, replay", flush=True)
    small = configs.ScanConfig("graph_small", 2, 700, 192, 16, "bf16", "s4d_real", "per_token", 1.0, 61)
    large = configs.ScanConfig("graph_large", 4, 6000, 640, 16, "bf16", "lognormal", "per_token", 1.0, 62)
    si = generate.scan_inputs(small, DEV)
    li = generate.scan_inputs(large, DEV)
    sargs = (si["x"], si["delta"], si["A"], si["B"], si["C"], si["D"])
    largs = (li["x"], li["delta"], li["A"], li["B"], li["C"], li["D"])
    y_e, h_e = ss.scan_fwd(*sargs)
    yl_e, hl_e = ss.scan_fwd(*largs)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y, hf = torch.empty_like(y_e), torch.empty_like(h_e)
    yl, hl = torch.empty_like(yl_e), torch.empty_like(hl_e)
    with torch.cuda.stream(s):
        ss.scan_fwd(*sargs, y=y, h_final=hf)  # sizes the stream's scratch for the small call only
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ss.scan_fwd(*sargs, y=y, h_final=hf)
    for k in range(3):
        with torch.cuda.stream(s):
            ss.scan_fwd(*largs, y=yl, h_final=hl)  # grows the scratch of stream s (first time)
            filler = torch.full((16 << 20,), float(k + 1), device=DEV)  # reuses freed memory if any
        s.synchronize()
        assert torch.equal(yl, yl_e) and torch.equal(hl, hl_e)
        y.zero_()
        hf.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_e), f"replay {k}: y differs"
        assert torch.equal(hf, h_e), f"replay {k}: h_final differs"
        del filler
    del g
    torch.cuda.synchronize()
    ss.release_workspaces()


def test_capture_with_too_little_scratch_is_refused(ss):
    """A capturing call never allocates or synchronises: with no scratch yet
    on the stream it fails with SSM_ERR_CAPTURE and records nothing."""
    print("case: capture without sized scratch", flush=True)
    cfg = configs.ScanConfig("graph_unsized", 2, 500, 128, 16, "bf16", "s4d_real", "per_token", 1.0, 63)
    inp = generate.scan_inputs(cfg, DEV)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"])
    y_e, h_e = ss.scan_fwd(*args)
    torch.cuda.synchronize()
    y, hf = torch.empty_like(y_e), torch.empty_like(h_e)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(ss.SSMError) as err:
        with torch.cuda.graph(g, stream=s):
            ss.scan_fwd(*args, y=y, h_final=hf)
    assert err.value.code == 10  # SSM_ERR_CAPTURE
    torch.cuda.synchronize()
    # the stream works normally afterwards
    with torch.cuda.stream(s):
        ss.scan_fwd(*args, y=y, h_final=hf)
    s.synchronize()
    assert torch.equal(y, y_e) and torch.equal(hf, h_e)
