"""Decode steps, scans and backwards captured in a HIP graph (through torch's
graph capture on the stream the binding launches on): every replay, with eager work and
synchronisation between replays, must equal the plain launches bit for bit."""
import pytest

from selective_state_space_63_amd import synth
from gpu_util import problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_63_amd import s6
    s6.load_library()
    return torch


def test_decode_graph_replays(torch_cuda):
    import torch
    from selective_state_space_63_amd import s6
    w = synth.custom(5, 300, 16, 8, synth.BF16, True, seed=31)
    d, _ = problem(w, True)
    S = w.seqlen
    sl = [{k: (None if d[k] is None else d[k][..., s].contiguous()) for k in ("x", "delta", "Bm", "Cm", "z")}
          for s in range(S)]
    y = torch.empty((w.batch, w.dim), device="cuda", dtype=torch.float32)

    def run(h):
        for s in range(S):
            t = sl[s]
            s6.state_update(h, t["x"], t["delta"], d["A"], t["Bm"], t["Cm"], D=d["D"], z=t["z"], y=y)

    h_ref = d["h0"].clone()
    run(h_ref)
    y_ref = y.clone()
    torch.cuda.synchronize()

    h = d["h0"].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(h)
    for rep in range(3):
        h.copy_(d["h0"])
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, h_ref), rep
        assert torch.equal(y, y_ref), rep


def test_scan_graph_replays(torch_cuda):
    """The fused scan (with final state and training checkpoints) captured in
    a HIP graph: it allocates nothing when the rows fill the GPU, so the
    capture holds just its kernel; every replay equals the eager call bit for
    bit."""
    import torch
    from selective_state_space_63_amd import s6
    w = synth.custom(8, 2600, 16, 256, synth.BF16, True, seed=32)  # 656 row blocks: not cut into segments
    d, _ = problem(w, True)
    y = torch.empty((w.batch, w.dim, w.seqlen), device="cuda", dtype=torch.float32)
    hl = torch.empty((w.batch, w.dim, w.dstate), device="cuda", dtype=torch.float32)
    ck = torch.empty(s6.ckpt_shape(w.batch, w.dim, w.seqlen, w.dstate), device="cuda", dtype=torch.float32)

    def run():
        s6.scan_fwd(d["x"], d["delta"], d["A"], d["Bm"], d["Cm"], D=d["D"], z=d["z"], h0=d["h0"], y=y, h_last=hl,
                    return_last_state=True, ckpt=ck)

    run()
    torch.cuda.synchronize()
    refs = (y.clone(), hl.clone(), ck.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for t in (y, hl, ck):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip((y, hl, ck), refs):
            assert torch.equal(t, r), rep


def _replay_check(torch, g, outs, refs, reps=3):
    """Replays g `reps` times with eager work (clearing the outputs, an
    unrelated product) and synchronisation between replays; every replay
    must reproduce refs bit for bit."""
    for rep in range(reps):
        for t in outs:
            t.fill_(float("nan"))
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del junk
        for t, r in zip(outs, refs):
            assert torch.equal(t, r), rep


def test_segmented_scan_graph_replays(torch_cuda):
    """A scan of one long row of 1536 channels (48 channel blocks: the
    sequence is cut into segments whose carries live in the caller's
    workspace, here allocated by the binding inside the capture) and its
    final-state-only form, captured and replayed."""
    import torch
    from selective_state_space_63_amd import s6
    w = synth.custom(1, 1536, 16, 65536, synth.BF16, True, seed=33)
    assert s6.workspace_size("scan_fwd", w.batch, w.dim, w.seqlen, w.dstate) > 0
    print(f"[case] segmented scan graph {w.name}", flush=True)
    d = synth.device_full(w)
    h0 = torch.randn((w.batch, w.dim, w.dstate), device="cuda", dtype=torch.float32)
    y = torch.empty((w.batch, w.dim, w.seqlen), device="cuda", dtype=torch.float32)
    hl = torch.empty((w.batch, w.dim, w.dstate), device="cuda", dtype=torch.float32)
    hs = torch.empty_like(hl)

    def run():
        s6.scan_fwd(d["x"], d["delta"], d["A"], d["Bm"], d["Cm"], D=d["Dskip"], z=d["z"], h0=h0, y=y, h_last=hl,
                    return_last_state=True)
        s6.last_state(d["x"], d["delta"], d["A"], d["Bm"], h0=h0, out=hs)

    run()
    torch.cuda.synchronize()
    refs = (y.clone(), hl.clone(), hs.clone())
    # the fused scan runs its last segment from the folded incoming state, the
    # final-state scan folds that segment's aggregate too: equal to rounding
    assert torch.allclose(hl, hs, rtol=1e-5, atol=1e-6)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    _replay_check(torch, g, (y, hl, hs), refs)


def test_segmented_ssd_graph_replays(torch_cuda):
    """The scalar-A scan of one long row (3 channel tiles: cut into
    segments, state-only pass, carry fold, scan from the folded states) with
    its workspace allocated inside the capture, replayed."""
    import torch
    from selective_state_space_63_amd import s6
    w = synth.custom(1, 48, 16, 16384, synth.BF16, True, seed=35)
    assert s6.workspace_size("ssd_scan_fwd", w.batch, w.dim, w.seqlen, w.dstate) > 0
    print(f"[case] segmented scalar-A scan graph {w.name}", flush=True)
    d = synth.device_full(w)
    a = synth.scalar_a_device(w)
    h0 = torch.randn((w.batch, w.dim, w.dstate), device="cuda", dtype=torch.float32)
    y = torch.empty((w.batch, w.dim, w.seqlen), device="cuda", dtype=torch.float32)
    hl = torch.empty((w.batch, w.dim, w.dstate), device="cuda", dtype=torch.float32)

    def run():
        s6.ssd_scan_fwd(d["x"], d["delta"], a, d["Bm"], d["Cm"], D=d["Dskip"], z=d["z"], h0=h0,
                        return_last_state=True, y=y, h_last=hl)

    run()
    torch.cuda.synchronize()
    refs = (y.clone(), hl.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    _replay_check(torch, g, (y, hl), refs)


@pytest.mark.parametrize("shape", [(2, 256, 1024), (1, 64, 8192), (8, 2592, 256)], ids=["rows", "parts", "chunks"])
def test_backward_graph_replays(torch_cuda, shape):
    """The backward (checkpoint pass, adjoint kernel, fixed-order reductions;
    with few long rows also the carry pass and fold over parts; with rows
    enough to fill the GPU the sequential first pass that stores every
    chunk's state) captured with its workspace and replayed: every gradient
    equal to the eager call bit for bit."""
    import torch
    from selective_state_space_63_amd import s6
    bsz, dim, L = shape
    w = synth.custom(bsz, dim, 16, L, synth.BF16, True, seed=34)
    print(f"[case] backward graph {w.name}", flush=True)
    d, _ = problem(w, True)
    dy = torch.randn((bsz, dim, L), device="cuda", dtype=torch.float32)
    dhl = torch.randn((bsz, dim, 16), device="cuda", dtype=torch.float32)
    res = {}

    def run():
        res.update(s6.scan_bwd(d["x"], d["delta"], d["A"], d["Bm"], d["Cm"], dy, D=d["D"], z=d["z"], h0=d["h0"],
                               dh_last=dhl))

    run()
    torch.cuda.synchronize()
    keys = sorted(res)
    refs = tuple(res[k].clone() for k in keys)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    _replay_check(torch, g, tuple(res[k] for k in keys), refs)
