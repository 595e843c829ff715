"""Decode steps captured in a HIP graph (through torch's graph capture on the
stream the binding launches on): every replay, with eager work and
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
