"""moe_forward captured into a HIP graph (through torch.cuda.CUDAGraph) and
replayed: after one eager call has sized the workspace, a call enqueues kernels
only, so it can be captured.  Every replay, with eager work and
synchronisation between replays and new values in the static input, must
equal the eager result bit for bit."""
import numpy as np
import pytest

from gpu_util import log, upload
from synth import make_inputs

pytestmark = pytest.mark.gpu


def _moe():
    import sparse_mixture_experts_22_amd as moe
    return moe


@pytest.mark.parametrize("T,d,f,n,K", [
    (32, 256, 384, 8, 2),     # decode form: fused routing block, weight-streaming kernels
    (2000, 192, 320, 4, 2),   # prefill form: scan/scatter, tiled GEMMs, split leftover tiles
])
def test_forward_graph_replays_match_eager(T, d, f, n, K):
    import torch
    moe = _moe()
    log(f"graph capture: T={T} d={d} f={f} n={n} K={K}")
    inp = make_inputs(T, d, f, n, K, dtype="bf16", seed=900 + T)
    dev = upload(inp)
    other = upload(make_inputs(T, d, f, n, K, dtype="bf16", seed=901 + T))
    w = (dev["Wg"], dev["W1"], dev["W3"], dev["W2"])
    x_static = dev["x"].clone()
    y_static = torch.empty((T, d), dtype=torch.float32, device=x_static.device)

    ref_a = moe.forward(dev["x"], *w, K).clone()          # eager; also sizes the workspace
    ref_b = moe.forward(other["x"], *w, K).clone()
    torch.cuda.synchronize()
    assert not torch.equal(ref_a, ref_b)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(x_static, *w, K, y=y_static)         # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        moe.forward(x_static, *w, K, y=y_static)

    for rep in range(4):
        src, ref = (dev["x"], ref_a) if rep % 2 == 0 else (other["x"], ref_b)
        x_static.copy_(src)
        y_static.fill_(float("nan"))
        g.replay()
        # eager work of the program between replays (another layer call and torch ops)
        scratch = moe.forward(other["x"], *w, K)
        _ = (scratch * 2.0).sum()
        torch.cuda.synchronize()
        assert torch.equal(y_static, ref), f"replay {rep} differs"
    assert np.isfinite(y_static.cpu().numpy()).all()


@pytest.mark.parametrize("T,d,f,n,K", [
    (32, 256, 384, 8, 2),     # decode form: weight streaming on packed weights
    (2000, 256, 384, 4, 2),   # prefill form: the work-list GEMMs, whose counters the router clears
])
def test_forward_packed_graph_replays_match_eager(T, d, f, n, K):
    import torch
    moe = _moe()
    log(f"graph capture (packed): T={T} d={d} f={f} n={n} K={K}")
    inp = make_inputs(T, d, f, n, K, dtype="bf16", seed=950 + T)
    dev = upload(inp)
    other = upload(make_inputs(T, d, f, n, K, dtype="bf16", seed=951 + T))
    p13 = moe.pack_up(dev["W1"], dev["W3"])
    p2 = moe.pack_down(dev["W2"])
    x_static = dev["x"].clone()
    y_static = torch.empty((T, d), dtype=torch.float32, device=x_static.device)

    ref_a = moe.forward_packed(dev["x"], dev["Wg"], p13, p2, f, K).clone()
    ref_b = moe.forward_packed(other["x"], dev["Wg"], p13, p2, f, K).clone()
    torch.cuda.synchronize()
    assert not torch.equal(ref_a, ref_b)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward_packed(x_static, dev["Wg"], p13, p2, f, K, y=y_static)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        moe.forward_packed(x_static, dev["Wg"], p13, p2, f, K, y=y_static)

    for rep in range(4):
        src, ref = (dev["x"], ref_a) if rep % 2 == 0 else (other["x"], ref_b)
        x_static.copy_(src)
        y_static.fill_(float("nan"))
        g.replay()
        # eager work between replays, including another call that uses (and leaves behind) the work lists
        scratch = moe.forward_packed(other["x"], dev["Wg"], p13, p2, f, K)
        _ = (scratch * 2.0).sum()
        torch.cuda.synchronize()
        assert torch.equal(y_static, ref), f"replay {rep} differs"
    assert np.isfinite(y_static.cpu().numpy()).all()


def test_graph_replays_after_the_workspace_grows():
    # a graph captured over a small call keeps addressing the workspace it was
    # captured with; a later, larger call grows the workspace, and the outgrown
    # buffer must stay valid for the graph's replays (it is freed only by
    # moe_release, which this test does not call)
    import torch
    moe = _moe()
    T, d, f, n, K = 32, 256, 384, 8, 2
    inp = make_inputs(T, d, f, n, K, dtype="bf16", seed=77)
    dev = upload(inp)
    w = (dev["Wg"], dev["W1"], dev["W3"], dev["W2"])
    torch.cuda.synchronize()
    moe.release()  # start from no workspace, so the calls below size it from small to large
    x_static = dev["x"].clone()
    y_static = torch.empty((T, d), dtype=torch.float32, device=x_static.device)
    ref = moe.forward(dev["x"], *w, K).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(x_static, *w, K, y=y_static)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        moe.forward(x_static, *w, K, y=y_static)
    # a much larger call: needs more workspace than any call since the release
    Tb = 4 * 1024 * 1024 // (K * (2 * f + 4 * d)) * 64   # a few hundred MiB of intermediates
    need = moe.workspace_bytes(Tb, d, f, n, K)
    log(f"growth call: T={Tb} workspace {need / 2**20:.0f} MiB")
    xb = torch.randn((Tb, d), device=x_static.device).to(torch.bfloat16)
    yb = moe.forward(xb, *w, K)
    torch.cuda.synchronize()
    assert torch.isfinite(yb).all()
    del yb, xb
    torch.cuda.empty_cache()
    # torch may now hand out memory; the graph must still use its own workspace
    filler = torch.full((64 << 20,), 3.0, device=x_static.device)
    for rep in range(3):
        y_static.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_static, ref), f"replay {rep} after growth differs"
    del filler
