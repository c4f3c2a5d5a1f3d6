"""moe_forward_noalloc (the entry point for callers that cannot allocate) on the
GPU, through the C ABI: its output against moe_forward's on the same inputs,
on two calls in a row, the second with a smaller batch, plus the size limit."""
import numpy as np
import pytest

import oracle
from gpu_util import log, upload
from parity import BF16_MAX_REL, BF16_MEAN_REL, assert_rows_close
from synth import make_inputs

pytestmark = pytest.mark.gpu


def _moe():
    import sparse_mixture_experts_22_amd as moe
    return moe


def _pair(inp, dev, T):
    """(moe_forward, moe_forward_noalloc) on the first T tokens of the upload."""
    import torch
    moe = _moe()
    x = dev["x"][:T]
    ref = moe.forward(x, dev["Wg"], dev["W1"], dev["W3"], dev["W2"], inp.K)
    y = torch.full((T, inp.d), float("nan"), dtype=torch.float32, device=x.device)
    moe.forward_noalloc(x, dev["Wg"], dev["W1"], dev["W3"], dev["W2"], inp.K, y)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), y.cpu().numpy()


@pytest.mark.parametrize("T0,T1,d,f,n,K", [
    (32, 12, 512, 1024, 8, 2),     # weight-streaming path (T*K <= 24 n)
    (96, 40, 256, 384, 8, 2),      # weight-streaming path, at its row limit
])
def test_noalloc_streaming_path_is_bitwise_forward(T0, T1, d, f, n, K):
    moe = _moe()
    inp = make_inputs(T0, d, f, n, K, dtype="bf16", seed=900 + T0)
    dev = upload(inp)
    for T in (T0, T1):  # the second call is smaller
        assert 0 < moe.noalloc_scratch_bytes(T, d, f, n, K) <= moe.NOALLOC_SCRATCH_BYTES
        ref, y = _pair(inp, dev, T)
        log(f"noalloc streaming T={T} d={d} f={f} n={n} K={K}")
        np.testing.assert_array_equal(y, ref)


def test_noalloc_tiled_path_matches_forward_and_oracle():
    # T*K = 3000 rows > 24 n: the tiled grouped GEMMs; every down-projection tile
    # runs whole here, so agreement with moe_forward is to fp32 summation order
    moe = _moe()
    T0, T1, d, f, n, K = 1500, 700, 256, 384, 8, 2
    inp = make_inputs(T0, d, f, n, K, dtype="bf16", seed=913)
    dev = upload(inp)
    for T in (T0, T1):
        need = moe.noalloc_scratch_bytes(T, d, f, n, K)
        assert 0 < need <= moe.NOALLOC_SCRATCH_BYTES
        ref, y = _pair(inp, dev, T)
        log(f"noalloc tiled T={T}: scratch {need} bytes")
        assert np.isfinite(y).all()
        assert_rows_close(y, ref, 1e-4, 1e-5, what="noalloc vs forward")
        yo = oracle.forward(inp.f64("x")[:T], inp.f64("Wg"), inp.f64("W1"), inp.f64("W3"), inp.f64("W2"), K)
        assert_rows_close(y, yo, BF16_MAX_REL, BF16_MEAN_REL, what="noalloc vs oracle")


def test_noalloc_mixtral_decode_shape():
    # the Mixtral decode batch (T = 32, d = 4096, f = 14336, n = 8, K = 2), then 8 tokens
    moe = _moe()
    T0, T1, d, f, n, K = 32, 8, 4096, 14336, 8, 2
    need = moe.noalloc_scratch_bytes(T0, d, f, n, K)
    log(f"noalloc mixtral decode: scratch {need} bytes")
    assert need <= 8 << 20
    inp = make_inputs(T0, d, f, n, K, dtype="bf16", seed=931)
    dev = upload(inp)
    for T in (T0, T1):
        ref, y = _pair(inp, dev, T)
        np.testing.assert_array_equal(y, ref)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    import torch
    moe = _moe()
    T, d, f, n, K = 20000, 512, 1024, 8, 2
    assert moe.noalloc_scratch_bytes(T, d, f, n, K) > moe.NOALLOC_SCRATCH_BYTES
    inp = make_inputs(64, d, f, n, K, dtype="bf16", seed=7)
    dev = upload(inp)
    x = torch.zeros((T, d), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, d), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoEError, match="scratch"):
        moe.forward_noalloc(x, dev["Wg"], dev["W1"], dev["W3"], dev["W2"], K, y)
    torch.cuda.synchronize()
    assert (y == 7.0).all()
