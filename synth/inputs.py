"""Seeded synthetic MoE-layer inputs (x, W_g, W1, W3, W2).

Recipe (stated once, used by tests and the benchmark alike):
  * generator: numpy PCG64.  ``SeedSequence(seed).spawn(5)`` gives one child per
    tensor, in the order x, W_g, W1, W3, W2.  Each tensor is drawn in blocks of
    whole rows along its first axis (R = max(1, 2**22 // elements_per_row) rows
    per block); block b uses ``default_rng(child.spawn(n_blocks)[b])``.  Blocks
    are independent, so they are drawn in parallel threads;
  * standard normals are drawn in float32 and scaled:
      x ~ N(0, 1); W_g, W1, W3 ~ N(0, 1/d); W2 ~ N(0, 1/f)   (fan-in scaling);
  * bf16 configurations round every tensor once, float32 -> bf16 with
    round-to-nearest-even; the fp32 configuration keeps float32;
  * ``routing="skewed"`` builds the router as W_g[:, i] = s_i * u_i + b_i * v with
    u_i, v ~ N(0, 1/d) (u from the W_g child's first spawned child, v from its
    second), s = (1, ..., 1, 0.1) and b = (+16, -16, ..., -16): expert 0
    wins the top-1 pick for roughly half the tokens and the last expert rarely does.

Shapes follow the layer equation of the Mixtral study deck (card 2.1): x is
[T][d], W_g is [d][n] (so logits = x @ W_g), W1 and W3 are [n][d][f], W2 is
[n][f][d].  The Mixtral model config quoted in "Why 8x7B Is Not 56B" (Part 4 of
"Mixture of Experts: Why Mixtral Only Wakes Up Two Specialists") fixes
d = 4096, f = 14336, n = 8, K = 2.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass

import numpy as np

SEED_BASE = 20240108

# name -> (T, d, f, n, K, dtype, routing, seed index)
CONFIGS = {
    "tiny_fp32": dict(T=256, d=64, f=128, n=8, K=2, dtype="f32", routing="uniform", index=0),
    "mixtral_prefill": dict(T=8192, d=4096, f=14336, n=8, K=2, dtype="bf16", routing="uniform", index=1),
    "mixtral_decode": dict(T=32, d=4096, f=14336, n=8, K=2, dtype="bf16", routing="uniform", index=2),
    "mixtral_skewed": dict(T=8192, d=4096, f=14336, n=8, K=2, dtype="bf16", routing="skewed", index=3),
    "many_experts": dict(T=32768, d=4096, f=1792, n=64, K=2, dtype="bf16", routing="uniform", index=4),
}

_CHUNK = 1 << 24  # elements per conversion chunk, bounds temporary memory


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in = a.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    for s in range(0, flat_in.size, _CHUNK):
        b = flat_in[s:s + _CHUNK]
        lsb = (b >> 16) & np.uint32(1)
        lsb += np.uint32(0x7FFF)
        lsb += b  # finite inputs: at most 0xFF7FFFFF + 0x8000, no uint32 overflow
        lsb >>= 16
        flat_out[s:s + _CHUNK] = lsb
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class MoEInputs:
    """One layer's inputs. For dtype 'bf16' the arrays hold uint16 bit patterns,
    for 'f32' they hold float32 values."""
    x: np.ndarray
    Wg: np.ndarray
    W1: np.ndarray
    W3: np.ndarray
    W2: np.ndarray
    T: int
    d: int
    f: int
    n: int
    K: int
    dtype: str

    def f64(self, name: str) -> np.ndarray:
        """The named tensor widened losslessly to float64 (what the oracle consumes)."""
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def expert_f64(self, name: str, e: int) -> np.ndarray:
        """One expert's slice of W1/W3/W2 widened to float64."""
        a = getattr(self, name)[e]
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


_THREADS = max(1, min(16, os.cpu_count() or 1))


def _draw(ss: np.random.SeedSequence, shape, scale: float, to_bf16: bool) -> np.ndarray:
    """N(0, scale^2) in float32 (or its bf16 bits), drawn block-wise along axis 0."""
    shape = tuple(int(v) for v in shape)
    rows = shape[0]
    per_row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    R = max(1, (1 << 22) // max(per_row, 1))
    nblk = (rows + R - 1) // R
    kids = ss.spawn(nblk)
    out = np.empty(shape, dtype=np.uint16 if to_bf16 else np.float32)

    def work(b):
        lo, hi = b * R, min(rows, (b + 1) * R)
        blk = np.random.default_rng(kids[b]).standard_normal(size=(hi - lo,) + shape[1:],
                                                             dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        out[lo:hi] = bf16_bits_from_f32(blk) if to_bf16 else blk

    if nblk == 1:
        work(0)
    else:
        with cf.ThreadPoolExecutor(max_workers=_THREADS) as ex:
            list(ex.map(work, range(nblk)))
    return out


def make_inputs(T: int, d: int, f: int, n: int, K: int, dtype: str = "bf16",
                seed: int = SEED_BASE, routing: str = "uniform",
                wg_zero: bool = False, router_only: bool = False) -> MoEInputs:
    """Draw one layer's inputs. ``wg_zero`` replaces the router by zeros
    (every logit ties), after the draws so the other tensors are unchanged.
    ``router_only`` stops after x and W_g (same values as the full draw) and
    leaves the expert weights as None."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    bf = dtype == "bf16"
    s_x, s_wg, s_w1, s_w3, s_w2 = np.random.SeedSequence(seed).spawn(5)
    x = _draw(s_x, (T, d), 1.0, bf)
    if routing == "uniform":
        wg = _draw(s_wg, (d, n), 1.0 / np.sqrt(d), False)
    elif routing == "skewed":
        s_u, s_v = s_wg.spawn(2)
        u = _draw(s_u, (d, n), 1.0 / np.sqrt(d), False)
        v = _draw(s_v, (d,), 1.0 / np.sqrt(d), False)
        sc = np.ones(n, dtype=np.float32)
        sc[n - 1] = 0.1
        b = np.full(n, -16.0, dtype=np.float32)
        b[0] = 16.0
        wg = u * sc[None, :] + v[:, None] * b[None, :]
    else:
        raise ValueError(routing)
    if wg_zero:
        wg = np.zeros_like(wg)
    wg = wg.astype(np.float32)
    Wg = bf16_bits_from_f32(wg) if bf else wg
    if router_only:
        return MoEInputs(x=x, Wg=Wg, W1=None, W3=None, W2=None, T=T, d=d, f=f, n=n, K=K, dtype=dtype)
    W1 = _draw(s_w1, (n, d, f), 1.0 / np.sqrt(d), bf)
    W3 = _draw(s_w3, (n, d, f), 1.0 / np.sqrt(d), bf)
    W2 = _draw(s_w2, (n, f, d), 1.0 / np.sqrt(f), bf)
    return MoEInputs(x=x, Wg=Wg, W1=W1, W3=W3, W2=W2, T=T, d=d, f=f, n=n, K=K, dtype=dtype)


def make_config_inputs(name: str, router_only: bool = False) -> MoEInputs:
    c = CONFIGS[name]
    return make_inputs(c["T"], c["d"], c["f"], c["n"], c["K"], dtype=c["dtype"],
                       seed=SEED_BASE + c["index"], routing=c["routing"],
                       router_only=router_only)
