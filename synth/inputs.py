"""Seeded synthetic MoE-layer inputs (x, W_g, W1, W3, W2).

Recipe (stated once, used by tests and the benchmark alike):
  * generator: numpy ``default_rng(seed)`` (PCG64); draw order x, W_g, W1, W3, W2;
  * standard normals are drawn in float32 and scaled:
      x ~ N(0, 1); W_g, W1, W3 ~ N(0, 1/d); W2 ~ N(0, 1/f)   (fan-in scaling);
  * bf16 configurations round every tensor once, float32 -> bf16 with
    round-to-nearest-even; the fp32 configuration keeps float32;
  * ``routing="skewed"`` builds the router as W_g[:, i] = s_i * u_i + b_i * v with
    u_i, v ~ N(0, 1/d), s = (1, ..., 1, 0.1) and b = (+16, -16, ..., -16): expert 0
    wins the top-1 pick for roughly half the tokens and the last expert rarely does.

Shapes follow the layer equation of the Mixtral study deck (card 2.1): x is
[T][d], W_g is [d][n] (so logits = x @ W_g), W1 and W3 are [n][d][f], W2 is
[n][f][d].  The Mixtral model config quoted in "Why 8x7B Is Not 56B" (Part 4 of
"Mixture of Experts: Why Mixtral Only Wakes Up Two Specialists") fixes
d = 4096, f = 14336, n = 8, K = 2.
"""
from __future__ import annotations

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
        b = flat_in[s:s + _CHUNK].astype(np.uint64)
        b += 0x7FFF + ((b >> 16) & 1)
        flat_out[s:s + _CHUNK] = (b >> 16).astype(np.uint16)
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


def _normal(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def make_inputs(T: int, d: int, f: int, n: int, K: int, dtype: str = "bf16",
                seed: int = SEED_BASE, routing: str = "uniform",
                wg_zero: bool = False, router_only: bool = False) -> MoEInputs:
    """Draw one layer's inputs. ``wg_zero`` replaces the router by zeros
    (every logit ties), after the draws so the other tensors are unchanged.
    ``router_only`` stops after x and W_g (same values as the full draw) and
    leaves the expert weights as None."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    conv = bf16_bits_from_f32 if dtype == "bf16" else (lambda a: a)
    x = conv(_normal(rng, (T, d), 1.0))
    if routing == "uniform":
        wg = _normal(rng, (d, n), 1.0 / np.sqrt(d))
    elif routing == "skewed":
        u = _normal(rng, (d, n), 1.0 / np.sqrt(d))
        v = _normal(rng, (d,), 1.0 / np.sqrt(d))
        s = np.ones(n, dtype=np.float32)
        s[n - 1] = 0.1
        b = np.full(n, -16.0, dtype=np.float32)
        b[0] = 16.0
        wg = u * s[None, :] + v[:, None] * b[None, :]
    else:
        raise ValueError(routing)
    if wg_zero:
        wg = np.zeros_like(wg)
    Wg = conv(wg.astype(np.float32))
    if router_only:
        return MoEInputs(x=x, Wg=Wg, W1=None, W3=None, W2=None, T=T, d=d, f=f, n=n, K=K, dtype=dtype)
    W1 = conv(_normal(rng, (n, d, f), 1.0 / np.sqrt(d)))
    W3 = conv(_normal(rng, (n, d, f), 1.0 / np.sqrt(d)))
    W2 = conv(_normal(rng, (n, f, d), 1.0 / np.sqrt(f)))
    return MoEInputs(x=x, Wg=Wg, W1=W1, W3=W3, W2=W2, T=T, d=d, f=f, n=n, K=K, dtype=dtype)


def make_config_inputs(name: str, router_only: bool = False) -> MoEInputs:
    c = CONFIGS[name]
    return make_inputs(c["T"], c["d"], c["f"], c["n"], c["K"], dtype=c["dtype"],
                       seed=SEED_BASE + c["index"], routing=c["routing"],
                       router_only=router_only)
