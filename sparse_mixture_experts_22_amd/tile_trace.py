"""Per-tile timeline of the packed prefill GEMMs (profiling tool).

    python3 -m sparse_mixture_experts_22_amd.tile_trace mixtral_prefill [many_experts ...]

Runs moe_forward_packed of the tile-trace build (libmoe_tiletrace.so, made by
build.build_tile_trace(); include/moe_tile_trace.h) on a synthetic workload of
the named shape, after warm-up calls, and summarises for each projection:

  - the time and shader-clock cycles of each phase of a tile (k-loop, closing
    barrier, the transition that issues the next tile's loads, the epilogue);
  - the k-loop's cycles per MFMA against the 32 cycles one
    v_mfma_f32_32x32x16_bf16 occupies the matrix core (the issue bound), and
    the clock the part held meanwhile;
  - k-loop time per class of tile (live 32-row blocks, k-steps);
  - how far apart the workgroups finished (idle tail).

Needs a GPU.  Inputs come from the seeded generators (synth); nothing here
checks results (the tests do: the traced library computes what libmoe.so does).
"""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np

PROJS, WGS, TILES, FIELDS = 2, 512, 64, 12
MFMA_CYCLES = 32  # v_mfma_f32_32x32x16_bf16: 8 passes of 4 cycles


def _lib():
    from . import build
    if not os.path.exists(build.TRACE_LIB):
        raise RuntimeError(f"{build.TRACE_LIB} is missing: run build.build_tile_trace() first")
    L = ctypes.CDLL(build.TRACE_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.moe_forward_packed.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp]
    L.moe_tile_trace_read.argtypes = [ctypes.POINTER(ctypes.c_longlong)]
    return L


def record(name: str, warmup: int = 5) -> np.ndarray:
    """One traced forward of workload `name` (a key of synth.CONFIGS): the raw
    trace, int64 [proj][wg][tile][field]."""
    import torch

    from synth import CONFIGS, make_config_inputs

    from . import _binding as moe
    L = _lib()
    c = CONFIGS[name]
    T, d, f, n, K = c["T"], c["d"], c["f"], c["n"], c["K"]
    inp = make_config_inputs(name)
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x, wg = up(inp.x), up(inp.Wg)
    p13 = moe.pack_up(up(inp.W1), up(inp.W3))
    p2 = moe.pack_down(up(inp.W2))
    del inp
    torch.cuda.empty_cache()
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream()

    def run():
        st = L.moe_forward_packed(x.data_ptr(), wg.data_ptr(), p13.data_ptr(), p2.data_ptr(), T, d, f, n, K,
                                  y.data_ptr(), s.cuda_stream)
        if st != 0:
            raise RuntimeError(f"moe_forward_packed returned {st}")

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    if L.moe_tile_trace_clear() != 0:
        raise RuntimeError("moe_tile_trace_clear failed")
    run()
    torch.cuda.synchronize()
    buf = np.zeros(PROJS * WGS * TILES * FIELDS, dtype=np.int64)
    if L.moe_tile_trace_read(buf.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong))) != 0:
        raise RuntimeError("moe_tile_trace_read failed")
    return buf.reshape(PROJS, WGS, TILES, FIELDS)


def summarize(tr: np.ndarray, name: str = "") -> str:
    out = []
    for proj, label in ((0, "gate/up projection (packed_gemm_kernel<1>)"),
                        (1, "down projection (packed_gemm_kernel<2>)")):
        P = tr[proj]
        valid = P[:, :, 4] != 0
        if not valid.any():
            out.append(f"[{name}] {label}: no tiles recorded (not the tiled path)")
            continue
        t0 = P[valid][:, 0].min()
        us = np.where(valid[..., None], (P[..., :5] - t0) / 100.0, np.nan)
        clk = np.where(valid[..., None], P[..., 5:10].astype(np.float64), np.nan)
        nb = P[:, :, 10] % 16          # live row blocks
        ksteps = P[:, :, 10] // 16
        mb = P[:, :, 11]               # row blocks multiplied
        per_wg = valid.sum(1)
        wgs = int((per_wg > 0).sum())
        out.append(f"[{name}] {label}: {int(valid.sum())} tiles on {wgs} workgroups "
                   f"({per_wg[per_wg > 0].min()}..{per_wg.max()} each)")
        out.append(f"  {'phase':38s} {'mean us':>9s} {'median':>9s} {'p90':>9s} {'cycles':>9s} {'GHz':>6s}")
        for k, ph in enumerate(["k-loop", "closing barrier", "transition (next tile's loads issued)",
                                "epilogue (rest)"]):
            v = us[:, :, k + 1] - us[:, :, k]
            c = clk[:, :, k + 1] - clk[:, :, k]
            m = ~np.isnan(v)
            out.append(f"  {ph:38s} {v[m].mean():9.2f} {np.median(v[m]):9.2f} {np.percentile(v[m], 90):9.2f} "
                       f"{c[m].mean():9.0f} {c[m].sum() / v[m].sum() / 1e3:6.2f}")
        gap = us[:, 1:, 0] - us[:, :-1, 4]
        g = gap[~np.isnan(gap)]
        if g.size:
            out.append(f"  {'epilogue end -> next k-loop':38s} {g.mean():9.2f} {np.median(g):9.2f}")
        # k-loop efficiency: MFMAs per wave = 2 (fragments) x blocks multiplied x 2 k16-steps per k-step
        loop_c = clk[:, :, 1] - clk[:, :, 0]
        loop_t = us[:, :, 1] - us[:, :, 0]
        mf = 2 * mb * 2 * ksteps
        sel = valid & (mf > 0)
        ratio = loop_c[sel].sum() / mf[sel].sum()
        out.append(f"  k-loop: {ratio:.1f} cycles per MFMA per wave (issue bound {MFMA_CYCLES}: "
                   f"{100 * MFMA_CYCLES / ratio:.1f}% of it), clock {loop_c[sel].sum() / loop_t[sel].sum() / 1e3:.2f} GHz")
        busy = (us[:, :, 4] - us[:, :, 0])
        tile_time = np.nansum(busy)
        loop_time = np.nansum(loop_t)
        act = np.array([np.nanmax(us[w, :, 4]) for w in range(us.shape[0]) if per_wg[w] > 0])
        span = act.max()
        out.append(f"  span {span:.1f} us: k-loops {100 * loop_time / (wgs * span):.1f}% of workgroup time, "
                   f"transitions+epilogues {100 * (tile_time - loop_time) / (wgs * span):.1f}%, "
                   f"idle tail {100 * (span - act).sum() / (wgs * span):.1f}% "
                   f"(workgroups end {act.min():.1f}..{act.max():.1f} us)")
        for kk in sorted(set(ksteps[valid].tolist())):
            for b in sorted(set(nb[valid & (ksteps == kk)].tolist())):
                s = valid & (ksteps == kk) & (nb == b)
                out.append(f"    k-steps {kk:4d}, live blocks {b} (multiplied {int(mb[s].max())}): "
                           f"{int(s.sum()):5d} tiles, k-loop {np.nanmean(loop_t[s]):8.2f} us, "
                           f"{loop_c[s].sum() / mf[s].sum():.1f} cycles/MFMA")
    return "\n".join(out)


def main(argv) -> int:
    names = argv or ["mixtral_prefill"]
    for name in names:
        print(summarize(record(name), name), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
