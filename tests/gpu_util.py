"""Helpers for the GPU parity tests: move seeded inputs to the device, run the library through
its binding, and compare with the fp64 oracle element by element."""
from __future__ import annotations

import math
import sys

import numpy as np

import workloads

TOL_BF16 = 2e-2   # max-abs, bf16 inputs, fp32 accumulation
TOL_F32 = 1e-5    # max-abs, fp32 inputs
TOL_LSE = 1e-3


def device():
    import pytest
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def to_dev(arr, dtype, dev):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_half_ulp(x):
    ax = np.maximum(np.abs(x), 1e-30)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def check(name, got, ref, tol, bf16_out):
    """Max-abs comparison.  The bar `tol` bounds the error of the fp32-accumulated result; a bf16
    output is in addition rounded once to bf16 when stored, so for bf16 outputs half a bf16 ulp of
    the reference value is added to the bar (0.0039 at 1 <= |x| < 2, 0.0156 at 4 <= |x| < 8,
    0.031 at 8 <= |x| < 16): the rounding of the output itself, which no kernel can avoid."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    lim = np.full(ref.shape, tol)
    if bf16_out:
        lim = tol + bf16_half_ulp(ref)
    bad = ~(err <= lim)
    emax = float(np.nanmax(err)) if err.size else 0.0
    say(f"  {name}: max|err| {emax:.3e}  max|ref| {float(np.abs(ref).max()) if ref.size else 0:.3f}  "
        f"n={ref.size}  over-{tol:g}: {int((err > tol).sum())}")
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err, -1)), ref.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} elements out of tolerance; worst at {i}: got {got[i]} "
                             f"ref {ref[i]} err {err[i]:.4e} (tol {lim[i]:.4e})")
    return emax


def check_lse(name, got, ref, tol=TOL_LSE):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    dead_r = np.isneginf(ref)
    dead_g = np.isneginf(got)
    assert np.array_equal(dead_r, dead_g), f"{name}: -inf pattern differs ({dead_r.sum()} vs {dead_g.sum()})"
    return check(name, got[~dead_r], ref[~dead_r], tol, False)


def run_lib(t: workloads.Tensors, scale, causal, dev, backward=True):
    """Run forward (and backward) on the device; returns torch tensors."""
    import torch

    import exact_io_aware_flash_amd as fa

    q = to_dev(t.q, t.dtype, dev)
    k = to_dev(t.k, t.dtype, dev)
    v = to_dev(t.v, t.dtype, dev)
    mask = torch.from_numpy(t.block_mask).to(dev) if t.block_mask is not None else None
    # outputs start as NaN, so that an element no workgroup wrote is caught on every size
    nan = lambda shape, dt: torch.full(shape, float("nan"), dtype=dt, device=dev)
    o, lse = fa.fwd(q, k, v, scale, causal, mask, out=nan(q.shape, q.dtype), lse=nan(q.shape[:3], torch.float32))
    out = {"o": o, "lse": lse}
    if backward:
        do = to_dev(t.do, t.dtype, dev)
        dq, dk, dv = fa.bwd(q, k, v, o, lse, do, scale, causal, mask, dq=nan(q.shape, q.dtype),
                            dk=nan(q.shape, q.dtype), dv=nan(q.shape, q.dtype))
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, x in out.items():
        assert not torch.isnan(x).any().item(), f"{name}: elements left unwritten (or NaN) on the device"
    return out


def compare_heads(t: workloads.Tensors, res, scale, causal, heads, backward=True, rows=None, cols=None, chunk=1024):
    """Compare device results with the oracle on the listed (b, h) heads.  rows / cols sample the
    query rows (O, LSE, dQ) and key rows (dK, dV) compared; None compares all."""
    import oracle

    bf16 = t.dtype == "bf16"
    tol = TOL_BF16 if bf16 else TOL_F32
    for (b, h) in heads:
        q = _head(t, "q", b, h)
        k = _head(t, "k", b, h)
        v = _head(t, "v", b, h)
        N = q.shape[0]
        r = np.arange(N) if rows is None else np.asarray(rows)
        O, L = oracle.forward_head(q, k, v, scale, causal, t.block_mask, rows=r, chunk=chunk)
        check(f"O[{b},{h}]", host_f64(res["o"][b, h][r]), O, tol, bf16)
        check_lse(f"LSE[{b},{h}]", res["lse"][b, h][r].cpu().numpy(), L)
        if backward:
            do = _head(t, "do", b, h)
            c = np.arange(N) if cols is None else np.asarray(cols)
            dQ, dK, dV = oracle.backward_head(q, k, v, do, scale, causal, t.block_mask, dq_rows=r, dkv_cols=c,
                                              chunk=chunk)
            check(f"dQ[{b},{h}]", host_f64(res["dq"][b, h][r]), dQ, tol, bf16)
            check(f"dK[{b},{h}]", host_f64(res["dk"][b, h][c]), dK, tol, bf16)
            check(f"dV[{b},{h}]", host_f64(res["dv"][b, h][c]), dV, tol, bf16)


def _head(t, name, b, h):
    a = getattr(t, name)[b, h]
    if t.dtype == "bf16":
        return workloads.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def sample_rows(N, n, seed):
    rng = np.random.default_rng(seed)
    base = {0, 1, N - 1, N // 2, min(N - 1, 127), min(N - 1, 128)}
    base |= set(rng.choice(N, size=min(N, n), replace=False).tolist())
    return np.array(sorted(base))


def tile_samples(N, seed, tile=128):
    """One seeded random index in every `tile`-sized block of [0, N) (the ragged last block too)."""
    rng = np.random.default_rng(seed)
    nt = (N + tile - 1) // tile
    return np.minimum(np.arange(nt) * tile + rng.integers(0, tile, nt), N - 1)


def compare_every_tile(t: workloads.Tensors, res, scale, causal, seed, kv_heads, backward=True):
    """Full-size comparison that reaches every tile: on every head, one query row of every
    128-row query tile (O, LSE and, with the backward, dQ); on the heads `kv_heads`, one key of
    every 128-key block (dK, dV).  Rows and keys are drawn per head."""
    import oracle

    B, H, N = t.q.shape[:3]
    bf16 = t.dtype == "bf16"
    tol = TOL_BF16 if bf16 else TOL_F32
    worst = {"O": 0.0, "LSE": 0.0, "dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for b in range(B):
        for h in range(H):
            q, k, v = _head(t, "q", b, h), _head(t, "k", b, h), _head(t, "v", b, h)
            r = tile_samples(N, seed + 1000 * b + h)
            O, L = oracle.forward_head(q, k, v, scale, causal, t.block_mask, rows=r)
            worst["O"] = max(worst["O"], check(f"O[{b},{h}] tiles", host_f64(res["o"][b, h][r]), O, tol, bf16))
            worst["LSE"] = max(worst["LSE"], check_lse(f"LSE[{b},{h}] tiles", res["lse"][b, h][r].cpu().numpy(), L))
            if backward:
                do = _head(t, "do", b, h)
                dQ, _, _ = oracle.backward_head(q, k, v, do, scale, causal, t.block_mask, dq_rows=r, dkv_cols=[])
                worst["dQ"] = max(worst["dQ"], check(f"dQ[{b},{h}] tiles", host_f64(res["dq"][b, h][r]), dQ, tol, bf16))
                if (b, h) in kv_heads:
                    c = tile_samples(N, seed + 7 + 1000 * b + h)
                    _, dK, dV = oracle.backward_head(q, k, v, do, scale, causal, t.block_mask, dq_rows=[], dkv_cols=c)
                    worst["dK"] = max(worst["dK"], check(f"dK[{b},{h}] blocks", host_f64(res["dk"][b, h][c]), dK, tol,
                                                         bf16))
                    worst["dV"] = max(worst["dV"], check(f"dV[{b},{h}] blocks", host_f64(res["dv"][b, h][c]), dV, tol,
                                                         bf16))
    say(f"  worst over all tiles: {worst}")
    return worst
