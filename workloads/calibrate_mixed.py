"""Calibration of the mixed-residency workload, written out as stored inputs.

Run as ``python -m workloads.calibrate_mixed [--B 32 --T 131072 --K 2048]``.

The workload asks for two things that depend on the indexer's own output:
* about 70 % of each request's top-K inside four 8K-token windows, reached by
  one additive bias beta on the window tokens, found by bisection;
* hot buffers pre-seeded so that about half of the current top-K hits:
  min(1024, #host-only selected tokens) of the host-only tokens of the current
  top-K, chosen uniformly.

Both need scores and a top-K, which only the oracle computes, so this script
runs the oracle once and stores (beta, hot tokens) under ``workloads/data/``;
the generator only reads them.  Nothing on the GPU path imports this module.
"""

from __future__ import annotations

import argparse
import time

import numpy as np

from oracle import indexer as o_indexer, topk as o_topk
from workloads import gen

TARGET = 0.70


def _fraction(S0: np.ndarray, wmask: np.ndarray, beta: float, K: int) -> float:
    """Mean over requests of |top-K inside windows| / K for scores S0 + beta * mask."""
    B, T = S0.shape
    fr = []
    b32 = float(np.float32(beta))
    for b in range(B):
        sel = o_topk.topk_row(S0[b] + b32 * wmask[b], T, K)
        fr.append(np.mean(wmask[b][sel]))
    return float(np.mean(fr))


def calibrate(seed: int = 1003, B: int = 32, T: int = 131072, K: int = 2048,
              tail: int = 4096, verbose: bool = False):
    """Returns (beta, hot_tokens [B, H]) for the mixed workload at these sizes."""
    C = 2 * K
    t0 = time.time()
    wl = gen.mixed_128k(seed=seed, B=B, T=T, K=K, tail=tail, beta=0.0,
                        hot_tokens=np.full((B, 0), -1, np.int32), latent=False)
    S0 = o_indexer.indexer_scores(wl.q_idx, wl.q_dtype, wl.w, wl.idx_pool, wl.k_dtype,
                                  wl.idx_scale, wl.idx_bt, wl.ctx_len, None,
                                  T_stride=wl.T_stride)[:, 0, :T]
    wmask = wl.info["window_mask"]
    if verbose:
        print(f"unbiased scores in {time.time() - t0:.1f}s; no-bias fraction "
              f"{_fraction(S0, wmask, 0.0, K):.3f}", flush=True)
    lo, hi = 0.0, float(np.max(S0) - np.min(S0))
    for _ in range(50):
        mid = 0.5 * (lo + hi)
        if _fraction(S0, wmask, mid, K) < TARGET:
            lo = mid
        else:
            hi = mid
    beta = hi
    frac = _fraction(S0, wmask, beta, K)
    if verbose:
        print(f"beta = {beta:.6g} -> fraction {frac:.4f}", flush=True)
    host_lim = (wl.T_stride // gen.BLOCK - (-(-tail // gen.BLOCK))) * gen.BLOCK
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(11)[10]))
    n_hot = min(1024, C // 4)
    hot = np.full((B, n_hot), -1, dtype=np.int32)
    b32 = float(np.float32(beta))
    for b in range(B):
        sel = o_topk.topk_row(S0[b] + b32 * wmask[b], T, K)
        host_sel = sel[sel < host_lim]
        m = min(n_hot, len(host_sel))
        hot[b, :m] = np.sort(rng.choice(host_sel, size=m, replace=False))
    return beta, hot, frac


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seed", type=int, default=1003)
    ap.add_argument("--B", type=int, default=32)
    ap.add_argument("--T", type=int, default=131072)
    ap.add_argument("--K", type=int, default=2048)
    a = ap.parse_args()
    beta, hot, frac = calibrate(a.seed, a.B, a.T, a.K, verbose=True)
    gen.DATA_DIR.mkdir(parents=True, exist_ok=True)
    f = gen.DATA_DIR / f"mixed_s{a.seed}_B{a.B}_T{a.T}_K{a.K}_C{2 * a.K}.npz"
    np.savez_compressed(f, beta=np.float64(beta), hot_tokens=hot, fraction=np.float64(frac))
    print(f"wrote {f}")


if __name__ == "__main__":
    main()
