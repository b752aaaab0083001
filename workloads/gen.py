"""Generators for the five synthetic workloads of the decode step.

Every array is drawn from numpy ``Generator(PCG64)`` streams spawned from
``SeedSequence(seed)``; the default seed of workload n is 1000 + n.  The ten
child streams are used for, in order:

    0 context lengths   1 block permutations   2 latent values
    3 attention queries 4 indexer queries      5 head weights
    6 indexer keys      7 bias / window centres 8 hot-buffer seeding
    9 query drift between steps

Large arrays are drawn in fixed-size chunks, each from its own spawned
stream, so the bytes do not depend on how many threads fill them.

Storage formats: float32 draws are rounded to bf16 (round to nearest even) or
quantized to FP8 E4M3FN with one fp32 scale per 64-token block,
scale = amax / 448 (1 when the block is all zeros), code = RNE(x / scale)
clamped to +-448 (torch's float8_e4m3fn conversion does the rounding).

Workload shapes (one GPU's share; "Un contexte d'un million sur huit H200",
"Les chiffres", and "vLLM sert GLM-5.3 en contexte 1M sur 16 H200",
"Les résultats", give the deployments these stand in for):

    tiny_fp32      B=1  T=4096              fp32 everywhere, all resident
    resident_fp8   B=8  T~U[16K,32K]        fp8 KV, attention-sink bias, all resident
    mixed_128k     B=32 T=131072            4096-token resident tail, host pool,
                                            hot buffers 2K pre-seeded, locality bias
    mtp3_agentic   B=64 P=4 T~74K..86K      40 % of rows fit the GPU pool, hot 5K
    norescache_1m  B=4  T=2^20  L=4         latent host-only, hot buffers start empty
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from pathlib import Path

import numpy as np
import torch

BLOCK = 64
D_LATENT = 576
E4M3_MAX = 448.0
DATA_DIR = Path(__file__).resolve().parent / "data"

_CHUNK = 1 << 22          # values per random chunk
_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8))


# --------------------------------------------------------------------------- random draws

def _children(seed: int) -> list:
    return np.random.SeedSequence(seed).spawn(10)


def _run(fn, n):
    if n == 1 or _THREADS == 1:
        for i in range(n):
            fn(i)
        return
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fn, range(n)))


def normal_f32(ss: np.random.SeedSequence, shape) -> np.ndarray:
    """float32 N(0,1) array, drawn in fixed chunks of spawned streams."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    n = flat.size
    nch = max(1, -(-n // _CHUNK))
    kids = ss.spawn(nch)

    def work(i):
        g = np.random.Generator(np.random.PCG64(kids[i]))
        g.standard_normal(out=flat[i * _CHUNK:(i + 1) * _CHUNK], dtype=np.float32)
    _run(work, nch)
    return out


def uniform_f32(ss: np.random.SeedSequence, shape) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    return g.random(shape, dtype=np.float64).astype(np.float32)


def bf16_bits(x) -> np.ndarray:
    """Round float32/float64 values to bf16 (RNE); returns the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """float32 values of bf16 bit patterns (via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.float().numpy()


def quantize_e4m3_blocks(x: np.ndarray):
    """x float32 [..., 64, D] -> (codes uint8 [..., 64, D], scale float32 [...]).

    One scale per 64-token block: amax / 448, or 1 for an all-zero block.
    """
    t = torch.from_numpy(x)
    amax = t.abs().amax(dim=(-2, -1))
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (t / scale[..., None, None]).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale.numpy().astype(np.float32)


def _fp8_rows(ss: np.random.SeedSequence, n_blocks: int, D: int, tokens_per_chunk: int = 16384):
    """N(0,1) rows quantized per block: codes [n_blocks, 64, D], scales [n_blocks]."""
    codes = np.empty((n_blocks, BLOCK, D), dtype=np.uint8)
    scales = np.empty((n_blocks,), dtype=np.float32)
    bpc = max(1, tokens_per_chunk // BLOCK)
    nch = max(1, -(-n_blocks // bpc))
    kids = ss.spawn(nch)

    def work(i):
        b0, b1 = i * bpc, min(n_blocks, (i + 1) * bpc)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        x = g.standard_normal(((b1 - b0), BLOCK, D), dtype=np.float32)
        c, s = quantize_e4m3_blocks(x)
        codes[b0:b1] = c
        scales[b0:b1] = s
    prev = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        _run(work, nch)
    finally:
        torch.set_num_threads(prev)
    return codes, scales


def _f32_rows(ss, n_blocks: int, D: int):
    return normal_f32(ss, (n_blocks, BLOCK, D))


# --------------------------------------------------------------------------- workload object

@dataclass
class Workload:
    """All inputs of a decode-step workload, as host numpy arrays.

    Per-token arrays use a row stride T_stride (a multiple of 64); block tables
    have T_stride // 64 columns.  Dtype tags: 'f32', 'bf16' (uint16 bits),
    'e4m3' (uint8 codes).
    """
    name: str
    seed: int
    B: int
    P: int
    K: int
    L: int
    Hq: int
    H_idx: int
    D_idx: int
    T_stride: int
    ctx_len: np.ndarray            # [B] int32
    C: int                         # hot capacity in rows per request (0 = none)
    q_dtype: str                   # 'f32' or 'bf16' (indexer and attention queries)
    k_dtype: str                   # 'f32' or 'e4m3' (indexer keys)
    kv_dtype: str                  # 'f32' or 'e4m3' (latent rows)
    sm_scale: float
    # indexer cache (always resident)
    w: np.ndarray                  # [B, P, H_idx] float32
    idx_pool: np.ndarray           # [N_idx_blocks, 64, D_idx]
    idx_scale: np.ndarray | None   # [N_idx_blocks] float32
    idx_bt: np.ndarray             # [B, max_blocks] int32 (-1 past the context)
    bias: np.ndarray | None        # [B, T_stride] float32
    # logical latent, one slice per attention layer (padding rows are zero)
    lat: np.ndarray                # [L, B, T_stride, 576]
    lat_scale: np.ndarray | None   # [L, B, T_stride // 64] float32
    # residency
    n_pool_blocks: int
    bt: np.ndarray                 # [B, max_blocks] int32, -1 = page not resident
    hot_blocks: np.ndarray         # [B, C // 64] int32
    tok2slot: np.ndarray           # [B, T_stride] int32
    slot2tok: np.ndarray           # [B, C] int32
    stamp: np.ndarray              # [B, C] int32
    step: int
    has_host: bool                 # host pool = the logical latent, row b*T_stride + t
    steps: int = 1                 # length of the step sequence
    _step_q: list = field(default_factory=list, repr=False)   # per step (q_idx, q)
    info: dict = field(default_factory=dict)
    # decode loop with KV append (None when the context stays fixed over the steps):
    # after step s < steps every request appends token ctx0[b] + s - 1, whose latent
    # rows (every layer) and page scale are already in `lat` / `lat_scale` past the
    # context, and whose key is app_keys[b, s - 1] (page scale app_key_scale[b, s - 1]).
    ctx0: np.ndarray | None = None            # [B] int32 context before the first append
    free_blocks: np.ndarray | None = None     # latent free list, bottom .. top (int32)
    idx_free_blocks: np.ndarray | None = None # indexer free list, bottom .. top (int32)
    app_keys: np.ndarray | None = None        # [B, steps - 1, D_idx] key codes
    app_key_scale: np.ndarray | None = None   # [B, steps - 1] scale of the key's page

    @property
    def max_blocks(self) -> int:
        return self.T_stride // BLOCK

    @property
    def host_bt(self) -> np.ndarray:
        """int64 [B, max_blocks]: host row of token 64*j of each page, -1 if none."""
        if not self.has_host:
            return np.full((self.B, self.max_blocks), -1, dtype=np.int64)
        b = np.arange(self.B, dtype=np.int64)[:, None]
        j = np.arange(self.max_blocks, dtype=np.int64)[None, :]
        hb = b * self.T_stride + j * BLOCK
        nblk = -(-self.ctx_len.astype(np.int64) // BLOCK)
        return np.where(j < nblk[:, None], hb, -1)

    @property
    def host_rows(self) -> np.ndarray:
        """[L, B * T_stride, 576] view of the logical latent (the host pool)."""
        return self.lat.reshape(self.L, self.B * self.T_stride, D_LATENT)

    @property
    def host_scale(self) -> np.ndarray | None:
        """[L, B * T_stride] per-row scales of the host pool."""
        if self.lat_scale is None:
            return None
        return np.repeat(self.lat_scale, BLOCK, axis=2).reshape(self.L, self.B * self.T_stride)

    @property
    def appends(self) -> bool:
        return self.ctx0 is not None

    def append_inputs(self, s: int):
        """Inputs of the KV append that follows step s (1 <= s < steps): one token per
        request.  Returns (n_new [B] int32, rows [B,1,L,576], row_scale [B,1,L] or
        None, keys [B,1,D_idx], key_scale [B,1] or None)."""
        assert self.appends and 1 <= s < self.steps
        i = s - 1
        t = self.ctx0.astype(np.int64) + i
        b = np.arange(self.B)
        rows = self.lat[:, b, t].transpose(1, 0, 2)[:, None]          # [B,1,L,576]
        rsc = None
        if self.lat_scale is not None:
            rsc = self.lat_scale[:, b, t // BLOCK].T[:, None].astype(np.float32)
        keys = self.app_keys[:, i][:, None]
        ksc = None if self.app_key_scale is None else self.app_key_scale[:, i][:, None]
        return (np.ones(self.B, np.int32), np.ascontiguousarray(rows),
                None if rsc is None else np.ascontiguousarray(rsc), np.ascontiguousarray(keys),
                None if ksc is None else np.ascontiguousarray(ksc))

    def step_inputs(self, s: int = 1):
        """(q_idx, q) of step s (1-based): q_idx [B,P,H,D], q [L,B,P,Hq,576]."""
        return self._step_q[s - 1]

    def physical_pool(self):
        """(pool [L, n_rows, 576], row_scale [L, n_rows] or None) of the initial
        state: what the device pool holds before the first step."""
        return build_pool(self)

    @property
    def q_idx(self):
        return self._step_q[0][0]

    @property
    def q(self):
        return self._step_q[0][1]


def build_pool(wl: Workload, pool_out: np.ndarray | None = None,
               scale_out: np.ndarray | None = None):
    """Physical pool contents of a workload's initial state.

    Returns pool [L, n_pool_blocks * 64, 576] and row_scale [L, n_rows] (None for
    fp32 rows): resident pages are copied from the logical latent according to
    ``bt``; every occupied hot slot holds the logical row of its token; all
    other rows are zero.
    """
    n_rows = wl.n_pool_blocks * BLOCK
    dt = np.float32 if wl.kv_dtype == "f32" else np.uint8
    pool = pool_out if pool_out is not None else np.zeros((wl.L, n_rows, D_LATENT), dtype=dt)
    rsc = None
    if wl.lat_scale is not None:
        rsc = scale_out if scale_out is not None else np.zeros((wl.L, n_rows), dtype=np.float32)
    for b in range(wl.B):
        nblk = -(-int(wl.ctx_len[b]) // BLOCK)
        js = np.nonzero(wl.bt[b, :nblk] >= 0)[0]
        if len(js):
            src = (js[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
            dst = (wl.bt[b, js].astype(np.int64)[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
            pool[:, dst] = wl.lat[:, b, src]
            if rsc is not None:
                rsc[:, dst] = wl.lat_scale[:, b, src // BLOCK]
        if wl.C:
            v = np.nonzero(wl.slot2tok[b] >= 0)[0]
            if len(v):
                t = wl.slot2tok[b, v].astype(np.int64)
                dst = wl.hot_blocks[b, v // BLOCK].astype(np.int64) * BLOCK + v % BLOCK
                pool[:, dst] = wl.lat[:, b, t]
                if rsc is not None:
                    rsc[:, dst] = wl.lat_scale[:, b, t // BLOCK]
    return pool, rsc


# --------------------------------------------------------------------------- pieces

def _round_up(x: int, m: int) -> int:
    return -(-x // m) * m


def _indexer_cache(ch, B, ctx_len, T_stride, D, fp8: bool):
    """Paged indexer keys ~N(0,1): pool, per-block scale, block table."""
    nblk = [-(-int(t) // BLOCK) for t in ctx_len]
    total = int(sum(nblk))
    g = np.random.Generator(np.random.PCG64(ch[1].spawn(1)[0]))
    perm = g.permutation(total).astype(np.int32)
    if fp8:
        codes, scales = _fp8_rows(ch[6], total, D)
    else:
        codes, scales = _f32_rows(ch[6], total, D), None
    # zero the padding rows past each context (never read)
    off = 0
    for b in range(B):
        pad = nblk[b] * BLOCK - int(ctx_len[b])
        if pad:
            codes[off + nblk[b] - 1, BLOCK - pad:] = 0
        off += nblk[b]
    pool = np.empty_like(codes)
    pool[perm] = codes
    scale = None
    if scales is not None:
        scale = np.empty_like(scales)
        scale[perm] = scales
    bt = np.full((B, T_stride // BLOCK), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    return pool, scale, bt


def _latent(ch, L, B, ctx_len, T_stride, fp8: bool):
    """Logical latent [L, B, T_stride, 576] ~N(0,1) and per-block scales."""
    nb = T_stride // BLOCK
    if fp8:
        codes, scales = _fp8_rows(ch[2], L * B * nb, D_LATENT)
        lat = codes.reshape(L, B, T_stride, D_LATENT)
        sc = scales.reshape(L, B, nb)
    else:
        lat = _f32_rows(ch[2], L * B * nb, D_LATENT).reshape(L, B, T_stride, D_LATENT)
        sc = None
    for b in range(B):
        T = int(ctx_len[b])
        lat[:, b, T:] = 0
    return lat, sc


def _queries(ss, shape, dtype: str):
    x = normal_f32(ss, shape)
    return x if dtype == "f32" else bf16_bits(x)


def _empty_hot(B, C, T_stride):
    return (np.full((B, T_stride), -1, dtype=np.int32), np.full((B, C), -1, dtype=np.int32),
            np.zeros((B, C), dtype=np.int32))


def _place_blocks(ch, B, resident: list, n_hot_blocks: int):
    """One shared pool: a seeded permutation over every resident (request, page)
    pair and every hot block, so tail pages and hot blocks interleave.

    resident[b] = list of logical pages of request b that are resident.
    Returns (n_pool_blocks, bt_entries per request, hot_blocks [B, n_hot_blocks]).
    """
    n_res = sum(len(r) for r in resident)
    total = n_res + B * n_hot_blocks
    g = np.random.Generator(np.random.PCG64(ch[1].spawn(1)[0]))
    perm = g.permutation(total).astype(np.int32)
    pages, off = [], 0
    for r in resident:
        pages.append(perm[off:off + len(r)])
        off += len(r)
    hot = perm[off:].reshape(B, n_hot_blocks) if n_hot_blocks else np.zeros((B, 0), np.int32)
    return total, pages, hot


def _bias_sigma(q_bits_bp: np.ndarray, w_bp: np.ndarray) -> float:
    """Standard deviation of a position's unbiased indexer score over keys
    drawn from the generator's key distribution k ~ N(0, I).

    For z_h = q_h . k the vector z is Gaussian with covariance G = Q Q^T, and
    the arc-cosine identity gives, with a_h = sqrt(G_hh), rho = G_hh'/(a_h a_h'),
    theta = arccos(rho):
        E[relu(z_h)]               = a_h / sqrt(2 pi)
        E[relu(z_h) relu(z_h')]    = a_h a_h' (sin theta + (pi - theta) cos theta) / (2 pi)
    so Var(sum_h w_h relu(z_h)) follows in closed form.  This is a moment of the
    input distribution, used only to size the attention-sink bias.
    """
    Q = bf16_values(q_bits_bp).astype(np.float64)           # [H, D]
    w = w_bp.astype(np.float64)
    G = Q @ Q.T
    a = np.sqrt(np.diag(G))
    rho = np.clip(G / np.outer(a, a), -1.0, 1.0)
    th = np.arccos(rho)
    m2 = np.outer(a, a) * (np.sin(th) + (np.pi - th) * np.cos(th)) / (2 * np.pi)
    m1 = a / math.sqrt(2 * np.pi)
    cov = m2 - np.outer(m1, m1)
    return float(math.sqrt(max(w @ cov @ w, 0.0)))


def _ar1_steps(ch, q0_f64: np.ndarray, steps: int, rho: float) -> list:
    """AR(1) drift of the indexer queries in float64: q_s = rho q_{s-1} + sqrt(1-rho^2) e_s."""
    out = [q0_f64]
    kids = ch[9].spawn(max(steps - 1, 1))
    for s in range(1, steps):
        g = np.random.Generator(np.random.PCG64(kids[s - 1]))
        e = g.standard_normal(q0_f64.shape)
        out.append(rho * out[-1] + math.sqrt(1 - rho * rho) * e)
    return out


# --------------------------------------------------------------------------- workloads

def tiny_fp32(K: int = 256, seed: int = 1001, T: int = 4096) -> Workload:
    """B=1, T=4096, K=256 (also run at K=4096 and 8192), 16 heads, fp32
    everywhere, indexer 4 heads x 64, one layer, all rows resident in a paged
    pool with a seeded block permutation, no host pool."""
    ch = _children(seed)
    B, P, Hq, H, D, L = 1, 1, 16, 4, 64, 1
    ctx = np.array([T], dtype=np.int32)
    Ts = _round_up(T, BLOCK)
    idx_pool, idx_scale, idx_bt = _indexer_cache(ch, B, ctx, Ts, D, fp8=False)
    lat, lat_scale = _latent(ch, L, B, ctx, Ts, fp8=False)
    nblk = -(-T // BLOCK)
    n_pool, pages, hot = _place_blocks(ch, B, [list(range(nblk))], 0)
    bt = np.full((B, Ts // BLOCK), -1, dtype=np.int32)
    bt[0, :nblk] = pages[0]
    q_idx = _queries(ch[4], (B, P, H, D), "f32")
    w = uniform_f32(ch[5], (B, P, H))
    q = _queries(ch[3], (L, B, P, Hq, D_LATENT), "f32")
    t2s, s2t, st = _empty_hot(B, 0, Ts)
    return Workload("tiny_fp32", seed, B, P, K, L, Hq, H, D, Ts, ctx, 0, "f32", "f32", "f32",
                    1.0 / math.sqrt(D_LATENT), w, idx_pool, idx_scale, idx_bt, None, lat,
                    lat_scale, n_pool, bt, hot, t2s, s2t, st, 0, False, 1, [(q_idx, q)])


def resident_fp8(seed: int = 1002, B: int = 8, T_lo: int = 16384, T_hi: int = 32768,
                 K: int = 2048, ctx_len=None) -> Workload:
    """B=8, T ~ U{16K..32K}, K=2048, 16 bf16 heads (one shard of 128), fp8
    latent and indexer keys with per-block scales, indexer 64 heads x 128, an
    attention-sink bias of +2 sigma on the first 64 and last 256 tokens, whole
    cache resident in shuffled blocks.  ctx_len, when given, fixes the context
    lengths (and B) instead of drawing them."""
    ch = _children(seed)
    P, Hq, H, D, L = 1, 16, 64, 128, 1
    g0 = np.random.Generator(np.random.PCG64(ch[0]))
    ctx = g0.integers(T_lo, T_hi + 1, size=B).astype(np.int32)
    if ctx_len is not None:
        ctx = np.asarray(ctx_len, dtype=np.int32)
        B = len(ctx)
    Ts = max(_round_up(int(ctx.max()), BLOCK), BLOCK)
    idx_pool, idx_scale, idx_bt = _indexer_cache(ch, B, ctx, Ts, D, fp8=True)
    q_idx = _queries(ch[4], (B, P, H, D), "bf16")
    w = uniform_f32(ch[5], (B, P, H))
    bias = np.zeros((B, Ts), dtype=np.float32)
    sig = np.zeros(B)
    for b in range(B):
        sig[b] = _bias_sigma(q_idx[b, 0], w[b, 0])
        T = int(ctx[b])
        bias[b, :min(64, T)] = np.float32(2.0 * sig[b])
        bias[b, max(T - 256, 0):T] = np.float32(2.0 * sig[b])
    lat, lat_scale = _latent(ch, L, B, ctx, Ts, fp8=True)
    res = [list(range(-(-int(t) // BLOCK))) for t in ctx]
    n_pool, pages, hot = _place_blocks(ch, B, res, 0)
    bt = np.full((B, Ts // BLOCK), -1, dtype=np.int32)
    for b in range(B):
        bt[b, :len(pages[b])] = pages[b]
    q = _queries(ch[3], (L, B, P, Hq, D_LATENT), "bf16")
    t2s, s2t, st = _empty_hot(B, 0, Ts)
    return Workload("resident_fp8", seed, B, P, K, L, Hq, H, D, Ts, ctx, 0, "bf16", "e4m3",
                    "e4m3", 1.0 / math.sqrt(D_LATENT), w, idx_pool, idx_scale, idx_bt, bias,
                    lat, lat_scale, n_pool, bt, hot, t2s, s2t, st, 0, False, 1, [(q_idx, q)],
                    info={"sigma": sig})


def mixed_windows(ch, B: int, T: int, n_centres: int = 4, half: int = 4096):
    """Locality windows: 4 centres per request, uniform in [4096, T - 8192],
    each window [c - 4096, c + 4096).  Returns (centres [B, 4], mask [B, T] bool)."""
    g = np.random.Generator(np.random.PCG64(ch[7]))
    lo, hi = half, max(T - 2 * half, half + 1)
    centres = g.integers(lo, hi, size=(B, n_centres))
    mask = np.zeros((B, T), dtype=bool)
    for b in range(B):
        for c in centres[b]:
            mask[b, max(c - half, 0):min(c + half, T)] = True
    return centres, mask


def mixed_128k_stored(seed: int, B: int, T: int, K: int, C: int):
    """(beta, hot tokens [B, n]) for the mixed-residency workload, as written by
    ``python -m workloads.calibrate_mixed`` (a script that runs the oracle)."""
    f = DATA_DIR / f"mixed_s{seed}_B{B}_T{T}_K{K}_C{C}.npz"
    if not f.exists():
        raise FileNotFoundError(f"{f} missing: run `python -m workloads.calibrate_mixed` "
                                "or pass beta and hot_tokens explicitly")
    z = np.load(f, allow_pickle=False)
    return float(z["beta"]), z["hot_tokens"]


def mixed_128k(seed: int = 1003, B: int = 32, T: int = 131072, K: int = 2048,
               tail: int = 4096, beta: float | None = None, hot_tokens=None,
               latent: bool = True) -> Workload:
    """Mixed residency at 128K: B=32, T=131072, K=2048, 16 heads, fp8 latent.
    The last 4096 tokens are resident and never evicted; older pages live only
    in the pinned host pool.  Hot buffers hold 2K = 4096 rows per request, drawn
    from the same shared pool, pre-seeded so that about half of the current
    top-K hits: ``hot_tokens[b]`` (host-only tokens of the current top-K, chosen
    by the calibration) go to random slots, the remaining slots hold other random
    host-only tokens, stamps are uniform in [1, 8] and the step counter is 8.
    Indexer scores get +beta on four 8K-token windows so that about 70 % of the
    top-K falls inside them.  ``latent=False`` skips the latent (indexer-only use).
    """
    ch = _children(seed)
    P, Hq, H, D, L = 1, 16, 64, 128, 1
    C = 2 * K
    ctx = np.full(B, T, dtype=np.int32)
    Ts = _round_up(T, BLOCK)
    idx_pool, idx_scale, idx_bt = _indexer_cache(ch, B, ctx, Ts, D, fp8=True)
    q_idx = _queries(ch[4], (B, P, H, D), "bf16")
    w = uniform_f32(ch[5], (B, P, H))
    centres, wmask = mixed_windows(ch, B, T)
    if beta is None or hot_tokens is None:
        b_st, h_st = mixed_128k_stored(seed, B, T, K, C)
        beta = b_st if beta is None else beta
        hot_tokens = h_st if hot_tokens is None else hot_tokens
    bias = np.zeros((B, Ts), dtype=np.float32)
    bias[:, :T][wmask] = np.float32(beta)
    nblk = Ts // BLOCK
    tail_blk = -(-tail // BLOCK)
    res = [list(range(nblk - tail_blk, nblk)) for _ in range(B)]
    n_pool, pages, hot = _place_blocks(ch, B, res, C // BLOCK)
    bt = np.full((B, nblk), -1, dtype=np.int32)
    for b in range(B):
        bt[b, nblk - tail_blk:] = pages[b]
    # hot seeding
    t2s, s2t, st = _empty_hot(B, C, Ts)
    g = np.random.Generator(np.random.PCG64(ch[8]))
    host_lim = (nblk - tail_blk) * BLOCK               # tokens below this are host-only
    for b in range(B):
        ht = np.asarray(hot_tokens[b])
        ht = ht[ht >= 0].astype(np.int64)
        if np.any(ht >= host_lim):
            raise ValueError("hot tokens must be host-only")
        others = g.choice(host_lim, size=C, replace=False)
        others = others[~np.isin(others, ht)][:C - len(ht)]
        toks = np.concatenate([ht, others])
        slots = g.permutation(C)
        s2t[b, slots] = toks
        t2s[b, toks] = slots
        st[b] = g.integers(1, 9, size=C)
    if latent:
        lat, lat_scale = _latent(ch, L, B, ctx, Ts, fp8=True)
    else:
        lat = np.zeros((L, B, 0, D_LATENT), dtype=np.uint8)
        lat_scale = np.zeros((L, B, 0), dtype=np.float32)
    q = _queries(ch[3], (L, B, P, Hq, D_LATENT), "bf16")
    return Workload("mixed_128k", seed, B, P, K, L, Hq, H, D, Ts, ctx, C, "bf16", "e4m3", "e4m3",
                    1.0 / math.sqrt(D_LATENT), w, idx_pool, idx_scale, idx_bt, bias, lat,
                    lat_scale, n_pool, bt, hot, t2s, s2t, st, 8, True, 1, [(q_idx, q)],
                    info={"beta": beta, "centres": centres, "window_mask": wmask,
                          "hot_tokens": hot_tokens})


def conversation_lengths(ss, B: int, first_turn: int = 74160, per_turn: int = 973,
                         turns: int = 13, out_max: int = 220) -> np.ndarray:
    """T = first_turn + (n - 1) * per_turn + j, turn n ~ U{1..turns}, j ~ U{1..out_max}."""
    g0 = np.random.Generator(np.random.PCG64(ss))
    n = g0.integers(1, turns + 1, size=B)
    j = g0.integers(1, out_max + 1, size=B)
    return (first_turn + (n - 1) * per_turn + j).astype(np.int32)


def mtp3_agentic(seed: int = 1004, B: int = 64, K: int = 2048, steps: int = 4,
                 rho: float = 0.95, pool_frac: float = 0.40, first_turn: int = 74160,
                 per_turn: int = 973, turns: int = 13, out_max: int = 220,
                 P: int = 4, C: int | None = None) -> Workload:
    """MTP3 agentic mix: 3 speculative tokens, so P = 4 query positions and hot
    buffers of (3 + 2) x K = 10240 rows per request.  Context lengths follow
    13-turn conversations (first turn 74,160 tokens, then +753 input and +220
    output per turn): T = 74160 + (n - 1) * 973 + j with turn n ~ U{1..13} and
    output position j ~ U{1..220}.  The GPU pool holds 40 % of all rows: the hot
    blocks plus an equal resident tail per request; the rest is host-only.
    Four steps with the indexer queries drifting as AR(1) (rho = 0.95) and fresh
    attention queries per step; hot buffers start empty.  ``P`` other than 4
    (P - 1 speculative tokens, hot buffers (P + 1) x K) serves smaller tests, as
    does ``C`` (hot rows per request, a multiple of 64 of at least P x K)."""
    ch = _children(seed)
    Hq, H, D, L = 16, 64, 128, 1
    C = (P + 1) * K if C is None else int(C)
    ctx = conversation_lengths(ch[0], B, first_turn, per_turn, turns, out_max)
    Ts = _round_up(int(ctx.max()), BLOCK)
    nblk = -(-ctx.astype(np.int64) // BLOCK)
    pool_blocks = int(math.floor(pool_frac * int(nblk.sum())))
    hot_b = C // BLOCK
    tail_b = (pool_blocks - B * hot_b) // B
    if tail_b <= 0:
        raise ValueError("pool too small for the hot buffers")
    idx_pool, idx_scale, idx_bt = _indexer_cache(ch, B, ctx, Ts, D, fp8=True)
    w = uniform_f32(ch[5], (B, P, H))
    res = [list(range(max(int(nb) - tail_b, 0), int(nb))) for nb in nblk]
    n_pool, pages, hot = _place_blocks(ch, B, res, hot_b)
    bt = np.full((B, Ts // BLOCK), -1, dtype=np.int32)
    for b in range(B):
        bt[b, res[b][0]:res[b][-1] + 1] = pages[b]
    lat, lat_scale = _latent(ch, L, B, ctx, Ts, fp8=True)
    g4 = np.random.Generator(np.random.PCG64(ch[4]))
    q0 = g4.standard_normal((B, P, H, D))
    qs = _ar1_steps(ch, q0, steps, rho)
    kq = ch[3].spawn(steps)
    step_q = [(bf16_bits(qs[s]), _queries(kq[s], (L, B, P, Hq, D_LATENT), "bf16"))
              for s in range(steps)]
    t2s, s2t, st = _empty_hot(B, C, Ts)
    return Workload("mtp3_agentic", seed, B, P, K, L, Hq, H, D, Ts, ctx, C, "bf16", "e4m3",
                    "e4m3", 1.0 / math.sqrt(D_LATENT), w, idx_pool, idx_scale, idx_bt, None,
                    lat, lat_scale, n_pool, bt, hot, t2s, s2t, st, 0, True, steps, step_q,
                    info={"tail_blocks": tail_b, "pool_blocks_target": pool_blocks})


def norescache_1m(seed: int = 1005, B: int = 4, T: int = 1 << 20, K: int = 2048, L: int = 4,
                  steps: int = 16, rho: float = 0.95, append: bool = False) -> Workload:
    """1M-token no-residency start: B=4, T=2^20, K=2048, 16 heads, fp8 latent,
    four sparse-MLA layers sharing one indexer layer.  The indexer cache is
    resident; the whole latent is host-only and the hot buffers (2K rows per
    request, shared by the four layers) start empty, so rows fault in as the
    indexer asks for them.  Sixteen steps with AR(1) drifting indexer queries
    (rho = 0.95) and fresh attention queries per layer per step.

    append: a decode loop -- after every step but the last each request appends
    one token (latent rows of every layer and an indexer key), so the context
    grows by one per step.  T must be a multiple of 64: the first appended token
    opens a new page, whose latent and indexer blocks come from two free lists of
    spare blocks (a seeded order).  The appended rows are the latent's own draws
    past the context (quantized per page like every page); keys come from one
    more page of N(0,1) keys per request, quantized per page."""
    ch = _children(seed)
    P, Hq, H, D = 1, 16, 64, 128
    C = 2 * K
    ctx = np.full(B, T, dtype=np.int32)
    n_app = steps - 1 if append else 0
    if append and T % BLOCK:
        raise ValueError("the append loop needs a page-aligned context")
    Ts = _round_up(T + n_app, BLOCK)
    idx_pool, idx_scale, idx_bt = _indexer_cache(ch, B, ctx, Ts, D, fp8=True)
    w = uniform_f32(ch[5], (B, P, H))
    n_pool, _, hot = _place_blocks(ch, B, [[] for _ in range(B)], C // BLOCK)
    bt = np.full((B, Ts // BLOCK), -1, dtype=np.int32)
    lat, lat_scale = _latent(ch, L, B, ctx + n_app, Ts, fp8=True)
    extra = {}
    if append:
        # spare blocks for the pages the appends open, on two stacks in a seeded order
        npg = -(-n_app // BLOCK)
        ss = np.random.SeedSequence(seed, spawn_key=(10,)).spawn(3)
        g = np.random.Generator(np.random.PCG64(ss[0]))
        free = (n_pool + g.permutation(B * npg)).astype(np.int32)
        n_idx = idx_pool.shape[0]
        idx_free = (n_idx + g.permutation(B * npg)).astype(np.int32)
        n_pool += B * npg
        idx_pool = np.concatenate([idx_pool, np.zeros((B * npg, BLOCK, D), idx_pool.dtype)])
        idx_scale = np.concatenate([idx_scale, np.zeros(B * npg, np.float32)])
        kc, ks = _fp8_rows(ss[1], B * npg, D)                # [B*npg, 64, D], [B*npg]
        i = np.arange(n_app)
        kc = kc.reshape(B, npg * BLOCK, D)[:, :n_app]
        ks = ks.reshape(B, npg)[:, i // BLOCK]
        extra = dict(ctx0=ctx.copy(), free_blocks=free, idx_free_blocks=idx_free,
                     app_keys=np.ascontiguousarray(kc), app_key_scale=np.ascontiguousarray(ks))
    g4 = np.random.Generator(np.random.PCG64(ch[4]))
    q0 = g4.standard_normal((B, P, H, D))
    qs = _ar1_steps(ch, q0, steps, rho)
    kq = ch[3].spawn(steps)
    step_q = [(bf16_bits(qs[s]), _queries(kq[s], (L, B, P, Hq, D_LATENT), "bf16"))
              for s in range(steps)]
    t2s, s2t, st = _empty_hot(B, C, Ts)
    return Workload("norescache_1m", seed, B, P, K, L, Hq, H, D, Ts, ctx, C, "bf16", "e4m3",
                    "e4m3", 1.0 / math.sqrt(D_LATENT), w, idx_pool, idx_scale, idx_bt, None,
                    lat, lat_scale, n_pool, bt, hot, t2s, s2t, st, 0, True, steps, step_q,
                    **extra)


def indexer_inputs(seed: int, ctx_len, T_stride: int, H: int = 64, D: int = 128,
                   bias: bool = True, P: int = 1) -> dict:
    """Indexer-only inputs (no latent cache) for many-request cases: bf16
    queries [B,P,H,D] ~N(0,1), head weights U[0,1), fp8 keys with per-block
    scales in a permuted paged pool, and a bias U[0,1) per token, or None."""
    ch = _children(seed)
    ctx = np.asarray(ctx_len, dtype=np.int32)
    B = len(ctx)
    idx_pool, idx_scale, idx_bt = _indexer_cache(ch, B, ctx, T_stride, D, fp8=True)
    return {"ctx_len": ctx, "T_stride": T_stride, "H": H, "D": D, "P": P,
            "q_idx": _queries(ch[4], (B, P, H, D), "bf16"), "w": uniform_f32(ch[5], (B, P, H)),
            "idx_pool": idx_pool, "idx_scale": idx_scale, "idx_bt": idx_bt,
            "bias": uniform_f32(ch[8], (B, T_stride)) if bias else None}


CONFIG_NAMES = ["tiny_fp32", "resident_fp8", "mixed_128k", "mtp3_agentic", "norescache_1m"]


def by_name(name: str, **kw) -> Workload:
    return {"tiny_fp32": tiny_fp32, "resident_fp8": resident_fp8, "mixed_128k": mixed_128k,
            "mtp3_agentic": mtp3_agentic, "norescache_1m": norescache_1m}[name](**kw)
