"""GPU parity of the E4M3-query indexer variant, through the C ABI.

hs_quantize_queries is compared with the oracle's quantization rule bit for
bit (codes and scaled head weights); the E4M3 x E4M3 indexer's scores with the
oracle's indexer over the oracle's own codes; the top-K exactly on the GPU
scores and within the near-tie rule on the oracle's; and the rest of the step
(resolve, copies, attention) as for the bf16 indexer.
"""
import sys

import numpy as np
import pytest

from oracle import numerics, quant
from workloads import gen
from workloads.calibrate_mixed import calibrate
import gpu_check as gc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_indexer_logits_amd import _lib
    _lib.load()


def _quantize_on_gpu(q_bits, w):
    from decode_indexer_logits_amd import _lib
    B, P, H, D = q_bits.shape
    ctx = torch.full((B,), 64, dtype=torch.int32, device="cuda")
    batch = _lib.make_batch(B, P, 64, ctx)
    qd = torch.from_numpy(q_bits.view(np.int16)).cuda()
    wd = torch.from_numpy(w).cuda()
    q8 = torch.full((B, P, H, D), 0x55, dtype=torch.uint8, device="cuda")
    ws = torch.full((B, P, H), 7.0, dtype=torch.float32, device="cuda")
    _lib.quantize_queries(batch, H, D, qd, wd, q8, ws)
    torch.cuda.synchronize()
    return q8.cpu().numpy(), ws.cpu().numpy()


@pytest.mark.parametrize("D", [64, 128])
def test_quantize_queries_bit_exact(D):
    _say(f"quantize D={D}")
    rng = np.random.default_rng(40 + D)
    B, P, H = 3, 2, 64
    q = (rng.standard_normal((B, P, H, D)) * np.exp(rng.uniform(-20, 20, (B, P, H, 1))))
    q = q.astype(np.float32)
    q[0, 0, 0] = 0.0                                    # zero head
    q[0, 0, 1] = 2.0 ** -70                             # below the 2^-64 floor
    q[0, 0, 2, :4] = [2.0 ** -64, -2.0 ** -65, 0, 0]    # at the floor
    q[0, 0, 2, 4:] = 0.0
    # amax 448 makes inv = 1: the codes are the hardware's own rounding of
    # every tie between neighbouring E4M3 values, both signs
    tab = numerics.e4m3fn_table()[:0x7F]
    mids = ((tab[:-1] + tab[1:]) / 2).astype(np.float32)
    for i, h in enumerate(range(3, 3 + 8)):
        d = np.arange(D)
        row = mids[(5 * d + 11 * i) % len(mids)] * np.where((d + i) % 2, -1, 1)
        row[i] = 448.0
        q[0, 1, h] = row
    q[1, 0, 5] = -q[1, 0, 5]
    bits = gen.bf16_bits(q)
    w = rng.standard_normal((B, P, H)).astype(np.float32)
    w[2, 1, :8] = -0.0
    q8, ws = _quantize_on_gpu(bits, w)
    gc.check_quantized(bits, w, q8, ws)
    codes, _, _ = quant.quantize_queries(bits, w)
    assert np.all(codes[0, 0, :2] == 0) and codes[0, 0, 2, 0] == 0x7E   # the floor cases


def _mixed_small(B=4, T=16384, K=512, tail=1024, seed=1003):
    beta, hot, _ = calibrate(seed=seed, B=B, T=T, K=K, tail=tail)
    return gen.mixed_128k(seed=seed, B=B, T=T, K=K, tail=tail, beta=beta, hot_tokens=hot)


def _workload(name):
    if name == "resident_fp8":
        return gen.resident_fp8(B=4)
    if name == "resident_ragged":
        return gen.resident_fp8(B=5, T_lo=1, T_hi=3000, K=512)
    if name == "mixed_small":
        return _mixed_small()
    if name == "mtp3_small":
        return gen.mtp3_agentic(B=3, K=128, steps=2, first_turn=6000, per_turn=300, turns=5,
                                out_max=50)
    if name in ("spec_p2", "spec_p3"):
        return gen.mtp3_agentic(B=3, K=128, steps=2, first_turn=9000, per_turn=300, turns=5,
                                out_max=50, P=int(name[-1]))
    raise KeyError(name)


@pytest.mark.parametrize("name", ["resident_fp8", "resident_ragged", "mixed_small", "mtp3_small",
                                  "spec_p2", "spec_p3"])
def test_e4m3_indexer_step_against_oracle(name):
    from decode_indexer_logits_amd.device import DeviceStep
    wl = _workload(name)
    _say(f"e4m3 indexer {name}: B={wl.B} P={wl.P} K={wl.K} ctx={wl.ctx_len.tolist()[:6]}")
    ds = DeviceStep(wl, indexer_q="e4m3")
    ost = gc.oracle_state(wl)
    for s in range(1, min(wl.steps, 2) + 1):
        if s > 1:
            ds.set_queries(s)
        ds.run()
        ost, rr, info = gc.full_check(ds, wl, ost, s=s, attn_tol=2e-2)
        _say(f"step {s}", {k: v for k, v in info.items() if k != "counts"})


def test_e4m3_indexer_fused_topk_matches_separate_calls():
    from decode_indexer_logits_amd.device import DeviceStep
    wl = gen.mtp3_agentic(B=3, K=128, steps=1, first_turn=6000, per_turn=300, turns=5, out_max=50)
    _say("e4m3 fused vs separate, P=4")
    ds = DeviceStep(wl, indexer_q="e4m3")
    ds.run_indexer()
    ds.run_topk()
    torch.cuda.synchronize()
    s1, t1 = ds.scores.cpu().numpy(), ds.topk.cpu().numpy()
    ds.run_indexer_topk()
    torch.cuda.synchronize()
    s2, t2 = ds.scores.cpu().numpy(), ds.topk.cpu().numpy()
    for b in range(wl.B):
        for p in range(wl.P):
            n = int(wl.ctx_len[b]) - wl.P + p + 1
            assert np.array_equal(s1[b, p, :n].view(np.uint32), s2[b, p, :n].view(np.uint32))
    assert np.array_equal(t1, t2)
