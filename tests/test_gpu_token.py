"""GPU parity of the token-level path (the granularity the pages compare MSA with): token
scores, top-budget token selection and attention over the selected tokens, against the
CPU oracle.  Scores within 1e-4 (scaled); the selection bit-exact against the oracle's
top-k on the GPU's scores; attention within the bf16 output gates."""
import numpy as np
import pytest
import torch

import block_sparse_long_06_amd as msa
import oracle
import synth
from synth import workloads as W
from tests.gpu_util import check_out, f64, gen, require_gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    (W.small("tok_bf16", S=3, T=1, N=5000, H=16, Hkv=2, d=128, dI=64, k=16, structure="sink_needles"), 2048),
    (W.small("tok_bf16_multi_q_d64", S=2, T=4, N=3000, H=8, Hkv=2, d=64, dI=32, k=8), 700),
    (W.small("tok_e4m3_keys", S=2, T=1, N=4100, H=16, Hkv=2, d=128, dI=64, k=16, kidx_dtype=synth.FP8), 2048),
    (W.small("tok_budget_covers_row", S=1, T=3, N=1500, H=8, Hkv=1, d=128, dI=128, k=16), 2048),
]


@pytest.mark.parametrize("wl,budget", CASES, ids=[c[0].name for c in CASES])
def test_token_decode_matches_the_oracle(wl, budget):
    require_gpu()
    say("case", wl.name, "budget", budget)
    inputs = gen(wl)
    prob = wl.problem()
    tb = msa.alloc_token_decode(prob, budget)
    msa.run_token_decode(prob, inputs["q"], inputs["k"], inputs["v"], inputs["q_idx"], inputs["k_idx"], tb, budget)
    torch.cuda.synchronize()
    pos = oracle.positions(wl.N, wl.T)
    qI, kI = f64(inputs["q_idx"]), f64(inputs["k_idx"])
    q, K, V = f64(inputs["q"]), f64(inputs["k"]), f64(inputs["v"])
    sc = tb.scores.cpu().numpy()
    sel = tb.sel_tok.cpu().numpy()
    out = f64(tb.out)
    G = wl.G
    causal = np.arange(wl.N)[None, :] <= pos[:, None]
    for s in range(wl.S):
        for g in range(wl.Hkv):
            ref = oracle.slice_token_scores(qI[s, g], pos, kI[s, g])
            err = np.abs(sc[s, g][causal] - ref[causal]) / np.maximum(np.abs(ref[causal]), 1.0)
            say("  s%d g%d token scores: max scaled err %.3e" % (s, g, float(err.max())))
            assert float(err.max()) <= 1e-4
            gpu_rows = np.where(causal, sc[s, g], np.nan)
            np.testing.assert_array_equal(sel[s, g], oracle.slice_token_topk(gpu_rows, pos, budget))
            ref_o = oracle.slice_token_attention(q[s][:, g * G:(g + 1) * G], pos, sel[s, g], K[s, g], V[s, g],
                                                 wl.scale)
            check_out(out[s][:, g * G:(g + 1) * G], ref_o, wl.dtype, what="token s%d g%d" % (s, g))


@pytest.mark.parametrize("kind", ["few_values", "all_equal", "signed_zero", "one_huge"])
def test_token_topk_adversarial_rows(kind):
    require_gpu()
    T, N, budget = 2, 70000, 2048
    wl = W.small("tok_adv", S=1, T=T, N=N, H=8, Hkv=1, d=128, dI=64, k=16)
    prob = wl.problem()
    pos = oracle.positions(N, T)
    rng = np.random.default_rng(5)
    if kind == "few_values":
        rows = rng.integers(0, 3, (T, N)).astype(np.float32)
    elif kind == "all_equal":
        rows = np.full((T, N), 1.5, np.float32)
    elif kind == "signed_zero":
        rows = np.where(rng.random((T, N)) < 0.5, -0.0, 0.0).astype(np.float32)
        rows[:, ::97] = -1.0
    else:
        rows = rng.standard_normal((T, N)).astype(np.float32)
        rows[:, 12345] = 3e38
    _check_topk(prob, rows, pos, budget)


def _check_topk(prob, rows, pos, budget):
    """msa_token_topk on rows [T, N] of one (sequence, group) against the oracle's top-k."""
    T, N = rows.shape
    sc = torch.from_numpy(rows).reshape(1, 1, T, N).cuda()
    sel = torch.empty((1, 1, T, budget), dtype=torch.int32, device="cuda")
    nws = msa.token_workspace_bytes(prob, budget)
    ws = torch.empty((nws,), dtype=torch.uint8, device="cuda")
    msa.token_topk(prob, budget, sc, sel, ws, nws)
    torch.cuda.synchronize()
    ref = oracle.slice_token_topk(np.where(np.arange(N)[None, :] <= pos[:, None], rows, np.nan), pos, budget)
    np.testing.assert_array_equal(sel.cpu().numpy()[0, 0], ref)


@pytest.mark.parametrize("N,budget", [(300000, 2048), (200001, 700), (1048576, 8192)])
def test_token_topk_long_rows(N, budget):
    """Rows of many 16384-position chunks (the chunked path): Gaussian scores plus a band
    of large values and a few equal maxima."""
    require_gpu()
    say("long rows", N, "budget", budget)
    T = 2
    wl = W.small("tok_long", S=1, T=T, N=N, H=8, Hkv=1, d=128, dI=64, k=16)
    pos = oracle.positions(N, T)
    rng = np.random.default_rng(N)
    rows = (3.0 * rng.standard_normal((T, N))).astype(np.float32)
    rows[:, 1000:1400] += 6.0
    rows[:, 77777 % N] = rows[:, 5 % N] = 50.0
    _check_topk(wl.problem(), rows, pos, budget)


def test_token_topk_overflow_and_normal_rows_in_one_call():
    """One row whose candidates exceed the chunked path's capacity (all equal: the one-
    workgroup path takes it) next to an ordinary row."""
    require_gpu()
    T, N, budget = 2, 100000, 2048
    wl = W.small("tok_mixed", S=1, T=T, N=N, H=8, Hkv=1, d=128, dI=64, k=16)
    pos = oracle.positions(N, T)
    rows = np.empty((T, N), np.float32)
    rows[0] = 0.25
    rows[1] = np.random.default_rng(3).standard_normal(N).astype(np.float32)
    _check_topk(wl.problem(), rows, pos, budget)
