"""GPU parity of the fused selection (index scores + top-k without the block-score matrix):
its output must be bit-identical to msa_index_scores followed by msa_block_topk (whose
selection the forward parity tests gate against the oracle), on shapes that span several
16-block chunks, several 1024-block spans, ragged tails, E4M3 keys and k in {1, 4, 16}."""
import numpy as np
import pytest
import torch

import block_sparse_long_06_amd as msa
import oracle
import synth
from synth import workloads as W
from tests.gpu_util import gen, require_gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    W.small("fused_bf16", S=1, T=3000, N=3000, H=16, Hkv=2, d=128, dI=64, k=16),
    W.small("fused_structured_ragged", S=2, T=1000, N=3333, H=16, Hkv=2, d=128, dI=64, k=16,
            structure="band_sink_needles"),
    W.small("fused_two_spans", S=1, T=300, N=140000, H=8, Hkv=1, d=128, dI=64, k=16),
    W.small("fused_e4m3_dI32_k4", S=1, T=2048, N=2600, H=8, Hkv=2, d=64, dI=32, k=4, kidx_dtype=synth.FP8),
    W.small("fused_dI128_k1", S=1, T=700, N=900, H=8, Hkv=1, d=128, dI=128, k=1),
    W.small("fused_short_T", S=2, T=40, N=5000, H=8, Hkv=2, d=128, dI=64, k=16),
]


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_fused_selection_equals_the_two_calls(wl):
    require_gpu()
    say("case", wl.name)
    x = gen(wl, names=("q_idx", "k_idx"))
    prob = wl.problem()
    scores = torch.empty((wl.S, wl.Hkv, wl.T, wl.nb), dtype=torch.float32, device="cuda")
    sel_ref = torch.empty((wl.S, wl.Hkv, wl.T, wl.k), dtype=torch.int32, device="cuda")
    msa.index_scores(prob, x["q_idx"], x["k_idx"], scores)
    msa.block_topk(prob, scores, sel_ref)
    ws = torch.empty((max(msa.workspace_bytes(prob, msa.MSA_CALL_INDEX_TOPK), 1),), dtype=torch.uint8, device="cuda")
    sel = torch.full((wl.S, wl.Hkv, wl.T, wl.k), -7, dtype=torch.int32, device="cuda")
    msa.index_topk(prob, x["q_idx"], x["k_idx"], sel, ws, ws.numel())
    torch.cuda.synchronize()
    a, b = sel.cpu().numpy(), sel_ref.cpu().numpy()
    say("  rows %d, equal rows %d" % (a.shape[0] * a.shape[1] * a.shape[2], int((a == b).all(-1).sum())))
    np.testing.assert_array_equal(a, b)
    # and the selection is the oracle's top-k of the (unfused) GPU scores on a sample of rows
    pos = oracle.positions(wl.N, wl.T)
    rows = np.unique(np.linspace(0, wl.T - 1, 64).astype(int))
    sc = scores.cpu().numpy()
    for s in range(wl.S):
        for g in range(wl.Hkv):
            np.testing.assert_array_equal(a[s, g][rows], oracle.slice_block_topk(sc[s, g][rows], pos[rows] // 128,
                                                                                wl.k))
    # the candidate workspace is far smaller than the block-score matrix it replaces
    if wl.T >= 256:
        assert ws.numel() < scores.numel() * 4 or wl.nb < 64
