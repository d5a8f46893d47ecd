"""GPU parity of the fused selection (index scores + top-k without the block-score matrix):
its output must be bit-identical to msa_index_scores followed by msa_block_topk (whose
selection the forward parity tests gate against the oracle), on shapes that span several
16-block chunks, several 1024-block spans, ragged tails, E4M3 keys and k in {1, 4, 16}.  Every
row is also checked against the oracle: its top-k of the GPU's scores (bit-exact) and its
index scores (1e-4 scaled)."""
import numpy as np
import pytest
import torch

import block_sparse_long_06_amd as msa
import oracle
import synth
from synth import workloads as W
from tests.gpu_util import check_scores, f64, gen, require_gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    W.small("fused_bf16", S=1, T=3000, N=3000, H=16, Hkv=2, d=128, dI=64, k=16),
    W.small("fused_structured_ragged", S=2, T=1000, N=3333, H=16, Hkv=2, d=128, dI=64, k=16,
            structure="band_sink_needles"),
    W.small("fused_two_spans", S=1, T=300, N=140000, H=8, Hkv=1, d=128, dI=64, k=16),
    W.small("fused_e4m3_dI32_k4", S=1, T=2048, N=2600, H=8, Hkv=2, d=64, dI=32, k=4, kidx_dtype=synth.FP8),
    W.small("fused_dI128_k1", S=1, T=700, N=900, H=8, Hkv=1, d=128, dI=128, k=1),
    W.small("fused_short_T", S=2, T=40, N=5000, H=8, Hkv=2, d=128, dI=64, k=16),
    # chunks far into their sequences: eight-wave workgroups (1024 query rows), a ragged
    # second row tile, and E4M3 keys at d_I = 32
    W.small("fused_chunk_at_end", S=2, T=1500, N=40000, H=8, Hkv=2, d=128, dI=64, k=16),
    W.small("fused_e4m3_chunk_at_end", S=1, T=700, N=30000, H=8, Hkv=2, d=64, dI=32, k=4, kidx_dtype=synth.FP8),
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
    # and on every row the selection is the oracle's top-k of the (unfused) GPU scores, and
    # those scores are the oracle's within the indexer tolerance
    pos = oracle.positions(wl.N, wl.T)
    sc = scores.cpu().numpy()
    qI, kI = f64(x["q_idx"]), f64(x["k_idx"])
    for s in range(wl.S):
        for g in range(wl.Hkv):
            np.testing.assert_array_equal(a[s, g], oracle.slice_block_topk(sc[s, g], pos // 128, wl.k))
            check_scores(sc[s, g], oracle.slice_index_scores(qI[s, g], pos, kI[s, g], 128), pos,
                         what="s%d g%d" % (s, g))
    # the candidate workspace is far smaller than the block-score matrix it replaces
    if wl.T >= 256:
        assert ws.numel() < scores.numel() * 4 or wl.nb < 64


E2E = [CASES[0], CASES[1], CASES[3]]


@pytest.mark.parametrize("wl", E2E, ids=[c.name for c in E2E])
def test_fused_prefill_pass_equals_the_unfused_pass(wl):
    """A whole prefill pass with the fused selection (alloc_prefill(fused_selection=True))
    gives the same selection, inversion and attention output, bit for bit, as the pass
    through the block-score matrix (which verify_prefill gates against the oracle)."""
    require_gpu()
    say("case", wl.name)
    x = gen(wl)
    prob = wl.problem()
    ref = msa.alloc_prefill(prob)
    fused = msa.alloc_prefill(prob, fused_selection=True)
    assert fused.scores is None and fused.ws_select is not None
    for bufs in (ref, fused):
        msa.run_prefill(prob, x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], bufs)
    torch.cuda.synchronize()
    for name in ("sel", "csr_offsets"):
        assert torch.equal(getattr(ref, name), getattr(fused, name)), name
    # csr_entries is sized for every pair; only the prefix the offsets cover is written
    used = int(ref.csr_offsets[-1, -1, -1])
    assert torch.equal(ref.csr_entries[:used], fused.csr_entries[:used])
    assert torch.equal(ref.out.view(torch.uint8), fused.out.view(torch.uint8))
    # a second fused pass over the same buffers repeats the first
    first = fused.out.clone()
    msa.run_prefill(prob, x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], fused)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.uint8), fused.out.view(torch.uint8))
