"""The allocation-free decode call (msa_sparse_attn_decode_noalloc) against the workspace
call it mirrors (msa_sparse_attn_decode), through the C ABI.

Both run the same kernels on the same selection, so the outputs must be bit-identical;
each is also held to the oracle's attention at the bf16 / fp32 gates.  Three calls in a
row share the library's static scratch: a large bf16 problem, then a smaller one (the
scratch then holds the first call's partials beyond the second's), then a float32 one."""
import numpy as np
import pytest
import torch

import block_sparse_long_06_amd as msa
import oracle
import synth
from synth import workloads as W
from tests.gpu_util import check_out, f64, gen, require_gpu, say

pytestmark = pytest.mark.gpu


def _compare(wl):
    say("case", wl.name)
    inputs = gen(wl)
    prob = wl.problem()
    need = msa.workspace_bytes(prob, msa.MSA_CALL_DECODE)
    assert 0 < need <= msa.DECODE_SCRATCH_BYTES
    db = msa.alloc_decode(prob)
    msa.run_decode(prob, inputs["q"], inputs["k"], inputs["v"], inputs["q_idx"], inputs["k_idx"], db)
    out = torch.full_like(db.out, float("nan"))
    msa.sparse_attn_decode_noalloc(prob, inputs["q"], inputs["k"], inputs["v"], db.sel, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), db.out.view(torch.uint8))
    pos = oracle.positions(wl.N, wl.T)
    q, K, V = f64(inputs["q"]), f64(inputs["k"]), f64(inputs["v"])
    sel, got = db.sel.cpu().numpy(), f64(out)
    G = wl.G
    for s in range(wl.S):
        for g in range(wl.Hkv):
            ref = oracle.slice_attention(q[s][:, g * G:(g + 1) * G], pos, sel[s, g], K[s, g], V[s, g], 128, wl.scale)
            check_out(got[s][:, g * G:(g + 1) * G], ref, wl.dtype, what="no-alloc decode s%d g%d" % (s, g))


def test_no_alloc_decode_equals_the_workspace_call_on_consecutive_calls():
    require_gpu()
    _compare(W.small("noalloc_big", S=6, T=3, N=6000, H=32, Hkv=4, d=128, dI=64, k=16, structure="sink_needles"))
    _compare(W.small("noalloc_small", S=2, T=1, N=2000, H=8, Hkv=2, d=64, dI=32, k=8))
    _compare(W.small("noalloc_fp32", S=2, T=2, N=1500, H=4, Hkv=2, d=64, dI=32, k=4, dtype=synth.F32))


def test_no_alloc_decode_rejects_a_problem_beyond_the_scratch():
    require_gpu()
    prob = msa.problem(16, 8, 1 << 20, 64, 8, 128, 64, 16)
    assert msa.workspace_bytes(prob, msa.MSA_CALL_DECODE) > msa.DECODE_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(msa.MSAError) as ei:
        msa.sparse_attn_decode_noalloc(prob, x, x, x, x, x)
    assert ei.value.status == msa.MSA_ERR_WORKSPACE_TOO_SMALL
