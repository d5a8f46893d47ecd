"""Helpers shared by the GPU parity tests: device inputs, host copies, comparisons.

Inputs come from the seeded generator (synth); expected values come only from the
CPU oracle.  Nothing here computes any step of the method."""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_sparse_long_06_amd as msa
import oracle
import synth

SCORE_RTOL = 1e-4                    # |d| <= 1e-4 * max(|ref|, 1)  (fp32 accumulation)
# |d| <= ATOL * max(|ref|, 1) per element: the absolute gate for outputs up to unit size
# (every default-scale workload: |o| ~ 0.03-0.05).  Above it the bf16 roundings scale with
# the value (P, the partial O and the output each carry 2^-9 relative), e.g. at a logit
# scale of 1.0, where softmax is peaked and |o| reaches ~4.
ATOL = {synth.BF16: 2e-2, synth.F32: 1e-4}
# bf16 outputs are also held to a relative RMS error of 1% (observed ~0.3%: bf16 inputs,
# P and output rounding).  2e-2 absolute alone cannot see one block too many or too few
# in a 16-block selection (outputs are ~0.03-0.05 in size); such an error is several %.
REL_RMS_MAX = {synth.BF16: 1e-2, synth.F32: 1e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    msa.lib()


def gen(wl, names=("q", "k", "v", "q_idx", "k_idx")):
    specs = wl.specs()
    return {n: synth.device_tensor(specs[n]) for n in names}


def f64(t) -> np.ndarray:
    return oracle.decode(t)


def check_scores(gpu_rows, ref_rows, pos, B=128, what=""):
    """gpu_rows/ref_rows [R, nb]: compare eligible entries (b <= own block)."""
    R, nb = ref_rows.shape
    elig = np.arange(nb)[None, :] <= (pos // B)[:, None]
    g = gpu_rows[elig].astype(np.float64)
    r = ref_rows[elig]
    err = np.abs(g - r) / np.maximum(np.abs(r), 1.0)
    worst = float(err.max()) if err.size else 0.0
    say("  scores %s: %d entries, max scaled err %.3e" % (what, err.size, worst))
    assert np.all(np.isfinite(g)), "non-finite GPU score"
    assert worst <= SCORE_RTOL, "index scores off by %.3e (scaled)" % worst


def check_out(gpu, ref, dtype, what=""):
    g = gpu.astype(np.float64)
    err = np.abs(g - ref)
    scaled = err / np.maximum(np.abs(ref), 1.0)
    rel_rms = float(np.sqrt(np.mean((g - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))
    say("  out %s: max abs err %.3e (scaled %.3e), rel rms %.3e" % (what, float(err.max()), float(scaled.max()),
                                                                   rel_rms))
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    assert float(scaled.max()) <= ATOL[dtype], "attention output off by %.3e (scaled)" % float(scaled.max())
    assert rel_rms <= REL_RMS_MAX[dtype], "attention output relative RMS error %.3e" % rel_rms
    return rel_rms


def full_prefill(wl, inputs, bufs=None):
    prob = wl.problem()
    bufs = bufs or msa.alloc_prefill(prob)
    msa.run_prefill(prob, inputs["q"], inputs["k"], inputs["v"], inputs["q_idx"], inputs["k_idx"], bufs)
    torch.cuda.synchronize()
    return prob, bufs


def verify_prefill(wl, inputs, bufs):
    """Every stage of one prefill pass against the oracle: scores, selection on the GPU's
    scores (bit-exact), inversion (bit-exact) and attention on the GPU's selection."""
    S, T, N, Hkv, G, nb, k = wl.S, wl.T, wl.N, wl.Hkv, wl.G, wl.nb, wl.k
    pos = oracle.positions(N, T)
    qI, kI = f64(inputs["q_idx"]), f64(inputs["k_idx"])
    q, K, V = f64(inputs["q"]), f64(inputs["k"]), f64(inputs["v"])
    sc = bufs.scores.cpu().numpy()
    sel = bufs.sel.cpu().numpy()
    off = bufs.csr_offsets.cpu().numpy()
    ent = bufs.csr_entries.cpu().numpy()
    out = f64(bufs.out)
    scale = wl.scale
    differ = 0
    for s in range(S):
        for g in range(Hkv):
            ref_sc = oracle.slice_index_scores(qI[s, g], pos, kI[s, g], 128)
            check_scores(sc[s, g], ref_sc, pos, what="s%d g%d" % (s, g))
            ref_sel = oracle.slice_block_topk(sc[s, g], pos // 128, k)
            np.testing.assert_array_equal(sel[s, g], ref_sel)
            differ += int(np.sum(np.any(oracle.slice_block_topk(ref_sc, pos // 128, k) != sel[s, g], axis=1)))
            r_off, r_ent = oracle.slice_invert(sel[s, g], nb)
            base = off[s, g, 0]
            np.testing.assert_array_equal(off[s, g] - base, r_off)
            np.testing.assert_array_equal(ent[base:base + r_off[-1]], r_ent)
            ref = oracle.slice_attention(q[s][:, g * G:(g + 1) * G], pos, sel[s, g], K[s, g], V[s, g], 128, scale)
            check_out(out[s][:, g * G:(g + 1) * G], ref, wl.dtype, what="s%d g%d" % (s, g))
    say("  rows whose independent oracle selection differs: %d of %d" % (differ, S * Hkv * T))
    assert off[-1, -1, -1] == np.sum(sel >= 0)
