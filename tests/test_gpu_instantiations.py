"""GPU parity of every kernel instantiation the C ABI accepts, against the CPU oracle.

The bf16 matrix-core kernels are compiled per (head dim d, group size G): the
Outer-Gather-Q kernel and the query-tile kernel of the prefill, the decode split-K
kernel and the attention backward.  The ABI accepts d in {64, 128} and G in
{1, 2, 4, 8, 16}, so each of those ten pairs runs here:

  * prefill through all three attention schedules -- the default (tile kernel on its
    own stream beside Outer-Gather-Q), the tile kernel on the caller's stream
    (MSA_TILE_OVERLAP=0, bit-identical to the default), and Outer-Gather-Q alone
    (MSA_HOT_TILES=0) -- each gated against the oracle.  The structured index inputs
    make both kernels take pairs (about 90 % tile-shared, the rest Outer-Gather-Q),
    which the test asserts from the selection;
  * decode at T = 1 and T = 3;
  * a non-default softmax_scale (1.0: logits of standard deviation sqrt(d), far past
    the default 1/sqrt(d)), for prefill in all three schedules, decode, and the float32
    kernels.

The attention backward's ten instantiations are covered in test_gpu_train.py."""
import numpy as np
import pytest
import torch

import bench
import block_sparse_long_06_amd as msa
import oracle
import synth
from synth import workloads as W
from tests.gpu_util import check_out, f64, full_prefill, gen, require_gpu, say, verify_prefill

pytestmark = pytest.mark.gpu

DG = [(d, G) for d in (128, 64) for G in (1, 2, 4, 8, 16)]


def _prefill_wl(d, G, scale=0.0, dtype=synth.BF16):
    Hkv = 1 if G == 16 else 2
    name = "prefill_d%d_g%d%s" % (d, G, "_scale%g" % scale if scale else "")
    # 1280 queries at the end of a 4096-key cache (ten query tiles, a ragged chunk offset)
    return W.small(name, S=1, T=1280, N=4096, H=G * Hkv, Hkv=Hkv, d=d, dI=64, k=16, dtype=dtype,
                   structure="band_sink_needles", softmax_scale=scale)


def _three_schedules(wl, monkeypatch):
    inputs = gen(wl)
    _, on = full_prefill(wl, inputs)
    monkeypatch.setenv("MSA_TILE_OVERLAP", "0")
    _, serial = full_prefill(wl, inputs)
    monkeypatch.delenv("MSA_TILE_OVERLAP")
    monkeypatch.setenv("MSA_HOT_TILES", "0")
    _, ogq = full_prefill(wl, inputs)
    monkeypatch.delenv("MSA_HOT_TILES")
    # both attention kernels must have had pairs to process
    hot, _ = bench.query_tile_split(wl, on.sel)
    n_hot, n_valid = int(hot.sum()), int((on.sel >= 0).sum())
    say("  pairs: %d tile-shared, %d Outer-Gather-Q" % (n_hot, n_valid - n_hot))
    assert 0 < n_hot < n_valid
    for bufs, what in ((on, "default"), (serial, "tile kernel on the caller's stream"),
                       (ogq, "Outer-Gather-Q only")):
        say("  schedule:", what)
        verify_prefill(wl, inputs, bufs)
    assert torch.equal(on.out.view(torch.uint8), serial.out.view(torch.uint8))
    check_out(f64(on.out), f64(ogq.out), wl.dtype, what="query tiles on vs off")


@pytest.mark.parametrize("d,G", DG, ids=["d%d_g%d" % x for x in DG])
def test_prefill_every_instantiation(d, G, monkeypatch):
    require_gpu()
    wl = _prefill_wl(d, G)
    say("case", wl.name)
    _three_schedules(wl, monkeypatch)


@pytest.mark.parametrize("d,G", [(128, 8), (64, 2), (128, 16)], ids=["d128_g8", "d64_g2", "d128_g16"])
def test_prefill_softmax_scale_one(d, G, monkeypatch):
    require_gpu()
    wl = _prefill_wl(d, G, scale=1.0)
    say("case", wl.name)
    _three_schedules(wl, monkeypatch)


def _decode_check(wl):
    inputs = gen(wl)
    prob = wl.problem()
    db = msa.alloc_decode(prob)
    msa.run_decode(prob, inputs["q"], inputs["k"], inputs["v"], inputs["q_idx"], inputs["k_idx"], db)
    torch.cuda.synchronize()
    pos = oracle.positions(wl.N, wl.T)
    q, K, V = f64(inputs["q"]), f64(inputs["k"]), f64(inputs["v"])
    sc, sel, out = db.scores.cpu().numpy(), db.sel.cpu().numpy(), f64(db.out)
    G = wl.G
    for s in range(wl.S):
        for g in range(wl.Hkv):
            np.testing.assert_array_equal(sel[s, g], oracle.slice_block_topk(sc[s, g], pos // 128, wl.k))
            ref = oracle.slice_attention(q[s][:, g * G:(g + 1) * G], pos, sel[s, g], K[s, g], V[s, g], 128,
                                         wl.scale)
            check_out(out[s][:, g * G:(g + 1) * G], ref, wl.dtype, what="decode s%d g%d" % (s, g))


@pytest.mark.parametrize("d,G", DG, ids=["d%d_g%d" % x for x in DG])
@pytest.mark.parametrize("T", [1, 3])
def test_decode_every_instantiation(d, G, T):
    require_gpu()
    Hkv = 1 if G == 16 else 2
    wl = W.small("decode_d%d_g%d_T%d" % (d, G, T), S=2, T=T, N=2900, H=G * Hkv, Hkv=Hkv, d=d, dI=64, k=16,
                 structure="sink_needles")
    say("case", wl.name)
    _decode_check(wl)


@pytest.mark.parametrize("d,G,dtype", [(128, 8, synth.BF16), (64, 16, synth.BF16), (64, 4, synth.F32),
                                       (128, 2, synth.F32)],
                         ids=["bf16_d128_g8", "bf16_d64_g16", "fp32_d64_g4", "fp32_d128_g2"])
def test_decode_softmax_scale_one(d, G, dtype):
    require_gpu()
    Hkv = 1 if G == 16 else 2
    wl = W.small("decode_scale1_d%d_g%d" % (d, G), S=2, T=2, N=2100, H=G * Hkv, Hkv=Hkv, d=d, dI=32, k=8,
                 dtype=dtype, softmax_scale=1.0)
    say("case", wl.name)
    _decode_check(wl)


@pytest.mark.parametrize("scale", [1.0, 0.02])
def test_prefill_float32_softmax_scale(scale):
    require_gpu()
    wl = W.small("prefill_fp32_scale%g" % scale, S=1, T=600, N=900, H=8, Hkv=2, d=64, dI=32, k=4,
                 dtype=synth.F32, softmax_scale=scale)
    say("case", wl.name)
    inputs = gen(wl)
    _, bufs = full_prefill(wl, inputs)
    verify_prefill(wl, inputs, bufs)
