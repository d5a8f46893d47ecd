"""GPU parity of the per-sequence decode calls: ragged cache lengths and paged caches.

Expected values come from the CPU oracle run per sequence on its first kv_lens[s]
positions: a ragged batch is S independent dense problems, and a paged cache only stores
the same rows elsewhere.  The pools are built on the device by copying the seeded dense
caches into shuffled pages.  Every page that no sequence owns, and every row past a
sequence's length, holds NaN, so any read outside a sequence shows up as a non-finite
score or output."""
import numpy as np
import pytest
import torch

import block_sparse_long_06_amd as msa
import oracle
import synth
from synth import workloads as W
from tests.gpu_util import check_out, check_scores, f64, gen, require_gpu, say

pytestmark = pytest.mark.gpu

B = 128

CASES = [
    (W.small("kv_bf16", S=5, T=1, N=3000, H=16, Hkv=2, d=128, dI=64, k=16, structure="sink_needles"),
     [3000, 1, 128, 1000, 2049]),
    (W.small("kv_fp32", S=3, T=1, N=2000, H=8, Hkv=2, d=64, dI=32, k=4, dtype=synth.F32), [2000, 700, 129]),
    (W.small("kv_bf16_multi_q_e4m3", S=3, T=4, N=2500, H=8, Hkv=2, d=64, dI=32, k=8, kidx_dtype=synth.FP8),
     [2500, 4, 1337]),
    (W.small("kv_bf16_g8_dI128", S=2, T=2, N=4000, H=16, Hkv=2, d=128, dI=128, k=16), [4000, 3900]),
]


def _nan_fill(t):
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(0x7FC0)
    elif t.dtype == torch.float8_e4m3fn:
        t.view(torch.uint8).fill_(0x7F)
    else:
        t.fill_(float("nan"))
    return t


def _page_table(lens, nb, seed, spare=3, extra_cols=2):
    """Shuffled page ids for the blocks each sequence holds; -1 elsewhere."""
    need = [(n + B - 1) // B for n in lens]
    num_pages = sum(need) + spare
    perm = np.random.default_rng(seed).permutation(num_pages)
    table = np.full((len(lens), nb + extra_cols), -1, dtype=np.int32)
    i = 0
    for s, m in enumerate(need):
        table[s, :m] = perm[i:i + m]
        i += m
    return table, num_pages


def _to_pool(dense, lens, table, num_pages):
    S, Hkv, N, w = dense.shape
    pool = _nan_fill(torch.empty((num_pages, Hkv, B, w), dtype=dense.dtype, device=dense.device))
    for s in range(S):
        for b in range((lens[s] + B - 1) // B):
            n = min(B, lens[s] - b * B)
            pool[int(table[s, b]), :, :n, :] = dense[s, :, b * B:b * B + n, :]
    return pool


def _ragged_dense(dense, lens):
    out = dense.clone()
    for s, n in enumerate(lens):
        _nan_fill(out[s, :, n:, :])
    return out


def _run(prob, lay, inputs, caches):
    db = msa.alloc_decode(prob)
    msa.run_decode_kv(prob, lay, inputs["q"], caches["k"], caches["v"], inputs["q_idx"], caches["k_idx"], db)
    torch.cuda.synchronize()
    return db


def _verify(wl, inputs, lens, db, what):
    qI, kI = f64(inputs["q_idx"]), f64(inputs["k_idx"])
    q, K, V = f64(inputs["q"]), f64(inputs["k"]), f64(inputs["v"])
    sc = db.scores.cpu().numpy()
    sel = db.sel.cpu().numpy()
    out = f64(db.out)
    G = wl.G
    for s in range(wl.S):
        n = lens[s]
        pos = oracle.positions(n, wl.T)
        for g in range(wl.Hkv):
            ref_sc = oracle.slice_index_scores(qI[s, g], pos, kI[s, g, :n], B)
            nbs = ref_sc.shape[1]
            check_scores(sc[s, g][:, :nbs], ref_sc, pos, what="%s s%d g%d len %d" % (what, s, g, n))
            np.testing.assert_array_equal(sel[s, g], oracle.slice_block_topk(sc[s, g][:, :nbs], pos // B, wl.k))
            ref = oracle.slice_attention(q[s][:, g * G:(g + 1) * G], pos, sel[s, g], K[s, g, :n], V[s, g, :n], B,
                                         wl.scale)
            check_out(out[s][:, g * G:(g + 1) * G], ref, wl.dtype, what="%s s%d g%d" % (what, s, g))


@pytest.mark.parametrize("wl,lens", CASES, ids=[c[0].name for c in CASES])
def test_ragged_and_paged_decode_match_the_oracle(wl, lens):
    require_gpu()
    say("case", wl.name, "lens", lens)
    inputs = gen(wl)
    prob = wl.problem()
    kv_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    # ragged dense caches (rows past each length are NaN)
    dense = {n: _ragged_dense(inputs[n], lens) for n in ("k", "v", "k_idx")}
    db_dense = _run(prob, msa.kv_layout(kv_lens), inputs, dense)
    _verify(wl, inputs, lens, db_dense, "ragged dense")
    # paged caches (shuffled pages; unowned pages and tails are NaN)
    table, num_pages = _page_table(lens, wl.nb, seed=wl.seed)
    tdev = torch.from_numpy(table).cuda()
    pools = {n: _to_pool(inputs[n], lens, table, num_pages) for n in ("k", "v", "k_idx")}
    db_paged = _run(prob, msa.kv_layout(kv_lens, tdev, num_pages), inputs, pools)
    _verify(wl, inputs, lens, db_paged, "paged")
    # same arithmetic, different addressing: bit-identical
    np.testing.assert_array_equal(db_paged.sel.cpu().numpy(), db_dense.sel.cpu().numpy())
    assert torch.equal(db_paged.out.view(torch.uint8), db_dense.out.view(torch.uint8))


def test_full_lengths_equal_the_dense_decode_call():
    require_gpu()
    wl = CASES[0][0]
    inputs = gen(wl)
    prob = wl.problem()
    ref = msa.alloc_decode(prob)
    msa.run_decode(prob, inputs["q"], inputs["k"], inputs["v"], inputs["q_idx"], inputs["k_idx"], ref)
    kv_lens = torch.full((wl.S,), wl.N, dtype=torch.int32, device="cuda")
    got = _run(prob, msa.kv_layout(kv_lens), inputs, {n: inputs[n] for n in ("k", "v", "k_idx")})
    np.testing.assert_array_equal(got.sel.cpu().numpy(), ref.sel.cpu().numpy())
    assert torch.equal(got.out.view(torch.uint8), ref.out.view(torch.uint8))


def test_out_of_contract_device_values_stay_in_bounds():
    """kv_lens outside [T, N] are clamped; a page id outside the pool reads as zeros."""
    require_gpu()
    wl = W.small("kv_bad_values", S=3, T=1, N=1500, H=8, Hkv=2, d=128, dI=64, k=8)
    inputs = gen(wl)
    prob = wl.problem()
    given = [0, wl.N + 500, 1000]
    lens = [wl.T, wl.N, 1000]            # what the kernels use
    table, num_pages = _page_table(lens, wl.nb, seed=7)
    pools = {n: _to_pool(inputs[n], lens, table, num_pages) for n in ("k", "v", "k_idx")}
    # block 3 of sequence 1 and block 0 of sequence 2 point outside the pool: they read as 0
    table[1, 3] = -5
    table[2, 0] = num_pages + 11
    zeroed = {n: inputs[n].clone() for n in ("k", "v", "k_idx")}
    for n in zeroed:
        zeroed[n][1, :, 3 * B:4 * B, :] = 0
        zeroed[n][2, :, 0:B, :] = 0
    kv_lens = torch.tensor(given, dtype=torch.int32, device="cuda")
    lay = msa.kv_layout(kv_lens, torch.from_numpy(table).cuda(), num_pages)
    db = _run(prob, lay, inputs, pools)
    ref_inputs = dict(inputs, **zeroed)
    _verify(wl, ref_inputs, lens, db, "clamped / zero pages")


PREFILL_CASES = [
    (W.small("kvp_bf16", S=3, T=300, N=4000, H=16, Hkv=2, d=128, dI=64, k=16, structure="band_sink_needles"),
     [4000, 300, 2345]),
    (W.small("kvp_fp32", S=2, T=260, N=1500, H=8, Hkv=2, d=64, dI=32, k=4, dtype=synth.F32), [1500, 777]),
    (W.small("kvp_e4m3_g1", S=2, T=512, N=3000, H=2, Hkv=2, d=128, dI=64, k=8, kidx_dtype=synth.FP8), [3000, 1029]),
]


def _run_prefill(prob, lay, inputs, caches):
    pb = msa.alloc_prefill(prob)
    msa.run_prefill_kv(prob, lay, inputs["q"], caches["k"], caches["v"], inputs["q_idx"], caches["k_idx"], pb)
    torch.cuda.synchronize()
    return pb


@pytest.mark.parametrize("wl,lens", PREFILL_CASES, ids=[c[0].name for c in PREFILL_CASES])
def test_ragged_and_paged_prefill_match_the_oracle(wl, lens):
    require_gpu()
    say("case", wl.name, "lens", lens)
    inputs = gen(wl)
    prob = wl.problem()
    kv_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dense = {n: _ragged_dense(inputs[n], lens) for n in ("k", "v", "k_idx")}
    pb_dense = _run_prefill(prob, msa.kv_layout(kv_lens), inputs, dense)
    _verify(wl, inputs, lens, pb_dense, "ragged dense prefill")
    table, num_pages = _page_table(lens, wl.nb, seed=wl.seed + 1)
    pools = {n: _to_pool(inputs[n], lens, table, num_pages) for n in ("k", "v", "k_idx")}
    pb_paged = _run_prefill(prob, msa.kv_layout(kv_lens, torch.from_numpy(table).cuda(), num_pages), inputs, pools)
    _verify(wl, inputs, lens, pb_paged, "paged prefill")
    np.testing.assert_array_equal(pb_paged.sel.cpu().numpy(), pb_dense.sel.cpu().numpy())
    assert torch.equal(pb_paged.out.view(torch.uint8), pb_dense.out.view(torch.uint8))
