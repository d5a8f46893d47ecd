"""GPU parity: every C-ABI call against the CPU oracle on seeded inputs.

Shapes here are small enough for the oracle to finish in seconds, yet span several
tiles of every kernel and ragged tails (T and N not multiples of the tile sizes,
T < N chunks, G in {1, 4, 8, 16}, d in {64, 128}, dI in {32, 64, 128}).

Gates: index scores within 1e-4 (scaled); selection bit-exact when the oracle is
fed the GPU's block scores; inversion bit-exact; attention within 2e-2 absolute
(bf16) / 1e-4 (fp32) on the GPU's selection."""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_long_06_amd as msa
import oracle
import synth
from synth import workloads as W
from tests.gpu_util import check_out, check_scores, f64, full_prefill, gen, require_gpu, say, verify_prefill

pytestmark = pytest.mark.gpu

CASES = [
    W.C0,
    W.small("bf16_g8_ragged_chunk", S=2, T=700, N=1000, H=16, Hkv=2, d=128, dI=64, k=4),
    W.small("bf16_g4_d64_dI32", S=1, T=3000, N=3000, H=8, Hkv=2, d=64, dI=32, k=16),
    W.small("bf16_g16_dI128_chunk", S=1, T=300, N=4500, H=16, Hkv=1, d=128, dI=128, k=8),
    W.small("bf16_g1_k3", S=1, T=1500, N=1500, H=2, Hkv=2, d=64, dI=64, k=3),
    W.small("bf16_short_T_full_budget", S=1, T=100, N=2000, H=16, Hkv=2, d=128, dI=64, k=16),
    W.small("bf16_k1_block_local", S=1, T=600, N=900, H=8, Hkv=1, d=128, dI=64, k=1),
    W.small("bf16_structured", S=1, T=4096, N=4096, H=16, Hkv=2, d=128, dI=64, k=16,
            structure="band_sink_needles"),
    W.small("bf16_structured_ragged", S=2, T=1000, N=3000, H=16, Hkv=2, d=128, dI=64, k=16,
            structure="band_sink_needles"),
    # k >= nb for most rows: every causal block is chosen by every row of a tile, so the
    # last tiles have more than 32 blocks that qualify as tile-shared (the cap applies)
    W.small("bf16_k64_all_blocks_shared", S=1, T=5120, N=5120, H=8, Hkv=1, d=128, dI=64, k=64),
    # k > 16 (the generic selection, inversion and merge paths) with structured selections,
    # queries from position 700: query tiles straddle the inversion's 64-row steps
    W.small("bf16_k24_structured_offset", S=1, T=1900, N=2600, H=16, Hkv=2, d=128, dI=64, k=24,
            structure="band_sink_needles"),
    # degenerate sizes: a cache that is one partial block (only the own block exists, every
    # row's selection is that block alone), and exactly one full block
    W.small("bf16_one_partial_block", S=2, T=77, N=77, H=8, Hkv=1, d=128, dI=64, k=16),
    W.small("bf16_exactly_one_block", S=1, T=128, N=128, H=16, Hkv=2, d=64, dI=64, k=4),
    W.small("fp32_one_partial_block", S=1, T=50, N=50, H=4, Hkv=1, d=64, dI=32, k=4, dtype=synth.F32),
    W.small("fp32_g2_d128", S=2, T=500, N=777, H=4, Hkv=2, d=128, dI=64, k=5, dtype=synth.F32),
    W.small("fp32_g8_d64", S=1, T=1200, N=1300, H=8, Hkv=1, d=64, dI=32, k=6, dtype=synth.F32),
]


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_prefill_pipeline_matches_oracle(wl):
    require_gpu()
    say("case", wl.name)
    inputs = gen(wl)
    _, bufs = full_prefill(wl, inputs)
    verify_prefill(wl, inputs, bufs)


# 1-byte index keys (OCP E4M3; the serving variant): matrix-core indexer (T >= 256),
# the row kernel (8 < T < 256) and, below, the decode stream.  The oracle decodes the
# same E4M3 bytes exactly.
FP8_CASES = [
    W.small("bf16_e4m3_keys_structured", S=1, T=2048, N=3000, H=16, Hkv=2, d=128, dI=64, k=16,
            structure="band_sink_needles", kidx_dtype=synth.FP8),
    W.small("bf16_e4m3_keys_rows_dI128", S=2, T=100, N=1500, H=8, Hkv=2, d=64, dI=128, k=8, kidx_dtype=synth.FP8),
    W.small("bf16_e4m3_keys_dI32", S=1, T=700, N=900, H=4, Hkv=1, d=64, dI=32, k=4, kidx_dtype=synth.FP8),
]


@pytest.mark.parametrize("wl", FP8_CASES, ids=[c.name for c in FP8_CASES])
def test_prefill_with_e4m3_index_keys(wl):
    require_gpu()
    say("case", wl.name)
    inputs = gen(wl)
    assert inputs["k_idx"].dtype == torch.float8_e4m3fn
    _, bufs = full_prefill(wl, inputs)
    verify_prefill(wl, inputs, bufs)


QT_OFF_CASES = [c for c in CASES if c.name in ("bf16_g8_ragged_chunk", "bf16_structured",
                                                 "bf16_k64_all_blocks_shared", "bf16_g1_k3")]


@pytest.mark.parametrize("wl", QT_OFF_CASES, ids=[c.name for c in QT_OFF_CASES])
def test_prefill_without_query_tiles(wl, monkeypatch):
    """MSA_HOT_TILES=0: every (row, block) pair takes the Outer-Gather-Q kernel.  The
    output matches the oracle, and the default run (query-tile pass for tile-shared
    blocks) within rounding."""
    require_gpu()
    say("case", wl.name, "(query tiles off)")
    inputs = gen(wl)
    _, on = full_prefill(wl, inputs)
    monkeypatch.setenv("MSA_HOT_TILES", "0")
    _, off = full_prefill(wl, inputs)
    monkeypatch.delenv("MSA_HOT_TILES")
    verify_prefill(wl, inputs, off)
    check_out(f64(on.out), f64(off.out), wl.dtype, what="query tiles on vs off")



@pytest.mark.parametrize("wl", QT_OFF_CASES[:2], ids=[c.name for c in QT_OFF_CASES[:2]])
def test_tile_kernel_on_its_own_stream_changes_no_bit(wl, monkeypatch):
    """The query-tile kernel runs on a second stream beside Outer-Gather-Q by default
    (MSA_TILE_OVERLAP=0 puts it back on the caller's stream after it).  The two write
    disjoint partials, so the outputs are bit-identical, and both match the oracle."""
    require_gpu()
    say("case", wl.name, "(tile kernel overlap on / off)")
    inputs = gen(wl)
    _, on = full_prefill(wl, inputs)
    monkeypatch.setenv("MSA_TILE_OVERLAP", "0")
    _, off = full_prefill(wl, inputs)
    monkeypatch.delenv("MSA_TILE_OVERLAP")
    verify_prefill(wl, inputs, on)
    assert torch.equal(on.out.view(torch.uint8), off.out.view(torch.uint8))


DEC_CASES = [
    W.small("dec_bf16", S=3, T=1, N=5000, H=16, Hkv=2, d=128, dI=64, k=16, structure="sink_needles"),
    W.small("dec_fp32", S=2, T=1, N=3333, H=8, Hkv=2, d=64, dI=32, k=4, dtype=synth.F32),
    W.small("dec_bf16_multi_q", S=2, T=5, N=2000, H=8, Hkv=1, d=128, dI=64, k=8),
    W.small("dec_e4m3_keys", S=3, T=1, N=5000, H=16, Hkv=2, d=128, dI=64, k=16, structure="sink_needles",
            kidx_dtype=synth.FP8),
    W.small("dec_e4m3_keys_multi_q_dI32", S=2, T=3, N=2100, H=8, Hkv=2, d=64, dI=32, k=8, kidx_dtype=synth.FP8),
    # every head-group size the bf16 decode kernel takes (its B operand holds up to 16 heads)
    W.small("dec_bf16_g16", S=2, T=1, N=3000, H=16, Hkv=1, d=128, dI=64, k=16),
    W.small("dec_bf16_g1_d64_multi_q", S=3, T=2, N=2500, H=2, Hkv=2, d=64, dI=64, k=8),
    W.small("dec_bf16_g2", S=2, T=1, N=1800, H=4, Hkv=2, d=128, dI=32, k=4),
    # the first token (one key: attention returns its value) and one key past a block
    # boundary (the own block holds a single key)
    W.small("dec_first_token", S=2, T=1, N=1, H=16, Hkv=2, d=128, dI=64, k=16),
    W.small("dec_one_past_a_block", S=2, T=1, N=129, H=8, Hkv=1, d=128, dI=64, k=16),
]


@pytest.mark.parametrize("wl", DEC_CASES, ids=[c.name for c in DEC_CASES])
def test_decode_matches_oracle_and_prefill(wl):
    require_gpu()
    say("case", wl.name)
    inputs = gen(wl)
    prob = wl.problem()
    db = msa.alloc_decode(prob)
    msa.run_decode(prob, inputs["q"], inputs["k"], inputs["v"], inputs["q_idx"], inputs["k_idx"], db)
    _, pb = full_prefill(wl, inputs)
    torch.cuda.synchronize()
    pos = oracle.positions(wl.N, wl.T)
    qI, kI = f64(inputs["q_idx"]), f64(inputs["k_idx"])
    q, K, V = f64(inputs["q"]), f64(inputs["k"]), f64(inputs["v"])
    sc = db.scores.cpu().numpy()
    sel = db.sel.cpu().numpy()
    out = f64(db.out)
    G = wl.G
    for s in range(wl.S):
        for g in range(wl.Hkv):
            ref_sc = oracle.slice_index_scores(qI[s, g], pos, kI[s, g], 128)
            check_scores(sc[s, g], ref_sc, pos, what="s%d g%d" % (s, g))
            np.testing.assert_array_equal(sel[s, g], oracle.slice_block_topk(sc[s, g], pos // 128, wl.k))
            ref = oracle.slice_attention(q[s][:, g * G:(g + 1) * G], pos, sel[s, g], K[s, g], V[s, g], 128,
                                         wl.scale)
            check_out(out[s][:, g * G:(g + 1) * G], ref, wl.dtype, what="decode s%d g%d" % (s, g))
    # the prefill path on the same problem agrees with the decode path
    np.testing.assert_array_equal(pb.sel.cpu().numpy(), sel)
    check_out(f64(pb.out), out, wl.dtype, what="prefill vs decode")


def test_runs_are_bit_identical():
    require_gpu()
    wl = CASES[1]
    inputs = gen(wl)
    _, b1 = full_prefill(wl, inputs)
    _, b2 = full_prefill(wl, inputs)
    pos = oracle.positions(wl.N, wl.T)
    elig = torch.from_numpy(np.arange(wl.nb)[None, :] <= (pos // 128)[:, None]).cuda()
    assert torch.equal(b1.scores.masked_select(elig.expand_as(b1.scores)),
                       b2.scores.masked_select(elig.expand_as(b2.scores)))
    for name in ("sel", "csr_offsets", "out"):
        assert torch.equal(getattr(b1, name), getattr(b2, name)), name
    n = int(b1.csr_offsets[-1, -1, -1])
    assert torch.equal(b1.csr_entries[:n], b2.csr_entries[:n])


def test_nan_poison_unselected_blocks():
    """Blocks no query selected are filled with NaN: the prefill and decode outputs stay finite
    and bit-identical to those of the unpoisoned run."""
    require_gpu()
    wl = W.small("poison", S=1, T=32, N=8192, H=16, Hkv=2, d=128, dI=64, k=2)
    inputs = gen(wl)
    prob, bufs = full_prefill(wl, inputs)
    ref_out = bufs.out.clone()
    # decode of the same rows before the poisoning (its selection is the prefill's)
    db = msa.alloc_decode(prob)
    msa.run_decode(prob, inputs["q"], inputs["k"], inputs["v"], inputs["q_idx"], inputs["k_idx"], db)
    torch.cuda.synchronize()
    assert torch.equal(db.sel, bufs.sel)
    ref_dec = db.out.clone()
    sel = bufs.sel.cpu().numpy()
    K, V = inputs["k"], inputs["v"]
    poisoned = 0
    for s in range(wl.S):
        for g in range(wl.Hkv):
            used = set(int(b) for b in np.unique(sel[s, g]) if b >= 0)
            for b in range(wl.nb):
                if b not in used:
                    K[s, g, b * 128:(b + 1) * 128] = float("nan")
                    V[s, g, b * 128:(b + 1) * 128] = float("nan")
                    poisoned += 1
    say("  poisoned %d of %d blocks" % (poisoned, wl.S * wl.Hkv * wl.nb))
    assert poisoned > 0
    msa.sparse_attn_prefill(prob, inputs["q"], K, V, bufs.csr_offsets, bufs.csr_entries, bufs.sel, bufs.out,
                            bufs.ws_prefill, bufs.ws_prefill.numel())
    torch.cuda.synchronize()
    assert torch.isfinite(bufs.out.float()).all()
    assert torch.equal(bufs.out, ref_out)
    # decode reads only its selected blocks as well: finite and bit-identical
    db.out.fill_(0)
    msa.run_decode(prob, inputs["q"], K, V, inputs["q_idx"], inputs["k_idx"], db)
    torch.cuda.synchronize()
    assert torch.isfinite(db.out.float()).all()
    assert torch.equal(db.out, ref_dec)


# ------------------------------------------------------------------ adversarial top-k
def _topk_case(scores_np, T, N, k):
    prob = msa.problem(1, T, N, 8, 1, 128, 64, k)
    sc = torch.from_numpy(scores_np.astype(np.float32)).cuda().reshape(1, 1, T, -1).contiguous()
    sel = torch.full((1, 1, T, k), -7, dtype=torch.int32, device="cuda")
    msa.block_topk(prob, sc, sel)
    torch.cuda.synchronize()
    pos = oracle.positions(N, T)
    ref = oracle.slice_block_topk(scores_np.astype(np.float32).astype(np.float64), pos // 128, k)
    np.testing.assert_array_equal(sel.cpu().numpy()[0, 0], ref)


@pytest.mark.parametrize("kind", ["all_equal", "signed_zero", "few_values", "neg_inf_and_huge",
                                  "long_all_equal", "long_random", "long_ties_at_threshold",
                                  "few_values_odd_nb", "long_random_odd_nb", "ties_at_threshold_odd_nb",
                                  "mid_random", "mid_all_equal", "mid_ties_at_threshold", "mid_neg_inf_and_huge",
                                  "mid_random_odd_nb", "int_ties", "mid_int_ties", "long_int_ties"])
@pytest.mark.parametrize("k", [1, 2, 16, 64])
def test_topk_adversarial_rows(kind, k):
    """Rows of up to 300 blocks (held in registers), 130 rows of 8192 blocks (a workgroup
    per row) and 16,500 rows of up to 1100 blocks (more rows than the workgroup-per-row
    kernel takes: rows past 1024 blocks stream the row twice, the rest stay in registers,
    in one launch)."""
    require_gpu()
    rng = np.random.default_rng(zlib.crc32(kind.encode()) * 100 + k)
    if kind.startswith("long"):
        T, N = 130, 8192 * 128
    elif kind.startswith("mid"):
        T, N = 16500, 1100 * 128
        kind = kind[len("mid_"):]
    else:
        T, N = 300, 300 * 128
    if kind.endswith("_odd_nb"):  # nb % 4 != 0: rows are not 16-byte aligned (scalar loads)
        N = N - 128 - 5
        kind = kind[: -len("_odd_nb")]
    nb = (N + 127) // 128
    if kind in ("all_equal", "long_all_equal"):
        sc = np.full((T, nb), 0.75)
    elif kind == "signed_zero":
        sc = rng.choice([-0.0, 0.0, -1.0, 1.0], size=(T, nb))
    elif kind == "few_values":
        sc = rng.integers(0, 3, size=(T, nb)).astype(np.float64)
    elif kind == "neg_inf_and_huge":
        sc = rng.choice([-np.inf, np.inf, -3e38, 3e38, 1e-45, -1e-45], size=(T, nb))
    elif kind in ("random", "long_random"):
        sc = rng.standard_normal((T, nb))
    elif kind in ("int_ties", "long_int_ties"):  # few candidates, often tied at the k-th value
        sc = rng.integers(0, 3 * nb // 2, size=(T, nb)).astype(np.float64)
    else:  # many ties exactly at the k-th value
        sc = rng.standard_normal((T, nb)) - 10
        sc[:, ::3] = 5.0
    _topk_case(sc, T, N, k)


def test_invert_skewed_selection():
    """Every query picks block 0 and its own block (sink-like skew), k = 2."""
    require_gpu()
    T = N = 8192 * 4
    k = 2
    own = oracle.positions(N, T) // 128
    sel_np = np.stack([np.zeros(T, dtype=np.int32), own.astype(np.int32)], axis=1)
    sel_np[own == 0, 1] = -1
    prob = msa.problem(1, T, N, 8, 1, 128, 64, k)
    sel = torch.from_numpy(sel_np).cuda().reshape(1, 1, T, k).contiguous()
    nb = prob.nb
    off = torch.empty((1, 1, nb + 1), dtype=torch.int32, device="cuda")
    ent = torch.empty((T * k,), dtype=torch.int32, device="cuda")
    ws = torch.empty((msa.workspace_bytes(prob, msa.MSA_CALL_INVERT),), dtype=torch.uint8, device="cuda")
    msa.invert_selection(prob, sel, off, ent, ws, ws.numel())
    torch.cuda.synchronize()
    r_off, r_ent = oracle.slice_invert(sel_np, nb)
    np.testing.assert_array_equal(off.cpu().numpy()[0, 0], r_off)
    np.testing.assert_array_equal(ent.cpu().numpy()[: r_off[-1]], r_ent)


def dedup_rows(sel):
    """sel with every repeat of a block id after its first slot in the row set to -1 (the
    inversion's documented handling of rows outside the distinct-ids contract)."""
    out = sel.copy()
    for r in range(out.shape[0]):
        seen = set()
        for i in range(out.shape[1]):
            b = int(out[r, i])
            if b in seen:
                out[r, i] = -1
            elif b >= 0:
                seen.add(b)
    return out


@pytest.mark.parametrize("k", [4, 16, 24])
def test_invert_rows_with_repeated_ids(k):
    """Rows that repeat a block id (outside the contract: msa_block_topk never does) list it
    once, at its first slot; every list position is written (no stale entry for a prefill
    to read as a row index)."""
    require_gpu()
    T, N = 1500, 1500 * 3
    nb = (N + 127) // 128
    rng = np.random.default_rng(1234 + k)
    sel_np = rng.integers(-1, nb, size=(T, k)).astype(np.int32)
    sel_np[:, 1] = sel_np[:, 0]                      # a repeat in every row
    sel_np[::7, -1] = sel_np[::7, 0]                  # and one at the far end
    sel_np[::5] = rng.integers(0, 3, size=(len(sel_np[::5]), k))  # heavy repeats
    # ascending rows (the form the top-k emits, where the kernels skip the pairwise check)
    # with a negative entry followed by a repeat, or a repeat right after its first slot
    asc = np.arange(k, dtype=np.int32) % nb
    for r in range(3, T, 11):
        row = asc.copy()
        if r % 2:
            row[k // 2] = -1
            row[k // 2 + 1] = row[0]
        else:
            row[-1] = row[-2]
        sel_np[r] = row
    sel_np[2::11] = asc                               # ascending, no repeat
    prob = msa.problem(1, T, N, 8, 1, 128, 64, k)
    sel = torch.from_numpy(sel_np).cuda().reshape(1, 1, T, k).contiguous()
    off = torch.empty((1, 1, nb + 1), dtype=torch.int32, device="cuda")
    ent = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty((msa.workspace_bytes(prob, msa.MSA_CALL_INVERT),), dtype=torch.uint8, device="cuda")
    msa.invert_selection(prob, sel, off, ent, ws, ws.numel())
    torch.cuda.synchronize()
    r_off, r_ent = oracle.slice_invert(dedup_rows(sel_np), nb)
    got = ent.cpu().numpy()
    np.testing.assert_array_equal(off.cpu().numpy()[0, 0], r_off)
    np.testing.assert_array_equal(got[: r_off[-1]], r_ent)
    assert np.all(got[: r_off[-1]] >= 0)


def test_generator_device_matches_host():
    require_gpu()
    for wl in (W.small("gen", S=2, T=300, N=700, H=4, Hkv=2, d=64, dI=32, k=4, structure="band_sink_needles"),
               W.small("gen32", S=1, T=100, N=260, H=2, Hkv=1, d=64, dI=32, k=4, dtype=synth.F32),
               W.small("gen_sn", S=3, T=1, N=1000, H=4, Hkv=2, d=64, dI=64, k=4, structure="sink_needles"),
               W.small("gen_f8", S=2, T=200, N=900, H=4, Hkv=2, d=64, dI=64, k=4, structure="band_sink_needles",
                       kidx_dtype=synth.FP8)):
        for name, spec in wl.specs().items():
            dev = synth.device_tensor(spec)
            host = synth.host_tensor(spec)
            if spec.dtype == synth.BF16:
                got = dev.cpu().view(torch.int16).numpy().view(np.uint16)
            elif spec.dtype == synth.FP8:
                got = dev.cpu().view(torch.uint8).numpy()
            else:
                got = dev.cpu().numpy()
            assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(host).view(np.uint8)), (wl.name, name)


def test_profiler_samples_add_up_to_the_totals():
    """The per-launch durations of the library timer sum to its totals, one per launch."""
    require_gpu()
    wl = W.small("prof", S=1, T=600, N=600, H=8, Hkv=2, d=64, dI=32, k=4)
    inputs = gen(wl)
    prob = wl.problem()
    pb = msa.alloc_prefill(prob)
    msa.profiler_read(None, reset=True)
    msa.profiler_enable(True)
    for _ in range(3):
        msa.run_prefill(prob, inputs["q"], inputs["k"], inputs["v"], inputs["q_idx"], inputs["k_idx"], pb)
    torch.cuda.synchronize()
    msa.profiler_enable(False)
    for name in ("idx_scores_mfma", "block_topk", "lse_merge", None):
        ms, n = msa.profiler_read(name, reset=False)
        xs = msa.profiler_samples(name)
        assert len(xs) == n and n >= 3 and all(x >= 0.0 for x in xs)
        assert abs(sum(xs) - ms) <= 1e-6 * max(1.0, ms) + 1e-3
    msa.profiler_read(None, reset=True)
    assert msa.profiler_samples(None) == []
