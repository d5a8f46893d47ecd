"""Benchmark of the MSA hot path on one MI355X.

One step = one full MSA prefill pass over the 131,072-token workload (index scores
+ block max-pool and top-k -- by default fused in one kernel that never writes the block
scores, bit-identical to the two separate calls, which are timed beside it; --selection
two-call times them in the step --, inversion, Outer-Gather-Q attention, LSE merge) followed by
one decode step of 16 sequences over 1,048,576-token caches (index scores, top-k,
split-K attention + merge).  Inputs are generated on the device before timing and
stay resident in HBM.

value  = prefill tokens/s = 131,072 / (device time of the prefill part of a step)
decode = us per decode step (all 16 sequences advance one token), and / 16

Per-kernel device times come from the library's own hipEvent timer (events recorded
on the launch stream around every launch) over the timed region: the mean per launch,
and p50 / p95 over the launches (by default 20 timed steps after 3 warm-ups).  The roofline
object prices the dominant kernel's ALGORITHMIC work (causal triangle, selected keys
only, every tensor read or written once) against MI355X peaks (bf16 dense MFMA
2.5 PFLOP/s, HBM 8 TB/s).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_BF16 = 2.5e15   # FLOP/s, dense
PEAK_HBM = 8.0e12         # B/s
METRIC = "MSA prefill tokens/s at 128K & decode µs/token at 1M; % MFMA/HBM peak"


# ------------------------------------------------------------------ work model
def positions(N, T):
    return np.arange(N - T, N, dtype=np.int64)


def prefill_model(S, T, N, H, Hkv, d, dI, k, B=128, esize=2, touched_blocks=None):
    """Algorithmic flops / bytes per stage of one prefill pass (per launch)."""
    G = H // Hkv
    p = positions(N, T)
    bt = p // B
    nb = (N + B - 1) // B
    slots = np.minimum(k, bt + 1)                        # valid selections per (t, g)
    keys = (slots - 1) * B + (p - bt * B) + 1            # attended keys per (t, g)
    n_slots = S * Hkv * int(slots.sum())
    m = {}
    m["idx_scores"] = dict(flops=2.0 * dI * S * Hkv * float((p + 1).sum()),
                           bytes=esize * S * Hkv * (T + N) * dI + 4.0 * S * Hkv * float((bt + 1).sum()))
    # fused selection: the same index products; its per-(row, span) candidate lists of 15
    # (score, id) are written once and read once by the merge
    nspan = (nb + 1023) // 1024
    cand = 8.0 * 15 * S * Hkv * T * nspan
    m["idx_topk"] = dict(flops=m["idx_scores"]["flops"],
                         bytes=esize * S * Hkv * (T + N) * dI + cand + 4.0 * S * Hkv * T * k)
    m["topk_merge"] = dict(flops=0.0, bytes=cand + 4.0 * S * Hkv * T * k)
    rows_reading = bt >= k                               # rows that must rank their past blocks
    m["block_topk"] = dict(flops=0.0, bytes=4.0 * S * Hkv * float((bt * rows_reading).sum()) + 4.0 * S * Hkv * T * k)
    m["invert"] = dict(flops=0.0, bytes=4.0 * S * Hkv * T * k + 4.0 * n_slots + 4.0 * S * Hkv * (nb + 1))
    if touched_blocks is None:
        touched_blocks = S * Hkv * nb
    part = n_slots * G * (d * esize + 4.0)
    m["ogq_attention"] = dict(flops=4.0 * d * G * S * Hkv * float(keys.sum()),
                              bytes=esize * S * T * H * d + touched_blocks * 2.0 * B * d * esize + part + 4.0 * n_slots)
    m["lse_merge"] = dict(flops=0.0, bytes=part + esize * S * T * H * d + 4.0 * S * Hkv * T * k)
    return m


def decode_model(S, N, H, Hkv, d, dI, k, B=128, esize=2):
    G = H // Hkv
    nb = (N + B - 1) // B
    m = {}
    m["idx_scores"] = dict(flops=2.0 * dI * S * Hkv * N, bytes=esize * S * Hkv * (N + 1) * dI + 4.0 * S * Hkv * nb)
    m["block_topk"] = dict(flops=0.0, bytes=4.0 * S * Hkv * (nb - 1) + 4.0 * S * Hkv * k)
    m["attention"] = dict(flops=4.0 * d * G * S * Hkv * k * B,
                          bytes=S * Hkv * k * 2.0 * B * d * esize + 2.0 * esize * S * H * d + 4.0 * S * Hkv * k)
    return m


def attention_reduction_ratio(G, d, dI, N, budget=2048):
    """Dense-attention flops / MSA flops (index branch + main branch) averaged over a
    causal prefill of N tokens: 2*G*d*n / (2*G*d*budget + dI*n) at n = N/2."""
    n = N / 2.0
    return (2.0 * G * d * n) / (2.0 * G * d * budget + dI * n)


def percentiles(samples):
    """p50 / p95 / p99 (ms) of per-launch or per-step times."""
    import numpy as np
    if not samples:
        return {}
    a = np.asarray(samples, dtype=np.float64)
    return dict(p50_ms=float(np.percentile(a, 50)), p95_ms=float(np.percentile(a, 95)),
                p99_ms=float(np.percentile(a, 99)))


def roofline(flops, nbytes, seconds):
    """Bound by whichever of MFMA or HBM the algorithmic work needs longer on."""
    t_mfma = flops / PEAK_MFMA_BF16
    t_hbm = nbytes / PEAK_HBM
    if t_mfma >= t_hbm:
        a = flops / seconds / 1e12
        return dict(bound="mfma", achieved=a, peak=PEAK_MFMA_BF16 / 1e12, unit="TFLOP/s", frac=a / (PEAK_MFMA_BF16 / 1e12))
    a = nbytes / seconds / 1e9
    return dict(bound="hbm", achieved=a, peak=PEAK_HBM / 1e9, unit="GB/s", frac=a / (PEAK_HBM / 1e9))


def query_tile_split(wl, sel, min_rows=32, cap=32, min_blocks=2):
    """Per-(row, slot) flag of the library's query-tile split, recomputed from sel for
    reporting: block b is tile-shared for (s, g, 128-position query tile) when at least
    max(min_rows, ceil(rows / 2)) of the tile's rows chose it and the tile has at least
    min_rows rows; at most `cap` such blocks are kept, the highest ids first, and a tile
    with fewer than `min_blocks` of them keeps none."""
    import torch
    S, Hkv, T, k = sel.shape
    dev = sel.device
    nb = wl.nb
    pos = torch.arange(wl.N - wl.T, wl.N, device=dev, dtype=torch.int64)
    qb = (pos // 128) - (wl.N - wl.T) // 128                                  # tile of each row
    nqb = int(qb.max()) + 1
    rows = torch.bincount(qb, minlength=nqb)                                  # rows per tile
    thr = torch.clamp((rows + 1) // 2, min=min_rows)
    s64 = sel.to(torch.int64)
    valid = s64 >= 0
    sg = torch.arange(S * Hkv, device=dev).view(S, Hkv, 1, 1)
    key = (sg * nqb + qb.view(1, 1, T, 1)) * nb + s64.clamp(min=0)
    cnt = torch.bincount(key[valid], minlength=S * Hkv * nqb * nb).view(S * Hkv, nqb, nb)
    cand = (cnt >= thr.view(1, nqb, 1)) & (rows >= min_rows).view(1, nqb, 1)
    from_top = torch.flip(torch.cumsum(torch.flip(cand.to(torch.int32), [2]), 2), [2])
    keep = cand & (from_top <= cap)
    keep &= (cand.sum(dim=2, keepdim=True) >= min_blocks)
    return valid & keep.view(-1)[key.clamp(min=0)], keep


def attention_split_model(wl, sel, hot, keep, esize=2):
    """Algorithmic work of the two attention kernels and the merge for one selection.
    Each kernel is priced for the (row, block) pairs it handles: scores and PV over the
    attended keys; Q of every row it serves once, K/V of every block it touches once,
    one partial (G x (d bf16 + lse)) per pair (Outer-Gather-Q) or per row (query tile)."""
    import torch
    S, Hkv, T, k = sel.shape
    G, d, B = wl.G, wl.d, 128
    pos = torch.arange(wl.N - wl.T, wl.N, device=sel.device, dtype=torch.int64).view(1, 1, T, 1)
    bt = pos // B
    s64 = sel.to(torch.int64)
    valid = s64 >= 0
    keys = torch.where(s64 == bt, pos - bt * B + 1, torch.full_like(s64, B)) * valid
    cold = valid & ~hot
    part = G * (d * esize + 4.0)
    qrow = G * d * esize
    kv = 2.0 * B * d * esize
    rows_hot = int(hot.any(dim=3).sum())
    rows_cold = int(cold.any(dim=3).sum())
    n_cold = int(cold.sum())
    sgb_cold = torch.zeros(S * Hkv * wl.nb, dtype=torch.bool, device=sel.device)
    sgi = torch.arange(S * Hkv, device=sel.device).view(S, Hkv, 1, 1) * wl.nb
    sgb_cold[(sgi + s64.clamp(min=0))[cold]] = True
    m = {}
    m["hot_mfma"] = dict(flops=4.0 * d * G * float((keys * hot).sum()),
                         bytes=rows_hot * (qrow + part) + int(keep.any(dim=1).sum()) * kv)
    m["ogq_mfma"] = dict(flops=4.0 * d * G * float((keys * cold).sum()),
                         bytes=rows_cold * qrow + int(sgb_cold.sum()) * kv + n_cold * (part + 4.0))
    m["lse_merge"] = dict(flops=0.0, bytes=(n_cold + rows_hot) * part + esize * S * T * wl.H * d
                          + S * Hkv * T * (4.0 * k + 8.0))
    m["pairs"] = dict(query_tile=int(hot.sum()), outer_gather_q=n_cold, rows_with_query_tile=rows_hot)
    return m


# kernel name (library profiler) -> model stage (the attention kernels and the merge
# are priced by attention_split_model from the run's own selection)
PREFILL_KERNELS = {"idx_scores_mfma": "idx_scores", "block_topk": "block_topk", "idx_topk_mfma": "idx_topk",
                   "topk_merge": "topk_merge", "ogq_mfma": "ogq_mfma", "hot_mfma": "hot_mfma",
                   "lse_merge": "lse_merge"}
KERNEL_SOURCES = {"ogq_mfma": "attention_mfma.hip", "hot_mfma": "attention_mfma.hip",
                  "idx_scores_mfma": "index_scores_mfma.hip", "lse_merge": "attention.hip", "block_topk": "topk.hip",
                  "idx_topk_mfma": "fused_topk.hip", "topk_merge": "fused_topk.hip"}


def source_sha(kernel):
    f = KERNEL_SOURCES.get(kernel)
    if f is None:
        return None
    with open(os.path.join(ROOT, "block_sparse_long_06_amd", "csrc", f), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if
    the summary is missing or was taken on a different version of the kernel."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_c2_prefill_128k.json" % kernel)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ CPU baseline
def achievable_peaks():
    """What this machine reaches with vendor-library kernels, for context beside the vendor
    peaks (the rooflines stay against the vendor peaks): a square bf16 GEMM (hipBLASLt via
    torch.matmul of contiguous operands), a device-to-device copy (bytes read + written)
    and a plain sum (bytes read), each the best of 5 timed repetitions."""
    import torch
    out = {}
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev0.record()
            fn()
            ev1.record()
            torch.cuda.synchronize()
            ts.append(ev0.elapsed_time(ev1) / 1e3)
        return min(ts)

    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    t = best(lambda: torch.matmul(a, b, out=c))
    out["bf16_gemm_8192_tflops"] = 2.0 * n ** 3 / t / 1e12
    del a, b, c
    x = torch.ones((1 << 31,), dtype=torch.bfloat16, device="cuda")   # 4 GiB
    y = torch.empty_like(x)
    t = best(lambda: y.copy_(x))
    out["hbm_copy_GBps"] = 2.0 * x.numel() * 2 / t / 1e9
    t = best(lambda: x.sum())
    out["hbm_read_sum_GBps"] = x.numel() * 2 / t / 1e9
    del x, y
    torch.cuda.empty_cache()
    out["vendor_peaks"] = dict(bf16_dense_tflops=PEAK_MFMA_BF16 / 1e12, hbm_GBps=PEAK_HBM / 1e9)
    return out


def cpu_baseline(wl, inputs, seconds_budget=12.0):
    """The oracle, as is, on a bounded sample of query rows of the same workload:
    index scores, top-k, inversion and attention for R rows x all groups, each stage
    timed on its own.  Returns tokens/s (= rows / oracle seconds), the thread count it
    used, and per stage the seconds spent, the time per row and the time the whole
    workload (T rows) would take at that rate."""
    import torch
    import oracle
    pos_all = positions(wl.N, wl.T)
    G = wl.G
    # host copies of one workload's inputs, decoded to float64 (not timed)
    kI = [oracle.decode(inputs["k_idx"][0, g]) for g in range(wl.Hkv)]
    K = [oracle.decode(inputs["k"][0, g]) for g in range(wl.Hkv)]
    V = [oracle.decode(inputs["v"][0, g]) for g in range(wl.Hkv)]
    rows_all = wl.sampled_rows(8192)
    done_rows = 0
    spent = dict(index_scores=0.0, block_topk=0.0, invert=0.0, attention=0.0)
    batch = 16
    i = 0
    while sum(spent.values()) < seconds_budget and i < len(rows_all):
        rows = rows_all[i:i + batch]
        i += batch
        idx = torch.from_numpy(rows).cuda()
        qI = [oracle.decode(inputs["q_idx"][0, g][idx]) for g in range(wl.Hkv)]
        q = oracle.decode(inputs["q"][0][idx])
        for g in range(wl.Hkv):
            t0 = time.perf_counter()
            sc = oracle.slice_index_scores(qI[g], pos_all[rows], kI[g], 128)
            t1 = time.perf_counter()
            sel = oracle.slice_block_topk(sc, pos_all[rows] // 128, wl.k)
            t2 = time.perf_counter()
            oracle.slice_invert(sel, wl.nb)
            t3 = time.perf_counter()
            oracle.slice_attention(q[:, g * G:(g + 1) * G], pos_all[rows], sel, K[g], V[g], 128, wl.scale)
            t4 = time.perf_counter()
            spent["index_scores"] += t1 - t0
            spent["block_topk"] += t2 - t1
            spent["invert"] += t3 - t2
            spent["attention"] += t4 - t3
        done_rows += len(rows)
    total = sum(spent.values())
    stages = {n: dict(s=v, ms_per_row=1e3 * v / done_rows, full_workload_s_extrapolated=v / done_rows * wl.T)
              for n, v in spent.items()}
    return dict(value=done_rows / total, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample="%d seeded query rows x %d groups of the %s workload (full index scan, top-k, "
                       "inversion, attention per row), %.1f s of CPU work" % (done_rows, wl.Hkv, wl.name, total),
                stages=stages)


def cpu_decode_baseline(wd, inputs, pairs=3):
    """The oracle, as is, on `pairs` seeded (sequence, group) rows of the decode step:
    index scores over the whole cache, top-k and attention over the selected blocks.  One
    decode row is one oracle row (its loops run over rows), so this runs on one thread.
    Reported per stage, and as the decode step's time at that rate (16 x 8 rows)."""
    import oracle
    rng = np.random.default_rng(wd.seed + 7)
    picks = sorted(set((int(rng.integers(wd.S)), int(rng.integers(wd.Hkv))) for _ in range(4 * pairs)))[:pairs]
    pos = positions(wd.N, wd.T)
    G = wd.G
    spent = dict(index_scores=0.0, block_topk=0.0, attention=0.0)
    for s_, g in picks:
        kI = oracle.decode(inputs["k_idx"][s_, g])
        K, V = oracle.decode(inputs["k"][s_, g]), oracle.decode(inputs["v"][s_, g])
        qI = oracle.decode(inputs["q_idx"][s_, g])
        q = oracle.decode(inputs["q"][s_])[:, g * G:(g + 1) * G]
        t0 = time.perf_counter()
        sc = oracle.slice_index_scores(qI, pos, kI, 128)
        t1 = time.perf_counter()
        sel = oracle.slice_block_topk(sc, pos // 128, wd.k)
        t2 = time.perf_counter()
        oracle.slice_attention(q, pos, sel, K, V, 128, wd.scale)
        t3 = time.perf_counter()
        spent["index_scores"] += t1 - t0
        spent["block_topk"] += t2 - t1
        spent["attention"] += t3 - t2
        del kI, K, V
    n = len(picks)
    rows_per_step = wd.S * wd.Hkv * wd.T
    per_row = sum(spent.values()) / n
    return dict(value=per_row * rows_per_step * 1e6, unit="us per decode step (extrapolated)", cores=1,
                kind="oracle",
                sample="%d seeded (sequence, group) rows of the %s workload (index scan of %d keys, top-k, "
                       "attention), %.1f s of CPU work; the step has %d such rows"
                       % (n, wd.name, wd.N, sum(spent.values()), rows_per_step),
                stages={k: dict(s=v, ms_per_row=1e3 * v / n) for k, v in spent.items()})


def selection_structure(wl, sel, csr_offsets):
    """Realised structure of one prefill selection (reported, never timed).

    Classes of each valid (query, group, slot), first match wins: own block; sink
    (block 0); needle (a boosted block of the generator other than 0); band (1-4
    blocks before the own one); other.  `tile_shared` is the fraction of valid slots
    whose block is also chosen by at least half of the queries in the same 128-position
    query block and group; `csr_rows` summarises the per-(group, block) row counts."""
    import torch
    S, Hkv, T, k = sel.shape
    dev = sel.device
    pos = torch.arange(wl.N - wl.T, wl.N, device=dev, dtype=torch.int64)
    bt = (pos // 128).view(1, 1, T, 1)
    s64 = sel.to(torch.int64)
    valid = s64 >= 0
    n_valid = int(valid.sum())
    own = valid & (s64 == bt)
    sink = valid & ~own & (s64 == 0)
    bm = wl.boost_mask()
    if bm is not None:
        boost = torch.from_numpy(bm.astype(np.bool_)).to(dev)                       # [S, Hkv, nb]
        sidx = torch.arange(S, device=dev).view(S, 1, 1, 1).expand_as(s64)
        gidx = torch.arange(Hkv, device=dev).view(1, Hkv, 1, 1).expand_as(s64)
        needle = valid & ~own & ~sink & boost[sidx, gidx, s64.clamp(min=0)]
    else:
        needle = torch.zeros_like(valid)
    band = valid & ~own & ~sink & ~needle & (s64 >= bt - 4)
    other = valid & ~own & ~sink & ~needle & ~band
    frac = {n: float(m.sum()) / max(n_valid, 1)
            for n, m in (("own", own), ("sink", sink), ("needle", needle), ("band", band), ("other", other))}
    # blocks shared inside a 128-position query block
    qb = bt - int((wl.N - wl.T) // 128)
    nqb = int(qb.max()) + 1
    nb = wl.nb
    sg = (torch.arange(S, device=dev).view(S, 1, 1, 1) * Hkv + torch.arange(Hkv, device=dev).view(1, Hkv, 1, 1))
    key = ((sg * nqb + qb) * nb + s64.clamp(min=0))
    cnt = torch.bincount(key[valid], minlength=S * Hkv * nqb * nb)
    rows_in_qb = torch.bincount(qb.view(-1), minlength=nqb).view(1, 1, nqb)           # queries per query block
    at = cnt[key.clamp(min=0)]
    tile_rows = rows_in_qb.view(-1)[qb.expand_as(s64)]
    shared = valid & (2 * at >= tile_rows)
    frac["tile_shared"] = float(shared.sum()) / max(n_valid, 1)
    counts = (csr_offsets[..., 1:] - csr_offsets[..., :-1]).reshape(-1).to(torch.float64)
    nz = counts[counts > 0]
    csr = dict(blocks_touched=int(nz.numel()), max=int(nz.max()) if nz.numel() else 0,
               p50=float(torch.quantile(nz, 0.5)) if nz.numel() else 0.0,
               p99=float(torch.quantile(nz, 0.99)) if nz.numel() else 0.0)
    return dict(fractions=frac, valid_slots=n_valid, csr_rows=csr)


# ------------------------------------------------------------------ main
def paged_decode(args, msa, wd, xd):
    """The decode workload over a ragged batch in a paged cache, outside the timed step:
    sequence lengths drawn (seeded) from [N/2, N], every 128-position block in its own
    page of a shuffled pool [pages, Hkv, 128, .] holding the same values as the dense
    cache.  Reports the step time and the index stream's rate over the bytes it must read
    (sum of lengths x Hkv x dI x 2)."""
    import numpy as np
    import torch
    S, N, Hkv, B = wd.S, wd.N, wd.Hkv, 128
    nb = N // B
    rng = np.random.default_rng(wd.seed + 8)
    lens = rng.integers(N // 2, N + 1, size=S)
    need = (lens + B - 1) // B
    num_pages = int(need.sum())
    perm = rng.permutation(num_pages)
    table = np.full((S, nb), -1, dtype=np.int32)
    flat, pages, i = [], [], 0
    for s in range(S):
        table[s, :need[s]] = perm[i:i + need[s]]
        flat.extend(range(s * nb, s * nb + int(need[s])))
        pages.extend(perm[i:i + need[s]].tolist())
        i += int(need[s])
    flat = torch.tensor(flat, dtype=torch.int64, device="cuda")
    pages = torch.tensor(pages, dtype=torch.int64, device="cuda")

    def to_pool(dense):
        w = dense.shape[-1]
        src = dense.view(S, Hkv, nb, B, w).permute(0, 2, 1, 3, 4).reshape(S * nb, Hkv, B, w)
        pool = torch.empty((num_pages, Hkv, B, w), dtype=dense.dtype, device="cuda")
        pool[pages] = src[flat]
        return pool

    pools = {n: to_pool(xd[n]) for n in ("k", "v", "k_idx")}
    kv_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    lay = msa.kv_layout(kv_lens, torch.from_numpy(table).cuda(), num_pages)
    prob = wd.problem()
    bufs = msa.alloc_decode(prob)

    def step():
        msa.run_decode_kv(prob, lay, xd["q"], pools["k"], pools["v"], xd["q_idx"], pools["k_idx"], bufs)
    step()
    torch.cuda.synchronize()
    ms, ms_timer = timed_then_profiled(msa, step, args.steps)
    st = {}
    for kn in ("idx_scores_stream", "block_topk_t1", "decode_attn", "decode_merge"):
        tms, nl = msa.profiler_read(kn, reset=False)
        if nl:
            st[kn] = dict(ms=tms / nl)
    msa.profiler_read(None, reset=True)
    if "idx_scores_stream" in st:
        kbytes = float(lens.sum()) * Hkv * wd.dI * 2.0 + 4.0 * float(need.sum()) * Hkv
        sec = st["idx_scores_stream"]["ms"] / 1e3
        st["idx_scores_stream"].update(roofline(2.0 * wd.dI * float(lens.sum()) * Hkv, kbytes, sec))
    del pools
    return dict(workload="%s, ragged lengths in [N/2, N] (mean %d), paged (%d shuffled 128-position pages)"
                % (wd.description, int(lens.mean()), num_pages),
                us_per_step=ms * 1e3, us_per_token_amortised=ms * 1e3 / S, stages=st)


def other_selection(args, msa, wp, xp, pb, fused):
    """The selection path the timed step does not use, on the prefill workload and outside
    the timed step: the fused index scores + top-k (fused=True; no [S, Hkv, T, nb] score
    matrix) or the two calls msa_index_scores + msa_block_topk.  Time per pass, per kernel,
    the workspace of the fused call against the score matrix, and whether its selection
    equals the timed step's."""
    import torch
    prob = wp.problem()
    sel = torch.empty_like(pb.sel)
    ws = torch.empty((max(msa.workspace_bytes(prob, msa.MSA_CALL_INDEX_TOPK), 1),), dtype=torch.uint8, device="cuda")
    scores = None if fused else torch.empty((wp.S, wp.Hkv, wp.T, wp.nb), dtype=torch.float32, device="cuda")

    def call():
        if fused:
            msa.index_topk(prob, xp["q_idx"], xp["k_idx"], sel, ws, ws.numel())
        else:
            msa.index_scores(prob, xp["q_idx"], xp["k_idx"], scores)
            msa.block_topk(prob, scores, sel)
    call()
    torch.cuda.synchronize()
    ms, ms_timer = timed_then_profiled(msa, call, args.steps)
    m = prefill_model(wp.S, wp.T, wp.N, wp.H, wp.Hkv, wp.d, wp.dI, wp.k)
    st = {}
    for kn in (("idx_topk_mfma", "topk_merge") if fused else ("idx_scores_mfma", "block_topk")):
        tms, nl = msa.profiler_read(kn, reset=False)
        if nl:
            stage = m[PREFILL_KERNELS[kn]]
            st[kn] = dict(ms=tms / nl, **roofline(stage["flops"], stage["bytes"], tms / nl / 1e3))
    msa.profiler_read(None, reset=True)
    same = bool(torch.equal(sel, pb.sel))
    return dict(workload=wp.description + (", index scores + top-k fused" if fused else
                                           ", index scores and top-k as two calls"),
                fused=fused, ms_per_pass=ms, stages=st, fused_workspace_bytes=int(ws.numel()),
                score_matrix_bytes=int(wp.S * wp.Hkv * wp.T * wp.nb * 4),
                selection_equal_to_the_timed_step=same)


def token_decode(args, msa, wd, xd, block_sel):
    """The decode workload with token-level selection at the block path's budget (16 x 128 =
    2048 tokens, the pages' granularity comparison), outside the timed step: step time per
    stage and the share of the token-level picks that fall inside the blocks the block-level
    step chose."""
    import torch
    budget = wd.k * 128
    prob = wd.problem()
    tb = msa.alloc_token_decode(prob, budget)

    def step():
        msa.run_token_decode(prob, xd["q"], xd["k"], xd["v"], xd["q_idx"], xd["k_idx"], tb, budget)
    step()
    torch.cuda.synchronize()
    ms, ms_timer = timed_then_profiled(msa, step, args.steps)
    st = {}
    for kn in ("token_scores", "token_topk", "token_attn", "token_merge"):
        tms, nl = msa.profiler_read(kn, reset=False)
        if nl:
            st[kn] = dict(ms=tms / nl)
    msa.profiler_read(None, reset=True)
    if "token_scores" in st:
        kbytes = wd.S * wd.Hkv * wd.N * wd.dI * 2.0 + 4.0 * wd.S * wd.Hkv * wd.N
        sec = st["token_scores"]["ms"] / 1e3
        st["token_scores"].update(roofline(2.0 * wd.dI * wd.S * wd.Hkv * wd.N, kbytes, sec))
    if "token_topk" in st:
        # algorithmic: every eligible score read once, the chosen positions written once
        sec = st["token_topk"]["ms"] / 1e3
        rows = wd.S * wd.Hkv * wd.T
        st["token_topk"].update(roofline(0.0, 4.0 * rows * wd.N + 4.0 * rows * budget, sec))
    tok = tb.sel_tok                                            # [S, Hkv, 1, budget]
    blk = block_sel                                             # [S, Hkv, 1, k]
    inside = ((tok.unsqueeze(-1) // 128) == blk.unsqueeze(-2)).any(-1) & (tok >= 0)
    share = inside.sum().item() / max(1, (tok >= 0).sum().item())
    del tb
    return dict(workload="%s, token-level selection of %d tokens" % (wd.description, budget),
                us_per_step=ms * 1e3, us_per_token_amortised=ms * 1e3 / wd.S, stages=st,
                share_of_token_picks_inside_the_block_selection=share)


def train_step(args, msa, wl):
    """One training step of wl, outside the timed prefill step: index scores, top-k,
    inversion, the forward with lse and teacher mass (every pair in Outer-Gather-Q order),
    the main-branch backward for a seeded upstream gradient, the index KL and the
    index-branch backward.  Stage times come from the library timer.  The attention
    backward is priced at 10 d flops per (row, head, attended key): five products (S, dP,
    dV, dK, dQ) of 2 d each, against the bf16 matrix-core peak."""
    import torch
    import synth
    specs = wl.specs()
    x = {n: synth.device_tensor(specs[n]) for n in specs}
    dout = synth.device_tensor(wl.dout_spec())
    prob = wl.problem()
    tb = msa.alloc_train(prob)

    def step():
        msa.run_train_step(prob, x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], dout, tb)
    step()
    torch.cuda.synchronize()
    ms, ms_timer = timed_then_profiled(msa, step, args.steps)
    st = {}
    for kn in ("idx_scores_mfma", "block_topk", "ogq_mfma", "lse_merge", "bwd_zero", "bwd_drow", "attn_bwd", "dq_merge",
               "index_kl", "index_bwd_zero", "index_bwd", "index_dq_gather"):
        tms, nl = msa.profiler_read(kn, reset=False)
        if nl:
            st[kn] = dict(ms=tms / nl)
    msa.profiler_read(None, reset=True)
    m = prefill_model(wl.S, wl.T, wl.N, wl.H, wl.Hkv, wl.d, wl.dI, wl.k)
    fwd_flops = m["ogq_attention"]["flops"]
    if "attn_bwd" in st:
        st["attn_bwd"].update(roofline(2.5 * fwd_flops, 0.0, st["attn_bwd"]["ms"] / 1e3), flops=2.5 * fwd_flops)
    if "ogq_mfma" in st:
        st["ogq_mfma"].update(roofline(fwd_flops, m["ogq_attention"]["bytes"], st["ogq_mfma"]["ms"] / 1e3))
    del tb, x
    return dict(workload=wl.description + ", training step (forward + backward + index KL)",
                ms_per_step=ms, ms_per_step_with_kernel_timer=ms_timer, tokens_per_s=wl.T / (ms / 1e3), stages=st)


PREFILL_TIMER_NAMES = ("idx_scores_mfma", "idx_scores_rows", "block_topk", "invert_count", "invert_scatter",
                       "invert_offsets", "scan_tile_sums", "scan_top", "scan_apply", "wl_count", "wl_emit", "ogq_mfma",
                       "ogq_simple", "lse_merge", "hot_select", "hot_compact", "cold_count", "cold_scatter",
                       "cold_offsets", "hot_mfma", "idx_topk_mfma", "topk_merge")


def timed_then_profiled(msa, step, steps):
    """Mean time of `steps` calls of step() without the library's per-kernel timer (its
    event records add a few microseconds per launch), then of as many with the timer on;
    the timer's records of the second run are left for the caller to read."""
    import torch

    def run():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    ms = run()
    msa.profiler_read(None, reset=True)
    msa.profiler_enable(True)
    ms_timer = run()
    msa.profiler_enable(False)
    return ms, ms_timer


def read_timer(msa, names):
    """Per-kernel totals, launch counts and per-launch samples of the library timer."""
    kern = {}
    for name in names:
        ms, n = msa.profiler_read(name, reset=False)
        if n:
            kern[name] = dict(total_ms=ms, launches=n, samples=msa.profiler_samples(name))
    return kern


def prefill_stage_report(wp, pb, kern, steps):
    """Per-stage device times and rooflines of the prefill passes recorded in `kern`
    (steps passes of wp whose last selection is in pb), priced by the algorithmic model."""
    import torch
    # algorithmic work of the prefill pass, with the blocks actually touched
    counts = pb.csr_offsets[..., 1:] - pb.csr_offsets[..., :-1]
    touched = int((counts > 0).sum())
    model = prefill_model(wp.S, wp.T, wp.N, wp.H, wp.Hkv, wp.d, wp.dI, wp.k, touched_blocks=touched)
    if os.environ.get("MSA_HOT_TILES", "1").startswith("0"):
        hot_flag = torch.zeros_like(pb.sel, dtype=torch.bool)
        keep = torch.zeros((1, 1, 1), dtype=torch.bool, device=pb.sel.device)
    else:
        hot_flag, keep = query_tile_split(wp, pb.sel)
    split = attention_split_model(wp, pb.sel, hot_flag, keep)
    model.update({kk: split[kk] for kk in ("hot_mfma", "ogq_mfma", "lse_merge")})
    stages = {}
    for kname, stage in PREFILL_KERNELS.items():
        if kname not in kern:
            continue
        per_launch_s = kern[kname]["total_ms"] / kern[kname]["launches"] / 1e3
        rf = roofline(model[stage]["flops"], model[stage]["bytes"], per_launch_s)
        stages[kname] = dict(ms=per_launch_s * 1e3, **percentiles(kern[kname]["samples"]),
                             flops=model[stage]["flops"], bytes=model[stage]["bytes"], **rf)
    inv_ms = sum(kern[n]["total_ms"] for n in ("invert_count", "invert_scatter", "invert_offsets") if n in kern)
    stages["invert(all launches)"] = dict(ms=inv_ms / steps, **roofline(0.0, model["invert"]["bytes"], inv_ms / steps / 1e3))
    split_ms = sum(kern[n]["total_ms"] for n in ("hot_select", "hot_compact", "cold_count", "cold_scatter", "cold_offsets")
                   if n in kern)
    stages["query_tile_split(all launches)"] = dict(ms=split_ms / steps)
    # a4 as a whole (both attention kernels) against the full a4 work
    a4_ms = sum(kern[n]["total_ms"] for n in ("ogq_mfma", "hot_mfma") if n in kern) / steps
    if a4_ms > 0:
        stages["a4_attention(ogq_mfma+hot_mfma)"] = dict(
            ms=a4_ms, flops=model["ogq_attention"]["flops"], bytes=model["ogq_attention"]["bytes"],
            **roofline(model["ogq_attention"]["flops"], model["ogq_attention"]["bytes"], a4_ms / 1e3))
    return stages, split


def other_prefill(args, msa, wl, fused):
    """One more prefill workload, timed on its own after the headline steps: tokens/s and
    the per-stage rooflines, with the same timer and model as the headline workload.  With
    fused, the pass selects blocks with the fused index scores + top-k (no block-score
    matrix) in place of the two separate calls."""
    import torch
    import synth
    specs = wl.specs()
    x = {n: synth.device_tensor(specs[n]) for n in specs}
    prob = wl.problem()
    pb = msa.alloc_prefill(prob, fused_selection=fused)

    def run():
        msa.run_prefill(prob, x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], pb)
    for _ in range(max(args.warmup, 1)):
        run()
    torch.cuda.synchronize()
    def timed():
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            ev[i][0].record()
            run()
            ev[i][1].record()
        torch.cuda.synchronize()
        return [e[0].elapsed_time(e[1]) for e in ev]
    # as for the headline workload: step times without the library's per-kernel timer,
    # then the same steps with it for the stage times
    steps_ms = timed()
    msa.profiler_read(None, reset=True)
    msa.profiler_enable(True)
    timer_ms = timed()
    msa.profiler_enable(False)
    kern = read_timer(msa, PREFILL_TIMER_NAMES)
    msa.profiler_read(None, reset=True)
    ms = sum(steps_ms) / len(steps_ms)
    stages, split = prefill_stage_report(wl, pb, kern, args.steps)
    del x, pb
    torch.cuda.empty_cache()
    desc = wl.description + (", fused index scores + top-k" if fused else ", index scores and top-k as two calls")
    return dict(workload=desc, tokens=wl.T, tokens_per_s=wl.T / (ms / 1e3), prefill_ms=ms,
                prefill_ms_with_kernel_timer=sum(timer_ms) / len(timer_ms),
                **{"prefill_" + k: v for k, v in percentiles(steps_ms).items()}, stages=stages,
                attention_pairs=split["pairs"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--prefill", default="C2", choices=["C1", "C2", "C4"],
                    help="prefill workload timed (default C2: the 131072-token headline configuration)")
    ap.add_argument("--no-fp8-decode", action="store_true",
                    help="skip the extra decode timing with the index keys stored as FP8 E4M3 (serving variant)")
    ap.add_argument("--no-paged-decode", action="store_true",
                    help="skip the extra decode timing over ragged lengths and a paged cache (serving variant)")
    ap.add_argument("--train", default="C1", choices=["C1", "C2", "none"],
                    help="workload of the extra training-step timing (default C1, 32768 tokens)")
    ap.add_argument("--other-prefill", default="C1,C4",
                    help="further prefill workloads timed after the headline steps with the same --selection "
                         "(comma list of C1, C2, C4, each optionally suffixed '+fused' or '+two-call' to override "
                         "the selection path, or 'none')")
    ap.add_argument("--selection", default="fused", choices=["fused", "two-call"],
                    help="block selection of the timed prefill pass: the fused index scores + top-k kernel "
                         "(default; no block-score matrix) or msa_index_scores + msa_block_topk; the other one is "
                         "timed beside it, outside the step (falls back to two-call where the fused call does not "
                         "apply: top-k > 16)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy 3 times (the known-size reference "
                         "for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MSA path shards by KV-head group and sequence with no "
              "exchange inside MSA; this library runs on one MI355X (--gpus %d is not supported)." % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_long_06_amd as msa
    import synth
    from synth import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    print("[bench] device: %s" % torch.cuda.get_device_name(0), file=sys.stderr, flush=True)
    if args.copy_probe:
        src = torch.ones((1 << 29,), dtype=torch.bfloat16, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] copy probe: 3 x 1 GiB device copies", file=sys.stderr, flush=True)
    wp, wd = {"C1": W.C1, "C2": W.C2, "C4": W.C4}[args.prefill], W.C3
    specs = wp.specs()
    xp = {n: synth.device_tensor(specs[n]) for n in specs}
    pprob = wp.problem()
    use_fused = args.selection == "fused" and wp.k <= 16
    pb = msa.alloc_prefill(pprob, fused_selection=use_fused)
    xd = db = dprob = None
    kidx8 = db8 = dprob8 = None
    if not args.no_decode:
        ds = wd.specs()
        xd = {n: synth.device_tensor(ds[n]) for n in ds}
        dprob = wd.problem()
        db = msa.alloc_decode(dprob)
        if not args.no_fp8_decode:
            kidx8 = synth.device_tensor(W.C3_FP8.specs()["k_idx"])   # the same values, stored as E4M3
            dprob8 = W.C3_FP8.problem()
            db8 = msa.alloc_decode(dprob8)
    torch.cuda.synchronize()
    print("[bench] inputs resident: prefill %s, decode %s" % (wp.name, wd.name), file=sys.stderr, flush=True)

    def prefill():
        msa.run_prefill(pprob, xp["q"], xp["k"], xp["v"], xp["q_idx"], xp["k_idx"], pb)

    def decode():
        msa.run_decode(dprob, xd["q"], xd["k"], xd["v"], xd["q_idx"], xd["k_idx"], db)

    for _ in range(args.warmup):
        prefill()
        if db is not None:
            decode()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    def timed_steps():
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record()
            prefill()
            ev[i][1].record()
            if db is not None:
                decode()
            ev[i][2].record()
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        pre = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
        dec = [ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)] if db else None
        return pre, dec, wall_s

    # The headline steps run without the library's per-kernel timer (its two event records
    # per launch add ~0.1-0.2 ms to a prefill step and ~35 us to a decode step); the same
    # number of steps then runs again with the timer on for the per-kernel times, the
    # stage rooflines and the dominant kernel's roofline.
    prefill_steps, decode_steps, wall = timed_steps()
    msa.profiler_read(None, reset=True)
    msa.profiler_enable(True)
    prefill_steps_timer, decode_steps_timer, _ = timed_steps()
    msa.profiler_enable(False)
    kern = read_timer(msa, PREFILL_TIMER_NAMES + ("idx_scores_stream", "block_topk_t1", "decode_attn",
                                                  "decode_simple", "decode_merge"))
    msa.profiler_read(None, reset=True)
    prefill_ms = sum(prefill_steps) / args.steps
    decode_ms = (sum(decode_steps) / args.steps) if db else None
    print("[bench] timed %d steps: prefill %.3f ms, decode %s ms" % (args.steps, prefill_ms,
          "%.3f" % decode_ms if decode_ms else "-"), file=sys.stderr, flush=True)

    stages, split = prefill_stage_report(wp, pb, kern, args.steps)
    dominant = max((k for k in stages if k in PREFILL_KERNELS), key=lambda k: stages[k]["ms"])
    dom = stages[dominant]
    traffic = measured_traffic(dominant) if wp is W.C2 else None
    roof = dict(kernel=dominant, bound=dom["bound"], achieved=dom["achieved"], peak=dom["peak"], unit=dom["unit"],
                frac=dom["frac"], traffic=traffic,
                algorithmic_bytes=dom["bytes"], algorithmic_flops=dom["flops"], ms_per_launch=dom["ms"])

    dec = None
    if db is not None:
        dm = decode_model(wd.S, wd.N, wd.H, wd.Hkv, wd.d, wd.dI, wd.k)
        dstages = {}
        for kn in ("idx_scores_stream", "idx_scores_rows"):
            if kn in kern:
                s_ = kern[kn]["total_ms"] / kern[kn]["launches"] / 1e3
                dstages[kn] = dict(ms=s_ * 1e3, **percentiles(kern[kn]["samples"]),
                                   **roofline(dm["idx_scores"]["flops"], dm["idx_scores"]["bytes"], s_))
        if "block_topk_t1" in kern:
            s_ = kern["block_topk_t1"]["total_ms"] / kern["block_topk_t1"]["launches"] / 1e3
            dstages["block_topk_t1"] = dict(ms=s_ * 1e3, **roofline(0.0, dm["block_topk"]["bytes"], s_))
        for kn in ("decode_attn", "decode_simple"):
            if kn in kern:
                s_ = kern[kn]["total_ms"] / kern[kn]["launches"] / 1e3
                dstages[kn] = dict(ms=s_ * 1e3, **roofline(dm["attention"]["flops"], dm["attention"]["bytes"], s_))
        if "decode_merge" in kern:
            dstages["decode_merge"] = dict(ms=kern["decode_merge"]["total_ms"] / kern["decode_merge"]["launches"])
        dec = dict(workload=wd.description, us_per_step=decode_ms * 1e3, us_per_token_amortised=decode_ms * 1e3 / wd.S,
                   us_per_step_p50=1e3 * percentiles(decode_steps)["p50_ms"],
                   us_per_step_p95=1e3 * percentiles(decode_steps)["p95_ms"],
                   us_per_step_p99=1e3 * percentiles(decode_steps)["p99_ms"],
                   us_per_step_with_kernel_timer=1e3 * sum(decode_steps_timer) / args.steps,
                   sequences=wd.S, kv_len=wd.N, stages=dstages)

    dec8 = None
    if db8 is not None:
        # serving variant, outside the timed step: the same decode with 1-byte index keys
        def decode8():
            msa.run_decode(dprob8, xd["q"], xd["k"], xd["v"], xd["q_idx"], kidx8, db8)
        decode8()
        torch.cuda.synchronize()
        ms8, _ = timed_then_profiled(msa, decode8, args.steps)
        k8 = {}
        for kn in ("idx_scores_stream", "block_topk_t1", "decode_attn", "decode_merge"):
            tms, nl = msa.profiler_read(kn, reset=False)
            if nl:
                k8[kn] = dict(ms=tms / nl)
        msa.profiler_read(None, reset=True)
        kbytes8 = wd.S * wd.Hkv * wd.N * wd.dI * 1.0 + 4.0 * wd.S * wd.Hkv * wd.nb
        if "idx_scores_stream" in k8:
            s8 = k8["idx_scores_stream"]["ms"] / 1e3
            k8["idx_scores_stream"].update(roofline(2.0 * wd.dI * wd.S * wd.Hkv * wd.N, kbytes8, s8))
        # share of the bf16-key selections (valid slots) that the E4M3-key run also chose
        a, b = db.sel, db8.sel
        hit = ((a.unsqueeze(-1) == b.unsqueeze(-2)).any(-1) & (a >= 0)).sum().item()
        overlap = hit / max(1, (a >= 0).sum().item())
        dec8 = dict(workload=W.C3_FP8.description, us_per_step=ms8 * 1e3, us_per_token_amortised=ms8 * 1e3 / wd.S,
                    stages=k8, selection_overlap_with_bf16_keys=overlap)
        print("[bench] decode with E4M3 index keys: %.3f ms per step" % ms8, file=sys.stderr, flush=True)

    osel = other_selection(args, msa, wp, xp, pb, fused=not use_fused) if wp.k <= 16 else None
    if osel is not None:
        print("[bench] selection %s, outside the step: %.3f ms (equal selection: %s)"
              % ("fused" if osel["fused"] else "as two calls", osel["ms_per_pass"],
                 osel["selection_equal_to_the_timed_step"]), file=sys.stderr, flush=True)

    dect = None
    if db is not None:
        dect = token_decode(args, msa, wd, xd, db.sel)
        print("[bench] decode with token-level selection: %.3f ms per step" % (dect["us_per_step"] / 1e3),
              file=sys.stderr, flush=True)

    decp = None
    if db is not None and not args.no_paged_decode:
        decp = paged_decode(args, msa, wd, xd)
        print("[bench] decode over ragged lengths and a paged cache: %.3f ms per step" % (decp["us_per_step"] / 1e3),
              file=sys.stderr, flush=True)

    trn = None
    if args.train != "none":
        trn = train_step(args, msa, {"C1": W.C1, "C2": W.C2}[args.train])
        print("[bench] training step (%s): %.3f ms" % (args.train, trn["ms_per_step"]), file=sys.stderr, flush=True)

    others = {}
    if args.other_prefill != "none":
        for name in [x for x in args.other_prefill.split(",") if x and x != args.prefill]:
            base, _, how = name.partition("+")
            wl = {"C1": W.C1, "C2": W.C2, "C4": W.C4}[base]
            fused = (how == "fused" or (how == "" and args.selection == "fused")) and wl.k <= 16
            others[name] = other_prefill(args, msa, wl, fused)
            print("[bench] prefill %s: %.3f ms (%.0f tokens/s)" % (name, others[name]["prefill_ms"],
                  others[name]["tokens_per_s"]), file=sys.stderr, flush=True)

    peaks = achievable_peaks()
    print("[bench] achievable: bf16 GEMM %.0f TFLOP/s, copy %.0f GB/s, read %.0f GB/s" % (
        peaks["bf16_gemm_8192_tflops"], peaks["hbm_copy_GBps"], peaks["hbm_read_sum_GBps"]), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] oracle CPU baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wp, xp)
        if xd is not None:
            print("[bench] oracle CPU baseline of the decode step ...", file=sys.stderr, flush=True)
            cpu["decode"] = cpu_decode_baseline(wd, xd)

    value = wp.T / (prefill_ms / 1e3)
    ms_per_step = (prefill_ms + (decode_ms or 0.0))
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wp.description, "batch": wp.S, "seq_len": wp.T, "num_heads": wp.H,
                   "num_kv_heads": wp.Hkv, "head_dim": wp.d, "index_dim": wp.dI, "block": 128, "topk": wp.k},
        "prefill_ms": prefill_ms, "prefill_ms_p50": percentiles(prefill_steps)["p50_ms"],
        "prefill_ms_p95": percentiles(prefill_steps)["p95_ms"], "prefill_ms_p99": percentiles(prefill_steps)["p99_ms"],
        "prefill_ms_with_kernel_timer": sum(prefill_steps_timer) / args.steps,
        "wall_s_timed": wall, "other_prefill": others,
        "selection": "fused" if use_fused else "two-call", "other_selection": osel,
        "decode": dec, "decode_e4m3_index_keys": dec8, "decode_ragged_paged": decp, "decode_token_level": dect,
        "training_step": trn, "stages": stages, "roofline": roof, "achievable_peaks": peaks, "cpu_baseline": cpu,
        "selection_structure": selection_structure(wp, pb.sel, pb.csr_offsets),
        "attention_pairs": split["pairs"],
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
