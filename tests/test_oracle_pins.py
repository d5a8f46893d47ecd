"""Pins for the CPU oracle (CPU only).

The pages print no worked MSA example, so the oracle is pinned by (a) a dense
brute force that reaches every result by a different route, (b) closed forms,
(c) special cases that reduce to textbook / library dense attention, and (d) the
invariants the pages state (own block always selected, a fixed budget of k
blocks).  Each test names the passage it pins."""
import numpy as np
import pytest
import torch

import oracle
from tests import brute_force as bf

RNG = np.random.default_rng(20260603)


def _pos(N, T):
    return np.arange(N - T, N, dtype=np.int64)


# ------------------------------------------------------------------ index scores
# "第一步：粗筛" items 1-2: score every token, block score = max inside the block.
@pytest.mark.parametrize("N,T,B,dI", [(16, 16, 4, 3), (37, 20, 8, 5), (300, 300, 128, 32),
                                      (129, 2, 128, 4), (1, 1, 4, 2)])
def test_scores_match_dense_brute_force(N, T, B, dI):
    qI = RNG.standard_normal((T, dI))
    kI = RNG.standard_normal((N, dI))
    pos = _pos(N, T)
    got = oracle.slice_index_scores(qI, pos, kI, B)
    ref = bf.scores(qI, kI, pos, B)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_allclose(got[ok], ref[ok], rtol=1e-12, atol=1e-12)


def test_scores_closed_forms():
    N, T, B, dI = 50, 50, 8, 6
    pos = _pos(N, T)
    nb = (N + B - 1) // B
    # zero keys -> every eligible block score is exactly 0
    s0 = oracle.slice_index_scores(RNG.standard_normal((T, dI)), pos, np.zeros((N, dI)), B)
    elig = np.arange(nb)[None, :] <= (pos // B)[:, None]
    assert np.all(s0[elig] == 0.0) and np.all(np.isnan(s0[~elig]))
    # q = k = e0 -> every eligible block score is exactly 1
    e0q = np.zeros((T, dI)); e0q[:, 0] = 1
    e0k = np.zeros((N, dI)); e0k[:, 0] = 1
    s1 = oracle.slice_index_scores(e0q, pos, e0k, B)
    assert np.all(s1[elig] == 1.0)


def test_scores_are_causal_inside_own_block():
    # key j's value grows with j: the own-block maximum must stop at j = pos.
    N, B = 24, 8
    kI = np.arange(N, dtype=np.float64)[:, None]
    qI = np.ones((N, 1))
    s = oracle.slice_index_scores(qI, _pos(N, N), kI, B)
    for t in range(N):
        bt = t // B
        assert s[t, bt] == t                      # max over keys bt*B..t is t itself
        for b in range(bt):
            assert s[t, b] == (b + 1) * B - 1     # full past blocks: their last key


def test_scores_hand_worked_example():
    # tiny example worked out by hand: B = 2, dI = 1, q = 1 for every row,
    # keys 3,-1 | 0,5 | 2 (ragged last block)
    kI = np.array([[3.0], [-1.0], [0.0], [5.0], [2.0]])
    qI = np.ones((5, 1))
    s = oracle.slice_index_scores(qI, _pos(5, 5), kI, 2)
    expect = np.array([[3, np.nan, np.nan],
                       [3, np.nan, np.nan],
                       [3, 0, np.nan],
                       [3, 5, np.nan],
                       [3, 5, 2]], dtype=np.float64)
    np.testing.assert_array_equal(s, expect)


# ------------------------------------------------------------------ selection
# "第一步：粗筛" item 3 and the head-pattern appendix: own block forced, the rest
# by score; ties -> lower block id (fixed tie-break).
@pytest.mark.parametrize("k", [1, 2, 4, 16, 64])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_matches_sort_brute_force(k, ties):
    T, nb = 200, 40
    own = RNG.integers(0, nb, size=T)
    sc = RNG.integers(0, 3, size=(T, nb)).astype(np.float64) if ties else RNG.standard_normal((T, nb))
    got = oracle.slice_block_topk(sc, own, k)
    ref = bf.topk(sc, own, k)
    np.testing.assert_array_equal(got, ref)


def test_topk_invariants():
    T, nb, k = 500, 64, 16
    own = RNG.integers(0, nb, size=T)
    sc = RNG.standard_normal((T, nb))
    sel = oracle.slice_block_topk(sc, own, k)
    for t in range(T):
        row = sel[t]
        valid = row[row >= 0]
        assert own[t] in valid                               # own block always present
        assert len(valid) == min(k, own[t] + 1)              # fixed budget
        assert np.all(valid <= own[t])                       # causal: no future block
        assert np.all(np.diff(valid) > 0)                    # ascending, distinct
        assert np.all(row[len(valid):] == -1)                # -1 padding at the end


def test_topk_all_equal_pins_tie_break():
    nb, k = 30, 5
    own = np.array([29, 10, 3, 0])
    sc = np.full((4, nb), 0.5)
    sel = oracle.slice_block_topk(sc, own, k)
    np.testing.assert_array_equal(sel[0], [0, 1, 2, 3, 29])
    np.testing.assert_array_equal(sel[1], [0, 1, 2, 3, 10])
    np.testing.assert_array_equal(sel[2], [0, 1, 2, 3, -1])
    np.testing.assert_array_equal(sel[3], [0, -1, -1, -1, -1])


def test_topk_signed_zero_is_a_tie():
    sc = np.array([[1.0, -0.0, 0.0, 0.0, 0.0]])
    sc[0, 0] = -1.0
    sel = oracle.slice_block_topk(sc, np.array([4]), 2)
    np.testing.assert_array_equal(sel[0], [1, 4])        # -0.0 == +0.0, lower id wins


def test_topk_boosted_block_always_selected():
    nb, k = 50, 4
    own = np.arange(nb)
    sc = RNG.standard_normal((nb, nb))
    sc[:, 17] += 100.0
    sel = oracle.slice_block_topk(sc, own, k)
    for t in range(18, nb):
        assert 17 in sel[t]


def test_topk_k_at_least_nb_selects_every_causal_block():
    nb = 12
    own = np.arange(nb)
    sel = oracle.slice_block_topk(RNG.standard_normal((nb, nb)), own, nb)
    for t in range(nb):
        np.testing.assert_array_equal(sel[t][: t + 1], np.arange(t + 1))


# ------------------------------------------------------------------ inversion
# "Kernel 创新：Outer Gather Q": gather, per KV block, every query that chose it.
def test_invert_matches_brute_force_and_round_trips():
    T, nb, k = 300, 20, 6
    own = np.minimum(np.arange(T) // 15, nb - 1)
    sel = oracle.slice_block_topk(RNG.standard_normal((T, nb)), own, k)
    off, ent = oracle.slice_invert(sel, nb)
    roff, rent = bf.invert(sel, nb)
    np.testing.assert_array_equal(off, roff)
    np.testing.assert_array_equal(ent, rent)
    assert off[-1] == np.sum(sel >= 0)
    for b in range(nb):
        lst = ent[off[b]:off[b + 1]]
        assert np.all(np.diff(lst // k) > 0)                 # ascending t, one slot per t
        assert np.all(sel.reshape(-1)[lst] == b)              # every entry maps back to b


# ------------------------------------------------------------------ attention
# "第二步：精算": exact softmax attention restricted to the chosen blocks.
def _rand_attn(N, T, G, d):
    return (RNG.standard_normal((T, G, d)), RNG.standard_normal((N, d)),
            RNG.standard_normal((N, d)))


def test_attention_matches_dense_masked_brute_force():
    N, T, G, d, B, k = 70, 33, 3, 8, 8, 3
    q, K, V = _rand_attn(N, T, G, d)
    pos = _pos(N, T)
    own = pos // B
    sel = oracle.slice_block_topk(RNG.standard_normal((T, (N + B - 1) // B)), own, k)
    got = oracle.slice_attention(q, pos, sel, K, V, B, 0.37)
    ref = bf.attention(q, K, V, pos, sel, B, 0.37)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_attention_full_budget_is_dense_causal_sdpa():
    # k >= nb: MSA reduces to dense causal attention (torch SDPA, fp64, explicit mask
    # because queries are the LAST T positions).
    N, T, G, d, B = 96, 40, 4, 16, 16
    nb = N // B
    q, K, V = _rand_attn(N, T, G, d)
    pos = _pos(N, T)
    sel = oracle.slice_block_topk(np.zeros((T, nb)), pos // B, nb)
    got = oracle.slice_attention(q, pos, sel, K, V, B, 1 / np.sqrt(d))
    qt = torch.from_numpy(q).permute(1, 0, 2)                 # [G, T, d]
    Kt = torch.from_numpy(K)[None].expand(G, N, d)
    Vt = torch.from_numpy(V)[None].expand(G, N, d)
    mask = torch.from_numpy(np.arange(N)[None, :] <= pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask)
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_attention_k1_is_block_local_causal():
    N, T, G, d, B = 64, 64, 2, 4, 16
    q, K, V = _rand_attn(N, T, G, d)
    pos = _pos(N, T)
    sel = oracle.slice_block_topk(RNG.standard_normal((T, N // B)), pos // B, 1)
    got = oracle.slice_attention(q, pos, sel, K, V, B, 0.5)
    for t in range(T):
        lo = (pos[t] // B) * B
        keys = np.arange(lo, pos[t] + 1)
        for h in range(G):
            lg = 0.5 * K[keys] @ q[t, h]
            w = np.exp(lg - lg.max()); w /= w.sum()
            np.testing.assert_allclose(got[t, h], w @ V[keys], rtol=1e-12, atol=1e-13)


def test_partials_merge_equals_direct_attention():
    # log-sum-exp merge over the per-block parts == softmax over the union
    N, T, G, d, B, k = 200, 60, 2, 8, 16, 5
    q, K, V = _rand_attn(N, T, G, d)
    pos = _pos(N, T)
    sel = oracle.slice_block_topk(RNG.standard_normal((T, (N + B - 1) // B)), pos // B, k)
    lse, Op = oracle.slice_attention_partials(q, pos, sel, K, V, B, 0.3)
    merged = oracle.slice_lse_merge(lse, Op)
    direct = oracle.slice_attention(q, pos, sel, K, V, B, 0.3)
    np.testing.assert_allclose(merged, direct, rtol=1e-11, atol=1e-13)
    # single-slot lse is the textbook log-sum-exp of that block's logits
    t, i, h = 59, 0, 1
    b = sel[t, i]
    keys = np.arange(b * B, min((b + 1) * B, pos[t] + 1))
    lg = 0.3 * K[keys] @ q[t, h]
    assert abs(lse[t, i, h] - (lg.max() + np.log(np.exp(lg - lg.max()).sum()))) < 1e-12
    assert np.all(np.isneginf(lse[sel == -1]))


def test_merge_of_random_partition_is_softmax_of_union():
    # arbitrary partition of one key set into 4 parts, merged with the oracle's merge
    n, d = 57, 6
    lg = RNG.standard_normal(n) * 3
    V = RNG.standard_normal((n, d))
    part = RNG.integers(0, 4, size=n)
    lse = np.full((1, 4, 1), -np.inf)
    Op = np.zeros((1, 4, 1, d))
    for i in range(4):
        m = part == i
        if m.any():
            lse[0, i, 0] = np.log(np.exp(lg[m]).sum())
            w = np.exp(lg[m] - lse[0, i, 0])
            Op[0, i, 0] = w @ V[m]
    out = oracle.slice_lse_merge(lse, Op)
    w = np.exp(lg - lg.max()); w /= w.sum()
    np.testing.assert_allclose(out[0, 0], w @ V, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ whole tensors
def test_whole_tensor_walk_matches_slices():
    S, Hkv, G, N, T, d, dI, B, k = 2, 2, 2, 40, 24, 4, 3, 8, 2
    q = RNG.standard_normal((S, T, Hkv * G, d))
    K = RNG.standard_normal((S, Hkv, N, d))
    V = RNG.standard_normal((S, Hkv, N, d))
    qI = RNG.standard_normal((S, Hkv, T, dI))
    kI = RNG.standard_normal((S, Hkv, N, dI))
    sc = oracle.index_scores(qI, kI, N, B)
    sel = oracle.block_topk(sc, N, B, k)
    out = oracle.attention(q, K, V, sel, B, 0.5)
    pos = _pos(N, T)
    for s in range(S):
        for g in range(Hkv):
            ref_sc = bf.scores(qI[s, g], kI[s, g], pos, B)
            np.testing.assert_allclose(np.nan_to_num(sc[s, g]), np.nan_to_num(ref_sc), rtol=1e-12)
            ref_sel = bf.topk(ref_sc, pos // B, k)
            np.testing.assert_array_equal(sel[s, g], ref_sel)
            ref = bf.attention(q[s][:, g * G:(g + 1) * G], K[s, g], V[s, g], pos, ref_sel, B, 0.5)
            np.testing.assert_allclose(out[s][:, g * G:(g + 1) * G], ref, rtol=1e-11, atol=1e-13)


# ------------------------------------------------------------------ 1-byte index keys
# Serving variant of the index keys: OCP FP8 E4M3 storage, decoded exactly.
def test_e4m3_table_matches_the_format_definition():
    t = oracle.e4m3_table()
    # values fixed by the format: bias 7, 3 mantissa bits, subnormals m * 2^-9, no infinity
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x08] == 2.0 ** -6                             # smallest normal
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9  # subnormals
    assert t[0x00] == 0.0 and np.signbit(t[0x80])           # +0 and -0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x39] == 1.125 and t[0x40] == 2.0
    finite = t[~np.isnan(t)]
    assert len(finite) == 254
    # monotone over the positive codes
    assert np.all(np.diff(t[0x00:0x7F]) > 0)


def test_e4m3_table_matches_torch_float8():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = oracle.e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(t))
    np.testing.assert_array_equal(t[~nan], ref[~nan])


def test_decode_handles_e4m3_tensors():
    codes = torch.tensor([0x38, 0x7E, 0x81, 0x00], dtype=torch.uint8)
    np.testing.assert_array_equal(oracle.decode(codes.view(torch.float8_e4m3fn)), [1.0, 448.0, -2.0 ** -9, 0.0])


# ------------------------------------------------------------------ training
# "索引分支训练：KL 对齐" (the index branch is taught by the main branch's attention
# distribution through a KL divergence, teacher cut from the gradient) and the MSA entry's
# "KL loss ... teacher stop-gradient".  The gradients are pinned against torch autograd
# in float64 on the dense masked formulation (a different route: autograd of the
# brute-force mask-and-softmax, not the oracle's hand-derived chain rule) and against
# finite differences of the oracle's own forward.
def _mask(pos, sel, N, B):
    blk = np.arange(N) // B
    m = np.zeros((len(pos), N), dtype=bool)
    for t in range(len(pos)):
        m[t] = np.isin(blk, sel[t][sel[t] >= 0]) & (np.arange(N) <= pos[t])
    return torch.from_numpy(m)


def _train_case(N=70, T=33, G=3, d=8, B=8, k=3):
    q, K, V = _rand_attn(N, T, G, d)
    pos = _pos(N, T)
    sel = oracle.slice_block_topk(RNG.standard_normal((T, (N + B - 1) // B)), pos // B, k)
    return q, K, V, pos, sel


def test_attention_train_lse_and_teacher_mass_match_brute_force():
    N, B, scale = 70, 8, 0.41
    q, K, V, pos, sel = _train_case(N=N, B=B)
    out, lse, mass = oracle.slice_attention_train(q, pos, sel, K, V, B, scale)
    np.testing.assert_allclose(out, oracle.slice_attention(q, pos, sel, K, V, B, scale), rtol=1e-12, atol=1e-13)
    logits = np.einsum("tgd,nd->tgn", q, K) * scale
    logits = np.where(_mask(pos, sel, N, B).numpy()[:, None, :], logits, -np.inf)
    m = logits.max(axis=2)
    ref_lse = m + np.log(np.exp(logits - m[..., None]).sum(axis=2))
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)
    P = np.exp(logits - ref_lse[..., None])               # dense probabilities [T, G, N]
    blk = np.arange(N) // B
    for t in range(len(pos)):
        for i, b in enumerate(sel[t]):
            want = 0.0 if b < 0 else P[t][:, blk == b].sum() / q.shape[1]
            assert abs(mass[t, i] - want) < 1e-12
    np.testing.assert_allclose(mass.sum(axis=1), 1.0, rtol=1e-12)


def test_attention_backward_matches_fp64_autograd():
    N, B, scale = 70, 8, 0.37
    q, K, V, pos, sel = _train_case(N=N, B=B)
    dout = RNG.standard_normal(q.shape)
    dq, dK, dV = oracle.slice_attention_backward(q, pos, sel, K, V, B, scale, dout)
    tq, tK, tV = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, K, V))
    logits = torch.einsum("tgd,nd->tgn", tq, tK) * scale
    logits = logits.masked_fill(~_mask(pos, sel, N, B)[:, None, :], float("-inf"))
    out = torch.einsum("tgn,nd->tgd", torch.softmax(logits, dim=2), tV)
    (out * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, tK.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, tV.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_attention_backward_finite_differences():
    N, T, G, d, B, k, scale = 24, 10, 2, 4, 8, 2, 0.5
    q, K, V, pos, sel = _train_case(N=N, T=T, G=G, d=d, B=B, k=k)
    dout = RNG.standard_normal(q.shape)
    dq, dK, dV = oracle.slice_attention_backward(q, pos, sel, K, V, B, scale, dout)

    def f(q_, K_, V_):
        return float((oracle.slice_attention(q_, pos, sel, K_, V_, B, scale) * dout).sum())
    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (K, dK, 1), (V, dV, 2)):
        for idx in [tuple(RNG.integers(0, s) for s in arr.shape) for _ in range(6)]:
            a, b = arr.copy(), arr.copy()
            a[idx] += eps
            b[idx] -= eps
            args_a = [q, K, V]
            args_b = [q, K, V]
            args_a[which], args_b[which] = a, b
            fd = (f(*args_a) - f(*args_b)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def test_index_kl_closed_forms():
    R, nb, k, sigma = 6, 9, 4, 0.7
    scores = RNG.standard_normal((R, nb))
    sel = np.array([np.sort(RNG.choice(nb, k, replace=False)) for _ in range(R)], dtype=np.int32)
    sel[0, 2:] = -1                                          # a row with two valid slots
    # teacher = student: zero loss, zero gradient
    z = sigma * np.take_along_axis(scores, np.maximum(sel, 0), axis=1)
    z = np.where(sel >= 0, z, -np.inf)
    pS = np.exp(z - z.max(axis=1, keepdims=True))
    pS /= pS.sum(axis=1, keepdims=True)
    loss, ds = oracle.slice_index_kl(scores, sel, pS * 3.0, sigma)   # any positive scale of the teacher
    np.testing.assert_allclose(loss, 0.0, atol=1e-12)
    np.testing.assert_allclose(ds, 0.0, atol=1e-12)
    # one-hot teacher: the loss is the student's negative log-probability of that block
    onehot = np.zeros((R, k))
    onehot[:, 1] = 1.0
    loss, ds = oracle.slice_index_kl(scores, sel, onehot, sigma)
    np.testing.assert_allclose(loss, -np.log(pS[:, 1]), rtol=1e-12)
    np.testing.assert_allclose(ds[:, 1], sigma * (pS[:, 1] - 1.0), rtol=1e-12)
    # equal scores: uniform student, loss = log(#valid) - entropy(teacher)
    pT = RNG.random((R, k))
    pT = np.where(sel >= 0, pT, 0.0)
    loss, ds = oracle.slice_index_kl(np.zeros((R, nb)), sel, pT, sigma)
    nv = (sel >= 0).sum(axis=1)
    q_ = pT / pT.sum(axis=1, keepdims=True)
    ent = -np.where(q_ > 0, q_ * np.log(np.where(q_ > 0, q_, 1.0)), 0.0).sum(axis=1)
    np.testing.assert_allclose(loss, np.log(nv) - ent, rtol=1e-12)
    np.testing.assert_allclose(ds.sum(axis=1), 0.0, atol=1e-12)   # probabilities on both sides sum to 1
    assert np.all(ds[sel < 0] == 0.0)


def test_index_kl_gradient_finite_differences():
    R, nb, k, sigma = 5, 8, 4, 1.3
    scores = RNG.standard_normal((R, nb))
    sel = np.array([np.sort(RNG.choice(nb, k, replace=False)) for _ in range(R)], dtype=np.int32)
    mass = RNG.random((R, k))
    loss, ds = oracle.slice_index_kl(scores, sel, mass, sigma)
    assert np.all(loss >= -1e-15)
    eps = 1e-6
    for r in range(R):
        for i in range(k):
            a, b = scores.copy(), scores.copy()
            a[r, sel[r, i]] += eps
            b[r, sel[r, i]] -= eps
            fd = (oracle.slice_index_kl(a, sel, mass, sigma)[0][r] - oracle.slice_index_kl(b, sel, mass, sigma)[0][r])
            assert abs(fd / (2 * eps) - ds[r, i]) < 1e-7


def test_index_backward_matches_fp64_autograd_through_the_max_pool():
    N, T, B, dI, k = 70, 33, 8, 5, 3
    qI, KI = RNG.standard_normal((T, dI)), RNG.standard_normal((N, dI))
    pos = _pos(N, T)
    sel = oracle.slice_block_topk(RNG.standard_normal((T, (N + B - 1) // B)), pos // B, k)
    dscore = RNG.standard_normal((T, k)) * (sel >= 0)
    dq, dK = oracle.slice_index_backward(qI, pos, sel, KI, B, dscore)
    tq = torch.tensor(qI, requires_grad=True)
    tK = torch.tensor(KI, requires_grad=True)
    nb = (N + B - 1) // B
    s = tq @ tK.T                                            # [T, N] token scores
    causal = torch.from_numpy(np.arange(N)[None, :] <= pos[:, None])
    s = s.masked_fill(~causal, float("-inf"))
    s = torch.nn.functional.pad(s, (0, nb * B - N), value=float("-inf")).view(T, nb, B)
    blockscore = s.amax(dim=2)                               # [T, nb] (no ties in random data)
    chosen = torch.from_numpy(np.maximum(sel, 0)).long()
    picked = torch.gather(blockscore, 1, chosen)
    (picked * torch.from_numpy(dscore)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dK, tK.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_index_backward_tie_goes_to_the_lowest_position():
    N, B, dI = 16, 8, 3
    KI = np.zeros((N, dI))
    KI[:, 0] = 1.0                                           # every key scores the same
    qI = np.array([[2.0, 0.0, 0.0]])
    pos = np.array([N - 1])
    sel = np.array([[0, 1]], dtype=np.int32)
    dq, dK = oracle.slice_index_backward(qI, pos, sel, KI, B, np.array([[1.0, 0.5]]))
    assert np.count_nonzero(dK.any(axis=1)) == 2
    np.testing.assert_allclose(dK[0], [2.0, 0.0, 0.0])
    np.testing.assert_allclose(dK[8], [1.0, 0.0, 0.0])
    np.testing.assert_allclose(dq[0], [1.5, 0.0, 0.0])


def test_index_argmax_and_scatter_agree_with_the_fused_backward():
    N, T, B, dI, k = 70, 33, 8, 5, 3
    qI, KI = RNG.standard_normal((T, dI)), RNG.standard_normal((N, dI))
    pos = _pos(N, T)
    sel = oracle.slice_block_topk(RNG.standard_normal((T, (N + B - 1) // B)), pos // B, k)
    dscore = RNG.standard_normal((T, k)) * (sel >= 0)
    jb, best, cv = oracle.slice_index_argmax(qI, pos, sel, KI, B, cand=None)
    # the block scores of the max-pool are the best values
    sc = oracle.slice_index_scores(qI, pos, KI, B)
    ok = sel >= 0
    np.testing.assert_allclose(best[ok], np.take_along_axis(sc, np.maximum(sel, 0), axis=1)[ok], rtol=1e-12)
    assert np.all(jb[~ok] == -1) and np.all(jb[ok] // B == sel[ok]) and np.all(jb[ok] <= pos[:, None].repeat(k, 1)[ok])
    # the score at a candidate position is reported; outside the block it is NaN
    _, _, cv = oracle.slice_index_argmax(qI, pos, sel, KI, B, cand=jb)
    np.testing.assert_array_equal(cv[ok], best[ok])
    _, _, cv2 = oracle.slice_index_argmax(qI, pos, sel, KI, B, cand=np.where(ok, jb + B, -1))
    assert np.all(np.isnan(cv2))
    a = oracle.slice_index_backward(qI, pos, sel, KI, B, dscore)
    b = oracle.slice_index_backward_at(qI, jb, KI, dscore)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------ token level
# "分歧一：颗粒度" (DSA: 2048 single tokens per query, MSA: 16 blocks x 128, same budget) and
# the DSA entry of "稀疏注意力速览" (top-k single tokens by the indexer's token scores).
@pytest.mark.parametrize("budget,ties", [(5, False), (5, True), (64, False), (300, False)])
def test_token_topk_matches_sort_brute_force(budget, ties):
    N, T = 200, 40
    pos = _pos(N, T)
    sc = RNG.integers(0, 4, (T, N)).astype(float) if ties else RNG.standard_normal((T, N))
    got = oracle.slice_token_topk(sc, pos, budget)
    for t in range(T):
        n = pos[t] + 1
        order = np.lexsort((np.arange(n), -sc[t, :n]))     # score desc, position asc
        want = np.sort(order[:min(budget, n)])
        np.testing.assert_array_equal(got[t, :len(want)], want)
        assert np.all(got[t, len(want):] == -1)


def test_token_scores_are_the_block_scores_of_block_size_one():
    N, T, dI = 60, 60, 7
    qI, kI = RNG.standard_normal((T, dI)), RNG.standard_normal((N, dI))
    pos = _pos(N, T)
    got = oracle.slice_token_scores(qI, pos, kI)
    ref = qI @ kI.T
    causal = np.arange(N)[None, :] <= pos[:, None]
    np.testing.assert_allclose(got[causal], ref[causal], rtol=1e-12, atol=1e-12)
    assert np.all(np.isnan(got[~causal]))


def test_token_attention_matches_dense_masked_brute_force():
    N, T, G, d = 90, 30, 3, 8
    q, K, V = _rand_attn(N, T, G, d)
    pos = _pos(N, T)
    sc = oracle.slice_token_scores(RNG.standard_normal((T, 5)), pos, RNG.standard_normal((N, 5)))
    tok = oracle.slice_token_topk(sc, pos, 17)
    got = oracle.slice_token_attention(q, pos, tok, K, V, 0.29)
    ref = bf.attention(q, K, V, pos, tok, 1, 0.29)              # block size 1 = single tokens
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    # the budget covers every causal token: dense causal attention
    full = oracle.slice_token_attention(q, pos, oracle.slice_token_topk(sc, pos, N), K, V, 0.29)
    dense = bf.attention(q, K, V, pos, np.tile(np.arange(N, dtype=np.int32), (T, 1)), 1, 0.29)
    np.testing.assert_allclose(full, dense, rtol=1e-12, atol=1e-13)
