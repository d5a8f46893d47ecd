"""Dense NumPy brute force for tiny MSA inputs -- a second route to every result
the oracle computes, used only to pin the oracle.

It never gathers: it builds the full [T, N] score matrix, pools it with a reshape,
ranks blocks with a lexicographic sort, and evaluates attention as a dense
softmax under a boolean [T, N] mask (selected blocks AND causal)."""
import numpy as np


def scores(qI, kI, pos, B):
    """qI [T, dI], kI [N, dI], pos [T] -> [T, nb] with NaN beyond the own block."""
    T = qI.shape[0]
    N = kI.shape[0]
    nb = (N + B - 1) // B
    dense = qI @ kI.T                                   # [T, N]
    causal = np.arange(N)[None, :] <= pos[:, None]
    dense = np.where(causal, dense, -np.inf)
    padded = np.full((T, nb * B), -np.inf)
    padded[:, :N] = dense
    pooled = padded.reshape(T, nb, B).max(axis=2)
    own = pos // B
    pooled[np.arange(nb)[None, :] > own[:, None]] = np.nan
    return pooled


def topk(sc, own, k):
    """Sort eligible blocks by (-score, block id); take k-1 best plus the own block."""
    T, nb = sc.shape
    out = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        bt = int(own[t])
        cand = np.arange(bt)
        order = np.lexsort((cand, -sc[t, :bt])) if bt > 0 else np.zeros(0, dtype=np.int64)
        chosen = sorted([bt] + list(cand[order[: k - 1]]))
        out[t, : len(chosen)] = chosen
    return out


def invert(sel, nb):
    T, k = sel.shape
    flat = sel.reshape(-1)
    offsets = [0]
    entries = []
    for b in range(nb):
        idx = np.nonzero(flat == b)[0]          # ascending flat index = ascending (t, slot)
        entries.extend(int(i) for i in idx)
        offsets.append(len(entries))
    return np.array(offsets, dtype=np.int64), np.array(entries, dtype=np.int32)


def attention(q, K, V, pos, sel, B, scale):
    """q [T, G, d], K/V [N, d], sel [T, k] -> [T, G, d] via a dense masked softmax."""
    T = q.shape[0]
    N = K.shape[0]
    blk = np.arange(N) // B
    mask = np.zeros((T, N), dtype=bool)
    for t in range(T):
        chosen = sel[t][sel[t] >= 0]
        mask[t] = np.isin(blk, chosen) & (np.arange(N) <= pos[t])
    logits = np.einsum("tgd,nd->tgn", q, K) * scale
    logits = np.where(mask[:, None, :], logits, -np.inf)
    m = logits.max(axis=2, keepdims=True)
    w = np.exp(logits - m)
    w = w / w.sum(axis=2, keepdims=True)
    return np.einsum("tgn,nd->tgd", w, V)
