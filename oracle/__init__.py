"""CPU oracle for MiniMax Sparse Attention (MSA) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library and its Python binding never touch it, and the two
share no code.  The arithmetic lives in ``msa_oracle.c`` (plain C, IEEE double,
OpenMP); this module only builds it, decodes stored inputs to float64 and walks
the (sequence, KV-group) slices of the tensor layouts:

    q      [S, T, H, d]      query heads; head h belongs to group h // (H // Hkv)
    K, V   [S, Hkv, N, d]
    q_idx  [S, Hkv, T, dI]   one index-query head per group
    k_idx  [S, Hkv, N, dI]   one index-key head per group
    scores [S, Hkv, T, nb]   block scores, NaN where not eligible (b > own block)
    sel    [S, Hkv, T, k]    ascending block ids, -1 padded

Queries are the last T of the N positions: row t sits at pos = N - T + t.

Sources: "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比"
(sections 第一步：粗筛, 第二步：精算, Kernel 创新：Outer Gather Q) and the MSA entry
of "稀疏注意力速览（Sparse Attention，2019 ~ 2026）".  Each C function states the
passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
# MSA_ORACLE_LIBRARY may name another build of the same source (the sanitizer build)
_LIB = os.environ.get("MSA_ORACLE_LIBRARY") or _DEFAULT_LIB
SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
CLANG = "/opt/rocm/llvm/bin/clang"

_lib = None


def build(force: bool = True) -> str:
    """Compile msa_oracle.c with gcc (IEEE semantics: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_DEFAULT_LIB):
        tmp = _DEFAULT_LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _DEFAULT_LIB)
    return _DEFAULT_LIB


def build_sanitized(force: bool = True) -> str:
    """The same source under AddressSanitizer + UndefinedBehaviorSanitizer (clang, whose
    ASan runtime the GPU library's host-sanitizer build shares; serial: no OpenMP)."""
    if force or not os.path.exists(SAN_LIB):
        tmp = SAN_LIB + ".tmp%d" % os.getpid()
        cmd = [CLANG, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared", "-fPIC", _SRC, "-o", tmp,
               "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, SAN_LIB)
    return SAN_LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        lib.orc_index_scores.argtypes = [i64, i32, i32, i64, P, P, P, P]
        lib.orc_block_topk.argtypes = [i64, i32, i64, P, P, P]
        lib.orc_invert.argtypes = [i64, i32, i64, P, P, P]
        lib.orc_attention.argtypes = [i64, i32, i32, i32, i32, i64, P, P, P, P, P, ctypes.c_double, P]
        lib.orc_attention_partials.argtypes = [i64, i32, i32, i32, i32, i64, P, P, P, P, P,
                                               ctypes.c_double, P, P]
        lib.orc_lse_merge.argtypes = [i32, i32, i32, i64, P, P, P]
        lib.orc_attention_train.argtypes = [i64, i32, i32, i32, i32, i64, P, P, P, P, P, ctypes.c_double,
                                            P, P, P]
        lib.orc_attention_backward.argtypes = [i64, i32, i32, i32, i32, i64, P, P, P, P, P, ctypes.c_double,
                                               P, P, P, P]
        lib.orc_index_kl.argtypes = [i64, i32, i64, P, P, P, ctypes.c_double, P, P]
        lib.orc_index_backward.argtypes = [i64, i32, i32, i32, i64, P, P, P, P, P, P, P]
        lib.orc_index_argmax.argtypes = [i64, i32, i32, i32, i64, P, P, P, P, P, P, P, P]
        lib.orc_index_backward_at.argtypes = [i64, i32, i32, i64, P, P, P, P, P, P]
        lib.orc_token_topk.argtypes = [i64, i32, i64, P, P, P]
        lib.orc_num_threads.restype = ctypes.c_int
        for f in ("orc_index_scores", "orc_block_topk", "orc_invert", "orc_attention",
                  "orc_attention_partials", "orc_lse_merge", "orc_attention_train", "orc_attention_backward",
                  "orc_index_kl", "orc_index_backward", "orc_index_argmax", "orc_index_backward_at",
                  "orc_token_topk"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().orc_num_threads())


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def e4m3_table() -> np.ndarray:
    """The 256 values of the OCP FP8 E4M3 format as float64: sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; code
    S.1111.111 is NaN (there is no infinity)."""
    c = np.arange(256)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    v = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = s * v
    v[(e == 15) & (m == 7)] = np.nan
    return v


def decode_e4m3(codes) -> np.ndarray:
    """uint8 E4M3 codes -> float64, exactly."""
    return e4m3_table()[np.asarray(codes, dtype=np.uint8)]


def decode(x) -> np.ndarray:
    """Stored input -> float64, exactly.  Accepts numpy float arrays, numpy uint16
    arrays holding bf16 bit patterns, or (CPU) torch tensors of float32, bfloat16 or
    float8_e4m3fn (decoded with e4m3_table)."""
    try:
        import torch  # noqa: F401  (torch is optional for pure-numpy callers)
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16).numpy().view(np.uint16)
            elif x.dtype == torch.float8_e4m3fn:
                return decode_e4m3(x.view(torch.uint8).numpy())
            else:
                x = x.numpy()
    except ImportError:
        pass
    x = np.asarray(x)
    if x.dtype == np.uint16:  # bf16 bit patterns: the high half of an IEEE float32
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def positions(N: int, T: int) -> np.ndarray:
    """Absolute positions of the T query rows: the last T of N."""
    return np.arange(N - T, N, dtype=np.int64)


# ---------------------------------------------------------------- per-slice calls
def slice_index_scores(qI_rows, pos, kI, B: int) -> np.ndarray:
    """qI_rows [R, dI], pos [R], kI [N, dI] -> [R, nb] (NaN beyond the own block)."""
    qI_rows = np.ascontiguousarray(qI_rows, dtype=np.float64)
    kI = np.ascontiguousarray(kI, dtype=np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    R, dI = qI_rows.shape
    N = kI.shape[0]
    nb = (N + B - 1) // B
    out = np.empty((R, nb), dtype=np.float64)
    _load().orc_index_scores(N, B, dI, R, _p(qI_rows), _p(pos), _p(kI), _p(out))
    return out


def slice_block_topk(scores, own, k: int) -> np.ndarray:
    """scores [R, nb] (float64 or float32 values), own [R] -> sel [R, k] int32."""
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    own = np.ascontiguousarray(own, dtype=np.int64)
    R, nb = scores.shape
    sel = np.empty((R, k), dtype=np.int32)
    _load().orc_block_topk(nb, k, R, _p(scores), _p(own), _p(sel))
    return sel


def slice_invert(sel, nb: int):
    """sel [T, k] -> (offsets [nb+1] int64, entries [offsets[-1]] int32)."""
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    T, k = sel.shape
    offsets = np.empty(nb + 1, dtype=np.int64)
    entries = np.empty(max(T * k, 1), dtype=np.int32)
    _load().orc_invert(T, k, nb, _p(sel), _p(offsets), _p(entries))
    return offsets, entries[: offsets[-1]].copy()


def slice_attention(q_rows, pos, sel_rows, K, V, B: int, scale: float) -> np.ndarray:
    """q_rows [R, G, d], pos [R], sel_rows [R, k], K/V [N, d] -> out [R, G, d]."""
    q_rows = np.ascontiguousarray(q_rows, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel_rows = np.ascontiguousarray(sel_rows, dtype=np.int32)
    R, G, d = q_rows.shape
    k = sel_rows.shape[1]
    out = np.empty((R, G, d), dtype=np.float64)
    _load().orc_attention(K.shape[0], B, d, G, k, R, _p(q_rows), _p(pos), _p(sel_rows),
                          _p(K), _p(V), float(scale), _p(out))
    return out


def slice_attention_partials(q_rows, pos, sel_rows, K, V, B: int, scale: float):
    """-> (lse [R, k, G], Op [R, k, G, d]); slots with sel -1 give lse -inf, Op 0."""
    q_rows = np.ascontiguousarray(q_rows, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel_rows = np.ascontiguousarray(sel_rows, dtype=np.int32)
    R, G, d = q_rows.shape
    k = sel_rows.shape[1]
    lse = np.empty((R, k, G), dtype=np.float64)
    Op = np.empty((R, k, G, d), dtype=np.float64)
    _load().orc_attention_partials(K.shape[0], B, d, G, k, R, _p(q_rows), _p(pos), _p(sel_rows),
                                   _p(K), _p(V), float(scale), _p(lse), _p(Op))
    return lse, Op


def slice_lse_merge(lse, Op) -> np.ndarray:
    """lse [R, k, G], Op [R, k, G, d] -> out [R, G, d]."""
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    Op = np.ascontiguousarray(Op, dtype=np.float64)
    R, k, G, d = Op.shape
    out = np.empty((R, G, d), dtype=np.float64)
    _load().orc_lse_merge(d, G, k, R, _p(lse), _p(Op), _p(out))
    return out


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def slice_attention_train(q_rows, pos, sel_rows, K, V, B: int, scale: float):
    """-> (out [R, G, d], lse [R, G] natural log, mass [R, k] teacher block masses)."""
    q_rows, K, V = _f64(q_rows), _f64(K), _f64(V)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel_rows = np.ascontiguousarray(sel_rows, dtype=np.int32)
    R, G, d = q_rows.shape
    k = sel_rows.shape[1]
    out = np.empty((R, G, d))
    lse = np.empty((R, G))
    mass = np.empty((R, k))
    _load().orc_attention_train(K.shape[0], B, d, G, k, R, _p(q_rows), _p(pos), _p(sel_rows), _p(K), _p(V),
                                float(scale), _p(out), _p(lse), _p(mass))
    return out, lse, mass


def slice_attention_backward(q_rows, pos, sel_rows, K, V, B: int, scale: float, dout):
    """Gradients of sum(dout * out) -> (dq [R, G, d], dK [N, d], dV [N, d])."""
    q_rows, K, V, dout = _f64(q_rows), _f64(K), _f64(V), _f64(dout)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel_rows = np.ascontiguousarray(sel_rows, dtype=np.int32)
    R, G, d = q_rows.shape
    k = sel_rows.shape[1]
    dq = np.empty((R, G, d))
    dK = np.empty(K.shape)
    dV = np.empty(V.shape)
    _load().orc_attention_backward(K.shape[0], B, d, G, k, R, _p(q_rows), _p(pos), _p(sel_rows), _p(K), _p(V),
                                   float(scale), _p(dout), _p(dq), _p(dK), _p(dV))
    return dq, dK, dV


def slice_index_kl(scores, sel_rows, mass, sigma: float):
    """scores [R, nb], sel [R, k], teacher mass [R, k] -> (loss [R], dscore [R, k])."""
    scores, mass = _f64(scores), _f64(mass)
    sel_rows = np.ascontiguousarray(sel_rows, dtype=np.int32)
    R, nb = scores.shape
    k = sel_rows.shape[1]
    loss = np.empty((R,))
    dscore = np.empty((R, k))
    _load().orc_index_kl(nb, k, R, _p(scores), _p(sel_rows), _p(mass), float(sigma), _p(loss), _p(dscore))
    return loss, dscore


def slice_index_backward(qI_rows, pos, sel_rows, KI, B: int, dscore):
    """-> (dqI [R, dI], dKI [N, dI]) through the causal block max-pool."""
    qI_rows, KI, dscore = _f64(qI_rows), _f64(KI), _f64(dscore)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel_rows = np.ascontiguousarray(sel_rows, dtype=np.int32)
    R, dI = qI_rows.shape
    k = sel_rows.shape[1]
    dqI = np.empty((R, dI))
    dKI = np.empty(KI.shape)
    _load().orc_index_backward(KI.shape[0], B, dI, k, R, _p(qI_rows), _p(pos), _p(sel_rows), _p(KI), _p(dscore),
                               _p(dqI), _p(dKI))
    return dqI, dKI


def slice_index_argmax(qI_rows, pos, sel_rows, KI, B: int, cand=None):
    """-> (jbest [R, k] int64, best [R, k], cand_val [R, k]): the max-pool arg-max (lowest
    position among equal scores), its score, and the score at the candidate positions."""
    qI_rows, KI = _f64(qI_rows), _f64(KI)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel_rows = np.ascontiguousarray(sel_rows, dtype=np.int32)
    R, dI = qI_rows.shape
    k = sel_rows.shape[1]
    jb = np.empty((R, k), dtype=np.int64)
    best = np.empty((R, k))
    cv = np.empty((R, k))
    c = None if cand is None else np.ascontiguousarray(cand, dtype=np.int64)
    _load().orc_index_argmax(KI.shape[0], B, dI, k, R, _p(qI_rows), _p(pos), _p(sel_rows), _p(KI),
                             _p(c) if c is not None else None, _p(jb), _p(best), _p(cv))
    return jb, best, cv


def slice_index_backward_at(qI_rows, jstar, KI, dscore):
    """The max-pool gradient scatter for given arg-max positions jstar [R, k] (-1 = none)."""
    qI_rows, KI, dscore = _f64(qI_rows), _f64(KI), _f64(dscore)
    jstar = np.ascontiguousarray(jstar, dtype=np.int64)
    R, dI = qI_rows.shape
    k = jstar.shape[1]
    dqI = np.empty((R, dI))
    dKI = np.empty(KI.shape)
    _load().orc_index_backward_at(KI.shape[0], dI, k, R, _p(qI_rows), _p(jstar), _p(KI), _p(dscore), _p(dqI),
                                  _p(dKI))
    return dqI, dKI


def slice_token_scores(qI_rows, pos, kI) -> np.ndarray:
    """Token-level index scores [R, N] (the block scores with block size 1; NaN past pos)."""
    return slice_index_scores(qI_rows, pos, kI, 1)


def slice_token_topk(scores, pos, budget: int) -> np.ndarray:
    """scores [R, N] -> [R, budget] ascending positions of the top tokens (-1 padded)."""
    scores = np.ascontiguousarray(np.nan_to_num(np.asarray(scores, dtype=np.float64), nan=-np.inf))
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    R, N = scores.shape
    out = np.empty((R, budget), dtype=np.int32)
    _load().orc_token_topk(N, budget, R, _p(scores), _p(pos), _p(out))
    return out


def slice_token_attention(q_rows, pos, tok_rows, K, V, scale: float) -> np.ndarray:
    """Attention over selected token positions (the block attention with block size 1)."""
    return slice_attention(q_rows, pos, tok_rows, K, V, 1, scale)


# ------------------------------------------------------- whole-tensor conveniences
def index_scores(q_idx, k_idx, N: int, B: int) -> np.ndarray:
    """q_idx [S, Hkv, T, dI], k_idx [S, Hkv, N, dI] -> scores [S, Hkv, T, nb]."""
    q_idx = decode(q_idx)
    k_idx = decode(k_idx)
    S, Hkv, T, _ = q_idx.shape
    nb = (N + B - 1) // B
    pos = positions(N, T)
    out = np.empty((S, Hkv, T, nb), dtype=np.float64)
    for s in range(S):
        for g in range(Hkv):
            out[s, g] = slice_index_scores(q_idx[s, g], pos, k_idx[s, g], B)
    return out


def block_topk(scores, N: int, B: int, k: int) -> np.ndarray:
    """scores [S, Hkv, T, nb] -> sel [S, Hkv, T, k]."""
    scores = np.asarray(scores)
    S, Hkv, T, nb = scores.shape
    own = positions(N, T) // B
    sel = np.empty((S, Hkv, T, k), dtype=np.int32)
    for s in range(S):
        for g in range(Hkv):
            sel[s, g] = slice_block_topk(scores[s, g], own, k)
    return sel


def invert(sel, nb: int):
    """sel [S, Hkv, T, k] -> list over (s, g) of (offsets, entries), row-major in (s, g)."""
    S, Hkv = sel.shape[:2]
    return [[slice_invert(sel[s, g], nb) for g in range(Hkv)] for s in range(S)]


def attention(q, K, V, sel, B: int, scale: float, rows=None) -> np.ndarray:
    """q [S, T, H, d], K/V [S, Hkv, N, d], sel [S, Hkv, T, k] -> out [S, R, H, d].

    rows: optional list of query-row indices t to compute (default: all T)."""
    q = decode(q)
    K = decode(K)
    V = decode(V)
    S, T, H, d = q.shape
    Hkv, N = K.shape[1], K.shape[2]
    G = H // Hkv
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = positions(N, T)[rows]
    out = np.empty((S, len(rows), H, d), dtype=np.float64)
    for s in range(S):
        for g in range(Hkv):
            qr = q[s][rows][:, g * G:(g + 1) * G, :]
            out[s, :, g * G:(g + 1) * G, :] = slice_attention(
                qr, pos, sel[s, g][rows], K[s, g], V[s, g], B, scale)
    return out


class Timer:
    """Wall-clock stopwatch for the CPU-baseline leg."""

    def __enter__(self):
        self.t0 = time.perf_counter()
        return self

    def __exit__(self, *exc):
        self.seconds = time.perf_counter() - self.t0
