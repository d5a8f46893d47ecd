"""Python binding of libmsa.so -- MiniMax Sparse Attention (MSA) on MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.  PyTorch
is used for device memory and streams.  The names mirror the C ABI in
include/msa.h (without the ``msa_`` prefix); tensors are passed as torch tensors
(their ``data_ptr()``) or raw integer device addresses.

If the library is missing the import still succeeds, but every call raises
``MSAError``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
# MSA_LIBRARY may name another build of the same library (e.g. a debug build).
LIB_PATH = os.environ.get("MSA_LIBRARY") or os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARGUMENT, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE_TOO_SMALL, MSA_ERR_DEVICE = range(5)
MSA_F32, MSA_BF16, MSA_FP8_E4M3 = 0, 1, 2
(MSA_CALL_INVERT, MSA_CALL_PREFILL, MSA_CALL_DECODE, MSA_CALL_BACKWARD, MSA_CALL_INDEX_BACKWARD,
 MSA_CALL_TOKEN_DECODE, MSA_CALL_INDEX_TOPK) = 2, 3, 4, 5, 6, 7, 8

EXPORTED = ("msa_index_scores", "msa_block_topk", "msa_invert_selection", "msa_sparse_attn_prefill",
            "msa_sparse_attn_decode", "msa_workspace_bytes", "msa_status_string",
            "msa_last_error_message", "msa_profiler_enable", "msa_profiler_read", "msa_profiler_samples",
            "msa_index_scores_kv",
            "msa_block_topk_kv", "msa_sparse_attn_decode_kv", "msa_sparse_attn_prefill_train",
            "msa_sparse_attn_backward", "msa_index_kl", "msa_index_backward", "msa_token_scores",
            "msa_token_topk", "msa_token_attn_decode", "msa_token_workspace_bytes", "msa_index_topk",
            "msa_sparse_attn_prefill_kv", "msa_sparse_attn_decode_noalloc")


class MSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Problem(ctypes.Structure):
    """msa_problem (include/msa.h)."""
    _fields_ = [("batch", ctypes.c_int32), ("num_q", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("topk", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("index_key_dtype", ctypes.c_int32)]

    @property
    def nb(self) -> int:
        return (self.kv_len + self.block_size - 1) // self.block_size

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    def __repr__(self):
        return "Problem(" + ", ".join("%s=%r" % (f, getattr(self, f)) for f, _ in self._fields_) + ")"


class KVLayout(ctypes.Structure):
    """msa_kv_layout: per-sequence lengths and an optional page table (device pointers)."""
    _fields_ = [("kv_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("table_stride", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


def kv_layout(kv_lens, block_table=None, num_pages: int = 0) -> KVLayout:
    """Layout for the per-sequence calls: kv_lens int32 [S] on the device; block_table int32
    [S, stride] on the device (or None for dense caches); num_pages = pages in each pool."""
    lay = KVLayout()
    lay.kv_lens = kv_lens.data_ptr()
    lay.block_table = block_table.data_ptr() if block_table is not None else None
    lay.table_stride = int(block_table.shape[1]) if block_table is not None else 0
    lay.num_pages = int(num_pages)
    lay._keep = (kv_lens, block_table)  # the tensors must outlive the calls
    return lay


def problem(batch, num_q, kv_len, num_heads, num_kv_heads, head_dim, index_dim, topk,
            dtype=MSA_BF16, block_size=128, softmax_scale=0.0, index_key_dtype=0) -> Problem:
    return Problem(batch, num_q, kv_len, num_heads, num_kv_heads, head_dim, index_dim, block_size,
                   topk, dtype, softmax_scale, index_key_dtype)


_lib = None


def lib():
    """The loaded libmsa.so (raises MSAError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MSAError(MSA_ERR_DEVICE, "libmsa.so not built at %s (run __graft_entry__.build())" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        PP = ctypes.POINTER(Problem)
        st = ctypes.c_int
        L.msa_index_scores.argtypes = [PP, P, P, P, P]
        L.msa_block_topk.argtypes = [PP, P, P, P]
        L.msa_invert_selection.argtypes = [PP, P, P, P, P, ctypes.c_size_t, P]
        L.msa_sparse_attn_prefill.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_sparse_attn_decode.argtypes = [PP, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_sparse_attn_decode_noalloc.argtypes = [PP, P, P, P, P, P, P]
        L.msa_sparse_attn_decode_noalloc.restype = st
        LP = ctypes.POINTER(KVLayout)
        L.msa_index_scores_kv.argtypes = [PP, LP, P, P, P, P]
        L.msa_block_topk_kv.argtypes = [PP, LP, P, P, P]
        L.msa_sparse_attn_decode_kv.argtypes = [PP, LP, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_sparse_attn_prefill_train.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_sparse_attn_backward.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_index_kl.argtypes = [PP, P, P, P, ctypes.c_float, P, P, P]
        L.msa_index_backward.argtypes = [PP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_sparse_attn_prefill_kv.argtypes = [PP, ctypes.POINTER(KVLayout), P, P, P, P, P, P, P, P,
                                                 ctypes.c_size_t, P]
        L.msa_sparse_attn_prefill_kv.restype = st
        L.msa_index_topk.argtypes = [PP, P, P, P, P, ctypes.c_size_t, P]
        L.msa_index_topk.restype = st
        L.msa_token_scores.argtypes = [PP, P, P, P, P]
        L.msa_token_topk.argtypes = [PP, ctypes.c_int32, P, P, P, ctypes.c_size_t, P]
        L.msa_token_attn_decode.argtypes = [PP, ctypes.c_int32, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_token_workspace_bytes.argtypes = [PP, ctypes.c_int32]
        L.msa_token_workspace_bytes.restype = ctypes.c_size_t
        for f in ("msa_token_scores", "msa_token_topk", "msa_token_attn_decode"):
            getattr(L, f).restype = st
        for f in ("msa_index_scores", "msa_block_topk", "msa_invert_selection",
                  "msa_sparse_attn_prefill", "msa_sparse_attn_decode", "msa_index_scores_kv",
                  "msa_block_topk_kv", "msa_sparse_attn_decode_kv", "msa_sparse_attn_prefill_train",
                  "msa_sparse_attn_backward", "msa_index_kl", "msa_index_backward"):
            getattr(L, f).restype = st
        L.msa_workspace_bytes.argtypes = [PP, ctypes.c_int]
        L.msa_workspace_bytes.restype = ctypes.c_size_t
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_last_error_message.argtypes = []
        L.msa_last_error_message.restype = ctypes.c_char_p
        L.msa_profiler_enable.argtypes = [ctypes.c_int]
        L.msa_profiler_enable.restype = st
        L.msa_profiler_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
        L.msa_profiler_read.restype = st
        L.msa_profiler_samples.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_float), ctypes.c_int64,
                                           ctypes.POINTER(ctypes.c_int64)]
        L.msa_profiler_samples.restype = st
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return ctypes.c_void_p(x)
    return ctypes.c_void_p(x.data_ptr())


def _stream(stream, *tensors):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    for t in tensors:
        if hasattr(t, "is_cuda") and t.is_cuda:
            import torch
            return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(0)


def _check(status: int):
    if status != MSA_OK:
        L = lib()
        raise MSAError(status, "%s: %s" % (L.msa_status_string(status).decode(),
                                           L.msa_last_error_message().decode()))


def status_string(status: int) -> str:
    return lib().msa_status_string(status).decode()


def last_error_message() -> str:
    return lib().msa_last_error_message().decode()


def workspace_bytes(prob: Problem, which_call: int) -> int:
    return int(lib().msa_workspace_bytes(ctypes.byref(prob), which_call))


def index_scores(prob: Problem, q_idx, k_idx, scores, stream=None) -> None:
    _check(lib().msa_index_scores(ctypes.byref(prob), _ptr(q_idx), _ptr(k_idx), _ptr(scores),
                                  _stream(stream, q_idx)))


def index_topk(prob: Problem, q_idx, k_idx, sel, workspace, workspace_bytes_: int, stream=None) -> None:
    """Fused scores + top-k: the selection without the [S, Hkv, T, nb] block scores."""
    _check(lib().msa_index_topk(ctypes.byref(prob), _ptr(q_idx), _ptr(k_idx), _ptr(sel), _ptr(workspace),
                                workspace_bytes_, _stream(stream, q_idx)))


def block_topk(prob: Problem, scores, sel, stream=None) -> None:
    _check(lib().msa_block_topk(ctypes.byref(prob), _ptr(scores), _ptr(sel), _stream(stream, scores)))


def invert_selection(prob: Problem, sel, csr_offsets, csr_entries, workspace, workspace_bytes_: int,
                     stream=None) -> None:
    _check(lib().msa_invert_selection(ctypes.byref(prob), _ptr(sel), _ptr(csr_offsets), _ptr(csr_entries),
                                      _ptr(workspace), workspace_bytes_, _stream(stream, sel)))


def sparse_attn_prefill(prob: Problem, q, k, v, csr_offsets, csr_entries, sel, out, workspace,
                        workspace_bytes_: int, stream=None) -> None:
    _check(lib().msa_sparse_attn_prefill(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(csr_offsets),
                                         _ptr(csr_entries), _ptr(sel), _ptr(out), _ptr(workspace),
                                         workspace_bytes_, _stream(stream, q)))


def sparse_attn_decode(prob: Problem, q, k_cache, v_cache, sel, out, workspace, workspace_bytes_: int,
                       stream=None) -> None:
    _check(lib().msa_sparse_attn_decode(ctypes.byref(prob), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(sel), _ptr(out), _ptr(workspace), workspace_bytes_,
                                        _stream(stream, q)))


DECODE_SCRATCH_BYTES = 32 << 20  # MSA_DECODE_SCRATCH_BYTES


def sparse_attn_decode_noalloc(prob: Problem, q, k_cache, v_cache, sel, out, stream=None) -> None:
    """msa_sparse_attn_decode with the library's static scratch instead of a workspace (no
    allocation; calls that overlap on one device race)."""
    _check(lib().msa_sparse_attn_decode_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                _ptr(sel), _ptr(out), _stream(stream, q)))


def _lay(layout):
    return ctypes.byref(layout) if layout is not None else None


def index_scores_kv(prob: Problem, layout: KVLayout, q_idx, k_idx, scores, stream=None) -> None:
    _check(lib().msa_index_scores_kv(ctypes.byref(prob), _lay(layout), _ptr(q_idx), _ptr(k_idx), _ptr(scores),
                                     _stream(stream, q_idx)))


def block_topk_kv(prob: Problem, layout: KVLayout, scores, sel, stream=None) -> None:
    _check(lib().msa_block_topk_kv(ctypes.byref(prob), _lay(layout), _ptr(scores), _ptr(sel),
                                   _stream(stream, scores)))


def sparse_attn_prefill_kv(prob: Problem, layout: KVLayout, q, k, v, csr_offsets, csr_entries, sel, out, workspace,
                           workspace_bytes_: int, stream=None) -> None:
    _check(lib().msa_sparse_attn_prefill_kv(ctypes.byref(prob), _lay(layout), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(csr_offsets), _ptr(csr_entries), _ptr(sel), _ptr(out),
                                            _ptr(workspace), workspace_bytes_, _stream(stream, q)))


def sparse_attn_decode_kv(prob: Problem, layout: KVLayout, q, k_cache, v_cache, sel, out, workspace,
                          workspace_bytes_: int, stream=None) -> None:
    _check(lib().msa_sparse_attn_decode_kv(ctypes.byref(prob), _lay(layout), _ptr(q), _ptr(k_cache),
                                           _ptr(v_cache), _ptr(sel), _ptr(out), _ptr(workspace),
                                           workspace_bytes_, _stream(stream, q)))


def sparse_attn_prefill_train(prob: Problem, q, k, v, csr_offsets, csr_entries, sel, out, lse, block_mass,
                              workspace, workspace_bytes_: int, stream=None) -> None:
    _check(lib().msa_sparse_attn_prefill_train(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(csr_offsets),
                                               _ptr(csr_entries), _ptr(sel), _ptr(out), _ptr(lse), _ptr(block_mass),
                                               _ptr(workspace), workspace_bytes_, _stream(stream, q)))


def sparse_attn_backward(prob: Problem, q, k, v, out, dout, lse, sel, csr_offsets, csr_entries, dq, dk, dv,
                         workspace, workspace_bytes_: int, stream=None) -> None:
    _check(lib().msa_sparse_attn_backward(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                          _ptr(lse), _ptr(sel), _ptr(csr_offsets), _ptr(csr_entries), _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(workspace), workspace_bytes_,
                                          _stream(stream, q)))


def index_kl(prob: Problem, scores, sel, block_mass, sigma: float, loss, dscores, stream=None) -> None:
    _check(lib().msa_index_kl(ctypes.byref(prob), _ptr(scores), _ptr(sel), _ptr(block_mass), float(sigma),
                              _ptr(loss), _ptr(dscores), _stream(stream, scores)))


def index_backward(prob: Problem, q_idx, k_idx, csr_offsets, csr_entries, dscores, dq_idx, dk_idx, argmax,
                   workspace, workspace_bytes_: int, stream=None) -> None:
    _check(lib().msa_index_backward(ctypes.byref(prob), _ptr(q_idx), _ptr(k_idx), _ptr(csr_offsets),
                                    _ptr(csr_entries), _ptr(dscores), _ptr(dq_idx), _ptr(dk_idx), _ptr(argmax),
                                    _ptr(workspace), workspace_bytes_, _stream(stream, q_idx)))


def token_scores(prob: Problem, q_idx, k_idx, scores, stream=None) -> None:
    _check(lib().msa_token_scores(ctypes.byref(prob), _ptr(q_idx), _ptr(k_idx), _ptr(scores), _stream(stream, q_idx)))


def token_topk(prob: Problem, budget: int, scores, sel_tok, workspace, workspace_bytes_: int,
               stream=None) -> None:
    _check(lib().msa_token_topk(ctypes.byref(prob), int(budget), _ptr(scores), _ptr(sel_tok), _ptr(workspace),
                                workspace_bytes_, _stream(stream, scores)))


def token_workspace_bytes(prob: Problem, budget: int) -> int:
    return int(lib().msa_token_workspace_bytes(ctypes.byref(prob), int(budget)))


def token_attn_decode(prob: Problem, budget: int, q, k_cache, v_cache, sel_tok, out, workspace,
                      workspace_bytes_: int, stream=None) -> None:
    _check(lib().msa_token_attn_decode(ctypes.byref(prob), int(budget), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(sel_tok), _ptr(out), _ptr(workspace), workspace_bytes_,
                                       _stream(stream, q)))


def profiler_enable(on: bool) -> None:
    _check(lib().msa_profiler_enable(1 if on else 0))


def profiler_read(kernel: str | None = None, reset: bool = True):
    """(total device ms, launches) of `kernel` (None = all) since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().msa_profiler_read(kernel.encode() if kernel else None, ctypes.byref(ms), ctypes.byref(n),
                                   1 if reset else 0))
    return ms.value, n.value


def profiler_samples(kernel: str | None = None) -> list:
    """The individual launch durations (ms) of `kernel` (None = all) since the last reset."""
    n = ctypes.c_int64()
    name = kernel.encode() if kernel else None
    _check(lib().msa_profiler_samples(name, None, 0, ctypes.byref(n)))
    buf = (ctypes.c_float * max(n.value, 1))()
    _check(lib().msa_profiler_samples(name, buf, n.value, ctypes.byref(n)))
    return [float(buf[i]) for i in range(n.value)]


# ------------------------------------------------------------------ allocating helpers
@dataclass
class PrefillBuffers:
    scores: object
    sel: object
    csr_offsets: object
    csr_entries: object
    ws_invert: object
    ws_prefill: object
    out: object
    ws_select: object = None  # fused selection's workspace (scores is then None)


def alloc_prefill(prob: Problem, device="cuda", fused_selection: bool = False) -> PrefillBuffers:
    """Allocate (torch) every output and workspace of one prefill pass.  With
    fused_selection the pass selects blocks with msa_index_topk (no block-score matrix:
    bf16 queries and top-k <= 16)."""
    import torch
    S, T, Hkv, nb, k = prob.batch, prob.num_q, prob.num_kv_heads, prob.nb, prob.topk
    odt = torch.bfloat16 if prob.dtype == MSA_BF16 else torch.float32
    wi = max(workspace_bytes(prob, MSA_CALL_INVERT), 1)
    wp = max(workspace_bytes(prob, MSA_CALL_PREFILL), 1)
    ws_select = None
    if fused_selection:
        ws_select = torch.empty((max(workspace_bytes(prob, MSA_CALL_INDEX_TOPK), 1),), dtype=torch.uint8,
                                device=device)
    return PrefillBuffers(
        scores=None if fused_selection else torch.empty((S, Hkv, T, nb), dtype=torch.float32, device=device),
        sel=torch.empty((S, Hkv, T, k), dtype=torch.int32, device=device),
        csr_offsets=torch.empty((S, Hkv, nb + 1), dtype=torch.int32, device=device),
        csr_entries=torch.empty((S * Hkv * T * k,), dtype=torch.int32, device=device),
        ws_invert=torch.empty((wi,), dtype=torch.uint8, device=device),
        ws_prefill=torch.empty((wp,), dtype=torch.uint8, device=device),
        out=torch.empty((S, T, prob.num_heads, prob.head_dim), dtype=odt, device=device),
        ws_select=ws_select)


def run_prefill(prob: Problem, q, k, v, q_idx, k_idx, bufs: PrefillBuffers, stream=None) -> None:
    """The prefill pass: scores -> top-k (or the fused selection when bufs were allocated
    with fused_selection) -> inversion -> attention + merge."""
    if bufs.scores is None:
        index_topk(prob, q_idx, k_idx, bufs.sel, bufs.ws_select, bufs.ws_select.numel(), stream)
    else:
        index_scores(prob, q_idx, k_idx, bufs.scores, stream)
        block_topk(prob, bufs.scores, bufs.sel, stream)
    invert_selection(prob, bufs.sel, bufs.csr_offsets, bufs.csr_entries, bufs.ws_invert,
                     bufs.ws_invert.numel(), stream)
    sparse_attn_prefill(prob, q, k, v, bufs.csr_offsets, bufs.csr_entries, bufs.sel, bufs.out,
                        bufs.ws_prefill, bufs.ws_prefill.numel(), stream)


@dataclass
class DecodeBuffers:
    scores: object
    sel: object
    ws_decode: object
    out: object


def alloc_decode(prob: Problem, device="cuda") -> DecodeBuffers:
    import torch
    S, T, Hkv, nb, k = prob.batch, prob.num_q, prob.num_kv_heads, prob.nb, prob.topk
    odt = torch.bfloat16 if prob.dtype == MSA_BF16 else torch.float32
    wd = max(workspace_bytes(prob, MSA_CALL_DECODE), 1)
    return DecodeBuffers(
        scores=torch.empty((S, Hkv, T, nb), dtype=torch.float32, device=device),
        sel=torch.empty((S, Hkv, T, k), dtype=torch.int32, device=device),
        ws_decode=torch.empty((wd,), dtype=torch.uint8, device=device),
        out=torch.empty((S, T, prob.num_heads, prob.head_dim), dtype=odt, device=device))


def run_decode(prob: Problem, q, k_cache, v_cache, q_idx, k_idx, bufs: DecodeBuffers, stream=None) -> None:
    """One decode step: scores -> top-k -> query-centric split-K attention + merge."""
    index_scores(prob, q_idx, k_idx, bufs.scores, stream)
    block_topk(prob, bufs.scores, bufs.sel, stream)
    sparse_attn_decode(prob, q, k_cache, v_cache, bufs.sel, bufs.out, bufs.ws_decode,
                       bufs.ws_decode.numel(), stream)


def run_decode_kv(prob: Problem, layout: KVLayout, q, k_cache, v_cache, q_idx, k_idx, bufs: DecodeBuffers,
                  stream=None) -> None:
    """One decode step over ragged / paged caches (same stages as run_decode)."""
    index_scores_kv(prob, layout, q_idx, k_idx, bufs.scores, stream)
    block_topk_kv(prob, layout, bufs.scores, bufs.sel, stream)
    sparse_attn_decode_kv(prob, layout, q, k_cache, v_cache, bufs.sel, bufs.out, bufs.ws_decode,
                          bufs.ws_decode.numel(), stream)


@dataclass
class TrainBuffers:
    """Outputs and workspaces of one training step (forward with lse and teacher, main-branch
    backward, index KL and index backward)."""
    fwd: PrefillBuffers
    lse: object
    mass: object
    dq: object
    dk: object
    dv: object
    ws_bwd: object
    loss: object
    dscores: object
    dq_idx: object
    dk_idx: object
    argmax: object
    ws_ibwd: object


def alloc_train(prob: Problem, device="cuda") -> TrainBuffers:
    import torch
    S, T, N, H, Hkv, d, dI, k = (prob.batch, prob.num_q, prob.kv_len, prob.num_heads, prob.num_kv_heads,
                                 prob.head_dim, prob.index_dim, prob.topk)
    f32 = dict(dtype=torch.float32, device=device)
    return TrainBuffers(
        fwd=alloc_prefill(prob, device),
        lse=torch.empty((S, T, H), **f32), mass=torch.empty((S, Hkv, T, k), **f32),
        dq=torch.empty((S, T, H, d), **f32), dk=torch.empty((S, Hkv, N, d), **f32),
        dv=torch.empty((S, Hkv, N, d), **f32),
        ws_bwd=torch.empty((max(workspace_bytes(prob, MSA_CALL_BACKWARD), 1),), dtype=torch.uint8, device=device),
        loss=torch.empty((S, Hkv, T), **f32), dscores=torch.empty((S, Hkv, T, k), **f32),
        dq_idx=torch.empty((S, Hkv, T, dI), **f32), dk_idx=torch.empty((S, Hkv, N, dI), **f32),
        argmax=torch.full((S, Hkv, T, k), -1, dtype=torch.int32, device=device),
        ws_ibwd=torch.empty((max(workspace_bytes(prob, MSA_CALL_INDEX_BACKWARD), 1),), dtype=torch.uint8,
                            device=device))


def run_train_step(prob: Problem, q, k, v, q_idx, k_idx, dout, bufs: TrainBuffers, sigma: float = 0.0,
                   stream=None) -> None:
    """Forward (scores, top-k, inversion, attention with lse and teacher), then the main-branch
    backward for the upstream gradient dout, the index KL and the index-branch backward."""
    f = bufs.fwd
    index_scores(prob, q_idx, k_idx, f.scores, stream)
    block_topk(prob, f.scores, f.sel, stream)
    invert_selection(prob, f.sel, f.csr_offsets, f.csr_entries, f.ws_invert, f.ws_invert.numel(), stream)
    sparse_attn_prefill_train(prob, q, k, v, f.csr_offsets, f.csr_entries, f.sel, f.out, bufs.lse, bufs.mass,
                              f.ws_prefill, f.ws_prefill.numel(), stream)
    sparse_attn_backward(prob, q, k, v, f.out, dout, bufs.lse, f.sel, f.csr_offsets, f.csr_entries, bufs.dq,
                         bufs.dk, bufs.dv, bufs.ws_bwd, bufs.ws_bwd.numel(), stream)
    index_kl(prob, f.scores, f.sel, bufs.mass, sigma, bufs.loss, bufs.dscores, stream)
    index_backward(prob, q_idx, k_idx, f.csr_offsets, f.csr_entries, bufs.dscores, bufs.dq_idx, bufs.dk_idx,
                   bufs.argmax, bufs.ws_ibwd, bufs.ws_ibwd.numel(), stream)


@dataclass
class TokenBuffers:
    scores: object
    sel_tok: object
    ws: object
    out: object


def alloc_token_decode(prob: Problem, budget: int = 2048, device="cuda") -> TokenBuffers:
    import torch
    S, T, N, Hkv = prob.batch, prob.num_q, prob.kv_len, prob.num_kv_heads
    odt = torch.bfloat16
    return TokenBuffers(
        scores=torch.empty((S, Hkv, T, N), dtype=torch.float32, device=device),
        sel_tok=torch.empty((S, Hkv, T, budget), dtype=torch.int32, device=device),
        ws=torch.empty((max(token_workspace_bytes(prob, budget), 1),), dtype=torch.uint8, device=device),
        out=torch.empty((S, T, prob.num_heads, prob.head_dim), dtype=odt, device=device))


def run_token_decode(prob: Problem, q, k_cache, v_cache, q_idx, k_idx, bufs: TokenBuffers, budget: int = 2048,
                     stream=None) -> None:
    """Token-level decode step: token scores -> top-budget tokens -> attention over them."""
    token_scores(prob, q_idx, k_idx, bufs.scores, stream)
    token_topk(prob, budget, bufs.scores, bufs.sel_tok, bufs.ws, bufs.ws.numel(), stream)
    token_attn_decode(prob, budget, q, k_cache, v_cache, bufs.sel_tok, bufs.out, bufs.ws, bufs.ws.numel(), stream)


def run_prefill_kv(prob: Problem, layout: KVLayout, q, k, v, q_idx, k_idx, bufs: PrefillBuffers, stream=None) -> None:
    """Batched chunked prefill over ragged / paged caches (same stages as run_prefill)."""
    index_scores_kv(prob, layout, q_idx, k_idx, bufs.scores, stream)
    block_topk_kv(prob, layout, bufs.scores, bufs.sel, stream)
    invert_selection(prob, bufs.sel, bufs.csr_offsets, bufs.csr_entries, bufs.ws_invert, bufs.ws_invert.numel(),
                     stream)
    sparse_attn_prefill_kv(prob, layout, q, k, v, bufs.csr_offsets, bufs.csr_entries, bufs.sel, bufs.out,
                           bufs.ws_prefill, bufs.ws_prefill.numel(), stream)
