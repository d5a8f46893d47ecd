"""Host-side tests of the C ABI (CPU only; no kernel is launched).

The library must load, export every entry point declared in include/msa.h, and
reject bad arguments on the host before touching the device."""
import ctypes
import os
import re

import pytest

import block_sparse_long_06_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "msa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_hot_path_calls():
    names = _declared()
    for f in ("msa_index_scores", "msa_block_topk", "msa_invert_selection", "msa_sparse_attn_prefill",
              "msa_sparse_attn_decode"):
        assert f in names


def test_library_defines_every_kernel_launch_stub():
    """Every kernel the library launches has its host launch stub (a stub dropped by the
    host compiler pass leaves an undefined symbol that only loading would report)."""
    from block_sparse_long_06_amd import _build
    assert _build.undefined_kernel_stubs(msa.LIB_PATH) == []


def test_library_exports_every_declared_symbol():
    L = msa.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert set(_declared()) == set(msa.EXPORTED)


def _good(**kw):
    p = dict(batch=1, num_q=300, kv_len=1000, num_heads=8, num_kv_heads=2, head_dim=128, index_dim=64,
             topk=16, dtype=msa.MSA_BF16)
    p.update(kw)
    return msa.problem(**p)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(num_q=0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(num_q=1001), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(num_heads=7), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(topk=0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(softmax_scale=-1.0), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(softmax_scale=float("nan")), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(block_size=64), msa.MSA_ERR_UNSUPPORTED),
    (dict(topk=65), msa.MSA_ERR_UNSUPPORTED),
    (dict(kv_len=8192 * 128 + 1, num_q=1), msa.MSA_ERR_UNSUPPORTED),
    (dict(index_dim=48), msa.MSA_ERR_UNSUPPORTED),
    (dict(index_key_dtype=5), msa.MSA_ERR_INVALID_ARGUMENT),
    (dict(index_key_dtype=msa.MSA_FP8_E4M3, dtype=msa.MSA_F32), msa.MSA_ERR_UNSUPPORTED),
    (dict(num_q=1 << 20, kv_len=1 << 20, num_kv_heads=128, num_heads=128), msa.MSA_ERR_UNSUPPORTED),
])
def test_bad_problem_is_rejected_before_any_launch(kw, status):
    p = _good(**kw)
    with pytest.raises(msa.MSAError) as ei:
        msa.index_scores(p, 1, 1, 1, stream=0)
    assert ei.value.status == status
    assert msa.last_error_message() != ""


@pytest.mark.parametrize("kw", [dict(head_dim=96), dict(num_heads=6, num_kv_heads=2),
                                dict(num_heads=64, num_kv_heads=2)])
def test_main_branch_limits(kw):
    p = _good(**kw)
    with pytest.raises(msa.MSAError) as ei:
        msa.sparse_attn_decode(p, 1, 1, 1, 1, 1, 1, 1 << 40, stream=0)
    assert ei.value.status == msa.MSA_ERR_UNSUPPORTED
    assert msa.workspace_bytes(p, msa.MSA_CALL_DECODE) == 0


def test_null_pointers_are_rejected():
    p = _good()
    for call in (lambda: msa.index_scores(p, None, 1, 1, stream=0),
                 lambda: msa.index_scores(p, 1, 1, None, stream=0),
                 lambda: msa.block_topk(p, None, 1, stream=0),
                 lambda: msa.invert_selection(p, 1, None, 1, 1, 1 << 40, stream=0),
                 lambda: msa.sparse_attn_prefill(p, 1, 1, 1, 1, 1, 1, None, 1, 1 << 40, stream=0),
                 lambda: msa.sparse_attn_decode(p, 1, None, 1, 1, 1, 1, 1 << 40, stream=0)):
        with pytest.raises(msa.MSAError) as ei:
            call()
        assert ei.value.status == msa.MSA_ERR_INVALID_ARGUMENT
        assert "NULL" in msa.last_error_message()


def test_workspace_too_small_is_rejected():
    p = _good()
    need = msa.workspace_bytes(p, msa.MSA_CALL_PREFILL)
    assert need > 0
    with pytest.raises(msa.MSAError) as ei:
        msa.sparse_attn_prefill(p, 1, 1, 1, 1, 1, 1, 1, 1, need - 1, stream=0)
    assert ei.value.status == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    need_i = msa.workspace_bytes(p, msa.MSA_CALL_INVERT)
    with pytest.raises(msa.MSAError) as ei:
        msa.invert_selection(p, 1, 1, 1, 1, need_i - 1, stream=0)
    assert ei.value.status == msa.MSA_ERR_WORKSPACE_TOO_SMALL


def test_token_topk_needs_its_workspace():
    # per row: a histogram, a chunk table and up to 16384 candidates (key + position)
    p = _good(num_q=2, kv_len=300000)
    need = msa.token_workspace_bytes(p, 2048)
    rows = p.batch * p.num_kv_heads * p.num_q
    assert need >= rows * 2 * 16384 * 4
    with pytest.raises(msa.MSAError) as ei:
        msa.token_topk(p, 2048, 1, 1, 1, need - 1, stream=0)
    assert ei.value.status == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(msa.MSAError) as ei:
        msa.token_topk(p, 2048, 1, 1, None, need, stream=0)
    assert ei.value.status == msa.MSA_ERR_INVALID_ARGUMENT


def test_workspace_sizes_scale_with_partials():
    # prefill workspace holds T*Hkv*k*G partials of (d bf16 + 1 fp32)
    p = _good(num_q=1000, kv_len=1000)
    w = msa.workspace_bytes(p, msa.MSA_CALL_PREFILL)
    npart = 1000 * 2 * 16 * 4
    assert w >= npart * (128 * 2 + 4)
    assert w < npart * (128 * 2 + 4) * 1.2 + (1 << 20)
    assert msa.workspace_bytes(p, 99) == 0


def test_status_strings():
    assert msa.status_string(msa.MSA_OK) == "MSA_OK"
    assert msa.status_string(msa.MSA_ERR_WORKSPACE_TOO_SMALL) == "MSA_ERR_WORKSPACE_TOO_SMALL"
    assert msa.status_string(42) == "MSA_ERR_UNKNOWN"


def test_profiler_read_without_records():
    msa.profiler_enable(False)
    ms, n = msa.profiler_read(None)
    assert ms == 0.0 and n == 0
    assert msa.profiler_samples(None) == []
    assert msa.profiler_samples("idx_scores_mfma") == []


def _layout(kv_lens=1, block_table=None, stride=0, pages=0):
    lay = msa.KVLayout()
    lay.kv_lens = kv_lens
    lay.block_table = block_table
    lay.table_stride = stride
    lay.num_pages = pages
    return lay


@pytest.mark.parametrize("lay,kw,status", [
    (None, {}, msa.MSA_ERR_INVALID_ARGUMENT),                                    # no layout
    ("nolens", {}, msa.MSA_ERR_INVALID_ARGUMENT),                                # kv_lens NULL
    ("hugepool", {}, msa.MSA_ERR_UNSUPPORTED),                                    # pool beyond 2^40 elements
    ("shortstride", {}, msa.MSA_ERR_INVALID_ARGUMENT),                           # table_stride < nb
    ("nopages", {}, msa.MSA_ERR_INVALID_ARGUMENT),                               # num_pages < 1
])
def test_kv_layout_is_validated_on_the_host(lay, kw, status):
    p = _good(**dict(dict(num_q=1, kv_len=1000), **kw))
    layouts = {None: None, "nolens": _layout(kv_lens=None), "hugepool": _layout(block_table=1, stride=8, pages=1 << 30),
               "shortstride": _layout(block_table=1, stride=7, pages=10),   # nb = 8
               "nopages": _layout(block_table=1, stride=8, pages=0)}
    L = layouts[lay]
    for call in (lambda: msa.index_scores_kv(p, L, 1, 1, 1, stream=0),
                 lambda: msa.block_topk_kv(p, L, 1, 1, stream=0),
                 lambda: msa.sparse_attn_decode_kv(p, L, 1, 1, 1, 1, 1, 1, 1 << 40, stream=0),
                 lambda: msa.sparse_attn_prefill_kv(p, L, 1, 1, 1, 1, 1, 1, 1, 1, 1 << 40, stream=0)):
        with pytest.raises(msa.MSAError) as ei:
            call()
        assert ei.value.status == status
        assert msa.last_error_message() != ""


def test_kv_calls_reject_null_pointers_and_small_workspace():
    p = _good(num_q=1, kv_len=1000)
    L = _layout(block_table=1, stride=8, pages=3)
    with pytest.raises(msa.MSAError) as ei:
        msa.index_scores_kv(p, L, 1, None, 1, stream=0)
    assert ei.value.status == msa.MSA_ERR_INVALID_ARGUMENT
    need = msa.workspace_bytes(p, msa.MSA_CALL_DECODE)
    with pytest.raises(msa.MSAError) as ei:
        msa.sparse_attn_decode_kv(p, L, 1, 1, 1, 1, 1, 1, need - 1, stream=0)
    assert ei.value.status == msa.MSA_ERR_WORKSPACE_TOO_SMALL


def test_no_alloc_decode_is_validated_on_the_host():
    """Argument checks and the scratch-size limit come before any device call."""
    prob = msa.problem(16, 8, 1 << 20, 64, 8, 128, 64, 16)
    need = msa.workspace_bytes(prob, msa.MSA_CALL_DECODE)
    assert need > msa.DECODE_SCRATCH_BYTES
    L = msa.lib()
    p = ctypes.c_void_p(16)
    st = L.msa_sparse_attn_decode_noalloc(ctypes.byref(prob), p, p, p, p, p, None)
    assert st == msa.MSA_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in msa.last_error_message()
    small = msa.problem(16, 1, 1 << 20, 64, 8, 128, 64, 16)
    assert msa.workspace_bytes(small, msa.MSA_CALL_DECODE) <= msa.DECODE_SCRATCH_BYTES
    st = L.msa_sparse_attn_decode_noalloc(ctypes.byref(small), p, None, p, p, p, None)
    assert st == msa.MSA_ERR_INVALID_ARGUMENT
    st = L.msa_sparse_attn_decode_noalloc(ctypes.byref(_good(head_dim=96)), p, p, p, p, p, None)
    assert st == msa.MSA_ERR_UNSUPPORTED

