"""Seeded synthetic inputs for MSA, shared by the GPU tests, the oracle tests and the bench.

This module holds input generation only -- none of the attention method's
arithmetic.  Every element is a pure function of (seed, tensor id, flat index):

    value = TABLE[h16(seed, tensor_id, flat_index)]            (iid N(0,1))

* h16 is the top 16 bits of the SplitMix64 generator (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014): the stream
  key is mix64(seed * 256 + tensor_id) and the i-th output is
  mix64(key + (i + 1) * 0x9E3779B97F4A7C15), mix64 being the published
  variant-13 finaliser (shifts 30/27/31).
* TABLE[u] = Phi^-1((u + 0.5) / 65536), the standard-normal quantile at 65,536
  mid-points, computed once on the host in float64 and rounded to float32.

The device generator (``synth_dev.hip`` -> ``libmsa_synth.so``) implements the
same hash and reads the same table, so host and device agree bit for bit.
Structure (index keys with sink / needle / recent-band boosts) is added in
float32 and rounded once to the storage dtype (bf16 round-to-nearest-even; for
1-byte index keys OCP E4M3, round-to-nearest-even, saturating at 448).

Structured index inputs (the emergent head patterns: a diagonal band of recent
context, a leftmost sink column and per-group stripes at other distances):
* boost channel: coordinate 0 of every index query is 1.0; coordinate 0 of every
  index key in a boosted block (block 0 and 8 "needle" blocks per (sequence,
  group)) gets +boost, so those blocks' scores shift by exactly +boost;
* recent band: coordinates 1..16 carry 8 rotary planes a*(cos, sin)(theta_i * x)
  at absolute position x, theta_i = 2*pi / (1024 * 2**(i/2)), a**2 = band_a2,
  so the q.k contribution is band_a2 * sum_i cos(theta_i * (p - j)).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_DEV_SRC = os.path.join(_HERE, "synth_dev.hip")
_DEV_LIB = os.path.join(_HERE, "libmsa_synth.so")

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)

TID_Q, TID_K, TID_V, TID_QI, TID_KI, TID_NEEDLE, TID_ROWS, TID_DOUT = 1, 2, 3, 4, 5, 6, 7, 9
KIND_IID, KIND_QIDX, KIND_KIDX = 0, 1, 2
F32, BF16, FP8 = 0, 1, 2   # FP8: OCP E4M3 (index keys only)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor_id: int) -> np.uint64:
    with np.errstate(over="ignore"):
        base = np.uint64(seed) * np.uint64(256) + np.uint64(tensor_id)
    return _mix64(np.array([base], dtype=np.uint64))[0]


def h16(seed: int, tensor_id: int, flat_index) -> np.ndarray:
    """Top 16 bits of the (flat_index)-th SplitMix64 output of stream (seed, tensor_id)."""
    key = stream_key(seed, tensor_id)
    i = np.asarray(flat_index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + (i + np.uint64(1)) * GOLDEN
    return (_mix64(z) >> np.uint64(48)).astype(np.int64)


_TABLE = None


def normal_table() -> np.ndarray:
    """65,536 float32 standard-normal quantiles at (u + 0.5) / 65536."""
    global _TABLE
    if _TABLE is None:
        from scipy.special import ndtri
        u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _TABLE = ndtri(u).astype(np.float32)
    return _TABLE


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even, returning the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def band_table(length: int, band_a2: float) -> np.ndarray:
    """[length, 16] float32: a*cos(theta_i x), a*sin(theta_i x) for planes i = 0..7."""
    a = np.sqrt(band_a2)
    x = np.arange(length, dtype=np.float64)[:, None]
    i = np.arange(8, dtype=np.float64)[None, :]
    theta = 2.0 * np.pi / (1024.0 * 2.0 ** (i / 2.0))
    out = np.empty((length, 16), dtype=np.float64)
    out[:, 0::2] = a * np.cos(theta * x)
    out[:, 1::2] = a * np.sin(theta * x)
    return out.astype(np.float32)


def needle_blocks(seed: int, S: int, Hkv: int, nb: int, count: int = 8) -> np.ndarray:
    """[S, Hkv, count] distinct block ids in [1, nb-1] per (sequence, group), drawn from
    stream (seed, TID_NEEDLE) by rejection of repeats."""
    out = np.zeros((S, Hkv, count), dtype=np.int64)
    if nb <= 1:
        return out
    count = min(count, nb - 1)
    for s in range(S):
        for g in range(Hkv):
            got = []
            i = 0
            base = (s * Hkv + g) << 20
            while len(got) < count:
                v = int(h16(seed, TID_NEEDLE, base + i)[()]) * 65536 + int(h16(seed, TID_NEEDLE, base + i + (1 << 19))[()])
                b = 1 + v % (nb - 1)
                if b not in got:
                    got.append(b)
                i += 1
            out[s, g, :count] = got
    return out


@dataclass
class TensorSpec:
    """A generated tensor of logical shape [S, A, L, D] (flat row-major index)."""
    shape: tuple
    seed: int
    tensor_id: int
    dtype: int = BF16
    kind: int = KIND_IID
    pos_offset: int = 0            # absolute position of row l is pos_offset + l
    boost: float = 0.0             # KIND_KIDX: added to coordinate 0 in boosted blocks
    block: int = 128               # block size for the boost mask
    boost_mask: np.ndarray = None  # [S, A, nbb] uint8, KIND_KIDX only
    band: np.ndarray = None        # [max_pos, 16] float32 or None (no band)
    extra: dict = field(default_factory=dict)


def values_at(spec: TensorSpec, flat: np.ndarray) -> np.ndarray:
    """Float32 values (before storage rounding) of the elements at flat indices."""
    flat = np.asarray(flat, dtype=np.int64)
    S, A, L, D = spec.shape
    c = flat % D
    l = (flat // D) % L
    a = (flat // (D * L)) % A
    s = flat // (D * L * A)
    v = normal_table()[h16(spec.seed, spec.tensor_id, flat)].astype(np.float32)
    if spec.kind == KIND_QIDX:
        v = np.where(c == 0, np.float32(1.0), v)
        if spec.band is not None:
            inb = (c >= 1) & (c <= 16)
            pos = spec.pos_offset + l
            bv = spec.band[np.where(inb, pos, 0), np.where(inb, c - 1, 0)]
            v = np.where(inb, bv, v)
    elif spec.kind == KIND_KIDX:
        if spec.boost_mask is not None:
            blk = (spec.pos_offset + l) // spec.block
            m = spec.boost_mask[s, a, blk].astype(bool) & (c == 0)
            v = np.where(m, (v + np.float32(spec.boost)).astype(np.float32), v)
        if spec.band is not None:
            inb = (c >= 1) & (c <= 16)
            pos = spec.pos_offset + l
            bv = spec.band[np.where(inb, pos, 0), np.where(inb, c - 1, 0)]
            v = np.where(inb, bv, v)
    return v.astype(np.float32)


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 codes (uint8): round to nearest even, magnitudes beyond the
    largest finite value (448) saturate to it.  Finite inputs only.  Storage encoding of
    the generator (the device generator implements the same steps)."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    sign = ((u >> np.uint32(24)) & np.uint32(0x80)).astype(np.uint32)
    a = np.abs(x)
    au = a.view(np.uint32)
    # normal range: 3 mantissa bits kept, round half to even on the 20 dropped bits
    e = (au >> np.uint32(23)).astype(np.int64) - 127
    mant = (au & np.uint32(0x7FFFFF)).astype(np.int64)
    keep = mant >> 20
    rem = mant & 0xFFFFF
    up = (rem > 0x80000) | ((rem == 0x80000) & ((keep & 1) == 1))
    keep = keep + up
    e = np.where(keep == 8, e + 1, e)
    keep = np.where(keep == 8, 0, keep)
    normal = np.minimum(((e + 7) << 3) | keep, 0x7E)
    # below the smallest normal (2^-6): multiples of 2^-9, rounded half to even
    sub = np.rint(a.astype(np.float64) * 512.0).astype(np.int64)
    code = np.where(a < np.float32(0.015625), sub, normal)
    code = np.where(a >= np.float32(448.0), 0x7E, code)
    return (code.astype(np.uint32) | sign).astype(np.uint8)


def host_tensor(spec: TensorSpec) -> np.ndarray:
    """The whole tensor on the host, in storage form (float32 array, uint16 bf16 bits,
    or uint8 E4M3 codes)."""
    n = int(np.prod(spec.shape))
    v = values_at(spec, np.arange(n, dtype=np.int64)).reshape(spec.shape)
    if spec.dtype == F32:
        return v
    return f32_to_bf16_bits(v) if spec.dtype == BF16 else f32_to_e4m3(v)


# ------------------------------------------------------------------ device side
_dev = None


def build_device(force: bool = True) -> str:
    if force or not os.path.exists(_DEV_LIB):
        tmp = _DEV_LIB + ".tmp%d" % os.getpid()
        cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               _DEV_SRC, "-o", tmp]
        subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
        os.replace(tmp, _DEV_LIB)
    return _DEV_LIB


def _load_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(_DEV_LIB):
            raise RuntimeError("libmsa_synth.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_DEV_LIB)
        P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.synth_fill.argtypes = [P, i32, i64, i64, i64, i64, ctypes.c_uint64, i32, P, i32,
                                   i64, ctypes.c_float, i32, P, i64, P, P]
        lib.synth_fill.restype = i32
        _dev = lib
    return _dev


def device_tensor(spec: TensorSpec, device="cuda"):
    """Generate the tensor directly in device memory (torch tensor of float32, bfloat16 or
    float8_e4m3fn).

    Bit-identical to host_tensor(spec).  Small side tables (the normal table, the
    band table, the boost mask) are copied up; the bulk never crosses PCIe."""
    import torch
    lib = _load_dev()
    S, A, L, D = spec.shape
    tdt = {F32: torch.float32, BF16: torch.bfloat16, FP8: torch.float8_e4m3fn}[spec.dtype]
    out = torch.empty((S, A, L, D), dtype=tdt, device=device)
    table = torch.from_numpy(normal_table()).to(device)
    band = torch.from_numpy(np.ascontiguousarray(spec.band)).to(device) if spec.band is not None else None
    mask = None
    nbb = 0
    if spec.boost_mask is not None:
        mask = torch.from_numpy(np.ascontiguousarray(spec.boost_mask, dtype=np.uint8)).to(device)
        nbb = spec.boost_mask.shape[-1]
    stream = torch.cuda.current_stream(out.device).cuda_stream
    rc = lib.synth_fill(out.data_ptr(), spec.dtype, S, A, L, D, spec.seed, spec.tensor_id,
                        table.data_ptr(), spec.kind, spec.pos_offset, float(spec.boost), spec.block,
                        mask.data_ptr() if mask is not None else None, nbb,
                        band.data_ptr() if band is not None else None, ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError("synth_fill failed with HIP error %d" % rc)
    # keep side tables alive until the fill has run
    torch.cuda.current_stream(out.device).synchronize()
    return out
