// attention_mfma.hip -- a4 for bf16 prefill on gfx950 matrix cores: the Outer-Gather-Q
// kernel of page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比", section
// Kernel 创新：Outer Gather Q (the KV block is the outer loop; every query that chose
// it is gathered and processed against one on-chip copy), computing the exact
// block-restricted softmax of section 第二步：精算.
//
// Work item = one (sequence, group, KV block) and up to R = 128 / G query rows of its
// inverted list (ascending rows).  M-rows = (query row, head) pairs, head fastest,
// so one query row's G heads are G consecutive M-rows; each of the 4 waves owns 32.
//
//  * K (128 x d) is staged in LDS row-major with a 16-byte row pad; V is staged
//    TRANSPOSED (d x 128, 8-byte row pad) so a lane can fetch 4 consecutive keys of
//    one head dimension with one 8-byte read.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys, B = 32 M-rows): the
//    output column of lane n = lane % 32 is one M-row, so the row max and row sum
//    are in-lane over 64 values plus one exchange with lane ^ 32.
//  * P = exp2(s - m) stays in registers: accumulator registers 8p..8p+7 of key tile
//    kt hold 8 keys of the lane's M-row, exactly the 8 k-elements a lane supplies
//    to a B operand.  So O^T = V^T P^T is accumulated with k-step = (kt, p) whose
//    key order is the accumulator's row order; the V^T A-operand reads the same
//    keys from the transposed LDS copy (two runs of 4 consecutive keys).
//  * 32x32 accumulator layout: output row i is held by lane half (i % 8) / 4 in
//    register 4 * (i / 8) + i % 4.  The QK contraction visits head dims in the
//    order lane half h, k-step s -> dims [64 h + 8 s, +8) (any order works as long
//    as A and B agree), letting each lane read one contiguous 128-byte half row.
//
// Output: per (row, slot, head) partial O (bf16, normalised) and lse (fp32, natural
// log), merged by lse_merge.
#include "msa_internal.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlk = 128;
constexpr int kKPad = 16;  // bytes of pad per K row
constexpr int kVPad = 8;   // bytes of pad per V^T row

template <int DH>
struct OgqLds {
  static constexpr int KROW = DH * 2 + kKPad;
  static constexpr int VROW = kBlk * 2 + kVPad;
  unsigned char k[kBlk * KROW];
  unsigned char vt[DH * VROW];
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

template <int DH>
__device__ __forceinline__ void stage_kv(OgqLds<DH>& L, const uint16_t* kb, const uint16_t* vb, int nvalid) {
  // K: 16-byte chunks, row-major copy with a pad
  constexpr int CPR = DH / 8;
#pragma unroll
  for (int u = 0; u < kBlk * CPR / 256; ++u) {
    const int c = threadIdx.x + 256 * u;
    const int row = c / CPR, col = c % CPR;
    const uint4 val = row < nvalid ? *reinterpret_cast<const uint4*>(kb + row * DH + col * 8)
                                   : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(&L.k[row * OgqLds<DH>::KROW + col * 16]) = val;
  }
  // V^T: thread = (4 consecutive keys, 8 consecutive dims); 4x8 transpose in registers
  const int kg = threadIdx.x & 31;
#pragma unroll
  for (int u = 0; u < DH / 64; ++u) {
    const int dc = (threadIdx.x >> 5) + 8 * u;
    uint32_t w[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 4 * kg + i;
      const uint4 x = key < nvalid ? *reinterpret_cast<const uint4*>(vb + key * DH + dc * 8)
                                   : make_uint4(0u, 0u, 0u, 0u);
      w[i][0] = x.x; w[i][1] = x.y; w[i][2] = x.z; w[i][3] = x.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t k0 = (w[0][e >> 1] >> sh) & 0xFFFFu, k1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t k2 = (w[2][e >> 1] >> sh) & 0xFFFFu, k3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
      uint2 o;
      o.x = k0 | (k1 << 16);
      o.y = k2 | (k3 << 16);
      *reinterpret_cast<uint2*>(&L.vt[(dc * 8 + e) * OgqLds<DH>::VROW + kg * 8]) = o;
    }
  }
}

template <int DH, int G>
__global__ void __launch_bounds__(256, 2) ogq_mfma(Dims D, const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   const int4* __restrict__ wl,
                                                   const int* __restrict__ n_items,
                                                   const int32_t* __restrict__ entries,
                                                   float* __restrict__ part_lse,
                                                   uint16_t* __restrict__ part_o) {
  constexpr int KS = DH / 16;  // k-steps of the QK contraction
  constexpr int DT = DH / 32;  // output dim tiles of PV
  constexpr int RPW = 32 / G;  // query rows per wave
  __shared__ OgqLds<DH> L;

  // XCD-aware item order: the 8 XCDs receive workgroups round-robin, so give each
  // XCD a contiguous range of items (consecutive items share a KV block).
  const int n = *n_items;
  const int per_xcd = (n + 7) / 8;
  const int slot_in_xcd = blockIdx.x >> 3;
  const int item = (blockIdx.x & 7) * per_xcd + slot_in_xcd;
  if (slot_in_xcd >= per_xcd || item >= n) return;

  const int4 w = wl[item];
  const int64_t sg = w.x / D.nb;
  const int b = w.x % D.nb;
  const int s = (int)(sg / D.Hkv), g = (int)(sg % D.Hkv);
  const int j0 = b * kBlk;
  const int nvalid = min(kBlk, D.N - j0);
  stage_kv<DH>(L, k + (sg * D.N + j0) * DH, v + (sg * D.N + j0) * DH, nvalid);

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int nl = lane & 31;
  const int rr = wave * RPW + nl / G;  // local query row of this lane's M-row
  const int hh = nl % G;               // head within the group
  const bool row_ok = rr < w.z;
  const int e = entries[w.y + (row_ok ? rr : 0)];
  const int t = e / D.k;
  const int slot = e % D.k;
  const int p = D.pos0 + t;

  // B operand of S^T: this lane's M-row, head dims [64h + 8ks, +8)
  bf16x8 qf[KS];
  {
    const uint16_t* qp = q + (((int64_t)s * D.T + t) * D.H + g * G + hh) * DH + (DH / 2) * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 8 * ks);
  }
  __syncthreads();
  const bool wave_live = wave * RPW < w.z;
  if (!wave_live) return;  // no rows for this wave (no later barrier)

  // S^T = K Q^T for the 4 key tiles
  f32x16 sacc[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    sacc[kt] = f32x16{};
    const unsigned char* arow = &L.k[(kt * 32 + nl) * OgqLds<DH>::KROW + DH * h];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 16 * ks);
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kt], 0, 0, 0);
    }
  }
  // scale into log2 units, causal mask inside the own block, row max
  const float sc = D.scale * kLog2e;
  const bool need_mask = __ballot(row_ok && p < j0 + kBlk - 1) != 0ull;
  float m = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = sacc[kt][r] * sc;
      if (need_mask) {
        const int j = j0 + kt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (j > p) x = -INFINITY;
      }
      sacc[kt][r] = x;
      m = fmaxf(m, x);
    }
  }
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  // P = exp2(s - m); row sum in fp32; P packed to bf16 as PV B-operands
  float l = 0.0f;
  bf16x8 pf[4][2];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = exp2f(sacc[kt][8 * pp + 2 * i] - m);
        const float c = exp2f(sacc[kt][8 * pp + 2 * i + 1] - m);
        l += a + c;
        pk[i] = pack_bf16x2(a, c);
      }
      pf[kt][pp] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
  }
  l += __shfl_xor(l, 32, 64);

  // O^T = V^T P^T
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int kb0 = (kt * 32 + 16 * pp + 4 * h) * 2;  // byte offset of the first key run
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const unsigned char* vrow = &L.vt[(dt * 32 + nl) * OgqLds<DH>::VROW];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + kb0);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + kb0 + 16);
        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kt][pp], oacc[dt], 0, 0, 0);
      }
    }
  }

  if (!row_ok) return;
  const int64_t pidx = (((int64_t)s * D.T + t) * D.Hkv + g) * D.k + slot;
  const float inv = 1.0f / l;
  uint16_t* op = part_o + (pidx * G + hh) * DH + 4 * h;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      uint2 o;
      o.x = pack_bf16x2(oacc[dt][4 * qd] * inv, oacc[dt][4 * qd + 1] * inv);
      o.y = pack_bf16x2(oacc[dt][4 * qd + 2] * inv, oacc[dt][4 * qd + 3] * inv);
      *reinterpret_cast<uint2*>(op + dt * 32 + 8 * qd) = o;
    }
  }
  if (h == 0) part_lse[pidx * G + hh] = (m + log2f(l)) * kLn2;
}

template <int DH, int G>
hipError_t launch_t(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int4* wl,
                    const int* n_items, int64_t grid, const int32_t* entries, float* part_lse,
                    uint16_t* part_o, hipStream_t st) {
  LaunchScope scope("ogq_mfma", st);
  hipLaunchKernelGGL((ogq_mfma<DH, G>), dim3((unsigned)grid), dim3(256), 0, st, D, q, k, v, wl, n_items,
                     entries, part_lse, part_o);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_dh(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int4* wl,
                     const int* n_items, int64_t grid, const int32_t* entries, float* part_lse,
                     uint16_t* part_o, hipStream_t st) {
  switch (D.G) {
    case 1: return launch_t<DH, 1>(D, q, k, v, wl, n_items, grid, entries, part_lse, part_o, st);
    case 2: return launch_t<DH, 2>(D, q, k, v, wl, n_items, grid, entries, part_lse, part_o, st);
    case 4: return launch_t<DH, 4>(D, q, k, v, wl, n_items, grid, entries, part_lse, part_o, st);
    case 8: return launch_t<DH, 8>(D, q, k, v, wl, n_items, grid, entries, part_lse, part_o, st);
    default: return launch_t<DH, 16>(D, q, k, v, wl, n_items, grid, entries, part_lse, part_o, st);
  }
}

}  // namespace

bool ogq_mfma_supported(const Dims& D) {
  return D.dtype == MSA_BF16 && (D.d == 64 || D.d == 128) &&
         (D.G == 1 || D.G == 2 || D.G == 4 || D.G == 8 || D.G == 16);
}

int ogq_mfma_rows_per_item(const Dims& D) { return 128 / D.G; }

hipError_t launch_ogq_mfma(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int4* wl, const int* n_items, int64_t ub, const int32_t* entries,
                           float* part_lse, uint16_t* part_o, hipStream_t st) {
  const int64_t grid = (ub + 7) / 8 * 8 + 8;  // >= 8 * ceil(n_items / 8) for any n_items <= ub
  if (D.d == 64) return launch_dh<64>(D, q, k, v, wl, n_items, grid, entries, part_lse, part_o, st);
  return launch_dh<128>(D, q, k, v, wl, n_items, grid, entries, part_lse, part_o, st);
}

}  // namespace msa
