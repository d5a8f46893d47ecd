// decode_attn.hip -- a6: the decode main branch of page "MSA 稀疏注意力三国杀：NSA / DSA /
// MoBA / MSA 四方案深度对比", section 第二步：精算 (exact softmax attention over the selected
// blocks only), in the query-centric split-K form: every (sequence, query row, group,
// slot) is one work item that attends the row's G heads to ONE selected 128-key block and
// writes that slot's partial (normalised O and its log-sum-exp); the LSE merge combines a
// row's slots.
//
// At decode the items hold one row each, so the matrix-core prefill kernel (built for
// hundreds of rows per staged block) would stage 64 KB of K/V per row through LDS with
// eight waves and compute with one.  This kernel is sized for that shape instead: one
// 256-thread workgroup per item, ~39 KB of LDS, so four items run per CU and their block
// reads overlap.
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 dims read straight from
//    global memory into registers (wave w owns keys 32 w .. 32 w + 31), B = the G query
//    heads (columns >= G are zero).  Output lane l holds keys 4 (l / 16) + {0..3} of a
//    16-key tile for head l % 16, so the row statistics need only lane exchanges within a
//    wave and one small LDS table across the 4 waves.
//  * The contraction pairs A and B element by element in the same (lane group, element)
//    order, so any assignment of dims (QK) or keys (PV) to that order is valid.  QK uses
//    contiguous 16-byte runs; PV uses the key order in which S^T left P in the registers:
//    elements 0..3 = keys 4 g + {0..3} of the chunk's first 16-key tile, 4..7 = the same
//    of its second.
//  * V goes to LDS with 16-byte direct global -> LDS loads, rows padded to DH * 2 + 16
//    bytes; the V^T operand of O^T = V^T P^T is read with ds_read_b64_tr_b16, two reads
//    per operand (rows 4 g and 16 + 4 g of the chunk).  The waves split the output dims
//    (DH / 4 each) and read the four chunks' P operands from LDS.
#include "msa_internal.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kB = 128;  // keys per block

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// 16x16x32 A operand read transposed out of a row-major bf16 tile: lane (n = lane % 16,
// group g = lane / 16) gets column col0 + n of rows r0(g) + {0..3} (elements 0..3) and
// r1(g) + {0..3} (elements 4..7).  ds_read_b64_tr_b16 works in groups of 16 lanes:
// destination lane i receives, as element j, the (i % 4)-th 16-bit value of the 8 bytes
// addressed by source lane 4 j + i / 4; so source lane 4 j + q addresses row r + j at
// columns col0 + 4 q .. + 3.
__device__ __forceinline__ bf16x8 tr16_operand(const unsigned char* tile, int row_bytes, int r0, int r1, int col0,
                                               int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  const int sl = lane & 15, j = sl >> 2, q = sl & 3;
  const int col = col0 + 4 * q;
  const lds_u8* t = (const lds_u8*)tile;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (r0 + j) * row_bytes + col * 2));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (r1 + j) * row_bytes + col * 2));
  const s16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, ab);
}

template <int DH>
__global__ void __launch_bounds__(256) decode_attn(Dims D, const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   const int32_t* __restrict__ sel, float* __restrict__ part_lse,
                                                   uint16_t* __restrict__ part_o) {
  // padded V row: a transposing read (16 rows x 32 bytes per 16-lane group) then hits
  // each bank twice, the minimum for its 512 bytes
  constexpr int VROW = DH * 2 + 16;
  constexpr int VB = kB * VROW;                // bytes of the V tile
  constexpr int NINST = VB / 1024;             // 1 KB direct-load instructions (wave w: w, w + 4, ...)
  static_assert(NINST * 1024 == VB, "whole direct-load instructions");
  constexpr int KS = DH / 32;                  // k-steps of the QK contraction
  constexpr int DTW = DH / 64;                 // 16-dim output tiles per wave
  __shared__ __attribute__((aligned(16))) unsigned char vt[VB];
  __shared__ u32x4 pb[4][64];                  // each wave's P operand (its 32-key chunk)
  __shared__ float red[2][4][16];              // per wave and head: max, then sum

  // item = partial index ((s * T + t) * Hkv + g) * k + slot; sel is [S, Hkv, T, k]
  const int64_t item = blockIdx.x;
  const int64_t pidx = item;
  const int slot = (int)(item % D.k);
  const int64_t row = item / D.k;  // (s * T + t) * Hkv + g
  const int g = (int)(row % D.Hkv);
  const int64_t st_ = row / D.Hkv;  // s * T + t
  const int t = (int)(st_ % D.T);
  const int s = (int)(st_ / D.T);
  const int b = sel[(((int64_t)s * D.Hkv + g) * D.T + t) * D.k + slot];
  if (b < 0 || b >= D.nb) return;  // an empty slot (uniform across the workgroup)

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;   // key / head / dim index within a 16-wide tile
  const int gl = lane >> 4;  // lane group
  const int G = D.G;
  const int j0 = b * kB;
  const int p = seq_pos0(D, s) + t;
  const int64_t kv0 = kv_row(D, s, g, j0, DH);  // a block is contiguous; an invalid page reads as 0
  const int nvalid = kv0 < 0 ? 0 : min(kB, seq_len(D, s) - j0);

  // V -> LDS (direct loads; pad slots re-read a chunk of the same row, never read back;
  // rows past the end repeat row 0: their keys are masked causally, so P = 0 there).  K and
  // V are read once per step, with non-temporal loads: after the index stream's
  // non-temporal sweep of the index keys, ordinary loads here measured 50 against 35 us.
  if (kv0 >= 0) {
    typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
    for (int u = wave; u < NINST; u += 4) {
      const int off = u * 1024;
      const int x = off + 16 * lane;
      const int r = x / VROW, o = x % VROW;
      const int c = o < DH * 2 ? o / 16 : 0;
      const int rr = r < nvalid ? r : 0;
      __builtin_amdgcn_global_load_lds(v + kv0 + (int64_t)rr * DH + c * 8, (lds_void*)(vt + off), 16, 0, 2);
    }
  } else {
    for (int i = threadIdx.x; i < VB / 16; i += 256) reinterpret_cast<u32x4*>(vt)[i] = u32x4{0u, 0u, 0u, 0u};
  }

  // K (A operands, straight to registers) and Q (B operands)
  bf16x8 ka[2][KS], qb[KS];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int key = 32 * wave + 16 * tt + n;
    const int rr = key < nvalid ? key : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ka[tt][ks] = kv0 >= 0 ? __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                  k + kv0 + (int64_t)rr * DH + 32 * ks + 8 * gl)))
                            : bf16x8{};
  }
  const bool head_ok = n < G;
  const uint16_t* qp = q + ((st_ * D.H) + (int64_t)g * G + (head_ok ? n : 0)) * DH + 8 * gl;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qb[ks] = head_ok ? *reinterpret_cast<const bf16x8*>(qp + 32 * ks) : bf16x8{};

  // S^T for the wave's two 16-key tiles; causal mask (keys j > p)
  f32x4 sacc[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    sacc[tt] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tt][ks], qb[ks], sacc[tt], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (j0 + 32 * wave + 16 * tt + 4 * gl + i > p) sacc[tt][i] = -INFINITY;
  }
  const float sc = D.scale * kLog2e;
  float mx = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[tt][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (gl == 0) red[0][wave][n] = mx;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0][0][n], red[0][1][n]), fmaxf(red[0][2][n], red[0][3][n]));
  const float msc = m * sc;  // the block always holds a key <= p, so m is finite

  float l = 0.0f;
  uint32_t pk[4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = __builtin_amdgcn_exp2f(fmaf(sacc[tt][i], sc, -msc));
      l += e[i];
    }
    pk[2 * tt] = pack_bf16x2(e[0], e[1]);
    pk[2 * tt + 1] = pack_bf16x2(e[2], e[3]);
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (gl == 0) red[1][wave][n] = l;
  pb[wave][lane] = u32x4{pk[0], pk[1], pk[2], pk[3]};
  __syncthreads();  // also completes the V direct loads (the compiler waits for them)
  l = red[1][0][n] + red[1][1][n] + red[1][2][n] + red[1][3][n];

  // O^T = V^T P^T for this wave's output dims, over the four 32-key chunks
  const float inv = 1.0f / l;
#pragma unroll
  for (int dl = 0; dl < DTW; ++dl) {
    const int dt = wave * DTW + dl;
    f32x4 oacc = f32x4{};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 a = tr16_operand(vt, VROW, 32 * c + 4 * gl, 32 * c + 16 + 4 * gl, 16 * dt, lane);
      const bf16x8 bp = __builtin_bit_cast(bf16x8, pb[c][lane]);
      oacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp, oacc, 0, 0, 0);
    }
    // lane holds O^T[dims 16 dt + 4 gl + {0..3}][head n]
    if (head_ok) {
      uint2 o;
      o.x = pack_bf16x2(oacc[0] * inv, oacc[1] * inv);
      o.y = pack_bf16x2(oacc[2] * inv, oacc[3] * inv);
      *reinterpret_cast<uint2*>(part_o + (pidx * G + n) * DH + 16 * dt + 4 * gl) = o;
    }
  }
  if (wave == 0 && gl == 0 && head_ok) part_lse[pidx * G + n] = (msc + __builtin_amdgcn_logf(l)) * kLn2;
}

}  // namespace

bool decode_attn_supported(const Dims& D) {
  return D.dtype == MSA_BF16 && (D.d == 64 || D.d == 128) &&
         (D.G == 1 || D.G == 2 || D.G == 4 || D.G == 8 || D.G == 16);
}

hipError_t launch_decode_attn(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* sel, float* part_lse, uint16_t* part_o, hipStream_t st) {
  const int64_t n = (int64_t)D.S * D.T * D.Hkv * D.k;
  if (n <= 0) return hipSuccess;
  if (n >= (1ll << 31)) return hipErrorInvalidValue;
  LaunchScope scope("decode_attn", st);
  if (D.d == 128)
    hipLaunchKernelGGL((decode_attn<128>), dim3((unsigned)n), dim3(256), 0, st, D, q, k, v, sel, part_lse, part_o);
  else
    hipLaunchKernelGGL((decode_attn<64>), dim3((unsigned)n), dim3(256), 0, st, D, q, k, v, sel, part_lse, part_o);
  return hipGetLastError();
}

}  // namespace msa
