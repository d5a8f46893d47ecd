// index_scores_mfma.hip -- a1 for bf16 prefill on gfx950 matrix cores.
// Computes the index scores of page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA
// 四方案深度对比", section 第一步：粗筛 items 1-2 (token scores, max over each 128-token
// block), causal inside the query's own block.
//
// Work unit (one workgroup, 4 waves): 512 consecutive query rows of one
// (sequence, group) x a chunk of up to kChunk key blocks.  Each wave owns 128
// queries as four 32-query MFMA B-operands held in registers for the whole unit,
// so each key fragment read from LDS feeds four MFMAs.  Key blocks (128 keys x dI
// bf16) are staged through LDS, double buffered, with a 16-byte row pad so the
// per-lane 16-byte reads are bank-conflict free.
//
// v_mfma_f32_32x32x16_bf16 with A = 32 keys, B = 32 queries: output column
// n = lane % 32 is one query, so a lane's 16 accumulators are 16 keys of ONE
// query and the block max is an in-register max3 chain plus one exchange with
// lane ^ 32 (which holds the other 16 keys of each 32-key tile).  Key tile kt-1 is
// reduced only after the MFMAs of tile kt are issued, so the max chain overlaps the
// matrix core.  The causal mask is applied only in blocks that reach a query's
// position (a separate instantiation of the block body).  Output row i of the
// 32x32 tile lives in lane half (i % 8) / 4, register 4 * (i / 8) + i % 4.  The
// contraction over dI may visit the index dimensions in any order as long as A and
// B agree; here lane half h of k-step s covers dims [16 s + 8 h, +8).
//
// Each row's block maxima of the chunk are collected in LDS and written at the end
// as one contiguous run per row.
#include "msa_internal.hpp"
#include <type_traits>

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQT = 4;
constexpr int kQW = 32 * kQT;    // queries per wave
constexpr int kQB = 4 * kQW;     // queries per workgroup
constexpr int kChunk = 16;       // key blocks per workgroup
constexpr int kBlk = 128;        // block size
constexpr int kOutPad = kChunk + 1;

__device__ __forceinline__ float max16(const f32x16& a) {
  float m = __builtin_fmaxf(__builtin_fmaxf(a[0], a[1]), a[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, a[r]), a[r + 1]);
  return __builtin_fmaxf(m, a[15]);
}

// Bytes B and B+1 of a word of OCP E4M3 codes -> two bf16 in one word.  Exact: E4M3
// values have 3 mantissa bits and exponents inside the bf16 range, so each float's low
// 16 bits are zero.  One hardware conversion per byte (the packed two-value builtin had
// its second result replaced by its first by this compiler).
template <int B>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  const float f0 = __builtin_amdgcn_cvt_f32_fp8((int)w, B);
  const float f1 = __builtin_amdgcn_cvt_f32_fp8((int)w, B + 1);
  return (__builtin_bit_cast(uint32_t, f0) >> 16) | (__builtin_bit_cast(uint32_t, f1) & 0xFFFF0000u);
}

// dI = 128 doubles the resident B operands, which leaves room for one wave per SIMD only.
// TK: uint16_t (bf16 keys) or uint8_t (E4M3 keys, widened to bf16 when staged).
template <int DI, typename TK>
__global__ void __launch_bounds__(256, DI == 128 ? 1 : 2) idx_scores_mfma(Dims D, const uint16_t* __restrict__ q_idx,
                                                          const TK* __restrict__ k_idx,
                                                          float* __restrict__ scores) {
  constexpr int KS = DI / 16;
  constexpr int ROWB = DI * 2 + 16;
  constexpr int CPR = DI / 8;
  constexpr int PER_T = kBlk * CPR / 256;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][kBlk * ROWB];
  __shared__ float outb[4][kQW][kOutPad];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int n = lane & 31;
  const int64_t sg = blockIdx.z;
  const int s = (int)(sg / D.Hkv), g = (int)(sg % D.Hkv);
  const int ns = seq_len(D, s);      // N, or this sequence's length (per-sequence calls)
  const int pos0 = ns - D.T;
  const int t_first = blockIdx.x * kQB;
  const int t_last = min(t_first + kQB - 1, D.T - 1);
  const int bmax = (pos0 + t_last) / kBlk;
  const int b0 = blockIdx.y * kChunk;
  if (b0 > bmax) return;
  const int b1 = min(b0 + kChunk - 1, bmax);

  bf16x8 qf[kQT][KS];
  int pq[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int t = t_first + wave * kQW + qt * 32 + n;
    const int tc = t < D.T ? t : D.T - 1;
    pq[qt] = t < D.T ? pos0 + t : 0x7FFFFFFF;
    const uint16_t* qp = q_idx + (sg * D.T + tc) * DI + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[qt][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }
  const int t_w0 = min(t_first + wave * kQW, D.T - 1);
  const int bmask = (pos0 + t_w0) / kBlk;

  // one piece = 8 key dims: 16 bytes of bf16 or 8 bytes of E4M3
  typedef typename std::conditional<sizeof(TK) == 2, uint4, uint2>::type Piece;
  Piece stage[PER_T];
  auto gload = [&](int b) {
    // a block's keys are contiguous (dense cache or one page); an invalid page reads as 0
    const int64_t kb0 = kv_row(D, s, g, b * kBlk, DI);
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int c = threadIdx.x + 256 * u;
      const int row = c / CPR, col = c % CPR;
      const int j = b * kBlk + row;
      stage[u] = kb0 >= 0 && j < ns ? *reinterpret_cast<const Piece*>(k_idx + kb0 + (int64_t)row * DI + col * 8)
                                    : Piece{};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int c = threadIdx.x + 256 * u;
      const int row = c / CPR, col = c % CPR;
      uint4 w;
      if constexpr (sizeof(TK) == 2) {
        w = stage[u];
      } else {
        w = make_uint4(e4m3x2_to_bf16x2<0>(stage[u].x), e4m3x2_to_bf16x2<2>(stage[u].x),
                       e4m3x2_to_bf16x2<0>(stage[u].y), e4m3x2_to_bf16x2<2>(stage[u].y));
      }
      *reinterpret_cast<uint4*>(&lds[buf][row * ROWB + col * 16]) = w;
    }
  };

  gload(b0);
  lstore(0);
  __syncthreads();

  for (int b = b0; b <= b1; ++b) {
    const int buf = (b - b0) & 1;
    if (b < b1) gload(b + 1);
    float rmax[kQT];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) rmax[qt] = -INFINITY;
    auto body = [&](auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      f32x16 acc[2][kQT];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        bf16x8 af[KS];
        const unsigned char* arow = &lds[buf][(kt * 32 + n) * ROWB + 16 * h];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) af[ks] = *reinterpret_cast<const bf16x8*>(arow + ks * 32);
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) {
          acc[kt & 1][qt] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc[kt & 1][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], qf[qt][ks], acc[kt & 1][qt], 0, 0, 0);
        }
        if (kt >= 1) {
          const int pk = (kt - 1) & 1;
#pragma unroll
          for (int qt = 0; qt < kQT; ++qt) {
            if (MASKED) {
              const int jb = b * kBlk + (kt - 1) * 32 + 4 * h;
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (jb + 8 * (r >> 2) + (r & 3) > pq[qt]) acc[pk][qt][r] = -INFINITY;
            }
            rmax[qt] = __builtin_fmaxf(rmax[qt], max16(acc[pk][qt]));
          }
        }
      }
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) {
        if (MASKED) {
          const int jb = b * kBlk + 3 * 32 + 4 * h;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (jb + 8 * (r >> 2) + (r & 3) > pq[qt]) acc[1][qt][r] = -INFINITY;
        }
        rmax[qt] = __builtin_fmaxf(rmax[qt], max16(acc[1][qt]));
      }
    };
    if (b >= bmask) body(std::true_type{});
    else body(std::false_type{});
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) rmax[qt] = __builtin_fmaxf(rmax[qt], __shfl_xor(rmax[qt], 32, 64));
    // lane half h records query tiles 2h and 2h + 1
    outb[wave][(2 * h) * 32 + n][b - b0] = h == 0 ? rmax[0] : rmax[2];
    outb[wave][(2 * h + 1) * 32 + n][b - b0] = h == 0 ? rmax[1] : rmax[3];
    if (b < b1) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int rr = 0; rr < kQW / 64; ++rr) {
    const int rl = lane + 64 * rr;
    const int t_out = t_first + wave * kQW + rl;
    if (t_out < D.T) {
      const int bt = (pos0 + t_out) / kBlk;
      const int len = min(b1, bt) - b0 + 1;
      float* out_row = scores + (sg * D.T + t_out) * (int64_t)D.nb + b0;
      const float* src = outb[wave][rl];
      int u = 0;
      if ((D.nb & 3) == 0)
        for (; u + 4 <= len; u += 4) *reinterpret_cast<float4*>(out_row + u) = make_float4(src[u], src[u + 1], src[u + 2], src[u + 3]);
      for (; u < len; ++u) out_row[u] = src[u];
    }
  }
}

template <typename TK>
void launch_mfma_t(const Dims& D, dim3 grid, const uint16_t* q_idx, const TK* k_idx, float* scores, hipStream_t st) {
  switch (D.dI) {
    case 32: hipLaunchKernelGGL((idx_scores_mfma<32, TK>), grid, dim3(256), 0, st, D, q_idx, k_idx, scores); break;
    case 64: hipLaunchKernelGGL((idx_scores_mfma<64, TK>), grid, dim3(256), 0, st, D, q_idx, k_idx, scores); break;
    default: hipLaunchKernelGGL((idx_scores_mfma<128, TK>), grid, dim3(256), 0, st, D, q_idx, k_idx, scores); break;
  }
}

}  // namespace

hipError_t launch_index_scores_mfma(const Dims& D, const uint16_t* q_idx, const void* k_idx,
                                    float* scores, hipStream_t st) {
  const int nq = (D.T + kQB - 1) / kQB;
  const int bmax = (D.N - 1) / kBlk;
  const int nchunk = bmax / kChunk + 1;
  dim3 grid((unsigned)nq, (unsigned)nchunk, (unsigned)(D.S * D.Hkv));
  LaunchScope scope("idx_scores_mfma", st);
  if (D.kdtype == MSA_FP8_E4M3) launch_mfma_t(D, grid, q_idx, static_cast<const uint8_t*>(k_idx), scores, st);
  else launch_mfma_t(D, grid, q_idx, static_cast<const uint16_t*>(k_idx), scores, st);
  return hipGetLastError();
}

}  // namespace msa
