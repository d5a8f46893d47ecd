// index_scores.hip -- a1: index-branch scoring fused with the causal block max-pool.
// Page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比", section 第一步：粗筛
// items 1-2 (score every token of a 128-token block, block score = the maximum,
// "block max pooling"); MSA entry of "稀疏注意力速览（Sparse Attention，2019 ~ 2026）"
// (one index-query head and a shared index-key head per GQA group, max-pool
// inside the block).
//
//   scores[s,g,t,b] = max_{bB <= j <= min((b+1)B-1, p_t)} q_idx[s,g,t,:] . k_idx[s,g,j,:]
//
// Kernels:
//  * idx_scores_rows: one wave per (row, block), lane per key, fp32 FMAs (float32
//    inputs and mid-sized query counts).
//  * idx_scores_stream: the decode shape (a few queries), a stream over the keys.
//  * idx_scores_mfma (index_scores_mfma.hip): bf16 prefill on matrix cores.
// Index keys are bf16 / float32 like the queries, or OCP E4M3 bytes (bf16 problems),
// decoded exactly with the hardware converter before the products.
#include "msa_internal.hpp"

namespace msa {

hipError_t launch_index_scores_mfma(const Dims& D, const uint16_t* q_idx, const void* k_idx,
                                    float* scores, hipStream_t st);

namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ void load8(const uint16_t* p, float* o) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  o[0] = __builtin_bit_cast(float, u.x << 16);
  o[1] = __builtin_bit_cast(float, u.x & 0xFFFF0000u);
  o[2] = __builtin_bit_cast(float, u.y << 16);
  o[3] = __builtin_bit_cast(float, u.y & 0xFFFF0000u);
  o[4] = __builtin_bit_cast(float, u.z << 16);
  o[5] = __builtin_bit_cast(float, u.z & 0xFFFF0000u);
  o[6] = __builtin_bit_cast(float, u.w << 16);
  o[7] = __builtin_bit_cast(float, u.w & 0xFFFF0000u);
}
// 4 OCP E4M3 bytes of a word -> 4 floats (exact), one hardware conversion per byte.
// (The single-byte form: the packed two-value builtin had its second result replaced
// by its first by this compiler.)
__device__ __forceinline__ void e4m3x4(uint32_t w, float* o) {
  o[0] = __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
  o[1] = __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
  o[2] = __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
  o[3] = __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
}
// 8 OCP E4M3 bytes -> 8 floats (exact).
__device__ __forceinline__ void load8(const uint8_t* p, float* o) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  e4m3x4(u.x, o);
  e4m3x4(u.y, o + 4);
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// grid: (rows = S*Hkv*T, ceil(nb / kWaves)); wave w of block (r, y) scores block y*kWaves + w.
template <typename T, typename TK>
__global__ void __launch_bounds__(kWaves * 64) idx_scores_rows(Dims D, const T* __restrict__ q_idx,
                                                               const TK* __restrict__ k_idx,
                                                               float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x;
  const int b = blockIdx.y * kWaves + (threadIdx.x >> 6);
  const int t = (int)(row % D.T);
  const int64_t sg = row / D.T;
  const int s = (int)(sg / D.Hkv), g = (int)(sg % D.Hkv);
  const int p = seq_pos0(D, s) + t;
  const int bt = p / D.B;
  if (b > bt) return;
  const T* q = q_idx + row * D.dI;
  const int64_t kb0 = kv_row(D, s, g, b * D.B, D.dI);  // a block's rows are contiguous
  float best = kb0 < 0 ? 0.0f : -INFINITY;               // rows of an invalid page read as 0
  for (int j = b * D.B + lane; kb0 >= 0 && j < (b + 1) * D.B && j <= p; j += 64) {
    const TK* kk = k_idx + kb0 + (int64_t)(j - b * D.B) * D.dI;
    float acc = 0.0f;
    for (int c = 0; c < D.dI; c += 8) {
      float qv[8], kv[8];
      load8(q + c, qv);
      load8(kk + c, kv);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf(qv[u], kv[u], acc);
    }
    best = fmaxf(best, acc);
  }
  best = wave_max(best);
  if (lane == 0) scores[row * D.nb + b] = best;
}

// Decode shape (T <= kStreamT queries per (s, g)): a stream over the index keys.  One
// workgroup scores kStreamBlocks consecutive blocks of one (s, g) for all its queries.
// Thread = (key slot, 16-byte column of the key row): every load instruction of the
// workgroup covers one contiguous 4 KB run of keys.  The lanes sharing a key add
// their partial dots with xor shuffles; the block max is a wave reduction over key
// slots plus an LDS step across the 4 waves.
typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamT = 8;
constexpr int kStreamBlocks = 8;

// TK = uint16_t (bf16 keys: 8 dims per 16-byte lane load) or uint8_t (E4M3 keys: 16
// dims per 16-byte lane load, decoded with the hardware converter).  TOKEN: write every
// causal key's score to tok [S, Hkv, T, N] instead of the block maxima (token-level
// selection).
template <int DI, int TQ, typename TK, bool TOKEN = false>
__global__ void __launch_bounds__(256) idx_scores_stream(Dims D, const uint16_t* __restrict__ q_idx,
                                                         const TK* __restrict__ k_idx,
                                                         float* __restrict__ scores) {
  constexpr int DPL = 16 / (int)sizeof(TK);  // dims per lane and key
  constexpr int CPR = DI / DPL;              // lanes per key row
  constexpr int KPP = 256 / CPR;             // keys per pass of the workgroup
  constexpr int PASSES = 128 / KPP;          // passes per block
  __shared__ float red[kStreamBlocks][4][TQ];  // per (block, wave) maxima, combined at the end
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = threadIdx.x % CPR;
  const int kslot = threadIdx.x / CPR;
  const int64_t sg = blockIdx.y;
  const int s = (int)(sg / D.Hkv), g = (int)(sg % D.Hkv);
  const int b0 = blockIdx.x * kStreamBlocks;
  const int T = D.T;
  const int ns = seq_len(D, s);
  float qv[TQ][DPL];
  int pq[TQ];
#pragma unroll
  for (int tq = 0; tq < TQ; ++tq) {
    const int t = tq < T ? tq : T - 1;
    pq[tq] = tq < T ? ns - T + tq : -1;
#pragma unroll
    for (int x = 0; x < DPL; x += 8) load8(q_idx + (sg * T + t) * DI + col * DPL + x, &qv[tq][x]);
  }
  const int bend = min(b0 + kStreamBlocks, (ns + 127) / 128);
  // a block's rows are contiguous (dense cache or one page); an invalid page reads as 0.
  // Loads run ahead in registers so the next blocks' HBM reads overlap this block's dot
  // products and reductions; each key is read once (non-temporal loads).
  // Each wave leaves its maximum of every block in LDS; the workgroup's four are combined
  // once, after its last block, so the loop has no barrier.
  auto gload = [&](int b, uint4 (&kr)[PASSES]) {
    const int64_t kb0 = kv_row(D, s, g, b * 128, DI);
    const TK* kbase = k_idx + (kb0 < 0 ? 0 : kb0) + col * DPL;
#pragma unroll
    for (int u = 0; u < PASSES; ++u) {
      const int jj = u * KPP + kslot;
      kr[u] = kb0 >= 0 && b * 128 + jj < ns
                  ? __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                        reinterpret_cast<const nt_u32x4*>(kbase + (int64_t)jj * DI)))
                  : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  // (two ahead with one query row, the decode shape; one ahead with TQ rows, whose query
  // registers leave no room for a third set)
  constexpr bool AHEAD2 = TQ == 1;
  uint4 kr[PASSES], kn[PASSES], kn2[AHEAD2 ? PASSES : 1];
  if (b0 < bend) gload(b0, kn);
  if constexpr (AHEAD2) {
    if (b0 + 1 < bend) gload(b0 + 1, kn2);
  }
#pragma unroll
  for (int i = 0; i < kStreamBlocks; ++i) {
    const int b = b0 + i;
    if (b >= bend) break;
#pragma unroll
    for (int u = 0; u < PASSES; ++u) kr[u] = kn[u];
    if constexpr (AHEAD2) {
#pragma unroll
      for (int u = 0; u < PASSES; ++u) kn[u] = kn2[u];
      if (b + 2 < bend) gload(b + 2, kn2);
    } else {
      if (b + 1 < bend) gload(b + 1, kn);
    }
    float m[TQ];
#pragma unroll
    for (int tq = 0; tq < TQ; ++tq) m[tq] = -INFINITY;
#pragma unroll
    for (int u = 0; u < PASSES; ++u) {
      const int j = b * 128 + u * KPP + kslot;
      const uint32_t w4[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
      float kv[DPL];
      if constexpr (sizeof(TK) == 2) {
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          kv[2 * i2] = __builtin_bit_cast(float, w4[i2] << 16);
          kv[2 * i2 + 1] = __builtin_bit_cast(float, w4[i2] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) e4m3x4(w4[i2], &kv[4 * i2]);
      }
#pragma unroll
      for (int tq = 0; tq < TQ; ++tq) {
        float acc = 0.0f;
#pragma unroll
        for (int x = 0; x < DPL; ++x) acc = fmaf(qv[tq][x], kv[x], acc);
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
        if constexpr (TOKEN) {
          if (col == 0 && tq < T && j <= pq[tq])
            __builtin_nontemporal_store(acc, &scores[(sg * T + tq) * (int64_t)D.N + j]);
        } else {
          if (j <= pq[tq]) m[tq] = fmaxf(m[tq], acc);
        }
      }
    }
    if constexpr (TOKEN) continue;
#pragma unroll
    for (int tq = 0; tq < TQ; ++tq) {
      float x = m[tq];
#pragma unroll
      for (int o = CPR; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
      if (lane == 0) red[i][wave][tq] = x;
    }
  }
  if constexpr (!TOKEN) {
    __syncthreads();
    if (threadIdx.x < TQ && threadIdx.x < T) {
      const int tq = threadIdx.x;
#pragma unroll
      for (int i = 0; i < kStreamBlocks; ++i) {
        const int b = b0 + i;
        if (b < bend && b <= pq[tq] / 128)
          scores[(sg * T + tq) * (int64_t)D.nb + b] =
              fmaxf(fmaxf(red[i][0][tq], red[i][1][tq]), fmaxf(red[i][2][tq], red[i][3][tq]));
      }
    }
  }
}

template <int DI, typename TK>
void launch_stream_di(const Dims& D, const uint16_t* q, const TK* k, float* sc, hipStream_t st) {
  dim3 grid((unsigned)((D.nb + kStreamBlocks - 1) / kStreamBlocks), (unsigned)(D.S * D.Hkv));
  if (D.T == 1)
    hipLaunchKernelGGL((idx_scores_stream<DI, 1, TK>), grid, dim3(256), 0, st, D, q, k, sc);
  else
    hipLaunchKernelGGL((idx_scores_stream<DI, kStreamT, TK>), grid, dim3(256), 0, st, D, q, k, sc);
}

template <typename TK>
void launch_stream(const Dims& D, const uint16_t* q, const TK* k, float* sc, hipStream_t st) {
  if (D.dI == 32) launch_stream_di<32>(D, q, k, sc, st);
  else if (D.dI == 64) launch_stream_di<64>(D, q, k, sc, st);
  else launch_stream_di<128>(D, q, k, sc, st);
}

template <int DI, typename TK>
void launch_token_di(const Dims& D, const uint16_t* q, const TK* k, float* tok, hipStream_t st) {
  dim3 grid((unsigned)((D.nb + kStreamBlocks - 1) / kStreamBlocks), (unsigned)(D.S * D.Hkv));
  if (D.T == 1)
    hipLaunchKernelGGL((idx_scores_stream<DI, 1, TK, true>), grid, dim3(256), 0, st, D, q, k, tok);
  else
    hipLaunchKernelGGL((idx_scores_stream<DI, kStreamT, TK, true>), grid, dim3(256), 0, st, D, q, k, tok);
}

template <typename TK>
void launch_token(const Dims& D, const uint16_t* q, const TK* k, float* tok, hipStream_t st) {
  if (D.dI == 32) launch_token_di<32>(D, q, k, tok, st);
  else if (D.dI == 64) launch_token_di<64>(D, q, k, tok, st);
  else launch_token_di<128>(D, q, k, tok, st);
}

}  // namespace

// Token-level scores for decode shapes (bf16 queries, T <= kStreamT): tok [S, Hkv, T, N].
hipError_t launch_token_scores(const Dims& D, const void* q_idx, const void* k_idx, float* tok, hipStream_t st) {
  if (D.dtype != MSA_BF16 || D.T > kStreamT) return hipErrorInvalidValue;
  const uint16_t* q = static_cast<const uint16_t*>(q_idx);
  LaunchScope scope("token_scores", st);
  if (D.kdtype == MSA_FP8_E4M3) launch_token(D, q, static_cast<const uint8_t*>(k_idx), tok, st);
  else launch_token(D, q, static_cast<const uint16_t*>(k_idx), tok, st);
  return hipGetLastError();
}

hipError_t launch_index_scores(const Dims& D, const void* q_idx, const void* k_idx, float* scores,
                               hipStream_t st) {
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  const bool f8 = D.kdtype == MSA_FP8_E4M3;
  if (D.dtype == MSA_BF16 && D.T >= 256)
    return launch_index_scores_mfma(D, static_cast<const uint16_t*>(q_idx), k_idx, scores, st);
  if (D.dtype == MSA_BF16 && D.T <= kStreamT) {
    const uint16_t* q = static_cast<const uint16_t*>(q_idx);
    LaunchScope scope("idx_scores_stream", st);
    if (f8) launch_stream(D, q, static_cast<const uint8_t*>(k_idx), scores, st);
    else launch_stream(D, q, static_cast<const uint16_t*>(k_idx), scores, st);
    return hipGetLastError();
  }
  dim3 grid((unsigned)rows, (unsigned)((D.nb + kWaves - 1) / kWaves));
  LaunchScope scope("idx_scores_rows", st);
  if (D.dtype == MSA_BF16 && f8)
    hipLaunchKernelGGL((idx_scores_rows<uint16_t, uint8_t>), grid, dim3(kWaves * 64), 0, st, D,
                       static_cast<const uint16_t*>(q_idx), static_cast<const uint8_t*>(k_idx), scores);
  else if (D.dtype == MSA_BF16)
    hipLaunchKernelGGL((idx_scores_rows<uint16_t, uint16_t>), grid, dim3(kWaves * 64), 0, st, D,
                       static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx), scores);
  else
    hipLaunchKernelGGL((idx_scores_rows<float, float>), grid, dim3(kWaves * 64), 0, st, D,
                       static_cast<const float*>(q_idx), static_cast<const float*>(k_idx), scores);
  return hipGetLastError();
}

}  // namespace msa
