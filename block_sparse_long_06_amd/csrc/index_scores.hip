// index_scores.hip -- a1: index-branch scoring fused with the causal block max-pool.
// Page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比", section 第一步：粗筛
// items 1-2 (score every token of a 128-token block, block score = the maximum,
// "block max pooling"); MSA entry of "稀疏注意力速览（Sparse Attention，2019 ~ 2026）"
// (one index-query head and a shared index-key head per GQA group, max-pool
// inside the block).
//
//   scores[s,g,t,b] = max_{bB <= j <= min((b+1)B-1, p_t)} q_idx[s,g,t,:] . k_idx[s,g,j,:]
//
// Two kernels:
//  * idx_scores_rows: one wave per (row, block), lane per key, fp32 FMAs.  Used
//    for float32 inputs and for short query counts (the decode shape, where the
//    stage is a stream over the index keys).
//  * idx_scores_mfma (index_scores_mfma.hip): bf16 prefill on matrix cores.
#include "msa_internal.hpp"

namespace msa {

hipError_t launch_index_scores_mfma(const Dims& D, const uint16_t* q_idx, const uint16_t* k_idx,
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
__device__ __forceinline__ void load8(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// grid: (rows = S*Hkv*T, ceil(nb / kWaves)); wave w of block (r, y) scores block y*kWaves + w.
template <typename T>
__global__ void __launch_bounds__(kWaves * 64) idx_scores_rows(Dims D, const T* __restrict__ q_idx,
                                                               const T* __restrict__ k_idx,
                                                               float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x;
  const int b = blockIdx.y * kWaves + (threadIdx.x >> 6);
  const int t = (int)(row % D.T);
  const int64_t sg = row / D.T;
  const int p = D.pos0 + t;
  const int bt = p / D.B;
  if (b > bt) return;
  const T* q = q_idx + row * D.dI;
  const T* kbase = k_idx + sg * (int64_t)D.N * D.dI;
  float best = -INFINITY;
  for (int j = b * D.B + lane; j < (b + 1) * D.B && j <= p; j += 64) {
    const T* kk = kbase + (int64_t)j * D.dI;
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
// workgroup covers one contiguous 4 KB run of keys.  The DI/8 lanes sharing a key add
// their partial dots with xor shuffles; the block max is a wave reduction over key
// slots plus an LDS step across the 4 waves.
constexpr int kStreamT = 8;
constexpr int kStreamBlocks = 8;

template <int DI, int TQ>
__global__ void __launch_bounds__(256) idx_scores_stream(Dims D, const uint16_t* __restrict__ q_idx,
                                                         const uint16_t* __restrict__ k_idx,
                                                         float* __restrict__ scores) {
  constexpr int CPR = DI / 8;            // lanes per key row
  constexpr int KPP = 256 / CPR;         // keys per pass of the workgroup
  constexpr int PASSES = 128 / KPP;      // passes per block
  __shared__ float red[4][TQ];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = threadIdx.x % CPR;
  const int kslot = threadIdx.x / CPR;
  const int64_t sg = blockIdx.y;
  const int b0 = blockIdx.x * kStreamBlocks;
  const int T = D.T;
  float qv[TQ][8];
  int pq[TQ];
#pragma unroll
  for (int tq = 0; tq < TQ; ++tq) {
    const int t = tq < T ? tq : T - 1;
    pq[tq] = tq < T ? D.pos0 + tq : -1;
    load8(q_idx + (sg * T + t) * DI + col * 8, qv[tq]);
  }
  const uint16_t* kbase = k_idx + sg * (int64_t)D.N * DI + col * 8;
  const int bend = min(b0 + kStreamBlocks, D.nb);
  for (int b = b0; b < bend; ++b) {
    uint4 kr[PASSES];
#pragma unroll
    for (int u = 0; u < PASSES; ++u) {
      const int j = b * 128 + u * KPP + kslot;
      kr[u] = j < D.N ? *reinterpret_cast<const uint4*>(kbase + (int64_t)j * DI) : make_uint4(0u, 0u, 0u, 0u);
    }
    float m[TQ];
#pragma unroll
    for (int tq = 0; tq < TQ; ++tq) m[tq] = -INFINITY;
#pragma unroll
    for (int u = 0; u < PASSES; ++u) {
      const int j = b * 128 + u * KPP + kslot;
      const uint32_t w4[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
      float kv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kv[2 * i] = __builtin_bit_cast(float, w4[i] << 16);
        kv[2 * i + 1] = __builtin_bit_cast(float, w4[i] & 0xFFFF0000u);
      }
#pragma unroll
      for (int tq = 0; tq < TQ; ++tq) {
        float acc = 0.0f;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc = fmaf(qv[tq][x], kv[x], acc);
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
        if (j <= pq[tq]) m[tq] = fmaxf(m[tq], acc);
      }
    }
#pragma unroll
    for (int tq = 0; tq < TQ; ++tq) {
      float x = m[tq];
#pragma unroll
      for (int o = CPR; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
      if (lane == 0) red[wave][tq] = x;
    }
    __syncthreads();
    if (threadIdx.x < TQ && threadIdx.x < T) {
      const int tq = threadIdx.x;
      const float x = fmaxf(fmaxf(red[0][tq], red[1][tq]), fmaxf(red[2][tq], red[3][tq]));
      if (b <= pq[tq] / 128) scores[(sg * T + tq) * (int64_t)D.nb + b] = x;
    }
    __syncthreads();
  }
}

template <int DI>
void launch_stream_di(const Dims& D, const uint16_t* q, const uint16_t* k, float* sc, hipStream_t st) {
  dim3 grid((unsigned)((D.nb + kStreamBlocks - 1) / kStreamBlocks), (unsigned)(D.S * D.Hkv));
  if (D.T == 1)
    hipLaunchKernelGGL((idx_scores_stream<DI, 1>), grid, dim3(256), 0, st, D, q, k, sc);
  else
    hipLaunchKernelGGL((idx_scores_stream<DI, kStreamT>), grid, dim3(256), 0, st, D, q, k, sc);
}

}  // namespace

hipError_t launch_index_scores(const Dims& D, const void* q_idx, const void* k_idx, float* scores,
                               hipStream_t st) {
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  if (D.dtype == MSA_BF16 && D.T >= 256)
    return launch_index_scores_mfma(D, static_cast<const uint16_t*>(q_idx),
                                    static_cast<const uint16_t*>(k_idx), scores, st);
  if (D.dtype == MSA_BF16 && D.T <= kStreamT) {
    const uint16_t* q = static_cast<const uint16_t*>(q_idx);
    const uint16_t* k = static_cast<const uint16_t*>(k_idx);
    LaunchScope scope("idx_scores_stream", st);
    if (D.dI == 32) launch_stream_di<32>(D, q, k, scores, st);
    else if (D.dI == 64) launch_stream_di<64>(D, q, k, scores, st);
    else launch_stream_di<128>(D, q, k, scores, st);
    return hipGetLastError();
  }
  dim3 grid((unsigned)rows, (unsigned)((D.nb + kWaves - 1) / kWaves));
  LaunchScope scope("idx_scores_rows", st);
  if (D.dtype == MSA_BF16)
    hipLaunchKernelGGL(idx_scores_rows<uint16_t>, grid, dim3(kWaves * 64), 0, st, D,
                       static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx), scores);
  else
    hipLaunchKernelGGL(idx_scores_rows<float>, grid, dim3(kWaves * 64), 0, st, D,
                       static_cast<const float*>(q_idx), static_cast<const float*>(k_idx), scores);
  return hipGetLastError();
}

}  // namespace msa
