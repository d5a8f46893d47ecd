// attention.hip -- a4/a5/a6: the main branch.  Exact softmax attention restricted to
// the selected blocks (page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比",
// section 第二步：精算; MSA entry of "稀疏注意力速览（Sparse Attention，2019 ~ 2026）":
// the main branch attends exactly, with softmax, to the chosen blocks only), organised in the
// Outer-Gather-Q order of section Kernel 创新：Outer Gather Q for prefill (the KV block
// is the outer loop, staged on chip once for every query row that chose it) and
// query-centric split-K for decode (one workgroup per (query row, selected block)).
//
// Both produce per-(query row, slot, head) partials over ONE block:
//   lse = m + log(l),  O = (sum_j exp(s_j - m) v_j) / l,   s_j = scale * q . k_j,
// over the block's keys j <= p_t, and lse_merge combines the slots of a row:
//   out = sum_i exp(lse_i - L) O_i,  L = log sum_i exp(lse_i).
// Partial index of (s, t, g, slot): pidx = ((s*T + t)*Hkv + g)*k + slot;
//   part_lse[pidx*G + h], part_o[(pidx*G + h)*d + c].
//
// This file holds the work-list builder, the VALU kernels (float32 problems, and
// any problem the matrix-core kernel does not cover), the decode kernel and the
// merge; the bf16 matrix-core prefill kernel is in attention_mfma.hip.
#include "msa_internal.hpp"
#include "scan.hpp"

#include <stdlib.h>

#include <mutex>

namespace msa {

// matrix-core Outer-Gather-Q kernel (attention_mfma.hip)
bool ogq_mfma_supported(const Dims& D);
int ogq_mfma_rows_per_item(const Dims& D);
hipError_t launch_ogq_mfma(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int4* worklist, const int* n_items, int64_t grid,
                           const int32_t* entries, float* part_lse, uint16_t* part_o, hipStream_t st);
hipError_t launch_hot_mfma(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v, const HotSplit& h,
                           float* part_lse, uint16_t* part_o, hipStream_t st);
// decode attention, one workgroup per (row, group, slot) (decode_attn.hip)
bool decode_attn_supported(const Dims& D);
hipError_t launch_decode_attn(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* sel, float* part_lse, uint16_t* part_o, hipStream_t st);

namespace {

constexpr int kSimpleRows = 16;  // query rows per work item of the VALU kernel

// ------------------------------------------------------------------ work list
// Work item = (sgb = (s*Hkv + g)*nb + b, first csr position, row count <= R).
__global__ void __launch_bounds__(256) wl_count(Dims D, const int32_t* __restrict__ off,
                                                int* __restrict__ items, int R) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nsgb = (int64_t)D.S * D.Hkv * D.nb;
  if (i >= nsgb) return;
  const int64_t sg = i / D.nb;
  const int b = (int)(i % D.nb);
  const int64_t o = sg * (D.nb + 1) + b;
  const int len = off[o + 1] - off[o];
  items[i] = (len + R - 1) / R;
}

__global__ void __launch_bounds__(256) wl_emit(Dims D, const int32_t* __restrict__ off,
                                               const int* __restrict__ items,
                                               const int* __restrict__ itempos,
                                               int4* __restrict__ wl, int R) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nsgb = (int64_t)D.S * D.Hkv * D.nb;
  if (i >= nsgb) return;
  const int64_t sg = i / D.nb;
  const int b = (int)(i % D.nb);
  const int64_t o = sg * (D.nb + 1) + b;
  const int beg = off[o];
  const int len = off[o + 1] - beg;
  const int n = items[i];
  const int p0 = itempos[i];
  for (int j = 0; j < n; ++j) wl[p0 + j] = make_int4((int)i, beg + j * R, min(R, len - j * R), 0);
}

// ------------------------------------------------------------------ VALU block kernel
// Stages K (as float, row stride DH+1: conflict-free lane-per-key reads) and V of one
// block in LDS, then one wave per (row, head) pair computes the block-local softmax.
template <typename T, int DH>
struct BlockLds {
  float K[128][DH + 1];
  T V[128][DH];
  float P[4][128];
  float Q[4][DH];
};

template <typename T, int DH>
__device__ void stage_block(const Dims& D, BlockLds<T, DH>& L, const T* k, const T* v, int64_t sg,
                            int b) {
  const int j0 = b * 128;
  const int s = (int)(sg / D.Hkv), g = (int)(sg % D.Hkv);
  const int64_t kv0 = kv_row(D, s, g, j0, DH);  // a block is contiguous; an invalid page reads as 0
  const int nvalid = kv0 < 0 ? 0 : min(128, seq_len(D, s) - j0);
  const T* kb = k + (kv0 < 0 ? 0 : kv0);
  const T* vb = v + (kv0 < 0 ? 0 : kv0);
  for (int i = threadIdx.x; i < 128 * DH; i += 256) {
    const int row = i / DH, c = i % DH;
    const bool ok = row < nvalid;
    L.K[row][c] = ok ? ldf(kb, i) : 0.0f;
    L.V[row][c] = ok ? vb[i] : T(0);
  }
}

// One (row t, slot, head h) against the staged block.
template <typename T, typename PT, int DH>
__device__ void attend_one(const Dims& D, BlockLds<T, DH>& L, const T* q, int s, int g, int b, int t,
                           int slot, int h, float* part_lse, PT* part_o) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int p = seq_pos0(D, s) + t;
  const T* qv = q + (((int64_t)s * D.T + t) * D.H + g * D.G + h) * DH;
  for (int c = lane; c < DH; c += 64) L.Q[wave][c] = ldf(qv, c);
  __builtin_amdgcn_wave_barrier();
  float lg[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = lane + 64 * u;
    lg[u] = -INFINITY;
    if (b * 128 + j <= p) {
      float acc = 0.0f;
      for (int c = 0; c < DH; ++c) acc = fmaf(L.Q[wave][c], L.K[j][c], acc);
      lg[u] = acc * D.scale;
    }
  }
  const float m = wave_max(fmaxf(lg[0], lg[1]));
  const float p0 = lg[0] == -INFINITY ? 0.0f : exp2f((lg[0] - m) * kLog2e);
  const float p1 = lg[1] == -INFINITY ? 0.0f : exp2f((lg[1] - m) * kLog2e);
  const float l = wave_sum(p0 + p1);
  L.P[wave][lane] = p0;
  L.P[wave][lane + 64] = p1;
  __builtin_amdgcn_wave_barrier();
  const int64_t pidx = (((int64_t)s * D.T + t) * D.Hkv + g) * D.k + slot;
  const float inv = 1.0f / l;
  for (int c = lane; c < DH; c += 64) {
    float acc = 0.0f;
    for (int j = 0; j < 128; ++j) acc = fmaf(L.P[wave][j], ldf(&L.V[0][0], j * DH + c), acc);
    stf(part_o, (pidx * D.G + h) * DH + c, acc * inv);
  }
  if (lane == 0) part_lse[pidx * D.G + h] = m + log2f(l) * kLn2;
  __builtin_amdgcn_wave_barrier();
}

template <typename T, typename PT, int DH>
__global__ void __launch_bounds__(256) ogq_simple(Dims D, const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ v, const int4* __restrict__ wl,
                                                  const int* __restrict__ n_items,
                                                  const int32_t* __restrict__ entries,
                                                  float* __restrict__ part_lse, PT* __restrict__ part_o) {
  extern __shared__ unsigned char smem[];
  BlockLds<T, DH>& L = *reinterpret_cast<BlockLds<T, DH>*>(smem);
  if ((int)blockIdx.x >= *n_items) return;
  const int4 w = wl[blockIdx.x];
  const int64_t sg = w.x / D.nb;
  const int b = w.x % D.nb;
  const int s = (int)(sg / D.Hkv), g = (int)(sg % D.Hkv);
  stage_block<T, DH>(D, L, k, v, sg, b);
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  for (int pr = wave; pr < w.z * D.G; pr += 4) {
    const int e = entries[w.y + pr / D.G];
    attend_one<T, PT, DH>(D, L, q, s, g, b, e / D.k, e % D.k, pr % D.G, part_lse, part_o);
  }
}

// Decode: one workgroup per (row = (s, t, g), slot); unused slots get lse = -inf.
template <typename T, int DH>
__global__ void __launch_bounds__(256) decode_simple(Dims D, const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, const int32_t* __restrict__ sel,
                                                     float* __restrict__ part_lse, float* __restrict__ part_o) {
  extern __shared__ unsigned char smem[];
  BlockLds<T, DH>& L = *reinterpret_cast<BlockLds<T, DH>*>(smem);
  const int slot = blockIdx.y;
  const int64_t row = blockIdx.x;  // ((s*T + t)*Hkv + g)
  const int g = (int)(row % D.Hkv);
  const int t = (int)((row / D.Hkv) % D.T);
  const int s = (int)(row / ((int64_t)D.Hkv * D.T));
  const int64_t sg = (int64_t)s * D.Hkv + g;
  const int b = sel[(sg * D.T + t) * D.k + slot];
  if (b < 0) {
    const int64_t pidx = row * D.k + slot;
    for (int h = threadIdx.x; h < D.G; h += 256) part_lse[pidx * D.G + h] = -INFINITY;
    return;
  }
  stage_block<T, DH>(D, L, k, v, sg, b);
  __syncthreads();
  for (int h = threadIdx.x >> 6; h < D.G; h += 4)
    attend_one<T, float, DH>(D, L, q, s, g, b, t, slot, h, part_lse, part_o);
}

// ------------------------------------------------------------------ merge
__device__ __forceinline__ void load8f(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 c = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = c.x; o[5] = c.y; o[6] = c.z; o[7] = c.w;
}
__device__ __forceinline__ void load8f(const uint16_t* p, float* o) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    o[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  uint4 u;
  u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  u.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
  u.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
  // the merged output is not read again by this library: a non-temporal store
  typedef unsigned u32x4_st __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_st, u), reinterpret_cast<u32x4_st*>(p));
}

// One wave per row (s, t, g).  The row's slot lse values (k x G floats, contiguous)
// are loaded with one coalesced access into LDS, turned there into normalised
// weights w[i][h] = exp(lse_i - max) / sum, and lane l then accumulates the 8
// consecutive outputs of chunks l, l + 64, ... with the partial loads of 8 slots
// issued back to back.  Invalid slots (sel = -1) get weight 0 and are not loaded.
constexpr int kMergeMaxKG = 64 * 16;  // k * G

template <typename T, typename PT>
__global__ void __launch_bounds__(256) lse_merge_kernel(Dims D, const int32_t* __restrict__ sel,
                                                        const float* __restrict__ part_lse,
                                                        const PT* __restrict__ part_o,
                                                        const uint64_t* __restrict__ hotmask, T* __restrict__ out,
                                                        float* __restrict__ lse_out, float* __restrict__ mass_out) {
  __shared__ float wbuf[4][kMergeMaxKG];
  __shared__ float hstat[4][2][16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  const int64_t rows = (int64_t)D.S * D.T * D.Hkv;
  if (row >= rows) return;
  const int g = (int)(row % D.Hkv);
  const int t = (int)((row / D.Hkv) % D.T);
  const int s = (int)(row / ((int64_t)D.Hkv * D.T));
  const int32_t* sl = sel + (((int64_t)s * D.Hkv + g) * D.T + t) * D.k;
  uint64_t vmask = __ballot(lane < D.k && sl[lane < D.k ? lane : 0] >= 0);
  if (hotmask != nullptr) {
    const uint64_t hm = hotmask[row];
    vmask &= ~(hm & (hm - 1));  // hot slots other than the lowest
  }
  const int G = D.G, KG = D.k * D.G, GD = D.G * D.d;
  const float* lrow = part_lse + row * KG;
  const PT* prow = part_o + row * (int64_t)D.k * GD;
  T* orow = out + (((int64_t)s * D.T + t) * D.H + g * G) * D.d;
  float* wb = wbuf[wave];
  for (int x = lane; x < KG; x += 64) wb[x] = ((vmask >> (x / G)) & 1ull) ? lrow[x] : -INFINITY;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < G) {
    float m = -INFINITY;
    for (int i = 0; i < D.k; ++i) m = fmaxf(m, wb[i * G + lane]);
    float tot = 0.0f;
    for (int i = 0; i < D.k; ++i) tot += __builtin_amdgcn_exp2f((wb[i * G + lane] - m) * kLog2e);
    hstat[wave][0][lane] = m;
    hstat[wave][1][lane] = 1.0f / tot;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int x = lane; x < KG; x += 64) {
    const int hh = x % G;
    wb[x] = __builtin_amdgcn_exp2f((wb[x] - hstat[wave][0][hh]) * kLog2e) * hstat[wave][1][hh];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // training outputs: the row's log-sum-exp per head, and per slot the share of the
  // attention that falls on that block, averaged over the group's heads
  if (lse_out != nullptr && lane < G)
    lse_out[((int64_t)s * D.T + t) * D.H + g * G + lane] = hstat[wave][0][lane] - __logf(hstat[wave][1][lane]);
  if (mass_out != nullptr && lane < D.k) {
    float mw = 0.0f;
    for (int hh = 0; hh < G; ++hh) mw += wb[lane * G + hh];
    mass_out[(((int64_t)s * D.Hkv + g) * D.T + t) * D.k + lane] = mw / (float)G;
  }
  for (int c8 = lane; c8 * 8 < GD; c8 += 64) {
    const int hh = c8 * 8 / D.d;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i0 = 0; i0 < D.k; i0 += 8) {
      float o[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u;
        if (i < D.k && ((vmask >> i) & 1ull)) {
          load8f(prow + (int64_t)i * GD + c8 * 8, o[u]);
        } else {
#pragma unroll
          for (int x = 0; x < 8; ++x) o[u][x] = 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u;
        const float w = i < D.k ? wb[i * G + hh] : 0.0f;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] = fmaf(w, o[u][x], acc[x]);
      }
    }
    store8(orow + c8 * 8, acc);
  }
}

// 16 bytes read once (a partial): a non-temporal load.
__device__ __forceinline__ uint4 load_once(const uint16_t* p) {
  typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p)));
}

// The same merge for the common shape (bf16 partials, k <= 16, G * d = 512 * CPL).
// Without a hot mask every partial load of the lane (up to 16 slots x CPL 16-byte
// chunks) is issued first, and the selection mask, lse values and weights are worked
// out while they are in flight (loads of invalid slots read unused workspace and are
// never accumulated).  With a hot mask (HOT) the slot mask is formed first and only
// the slots that are read are loaded: skipped hot slots hold no partial.  lse_out and
// mass_out (optional, training) as in lse_merge_kernel.
template <typename T, int CPL, bool HOT>
__global__ void __launch_bounds__(256) lse_merge_bf16_k16(Dims D, const int32_t* __restrict__ sel,
                                                          const float* __restrict__ part_lse,
                                                          const uint16_t* __restrict__ part_o,
                                                          const uint64_t* __restrict__ hotmask, T* __restrict__ out,
                                                          float* __restrict__ lse_out, float* __restrict__ mass_out) {
  __shared__ float wbuf[4][16 * 16];
  __shared__ float hstat[4][2][16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  const int64_t rows = (int64_t)D.S * D.T * D.Hkv;
  if (row >= rows) return;
  const int G = D.G, KG = D.k * D.G, GD = D.G * D.d;
  const uint16_t* prow = part_o + row * (int64_t)D.k * GD;
  const int g = (int)(row % D.Hkv);
  const int t = (int)((row / D.Hkv) % D.T);
  const int s = (int)(row / ((int64_t)D.Hkv * D.T));
  const int32_t* sl = sel + (((int64_t)s * D.Hkv + g) * D.T + t) * D.k;
  uint4 raw[16][CPL];
  uint64_t vmask;
  if (HOT) {
    vmask = __ballot(lane < D.k && sl[lane < D.k ? lane : 0] >= 0);
    const uint64_t hm = hotmask[row];
    vmask &= ~(hm & (hm - 1));
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        raw[i][c] = (vmask >> i) & 1ull ? load_once(prow + (int64_t)i * GD + (lane + 64 * c) * 8)
                                        : make_uint4(0u, 0u, 0u, 0u);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        raw[i][c] = i < D.k ? load_once(prow + (int64_t)i * GD + (lane + 64 * c) * 8) : make_uint4(0u, 0u, 0u, 0u);
    vmask = __ballot(lane < D.k && sl[lane < D.k ? lane : 0] >= 0);
  }
  const float* lrow = part_lse + row * KG;
  float* wb = wbuf[wave];
  for (int x = lane; x < KG; x += 64) wb[x] = ((vmask >> (x / G)) & 1ull) ? lrow[x] : -INFINITY;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < G) {
    float m = -INFINITY;
    for (int i = 0; i < D.k; ++i) m = fmaxf(m, wb[i * G + lane]);
    float tot = 0.0f;
    for (int i = 0; i < D.k; ++i) tot += __builtin_amdgcn_exp2f((wb[i * G + lane] - m) * kLog2e);
    hstat[wave][0][lane] = m;
    hstat[wave][1][lane] = 1.0f / tot;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int x = lane; x < KG; x += 64) {
    const int hh = x % G;
    wb[x] = __builtin_amdgcn_exp2f((wb[x] - hstat[wave][0][hh]) * kLog2e) * hstat[wave][1][hh];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // training outputs: the row's log-sum-exp per head, and per slot the share of the
  // attention that falls on that block, averaged over the group's heads
  if (lse_out != nullptr && lane < G)
    lse_out[((int64_t)s * D.T + t) * D.H + g * G + lane] = hstat[wave][0][lane] - __logf(hstat[wave][1][lane]);
  if (mass_out != nullptr && lane < D.k) {
    float mw = 0.0f;
    for (int hh = 0; hh < G; ++hh) mw += wb[lane * G + hh];
    mass_out[(((int64_t)s * D.Hkv + g) * D.T + t) * D.k + lane] = mw / (float)G;
  }
  T* orow = out + (((int64_t)s * D.T + t) * D.H + g * G) * D.d;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int c8 = lane + 64 * c;
    const int hh = c8 * 8 / D.d;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < D.k && ((vmask >> i) & 1ull)) {  // wave-uniform
        const float w = wb[i * G + hh];
        const uint32_t q4[4] = {raw[i][c].x, raw[i][c].y, raw[i][c].z, raw[i][c].w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          acc[2 * x] = fmaf(w, __builtin_bit_cast(float, q4[x] << 16), acc[2 * x]);
          acc[2 * x + 1] = fmaf(w, __builtin_bit_cast(float, q4[x] & 0xFFFF0000u), acc[2 * x + 1]);
        }
      }
    }
    store8(orow + c8 * 8, acc);
  }
}

struct PrefillWs {
  int* items;
  int* itempos;
  int* n_items;
  void* scan_ws;
  int4* wl;
  float* part_lse;
  void* part_o;
  int64_t ub;
  bool has_hot;
  HotSplit hs;  // query-tile split (matrix-core problems)
};

int rows_per_item(const Dims& D) {
  return ogq_mfma_supported(D) ? ogq_mfma_rows_per_item(D) : kSimpleRows;
}

PrefillWs prefill_layout(const Dims& D, void* base, size_t* total) {
  const int64_t nsgb = (int64_t)D.S * D.Hkv * D.nb;
  const int64_t npart = (int64_t)D.S * D.T * D.Hkv * D.k;
  const int R = rows_per_item(D);
  PrefillWs w;
  w.ub = nsgb + (npart + R - 1) / R;
  unsigned char* p = static_cast<unsigned char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* r = p ? p + off : nullptr;
    off += align_up(bytes, 256);
    return r;
  };
  w.items = static_cast<int*>(take(nsgb * sizeof(int)));
  w.itempos = static_cast<int*>(take(nsgb * sizeof(int)));
  w.n_items = static_cast<int*>(take(sizeof(int)));
  w.scan_ws = take(scan_workspace_bytes(nsgb));
  w.wl = static_cast<int4*>(take(w.ub * sizeof(int4)));
  w.part_lse = static_cast<float*>(take(npart * D.G * sizeof(float)));
  const size_t pelem = D.dtype == MSA_BF16 ? 2 : 4;
  w.part_o = take((size_t)npart * D.G * D.d * pelem);
  w.has_hot = ogq_mfma_supported(D);
  w.hs = HotSplit{};
  if (w.has_hot) {
    size_t hb = 0;
    (void)hot_split_layout(D, nullptr, &hb);
    void* hbase = take(hb);
    w.hs = hot_split_layout(D, hbase, &hb);
  }
  *total = off;
  return w;
}

// The query-tile pass is on unless the environment sets MSA_HOT_TILES=0.
bool hot_tiles_enabled() {
  const char* e = getenv("MSA_HOT_TILES");
  return !(e != nullptr && e[0] == '0');
}

bool tile_overlap_enabled() {
  const char* e = getenv("MSA_TILE_OVERLAP");
  return !(e != nullptr && e[0] == '0');
}

// A second stream per device (default priority) for the query-tile kernel, with the two
// events that fork it from and join it to the caller's stream.  The tile kernel keeps one
// persistent workgroup per CU with a static share of tiles; launched first on its own
// stream, the Outer-Gather-Q workgroups queued behind it on the caller's stream take each
// CU as its tile workgroup retires, so neither kernel waits for the other's slowest CU.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;  // held from the fork record to the join wait: the events are shared
SideStream g_side[kMaxDevices];

hipError_t side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SideStream& x = g_side[dev];
  if (x.s == nullptr) {
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    x.s = s;
    x.fork = f;
    x.join = j;
  }
  *out = &x;
  return hipSuccess;
}

template <typename T, typename PT, int DH>
hipError_t launch_ogq_simple_t(const Dims& D, const void* q, const void* k, const void* v,
                               const PrefillWs& w, const int32_t* entries, hipStream_t st) {
  const size_t lds = sizeof(BlockLds<T, DH>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(ogq_simple<T, PT, DH>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  LaunchScope scope("ogq_simple", st);
  hipLaunchKernelGGL((ogq_simple<T, PT, DH>), dim3((unsigned)w.ub), dim3(256), lds, st, D,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), w.wl,
                     w.n_items, entries, w.part_lse, static_cast<PT*>(w.part_o));
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t launch_decode_t(const Dims& D, const void* q, const void* k, const void* v, const int32_t* sel,
                           float* part_lse, float* part_o, hipStream_t st) {
  const size_t lds = sizeof(BlockLds<T, DH>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_simple<T, DH>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)D.S * D.T * D.Hkv;
  LaunchScope scope("decode_simple", st);
  hipLaunchKernelGGL((decode_simple<T, DH>), dim3((unsigned)rows, (unsigned)D.k), dim3(256), lds, st, D,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), sel,
                     part_lse, part_o);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const Dims& D, const int32_t* sel, const float* part_lse, const void* part_o,
                            int part_o_is_bf16, const uint64_t* hotmask, void* out, hipStream_t st,
                            const char* name, float* lse_out, float* mass_out) {
  const int64_t rows = (int64_t)D.S * D.T * D.Hkv;
  const dim3 grid((unsigned)((rows + 3) / 4));
  LaunchScope scope(name, st);
  const int gd = D.G * D.d;
  const uint16_t* pb = static_cast<const uint16_t*>(part_o);
  uint16_t* ob = static_cast<uint16_t*>(out);
  const bool train = lse_out != nullptr || mass_out != nullptr;
  if (D.dtype == MSA_BF16 && part_o_is_bf16 && D.k <= 16 && (gd == 512 || gd == 1024) && !(train && hotmask)) {
    if (gd == 1024 && hotmask)
      hipLaunchKernelGGL((lse_merge_bf16_k16<uint16_t, 2, true>), grid, dim3(256), 0, st, D, sel, part_lse, pb,
                         hotmask, ob, lse_out, mass_out);
    else if (gd == 1024)
      hipLaunchKernelGGL((lse_merge_bf16_k16<uint16_t, 2, false>), grid, dim3(256), 0, st, D, sel, part_lse, pb,
                         hotmask, ob, lse_out, mass_out);
    else if (hotmask)
      hipLaunchKernelGGL((lse_merge_bf16_k16<uint16_t, 1, true>), grid, dim3(256), 0, st, D, sel, part_lse, pb,
                         hotmask, ob, lse_out, mass_out);
    else
      hipLaunchKernelGGL((lse_merge_bf16_k16<uint16_t, 1, false>), grid, dim3(256), 0, st, D, sel, part_lse, pb,
                         hotmask, ob, lse_out, mass_out);
  } else if (D.dtype == MSA_BF16) {
    if (part_o_is_bf16)
      hipLaunchKernelGGL((lse_merge_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, st, D, sel, part_lse, pb,
                         hotmask, ob, lse_out, mass_out);
    else
      hipLaunchKernelGGL((lse_merge_kernel<uint16_t, float>), grid, dim3(256), 0, st, D, sel, part_lse,
                         static_cast<const float*>(part_o), hotmask, ob, lse_out, mass_out);
  } else {
    hipLaunchKernelGGL((lse_merge_kernel<float, float>), grid, dim3(256), 0, st, D, sel, part_lse,
                       static_cast<const float*>(part_o), hotmask, static_cast<float*>(out), lse_out, mass_out);
  }
  return hipGetLastError();
}

WorkList work_list_layout(const Dims& D, int R, void* base, size_t* total) {
  const int64_t nsgb = (int64_t)D.S * D.Hkv * D.nb;
  const int64_t npart = (int64_t)D.S * D.T * D.Hkv * D.k;
  WorkList w;
  w.ub = nsgb + (npart + R - 1) / R;
  unsigned char* p = static_cast<unsigned char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* r = p ? p + off : nullptr;
    off += align_up(bytes, 256);
    return r;
  };
  w.items = static_cast<int*>(take(nsgb * sizeof(int)));
  w.itempos = static_cast<int*>(take(nsgb * sizeof(int)));
  w.n_items = static_cast<int*>(take(sizeof(int)));
  w.scan_ws = take(scan_workspace_bytes(nsgb));
  w.wl = static_cast<int4*>(take(w.ub * sizeof(int4)));
  *total = off;
  return w;
}

hipError_t launch_work_list(const Dims& D, const int32_t* off, int R, const WorkList& w, hipStream_t st) {
  const int64_t nsgb = (int64_t)D.S * D.Hkv * D.nb;
  const unsigned g256 = (unsigned)((nsgb + 255) / 256);
  {
    LaunchScope s("wl_count", st);
    hipLaunchKernelGGL(wl_count, dim3(g256), dim3(256), 0, st, D, off, w.items, R);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_exclusive_scan(w.items, w.itempos, nsgb, w.n_items, w.scan_ws, st);
  if (e != hipSuccess) return e;
  LaunchScope s("wl_emit", st);
  hipLaunchKernelGGL(wl_emit, dim3(g256), dim3(256), 0, st, D, off, w.items, w.itempos, w.wl, R);
  return hipGetLastError();
}

size_t prefill_workspace_bytes(const Dims& D) {
  size_t total = 0;
  (void)prefill_layout(D, nullptr, &total);
  return total;
}

hipError_t launch_prefill(const Dims& D, const void* q, const void* k, const void* v, const int32_t* off,
                          const int32_t* entries, const int32_t* sel, void* out, void* ws, hipStream_t st,
                          float* lse_out, float* mass_out) {
  size_t total = 0;
  const PrefillWs w = prefill_layout(D, ws, &total);
  const int64_t nsgb = (int64_t)D.S * D.Hkv * D.nb;
  const int R = rows_per_item(D);
  const unsigned g256 = (unsigned)((nsgb + 255) / 256);
  hipError_t e;
  // the training outputs need one partial per (row, slot): no query-tile pass then
  // (nor with per-sequence lengths: the tile pass maps tiles through one position offset)
  const bool hot = w.has_hot && hot_tiles_enabled() && lse_out == nullptr && mass_out == nullptr &&
                   D.kv_lens == nullptr;
  const bool overlap = hot && tile_overlap_enabled();
  std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
  SideStream* side = nullptr;
  // on an early error return the caller's stream still waits for the tile kernel
  struct Join {
    hipStream_t st;
    SideStream* side;
    ~Join() {
      if (side != nullptr) (void)hipStreamWaitEvent(st, side->join, 0);
    }
  } join{st, nullptr};
  if (hot) {  // Outer-Gather-Q then takes only the cold part of the CSR
    e = launch_hot_split(D, sel, w.hs, st);
    if (e != hipSuccess) return e;
    off = w.hs.cold_off;
    entries = w.hs.cold_ent;
  }
  if (overlap) {  // the tile kernel first, on the side stream, once its tile lists are done
    side_lock.lock();
    e = side_stream(&side);
    if (e == hipSuccess) e = hipEventRecord(side->fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e == hipSuccess)
      e = launch_hot_mfma(D, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), w.hs, w.part_lse, static_cast<uint16_t*>(w.part_o),
                          side->s);
    if (e == hipSuccess) e = hipEventRecord(side->join, side->s);
    if (e != hipSuccess) return e;
    join.side = side;
  }
  if (hot) {  // the cold lists: the inversion of the selections without the tile-shared slots
    e = launch_invert(D, sel, w.hs.cold_off, w.hs.cold_ent, w.hs.inv_ws, st, w.hs.hotmask);
    if (e != hipSuccess) return e;
  }
  {
    LaunchScope s("wl_count", st);
    hipLaunchKernelGGL(wl_count, dim3(g256), dim3(256), 0, st, D, off, w.items, R);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_exclusive_scan(w.items, w.itempos, nsgb, w.n_items, w.scan_ws, st);
  if (e != hipSuccess) return e;
  {
    LaunchScope s("wl_emit", st);
    hipLaunchKernelGGL(wl_emit, dim3(g256), dim3(256), 0, st, D, off, w.items, w.itempos, w.wl, R);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ogq_mfma_supported(D)) {
    e = launch_ogq_mfma(D, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                        static_cast<const uint16_t*>(v), w.wl, w.n_items, w.ub, entries, w.part_lse,
                        static_cast<uint16_t*>(w.part_o), st);
  } else {  // float32 (every bf16 problem the ABI accepts takes the matrix-core kernel)
    e = D.d == 64 ? launch_ogq_simple_t<float, float, 64>(D, q, k, v, w, entries, st)
                  : launch_ogq_simple_t<float, float, 128>(D, q, k, v, w, entries, st);
  }
  // a failed Outer-Gather-Q launch is reported as it is (the Join still makes the
  // caller's stream wait for the tile kernel, with the side-stream lock held)
  if (e != hipSuccess) return e;
  if (overlap) {  // the merge reads both kernels' partials
    join.side = nullptr;
    e = hipStreamWaitEvent(st, side->join, 0);
    side_lock.unlock();
  } else if (hot) {
    e = launch_hot_mfma(D, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                        static_cast<const uint16_t*>(v), w.hs, w.part_lse, static_cast<uint16_t*>(w.part_o), st);
  }
  if (e != hipSuccess) return e;
  return launch_lse_merge(D, sel, w.part_lse, w.part_o, D.dtype == MSA_BF16, hot ? w.hs.hotmask : nullptr, out,
                          st, "lse_merge", lse_out, mass_out);
}

// Decode workspace: partial lse / O per (s, t, g, slot, head), plus (bf16 path) the
// per-slot work items of the matrix-core kernel.
struct DecodeWs {
  float* part_lse;
  void* part_o;
};

static DecodeWs decode_layout(const Dims& D, void* base, size_t* total) {
  const int64_t nslot = (int64_t)D.S * D.T * D.Hkv * D.k;
  const int64_t npart = nslot * D.G;
  const bool mfma = decode_attn_supported(D);  // bf16 partials
  unsigned char* p = static_cast<unsigned char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* r = p ? p + off : nullptr;
    off += align_up(bytes, 256);
    return r;
  };
  DecodeWs w{};
  w.part_lse = static_cast<float*>(take(npart * sizeof(float)));
  w.part_o = take((size_t)npart * D.d * (mfma ? 2 : 4));
  *total = off;
  return w;
}

size_t decode_workspace_bytes(const Dims& D) {
  size_t total = 0;
  (void)decode_layout(D, nullptr, &total);
  return total;
}

hipError_t launch_decode(const Dims& D, const void* q, const void* k, const void* v, const int32_t* sel,
                         void* out, void* ws, hipStream_t st) {
  size_t total = 0;
  const DecodeWs w = decode_layout(D, ws, &total);
  hipError_t e;
  if (decode_attn_supported(D)) {
    e = launch_decode_attn(D, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), sel, w.part_lse, static_cast<uint16_t*>(w.part_o), st);
    if (e != hipSuccess) return e;
    return launch_lse_merge(D, sel, w.part_lse, w.part_o, 1, nullptr, out, st, "decode_merge");
  }
  float* po = static_cast<float*>(w.part_o);  // float32 problems
  e = D.d == 64 ? launch_decode_t<float, 64>(D, q, k, v, sel, w.part_lse, po, st)
                : launch_decode_t<float, 128>(D, q, k, v, sel, w.part_lse, po, st);
  if (e != hipSuccess) return e;
  return launch_lse_merge(D, sel, w.part_lse, w.part_o, 0, nullptr, out, st, "decode_merge");
}

}  // namespace msa
