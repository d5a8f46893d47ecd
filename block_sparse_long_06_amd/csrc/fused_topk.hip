// fused_topk.hip -- a1 + a2 fused: index scores, block max-pool and per-group top-k
// without materialising the [T, nb] block scores.  Page "MSA 稀疏注意力三国杀：NSA / DSA /
// MoBA / MSA 四方案深度对比", section 第一步：粗筛 (score every token, block max pooling,
// 16 blocks with the current position's block always chosen, the rest by score).
//
// idx_topk_mfma: one workgroup = 256 query rows of one (sequence, group) x a span of up to
// kSpan key blocks.  The block maxima are formed exactly as in the unfused matrix-core
// indexer (same k-step order, same max chain), 16 blocks (a chunk) at a time into LDS; after
// each chunk one thread per row merges the chunk's maxima into the row's running list of
// its 15 best blocks (score descending, id ascending), kept in LDS.  Within a span the ids
// arrive in ascending order, so a block enters a full list only with a score strictly
// above the list's last one.  Only blocks b < b_t (strictly in the row's past) are ranked:
// the own block is forced, later blocks are not eligible -- so no causal mask is needed.
// Each (row, span) list is written out (score, id; id -1 for empty entries).
//
// topk_merge: one thread per row merges its spans' lists into the k-1 best blocks (score
// descending, id ascending), appends the own block and writes them in ascending order,
// padded with -1: the output of msa_block_topk.
#include "msa_internal.hpp"

#include <type_traits>

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQT = 2;
constexpr int kQW = 32 * kQT;    // queries per wave
constexpr int kQB = 4 * kQW;     // queries per workgroup
constexpr int kChunk = 16;       // blocks merged per step
constexpr int kSpan = 1024;      // blocks per span (workgroup)
constexpr int kBlk = 128;
constexpr int kList = 15;        // list length: k - 1 <= 15

__device__ __forceinline__ float max16(const f32x16& a) {
  float m = __builtin_fmaxf(__builtin_fmaxf(a[0], a[1]), a[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, a[r]), a[r + 1]);
  return __builtin_fmaxf(m, a[15]);
}

template <int B>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  const float f0 = __builtin_amdgcn_cvt_f32_fp8((int)w, B);
  const float f1 = __builtin_amdgcn_cvt_f32_fp8((int)w, B + 1);
  return (__builtin_bit_cast(uint32_t, f0) >> 16) | (__builtin_bit_cast(uint32_t, f1) & 0xFFFF0000u);
}

template <int DI, typename TK>
__global__ void __launch_bounds__(256, DI == 128 ? 1 : 2) idx_topk_mfma(Dims D, const uint16_t* __restrict__ q_idx,
                                                        const TK* __restrict__ k_idx, float* __restrict__ cand_sc,
                                                        int32_t* __restrict__ cand_id, int nspan) {
  constexpr int KS = DI / 16;
  constexpr int ROWB = DI * 2 + 16;
  constexpr int CPR = DI / 8;
  constexpr int PER_T = kBlk * CPR / 256;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][kBlk * ROWB];
  __shared__ __attribute__((aligned(16))) float outb[4][kQW][kChunk + 4];  // 16-byte aligned rows
  __shared__ float lsc[kQB][kList];
  __shared__ uint16_t lid[kQB][kList];  // block ids < 8192

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int n = lane & 31;
  const int64_t sg = blockIdx.z;
  const int t_first = blockIdx.x * kQB;
  const int t_last = min(t_first + kQB - 1, D.T - 1);
  const int span = blockIdx.y;
  const int b_lo = span * kSpan;
  const int b_hi = min(b_lo + kSpan, (D.pos0 + t_last) / kBlk);  // exclusive: only past blocks are ranked
  // this thread's row for the merges
  const int tr = t_first + threadIdx.x;
  const int bt_r = tr < D.T ? (D.pos0 + tr) / kBlk : 0;
  int cnt = 0;
  float theta = -INFINITY;  // the list's last score once it is full: the entry bar

  if (b_lo < b_hi) {
    bf16x8 qf[kQT][KS];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      const int t = t_first + wave * kQW + qt * 32 + n;
      const int tc = t < D.T ? t : D.T - 1;
      const uint16_t* qp = q_idx + (sg * D.T + tc) * DI + 8 * h;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[qt][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
    }
    const TK* kbase = k_idx + sg * (int64_t)D.N * DI;
    typedef typename std::conditional<sizeof(TK) == 2, uint4, uint2>::type Piece;
    Piece stage[PER_T];
    auto gload = [&](int b) {
#pragma unroll
      for (int u = 0; u < PER_T; ++u) {
        const int c = threadIdx.x + 256 * u;
        const int row = c / CPR, col = c % CPR;
        const int j = b * kBlk + row;
        stage[u] = j < D.N ? *reinterpret_cast<const Piece*>(kbase + (int64_t)j * DI + col * 8) : Piece{};
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

    gload(b_lo);
    lstore(0);
    __syncthreads();
    for (int b = b_lo; b < b_hi; ++b) {
      const int buf = (b - b_lo) & 1;
      if (b + 1 < b_hi) gload(b + 1);
      float rmax[kQT];
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) rmax[qt] = -INFINITY;
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
#pragma unroll
          for (int qt = 0; qt < kQT; ++qt) rmax[qt] = __builtin_fmaxf(rmax[qt], max16(acc[(kt - 1) & 1][qt]));
        }
      }
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) rmax[qt] = __builtin_fmaxf(rmax[qt], max16(acc[1][qt]));
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) rmax[qt] = __builtin_fmaxf(rmax[qt], __shfl_xor(rmax[qt], 32, 64));
      // lane half h records query tile h
      outb[wave][h * 32 + n][(b - b_lo) % kChunk] = h == 0 ? rmax[0] : rmax[1];
      if (b + 1 < b_hi) lstore(buf ^ 1);
      __syncthreads();
      if ((b - b_lo) % kChunk == kChunk - 1 || b + 1 == b_hi) {
        // merge the chunk's maxima into this thread's row list
        const int c0 = b - (b - b_lo) % kChunk;
        const float* src = outb[threadIdx.x >> 6][threadIdx.x & 63];
        float v[kChunk];
#pragma unroll
        for (int q4 = 0; q4 < kChunk / 4; ++q4) {
          const float4 f = *reinterpret_cast<const float4*>(src + 4 * q4);
          v[4 * q4] = f.x; v[4 * q4 + 1] = f.y; v[4 * q4 + 2] = f.z; v[4 * q4 + 3] = f.w;
        }
        float* ls = lsc[threadIdx.x];
        uint16_t* li = lid[threadIdx.x];
        const int nv = min(b, bt_r - 1) - c0 + 1;  // this row's eligible blocks of the chunk
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
          const float s = v[j];
          if (j >= nv || !(s > theta)) continue;  // ids ascend: a tie with the bar stays out
          int pos = cnt < kList ? cnt : kList - 1;
          while (pos > 0 && ls[pos - 1] < s) {
            ls[pos] = ls[pos - 1];
            li[pos] = li[pos - 1];
            --pos;
          }
          ls[pos] = s;
          li[pos] = (uint16_t)(c0 + j);
          cnt = cnt < kList ? cnt + 1 : kList;
          if (cnt == kList) theta = ls[kList - 1];
        }
        __syncthreads();  // outb is rewritten by the next chunk
      }
    }
  }
  if (tr < D.T) {
    const int64_t o = ((sg * D.T + tr) * nspan + span) * kList;
    for (int i = 0; i < kList; ++i) {
      cand_sc[o + i] = i < cnt ? lsc[threadIdx.x][i] : 0.0f;
      cand_id[o + i] = i < cnt ? (int32_t)lid[threadIdx.x][i] : -1;
    }
  }
}

// One thread per row: the k-1 best of the spans' candidates, plus the own block, ascending.
__global__ void __launch_bounds__(256) topk_merge(Dims D, int nspan, const float* __restrict__ cand_sc,
                                                  const int32_t* __restrict__ cand_id, int32_t* __restrict__ sel) {
  __shared__ float bs[256][kList];
  __shared__ int32_t bi[256][kList + 1];
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (s, g, t)
  if (row >= (int64_t)D.S * D.Hkv * D.T) return;
  const int t = (int)(row % D.T);
  const int bt = (D.pos0 + t) / kBlk;
  const int want = min(D.k - 1, bt);
  float* ls = bs[threadIdx.x];
  int32_t* li = bi[threadIdx.x];
  int cnt = 0;
  for (int sp = 0; sp < nspan; ++sp) {
    const int64_t o = (row * nspan + sp) * kList;
    for (int i = 0; i < kList; ++i) {
      const int32_t id = cand_id[o + i];
      if (id < 0) break;
      const float s = cand_sc[o + i];
      // better = higher score, then lower id
      if (cnt == want && want > 0) {
        const float ws = ls[want - 1];
        const int32_t wi = li[want - 1];
        if (!(s > ws || (s == ws && id < wi))) continue;
      }
      if (want == 0) break;
      int pos = cnt < want ? cnt : want - 1;
      while (pos > 0 && (ls[pos - 1] < s || (ls[pos - 1] == s && li[pos - 1] > id))) {
        ls[pos] = ls[pos - 1];
        li[pos] = li[pos - 1];
        --pos;
      }
      ls[pos] = s;
      li[pos] = id;
      cnt = cnt < want ? cnt + 1 : want;
    }
  }
  li[cnt++] = bt;  // the own block
  // ascending ids (insertion sort; at most 16 entries)
  for (int i = 1; i < cnt; ++i) {
    const int32_t x = li[i];
    int j = i - 1;
    while (j >= 0 && li[j] > x) {
      li[j + 1] = li[j];
      --j;
    }
    li[j + 1] = x;
  }
  int32_t* out = sel + row * D.k;
  for (int i = 0; i < D.k; ++i) out[i] = i < cnt ? li[i] : -1;
}

template <int DI, typename TK>
void launch_fused_t(const Dims& D, dim3 grid, const uint16_t* q, const TK* k, float* cs, int32_t* ci, int nspan,
                    hipStream_t st) {
  hipLaunchKernelGGL((idx_topk_mfma<DI, TK>), grid, dim3(256), 0, st, D, q, k, cs, ci, nspan);
}

template <typename TK>
void launch_fused(const Dims& D, dim3 grid, const uint16_t* q, const TK* k, float* cs, int32_t* ci, int nspan,
                  hipStream_t st) {
  if (D.dI == 32) launch_fused_t<32, TK>(D, grid, q, k, cs, ci, nspan, st);
  else if (D.dI == 64) launch_fused_t<64, TK>(D, grid, q, k, cs, ci, nspan, st);
  else launch_fused_t<128, TK>(D, grid, q, k, cs, ci, nspan, st);
}

int num_spans(const Dims& D) { return (D.nb + kSpan - 1) / kSpan; }

}  // namespace

// Below this many query rows the unfused indexer takes its row / streaming kernels (another
// float32 summation order); the fused call then runs those two kernels itself, into a
// workspace of block scores bounded by T < kFusedMinT, so that its selection stays
// bit-identical to the two separate calls for every problem.
constexpr int kFusedMinT = 256;

size_t index_topk_workspace_bytes(const Dims& D) {
  if (D.T < kFusedMinT) return align_up((size_t)D.S * D.Hkv * D.T * D.nb * sizeof(float), 256);
  const size_t n = (size_t)D.S * D.Hkv * D.T * num_spans(D) * kList;
  return align_up(n * sizeof(float), 256) + align_up(n * sizeof(int32_t), 256);
}

hipError_t launch_index_topk(const Dims& D, const void* q_idx, const void* k_idx, int32_t* sel, void* ws,
                             hipStream_t st) {
  if (D.T < kFusedMinT) {
    float* sc = static_cast<float*>(ws);
    hipError_t e = launch_index_scores(D, q_idx, k_idx, sc, st);
    return e != hipSuccess ? e : launch_block_topk(D, sc, sel, st);
  }
  const int nspan = num_spans(D);
  const size_t n = (size_t)D.S * D.Hkv * D.T * nspan * kList;
  float* cs = static_cast<float*>(ws);
  int32_t* ci = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(ws) + align_up(n * sizeof(float), 256));
  {
    const dim3 grid((unsigned)((D.T + kQB - 1) / kQB), (unsigned)nspan, (unsigned)(D.S * D.Hkv));
    LaunchScope scope("idx_topk_mfma", st);
    const uint16_t* q = static_cast<const uint16_t*>(q_idx);
    if (D.kdtype == MSA_FP8_E4M3) launch_fused(D, grid, q, static_cast<const uint8_t*>(k_idx), cs, ci, nspan, st);
    else launch_fused(D, grid, q, static_cast<const uint16_t*>(k_idx), cs, ci, nspan, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  LaunchScope scope("topk_merge", st);
  hipLaunchKernelGGL(topk_merge, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, D, nspan, cs, ci, sel);
  return hipGetLastError();
}

}  // namespace msa
