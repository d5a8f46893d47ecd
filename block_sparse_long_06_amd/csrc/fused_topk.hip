// fused_topk.hip -- a1 + a2 fused: index scores, block max-pool and per-group top-k
// without materialising the [T, nb] block scores.  Page "MSA 稀疏注意力三国杀：NSA / DSA /
// MoBA / MSA 四方案深度对比", section 第一步：粗筛 (score every token, block max pooling,
// 16 blocks with the current position's block always chosen, the rest by score).
//
// idx_topk_mfma: one workgroup = 512 query rows of one (sequence, group) x a span of up to
// kSpan key blocks; each wave holds four 32-query tiles as resident MFMA operands, so a key
// fragment read from LDS feeds four products.  The block maxima are formed exactly as in
// the unfused matrix-core indexer (same k-step order; a maximum does not depend on the
// order it is taken in).  Lane (h, n) of a wave ends each block with the maxima of rows
// 2h * 32 + n and (2h + 1) * 32 + n of its query tiles and is also the thread that ranks
// those two rows, so the maxima of 16 blocks (a chunk) go to lane-private LDS rows and
// need no barrier.  After each chunk the lane merges them into each row's running list of
// its 15 best blocks (score descending, id ascending), held in registers: only the chunk's
// values above the list's last score are visited, each inserted by a branch-free shift.  Within a
// span the ids arrive in ascending order, so a block enters only with a score strictly
// above the list's last one (-inf while the list has room, so -inf and NaN never enter).
// Only blocks b < b_t (strictly in the row's past) are ranked: the own block is forced,
// later blocks are not eligible -- so no causal mask is needed.  Each (row, span) list is
// written out (score, id; id -1 for empty entries) -- or, when the keys fit one span
// (nb <= kSpan), the list already is the row's ranking and the lane writes the row's
// selection itself.
//
// topk_merge (several spans): one thread per row merges its spans' lists into the k-1 best blocks (score
// descending, id ascending), appends the own block and writes them in ascending order,
// padded with -1: the output of msa_block_topk.
#include "msa_internal.hpp"

#include <type_traits>

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQT = 4;           // 32-query tiles per wave
constexpr int kQW = 32 * kQT;    // queries per wave
// Waves per workgroup W: 4 (512 query rows), or 8 (1024 rows sharing each staged key block:
// fewer staging loads per product) where each row tile has about the same work -- a chunk
// far into its sequence -- and the registers allow two waves per SIMD (d_I <= 64); with
// causal row tiles the longer tiles of eight waves made the launch's tail longer.
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

// The row's list of its kList best blocks so far (score descending, id ascending; empty
// entries hold score -inf and id -1, so ls[kList - 1] is the entry bar), and the merge of
// one chunk's maxima src[0..nv) -- block ids c0 + j, above every id in the list.
struct RowList {
  float ls[kList];
  int li[kList];
};

__device__ __forceinline__ void list_init(RowList& L) {
#pragma unroll
  for (int i = 0; i < kList; ++i) {
    L.ls[i] = -INFINITY;
    L.li[i] = -1;
  }
}

__device__ __forceinline__ void list_merge(RowList& L, const float* src, int nv, int c0) {
  const float bar = L.ls[kList - 1];
  uint32_t m = 0;
#pragma unroll
  for (int q4 = 0; q4 < kChunk / 4; ++q4) {
    const float4 f = *reinterpret_cast<const float4*>(src + 4 * q4);
    m |= (f.x > bar ? 1u : 0u) << (4 * q4);
    m |= (f.y > bar ? 2u : 0u) << (4 * q4);
    m |= (f.z > bar ? 4u : 0u) << (4 * q4);
    m |= (f.w > bar ? 8u : 0u) << (4 * q4);
  }
  m &= nv >= kChunk ? 0xFFFFu : (nv > 0 ? (1u << nv) - 1u : 0u);
  while (m) {  // ascending ids: a tie with an entry places the new block after it
    const int j = __builtin_ctz(m);
    m &= m - 1;
    const float sc = src[j];
    if (!(sc > L.ls[kList - 1])) continue;
    bool gt[kList];
#pragma unroll
    for (int i = 0; i < kList; ++i) gt[i] = sc > L.ls[i];
#pragma unroll
    for (int i = kList - 1; i >= 1; --i) {
      L.ls[i] = gt[i - 1] ? L.ls[i - 1] : (gt[i] ? sc : L.ls[i]);
      L.li[i] = gt[i - 1] ? L.li[i - 1] : (gt[i] ? c0 + j : L.li[i]);
    }
    L.ls[0] = gt[0] ? sc : L.ls[0];
    L.li[0] = gt[0] ? c0 + j : L.li[0];
  }
}

// The row's selection from its list of best blocks (score descending, id ascending): the
// first min(k - 1, b_t) entries ranked by id (ids are distinct), then the own block b_t,
// then -1 padding -- the output of msa_block_topk.
__device__ __forceinline__ void emit_row(const Dims& D, const int (&li)[kList], int bt, int32_t* out) {
  const int want = min(D.k - 1, bt);
  int v[kList];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < kList; ++i) {
    const bool ok = i < want && li[i] >= 0;
    v[i] = ok ? li[i] : INT_MAX;
    cnt += ok ? 1 : 0;
  }
#pragma unroll
  for (int i = 0; i < kList; ++i) {
    int r = 0;
#pragma unroll
    for (int j = 0; j < kList; ++j) r += v[j] < v[i] ? 1 : 0;
    if (v[i] != INT_MAX) out[r] = v[i];
  }
  out[cnt] = bt;
  for (int i = cnt + 1; i < D.k; ++i) out[i] = -1;
}

template <int DI, typename TK, int W>
__global__ void __launch_bounds__(64 * W, (DI == 128 || W == 8) ? 1 : 2) idx_topk_mfma(Dims D, const uint16_t* __restrict__ q_idx,
                                                        const TK* __restrict__ k_idx, float* __restrict__ cand_sc,
                                                        int32_t* __restrict__ cand_id, int nspan,
                                                        int32_t* __restrict__ sel) {
  constexpr int KS = DI / 16;
  constexpr int ROWB = DI * 2 + 16;
  constexpr int CPR = DI / 8;
  constexpr int NT = 64 * W;
  constexpr int kQB = W * kQW;  // queries per workgroup
  constexpr int PER_T = kBlk * CPR / NT;
  static_assert(PER_T >= 1 && PER_T * NT == kBlk * CPR, "whole 16-byte pieces per thread");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][kBlk * ROWB];
  __shared__ __attribute__((aligned(16))) float outb[W][kQW][kChunk + 4];  // 16-byte aligned rows

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int n = lane & 31;
  // grid (sequence x group, span, row tile from the last): the longest (latest) row tiles
  // are dispatched first, and consecutive workgroups -- spread over the XCDs in turn --
  // take different (sequence, group)s, so each XCD's L2 holds fewer groups' index keys
  const int64_t sg = blockIdx.x;
  const int t_first = (int)(gridDim.z - 1 - blockIdx.z) * kQB;
  const int t_last = min(t_first + kQB - 1, D.T - 1);
  const int span = blockIdx.y;
  const int b_lo = span * kSpan;
  const int b_hi = min(b_lo + kSpan, (D.pos0 + t_last) / kBlk);  // exclusive: only past blocks are ranked
  // this lane ranks rows (2h) * 32 + n and (2h + 1) * 32 + n of its wave's query tiles
  const int rw0 = (2 * h) * 32 + n, rw1 = rw0 + 32;
  const int tr0 = t_first + wave * kQW + rw0, tr1 = tr0 + 32;
  const int bt0 = tr0 < D.T ? (D.pos0 + tr0) / kBlk : 0;
  const int bt1 = tr1 < D.T ? (D.pos0 + tr1) / kBlk : 0;
  RowList L0, L1;
  list_init(L0);
  list_init(L1);

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
        const int c = threadIdx.x + NT * u;
        const int row = c / CPR, col = c % CPR;
        const int j = b * kBlk + row;
        stage[u] = j < D.N ? *reinterpret_cast<const Piece*>(kbase + (int64_t)j * DI + col * 8) : Piece{};
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int u = 0; u < PER_T; ++u) {
        const int c = threadIdx.x + NT * u;
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
      // (key tile, query tile) steps in turn; each step's accumulator is reduced after the
      // next step's products are issued, so two accumulators are live
      f32x16 acc[2];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        bf16x8 af[KS];
        const unsigned char* arow = &lds[buf][(kt * 32 + n) * ROWB + 16 * h];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) af[ks] = *reinterpret_cast<const bf16x8*>(arow + ks * 32);
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) {
          const int step = kt * kQT + qt;
          acc[step & 1] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc[step & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], qf[qt][ks], acc[step & 1], 0, 0, 0);
          if (step >= 1) {
            const int pq = (qt + kQT - 1) % kQT;
            rmax[pq] = __builtin_fmaxf(rmax[pq], max16(acc[(step - 1) & 1]));
          }
        }
      }
      rmax[kQT - 1] = __builtin_fmaxf(rmax[kQT - 1], max16(acc[(4 * kQT - 1) & 1]));
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) rmax[qt] = __builtin_fmaxf(rmax[qt], __shfl_xor(rmax[qt], 32, 64));
      // lane half h records query tiles 2h and 2h + 1: its own two rows
      const int col = (b - b_lo) % kChunk;
      outb[wave][rw0][col] = h == 0 ? rmax[0] : rmax[2];
      outb[wave][rw1][col] = h == 0 ? rmax[1] : rmax[3];
      if (b + 1 < b_hi) lstore(buf ^ 1);
      __syncthreads();
      if (col == kChunk - 1 || b + 1 == b_hi) {
        const int c0 = b - col;
        list_merge(L0, outb[wave][rw0], min(b, bt0 - 1) - c0 + 1, c0);
        list_merge(L1, outb[wave][rw1], min(b, bt1 - 1) - c0 + 1, c0);
      }
    }
  }
  auto put = [&](const RowList& L, int tr) {
    if (tr >= D.T) return;
    if (sel != nullptr) {  // one span: the list is the row's final ranking
      emit_row(D, L.li, (D.pos0 + tr) / kBlk, sel + (sg * D.T + tr) * D.k);
      return;
    }
    const int64_t o = ((sg * D.T + tr) * nspan + span) * kList;
#pragma unroll
    for (int i = 0; i < kList; ++i) {
      cand_sc[o + i] = L.li[i] >= 0 ? L.ls[i] : 0.0f;
      cand_id[o + i] = L.li[i];
    }
  };
  put(L0, tr0);
  put(L1, tr1);
}

// One thread per row: the k-1 best of the spans' candidates, plus the own block, ascending.
// With one span the row's list already is its best 15 in order; with several, each span's
// list is merged into a register list (score descending, id ascending: a span's entries
// arrive in its own order and every id is above the earlier spans', so a new entry goes
// after the equal scores already held).  The chosen ids are placed by rank (they are
// distinct), and the own block, above every ranked id, follows them.
__global__ void __launch_bounds__(256) topk_merge(Dims D, int nspan, const float* __restrict__ cand_sc,
                                                  const int32_t* __restrict__ cand_id, int32_t* __restrict__ sel) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (s, g, t)
  if (row >= (int64_t)D.S * D.Hkv * D.T) return;
  const int t = (int)(row % D.T);
  const int bt = (D.pos0 + t) / kBlk;
  int li[kList];
  if (nspan == 1) {
#pragma unroll
    for (int i = 0; i < kList; ++i) li[i] = cand_id[row * kList + i];
  } else {
    float ls[kList];
#pragma unroll
    for (int i = 0; i < kList; ++i) {
      ls[i] = -INFINITY;
      li[i] = -1;
    }
    for (int sp = 0; sp < nspan; ++sp) {
      const int64_t o = (row * nspan + sp) * kList;
      for (int j = 0; j < kList; ++j) {
        const int32_t id = cand_id[o + j];
        if (id < 0) break;  // the span's list ends
        const float sc = cand_sc[o + j];
        if (!(sc > ls[kList - 1])) break;  // the span's later entries score no higher
        bool gt[kList];
#pragma unroll
        for (int i = 0; i < kList; ++i) gt[i] = sc > ls[i];
#pragma unroll
        for (int i = kList - 1; i >= 1; --i) {
          ls[i] = gt[i - 1] ? ls[i - 1] : (gt[i] ? sc : ls[i]);
          li[i] = gt[i - 1] ? li[i - 1] : (gt[i] ? id : li[i]);
        }
        ls[0] = gt[0] ? sc : ls[0];
        li[0] = gt[0] ? id : li[0];
      }
    }
  }
  emit_row(D, li, bt, sel + row * D.k);
}

template <int DI, typename TK, int W>
void launch_fused_w(const Dims& D, dim3 grid, const uint16_t* q, const TK* k, float* cs, int32_t* ci, int nspan,
                    int32_t* sel, hipStream_t st) {
  const dim3 g(grid.x, grid.y, (unsigned)((D.T + W * kQW - 1) / (W * kQW)));
  hipLaunchKernelGGL((idx_topk_mfma<DI, TK, W>), g, dim3(64 * W), 0, st, D, q, k, cs, ci, nspan, sel);
}

template <int DI, typename TK>
void launch_fused_t(const Dims& D, dim3 grid, const uint16_t* q, const TK* k, float* cs, int32_t* ci, int nspan,
                    int32_t* sel, hipStream_t st) {
  if constexpr (DI <= 64) {
    if ((int64_t)D.pos0 >= 4 * (int64_t)D.T) return launch_fused_w<DI, TK, 8>(D, grid, q, k, cs, ci, nspan, sel, st);
  }
  launch_fused_w<DI, TK, 4>(D, grid, q, k, cs, ci, nspan, sel, st);
}

template <typename TK>
void launch_fused(const Dims& D, dim3 grid, const uint16_t* q, const TK* k, float* cs, int32_t* ci, int nspan,
                  int32_t* sel, hipStream_t st) {
  if (D.dI == 32) launch_fused_t<32, TK>(D, grid, q, k, cs, ci, nspan, sel, st);
  else if (D.dI == 64) launch_fused_t<64, TK>(D, grid, q, k, cs, ci, nspan, sel, st);
  else launch_fused_t<128, TK>(D, grid, q, k, cs, ci, nspan, sel, st);
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
  // with one span (nb <= kSpan) the kernel's lists are final: it writes sel itself and no
  // merge pass runs
  int32_t* direct = nspan == 1 ? sel : nullptr;
  {
    const dim3 grid((unsigned)(D.S * D.Hkv), (unsigned)nspan, 1u);  // row tiles: set per d_I at launch
    LaunchScope scope("idx_topk_mfma", st);
    const uint16_t* q = static_cast<const uint16_t*>(q_idx);
    if (D.kdtype == MSA_FP8_E4M3)
      launch_fused(D, grid, q, static_cast<const uint8_t*>(k_idx), cs, ci, nspan, direct, st);
    else
      launch_fused(D, grid, q, static_cast<const uint16_t*>(k_idx), cs, ci, nspan, direct, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || direct != nullptr) return e;
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  LaunchScope scope("topk_merge", st);
  hipLaunchKernelGGL(topk_merge, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, D, nspan, cs, ci, sel);
  return hipGetLastError();
}

}  // namespace msa
