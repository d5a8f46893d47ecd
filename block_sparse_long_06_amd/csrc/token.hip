// token.hip -- token-level selection on the same indexer, for the granularity comparison of
// page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比", section 分歧一：颗粒度
// (DSA picks 2048 single tokens per query where MSA picks 16 blocks x 128: the same
// budget) and the DSA entry of "稀疏注意力速览（Sparse Attention，2019 ~ 2026）" (the
// indexer scores every earlier token, the top-k single tokens are kept).
//
//  * token top-k: the `budget` causal tokens with the largest scores, ties to the lower
//    position, as ascending positions; exact, over order-preserving uint32 keys.  Rows are
//    cut into chunks of kTkChunk positions, one workgroup each (the whole chip works on a
//    few rows):
//      tk_hist   : a histogram of each row's top 11 key bits (per-wave LDS histograms,
//                  then global atomics of the nonzero bins);
//      tk_filter : every chunk derives the row's threshold bin b1 (where the count from the
//                  top reaches `budget`) and appends its keys with top bits >= b1, in
//                  position order, to the row's candidate list (one contiguous run per
//                  chunk, placed by an atomic counter, recorded in a chunk table);
//      tk_finish : one workgroup per row reads the candidates back in chunk order (= position
//                  order), radix-selects the remaining 21 bits among the b1 bin, and
//                  compacts the chosen positions.
//    A row whose candidates exceed kTkCap (heavy ties, coarse score distributions) is left
//    to token_topk, the one-workgroup radix select (digits of 11, 11 and 10 bits over the
//    whole row, then a compaction pass), which runs only for such rows.
//  * token_attn: one workgroup per (row, group, chunk of 128 selected tokens) gathers the
//    chunk's K / V rows into LDS, one wave per query head forms the chunk-local softmax
//    partial (lse, O); the log-sum-exp merge of the block path combines a row's chunks.
#include "msa_internal.hpp"

namespace msa {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kChunk = 128;  // selected tokens per attention work item

__device__ __forceinline__ uint32_t ord_key(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u << 1) == 0u) u = 0u;  // -0 and +0 are the same value
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix sum over the workgroup's 1024 threads; *total receives the sum.
__device__ int block_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (threadIdx.x < 64) {
    int w = threadIdx.x < kTkWaves ? wsum[threadIdx.x] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(w, o, 64);
      if (threadIdx.x >= o) w += y;
    }
    if (threadIdx.x < kTkWaves) wsum[threadIdx.x] = w;  // inclusive over waves
  }
  __syncthreads();
  const int before = (wave > 0 ? wsum[wave - 1] : 0) + x - v;
  const int tot = wsum[kTkWaves - 1];
  __syncthreads();  // wsum may be reused by the next call
  *total = tot;
  return before;
}

// ---------------------------------------------------------------- chunked top-k
constexpr int kTkChunk = 16384;  // positions per tk_hist / tk_filter workgroup
constexpr int kTkCap = 16384;    // candidates a row may keep (more: the one-workgroup path)
constexpr int kTkLocal = 4096;   // candidates a tk_filter workgroup buffers in LDS
constexpr int kTkBins = 2048;    // first digit: the top 11 key bits
constexpr int kTkShift = 21;

// Per-row scratch (global memory), kTkRow32(nch) 32-bit words per row.
struct TkRow {
  uint32_t* hist;     // [kTkBins] counts of the top 11 key bits
  uint32_t* head;     // [4]: candidate count, overflow flag, b1, keys above bin b1
  uint32_t* coff;     // [nch] a chunk's first candidate
  uint32_t* ccnt;     // [nch] its number of candidates
  uint32_t* ckey;     // [kTkCap] candidate keys
  int32_t* cpos;      // [kTkCap] candidate positions
};
__host__ __device__ inline int64_t tk_row_words(int nch) {
  return ((int64_t)kTkBins + 4 + 2 * (int64_t)nch + 2 * (int64_t)kTkCap + 63) / 64 * 64;
}
__device__ __forceinline__ TkRow tk_row(uint32_t* base, int nch, int64_t row) {
  TkRow r;
  uint32_t* p = base + row * tk_row_words(nch);
  r.hist = p;
  r.head = p + kTkBins;
  r.coff = r.head + 4;
  r.ccnt = r.coff + nch;
  r.ckey = r.ccnt + nch;
  r.cpos = reinterpret_cast<int32_t*>(r.ckey + kTkCap);
  return r;
}

__device__ __forceinline__ int tk_eligible(const Dims& D, int64_t row) {  // row = (s, g, t)
  const int t = (int)(row % D.T);
  const int s = (int)(row / ((int64_t)D.Hkv * D.T));
  return seq_pos0(D, s) + t + 1;
}

__global__ void __launch_bounds__(kTkThreads) token_topk(Dims D, int budget, const float* __restrict__ tok,
                                                         int32_t* __restrict__ out,
                                                         const uint32_t* __restrict__ ws, int nch) {
  __shared__ int hist[2048];
  __shared__ int wsum[kTkWaves];
  __shared__ int s_bin, s_above;
  const int64_t row = blockIdx.x;  // (s, g, t)
  // only the rows the chunked path gave up on (candidate overflow)
  if (ws != nullptr && ws[row * tk_row_words(nch) + kTkBins + 1] == 0u) return;
  const int t = (int)(row % D.T);
  const int s = (int)(row / ((int64_t)D.Hkv * D.T));
  const int n = seq_pos0(D, s) + t + 1;  // eligible positions 0 .. n-1
  const float* sc = tok + row * (int64_t)D.N;
  int32_t* o = out + row * (int64_t)budget;
  const int tid = threadIdx.x;
  if (n <= budget) {
    for (int i = tid; i < budget; i += kTkThreads) o[i] = i < n ? i : -1;
    return;
  }
  // ---- radix select of the budget-th largest key tau
  uint32_t prefix = 0;
  int need = budget;  // still to take among the keys that match the prefix
  const int shifts[3] = {21, 10, 0}, widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass], wd = widths[pass];
    const int nbins = 1 << wd;
    const uint32_t hi_mask = pass == 0 ? 0u : ~((1u << (sh + wd)) - 1u);
    for (int i = tid; i < nbins; i += kTkThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += kTkThreads) {
      const uint32_t k = ord_key(sc[j]);
      if ((k & hi_mask) == prefix) atomicAdd(&hist[(k >> sh) & (nbins - 1)], 1);
    }
    __syncthreads();
    // thread i owns bins nbins-1-2i and nbins-2-2i (descending); find the bin where the
    // count from the top reaches `need`
    const int b0 = nbins - 1 - 2 * tid, b1 = nbins - 2 - 2 * tid;
    const int c0 = b0 >= 0 ? hist[b0] : 0, c1 = b1 >= 0 ? hist[b1] : 0;
    int tot;
    const int before = block_scan(c0 + c1, wsum, &tot);
    if (before < need && need <= before + c0) {
      s_bin = b0;
      s_above = before;
    } else if (before + c0 < need && need <= before + c0 + c1) {
      s_bin = b1;
      s_above = before + c0;
    }
    __syncthreads();
    prefix |= (uint32_t)s_bin << sh;
    need -= s_above;
    __syncthreads();
  }
  const uint32_t tau = prefix;  // keys > tau: all taken; keys == tau: the first `need`
  // ---- compaction in ascending position order: wave w owns positions [w*span, (w+1)*span),
  // its lanes stride through them 64 at a time (coalesced), ballots rank within a step
  const int lane = tid & 63, wave = tid >> 6;
  const int span = (n + kTkWaves - 1) / kTkWaves;
  const int j0 = wave * span, j1 = min(n, j0 + span);
  int gt = 0, eq = 0;  // per wave (lane 0's copy is used)
  for (int jb = j0; jb < j1; jb += 64) {
    const int j = jb + lane;
    const uint32_t k = j < j1 ? ord_key(sc[j]) : 0u;
    gt += __popcll(__ballot(j < j1 && k > tau));
    eq += __popcll(__ballot(j < j1 && k == tau));
  }
  int tot;
  const int eq_before = block_scan(lane == 0 ? eq : 0, wsum, &tot);        // exclusive over waves
  const int eq_before_w = __shfl(eq_before, 0, 64);
  const int eq_take = max(0, min(eq, need - eq_before_w));
  const int out_before = block_scan(lane == 0 ? gt + eq_take : 0, wsum, &tot);
  int w = __shfl(out_before, 0, 64);
  int eq_seen = eq_before_w;
  for (int jb = j0; jb < j1; jb += 64) {
    const int j = jb + lane;
    const uint32_t k = j < j1 ? ord_key(sc[j]) : 0u;
    const bool is_eq = j < j1 && k == tau;
    const uint64_t eqm = __ballot(is_eq);
    const bool take = (j < j1 && k > tau) || (is_eq && eq_seen + lanes_below(eqm) < need);
    const uint64_t tm = __ballot(take);
    if (take && w + lanes_below(tm) < budget) o[w + lanes_below(tm)] = j;  // exactly budget are taken
    w += __popcll(tm);
    eq_seen += __popcll(eqm);
  }
}

// Exclusive prefix sum over a 256-thread workgroup; *total receives the sum.
__device__ int block_scan256(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  const int w0 = wsum[0], w1 = wsum[1], w2 = wsum[2], w3 = wsum[3];
  const int before = (wave > 0 ? w0 : 0) + (wave > 1 ? w1 : 0) + (wave > 2 ? w2 : 0) + x - v;
  __syncthreads();  // wsum may be reused by the next call
  *total = w0 + w1 + w2 + w3;
  return before;
}

__global__ void __launch_bounds__(kTkThreads) tk_zero(uint32_t* __restrict__ base, int nch, int64_t rows) {
  // clear each row's histogram and head (the other fields are written before they are read)
  const int64_t row = blockIdx.x;
  if (row >= rows) return;
  uint32_t* p = base + row * tk_row_words(nch);
  for (int i = threadIdx.x; i < kTkBins + 4; i += kTkThreads) p[i] = 0u;
}

__global__ void __launch_bounds__(256) tk_hist(Dims D, int budget, int nch, const float* __restrict__ tok,
                                               uint32_t* __restrict__ ws) {
  __shared__ uint32_t h[4][kTkBins];  // one histogram per wave: fewer colliding atomics
  const int64_t row = blockIdx.y;
  const int n = tk_eligible(D, row);
  const int j0 = blockIdx.x * kTkChunk;
  if (n <= budget || j0 >= n) return;
  const int j1 = min(n, j0 + kTkChunk);
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * kTkBins; i += 256) (&h[0][0])[i] = 0u;
  __syncthreads();
  const float* sc = tok + row * (int64_t)D.N;
  for (int j = j0 + (int)threadIdx.x; j < j1; j += 1024) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = j + 256 * u < j1 ? sc[j + 256 * u] : 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j + 256 * u < j1) atomicAdd(&h[wave][ord_key(v[u]) >> kTkShift], 1u);
  }
  __syncthreads();
  TkRow r = tk_row(ws, nch, row);
  for (int b = threadIdx.x; b < kTkBins; b += 256) {
    const uint32_t c = h[0][b] + h[1][b] + h[2][b] + h[3][b];
    if (c) atomicAdd(&r.hist[b], c);
  }
}

__global__ void __launch_bounds__(256) tk_filter(Dims D, int budget, int nch, const float* __restrict__ tok,
                                                 uint32_t* __restrict__ ws) {
  __shared__ uint32_t lkey[kTkLocal];
  __shared__ int32_t lpos[kTkLocal];
  __shared__ int wsum[4];
  __shared__ int s_bin, s_above;
  const int64_t row = blockIdx.y;
  const int n = tk_eligible(D, row);
  const int chunk = blockIdx.x;
  const int j0 = chunk * kTkChunk;
  if (n <= budget || j0 >= n) return;
  const int j1 = min(n, j0 + kTkChunk);
  TkRow r = tk_row(ws, nch, row);
  // ---- the threshold bin: thread i holds bins 2047 - 8i .. 2040 - 8i (descending)
  uint32_t c8[8];
  int csum = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    c8[e] = r.hist[kTkBins - 1 - 8 * (int)threadIdx.x - e];
    csum += (int)c8[e];
  }
  int tot;
  int before = block_scan256(csum, wsum, &tot);
  if (before < budget && budget <= before + csum) {
    int acc = before;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (acc < budget && budget <= acc + (int)c8[e]) {
        s_bin = kTkBins - 1 - 8 * (int)threadIdx.x - e;
        s_above = acc;
      }
      acc += (int)c8[e];
    }
  }
  __syncthreads();
  const uint32_t b1 = (uint32_t)s_bin;
  const uint32_t t1 = b1 << kTkShift;  // candidates: keys >= t1
  if (chunk == 0 && threadIdx.x == 0) {
    r.head[2] = b1;
    r.head[3] = (uint32_t)s_above;
  }
  // ---- candidates of the chunk in position order: wave w takes the chunk's w-th quarter,
  // 256 positions per step (4 consecutive per lane), ranks its candidates with a wave scan
  // and keeps them in its quarter of the LDS buffer; the quarters follow in wave order
  const float* sc = tok + row * (int64_t)D.N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kQuarter = kTkLocal / 4;
  uint32_t* wkey = lkey + wave * kQuarter;
  int32_t* wpos = lpos + wave * kQuarter;
  const int q0 = j0 + wave * (kTkChunk / 4), q1 = min(j1, q0 + kTkChunk / 4);
  int cw = 0;
  for (int base = q0; base < q1; base += 256) {
    const int j = base + 4 * lane;
    uint32_t k4[4];
    int f = 0;
    if (j + 3 < q1 && ((reinterpret_cast<uintptr_t>(sc + j) & 15) == 0)) {
      const float4 v4 = *reinterpret_cast<const float4*>(sc + j);
      k4[0] = ord_key(v4.x); k4[1] = ord_key(v4.y); k4[2] = ord_key(v4.z); k4[3] = ord_key(v4.w);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) k4[u] = j + u < q1 ? ord_key(sc[j + u]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) f += (j + u < q1 && k4[u] >= t1) ? 1 : 0;
    int x = f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    int at = cw + x - f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j + u < q1 && k4[u] >= t1) {
        if (at < kQuarter) {
          wkey[at] = k4[u];
          wpos[at] = j + u;
        }
        ++at;
      }
    cw += __shfl(x, 63, 64);
  }
  if (lane == 0) wsum[wave] = cw;
  __syncthreads();
  const int c0 = wsum[0], c1 = wsum[1], c2 = wsum[2], c3 = wsum[3];
  const int C = c0 + c1 + c2 + c3;
  const bool wover = c0 > kQuarter || c1 > kQuarter || c2 > kQuarter || c3 > kQuarter;
  __shared__ uint32_t s_base;
  if (threadIdx.x == 0) {
    const uint32_t b = wover ? (uint32_t)kTkCap + 1u : atomicAdd(&r.head[0], (uint32_t)C);
    const bool over = wover || b + (uint32_t)C > (uint32_t)kTkCap;
    if (over) atomicOr(&r.head[1], 1u);
    s_base = over ? 0xFFFFFFFFu : b;
    r.coff[chunk] = over ? 0u : b;
    r.ccnt[chunk] = over ? 0u : (uint32_t)C;
  }
  __syncthreads();
  const uint32_t b = s_base;
  if (b == 0xFFFFFFFFu) return;
  const uint32_t wb = b + (uint32_t)((wave > 0 ? c0 : 0) + (wave > 1 ? c1 : 0) + (wave > 2 ? c2 : 0));
  for (int i = lane; i < cw; i += 64) {
    r.ckey[wb + i] = wkey[i];
    r.cpos[wb + i] = wpos[i];
  }
}

// One workgroup per row: the exact selection among the candidates, in position order.
__global__ void __launch_bounds__(kTkThreads) tk_finish(Dims D, int budget, int nch, uint32_t* __restrict__ ws,
                                                        int32_t* __restrict__ out) {
  __shared__ uint32_t key[kTkCap];
  __shared__ int32_t pos[kTkCap];
  __shared__ int hist[2048];
  __shared__ int wsum[kTkWaves];
  __shared__ int s_bin, s_above;
  const int64_t row = blockIdx.x;
  const int n = tk_eligible(D, row);
  int32_t* o = out + row * (int64_t)budget;
  const int tid = threadIdx.x;
  if (n <= budget) {
    for (int i = tid; i < budget; i += kTkThreads) o[i] = i < n ? i : -1;
    return;
  }
  TkRow r = tk_row(ws, nch, row);
  if (r.head[1] != 0u) return;  // overflow: token_topk takes the row
  // ---- candidates back in chunk order
  const int nchr = (n + kTkChunk - 1) / kTkChunk;
  int M = 0;
  for (int c = 0; c < nchr; ++c) {
    const int off = (int)r.coff[c], cnt = (int)r.ccnt[c];
    for (int i = tid; i < cnt; i += kTkThreads) {
      key[M + i] = r.ckey[off + i];
      pos[M + i] = r.cpos[off + i];
    }
    M += cnt;
  }
  const uint32_t b1 = r.head[2];
  const int above1 = (int)r.head[3];
  __syncthreads();
  // ---- radix select of the remaining bits (11 then 10) among the b1 bin
  uint32_t prefix = b1 << kTkShift;
  int need = budget - above1;  // >= 1: to take among the keys that match the prefix
  const int shifts[2] = {10, 0}, widths[2] = {11, 10};
  for (int pass = 0; pass < 2; ++pass) {
    const int sh = shifts[pass], wd = widths[pass];
    const int nbins = 1 << wd;
    const uint32_t hi_mask = ~((1u << (sh + wd)) - 1u);
    for (int i = tid; i < nbins; i += kTkThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < M; i += kTkThreads) {
      const uint32_t k = key[i];
      if ((k & hi_mask) == prefix) atomicAdd(&hist[(k >> sh) & (nbins - 1)], 1);
    }
    __syncthreads();
    const int bb0 = nbins - 1 - 2 * tid, bb1 = nbins - 2 - 2 * tid;
    const int c0 = bb0 >= 0 ? hist[bb0] : 0, c1 = bb1 >= 0 ? hist[bb1] : 0;
    int tot;
    const int before = block_scan(c0 + c1, wsum, &tot);
    if (before < need && need <= before + c0) {
      s_bin = bb0;
      s_above = before;
    } else if (before + c0 < need && need <= before + c0 + c1) {
      s_bin = bb1;
      s_above = before + c0;
    }
    __syncthreads();
    prefix |= (uint32_t)s_bin << sh;
    need -= s_above;
    __syncthreads();
  }
  const uint32_t tau = prefix;  // keys > tau: all taken; keys == tau: the first `need` by position
  // ---- compaction in position order: thread i owns candidates [i * per, (i + 1) * per)
  const int per = (M + kTkThreads - 1) / kTkThreads;
  const int a0 = min(M, tid * per), a1 = min(M, a0 + per);
  int gt = 0, eq = 0;
  for (int i = a0; i < a1; ++i) {
    gt += key[i] > tau ? 1 : 0;
    eq += key[i] == tau ? 1 : 0;
  }
  int tot;
  const int eq_before = block_scan(eq, wsum, &tot);
  const int eq_take = max(0, min(eq, need - eq_before));
  int w = block_scan(gt + eq_take, wsum, &tot);
  int eq_seen = eq_before;
  for (int i = a0; i < a1; ++i) {
    const uint32_t k = key[i];
    const bool take = k > tau || (k == tau && eq_seen < need);
    eq_seen += k == tau ? 1 : 0;
    if (take) {
      if (w < budget) o[w] = pos[i];  // exactly budget are taken
      ++w;
    }
  }
}

template <int DH>
struct TokLds {
  uint16_t k[kChunk][DH + 2];  // bf16, rows of DH / 2 + 1 words: lane-per-key reads are conflict-free
  uint16_t v[kChunk][DH];
  int32_t pos[kChunk];
  float p[16][kChunk];         // per head (wave): probabilities
  uint16_t q[16][DH];          // bf16 (78 KB in all: two workgroups per CU)
};

// Work item (row (s, t, g), chunk c): tokens sel_tok[(s, g, t), c*128 ...]; wave h = head h.
template <int DH>
__global__ void __launch_bounds__(1024) token_attn(Dims D, int budget, int nch, const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                   const int32_t* __restrict__ sel_tok, float* __restrict__ part_lse,
                                                   float* __restrict__ part_o, int32_t* __restrict__ chunk_sel) {
  __shared__ TokLds<DH> L;
  const int64_t row = blockIdx.x;  // (s, t, g)
  const int c = blockIdx.y;
  const int g = (int)(row % D.Hkv);
  const int t = (int)((row / D.Hkv) % D.T);
  const int s = (int)(row / ((int64_t)D.Hkv * D.T));
  const int32_t* tl = sel_tok + (((int64_t)s * D.Hkv + g) * D.T + t) * budget + (int64_t)c * kChunk;
  const int ntok = min(kChunk, budget - c * kChunk);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ns = seq_len(D, s);
  for (int i = threadIdx.x; i < kChunk; i += blockDim.x) {
    const int pj = i < ntok ? tl[i] : -1;
    L.pos[i] = pj < ns ? pj : -1;  // a position outside the sequence counts as empty
  }
  __syncthreads();
  const bool any = L.pos[0] >= 0;  // positions ascend, -1 padding last
  if (threadIdx.x == 0) chunk_sel[(((int64_t)s * D.Hkv + g) * D.T + t) * nch + c] = any ? c : -1;
  if (!any) return;
  for (int i = threadIdx.x; i < kChunk * DH / 8; i += blockDim.x) {
    const int j = i / (DH / 8), cc = (i % (DH / 8)) * 8;
    const int pj = L.pos[j];
    const int64_t off = pj >= 0 ? kv_row(D, s, g, pj, DH) : -1;
    uint4 kk = make_uint4(0u, 0u, 0u, 0u), vv = make_uint4(0u, 0u, 0u, 0u);
    if (off >= 0) {
      kk = *reinterpret_cast<const uint4*>(k + off + cc);
      vv = *reinterpret_cast<const uint4*>(v + off + cc);
    }
    const uint32_t wk[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
    for (int x = 0; x < 4; ++x) *reinterpret_cast<uint32_t*>(&L.k[j][cc + 2 * x]) = wk[x];
    *reinterpret_cast<uint4*>(&L.v[j][cc]) = vv;
  }
  const int h = wave;  // one wave per query head of the group
  const uint16_t* qv = q + (((int64_t)s * D.T + t) * D.H + (int64_t)g * D.G + h) * DH;
  if (h < D.G)
    for (int cc = lane; cc < DH; cc += 64) L.q[h][cc] = qv[cc];
  __syncthreads();
  if (h >= D.G) return;
  float lg[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = lane + 64 * u;
    lg[u] = -INFINITY;
    if (L.pos[j] >= 0) {
      float acc = 0.0f;
      for (int cc = 0; cc < DH; cc += 2) {
        const uint32_t kw = *reinterpret_cast<const uint32_t*>(&L.k[j][cc]);
        const uint32_t qw = *reinterpret_cast<const uint32_t*>(&L.q[h][cc]);
        acc = fmaf(bf16_to_f32((uint16_t)(qw & 0xFFFFu)), bf16_to_f32((uint16_t)(kw & 0xFFFFu)), acc);
        acc = fmaf(bf16_to_f32((uint16_t)(qw >> 16)), bf16_to_f32((uint16_t)(kw >> 16)), acc);
      }
      lg[u] = acc * D.scale;
    }
  }
  const float m = wave_max(fmaxf(lg[0], lg[1]));
  const float p0 = lg[0] == -INFINITY ? 0.0f : __expf(lg[0] - m);
  const float p1 = lg[1] == -INFINITY ? 0.0f : __expf(lg[1] - m);
  const float l = wave_sum(p0 + p1);
  L.p[h][lane] = p0;
  L.p[h][lane + 64] = p1;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int64_t pi = (row * nch + c) * D.G + h;
  const float inv = 1.0f / l;
  for (int cc = lane; cc < DH; cc += 64) {
    float acc = 0.0f;
    for (int j = 0; j < kChunk; ++j) acc = fmaf(L.p[h][j], bf16_to_f32(L.v[j][cc]), acc);
    part_o[pi * DH + cc] = acc * inv;
  }
  if (lane == 0) part_lse[pi] = m + __logf(l);
}

struct TokWs {
  float* part_lse;
  float* part_o;
  int32_t* chunk_sel;
};

TokWs token_layout(const Dims& D, int budget, void* base, size_t* total) {
  const int nch = (budget + kChunk - 1) / kChunk;
  const int64_t nslot = (int64_t)D.S * D.T * D.Hkv * nch;
  unsigned char* p = static_cast<unsigned char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* r = p ? p + off : nullptr;
    off += align_up(bytes, 256);
    return r;
  };
  TokWs w;
  w.part_lse = static_cast<float*>(take(nslot * D.G * sizeof(float)));
  w.part_o = static_cast<float*>(take(nslot * D.G * D.d * sizeof(float)));
  w.chunk_sel = static_cast<int32_t*>(take(nslot * sizeof(int32_t)));
  *total = off;
  return w;
}

}  // namespace

size_t token_topk_workspace_bytes(const Dims& D) {
  const int nch = (D.N + kTkChunk - 1) / kTkChunk;
  return (size_t)D.S * D.Hkv * D.T * (size_t)tk_row_words(nch) * sizeof(uint32_t);
}

hipError_t launch_token_topk(const Dims& D, int budget, const float* tok, int32_t* sel_tok, void* ws,
                             hipStream_t st) {
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  const int nch = (D.N + kTkChunk - 1) / kTkChunk;
  uint32_t* w = static_cast<uint32_t*>(ws);
  LaunchScope scope("token_topk", st);
  hipLaunchKernelGGL(tk_zero, dim3((unsigned)rows), dim3(kTkThreads), 0, st, w, nch, rows);
  hipLaunchKernelGGL(tk_hist, dim3((unsigned)nch, (unsigned)rows), dim3(256), 0, st, D, budget, nch, tok, w);
  hipLaunchKernelGGL(tk_filter, dim3((unsigned)nch, (unsigned)rows), dim3(256), 0, st, D, budget, nch, tok, w);
  hipLaunchKernelGGL(tk_finish, dim3((unsigned)rows), dim3(kTkThreads), 0, st, D, budget, nch, w, sel_tok);
  // rows whose candidates overflowed (the flag in each row's head) take the one-workgroup path
  hipLaunchKernelGGL(token_topk, dim3((unsigned)rows), dim3(kTkThreads), 0, st, D, budget, tok, sel_tok,
                     static_cast<const uint32_t*>(w), nch);
  return hipGetLastError();
}

size_t token_workspace_bytes(const Dims& D, int budget) {
  // one buffer serves the top-k call and then the attention call
  size_t total = 0;
  (void)token_layout(D, budget, nullptr, &total);
  const size_t tk = token_topk_workspace_bytes(D);
  return total > tk ? total : tk;
}

hipError_t launch_token_attn(const Dims& D, int budget, const void* q, const void* k, const void* v,
                             const int32_t* sel_tok, void* out, void* ws, hipStream_t st) {
  size_t total = 0;
  const TokWs w = token_layout(D, budget, ws, &total);
  const int nch = (budget + kChunk - 1) / kChunk;
  const int64_t rows = (int64_t)D.S * D.T * D.Hkv;
  {
    LaunchScope scope("token_attn", st);
    const dim3 grid((unsigned)rows, (unsigned)nch);
    const dim3 block((unsigned)(64 * D.G));
    if (D.d == 64)
      hipLaunchKernelGGL(token_attn<64>, grid, block, 0, st, D, budget, nch, static_cast<const uint16_t*>(q),
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), sel_tok, w.part_lse,
                         w.part_o, w.chunk_sel);
    else
      hipLaunchKernelGGL(token_attn<128>, grid, block, 0, st, D, budget, nch, static_cast<const uint16_t*>(q),
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), sel_tok, w.part_lse,
                         w.part_o, w.chunk_sel);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Dims Dc = D;
  Dc.k = nch;  // the merge treats a row's chunks as its slots
  return launch_lse_merge(Dc, w.chunk_sel, w.part_lse, w.part_o, 0, nullptr, out, st, "token_merge");
}

}  // namespace msa
