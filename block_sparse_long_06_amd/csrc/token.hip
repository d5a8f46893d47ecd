// token.hip -- token-level selection on the same indexer, for the granularity comparison of
// page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比", section 分歧一：颗粒度
// (DSA picks 2048 single tokens per query where MSA picks 16 blocks x 128: the same
// budget) and the DSA entry of "稀疏注意力速览（Sparse Attention，2019 ~ 2026）" (the
// indexer scores every earlier token, the top-k single tokens are kept).
//
//  * token_topk: one 1024-thread workgroup per (sequence, group, query row) selects the
//    `budget` causal tokens with the largest scores, ties to the lower position, by an
//    exact radix select over order-preserving uint32 keys (digits of 11, 11 and 10 bits,
//    LDS histograms, a block scan to find each digit), then a compaction pass writes the
//    chosen positions in ascending order.
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

__global__ void __launch_bounds__(kTkThreads) token_topk(Dims D, int budget, const float* __restrict__ tok,
                                                         int32_t* __restrict__ out) {
  __shared__ int hist[2048];
  __shared__ int wsum[kTkWaves];
  __shared__ int s_bin, s_above;
  const int64_t row = blockIdx.x;  // (s, g, t)
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
  int above = 0;      // keys already known to be > tau
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
    above += s_above;
    __syncthreads();
  }
  const uint32_t tau = prefix;  // keys > tau: `above` of them, all taken; keys == tau: the first `need`
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

template <int DH>
struct TokLds {
  float k[kChunk][DH + 1];  // padded: lane-per-key reads are conflict-free
  uint16_t v[kChunk][DH];
  int32_t pos[kChunk];
  float p[16][kChunk];       // per head (wave): probabilities
  float q[16][DH];
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
    for (int x = 0; x < 4; ++x) {
      L.k[j][cc + 2 * x] = bf16_to_f32((uint16_t)(wk[x] & 0xFFFFu));
      L.k[j][cc + 2 * x + 1] = bf16_to_f32((uint16_t)(wk[x] >> 16));
    }
    *reinterpret_cast<uint4*>(&L.v[j][cc]) = vv;
  }
  const int h = wave;  // one wave per query head of the group
  const uint16_t* qv = q + (((int64_t)s * D.T + t) * D.H + (int64_t)g * D.G + h) * DH;
  if (h < D.G)
    for (int cc = lane; cc < DH; cc += 64) L.q[h][cc] = bf16_to_f32(qv[cc]);
  __syncthreads();
  if (h >= D.G) return;
  float lg[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = lane + 64 * u;
    lg[u] = -INFINITY;
    if (L.pos[j] >= 0) {
      float acc = 0.0f;
      for (int cc = 0; cc < DH; ++cc) acc = fmaf(L.q[h][cc], L.k[j][cc], acc);
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

hipError_t launch_token_topk(const Dims& D, int budget, const float* tok, int32_t* sel_tok, hipStream_t st) {
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  LaunchScope scope("token_topk", st);
  hipLaunchKernelGGL(token_topk, dim3((unsigned)rows), dim3(kTkThreads), 0, st, D, budget, tok, sel_tok);
  return hipGetLastError();
}

size_t token_workspace_bytes(const Dims& D, int budget) {
  size_t total = 0;
  (void)token_layout(D, budget, nullptr, &total);
  return total;
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
