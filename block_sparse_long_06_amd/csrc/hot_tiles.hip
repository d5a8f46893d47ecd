// hot_tiles.hip -- split of the prefill selection into query-tile ("hot") blocks and
// Outer-Gather-Q ("cold") pairs.
//
// The pages' head-pattern appendix (page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA
// 四方案深度对比") shows that neighbouring queries choose largely the same blocks: the
// diagonal (own and adjacent blocks), the sink and per-group stripes.  A block chosen by
// most rows of one 128-position query tile is cheaper to process tile-wise -- the tile's
// Q rows stay on chip while the block streams past once, and the row keeps ONE partial
// for all such blocks -- than to gather every row's Q again and write one partial per
// (row, block).  The remaining (row, block) pairs keep the Outer-Gather-Q order of
// section Kernel 创新：Outer Gather Q.  Both halves compute exact block-restricted
// softmax terms, so the merged result is the same exact attention.
//
// Query tile tau = absolute positions [128 tau, 128 tau + 127] intersected with the
// query rows [N - T, N).  A block b is hot for (s, g, tau) when at least half of the
// tile's rows, and at least kHotMinRows rows, selected it; at most kHotMax hot blocks
// are kept, taken in descending id order so the tile's own block (chosen by every row)
// always stays.  A tile with fewer than kHotMinBlocks such blocks (typically its own
// block alone) keeps all its pairs on the Outer-Gather-Q path.  Outputs, per row (s, t, g):
//   hotmask  uint64: bit slot set if sel[s,g,t,slot] is a hot block of the row's tile;
//   selbits  uint32: bit i set if the row selected hot block i of its tile;
// per (s, g, tau): hot list {count, ids...} (kHotStride ints).
// The cold CSR -- the selection inversion of the entries whose slot bit is clear, in the
// same format and order as the full inversion (flat (s, g, b) offsets, ascending rows) --
// is built afterwards by the inversion kernels themselves, with hotmask as their skip mask
// (the tile kernel needs only the outputs above, so it can start before that).
#include "msa_internal.hpp"

namespace msa {
namespace {

constexpr int kHotMinRows = 32;
constexpr int kHotMinBlocks = 2;
constexpr int kMaxNb = 8192;  // dynamic LDS of the histogram: nb <= kMaxNb

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Rows [t_lo, t_end) of query tile `ti` (0-based from the tile holding row 0).
__device__ __forceinline__ void tile_rows(const Dims& D, int ti, int& t_lo, int& t_end) {
  const int tau = D.pos0 / kHotTile + ti;
  t_lo = max(tau * kHotTile, D.pos0) - D.pos0;
  t_end = min(tau * kHotTile + kHotTile, D.N) - D.pos0;
}

// One workgroup per (s, g, tile): block histogram of the tile's selections in LDS
// (dynamic: nb counts, then -- for k <= 16 -- the tile's selections themselves, row pitch
// k | 1 so that one row per lane reads without bank conflicts, and the row pass needs no
// second global read).  The flattened (row, slot) loads keep a wave's 64 histogram
// updates on at most four rows.  The hot blocks are found in descending id order by the
// four waves at once, each over a quarter of the blocks, then concatenated.
__global__ void __launch_bounds__(256) hot_select(Dims D, const int32_t* __restrict__ sel,
                                                  int32_t* __restrict__ hot, int32_t* __restrict__ nhot,
                                                  uint64_t* __restrict__ hotmask, uint32_t* __restrict__ selbits,
                                                  int ntiles) {
  extern __shared__ int smem[];
  int* hist = smem;
  int* rowsel = smem + D.nb;
  __shared__ int s_hot[4][kHotMax];
  __shared__ int s_cnt[4];
  __shared__ int s_list[kHotMax];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ti = blockIdx.x;
  const int64_t sg = blockIdx.y;
  const int s = (int)(sg / D.Hkv), g = (int)(sg % D.Hkv);
  int t_lo, t_end;
  tile_rows(D, ti, t_lo, t_end);
  const int rows = t_end - t_lo;
  const int32_t* srow = sel + (sg * D.T + t_lo) * D.k;
  const bool active = rows >= kHotMinRows;
  const bool cached = D.k <= 16;
  const int kp = D.k | 1;
  int nh = 0;
  if (active) {  // uniform over the workgroup
    for (int b = tid; b < D.nb; b += 256) hist[b] = 0;
    __syncthreads();
    const int n = rows * D.k;
    const int dr = 256 / D.k, ds = 256 % D.k;
    int r = tid / D.k, sl = tid % D.k;
    for (int i = tid; i < n; i += 256) {
      const int b = srow[i];
      if (cached) rowsel[r * kp + sl] = b;
      if (b >= 0 && b < D.nb) atomicAdd(&hist[b], 1);
      r += dr;
      sl += ds;
      if (sl >= D.k) {
        sl -= D.k;
        ++r;
      }
    }
    __syncthreads();
    const int thr = max(kHotMinRows, (rows + 1) / 2);
    const int q = ((D.nb + 3) / 4 + 63) / 64 * 64;  // blocks per wave, a multiple of 64
    int nw = 0;
    for (int j = 0; j < q && nw < kHotMax; j += 64) {
      const int bb = D.nb - 1 - wave * q - j - lane;
      const bool f = bb >= 0 && hist[bb] >= thr;
      const uint64_t m = __ballot(f);
      const int at = nw + lanes_below(m);
      if (f && at < kHotMax) s_hot[wave][at] = bb;
      nw += __popcll(m);
    }
    if (lane == 0) s_cnt[wave] = min(nw, kHotMax);
    __syncthreads();
    const int total = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
    // a tile whose only shared block is its own is left to Outer-Gather-Q: staging one
    // block per workgroup slice costs more than it saves
    nh = total >= kHotMinBlocks ? min(total, kHotMax) : 0;
    if (tid < nh) {
      int w = 0, off = 0;
      while (tid >= off + s_cnt[w]) {
        off += s_cnt[w];
        ++w;
      }
      const int bh = s_hot[w][tid - off];
      s_list[tid] = bh;
      hist[bh] = -1 - tid;  // hot index, negated
    }
    __syncthreads();
  }
  for (int r = tid; r < rows; r += 256) {
    uint64_t hm = 0;
    uint32_t sb = 0;
    if (nh > 0) {
      for (int slot = 0; slot < D.k; ++slot) {
        const int b = cached ? rowsel[r * kp + slot] : srow[r * D.k + slot];
        if (b >= 0 && b < D.nb) {
          const int x = hist[b];
          if (x < 0) {
            hm |= 1ull << slot;
            sb |= 1u << (-1 - x);
          }
        }
      }
    }
    const int64_t row = ((int64_t)s * D.T + t_lo + r) * D.Hkv + g;
    hotmask[row] = hm;
    selbits[row] = sb;
  }
  if (tid <= kHotMax) hot[(sg * ntiles + ti) * kHotStride + tid] = tid == 0 ? nh : (tid - 1 < nh ? s_list[tid - 1] : -1);
  if (tid == 0) nhot[sg * ntiles + ti] = nh;
}

// One workgroup lists, in (s, g, tile) order, the tiles that have shared blocks: each
// thread takes 8 consecutive tile counts per round (two 16-byte loads, all issued before
// the scan).
__global__ void __launch_bounds__(1024) hot_compact(const int32_t* __restrict__ nhot, int64_t ntot,
                                                    int32_t* __restrict__ tiles, int* __restrict__ count) {
  constexpr int kPer = 8;
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int run = 0;
  for (int64_t base = 0; base < ntot; base += 1024 * kPer) {
    const int64_t i0 = base + (int64_t)threadIdx.x * kPer;
    int nv[kPer];
    if (i0 + kPer <= ntot) {  // nhot is 256-byte aligned and i0 a multiple of 8
      const int4 a = *reinterpret_cast<const int4*>(nhot + i0);
      const int4 b = *reinterpret_cast<const int4*>(nhot + i0 + 4);
      nv[0] = a.x; nv[1] = a.y; nv[2] = a.z; nv[3] = a.w;
      nv[4] = b.x; nv[5] = b.y; nv[6] = b.z; nv[7] = b.w;
    } else {
#pragma unroll
      for (int u = 0; u < kPer; ++u) nv[u] = i0 + u < ntot ? nhot[i0 + u] : 0;
    }
    bool f[kPer];
    int c = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      f[u] = nv[u] > 0;
      c += f[u] ? 1 : 0;
    }
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int x = __shfl_up(incl, o, 64);
      if (lane >= o) incl += x;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int p = run + incl - c, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int x = wsum[w];
      p += w < wave ? x : 0;
      tot += x;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (f[u]) tiles[p++] = (int32_t)(i0 + u);
    run += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) *count = run;
}

}  // namespace

int hot_num_tiles(const Dims& D) { return (D.N - 1) / kHotTile - D.pos0 / kHotTile + 1; }

HotSplit hot_split_layout(const Dims& D, void* base, size_t* total) {
  const int64_t rows = (int64_t)D.S * D.T * D.Hkv;
  const int64_t npart = rows * D.k;
  const int64_t nflat = (int64_t)D.S * D.Hkv * (D.nb + 1);
  unsigned char* p = static_cast<unsigned char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* r = p ? p + off : nullptr;
    off += align_up(bytes, 256);
    return r;
  };
  HotSplit h{};
  h.ntiles = hot_num_tiles(D);
  h.hot = static_cast<int32_t*>(take((size_t)D.S * D.Hkv * h.ntiles * kHotStride * sizeof(int32_t)));
  h.nhot = static_cast<int32_t*>(take((size_t)D.S * D.Hkv * h.ntiles * sizeof(int32_t)));
  h.tiles = static_cast<int32_t*>(take((size_t)D.S * D.Hkv * h.ntiles * sizeof(int32_t)));
  h.ntile = static_cast<int*>(take(sizeof(int)));
  h.hotmask = static_cast<uint64_t*>(take(rows * sizeof(uint64_t)));
  h.selbits = static_cast<uint32_t*>(take(rows * sizeof(uint32_t)));
  h.cold_off = static_cast<int32_t*>(take(nflat * sizeof(int32_t)));
  h.cold_ent = static_cast<int32_t*>(take(npart * sizeof(int32_t)));
  h.inv_ws = take(invert_workspace_bytes(D));
  *total = off;
  return h;
}

hipError_t launch_hot_split(const Dims& D, const int32_t* sel, const HotSplit& h, hipStream_t st) {
  if (D.nb > kMaxNb) return hipErrorInvalidValue;
  {
    LaunchScope s("hot_select", st);
    const size_t lds = ((size_t)D.nb + (D.k <= 16 ? (size_t)kHotTile * (D.k | 1) : 0)) * sizeof(int);
    hipLaunchKernelGGL(hot_select, dim3((unsigned)h.ntiles, (unsigned)(D.S * D.Hkv)), dim3(256), lds, st, D, sel,
                       h.hot, h.nhot, h.hotmask, h.selbits, h.ntiles);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    LaunchScope s("hot_compact", st);
    hipLaunchKernelGGL(hot_compact, dim3(1), dim3(1024), 0, st, h.nhot, (int64_t)D.S * D.Hkv * h.ntiles, h.tiles,
                       h.ntile);
  }
  return hipGetLastError();
}

}  // namespace msa
