// invert.hip -- a3: inversion of the per-query block selections into per-(sequence,
// group, block) lists of query rows: the index behind the Outer-Gather-Q order of
// page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比", section
// Kernel 创新：Outer Gather Q (KV block as the outer loop; gather every query that
// chose the block).
//
// A stable counting sort, deterministic (no order depends on timing):
//  1. count:   per chunk of `ct` query rows of one (s, g), an LDS histogram over
//              blocks, stored as cnt[(sg, b, chunk)] (chunk fastest);
//  2. scan:    exclusive prefix sum over cnt in (sg, b, chunk) order = the global
//              position of the first entry of each (sg, b, chunk);
//  3. offsets: csr_offsets[sg, b] = position of (sg, b, chunk 0);
//  4. scatter: one wave per chunk walks its rows 64 at a time (lane = row).  For
//              each block, a 64-bit LDS mask of the lanes that chose it gives each
//              lane its rank among the earlier lanes (popcount of the lower bits),
//              and a per-block LDS word holding the list position of the block's next
//              entry carries ranks across steps, so every list comes out in ascending
//              row order.
#include "msa_internal.hpp"
#include "scan.hpp"

namespace msa {
namespace {

// Query rows per chunk: 256 .. 1024, the largest power of two that still gives about
// 2048 chunks (one wave each in the scatter: the ranking is latency-bound, so it wants
// many waves; larger chunks mean fewer counts to scan and fewer masks to clear).
int chunk_rows(const Dims& D) {
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  int c = 256;
  while (c < 1024 && rows / (2 * c) >= 2048) c *= 2;
  return c;
}

// An entry whose slot bit is set in its row's mask (hotmask [S, T, Hkv], nullable) is left
// out: the same inversion then builds the list of the remaining entries only.
__device__ __forceinline__ uint64_t row_skip(const Dims& D, const uint64_t* hotmask, int64_t sg, int t) {
  if (hotmask == nullptr) return 0ull;
  const int64_t s = sg / D.Hkv, g = sg % D.Hkv;
  return hotmask[(s * D.T + t) * D.Hkv + g];
}

// The k <= KR selections of a row, -1 beyond k or where ok is false.
template <int KR>
__device__ __forceinline__ void row_load(const Dims& D, const int32_t* srow, bool ok, int (&bl)[KR]) {
  if (KR % 4 == 0 && (D.k & 3) == 0 && (reinterpret_cast<uintptr_t>(srow) & 15) == 0) {
    // 16-byte loads: the row starts 16-byte aligned and holds whole groups of four
#pragma unroll
    for (int i = 0; i < KR / 4; ++i) {
      const int4 v = ok && 4 * i < D.k ? reinterpret_cast<const int4*>(srow)[i] : make_int4(-1, -1, -1, -1);
      bl[4 * i] = v.x;
      bl[4 * i + 1] = v.y;
      bl[4 * i + 2] = v.z;
      bl[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < KR; ++i) bl[i] = ok && i < D.k ? srow[i] : -1;
  }
}

// Rows hold distinct block ids (msa_block_topk's rows do).  A repeated id is outside
// that contract; its later slots are dropped here, by the count and the scatter alike,
// so that every list position the count reserves is written.  A row that is strictly
// ascending up to its first negative entry, and negative after it (the form both top-k
// paths emit), has no repeat, and skips the pairwise check.  Skipped slots become -1.
template <int KR>
__device__ __forceinline__ void row_clean(uint64_t skip, int (&bl)[KR]) {
  bool asc = true;
#pragma unroll
  for (int i = 1; i < KR; ++i) asc = asc && ((bl[i] > bl[i - 1] && bl[i - 1] >= 0) || bl[i] < 0);
  if (!asc) {
#pragma unroll
    for (int i = 1; i < KR; ++i) {
      bool rep = false;
#pragma unroll
      for (int j = 0; j < i; ++j) rep |= bl[j] == bl[i];
      if (rep) bl[i] = -1;
    }
  }
#pragma unroll
  for (int i = 0; i < KR; ++i)
    if ((skip >> i) & 1ull) bl[i] = -1;
}

// Slot i of a row held in memory (any k): its block, or -1 if skipped, out of range or
// a repeat of an earlier slot.
__device__ __forceinline__ int row_block_at(const Dims& D, const int32_t* srow, uint64_t skip, int i) {
  const int b = srow[i];
  if (b < 0 || b >= D.nb) return -1;
  for (int j = 0; j < i; ++j)
    if (srow[j] == b) return -1;
  return ((skip >> i) & 1ull) ? -1 : b;
}

// LDS update for block b of every lane with ok set, where lanes that share the first
// pending lane's block (up to two such groups of at least four) are served by one update
// of their group's leader: in one slot of consecutive rows the sink, the own block and the
// band blocks are usually one block for most lanes, whose individual atomics would
// serialise on one address.  upd(b, m) applies the update for block b and lane mask m.
template <typename Upd>
__device__ __forceinline__ void peeled_update(int b, bool ok, Upd upd) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const uint64_t pend = __ballot(ok);
    if (pend == 0ull) return;
    const int v = __builtin_amdgcn_readlane(b, __builtin_ctzll(pend));
    const uint64_t m = __ballot(ok && b == v);
    if (__popcll(m) < 4) break;
    if (lane == __builtin_ctzll(m)) upd(v, m);
    ok = ok && b != v;
  }
  if (ok) upd(b, 1ull << lane);
}

// One thread per query row of the chunk.
template <int KR>
__global__ void __launch_bounds__(256) invert_count(Dims D, const int32_t* __restrict__ sel,
                                                    const uint64_t* __restrict__ hotmask,
                                                    int* __restrict__ cnt, int nchunks, int ct) {
  extern __shared__ int hist[];
  const int c = blockIdx.x;
  const int64_t sg = blockIdx.y;
  for (int b = threadIdx.x; b < D.nb; b += 256) hist[b] = 0;
  __syncthreads();
  const int t0 = c * ct;
  const int t1 = min(t0 + ct, D.T);
  if constexpr (KR > 0) {
    // every row of this thread (ct <= 4 * 256) loaded before the first update
    constexpr int kMaxR = 4;
    int bl[kMaxR][KR];
    uint64_t sk[kMaxR];
#pragma unroll
    for (int r = 0; r < kMaxR; ++r) {
      const int t = t0 + (int)threadIdx.x + 256 * r;
      const bool ok = 256 * r < ct && t < t1;
      row_load<KR>(D, sel + (sg * D.T + (ok ? t : t0)) * D.k, ok, bl[r]);
      sk[r] = ok ? row_skip(D, hotmask, sg, t) : 0ull;
    }
#pragma unroll
    for (int r = 0; r < kMaxR; ++r) {
      if (256 * r >= ct) break;
      row_clean<KR>(sk[r], bl[r]);
      if (hotmask == nullptr) {  // the full selection: shared blocks are common in a slot
#pragma unroll
        for (int i = 0; i < KR; ++i)
          peeled_update(bl[r][i], bl[r][i] >= 0 && bl[r][i] < D.nb,
                        [&](int b, uint64_t m) { atomicAdd(&hist[b], __popcll(m)); });
      } else {  // the tile-shared entries are skipped: what remains rarely coincides
#pragma unroll
        for (int i = 0; i < KR; ++i)
          if (bl[r][i] >= 0 && bl[r][i] < D.nb) atomicAdd(&hist[bl[r][i]], 1);
      }
    }
  } else {
    for (int t = t0 + (int)threadIdx.x; t < t1; t += 256) {
      const int32_t* srow = sel + (sg * D.T + t) * D.k;
      const uint64_t skip = row_skip(D, hotmask, sg, t);
      for (int i = 0; i < D.k; ++i) {
        const int b = row_block_at(D, srow, skip, i);
        if (b >= 0) atomicAdd(&hist[b], 1);
      }
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < D.nb; b += 256) cnt[(sg * D.nb + b) * nchunks + c] = hist[b];
}

__global__ void __launch_bounds__(256) invert_offsets(Dims D, const int* __restrict__ pos,
                                                      const int* __restrict__ total,
                                                      int32_t* __restrict__ offsets, int nchunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nsg = (int64_t)D.S * D.Hkv;
  if (i >= nsg * (D.nb + 1)) return;
  const int64_t sg = i / (D.nb + 1);
  const int b = (int)(i % (D.nb + 1));
  int v;
  if (b < D.nb)
    v = pos[(sg * D.nb + b) * nchunks];
  else
    v = sg + 1 < nsg ? pos[((sg + 1) * D.nb) * nchunks] : *total;
  offsets[i] = v;
}

// KR > 0: the row's k <= KR selections are read once into registers (the next step's
// while this one is ranked); KR == 0: any k, re-read from memory in each phase.  Per
// block the LDS holds the lane mask of the current step and `at`, the list position of
// the block's next entry (the chunk's start position, gathered first, plus the entries
// already placed), so ranking an entry needs no memory access.
template <int KR>
__global__ void __launch_bounds__(64) invert_scatter(Dims D, const int32_t* __restrict__ sel,
                                                     const uint64_t* __restrict__ hotmask,
                                                     const int* __restrict__ pos,
                                                     int32_t* __restrict__ entries, int nchunks, int ct) {
  extern __shared__ unsigned char smem[];
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);
  int* at = reinterpret_cast<int*>(smem + sizeof(unsigned long long) * D.nb);
  const int lane = threadIdx.x;
  const int c = blockIdx.x;
  const int64_t sg = blockIdx.y;
  const int* pos_c = pos + (sg * D.nb) * nchunks + c;  // pos of (sg, b, c) = pos_c[b * nchunks]
  for (int b = lane; b < D.nb; b += 64) {
    mask[b] = 0ull;
    at[b] = pos_c[(int64_t)b * nchunks];
  }
  __syncthreads();
  const int t0 = c * ct;
  const int t1 = min(t0 + ct, D.T);
  const unsigned long long lower = (1ull << lane) - 1ull;
  int nx[KR > 0 ? KR : 1];
  uint64_t nskip = 0ull;
  auto fetch = [&](int tb) {
    if constexpr (KR > 0) {
      const int t = tb + lane;
      const bool ok = t < t1;
      row_load<KR>(D, sel + (sg * D.T + (ok ? t : t0)) * D.k, ok, nx);
      nskip = ok ? row_skip(D, hotmask, sg, t) : 0ull;
    }
  };
  fetch(t0);
  for (int tb = t0; tb < t1; tb += 64) {
    const int t = tb + lane;
    if constexpr (KR > 0) {
      int bl[KR];
#pragma unroll
      for (int i = 0; i < KR; ++i) bl[i] = nx[i];
      const uint64_t sk = nskip;
      if (tb + 64 < t1) fetch(tb + 64);
      row_clean<KR>(sk, bl);
      // phase 1: mark the lanes that chose each block
#pragma unroll
      for (int i = 0; i < KR; ++i)
        if (bl[i] >= 0 && bl[i] < D.nb) atomicOr(&mask[bl[i]], 1ull << lane);
      __syncthreads();
      // phase 2: rank among the earlier lanes -> list position; mask and position kept
      unsigned long long m[KR];
      int p[KR];
#pragma unroll
      for (int i = 0; i < KR; ++i) {
        m[i] = 0ull;
        p[i] = 0;
        if (bl[i] >= 0 && bl[i] < D.nb) {
          m[i] = mask[bl[i]];
          p[i] = at[bl[i]];
          entries[p[i] + __popcll(m[i] & lower)] = t * D.k + i;
        }
      }
      __syncthreads();
      // phase 3: the lowest lane of each block advances its position and clears its mask
#pragma unroll
      for (int i = 0; i < KR; ++i) {
        if (bl[i] >= 0 && bl[i] < D.nb && (m[i] & lower) == 0ull) {
          at[bl[i]] = p[i] + __popcll(m[i]);
          mask[bl[i]] = 0ull;
        }
      }
      __syncthreads();
    } else {
      const int32_t* srow = sel + (sg * D.T + t) * D.k;
      const uint64_t skip = t < t1 ? row_skip(D, hotmask, sg, t) : 0ull;
      auto blk = [&](int i) { return t < t1 ? row_block_at(D, srow, skip, i) : -1; };
      for (int i = 0; i < D.k; ++i) {
        const int b = blk(i);
        if (b >= 0) atomicOr(&mask[b], 1ull << lane);
      }
      __syncthreads();
      for (int i = 0; i < D.k; ++i) {
        const int b = blk(i);
        if (b >= 0) entries[at[b] + __popcll(mask[b] & lower)] = t * D.k + i;
      }
      __syncthreads();
      // a lane that reads a mask its block's leader already cleared adds nothing
      for (int i = 0; i < D.k; ++i) {
        const int b = blk(i);
        if (b >= 0) {
          const unsigned long long mm = mask[b];
          if ((mm & lower) == 0ull) {
            atomicAdd(&at[b], __popcll(mm));
            mask[b] = 0ull;
          }
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace

static int invert_chunks(const Dims& D) { return (D.T + chunk_rows(D) - 1) / chunk_rows(D); }

size_t invert_workspace_bytes(const Dims& D) {
  const int64_t m = (int64_t)D.S * D.Hkv * D.nb * invert_chunks(D);
  return 2 * align_up((size_t)m * sizeof(int), 256) + align_up(sizeof(int), 256) +
         scan_workspace_bytes(m);
}

// With a skip mask the kernels are timed under the cold_* names (the tile split's lists).
hipError_t launch_invert(const Dims& D, const int32_t* sel, int32_t* offsets, int32_t* entries,
                         void* ws, hipStream_t st, const uint64_t* hotmask) {
  const int nchunks = invert_chunks(D);
  const int64_t nsg = (int64_t)D.S * D.Hkv;
  const int64_t m = nsg * D.nb * nchunks;
  unsigned char* w = static_cast<unsigned char*>(ws);
  int* cnt = reinterpret_cast<int*>(w);
  w += align_up((size_t)m * sizeof(int), 256);
  int* pos = reinterpret_cast<int*>(w);
  w += align_up((size_t)m * sizeof(int), 256);
  int* total = reinterpret_cast<int*>(w);
  w += align_up(sizeof(int), 256);
  void* scan_ws = w;
  {
    LaunchScope s(hotmask ? "cold_count" : "invert_count", st);
    if (D.k <= 16)
      hipLaunchKernelGGL(invert_count<16>, dim3(nchunks, (unsigned)nsg), dim3(256), D.nb * sizeof(int), st, D,
                         sel, hotmask, cnt, nchunks, chunk_rows(D));
    else
      hipLaunchKernelGGL(invert_count<0>, dim3(nchunks, (unsigned)nsg), dim3(256), D.nb * sizeof(int), st, D,
                         sel, hotmask, cnt, nchunks, chunk_rows(D));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_exclusive_scan(cnt, pos, m, total, scan_ws, st);
  if (e != hipSuccess) return e;
  {
    const int64_t n = nsg * (D.nb + 1);
    LaunchScope s(hotmask ? "cold_offsets" : "invert_offsets", st);
    hipLaunchKernelGGL(invert_offsets, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, D, pos, total,
                       offsets, nchunks);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    const size_t lds = (size_t)D.nb * (sizeof(unsigned long long) + sizeof(int));
    const void* kern = D.k <= 16 ? reinterpret_cast<const void*>(invert_scatter<16>)
                                 : reinterpret_cast<const void*>(invert_scatter<0>);
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    LaunchScope s(hotmask ? "cold_scatter" : "invert_scatter", st);
    if (D.k <= 16)
      hipLaunchKernelGGL(invert_scatter<16>, dim3(nchunks, (unsigned)nsg), dim3(64), lds, st, D, sel, hotmask,
                         pos, entries, nchunks, chunk_rows(D));
    else
      hipLaunchKernelGGL(invert_scatter<0>, dim3(nchunks, (unsigned)nsg), dim3(64), lds, st, D, sel, hotmask,
                         pos, entries, nchunks, chunk_rows(D));
  }
  return hipGetLastError();
}

}  // namespace msa
