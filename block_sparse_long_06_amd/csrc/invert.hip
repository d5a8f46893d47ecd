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
//              and a per-block running count carries ranks across steps, so every
//              list comes out in ascending row order.
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
  const int64_t e0 = (sg * D.T + t0) * D.k;
  const int64_t e1 = (sg * D.T + t1) * D.k;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += 256) {
    const int b = sel[e];
    const int64_t r = e / D.k;  // sg * T + t
    const int slot = (int)(e - r * D.k);
    const bool skip = (row_skip(D, hotmask, sg, (int)(r - sg * D.T)) >> slot) & 1ull;
    if (b >= 0 && b < D.nb && !skip) atomicAdd(&hist[b], 1);
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

// KR > 0: the row's k <= KR selections are read once into registers; KR == 0: any k,
// re-read from memory in each phase.  The chunk's per-block start positions are gathered
// into LDS first, so ranking an entry needs no memory access.
template <int KR>
__global__ void __launch_bounds__(64) invert_scatter(Dims D, const int32_t* __restrict__ sel,
                                                     const uint64_t* __restrict__ hotmask,
                                                     const int* __restrict__ pos,
                                                     int32_t* __restrict__ entries, int nchunks, int ct) {
  extern __shared__ unsigned char smem[];
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);
  int* base = reinterpret_cast<int*>(smem + sizeof(unsigned long long) * D.nb);
  uint16_t* run = reinterpret_cast<uint16_t*>(smem + (sizeof(unsigned long long) + sizeof(int)) * D.nb);
  const int lane = threadIdx.x;
  const int c = blockIdx.x;
  const int64_t sg = blockIdx.y;
  const int* pos_c = pos + (sg * D.nb) * nchunks + c;  // pos of (sg, b, c) = pos_c[b * nchunks]
  for (int b = lane; b < D.nb; b += 64) {
    mask[b] = 0ull;
    run[b] = 0;
    base[b] = pos_c[(int64_t)b * nchunks];
  }
  __syncthreads();
  const int t0 = c * ct;
  const int t1 = min(t0 + ct, D.T);
  const unsigned long long lower = (1ull << lane) - 1ull;
  const int k = KR > 0 ? KR : D.k;
  for (int tb = t0; tb < t1; tb += 64) {
    const int t = tb + lane;
    const int32_t* srow = sel + (sg * D.T + t) * D.k;
    const uint64_t skip = t < t1 ? row_skip(D, hotmask, sg, t) : 0ull;
    int bl[KR > 0 ? KR : 1];
    if constexpr (KR > 0) {
#pragma unroll
      for (int i = 0; i < KR; ++i) bl[i] = t < t1 && i < D.k && !((skip >> i) & 1ull) ? srow[i] : -1;
    }
    auto blk = [&](int i) { return KR > 0 ? bl[i] : (t < t1 && !((skip >> i) & 1ull) ? srow[i] : -1); };
    // phase 1: mark the lanes that chose each block
#pragma unroll
    for (int i = 0; i < k; ++i) {
      const int b = blk(i);
      if (b >= 0 && b < D.nb) atomicOr(&mask[b], 1ull << lane);
    }
    __syncthreads();
    // phase 2: rank among earlier lanes + running count -> global position
#pragma unroll
    for (int i = 0; i < k; ++i) {
      const int b = blk(i);
      if (b >= 0 && b < D.nb) {
        const unsigned long long m = mask[b];
        entries[base[b] + run[b] + __popcll(m & lower)] = t * D.k + i;
      }
    }
    __syncthreads();
    // phase 3: the lowest lane of each block advances its count and clears its mask
#pragma unroll
    for (int i = 0; i < k; ++i) {
      const int b = blk(i);
      if (b >= 0 && b < D.nb) {
        const unsigned long long m = mask[b];
        if ((m & lower) == 0ull) {
          run[b] = (uint16_t)(run[b] + __popcll(m));
          mask[b] = 0ull;
        }
      }
    }
    __syncthreads();
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
    hipLaunchKernelGGL(invert_count, dim3(nchunks, (unsigned)nsg), dim3(256), D.nb * sizeof(int), st, D,
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
    const size_t lds = (size_t)D.nb * (sizeof(unsigned long long) + sizeof(int) + sizeof(uint16_t));
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
