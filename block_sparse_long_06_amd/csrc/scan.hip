// scan.hip -- device-wide exclusive prefix sum of int32 counts (three launches:
// tile sums, a one-workgroup scan of the tile sums, tile-local scans).  Used to
// turn per-(group, block, chunk) counts into list positions.
#include "msa_internal.hpp"
#include "scan.hpp"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 8;
constexpr int kTile = kThreads * kItems;
constexpr int kTopThreads = 1024;

// Inclusive scan over a wave64.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Exclusive scan across the workgroup; returns the workgroup total in *total.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* total) {
  __shared__ int wsum[NT / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v, lane);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int s = wsum[w];
    if (w < wave) before += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

__global__ void __launch_bounds__(kThreads) scan_tile_sums(const int* __restrict__ in, int64_t n,
                                                           int* __restrict__ tile_sum) {
  const int64_t base = (int64_t)blockIdx.x * kTile;
  int s = 0;
#pragma unroll
  for (int u = 0; u < kItems; ++u) {
    const int64_t i = base + (int64_t)u * kThreads + threadIdx.x;
    if (i < n) s += in[i];
  }
  int tot;
  (void)block_excl_scan<kThreads>(s, &tot);
  if (threadIdx.x == 0) tile_sum[blockIdx.x] = tot;
}

__global__ void __launch_bounds__(kTopThreads) scan_top(int* __restrict__ tile_sum, int64_t ntiles,
                                                        int* __restrict__ total) {
  int carry = 0;
  for (int64_t base = 0; base < ntiles; base += kTopThreads) {
    const int64_t i = base + threadIdx.x;
    const int v = i < ntiles ? tile_sum[i] : 0;
    int tot;
    const int ex = block_excl_scan<kTopThreads>(v, &tot);
    if (i < ntiles) tile_sum[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0 && total != nullptr) *total = carry;
}

__global__ void __launch_bounds__(kThreads) scan_apply(const int* __restrict__ in, int64_t n,
                                                       const int* __restrict__ tile_off,
                                                       int* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kItems;
  int v[kItems];
  int s = 0;
#pragma unroll
  for (int u = 0; u < kItems; ++u) {
    v[u] = base + u < n ? in[base + u] : 0;
    s += v[u];
  }
  int tot;
  int run = block_excl_scan<kThreads>(s, &tot) + tile_off[blockIdx.x];
#pragma unroll
  for (int u = 0; u < kItems; ++u) {
    if (base + u < n) out[base + u] = run;
    run += v[u];
  }
}

}  // namespace

size_t scan_workspace_bytes(int64_t n) {
  const int64_t ntiles = (n + kTile - 1) / kTile;
  return align_up((size_t)(ntiles > 0 ? ntiles : 1) * sizeof(int), 256);
}

hipError_t launch_exclusive_scan(const int* in, int* out, int64_t n, int* total, void* ws,
                                 hipStream_t st) {
  const int64_t ntiles = (n + kTile - 1) / kTile;
  int* tile = static_cast<int*>(ws);
  if (ntiles > 0) {
    LaunchScope s1("scan_tile_sums", st);
    hipLaunchKernelGGL(scan_tile_sums, dim3((unsigned)ntiles), dim3(kThreads), 0, st, in, n, tile);
  }
  {
    LaunchScope s2("scan_top", st);
    hipLaunchKernelGGL(scan_top, dim3(1), dim3(kTopThreads), 0, st, tile, ntiles, total);
  }
  if (ntiles > 0) {
    LaunchScope s3("scan_apply", st);
    hipLaunchKernelGGL(scan_apply, dim3((unsigned)ntiles), dim3(kThreads), 0, st, in, n, tile, out);
  }
  return hipGetLastError();
}

}  // namespace msa
