// synth_dev.hip -- device twin of synth/__init__.py's seeded input generator.
//
// Element (s, a, l, c) of a [S, A, L, D] tensor, flat index f:
//   v = TABLE[top16(splitmix64 output number f of stream (seed, tensor_id))]
// plus the optional structure of index queries / keys (boost channel,
// boosted blocks, rotary band planes read from a host-built table), added in
// float32 and rounded once to the storage dtype.  Generation only: nothing of
// the attention method is computed here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float32 -> OCP E4M3 code: round to nearest even, saturating at 448 (finite inputs).
// The same steps as synth.f32_to_e4m3 on the host.
__device__ __forceinline__ uint8_t f32_to_e4m3_rne(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    code = (uint32_t)(int)rintf(a * 512.0f);
  } else {
    const uint32_t au = __builtin_bit_cast(uint32_t, a);
    int e = (int)(au >> 23) - 127;
    const uint32_t mant = au & 0x7FFFFFu;
    uint32_t keep = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;
    if (keep == 8u) {
      keep = 0u;
      ++e;
    }
    code = min((uint32_t)(((e + 7) << 3) | (int)keep), 0x7Eu);
  }
  return (uint8_t)(code | sign);
}

struct FillArgs {
  void* dst;
  int dtype;  // 0 f32, 1 bf16, 2 OCP E4M3
  int64_t S, A, L, D;
  uint64_t key;
  const float* table;
  int kind;  // 0 iid, 1 index query, 2 index key
  int64_t pos_offset;
  float boost;
  int block;
  const uint8_t* mask;  // [S, A, nbb]
  int64_t nbb;
  const float* band;  // [positions, 16]
};

__global__ void __launch_bounds__(256) fill_kernel(FillArgs p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; f < n; f += stride) {
    const uint64_t z = mix64(p.key + (uint64_t)(f + 1) * 0x9E3779B97F4A7C15ull);
    float v = p.table[z >> 48];
    if (p.kind != 0) {
      const int64_t c = f % p.D;
      const int64_t l = (f / p.D) % p.L;
      const int64_t a = (f / (p.D * p.L)) % p.A;
      const int64_t s = f / (p.D * p.L * p.A);
      const int64_t pos = p.pos_offset + l;
      if (p.kind == 1 && c == 0) v = 1.0f;
      if (p.kind == 2 && c == 0 && p.mask != nullptr) {
        const int64_t blk = pos / p.block;
        if (p.mask[(s * p.A + a) * p.nbb + blk]) v = v + p.boost;
      }
      if (p.band != nullptr && c >= 1 && c <= 16) v = p.band[pos * 16 + (c - 1)];
    }
    if (p.dtype == 0)
      static_cast<float*>(p.dst)[f] = v;
    else if (p.dtype == 1)
      static_cast<uint16_t*>(p.dst)[f] = f32_to_bf16_rne(v);
    else
      static_cast<uint8_t*>(p.dst)[f] = f32_to_e4m3_rne(v);
  }
}

uint64_t host_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

// Returns 0 on success, else the hipError_t of the failed launch.
extern "C" int synth_fill(void* dst, int dtype, int64_t S, int64_t A, int64_t L, int64_t D,
                          uint64_t seed, int tensor_id, const float* table, int kind,
                          int64_t pos_offset, float boost, int block, const uint8_t* mask,
                          int64_t nbb, const float* band, void* stream) {
  FillArgs p;
  p.dst = dst;
  p.dtype = dtype;
  p.S = S; p.A = A; p.L = L; p.D = D;
  p.key = host_mix64(seed * 256ull + (uint64_t)tensor_id);
  p.table = table;
  p.kind = kind;
  p.pos_offset = pos_offset;
  p.boost = boost;
  p.block = block;
  p.mask = mask;
  p.nbb = nbb;
  p.band = band;
  const int64_t n = S * A * L * D;
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p, n);
  return (int)hipGetLastError();
}
