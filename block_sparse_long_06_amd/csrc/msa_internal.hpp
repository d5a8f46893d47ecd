// msa_internal.hpp -- shared declarations of libmsa's translation units.
// Host launchers are declared here; device helpers are inline below.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/msa.h"

namespace msa {

// Problem sizes after validation (host and device copy by value).
struct Dims {
  int S, T, N, H, Hkv, G, d, dI, B, k, nb;
  int pos0;      // N - T: absolute position of query row 0
  int dtype;     // msa_dtype
  float scale;   // main-branch logit scale (resolved, never 0)
  int kdtype;    // msa_dtype of k_idx (resolved: dtype or MSA_FP8_E4M3)
  // Cache layout of the per-sequence calls (null: dense [S, Hkv, N, .] caches, every
  // sequence N positions long).
  const int32_t* kv_lens;      // [S] device: sequence s holds positions 0 .. kv_lens[s]-1
  const int32_t* block_table;  // [S, bt_stride] device: page of logical block b, or null
  int bt_stride;
  int num_pages;               // pages of the pools [num_pages, Hkv, B, .]
};

// ----------------------------------------------------------------- profiler
// Brackets a launch with hipEvents when the profiler is enabled.
struct LaunchScope {
  LaunchScope(const char* name, hipStream_t s);
  ~LaunchScope();
  int slot;
  hipStream_t stream;
};

// ----------------------------------------------------------------- launchers
// Each returns hipSuccess or the error of its first failing launch.
hipError_t launch_index_scores(const Dims& D, const void* q_idx, const void* k_idx,
                               float* scores, hipStream_t st);
hipError_t launch_block_topk(const Dims& D, const float* scores, int32_t* sel, hipStream_t st);

size_t invert_workspace_bytes(const Dims& D);
hipError_t launch_invert(const Dims& D, const int32_t* sel, int32_t* offsets, int32_t* entries,
                         void* ws, hipStream_t st,
                         const uint64_t* hotmask = nullptr);

size_t prefill_workspace_bytes(const Dims& D);
// lse_out [S, T, H] and mass_out [S, Hkv, T, k] (both optional) are the training outputs.
hipError_t launch_prefill(const Dims& D, const void* q, const void* k, const void* v,
                          const int32_t* offsets, const int32_t* entries, const int32_t* sel,
                          void* out, void* ws, hipStream_t st, float* lse_out = nullptr,
                          float* mass_out = nullptr);

size_t decode_workspace_bytes(const Dims& D);

// Work list over an inverted selection (attention.hip): one item per (s, g, b) and run of
// at most R rows of its list, as int4 {(s*Hkv + g)*nb + b, first csr position, rows, 0}.
struct WorkList {
  int* items;
  int* itempos;
  int* n_items;
  void* scan_ws;
  int4* wl;
  int64_t ub;  // upper bound on the number of items
};
WorkList work_list_layout(const Dims& D, int R, void* base, size_t* total);
hipError_t launch_work_list(const Dims& D, const int32_t* off, int R, const WorkList& w, hipStream_t st);

// a1 + a2 fused (fused_topk.hip): selection without materialising the block scores.
size_t index_topk_workspace_bytes(const Dims& D);
hipError_t launch_index_topk(const Dims& D, const void* q_idx, const void* k_idx, int32_t* sel, void* ws,
                             hipStream_t st);

// Token-level selection (index_scores.hip, token.hip).
hipError_t launch_token_scores(const Dims& D, const void* q_idx, const void* k_idx, float* tok, hipStream_t st);
hipError_t launch_token_topk(const Dims& D, int budget, const float* tok, int32_t* sel_tok, void* ws,
                             hipStream_t st);
size_t token_topk_workspace_bytes(const Dims& D);
size_t token_workspace_bytes(const Dims& D, int budget);
hipError_t launch_token_attn(const Dims& D, int budget, const void* q, const void* k, const void* v,
                             const int32_t* sel_tok, void* out, void* ws, hipStream_t st);

// Training path (backward.hip).
size_t backward_workspace_bytes(const Dims& D);
hipError_t launch_attn_backward(const Dims& D, const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse, const int32_t* sel, const int32_t* off,
                                const int32_t* entries, float* dq, float* dk, float* dv, void* ws, hipStream_t st);
hipError_t launch_index_kl(const Dims& D, const float* scores, const int32_t* sel, const float* mass, float sigma,
                           float* loss, float* dscore, hipStream_t st);
size_t index_backward_workspace_bytes(const Dims& D);
hipError_t launch_index_backward(const Dims& D, const void* q_idx, const void* k_idx, const int32_t* off,
                                 const int32_t* entries, const float* dscore, float* dq_idx, float* dk_idx,
                                 int32_t* argmax, void* ws, hipStream_t st);
hipError_t launch_decode(const Dims& D, const void* q, const void* k, const void* v,
                         const int32_t* sel, void* out, void* ws, hipStream_t st);

// Shared by the prefill and decode paths: merge per-slot partials into out.  With
// hotmask (per row (s, t, g)), only the lowest hot slot of a row is read: it holds
// the row's partial over all of its hot blocks; the other hot slots are skipped.
hipError_t launch_lse_merge(const Dims& D, const int32_t* sel, const float* part_lse,
                            const void* part_o, int part_o_is_bf16, const uint64_t* hotmask, void* out,
                            hipStream_t st, const char* name, float* lse_out = nullptr,
                            float* mass_out = nullptr);

// Query-tile / Outer-Gather-Q split of a prefill selection (hot_tiles.hip).
constexpr int kHotTile = 128;            // query tile: one 128-position block
constexpr int kHotMax = 32;              // hot blocks kept per (sequence, group, tile)
constexpr int kHotStride = kHotMax + 1;  // {count, ids...} per (sequence, group, tile)
struct HotSplit {
  int ntiles;
  int32_t* hot;         // [S*Hkv, ntiles, kHotStride]
  int32_t* nhot;        // [S*Hkv, ntiles]: the count of each tile's list, contiguous
  int32_t* tiles;       // (s*Hkv + g)*ntiles + tile of every tile with shared blocks, in order
  int* ntile;           // their number
  uint64_t* hotmask;    // [S, T, Hkv]
  uint32_t* selbits;    // [S, T, Hkv]
  int32_t* cold_off;    // [S, Hkv, nb + 1]
  int32_t* cold_ent;    // [S*T*Hkv*k] capacity
  void* inv_ws;         // workspace of the inversion that builds the cold lists
};
int hot_num_tiles(const Dims& D);
HotSplit hot_split_layout(const Dims& D, void* base, size_t* total);
hipError_t launch_hot_split(const Dims& D, const int32_t* sel, const HotSplit& h, hipStream_t st);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ----------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {  // round to nearest even
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float ldf(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void stf(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void stf(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

// Wave64 reductions through cross-lane shuffles.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Length of sequence s: kv_lens[s] clamped to [T, N] (a device-side value outside the
// contract can never address memory outside the caller's buffers), N without kv_lens.
__device__ __forceinline__ int seq_len(const Dims& D, int s) {
  if (D.kv_lens == nullptr) return D.N;
  const int n = D.kv_lens[s];
  return n < D.T ? D.T : (n > D.N ? D.N : n);
}
// Absolute position of query row 0 of sequence s (its queries are its last T positions).
__device__ __forceinline__ int seq_pos0(const Dims& D, int s) { return seq_len(D, s) - D.T; }
// Element offset of cache row j of (sequence s, group g) in a cache of row width w: dense
// [S, Hkv, N, w], or the pool [num_pages, Hkv, B, w] through the block table (one page =
// one 128-position block).  -1 for a page id outside [0, num_pages): such rows read as 0.
__device__ __forceinline__ int64_t kv_row(const Dims& D, int s, int g, int j, int w) {
  if (D.block_table == nullptr) return (((int64_t)s * D.Hkv + g) * D.N + j) * w;
  const int page = D.block_table[(int64_t)s * D.bt_stride + (j >> 7)];
  if ((unsigned)page >= (unsigned)D.num_pages) return -1;
  return (((int64_t)page * D.Hkv + g) * 128 + (j & 127)) * w;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// An MFMA operand (8 bf16) read TRANSPOSED out of a row-major bf16 tile in LDS with
// gfx950's ds_read_b64_tr_b16: lane (n = lane % 32, half h = lane / 32) gets column
// col0 + n of rows r0 + {0..3} (elements 0..3) and r1 + {0..3} (elements 4..7); r0 and r1
// may depend on h.  The instruction works in groups of 16 lanes: destination lane i
// receives, as element j, the (i % 4)-th 16-bit value of the 8 bytes addressed by source
// lane 4 j + i / 4 (established with an in-bounds probe), so source lane s = 4 j + q
// addresses row r + j at columns col0 + 16 * (lane / 16 % 2) + 4 q .. + 3.  Addresses are
// 8-byte aligned when row_bytes and col0 are multiples of 8 bytes / 4 elements.
typedef __bf16 tr_bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ tr_bf16x8 tr_operand(const unsigned char* tile, int row_bytes, int r0, int r1, int col0,
                                                int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  const int sl = lane & 15, j = sl >> 2, q = sl & 3;
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * q;
  const lds_u8* t = (const lds_u8*)tile;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (r0 + j) * row_bytes + col * 2));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (r1 + j) * row_bytes + col * 2));
  const s16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(tr_bf16x8, ab);
}

}  // namespace msa
