// topk.hip -- a2: per-(sequence, group, query) block selection with the own block
// forced.  Page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比", section
// 第一步：粗筛 item 3 (16 blocks, the current position's block always chosen, the
// rest by score) and the head-pattern appendix (the own block is the only forced
// rule); MSA entry of "稀疏注意力速览（Sparse Attention，2019 ~ 2026）".
//
// One wave64 per row.  The order key of a block is (score desc, id asc); scores
// are mapped to order-preserving uint32 ("ord"), with -0 folded onto +0 so they
// tie as IEEE values do.  Selecting the `need = k-1` best of n = b_t blocks:
//   A. every lane keeps the max ord of its strided share of the row;
//   B. tau1 = a lower bound of the need-th largest lane maximum with at least
//      `need` lane maxima >= tau1 (bitwise radix search with wave ballots).  At
//      least `need` scores are >= tau1, so every selected block is >= tau1; those
//      candidates are compacted into LDS in ascending id order;
//   C. tau = the need-th largest ord among the candidates (same radix search),
//      or a value that exactly `need` candidates reach; blocks with ord > tau are
//      taken, and among ord == tau the lowest ids fill the remaining places;
//   D. the taken ids are compacted in ascending order and the own block appended.
// The register searches start below the high bits that every key shares (a wave
// max / min) and stop as soon as exactly `need` keys reach the prefix.
// If more than kCap candidates pass step B (heavy ties), steps C-D read the row
// from memory instead of LDS: slower, same result.
#include "msa_internal.hpp"

namespace msa {
namespace {

constexpr int kWaves = 4;
constexpr int kCap = 512;
constexpr int kRegPerLane = 16;  // rows of up to 1024 blocks are held in registers

__device__ __forceinline__ uint32_t ord_key(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u << 1) == 0u) u = 0u;  // -0 and +0 are the same value
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of ord_key (ord_key(ord_inv(o)) == o for every o that ord_key produces).
__device__ __forceinline__ float ord_inv(uint32_t o) {
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Lane exchange within rows of 16 lanes (DPP); every lane of the wave is active here.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kHalfRowMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Wave-uniform maximum and minimum of a per-lane value: a butterfly inside each row
// of 16 lanes, then the four row results.
__device__ __forceinline__ void wave_umax_umin(uint32_t a, uint32_t b, uint32_t& mx, uint32_t& mn) {
  a = max(a, dpp<kQuadSwap1>(a));
  b = min(b, dpp<kQuadSwap1>(b));
  a = max(a, dpp<kQuadSwap2>(a));
  b = min(b, dpp<kQuadSwap2>(b));
  a = max(a, dpp<kHalfRowMirror>(a));
  b = min(b, dpp<kHalfRowMirror>(b));
  a = max(a, dpp<kRowMirror>(a));
  b = min(b, dpp<kRowMirror>(b));
  const uint32_t a0 = __builtin_amdgcn_readlane(a, 0), a1 = __builtin_amdgcn_readlane(a, 16);
  const uint32_t a2 = __builtin_amdgcn_readlane(a, 32), a3 = __builtin_amdgcn_readlane(a, 48);
  const uint32_t b0 = __builtin_amdgcn_readlane(b, 0), b1 = __builtin_amdgcn_readlane(b, 16);
  const uint32_t b2 = __builtin_amdgcn_readlane(b, 32), b3 = __builtin_amdgcn_readlane(b, 48);
  mx = max(max(a0, a1), max(a2, a3));
  mn = min(min(b0, b1), min(b2, b3));
}

// One key per lane (`live` lanes only; at least `want` of them).  Returns x with
// #{live keys >= x} >= want and x <= the want-th largest live key: either that key
// itself, or a prefix of it that exactly `want` live keys reach (the search stops
// there: the prefix then separates the `want` largest from the rest).  The search
// runs over the bits below those that every live key shares.
__device__ __forceinline__ uint32_t lane_kth(uint32_t key, bool live, int want) {
  uint32_t hi, lo;
  wave_umax_umin(live ? key : 0u, live ? key : 0xFFFFFFFFu, hi, lo);
  const uint32_t diff = hi ^ lo;
  if (diff == 0u) return hi;
  const int top = 31 - __builtin_clz(diff);
  uint32_t prefix = hi & ~((2u << top) - 1u);  // <= lo: every live key reaches it
  const uint32_t k = live ? key : 0u;          // 0 never reaches a candidate (cand > 0)
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    const int c = __popcll(__ballot(k >= cand));
    if (c >= want) {
      prefix = cand;
      if (c == want) break;
    }
  }
  return prefix;
}

// Candidate sources: element c (ascending c = ascending block id) -> (ord, id).
struct LdsSrc {
  const uint32_t* ord;
  const int32_t* id;
  int n;
  __device__ uint32_t key(int c) const { return ord[c]; }
  __device__ int32_t idx(int c) const { return id[c]; }
};
struct LdsFloatSrc {
  const float* val;
  const int32_t* id;
  int n;
  __device__ uint32_t key(int c) const { return ord_key(val[c]); }
  __device__ int32_t idx(int c) const { return id[c]; }
};
struct RowSrc {
  const float* sc;
  int n;
  __device__ uint32_t key(int c) const { return ord_key(sc[c]); }
  __device__ int32_t idx(int c) const { return c; }
};

// Largest x with #{elements e : f(e) >= x} >= want, where f(e) = key (mode 0) or
// (key == tau ? ~id : 0) (mode 1).  Requires at least `want` elements.
template <class Src>
__device__ __forceinline__ uint32_t radix_kth(const Src& src, int lane, int want, int mode, uint32_t tau) {
  uint32_t prefix = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    int cnt = 0;
    for (int base = 0; base < src.n; base += 64) {
      const int c = base + lane;
      bool f = false;
      if (c < src.n) {
        const uint32_t o = src.key(c);
        const uint32_t v = mode == 0 ? o : (o == tau ? ~(uint32_t)src.idx(c) : 0u);
        f = v >= cand;
      }
      cnt += __popcll(__ballot(f));
    }
    if (cnt >= want) prefix = cand;
  }
  return prefix;
}

template <class Src>
__device__ __forceinline__ void select_and_write(const Src& src, int lane, int need, int32_t* out) {
  const uint32_t tau = radix_kth(src, lane, need, 0, 0u);
  int c_gt = 0, c_eq = 0;
  for (int base = 0; base < src.n; base += 64) {
    const int c = base + lane;
    const uint32_t o = c < src.n ? src.key(c) : 0u;
    c_gt += __popcll(__ballot(c < src.n && o > tau));
    c_eq += __popcll(__ballot(c < src.n && o == tau));
  }
  const int need_eq = need - c_gt;  // 1 <= need_eq <= c_eq
  uint32_t iota = 0xFFFFFFFFu;      // ties with id <= iota are taken
  if (need_eq < c_eq) iota = ~radix_kth(src, lane, need_eq, 1, tau);
  int pos = 0;
  for (int base = 0; base < src.n; base += 64) {
    const int c = base + lane;
    bool f = false;
    int32_t id = 0;
    if (c < src.n) {
      const uint32_t o = src.key(c);
      id = src.idx(c);
      f = o > tau || (o == tau && (uint32_t)id <= iota);
    }
    const uint64_t m = __ballot(f);
    const int at = pos + lanes_below(m);
    if (f && at < need) out[at] = id;  // exactly `need` are flagged; the bound is insurance
    pos += __popcll(m);
  }
}

// Candidates held one per lane (lanes below C, in ascending id order, C >= need):
// writes the `need` best by (ord desc, id asc) to out[0 .. need-1] in ascending id order.
__device__ __forceinline__ void pick_from_lanes(uint32_t co, int32_t cid, bool have, int lane, int need,
                                                int32_t* out) {
  // when the search stops early exactly `need` candidates are >= tau and every one
  // equal to tau is taken below
  const uint32_t tau = lane_kth(co, have, need);
  const int c_gt = __popcll(__ballot(have && co > tau));
  const uint64_t eqm = __ballot(have && co == tau);
  const int need_eq = need - c_gt;
  // ties at tau: the lowest ids win; candidates are in ascending id order, so the
  // first need_eq set bits of eqm are taken
  uint64_t take_eq = eqm;
  for (int drop = __popcll(eqm) - need_eq; drop > 0; --drop) take_eq &= ~(1ull << (63 - __builtin_clzll(take_eq)));
  const bool f = have && (co > tau || ((take_eq >> lane) & 1ull));
  const uint64_t m = __ballot(f);
  const int at = lanes_below(m);
  if (f && at < need) out[at] = cid;
}

// Completes this wave's earlier LDS accesses before its later ones (lanes exchange data
// through LDS).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// VEC: rows start 16-byte aligned (nb % 4 == 0), so each lane fetches 4 consecutive
// scores per load; the row is then re-distributed through LDS so that lane l holds
// blocks l, l + 64, ... (the layout the ascending-id compaction below relies on).
template <bool VEC>
__global__ void __launch_bounds__(kWaves * 64) block_topk_kernel(Dims D, const float* __restrict__ scores,
                                                                  int32_t* __restrict__ sel) {
  __shared__ __attribute__((aligned(16))) uint32_t s_buf[kWaves][2 * kCap];  // row staging / candidates
  uint32_t* const s_ord_w = s_buf[threadIdx.x >> 6];
  int32_t* const s_id_w = reinterpret_cast<int32_t*>(s_buf[threadIdx.x >> 6] + kCap);
  // the wave index is uniform: the row's index arithmetic runs on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  if (row >= rows) return;
  // rows < 2^32 (checked at launch): 32-bit division
  const uint32_t r32 = (uint32_t)row;
  const int t = (int)(r32 % (uint32_t)D.T);
  const int bt = (seq_pos0(D, (int)(r32 / ((uint32_t)D.Hkv * (uint32_t)D.T))) + t) / D.B;
  const int k = D.k;
  int32_t* out = sel + row * k;
  const int n = bt;        // eligible blocks other than the own one: 0 .. bt-1
  const int need = k - 1;  // how many of them are taken
  if (need >= n) {         // budget covers every causal block
    for (int i = lane; i < k; i += 64) out[i] = i <= bt ? i : -1;
    return;
  }
  if (need == 0) {         // k == 1: the own block alone
    if (lane == 0) out[0] = bt;
    return;
  }
  const float* sc = scores + row * (int64_t)D.nb;
  if (n <= 64 * kRegPerLane) {
    // Fast path: the row lives in registers (element i*64 + lane in slot i), compared
    // as IEEE floats (the same order as ord_key, -0 == +0 included); only the lane
    // maxima and the candidates are mapped to ord_key for the bitwise searches.
    // Elements at n and beyond are -inf.
    float* const s_f = reinterpret_cast<float*>(s_ord_w);  // row staging: the whole candidate buffer
    const int ni = (n + 63) >> 6;                           // 64-element segments holding the row
    float o[kRegPerLane];
    if (VEC) {
      static_assert(2 * kCap >= 64 * kRegPerLane, "row staging fits the candidate buffer");
      // every load is issued before the first store, none under a branch: out-of-row
      // lanes re-read the row's first four scores (in bounds) and store them past the
      // row's end, where the -inf tail below or nothing reads them
      float4 x[kRegPerLane / 4];
#pragma unroll
      for (int i = 0; i < kRegPerLane / 4; ++i) {
        const int c = i * 256 + 4 * lane;
        x[i] = *reinterpret_cast<const float4*>(sc + (c < n ? c : 0));
      }
#pragma unroll
      for (int i = 0; i < kRegPerLane / 4; ++i) *reinterpret_cast<float4*>(&s_f[i * 256 + 4 * lane]) = x[i];
      wave_lds_sync();
      if (n + lane < ni * 64) s_f[n + lane] = -INFINITY;  // tail of the last segment
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < kRegPerLane; ++i) o[i] = i < ni ? s_f[i * 64 + lane] : -INFINITY;
      wave_lds_sync();  // the staging area takes the candidates next
    } else {
#pragma unroll
      for (int i = 0; i < kRegPerLane; ++i) {
        const int c = i * 64 + lane;
        o[i] = sc[c < n ? c : 0];  // all loads in flight; out-of-row lanes masked below
      }
#pragma unroll
      for (int i = 0; i < kRegPerLane; ++i)
        if (!(i < ni && i * 64 + lane < n)) o[i] = -INFINITY;
    }
    float lmf = o[0];
#pragma unroll
    for (int i = 1; i < kRegPerLane; ++i) lmf = fmaxf(lmf, o[i]);
    // lanes past the row's end hold no element; the others number min(n, 64) > need
    const uint32_t t1 = lane_kth(ord_key(lmf), lane < n, need);
    const float t1f = ord_inv(t1);
    if (t1f > -INFINITY) {  // otherwise -inf scores reach the threshold: generic path below
      // candidates (value >= t1) compacted in ascending id order; -inf padding never passes
      int C = 0;
#pragma unroll
      for (int i = 0; i < kRegPerLane; ++i) {
        if (i < ni) {
          const bool f = o[i] >= t1f;
          const uint64_t m = __ballot(f);
          if (m != 0ull) {
            const int p = C + lanes_below(m);
            if (f && p < kCap) {
              s_f[p] = o[i];
              s_id_w[p] = i * 64 + lane;
            }
            C += __popcll(m);
          }
        }
      }
      if (C <= 64) {
        const bool have = lane < C;
        pick_from_lanes(have ? ord_key(s_f[lane]) : 0u, have ? s_id_w[lane] : 0, have, lane, need, out);
        if (lane == 0) out[need] = bt;
        return;
      }
      if (C <= kCap) {
        LdsFloatSrc src{s_f, s_id_w, C};
        select_and_write(src, lane, need, out);
        if (lane == 0) out[need] = bt;
        return;
      }
    }
    RowSrc src{sc, n};
    select_and_write(src, lane, need, out);
    if (lane == 0) out[need] = bt;
    return;
  }
  // A. lane maxima over a share of the row (any split works: only the maxima matter);
  // four loads in flight per lane
  constexpr int kU = 4;
  uint32_t lmax = 0;
  if (VEC) {
    for (int c0 = 4 * lane; c0 < n; c0 += kU * 256) {
      float4 x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + u * 256;  // c < n keeps c + 3 < nb (rows are a multiple of 4 long)
        x[u] = *reinterpret_cast<const float4*>(sc + (c < n ? c : 0));
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + u * 256;
        const uint32_t a = c < n ? ord_key(x[u].x) : 0u;
        const uint32_t b = c + 1 < n ? ord_key(x[u].y) : 0u;
        const uint32_t d = c + 2 < n ? ord_key(x[u].z) : 0u;
        const uint32_t e = c + 3 < n ? ord_key(x[u].w) : 0u;
        lmax = max(max(lmax, a), max(b, max(d, e)));
      }
    }
  } else {
    for (int i0 = lane; i0 < n; i0 += kU * 64) {
      uint32_t o[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) o[u] = ord_key(sc[i0 + u * 64 < n ? i0 + u * 64 : 0]);
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (i0 + u * 64 >= n) o[u] = 0u;
#pragma unroll
      for (int u = 0; u < kU; ++u) lmax = max(lmax, o[u]);
    }
  }
  // B. tau1 <= the need-th largest lane maximum (every lane holds elements: n > 1024);
  // compact ord >= tau1 into LDS (ascending id), eight loads in flight per lane
  const uint32_t tau1 = lane_kth(lmax, true, need);
  constexpr int kV = 8;
  int C = 0;
  for (int b0 = 0; b0 < n; b0 += kV * 64) {
    uint32_t o[kV];
#pragma unroll
    for (int u = 0; u < kV; ++u) {
      const int i = b0 + u * 64 + lane;
      o[u] = ord_key(sc[i < n ? i : 0]);  // out-of-row lanes are masked below
    }
#pragma unroll
    for (int u = 0; u < kV; ++u) {
      const int i = b0 + u * 64 + lane;
      const bool f = i < n && o[u] >= tau1;
      const uint64_t m = __ballot(f);
      const int p = C + lanes_below(m);
      if (f && p < kCap) {
        s_ord_w[p] = o[u];
        s_id_w[p] = i;
      }
      C += __popcll(m);
    }
  }
  if (C <= 64) {
    const bool have = lane < C;
    pick_from_lanes(have ? s_ord_w[lane] : 0u, have ? s_id_w[lane] : 0, have, lane, need, out);
  } else if (C <= kCap) {
    LdsSrc src{s_ord_w, s_id_w, C};
    select_and_write(src, lane, need, out);
  } else {
    RowSrc src{sc, n};
    select_and_write(src, lane, need, out);
  }
  if (lane == 0) out[need] = bt;  // the own block is the largest id of the row
}

}  // namespace

hipError_t launch_block_topk(const Dims& D, const float* scores, int32_t* sel, hipStream_t st) {
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  const int64_t grid = (rows + kWaves - 1) / kWaves;
  if (rows > (int64_t)UINT32_MAX || (int64_t)D.Hkv * D.T > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
  LaunchScope scope(D.T == 1 ? "block_topk_t1" : "block_topk", st);
  const bool vec = D.nb % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15u) == 0;
  if (vec)
    hipLaunchKernelGGL(block_topk_kernel<true>, dim3((unsigned)grid), dim3(kWaves * 64), 0, st, D, scores, sel);
  else
    hipLaunchKernelGGL(block_topk_kernel<false>, dim3((unsigned)grid), dim3(kWaves * 64), 0, st, D, scores, sel);
  return hipGetLastError();
}

}  // namespace msa
