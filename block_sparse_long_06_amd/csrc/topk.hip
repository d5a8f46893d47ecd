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

// DPP row broadcasts: the last lane of one row of 16 to the next row(s).
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

// Wave-uniform maximum and minimum of a per-lane value: a butterfly inside each row
// of 16 lanes, then the row results carried to lane 63 by two row broadcasts.
__device__ __forceinline__ void wave_umax_umin(uint32_t a, uint32_t b, uint32_t& mx, uint32_t& mn) {
  a = max(a, dpp<kQuadSwap1>(a));
  b = min(b, dpp<kQuadSwap1>(b));
  a = max(a, dpp<kQuadSwap2>(a));
  b = min(b, dpp<kQuadSwap2>(b));
  a = max(a, dpp<kHalfRowMirror>(a));
  b = min(b, dpp<kHalfRowMirror>(b));
  a = max(a, dpp<kRowMirror>(a));
  b = min(b, dpp<kRowMirror>(b));
  // rows 1 and 3 take the row below; then rows 2 and 3 take row 1 (rows 0 and 2 of the
  // first step, rows 0 and 1 of the second keep their value)
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp((int)a, (int)a, kRowBcast15, 0xA, 0xF, false));
  b = min(b, (uint32_t)__builtin_amdgcn_update_dpp((int)b, (int)b, kRowBcast15, 0xA, 0xF, false));
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp((int)a, (int)a, kRowBcast31, 0xC, 0xF, false));
  b = min(b, (uint32_t)__builtin_amdgcn_update_dpp((int)b, (int)b, kRowBcast31, 0xC, 0xF, false));
  mx = __builtin_amdgcn_readlane(a, 63);
  mn = __builtin_amdgcn_readlane(b, 63);
}

constexpr int kQuadMirror = 0x1B;  // quad_perm [3,2,1,0]

// Compare-exchange between the lane pairs of a DPP pattern: lanes with keep_max take the
// larger key, their partners the smaller.
template <int CTRL>
__device__ __forceinline__ uint32_t cmpx(uint32_t x, bool keep_max) {
  const uint32_t p = dpp<CTRL>(x);
  return keep_max ? max(x, p) : min(x, p);
}

// Rotations within rows of 16 lanes: with row_ror:n lane i reads lane (i - n) mod 16.
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kRowRor12 = 0x12C;

// Compare-exchange with the lane at distance 4 inside the row (lane i ^ 4).
__device__ __forceinline__ uint32_t cmpx4(uint32_t x, bool keep_max, bool bit2) {
  const uint32_t up = dpp<kRowRor12>(x);  // lane i + 4 (mod 16)
  const uint32_t dn = dpp<kRowRor4>(x);   // lane i - 4 (mod 16)
  const uint32_t p = bit2 ? dn : up;
  return keep_max ? max(x, p) : min(x, p);
}

// The key of lane i ^ 16 (the neighbouring row, same position).  permlane16_swap trades
// the odd rows of its first operand for the even rows of its second; with both operands
// x, one result holds x and the other the neighbouring row's key, whichever is which.
__device__ __forceinline__ uint32_t row_partner(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return (uint32_t)r[0] ^ (uint32_t)r[1] ^ x;
}

// The need-th largest (1 <= need <= 16) of the keys in lanes 0..31.  Each row of 16
// lanes is sorted in descending lane order (bitonic merges in the flip form: quads, then
// halves, then the row); the 16 largest of rows 0 and 1 are the pairwise maxima of row 0
// against row 1 reversed, a bitonic sequence that four half-cleaner steps sort.
__device__ __forceinline__ uint32_t kth_of_32(uint32_t x, int lane, int need) {
  const bool b0 = (lane & 1) == 0, b1 = (lane & 2) == 0, b2 = (lane & 4) == 0, b3 = (lane & 8) == 0;
  x = cmpx<kQuadSwap1>(x, b0);
  x = cmpx<kQuadMirror>(x, b1);
  x = cmpx<kQuadSwap1>(x, b0);
  x = cmpx<kHalfRowMirror>(x, b2);
  x = cmpx<kQuadSwap2>(x, b1);
  x = cmpx<kQuadSwap1>(x, b0);
  x = cmpx<kRowMirror>(x, b3);
  x = cmpx4(x, b2, !b2);
  x = cmpx<kQuadSwap2>(x, b1);
  x = cmpx<kQuadSwap1>(x, b0);
  x = max(x, row_partner(dpp<kRowMirror>(x)));  // row 0: lane i against lane 31 - i
  x = cmpx<kRowRor8>(x, b3);                     // lane i ^ 8
  x = cmpx4(x, b2, !b2);
  x = cmpx<kQuadSwap2>(x, b1);
  x = cmpx<kQuadSwap1>(x, b0);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, need - 1);
}

// One key per lane (`live` lanes only; at least `want` of them), every live key in
// [lo, hi].  Returns x with #{live keys >= x} >= want and x <= the want-th largest live
// key: either that key itself, or a prefix of it that exactly `want` live keys reach
// (the search stops there: the prefix then separates the `want` largest from the
// rest).  The search runs over the bits below those that hi and lo share (every live
// key shares them too); its state is wave-uniform and stays on the scalar unit.
__device__ __forceinline__ uint32_t lane_kth_in(uint32_t key, bool live, int want, uint32_t hi, uint32_t lo) {
  const uint32_t diff = hi ^ lo;
  if (diff == 0u) return hi;
  const uint32_t top = 0x80000000u >> __builtin_clz(diff);
  uint32_t prefix = hi & ~(top + top - 1u);  // <= lo: every live key reaches it
  uint32_t k = live ? key : 0u;  // 0 never reaches a candidate (cand > 0)
  // one register holding the masked key: the compares below read it as is
  __asm__ volatile("" : "+v"(k));
  // two bits per pass (the exit is tested once per pass: a pass that starts with exactly
  // `want` keys at the prefix keeps it so; past bit 0 the second step re-tests the prefix)
  uint32_t b = top;
  do {
    uint32_t cand = prefix | b;
    const int c1 = __popcll(__ballot(k >= cand));
    prefix = c1 >= want ? cand : prefix;
    cand = prefix | (b >> 1);
    const int c2 = __popcll(__ballot(k >= cand));
    prefix = c2 >= want ? cand : prefix;
    b = (c1 == want || c2 == want) ? 0u : b >> 2;
  } while (b != 0u);
  return prefix;
}

__device__ __forceinline__ uint32_t lane_kth(uint32_t key, bool live, int want) {
  uint32_t hi, lo;
  wave_umax_umin(live ? key : 0u, live ? key : 0xFFFFFFFFu, hi, lo);
  return lane_kth_in(key, live, want, hi, lo);
}

// Candidate sources: element c (ascending c = ascending block id) -> (ord, id).
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

// Candidates held one per lane (lanes below C, in ascending id order, C >= need), every
// candidate key in [lo, hi]: writes the `need` best by (ord desc, id asc) to
// out[0 .. need-1] in ascending id order.
__device__ __forceinline__ void pick_from_lanes_in(uint32_t co, int32_t cid, bool have, int lane, int need,
                                                   int32_t* out, uint32_t hi, uint32_t lo, bool small) {
  // small (at most 32 candidates, need <= 16): tau is the need-th largest key, from a
  // sorting network; otherwise a bitwise search, which may stop at a prefix that exactly
  // `need` candidates reach (every candidate equal to tau is then taken below)
  const uint32_t tau = small ? kth_of_32(have ? co : 0u, lane, need) : lane_kth_in(co, have, need, hi, lo);
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

// The same for C candidates with no known key bounds.
__device__ __forceinline__ void pick_from_lanes(uint32_t co, int32_t cid, bool have, int lane, int need, int C,
                                                int32_t* out) {
  uint32_t hi = 0u, lo = 0u;
  const bool small = C <= 32 && need <= 16;
  if (!small) wave_umax_umin(have ? co : 0u, have ? co : 0xFFFFFFFFu, hi, lo);
  pick_from_lanes_in(co, cid, have, lane, need, out, hi, lo, small);
}

// Completes this wave's earlier LDS accesses before its later ones (lanes exchange data
// through LDS).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Writes the selection of a row from its candidates in LDS (values s_f[0 .. C-1] with ids
// s_id[...], ascending id order; C >= need; the buffer holds only the first kCap of them,
// so beyond kCap the row is read again from memory).  Every candidate key lies in
// [t1, hi].
__device__ __forceinline__ void select_candidates(const float* s_f, const int32_t* s_id, int C, const float* sc,
                                                  int n, int lane, int need, uint32_t hi, uint32_t t1,
                                                  int32_t* out) {
  if (C <= 64) {
    const bool have = lane < C;
    pick_from_lanes_in(have ? ord_key(s_f[lane]) : 0u, have ? s_id[lane] : 0, have, lane, need, out, hi, t1,
                       C <= 32 && need <= 16);
  } else if (C <= kCap) {
    LdsFloatSrc src{s_f, s_id, C};
    select_and_write(src, lane, need, out);
  } else {
    RowSrc src{sc, n};
    select_and_write(src, lane, need, out);
  }
}

// Appends the scores of one 64-wide segment (element id0 + lane) that pass `f` to the
// candidate buffer in ascending id order.  Positions wrap at kCap: past kCap candidates
// the buffer is not read.
__device__ __forceinline__ void append_candidates(bool f, float v, int id, int lane, float* s_f, int32_t* s_id,
                                                  int& C) {
  const uint64_t m = __ballot(f);
  if (m != 0ull) {
    const int p = (C + lanes_below(m)) & (kCap - 1);
    if (f) {
      s_f[p] = v;
      s_id[p] = id;
    }
    C += __popcll(m);
  }
}

// Grid: (ceil(T / kWaves), S * H_kv) when T >= kWaves (the workgroup's rows share the
// sequence and group: no integer division per row), else (ceil(rows / kWaves)).
// VEC: rows start 16-byte aligned (nb % 4 == 0), so each lane fetches 4 consecutive
// scores per load; the row is then re-distributed through LDS so that lane l holds
// blocks l, l + 64, ... (the layout the ascending-id compaction below relies on).
template <bool VEC>
__global__ void __launch_bounds__(kWaves * 64) block_topk_kernel(Dims D, const float* __restrict__ scores,
                                                                  int32_t* __restrict__ sel) {
  __shared__ __attribute__((aligned(16))) uint32_t s_buf[kWaves][2 * kCap];  // row staging / candidates
  float* const s_f = reinterpret_cast<float*>(s_buf[threadIdx.x >> 6]);
  int32_t* const s_id_w = reinterpret_cast<int32_t*>(s_buf[threadIdx.x >> 6] + kCap);
  // the wave index is uniform: the row's index arithmetic runs on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int t, sg;
  if (D.T >= kWaves) {
    t = (int)blockIdx.x * kWaves + wave;
    sg = (int)blockIdx.y;
    if (t >= D.T) return;
  } else {
    // rows < 2^32 (checked at launch): 32-bit division
    const int64_t r = (int64_t)blockIdx.x * kWaves + wave;
    if (r >= (int64_t)D.S * D.Hkv * D.T) return;
    t = (int)((uint32_t)r % (uint32_t)D.T);
    sg = (int)((uint32_t)r / (uint32_t)D.T);
  }
  const int64_t row = (int64_t)sg * D.T + t;
  const int p0 = D.kv_lens != nullptr ? seq_pos0(D, sg / D.Hkv) : D.pos0;
  const int bt = (p0 + t) >> 7;  // blocks of 128 positions
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
    float o[kRegPerLane];
    if (VEC) {
      static_assert(2 * kCap >= 64 * kRegPerLane, "row staging fits the candidate buffer");
      // every load is issued before the first store, none under a branch: out-of-row
      // lanes re-read the row's first four scores (in bounds) and store -inf instead
      float4 x[kRegPerLane / 4];
#pragma unroll
      for (int i = 0; i < kRegPerLane / 4; ++i) {
        const int c = i * 256 + 4 * lane;
        x[i] = *reinterpret_cast<const float4*>(sc + (c < n ? c : 0));
      }
#pragma unroll
      for (int i = 0; i < kRegPerLane / 4; ++i) {
        const int c = i * 256 + 4 * lane;
        if (!(c < n)) x[i] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        *reinterpret_cast<float4*>(&s_f[c]) = x[i];
      }
      wave_lds_sync();
      if (lane < ((4 - (n & 3)) & 3)) s_f[n + lane] = -INFINITY;  // the row's last, partial float4
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < kRegPerLane; ++i) o[i] = s_f[i * 64 + lane];
      wave_lds_sync();  // the staging area takes the candidates next
    } else {
#pragma unroll
      for (int i = 0; i < kRegPerLane; ++i) {
        const int c = i * 64 + lane;
        o[i] = sc[c < n ? c : 0];  // all loads in flight; out-of-row lanes masked below
      }
#pragma unroll
      for (int i = 0; i < kRegPerLane; ++i)
        if (!(i * 64 + lane < n)) o[i] = -INFINITY;
    }
    float lmf = o[0];
#pragma unroll
    for (int i = 1; i < kRegPerLane; ++i) lmf = fmaxf(lmf, o[i]);
    // lanes past the row's end hold no element; the others number min(n, 64) > need
    const bool live = lane < n;
    const uint32_t lk = ord_key(lmf);
    uint32_t hi, lo;
    wave_umax_umin(live ? lk : 0u, live ? lk : 0xFFFFFFFFu, hi, lo);
    const uint32_t t1 = lane_kth_in(lk, live, need, hi, lo);
    const float t1f = ord_inv(t1);
    if (t1f > -INFINITY) {  // otherwise -inf (or NaN) scores reach the threshold: the row from memory
      // candidates (value >= t1) compacted in ascending id order; -inf padding never passes
      int C = 0;
#pragma unroll
      for (int i = 0; i < kRegPerLane; ++i) append_candidates(o[i] >= t1f, o[i], i * 64 + lane, lane, s_f, s_id_w, C);
      select_candidates(s_f, s_id_w, C, sc, n, lane, need, hi, t1, out);
    } else {
      RowSrc src{sc, n};
      select_and_write(src, lane, need, out);
    }
    if (lane == 0) out[need] = bt;
    return;
  }
  // A. lane maxima over a share of the row (any split works: only the maxima matter),
  // in the float domain; whole chunks with four loads in flight per lane, then the rest
  float lmf = -INFINITY;
  if (VEC) {
    constexpr int kU = 4;
    int c0 = 0;
    for (; c0 + kU * 256 <= n; c0 += kU * 256) {
      float4 x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) x[u] = *reinterpret_cast<const float4*>(sc + c0 + u * 256 + 4 * lane);
#pragma unroll
      for (int u = 0; u < kU; ++u) lmf = fmaxf(lmf, fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w)));
    }
    for (; c0 < n; c0 += 256) {
      const int c = c0 + 4 * lane;  // c < n keeps c + 3 < nb (rows are a multiple of 4 long)
      const float4 x = *reinterpret_cast<const float4*>(sc + (c < n ? c : 0));
      if (c < n) lmf = fmaxf(lmf, x.x);
      if (c + 1 < n) lmf = fmaxf(lmf, x.y);
      if (c + 2 < n) lmf = fmaxf(lmf, x.z);
      if (c + 3 < n) lmf = fmaxf(lmf, x.w);
    }
  } else {
    constexpr int kU = 4;
    int i0 = 0;
    for (; i0 + kU * 64 <= n; i0 += kU * 64) {
      float x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) x[u] = sc[i0 + u * 64 + lane];
#pragma unroll
      for (int u = 0; u < kU; ++u) lmf = fmaxf(lmf, x[u]);
    }
    for (; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      const float x = sc[i < n ? i : 0];
      if (i < n) lmf = fmaxf(lmf, x);
    }
  }
  // B. t1 <= the need-th largest lane maximum (every lane holds elements: n > 1024);
  // scores >= t1 compacted into LDS in ascending id order, eight loads in flight per lane
  const uint32_t lk = ord_key(lmf);
  uint32_t hi, lo;
  wave_umax_umin(lk, lk, hi, lo);
  const uint32_t t1 = lane_kth_in(lk, true, need, hi, lo);
  const float t1f = ord_inv(t1);
  if (!(t1f > -INFINITY)) {  // -inf (or NaN) scores reach the threshold: the row from memory
    RowSrc src{sc, n};
    select_and_write(src, lane, need, out);
    if (lane == 0) out[need] = bt;
    return;
  }
  constexpr int kV = 8;
  int C = 0;
  int b0 = 0;
  for (; b0 + kV * 64 <= n; b0 += kV * 64) {
    float o[kV];
#pragma unroll
    for (int u = 0; u < kV; ++u) o[u] = sc[b0 + u * 64 + lane];
#pragma unroll
    for (int u = 0; u < kV; ++u) append_candidates(o[u] >= t1f, o[u], b0 + u * 64 + lane, lane, s_f, s_id_w, C);
  }
  for (; b0 < n; b0 += 64) {
    const int i = b0 + lane;
    const float v = sc[i < n ? i : 0];
    append_candidates(i < n && v >= t1f, v, i, lane, s_f, s_id_w, C);
  }
  select_candidates(s_f, s_id_w, C, sc, n, lane, need, hi, t1, out);
  if (lane == 0) out[need] = bt;  // the own block is the largest id of the row
}

// Long rows and few of them (decode: one row per (sequence, group), ~8K past blocks): one
// 1024-thread workgroup per row reads the whole row in one pass, 8 consecutive scores per
// thread (ids 8 tid .. 8 tid + 7), as order keys (0 = not eligible).
//   1. each wave's threshold tau_w <= the need-th largest of its 512 keys (lane maxima,
//      lane_kth); tau = the largest tau_w is still <= the row's need-th largest key, so
//      every selected block has key >= tau;
//   2. the keys >= tau are compacted into LDS in ascending id order (a scan of the
//      per-thread counts inside each wave, then the wave totals);
//   3. wave 0 holds the candidates in registers (candidate c in slot c / 64 of lane c % 64,
//      so slot-major order is id order), finds the need-th largest key by a radix search
//      over them, takes every larger key and, among keys equal to it, the lowest ids.
//      More than kLongCap candidates (ties at the threshold) fall back to the row in memory.
constexpr int kLongThreads = 1024;
constexpr int kLongWaves = kLongThreads / 64;
constexpr int kLongPer = 8;
constexpr int kLongCap = 1024;
constexpr int kLongSlots = kLongCap / 64;
constexpr int64_t kLongRows = 16384;  // up to 16K rows (workgroups of 16 waves)

// 3. (one wave) the need-th largest of C > 64 candidates held in LDS in ascending id
// order, NS per lane (candidate c in slot c / 64 of lane c % 64, so slot-major order is id
// order, NS * 64 >= C): a radix search for its key, then every larger key and, among keys
// equal to it, the lowest ids.  Empty slots hold key 0, which no candidate prefix reaches,
// so no slot needs a guard.
template <int NS>
__device__ __forceinline__ void long_select(const uint32_t* s_ord, const int32_t* s_id, int C, int lane, int need,
                                            int32_t* out) {
  uint32_t ck[NS];
  int32_t ci[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int cc = lane + 64 * u;
    ck[u] = cc < C ? s_ord[cc] : 0u;
    ci[u] = cc < C ? s_id[cc] : 0;
  }
  // prefix: the need-th largest candidate key, or a prefix of it that exactly `need`
  // candidates reach (the search then stops: it separates them from the rest).  The
  // search runs below the high bits every candidate shares.
  uint32_t hi = 0u, lo = 0xFFFFFFFFu;
#pragma unroll
  for (int u = 0; u < NS; ++u)
    if (lane + 64 * u < C) {
      hi = max(hi, ck[u]);
      lo = min(lo, ck[u]);
    }
  uint32_t whi, wlo;
  wave_umax_umin(hi, lo, whi, wlo);
  uint32_t prefix = whi;
  if (whi != wlo) {
    const int top = 31 - __builtin_clz(whi ^ wlo);
    prefix = whi & ~((2u << top) - 1u);  // <= every candidate
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < NS; ++u) cnt += __popcll(__ballot(ck[u] >= cand));
      if (cnt >= need) {
        prefix = cand;
        if (cnt == need) break;
      }
    }
  }
  int c_gt = 0;
#pragma unroll
  for (int u = 0; u < NS; ++u) c_gt += __popcll(__ballot(ck[u] > prefix));
  const int need_eq = need - c_gt;  // >= 0 (0 when the search stopped between keys)
  int pos = 0, eq_seen = 0;
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const bool eq = ck[u] == prefix;
    const uint64_t meq = __ballot(eq);
    const bool f = ck[u] > prefix || (eq && eq_seen + lanes_below(meq) < need_eq);
    const uint64_t m = __ballot(f);
    const int at = pos + lanes_below(m);
    if (f && at < need) out[at] = ci[u];
    pos += __popcll(m);
    eq_seen += __popcll(meq);
  }
}

template <bool VEC>
__global__ void __launch_bounds__(kLongThreads) block_topk_long(Dims D, const float* __restrict__ scores,
                                                               int32_t* __restrict__ sel) {
  __shared__ uint32_t s_ord[kLongCap];
  __shared__ int32_t s_id[kLongCap];
  __shared__ uint32_t s_tau[kLongWaves];
  __shared__ int s_cnt[kLongWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t r32 = blockIdx.x;
  const int t = (int)(r32 % (uint32_t)D.T);
  const int bt = (seq_pos0(D, (int)(r32 / ((uint32_t)D.Hkv * (uint32_t)D.T))) + t) / D.B;
  const int k = D.k;
  int32_t* out = sel + (int64_t)r32 * k;
  const int n = bt;
  const int need = k - 1;
  if (need >= n) {  // uniform over the workgroup
    for (int i = tid; i < k; i += kLongThreads) out[i] = i <= bt ? i : -1;
    return;
  }
  if (need == 0) {
    if (tid == 0) out[0] = bt;
    return;
  }
  const float* sc = scores + (int64_t)r32 * D.nb;
  const int base = kLongPer * tid;
  uint32_t key[kLongPer];
  if (VEC) {
    // base is a multiple of 4 and rows are a multiple of 4 long: base < n keeps base + 3
    // inside the row, base + 4 < n keeps base + 7 inside it
    const float4 a = *reinterpret_cast<const float4*>(sc + (base < n ? base : 0));
    const float4 b = *reinterpret_cast<const float4*>(sc + (base + 4 < n ? base + 4 : 0));
    const float v[kLongPer] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int u = 0; u < kLongPer; ++u) key[u] = base + u < n ? ord_key(v[u]) : 0u;
  } else {
    float v[kLongPer];
#pragma unroll
    for (int u = 0; u < kLongPer; ++u) v[u] = sc[base + u < n ? base + u : 0];
#pragma unroll
    for (int u = 0; u < kLongPer; ++u) key[u] = base + u < n ? ord_key(v[u]) : 0u;
  }
  uint32_t lm = key[0];
#pragma unroll
  for (int u = 1; u < kLongPer; ++u) lm = max(lm, key[u]);
  // 1. wave threshold (0 when fewer than `need` lanes of the wave hold eligible blocks)
  const bool live = base < n;
  const int nlive = __popcll(__ballot(live));
  const uint32_t tau_w = nlive >= need ? lane_kth(lm, live, need) : 0u;
  if (lane == 0) s_tau[wave] = tau_w;
  __syncthreads();
  uint32_t tau = 0u;
#pragma unroll
  for (int w = 0; w < kLongWaves; ++w) tau = max(tau, s_tau[w]);
  // 2. candidates (eligible keys are > 0), ascending id order
  int c = 0;
#pragma unroll
  for (int u = 0; u < kLongPer; ++u) c += (key[u] != 0u && key[u] >= tau) ? 1 : 0;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(incl, o, 64);
    if (lane >= o) incl += x;
  }
  if (lane == 63) s_cnt[wave] = incl;
  __syncthreads();
  int wbase = 0, C = 0;
#pragma unroll
  for (int w = 0; w < kLongWaves; ++w) {
    const int x = s_cnt[w];
    wbase += w < wave ? x : 0;
    C += x;
  }
  int p = wbase + incl - c;
#pragma unroll
  for (int u = 0; u < kLongPer; ++u) {
    if (key[u] != 0u && key[u] >= tau) {
      if (p < kLongCap) {
        s_ord[p] = key[u];
        s_id[p] = base + u;
      }
      ++p;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  if (C > kLongCap) {  // heavy ties at the threshold: the row from memory
    RowSrc src{sc, n};
    select_and_write(src, lane, need, out);
  } else if (C <= 64) {
    const bool have = lane < C;
    pick_from_lanes(have ? s_ord[lane] : 0u, have ? s_id[lane] : 0, have, lane, need, C, out);
  } else if (C <= 4 * 64) {
    long_select<4>(s_ord, s_id, C, lane, need, out);
  } else {
    long_select<kLongSlots>(s_ord, s_id, C, lane, need, out);
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
  // long rows and too few of them to fill the chip one wave each: a workgroup per row
  if (D.nb > 64 * kRegPerLane && rows <= kLongRows) {
    if (vec)
      hipLaunchKernelGGL(block_topk_long<true>, dim3((unsigned)rows), dim3(kLongThreads), 0, st, D, scores, sel);
    else
      hipLaunchKernelGGL(block_topk_long<false>, dim3((unsigned)rows), dim3(kLongThreads), 0, st, D, scores, sel);
    return hipGetLastError();
  }
  // S * H_kv <= 65535 (checked with the problem)
  const dim3 g2 = D.T >= kWaves ? dim3((unsigned)((D.T + kWaves - 1) / kWaves), (unsigned)(D.S * D.Hkv))
                                : dim3((unsigned)grid);
  if (vec)
    hipLaunchKernelGGL(block_topk_kernel<true>, g2, dim3(kWaves * 64), 0, st, D, scores, sel);
  else
    hipLaunchKernelGGL(block_topk_kernel<false>, g2, dim3(kWaves * 64), 0, st, D, scores, sel);
  return hipGetLastError();
}

}  // namespace msa
