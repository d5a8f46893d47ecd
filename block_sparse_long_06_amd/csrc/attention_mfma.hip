// attention_mfma.hip -- a4 for bf16 prefill on gfx950 matrix cores: the Outer-Gather-Q
// kernel of page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比", section
// Kernel 创新：Outer Gather Q (the KV block is the outer loop; every query that chose
// it is gathered and processed against one on-chip copy), computing the exact
// block-restricted softmax of section 第二步：精算.
//
// Work item = one (sequence, group, KV block) and up to kItemRows query rows of its
// inverted list (ascending rows).  One workgroup of 8 waves stages K and V once; the
// rows are then cut into sub-chunks of 32 M-rows (M-row = (query row, head), head
// fastest, so a sub-chunk is 32 / G query rows) and wave w walks sub-chunks w, w + 8,
// ...  Waves are independent after the staging barrier: each owns an LDS buffer that
// receives its gathered Q rows (coalesced 16-byte pieces; a query row's G heads are
// contiguous) and is then reused to transpose its outputs into coalesced stores.
// The next sub-chunk's Q rows are fetched into registers while the current one
// computes; two waves per SIMD overlap one wave's softmax with the other's MFMAs.
//
//  * LDS: K row-major (16-byte row pad), V TRANSPOSED (d x 128, 16-byte row pad).  In
//    a V^T row the keys of every 16-key group are stored in the order in which one lane
//    half feeds them to the PV contraction (see the P item below), so a lane fetches its
//    8 keys of one head dim with one 16-byte read.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys, B = 32 M-rows): a lane's
//    output column is one M-row, so row max and row sum are in-lane over 64 values
//    plus one exchange with lane ^ 32.
//  * P = exp2(s - m) stays in registers: accumulator registers 8p..8p+7 of key tile
//    kt hold 8 keys of the lane's M-row, exactly the 8 k-elements a lane supplies to
//    a B operand, so O^T = V^T P^T uses k-step (kt, p) with the accumulator's row
//    order.  Those 8 keys of lane half h are k0 + 4h + {0..3} and k0 + 8 + 4h + {0..3}
//    (k0 = 16 p); V^T stores key k0 + 8a + 4h + x at column k0 + 8h + 4a + x, so they
//    are one contiguous 16-byte run.
//  * 32x32 accumulator layout: output row i is held by lane half (i % 8) / 4 in
//    register 4 * (i / 8) + i % 4.  The QK contraction visits head dims in the order
//    lane half h, k-step s -> dims [d/2 * h + 8 s, +8) (any order works as long as A
//    and B agree).
//
// Output: per (row, slot, head) partial O (bf16, normalised) and lse (fp32, natural
// log), merged by lse_merge.  Partial O is written with non-temporal stores: it is
// read back only by the merge, long after, and should not evict K/V or Q lines.
#include "msa_internal.hpp"

#include <type_traits>

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlk = 128;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kItemRows = 512;  // query rows per work item

template <int DH>
struct __attribute__((aligned(16))) OgqLds {
  static constexpr int KROW = DH * 2 + 16;   // K row, padded
  static constexpr int VROW = kBlk * 2 + 16;  // V^T row, padded
  static constexpr int QROW = DH * 2 + 16;   // per-wave Q / O row, padded
  __attribute__((aligned(16))) unsigned char k[kBlk * KROW];
  __attribute__((aligned(16))) unsigned char vt[DH * VROW];
  __attribute__((aligned(16))) unsigned char buf[kWaves][32 * QROW];
  int64_t qoff[kItemRows];   // element offset of the row's first head in q
  int64_t pidx[kItemRows];   // partial index ((s*T + t)*Hkv + g)*k + slot
  int pos[kItemRows];        // absolute position p_t
  float lse[kWaves][32];
};

// Completes this wave's earlier LDS accesses before its later ones and keeps the
// compiler from moving LDS accesses across (lanes exchange data through LDS).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// K/V staging in two halves (global -> registers, registers -> LDS) so that a kernel
// can fetch the next block while it computes on the current one.  Thread layout:
// K: 16-byte pieces, row-major; V^T: thread = (4 consecutive keys, 8 consecutive dims),
// transposed 4x8 in registers.
template <int DH>
struct KVRegs {
  static constexpr int KP = kBlk * DH / 8 / kThreads;  // K pieces per thread
  uint4 k[KP];
  uint4 v[4];
};

template <int DH>
__device__ __forceinline__ void gload_k(uint4 (&rk)[KVRegs<DH>::KP], const uint16_t* kb, int nvalid) {
  constexpr int CPR = DH / 8;
#pragma unroll
  for (int u = 0; u < KVRegs<DH>::KP; ++u) {
    const int c = threadIdx.x + kThreads * u;
    const int row = c / CPR, col = c % CPR;
    rk[u] = row < nvalid ? *reinterpret_cast<const uint4*>(kb + row * DH + col * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int DH>
__device__ __forceinline__ void gload_v(uint4 (&rv)[4], const uint16_t* vb, int nvalid) {
  const int kg = threadIdx.x & 31;
  const int dc = threadIdx.x >> 5;  // 0..15
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = 4 * kg + i;
    rv[i] = dc < DH / 8 && key < nvalid ? *reinterpret_cast<const uint4*>(vb + key * DH + dc * 8)
                                         : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int DH>
__device__ __forceinline__ void gload_kv(KVRegs<DH>& r, const uint16_t* kb, const uint16_t* vb, int nvalid) {
  gload_k<DH>(r.k, kb, nvalid);
  gload_v<DH>(r.v, vb, nvalid);
}

template <int DH>
__device__ __forceinline__ void lstore_k(unsigned char* lk, const uint4 (&rk)[KVRegs<DH>::KP]) {
  constexpr int CPR = DH / 8;
#pragma unroll
  for (int u = 0; u < KVRegs<DH>::KP; ++u) {
    const int c = threadIdx.x + kThreads * u;
    const int row = c / CPR, col = c % CPR;
    *reinterpret_cast<uint4*>(&lk[row * OgqLds<DH>::KROW + col * 16]) = rk[u];
  }
}

template <int DH>
__device__ __forceinline__ void lstore_vt(unsigned char* lvt, const uint4 (&rv)[4]) {
  const int kg = threadIdx.x & 31;
  const int dc = threadIdx.x >> 5;
  // keys 4 kg .. 4 kg + 3 = k0 + 8a + 4h + {0..3} go to columns k0 + 8h + 4a + {0..3}
  const int kc = (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1);
  if (dc < DH / 8) {
    const uint32_t w[4][4] = {{rv[0].x, rv[0].y, rv[0].z, rv[0].w}, {rv[1].x, rv[1].y, rv[1].z, rv[1].w},
                              {rv[2].x, rv[2].y, rv[2].z, rv[2].w}, {rv[3].x, rv[3].y, rv[3].z, rv[3].w}};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t k0 = (w[0][e >> 1] >> sh) & 0xFFFFu, k1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t k2 = (w[2][e >> 1] >> sh) & 0xFFFFu, k3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
      uint2 o;
      o.x = k0 | (k1 << 16);
      o.y = k2 | (k3 << 16);
      *reinterpret_cast<uint2*>(&lvt[(dc * 8 + e) * OgqLds<DH>::VROW + kc * 8]) = o;
    }
  }
}

template <int DH>
__device__ __forceinline__ void lstore_kv(unsigned char* lk, unsigned char* lvt, const KVRegs<DH>& r) {
  lstore_k<DH>(lk, r.k);
  lstore_vt<DH>(lvt, r.v);
}

template <int DH>
__device__ __forceinline__ void stage_kv(OgqLds<DH>& L, const uint16_t* kb, const uint16_t* vb, int nvalid) {
  KVRegs<DH> r;
  gload_kv<DH>(r, kb, vb, nvalid);
  lstore_kv<DH>(L.k, L.vt, r);
}

// One wave's gathered Q rows: piece p = lane + 64 u -> M-row p / (DH/8), column p % (DH/8).
template <int DH>
struct QRegs {
  static constexpr int PIECES = 32 * DH / 8 / 64;
  uint4 v[PIECES];
};

template <int DH, int G>
__device__ __forceinline__ void load_q(QRegs<DH>& qr, const OgqLds<DH>& L, const uint16_t* q, int r0, int nrows,
                                       int lane) {
  constexpr int CPR = DH / 8;
#pragma unroll
  for (int u = 0; u < QRegs<DH>::PIECES; ++u) {
    const int p = lane + 64 * u;
    const int mr = p / CPR, col = p % CPR;
    const int r = mr / G, hh = mr % G;
    qr.v[u] = r < nrows ? *reinterpret_cast<const uint4*>(q + L.qoff[r0 + r] + hh * DH + col * 8)
                        : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int DH>
__device__ __forceinline__ void put_q(unsigned char* buf, const QRegs<DH>& qr, int lane) {
  constexpr int CPR = DH / 8;
#pragma unroll
  for (int u = 0; u < QRegs<DH>::PIECES; ++u) {
    const int p = lane + 64 * u;
    *reinterpret_cast<uint4*>(buf + (p / CPR) * OgqLds<DH>::QROW + (p % CPR) * 16) = qr.v[u];
  }
}

template <int DH, int G>
__global__ void __launch_bounds__(kThreads) ogq_mfma(Dims D, const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v,
                                                     const int4* __restrict__ wl,
                                                     const int* __restrict__ n_items,
                                                     const int32_t* __restrict__ entries,
                                                     float* __restrict__ part_lse,
                                                     uint16_t* __restrict__ part_o) {
  constexpr int KS = DH / 16;  // k-steps of the QK contraction
  constexpr int DT = DH / 32;  // output dim tiles of PV
  constexpr int RW = 32 / G;   // query rows per wave sub-chunk
  constexpr int CPR = DH / 8;
  __shared__ OgqLds<DH> L;

  // XCD-aware item order: the 8 XCDs receive workgroups round-robin, so give each
  // XCD a contiguous range of items (consecutive items share a KV block).
  const int n = *n_items;
  const int per_xcd = (n + 7) / 8;
  const int slot_in_xcd = blockIdx.x >> 3;
  const int item = (blockIdx.x & 7) * per_xcd + slot_in_xcd;
  if (slot_in_xcd >= per_xcd || item >= n) return;

  const int4 w = wl[item];
  if (w.z <= 0) return;  // empty item
  const int64_t sg = w.x / D.nb;
  const int b = w.x % D.nb;
  const int s = (int)(sg / D.Hkv), g = (int)(sg % D.Hkv);
  const int j0 = b * kBlk;
  const int pos0 = seq_pos0(D, s);
  const int64_t kv0 = kv_row(D, s, g, j0, DH);  // a block is contiguous; an invalid page reads as 0
  const int nvalid = kv0 < 0 ? 0 : min(kBlk, seq_len(D, s) - j0);
  const int rows = w.z;

  // per-row tables (one division per row, once per item)
  for (int r = threadIdx.x; r < rows; r += kThreads) {
    const int e = entries[w.y + r];
    const int t = e / D.k;
    const int slot = e - t * D.k;
    L.qoff[r] = (((int64_t)s * D.T + t) * D.H + (int64_t)g * G) * DH;
    L.pidx[r] = (((int64_t)s * D.T + t) * D.Hkv + g) * D.k + slot;
    L.pos[r] = pos0 + t;
  }
  stage_kv<DH>(L, k + (kv0 < 0 ? 0 : kv0), v + (kv0 < 0 ? 0 : kv0), nvalid);
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int nl = lane & 31;
  const int nsub = (rows + RW - 1) / RW;
  int j = wave;
  if (j >= nsub) return;
  unsigned char* buf = L.buf[wave];
  const float sc = D.scale * kLog2e;

  QRegs<DH> qn;
  load_q<DH, G>(qn, L, q, j * RW, min(RW, rows - j * RW), lane);
  put_q<DH>(buf, qn, lane);
  wave_lds_sync();
  if (j + kWaves < nsub) load_q<DH, G>(qn, L, q, (j + kWaves) * RW, min(RW, rows - (j + kWaves) * RW), lane);

  while (true) {
    const int r0 = j * RW;
    const int nrows = min(RW, rows - r0);
    const int rr = nl / G;  // this lane's query row within the sub-chunk
    const bool row_ok = rr < nrows;
    const int p = L.pos[r0 + (row_ok ? rr : 0)];

    // S^T = K Q^T for the 4 key tiles
    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) sacc[kt] = f32x16{};
    {
      const unsigned char* qrow = buf + nl * OgqLds<DH>::QROW + DH * h;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 bq = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              &L.k[(kt * 32 + nl) * OgqLds<DH>::KROW + DH * h + 16 * ks]);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, sacc[kt], 0, 0, 0);
        }
      }
    }
    // causal mask inside the own block; row max of the raw scores (scale > 0)
    if (__ballot(row_ok && p < j0 + kBlk - 1) != 0ull) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j0 + kt * 32 + 8 * (r >> 2) + 4 * h + (r & 3) > p) sacc[kt][r] = -INFINITY;
    }
    float m = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, sacc[kt][r]);
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    const float msc = m * sc;
    float l = 0.0f;
    bf16x8 pf[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = __builtin_amdgcn_exp2f(fmaf(sacc[kt][8 * pp + 2 * i], sc, -msc));
          const float c = __builtin_amdgcn_exp2f(fmaf(sacc[kt][8 * pp + 2 * i + 1], sc, -msc));
          l += a + c;
          pk[i] = cvt_bf16x2(a, c);
        }
        pf[kt][pp] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
      }
    }
    l += __shfl_xor(l, 32, 64);

    // O^T = V^T P^T
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int kb0 = (kt * 32 + 16 * pp + 8 * h) * 2;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&L.vt[(dt * 32 + nl) * OgqLds<DH>::VROW + kb0]);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kt][pp], oacc[dt], 0, 0, 0);
        }
      }
    }
    wave_lds_sync();  // this wave's Q rows are consumed: the buffer takes the outputs

    const float inv = 1.0f / l;
    unsigned char* orow = buf + nl * OgqLds<DH>::QROW + 8 * h;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        uint2 o;
        o.x = cvt_bf16x2(oacc[dt][4 * qd] * inv, oacc[dt][4 * qd + 1] * inv);
        o.y = cvt_bf16x2(oacc[dt][4 * qd + 2] * inv, oacc[dt][4 * qd + 3] * inv);
        *reinterpret_cast<uint2*>(orow + (dt * 32 + 8 * qd) * 2) = o;
      }
    }
    if (h == 0) L.lse[wave][nl] = (msc + __builtin_amdgcn_logf(l)) * kLn2;
    wave_lds_sync();

    // coalesced partial stores: (row, slot) -> G heads x d contiguous
#pragma unroll
    for (int u = 0; u < QRegs<DH>::PIECES; ++u) {
      const int pc = lane + 64 * u;
      const int mr = pc / CPR, col = pc % CPR;
      const int r = mr / G, hh = mr % G;
      if (r < nrows)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(buf + mr * OgqLds<DH>::QROW + col * 16),
                                    reinterpret_cast<u32x4*>(part_o + (L.pidx[r0 + r] * G + hh) * DH + col * 8));
    }
    if (lane < 32 && lane / G < nrows)
      __builtin_nontemporal_store(L.lse[wave][lane], &part_lse[L.pidx[r0 + lane / G] * G + lane % G]);

    j += kWaves;
    if (j >= nsub) break;
    wave_lds_sync();  // outputs read back: the buffer takes the next Q rows
    put_q<DH>(buf, qn, lane);
    wave_lds_sync();
    if (j + kWaves < nsub) load_q<DH, G>(qn, L, q, (j + kWaves) * RW, min(RW, rows - (j + kWaves) * RW), lane);
  }
}

// ------------------------------------------------------------------ query-tile pass
// Shared blocks of a 128-position query tile (chosen by most of its rows;
// hot_tiles.hip) are processed tile-wise.  Work item = one 8-wave slice of a tile:
// 8 waves x 32 M-rows (32 query rows at G = 8).  Each wave's Q B-operands stay in
// registers while the tile's shared blocks stream through double-buffered LDS (the
// next block's K is fetched during the first 64-key half of the current block, its V
// during the second; one barrier per block).  Online softmax over the blocks with a
// lazy reference max m: it is raised only when a row's max exceeds it by more than
// kLazy in exp2 units, so P <= 2^kLazy and the O^T accumulators are rescaled rarely
// (any reference gives the same normalised result).  A row that did not choose a
// block gets P = 0 through an infinite exponent offset; the causal mask applies
// inside the own block.  Each row with shared slots writes ONE partial (over all its
// shared blocks) at its lowest shared slot; the merge skips its other shared slots.
//
// The kernel is persistent: one workgroup per CU walks a contiguous range of the
// compacted item list of its XCD (neighbouring tiles of one group share most of their
// blocks, so they stay in that XCD's L2).  The next item's first block is staged into
// the idle buffer during the current item's last block, and its Q rows are fetched
// while the current item writes its outputs, so only the first item pays the
// start-up latency.
template <int DH>
struct __attribute__((aligned(16))) HotLds {
  static constexpr int KROW = OgqLds<DH>::KROW, VROW = OgqLds<DH>::VROW;
  static constexpr int QROW = DH * 2 + 8;             // output transpose row
  static constexpr int KB = kBlk * KROW;              // K part of a buffer
  static constexpr int BUF = KB + DH * VROW;          // K | V^T
  // buf[b] holds one block; the buffer freed by an item's last block receives that
  // item's transposed outputs (8 waves x 32 rows x QROW bytes)
  __attribute__((aligned(16))) unsigned char buf[2][BUF];
  int64_t pidx[2][kWaves][32];  // per item parity: partial index of the wave's rows, -1 if none
  float lse[kWaves][32];
};

// Per-item values of one lane.
struct HotItem {
  const int32_t* hl;  // {count, block ids...}
  int nh;
  int64_t sg;
  int s, g;
  int t_end;          // one past the tile's last row
  int tq0;            // the wave's first query row
  bool row_ok;
  uint32_t sb;        // shared blocks chosen by the lane's row
  int p;              // the row's position
};

template <int DH, int G>
__device__ __forceinline__ void hot_item_load(HotItem& it, bf16x8 (&bq)[DH / 16], const Dims& D, const uint16_t* q,
                                              const int32_t* hot, const int32_t* tiles, const uint64_t* hotmask,
                                              const uint32_t* selbits, int item, int ntiles, int wpt,
                                              int64_t (&pidx)[kWaves][32]) {
  constexpr int KS = DH / 16;
  constexpr int RW = 32 / G;
  constexpr int QWG = kWaves * RW;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int nl = lane & 31;
  const int part = item % wpt;
  const int tl = tiles[item / wpt];
  const int ti = tl % ntiles;
  it.sg = tl / ntiles;
  it.hl = hot + (int64_t)tl * kHotStride;
  it.nh = it.hl[0];
  it.s = (int)(it.sg / D.Hkv);
  it.g = (int)(it.sg % D.Hkv);
  const int tau = D.pos0 / kHotTile + ti;
  const int t_lo = max(tau * kHotTile, D.pos0) - D.pos0;
  it.t_end = min(tau * kHotTile + kHotTile, D.N) - D.pos0;
  it.tq0 = t_lo + part * QWG + wave * RW;
  const int t = it.tq0 + nl / G;  // this lane's M-row = (t, head nl % G)
  it.row_ok = t < it.t_end;
  const int tt = it.row_ok ? t : 0;
  const int64_t rowid = ((int64_t)it.s * D.T + tt) * D.Hkv + it.g;
  it.sb = it.row_ok ? selbits[rowid] : 0u;
  it.p = D.pos0 + tt;
  // Q B-operands: lane half h, k-step ks -> head dims [DH/2 h + 8 ks, +8)
  const uint16_t* qp = q + (((int64_t)it.s * D.T + tt) * D.H + (int64_t)it.g * G + nl % G) * DH + (DH / 2) * h;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) bq[ks] = it.row_ok ? *reinterpret_cast<const bf16x8*>(qp + 8 * ks) : bf16x8{};
  if (h == 0 && nl % G == 0) {
    int64_t pi = -1;
    if (it.row_ok) {
      const uint64_t hm = hotmask[rowid];
      if (hm != 0ull) pi = rowid * D.k + __builtin_ctzll(hm);
    }
    pidx[wave][nl / G] = pi;
  }
}

template <int DH, int G>
__global__ void __launch_bounds__(kThreads) hot_mfma(Dims D, const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v,
                                                     const int32_t* __restrict__ hot,
                                                     const int32_t* __restrict__ tiles,
                                                     const int* __restrict__ ntile,
                                                     const uint64_t* __restrict__ hotmask,
                                                     const uint32_t* __restrict__ selbits,
                                                     float* __restrict__ part_lse,
                                                     uint16_t* __restrict__ part_o, int ntiles, int wpt) {
  constexpr int KS = DH / 16;
  constexpr int DT = DH / 32;
  constexpr int CPR = DH / 8;
  constexpr int QROW = HotLds<DH>::QROW;
  static_assert(kWaves * 32 * QROW <= HotLds<DH>::BUF, "output transpose fits one buffer");
  __shared__ HotLds<DH> L;

  // this workgroup's items: a round-robin share of its XCD's contiguous range
  const int nitems = *ntile * wpt;
  const int per_xcd = (nitems + 7) / 8;
  const int xcd = blockIdx.x & 7;
  const int nwx = ((int)gridDim.x - xcd + 7) / 8;  // workgroups on this XCD
  const int end = min((xcd + 1) * per_xcd, nitems);
  int item = xcd * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= end) return;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int nl = lane & 31;
  const float sc = D.scale * kLog2e;
  constexpr float kLazy = 8.0f;

  HotItem it;
  bf16x8 bq[KS];
  int par = 0;
  hot_item_load<DH, G>(it, bq, D, q, hot, tiles, hotmask, selbits, item, ntiles, wpt, L.pidx[par]);
  KVRegs<DH> nx;
  {
    const int b = it.hl[1];
    const int64_t kv0 = (it.sg * D.N + (int64_t)b * kBlk) * DH;
    gload_kv<DH>(nx, k + kv0, v + kv0, min(kBlk, D.N - b * kBlk));
    lstore_k<DH>(L.buf[0], nx.k);
    lstore_vt<DH>(L.buf[0] + HotLds<DH>::KB, nx.v);
  }
  __syncthreads();
  int cur = 0;

  while (true) {
    const int next_item = item + nwx;
    const bool has_next = next_item < end;
    // the first block of the next item (its hot list is all that is needed now)
    int nb_first = 0;
    int64_t nsg = 0;
    if (has_next) {
      const int ntl = tiles[next_item / wpt];
      nsg = ntl / ntiles;
      nb_first = hot[(int64_t)ntl * kHotStride + 1];
    }

    // running reference max in exp2 units (raw score times sc); a finite start keeps
    // (ms - mn) finite, and no product with sc can overflow it whatever the scale
    float ms = -3.0e38f;
    float l = 0.0f;
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};

    for (int i = 0; i < it.nh; ++i) {
      // next block: this item's next one, else the next item's first, else this one again
      // (a harmless reload into the idle buffer)
      int bn = it.hl[1 + min(i + 1, it.nh - 1)];
      int64_t bsg = it.sg;
      if (i + 1 == it.nh && has_next) {
        bn = nb_first;
        bsg = nsg;
      }
      const int nvn = min(kBlk, D.N - bn * kBlk);
      const int64_t kvn = (bsg * D.N + (int64_t)bn * kBlk) * DH;
      gload_k<DH>(nx.k, k + kvn, nvn);
      const int j0 = it.hl[1 + i] * kBlk;
      const bool chose = (it.sb >> i) & 1u;
      const bool any = __ballot(chose) != 0ull;
      // causal mask (keys j > p) only where a row that chose the block ends inside it; a row
      // that did not choose the block gets P = 0 through an infinite exponent offset below
      const bool need_mask = __ballot(chose && it.p < j0 + kBlk - 1) != 0ull;
      const unsigned char* lk = L.buf[cur];
      const unsigned char* lvt = L.buf[cur] + HotLds<DH>::KB;
      auto half = [&](auto hf_tag) {
        constexpr int HF = decltype(hf_tag)::value;
        f32x16 sacc[2];
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int kt = 2 * HF + k2;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&lk[(kt * 32 + nl) * HotLds<DH>::KROW + DH * h + 16 * ks]);
            sacc[k2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[ks], sacc[k2], 0, 0, 0);
          }
        }
        if (need_mask) {
          // key j0 + 64 HF + 32 k2 + 8 (r / 4) + 4 h + r % 4 > p, constant part on the left
          const int bound = it.p - j0 - 64 * HF - 4 * h;
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * k2 + 8 * (r >> 2) + (r & 3) > bound) sacc[k2][r] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[k2][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (!chose) mx = -INFINITY;
        const float mxs = mx * sc;  // -inf for a row that did not choose the block
        if (__ballot(mxs > ms + kLazy) != 0ull) {
          const float mn = fmaxf(ms, mxs);
          const float alpha = __builtin_amdgcn_exp2f(ms - mn);
          ms = mn;
          l *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        }
        // exponent offset; +inf for a row that did not choose the block: fma(s, sc, -inf) is
        // -inf for every finite or -inf score, so its P is exactly 0
        const float msc = chose ? ms : INFINITY;
        bf16x8 pf[2][2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            uint32_t pk[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const float a = __builtin_amdgcn_exp2f(fmaf(sacc[k2][8 * pp + 2 * x], sc, -msc));
              const float c = __builtin_amdgcn_exp2f(fmaf(sacc[k2][8 * pp + 2 * x + 1], sc, -msc));
              l += a + c;
              pk[x] = cvt_bf16x2(a, c);
            }
            pf[k2][pp] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
          }
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const int kb0 = ((2 * HF + k2) * 32 + 16 * pp + 8 * h) * 2;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const bf16x8 a = *reinterpret_cast<const bf16x8*>(&lvt[(dt * 32 + nl) * HotLds<DH>::VROW + kb0]);
              oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[k2][pp], oacc[dt], 0, 0, 0);
            }
          }
        }
      };
      if (any) half(std::integral_constant<int, 0>{});
      lstore_k<DH>(L.buf[cur ^ 1], nx.k);
      gload_v<DH>(nx.v, v + kvn, nvn);
      if (any) half(std::integral_constant<int, 1>{});
      lstore_vt<DH>(L.buf[cur ^ 1] + HotLds<DH>::KB, nx.v);
      __syncthreads();
      cur ^= 1;
    }
    l += __shfl_xor(l, 32, 64);

    // buf[cur] holds the next item's first block; buf[cur ^ 1] (this item's last block)
    // takes the transposed outputs
    const HotItem done = it;
    const int dpar = par;
    if (has_next) {
      par ^= 1;
      hot_item_load<DH, G>(it, bq, D, q, hot, tiles, hotmask, selbits, next_item, ntiles, wpt, L.pidx[par]);
    }
    unsigned char* buf = L.buf[cur ^ 1] + wave * 32 * QROW;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    unsigned char* orow = buf + nl * QROW + 8 * h;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        uint2 o;
        o.x = cvt_bf16x2(oacc[dt][4 * qd] * inv, oacc[dt][4 * qd + 1] * inv);
        o.y = cvt_bf16x2(oacc[dt][4 * qd + 2] * inv, oacc[dt][4 * qd + 3] * inv);
        *reinterpret_cast<uint2*>(orow + (dt * 32 + 8 * qd) * 2) = o;
      }
    }
    if (h == 0) L.lse[wave][nl] = (ms + __builtin_amdgcn_logf(l)) * kLn2;
    wave_lds_sync();
#pragma unroll
    for (int u = 0; u < QRegs<DH>::PIECES; ++u) {
      const int pc = lane + 64 * u;
      const int mr = pc / CPR, col = pc % CPR;
      const int r = mr / G, hh = mr % G;
      const int64_t pi = L.pidx[dpar][wave][r];
      if (done.tq0 + r < done.t_end && pi >= 0) {
        // rows are QROW = 8 (mod 16) bytes apart: two 8-byte LDS reads
        const unsigned char* src = buf + mr * QROW + col * 16;
        const uint2 lo = *reinterpret_cast<const uint2*>(src);
        const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
        const u32x4 val = {lo.x, lo.y, hi.x, hi.y};
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(part_o + (pi * G + hh) * DH + col * 8));
      }
    }
    if (lane < 32) {
      const int r = lane / G;
      const int64_t pi = L.pidx[dpar][wave][r];
      if (done.tq0 + r < done.t_end && pi >= 0) part_lse[pi * G + lane % G] = L.lse[wave][lane];
    }
    if (!has_next) break;
    item = next_item;
    // every wave has read its outputs back before the next item's first block stages its
    // successor into this buffer
    __syncthreads();
  }
}

template <int DH, int G>
void launch_t(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int4* wl,
              const int* n_items, int64_t grid, const int32_t* entries, float* part_lse, uint16_t* part_o,
              hipStream_t st) {
  hipLaunchKernelGGL((ogq_mfma<DH, G>), dim3((unsigned)grid), dim3(kThreads), 0, st, D, q, k, v, wl, n_items,
                     entries, part_lse, part_o);
}

void launch_any(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int4* wl,
                const int* n_items, int64_t grid, const int32_t* entries, float* part_lse, uint16_t* part_o,
                hipStream_t st) {
#define MSA_OGQ_CASE(DH_, G_) \
  if (D.d == DH_ && D.G == G_) return launch_t<DH_, G_>(D, q, k, v, wl, n_items, grid, entries, part_lse, part_o, st)
  MSA_OGQ_CASE(128, 8); MSA_OGQ_CASE(128, 1); MSA_OGQ_CASE(128, 2); MSA_OGQ_CASE(128, 4); MSA_OGQ_CASE(128, 16);
  MSA_OGQ_CASE(64, 8); MSA_OGQ_CASE(64, 1); MSA_OGQ_CASE(64, 2); MSA_OGQ_CASE(64, 4); MSA_OGQ_CASE(64, 16);
#undef MSA_OGQ_CASE
}

template <int DH, int G>
void launch_hot_t(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v, const HotSplit& h,
                  float* part_lse, uint16_t* part_o, int wpt, int grid, hipStream_t st) {
  hipLaunchKernelGGL((hot_mfma<DH, G>), dim3((unsigned)grid), dim3(kThreads), 0, st, D, q, k, v, h.hot, h.tiles,
                     h.ntile, h.hotmask, h.selbits, part_lse, part_o, h.ntiles, wpt);
}

}  // namespace

hipError_t launch_hot_mfma(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v, const HotSplit& h,
                           float* part_lse, uint16_t* part_o, hipStream_t st) {
  const int qwg = kWaves * (32 / D.G);
  const int wpt = (kHotTile + qwg - 1) / qwg;
  if ((int64_t)D.S * D.Hkv * h.ntiles * wpt >= (1ll << 31)) return hipErrorInvalidValue;
  // persistent: one workgroup per CU (the LDS footprint allows one)
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int grid = max(ncu, 8);
  LaunchScope scope("hot_mfma", st);
#define MSA_HOT_CASE(DH_, G_) \
  if (D.d == DH_ && D.G == G_) { launch_hot_t<DH_, G_>(D, q, k, v, h, part_lse, part_o, wpt, grid, st); return hipGetLastError(); }
  MSA_HOT_CASE(128, 8); MSA_HOT_CASE(128, 1); MSA_HOT_CASE(128, 2); MSA_HOT_CASE(128, 4); MSA_HOT_CASE(128, 16);
  MSA_HOT_CASE(64, 8); MSA_HOT_CASE(64, 1); MSA_HOT_CASE(64, 2); MSA_HOT_CASE(64, 4); MSA_HOT_CASE(64, 16);
#undef MSA_HOT_CASE
  return hipErrorInvalidValue;
}

bool ogq_mfma_supported(const Dims& D) {
  return D.dtype == MSA_BF16 && (D.d == 64 || D.d == 128) &&
         (D.G == 1 || D.G == 2 || D.G == 4 || D.G == 8 || D.G == 16);
}

int ogq_mfma_rows_per_item(const Dims& D) {
  (void)D;
  return kItemRows;
}

hipError_t launch_ogq_mfma(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int4* wl, const int* n_items, int64_t ub, const int32_t* entries,
                           float* part_lse, uint16_t* part_o, hipStream_t st) {
  const int64_t grid = (ub + 7) / 8 * 8 + 8;  // >= 8 * ceil(n_items / 8) for any n_items <= ub
  LaunchScope scope("ogq_mfma", st);
  launch_any(D, q, k, v, wl, n_items, grid, entries, part_lse, part_o, st);
  return hipGetLastError();
}

}  // namespace msa
