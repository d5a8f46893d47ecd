// backward.hip -- the training path of MSA on gfx950.
//
// Page "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比", section 索引分支训练：
// KL 对齐 (the index branch is taught by the main branch's attention distribution through
// a KL divergence; the training signal reaches only the index branch), and the MSA entry of
// "稀疏注意力速览（Sparse Attention，2019 ~ 2026）" (KL loss, teacher stop-gradient).
//
//  * attn_bwd: gradients of the block-sparse main branch (dQ, dK, dV) in the Outer-Gather-Q
//    order of section Kernel 创新：Outer Gather Q: one work item = (sequence, group, KV
//    block) and up to kRows rows of its inverted list; the block's K, V and K^T are staged
//    once and every gathered row is processed against them.  Each of the 8 waves owns 16
//    keys (two waves per SIMD).  Per sub-chunk of 32 M-rows (M-row = (row, head)):
//        S = Q K^T and dP = dO V^T          (v_mfma_f32_16x16x32_bf16, two 16-M-row
//                                              tiles; lane column = key)
//        P = exp2(S scale log2e - lse log2e),  dS = P (dP - D)      (D = rowsum(dO o O))
//        dV^T += dO^T P,  dK^T += Q^T dS    (the P / dS registers are the B operands, in
//                                              the accumulator's M-row order; dO^T and Q^T
//                                              are read transposed out of the row-major
//                                              tiles in that order)
//        dQ = dS K                          (dS through LDS, wave w takes head dims
//                                              [16w, 16w+16); K^T in registers)
//    dQ of each (row, slot, head) is stored as a bf16 partial (a row's k slots are
//    different items) and a merge kernel sums a row's partials; dK, dV are accumulated in
//    registers over the item's rows and added once per item with float atomics (a block's
//    list can span several items).
//  * index_kl: per row, KL(teacher || student) over the selected blocks and its gradient
//    with respect to the block scores (teacher = the forward's block masses).
//  * index_bwd + index_dq_gather: the gradient of the block scores through the causal
//    max-pool: per (row, selected block) the arg-max key (lowest position among equal
//    maxima; scores as the matrix cores sum them in float32) takes dscore * q_I, and the
//    row takes dscore * k_I[j*] summed over its slots.
#include "msa_internal.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlk = 128;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 512;  // query rows per work item

__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// (transposed operand reads: tr_operand, msa_internal.hpp)

// M-row held by accumulator register r of lane half h (32x32 output layout).
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int DH>
struct __attribute__((aligned(16))) BwdLds {
  static constexpr int KROW = DH * 2 + 16;    // K / V row-major, bytes
  // Q / dO row-major (32 M-rows): a row pitch of 20 banks (mod 64) keeps the 16-byte row
  // reads conflict-free and spreads the transposed 8-byte reads (4 rows x 32 bytes per 16
  // lanes) over at most two lanes per bank
  static constexpr int QROW = DH * 2 + ((80 - DH * 2) % 256 + 256) % 256;
  static constexpr int SROW = kBlk * 2 + 16;  // dS row (one M-row over the block's keys)
  __attribute__((aligned(16))) unsigned char kr[kBlk * KROW];
  __attribute__((aligned(16))) unsigned char vr[kBlk * KROW];
  __attribute__((aligned(16))) unsigned char qs[32 * QROW];
  __attribute__((aligned(16))) unsigned char dos[32 * QROW];
  __attribute__((aligned(16))) unsigned char ds[32 * SROW];
  __attribute__((aligned(16))) float lse2[32];  // lse * log2(e); +inf for an M-row past the item's rows
  __attribute__((aligned(16))) float drow[32];
  __attribute__((aligned(16))) int pos[32];
  __attribute__((aligned(16))) unsigned char dqt[32 * QROW];  // a sub-chunk's dQ (bf16), stored next iteration
  int64_t dqoff[2][32];  // by sub-chunk parity: element offset of the M-row's dQ partial (scratch row if none)
  int rowt[kRows];     // the item's rows: query row t and slot, decoded once per item, so
  int rslot[kRows];    // that no per-sub-chunk load waits on another global load
};

// D[s, t, h] = sum_c dO[s, t, h, c] O[s, t, h, c] (fp32), 16 lanes per row.
template <int DH>
__global__ void __launch_bounds__(256) drow_kernel(int64_t rows, const uint16_t* __restrict__ out,
                                                   const uint16_t* __restrict__ dout, float* __restrict__ drow) {
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  float acc = 0.0f;
  if (r < rows) {
    for (int c = sub * 8; c < DH; c += 128) {
      const uint4 a = *reinterpret_cast<const uint4*>(out + r * DH + c);
      const uint4 b = *reinterpret_cast<const uint4*>(dout + r * DH + c);
      const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(bf16_to_f32((uint16_t)(wa[i] & 0xFFFFu)), bf16_to_f32((uint16_t)(wb[i] & 0xFFFFu)), acc);
        acc = fmaf(bf16_to_f32((uint16_t)(wa[i] >> 16)), bf16_to_f32((uint16_t)(wb[i] >> 16)), acc);
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (r < rows && sub == 0) drow[r] = acc;
}

__global__ void __launch_bounds__(256) zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

// ---- attention backward: 8 waves of 16 keys each (v_mfma_f32_16x16x32_bf16)
// Sixteen keys per wave halve the per-wave accumulators (dK^T, dV^T: 16 keys x d), the
// register-held K / V / K^T operands and the score tiles, so the kernel fits 256 registers
// and runs two waves per SIMD: one wave's products overlap the other's softmax, LDS
// traffic and barriers.  The price is twice the LDS operand reads per product (each wave
// reads the whole Q / dO / dS tiles for its 16 keys).  16x16 layout: lane (c = lane % 16,
// g = lane / 16); A operand = row c of the A tile, 8 k-values; B operand = column c, the
// same 8 k-values; output register i of a 16x16 tile = row 4 g + i, column c.  A k-step's
// 8 values of group g are k0 + 8 g + {0..7} for the row-major operands, or rows chosen to
// match the accumulator (the P / dS operands below): any order works as long as A and B
// agree.
constexpr int kWaves16 = 8;
constexpr int kThreads16 = kWaves16 * 64;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Transposed operand for the 16x16x32 layout: lane (c, g) gets column col0 + c of rows
// r0 + {0..3} (elements 0..3) and r1 + {0..3} (elements 4..7), r0 and r1 chosen per group
// (the transposing read works within each 16-lane group: destination lane i takes, as
// element j, value i % 4 of the 8 bytes addressed by source lane 4 j + i / 4, so source
// lane 4 j + q addresses row r + j at columns col0 + 4 q .. + 3).
__device__ __forceinline__ bf16x8 tr_operand16(const unsigned char* tile, int row_bytes, int r0, int r1, int col0,
                                               int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  const int sl = lane & 15, j = sl >> 2, q = sl & 3;
  const int col = col0 + 4 * q;
  const lds_u8* t = (const lds_u8*)tile;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (r0 + j) * row_bytes + col * 2));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (r1 + j) * row_bytes + col * 2));
  const s16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, ab);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int DH, int G>
__global__ void __launch_bounds__(kThreads16, 1) attn_bwd(Dims D, const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const uint16_t* __restrict__ dout,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ drow,
                                                            const int4* __restrict__ wl, const int* __restrict__ n_items,
                                                            const int32_t* __restrict__ entries,
                                                            uint16_t* __restrict__ part_dq, float* __restrict__ dk,
                                                            float* __restrict__ dv) {
  using L_ = BwdLds<DH>;
  constexpr int KS = DH / 32;  // 32-dim k-steps of S and dP
  constexpr int DT = DH / 16;  // 16-dim tiles of dK^T, dV^T (and the waves that form dQ)
  constexpr int CPR = DH / 8;  // 16-byte pieces per row
  constexpr int NPC = 32 * CPR;  // 16-byte pieces of a sub-chunk's Q (or dO)
  static_assert(NPC <= kThreads16 && kThreads16 % NPC == 0, "each thread one piece of Q and one of dO");
  __shared__ L_ L;
  // Sub-chunk i uses tile set i % 2 (Q, dO, dS, per-M-row values) and dQ tile i % 3, so
  // only two barriers per sub-chunk remain (see the step below).  Set 1 and dQ tiles 1, 2
  // live in the K / V staging area, idle during the sub-chunk loop (K, V, K^T are in
  // registers by then), when it is large enough (d = 128), else in an array of their own.
  constexpr int QB = 32 * L_::QROW, SB = 32 * L_::SROW;
  constexpr int SET1 = 4 * QB + SB;  // qs, dos, ds of set 1; dQ tiles 1 and 2
  constexpr bool IN_KV = SET1 <= 2 * kBlk * L_::KROW;
  __shared__ __attribute__((aligned(16))) unsigned char xbuf[IN_KV ? 16 : SET1];
  __shared__ __attribute__((aligned(16))) float tl2[2][32];
  __shared__ __attribute__((aligned(16))) float tdr[2][32];
  __shared__ __attribute__((aligned(16))) int tpos[2][32];
  __shared__ int64_t tdq[3][32];
  unsigned char* const s1 = IN_KV ? L.kr : xbuf;

  const int n = *n_items;
  const int per_xcd = (n + 7) / 8;
  const int slot_in_xcd = blockIdx.x >> 3;
  const int item = (blockIdx.x & 7) * per_xcd + slot_in_xcd;
  if (slot_in_xcd >= per_xcd || item >= n) return;
  const int4 w = wl[item];
  if (w.z <= 0) return;
  const int64_t sg = w.x / D.nb;
  const int b = w.x % D.nb;
  const int s = (int)(sg / D.Hkv), g = (int)(sg % D.Hkv);
  const int j0 = b * kBlk;
  const int nvalid = min(kBlk, D.N - j0);
  const int rows = w.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, grp = lane >> 4, c = lane & 15;
  const float sc = D.scale * kLog2e;

  {
    const uint16_t* kb = k + (sg * D.N + j0) * DH;
    const uint16_t* vb = v + (sg * D.N + j0) * DH;
    for (int x = threadIdx.x; x < kBlk * CPR; x += kThreads16) {
      const int row = x / CPR, col = x % CPR;
      const bool ok = row < nvalid;
      const uint4 kk = ok ? *reinterpret_cast<const uint4*>(kb + row * DH + col * 8) : make_uint4(0u, 0u, 0u, 0u);
      const uint4 vv = ok ? *reinterpret_cast<const uint4*>(vb + row * DH + col * 8) : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&L.kr[row * L_::KROW + col * 16]) = kk;
      *reinterpret_cast<uint4*>(&L.vr[row * L_::KROW + col * 16]) = vv;
    }
  }
  f32x4 dkt[DT], dvt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dkt[dt] = f32x4{};
    dvt[dt] = f32x4{};
  }
  for (int r = threadIdx.x; r < rows; r += kThreads16) {
    const int e = entries[w.y + r];
    const int t = e / D.k;
    L.rowt[r] = t;
    L.rslot[r] = e - t * D.k;
  }
  __syncthreads();
  const int mrows = rows * G;
  const int first_pos = D.pos0 + L.rowt[0];
  const int64_t dq_trash = (int64_t)D.S * D.T * D.Hkv * D.k * G * DH;
  const bool need_mask = first_pos < j0 + kBlk - 1;
  const int key = j0 + 16 * wave + c;  // this lane's key (S, dP, dK, dV columns)
  // K and V rows of this wave's 16 keys (B operands of S and dP: k-step ks = head dims
  // 32 ks + 8 grp + {0..7}) and, for dQ, K^T for head dims [16 wave, +16) (k-step ks = keys
  // 32 ks + 8 grp + {0..7}), read from LDS once per item
  bf16x8 kop[KS], vop[KS], ktop[kBlk / 32];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kop[ks] = *reinterpret_cast<const bf16x8*>(&L.kr[(16 * wave + c) * L_::KROW + (32 * ks + 8 * grp) * 2]);
    vop[ks] = *reinterpret_cast<const bf16x8*>(&L.vr[(16 * wave + c) * L_::KROW + (32 * ks + 8 * grp) * 2]);
  }
#pragma unroll
  for (int ks = 0; ks < kBlk / 32; ++ks)
    ktop[ks] = wave < DT ? tr_operand16(L.kr, L_::KROW, 32 * ks + 8 * grp, 32 * ks + 8 * grp + 4, 16 * wave, lane)
                         : bf16x8{};

  // a sub-chunk's Q and dO: thread x takes piece x % NPC (M-row % 32, 16-byte column / 32)
  struct Pre {
    uint4 q, g;
    float lse, drow;
    int t, slot;
  };
  const int pc = threadIdx.x % NPC;
  const int pm = pc % 32, pcol = pc / 32;
  auto fetch = [&](Pre& pr, int m0n) __attribute__((always_inline)) {
    {
      const int mr = m0n + pm;
      const int mc = mr < mrows ? mr : 0;
      const int t = L.rowt[mc / G];
      const int64_t off = (((int64_t)s * D.T + t) * D.H + (int64_t)g * G + mc % G) * DH + pcol * 8;
      pr.q = *reinterpret_cast<const uint4*>(q + off);
      pr.g = *reinterpret_cast<const uint4*>(dout + off);
    }
    const int mr = m0n + (int)(threadIdx.x & 31);
    const int mc = mr < mrows ? mr : 0;
    pr.t = L.rowt[mc / G];
    pr.slot = L.rslot[mc / G];
    const int64_t hr = ((int64_t)s * D.T + pr.t) * D.H + (int64_t)g * G + mc % G;
    pr.lse = lse[hr];
    pr.drow = drow[hr];
  };
  Pre pa, pb;
  fetch(pa, 0);
  fetch(pb, 32);

  // dQ tiles of "sub-chunks" -2 and -1 go to the scratch row (every thread reads these
  // offsets in the first two sub-chunks: a barrier before them)
  if (threadIdx.x < 32) {
    tdq[1][threadIdx.x] = dq_trash;
    tdq[2][threadIdx.x] = dq_trash;
  }
  __syncthreads();
  auto dqt_of = [&](int tri) __attribute__((always_inline)) {
    return tri == 0 ? L.dqt : s1 + 2 * QB + SB + (tri - 1) * QB;
  };
  auto store_dq = [&](int tri) {
    const unsigned char* src = dqt_of(tri);
    for (int x = threadIdx.x; x < NPC; x += kThreads16) {
      const int m = x / CPR, col = x % CPR;
      const uint4 val = *reinterpret_cast<const uint4*>(&src[m * L_::QROW + col * 16]);
      *reinterpret_cast<uint4*>(part_dq + tdq[tri][m] + col * 8) = val;
    }
  };

  // Sub-chunk i: (a) store the dQ tile of sub-chunk i - 2 and stage this one's Q, dO and
  // per-M-row values into set i % 2; barrier; (b) S, dP, P, dS, dV, dK, dS into set i % 2;
  // barrier; (c) dQ into tile i % 3.  No barrier ends (c): a wave still in (c) of i only
  // reads dS of set i % 2 and writes dQ tile i % 3, while a wave already in (a) of i + 1
  // writes set (i + 1) % 2 and stores dQ tile (i - 1) % 3 -- finished by every wave
  // before the barrier in (a) of i.  Set i % 2 is next written in (a) of i + 2 and dQ
  // tile i % 3 in (c) of i + 3, both after barriers that follow every use.
  auto step = [&](Pre& pr, int m0) __attribute__((always_inline)) {
    const int si = m0 >> 5;
    const int par = si & 1, tri = si % 3;
    unsigned char* const qsb = par ? s1 : L.qs;
    unsigned char* const dosb = par ? s1 + QB : L.dos;
    unsigned char* const dsb = par ? s1 + 2 * QB : L.ds;
    store_dq((si + 1) % 3);  // sub-chunk si - 2
    if (threadIdx.x < NPC) {
      const bool ok = m0 + pm < mrows;
      *reinterpret_cast<uint4*>(&qsb[pm * L_::QROW + pcol * 16]) = ok ? pr.q : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&dosb[pm * L_::QROW + pcol * 16]) = ok ? pr.g : make_uint4(0u, 0u, 0u, 0u);
    }
    if (threadIdx.x < 32) {
      const int m = threadIdx.x, mr = m0 + m;
      const bool ok = mr < mrows;
      const int64_t pidx = (((int64_t)s * D.T + pr.t) * D.Hkv + g) * D.k + pr.slot;
      tl2[par][m] = ok ? pr.lse * kLog2e : INFINITY;
      tdr[par][m] = ok ? pr.drow : 0.0f;
      tpos[par][m] = ok ? D.pos0 + pr.t : -1;
      tdq[tri][m] = ok ? (pidx * G + mr % G) * DH : dq_trash;
    }
    fetch(pr, m0 + 64);
    __syncthreads();

    // S = Q K^T, dP = dO V^T for this wave's 16 keys: M-row tiles mt = 0, 1
    f32x4 sacc[2], pacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x4{};
      pacc[mt] = f32x4{};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int ro = (16 * mt + c) * L_::QROW + (32 * ks + 8 * grp) * 2;
        sacc[mt] = mfma16(*reinterpret_cast<const bf16x8*>(&qsb[ro]), kop[ks], sacc[mt]);
        pacc[mt] = mfma16(*reinterpret_cast<const bf16x8*>(&dosb[ro]), vop[ks], pacc[mt]);
      }
    }
    // P, dS: register i of tile mt holds M-row 16 mt + 4 grp + i of this lane's key
    float pv[2][4], dsv[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const float4 l4 = *reinterpret_cast<const float4*>(&tl2[par][16 * mt + 4 * grp]);
      const float4 d4 = *reinterpret_cast<const float4*>(&tdr[par][16 * mt + 4 * grp]);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
      int pq[4] = {0, 0, 0, 0};
      if (need_mask) {
        const int4 p4 = *reinterpret_cast<const int4*>(&tpos[par][16 * mt + 4 * grp]);
        pq[0] = p4.x; pq[1] = p4.y; pq[2] = p4.z; pq[3] = p4.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[mt][i], sc, -lv[i]));
        if (need_mask && key > pq[i]) p = 0.0f;
        pv[mt][i] = p;
        dsv[mt][i] = p * (pacc[mt][i] - dv4[i]);
      }
    }
    // B operands of dV^T and dK^T (k = M-rows): elements 0..3 = tile 0's registers (M-rows
    // 4 grp + {0..3}), 4..7 = tile 1's (M-rows 16 + 4 grp + {0..3})
    const uint32_t wp[4] = {cvt_bf16x2(pv[0][0], pv[0][1]), cvt_bf16x2(pv[0][2], pv[0][3]),
                            cvt_bf16x2(pv[1][0], pv[1][1]), cvt_bf16x2(pv[1][2], pv[1][3])};
    const uint32_t wsd[4] = {cvt_bf16x2(dsv[0][0], dsv[0][1]), cvt_bf16x2(dsv[0][2], dsv[0][3]),
                             cvt_bf16x2(dsv[1][0], dsv[1][1]), cvt_bf16x2(dsv[1][2], dsv[1][3])};
    const bf16x8 pbo = __builtin_bit_cast(bf16x8, make_uint4(wp[0], wp[1], wp[2], wp[3]));
    const bf16x8 sbo = __builtin_bit_cast(bf16x8, make_uint4(wsd[0], wsd[1], wsd[2], wsd[3]));
    // dV^T += dO^T P, dK^T += Q^T dS: A = head dims 16 dt + c over the same M-rows (transposed reads)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dvt[dt] = mfma16(tr_operand16(dosb, L_::QROW, 4 * grp, 16 + 4 * grp, 16 * dt, lane), pbo, dvt[dt]);
      dkt[dt] = mfma16(tr_operand16(qsb, L_::QROW, 4 * grp, 16 + 4 * grp, 16 * dt, lane), sbo, dkt[dt]);
    }
    // dS to LDS (M-row major) for dQ
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint32_t wv = wsd[2 * mt + x];
        unsigned char* d0 = &dsb[(16 * mt + 4 * grp + 2 * x) * L_::SROW + (16 * wave + c) * 2];
        *reinterpret_cast<uint16_t*>(d0) = (uint16_t)(wv & 0xFFFFu);
        *reinterpret_cast<uint16_t*>(d0 + L_::SROW) = (uint16_t)(wv >> 16);
      }
    __syncthreads();
    // dQ = scale * dS K for head dims [16 wave, 16 wave + 16): two M-row tiles, k = keys
    if (wave < DT) {
      unsigned char* const dqb = dqt_of(tri);
      f32x4 qa[2] = {f32x4{}, f32x4{}};
#pragma unroll
      for (int ks = 0; ks < kBlk / 32; ++ks)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          qa[mt] = mfma16(*reinterpret_cast<const bf16x8*>(&dsb[(16 * mt + c) * L_::SROW + (32 * ks + 8 * grp) * 2]),
                          ktop[ks], qa[mt]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const uint32_t wq = cvt_bf16x2(qa[mt][2 * x] * D.scale, qa[mt][2 * x + 1] * D.scale);
          unsigned char* d0 = &dqb[(16 * mt + 4 * grp + 2 * x) * L_::QROW + (16 * wave + c) * 2];
          *reinterpret_cast<uint16_t*>(d0) = (uint16_t)(wq & 0xFFFFu);
          *reinterpret_cast<uint16_t*>(d0 + L_::QROW) = (uint16_t)(wq >> 16);
        }
    }
  };
  int nsub = 0;
  for (int m0 = 0; m0 < mrows; m0 += 64) {
    step(pa, m0);
    step(pb, m0 + 32);
    nsub += 2;
  }
  __syncthreads();
  store_dq((nsub - 2) % 3);  // the last two sub-chunks' dQ tiles
  store_dq((nsub - 1) % 3);

  __syncthreads();
  float* red = reinterpret_cast<float*>(L.kr);
  static_assert(sizeof(float) * kBlk * DH <= 2 * kBlk * BwdLds<DH>::KROW, "reduction buffer fits");
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float val = which == 0 ? dkt[dt][i] * D.scale : dvt[dt][i];
        red[(16 * wave + c) * DH + 16 * dt + 4 * grp + i] = val;
      }
    __syncthreads();
    float* dst = (which == 0 ? dk : dv) + (sg * D.N + j0) * DH;
    for (int i = threadIdx.x; i < nvalid * DH; i += kThreads16) unsafeAtomicAdd(dst + i, red[i]);
    __syncthreads();
  }
}

// dq[s, t, h, :] = sum over the valid slots of row (s, t, g) of its bf16 partials; one
// thread per 8 head dims.
template <int KR>
__global__ void __launch_bounds__(256) dq_merge(Dims D, const int32_t* __restrict__ sel,
                                                const uint16_t* __restrict__ part_dq, float* __restrict__ dq) {
  typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int gd8 = D.G * D.d / 8;
  const int64_t row = i / gd8;  // (s, t, g)
  if (row >= (int64_t)D.S * D.T * D.Hkv) return;
  const int c8 = (int)(i % gd8);
  const int g = (int)(row % D.Hkv);
  const int t = (int)((row / D.Hkv) % D.T);
  const int s = (int)(row / ((int64_t)D.Hkv * D.T));
  const int32_t* sl = sel + (((int64_t)s * D.Hkv + g) * D.T + t) * D.k;
  const uint16_t* pr = part_dq + row * D.k * (int64_t)D.G * D.d + c8 * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add = [&](const uint4& u) {
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      acc[2 * x] += bf16_to_f32((uint16_t)(wv[x] & 0xFFFFu));
      acc[2 * x + 1] += bf16_to_f32((uint16_t)(wv[x] >> 16));
    }
  };
  if constexpr (KR > 0) {
    // k <= KR: every partial of the thread is loaded (read once: non-temporal) before the
    // first add; the adds keep the ascending slot order
    uint4 u[KR];
    bool ok[KR];
#pragma unroll
    for (int slot = 0; slot < KR; ++slot) {
      ok[slot] = slot < D.k && sl[slot < D.k ? slot : 0] >= 0;
      u[slot] = ok[slot] ? __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(
                               pr + slot * (int64_t)D.G * D.d)))
                         : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int slot = 0; slot < KR; ++slot)
      if (ok[slot]) add(u[slot]);
  } else {
    for (int slot = 0; slot < D.k; ++slot) {
      if (sl[slot] < 0) continue;
      add(*reinterpret_cast<const uint4*>(pr + slot * (int64_t)D.G * D.d));
    }
  }
  // dq is not read again by this library: non-temporal stores
  typedef float f32x4_st __attribute__((ext_vector_type(4)));
  f32x4_st* o = reinterpret_cast<f32x4_st*>(dq + (((int64_t)s * D.T + t) * D.H + (int64_t)g * D.G) * D.d + c8 * 8);
  __builtin_nontemporal_store(f32x4_st{acc[0], acc[1], acc[2], acc[3]}, o);
  __builtin_nontemporal_store(f32x4_st{acc[4], acc[5], acc[6], acc[7]}, o + 1);
}

// Per row: KL(teacher || student) over the selected blocks and d loss / d block score.
// The row's selections, their block scores (a gather) and masses are all loaded before the
// first is used (KR >= k slots held in registers; KR = 0: any k, from memory).
template <int KR>
__global__ void __launch_bounds__(256) index_kl_kernel(Dims D, const float* __restrict__ scores,
                                                       const int32_t* __restrict__ sel,
                                                       const float* __restrict__ mass, float sigma,
                                                       float* __restrict__ loss, float* __restrict__ dscore) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (s, g, t)
  if (row >= (int64_t)D.S * D.Hkv * D.T) return;
  const int32_t* sl = sel + row * D.k;
  const float* ms = mass + row * D.k;
  const float* sc = scores + row * (int64_t)D.nb;
  constexpr int NR = KR > 0 ? KR : 1;
  bool ok[NR];
  float sv[NR], mv[NR];
  if constexpr (KR > 0) {
    int b[KR];
#pragma unroll
    for (int i = 0; i < KR; ++i) b[i] = i < D.k ? sl[i] : -1;
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      ok[i] = b[i] >= 0 && b[i] < D.nb;
      sv[i] = sc[ok[i] ? b[i] : 0];
      mv[i] = i < D.k ? ms[i] : 0.0f;
    }
  }
  auto slot = [&](int i, float& s_i, float& m_i) -> bool {  // block score and mass of slot i
    if constexpr (KR > 0) {
      s_i = sv[i];
      m_i = mv[i];
      return ok[i];
    } else {
      const int b = sl[i];
      const bool v = b >= 0 && b < D.nb;
      s_i = v ? sc[b] : 0.0f;
      m_i = ms[i];
      return v;
    }
  };
  const int k = KR > 0 ? KR : D.k;
  float mx = -INFINITY, tm = 0.0f;
#pragma unroll
  for (int i = 0; i < k; ++i) {
    float s_i, m_i;
    if (!slot(i, s_i, m_i)) continue;
    mx = fmaxf(mx, sigma * s_i);
    tm += m_i;
  }
  float l = 0.0f;
#pragma unroll
  for (int i = 0; i < k; ++i) {
    float s_i, m_i;
    if (slot(i, s_i, m_i)) l += expf(sigma * s_i - mx);
  }
  const float logl = logf(l);
  float L = 0.0f;
#pragma unroll
  for (int i = 0; i < k; ++i) {
    if (i >= D.k) break;
    float s_i, m_i;
    float gsc = 0.0f;
    if (slot(i, s_i, m_i)) {
      const float logps = sigma * s_i - mx - logl;
      const float pt = tm > 0.0f ? m_i / tm : 0.0f;
      if (pt > 0.0f) L += pt * (logf(pt) - logps);
      gsc = sigma * (expf(logps) - pt);
    }
    dscore[row * D.k + i] = gsc;
  }
  loss[row] = L;
}

// One KV block's index keys in LDS (bf16 row-major, 16-byte row pad: the per-lane 16-byte
// operand reads of a wave are bank-conflict free), the item's rows, and for a round of RP
// rows their index queries (row-major, the B operands of the key-gradient product) with
// each row's arg-max key and split dscore (its A operands).
template <int DI>
struct IdxBwdLds {
  static constexpr int ROW = DI * 2 + 16;
  static constexpr int RP = DI == 128 ? 128 : 256;  // rows per round
  static constexpr int QP = DI * 2 + 16;             // query-row pitch
  __attribute__((aligned(16))) unsigned char k[kBlk * ROW];
  __attribute__((aligned(16))) unsigned char qr[RP * QP];
  int rts[kRows];           // the item's rows, decoded once: query row t * 64 + slot (k <= 64)
  int sjs[RP];              // a round's arg-max keys (-1: none)
  uint32_t sw[RP];          // its dscores as two bf16 terms (hi | lo << 16)
};

// Arg-max of the causal block max-pool per (row, selected block) on the matrix cores, and
// the key side of its gradient.  Work item = (sequence, group, KV block) and up to kRows
// rows of its inverted list, taken in rounds of RP rows:
//  1. each wave takes 32 rows at a time: S^T = K_I q_I^T with v_mfma_f32_32x32x16_bf16 (A =
//     32 keys from LDS, B = the 32 rows' index queries from memory, k-step ks / lane half h
//     = index dims [16 ks + 8 h, +8)), so a lane's accumulators are 64 keys of ONE row; the
//     row's maximum over its causal keys and the lowest key holding it are in-register
//     scans plus one exchange with lane ^ 32 (scores are the matrix cores' float32 sums of
//     the exact bf16 products).  The arg-max goes to am (and to argmax when given); the
//     row's query, arg-max key and dscore go to LDS;
//  2. wave w owns keys [32 w, 32 w + 32): dK += A B over the round's rows, with A[key][row] =
//     the row's dscore if its arg-max is that key, else 0 (one-hot, dscore split into two
//     bf16 terms so that the sum keeps float32 precision) and B = the rows' queries.
// Each wave's dK tile goes to memory once per item with float atomics (float atomics into
// LDS, one per (row, index dim), were an order of magnitude slower).  The query side dq_idx
// is gathered per row afterwards (index_dq_gather).
template <int DI>
__global__ void __launch_bounds__(kThreads) index_bwd(Dims D, const uint16_t* __restrict__ q_idx,
                                                      const uint16_t* __restrict__ k_idx,
                                                      const int4* __restrict__ wl, const int* __restrict__ n_items,
                                                      const int32_t* __restrict__ entries,
                                                      const float* __restrict__ dscore, float* __restrict__ dk_idx,
                                                      int32_t* __restrict__ am, int32_t* __restrict__ argmax) {
  using L_ = IdxBwdLds<DI>;
  constexpr int KS = DI / 16;
  constexpr int CPR = DI / 8;
  constexpr int NT = DI / 32;  // index-dim tiles of the key gradient
  constexpr int RP = L_::RP;
  static_assert(kWaves * 32 == kBlk, "one 32-key tile per wave");
  __shared__ L_ L;
  const int n = *n_items;
  const int per_xcd = (n + 7) / 8;
  const int slot_in_xcd = blockIdx.x >> 3;
  const int item = (blockIdx.x & 7) * per_xcd + slot_in_xcd;
  if (slot_in_xcd >= per_xcd || item >= n) return;
  const int4 w = wl[item];
  if (w.z <= 0) return;
  const int64_t sg = w.x / D.nb;
  const int b = w.x % D.nb;
  const int j0 = b * kBlk;
  const int nvalid = min(kBlk, D.N - j0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, nl = lane & 31;
  const uint16_t* kb = k_idx + (sg * D.N + j0) * DI;
  for (int c = threadIdx.x; c < kBlk * CPR; c += kThreads) {
    const int key = c / CPR, col = c % CPR;
    *reinterpret_cast<uint4*>(&L.k[key * L_::ROW + col * 16]) =
        key < nvalid ? *reinterpret_cast<const uint4*>(kb + key * DI + col * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
  for (int r = threadIdx.x; r < w.z; r += kThreads) {
    const int e = entries[w.y + r];
    const int t = e / D.k;
    L.rts[r] = t * 64 + (e - t * D.k);
  }
  __syncthreads();
  // A lane's row of one 32-row step (both lane halves): its index query, dscore and place,
  // fetched one step ahead into one of two register sets (the loop is unrolled by two).
  // Loads are unconditional: a lane past the item's rows reads the item's first row and
  // writes nothing to memory.
  struct RowIn {
    bf16x8 q[KS];
    float gsc;
    int t, slot;
    bool ok;
  };
  auto fetch = [&](RowIn& x, int r0) __attribute__((always_inline)) {  // rows r0 + nl
    const int r = r0 + nl;
    x.ok = r < w.z;
    const int rs = L.rts[x.ok ? r : 0];
    x.t = rs >> 6;
    x.slot = rs & 63;
    const int64_t qi = sg * D.T + x.t;  // (s, g, t)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) x.q[ks] = *reinterpret_cast<const bf16x8*>(q_idx + qi * DI + 16 * ks + 8 * h);
    x.gsc = dscore[qi * D.k + x.slot];
  };
  constexpr int kStride = kWaves * 32;
  // phase 1 of one 32-row step of round `base` (rows base + r0 + nl)
  auto argmax_step = [&](RowIn& x, int base, int r0) __attribute__((always_inline)) {
    const int64_t qi = sg * D.T + x.t;
    f32x16 acc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      acc[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&L.k[(kt * 32 + nl) * L_::ROW + (16 * ks + 8 * h) * 2]);
        acc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, x.q[ks], acc[kt], 0, 0, 0);
      }
    }
    // keys kk <= lim are inside the block and causal for the row (kk = 0 always is: the
    // block is one the row selected)
    const int lim = min(nvalid - 1, D.pos0 + x.t - j0);
    float best = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (kt * 32 + acc_row(q, h) <= lim) best = fmaxf(best, acc[kt][q]);
    best = fmaxf(best, __shfl_xor(best, 32, 64));
    // lowest key holding the maximum (none when every causal score is NaN: no update)
    int idx = 0x7FFFFFFF;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int kk = kt * 32 + acc_row(q, h);
        if (kk <= lim && acc[kt][q] == best) idx = min(idx, kk);
      }
    idx = min(idx, __shfl_xor(idx, 32, 64));
    const int js = idx == 0x7FFFFFFF ? -1 : idx;
    if (x.ok && h == 0) {
      am[qi * D.k + x.slot] = js >= 0 ? j0 + js : -1;
      if (argmax != nullptr) argmax[qi * D.k + x.slot] = js >= 0 ? j0 + js : -1;
    }
    // the row's query and its A-operand entry for phase 2 (rows past the item: key -1)
    const int rl = r0 + nl;  // row within the round (< RP: r0 is a multiple of 32 below RP)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      *reinterpret_cast<bf16x8*>(&L.qr[rl * L_::QP + (16 * ks + 8 * h) * 2]) = x.q[ks];
    if (h == 0) {
      const uint32_t hi = cvt_bf16x2(x.gsc, 0.0f) & 0xFFFFu;
      const uint32_t lo = cvt_bf16x2(x.gsc - bf16_to_f32((uint16_t)hi), 0.0f) & 0xFFFFu;
      L.sjs[rl] = x.ok && js >= 0 ? js : -1;
      L.sw[rl] = hi | (lo << 16);
    }
    fetch(x, base + r0 + 2 * kStride);
  };
  f32x16 dka[NT];  // this wave's dK: keys [32 wave, +32), index-dim tile nt
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) dka[nt] = f32x16{};
  const int key = 32 * wave + nl;  // this lane's key (A-operand row) in phase 2
  for (int base = 0; base < w.z; base += RP) {
    const int rows = min(RP, w.z - base);
    RowIn xa, xb;
    fetch(xa, base + wave * 32);
    fetch(xb, base + wave * 32 + kStride);
    // steps in pairs, the second possibly past the round's rows (it then writes no memory;
    // its LDS entries lie past the round's rows and are not read)
    for (int r0 = wave * 32; r0 < rows; r0 += 2 * kStride) {
      argmax_step(xa, base, r0);
      if (r0 + kStride < RP) argmax_step(xb, base, r0 + kStride);
    }
    __syncthreads();
    // phase 2: 16 rows per k-step, rows 16 s + 8 h + {0..7} of this lane half
    for (int s0 = 0; s0 < rows; s0 += 16) {
      const int rb = s0 + 8 * h;
      const int4 j0v = *reinterpret_cast<const int4*>(&L.sjs[rb]);
      const int4 j1v = *reinterpret_cast<const int4*>(&L.sjs[rb + 4]);
      const uint4 w0v = *reinterpret_cast<const uint4*>(&L.sw[rb]);
      const uint4 w1v = *reinterpret_cast<const uint4*>(&L.sw[rb + 4]);
      const int jr[8] = {j0v.x, j0v.y, j0v.z, j0v.w, j1v.x, j1v.y, j1v.z, j1v.w};
      const uint32_t wr[8] = {w0v.x, w0v.y, w0v.z, w0v.w, w1v.x, w1v.y, w1v.z, w1v.w};
      uint32_t ah[4], al[4];
#pragma unroll
      for (int pq = 0; pq < 4; ++pq) {
        // a row past the round's rows holds a stale entry: never matched (s0 + 16 <= RP,
        // and rows >= `rows` are masked here)
        const bool v0 = rb + 2 * pq < rows, v1 = rb + 2 * pq + 1 < rows;
        const uint32_t w0 = v0 && jr[2 * pq] == key ? wr[2 * pq] : 0u;
        const uint32_t w1 = v1 && jr[2 * pq + 1] == key ? wr[2 * pq + 1] : 0u;
        ah[pq] = (w0 & 0xFFFFu) | (w1 << 16);
        al[pq] = (w0 >> 16) | (w1 & 0xFFFF0000u);
      }
      const bf16x8 a_hi = __builtin_bit_cast(bf16x8, make_uint4(ah[0], ah[1], ah[2], ah[3]));
      const bf16x8 a_lo = __builtin_bit_cast(bf16x8, make_uint4(al[0], al[1], al[2], al[3]));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 bq = tr_operand(L.qr, L_::QP, rb, rb + 4, 32 * nt, lane);
        dka[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi, bq, dka[nt], 0, 0, 0);
        dka[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo, bq, dka[nt], 0, 0, 0);
      }
    }
    __syncthreads();  // the round's LDS rows are consumed
  }
  // this wave's dK tile (rows = keys 32 wave + acc_row(r, h), columns = index dims 32 nt + nl)
  float* dst = dk_idx + (sg * D.N + j0) * DI;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = dka[nt][r];
      if (x != 0.0f) unsafeAtomicAdd(dst + (32 * wave + acc_row(r, h)) * DI + 32 * nt + nl, x);
    }
}

// dq_idx[s, g, t] = sum over the row's slots with an arg-max j of dscore * k_I[s, g, j], in
// slot order; 16 threads per row, DI / 16 index dims each.
template <int DI>
__global__ void __launch_bounds__(256) index_dq_gather(Dims D, const uint16_t* __restrict__ k_idx,
                                                       const int32_t* __restrict__ am,
                                                       const float* __restrict__ dscore,
                                                       float* __restrict__ dq_idx) {
  constexpr int PER = DI / 16;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 4;  // (s, g, t)
  if (row >= (int64_t)D.S * D.Hkv * D.T) return;
  const int c0 = (int)(gid & 15) * PER;
  const int64_t sg = row / D.T;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  for (int slot = 0; slot < D.k; ++slot) {
    const int j = am[row * D.k + slot];
    if (j < 0) continue;
    const float gsc = dscore[row * D.k + slot];
    const uint16_t* kp = k_idx + (sg * D.N + j) * DI + c0;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = fmaf(gsc, bf16_to_f32(kp[i]), acc[i]);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) dq_idx[row * DI + c0 + i] = acc[i];
}

__global__ void __launch_bounds__(256) fill_neg1(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = -1;
}

struct BwdWs {
  WorkList wlst;
  float* drow;
  uint16_t* part_dq;  // [S, T, Hkv, k, G, d] bf16
};

BwdWs backward_layout(const Dims& D, void* base, size_t* total) {
  BwdWs w;
  size_t wlb = 0;
  (void)work_list_layout(D, kRows, nullptr, &wlb);
  unsigned char* p = static_cast<unsigned char*>(base);
  w.wlst = work_list_layout(D, kRows, p, &wlb);
  size_t off = align_up(wlb, 256);
  w.drow = p ? reinterpret_cast<float*>(p + off) : nullptr;
  off += align_up((size_t)D.S * D.T * D.H * sizeof(float), 256);
  w.part_dq = p ? reinterpret_cast<uint16_t*>(p + off) : nullptr;
  // + one scratch row (d values) that M-rows past an item's list write to
  off += align_up(((size_t)D.S * D.T * D.Hkv * D.k * D.G + 1) * D.d * sizeof(uint16_t), 256);
  *total = off;
  return w;
}

hipError_t zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

template <int DH, int G>
void launch_bwd_t(const Dims& D, const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                  const float* lse, const float* drow, const WorkList& wl, const int32_t* entries,
                  uint16_t* part_dq, float* dk, float* dv, hipStream_t st) {
  const int64_t grid = (wl.ub + 7) / 8 * 8 + 8;
  hipLaunchKernelGGL((attn_bwd<DH, G>), dim3((unsigned)grid), dim3(kThreads16), 0, st, D, q, k, v, dout, lse, drow,
                     wl.wl, wl.n_items, entries, part_dq, dk, dv);
}

}  // namespace

size_t backward_workspace_bytes(const Dims& D) {
  size_t total = 0;
  (void)backward_layout(D, nullptr, &total);
  return total;
}

hipError_t launch_attn_backward(const Dims& D, const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse, const int32_t* sel, const int32_t* off,
                                const int32_t* entries, float* dq, float* dk, float* dv, void* ws, hipStream_t st) {
  size_t total = 0;
  const BwdWs w = backward_layout(D, ws, &total);
  hipError_t e;
  {
    LaunchScope scope("bwd_zero", st);
    e = zero(dk, (int64_t)D.S * D.Hkv * D.N * D.d, st);
    if (e == hipSuccess) e = zero(dv, (int64_t)D.S * D.Hkv * D.N * D.d, st);
  }
  if (e != hipSuccess) return e;
  {
    const int64_t rows = (int64_t)D.S * D.T * D.H;
    LaunchScope scope("bwd_drow", st);
    const dim3 grid((unsigned)((rows * 16 + 255) / 256));
    if (D.d == 64)
      hipLaunchKernelGGL(drow_kernel<64>, grid, dim3(256), 0, st, rows, static_cast<const uint16_t*>(out),
                         static_cast<const uint16_t*>(dout), w.drow);
    else
      hipLaunchKernelGGL(drow_kernel<128>, grid, dim3(256), 0, st, rows, static_cast<const uint16_t*>(out),
                         static_cast<const uint16_t*>(dout), w.drow);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  e = launch_work_list(D, off, kRows, w.wlst, st);
  if (e != hipSuccess) return e;
  const uint16_t *qb = static_cast<const uint16_t*>(q), *kb = static_cast<const uint16_t*>(k),
                 *vb = static_cast<const uint16_t*>(v), *gb = static_cast<const uint16_t*>(dout);
  bool launched = false;
  {
    LaunchScope scope("attn_bwd", st);
#define MSA_BWD_CASE(DH_, G_)                                                                          \
  if (!launched && D.d == DH_ && D.G == G_) {                                                          \
    launch_bwd_t<DH_, G_>(D, qb, kb, vb, gb, lse, w.drow, w.wlst, entries, w.part_dq, dk, dv, st);   \
    launched = true;                                                                                   \
  }
    MSA_BWD_CASE(128, 8); MSA_BWD_CASE(128, 1); MSA_BWD_CASE(128, 2); MSA_BWD_CASE(128, 4); MSA_BWD_CASE(128, 16);
    MSA_BWD_CASE(64, 8); MSA_BWD_CASE(64, 1); MSA_BWD_CASE(64, 2); MSA_BWD_CASE(64, 4); MSA_BWD_CASE(64, 16);
#undef MSA_BWD_CASE
  }
  if (!launched) return hipErrorInvalidValue;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nthreads = (int64_t)D.S * D.T * D.Hkv * (D.G * D.d / 8);
  LaunchScope scope("dq_merge", st);
  if (D.k <= 16)
    hipLaunchKernelGGL(dq_merge<16>, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, st, D, sel, w.part_dq, dq);
  else
    hipLaunchKernelGGL(dq_merge<0>, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, st, D, sel, w.part_dq, dq);
  return hipGetLastError();
}

hipError_t launch_index_kl(const Dims& D, const float* scores, const int32_t* sel, const float* mass, float sigma,
                           float* loss, float* dscore, hipStream_t st) {
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  LaunchScope scope("index_kl", st);
  const dim3 grid((unsigned)((rows + 255) / 256));
  if (D.k <= 16)
    hipLaunchKernelGGL(index_kl_kernel<16>, grid, dim3(256), 0, st, D, scores, sel, mass, sigma, loss, dscore);
  else
    hipLaunchKernelGGL(index_kl_kernel<0>, grid, dim3(256), 0, st, D, scores, sel, mass, sigma, loss, dscore);
  return hipGetLastError();
}

namespace {
// index-backward workspace: the work list, then the arg-max of every (row, slot)
WorkList index_bwd_layout(const Dims& D, void* base, int32_t** am, size_t* total) {
  size_t wlb = 0;
  (void)work_list_layout(D, kRows, nullptr, &wlb);
  unsigned char* p = static_cast<unsigned char*>(base);
  const WorkList wl = work_list_layout(D, kRows, p, &wlb);
  const size_t off = align_up(wlb, 256);
  *am = p ? reinterpret_cast<int32_t*>(p + off) : nullptr;
  *total = off + align_up((size_t)D.S * D.Hkv * D.T * D.k * sizeof(int32_t), 256);
  return wl;
}
}  // namespace

size_t index_backward_workspace_bytes(const Dims& D) {
  size_t total = 0;
  int32_t* am = nullptr;
  (void)index_bwd_layout(D, nullptr, &am, &total);
  return total;
}

hipError_t launch_index_backward(const Dims& D, const void* q_idx, const void* k_idx, const int32_t* off,
                                 const int32_t* entries, const float* dscore, float* dq_idx, float* dk_idx,
                                 int32_t* argmax, void* ws, hipStream_t st) {
  size_t total = 0;
  int32_t* am = nullptr;
  const WorkList wl = index_bwd_layout(D, ws, &am, &total);
  const int64_t nam = (int64_t)D.S * D.Hkv * D.T * D.k;
  hipError_t e;
  {
    LaunchScope scope("index_bwd_zero", st);
    e = zero(dk_idx, (int64_t)D.S * D.Hkv * D.N * D.dI, st);
    if (e == hipSuccess && nam > 0) {
      const int64_t blocks = (nam + 255) / 256 < 65536 ? (nam + 255) / 256 : 65536;
      hipLaunchKernelGGL(fill_neg1, dim3((unsigned)blocks), dim3(256), 0, st, am, nam);
      e = hipGetLastError();
    }
  }
  if (e != hipSuccess) return e;
  e = launch_work_list(D, off, kRows, wl, st);
  if (e != hipSuccess) return e;
  const int64_t grid = (wl.ub + 7) / 8 * 8 + 8;
  const uint16_t *qb = static_cast<const uint16_t*>(q_idx), *kb = static_cast<const uint16_t*>(k_idx);
  {
    LaunchScope scope("index_bwd", st);
    if (D.dI == 32)
      hipLaunchKernelGGL(index_bwd<32>, dim3((unsigned)grid), dim3(kThreads), 0, st, D, qb, kb, wl.wl, wl.n_items,
                         entries, dscore, dk_idx, am, argmax);
    else if (D.dI == 64)
      hipLaunchKernelGGL(index_bwd<64>, dim3((unsigned)grid), dim3(kThreads), 0, st, D, qb, kb, wl.wl, wl.n_items,
                         entries, dscore, dk_idx, am, argmax);
    else
      hipLaunchKernelGGL(index_bwd<128>, dim3((unsigned)grid), dim3(kThreads), 0, st, D, qb, kb, wl.wl, wl.n_items,
                         entries, dscore, dk_idx, am, argmax);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  LaunchScope scope("index_dq_gather", st);
  const dim3 g2((unsigned)((rows * 16 + 255) / 256));
  if (D.dI == 32)
    hipLaunchKernelGGL(index_dq_gather<32>, g2, dim3(256), 0, st, D, kb, am, dscore, dq_idx);
  else if (D.dI == 64)
    hipLaunchKernelGGL(index_dq_gather<64>, g2, dim3(256), 0, st, D, kb, am, dscore, dq_idx);
  else
    hipLaunchKernelGGL(index_dq_gather<128>, g2, dim3(256), 0, st, D, kb, am, dscore, dq_idx);
  return hipGetLastError();
}

}  // namespace msa
