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
//    once and every gathered row is processed against them.  Each of the 4 waves owns 32
//    keys.  Per sub-chunk of 32 M-rows (M-row = (row, head)):
//        S = Q K^T and dP = dO V^T          (v_mfma_f32_32x32x16_bf16; lane = key,
//                                              registers = M-rows)
//        P = exp2(S scale log2e - lse log2e),  dS = P (dP - D)      (D = rowsum(dO o O))
//        dV^T += dO^T P,  dK^T += Q^T dS    (the P / dS registers are the B operands: their
//                                              M-row order is the accumulator's; dO^T and
//                                              Q^T are stored in LDS in that order)
//        dQ = dS K                          (dS through LDS, wave w takes head dims
//                                              [32w, 32w+32); K^T in LDS is the B operand)
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
  static constexpr int QROW = DH * 2 + 16;    // Q / dO row-major (32 M-rows)
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

template <int DH, int G>
__global__ void __launch_bounds__(kThreads, 1) attn_bwd(Dims D, const uint16_t* __restrict__ q,
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
  constexpr int KS = DH / 16;  // k-steps over the head dims
  constexpr int DT = DH / 32;  // head-dim tiles
  constexpr int CPR = DH / 8;  // 16-byte pieces per row
  __shared__ L_ L;

  // XCD-aware order: consecutive items (same KV block) in one XCD's L2
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
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, nl = lane & 31;
  const float sc = D.scale * kLog2e;

  // ---- stage K, V (row-major)
  {
    const uint16_t* kb = k + (sg * D.N + j0) * DH;
    const uint16_t* vb = v + (sg * D.N + j0) * DH;
    for (int c = threadIdx.x; c < kBlk * CPR; c += kThreads) {
      const int row = c / CPR, col = c % CPR;
      const bool ok = row < nvalid;
      const uint4 kk = ok ? *reinterpret_cast<const uint4*>(kb + row * DH + col * 8) : make_uint4(0u, 0u, 0u, 0u);
      const uint4 vv = ok ? *reinterpret_cast<const uint4*>(vb + row * DH + col * 8) : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&L.kr[row * L_::KROW + col * 16]) = kk;
      *reinterpret_cast<uint4*>(&L.vr[row * L_::KROW + col * 16]) = vv;
    }
  }

  f32x16 dkt[DT], dvt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dkt[dt] = f32x16{};
    dvt[dt] = f32x16{};
  }
  for (int r = threadIdx.x; r < rows; r += kThreads) {
    const int e = entries[w.y + r];
    const int t = e / D.k;
    L.rowt[r] = t;
    L.rslot[r] = e - t * D.k;
  }
  __syncthreads();
  const int mrows = rows * G;
  const int first_pos = D.pos0 + L.rowt[0];  // rows ascend: the smallest position
  // M-rows past the list store their dQ here: one scratch row after the partials
  const int64_t dq_trash = (int64_t)D.S * D.T * D.Hkv * D.k * G * DH;
  const bool need_mask = first_pos < j0 + kBlk - 1;
  const int key = j0 + 32 * wave + nl;                // this lane's key

  // Q and dO pieces of a sub-chunk: piece c -> M-row c % 32, 16-byte column c / 32 (lanes
  // of a wave take consecutive M-rows, so the transposed 2-byte LDS writes of one
  // instruction fall in distinct dwords).  The next sub-chunk's pieces are fetched into
  // registers while the current one computes.
  constexpr int NP = 32 * CPR / kThreads;
  static_assert(NP >= 1 && 32 * CPR == NP * kThreads, "whole pieces per thread");
  uint4 nq[NP], ng[NP];
  // Every load is unconditional (a row past the list reads row 0 and is zeroed after the
  // load), and so are the dQ stores below: with no memory operation under a branch the
  // compiler counts them exactly, and the loop head waits only for the previous
  // iteration's loads, not for its dQ stores.
  // (the zeroing of rows past the list happens where the data is stored to LDS, so that
  // no instruction right after the loads waits for them)
  auto fetch = [&](int m0n) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int c = threadIdx.x + kThreads * u;
      const int mr = m0n + c % 32, col = c / 32;
      const int mc = mr < mrows ? mr : 0;
      const int t = L.rowt[mc / G];
      const int64_t off = (((int64_t)s * D.T + t) * D.H + (int64_t)g * G + mc % G) * DH + col * 8;
      nq[u] = *reinterpret_cast<const uint4*>(q + off);
      ng[u] = *reinterpret_cast<const uint4*>(dout + off);
    }
  };
  // per-M-row values of the next sub-chunk (threads 0..31), fetched with its Q and dO;
  // lse is scaled only when it is stored (the load's result is not needed before)
  float n_lse = 0.0f, n_drow = 0.0f;
  int n_t = 0, n_slot = 0;
  auto fetch_meta = [&](int m0n) {  // every thread (no branch); threads 0..31 store them
    const int mr = m0n + (int)(threadIdx.x & 31);
    const int mc = mr < mrows ? mr : 0;
    n_t = L.rowt[mc / G];
    n_slot = L.rslot[mc / G];
    const int64_t hr = ((int64_t)s * D.T + n_t) * D.H + (int64_t)g * G + mc % G;
    n_lse = lse[hr];
    n_drow = drow[hr];
  };
  fetch(0);
  fetch_meta(0);

  // dQ of a sub-chunk goes to an LDS tile and is stored at the start of the next
  // iteration, before that iteration's prefetch: the loads waited for at a loop head are
  // then never queued behind stores issued just before (this chip's counter does not
  // order a store ahead of a later load); the first iteration stores to the scratch row
  if (threadIdx.x < 32) L.dqoff[1][threadIdx.x] = dq_trash;
  constexpr int OP = 32 * CPR / kThreads;  // 16-byte dQ pieces per thread
  auto store_dq = [&](int par) {
#pragma unroll
    for (int u = 0; u < OP; ++u) {
      const int c = threadIdx.x + kThreads * u;
      const int m = c / CPR, col = c % CPR;  // a row's pieces in consecutive lanes
      const uint4 x = *reinterpret_cast<const uint4*>(&L.dqt[m * L_::QROW + col * 16]);
      *reinterpret_cast<uint4*>(part_dq + L.dqoff[par][m] + col * 8) = x;
    }
  };

  for (int m0 = 0; m0 < mrows; m0 += 32) {
    const int par = (m0 >> 5) & 1;
    __syncthreads();  // previous sub-chunk's buffers are free (and the staging is complete)
    store_dq(par ^ 1);  // the previous sub-chunk's dQ
    // ---- this sub-chunk's Q and dO (rows past the list as zeros)
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int c = threadIdx.x + kThreads * u;
      const int m = c % 32, col = c / 32;
      const bool ok = m0 + m < mrows;
      *reinterpret_cast<uint4*>(&L.qs[m * L_::QROW + col * 16]) = ok ? nq[u] : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&L.dos[m * L_::QROW + col * 16]) = ok ? ng[u] : make_uint4(0u, 0u, 0u, 0u);
    }
    if (threadIdx.x < 32) {
      const int m = threadIdx.x, mr = m0 + m;
      const bool ok = mr < mrows;
      const int64_t pidx = (((int64_t)s * D.T + n_t) * D.Hkv + g) * D.k + n_slot;
      L.lse2[m] = ok ? n_lse * kLog2e : INFINITY;  // P = 0 for an M-row past the list
      L.drow[m] = ok ? n_drow : 0.0f;
      L.pos[m] = ok ? D.pos0 + n_t : -1;
      L.dqoff[par][m] = ok ? (pidx * G + mr % G) * DH : dq_trash;
    }
    fetch(m0 + 32);  // past the last sub-chunk: row-0 loads, never used
    fetch_meta(m0 + 32);
    __syncthreads();

    // ---- S = Q K^T and dP = dO V^T for this wave's 32 keys
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&L.qs[nl * L_::QROW + (16 * ks + 8 * h) * 2]);
      const bf16x8 bk = *reinterpret_cast<const bf16x8*>(&L.kr[(32 * wave + nl) * L_::KROW + (16 * ks + 8 * h) * 2]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, sacc, 0, 0, 0);
      const bf16x8 ag = *reinterpret_cast<const bf16x8*>(&L.dos[nl * L_::QROW + (16 * ks + 8 * h) * 2]);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&L.vr[(32 * wave + nl) * L_::KROW + (16 * ks + 8 * h) * 2]);
      pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, bv, pacc, 0, 0, 0);
    }
    // ---- P, dS (registers r hold M-rows acc_row(r, h) of this lane's key)
    // per-M-row values of registers 4a .. 4a+3: M-rows 8a + 4h + {0..3}, one 16-byte read each
    float pv[16], dsv[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 l4 = *reinterpret_cast<const float4*>(&L.lse2[8 * a + 4 * h]);
      const float4 d4 = *reinterpret_cast<const float4*>(&L.drow[8 * a + 4 * h]);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
      int pq[4] = {0, 0, 0, 0};
      if (need_mask) {
        const int4 p4 = *reinterpret_cast<const int4*>(&L.pos[8 * a + 4 * h]);
        pq[0] = p4.x; pq[1] = p4.y; pq[2] = p4.z; pq[3] = p4.w;
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = 4 * a + x;
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], sc, -lv[x]));
        if (need_mask && key > pq[x]) p = 0.0f;
        pv[r] = p;
        dsv[r] = p * (pacc[r] - dv4[x]);
      }
    }
    bf16x8 pb[2], sb[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      uint32_t wp[4], wsd[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        wp[x] = cvt_bf16x2(pv[8 * pp + 2 * x], pv[8 * pp + 2 * x + 1]);
        wsd[x] = cvt_bf16x2(dsv[8 * pp + 2 * x], dsv[8 * pp + 2 * x + 1]);
      }
      pb[pp] = __builtin_bit_cast(bf16x8, make_uint4(wp[0], wp[1], wp[2], wp[3]));
      sb[pp] = __builtin_bit_cast(bf16x8, make_uint4(wsd[0], wsd[1], wsd[2], wsd[3]));
    }
    // ---- dV^T += dO^T P, dK^T += Q^T dS (k-step pp = M-rows of register group pp)
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        // rows (M-rows) 16 pp + 4 h + {0..3} and 16 pp + 8 + 4 h + {0..3}: register group pp
        const bf16x8 ag = tr_operand(L.dos, L_::QROW, 16 * pp + 4 * h, 16 * pp + 8 + 4 * h, 32 * dt, lane);
        dvt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, pb[pp], dvt[dt], 0, 0, 0);
        const bf16x8 aq = tr_operand(L.qs, L_::QROW, 16 * pp + 4 * h, 16 * pp + 8 + 4 * h, 32 * dt, lane);
        dkt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sb[pp], dkt[dt], 0, 0, 0);
      }
    }
    // ---- dS to LDS (M-row major) for dQ
#pragma unroll
    for (int r = 0; r < 16; ++r)
      *reinterpret_cast<uint16_t*>(&L.ds[acc_row(r, h) * L_::SROW + (32 * wave + nl) * 2]) =
          (uint16_t)(cvt_bf16x2(dsv[r], 0.0f) & 0xFFFFu);
    __syncthreads();
    // ---- dQ = scale * dS K for head dims [32 wave, 32 wave + 32)
    if (wave < DT) {
      f32x16 qacc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kBlk / 16; ++ks) {
        const bf16x8 as = *reinterpret_cast<const bf16x8*>(&L.ds[nl * L_::SROW + (16 * ks + 8 * h) * 2]);
        // keys 16 ks + 8 h + {0..7}, the order of the dS row read above
        const bf16x8 bk = tr_operand(L.kr, L_::KROW, 16 * ks + 8 * h, 16 * ks + 8 * h + 4, 32 * wave, lane);
        qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as, bk, qacc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        *reinterpret_cast<uint16_t*>(&L.dqt[acc_row(r, h) * L_::QROW + (32 * wave + nl) * 2]) =
            f32_to_bf16(qacc[r] * D.scale);
    }
  }
  __syncthreads();
  store_dq(((mrows - 1) >> 5) & 1);  // the last sub-chunk's dQ

  // ---- dK, dV of the block: through LDS (row-major fp32 over the K / V staging area) so
  // that the atomic adds of a wave cover contiguous head dims
  __syncthreads();
  float* red = reinterpret_cast<float*>(L.kr);  // kBlk x DH fp32 fits K + V staging
  static_assert(sizeof(float) * kBlk * DH <= 2 * kBlk * BwdLds<DH>::KROW, "reduction buffer fits");
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float val = which == 0 ? dkt[dt][r] * D.scale : dvt[dt][r];
        red[(32 * wave + nl) * DH + 32 * dt + acc_row(r, h)] = val;
      }
    __syncthreads();
    float* dst = (which == 0 ? dk : dv) + (sg * D.N + j0) * DH;
    for (int i = threadIdx.x; i < nvalid * DH; i += kThreads) unsafeAtomicAdd(dst + i, red[i]);
    __syncthreads();
  }
}

// dq[s, t, h, :] = sum over the valid slots of row (s, t, g) of its bf16 partials; one
// thread per 8 head dims.
__global__ void __launch_bounds__(256) dq_merge(Dims D, const int32_t* __restrict__ sel,
                                                const uint16_t* __restrict__ part_dq, float* __restrict__ dq) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int gd8 = D.G * D.d / 8;
  const int64_t row = i / gd8;  // (s, t, g)
  if (row >= (int64_t)D.S * D.T * D.Hkv) return;
  const int c8 = (int)(i % gd8);
  const int g = (int)(row % D.Hkv);
  const int t = (int)((row / D.Hkv) % D.T);
  const int s = (int)(row / ((int64_t)D.Hkv * D.T));
  const int32_t* sl = sel + (((int64_t)s * D.Hkv + g) * D.T + t) * D.k;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int slot = 0; slot < D.k; ++slot) {
    if (sl[slot] < 0) continue;
    const uint4 u = *reinterpret_cast<const uint4*>(part_dq + (row * D.k + slot) * (int64_t)D.G * D.d + c8 * 8);
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      acc[2 * x] += bf16_to_f32((uint16_t)(wv[x] & 0xFFFFu));
      acc[2 * x + 1] += bf16_to_f32((uint16_t)(wv[x] >> 16));
    }
  }
  float* o = dq + (((int64_t)s * D.T + t) * D.H + (int64_t)g * D.G) * D.d + c8 * 8;
  *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// Per row: KL(teacher || student) over the selected blocks and d loss / d block score.
__global__ void __launch_bounds__(256) index_kl_kernel(Dims D, const float* __restrict__ scores,
                                                       const int32_t* __restrict__ sel,
                                                       const float* __restrict__ mass, float sigma,
                                                       float* __restrict__ loss, float* __restrict__ dscore) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (s, g, t)
  if (row >= (int64_t)D.S * D.Hkv * D.T) return;
  const int32_t* sl = sel + row * D.k;
  const float* ms = mass + row * D.k;
  const float* sc = scores + row * (int64_t)D.nb;
  float mx = -INFINITY, tm = 0.0f;
  for (int i = 0; i < D.k; ++i) {
    const int b = sl[i];
    if (b < 0 || b >= D.nb) continue;
    mx = fmaxf(mx, sigma * sc[b]);
    tm += ms[i];
  }
  float l = 0.0f;
  for (int i = 0; i < D.k; ++i) {
    const int b = sl[i];
    if (b >= 0 && b < D.nb) l += expf(sigma * sc[b] - mx);
  }
  const float logl = logf(l);
  float L = 0.0f;
  for (int i = 0; i < D.k; ++i) {
    const int b = sl[i];
    float gsc = 0.0f;
    if (b >= 0 && b < D.nb) {
      const float logps = sigma * sc[b] - mx - logl;
      const float pt = tm > 0.0f ? ms[i] / tm : 0.0f;
      if (pt > 0.0f) L += pt * (logf(pt) - logps);
      gsc = sigma * (expf(logps) - pt);
    }
    dscore[row * D.k + i] = gsc;
  }
  loss[row] = L;
}

// One KV block's index keys in LDS (bf16 row-major, 16-byte row pad: the per-lane 16-byte
// operand reads of a wave are bank-conflict free), plus the block's key-gradient
// accumulator (fp32, one float of row pad).
template <int DI>
struct IdxBwdLds {
  static constexpr int ROW = DI * 2 + 16;
  __attribute__((aligned(16))) unsigned char k[kBlk * ROW];
  float dk[kBlk][DI + 1];
};

// Arg-max of the causal block max-pool per (row, selected block) on the matrix cores, and
// the key side of its gradient.  Work item = (sequence, group, KV block) and up to kRows
// rows of its inverted list; each wave takes 32 rows at a time:
//   S^T = K_I q_I^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys from LDS, B = the 32 rows'
//   index queries straight from memory, k-step ks / lane half h = index dims
//   [16 ks + 8 h, +8)), so a lane's accumulators are 64 keys of ONE row; the row's
//   maximum over its causal keys and the lowest key holding it are in-register scans plus
//   one exchange with lane ^ 32.  Scores are the matrix cores' float32 sums of the exact
//   bf16 products.
// The arg-max goes to am (and to argmax when given); dk_idx[j*] += dscore * q_I[row] is
// accumulated in LDS per item and added to memory once per item with float atomics.  The
// query side dq_idx is gathered per row afterwards (index_dq_gather).
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
  for (int i = threadIdx.x; i < kBlk * (DI + 1); i += kThreads) (&L.dk[0][0])[i] = 0.0f;
  __syncthreads();
  for (int r0 = wave * 32; r0 < w.z; r0 += kWaves * 32) {
    const int r = r0 + nl;  // this lane's row of the item (both lane halves)
    const bool ok = r < w.z;
    int t = 0, slot = 0;
    if (ok) {
      const int e = entries[w.y + r];
      t = e / D.k;
      slot = e - t * D.k;
    }
    const int64_t qr = sg * D.T + t;  // (s, g, t)
    bf16x8 bq[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bq[ks] = ok ? *reinterpret_cast<const bf16x8*>(q_idx + qr * DI + 16 * ks + 8 * h) : bf16x8{};
    f32x16 acc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      acc[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&L.k[(kt * 32 + nl) * L_::ROW + (16 * ks + 8 * h) * 2]);
        acc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[ks], acc[kt], 0, 0, 0);
      }
    }
    // keys kk <= lim are inside the block and causal for the row (kk = 0 always is: the
    // block is one the row selected)
    const int lim = min(nvalid - 1, D.pos0 + t - j0);
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
    if (ok && h == 0) {
      am[qr * D.k + slot] = js >= 0 ? j0 + js : -1;
      if (argmax != nullptr) argmax[qr * D.k + slot] = js >= 0 ? j0 + js : -1;
    }
    if (ok && js >= 0) {
      const float gsc = dscore[qr * D.k + slot];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) atomicAdd(&L.dk[js][16 * ks + 8 * h + i], gsc * (float)bq[ks][i]);
    }
  }
  __syncthreads();
  float* dst = dk_idx + (sg * D.N + j0) * DI;
  for (int i = threadIdx.x; i < nvalid * DI; i += kThreads) {
    const float x = L.dk[i / DI][i % DI];
    if (x != 0.0f) unsafeAtomicAdd(dst + i, x);
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
  hipLaunchKernelGGL((attn_bwd<DH, G>), dim3((unsigned)grid), dim3(kThreads), 0, st, D, q, k, v, dout, lse, drow,
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
  hipLaunchKernelGGL(dq_merge, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, st, D, sel, w.part_dq, dq);
  return hipGetLastError();
}

hipError_t launch_index_kl(const Dims& D, const float* scores, const int32_t* sel, const float* mass, float sigma,
                           float* loss, float* dscore, hipStream_t st) {
  const int64_t rows = (int64_t)D.S * D.Hkv * D.T;
  LaunchScope scope("index_kl", st);
  hipLaunchKernelGGL(index_kl_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, D, scores, sel, mass,
                     sigma, loss, dscore);
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
