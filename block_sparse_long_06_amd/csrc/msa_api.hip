// msa_api.hip -- the C ABI of libmsa.so: host-side validation, workspace sizing,
// error reporting, the opt-in kernel timer, and dispatch to the kernel launchers.
// The operations themselves are documented in include/msa.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "msa_internal.hpp"

namespace {

thread_local std::string g_last_error;

msa_status fail(msa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
msa_status fail(msa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

msa_status ok() {
  g_last_error.clear();
  return MSA_OK;
}

msa_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MSA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool pow2_upto16(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// Validates the problem and fills D.  `need_index` / `need_main` select which
// of the index-branch and main-branch fields must be supported.
msa_status check_problem(const msa_problem* p, msa::Dims* D, bool need_index, bool need_main) {
  if (p == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->batch < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", p->batch);
  if (p->kv_len < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "kv_len must be >= 1 (got %d)", p->kv_len);
  if (p->num_q < 1 || p->num_q > p->kv_len)
    return fail(MSA_ERR_INVALID_ARGUMENT, "num_q must be in [1, kv_len] (got %d, kv_len %d)",
                p->num_q, p->kv_len);
  if (p->num_kv_heads < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "num_kv_heads must be >= 1");
  if (p->num_heads < 1 || p->num_heads % p->num_kv_heads != 0)
    return fail(MSA_ERR_INVALID_ARGUMENT, "num_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                p->num_heads, p->num_kv_heads);
  if (p->block_size < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "block_size must be >= 1");
  if (p->topk < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "topk must be >= 1 (got %d)", p->topk);
  if (p->dtype != MSA_F32 && p->dtype != MSA_BF16)
    return fail(MSA_ERR_INVALID_ARGUMENT, "dtype must be MSA_F32 or MSA_BF16 (got %d)", p->dtype);
  if (p->index_key_dtype != 0 && p->index_key_dtype != p->dtype && p->index_key_dtype != MSA_FP8_E4M3)
    return fail(MSA_ERR_INVALID_ARGUMENT, "index_key_dtype must be 0, dtype or MSA_FP8_E4M3 (got %d)",
                p->index_key_dtype);
  if (p->index_key_dtype == MSA_FP8_E4M3 && p->dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "MSA_FP8_E4M3 index keys need dtype MSA_BF16");
  if (!(p->softmax_scale >= 0.0f) || isinf(p->softmax_scale))
    return fail(MSA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  if (p->block_size != 128)
    return fail(MSA_ERR_UNSUPPORTED, "block_size must be 128 (got %d)", p->block_size);
  if (p->topk > 64) return fail(MSA_ERR_UNSUPPORTED, "topk must be <= 64 (got %d)", p->topk);
  const int64_t nb = ((int64_t)p->kv_len + p->block_size - 1) / p->block_size;
  if (nb > 8192)
    return fail(MSA_ERR_UNSUPPORTED, "kv_len %d gives %lld blocks; at most 8192 are supported",
                p->kv_len, (long long)nb);
  const int64_t rows = (int64_t)p->batch * p->num_kv_heads * p->num_q;
  if (rows * p->topk >= (int64_t(1) << 31))
    return fail(MSA_ERR_UNSUPPORTED, "batch * num_kv_heads * num_q * topk must be < 2^31");
  if ((int64_t)p->batch * p->num_kv_heads > 65535)
    return fail(MSA_ERR_UNSUPPORTED, "batch * num_kv_heads must be <= 65535");
  if (rows * nb >= (int64_t(1) << 40))
    return fail(MSA_ERR_UNSUPPORTED, "block-score matrix too large");
  if (need_index && p->index_dim != 32 && p->index_dim != 64 && p->index_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "index_dim must be 32, 64 or 128 (got %d)", p->index_dim);
  const int G = p->num_heads / p->num_kv_heads;
  if (need_main) {
    if (p->head_dim != 64 && p->head_dim != 128)
      return fail(MSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
    if (!pow2_upto16(G))
      return fail(MSA_ERR_UNSUPPORTED, "num_heads / num_kv_heads must be 1, 2, 4, 8 or 16 (got %d)", G);
  }
  D->S = p->batch;
  D->T = p->num_q;
  D->N = p->kv_len;
  D->H = p->num_heads;
  D->Hkv = p->num_kv_heads;
  D->G = G;
  D->d = p->head_dim;
  D->dI = p->index_dim;
  D->B = p->block_size;
  D->k = p->topk;
  D->nb = (int)nb;
  D->pos0 = p->kv_len - p->num_q;
  D->dtype = p->dtype;
  D->kdtype = p->index_key_dtype == MSA_FP8_E4M3 ? MSA_FP8_E4M3 : p->dtype;
  D->kv_lens = nullptr;
  D->block_table = nullptr;
  D->bt_stride = 0;
  D->num_pages = 0;
  D->scale = p->softmax_scale > 0.0f ? p->softmax_scale : 1.0f / sqrtf((float)p->head_dim);
  return MSA_OK;
}

// Validates a per-sequence cache layout on the host and records it in D.
msa_status apply_layout(const msa_kv_layout* L, msa::Dims* D) {
  if (L == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "layout is NULL");
  if (L->kv_lens == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "layout->kv_lens is NULL");
  if (L->block_table != nullptr) {
    if (L->table_stride < D->nb)
      return fail(MSA_ERR_INVALID_ARGUMENT, "layout->table_stride %d < ceil(kv_len / block_size) = %d",
                  L->table_stride, D->nb);
    if (L->num_pages < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "layout->num_pages must be >= 1");
    if ((int64_t)L->num_pages * D->Hkv * D->B * (D->d > D->dI ? D->d : D->dI) >= (int64_t(1) << 40))
      return fail(MSA_ERR_UNSUPPORTED, "page pool too large");
  }
  D->kv_lens = L->kv_lens;
  D->block_table = L->block_table;
  D->bt_stride = L->block_table != nullptr ? L->table_stride : 0;
  D->num_pages = L->block_table != nullptr ? L->num_pages : 0;
  return MSA_OK;
}

// The fused selection: bf16 queries, lists of 15 blocks.
msa_status check_fused(const msa::Dims& D) {
  if (D.dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "msa_index_topk needs dtype MSA_BF16");
  if (D.k > 16) return fail(MSA_ERR_UNSUPPORTED, "msa_index_topk supports topk <= 16 (got %d)", D.k);
  return MSA_OK;
}

// The token-level calls: decode shapes, bf16 queries.
msa_status check_token(const msa::Dims& D, int budget) {
  if (D.dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "the token-level calls need dtype MSA_BF16");
  if (D.T > 8) return fail(MSA_ERR_UNSUPPORTED, "the token-level calls take num_q <= 8 (got %d)", D.T);
  if (budget < 1 || budget > 8192) return fail(MSA_ERR_UNSUPPORTED, "budget must be in 1 .. 8192 (got %d)", budget);
  if ((int64_t)D.S * D.Hkv * D.T > 0x7FFFFFFF) return fail(MSA_ERR_UNSUPPORTED, "too many rows");
  return MSA_OK;
}

// The training calls run the bf16 kernels only.
msa_status check_train(const msa::Dims& D, bool index) {
  if (D.dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "the training calls need dtype MSA_BF16");
  if (index && D.kdtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "the index-branch training calls need bf16 index keys");
  return MSA_OK;
}

#define REQUIRE_PTR(x)                                                         \
  do {                                                                         \
    if ((x) == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, #x " is NULL"); \
  } while (0)

// ------------------------------------------------------------------ profiler state
struct ProfRecord {
  std::string name;
  hipEvent_t start, stop;
  bool used;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof;

// ------------------------------------------------------------------ allocation-free decode
// The decode partials of msa_sparse_attn_decode_noalloc live in this file-scope device array
// (one copy per device, held until the process ends).  In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the address hipGetSymbolAddress
// returns for the current device, resolved once per device and kept here.
static __device__ __align__(256) unsigned char scratch[MSA_DECODE_SCRATCH_BYTES];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

msa_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(MSA_ERR_DEVICE, "device %d outside the %d devices the scratch table holds", dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MSA_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

namespace msa {

LaunchScope::LaunchScope(const char* name, hipStream_t s) : slot(-1), stream(s) {
  if (!g_prof_on) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (size_t i = 0; i < g_prof.size(); ++i)
    if (!g_prof[i].used) { slot = (int)i; break; }
  if (slot < 0) {
    ProfRecord r;
    if (hipEventCreate(&r.start) != hipSuccess) return;
    if (hipEventCreate(&r.stop) != hipSuccess) { (void)hipEventDestroy(r.start); return; }
    r.used = false;
    g_prof.push_back(r);
    slot = (int)g_prof.size() - 1;
  }
  g_prof[slot].used = true;
  g_prof[slot].name = name;
  (void)hipEventRecord(g_prof[slot].start, stream);
}

LaunchScope::~LaunchScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  (void)hipEventRecord(g_prof[slot].stop, stream);
}

}  // namespace msa

extern "C" {

const char* msa_status_string(msa_status s) {
  // a C caller may pass any int: read the bits as one, not as the C++ enum (whose range
  // stops at 7), so an unknown value is not undefined behaviour here
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARGUMENT: return "MSA_ERR_INVALID_ARGUMENT";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
    case MSA_ERR_DEVICE: return "MSA_ERR_DEVICE";
  }
  return "MSA_ERR_UNKNOWN";
}

const char* msa_last_error_message(void) { return g_last_error.c_str(); }

size_t msa_workspace_bytes(const msa_problem* prob, int which) {
  msa::Dims D;
  switch (which) {
    case MSA_CALL_INVERT:
      if (check_problem(prob, &D, false, false) != MSA_OK) return 0;
      return msa::invert_workspace_bytes(D);
    case MSA_CALL_PREFILL:
      if (check_problem(prob, &D, false, true) != MSA_OK) return 0;
      return msa::prefill_workspace_bytes(D);
    case MSA_CALL_DECODE:
      if (check_problem(prob, &D, false, true) != MSA_OK) return 0;
      return msa::decode_workspace_bytes(D);
    case MSA_CALL_BACKWARD:
      if (check_problem(prob, &D, false, true) != MSA_OK || check_train(D, false) != MSA_OK) return 0;
      return msa::backward_workspace_bytes(D);
    case MSA_CALL_INDEX_TOPK:
      if (check_problem(prob, &D, true, false) != MSA_OK || check_fused(D) != MSA_OK) return 0;
      return msa::index_topk_workspace_bytes(D);
    case MSA_CALL_TOKEN_DECODE:
      if (check_problem(prob, &D, false, true) != MSA_OK || check_token(D, 2048) != MSA_OK) return 0;
      return msa::token_workspace_bytes(D, 2048);
    case MSA_CALL_INDEX_BACKWARD:
      if (check_problem(prob, &D, true, false) != MSA_OK || check_train(D, true) != MSA_OK) return 0;
      return msa::index_backward_workspace_bytes(D);
    default:
      return 0;
  }
}

msa_status msa_index_scores(const msa_problem* prob, const void* q_idx, const void* k_idx,
                            float* scores, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, true, false);
  if (st != MSA_OK) return st;
  REQUIRE_PTR(q_idx);
  REQUIRE_PTR(k_idx);
  REQUIRE_PTR(scores);
  return device_status(msa::launch_index_scores(D, q_idx, k_idx, scores, (hipStream_t)stream),
                       "msa_index_scores launch");
}

msa_status msa_index_topk(const msa_problem* prob, const void* q_idx, const void* k_idx, int32_t* sel,
                          void* workspace, size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, true, false);
  if (st != MSA_OK) return st;
  if ((st = check_fused(D)) != MSA_OK) return st;
  REQUIRE_PTR(q_idx);
  REQUIRE_PTR(k_idx);
  REQUIRE_PTR(sel);
  const size_t need = msa::index_topk_workspace_bytes(D);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "msa_index_topk needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  REQUIRE_PTR(workspace);
  return device_status(msa::launch_index_topk(D, q_idx, k_idx, sel, workspace, (hipStream_t)stream),
                       "msa_index_topk launch");
}

msa_status msa_block_topk(const msa_problem* prob, const float* scores, int32_t* sel,
                          void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, false);
  if (st != MSA_OK) return st;
  REQUIRE_PTR(scores);
  REQUIRE_PTR(sel);
  return device_status(msa::launch_block_topk(D, scores, sel, (hipStream_t)stream),
                       "msa_block_topk launch");
}

msa_status msa_invert_selection(const msa_problem* prob, const int32_t* sel,
                                int32_t* csr_offsets, int32_t* csr_entries, void* workspace,
                                size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, false);
  if (st != MSA_OK) return st;
  REQUIRE_PTR(sel);
  REQUIRE_PTR(csr_offsets);
  REQUIRE_PTR(csr_entries);
  const size_t need = msa::invert_workspace_bytes(D);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "msa_invert_selection needs %zu workspace bytes, got %zu",
                need, workspace_bytes);
  if (need > 0) REQUIRE_PTR(workspace);
  return device_status(
      msa::launch_invert(D, sel, csr_offsets, csr_entries, workspace, (hipStream_t)stream),
      "msa_invert_selection launch");
}

msa_status msa_sparse_attn_prefill(const msa_problem* prob, const void* q, const void* k,
                                   const void* v, const int32_t* csr_offsets,
                                   const int32_t* csr_entries, const int32_t* sel, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, true);
  if (st != MSA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(csr_offsets);
  REQUIRE_PTR(csr_entries);
  REQUIRE_PTR(sel);
  REQUIRE_PTR(out);
  const size_t need = msa::prefill_workspace_bytes(D);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "msa_sparse_attn_prefill needs %zu workspace bytes, got %zu", need, workspace_bytes);
  REQUIRE_PTR(workspace);
  return device_status(msa::launch_prefill(D, q, k, v, csr_offsets, csr_entries, sel, out,
                                           workspace, (hipStream_t)stream),
                       "msa_sparse_attn_prefill launch");
}

msa_status msa_sparse_attn_decode(const msa_problem* prob, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* sel, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, true);
  if (st != MSA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(sel);
  REQUIRE_PTR(out);
  const size_t need = msa::decode_workspace_bytes(D);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "msa_sparse_attn_decode needs %zu workspace bytes, got %zu", need, workspace_bytes);
  REQUIRE_PTR(workspace);
  return device_status(
      msa::launch_decode(D, q, k_cache, v_cache, sel, out, workspace, (hipStream_t)stream),
      "msa_sparse_attn_decode launch");
}

msa_status msa_sparse_attn_decode_noalloc(const msa_problem* prob, const void* q, const void* k_cache,
                                          const void* v_cache, const int32_t* sel, void* out, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, true);
  if (st != MSA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(sel);
  REQUIRE_PTR(out);
  const size_t need = msa::decode_workspace_bytes(D);
  if (need > (size_t)MSA_DECODE_SCRATCH_BYTES)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "msa_sparse_attn_decode_noalloc: the problem needs %zu bytes of partials, above the %zu-byte "
                "static scratch (use msa_sparse_attn_decode with a workspace)",
                need, (size_t)MSA_DECODE_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws)) != MSA_OK) return st;
  return device_status(msa::launch_decode(D, q, k_cache, v_cache, sel, out, ws, (hipStream_t)stream),
                       "msa_sparse_attn_decode_noalloc launch");
}

msa_status msa_index_scores_kv(const msa_problem* prob, const msa_kv_layout* layout, const void* q_idx,
                               const void* k_idx, float* scores, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, true, false);
  if (st != MSA_OK) return st;
  st = apply_layout(layout, &D);
  if (st != MSA_OK) return st;
  REQUIRE_PTR(q_idx);
  REQUIRE_PTR(k_idx);
  REQUIRE_PTR(scores);
  return device_status(msa::launch_index_scores(D, q_idx, k_idx, scores, (hipStream_t)stream),
                       "msa_index_scores_kv launch");
}

msa_status msa_block_topk_kv(const msa_problem* prob, const msa_kv_layout* layout, const float* scores,
                             int32_t* sel, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, false);
  if (st != MSA_OK) return st;
  st = apply_layout(layout, &D);
  if (st != MSA_OK) return st;
  REQUIRE_PTR(scores);
  REQUIRE_PTR(sel);
  return device_status(msa::launch_block_topk(D, scores, sel, (hipStream_t)stream), "msa_block_topk_kv launch");
}

msa_status msa_sparse_attn_decode_kv(const msa_problem* prob, const msa_kv_layout* layout, const void* q,
                                     const void* k_cache, const void* v_cache, const int32_t* sel, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, true);
  if (st != MSA_OK) return st;
  st = apply_layout(layout, &D);
  if (st != MSA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(sel);
  REQUIRE_PTR(out);
  const size_t need = msa::decode_workspace_bytes(D);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "msa_sparse_attn_decode_kv needs %zu workspace bytes, got %zu", need, workspace_bytes);
  REQUIRE_PTR(workspace);
  return device_status(
      msa::launch_decode(D, q, k_cache, v_cache, sel, out, workspace, (hipStream_t)stream),
      "msa_sparse_attn_decode_kv launch");
}

msa_status msa_sparse_attn_prefill_train(const msa_problem* prob, const void* q, const void* k,
                                         const void* v, const int32_t* csr_offsets,
                                         const int32_t* csr_entries, const int32_t* sel, void* out,
                                         float* lse, float* block_mass, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, true);
  if (st != MSA_OK) return st;
  if ((st = check_train(D, false)) != MSA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(csr_offsets);
  REQUIRE_PTR(csr_entries);
  REQUIRE_PTR(sel);
  REQUIRE_PTR(out);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(block_mass);
  const size_t need = msa::prefill_workspace_bytes(D);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "msa_sparse_attn_prefill_train needs %zu workspace bytes, got %zu", need, workspace_bytes);
  REQUIRE_PTR(workspace);
  return device_status(msa::launch_prefill(D, q, k, v, csr_offsets, csr_entries, sel, out, workspace,
                                           (hipStream_t)stream, lse, block_mass),
                       "msa_sparse_attn_prefill_train launch");
}

msa_status msa_sparse_attn_backward(const msa_problem* prob, const void* q, const void* k,
                                    const void* v, const void* out, const void* dout,
                                    const float* lse, const int32_t* sel, const int32_t* csr_offsets,
                                    const int32_t* csr_entries, float* dq, float* dk, float* dv,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, true);
  if (st != MSA_OK) return st;
  if ((st = check_train(D, false)) != MSA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  REQUIRE_PTR(dout);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(sel);
  REQUIRE_PTR(csr_offsets);
  REQUIRE_PTR(csr_entries);
  REQUIRE_PTR(dq);
  REQUIRE_PTR(dk);
  REQUIRE_PTR(dv);
  const size_t need = msa::backward_workspace_bytes(D);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "msa_sparse_attn_backward needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  REQUIRE_PTR(workspace);
  return device_status(msa::launch_attn_backward(D, q, k, v, out, dout, lse, sel, csr_offsets, csr_entries, dq, dk,
                                                 dv, workspace, (hipStream_t)stream),
                       "msa_sparse_attn_backward launch");
}

msa_status msa_index_kl(const msa_problem* prob, const float* scores, const int32_t* sel,
                        const float* block_mass, float sigma, float* loss, float* dscores,
                        void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, true, false);
  if (st != MSA_OK) return st;
  if ((st = check_train(D, true)) != MSA_OK) return st;
  if (!(sigma >= 0.0f) || isinf(sigma)) return fail(MSA_ERR_INVALID_ARGUMENT, "sigma must be finite and >= 0");
  REQUIRE_PTR(scores);
  REQUIRE_PTR(sel);
  REQUIRE_PTR(block_mass);
  REQUIRE_PTR(loss);
  REQUIRE_PTR(dscores);
  const float sg = sigma > 0.0f ? sigma : 1.0f / sqrtf((float)D.dI);
  return device_status(msa::launch_index_kl(D, scores, sel, block_mass, sg, loss, dscores, (hipStream_t)stream),
                       "msa_index_kl launch");
}

msa_status msa_index_backward(const msa_problem* prob, const void* q_idx, const void* k_idx,
                              const int32_t* csr_offsets, const int32_t* csr_entries,
                              const float* dscores, float* dq_idx, float* dk_idx, int32_t* argmax,
                              void* workspace, size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, true, false);
  if (st != MSA_OK) return st;
  if ((st = check_train(D, true)) != MSA_OK) return st;
  REQUIRE_PTR(q_idx);
  REQUIRE_PTR(k_idx);
  REQUIRE_PTR(csr_offsets);
  REQUIRE_PTR(csr_entries);
  REQUIRE_PTR(dscores);
  REQUIRE_PTR(dq_idx);
  REQUIRE_PTR(dk_idx);
  const size_t need = msa::index_backward_workspace_bytes(D);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "msa_index_backward needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  REQUIRE_PTR(workspace);
  return device_status(msa::launch_index_backward(D, q_idx, k_idx, csr_offsets, csr_entries, dscores, dq_idx,
                                                  dk_idx, argmax, workspace, (hipStream_t)stream),
                       "msa_index_backward launch");
}

msa_status msa_token_scores(const msa_problem* prob, const void* q_idx, const void* k_idx, float* scores,
                            void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, true, false);
  if (st != MSA_OK) return st;
  if ((st = check_token(D, 1)) != MSA_OK) return st;
  REQUIRE_PTR(q_idx);
  REQUIRE_PTR(k_idx);
  REQUIRE_PTR(scores);
  return device_status(msa::launch_token_scores(D, q_idx, k_idx, scores, (hipStream_t)stream),
                       "msa_token_scores launch");
}

msa_status msa_token_topk(const msa_problem* prob, int32_t budget, const float* scores, int32_t* sel_tok,
                          void* workspace, size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, false);
  if (st != MSA_OK) return st;
  if ((st = check_token(D, budget)) != MSA_OK) return st;
  REQUIRE_PTR(scores);
  REQUIRE_PTR(sel_tok);
  const size_t need = msa::token_topk_workspace_bytes(D);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "msa_token_topk needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  REQUIRE_PTR(workspace);
  return device_status(msa::launch_token_topk(D, budget, scores, sel_tok, workspace, (hipStream_t)stream),
                       "msa_token_topk launch");
}

size_t msa_token_workspace_bytes(const msa_problem* prob, int32_t budget) {
  msa::Dims D;
  if (check_problem(prob, &D, false, true) != MSA_OK || check_token(D, budget) != MSA_OK) return 0;
  return msa::token_workspace_bytes(D, budget);
}

msa_status msa_token_attn_decode(const msa_problem* prob, int32_t budget, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* sel_tok, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, true);
  if (st != MSA_OK) return st;
  if ((st = check_token(D, budget)) != MSA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(sel_tok);
  REQUIRE_PTR(out);
  const size_t need = msa::token_workspace_bytes(D, budget);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "msa_token_attn_decode needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  REQUIRE_PTR(workspace);
  return device_status(msa::launch_token_attn(D, budget, q, k_cache, v_cache, sel_tok, out, workspace,
                                              (hipStream_t)stream),
                       "msa_token_attn_decode launch");
}

msa_status msa_sparse_attn_prefill_kv(const msa_problem* prob, const msa_kv_layout* layout, const void* q,
                                      const void* k, const void* v, const int32_t* csr_offsets,
                                      const int32_t* csr_entries, const int32_t* sel, void* out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  msa::Dims D;
  msa_status st = check_problem(prob, &D, false, true);
  if (st != MSA_OK) return st;
  st = apply_layout(layout, &D);
  if (st != MSA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(csr_offsets);
  REQUIRE_PTR(csr_entries);
  REQUIRE_PTR(sel);
  REQUIRE_PTR(out);
  const size_t need = msa::prefill_workspace_bytes(D);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "msa_sparse_attn_prefill_kv needs %zu workspace bytes, got %zu", need, workspace_bytes);
  REQUIRE_PTR(workspace);
  return device_status(msa::launch_prefill(D, q, k, v, csr_offsets, csr_entries, sel, out, workspace,
                                           (hipStream_t)stream),
                       "msa_sparse_attn_prefill_kv launch");
}

msa_status msa_profiler_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return ok();
}

msa_status msa_profiler_read(const char* kernel, double* total_ms, int64_t* launches, int reset) {
  if (total_ms == nullptr || launches == nullptr)
    return fail(MSA_ERR_INVALID_ARGUMENT, "total_ms and launches must not be NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : g_prof) {
    if (!r.used) continue;
    if (kernel != nullptr && kernel[0] != '\0' && r.name != kernel) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return device_status(e, "profiler event wait");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return device_status(e, "profiler elapsed time");
    tot += ms;
    ++n;
  }
  if (reset)
    for (auto& r : g_prof) r.used = false;
  *total_ms = tot;
  *launches = n;
  return ok();
}

msa_status msa_profiler_samples(const char* kernel, float* ms_out, int64_t capacity, int64_t* count) {
  if (count == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "count must not be NULL");
  if (capacity > 0 && ms_out == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "ms_out must not be NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int64_t n = 0;
  for (auto& r : g_prof) {
    if (!r.used) continue;
    if (kernel != nullptr && kernel[0] != '\0' && r.name != kernel) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return device_status(e, "profiler event wait");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return device_status(e, "profiler elapsed time");
    if (n < capacity) ms_out[n] = ms;
    ++n;
  }
  *count = n;
  return ok();
}

}  // extern "C"
