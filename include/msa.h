/*
 * msa.h -- C ABI of libmsa.so: MiniMax Sparse Attention (MSA) prefill and decode
 * on AMD Instinct MI355X (gfx950).
 *
 * Method, as described on the pages (cited by page title and section):
 *   [P1] "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比",
 *        sections 第一步：粗筛 (index branch, block max pooling, top-16 blocks with
 *        the query's own block forced), 第二步：精算 (exact attention over the
 *        16 x 128 = 2048 selected tokens), Kernel 创新：Outer Gather Q (KV block as
 *        the outer loop: gather every query that chose a block, read it once).
 *   [P3] "稀疏注意力速览（Sparse Attention，2019 ~ 2026）", entry "MiniMax Sparse
 *        Attention（MSA）" (GQA groups, one index-query head and a shared index-key
 *        head per group, in-block max-pool, per-group top-k, forced local block).
 *
 * Conventions for every call:
 *   - All tensor arguments are DEVICE pointers to dense row-major arrays owned by
 *     the caller; the library never allocates, frees or retains device memory
 *     and never keeps a pointer after the call returns.
 *   - The problem struct is a HOST pointer read during the call only.
 *   - Each call validates its arguments on the host, then enqueues its kernels
 *     asynchronously on `stream` (a hipStream_t; NULL = the default stream). It
 *     never synchronises the device.
 *   - On any status other than MSA_OK nothing was enqueued and no output was
 *     touched; msa_last_error_message() describes the failure (thread-local).
 *     Launch failures report MSA_ERR_DEVICE.  Asynchronous device faults surface
 *     at the caller's next synchronisation.
 *   - Calls keep no state between them, with two exceptions.  The bf16 prefill
 *     call creates, on its first use per device, one extra stream (default priority)
 *     and two events that it keeps until the process ends; a process-wide lock
 *     serialises its use of them, so prefill calls from several host threads take
 *     turns for that part of the call (see msa_sparse_attn_prefill).  The opt-in
 *     profiler below is global state.  Calls are otherwise thread-safe.
 *
 * Shapes (S = batch, T = queries per sequence, N = kv length, H = query heads,
 * Hkv = KV heads = GQA groups, G = H / Hkv, d = head dim, dI = index dim,
 * B = block size, nb = ceil(N / B), k = top-k):
 *   q       [S, T, H, d]     query head h belongs to group g = h / G
 *   k, v    [S, Hkv, N, d]   keys / values (the full, uncompressed cache)
 *   q_idx   [S, Hkv, T, dI]  one index-query head per group
 *   k_idx   [S, Hkv, N, dI]  one index-key head per group
 *   scores  [S, Hkv, T, nb]  float32 block scores
 *   sel     [S, Hkv, T, k]   int32 selected block ids
 *   out     [S, T, H, d]     attention output (same dtype as q)
 * The T queries are the LAST T positions: query row t sits at p_t = N - T + t and
 * owns block b_t = floor(p_t / B).  Element types follow problem.dtype (float32
 * or bfloat16 bit patterns); scores and log-sum-exps are always float32.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, inconsistent or out-of-range sizes */
  MSA_ERR_UNSUPPORTED = 2,        /* valid problem outside what the kernels implement */
  MSA_ERR_WORKSPACE_TOO_SMALL = 3,
  MSA_ERR_DEVICE = 4              /* a HIP runtime call or kernel launch failed */
} msa_status;

typedef enum {
  MSA_F32 = 0,
  MSA_BF16 = 1,
  MSA_FP8_E4M3 = 2  /* OCP FP8 E4M3 (bias 7, max 448, NaN 0x7F/0xFF): index keys only */
} msa_dtype;

typedef struct {
  int32_t batch;         /* S >= 1 */
  int32_t num_q;         /* T, 1 <= T <= N */
  int32_t kv_len;        /* N, 1 <= N <= 8192 * block_size (need not be a multiple of it) */
  int32_t num_heads;     /* H, a multiple of num_kv_heads */
  int32_t num_kv_heads;  /* Hkv >= 1; G = H / Hkv must be 1, 2, 4, 8 or 16 */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t index_dim;     /* dI: 32, 64 or 128 */
  int32_t block_size;    /* B: 128 */
  int32_t topk;          /* k: 1..64 */
  int32_t dtype;         /* msa_dtype of q, k, v, q_idx, out (and k_idx, see below) */
  float softmax_scale;   /* main-branch logit scale; 0 selects 1/sqrt(d) */
  int32_t index_key_dtype; /* element type of k_idx: 0 = dtype, or MSA_FP8_E4M3 (with
                              dtype MSA_BF16): 1-byte index keys halve the bytes the
                              decode-time index stream reads.  Any scale of the keys is
                              the caller's to fold into q_idx (scores are bilinear). */
} msa_problem;

/* Which call a workspace size is asked for (msa_workspace_bytes). */
enum { MSA_CALL_INVERT = 2, MSA_CALL_PREFILL = 3, MSA_CALL_DECODE = 4, MSA_CALL_BACKWARD = 5,
       MSA_CALL_INDEX_BACKWARD = 6, MSA_CALL_TOKEN_DECODE = 7, MSA_CALL_INDEX_TOPK = 8 };

/*
 * a1. Index branch scoring fused with the causal block max-pool
 *     ([P1] 第一步：粗筛 items 1-2; [P3] MSA entry).
 *   scores[s,g,t,b] = max_{j in [bB, min((b+1)B-1, p_t)]} sum_c q_idx[s,g,t,c] k_idx[s,g,j,c]
 *   for b <= b_t, accumulated in float32 (bf16 products are exact in fp32).
 *   Entries with b > b_t are NOT written (they are not eligible).
 *   Raw dot product: no scale and no activation (both are monotone and would not
 *   change the selection).
 *   With index_key_dtype = MSA_FP8_E4M3, k_idx holds one E4M3 byte per element; each
 *   key is decoded exactly (E4M3 values are bf16 values) and the products are formed
 *   as for bf16 keys.
 */
msa_status msa_index_scores(const msa_problem* prob, const void* q_idx, const void* k_idx,
                            float* scores, void* stream);

/*
 * a2. Per-group block top-k with the own block forced
 *     ([P1] 第一步：粗筛 item 3 and the head-pattern appendix: the only forced rule
 *     is that the query's own block is selected; [P3] MSA entry).
 *   sel[s,g,t,:] = {b_t} plus the k-1 best blocks b < b_t ordered by
 *   (score descending, block id ascending); fewer if b_t + 1 < k.
 *   Written in ascending block order, padded with -1 to k entries.
 *   Scores are compared as IEEE float32 values (+0 == -0); NaN scores are
 *   outside the contract.  Reads only scores[s,g,t,0..b_t].
 */
msa_status msa_block_topk(const msa_problem* prob, const float* scores, int32_t* sel,
                          void* stream);

/*
 * a1 + a2 fused: the selection of msa_block_topk computed straight from the index keys,
 *     without the [S, Hkv, T, nb] block scores ([P1] 第一步：粗筛).  Each row's block
 *     maxima are formed as in msa_index_scores and merged, 16 blocks at a time, into a
 *     running list of the row's 15 best past blocks (per span of 1024 blocks); a second
 *     kernel merges the spans' lists and appends the own block.  The result is bit-identical
 *     to msa_index_scores followed by msa_block_topk.  dtype MSA_BF16 (index keys bf16 or
 *     E4M3), topk <= 16; other problems return MSA_ERR_UNSUPPORTED.  With num_q < 256 the
 *     call runs those two kernels itself into the workspace (scores of fewer than 256 rows).
 *   workspace: msa_workspace_bytes(prob, MSA_CALL_INDEX_TOPK) bytes
 *     (S * Hkv * T * ceil(nb / 1024) * 15 candidates of 8 bytes; S * Hkv * T * nb floats
 *     when num_q < 256).
 */
msa_status msa_index_topk(const msa_problem* prob, const void* q_idx, const void* k_idx, int32_t* sel,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * a3. Selection inversion into per-(sequence, group, block) query lists: the index
 *     of the Outer-Gather-Q order ([P1] Kernel 创新：Outer Gather Q).
 *   csr_offsets [S, Hkv, nb + 1] int32: global positions into csr_entries; the list
 *     of (s, g, b) is csr_entries[csr_offsets[s,g,b] .. csr_offsets[s,g,b+1]).
 *     csr_offsets[s,g,nb] == csr_offsets[s,g+1,0] (one flat array, (s, g, b) order).
 *   csr_entries [S * Hkv * T * k] int32 (capacity): entry value t * k + slot for every
 *     query row t whose sel[s,g,t,slot] == b, in ascending t.  Deterministic.
 *   workspace: msa_workspace_bytes(prob, MSA_CALL_INVERT) bytes of device memory.
 *   Requires S * Hkv * T * k < 2^31.  Entries of sel outside [0, nb) count as -1.
 *   Each row of sel must hold distinct block ids (msa_block_topk's rows do).  A row
 *   that repeats an id is outside the contract: the id is listed once, for its first
 *   slot, and the later slots are treated as -1 (so every position up to
 *   csr_offsets[S-1, Hkv-1, nb] is written); msa_sparse_attn_prefill's output for such
 *   a row is then unspecified.
 */
msa_status msa_invert_selection(const msa_problem* prob, const int32_t* sel,
                                int32_t* csr_offsets, int32_t* csr_entries, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * a4 + a5. Prefill main branch in Outer-Gather-Q order plus the log-sum-exp merge
 *     ([P1] 第二步：精算 and Kernel 创新：Outer Gather Q; [P3] MSA entry: the main branch
 *     attends exactly, with softmax, to those blocks only).
 *   For every (s, g, b) the K/V block is staged on chip once and every query row of
 *   its csr list (all G heads of the group) is processed against it, giving a
 *   per-(row, slot, head) partial (lse, O).  A second kernel merges the partials:
 *     out[s,t,h,:] = sum_{j in J} softmax_j(scale * q[s,t,h,:] . k[s,g,j,:]) v[s,g,j,:]
 *     J = union over valid slots of [bB, (b+1)B) intersected with [0, p_t].
 *   sel, csr_offsets and csr_entries are the outputs of the two calls above (sel rows
 *   hold distinct blocks b <= b_t).
 *   bf16 problems: a block chosen by at least half (and at least 32) of the rows of one
 *   128-position query tile that has at least two such blocks is instead processed
 *   tile-wise -- the tile's Q rows stay on chip while the block streams past, and each
 *   row keeps one partial over all such blocks -- and only the remaining (row, block)
 *   entries of the CSR take the Outer-Gather-Q kernel.  The result is the same exact attention.  Setting the
 *   environment variable MSA_HOT_TILES=0 (read at each call) sends every entry through
 *   the Outer-Gather-Q kernel.  The tile-wise kernel runs on a second stream the library
 *   creates once per device (default priority), forked from `stream` by an event after
 *   the split and joined back into it by an event before the merge, so all work is still
 *   ordered on `stream` when the call returns; MSA_TILE_OVERLAP=0 keeps it on `stream`.
 *   Calls on several host threads take turns between that fork and join.
 *   workspace: msa_workspace_bytes(prob, MSA_CALL_PREFILL) bytes (partials, work list,
 *   query-tile split).
 */
msa_status msa_sparse_attn_prefill(const msa_problem* prob, const void* q, const void* k,
                                   const void* v, const int32_t* csr_offsets,
                                   const int32_t* csr_entries, const int32_t* sel, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * a6. Decode main branch: query-centric split-K over each query's selected blocks
 *     ([P1] 第二步：精算 -- every generated token attends to a fixed 2048 tokens;
 *     the whole uncompressed cache stays resident).  Same output definition as the
 *     prefill call; any T is accepted, no inversion is needed.
 *   k, v are the cache [S, Hkv, N, d]; q is [S, T, H, d] (T = 1 for plain decode).
 *   workspace: msa_workspace_bytes(prob, MSA_CALL_DECODE) bytes.
 */
msa_status msa_sparse_attn_decode(const msa_problem* prob, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* sel, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * msa_sparse_attn_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, kernels and output as msa_sparse_attn_decode; the decode
 * partials go to a static device array of MSA_DECODE_SCRATCH_BYTES owned by the library
 * (one per device, held until the process ends).  The call allocates and frees nothing.
 *   - A problem whose msa_workspace_bytes(prob, MSA_CALL_DECODE) exceeds
 *     MSA_DECODE_SCRATCH_BYTES returns MSA_ERR_WORKSPACE_TOO_SMALL (at bf16 and d = 128 a
 *     partial takes 260 bytes, so 32 MiB holds S * T * Hkv * k * G of about 129,000: 16
 *     sequences x 7 queries of the 64-head, top-16 shape).
 *   - Every call on one device uses that device's one array: calls that may overlap on a
 *     device (several streams, or several host threads) race and must be serialised by
 *     the caller.  Nothing in the array needs to start at zero; it keeps the last call's
 *     partials.
 *   - The first call on a device looks up the array's device address (no allocation);
 *     make one call outside any graph capture first if the capture must not see it.
 */
#define MSA_DECODE_SCRATCH_BYTES (32u << 20)
msa_status msa_sparse_attn_decode_noalloc(const msa_problem* prob, const void* q, const void* k_cache,
                                          const void* v_cache, const int32_t* sel, void* out, void* stream);

/*
 * Serving variants of the decode step: ragged per-sequence cache lengths and paged caches
 * ([P1] 第二步：精算 -- the whole uncompressed cache stays resident, and each new token
 * reads 16 of its 128-token blocks; one page here IS one such block).
 *
 *   kv_lens      DEVICE int32 [S]: sequence s holds positions 0 .. kv_lens[s]-1, and its
 *                T queries are its last T positions (p = kv_lens[s] - T + t).  Required.
 *                Contract: T <= kv_lens[s] <= prob->kv_len; a value outside is clamped to
 *                that range on the device (never an out-of-bounds access).
 *   block_table  DEVICE int32 [S, table_stride] or NULL.  NULL: the caches are dense
 *                [S, Hkv, kv_len, w] (w = head_dim for k/v, index_dim for k_idx) and only
 *                kv_lens applies.  Otherwise every cache argument is a page pool
 *                [num_pages, Hkv, block_size, w] and logical block b of sequence s is page
 *                block_table[s * table_stride + b] (entries for b < ceil(kv_lens[s] / B) are
 *                read).  A page id outside [0, num_pages) reads as zeros (its scores and
 *                attention contributions are then meaningless, but no memory outside the
 *                pools is touched).
 *   table_stride >= ceil(kv_len / block_size) when block_table != NULL.
 *   num_pages    >= 1 when block_table != NULL.
 * The problem's kv_len is the capacity (the largest allowed length); nb = ceil(kv_len / B)
 * sizes the scores rows.  Any num_q: decode, speculative decode and batched chunked prefill
 * (every sequence appends num_q queries at its end).  The prefill call runs every pair in
 * the Outer-Gather-Q order (no query-tile pass); msa_invert_selection needs no layout.
 */
typedef struct {
  const int32_t* kv_lens;
  const int32_t* block_table;
  int32_t table_stride;
  int32_t num_pages;
} msa_kv_layout;

/* a1 of msa_index_scores for the layout: scores [S, Hkv, T, nb], entries b > b_t of each
 * row not written, b_t = floor((kv_lens[s] - T + t) / B). */
msa_status msa_index_scores_kv(const msa_problem* prob, const msa_kv_layout* layout, const void* q_idx,
                               const void* k_idx, float* scores, void* stream);

/* a2 of msa_block_topk with the own block b_t of each row taken from kv_lens (only
 * layout->kv_lens is read). */
msa_status msa_block_topk_kv(const msa_problem* prob, const msa_kv_layout* layout, const float* scores,
                             int32_t* sel, void* stream);

/* a4 + a5 of msa_sparse_attn_prefill for the layout (workspace: msa_workspace_bytes(prob,
 * MSA_CALL_PREFILL) bytes). */
msa_status msa_sparse_attn_prefill_kv(const msa_problem* prob, const msa_kv_layout* layout, const void* q,
                                      const void* k, const void* v, const int32_t* csr_offsets,
                                      const int32_t* csr_entries, const int32_t* sel, void* out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* a6 of msa_sparse_attn_decode for the layout (workspace: msa_workspace_bytes(prob,
 * MSA_CALL_DECODE) bytes). */
msa_status msa_sparse_attn_decode_kv(const msa_problem* prob, const msa_kv_layout* layout, const void* q,
                                     const void* k_cache, const void* v_cache, const int32_t* sel, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training path ([P1] 索引分支训练：KL 对齐 -- the index branch learns from the main
 * branch's attention distribution through a KL divergence and only it receives that
 * signal; [P3] MSA entry: KL loss, teacher stop-gradient).  dtype MSA_BF16, index keys
 * bf16 (index_key_dtype 0 or MSA_BF16); other problems return MSA_ERR_UNSUPPORTED.
 * Gradients are float32 and are OVERWRITTEN (the calls zero them first).
 *
 * Readings of the pages used here:
 *   teacher  mass[s,g,t,i] = the main branch's attention on block sel[s,g,t,i] for row t,
 *            averaged over the G heads of group g (0 for a -1 slot; a row sums to 1);
 *   student  softmax over the row's selected blocks of sigma * scores[s,g,t,b];
 *   loss     KL(teacher / sum(teacher) || student) per row; gradients are those of the SUM
 *            of row losses, the teacher held fixed;
 *   max-pool the gradient of a block score reaches its arg-max key (lowest position among
 *            equal maxima, scores accumulated in float32).
 */

/* a4 + a5 of msa_sparse_attn_prefill with the training outputs (every pair takes the
 * Outer-Gather-Q kernel, whatever MSA_HOT_TILES says):
 *   lse        float32 [S, T, H]: log sum_j exp(scale q.K_j) over the row's attended keys;
 *   block_mass float32 [S, Hkv, T, k]: the teacher above.
 * workspace: msa_workspace_bytes(prob, MSA_CALL_PREFILL) bytes. */
msa_status msa_sparse_attn_prefill_train(const msa_problem* prob, const void* q, const void* k,
                                         const void* v, const int32_t* csr_offsets,
                                         const int32_t* csr_entries, const int32_t* sel, void* out,
                                         float* lse, float* block_mass, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* Gradients of sum(dout * out) for the main branch, out being the prefill output for the
 * same q, k, v and selection (dout, out bf16 [S, T, H, d]; lse from the call above; sel and
 * the csr lists of the forward):
 *   dq float32 [S, T, H, d], dk and dv float32 [S, Hkv, N, d].
 * The KV block is the outer loop.  dq is summed from bf16 per-(row, slot) partials; dk and
 * dv combine work items with float atomics (exact up to the order of float32 additions).
 * workspace: msa_workspace_bytes(prob, MSA_CALL_BACKWARD) bytes (it holds the dq partials:
 * S * T * Hkv * k * G * d bf16 values). */
msa_status msa_sparse_attn_backward(const msa_problem* prob, const void* q, const void* k,
                                    const void* v, const void* out, const void* dout,
                                    const float* lse, const int32_t* sel, const int32_t* csr_offsets,
                                    const int32_t* csr_entries, float* dq, float* dk, float* dv,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* The index-branch KL per row and its gradient with respect to the selected block scores:
 *   scores float32 [S, Hkv, T, nb] (msa_index_scores), sel [S, Hkv, T, k],
 *   block_mass [S, Hkv, T, k] (teacher), sigma > 0 (0 selects 1 / sqrt(index_dim));
 *   loss float32 [S, Hkv, T]; dscores float32 [S, Hkv, T, k] (0 for -1 slots). */
msa_status msa_index_kl(const msa_problem* prob, const float* scores, const int32_t* sel,
                        const float* block_mass, float sigma, float* loss, float* dscores,
                        void* stream);

/* Index-branch input gradients through the causal block max-pool, in Outer-Gather-Q order:
 *   dq_idx float32 [S, Hkv, T, dI], dk_idx float32 [S, Hkv, N, dI];
 *   argmax int32 [S, Hkv, T, k] (optional, may be NULL): the arg-max position of each
 *   selected block; entries of -1 slots are left untouched.
 * workspace: msa_workspace_bytes(prob, MSA_CALL_INDEX_BACKWARD) bytes. */
msa_status msa_index_backward(const msa_problem* prob, const void* q_idx, const void* k_idx,
                              const int32_t* csr_offsets, const int32_t* csr_entries,
                              const float* dscores, float* dq_idx, float* dk_idx, int32_t* argmax,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Token-level selection on the same indexer, the granularity the pages compare MSA with
 * ([P1] 分歧一：颗粒度: DSA keeps 2048 single tokens per query, MSA 16 blocks x 128 -- the
 * same budget; [P3] DSA entry).  Decode shapes: num_q <= 8, dtype MSA_BF16 (index keys
 * bf16 or E4M3); other problems return MSA_ERR_UNSUPPORTED.  budget: 1 .. 8192.
 *
 * msa_token_scores: scores [S, Hkv, T, N] float32, scores[s,g,t,j] = q_idx[s,g,t] . k_idx[s,g,j]
 *   for j <= p_t; entries j > p_t are not written.
 * msa_token_topk: sel_tok [S, Hkv, T, budget] int32: the budget positions j <= p_t with the
 *   largest scores (ties to the lower position; no forced token), in ascending order, -1
 *   padded when fewer are eligible.  Reads only scores[s,g,t,0..p_t].  workspace: at least
 *   msa_token_workspace_bytes(prob, budget) bytes (per-row histograms and candidate lists;
 *   MSA_ERR_WORKSPACE_TOO_SMALL otherwise); the same buffer may then serve
 *   msa_token_attn_decode on the same stream.
 * msa_token_attn_decode: out [S, T, H, d]: for each query head, the exact softmax attention
 *   over the row's selected positions (the block-level definition with block size 1).
 *   workspace: msa_workspace_bytes(prob, MSA_CALL_TOKEN_DECODE) bytes for budget = 2048;
 *   use msa_token_workspace_bytes for another budget.
 */
msa_status msa_token_scores(const msa_problem* prob, const void* q_idx, const void* k_idx, float* scores,
                            void* stream);
msa_status msa_token_topk(const msa_problem* prob, int32_t budget, const float* scores, int32_t* sel_tok,
                          void* workspace, size_t workspace_bytes, void* stream);
msa_status msa_token_attn_decode(const msa_problem* prob, int32_t budget, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* sel_tok, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream);
size_t msa_token_workspace_bytes(const msa_problem* prob, int32_t budget);

/* Device workspace needed by a call (MSA_CALL_*); 0 for an invalid problem or call. */
size_t msa_workspace_bytes(const msa_problem* prob, int which_call);

/* Static description of a status code. */
const char* msa_status_string(msa_status status);

/* Thread-local detail of this thread's last failed call ("" if none). */
const char* msa_last_error_message(void);

/*
 * Opt-in per-kernel timer (measurement aid).  While enabled, every launch of the
 * library's kernels is bracketed by a pair of hipEvents recorded on the launch
 * stream.  msa_profiler_read() waits for the recorded events, returns the summed
 * device time (ms) and launch count of the kernel named `kernel` (NULL or "" =
 * every kernel) since the last reset, and resets=1 clears the records.  Global
 * state: not for concurrent use from several threads.
 */
msa_status msa_profiler_enable(int on);
msa_status msa_profiler_read(const char* kernel, double* total_ms, int64_t* launches, int reset);
/* The individual launch durations (ms) of `kernel` (NULL or "" = every kernel) recorded
 * since the last reset, in no particular order (for percentiles): the first
 * min(capacity, count) are written to ms_out (caller-owned host memory, may be NULL when
 * capacity is 0) and *count receives the number recorded.  Does not reset. */
msa_status msa_profiler_samples(const char* kernel, float* ms_out, int64_t capacity, int64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
