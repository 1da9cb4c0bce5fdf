/*
 * mla.h -- C ABI of libmla.so: Multi-head Latent Attention over a paged
 * latent cache, hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * The method (sources are the pages this library is built from):
 *   - Per token, the hidden state h is projected to a small latent
 *     c_KV = W_DKV h and a separate rotary key k_R = RoPE(W_KR h, p); only the
 *     row [c_KV | k_R] is cached, one per token per layer, shared by every head
 *     (yapayzekasozluk.tr "Multi-head Latent Attention (MLA) Nedir?", section
 *     "MLA nasil calisir?"; LLMScale "GQA, MQA ve MLA", section "Multi-head
 *     latent attention (MLA)").
 *   - The step order is: project to the latent, write the cache in the
 *     engine's layout, read it with merged matrices or an equivalent kernel
 *     (openarchlab "MLA - latent KV, decoupled RoPE va matrix absorption",
 *     section 2).
 *   - Reading uses matrix absorption: W_UK is folded into the query and W_UV
 *     is applied after the softmax-weighted latent sum, changing the order of
 *     computation but not the function (same page, sections 1 and 6).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises.  Work is enqueued on `stream`
 *     and the call returns at once.  Scalar/struct pointers (dims, out
 *     parameters of the size helpers) are HOST pointers.
 *   - All tensors are dense row-major with the shapes written below.
 *     `dtype` selects fp32 or bf16 storage for every floating tensor except
 *     `lse` (always fp32) and workspaces (library-defined).  Arithmetic is
 *     fp32 (bf16 operands, fp32 accumulation) in either case.
 *   - Argument errors are detected on the host before anything is launched
 *     and return a negative mla_status; nothing is written.  A failed kernel
 *     launch returns MLA_ERR_HIP.
 *   - Device-side values (block-table entries, slots, sequence lengths and
 *     offsets) are read by the kernels.  Lengths are always clamped on the
 *     device to the host-side bounds the call passes (max_seq_len,
 *     max_q_len, max_kv_len, totals), which the host checks against the
 *     block-table capacity, so a length never takes a read past a
 *     sequence's block-table row.  Block-table entries must lie in
 *     [0, num_pages) and slots in [-1, num_pages * P): a release build does
 *     not check them.  A library built with MLA_DEBUG (libmla_debug.so,
 *     same ABI) compares every entry and slot with num_pages before it forms
 *     an address: an entry out of range sets a bit of the device error word
 *     (MLA_DEVERR_*, read with mla_get_device_error) and is replaced by
 *     page 0 (a slot is skipped), so no access leaves the pool; a clamped
 *     length sets MLA_DEVERR_LENGTH.
 *   - Calls on one stream are ordered; calls that share an output or a
 *     workspace on different streams race.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,      /* a required pointer is NULL                        */
  MLA_ERR_DIMS = -2,      /* unsupported or inconsistent dimensions            */
  MLA_ERR_DTYPE = -3,     /* unknown dtype code                                */
  MLA_ERR_WORKSPACE = -4, /* workspace smaller than the *_workspace_size value */
  MLA_ERR_CAPACITY = -5,  /* max_seq_len exceeds max_pages_per_seq * page_size */
  MLA_ERR_HIP = -6,       /* a HIP launch or device query failed               */
  MLA_ERR_ARG = -7        /* other invalid argument (negative count, bad flag,
                             softmax_scale <= 0, an empty pool for work)       */
} mla_status;

/* Bits of the device error word (set only by MLA_DEBUG builds). */
enum {
  MLA_DEVERR_PAGE = 1,   /* a block-table entry outside [0, num_pages)          */
  MLA_DEVERR_SLOT = 2,   /* a slot_mapping entry outside [-1, num_pages * P)    */
  MLA_DEVERR_LENGTH = 4  /* a device length or offset beyond its host bound    */
};

enum { MLA_F32 = 0, MLA_BF16 = 1 };

/* flags (bitwise or):
 *   MLA_FLAG_GENERIC forces the plain (VALU, any-shape) kernels even where
 *   the MFMA kernels apply; used to cross-check the two on one input.
 *   MLA_FLAG_FP8_CACHE selects the 8-bit cache (yapayzekasozluk.tr, section
 *   "MLA ve diger optimizasyonlarla iliskisi": the cached vector may be stored
 *   with 8 bits per value; openarchlab section 3 names the quantization
 *   scales that the ideal-size formula leaves out).  Requires dtype MLA_BF16
 *   (h, weights, queries and outputs stay bf16).  A page then holds, for its
 *   P tokens, first the P rows of d_c + d_r E4M3 codes (1 sign, 4 exponent
 *   bits with bias 7, 3 mantissa bits; 448 is the largest value), then P
 *   float32 row scales: page bytes = P * (d_c + d_r + 4), see
 *   mla_page_bytes.  A row stores value x as the E4M3 code nearest to
 *   x / 2^e (ties to even, -0 stored as +0), where 2^e is the row's scale:
 *   the smallest power of two, at least 2^-126, with max |x| <= 448 * 2^e,
 *   taken over the row after rounding it to bf16.  The stored value is
 *   E4M3(code) * 2^e.  mla_write_cache_ws writes such rows, mla_decode reads
 *   them; prefill does not read an 8-bit pool (MLA_ERR_DTYPE).  Rows whose
 *   largest magnitude is at or above 2^126 or below 2^-117 lose range. */
enum { MLA_FLAG_GENERIC = 1, MLA_FLAG_FP8_CACHE = 2 };

typedef struct {
  int32_t hidden;      /* D: width of h                                         */
  int32_t num_heads;   /* H: query heads                                        */
  int32_t d_c;         /* latent width (kv_lora_rank), even                     */
  int32_t d_r;         /* rotary key width (qk_rope_head_dim), even             */
  int32_t qk_nope;     /* d_n: per-head non-rotary query/key width              */
  int32_t v_head;      /* d_v: per-head value width                             */
  int32_t page_size;   /* P: tokens per cache page                              */
  int32_t dtype;       /* MLA_F32 or MLA_BF16                                   */
  float rope_base;     /* RoPE base (10000 in the pages' models), > 0           */
  float softmax_scale; /* sigma > 0, multiplies every score                     */
  int32_t flags;       /* 0 or MLA_FLAG_* bits                                  */
} mla_dims_t;

/*
 * Step 1 + 2: project and write the cache (openarchlab section 2, steps 1-2;
 * compression and decoupled RoPE as in yapayzekasozluk.tr "MLA nasil calisir?").
 *
 * For n < n_tokens with slot_mapping[n] >= 0:
 *   row = [ W_DKV h_n  |  RoPE(W_KR h_n, positions[n]) ]      (fp32, then dtype, RNE)
 *   pool[slot / P][slot % P][0 : d_c + d_r] = row
 * RoPE rotates adjacent pairs (2i, 2i+1) by positions[n] * rope_base^(-2i/d_r).
 *
 *   h            [n_tokens, D]                 dtype
 *   w_dkr        [d_c + d_r, D]                dtype  rows 0..d_c-1 = W_DKV, rest = W_KR
 *   positions    [n_tokens]                    int32
 *   slot_mapping [n_tokens]                    int64  page * P + offset, -1 = skip
 *   pool         [num_pages, P, d_c + d_r]     dtype  updated in place
 * Slots must be distinct and < num_pages * P (checked on the device only by
 * MLA_DEBUG builds).  n_tokens == 0 is a no-op; otherwise num_pages >= 1.
 */
int mla_write_cache(const mla_dims_t* dims, const void* h, const void* w_dkr,
                    const int32_t* positions, const int64_t* slot_mapping, int32_t n_tokens,
                    void* pool, int32_t num_pages, hipStream_t stream);

/* Bytes of workspace mla_write_cache_ws needs for n_tokens rows: 0 for bf16
 * and fp32 caches, n_tokens * (d_c + d_r) * 2 for the 8-bit cache. */
size_t mla_write_cache_workspace_size(const mla_dims_t* dims, int32_t n_tokens);

/*
 * mla_write_cache with a workspace, for every cache format.  With
 * MLA_FLAG_FP8_CACHE the rows are computed as in mla_write_cache (bf16,
 * round to nearest even) into the workspace, then each row with
 * slot_mapping[n] >= 0 is quantized (see MLA_FLAG_FP8_CACHE) and its codes
 * and scale are stored at its slot of the 8-bit pool.  mla_write_cache is
 * this call with no workspace, so it returns MLA_ERR_WORKSPACE for an 8-bit
 * cache.
 *   workspace  >= mla_write_cache_workspace_size(dims, n_tokens) bytes
 *              (may be NULL when that size is 0)
 */
int mla_write_cache_ws(const mla_dims_t* dims, const void* h, const void* w_dkr,
                       const int32_t* positions, const int64_t* slot_mapping, int32_t n_tokens,
                       void* pool, int32_t num_pages, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Bytes of one cache page: P * (d_c + d_r) * element bytes, or
 * P * (d_c + d_r + 4) for the 8-bit cache (0 for invalid dims). */
size_t mla_page_bytes(const mla_dims_t* dims);

/*
 * Query absorption (openarchlab sections 1 and 6: W_UK folded into the query).
 *   q_abs[n][h][0 : d_c]       = W_UK,h^T q[n][h][0 : d_n]
 *   q_abs[n][h][d_c : d_c+d_r] = RoPE(q[n][h][d_n : d_n + d_r], positions[n])
 *
 *   q      [n_tokens, H, d_n + d_r]  dtype  pre-RoPE query, per head [q_C | q_R]
 *   w_uk   [H, d_n, d_c]             dtype  K_C,h = W_UK,h c
 *   q_abs  [n_tokens, H, d_c + d_r]  dtype  output
 */
int mla_absorb_q(const mla_dims_t* dims, const void* q, const void* w_uk,
                 const int32_t* positions, int32_t n_tokens, void* q_abs, hipStream_t stream);

/* Bytes of workspace mla_write_absorb needs for n_write rows (0 on invalid
 * arguments): 256 bytes of counters, then the split-K partials of the fused
 * launch (2 MiB at D = 7168, d_c + d_r = 576) or, for an 8-bit cache, the
 * bf16 staging of the rows. */
size_t mla_write_absorb_workspace_size(const mla_dims_t* dims, int32_t n_write);

/*
 * The decode step's cache write and query absorption in one call
 * (openarchlab section 2 steps 1-2).  The result is that of
 * mla_write_cache_ws(dims, h, w_dkr, positions, slot_mapping, n_write, pool,
 * num_pages) followed by mla_absorb_q(dims, q, w_uk, q_positions, n_q,
 * q_abs), with the same arguments, layouts and errors (the two are
 * independent: the absorption does not read the pool).
 *
 * With bf16 operands on the MFMA paths, n_write and n_q in [1, 64], d_n = 128,
 * d_c = 512, D a multiple of 64 up to 8192 and d_c + d_r a multiple of 64,
 * both run in one launch, so the absorption uses the CUs the cache write
 * leaves idle; otherwise the two calls run in sequence.  In the one launch
 * the rows are written by a split-K product: each row is the same fp32 sum
 * as mla_write_cache's, added in another order, then rounded once to bf16
 * (so a value can differ from mla_write_cache's by one bf16 unit in the
 * last place); the order is fixed, so the call is deterministic.  q_abs is
 * bit-identical to mla_absorb_q's.
 *
 *   workspace  >= mla_write_absorb_workspace_size(dims, n_write) bytes, of
 *              device memory that only this call uses.  Its first 256
 *              bytes must be zero before the first call (a zero-filled
 *              allocation); every call leaves them zero.  Calls that share
 *              a workspace must not overlap (one stream, or ordered).
 *              NULL is accepted when the size is 0.
 */
int mla_write_absorb(const mla_dims_t* dims, const void* h, const void* w_dkr, const int32_t* positions,
                     const int64_t* slot_mapping, int32_t n_write, void* pool, int32_t num_pages, const void* q,
                     const void* w_uk, const int32_t* q_positions, int32_t n_q, void* q_abs, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace mla_decode needs for `batch` sequences of at most
 * max_seq_len tokens (0 on invalid arguments or when no device is present). */
size_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t max_seq_len);

/*
 * Step 3, decode (openarchlab section 2 step 3; absorption, sections 1 and 6).
 * Sequence b has seq_lens[b] cached rows; token t lives at
 * pool[block_table[b][t / P]][t % P].  Its query q_abs[b] attends to all of
 * them (it sits at position seq_lens[b]-1, its own row already written):
 *   s_h,t  = softmax_scale * q_abs[b][h] . row_t              (all d_c + d_r)
 *   lat_h  = sum_t softmax_t(s_h) row_t[0 : d_c]
 *   out[b][h] = W_UV,h lat_h,   lse[b][h] = ln sum_t exp(s_h,t)
 * Empty sequences give out = 0, lse = -inf.
 *
 *   q_abs       [batch, H, d_c + d_r]           dtype
 *   pool        [num_pages, P, d_c + d_r]       dtype, or num_pages 8-bit
 *                                               pages (MLA_FLAG_FP8_CACHE);
 *                                               row_t is then the stored
 *                                               value E4M3(code) * scale
 *   block_table [batch, max_pages_per_seq]      int32
 *   seq_lens    [batch]                         int32 (device); lengths are
 *                                                clamped to [0, max_seq_len]
 *   w_uv        [H, d_v, d_c]                   dtype
 *   out         [batch, H, d_v]                 dtype
 *   lse         [batch, H]                      fp32, may be NULL
 *   workspace   >= mla_decode_workspace_size(dims, batch, max_seq_len) bytes
 * max_seq_len is a host-side bound on seq_lens: it must not exceed
 * max_pages_per_seq * P (MLA_ERR_CAPACITY) and it sizes the workspace.
 * Results do not depend on the page permutation (token-space split
 * boundaries, fixed merge order): two calls on permuted pools give identical
 * bits.  num_pages >= 1.
 * Range: the fast path accumulates unnormalised softmax numerators below
 * 2^100 (larger ones are detected and the affected partial is recomputed
 * exactly), so cached values must stay below 2^28 in magnitude for the fp32
 * latent sums to stay finite.
 * Precision: on the fast path each split's latent sums (fp32 inside the
 * split) are stored as bf16 (round to nearest even) between the two passes;
 * the merge itself, the (max, sum) pairs and the W_UV product stay fp32.
 */
int mla_decode(const mla_dims_t* dims, const void* q_abs, const void* pool, int32_t num_pages,
               const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
               int32_t batch, int32_t max_seq_len, const void* w_uv, void* out, float* lse,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments, results and errors as mla_decode, without the
 * workspace.  The split pass keeps its partial results in a device array
 * inside the library, MLA_NOALLOC_SCRATCH_BYTES per device, which each device
 * holds from the library's load until the process ends.  The call allocates
 * nothing and calls no allocating routine.
 * Size limit: the plan needs up to max(S, ceil(batch * max_seq_len / 8192)) +
 * batch work items of num_heads * (d_c + 2) * 4 bytes each, where S is the
 * number of split work-groups the device holds at once (its CU count, or
 * twice that for a bf16 cache with num_heads <= 32); a call whose items do
 * not fit returns MLA_ERR_WORKSPACE and launches nothing.  At num_heads 128,
 * d_c 512 on a 256-CU MI355X that is about 510 items, for example 64
 * sequences of up to 57k tokens or 192 of up to 8k.
 * Every call on one device shares its array and leaves its last contents
 * there: calls on one device that overlap (other streams, other threads)
 * race.  Nothing in the array needs clearing between calls.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (128u << 20)
int mla_decode_noalloc(const mla_dims_t* dims, const void* q_abs, const void* pool, int32_t num_pages,
                       const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                       int32_t batch, int32_t max_seq_len, const void* w_uv, void* out, float* lse,
                       hipStream_t stream);

/* Bytes of workspace mla_prefill needs for `total_tokens` query tokens, and
 * mla_prefill_kv for `total_tokens` key tokens (pass its total_kv): the
 * up-projected K_C and V of every key token, H * (d_n + d_v) values per token
 * (plus at most 255 bytes of alignment), stored as bf16 on the MFMA path
 * (mla_uses_fast_path(dims, 3) == 1) and as fp32 otherwise. */
size_t mla_prefill_workspace_size(const mla_dims_t* dims, int32_t total_tokens);

/*
 * Causal prefill of fresh sequences (openarchlab section 4 asks for prefill
 * and decode to be measured on the target kernel; decompression of K and V
 * from c_KV, yapayzekasozluk.tr "MLA nasil calisir?").  Sequence i holds
 * tokens cu_seqlens[i] .. cu_seqlens[i+1]-1 of q/out, at positions
 * 0 .. len-1, and its rows are already in the pool.  For each head h:
 *   K_h,t = [W_UK,h c_t | k_R,t],  V_h,t = W_UV,h c_t,
 *   Q_h,i = [q_C | RoPE(q_R, i)],  out[i][h] = softmax_{t<=i}(sigma Q.K) V,
 *   lse[i][h] = ln sum_{t<=i} exp(sigma Q.K).
 *
 *   q           [total_tokens, H, d_n + d_r]   dtype  pre-RoPE
 *   cu_seqlens  [num_seqs + 1]                  int32 (device), cu[0] = 0,
 *                                               cu[num_seqs] = total_tokens
 *   out         [total_tokens, H, d_v]          dtype
 *   lse         [total_tokens, H]               fp32, may be NULL
 * max_seq_len bounds every sequence length (capacity check and tiling).
 * Device offsets are clamped as in mla_prefill_kv; num_pages >= 1.
 */
int mla_prefill(const mla_dims_t* dims, const void* q, const void* pool, int32_t num_pages,
                const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* cu_seqlens,
                int32_t num_seqs, int32_t total_tokens, int32_t max_seq_len, const void* w_uk,
                const void* w_uv, void* out, float* lse, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * Prefill of new tokens onto sequences that may already hold a cached prefix
 * (chunked prefill).  openarchlab section 4 asks for prefill to be measured
 * under real serving shapes; the pages do not spell out chunking, and the
 * reading taken is causal attention by position: sequence i has
 * kv_len = cu_seqlens_kv[i+1] - cu_seqlens_kv[i] cached tokens in the pool
 * (positions 0 .. kv_len-1, the new tokens' rows already written), of which
 * the last q_len = cu_seqlens_q[i+1] - cu_seqlens_q[i] are the new tokens,
 * rows cu_seqlens_q[i] .. of q/out.  New token j sits at position
 * prefix + j, prefix = kv_len - q_len, and attends to cache positions
 * 0 .. prefix + j, with the same K, V, score and LSE as mla_prefill.
 *
 *   cu_seqlens_q   [num_seqs + 1]  int32 (device), cu_q[num_seqs] = total_q
 *   cu_seqlens_kv  [num_seqs + 1]  int32 (device), cu_kv[num_seqs] = total_kv,
 *                                  kv_len >= q_len for every sequence
 *   max_q_len, max_kv_len          bounds of q_len and kv_len (tiling and the
 *                                  capacity check against max_pages_per_seq)
 *   workspace                      mla_prefill_workspace_size(dims, total_kv)
 * Other arguments, layouts and errors as mla_prefill; MLA_ERR_ARG also when
 * total_kv < total_q or max_kv_len < max_q_len.  mla_prefill is this call
 * with cu_seqlens_kv = cu_seqlens_q (no prefix).
 * The kernels clamp the device offsets of sequence i before use:
 *   q0 = clamp(cu_q[i], 0, total_q),   q_len  = clamp(cu_q[i+1] - q0, 0, min(max_q_len, total_q - q0)),
 *   k0 = clamp(cu_kv[i], 0, total_kv), kv_len = clamp(cu_kv[i+1] - k0, 0, min(max_kv_len, total_kv - k0)),
 *   q_len = min(q_len, kv_len),
 * so inconsistent offsets give wrong rows but no access outside the
 * caller's buffers (MLA_DEVERR_LENGTH in MLA_DEBUG builds); query rows that
 * no clamped sequence covers are left unwritten.
 */
int mla_prefill_kv(const mla_dims_t* dims, const void* q, const void* pool, int32_t num_pages,
                   const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* cu_seqlens_q,
                   const int32_t* cu_seqlens_kv, int32_t num_seqs, int32_t total_q, int32_t total_kv,
                   int32_t max_q_len, int32_t max_kv_len, const void* w_uk, const void* w_uv, void* out,
                   float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Query low-rank compression and the output projection (yapayzekasozluk.tr
 * "MLA nasil calisir?", last paragraph: the queries get the same kind of
 * compression as K and V; openarchlab section 1: the decompression matrices
 * are folded into the query and the output matrices).
 *
 * mla_project_q: from the hidden states to the absorbed queries that
 * mla_decode reads, for n_tokens tokens:
 *   c_Q[n]       = W_DQ h[n]                                  (d_cq wide)
 *   q[n][h]      = W_UQ,h c_Q[n] = [q_C | q_R]                (d_n + d_r)
 *   q_abs[n][h]  = [W_UK,h^T q_C | RoPE(q_R, positions[n])]   (as mla_absorb_q)
 * c_Q and q are rounded to dtype (bf16: nearest even) in the workspace before
 * the next product.  The products run in this order (W_UK applied to q_C,
 * not folded into W_UQ beforehand): the same function as the folded matrix
 * W_UK,h^T W_UQ,h, with 192 d_cq + 64 K weights per head instead of
 * 576 d_cq at the DeepSeek-V3 shapes.
 *   h       [n_tokens, D]                 dtype
 *   w_dq    [d_cq, D]                     dtype
 *   w_uq    [H, d_n + d_r, d_cq]          dtype
 *   w_uk    [H, d_n, d_c]                 dtype
 *   q_abs   [n_tokens, H, d_c + d_r]      dtype  output
 *   workspace >= mla_project_q_workspace_size(dims, d_cq, n_tokens) bytes
 * d_cq >= 1.  n_tokens == 0 is a no-op.
 *
 * mla_project_out: the attention output through W_O, y[n] = W_O [o[n][0] |
 * ... | o[n][H-1]], head h at columns h d_v .. h d_v + d_v - 1 of W_O.  With
 * mla_decode's W_UV this is y = sum_h (W_O,h W_UV,h) lat_h, the folded output
 * matrix applied in two steps (d_v (D + d_c) weights per head instead of
 * D d_c).
 *   o       [n_tokens, H, d_v]            dtype  (mla_decode's out)
 *   w_o     [D, H d_v]                    dtype
 *   y       [n_tokens, D]                 dtype  output
 *   workspace >= mla_project_out_workspace_size(dims, n_tokens) bytes (may
 *             be 0: then NULL is accepted)
 */
size_t mla_project_q_workspace_size(const mla_dims_t* dims, int32_t d_cq, int32_t n_tokens);
int mla_project_q(const mla_dims_t* dims, int32_t d_cq, const void* h, const void* w_dq, const void* w_uq,
                  const void* w_uk, const int32_t* positions, int32_t n_tokens, void* q_abs, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);
size_t mla_project_out_workspace_size(const mla_dims_t* dims, int32_t n_tokens);
int mla_project_out(const mla_dims_t* dims, const void* o, const void* w_o, int32_t n_tokens, void* y,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Ideal cache bytes of `tokens` tokens over `layers` layers:
 * layers x tokens x (d_c + d_r) x element bytes (openarchlab section 3;
 * LLMScale "Multi-head latent attention (MLA)": the head count drops out).
 * The 8-bit cache counts one byte per value; like the pages' formula, the
 * figure leaves out the scales.  Returns 0 for invalid dims.
 */
size_t mla_cache_bytes(const mla_dims_t* dims, int64_t tokens, int32_t layers);

/* Static string naming a status code. */
const char* mla_status_string(int status);

/*
 * Which kernels a call with these dims would use: 1 = MFMA fast path,
 * 0 = generic path, negative = invalid dims.  `op` is 0 write_cache,
 * 1 absorb_q, 2 decode, 3 prefill.  The answer depends on the dims alone:
 * no batch size or length moves a call off the path reported here.
 */
int mla_uses_fast_path(const mla_dims_t* dims, int32_t op);

/*
 * The device error word of the current device: waits for `stream`, stores
 * the word (MLA_DEVERR_* bits, 0 if nothing was found) in *error_bits and
 * clears it.  The word is shared by every call on the device since the last
 * read, whatever its stream.  Only a library built with MLA_DEBUG ever sets
 * a bit (see the conventions above); mla_debug_build tells which build this
 * is.  Returns MLA_ERR_NULL for a NULL error_bits, MLA_ERR_HIP if the wait
 * or the copy fails.
 */
int mla_get_device_error(int32_t* error_bits, hipStream_t stream);

/* 1 for a library built with MLA_DEBUG (device-side index checks), else 0. */
int mla_debug_build(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
