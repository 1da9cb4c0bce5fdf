// C ABI of libmla: argument validation, workspace sizing, kernel dispatch.
// Every check runs on the host before any launch; see include/mla.h.
#include <math.h>
#include <string.h>

#include <atomic>

#include "mla_device.h"
#include "mla_internal.h"

using namespace mla;

namespace {

int elem_bytes(int dtype) { return dtype == MLA_BF16 ? 2 : 4; }

bool fp8_cache(const mla_dims_t* d) { return (d->flags & MLA_FLAG_FP8_CACHE) != 0; }

// bytes of one cached value
int cache_elem_bytes(const mla_dims_t* d) { return fp8_cache(d) ? 1 : elem_bytes(d->dtype); }

int check_dims(const mla_dims_t* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (d->flags & ~(MLA_FLAG_GENERIC | MLA_FLAG_FP8_CACHE)) return MLA_ERR_ARG;
  if (d->hidden < 1 || d->num_heads < 1 || d->d_c < 2 || d->d_r < 2 || d->qk_nope < 1 || d->v_head < 1 ||
      d->page_size < 1)
    return MLA_ERR_DIMS;
  if ((d->d_c & 1) || (d->d_r & 1)) return MLA_ERR_DIMS;
  if (!(d->rope_base > 0.f) || !isfinite(d->rope_base) || !isfinite(d->softmax_scale)) return MLA_ERR_ARG;
  if (fp8_cache(d)) {
    if (d->dtype != MLA_BF16) return MLA_ERR_DTYPE;
    // the float32 scales after the rows of a page stay 4-byte aligned
    if (((long long)d->page_size * (d->d_c + d->d_r)) % 4 != 0) return MLA_ERR_DIMS;
  }
  return MLA_OK;
}

// CU count of the current device, cached per device id.
int current_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return -1;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool bf16_fast(const mla_dims_t* d) { return d->dtype == MLA_BF16 && !(d->flags & MLA_FLAG_GENERIC); }

bool write_fast(const mla_dims_t* d) { return bf16_fast(d) && write_mfma_supported(d->hidden, d->d_c, d->d_r); }

bool absorb_fast(const mla_dims_t* d) {
  return bf16_fast(d) && absorb_mfma_supported(d->num_heads, d->qk_nope, d->d_c, d->d_r);
}

bool prefill_fast(const mla_dims_t* d) {
  return bf16_fast(d) && prefill_mfma_supported(d->qk_nope, d->v_head, d->d_r, d->d_c, d->page_size);
}

bool decode_fast(const mla_dims_t* d, int batch) {
  return d->dtype == MLA_BF16 && !(d->flags & MLA_FLAG_GENERIC) &&
         decode_mfma_supported(d->num_heads, d->d_c, d->d_r, d->v_head, d->page_size, batch);
}

struct DecodeLayout {
  int slots, max_items;
  size_t acc_bytes, ml_bytes, plan_bytes;
  size_t total() const { return acc_bytes + ml_bytes + plan_bytes; }
};

// Returns false when the device cannot be queried.  Items per call are at
// most max(4 * slots, total / kMaxChunk) + batch (see make_decode_plan).
bool decode_layout(const mla_dims_t* d, int batch, int max_seq_len, DecodeLayout& L) {
  const int cus = current_cus();
  if (cus <= 0) return false;
  L.slots = decode_fast(d, batch) ? decode_mfma_slots(d->num_heads, cus, fp8_cache(d)) : cus;
  const long long by_len = ((long long)batch * max_seq_len + kMaxChunk - 1) / kMaxChunk;
  const long long base = (long long)kMaxChunksPerSlot * L.slots;
  L.max_items = (int)((by_len > base ? by_len : base) + batch);
  L.acc_bytes = (size_t)L.max_items * d->num_heads * d->d_c * sizeof(float);
  L.acc_bytes = (L.acc_bytes + 255) & ~(size_t)255;
  L.ml_bytes = (size_t)L.max_items * d->num_heads * 2 * sizeof(float);
  L.ml_bytes = (L.ml_bytes + 255) & ~(size_t)255;
  L.plan_bytes = (size_t)(2 * batch + 2) * sizeof(int);
  return true;
}

size_t prefill_ws_bytes(const mla_dims_t* d, int total) {
  size_t k = (size_t)total * d->num_heads * d->qk_nope * sizeof(float);
  k = (k + 255) & ~(size_t)255;
  return k + (size_t)total * d->num_heads * d->v_head * sizeof(float);
}

int launched(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_DIMS: return "MLA_ERR_DIMS: unsupported or inconsistent dimensions";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unknown dtype";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small";
    case MLA_ERR_CAPACITY: return "MLA_ERR_CAPACITY: sequence length exceeds block-table capacity";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP launch or device query failed";
    case MLA_ERR_ARG: return "MLA_ERR_ARG: invalid argument";
    default: return "unknown mla status";
  }
}

size_t mla_cache_bytes(const mla_dims_t* dims, int64_t tokens, int32_t layers) {
  if (check_dims(dims) != MLA_OK || tokens < 0 || layers < 0) return 0;
  return (size_t)layers * (size_t)tokens * (size_t)(dims->d_c + dims->d_r) * (size_t)cache_elem_bytes(dims);
}

size_t mla_page_bytes(const mla_dims_t* dims) {
  if (check_dims(dims) != MLA_OK) return 0;
  const size_t R = (size_t)(dims->d_c + dims->d_r);
  return (size_t)dims->page_size * (fp8_cache(dims) ? R + 4 : R * (size_t)elem_bytes(dims->dtype));
}

size_t mla_write_cache_workspace_size(const mla_dims_t* dims, int32_t n_tokens) {
  if (check_dims(dims) != MLA_OK || n_tokens < 0) return 0;
  return fp8_cache(dims) ? (size_t)n_tokens * (size_t)(dims->d_c + dims->d_r) * 2 : 0;
}

int mla_uses_fast_path(const mla_dims_t* dims, int32_t op) {
  const int st = check_dims(dims);
  if (st != MLA_OK) return st;
  switch (op) {
    case 0: return write_fast(dims) ? 1 : 0;
    case 1: return absorb_fast(dims) ? 1 : 0;
    case 2: return decode_fast(dims, 1) ? 1 : 0;
    case 3: return (prefill_fast(dims) && !fp8_cache(dims)) ? 1 : 0;
    default: return MLA_ERR_ARG;
  }
}

int mla_write_cache_ws(const mla_dims_t* dims, const void* h, const void* w_dkr, const int32_t* positions,
                       const int64_t* slot_mapping, int32_t n_tokens, void* pool, int32_t num_pages, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0 || num_pages < 0) return MLA_ERR_ARG;
  if (n_tokens == 0) return MLA_OK;
  if (!h || !w_dkr || !positions || !slot_mapping || !pool) return MLA_ERR_NULL;
  const size_t need = mla_write_cache_workspace_size(dims, n_tokens);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  const bool f8 = fp8_cache(dims);
  // 8-bit cache: the bf16 rows go to the workspace (row n at row n), then
  // each is quantized into its slot
  WriteCacheArgs a{h, w_dkr, positions, slot_mapping, f8 ? workspace : pool, n_tokens, dims->hidden, dims->d_c,
                   dims->d_r, dims->page_size, dims->rope_base, f8 ? 1 : 0};
  hipError_t e = write_fast(dims) ? write_cache_mfma(a, stream)
                                  : write_cache_generic(a, dims->dtype == MLA_BF16, stream);
  if (e != hipSuccess || !f8) return launched(e);
  return launched(quantize_rows_fp8((const uint16_t*)workspace, slot_mapping, pool, n_tokens, dims->d_c + dims->d_r,
                                    dims->page_size, stream));
}

int mla_write_cache(const mla_dims_t* dims, const void* h, const void* w_dkr, const int32_t* positions,
                    const int64_t* slot_mapping, int32_t n_tokens, void* pool, int32_t num_pages,
                    hipStream_t stream) {
  return mla_write_cache_ws(dims, h, w_dkr, positions, slot_mapping, n_tokens, pool, num_pages, nullptr, 0, stream);
}

int mla_absorb_q(const mla_dims_t* dims, const void* q, const void* w_uk, const int32_t* positions,
                 int32_t n_tokens, void* q_abs, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0) return MLA_ERR_ARG;
  if (n_tokens == 0) return MLA_OK;
  if (!q || !w_uk || !positions || !q_abs) return MLA_ERR_NULL;
  AbsorbArgs a{q, w_uk, positions, q_abs, n_tokens, dims->num_heads, dims->qk_nope, dims->d_c, dims->d_r,
               dims->rope_base};
  if (absorb_fast(dims)) return launched(absorb_mfma(a, stream));
  return launched(absorb_generic(a, dims->dtype == MLA_BF16, stream));
}

size_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t max_seq_len) {
  if (check_dims(dims) != MLA_OK || batch < 0 || batch > kMaxDecodeBatch || max_seq_len < 0) return 0;
  DecodeLayout L;
  if (!decode_layout(dims, batch, max_seq_len, L)) return 0;
  return L.total();
}

int mla_decode(const mla_dims_t* dims, const void* q_abs, const void* pool, int32_t num_pages,
               const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
               int32_t max_seq_len, const void* w_uv, void* out, float* lse, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || max_seq_len < 0 || num_pages < 0 || max_pages_per_seq < 0) return MLA_ERR_ARG;
  if (batch > kMaxDecodeBatch) return MLA_ERR_DIMS;
  if (batch == 0) return MLA_OK;
  if (!q_abs || !pool || !block_table || !seq_lens || !w_uv || !out || !workspace) return MLA_ERR_NULL;
  if ((int64_t)max_seq_len > (int64_t)max_pages_per_seq * dims->page_size) return MLA_ERR_CAPACITY;
  DecodeLayout L;
  if (!decode_layout(dims, batch, max_seq_len, L)) return MLA_ERR_HIP;
  if (workspace_bytes < L.total()) return MLA_ERR_WORKSPACE;
  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.q_abs = q_abs;
  a.pool = pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.w_uv = w_uv;
  a.out = out;
  a.lse = lse;
  a.part_acc = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + L.acc_bytes);
  a.plan = (int*)((char*)workspace + L.acc_bytes + L.ml_bytes);
  a.batch = batch;
  a.H = dims->num_heads;
  a.d_c = dims->d_c;
  a.d_r = dims->d_r;
  a.d_v = dims->v_head;
  a.P = dims->page_size;
  a.max_pages_per_seq = max_pages_per_seq;
  a.len_cap = max_seq_len;
  a.slots = L.slots;
  a.max_items = L.max_items;
  a.min_chunk = 256;
  // partial (m, l, acc) written and read back, in cache-row equivalents
  a.ovh_tokens = (int)((2.0 * dims->num_heads * (dims->d_c + 2) * 4.0) /
                       ((double)(dims->d_c + dims->d_r) * cache_elem_bytes(dims)));
  a.scale_log2 = dims->softmax_scale * kLog2e;
  a.fp8 = fp8_cache(dims) ? 1 : 0;
  // the MFMA path addresses partials with 32-bit offsets
  if (decode_fast(dims, batch) && L.acc_bytes < ((size_t)1 << 32)) return launched(decode_mfma(a, stream));
  return launched(decode_generic(a, dims->dtype == MLA_BF16, stream));
}

size_t mla_prefill_workspace_size(const mla_dims_t* dims, int32_t total_tokens) {
  if (check_dims(dims) != MLA_OK || fp8_cache(dims) || total_tokens < 0) return 0;
  return prefill_ws_bytes(dims, total_tokens);
}

int mla_prefill_kv(const mla_dims_t* dims, const void* q, const void* pool, int32_t num_pages,
                   const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* cu_seqlens_q,
                   const int32_t* cu_seqlens_kv, int32_t num_seqs, int32_t total_q, int32_t total_kv,
                   int32_t max_q_len, int32_t max_kv_len, const void* w_uk, const void* w_uv, void* out,
                   float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (fp8_cache(dims)) return MLA_ERR_DTYPE;  // prefill reads bf16 / fp32 pools only
  if (num_seqs < 0 || total_q < 0 || total_kv < 0 || max_q_len < 0 || max_kv_len < 0 || num_pages < 0 ||
      max_pages_per_seq < 0)
    return MLA_ERR_ARG;
  if (total_kv < total_q || max_kv_len < max_q_len) return MLA_ERR_ARG;
  if (dims->v_head > 256) return MLA_ERR_DIMS;
  if (num_seqs == 0 || total_q == 0) return MLA_OK;
  if (!q || !pool || !block_table || !cu_seqlens_q || !cu_seqlens_kv || !w_uk || !w_uv || !out || !workspace)
    return MLA_ERR_NULL;
  if ((int64_t)max_kv_len > (int64_t)max_pages_per_seq * dims->page_size) return MLA_ERR_CAPACITY;
  if (workspace_bytes < prefill_ws_bytes(dims, total_kv)) return MLA_ERR_WORKSPACE;
  size_t kb = (size_t)total_kv * dims->num_heads * dims->qk_nope * sizeof(float);
  kb = (kb + 255) & ~(size_t)255;
  PrefillArgs a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.pool = pool;
  a.block_table = block_table;
  a.cu_q = cu_seqlens_q;
  a.cu_kv = cu_seqlens_kv;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.out = out;
  a.lse = lse;
  a.ws_k = workspace;
  a.ws_v = (char*)workspace + kb;
  a.num_seqs = num_seqs;
  a.total = total_q;
  a.total_kv = total_kv;
  a.max_seq_len = max_q_len;
  a.H = dims->num_heads;
  a.d_n = dims->qk_nope;
  a.d_r = dims->d_r;
  a.d_c = dims->d_c;
  a.d_v = dims->v_head;
  a.P = dims->page_size;
  a.max_pages_per_seq = max_pages_per_seq;
  a.rope_base = dims->rope_base;
  a.scale = dims->softmax_scale;
  if (prefill_fast(dims)) return launched(prefill_mfma(a, stream));
  return launched(prefill_generic(a, dims->dtype == MLA_BF16, stream));
}

int mla_prefill(const mla_dims_t* dims, const void* q, const void* pool, int32_t num_pages,
                const int32_t* block_table, int32_t max_pages_per_seq, const int32_t* cu_seqlens,
                int32_t num_seqs, int32_t total_tokens, int32_t max_seq_len, const void* w_uk, const void* w_uv,
                void* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // fresh sequences: the keys are exactly the new tokens
  return mla_prefill_kv(dims, q, pool, num_pages, block_table, max_pages_per_seq, cu_seqlens, cu_seqlens, num_seqs,
                        total_tokens, total_tokens, max_seq_len, max_seq_len, w_uk, w_uv, out, lse, workspace,
                        workspace_bytes, stream);
}

}  // extern "C"
