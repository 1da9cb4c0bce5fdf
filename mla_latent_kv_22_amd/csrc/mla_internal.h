// Internal interface between the C ABI (mla_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

// Largest batch the decode kernels plan for (two int arrays of this size sit in LDS).
constexpr int kMaxDecodeBatch = 4096;
// Decode split: k in {1,2,4} chunks per slot, so items <= 4 * slots + batch.
constexpr int kMaxChunksPerSlot = 4;
// Longest token range of one decode work item, and the pages it can touch.
constexpr int kMaxChunk = 8192;
constexpr int kMaxItemPages = kMaxChunk / 32 + 2;

struct WriteCacheArgs {
  const void* h;
  const void* w_dkr;
  const int32_t* positions;
  const int64_t* slots;
  void* pool;
  int n_tokens, D, d_c, d_r, P;
  float rope_base;
  int dense;  // 1: row n goes to row n of `pool` (a [n_tokens][R] staging buffer), slots unused
  int num_pages;
  int* err;   // device error word (set by MLA_DEBUG builds only)
};

struct AbsorbArgs {
  const void* q;
  const void* w_uk;
  const int32_t* positions;
  void* q_abs;
  int n_tokens, H, d_n, d_c, d_r;
  float rope_base;
};

struct DecodeArgs {
  const void* q_abs;
  const void* pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* w_uv;
  void* out;
  float* lse;
  float* part_acc;  // [max_items, H, d_c] fp32 (plain kernels)
  uint16_t* part_lat;  // [max_items, H, d_c] bf16, the same buffer (MFMA kernels)
  float* part_ml;   // [max_items, H, 2]  (reference max in log2 units, sum)
  int* plan;        // [2 batch + 2]: first item per sequence (batch + 1), lengths, chunk
  int batch, H, d_c, d_r, d_v, P, max_pages_per_seq;
  int len_cap;      // lengths are clamped to min(max_seq_len, block-table capacity)
  int slots;        // concurrent work-groups the split kernel can hold
  int max_items;    // capacity of the partial buffers
  int min_chunk, ovh_tokens;
  int round_ovh_tokens;  // planner: what a round costs besides its tokens, in cache rows
  float scale_log2; // softmax_scale * log2(e)
  int fp8;          // 1: 8-bit pool (E4M3 rows + float32 row scales per page)
  int num_pages;
  int* err;         // device error word (set by MLA_DEBUG builds only)
};

struct PrefillArgs {
  const void* q;
  const void* pool;
  const int32_t* block_table;
  const int32_t* cu_q;   // [num_seqs + 1] new (query) tokens per sequence
  const int32_t* cu_kv;  // [num_seqs + 1] all tokens per sequence (prefix + new), keys
  const void* w_uk;
  const void* w_uv;
  void* out;
  float* lse;
  void* ws_k;  // up-projected K_C: fp32 [total_kv, H, d_n] (generic) or bf16 [H, total_kv, d_n] (MFMA)
  void* ws_v;  // up-projected V:   fp32 [total_kv, H, d_v] (generic) or bf16 [H, total_kv, d_v] (MFMA)
  int num_seqs, total, total_kv, max_seq_len, H, d_n, d_r, d_c, d_v, P, max_pages_per_seq;
  float rope_base, scale;
  int max_kv_len;  // bound of every sequence's key count (max_seq_len bounds its new tokens)
  int num_pages;
  int* err;        // device error word (set by MLA_DEBUG builds only)
};

// 8-bit cache: quantize the bf16 rows of a [n_tokens][R] staging buffer into
// their slots of an 8-bit pool
hipError_t quantize_rows_fp8(const uint16_t* rows, const int64_t* slots, void* pool8, int n_tokens, int R, int P,
                             int num_pages, int* err, hipStream_t s);

// generic kernels (any shape, fp32 or bf16 storage)
hipError_t write_cache_generic(const WriteCacheArgs& a, bool bf16, hipStream_t s);
hipError_t absorb_generic(const AbsorbArgs& a, bool bf16, hipStream_t s);
hipError_t decode_generic(const DecodeArgs& a, bool bf16, hipStream_t s);  // a.fp8: bf16 queries, 8-bit pool
hipError_t prefill_generic(const PrefillArgs& a, bool bf16, hipStream_t s);

// MFMA projection kernels (bf16)
bool write_mfma_supported(int D, int d_c, int d_r);
hipError_t write_cache_mfma(const WriteCacheArgs& a, hipStream_t s);
bool absorb_mfma_supported(int H, int d_n, int d_c, int d_r);
hipError_t absorb_mfma(const AbsorbArgs& a, hipStream_t s);
// the decode step's cache write and absorption in one launch (at most 64
// tokens each, d_n = 128, d_c = 512): bit-identical to write_cache_mfma then
// absorb_mfma
// the fused cache write + absorption (k_write_absorb): its write part, its
// absorption part, its workspace (counters, then split-K partials)
bool write_absorb_fused_supported(int n_write, int D, int d_c, int d_r);
bool write_absorb_absorb_supported(int n_q, int H, int d_n, int d_c, int d_r);
size_t write_absorb_ws_bytes(int D, int d_c, int d_r);
hipError_t write_absorb_mfma(const WriteCacheArgs& wa, const AbsorbArgs& aa, void* workspace, int cus, hipStream_t s);

// MFMA decode kernels (bf16, latent width 512, rotary width 64)
bool decode_mfma_supported(int H, int d_c, int d_r, int d_v, int P, int batch);
int decode_mfma_slots(int H, int cus, bool fp8);
hipError_t decode_mfma(const DecodeArgs& a, hipStream_t s);
// Y[N, M] = X[N, K] W[M, K]^T (query compression, output projection): MFMA
// for bf16 with M % 64 == 0 and K % 64 == 0 (K split over work-groups when
// the tiles do not fill the GPU; part: gemm_workspace_bytes of fp32 partials),
// else plain kernels (fp32 or bf16 storage, fp32 arithmetic).
bool gemm_mfma_supported(int N, int M, int K);
int gemm_splits(int N, int M, int K, int cus);
size_t gemm_workspace_bytes(int N, int M, int K, int cus);
hipError_t gemm_bt(const void* X, const void* W, void* Y, int N, int M, int K, bool bf16, bool mfma, float* part,
                   int cus, hipStream_t s);
// MFMA prefill: d_n = d_v = 128, d_R = 64, bf16; workspace K_C and V as bf16 [H][total][128]
bool prefill_mfma_supported(int d_n, int d_v, int d_r, int d_c, int P);
hipError_t prefill_mfma(const PrefillArgs& a, hipStream_t s);

}  // namespace mla
