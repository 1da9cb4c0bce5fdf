// Plain (VALU) kernels for every step, any dimensions, fp32 or bf16 storage.
// They are the library's path for shapes the MFMA kernels do not cover (for
// example the fp32 workloads) and a second implementation to cross-check the
// MFMA kernels on the same inputs.  Arithmetic is fp32 throughout.
#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

// --------------------------------------------------------------------------
// cache write: row = [W_DKV h | RoPE(W_KR h, p)], scattered to its slot.
// One thread per latent element or per rotary pair.
template <typename T>
__global__ void __launch_bounds__(256) k_write_cache(WriteCacheArgs a) {
  const int J = a.d_c + a.d_r / 2;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)a.n_tokens * J) return;
  const int n = (int)(idx / J), j = (int)(idx % J);
  const long long slot = a.dense ? (long long)n : checked_slot(a.slots[n], a.num_pages, a.P, a.err);
  if (slot < 0) return;
  const int R = a.d_c + a.d_r;
  const T* h = (const T*)a.h + (size_t)n * a.D;
  const T* W = (const T*)a.w_dkr;
  T* row = (T*)a.pool + (size_t)slot * R;
  if (j < a.d_c) {
    const T* w = W + (size_t)j * a.D;
    float acc = 0.f;
    for (int d = 0; d < a.D; ++d) acc += ld(w, d) * ld(h, d);
    st(row, j, acc);
  } else {
    const int i = j - a.d_c;
    const T* w0 = W + (size_t)(a.d_c + 2 * i) * a.D;
    const T* w1 = w0 + a.D;
    float x0 = 0.f, x1 = 0.f;
    for (int d = 0; d < a.D; ++d) {
      const float hv = ld(h, d);
      x0 += ld(w0, d) * hv;
      x1 += ld(w1, d) * hv;
    }
    float c, s;
    rope_cs(a.positions[n], i, a.d_r, a.rope_base, c, s);
    st(row, a.d_c + 2 * i, x0 * c - x1 * s);
    st(row, a.d_c + 2 * i + 1, x0 * s + x1 * c);
  }
}

// --------------------------------------------------------------------------
// query absorption: q~ = [W_UK,h^T q_C | RoPE(q_R, p)].
template <typename T>
__global__ void __launch_bounds__(256) k_absorb(AbsorbArgs a) {
  const int J = a.d_c + a.d_r / 2;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)a.n_tokens * a.H * J) return;
  const int j = (int)(idx % J);
  const long long nh = idx / J;
  const int h = (int)(nh % a.H), n = (int)(nh / a.H);
  const T* qv = (const T*)a.q + (size_t)nh * (a.d_n + a.d_r);
  T* out = (T*)a.q_abs + (size_t)nh * (a.d_c + a.d_r);
  if (j < a.d_c) {
    const T* w = (const T*)a.w_uk + (size_t)h * a.d_n * a.d_c + j;
    float acc = 0.f;
    for (int k = 0; k < a.d_n; ++k) acc += ld(qv, k) * ld(w, (size_t)k * a.d_c);
    st(out, j, acc);
  } else {
    const int i = j - a.d_c;
    const float x0 = ld(qv, a.d_n + 2 * i), x1 = ld(qv, a.d_n + 2 * i + 1);
    float c, s;
    rope_cs(a.positions[n], i, a.d_r, a.rope_base, c, s);
    st(out, a.d_c + 2 * i, x0 * c - x1 * s);
    st(out, a.d_c + 2 * i + 1, x0 * s + x1 * c);
  }
}

// --------------------------------------------------------------------------
// decode pass 1: one wave per (work item, head).  Online softmax over the
// item's token range in tiles of 64 tokens (one score per lane), latent
// accumulator in LDS.  Emits (m, l, acc) in log2 units.
// With F8 the pool is 8-bit (queries stay T = bf16): a row's score is its
// code values' dot product times the row scale, and the row scale rides with
// the numerator into the latent sum (p 2^e times the code values), while the
// softmax sum takes p itself.
template <typename T, bool F8 = false>
__global__ void __launch_bounds__(64) k_decode_split(DecodeArgs a) {
  extern __shared__ float dyn[];
  int* s_len = (int*)dyn;
  int* s_items = s_len + (a.batch + 1);
  int* red = s_items + (a.batch + 1);
  const int R = a.d_c + a.d_r;
  float* q_s = (float*)(red + 16);
  float* p_s = q_s + R;
  float* acc = p_s + 64;
  typedef typename std::conditional<F8, uint8_t, T>::type RowT;
  const RowT** rows = (const RowT**)(acc + a.d_c + (a.d_c & 1));  // 8-byte aligned: all sizes above are ints

  const int cap = a.len_cap;
  const DecodePlan plan = make_decode_plan(a.seq_lens, a.batch, cap, a.slots, a.min_chunk, kMaxChunk, a.ovh_tokens, a.round_ovh_tokens,
                                           s_len, s_items, red, a.err, a.max_items);
  const int item = blockIdx.x;
  if (item >= plan.n_items) return;
  const int h = blockIdx.y, lane = threadIdx.x;
  const int b = item_seq(s_items, a.batch, item);
  const int t0 = (item - s_items[b]) * plan.chunk;
  const int t1 = min(s_len[b], t0 + plan.chunk);

  const T* q = (const T*)a.q_abs + ((size_t)b * a.H + h) * R;
  for (int r = lane; r < R; r += 64) q_s[r] = ld(q, r);
  for (int c = lane; c < a.d_c; c += 64) acc[c] = 0.f;
  __syncthreads();
  float m = -INFINITY, l = 0.f;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages_per_seq;
  for (int tb = t0; tb < t1; tb += 64) {
    const int t = tb + lane;
    const bool valid = t < t1;
    float s = -INFINITY, rscale = 1.f;
    const RowT* row = nullptr;
    if (valid) {
      const long long slot = (long long)checked_page(bt[t / a.P], a.num_pages, a.err) * a.P + (t % a.P);
      float dot = 0.f;
      if constexpr (F8) {
        row = fp8_row(a.pool, slot, a.P, R);
        rscale = fp8_scale(a.pool, slot, a.P, R);
        for (int r = 0; r < R; ++r) dot += q_s[r] * e4m3_to_f32(row[r]);
        dot *= rscale;
      } else {
        row = (const T*)a.pool + (size_t)slot * R;
        for (int r = 0; r < R; ++r) dot += q_s[r] * ld(row, r);
      }
      s = dot * a.scale_log2;
    }
    float mt = s;
    for (int o = 32; o > 0; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o));
    const float m_new = fmaxf(m, mt);
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
    const float p = valid ? exp2f(s - m_new) : 0.f;
    float ps = p;
    for (int o = 32; o > 0; o >>= 1) ps += __shfl_xor(ps, o);
    l = l * alpha + ps;
    m = m_new;
    p_s[lane] = valid ? p * rscale : 0.f;
    rows[lane] = row;
    __syncthreads();
    const int nt = min(64, t1 - tb);
    for (int c = lane; c < a.d_c; c += 64) {
      float v = acc[c] * alpha;
      if constexpr (F8) {
        for (int k = 0; k < nt; ++k) v += p_s[k] * e4m3_to_f32(rows[k][c]);
      } else {
        for (int k = 0; k < nt; ++k) v += p_s[k] * ld(rows[k], c);
      }
      acc[c] = v;
    }
    __syncthreads();
  }
  float* pa = a.part_acc + ((size_t)item * a.H + h) * a.d_c;
  for (int c = lane; c < a.d_c; c += 64) pa[c] = acc[c];
  if (lane == 0) {
    a.part_ml[((size_t)item * a.H + h) * 2 + 0] = m;
    a.part_ml[((size_t)item * a.H + h) * 2 + 1] = l;
  }
}

// decode pass 2: merge the items of one sequence for one head, then W_UV.
template <typename T>
__global__ void __launch_bounds__(128) k_decode_combine(DecodeArgs a) {
  extern __shared__ float dyn[];
  int* s_len = (int*)dyn;
  int* s_items = s_len + (a.batch + 1);
  int* red = s_items + (a.batch + 1);
  float* lat = (float*)(red + 16);
  float* stat = lat + a.d_c;  // m*, 1/L

  const int cap = a.len_cap;
  make_decode_plan(a.seq_lens, a.batch, cap, a.slots, a.min_chunk, kMaxChunk, a.ovh_tokens, a.round_ovh_tokens, s_len, s_items, red, a.err, a.max_items);
  const int b = blockIdx.x, h = blockIdx.y;
  const int i0 = s_items[b], i1 = s_items[b + 1];
  T* out = (T*)a.out + ((size_t)b * a.H + h) * a.d_v;
  if (i0 == i1) {
    for (int v = threadIdx.x; v < a.d_v; v += blockDim.x) st(out, v, 0.f);
    if (a.lse && threadIdx.x == 0) a.lse[(size_t)b * a.H + h] = -INFINITY;
    return;
  }
  if (threadIdx.x == 0) {
    float ms = -INFINITY;
    for (int i = i0; i < i1; ++i) ms = fmaxf(ms, a.part_ml[((size_t)i * a.H + h) * 2]);
    float L = 0.f;
    for (int i = i0; i < i1; ++i) {
      const float mi = a.part_ml[((size_t)i * a.H + h) * 2];
      L += exp2f(mi - ms) * a.part_ml[((size_t)i * a.H + h) * 2 + 1];
    }
    stat[0] = ms;
    stat[1] = 1.f / L;
    if (a.lse) a.lse[(size_t)b * a.H + h] = (ms + log2f(L)) * kLn2;
  }
  __syncthreads();
  const float ms = stat[0], invL = stat[1];
  for (int c = threadIdx.x; c < a.d_c; c += blockDim.x) {
    float v = 0.f;
    for (int i = i0; i < i1; ++i) {
      const float w = exp2f(a.part_ml[((size_t)i * a.H + h) * 2] - ms);
      v += w * a.part_acc[((size_t)i * a.H + h) * a.d_c + c];
    }
    lat[c] = v * invL;
  }
  __syncthreads();
  const T* wuv = (const T*)a.w_uv + (size_t)h * a.d_v * a.d_c;
  for (int v = threadIdx.x; v < a.d_v; v += blockDim.x) {
    float o = 0.f;
    for (int c = 0; c < a.d_c; ++c) o += ld(wuv, (size_t)v * a.d_c + c) * lat[c];
    st(out, v, o);
  }
}

// --------------------------------------------------------------------------
// prefill: up-project K_C and V per head into an fp32 workspace (every key
// token: cached prefix and new tokens), then causal attention with one
// work-group per (new query token, head).
__device__ __forceinline__ int seq_of(const int32_t* cu, int num_seqs, int n) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= n) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <typename T>
__global__ void __launch_bounds__(256) k_prefill_upproj(PrefillArgs a) {
  const int J = a.d_n + a.d_v;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)a.total_kv * a.H * J) return;
  const int j = (int)(idx % J);
  const long long nh = idx / J;
  const int h = (int)(nh % a.H), n = (int)(nh / a.H);  // n: key token (prefix and new)
  const int sq = seq_of(a.cu_kv, a.num_seqs, n);
  // clamped so that the block-table read stays in row sq (max_kv_len <= capacity)
  const int t = key_position(n, a.cu_kv[sq], a.max_kv_len, a.err);
  const int R = a.d_c + a.d_r;
  const int page = checked_page(a.block_table[(size_t)sq * a.max_pages_per_seq + t / a.P], a.num_pages, a.err);
  const T* row = (const T*)a.pool + ((size_t)page * a.P + t % a.P) * R;
  const T* w = (j < a.d_n) ? (const T*)a.w_uk + ((size_t)h * a.d_n + j) * a.d_c
                           : (const T*)a.w_uv + ((size_t)h * a.d_v + (j - a.d_n)) * a.d_c;
  float acc = 0.f;
  for (int c = 0; c < a.d_c; ++c) acc += ld(row, c) * ld(w, c);
  if (j < a.d_n) ((float*)a.ws_k)[(size_t)nh * a.d_n + j] = acc;
  else ((float*)a.ws_v)[(size_t)nh * a.d_v + (j - a.d_n)] = acc;
}

template <typename T>
__global__ void __launch_bounds__(128) k_prefill_attn(PrefillArgs a) {
  extern __shared__ float dyn[];
  float* qs = dyn;                     // d_n + d_r
  float* ps = qs + a.d_n + a.d_r;      // 128
  float* red = ps + 128;               // 4
  const int n = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int sq = seq_of(a.cu_q, a.num_seqs, n);
  const PrefillSeq sd = prefill_seq(a.cu_q, a.cu_kv, sq, a.total, a.total_kv, a.max_seq_len, a.max_kv_len, a.err);
  if (n < sd.q0 || n >= sd.q0 + sd.q_len) return;  // a row no (clamped) sequence covers
  const int base = sd.k0;  // first key token of the sequence in the workspace
  const int prefix = sd.kv_len - sd.q_len;
  const int i = prefix + n - sd.q0;  // position of this query in its sequence
  const int R = a.d_c + a.d_r;
  const T* qv = (const T*)a.q + ((size_t)n * a.H + h) * (a.d_n + a.d_r);
  for (int k = tid; k < a.d_n; k += 128) qs[k] = ld(qv, k);
  for (int p = tid; p < a.d_r / 2; p += 128) {
    float c, s;
    rope_cs(i, p, a.d_r, a.rope_base, c, s);
    const float x0 = ld(qv, a.d_n + 2 * p), x1 = ld(qv, a.d_n + 2 * p + 1);
    qs[a.d_n + 2 * p] = x0 * c - x1 * s;
    qs[a.d_n + 2 * p + 1] = x0 * s + x1 * c;
  }
  __syncthreads();
  const float* K = (const float*)a.ws_k;
  const float* V = (const float*)a.ws_v;
  const float sl2 = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  const int32_t* bt = a.block_table + (size_t)sq * a.max_pages_per_seq;
  for (int tb = 0; tb <= i; tb += 128) {
    const int t = tb + tid;
    float s = -INFINITY;
    if (t <= i) {
      const float* kc = K + ((size_t)(base + t) * a.H + h) * a.d_n;
      const T* row = (const T*)a.pool + ((size_t)checked_page(bt[t / a.P], a.num_pages, a.err) * a.P + t % a.P) * R;
      float dot = 0.f;
      for (int k = 0; k < a.d_n; ++k) dot += qs[k] * kc[k];
      for (int r = 0; r < a.d_r; ++r) dot += qs[a.d_n + r] * ld(row, a.d_c + r);
      s = dot * sl2;
    }
    float mt = s;
    for (int o = 32; o > 0; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o));
    if ((tid & 63) == 0) red[tid >> 6] = mt;
    __syncthreads();
    mt = fmaxf(red[0], red[1]);
    const float m_new = fmaxf(m, mt);
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
    const float p = (t <= i) ? exp2f(s - m_new) : 0.f;
    ps[tid] = p;
    float psum = p;
    for (int o = 32; o > 0; o >>= 1) psum += __shfl_xor(psum, o);
    __syncthreads();
    if ((tid & 63) == 0) red[2 + (tid >> 6)] = psum;
    __syncthreads();
    l = l * alpha + red[2] + red[3];
    m = m_new;
    const int nt = min(128, i + 1 - tb);
    acc0 *= alpha;
    acc1 *= alpha;
    for (int k = 0; k < nt; ++k) {
      const float* vv = V + ((size_t)(base + tb + k) * a.H + h) * a.d_v;
      const float pk = ps[k];
      if (tid < a.d_v) acc0 += pk * vv[tid];
      if (tid + 128 < a.d_v) acc1 += pk * vv[tid + 128];
    }
    __syncthreads();
  }
  T* out = (T*)a.out + ((size_t)n * a.H + h) * a.d_v;
  const float invl = 1.f / l;
  if (tid < a.d_v) st(out, tid, acc0 * invl);
  if (tid + 128 < a.d_v) st(out, tid + 128, acc1 * invl);
  if (a.lse && tid == 0) a.lse[(size_t)n * a.H + h] = (m + log2f(l)) * kLn2;
}

// --------------------------------------------------------------------------
// 8-bit cache rows: one wave per token.  amax = largest |x| of the bf16 row;
// scale 2^e with e the smallest exponent >= -126 such that amax <= 448 2^e
// (amax = f 2^k with 1 <= f < 2 and 448 = 1.75 2^8: e = k - 8, plus one when
// f > 1.75); codes = E4M3 nearest x / 2^e (the hardware conversion rounds to
// nearest even; x / 2^e is exact), a -0 result stored as +0.
__global__ void __launch_bounds__(256) k_quantize_rows(const uint16_t* __restrict__ rows,
                                                       const int64_t* __restrict__ slots, uint8_t* __restrict__ pool8,
                                                       int n_tokens, int R, int P, int num_pages, int* err) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (n >= n_tokens) return;
  const long long slot = checked_slot(slots[n], num_pages, P, err);
  if (slot < 0) return;
  const uint16_t* row = rows + (size_t)n * R;
  float amax = 0.f;
  for (int c = lane; c < R; c += 64) amax = fmaxf(amax, fabsf(bf16_to_f32(row[c])));
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  int e = 0;
  if (amax > 0.f) {
    const uint32_t bits = __float_as_uint(amax);
    const int k = (int)(bits >> 23) - 127;  // a subnormal amax gives k = -127: clamped below
    e = max(k - 8 + ((bits & 0x7fffffu) > 0x600000u ? 1 : 0), -126);
  }
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-126, 120]
  uint8_t* page = pool8 + (size_t)(slot / P) * fp8_page_bytes(P, R);
  const int t = (int)(slot % P);
  for (int c = lane; c < R; c += 64) {
    uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(bf16_to_f32(row[c]) * inv, 0.f, 0, false) & 0xffu;
    if (code == 0x80u) code = 0u;
    page[(size_t)t * R + c] = (uint8_t)code;
  }
  if (lane == 0) *(float*)(page + (size_t)P * R + 4 * t) = __uint_as_float((uint32_t)(127 + e) << 23);
}

inline unsigned blocks_for(long long n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

// --------------------------------------------------------------------------
hipError_t write_cache_generic(const WriteCacheArgs& a, bool bf16, hipStream_t s) {
  const long long n = (long long)a.n_tokens * (a.d_c + a.d_r / 2);
  if (n == 0) return hipSuccess;
  if (bf16) hipLaunchKernelGGL(k_write_cache<uint16_t>, dim3(blocks_for(n, 256)), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_write_cache<float>, dim3(blocks_for(n, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t quantize_rows_fp8(const uint16_t* rows, const int64_t* slots, void* pool8, int n_tokens, int R, int P,
                             int num_pages, int* err, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_rows, dim3(blocks_for(n_tokens, 4)), dim3(256), 0, s, rows, slots, (uint8_t*)pool8,
                     n_tokens, R, P, num_pages, err);
  return hipGetLastError();
}

hipError_t absorb_generic(const AbsorbArgs& a, bool bf16, hipStream_t s) {
  const long long n = (long long)a.n_tokens * a.H * (a.d_c + a.d_r / 2);
  if (n == 0) return hipSuccess;
  if (bf16) hipLaunchKernelGGL(k_absorb<uint16_t>, dim3(blocks_for(n, 256)), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_absorb<float>, dim3(blocks_for(n, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t decode_generic(const DecodeArgs& a, bool bf16, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const size_t plan_bytes = (size_t)(2 * (a.batch + 1) + 16) * sizeof(int);
  const size_t split_lds = plan_bytes + (size_t)(a.d_c + a.d_r + 64 + a.d_c + 1) * sizeof(float) +
                           64 * sizeof(void*) + 8;
  const size_t comb_lds = plan_bytes + (size_t)(a.d_c + 2) * sizeof(float);
  const dim3 g1(a.max_items, a.H), g2(a.batch, a.H);
  if (a.fp8) {
    hipLaunchKernelGGL((k_decode_split<uint16_t, true>), g1, dim3(64), split_lds, s, a);
    hipLaunchKernelGGL(k_decode_combine<uint16_t>, g2, dim3(128), comb_lds, s, a);
  } else if (bf16) {
    hipLaunchKernelGGL(k_decode_split<uint16_t>, g1, dim3(64), split_lds, s, a);
    hipLaunchKernelGGL(k_decode_combine<uint16_t>, g2, dim3(128), comb_lds, s, a);
  } else {
    hipLaunchKernelGGL(k_decode_split<float>, g1, dim3(64), split_lds, s, a);
    hipLaunchKernelGGL(k_decode_combine<float>, g2, dim3(128), comb_lds, s, a);
  }
  return hipGetLastError();
}

hipError_t prefill_generic(const PrefillArgs& a, bool bf16, hipStream_t s) {
  if (a.total == 0) return hipSuccess;
  const long long n = (long long)a.total_kv * a.H * (a.d_n + a.d_v);
  const size_t lds = (size_t)(a.d_n + a.d_r + 128 + 4) * sizeof(float);
  if (bf16) {
    hipLaunchKernelGGL(k_prefill_upproj<uint16_t>, dim3(blocks_for(n, 256)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_prefill_attn<uint16_t>, dim3(a.total, a.H), dim3(128), lds, s, a);
  } else {
    hipLaunchKernelGGL(k_prefill_upproj<float>, dim3(blocks_for(n, 256)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_prefill_attn<float>, dim3(a.total, a.H), dim3(128), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
