// Device helpers shared by the HIP kernels of libmla (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_checks.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- storage
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- 8-bit cache
// E4M3 code (low byte) -> float, exact (the two NaN codes give NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false)[0];
}
// 8-bit pool page: P rows of R codes, then P float32 row scales.
__device__ __forceinline__ size_t fp8_page_bytes(int P, int R) { return (size_t)P * (size_t)(R + 4); }
__device__ __forceinline__ const uint8_t* fp8_row(const void* pool, long long slot, int P, int R) {
  return (const uint8_t*)pool + (size_t)(slot / P) * fp8_page_bytes(P, R) + (size_t)(slot % P) * R;
}
__device__ __forceinline__ float fp8_scale(const void* pool, long long slot, int P, int R) {
  return *(const float*)((const uint8_t*)pool + (size_t)(slot / P) * fp8_page_bytes(P, R) + (size_t)P * R +
                         4 * (size_t)(slot % P));
}

__device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }


// ---------------------------------------------------------------- LDS DMA
// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]; the other counters left at their maximum).
__device__ __forceinline__ constexpr int waitcnt_vm(int n) {
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14);
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One wave-wide direct-to-LDS load: lane l copies 16 bytes from
// sbase + voff(l) to LDS byte M0 + 16 l (M0 = lds_addr).  Written as inline
// asm so that the compiler adds no wait of its own before later LDS reads;
// callers wait with s_waitcnt vmcnt for exactly the loads they need.  The
// instruction writes no VGPR.  (The immediate offset of the instruction
// would move the LDS destination as well, so column offsets go into sbase.)
template <int COL>
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 offset:%3"
      :
      : "v"(voff), "s"(sbase), "s"(lds_addr), "i"(COL)
      : "memory", "m0");
}

// Direct-to-LDS load from a 64-bit per-lane address (rows gathered through
// a block table can lie anywhere in a pool larger than 4 GiB).
__device__ __forceinline__ void dma16_v(const void* p, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(p), "s"(lds_addr)
      : "memory", "m0");
}

// ---------------------------------------------------------------- RoPE
// Rotation of pair i of a d-wide vector at position pos: angle pos * theta_i,
// theta_i = base^(-2i/d).
//
// theta_i, in double.
__device__ __forceinline__ double rope_inv_freq(int i, int d, float base) {
  return exp2(-(2.0 * (double)i / (double)d) * log2((double)base));
}

// cos and sin of pos * theta.  The angle is formed and reduced in double,
// f = angle - k pi/2 with |f| <= pi/4 (pi/2 rounded to double is off by 6e-17,
// so k pi/2 is off by k * 6e-17 rad), and sin f, cos f are then the fp32
// Taylor series to f^9 and f^10 (the terms left out are below 2e-9 for
// |f| <= pi/4); k mod 4 picks the quadrant.  This keeps full fp32 accuracy
// at any position (pair 0 turns through tens of thousands of radians at long
// positions) for a few double operations.
__device__ __forceinline__ void rope_cs_theta(int pos, double theta, float& c, float& s) {
  const double ang = (double)pos * theta;
  const double k = rint(ang * 0.63661977236758134);         // 2 / pi
  const float f = (float)fma(-k, 1.5707963267948966, ang);  // pi / 2
  const float f2 = f * f;
  float sp = fmaf(f2, 1.f / 362880.f, -1.f / 5040.f);  // 1/9!, -1/7!
  sp = fmaf(sp, f2, 1.f / 120.f);
  sp = fmaf(sp, f2, -1.f / 6.f);
  const float sf = fmaf(f * f2, sp, f);
  float cp = fmaf(f2, -1.f / 3628800.f, 1.f / 40320.f);  // -1/10!, 1/8!
  cp = fmaf(cp, f2, -1.f / 720.f);
  cp = fmaf(cp, f2, 1.f / 24.f);
  cp = fmaf(cp, f2, -0.5f);
  const float cf = fmaf(cp, f2, 1.f);
  const int q = (int)(long long)k & 3;
  const float cs = (q & 1) ? sf : cf, sn = (q & 1) ? cf : sf;
  c = (q == 1 || q == 2) ? -cs : cs;
  s = (q & 2) ? -sn : sn;
}

__device__ __forceinline__ void rope_cs(int pos, int i, int d, float base, float& c, float& s) {
  rope_cs_theta(pos, rope_inv_freq(i, d, base), c, s);
}

// ---------------------------------------------------------------- decode work split
// The token axis of every sequence is cut into chunks of `chunk` tokens
// (a multiple of 32); chunk k of sequence b is work item s_items[b] + k.  The
// plan is a pure function of the clamped lengths, the slot count and the
// overhead estimate, so every work-group (and the combine kernel) computes
// the same plan without a host round trip, and the split points never depend
// on where pages live.
struct DecodePlan {
  int chunk;
  int n_items;
};

__device__ __forceinline__ int clamp_len(int len, int cap, int* err) { return clamp_report(len, 0, cap, err); }

// Candidate chunk sizes: the total token count spread over k * slots items
// for k = 1, 2, 4, rounded up to 32 and clamped to [min_chunk, max_chunk].  The chosen one
// minimises (rounds of `slots` items) * chunk + the partial-result overhead
// (ovh_tokens token-equivalents per item, spread over the slots), among the
// candidates whose item count fits the partial buffers (max_items; the host
// sizes them so that k = 1 always fits).
// The first wave computes the plan with wave reductions (no barrier inside);
// one barrier then publishes it.  s_len, s_items: LDS, >= batch + 1 ints;
// red: LDS, >= 16 ints.  All threads call.
__device__ __forceinline__ long long wave_sum_ll(long long v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline DecodePlan make_decode_plan(const int32_t* __restrict__ seq_lens, int batch, int cap,
                                              int slots, int min_chunk, int max_chunk, int ovh_tokens, int round_ovh,
                                              int* s_len,
                                              int* s_items, int* red, int* err, int max_items) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    long long part = 0;
    for (int b = lane; b < batch; b += 64) {
      const int L = clamp_len(seq_lens[b], cap, blockIdx.x == 0 ? err : nullptr);
      s_len[b] = L;
      part += L;
    }
    const long long total = wave_sum_ll(part);
    // items at chunk ch: this lane's own entries, summed over the wave
    // (the lengths were written above by the same lanes)
    const int best_chunk =
        choose_chunk(total, batch, slots, min_chunk, max_chunk, ovh_tokens, round_ovh, max_items, [&](int ch) {
          long long it = 0;
          for (int b = lane; b < batch; b += 64) it += (s_len[b] + ch - 1) / ch;
          return wave_sum_ll(it);
        });
    // exclusive prefix of item counts: lane l owns the contiguous run of
    // sequences [l per, l per + per); LDS operations of one wave complete in
    // order, so the lengths written above are visible here
    const int per = (batch + 63) / 64;
    const int b0 = lane * per, b1 = min(batch, b0 + per);
    int mine = 0;
    for (int b = b0; b < b1; ++b) mine += (s_len[b] + best_chunk - 1) / best_chunk;
    int x = mine;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    int pre = x - mine;
    for (int b = b0; b < b1; ++b) {
      s_items[b] = pre;
      pre += (s_len[b] + best_chunk - 1) / best_chunk;
    }
    if (lane == 63) {
      s_items[batch] = x;
      red[0] = best_chunk;
    }
  }
  __syncthreads();
  DecodePlan p;
  p.chunk = red[0];
  p.n_items = s_items[batch];
  return p;
}

// Sequence owning work item `item` (s_items ascending, s_items[batch] > item).
__device__ __forceinline__ int item_seq(const int* s_items, int batch, int item) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_items[mid] <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace mla
