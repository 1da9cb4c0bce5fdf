// MFMA kernels for the two projections around the cache (gfx950, bf16):
//
// cache write   rows^T[R x N] = W_DKR[R x D] . h^T[D x N]   (16x16x32 MFMA)
//   One work-group per (16 cached features, 16 * TB4 tokens); its waves split
//   the hidden axis and meet in LDS.  In the accumulator each lane holds
//   4 consecutive features of one token, so the rotary pairs (2i, 2i+1) of
//   the k_R branch are rotated in registers before the bf16 store to the
//   token's slot.
//
// query absorption   q~[n][h][0:d_c] = q_C[n][h] . W_UK,h   (32x32x16 MFMA)
//   One work-group per (head, 128 latent columns, 64 tokens).  The W_UK,h
//   column block is staged row-major in LDS; its k-major operand fragments
//   come from the LDS transpose read.  The rotary half q_R is rotated by the
//   column-block-0 work-group of each head.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- cache write
template <int TB4, int NWV>
__global__ void __launch_bounds__(64 * NWV) k_write_mfma(WriteCacheArgs a) {
  __shared__ f32x4 part[NWV][TB4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int R = a.d_c + a.d_r;
  const int r0 = blockIdx.x * 16;
  const int n0 = blockIdx.y * 16 * TB4;
  const uint16_t* __restrict__ W = (const uint16_t*)a.w_dkr;
  const uint16_t* __restrict__ H = (const uint16_t*)a.h;
  const int D = a.D, ksteps = D / 32;
  const int m = lane & 15, kq = 8 * (lane >> 4);

  f32x4 acc[TB4];
#pragma unroll
  for (int t = 0; t < TB4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wp = W + (size_t)(r0 + m) * D + kq;
  const uint16_t* hp[TB4];
  bool hv[TB4];
#pragma unroll
  for (int t = 0; t < TB4; ++t) {
    const int n = n0 + 16 * t + m;
    hv[t] = n < a.n_tokens;
    hp[t] = H + (size_t)(hv[t] ? n : 0) * D + kq;
  }
#pragma unroll 8
  for (int ks = w; ks < ksteps; ks += NWV) {
    const u32x4 av = *(const u32x4*)(wp + 32 * ks);
#pragma unroll
    for (int t = 0; t < TB4; ++t) {
      u32x4 bv = *(const u32x4*)(hp[t] + 32 * ks);
      if (!hv[t]) bv = u32x4{0, 0, 0, 0};
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc[t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int t = 0; t < TB4; ++t) part[w][t][lane] = acc[t];
  __syncthreads();
  // epilogue: waves take token sub-blocks; fixed summation order over waves
  for (int t = w; t < TB4; t += NWV) {
    f32x4 v = part[0][t][lane];
#pragma unroll
    for (int k = 1; k < NWV; ++k) v += part[k][t][lane];
    const int n = n0 + 16 * t + m;  // D: lane holds token n = lane % 16, features 4 (lane / 16) + j
    if (n >= a.n_tokens) continue;
    const long long slot = a.slots[n];
    if (slot < 0) continue;
    const int rf = r0 + 4 * (lane >> 4);
    float o[4] = {v[0], v[1], v[2], v[3]};
    if (rf >= a.d_c) {
      const int pos = a.positions[n];
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        float c, s;
        rope_cs(pos, (rf - a.d_c) / 2 + pr, a.d_r, a.rope_base, c, s);
        const float x0 = o[2 * pr], x1 = o[2 * pr + 1];
        o[2 * pr] = x0 * c - x1 * s;
        o[2 * pr + 1] = x0 * s + x1 * c;
      }
    }
    const uint32_t lo = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
    uint16_t* dst = (uint16_t*)a.pool + (size_t)slot * R + rf;
    *(uint2*)dst = make_uint2(lo, hi);
  }
}

// ---------------------------------------------------------------- absorption
constexpr int AB_C = 128;  // latent columns per work-group
constexpr int AB_T = 64;   // tokens per work-group

__global__ void __launch_bounds__(256) k_absorb_mfma(AbsorbArgs a) {
  // W_UK,h[j][cb*128 .. +128] row-major, 256 bytes per row j; 16-byte chunk
  // slot XOR 2*(j % 4) makes the 4-row transpose reads conflict-free
  extern __shared__ __attribute__((aligned(16))) char wtile[];
  const int h = blockIdx.x, cb = blockIdx.y, n0 = blockIdx.z * AB_T;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int H = a.H, dn = a.d_n, dc = a.d_c, dq = a.d_n + a.d_r, R = a.d_c + a.d_r;
  const uint16_t* __restrict__ wuk = (const uint16_t*)a.w_uk + (size_t)h * dn * dc + cb * AB_C;
  // staged 8 chunks per thread at a time, all loads in flight before the stores
  for (int u0 = 0; u0 < dn * (AB_C / 8); u0 += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int u = u0 + k * 256 + tid, j = u >> 4, ch = u & 15;
      if (u < dn * (AB_C / 8)) v[k] = *(const u32x4*)(wuk + (size_t)j * dc + 8 * ch);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int u = u0 + k * 256 + tid, j = u >> 4, ch = u & 15;
      if (u < dn * (AB_C / 8)) *(u32x4*)(wtile + j * 256 + 16 * (ch ^ (2 * (j & 3)))) = v[k];
    }
  }
  __syncthreads();

  const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
  uint16_t* __restrict__ out = (uint16_t*)a.q_abs;
  const int g = lane >> 5, r = lane & 31;
  const int grp = lane >> 4, jl = lane & 15;
  // B operand (W^T fragment): lane gets W[k0 .. k0+3][col], col = 32 w + lane % 32
  const int tcol = 32 * w + 16 * (grp & 1) + 4 * (jl & 3);  // first column of the lane's 8-byte load
  for (int tb = 0; tb < AB_T / 32; ++tb) {
    const int n = n0 + 32 * tb + r;  // A operand: token = lane % 32
    const bool nv = n < a.n_tokens;
    const uint16_t* qp = Q + ((size_t)(nv ? n : 0) * H + h) * dq + 8 * g;
    f32x16 acc = f32x16{};
#pragma unroll 8
    for (int ks = 0; ks < dn / 16; ++ks) {
      u32x4 av = *(const u32x4*)(qp + 16 * ks);
      if (!nv) av = u32x4{0, 0, 0, 0};
      const int k0 = 16 * ks + 8 * g;
      const int j1 = k0 + (jl >> 2), j2 = j1 + 4;
      const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(wtile + j1 * 256 + 16 * ((tcol >> 3) ^ (2 * (j1 & 3))) + 2 * (tcol & 7)));
      const s16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(wtile + j2 * 256 + 16 * ((tcol >> 3) ^ (2 * (j2 & 3))) + 2 * (tcol & 7)));
      const s16x8 bv = s16x8{b1[0], b1[1], b1[2], b1[3], b2[0], b2[1], b2[2], b2[3]};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    }
    // D[token][col]: lane holds col = 32 w + lane % 32, tokens 8 (j/4) + 4 g + j % 4
    const int col = cb * AB_C + 32 * w + r;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int nn = n0 + 32 * tb + 8 * (j >> 2) + 4 * g + (j & 3);
      if (nn < a.n_tokens) out[((size_t)nn * H + h) * R + col] = f32_to_bf16(acc[j]);
    }
  }
  if (cb == 0) {
    const int np = a.d_r / 2;
    for (int u = tid; u < AB_T * np; u += 256) {
      const int nn = n0 + u / np, i = u % np;
      if (nn >= a.n_tokens) continue;
      const uint16_t* qr = Q + ((size_t)nn * H + h) * dq + dn;
      const float x0 = bf16_to_f32(qr[2 * i]), x1 = bf16_to_f32(qr[2 * i + 1]);
      float c, s;
      rope_cs(a.positions[nn], i, a.d_r, a.rope_base, c, s);
      uint16_t* o = out + ((size_t)nn * H + h) * R + dc;
      o[2 * i] = f32_to_bf16(x0 * c - x1 * s);
      o[2 * i + 1] = f32_to_bf16(x0 * s + x1 * c);
    }
  }
}

}  // namespace

bool write_mfma_supported(int D, int d_c, int d_r) { return D % 32 == 0 && d_c % 16 == 0 && d_r % 16 == 0; }

hipError_t write_cache_mfma(const WriteCacheArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  const int R = a.d_c + a.d_r;
  // few tokens (decode): W_DKR dominates the bytes, so 16 waves per work-group
  // split the hidden axis and keep many loads in flight; many tokens: 4 token
  // blocks per work-group reuse each W fragment 4 times
  if (a.n_tokens <= 1024) {
    hipLaunchKernelGGL((k_write_mfma<1, 16>), dim3(R / 16, (a.n_tokens + 15) / 16), dim3(1024), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_write_mfma<4, 4>), dim3(R / 16, (a.n_tokens + 63) / 64), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

bool absorb_mfma_supported(int H, int d_n, int d_c, int d_r) {
  return d_n % 16 == 0 && d_n <= 256 && d_c % AB_C == 0 && d_r % 2 == 0 && H >= 1;
}

hipError_t absorb_mfma(const AbsorbArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  const dim3 grid(a.H, a.d_c / AB_C, (a.n_tokens + AB_T - 1) / AB_T);
  hipLaunchKernelGGL(k_absorb_mfma, grid, dim3(256), (size_t)a.d_n * 256, s, a);
  return hipGetLastError();
}

}  // namespace mla
