// Dense products of the query compression and the output projection:
// Y[N, M] = X[N, K] W[M, K]^T, bf16 operands, fp32 accumulation (MFMA
// 32x32x16 for gfx950), and plain VALU kernels for fp32 or other shapes.
// At decode sizes (N of the order of the batch) these products stream their
// weight matrix once and are bound by HBM; the K axis is split over
// work-groups when the output tiles alone would not fill the GPU, and the
// fp32 partial sums are added by a second pass.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

constexpr int GM = 64;  // output columns (rows of W) per work-group
constexpr int GN = 64;  // output rows (rows of X) per work-group
constexpr int GK = 64;  // k per stage: one 128-byte row segment
constexpr int GSTAGE = (GM + GN) * GK * 2;  // 16 KiB: 64 W rows, then 64 X rows
constexpr int GNST = 3;

// LDS row r (128 bytes): 16-byte chunk c at slot c ^ ((r >> 1) & 7), so that
// the 16 lanes of one LDS cycle (rows r .. r + 15, one chunk) hit 16
// different 4-bank groups.
__device__ __forceinline__ int gslot(int r, int c) { return c ^ ((r >> 1) & 7); }

// Work-group (mt, nt, z): W rows 64 mt .. +63, X rows 64 nt .. +63, k range
// [z kc, (z + 1) kc).  Wave w computes the 32 x 32 block (m half w & 1,
// n half w >> 1): D[m][n] = sum_k W[m][k] X[n][k], A = W rows, B = X^T.
// OUT: 0 = bf16 Y (z must be 0), 1 = fp32 partial [z][N][M].
template <int OUT>
__global__ void __launch_bounds__(256, 2) k_gemm_bt(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                    void* __restrict__ Y, int N, int M, int K, int kc) {
  __shared__ __attribute__((aligned(16))) char smem[GNST * GSTAGE];
  const int mt = blockIdx.x, nt = blockIdx.y, z = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const uint32_t lds0 = lds_addr_of(smem);
  const int k0 = z * kc, nk = kc / GK;

  // loads: instruction i = w + 4 j (j < 4) of a stage fills LDS bytes
  // [1024 i, +1024): rows 8 (i % 8) + lane / 8 of the W block (i < 8) or of
  // the X block (i >= 8), slot lane % 8 (source chunk slot ^ row swizzle)
  const char* src[4];
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = w + 4 * j;
    const int r = 8 * (i & 7) + (lane >> 3);
    const int c = gslot(r, lane & 7);
    if (i < 8) {
      src[j] = (const char*)(W + (size_t)(GM * mt + r) * K + k0);
    } else {
      const int n = min(GN * nt + r, N - 1);  // rows past N repeat the last one (not stored)
      src[j] = (const char*)(X + (size_t)n * K + k0);
    }
    voff[j] = 16u * c;
  }
  auto issue = [&](int kb, int st) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // per-lane source rows: a 64-bit per-lane address
      dma16_v(src[j] + 128 * kb + voff[j], lds0 + st * GSTAGE + 1024 * (w + 4 * j));
    }
  };

  f32x16 acc = f32x16{};
  const int mb = w & 1, nb = w >> 1;
  const int ra = 32 * mb + r32, rb = GM + 32 * nb + r32;  // LDS rows of this lane's A and B fragments
#pragma unroll
  for (int s = 0; s < GNST - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kb = 0; kb < nk; ++kb) {
    // stage kb landed once only the later stages' loads remain
    if (kb + 1 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();  // stage kb visible; stage kb - 1 no longer read
    asm volatile("" ::: "memory");
    if (kb + GNST - 1 < nk) issue(kb + GNST - 1, (kb + GNST - 1) % GNST);
    const char* st = smem + (kb % GNST) * GSTAGE;
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      const int c = 2 * ks + g;
      const u32x4 av = *(const u32x4*)(st + ra * 128 + 16 * gslot(ra, c));
      const u32x4 bv = *(const u32x4*)(st + rb * 128 + 16 * gslot(rb, c));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bv), acc, 0, 0, 0);
    }
  }
  // D: lane holds column n = r32 of its block, rows m = 8 (j / 4) + 4 g + j % 4
  const int n = GN * nt + 32 * nb + r32;
  if (n >= N) return;
  const int m0 = GM * mt + 32 * mb + 4 * g;
  if constexpr (OUT == 0) {
    uint16_t* y = (uint16_t*)Y + (size_t)n * M + m0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(u32x2*)(y + 8 * q) = u32x2{pack_bf16(acc[4 * q], acc[4 * q + 1]), pack_bf16(acc[4 * q + 2], acc[4 * q + 3])};
  } else {
    float* y = (float*)Y + ((size_t)z * N + n) * M + m0;
#pragma unroll
    for (int q = 0; q < 4; ++q) *(f32x4*)(y + 8 * q) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
  }
}

// Weight-streaming form for few rows of X (N <= 64, the decode batch): a
// work-group takes 256 rows of W against all N rows of X, so each X k block
// it loads serves four times as many W rows as in k_gemm_bt and the bytes
// through a CU are mostly weights.  Wave w computes W rows 64 w .. +63 against
// the 64 X rows as 2 x 2 blocks of 32 x 32.  A stage is one 64-wide k block:
// 256 W rows then 64 X rows of 128 bytes (40 KiB, swizzled as gslot), filled
// by 40 direct-to-LDS loads (10 per wave); NST stages ring, NST - 1 ahead.
// Split z of `splits` takes k blocks [z kb / splits, (z + 1) kb / splits) of
// the kb = K / 64 (the splits need not divide kb).  OUT as k_gemm_bt.
constexpr int WSM = 256;                     // W rows per work-group
constexpr int WS_STAGE = (WSM + GN) * GK * 2;  // 40 KiB
constexpr int WS_LPW = (WSM + GN) / 8 / 4;     // loads per wave per stage (10)

template <int OUT, int NST>
__global__ void __launch_bounds__(256, 1) k_gemm_ws(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                     void* __restrict__ Y, int N, int M, int K, int splits) {
  __shared__ __attribute__((aligned(16))) char smem[NST * WS_STAGE];
  const int mt = blockIdx.x, z = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const uint32_t lds0 = lds_addr_of(smem);
  const int kb_all = K / GK, kb0 = z * kb_all / splits, kb1 = (z + 1) * kb_all / splits;
  const int k0 = kb0 * GK, nk = kb1 - kb0;

  // load j of this wave fills LDS bytes [1024 i, +1024) of a stage, i = w + 4 j:
  // rows 8 i + lane / 8 (W rows below 256, then X rows), slot lane % 8
  const char* src[WS_LPW];
#pragma unroll
  for (int j = 0; j < WS_LPW; ++j) {
    const int i = w + 4 * j;
    const int r = 8 * i + (lane >> 3);
    const int c = gslot(r, lane & 7);
    if (r < WSM) {
      src[j] = (const char*)(W + (size_t)(WSM * mt + r) * K + k0 + 8 * c);
    } else {
      const int n = min(r - WSM, N - 1);  // rows past N repeat the last one (not stored)
      src[j] = (const char*)(X + (size_t)n * K + k0 + 8 * c);
    }
  }
  auto issue = [&](int kb, int st) {
#pragma unroll
    for (int j = 0; j < WS_LPW; ++j) dma16_v(src[j] + 128 * kb, lds0 + st * WS_STAGE + 1024 * (w + 4 * j));
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{};
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kb = 0; kb < nk; ++kb) {
    // stage kb landed once only the later stages' loads remain (NST - 2 of
    // them at most: stage kb + NST - 1 is requested after this wait)
    static_assert(NST >= 2 && NST <= 4, "wait counts below");
    if (NST == 4 && kb + 2 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * WS_LPW));
    else if (NST >= 3 && kb + 1 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_vm(WS_LPW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();  // stage kb visible; stage kb - 1 no longer read
    asm volatile("" ::: "memory");
    if (kb + NST - 1 < nk) issue(kb + NST - 1, (kb + NST - 1) % NST);
    const char* st = smem + (kb % NST) * WS_STAGE;
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      const int c = 2 * ks + g;
      u32x4 av[2], bv[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int ra = 64 * w + 32 * mb + r32;
        av[mb] = *(const u32x4*)(st + ra * 128 + 16 * gslot(ra, c));
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int rb = WSM + 32 * nb + r32;
        bv[nb] = *(const u32x4*)(st + rb * 128 + 16 * gslot(rb, c));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[mb]), as_bf16x8(bv[nb]), acc[mb][nb], 0,
                                                                0, 0);
    }
  }
  // D: lane holds column n = r32 of its block, rows m = 8 (j / 4) + 4 g + j % 4
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = 32 * nb + r32;
    if (n >= N) continue;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int m0 = WSM * mt + 64 * w + 32 * mb + 4 * g;
      const f32x16& v = acc[mb][nb];
      if constexpr (OUT == 0) {
        uint16_t* y = (uint16_t*)Y + (size_t)n * M + m0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(u32x2*)(y + 8 * q) = u32x2{pack_bf16(v[4 * q], v[4 * q + 1]), pack_bf16(v[4 * q + 2], v[4 * q + 3])};
      } else {
        float* y = (float*)Y + ((size_t)z * N + n) * M + m0;
#pragma unroll
        for (int q = 0; q < 4; ++q) *(f32x4*)(y + 8 * q) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
      }
    }
  }
}

// Y[n][m] = sum over the splits of the fp32 partials, rounded to bf16;
// four outputs per thread.  Eight partials are requested at a time into
// separate sums (z % 8), which are then added in a fixed order.
__global__ void __launch_bounds__(256) k_gemm_reduce(const float* __restrict__ part, uint16_t* __restrict__ Y,
                                                     int NM, int splits) {
  const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (i >= NM) return;
  f32x4 s8[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) s8[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  int z = 0;
  for (; z + 8 <= splits; z += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) s8[u] += *(const f32x4*)(part + (size_t)(z + u) * NM + i);
  }
#pragma unroll
  for (int u = 0; u < 7; ++u)
    if (z + u < splits) s8[u] += *(const f32x4*)(part + (size_t)(z + u) * NM + i);
  const f32x4 s = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
  *(u32x2*)(Y + i) = u32x2{pack_bf16(s[0], s[1]), pack_bf16(s[2], s[3])};
}

// Plain kernel: one thread per output, fp32 arithmetic, any shape.
template <typename T>
__global__ void __launch_bounds__(256) k_gemm_generic(const T* __restrict__ X, const T* __restrict__ W,
                                                      T* __restrict__ Y, int N, int M, int K) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)N * M) return;
  const int n = (int)(idx / M), m = (int)(idx % M);
  const T* x = X + (size_t)n * K;
  const T* wr = W + (size_t)m * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc += ld(x, k) * ld(wr, k);
  st(Y, idx, acc);
}

}  // namespace

bool gemm_mfma_supported(int N, int M, int K) { return N >= 1 && M % GM == 0 && K % GK == 0 && K >= GK; }

// The weight-streaming form takes N <= 64 and M % 256 == 0.
static bool gemm_ws_form(int N, int M, int K) { return N >= 1 && N <= GN && M % WSM == 0 && K % GK == 0 && K >= GK; }

// Its K splits: as many as keep one work-group per CU at most (M / 256 tiles
// times the splits) and at least four 64-wide k blocks per split.
static int gemm_ws_splits(int M, int K, int cus) {
  const int tiles = M / WSM, kb = K / GK;
  int sp = cus / tiles;
  if (sp > kb / 4) sp = kb / 4;
  return sp > 1 ? sp : 1;
}

// K splits of k_gemm_bt: enough work-groups for about two per CU, each split
// a whole number of 64-wide k blocks.
int gemm_splits(int N, int M, int K, int cus) {
  if (gemm_ws_form(N, M, K)) return gemm_ws_splits(M, K, cus);
  const long long tiles = (long long)(M / GM) * ((N + GN - 1) / GN);
  const int kb = K / GK;
  int s = 1;
  while (tiles * s < 2LL * cus && s < kb) {
    int t = s + 1;
    while (t <= kb && kb % t != 0) ++t;
    if (t > kb) break;
    s = t;
  }
  return s;
}

size_t gemm_workspace_bytes(int N, int M, int K, int cus) {
  if (!gemm_mfma_supported(N, M, K)) return 0;
  const int splits = gemm_splits(N, M, K, cus);
  return splits > 1 ? (size_t)splits * N * M * sizeof(float) : 0;
}

hipError_t gemm_bt(const void* X, const void* W, void* Y, int N, int M, int K, bool bf16, bool mfma, float* part,
                   int cus, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (mfma && gemm_ws_form(N, M, K)) {
    const int splits = gemm_ws_splits(M, K, cus);
    const dim3 grid(M / WSM, 1, splits);
    if (splits == 1) {
      hipLaunchKernelGGL((k_gemm_ws<0, 4>), grid, dim3(256), 0, s, (const uint16_t*)X, (const uint16_t*)W, Y, N, M, K,
                         1);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((k_gemm_ws<1, 4>), grid, dim3(256), 0, s, (const uint16_t*)X, (const uint16_t*)W, (void*)part,
                       N, M, K, splits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int NM = N * M;
    hipLaunchKernelGGL(k_gemm_reduce, dim3((NM / 4 + 255) / 256), dim3(256), 0, s, part, (uint16_t*)Y, NM, splits);
    return hipGetLastError();
  }
  if (mfma) {
    const int splits = gemm_splits(N, M, K, cus);
    const dim3 grid(M / GM, (N + GN - 1) / GN, splits);
    if (splits == 1) {
      hipLaunchKernelGGL(k_gemm_bt<0>, grid, dim3(256), 0, s, (const uint16_t*)X, (const uint16_t*)W, Y, N, M, K, K);
    } else {
      hipLaunchKernelGGL(k_gemm_bt<1>, grid, dim3(256), 0, s, (const uint16_t*)X, (const uint16_t*)W, (void*)part, N,
                         M, K, K / splits);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int NM = N * M;  // M % 64 == 0: a multiple of 4
      hipLaunchKernelGGL(k_gemm_reduce, dim3((NM / 4 + 255) / 256), dim3(256), 0, s, part, (uint16_t*)Y, NM, splits);
    }
    return hipGetLastError();
  }
  const long long total = (long long)N * M;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(k_gemm_generic<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)X, (const uint16_t*)W,
                       (uint16_t*)Y, N, M, K);
  else
    hipLaunchKernelGGL(k_gemm_generic<float>, grid, dim3(256), 0, s, (const float*)X, (const float*)W, (float*)Y, N, M,
                       K);
  return hipGetLastError();
}

}  // namespace mla
