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

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// ---------------------------------------------------------------- cache write
// Every wave owns a contiguous range of 64-wide k chunks.  A chunk of the 16
// W rows and 16 * TB4 h rows is fetched with whole 128-byte lines per row (8
// lanes x 16 bytes), staged in the wave's own LDS slice and read back as MFMA
// fragments: row-scattered 16-byte fragment loads run at a fraction of the
// coalesced rate on this part.  LDS slice row layout: 8 16-byte pieces,
// piece p of row r at slot p ^ (r % 8) (conflict-free fragment reads).
// KB chunks are loaded into registers at a time (all of a wave's chunks in
// one round trip when KB covers them) and pass through NSL LDS slices.
template <int TB4, int NWV, int NSL>
struct WriteLds {
  uint16_t stage[NWV][NSL][(16 + 16 * TB4) * 64];  // W rows, then h rows
  f32x4 part[NWV][TB4][64];
};

// One work-group's tile (features 16 bx .. +15, tokens 16 TB4 by ..) of the cache write.
template <int TB4, int NWV, int KB, int NSL>
__device__ __forceinline__ void write_tile(const WriteCacheArgs& a, int bx, int by, WriteLds<TB4, NWV, NSL>& lds) {
  constexpr int ROWS = 16 + 16 * TB4;  // W rows, then h rows
  auto& stage = lds.stage;
  auto& part = lds.part;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int R = a.d_c + a.d_r;
  const int r0 = bx * 16;
  const int n0 = by * 16 * TB4;
  const uint16_t* __restrict__ W = (const uint16_t*)a.w_dkr;
  const uint16_t* __restrict__ H = (const uint16_t*)a.h;
  const int D = a.D, nchunk = D / 64;
  const int per = (nchunk + NWV - 1) / NWV;
  const int cbeg = w * per, cend = min(nchunk, cbeg + per);
  const int lrow = lane >> 3, lpc = lane & 7;  // loader: rows lrow + 8 i, 16-byte piece lpc
  const int m = lane & 15, q = lane >> 4;      // fragment: row m, k group q

  long long slot[TB4];
  int pos[TB4];

  f32x4 acc[TB4];
#pragma unroll
  for (int t = 0; t < TB4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // 32-bit byte offsets of this lane's rows from W_DKR and from the
  // work-group's h block
  const char* __restrict__ Wb = (const char*)W;
  const char* __restrict__ Hb = (const char*)H + (size_t)n0 * D * 2;
  uint32_t roff[ROWS / 8];
  bool rvalid[ROWS / 8];
#pragma unroll
  for (int i = 0; i < ROWS / 8; ++i) {
    const int row = lrow + 8 * i;
    if (row < 16) {
      roff[i] = (uint32_t)((r0 + row) * D * 2 + 16 * lpc);
      rvalid[i] = true;
    } else {
      roff[i] = (uint32_t)((row - 16) * D * 2 + 16 * lpc);
      rvalid[i] = n0 + row - 16 < a.n_tokens;
    }
  }
  for (int c0 = cbeg; c0 < cend; c0 += KB) {
    u32x4 v[KB][ROWS / 8];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const bool ok = c0 + u < cend;
      const uint32_t kb = 128u * (uint32_t)(c0 + u);
#pragma unroll
      for (int i = 0; i < ROWS / 8; ++i) {
        const int row = lrow + 8 * i;
        const char* base = row < 16 ? Wb : Hb;
        v[u][i] = (ok && rvalid[i]) ? *(const u32x4*)(base + (roff[i] + kb)) : u32x4{0, 0, 0, 0};
      }
    }
    if (c0 == cbeg) {
      // slot and position of the epilogue's token, in flight with the first
      // batch (unconditional loads from a clamped index; -1 marks no store)
#pragma unroll
      for (int t = 0; t < TB4; ++t) {
        const int n = n0 + 16 * t + m;
        const int nc = min(n, a.n_tokens - 1);
        const long long sl = a.dense ? (long long)nc : a.slots[nc];
        pos[t] = a.positions[nc];
        slot[t] = ((t % NWV) == w && n < a.n_tokens) ? checked_slot(sl, a.num_pages, a.P, a.err) : -1;
      }
    }
    // the slices are private to the wave and LDS operations of one wave
    // complete in order, so fragment reads see the stores before them and
    // precede the store that reuses their slice, without a barrier
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (c0 + u >= cend) break;
      uint16_t* sl_base = stage[w][u % NSL];
#pragma unroll
      for (int i = 0; i < ROWS / 8; ++i) {
        const int row = lrow + 8 * i;
        *(u32x4*)(sl_base + row * 64 + 8 * (lpc ^ (row & 7))) = v[u][i];
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int sl = (4 * kk + q) ^ (m & 7);
        const u32x4 av = *(const u32x4*)(sl_base + m * 64 + 8 * sl);
#pragma unroll
        for (int t = 0; t < TB4; ++t) {
          const u32x4 bv = *(const u32x4*)(sl_base + (16 + 16 * t + m) * 64 + 8 * sl);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc[t], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TB4; ++t) part[w][t][lane] = acc[t];
  __syncthreads();
  // rotary frequencies of this lane's two feature pairs (k_R rows only)
  double th[2] = {0.0, 0.0};
  if (r0 + 4 * (lane >> 4) >= a.d_c) {
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) th[pr] = rope_inv_freq((r0 + 4 * (lane >> 4) - a.d_c) / 2 + pr, a.d_r, a.rope_base);
  }
  // epilogue: waves take token sub-blocks; fixed summation order over waves
#pragma unroll
  for (int t = 0; t < TB4; ++t) {
    if ((t % NWV) != w || slot[t] < 0) continue;
    f32x4 v = part[0][t][lane];
#pragma unroll
    for (int k = 1; k < NWV; ++k) v += part[k][t][lane];
    // D: lane holds token n = lane % 16, features 4 (lane / 16) + j
    const int rf = r0 + 4 * (lane >> 4);
    float o[4] = {v[0], v[1], v[2], v[3]};
    if (rf >= a.d_c) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        float c, s;
        rope_cs_theta(pos[t], th[pr], c, s);
        const float x0 = o[2 * pr], x1 = o[2 * pr + 1];
        o[2 * pr] = x0 * c - x1 * s;
        o[2 * pr + 1] = x0 * s + x1 * c;
      }
    }
    const uint32_t lo = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
    uint16_t* dst = (uint16_t*)a.pool + (size_t)slot[t] * R + rf;
    *(uint2*)dst = make_uint2(lo, hi);
  }
}

template <int TB4, int NWV, int KB, int NSL>
__global__ void __launch_bounds__(64 * NWV) k_write_mfma(WriteCacheArgs a) {
  __shared__ __attribute__((aligned(16))) WriteLds<TB4, NWV, NSL> lds;
  write_tile<TB4, NWV, KB, NSL>(a, blockIdx.x, blockIdx.y, lds);
}

// Cache write for many tokens (a prefill chunk): one work-group per (128
// tokens, 192 cached features) with the whole hidden axis, so each h row is
// fetched by the R / 192 work-groups of its token block only, and those run
// on one XCD at the same time (its L2 serves the other fetches).  64-wide
// k chunks of the 192 W rows and 128 h rows pass through two LDS stages by
// direct-to-LDS loads (128-byte rows, 16-byte piece c at slot
// c ^ ((row / 2) % 8)).  The products are D^T: wave (wf, wt) holds features
// 96 wf .. +95 against tokens 64 wt .. +63, each lane four consecutive
// features of one token per accumulator group, so the rotary pairs of the
// k_R branch are rotated in registers and stored as one 8-byte group.
constexpr int WB_T = 128, WB_F = 192, WB_K = 64;
constexpr int WB_STAGE = (WB_F + WB_T) * WB_K * 2;  // 40 KiB
constexpr int WB_LPW = (WB_F + WB_T) / 8 / 4;       // loads per wave per stage (10)

__device__ __forceinline__ int wb_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

__global__ void __launch_bounds__(256, 2) k_write_big(WriteCacheArgs a, int n_fb) {
  __shared__ __attribute__((aligned(16))) char smem[2 * WB_STAGE];
  // work-group i runs on XCD i % 8: the n_fb feature blocks of a token block
  // take consecutive slots of one XCD
  const int id = blockIdx.x, xcd = id & 7, sl = id >> 3;
  const int tb_blk = (sl / n_fb) * 8 + xcd, fblk = sl % n_fb;
  const int n0 = tb_blk * WB_T, r0 = fblk * WB_F;
  if (n0 >= a.n_tokens) return;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int wf = w >> 1, wt = w & 1;
  const int N = a.n_tokens, D = a.D, R = a.d_c + a.d_r;
  const char* __restrict__ Wb = (const char*)a.w_dkr + (size_t)r0 * D * 2;
  const char* __restrict__ Hb = (const char*)a.h + (size_t)n0 * D * 2;
  const uint32_t lds0 = lds_addr_of(smem);

  // loads: instruction u (0..39) of a stage fills LDS bytes [1024 u, +1024):
  // stage rows 8 u + lane / 8 (rows < 192: W row r0 + row; else h row
  // n0 + row - 192, clamped to the last token), slot lane % 8.  Wave w
  // issues u = w + 4 i.
  uint32_t voff[WB_LPW];
#pragma unroll
  for (int i = 0; i < WB_LPW; ++i) {
    const int u = w + 4 * i, r = 8 * u + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int row = r < WB_F ? r : min(r - WB_F, N - 1 - n0);
    voff[i] = (uint32_t)(row * D * 2 + 16 * c);
  }
  auto issue = [&](int kc, int st) {
    const uint32_t base = lds0 + st * WB_STAGE;
#pragma unroll
    for (int i = 0; i < WB_LPW; ++i) {
      const int u = w + 4 * i;
      dma16<0>((8 * u < WB_F ? Wb : Hb) + 128 * kc, voff[i], base + 1024 * u);
    }
  };

  f32x16 acc[3][2];
#pragma unroll
  for (int fb = 0; fb < 3; ++fb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) acc[fb][tb] = f32x16{};
  const int nk = D / WB_K;
  issue(0, 0);
  for (int kc = 0; kc < nk; ++kc) {
    if (kc + 1 < nk) {
      issue(kc + 1, (kc + 1) & 1);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(WB_LPW));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* st = smem + (kc & 1) * WB_STAGE;
#pragma unroll
    for (int ks = 0; ks < WB_K / 16; ++ks) {
      const int c = 2 * ks + g;
      u32x4 bv[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int rb = WB_F + 64 * wt + 32 * tb + r32;  // B column: token
        bv[tb] = *(const u32x4*)(st + rb * 128 + 16 * wb_slot(rb, c));
      }
#pragma unroll
      for (int fb = 0; fb < 3; ++fb) {
        const int ra = 96 * wf + 32 * fb + r32;  // A row: feature
        const u32x4 av = *(const u32x4*)(st + ra * 128 + 16 * wb_slot(ra, c));
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bv[tb]), acc[fb][tb], 0, 0, 0);
      }
    }
    __syncthreads();  // the stage is free for the load two chunks on
  }

  // D^T[feature][token]: lane holds token 64 wt + 32 tb + lane % 32 and
  // features 96 wf + 32 fb + 8 (e/4) + 4 g + e % 4
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int n = n0 + 64 * wt + 32 * tb + r32;
    if (n >= N) continue;
    const long long slot = a.dense ? (long long)n : checked_slot(a.slots[n], a.num_pages, a.P, a.err);
    if (slot < 0) continue;
    const int pos = a.positions[n];
    uint16_t* dst = (uint16_t*)a.pool + (size_t)slot * R;
#pragma unroll
    for (int fb = 0; fb < 3; ++fb)
#pragma unroll
      for (int eg = 0; eg < 4; ++eg) {
        const int f0 = r0 + 96 * wf + 32 * fb + 8 * eg + 4 * g;
        float o[4] = {acc[fb][tb][4 * eg], acc[fb][tb][4 * eg + 1], acc[fb][tb][4 * eg + 2], acc[fb][tb][4 * eg + 3]};
        if (f0 >= a.d_c) {
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            float c, sn;
            rope_cs_theta(pos, rope_inv_freq((f0 - a.d_c) / 2 + pr, a.d_r, a.rope_base), c, sn);
            const float x0 = o[2 * pr], x1 = o[2 * pr + 1];
            o[2 * pr] = x0 * c - x1 * sn;
            o[2 * pr + 1] = x0 * sn + x1 * c;
          }
        }
        *(uint2*)(dst + f0) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      }
  }
}

// ---------------------------------------------------------------- absorption
constexpr int AB_C = 128;  // latent columns per work-group
constexpr int AB_T = 64;   // tokens per work-group
constexpr int AB_DR = 64;  // rotary width on this path

// LDS: W_UK,h column block (d_n rows x 256 bytes), the q_C block (64 tokens x
// d_n) and the output tile (64 tokens x 128 columns).  q and the output move
// between HBM and LDS in whole rows (16 lanes x 16 bytes per 256-byte row
// segment); the MFMA fragments are LDS reads.
template <int DN>
__global__ void __launch_bounds__(256) k_absorb_mfma(AbsorbArgs a) {
  constexpr int KMAX = DN / 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int dn = DN;
  char* wtile = smem;                          // dn x 256 B, chunk slot ch ^ 2 (j % 4)
  char* qtile = smem + dn * 256;               // 64 x (2 dn) B, piece p at slot p ^ (row % 8)
  char* otile = qtile + AB_T * 2 * dn;         // 64 x 256 B, piece p at slot p ^ (row % 8)
  const int h = blockIdx.x, cb = blockIdx.y, n0 = blockIdx.z * AB_T;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int H = a.H, dc = a.d_c, dq = a.d_n + a.d_r, R = a.d_c + a.d_r;
  constexpr int qp_row = DN / 8;  // 16-byte pieces per q_C row
  const uint16_t* __restrict__ wuk = (const uint16_t*)a.w_uk + (size_t)h * dn * dc + cb * AB_C;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
  uint16_t* __restrict__ out = (uint16_t*)a.q_abs;

  // loads, in this order: the rotary inputs (column-block-0 work-groups: 8
  // (token, pair) units per thread), then the W_UK block and the q_C block
  // (8 + 4 chunks per thread at d_n = 128).  vmcnt retires loads in issue
  // order, so the rotation can run while the staging loads are in flight.  q
  // rows past the last token are clamped and zeroed at the LDS store; no load
  // sits behind a branch.
  constexpr int np = AB_DR / 2;
  static_assert(AB_T * np == 8 * 256, "one batch of rotary units");
  uint32_t pr[8];
  int ps[8];
  if (cb == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int u = 256 * k + tid;
      const int nn = min(n0 + u / np, a.n_tokens - 1), i = u % np;
      pr[k] = *(const uint32_t*)(Q + ((size_t)nn * H + h) * dq + dn + 2 * i);
      ps[k] = a.positions[nn];
    }
  }
  constexpr int NWC = DN * (AB_C / 8) / 256, NQC = AB_T * (DN / 8) / 256;
  static_assert(DN * (AB_C / 8) % 256 == 0 && AB_T * (DN / 8) % 256 == 0, "whole chunks per thread");
  u32x4 wv[NWC], qv[NQC];
#pragma unroll
  for (int k = 0; k < NWC; ++k) {
    const int u = k * 256 + tid, j = u >> 4, ch = u & 15;
    wv[k] = *(const u32x4*)(wuk + (size_t)j * dc + 8 * ch);
  }
#pragma unroll
  for (int k = 0; k < NQC; ++k) {
    const int u = k * 256 + tid, t = u / qp_row, pc = u % qp_row;
    qv[k] = *(const u32x4*)(Q + ((size_t)min(n0 + t, a.n_tokens - 1) * H + h) * dq + 8 * pc);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the rotation starts
  if (cb == 0) {
    static_assert(256 % np == 0, "pair index fixed per thread");
    const double th = rope_inv_freq(tid % np, AB_DR, a.rope_base);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int u = 256 * k + tid;
      const int nn = n0 + u / np, i = u % np;
      if (nn >= a.n_tokens) continue;
      float c, s;
      rope_cs_theta(ps[k], th, c, s);
      const float x0 = __uint_as_float(pr[k] << 16), x1 = __uint_as_float(pr[k] & 0xffff0000u);
      const uint32_t o = (uint32_t)f32_to_bf16(x0 * c - x1 * s) | ((uint32_t)f32_to_bf16(x0 * s + x1 * c) << 16);
      *(uint32_t*)(out + ((size_t)nn * H + h) * R + dc + 2 * i) = o;
    }
  }
#pragma unroll
  for (int k = 0; k < NWC; ++k) {
    const int u = k * 256 + tid, j = u >> 4, ch = u & 15;
    *(u32x4*)(wtile + j * 256 + 16 * (ch ^ (2 * (j & 3)))) = wv[k];
  }
#pragma unroll
  for (int k = 0; k < NQC; ++k) {
    const int u = k * 256 + tid, t = u / qp_row, pc = u % qp_row;
    *(u32x4*)(qtile + t * 2 * dn + 16 * (pc ^ (t & 7))) = (n0 + t < a.n_tokens) ? qv[k] : u32x4{0, 0, 0, 0};
  }
  __syncthreads();

  const int g = lane >> 5, r = lane & 31;
  const int grp = lane >> 4, jl = lane & 15;
  // B operand (W^T fragment): lane gets W[k0 .. k0+3][col], col = 32 w + lane % 32
  const int tcol = 32 * w + 16 * (grp & 1) + 4 * (jl & 3);  // first column of the lane's 8-byte load
#pragma unroll
  for (int tb = 0; tb < AB_T / 32; ++tb) {
    const int trow = 32 * tb + r;  // A operand: token row = lane % 32
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KMAX; ++ks) {
      if (ks >= dn / 16) continue;
      const int pc = 2 * ks + g;
      const u32x4 av = *(const u32x4*)(qtile + trow * 2 * dn + 16 * (pc ^ (trow & 7)));
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
    const int col = 32 * w + r;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = 32 * tb + 8 * (j >> 2) + 4 * g + (j & 3);
      *(uint16_t*)(otile + t * 256 + 16 * ((col >> 3) ^ (t & 7)) + 2 * (col & 7)) = f32_to_bf16(acc[j]);
    }
  }
  __syncthreads();
  // output tile to HBM in whole 256-byte row segments
#pragma unroll
  for (int k = 0; k < AB_T * 16 / 256; ++k) {
    const int u = k * 256 + tid, t = u >> 4, pc = u & 15;
    const int n = n0 + t;
    if (n < a.n_tokens)
      *(u32x4*)(out + ((size_t)n * H + h) * R + cb * AB_C + 8 * pc) =
          *(const u32x4*)(otile + t * 256 + 16 * (pc ^ (t & 7)));
  }
}

// ---------------------------------------------------------------- write + absorption, one launch
// A decode step's cache write and absorption each leave most CUs idle and do
// not depend on each other.  k_write_absorb runs both in one grid of
// 1024-thread work-groups: the first nfb * S are split-K tiles of the cache
// write, the rest each take whole heads of the absorption (d_n = 128,
// d_c = 512, at most 64 tokens).
//
// Cache write, split over the hidden axis: work-group (fb, s) computes
// features 64 fb .. +63 against every token (at most 64) over hidden chunks
// [s nchunk / S, (s + 1) nchunk / S) of 64.  The W and h rows of its chunks
// arrive by direct-to-LDS loads in one batch (at most WS_MAXC chunks of
// 128 rows x 128 bytes, 16-byte piece p of row r at slot p ^ (r % 8)), so a
// work-group waits for memory once; a tile that covers the whole hidden axis
// instead moves its bytes through one CU in several dependent rounds.  Wave w
// computes features 16 (w % 4) .. +15 x tokens 16 (w / 4) .. +15 (16x16x32
// MFMA, chunks in order) and stores that fp32 partial.  A device-scope
// counter per feature block elects the block's last work-group to finish; it
// adds the S partials in slice order (a fixed order: the rows do not depend
// on which work-group finishes last), rotates the k_R pairs and stores the
// bf16 rows to their slots, and returns the counter to zero.
//
// Absorption: for a head, sub-group s (threads 256 s .. +255, four waves)
// computes latent columns 128 s .. +127 exactly as one k_absorb_mfma
// work-group does (same operands, same k order, so the results are
// bit-identical); the q_C block is staged once for the four, and each
// sub-group's W_UK column block is overwritten by its output tile once every
// wave has finished reading it.
constexpr int WA_WBLK = 32768;                 // one W_UK column block: 128 rows x 256 bytes
constexpr int WA_LDS = 4 * WA_WBLK + AB_T * 256;  // + the q_C block: 147456 bytes
constexpr int WS_MAXC = 8;                     // hidden chunks of 64 per split-K tile (16 KiB of LDS each)
constexpr int WS_MAXS = 16;                    // split-K slices
constexpr int WS_PART = 64 * 64;               // floats of one tile's partial: [64 tokens][64 features]
static_assert(WS_MAXC * 16384 <= WA_LDS, "split-K tile fits the fused kernel's LDS");

// buffer resource word 3 for raw 32-bit accesses, and the sc1 cache-policy
// bit of buffer loads and stores (device-coherent across the XCDs' L2 caches)
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCoherent = 16;

struct WriteSplit {
  int S, nfb;     // slices of the hidden axis, 64-feature blocks (R / 64)
  int* counters;  // [nfb], zero between calls
  float* part;    // [S][nfb][WS_PART]
};

__device__ __forceinline__ void write_split_tile(const WriteCacheArgs& a, const WriteSplit& ws, int fb, int s,
                                                 char* smem) {
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int D = a.D, nchunk = D / 64;
  const int c0 = s * nchunk / ws.S, nc = (s + 1) * nchunk / ws.S - c0;  // nc <= WS_MAXC
  // wave w loads rows 8 w .. 8 w + 7 of every chunk: waves 0-7 W rows
  // 64 fb + 8 w + l / 8, waves 8-15 h rows (tokens past the last repeat it;
  // their products are not stored); lane l fills slot l % 8 with source piece
  // (l % 8) ^ (row % 8)
  {
    const int row = 8 * w + (lane >> 3), piece = (lane & 7) ^ (row & 7);
    const char* src = w < 8 ? (const char*)a.w_dkr + ((size_t)(64 * fb + row) * D + 64 * c0 + 8 * piece) * 2
                            : (const char*)a.h + ((size_t)min(row - 64, a.n_tokens - 1) * D + 64 * c0 + 8 * piece) * 2;
    const uint32_t lds = lds_addr_of(smem) + 1024 * w;
#pragma unroll
    for (int i = 0; i < WS_MAXC; ++i)
      if (i < nc) dma16_v(src + 128 * i, lds + 16384 * i);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  asm volatile("" ::: "memory");
  const int m = lane & 15, q = lane >> 4;
  const int fw = w & 3, tw = w >> 2;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < WS_MAXC; ++i) {
    if (i >= nc) break;
    const char* cb = smem + 16384 * i;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int sl = (4 * kk + q) ^ (m & 7);
      const u32x4 av = *(const u32x4*)(cb + (16 * fw + m) * 128 + 16 * sl);
      const u32x4 bv = *(const u32x4*)(cb + (64 + 16 * tw + m) * 128 + 16 * sl);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc, 0, 0, 0);
    }
  }
  // D: lane holds token 16 tw + m, features 16 fw + 4 q + j.  The partial
  // goes out as device-coherent stores (written through to the level every
  // XCD reads), and every wave waits for them before the work-group counts
  // its slice in: the reducer's device-coherent loads then see them.  No
  // cache-wide write-back or invalidation is needed (nothing else of this
  // exchange passes through the per-XCD L2 caches).
  // (16-byte buffer accesses with the sc1 cache policy, the device-coherent
  // form; the resource covers exactly the partials)
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      ws.part, (short)0, ws.S * ws.nfb * WS_PART * (int)sizeof(float), kBufferRsrcWord3);
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(u32x4, acc), prs,
      (int)sizeof(float) * ((s * ws.nfb + fb) * WS_PART + (16 * tw + m) * 64 + 16 * fw + 4 * q), 0, kCoherent);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  if (tid == 0) {
    const int last = atomicAdd(ws.counters + fb, 1) == ws.S - 1;
    if (last) atomicExch(ws.counters + fb, 0);  // every slice has counted: ready for the next call
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  const int t = tid >> 4, f4 = tid & 15;
  if (t >= a.n_tokens) return;
  const int pb = (int)sizeof(float) * (fb * WS_PART + t * 64 + 4 * f4);
  // all WS_MAXS loads in flight at once: slices k >= S lie past the end of
  // the resource, where buffer loads return zero (and their values are not used)
  f32x4 pv[WS_MAXS];
#pragma unroll
  for (int k = 0; k < WS_MAXS; ++k)
    pv[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          prs, pb + (int)sizeof(float) * k * ws.nfb * WS_PART, 0, kCoherent));
  const long long sl = a.dense ? (long long)t : a.slots[t];
  const int pos = a.positions[t];
  f32x4 v = pv[0];
#pragma unroll
  for (int k = 1; k < WS_MAXS; ++k) {
    const f32x4 sum = v + pv[k];
    v = k < ws.S ? sum : v;
  }
  const long long slot = checked_slot(sl, a.num_pages, a.P, a.err);
  if (slot < 0) return;
  const int R = a.d_c + a.d_r, rf = 64 * fb + 4 * f4;
  float o[4] = {v[0], v[1], v[2], v[3]};
  if (rf >= a.d_c) {
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      float c, sn;
      rope_cs_theta(pos, rope_inv_freq((rf - a.d_c) / 2 + pr, a.d_r, a.rope_base), c, sn);
      const float x0 = o[2 * pr], x1 = o[2 * pr + 1];
      o[2 * pr] = x0 * c - x1 * sn;
      o[2 * pr + 1] = x0 * sn + x1 * c;
    }
  }
  const uint32_t lo = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
  *(uint2*)((uint16_t*)a.pool + (size_t)slot * R + rf) = make_uint2(lo, hi);
}

__device__ __forceinline__ void absorb_head16(const AbsorbArgs& a, int h, char* smem) {
  constexpr int DN = 128, NP = AB_DR / 2;
  const int tid = threadIdx.x, ts = tid & 255, lane = tid & 63;
  const int wv16 = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave within the work-group (uniform)
  const int sg = wv16 >> 2, ws = wv16 & 3;                     // sub-group, wave within it
  const int H = a.H, dc = a.d_c, dq = a.d_n + a.d_r, R = a.d_c + a.d_r;
  const int cb = sg;
  char* wtile = smem + cb * WA_WBLK;  // W_UK column block, later the output tile
  char* qtile = smem + 4 * WA_WBLK;   // 64 x 256 B, piece p at slot p ^ (row % 8)
  const uint16_t* __restrict__ wuk = (const uint16_t*)a.w_uk + (size_t)h * DN * dc + cb * AB_C;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
  uint16_t* __restrict__ out = (uint16_t*)a.q_abs;
  // loads, in this order: the rotary inputs (sub-group 0), then the W_UK
  // block and the q_C block straight into LDS (vmcnt retires in issue order,
  // so the rotation waits only for its own loads).  Direct-to-LDS load i of a
  // sub-group fills rows 4 i .. 4 i + 3 of its W block (lane l: row
  // 4 i + l / 16, slot l % 16, whose source chunk is slot ^ 2 (row % 4)); load
  // w16 of the work-group fills q_C rows 4 w16 .. +3 (slot l % 16, source
  // piece slot ^ (row % 8); rows past the last token repeat it: their outputs
  // are not stored).
  constexpr int RK = AB_T * NP / 1024;  // rotary units per thread (2): every thread takes part
  uint32_t pr[RK];
  int ps[RK];
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    const int u = 1024 * k + tid;
    const int nn = min(u / NP, a.n_tokens - 1), i = u % NP;
    pr[k] = *(const uint32_t*)(Q + ((size_t)nn * H + h) * dq + DN + 2 * i);
    ps[k] = a.positions[nn];
  }
  const uint32_t lds_w = lds_addr_of(wtile), lds_q = lds_addr_of(qtile);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = 4 * k + ws;  // this wave's load k of the sub-group's 32
    const int j = 4 * i + (lane >> 4), slot = lane & 15;
    dma16_v(wuk + (size_t)j * dc + 8 * (slot ^ (2 * (j & 3))), lds_w + 1024 * i);
  }
  {
    const int t = 4 * wv16 + (lane >> 4), slot = lane & 15;
    dma16_v(Q + ((size_t)min(t, a.n_tokens - 1) * H + h) * dq + 8 * (slot ^ (t & 7)), lds_q + 1024 * wv16);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));  // the rotary inputs (the 9 loads into LDS may remain)
  {
    static_assert(1024 % NP == 0, "pair index fixed per thread");
    const double th = rope_inv_freq(tid % NP, AB_DR, a.rope_base);
#pragma unroll
    for (int k = 0; k < RK; ++k) {
      const int u = 1024 * k + tid;
      const int nn = u / NP, i = u % NP;
      if (nn >= a.n_tokens) continue;
      float c, sn;
      rope_cs_theta(ps[k], th, c, sn);
      const float x0 = __uint_as_float(pr[k] << 16), x1 = __uint_as_float(pr[k] & 0xffff0000u);
      const uint32_t o = (uint32_t)f32_to_bf16(x0 * c - x1 * sn) | ((uint32_t)f32_to_bf16(x0 * sn + x1 * c) << 16);
      *(uint32_t*)(out + ((size_t)nn * H + h) * R + dc + 2 * i) = o;
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();  // W_UK blocks and the q_C block are in LDS
  asm volatile("" ::: "memory");

  const int g = lane >> 5, r = lane & 31;
  const int grp = lane >> 4, jl = lane & 15;
  const int tcol = 32 * ws + 16 * (grp & 1) + 4 * (jl & 3);
  // k-steps outer: each W_UK^T fragment (two transpose reads) serves both
  // 32-token blocks, and the unrolled loop lets the LDS reads run ahead of
  // the MFMAs (same operands and k order as before, so the same bits)
  f32x16 acc[AB_T / 32];
#pragma unroll
  for (int tb = 0; tb < AB_T / 32; ++tb) acc[tb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < DN / 16; ++ks) {
    const int pc = 2 * ks + g;
    const int k0 = 16 * ks + 8 * g;
    const int j1 = k0 + (jl >> 2), j2 = j1 + 4;
    const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(wtile + j1 * 256 + 16 * ((tcol >> 3) ^ (2 * (j1 & 3))) + 2 * (tcol & 7)));
    const s16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(wtile + j2 * 256 + 16 * ((tcol >> 3) ^ (2 * (j2 & 3))) + 2 * (tcol & 7)));
    const s16x8 bv = s16x8{b1[0], b1[1], b1[2], b1[3], b2[0], b2[1], b2[2], b2[3]};
#pragma unroll
    for (int tb = 0; tb < AB_T / 32; ++tb) {
      const int trow = 32 * tb + r;
      const u32x4 av = *(const u32x4*)(qtile + trow * 256 + 16 * (pc ^ (trow & 7)));
      acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), __builtin_bit_cast(bf16x8, bv), acc[tb], 0, 0,
                                                        0);
    }
  }
  __syncthreads();  // every wave has read its W_UK block: it becomes the output tile
  char* otile = wtile;  // 64 x 256 B, piece p at slot p ^ (row % 8)
  const int col = 32 * ws + r;
#pragma unroll
  for (int tb = 0; tb < AB_T / 32; ++tb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = 32 * tb + 8 * (j >> 2) + 4 * g + (j & 3);
      *(uint16_t*)(otile + t * 256 + 16 * ((col >> 3) ^ (t & 7)) + 2 * (col & 7)) = f32_to_bf16(acc[tb][j]);
    }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < AB_T * 16 / 256; ++k) {
    const int u = k * 256 + ts, t = u >> 4, pc = u & 15;
    if (t < a.n_tokens)
      *(u32x4*)(out + ((size_t)t * H + h) * R + cb * AB_C + 8 * pc) = *(const u32x4*)(otile + t * 256 + 16 * (pc ^ (t & 7)));
  }
}

// Work-group roles as wa_role (mla_checks.h) deals them: split-K write
// tiles grouped by XCD, then absorption heads rank, rank + n_ablocks, ...
__global__ void __launch_bounds__(1024, 1) k_write_absorb(WriteCacheArgs wa, AbsorbArgs aa, WriteSplit ws,
                                                          int n_ablocks) {
  __shared__ __attribute__((aligned(16))) char smem[WA_LDS];
  const WaRole role = wa_role(blockIdx.x, ws.S, ws.nfb);
  if (role.write) {
    write_split_tile(wa, ws, role.fb, role.s, smem);
    return;
  }
  const int rank = role.rank;
  for (int h = rank; h < aa.H; h += n_ablocks) {
    absorb_head16(aa, h, smem);
    __syncthreads();  // the next head reuses the LDS
  }
}

}  // namespace

static int write_split_slices(int D) { return (D / 64 + WS_MAXC - 1) / WS_MAXC; }

bool write_absorb_fused_supported(int n_write, int D, int d_c, int d_r) {
  const int R = d_c + d_r;
  return n_write >= 1 && n_write <= 64 && D % 64 == 0 && D >= 64 && write_split_slices(D) <= WS_MAXS && R % 64 == 0 &&
         R / 64 <= 64 && d_c == 4 * AB_C && d_r % 2 == 0;
}

bool write_absorb_absorb_supported(int n_q, int H, int d_n, int d_c, int d_r) {
  return n_q >= 1 && n_q <= AB_T && absorb_mfma_supported(H, d_n, d_c, d_r) && d_n == 128 && d_c == 4 * AB_C;
}

size_t write_absorb_ws_bytes(int D, int d_c, int d_r) {
  return 256 + (size_t)write_split_slices(D) * ((d_c + d_r) / 64) * WS_PART * sizeof(float);
}

hipError_t write_absorb_mfma(const WriteCacheArgs& wa, const AbsorbArgs& aa, void* workspace, int cus, hipStream_t s) {
  WriteSplit ws;
  ws.S = write_split_slices(wa.D);
  ws.nfb = (wa.d_c + wa.d_r) / 64;
  ws.counters = (int*)workspace;
  ws.part = (float*)((char*)workspace + 256);
  const int n_wblocks = ws.nfb * ws.S;
  int n_ablocks = cus - n_wblocks;
  if (n_ablocks > aa.H) n_ablocks = aa.H;
  if (n_ablocks < (aa.H + 1) / 2) n_ablocks = (aa.H + 1) / 2;  // at most two heads per work-group
  const int grid = wa_grid(ws.S, ws.nfb, n_ablocks);
  hipLaunchKernelGGL(k_write_absorb, dim3(grid), dim3(1024), 0, s, wa, aa, ws, n_ablocks);
  return hipGetLastError();
}

bool write_mfma_supported(int D, int d_c, int d_r) { return D % 64 == 0 && d_c % 16 == 0 && d_r % 16 == 0; }

hipError_t write_cache_mfma(const WriteCacheArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  const int R = a.d_c + a.d_r;
  // few tokens (decode): W_DKR dominates the bytes, so 16 waves per work-group
  // split the hidden axis, fetching their chunks in batches of 4 (two round
  // trips at D = 7168); many tokens: 4 token blocks per work-group reuse each W
  // fragment 4 times
  if (a.n_tokens >= 4096 && R % WB_F == 0 && a.D % WB_K == 0) {
    // many tokens: whole-hidden-axis tiles (the grid covers 8 token blocks per
    // XCD round; blocks past the last token return at once)
    const int n_fb = R / WB_F, n_tb = (a.n_tokens + WB_T - 1) / WB_T;
    hipLaunchKernelGGL(k_write_big, dim3(((n_tb + 7) / 8) * 8 * n_fb), dim3(256), 0, s, a, n_fb);
  } else if (a.n_tokens <= 1024) {
    hipLaunchKernelGGL((k_write_mfma<1, 16, 4, 2>), dim3(R / 16, (a.n_tokens + 15) / 16), dim3(1024), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_write_mfma<4, 4, 2, 2>), dim3(R / 16, (a.n_tokens + 63) / 64), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

bool absorb_mfma_supported(int H, int d_n, int d_c, int d_r) {
  return d_n % 64 == 0 && d_n <= 128 && d_c % AB_C == 0 && d_r == AB_DR && H >= 1;
}

hipError_t absorb_mfma(const AbsorbArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  const dim3 grid(a.H, a.d_c / AB_C, (a.n_tokens + AB_T - 1) / AB_T);
  const size_t lds = (size_t)a.d_n * 256 + (size_t)AB_T * 2 * a.d_n + (size_t)AB_T * 256;
  if (a.d_n == 128)
    hipLaunchKernelGGL(k_absorb_mfma<128>, grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL(k_absorb_mfma<64>, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace mla
