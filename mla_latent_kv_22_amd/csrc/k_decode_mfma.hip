// Split-T flash-decoding over the latent cache with matrix absorption, MFMA
// kernels for gfx950 (bf16 storage, latent width 512, rotary key width 64).
//
// Pass 1 (split): one work-group per work item = (sequence, token range).
// Its NW = ceil(H/32) waves each own 32 heads.  Cache rows stream
// HBM -> LDS once per item, 32 tokens per tile, three tiles in flight, with
// direct global->LDS loads; every wave then reads the tile twice from LDS:
//   scores  S^T[t][h] = row_t . q~_h          (MFMA 32x32x16, k = 576 features)
//   latent  O^T[f][h] += C^T[f][t] P^T[t][h]  (MFMA 32x32x16, k = 32 tokens)
// The C^T operand comes straight from the row-major tile through the LDS
// transpose read (ds_read_b64_tr_b16), so no transposed copy is staged.  The
// softmax is online with a lazily moved reference maximum: the accumulator is
// rescaled only when a head's running maximum grows by more than 8 (log2
// units), which keeps every exp2 below 256 and leaves the result exact.
// Pass 2 (combine): per (head, 32 sequences): LSE-merge of the items in a
// fixed order, the merged latent split into bf16 hi + lo parts, and W_UV
// applied with MFMA (so the fp32 latent reaches the product intact to ~2^-17).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int DC = 512;            // latent width
constexpr int DR = 64;             // rotary key width
constexpr int RW = DC + DR;        // cached row width (576 values, 1152 bytes)
constexpr int TT = 32;             // tokens per tile
constexpr int TILE_CHUNKS = TT * RW * 2 / 16;  // 2304 16-byte chunks
constexpr int TILE_BYTES = TILE_CHUNKS * 16;  // 36864
constexpr int LOADS_PER_TILE = TILE_CHUNKS / 64;  // 36 wave-wide 16-byte loads
constexpr int KS = RW / 16;        // 36 k-steps of the score MFMA
constexpr int FB = DC / 32;        // 16 f-blocks of the latent accumulator
constexpr float kLazy = 8.f;       // rescale threshold, log2 units

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Tile layout in LDS (36864 bytes per 32-token tile): the row is cut into 9
// column groups of 8 16-byte chunks; group cg holds 32 rows x 128 bytes, and
// inside a row the chunk slot is XOR-swizzled by the row:
//   byte(r, c) = 4096 * (c >> 3) + 128 * r + 16 * ((c & 7) ^ swz(r))
// swz takes all 8 values over any 8 aligned rows and distinct values of
// swz >> 1 over any 4 aligned rows (conflict-free 16-byte score reads of one
// chunk column, conflict-free 8-byte transpose reads); bit 3 of the row flips
// bit 1 so that rows r and r + 8 also differ.
__device__ __forceinline__ int swz(int r) { return (((r & 3) << 1) | ((r >> 2) & 1)) ^ ((r >> 2) & 2); }

__device__ __forceinline__ constexpr int waitcnt_vm(int n) {
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Wave-wide load i (0..35) of a tile fills LDS bytes [1024 i, 1024 i + 1024):
// column group cg = i / 4, rows 8 (i % 4) .. +7.  Lane l takes row
// r = 8 (i % 4) + l / 8 and the chunk whose swizzled slot is l % 8, so its
// global byte offset is lane_off(l, i % 2) + 9216 (i % 4) + 128 (i / 4): the
// swizzle of row r depends on bit 3 of r, which is the parity of i % 4.
__device__ __forceinline__ uint32_t load_lane_off(int lane, int odd) {
  const int r = lane >> 3;
  return (uint32_t)(r * (RW * 2) + (((lane & 7) ^ swz(r + 8 * odd)) << 4));
}

// One wave-wide 16-byte direct-to-LDS load: lane l's 16 bytes at
// sbase + voff land at LDS byte lds_addr + 16 l.  Written as inline asm so the
// compiler does not add its own conservative wait for every load in flight
// before each LDS read; the tile loop waits explicitly (s_waitcnt vmcnt +
// barrier) for exactly the tile it reads.  The instruction writes no VGPR.
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_addr)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr_of(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

template <int NW>
__device__ __forceinline__ void issue_tile(const char* __restrict__ tile_base, int nvalid, char* stage, int w,
                                           int lane, uint32_t lane_off0, uint32_t lane_off1) {
  const uint32_t lds0 = lds_addr_of(stage);
  if (nvalid == TT) {
#pragma unroll
    for (int i0 = 0; i0 < LOADS_PER_TILE; i0 += NW) {
      const int i = i0 + w;
      dma16(tile_base + (9216 * (i & 3) + 128 * (i >> 2)), (i & 1) ? lane_off1 : lane_off0, lds0 + 1024 * i);
    }
  } else {
    // ragged tail: rows past the last valid token repeat it (their p is 0)
#pragma unroll
    for (int i0 = 0; i0 < LOADS_PER_TILE; i0 += NW) {
      const int i = i0 + w;
      const int r = 8 * (i & 3) + (lane >> 3);
      const int rr = r < nvalid ? r : nvalid - 1;
      const int c = 8 * (i >> 2) + ((lane & 7) ^ swz(r));
      dma16(tile_base, (uint32_t)(rr * (RW * 2) + c * 16), lds0 + 1024 * i);
    }
  }
}

// Three stage buffers as separate LDS objects: the compiler can then tell the
// direct-to-LDS loads of one stage from reads of another and waits only for
// the tile being read instead of every load in flight.
template <int NW>
__global__ void __launch_bounds__(NW * 64, 1) k_split(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char tile0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char tile1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char tile2[TILE_BYTES];
  __shared__ int s_len[kMaxDecodeBatch + 1];
  __shared__ int s_items[kMaxDecodeBatch + 1];
  __shared__ int red[16];
  __shared__ int s_pages[kMaxItemPages];

  const int cap = a.len_cap;
  const DecodePlan plan = make_decode_plan(a.seq_lens, a.batch, cap, a.slots, a.min_chunk, kMaxChunk, a.ovh_tokens,
                                           s_len, s_items, red);
  const int n_items = plan.n_items;
  if ((int)blockIdx.x >= n_items) return;
  // consecutive items (same sequence) share an XCD: work-group i runs on XCD i % 8
  int item = blockIdx.x;
  if ((n_items & 7) == 0) item = (blockIdx.x & 7) * (n_items >> 3) + (blockIdx.x >> 3);

  // wave-uniform values read from LDS are moved to scalar registers so that
  // block-table reads and tile addresses stay scalar
  const int b = __builtin_amdgcn_readfirstlane(item_seq(s_items, a.batch, item));
  const int chunk = __builtin_amdgcn_readfirstlane(plan.chunk);
  const int t0 = (item - __builtin_amdgcn_readfirstlane(s_items[b])) * chunk;
  const int t1 = min(__builtin_amdgcn_readfirstlane(s_len[b]), t0 + chunk);
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, hl = lane & 31;
  const int hq = w * 32 + hl;
  const bool hvalid = hq < a.H;

  const char* __restrict__ pool = (const char*)a.pool;
  const int ntiles = (t1 - t0 + TT - 1) / TT;
  const uint32_t lane_off0 = load_lane_off(lane, 0), lane_off1 = load_lane_off(lane, 1);
  const int P = a.P;
  // the item's pages, staged once so the tile loop reads them from LDS
  {
    const int32_t* __restrict__ bt = a.block_table + (size_t)b * a.max_pages_per_seq;
    const int p0 = t0 / P, np = (t1 - 1) / P - p0 + 1;
    for (int i = threadIdx.x; i < np; i += blockDim.x) s_pages[i] = bt[p0 + i];
    __syncthreads();
  }
  const int page0 = t0 / P;

  auto tile_ptr = [&](int tile, int& nvalid) {
    const int tok0 = t0 + tile * TT;
    nvalid = min(TT, t1 - tok0);
    const int page = __builtin_amdgcn_readfirstlane(s_pages[tok0 / P - page0]);
    return pool + ((size_t)page * P + (tok0 % P)) * (RW * 2);
  };

  // prologue: the first two tiles in flight
  if (0 < ntiles) {
    int nv;
    const char* tp = tile_ptr(0, nv);
    issue_tile<NW>(tp, nv, tile0, w, lane, lane_off0, lane_off1);
  }
  if (1 < ntiles) {
    int nv;
    const char* tp = tile_ptr(1, nv);
    issue_tile<NW>(tp, nv, tile1, w, lane, lane_off0, lane_off1);
  }

  // absorbed query fragments: B operand of the score MFMA, k = features
  u32x4 qf[KS];
  {
    const uint16_t* qp = (const uint16_t*)a.q_abs + ((size_t)b * a.H + (hvalid ? hq : 0)) * RW + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = *(const u32x4*)(qp + 16 * ks);
      qf[ks] = hvalid ? v : u32x4{0, 0, 0, 0};
    }
  }

  f32x16 acc[FB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) acc[fb] = f32x16{};
  float m_ref = -INFINITY, lsum = 0.f;

  // per-lane LDS byte offsets of the operand reads (the rest is an immediate)
  int sbase[4];  // score A operand: row = lane % 32, chunk 2 ks + g
  {
    const int sw = swz(hl);
#pragma unroll
    for (int q = 0; q < 4; ++q) sbase[q] = 128 * hl + 16 * ((2 * q + g) ^ sw);
  }
  int tbase[2][2];  // transpose reads: [fb parity][upper 8 rows]
  {
    const int grp = lane >> 4, jl = lane & 15;
    const int trow = 4 * g + (jl >> 2);
    const int tchunk = 2 * (grp & 1) + ((jl >> 1) & 1);
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        tbase[par][hf] = 128 * trow + 16 * ((4 * par + tchunk) ^ swz(trow + 8 * hf)) + 8 * (jl & 1);
  }
  const float sl2 = a.scale_log2;

  // One tile step: `cur` holds tile it, `nxt2` receives tile it + 2.
  auto step = [&](int it, char* cur, char* nxt2) {
    // this wave's loads of tile `it` are done once at most the next tile's remain
    if (it + 1 < ntiles) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS_PER_TILE / NW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    // plain barrier: every wave has waited for its own loads of tile `it`, and
    // every wave is done reading the stage that the next loads overwrite
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (it + 2 < ntiles) {
      int nv;
      const char* tp = tile_ptr(it + 2, nv);
      issue_tile<NW>(tp, nv, nxt2, w, lane, lane_off0, lane_off1);
    }
    const char* tl = cur;
    const int tok0 = t0 + it * TT;

    // ---- scores: S^T[t][h], A = K rows (token = lane%32), B = q~
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 kf = *(const u32x4*)(tl + sbase[ks & 3] + 4096 * (ks >> 2));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[ks]), sacc, 0, 0, 0);
    }

    // ---- online softmax for head hl (this lane and lane^32 share it)
    float s[16];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = 8 * (j >> 2) + 4 * g + (j & 3);
      const float v = sacc[j] * sl2;
      s[j] = (tok0 + t < t1) ? v : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool need = mt > m_ref + kLazy;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mt : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) acc[fb] *= alpha;
      lsum *= alpha;
      m_ref = m_new;
    }
    u32x4 pb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t wds[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[8 * kk + e] - m_ref);
        const float p1 = __builtin_amdgcn_exp2f(s[8 * kk + e + 1] - m_ref);
        const uint16_t b0 = f32_to_bf16(p0), b1 = f32_to_bf16(p1);
        lsum += bf16_to_f32(b0) + bf16_to_f32(b1);
        wds[e >> 1] = (uint32_t)b0 | ((uint32_t)b1 << 16);
      }
      pb[kk] = u32x4{wds[0], wds[1], wds[2], wds[3]};
    }

    // ---- latent: O^T[f][h] += C^T[f][t] P^T[t][h]; A via LDS transpose reads
    //      rows 16 kk + 4 g + j/4 (+8), chunk 4 fb + ..., see tbase
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int imm = 4096 * (fb >> 1) + 128 * 16 * kk;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(tl + tbase[fb & 1][0] + imm));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(tl + tbase[fb & 1][1] + imm + 128 * 8));
        const s16x8 av = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                          as_bf16x8(pb[kk]), acc[fb], 0, 0, 0);
      }
    }
    };

  for (int it = 0; it < ntiles; it += 3) {
    step(it, tile0, tile2);
    if (it + 1 < ntiles) step(it + 1, tile1, tile0);
    if (it + 2 < ntiles) step(it + 2, tile2, tile1);
  }

  lsum += __shfl_xor(lsum, 32);
  if (hvalid) {
    float* pa = a.part_acc + ((size_t)item * a.H + hq) * DC + 4 * g;
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(f32x4*)(pa + 32 * fb + 8 * q4) =
            f32x4{acc[fb][4 * q4], acc[fb][4 * q4 + 1], acc[fb][4 * q4 + 2], acc[fb][4 * q4 + 3]};
    if (g == 0) {
      a.part_ml[((size_t)item * a.H + hq) * 2 + 0] = m_ref;
      a.part_ml[((size_t)item * a.H + hq) * 2 + 1] = lsum;
    }
  }
}

// --------------------------------------------------------------------------
// combine: grid (H, ceil(batch/32)), 256 threads.
constexpr int CB = 32;  // sequences per combine work-group
__global__ void __launch_bounds__(256) k_combine(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lat_hi[CB * DC];
  __shared__ __attribute__((aligned(16))) uint16_t lat_lo[CB * DC];
  __shared__ int s_len[kMaxDecodeBatch + 1];
  __shared__ int s_items[kMaxDecodeBatch + 1];
  __shared__ int red[16];
  __shared__ float s_m[CB], s_invl[CB];

  const int cap = a.len_cap;
  make_decode_plan(a.seq_lens, a.batch, cap, a.slots, a.min_chunk, kMaxChunk, a.ovh_tokens, s_len, s_items, red);
  const int h = blockIdx.x, b0 = blockIdx.y * CB;
  const int tid = threadIdx.x;

  // per-sequence merge statistics (fixed item order)
  if (tid < CB) {
    const int b = b0 + tid;
    float ms = -INFINITY, L = 0.f;
    if (b < a.batch) {
      const int i0 = s_items[b], i1 = s_items[b + 1];
      for (int i = i0; i < i1; ++i) ms = fmaxf(ms, a.part_ml[((size_t)i * a.H + h) * 2]);
      for (int i = i0; i < i1; ++i)
        L += exp2f(a.part_ml[((size_t)i * a.H + h) * 2] - ms) * a.part_ml[((size_t)i * a.H + h) * 2 + 1];
      if (a.lse) a.lse[(size_t)b * a.H + h] = (i1 > i0) ? (ms + log2f(L)) * kLn2 : -INFINITY;
    }
    s_m[tid] = ms;
    s_invl[tid] = (L > 0.f) ? 1.f / L : 0.f;
  }
  __syncthreads();

  // merged latent, split into bf16 hi + lo, stored with a 16-byte-chunk swizzle
  for (int u = tid; u < CB * (DC / 4); u += 256) {
    const int bl = u / (DC / 4), c4 = (u % (DC / 4)) * 4;
    const int b = b0 + bl;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (b < a.batch) {
      const int i0 = s_items[b], i1 = s_items[b + 1];
      const float ms = s_m[bl], invl = s_invl[bl];
      for (int i = i0; i < i1; ++i) {
        const float wgt = exp2f(a.part_ml[((size_t)i * a.H + h) * 2] - ms) * invl;
        v += wgt * *(const f32x4*)(a.part_acc + ((size_t)i * a.H + h) * DC + c4);
      }
    }
    const int chunk = c4 >> 3, within = c4 & 7;
    const int pos = bl * (DC / 8) + (chunk ^ (bl & 7));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t hb = f32_to_bf16(v[e]);
      const uint16_t lb = f32_to_bf16(v[e] - bf16_to_f32(hb));
      lat_hi[pos * 8 + within + e] = hb;
      lat_lo[pos * 8 + within + e] = lb;
    }
  }
  __syncthreads();

  // out[b][h][v] = sum_c lat[b][c] W_UV[h][v][c]: D[b][v], A = lat (b = lane%32), B = W_UV^T
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, r = lane & 31;
  const uint16_t* wuv = (const uint16_t*)a.w_uv + (size_t)h * a.d_v * DC;
  for (int vb = w; vb * 32 < a.d_v; vb += 4) {
    f32x16 acc = f32x16{};
    const uint16_t* wrow = wuv + (size_t)(vb * 32 + r) * DC + 8 * g;
#pragma unroll 4
    for (int ks = 0; ks < DC / 16; ++ks) {
      const u32x4 bw = *(const u32x4*)(wrow + 16 * ks);
      const int pos = r * (DC / 8) + ((2 * ks + g) ^ (r & 7));
      const u32x4 ah = *(const u32x4*)(lat_hi + pos * 8);
      const u32x4 al = *(const u32x4*)(lat_lo + pos * 8);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ah), as_bf16x8(bw), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(al), as_bf16x8(bw), acc, 0, 0, 0);
    }
    const int v = vb * 32 + r;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int bl = 8 * (j >> 2) + 4 * g + (j & 3);
      const int b = b0 + bl;
      if (b < a.batch) ((uint16_t*)a.out)[((size_t)b * a.H + h) * a.d_v + v] = f32_to_bf16(acc[j]);
    }
  }
}

}  // namespace

bool decode_mfma_supported(int H, int d_c, int d_r, int d_v, int P, int batch) {
  return d_c == DC && d_r == DR && H >= 1 && H <= 128 && d_v >= 32 && d_v % 32 == 0 && P >= TT && P % TT == 0 &&
         batch <= kMaxDecodeBatch;
}

int decode_mfma_slots(int H, int cus) {
  // one 4-wave work-group per CU (registers); narrower groups pack 4 waves per CU
  const int nw = (H + 31) / 32;
  return cus * (4 / nw);
}

hipError_t decode_mfma(const DecodeArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const int nw = (a.H + 31) / 32;
  const dim3 g1(a.max_items);
  switch (nw) {
    case 1: hipLaunchKernelGGL(k_split<1>, g1, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_split<2>, g1, dim3(128), 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_split<3>, g1, dim3(192), 0, s, a); break;
    default: hipLaunchKernelGGL(k_split<4>, g1, dim3(256), 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_combine, dim3(a.H, (a.batch + CB - 1) / CB), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
