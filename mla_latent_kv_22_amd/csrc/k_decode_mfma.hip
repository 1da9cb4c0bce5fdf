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
// transpose read (ds_read_b64_tr_b16), so no transposed copy is staged.  Each
// item fixes its per-head reference maximum on its first tile and never
// rescales the accumulator (the merge stays exact: every partial carries its
// own reference); a score more than 2^100 above the reference could overflow,
// so such an (item, head) -- detected from its sum of numerators -- is
// flagged and recomputed exactly by the combine.  A partial leaves as its
// (m, l) pair in fp32 and its 512 latent sums rounded to bf16 (same exponent
// range as fp32, relative rounding 2^-9; half the bytes of fp32 sums).
// Pass 2 (combine): per (head, 16 or 32 sequences): LSE-merge of the items in
// a fixed order in fp32, the merged latent split into bf16 hi + lo parts, and
// W_UV applied with MFMA (the fp32 merged latent reaches the product intact
// to ~2^-17).
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
constexpr float kHeadroom = 100.f;  // largest score above the item's reference, log2 units

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


__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// The score chain keeps its accumulator in VGPRs (inline asm) while the
// latent accumulator owns the AGPRs (compiler MFMA form).  Hazards the
// compiler cannot see for the asm chain are covered here: its operands come
// from LDS reads or global loads (waited for by the compiler through the asm
// inputs), and score_drain() puts 20 wait states between the last MFMA and
// the first VALU read of the scores (a 16-pass MFMA needs 18).
__device__ __forceinline__ void score_first(f32x16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_next(f32x16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_drain(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc));
}

// Direct-to-LDS loads of one tile.  Wave w of NW issues loads i = w, w+NW, ...
// of the 36; load i fills LDS bytes [1024 i, +1024) = column group i / 4,
// rows 8 (i % 4) .. +7, lane l taking row 8 (i % 4) + l / 8 and the chunk
// whose swizzled slot is l % 8.  Its global byte offset is
// lane_off(l, i % 4) + 128 (i / 4); with NW = 4 the row block i % 4 = w is
// fixed per wave, so one lane offset serves all nine loads.  Written as inline asm so the compiler adds no wait of its own
// before LDS reads; the tile loop waits explicitly for exactly the tile it
// reads.  The instruction writes no VGPR.
__device__ __forceinline__ uint32_t load_lane_off(int lane, int rb) {
  const int r = 8 * rb + (lane >> 3);
  return (uint32_t)(r * (RW * 2) + (((lane & 7) ^ swz(r)) << 4));
}



template <int NW, int I0>
__device__ __forceinline__ void issue_full(const char* tile_base, uint32_t lds0, int w, const uint32_t* lane_off) {
  if constexpr (I0 < LOADS_PER_TILE) {
    const int i = I0 + w;
    // column offset 128 * (i / 4) goes into the scalar base (the instruction's
    // immediate offset would move the LDS destination as well)
    if constexpr (NW == 4) {
      dma16<0>(tile_base + 32 * I0, lane_off[0], lds0 + 1024 * i);
    } else {
      dma16<0>(tile_base + 128 * (i >> 2), lane_off[i & 3], lds0 + 1024 * i);
    }
    issue_full<NW, I0 + NW>(tile_base, lds0, w, lane_off);
  }
}

template <int NW>
__device__ __forceinline__ void issue_tile(const char* __restrict__ tile_base, int nvalid, uint32_t lds0, int w,
                                           int lane, const uint32_t* lane_off) {
  if (nvalid == TT) {
    issue_full<NW, 0>(tile_base, lds0, w, lane_off);
  } else {
    // ragged tail: rows past the last valid token repeat it (their p is 0)
#pragma unroll
    for (int i0 = 0; i0 < LOADS_PER_TILE; i0 += NW) {
      const int i = i0 + w;
      const int r = 8 * (i & 3) + (lane >> 3);
      const int rr = r < nvalid ? r : nvalid - 1;
      const int c = 8 * (i >> 2) + ((lane & 7) ^ swz(r));
      dma16<0>(tile_base, (uint32_t)(rr * (RW * 2) + c * 16), lds0 + 1024 * i);
    }
  }
}

// Per-lane LDS byte offsets of the operand reads, relative to a buffer base.
struct ReadOffsets {
  int s[4];     // score A operand (row = lane % 32, chunk 2 ks + g): + 4096 (ks / 4)
  int t[2][2];  // transpose reads [fb parity][upper 8 rows]: + 4096 (fb / 2) + 2048 kk
  int p[2];     // P^T fragment of head lane % 32, [kk]: + 2048 hb
};

// P^T in LDS, bf16: head h owns 64 bytes = [kk][half g][8 tokens]; the 16-byte
// slot 2 kk + g is XOR-swizzled by (h >> 1) & 3 (conflict-free 16-byte reads
// and writes of 8 consecutive heads).
__device__ __forceinline__ int p_off(int h, int kk, int g) { return 64 * h + 16 * ((2 * kk + g) ^ ((h >> 1) & 3)); }

// Softmax numerators of one tile for head lane % 32: p = 2^(s sl2 - m_ref)
// rounded to bf16, written to the P^T buffer; their sum goes to lsum.
// Tokens at or past t1 (only in a ragged last tile) get p = 0; MAYBE_RAGGED
// false is for tiles known to be full (every tile but an item's last).
template <bool MAYBE_RAGGED>
__device__ __forceinline__ void tile_softmax(const f32x16& sacc, int tok0, int t1, int g, float sl2, float m_ref,
                                             char* pbuf, int head_off, float& lsum, const ReadOffsets& o) {
  const bool full = !MAYBE_RAGGED || tok0 + TT <= t1;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    uint32_t wds[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int j = 8 * kk + e;
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j], sl2, -m_ref));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j + 1], sl2, -m_ref));
      if (!full) {
        const int t = 8 * (j >> 2) + 4 * g + (j & 3);  // tokens of j and j + 1 are t and t + 1
        if (tok0 + t >= t1) p0 = 0.f;
        if (tok0 + t + 1 >= t1) p1 = 0.f;
      }
      const uint32_t pk = pack_bf16x2(p0, p1);  // hardware round-to-nearest-even
      // lsum += both rounded numerators: one bf16 dot product with (1, 1)
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                             lsum, false);
      wds[e >> 1] = pk;
    }
    *(u32x4*)(pbuf + head_off + o.p[kk]) = u32x4{wds[0], wds[1], wds[2], wds[3]};
  }
}

// Largest score of the tile for this lane's head (both lane halves), raw units.
__device__ __forceinline__ float tile_max(const f32x16& sacc, int tok0, int t1, int g) {
  float mt = -INFINITY;
  if (tok0 + TT <= t1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sacc[j]);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = 8 * (j >> 2) + 4 * g + (j & 3);
      if (tok0 + t < t1) mt = fmaxf(mt, sacc[j]);
    }
  }
  return fmaxf(mt, __shfl_xor(mt, 32));
}

// Work split inside one work-group of NW waves: for the scores, wave w owns
// heads [32 w, 32 w + 32) (HB = NW head blocks in all); for the latent update
// it owns the FBW = 16 / NW feature blocks [FBW w, FBW w + FBW) of every head,
// so each C^T fragment read from LDS serves HB MFMAs and each wave reads only
// its share of the tile through the transpose path.
// HBN = 1 is the few-heads split (at most 32 heads): every wave scores the
// one head block (the same products on each wave, which saves the P^T
// exchange between waves) and updates its FBW feature blocks of it.
template <int NW, int HBN = NW>
struct Split {
  static constexpr int HB = HBN;
  static constexpr int FBW = FB / NW;
  static constexpr int NPC = 2 * FBW * HB;  // latent MFMAs per tile (32; 8 for the few-heads split)
};

// Latent update of one tile, op i = (kk, fbl, hb) in that order: A = C^T
// fragment of feature block FBW w + fbl (two transpose reads, one group
// ahead), B = P^T fragment of head block hb (16-byte reads, reloaded as soon
// as its last use for kk = 0 has issued).  With SCORES, the 36 chained score
// MFMAs of the next tile are interleaved one for one.
template <int NW, bool SCORES, int HBN = NW>
__device__ __forceinline__ void tile_step(f32x16& sacc, const char* ts, const u32x4* qf, f32x16* acc, const char* tp,
                                          const char* pbuf, int w, const ReadOffsets& o) {
  using S = Split<NW, HBN>;
  constexpr int PF = 3;
  u32x4 kf[PF];
  if constexpr (SCORES) {
#pragma unroll
    for (int ks = 0; ks < PF; ++ks) kf[ks] = *(const u32x4*)(ts + o.s[ks & 3] + 4096 * (ks >> 2));
  }
  auto tr_a = [&](int kk, int fbl) {
    const int fb = S::FBW * w + fbl;
    const int imm = 4096 * (fb >> 1) + 2048 * kk;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tp + o.t[fb & 1][0] + imm));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tp + o.t[fb & 1][1] + imm + 1024));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };
  auto p_frag = [&](int kk, int hb) { return *(const u32x4*)(pbuf + 2048 * hb + o.p[kk]); };
  u32x4 af[2], pf[S::HB];
  af[0] = tr_a(0, 0);
#pragma unroll
  for (int hb = 0; hb < S::HB; ++hb) pf[hb] = p_frag(0, hb);
  constexpr int NOPS = SCORES ? KS : S::NPC;
#pragma unroll
  for (int op = 0; op < NOPS; ++op) {
    if constexpr (SCORES) {
      const u32x4 cur = kf[op % PF];
      if (op + PF < KS) kf[op % PF] = *(const u32x4*)(ts + o.s[(op + PF) & 3] + 4096 * ((op + PF) >> 2));
      if (op == 0) score_first(sacc, cur, qf[op]);
      else score_next(sacc, cur, qf[op]);
    }
    if (op < S::NPC) {
      const int kk = op / (S::FBW * S::HB), fbl = (op / S::HB) % S::FBW, hb = op % S::HB;
      const int grp = op / S::HB;  // (kk, fbl) group index 0 .. 2 FBW - 1
      if (hb == 0 && grp + 1 < 2 * S::FBW) af[(grp + 1) & 1] = tr_a((grp + 1) / S::FBW, (grp + 1) % S::FBW);
      const u32x4 bv = pf[hb];
      if (kk == 0 && fbl == S::FBW - 1) pf[hb] = p_frag(1, hb);  // last kk = 0 use of this slot
      acc[fbl * S::HB + hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[grp & 1]), as_bf16x8(bv),
                                                                      acc[fbl * S::HB + hb], 0, 0, 0);
    }
  }
  if constexpr (SCORES) score_drain(sacc);
}

// One step of the tile loop, fused: the 36 chained score MFMAs of tile it+1
// with the first NPA latent MFMAs of tile it interleaved, then the softmax
// numerators of tile it+1 (written to P^T buffer pbuf_wr, as tile_softmax;
// tile it+1 must be full) in eight pieces with the remaining latent MFMAs
// between them, so that the VALU work of the softmax runs beside MFMA work
// instead of after it.  The latent MFMAs keep the order and operand reads of
// tile_step.
template <int NW>
__device__ __forceinline__ void tile_step_fused(f32x16& sacc, const char* ts, const u32x4* qf, f32x16* acc,
                                                const char* tp, const char* pbuf_rd, int w, const ReadOffsets& o,
                                                int tok0, int g, float sl2, float m_ref, char* pbuf_wr, int head_off,
                                                float& lsum) {
  using S = Split<NW>;
  constexpr int PF = 3;
  // latent MFMAs beside the score chain: 36 + NPA MFMAs take about as long
  // as the dependent chain alone; the other 12 run beside the softmax
  constexpr int NPA = S::NPC - 12;
  u32x4 kf[PF];
#pragma unroll
  for (int ks = 0; ks < PF; ++ks) kf[ks] = *(const u32x4*)(ts + o.s[ks & 3] + 4096 * (ks >> 2));
  auto tr_a = [&](int kk, int fbl) {
    const int fb = S::FBW * w + fbl;
    const int imm = 4096 * (fb >> 1) + 2048 * kk;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tp + o.t[fb & 1][0] + imm));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tp + o.t[fb & 1][1] + imm + 1024));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };
  auto p_frag = [&](int kk, int hb) { return *(const u32x4*)(pbuf_rd + 2048 * hb + o.p[kk]); };
  u32x4 af[2], pf[S::HB];
  af[0] = tr_a(0, 0);
#pragma unroll
  for (int hb = 0; hb < S::HB; ++hb) pf[hb] = p_frag(0, hb);
  auto pv = [&](int op) {
    const int kk = op / (S::FBW * S::HB), fbl = (op / S::HB) % S::FBW, hb = op % S::HB;
    const int grp = op / S::HB;  // (kk, fbl) group index 0 .. 2 FBW - 1
    if (hb == 0 && grp + 1 < 2 * S::FBW) af[(grp + 1) & 1] = tr_a((grp + 1) / S::FBW, (grp + 1) % S::FBW);
    const u32x4 bv = pf[hb];
    if (kk == 0 && fbl == S::FBW - 1) pf[hb] = p_frag(1, hb);  // last kk = 0 use of this slot
    acc[fbl * S::HB + hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[grp & 1]), as_bf16x8(bv),
                                                                    acc[fbl * S::HB + hb], 0, 0, 0);
  };
#pragma unroll
  for (int c = 0; c < KS; ++c) {
    const u32x4 cur = kf[c % PF];
    if (c + PF < KS) kf[c % PF] = *(const u32x4*)(ts + o.s[(c + PF) & 3] + 4096 * ((c + PF) >> 2));
    if (c == 0) score_first(sacc, cur, qf[c]);
    else score_next(sacc, cur, qf[c]);
    // latent MFMAs c NPA / KS .. (c + 1) NPA / KS - 1 follow score MFMA c
#pragma unroll
    for (int op = c * NPA / KS; op < (c + 1) * NPA / KS; ++op) pv(op);
  }
  score_drain(sacc);
  __builtin_amdgcn_sched_barrier(0);
  (void)tok0;
  (void)g;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    uint32_t wds[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int j = 8 * kk + e;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j], sl2, -m_ref));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j + 1], sl2, -m_ref));
      const uint32_t pk = pack_bf16x2(p0, p1);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                             lsum, false);
      wds[e >> 1] = pk;
      // piece k = 4 kk + e / 2 is followed by latent MFMAs NPA + 3 k / 2 ..;
      // the scheduling barriers keep the VALU and MFMA work alternating
      const int k = 4 * kk + (e >> 1);
#pragma unroll
      for (int op = NPA + 3 * k / 2; op < NPA + 3 * (k + 1) / 2; ++op) pv(op);
      __builtin_amdgcn_sched_barrier(0);
    }
    *(u32x4*)(pbuf_wr + head_off + o.p[kk]) = u32x4{wds[0], wds[1], wds[2], wds[3]};
  }
}

// LDS map (160 KiB, the whole LDS of a CU):
//   [0, 147456)        four tile stages of 36864 bytes
//   [147456, 163840)   two P^T buffers of NW * 2048 bytes (8192 for NW = 4)
// The planner's per-sequence arrays and its reduction scratch live in stage 3
// until the first load into it (every read of them happens before the
// barrier that precedes that load).
constexpr int NSTAGE = 4;
constexpr int PBUF_BYTES = 4 * 2048;
constexpr int LDS_BYTES = NSTAGE * TILE_BYTES + 2 * PBUF_BYTES;
constexpr int PLAN_INTS = 2 * (kMaxDecodeBatch + 1) + 16;
static_assert(PLAN_INTS * 4 <= TILE_BYTES, "planner arrays must fit in one stage");
static_assert(LDS_BYTES <= 163840, "LDS budget");

// One work-group per CU, persistent over the work items: round r of work-group
// x takes item index x + r * gridDim.x (the host keeps rounds <= 64), so no
// work-group is launched without work.  FEW: at most 32 heads, four waves that
// all score them (Split<NW, 1>): each wave writes the numerators to its own
// P^T region and reads them back for its feature blocks.
template <int NW, bool FEW = false>
__global__ void __launch_bounds__(NW * 64, 1) k_split(DecodeArgs a) {
  using S = Split<NW, FEW ? 1 : NW>;
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  char* tiles = smem;
  char* pbufs = smem + NSTAGE * TILE_BYTES;
  int* s_len = (int*)(tiles + 3 * TILE_BYTES);
  int* s_items = s_len + (kMaxDecodeBatch + 1);
  int* red = s_items + (kMaxDecodeBatch + 1);

  const int cap = a.len_cap;
  const DecodePlan plan = make_decode_plan(a.seq_lens, a.batch, cap, a.slots, a.min_chunk, kMaxChunk,
                                           a.ovh_tokens, a.round_ovh_tokens, s_len, s_items, red, a.err, a.max_items);
  const int n_items = plan.n_items;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // work-group 0 publishes the plan for the combine pass:
  // [0, B] first item of each sequence, [B+1, 2B] clamped lengths, [2B+1] chunk
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i <= a.batch; i += blockDim.x) a.plan[i] = s_items[i];
    for (int i = threadIdx.x; i < a.batch; i += blockDim.x) a.plan[a.batch + 1 + i] = s_len[i];
    if (threadIdx.x == 0) a.plan[2 * a.batch + 1] = plan.chunk;
  }
  // lane r of every wave holds round r's item, sequence and token range.
  // Consecutive items (same sequence) share an XCD: work-group x runs on XCD x % 8.
  const int G = gridDim.x;
  const int rounds = (int)blockIdx.x < n_items ? (n_items - 1 - (int)blockIdx.x) / G + 1 : 0;
  int d_item = 0, d_b = 0, d_t0 = 0, d_t1 = 0;
  if (lane < rounds) {
    const int idx = blockIdx.x + lane * G;
    const int item = ((n_items & 7) == 0 && (G & 7) == 0) ? (idx & 7) * (n_items >> 3) + (idx >> 3) : idx;
    const int b = item_seq(s_items, a.batch, item);
    d_item = item;
    d_b = b;
    d_t0 = (item - s_items[b]) * plan.chunk;
    d_t1 = min(s_len[b], d_t0 + plan.chunk);
  }
  __syncthreads();  // the planner arrays in stage 3 are not read after this point

  const int g = lane >> 5, hl = lane & 31;
  const int hq = FEW ? hl : w * 32 + hl;
  const bool hvalid = hq < a.H;
  const int P = a.P, tpp = P / TT;
  const uint32_t page_bytes = (uint32_t)(P * RW * 2);
  const char* __restrict__ pool = (const char*)a.pool;
  const uint32_t lds_tiles = lds_addr_of(tiles);
  uint32_t lane_off[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) lane_off[rb] = load_lane_off(lane, NW == 4 ? w : rb);
  ReadOffsets ro;
  {
    const int sw = swz(hl);
#pragma unroll
    for (int q = 0; q < 4; ++q) ro.s[q] = 128 * hl + 16 * ((2 * q + g) ^ sw);
    const int grp = lane >> 4, jl = lane & 15;
    const int trow = 4 * g + (jl >> 2);
    const int tchunk = 2 * (grp & 1) + ((jl >> 1) & 1);
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        ro.t[par][hf] = 128 * trow + 16 * ((4 * par + tchunk) ^ swz(trow + 8 * hf)) + 8 * (jl & 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) ro.p[kk] = p_off(hl, kk, g);  // + 2048 hb (hb keeps (h >> 1) & 3)
  }
  const int head_off = 2048 * w;  // this wave's heads (FEW: its copy of the heads) in the P^T buffer
  const int rd_off = FEW ? head_off : 0;  // where the latent update reads P^T
  const float sl2 = a.scale_log2;
  constexpr int LPW = LOADS_PER_TILE / NW;  // loads per wave per tile

  for (int rd = 0; rd < rounds; ++rd) {
    const int item = __builtin_amdgcn_readlane(d_item, rd);
    const int b = __builtin_amdgcn_readlane(d_b, rd);
    const int t0 = __builtin_amdgcn_readlane(d_t0, rd);
    const int t1 = __builtin_amdgcn_readlane(d_t1, rd);
    // block-table entries are read through the constant address space: scalar
    // loads, counted by lgkmcnt, so they never wait for the tile loads in flight
    const __attribute__((address_space(4))) int32_t* btb =
        (const __attribute__((address_space(4))) int32_t*)(a.block_table + (size_t)b * a.max_pages_per_seq);
    const int ntiles = (t1 - t0 + TT - 1) / TT;
    // tiles are requested in order, so pages and in-page tiles are counted
    // (a tile lies in one page: P % 32 == 0, t0 % 32 == 0), and the next
    // tile's block-table entry is read one request ahead of its use
    const int pg_end = (t1 - 1) / P;
    int w_pg = t0 / P, w_in = (t0 % P) / TT;
    int w_page = checked_page(btb[w_pg], a.num_pages, a.err);
    auto tile_ptr = [&](int tile, int& nvalid) {
      nvalid = min(TT, t1 - (t0 + tile * TT));
      const char* tp = pool + (size_t)(uint32_t)w_page * page_bytes + (uint32_t)w_in * (TT * RW * 2);
      if (++w_in == tpp) {
        w_in = 0;
        ++w_pg;
      }
      w_page = checked_page(btb[min(w_pg, pg_end)], a.num_pages, a.err);
      return tp;
    };

    // prologue: the absorbed query fragments (B operand of the score MFMA:
    // head hq, k = 16 ks + 8 g .. +7), then tiles 0, 1 and 2.  No wait for
    // loads of this round may sit between the tile loads: in-order retirement
    // would make it wait for the tiles as well.  The tile waits below count
    // the loads issued after the ones they need.
    u32x4 qf[KS];
    {
      // uniform base plus a 32-bit lane offset, formed here (no 64-bit
      // per-lane pointer kept alive across the item loop)
      const char* qb = (const char*)a.q_abs + (size_t)b * a.H * (RW * 2);
      uint32_t qo = (uint32_t)((hvalid ? hq : 0) * (RW * 2) + 16 * g);
      asm volatile("" : "+v"(qo));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = *(const u32x4*)(qb + qo + 32 * ks);
        qf[ks] = hvalid ? v : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int st = 0; st < 3; ++st) {
      if (st < ntiles) {
        int nv;
        const char* tp = tile_ptr(st, nv);
        issue_tile<NW>(tp, nv, lds_tiles + st * TILE_BYTES, w, lane, lane_off);
      }
    }

    f32x16 acc[S::FBW * S::HB];
#pragma unroll
    for (int i = 0; i < S::FBW * S::HB; ++i) acc[i] = f32x16{};
    float lsum = 0.f;

    // tile 0: scores, reference maximum, numerators into P^T buffer 0
    if (ntiles >= 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPW));
    else if (ntiles == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    f32x16 sacc;
    {
      constexpr int PF = 3;
      u32x4 kf[PF];
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) kf[ks] = *(const u32x4*)(tiles + ro.s[ks & 3] + 4096 * (ks >> 2));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 cur = kf[ks % PF];
        if (ks + PF < KS) kf[ks % PF] = *(const u32x4*)(tiles + ro.s[(ks + PF) & 3] + 4096 * ((ks + PF) >> 2));
        if (ks == 0) score_first(sacc, cur, qf[ks]);
        else score_next(sacc, cur, qf[ks]);
      }
      score_drain(sacc);
    }
    const float m_ref = tile_max(sacc, t0, t1, g) * sl2;  // fixed for the whole item
    if (ntiles > 1) tile_softmax<false>(sacc, t0, t1, g, sl2, m_ref, pbufs, head_off, lsum, ro);
    else tile_softmax<true>(sacc, t0, t1, g, sl2, m_ref, pbufs, head_off, lsum, ro);

    // step it: latent update of tile it (P^T buffer it % 2) interleaved with the
    // scores of tile it+1, whose numerators go to P^T buffer (it+1) % 2
    auto step_sync = [&](int it) {
      int nv3 = 0;
      const char* tp3 = (it + 3 < ntiles) ? tile_ptr(it + 3, nv3) : nullptr;  // scalar page load, early
      // this wave's loads of tile it+1 are done once only tile it+2's remain
      if (it + 2 < ntiles) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPW));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      // all waves: tile it+1 in LDS, P^T of tile it written, tile it-1 and
      // P^T buffer (it+1) % 2 no longer read
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (it + 3 < ntiles) issue_tile<NW>(tp3, nv3, lds_tiles + ((it + 3) & 3) * TILE_BYTES, w, lane, lane_off);
    };
    // tile it+1 is full for it + 2 < ntiles: the fused step (softmax beside
    // the latent MFMAs)
    int it = 0;
    if constexpr (FEW) {
      // 8 latent MFMAs a tile: the score chain alone sets the step, and the
      // softmax follows it
      for (; it + 2 < ntiles; ++it) {
        step_sync(it);
        const char* cur = tiles + (it & 3) * TILE_BYTES;
        const char* nxt = tiles + ((it + 1) & 3) * TILE_BYTES;
        tile_step<NW, true, S::HB>(sacc, nxt, qf, acc, cur, pbufs + (it & 1) * PBUF_BYTES + rd_off, w, ro);
        const int tok1 = t0 + (it + 1) * TT;
        tile_softmax<false>(sacc, tok1, t1, g, sl2, m_ref, pbufs + ((it + 1) & 1) * PBUF_BYTES, head_off, lsum, ro);
      }
    } else {
      for (; it + 2 < ntiles; ++it) {
        step_sync(it);
        const char* cur = tiles + (it & 3) * TILE_BYTES;
        const char* nxt = tiles + ((it + 1) & 3) * TILE_BYTES;
        const int tok1 = t0 + (it + 1) * TT;
        tile_step_fused<NW>(sacc, nxt, qf, acc, cur, pbufs + (it & 1) * PBUF_BYTES, w, ro, tok1, g, sl2, m_ref,
                            pbufs + ((it + 1) & 1) * PBUF_BYTES, head_off, lsum);
      }
    }
    // the item's last tile (maybe ragged): scores, then its numerators
    if (it + 1 < ntiles) {
      step_sync(it);
      const char* cur = tiles + (it & 3) * TILE_BYTES;
      const char* nxt = tiles + ((it + 1) & 3) * TILE_BYTES;
      tile_step<NW, true, S::HB>(sacc, nxt, qf, acc, cur, pbufs + (it & 1) * PBUF_BYTES + rd_off, w, ro);
      const int tok1 = t0 + (it + 1) * TT;
      tile_softmax<true>(sacc, tok1, t1, g, sl2, m_ref, pbufs + ((it + 1) & 1) * PBUF_BYTES, head_off, lsum, ro);
    }
    // latent update of the last tile (its scores were taken in the last step)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    tile_step<NW, false, S::HB>(sacc, tiles, qf, acc, tiles + ((ntiles - 1) & 3) * TILE_BYTES,
                                pbufs + ((ntiles - 1) & 1) * PBUF_BYTES + rd_off, w, ro);

    lsum += __shfl_xor(lsum, 32);
    // a score more than kHeadroom (log2) above the item's reference makes its
    // numerator, and so lsum, at least 2^kHeadroom (or inf / NaN past the fp32
    // range): such a partial is flagged with m = +inf and recomputed exactly by
    // the combine pass.  Below that bound every numerator, sum and latent
    // product stays far inside the fp32 range.
    const bool overflow = !(lsum < 0x1p100f);
    if (hvalid && g == 0 && (!FEW || w == 0)) {  // FEW: every wave holds the same (m, l)
      a.part_ml[((size_t)item * a.H + hq) * 2 + 0] = overflow ? INFINITY : m_ref;
      a.part_ml[((size_t)item * a.H + hq) * 2 + 1] = lsum;
    }
    // acc[fbl * HB + hb] holds O^T rows f = 32 (FBW w + fbl) + 8 (j/4) + 4 g + j % 4
    // of head 32 hb + lane % 32
#pragma unroll
    for (int fbl = 0; fbl < S::FBW; ++fbl)
#pragma unroll
      for (int hb = 0; hb < S::HB; ++hb) {
        const int h = 32 * hb + hl;
        if (h >= a.H) continue;
        uint16_t* pa = a.part_lat + ((size_t)item * a.H + h) * DC + 32 * (S::FBW * w + fbl) + 4 * g;
        const f32x16& v = acc[fbl * S::HB + hb];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(uint2*)(pa + 8 * q4) =
              make_uint2(pack_bf16x2(v[4 * q4], v[4 * q4 + 1]), pack_bf16x2(v[4 * q4 + 2], v[4 * q4 + 3]));
      }
    // the next round's query loads and tiles reuse LDS and registers
    __syncthreads();
  }
}

// ============================================================================
// At most 16 heads (V2-Lite has 16): k_split16.  A 32-head MFMA block would
// be half padding, and the work per token is small, so the layout changes:
//   * 16-wide MFMAs: scores S^T[16 tokens][16 heads] with 16x16x32 (18 k
//     steps over the 576-wide row), the latent update O^T[16 features][16
//     heads] += C^T[16 features][16 tokens] P^T[16 tokens][16 heads] with
//     16x16x16.  The score accumulator leaves lane l holding tokens
//     4 (l / 16) .. +3 of head l % 16, which is exactly the lane's share of
//     the P^T operand, so the numerators go from the accumulator to the
//     latent MFMA in registers;
//   * token-parallel waves: wave w takes the item's 16-token tiles w, w + 4,
//     ... through a private two-stage ring (18 direct-to-LDS loads a tile),
//     with its own reference maximum, sum and 512 x 16 accumulator; no
//     barrier in the loop;
//   * at the item's end the four waves merge in LDS (each scaled by
//     2^(m_w - m*)) into one partial, in the layout the combine reads.
// Tile layout in a stage: column group cg (64 features, 128 bytes per row)
// of 16 rows at 2048 cg, 16-byte piece c of row r at slot c ^ ((r / 2) % 8):
// the score fragment reads (16 rows, one piece each) cover all 64 banks.
constexpr int T16 = 16;                        // tokens per tile
constexpr int T16_BYTES = T16 * RW * 2;        // 18432
constexpr int T16_LOADS = T16_BYTES / 1024;    // 18 wave-wide loads a tile
constexpr int T16_WAVE = 2 * T16_BYTES;        // two stages per wave
constexpr int T16_LDS = 4 * T16_WAVE;          // 147456
static_assert(PLAN_INTS * 4 <= T16_WAVE, "planner arrays fit in one wave's stages");
static_assert(4 * 16 * DC * 4 + 4 * 16 * 2 * 4 <= T16_LDS, "merge buffers fit");

__device__ __forceinline__ int s16sw(int r) { return (r >> 1) & 7; }

__global__ void __launch_bounds__(256, 1) k_split16(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[T16_LDS];
  int* s_len = (int*)(smem + 3 * T16_WAVE);  // wave 3's stages, before its first load
  int* s_items = s_len + (kMaxDecodeBatch + 1);
  int* red = s_items + (kMaxDecodeBatch + 1);

  const int cap = a.len_cap;
  const DecodePlan plan = make_decode_plan(a.seq_lens, a.batch, cap, a.slots, a.min_chunk, kMaxChunk,
                                           a.ovh_tokens, a.round_ovh_tokens, s_len, s_items, red, a.err, a.max_items);
  const int n_items = plan.n_items;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i <= a.batch; i += blockDim.x) a.plan[i] = s_items[i];
    for (int i = threadIdx.x; i < a.batch; i += blockDim.x) a.plan[a.batch + 1 + i] = s_len[i];
    if (threadIdx.x == 0) a.plan[2 * a.batch + 1] = plan.chunk;
  }
  const int G = gridDim.x;
  const int rounds = (int)blockIdx.x < n_items ? (n_items - 1 - (int)blockIdx.x) / G + 1 : 0;
  int d_item = 0, d_b = 0, d_t0 = 0, d_t1 = 0;
  if (lane < rounds) {
    const int idx = blockIdx.x + lane * G;
    const int item = ((n_items & 7) == 0 && (G & 7) == 0) ? (idx & 7) * (n_items >> 3) + (idx >> 3) : idx;
    const int b = item_seq(s_items, a.batch, item);
    d_item = item;
    d_b = b;
    d_t0 = (item - s_items[b]) * plan.chunk;
    d_t1 = min(s_len[b], d_t0 + plan.chunk);
  }
  __syncthreads();  // the planner arrays are not read after this point

  const int hl = lane & 15, q4 = lane >> 4;  // head; token quad / k group
  const bool hvalid = hl < a.H;
  const int P = a.P;
  const uint32_t page_bytes = (uint32_t)(P * RW * 2);
  const char* __restrict__ pool = (const char*)a.pool;
  char* wst = smem + w * T16_WAVE;  // this wave's two stages
  const uint32_t lds_w = lds_addr_of(wst);
  // load d of a tile: rows 8 (d % 2) + lane / 8 of column group d / 2, slot
  // lane % 8 holding source piece slot ^ (row / 2 % 8); the column offset
  // 128 (d / 2) goes into the scalar base
  uint32_t ld_off[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int row = 8 * hf + (lane >> 3);
    ld_off[hf] = (uint32_t)(row * (RW * 2) + 16 * ((lane & 7) ^ s16sw(row)));
  }
  // score A operand (token row hl, piece 4 (ks % 2) + q4 of group ks / 2)
  const int sc_row = 128 * hl;
  // transpose read for feature block fb: source lane l (in its 16-lane group
  // q4) gives row 4 q4 + (l % 16) / 4, 8 bytes at features 16 fb + 4 (l % 4):
  // piece 2 (fb % 4) + (l / 2) % 2 of group fb / 4, half l % 2
  int tr_off[4];
  {
    const int row = 4 * q4 + (hl >> 2);
#pragma unroll
    for (int f4 = 0; f4 < 4; ++f4) tr_off[f4] = row * 128 + 16 * ((2 * f4 + ((hl >> 1) & 1)) ^ s16sw(row)) + 8 * (hl & 1);
  }
  const float sl2 = a.scale_log2;

  for (int rd = 0; rd < rounds; ++rd) {
    const int item = __builtin_amdgcn_readlane(d_item, rd);
    const int b = __builtin_amdgcn_readlane(d_b, rd);
    const int t0 = __builtin_amdgcn_readlane(d_t0, rd);
    const int t1 = __builtin_amdgcn_readlane(d_t1, rd);
    const __attribute__((address_space(4))) int32_t* btb =
        (const __attribute__((address_space(4))) int32_t*)(a.block_table + (size_t)b * a.max_pages_per_seq);
    const int ntiles = (t1 - t0 + T16 - 1) / T16;
    const int nmine = w < ntiles ? (ntiles - 1 - w) / 4 + 1 : 0;  // tiles w, w + 4, ...
    auto tile_src = [&](int j) {  // first row of tile j (P % 16 == 0: a tile lies in one page)
      const int tok = t0 + T16 * j;
      const int page = checked_page(btb[tok / P], a.num_pages, a.err);
      return pool + (size_t)(uint32_t)page * page_bytes + (uint32_t)(tok % P) * (RW * 2);
    };
    auto issue = [&](int j, int st) {
      const char* src = tile_src(j);
      const int nv = min(T16, t1 - (t0 + T16 * j));
      const uint32_t dst = lds_w + st * T16_BYTES;
      if (nv == T16) {
#pragma unroll
        for (int d = 0; d < T16_LOADS; ++d) dma16<0>(src + 128 * (d >> 1), ld_off[d & 1], dst + 1024 * d);
      } else {
        // ragged tail: rows past the last token repeat it (their p is 0)
#pragma unroll
        for (int d = 0; d < T16_LOADS; ++d) {
          const int row = 8 * (d & 1) + (lane >> 3), rr = min(row, nv - 1);
          const uint32_t off = (uint32_t)(rr * (RW * 2) + 16 * ((lane & 7) ^ s16sw(row)));
          dma16<0>(src + 128 * (d >> 1), off, dst + 1024 * d);
        }
      }
    };

    // query fragments (B operand of S^T = K Q^T): head hl, features
    // 32 ks + 8 q4 .. +7; heads past H read head 0 (their results are not stored)
    u32x4 qf[RW / 32];
    {
      const char* qb = (const char*)a.q_abs + (size_t)b * a.H * (RW * 2);
      uint32_t qo = (uint32_t)((hvalid ? hl : 0) * (RW * 2) + 16 * q4);
      asm volatile("" : "+v"(qo));
#pragma unroll
      for (int ks = 0; ks < RW / 32; ++ks) qf[ks] = *(const u32x4*)(qb + qo + 64 * ks);
    }
    if (nmine > 0) issue(w, 0);
    if (nmine > 1) issue(w + 4, 1);

    f32x4 acc[DC / 16];
#pragma unroll
    for (int i = 0; i < DC / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, lsum = 0.f;
    for (int i = 0; i < nmine; ++i) {
      const int j = w + 4 * i;
      if (i + 1 < nmine) __builtin_amdgcn_s_waitcnt(waitcnt_vm(T16_LOADS));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      asm volatile("" ::: "memory");
      const char* st = wst + (i & 1) * T16_BYTES;
      // scores, K fragments three steps ahead
      constexpr int PF = 3;
      auto kfrag = [&](int ks) {
        return *(const u32x4*)(st + 2048 * (ks >> 1) + sc_row + 16 * ((4 * (ks & 1) + q4) ^ s16sw(hl)));
      };
      u32x4 kf[PF];
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) kf[ks] = kfrag(ks);
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < RW / 32; ++ks) {
        const u32x4 cur = kf[ks % PF];
        if (ks + PF < RW / 32) kf[ks % PF] = kfrag(ks + PF);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur), as_bf16x8(qf[ks]), sc, 0, 0, 0);
      }
      // sc[e]: token t0 + 16 j + 4 q4 + e against head hl
      const int tok = t0 + T16 * j + 4 * q4;
      if (i == 0) {
        // this wave's reference maximum: the largest score of its first tile
        float mt = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (tok + e < t1) mt = fmaxf(mt, sc[e]);
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        m_ref = mt * sl2;
      }
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], sl2, -m_ref));
        if (tok + e >= t1) pv[e] = 0.f;
      }
      const uint32_t p01 = pack_bf16x2(pv[0], pv[1]), p23 = pack_bf16x2(pv[2], pv[3]);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p01), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                             lsum, false);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p23), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                             lsum, false);
      const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{p01, p23});
      // latent: O^T[16 fb + ..][hl] += C^T[features][4 q4 ..] P^T, transpose
      // reads two blocks ahead
      auto cfrag = [&](int fb) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + 2048 * (fb >> 2) + tr_off[fb & 3]));
      };
      s16x4 cf[2];
      cf[0] = cfrag(0);
      cf[1] = cfrag(1);
#pragma unroll
      for (int fb = 0; fb < DC / 16; ++fb) {
        const s16x4 cur = cf[fb & 1];
        if (fb + 2 < DC / 16) cf[fb & 1] = cfrag(fb + 2);
        acc[fb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cur, pb, acc[fb], 0, 0, 0);
      }
      // the stage is read: tile i + 2 goes into it
      if (i + 2 < nmine) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this stage's reads have returned
        issue(j + 8, i & 1);
      }
    }

    // merge the four waves: m* = max m_w, L = sum 2^(m_w - m*) l_w,
    // acc = sum 2^(m_w - m*) acc_w.  A wave without tiles has m_w = -inf.
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    // a score more than kHeadroom (log2) above a wave's reference makes its
    // sum at least 2^kHeadroom (or inf / NaN): the partial is flagged and the
    // combine recomputes it exactly
    const float ovf = (nmine > 0 && !(lsum < 0x1p100f)) ? 1.f : 0.f;
    float* s_acc = (float*)smem;                         // [4 waves][16 heads][512]
    float* s_ml = (float*)(smem + 4 * 16 * DC * 4);      // [4 waves][16 heads][2]
    __syncthreads();  // every wave is done with its stages
    if (q4 == 0) {
      s_ml[(w * 16 + hl) * 2 + 0] = nmine > 0 ? m_ref : -INFINITY;
      s_ml[(w * 16 + hl) * 2 + 1] = ovf > 0.f ? INFINITY : lsum;
    }
    __syncthreads();
    float mstar = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) mstar = fmaxf(mstar, s_ml[(v * 16 + hl) * 2]);
    const float sw = nmine > 0 ? __builtin_amdgcn_exp2f(m_ref - mstar) : 0.f;
    // acc[fb]: features 16 fb + 4 q4 + e of head hl
#pragma unroll
    for (int fb = 0; fb < DC / 16; ++fb)
      *(f32x4*)(s_acc + (w * 16 + hl) * DC + 16 * fb + 4 * q4) = acc[fb] * sw;
    __syncthreads();
    // sum the four copies in wave order: thread t takes head t / 16 and
    // features 4 (t % 16) + 64 k, k < 8
    {
      const int h = threadIdx.x >> 4, c4 = threadIdx.x & 15;
      if (h < a.H) {
        uint16_t* pa = a.part_lat + ((size_t)item * a.H + h) * DC;
#pragma unroll
        for (int k = 0; k < DC / 64; ++k) {
          const int f = 4 * c4 + 64 * k;
          f32x4 v = *(const f32x4*)(s_acc + h * DC + f);
#pragma unroll
          for (int u = 1; u < 4; ++u) v += *(const f32x4*)(s_acc + (u * 16 + h) * DC + f);
          *(uint2*)(pa + f) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
        if (c4 == 0) {
          float ms = -INFINITY, L = 0.f;
          bool flag = false;
#pragma unroll
          for (int u = 0; u < 4; ++u) ms = fmaxf(ms, s_ml[(u * 16 + h) * 2]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float mu = s_ml[(u * 16 + h) * 2], lu = s_ml[(u * 16 + h) * 2 + 1];
            if (mu == -INFINITY) continue;
            if (!(lu < INFINITY)) flag = true;
            L += __builtin_amdgcn_exp2f(mu - ms) * lu;
          }
          a.part_ml[((size_t)item * a.H + h) * 2 + 0] = flag ? INFINITY : ms;
          a.part_ml[((size_t)item * a.H + h) * 2 + 1] = L;
        }
      }
    }
    // the next round's loads reuse the stages and the merge buffers
    __syncthreads();
  }
}

// ============================================================================
// 8-bit cache (MLA_FLAG_FP8_CACHE: E4M3 codes, one float32 power-of-two scale
// per row).  Same plan, item loop, ring of four stages and step order as
// k_split; what changes is the tile and how its operands are read:
//   * a tile is 32 rows of 576 codes (18432 bytes) plus the 32 row scales
//     (two 128-byte copies): 18 wave-wide row loads and one scale load;
//   * scores: the block-scaled 8-bit MFMA (v_mfma_scale_f32_32x32x64_f8f6f4)
//     takes the codes straight from LDS, 32 per lane (64 features per step),
//     with the row scale as the A-side scale (an E8M0 byte is the exponent
//     field of the float32 scale); the absorbed query enters as two E4M3
//     parts, hi = E4M3(q / 2^e) and lo = E4M3((q - hi 2^e) / 2^(e-4)), with
//     one exponent e per head (the smallest with max |q| <= 448 2^e).  The
//     bf16 query has 8 significant bits; hi holds the top 4 and lo the rest,
//     so hi 2^e + lo 2^(e-4) reproduces it except for elements some 2^13
//     below the head's largest, and 18 MFMAs (hi and lo for 9 steps) give
//     the scores of the stored values;
//   * latent operand: 8 codes of one feature for 8 tokens through the 8-bit
//     LDS transpose read (ds_read_b64_tr_b8), converted with scale 1; the row
//     scale rides with the numerator instead: P^T holds p 2^e (exact), while
//     the softmax sum takes p itself.
// Tile layout: 9 column groups of 64 codes; group cg holds 32 rows x 64 bytes
// with 16-byte chunk slots XOR-swizzled by bits 2 and 3 of the row:
//   byte(r, c) = 2048 (c >> 2) + 64 r + 16 ((c & 3) ^ swz8(r))
// A transpose read (rows {0..3, 8..11} + 4 j, two chunks per 32 lanes) then
// hits every bank once, and so does each 16-byte score read (16 rows, one
// chunk slot each).
constexpr int T8_ROWS = TT * RW;            // 18432 bytes of codes
constexpr int T8_SCALES = T8_ROWS;          // two 128-byte copies of the row scales
constexpr int TILE8_BYTES = T8_ROWS + 256;  // 18688
constexpr int LOADS8 = T8_ROWS / 1024;      // 18 wave-wide row loads
__device__ __forceinline__ int swz8(int r) { return (((r >> 3) & 1) << 1) | ((r >> 2) & 1); }

// loads per wave per tile: row loads i = w, w + NW, ... < 18, plus scale
// loads so that every wave issues the same count (the tile waits count loads)
template <int NW>
struct Load8 {
  static constexpr int LPW = NW == 4 ? 5 : (NW == 2 ? 10 : 19);
  // with four waves, waves 2 and 3 (four row loads each) load the scales
  static __device__ __forceinline__ bool scales(int w) { return NW == 4 ? w >= 2 : true; }
  static __device__ __forceinline__ int copy(int w) { return NW == 4 ? w - 2 : w; }
};

// source byte offset of lane `lane` in row load i (row half rh = i & 1),
// relative to the tile's first row
__device__ __forceinline__ uint32_t load8_lane_off(int lane, int rh) {
  const int r = 16 * rh + (lane >> 2);
  return (uint32_t)(r * RW + (((lane & 3) ^ swz8(r)) << 4));
}

// Load i fills LDS bytes [1024 i, +1024) = column group i >> 1, rows
// 16 (i & 1) .. +15: lane l takes row 16 (i & 1) + l / 4 and the chunk whose
// swizzled slot is l % 4.  The scale load uses lanes 0-7 (128 bytes).
template <int NW>
__device__ __forceinline__ void issue_tile8(const char* __restrict__ rows, const char* __restrict__ scales, int nvalid,
                                            uint32_t lds0, int w, int lane, const uint32_t* lane_off) {
  if (nvalid == TT) {
#pragma unroll
    for (int i0 = 0; i0 < LOADS8; i0 += NW) {
      const int i = i0 + w;
      if (i < LOADS8) dma16<0>(rows + 64 * (i >> 1), lane_off[i & 1], lds0 + 1024 * i);
    }
  } else {
    // ragged tail: rows past the last valid token repeat it (their p is 0)
#pragma unroll
    for (int i0 = 0; i0 < LOADS8; i0 += NW) {
      const int i = i0 + w;
      if (i < LOADS8) {
        const int r = 16 * (i & 1) + (lane >> 2);
        const int rr = r < nvalid ? r : nvalid - 1;
        const uint32_t off = (uint32_t)(rr * RW + 64 * (i >> 1) + (((lane & 3) ^ swz8(r)) << 4));
        dma16<0>(rows, off, lds0 + 1024 * i);
      }
    }
  }
  if (Load8<NW>::scales(w) && lane < 8) dma16<0>(scales, 16u * lane, lds0 + T8_SCALES + 128 * Load8<NW>::copy(w));
}

struct ReadOffsets8 {
  int s[2];  // score operand: row lane % 32, chunks 2 g and 2 g + 1 of the step's group: + 2048 kb
  int t[2];  // transpose reads [fb parity]: + 2048 (fb / 2) + 1024 kk
};

// 8 E4M3 codes -> 8 bf16 values (exact)
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2 v) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.f, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int KB8 = RW / 64;  // 9 score steps of 64 features

// Score MFMAs of the 8-bit path, inline asm like score_first / score_next
// (the accumulator stays in VGPRs).  a: 32 codes of the lane's row, b: 32
// codes of the lane's head, sa / sb: E8M0 scale bytes (bits 0-7).
__device__ __forceinline__ void score8_first(f32x16& acc, const i32x8& a, const i32x8& b, int sa, int sb) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
               : "=&v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
__device__ __forceinline__ void score8_next(f32x16& acc, const i32x8& a, const i32x8& b, int sa, int sb) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
// A VALU result read by an asm MFMA needs wait states the compiler does not
// add for asm (without them the scores of pipelined tiles came out wrong):
// the per-tile A-side scale passes through five before its first MFMA.
__device__ __forceinline__ void valu_to_mfma(int& v) { asm volatile("s_nop 4" : "+v"(v)); }

// 32 codes of one row for score step kb (two 16-byte chunks)
__device__ __forceinline__ i32x8 kfrag8(const char* ts, const ReadOffsets8& o, int kb) {
  const u32x4 x = *(const u32x4*)(ts + o.s[0] + 2048 * kb);
  const u32x4 y = *(const u32x4*)(ts + o.s[1] + 2048 * kb);
  return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
}

// 18 chained score MFMAs of one tile: for each step the hi then the lo part.
// The next step's fragment is read into the same registers once both MFMAs
// of a step have issued (they read their operands at issue).
__device__ __forceinline__ void score_tile8(f32x16& sacc, const char* ts, const ReadOffsets8& o, const i32x8* qh,
                                            const i32x8* ql, int sa, int sbh, int sbl) {
  i32x8 kf = kfrag8(ts, o, 0);
#pragma unroll
  for (int kb = 0; kb < KB8; ++kb) {
    if (kb == 0) score8_first(sacc, kf, qh[kb], sa, sbh);
    else score8_next(sacc, kf, qh[kb], sa, sbh);
    score8_next(sacc, kf, ql[kb], sa, sbl);
    if (kb + 1 < KB8) kf = kfrag8(ts, o, kb + 1);
  }
  score_drain(sacc);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Latent update of one tile from an 8-bit tile (op order and P^T reads as
// tile_step).  With SCORES the 18 score MFMAs of the next tile (ts) run
// first and the latent MFMAs fill the wait for each step's operands.
template <int NW, bool SCORES>
__device__ __forceinline__ void tile_step8(f32x16& sacc, const char* ts, int sa, const i32x8* qh, const i32x8* ql,
                                           int sbh, int sbl, f32x16* acc, const char* tp, const char* pbuf, int w,
                                           const ReadOffsets8& o, const ReadOffsets& op) {
  using S = Split<NW>;
  auto tr_a = [&](int kk, int fbl) {
    const int fb = S::FBW * w + fbl;
    const u32x2 v = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(tp + o.t[fb & 1] + 2048 * (fb >> 1) + 1024 * kk)));
    return fp8x8_to_bf16(v);
  };
  auto p_frag = [&](int kk, int hb) { return *(const u32x4*)(pbuf + 2048 * hb + op.p[kk]); };
  u32x4 af[2], pf[S::HB];
  af[0] = tr_a(0, 0);
#pragma unroll
  for (int hb = 0; hb < S::HB; ++hb) pf[hb] = p_frag(0, hb);
  i32x8 kf;
  if constexpr (SCORES) kf = kfrag8(ts, o, 0);
  auto pv = [&](int c) {
    const int kk = c / (S::FBW * S::HB), fbl = (c / S::HB) % S::FBW, hb = c % S::HB;
    const int grp = c / S::HB;
    if (hb == 0 && grp + 1 < 2 * S::FBW) af[(grp + 1) & 1] = tr_a((grp + 1) / S::FBW, (grp + 1) % S::FBW);
    const u32x4 bv = pf[hb];
    if (kk == 0 && fbl == S::FBW - 1) pf[hb] = p_frag(1, hb);
    acc[fbl * S::HB + hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[grp & 1]), as_bf16x8(bv),
                                                                    acc[fbl * S::HB + hb], 0, 0, 0);
  };
  if constexpr (SCORES) {
    // score step kb (two MFMAs) followed by latent MFMAs kb * NPC / KB8 ..
#pragma unroll
    for (int kb = 0; kb < KB8; ++kb) {
      if (kb == 0) score8_first(sacc, kf, qh[kb], sa, sbh);
      else score8_next(sacc, kf, qh[kb], sa, sbh);
      score8_next(sacc, kf, ql[kb], sa, sbl);
      if (kb + 1 < KB8) kf = kfrag8(ts, o, kb + 1);
#pragma unroll
      for (int c = kb * S::NPC / KB8; c < (kb + 1) * S::NPC / KB8; ++c) pv(c);
    }
    score_drain(sacc);
  } else {
#pragma unroll
    for (int c = 0; c < S::NPC; ++c) pv(c);
  }
}

// Softmax numerators of an 8-bit tile for head lane % 32: p = 2^(s sl2 - m_ref),
// the sum takes bf16(p), P^T takes bf16(p) times the token's row scale.
// scl: the tile's row scales in LDS.  Tokens at or past t1 get p = 0.
template <bool MAYBE_RAGGED>
__device__ __forceinline__ void tile_softmax8(const f32x16& sacc, int tok0, int t1, int g, float sl2, float m_ref,
                                              char* pbuf, int head_off, float& lsum, const ReadOffsets& o,
                                              const char* scl) {
  const bool full = !MAYBE_RAGGED || tok0 + TT <= t1;
  f32x4 sc4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) sc4[q] = *(const f32x4*)(scl + 4 * (8 * q + 4 * g));
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    uint32_t wds[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int j = 8 * kk + e;
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j], sl2, -m_ref));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j + 1], sl2, -m_ref));
      float s0 = sc4[j >> 2][j & 3], s1 = sc4[j >> 2][(j & 3) + 1];
      if (!full) {
        const int t = 8 * (j >> 2) + 4 * g + (j & 3);
        if (tok0 + t >= t1) p0 = s0 = 0.f;
        if (tok0 + t + 1 >= t1) p1 = s1 = 0.f;
      }
      const uint32_t pk = pack_bf16x2(p0, p1);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                             lsum, false);
      // bf16(p) 2^e = bf16(p 2^e): the scale is a power of two
      wds[e >> 1] = pack_bf16x2(p0 * s0, p1 * s1);
    }
    *(u32x4*)(pbuf + head_off + o.p[kk]) = u32x4{wds[0], wds[1], wds[2], wds[3]};
  }
}

// LDS map of k_split8: four tile stages of 18688 bytes, the two P^T buffers,
// then the planner's per-sequence arrays.
constexpr int LDS8_PBUF = NSTAGE * TILE8_BYTES;            // 74752
constexpr int LDS8_PLAN = LDS8_PBUF + 2 * PBUF_BYTES;      // 91136
constexpr int LDS8_BYTES = LDS8_PLAN + PLAN_INTS * 4;
static_assert(LDS8_BYTES <= 163840, "LDS budget");

template <int NW>
__global__ void __launch_bounds__(NW * 64, 1) k_split8(DecodeArgs a) {
  using S = Split<NW>;
  __shared__ __attribute__((aligned(16))) char smem[LDS8_BYTES];
  char* tiles = smem;
  char* pbufs = smem + LDS8_PBUF;
  int* s_len = (int*)(smem + LDS8_PLAN);
  int* s_items = s_len + (kMaxDecodeBatch + 1);
  int* red = s_items + (kMaxDecodeBatch + 1);

  const int cap = a.len_cap;
  const DecodePlan plan = make_decode_plan(a.seq_lens, a.batch, cap, a.slots, a.min_chunk, kMaxChunk,
                                           a.ovh_tokens, a.round_ovh_tokens, s_len, s_items, red, a.err, a.max_items);
  const int n_items = plan.n_items;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i <= a.batch; i += blockDim.x) a.plan[i] = s_items[i];
    for (int i = threadIdx.x; i < a.batch; i += blockDim.x) a.plan[a.batch + 1 + i] = s_len[i];
    if (threadIdx.x == 0) a.plan[2 * a.batch + 1] = plan.chunk;
  }
  const int G = gridDim.x;
  const int rounds = (int)blockIdx.x < n_items ? (n_items - 1 - (int)blockIdx.x) / G + 1 : 0;
  int d_item = 0, d_b = 0, d_t0 = 0, d_t1 = 0;
  if (lane < rounds) {
    const int idx = blockIdx.x + lane * G;
    const int item = ((n_items & 7) == 0 && (G & 7) == 0) ? (idx & 7) * (n_items >> 3) + (idx >> 3) : idx;
    const int b = item_seq(s_items, a.batch, item);
    d_item = item;
    d_b = b;
    d_t0 = (item - s_items[b]) * plan.chunk;
    d_t1 = min(s_len[b], d_t0 + plan.chunk);
  }

  const int g = lane >> 5, hl = lane & 31;
  const int hq = w * 32 + hl;
  const bool hvalid = hq < a.H;
  const int P = a.P, tpp = P / TT;
  const size_t page8 = (size_t)P * (RW + 4);
  const char* __restrict__ pool = (const char*)a.pool;
  const uint32_t lds_tiles = lds_addr_of(tiles);
  uint32_t lane_off[2];
#pragma unroll
  for (int rh = 0; rh < 2; ++rh) lane_off[rh] = load8_lane_off(lane, NW == 1 ? rh : (w & 1));
  ReadOffsets8 r8;
  ReadOffsets ro;
  {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) r8.s[h2] = 64 * hl + 16 * ((2 * g + h2) ^ swz8(hl));
    const int grp = lane >> 4, s = lane & 15, e = s >> 1;
    const int trow = 8 * (e >> 2) + 4 * (grp >> 1) + (e & 3);
#pragma unroll
    for (int par = 0; par < 2; ++par) r8.t[par] = 64 * trow + 16 * ((2 * par + (grp & 1)) ^ swz8(trow)) + 8 * (s & 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) ro.p[kk] = p_off(hl, kk, g);
  }
  const int head_off = 2048 * w;
  const float sl2 = a.scale_log2;
  constexpr int LPW = Load8<NW>::LPW;
  __syncthreads();  // planner arrays read

  for (int rd = 0; rd < rounds; ++rd) {
    const int item = __builtin_amdgcn_readlane(d_item, rd);
    const int b = __builtin_amdgcn_readlane(d_b, rd);
    const int t0 = __builtin_amdgcn_readlane(d_t0, rd);
    const int t1 = __builtin_amdgcn_readlane(d_t1, rd);
    const __attribute__((address_space(4))) int32_t* btb =
        (const __attribute__((address_space(4))) int32_t*)(a.block_table + (size_t)b * a.max_pages_per_seq);
    const int ntiles = (t1 - t0 + TT - 1) / TT;
    // tiles are requested in order: pages and in-page tiles are counted, and
    // the next tile's block-table entry is read one request ahead of its use
    const int pg_end = (t1 - 1) / P;
    int w_pg = t0 / P, w_in = (t0 % P) / TT;
    int w_page = checked_page(btb[w_pg], a.num_pages, a.err);
    auto tile_src = [&](int tile, int& nvalid, const char*& scales) {
      nvalid = min(TT, t1 - (t0 + tile * TT));
      const char* pg = pool + (size_t)(uint32_t)w_page * page8;
      scales = pg + (size_t)P * RW + 4 * TT * w_in;
      const char* rows = pg + (size_t)(TT * RW) * w_in;
      if (++w_in == tpp) {
        w_in = 0;
        ++w_pg;
      }
      w_page = checked_page(btb[min(w_pg, pg_end)], a.num_pages, a.err);
      return rows;
    };
    auto stage = [&](int tile) { return tiles + (tile & 3) * TILE8_BYTES; };
    // E8M0 scale byte of the lane's row in a tile (the exponent field of the
    // float32 power of two; 127 = 1 for rows past the end)
    auto row_scale = [&](int tile) {
      const uint32_t bits = *(const uint32_t*)(stage(tile) + T8_SCALES + 4 * hl);
      int sa = t0 + tile * TT + hl < t1 ? (int)((bits >> 23) & 0xffu) : 127;
      valu_to_mfma(sa);
      return sa;
    };

    // absorbed query of head hq: features 64 kb + 32 g + 8 j .. +7 (bf16) for
    // kb = 0..8, j = 0..3, split into the E4M3 parts hi and lo; a first pass
    // over the loads finds the head maximum, the second converts
    i32x8 qh[KB8], ql[KB8];
    int sbh, sbl;
    {
      const char* qb = (const char*)a.q_abs + (size_t)b * a.H * (RW * 2);
      uint32_t qo = (uint32_t)((hvalid ? hq : 0) * (RW * 2) + 64 * g);
      asm volatile("" : "+v"(qo));
      auto qload = [&](int kb, int j) {
        const u32x4 v = *(const u32x4*)(qb + qo + 128 * kb + 16 * j);
        return hvalid ? v : u32x4{0, 0, 0, 0};
      };
      // head maximum over both lane halves -> exponent e (smallest with
      // amax <= 448 2^e, at least -123 so that e - 4 stays an E8M0 value)
      float amax = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB8; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 v = qload(kb, j);
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(v[e2] << 16)), fabsf(__uint_as_float(v[e2] & 0xffff0000u))));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      int e = 0;
      if (amax > 0.f) {
        const uint32_t bits = __float_as_uint(amax);
        e = max((int)(bits >> 23) - 127 - 8 + ((bits & 0x7fffffu) > 0x600000u ? 1 : 0), -123);
      }
      const float inv_hi = __uint_as_float((uint32_t)(127 - e) << 23);      // 2^-e
      const float inv_lo = __uint_as_float((uint32_t)(127 - e + 4) << 23);  // 2^(4-e)
      const float sc_hi = __uint_as_float((uint32_t)(127 + e) << 23);       // 2^e
#pragma unroll
      for (int kb = 0; kb < KB8; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 v = qload(kb, j);
#pragma unroll
          for (int p2 = 0; p2 < 2; ++p2) {
            const uint32_t u0 = v[2 * p2], u1 = v[2 * p2 + 1];
            const float x0 = __uint_as_float(u0 << 16), x1 = __uint_as_float(u0 & 0xffff0000u);
            const float x2 = __uint_as_float(u1 << 16), x3 = __uint_as_float(u1 & 0xffff0000u);
            int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0 * inv_hi, x1 * inv_hi, 0, false);
            h = __builtin_amdgcn_cvt_pk_fp8_f32(x2 * inv_hi, x3 * inv_hi, h, true);
            const f32x2 d01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false), d23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
            // residuals are exact: bf16 minus its top 4 significant bits
            int l = __builtin_amdgcn_cvt_pk_fp8_f32((x0 - d01[0] * sc_hi) * inv_lo, (x1 - d01[1] * sc_hi) * inv_lo, 0,
                                                    false);
            l = __builtin_amdgcn_cvt_pk_fp8_f32((x2 - d23[0] * sc_hi) * inv_lo, (x3 - d23[1] * sc_hi) * inv_lo, l,
                                                true);
            qh[kb][2 * j + p2] = h;
            ql[kb][2 * j + p2] = l;
          }
        }
      }
      sbh = 127 + e;
      sbl = 127 + e - 4;
    }
#pragma unroll
    for (int st = 0; st < 3; ++st) {
      if (st < ntiles) {
        int nv;
        const char* sc;
        const char* tp = tile_src(st, nv, sc);
        issue_tile8<NW>(tp, sc, nv, lds_tiles + st * TILE8_BYTES, w, lane, lane_off);
      }
    }

    f32x16 acc[FB];
#pragma unroll
    for (int i = 0; i < FB; ++i) acc[i] = f32x16{};
    float lsum = 0.f;

    if (ntiles >= 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPW));
    else if (ntiles == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    f32x16 sacc;
    score_tile8(sacc, tiles, r8, qh, ql, row_scale(0), sbh, sbl);
    const float m_ref = tile_max(sacc, t0, t1, g) * sl2;
    if (ntiles > 1) tile_softmax8<false>(sacc, t0, t1, g, sl2, m_ref, pbufs, head_off, lsum, ro, tiles + T8_SCALES);
    else tile_softmax8<true>(sacc, t0, t1, g, sl2, m_ref, pbufs, head_off, lsum, ro, tiles + T8_SCALES);

    auto step_sync = [&](int it) {
      int nv3 = 0;
      const char* sc3 = nullptr;
      const char* tp3 = (it + 3 < ntiles) ? tile_src(it + 3, nv3, sc3) : nullptr;
      if (it + 2 < ntiles) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPW));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (it + 3 < ntiles) issue_tile8<NW>(tp3, sc3, nv3, lds_tiles + ((it + 3) & 3) * TILE8_BYTES, w, lane, lane_off);
    };
    int it = 0;
    for (; it + 2 < ntiles; ++it) {
      step_sync(it);
      tile_step8<NW, true>(sacc, stage(it + 1), row_scale(it + 1), qh, ql, sbh, sbl, acc, stage(it),
                           pbufs + (it & 1) * PBUF_BYTES, w, r8, ro);
      tile_softmax8<false>(sacc, t0 + (it + 1) * TT, t1, g, sl2, m_ref, pbufs + ((it + 1) & 1) * PBUF_BYTES,
                           head_off, lsum, ro, stage(it + 1) + T8_SCALES);
    }
    if (it + 1 < ntiles) {
      step_sync(it);
      tile_step8<NW, true>(sacc, stage(it + 1), row_scale(it + 1), qh, ql, sbh, sbl, acc, stage(it),
                           pbufs + (it & 1) * PBUF_BYTES, w, r8, ro);
      tile_softmax8<true>(sacc, t0 + (it + 1) * TT, t1, g, sl2, m_ref, pbufs + ((it + 1) & 1) * PBUF_BYTES,
                          head_off, lsum, ro, stage(it + 1) + T8_SCALES);
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    tile_step8<NW, false>(sacc, tiles, 127, qh, ql, sbh, sbl, acc, stage(ntiles - 1),
                          pbufs + ((ntiles - 1) & 1) * PBUF_BYTES, w, r8, ro);

    lsum += __shfl_xor(lsum, 32);
    const bool overflow = !(lsum < 0x1p100f);
    if (hvalid && g == 0) {
      a.part_ml[((size_t)item * a.H + hq) * 2 + 0] = overflow ? INFINITY : m_ref;
      a.part_ml[((size_t)item * a.H + hq) * 2 + 1] = lsum;
    }
#pragma unroll
    for (int fbl = 0; fbl < S::FBW; ++fbl)
#pragma unroll
      for (int hb = 0; hb < S::HB; ++hb) {
        const int h = 32 * hb + hl;
        if (h >= a.H) continue;
        uint16_t* pa = a.part_lat + ((size_t)item * a.H + h) * DC + 32 * (S::FBW * w + fbl) + 4 * g;
        const f32x16& v = acc[fbl * S::HB + hb];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(uint2*)(pa + 8 * q4) =
              make_uint2(pack_bf16x2(v[4 * q4], v[4 * q4 + 1]), pack_bf16x2(v[4 * q4 + 2], v[4 * q4 + 3]));
      }
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
// Exact two-pass partial (m, l, acc) of one (item, head) in fp32, stored as
// the split pass stores it (latent sums as bf16), used only for partials the
// split pass flagged.  scratch: >= 576 + 256 floats of LDS.
// The arguments are plain values (no pointer to the kernel's argument block,
// which would force that block into scratch memory in the caller).
// f8: the pool is 8-bit (row values E4M3(code) * row scale).
__device__ __noinline__ void recompute_partial(const void* __restrict__ pool, const int32_t* __restrict__ bt,
                                               const uint16_t* __restrict__ qa, uint16_t* __restrict__ pa,
                                               float* __restrict__ pml, int P, float scale_log2, int t0, int t1,
                                               float* scratch, int* red, int f8, int num_pages, int* err) {
  // blockDim.x in {256, 512, 1024}: thread tid keeps latent columns tid and
  // tid + blockDim.x, those below d_c
  const int nth = blockDim.x;
  float* q = scratch;          // 576
  float* p = scratch + RW;     // blockDim.x
  const int tid = threadIdx.x;
  __syncthreads();
  for (int f = tid; f < RW; f += nth) q[f] = bf16_to_f32(qa[f]);
  __syncthreads();
  // value f of token t's row
  auto val = [&](int t, int f) {
    const long long slot = (long long)checked_page(bt[t / P], num_pages, err) * P + t % P;
    return f8 ? e4m3_to_f32(fp8_row(pool, slot, P, RW)[f]) * fp8_scale(pool, slot, P, RW)
              : bf16_to_f32(((const uint16_t*)pool)[(size_t)slot * RW + f]);
  };
  auto score = [&](int t) {
    float d = 0.f;
    for (int f = 0; f < RW; ++f) d += q[f] * val(t, f);
    return d * scale_log2;
  };
  float m = -INFINITY;
  for (int t = t0 + tid; t < t1; t += nth) m = fmaxf(m, score(t));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = __float_as_int(m);
  __syncthreads();
  m = -INFINITY;
  for (int w = 0; w < (nth >> 6); ++w) m = fmaxf(m, __int_as_float(red[w]));
  const int c0 = tid, c1 = tid + nth;
  float acc0 = 0.f, acc1 = 0.f, l = 0.f;
  for (int tb = t0; tb < t1; tb += nth) {
    __syncthreads();
    const int t = tb + tid;
    p[tid] = (t < t1) ? exp2f(score(t) - m) : 0.f;
    __syncthreads();
    const int nt = min(nth, t1 - tb);
    for (int k = 0; k < nt; ++k) {
      const int tt = tb + k;
      const float pk = p[k];
      l += pk;  // every thread keeps the full sum
      if (c0 < DC) acc0 += pk * val(tt, c0);
      if (c1 < DC) acc1 += pk * val(tt, c1);
    }
  }
  if (c0 < DC) pa[c0] = f32_to_bf16(acc0);
  if (c1 < DC) pa[c1] = f32_to_bf16(acc1);
  if (tid == 0) {
    pml[0] = m;
    pml[1] = l;
  }
  __syncthreads();
}

// --------------------------------------------------------------------------
// combine: grid (H, ceil(batch / CB)), 512 threads (8 waves).  Work-group
// (h, sequences b0 .. b0+CB-1): merge the partials of every item of those
// sequences into the latent output (fp32), then o = W_UV,h lat with MFMA.
// CB = 16 with CNB = 2 item loads in flight per sequence when the grid fills
// the GPU; for small H x batch (few work-groups, many items per sequence)
// CB = 4 with CNB = 8 gives four times the work-groups and a quarter of the
// dependent load rounds.
constexpr int CNW = 8;   // waves per combine work-group
template <int CB, int CNB>
__global__ void __launch_bounds__(64 * CNW, 4) k_combine(DecodeArgs a) {
  constexpr int CBR = CB > 16 ? CB : 16;  // rows of the W_UV product (16-row MFMA blocks)
  __shared__ __attribute__((aligned(16))) uint16_t lat_hi[CBR * DC];  // [seq][512], 16-byte slot p ^ seq
  __shared__ __attribute__((aligned(16))) uint16_t lat_lo[CBR * DC];
  __shared__ __attribute__((aligned(16))) uint16_t o_st[CBR * 256];   // output rows (d_v <= 256)
  __shared__ int s_items[CB + 1], s_len[CB];
  __shared__ int red[16];
  __shared__ int s_chunk;

  const int h = blockIdx.x, b0 = blockIdx.y * CB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nb = min(CB, a.batch - b0);
  const float* __restrict__ pml = a.part_ml;
  const uint16_t* __restrict__ plat = a.part_lat;

  // the plan the split pass published
  if (tid <= nb) s_items[tid] = a.plan[b0 + tid];
  if (tid < nb) s_len[tid] = a.plan[a.batch + 1 + b0 + tid];
  if (tid == 0) s_chunk = a.plan[2 * a.batch + 1];
  __syncthreads();

  // thread: latent columns 4 cq .. 4 cq + 3 of sequences bl = tid / 128 + 4 k.
  // Online merge over the items in index order, CNB items per step:
  //   m = max(m, m_i);  v = v 2^(m_old - m) + sum_i 2^(m_i - m) acc_i;  L likewise.
  // A partial flagged by the split pass (m_i = +inf) is recomputed exactly
  // first and the merge redone.
  const int cq = tid & 127, blo = tid >> 7;
  constexpr int NS = CB / 4;
  f32x4 v[NS];
  float mrun[NS], lrun[NS];
  for (int pass = 0; pass < 2; ++pass) {
    int flagged = 0;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      mrun[k] = -INFINITY;
      lrun[k] = 0.f;
    }
    int maxn = 0;
    for (int k = 0; k < NS; ++k) {
      const int bl = blo + 4 * k;
      if (bl < nb) maxn = max(maxn, s_items[bl + 1] - s_items[bl]);
    }
    for (int j0 = 0; j0 < maxn; j0 += CNB) {
      float mi[NS][CNB], li[NS][CNB];
      f32x4 ai[NS][CNB];
#pragma unroll
      for (int k = 0; k < NS; ++k)
#pragma unroll
        for (int jj = 0; jj < CNB; ++jj) {
          const int bl = blo + 4 * k;
          const int i = (bl < nb) ? s_items[bl] + j0 + jj : 0;
          const bool ok = bl < nb && i < s_items[bl + 1];
          const size_t ih = (size_t)(ok ? i : 0) * (size_t)a.H + (size_t)h;
          const float2 ml = ok ? *(const float2*)(pml + 2 * ih) : make_float2(-INFINITY, 0.f);
          mi[k][jj] = ml.x;
          li[k][jj] = ml.y;
          const uint2 pb = ok ? *(const uint2*)(plat + DC * ih + 4 * cq) : make_uint2(0u, 0u);
          ai[k][jj] = f32x4{__uint_as_float(pb.x << 16), __uint_as_float(pb.x & 0xffff0000u),
                            __uint_as_float(pb.y << 16), __uint_as_float(pb.y & 0xffff0000u)};
        }
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        float mn = mrun[k];
#pragma unroll
        for (int jj = 0; jj < CNB; ++jj) {
          flagged |= mi[k][jj] == INFINITY;
          mn = fmaxf(mn, mi[k][jj]);
        }
        if (mn == -INFINITY) continue;  // no item yet
        const float sc = exp2f(mrun[k] - mn);  // 0 when mrun = -inf
        v[k] *= sc;
        lrun[k] *= sc;
#pragma unroll
        for (int jj = 0; jj < CNB; ++jj) {
          const float wgt = exp2f(mi[k][jj] - mn);  // 0 for absent items (m = -inf)
          v[k] += wgt * ai[k][jj];
          lrun[k] += wgt * li[k][jj];
        }
        mrun[k] = mn;
      }
    }
    if (__syncthreads_or(flagged) == 0) break;
    if (pass == 1) break;  // recomputed partials are finite
    for (int bl = 0; bl < nb; ++bl) {
      const int b = b0 + bl;
      for (int i = s_items[bl]; i < s_items[bl + 1]; ++i) {
        if (pml[((size_t)i * a.H + h) * 2] != INFINITY) continue;  // same value in every thread
        const int t0 = (i - s_items[bl]) * s_chunk;
        const int t1 = min(s_len[bl], t0 + s_chunk);
        const size_t ih = (size_t)i * a.H + h;
        recompute_partial(a.pool, a.block_table + (size_t)b * a.max_pages_per_seq,
                          (const uint16_t*)a.q_abs + ((size_t)b * a.H + h) * RW, a.part_lat + ih * DC,
                          a.part_ml + ih * 2, a.P, a.scale_log2, t0, t1, (float*)lat_hi, red, a.fp8, a.num_pages,
                          a.err);
      }
    }
    __syncthreads();
  }

  // lat = v / L as bf16 hi + lo (the pair carries the fp32 value to ~2^-17)
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int bl = blo + 4 * k;
    const float il = lrun[k] > 0.f ? 1.f / lrun[k] : 0.f;
    if (cq == 0 && bl < nb && a.lse)
      a.lse[(size_t)(b0 + bl) * a.H + h] = lrun[k] > 0.f ? (mrun[k] + log2f(lrun[k])) * kLn2 : -INFINITY;
    const f32x4 x = v[k] * il;
    const int pos = bl * (DC / 8) + ((cq >> 1) ^ bl);
    const int within = (cq & 1) * 4;
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const uint32_t hp = pack_bf16x2(x[e], x[e + 1]);
      const float h0 = __uint_as_float(hp << 16), h1 = __uint_as_float(hp & 0xffff0000u);
      hw[e >> 1] = hp;
      lw[e >> 1] = pack_bf16x2(x[e] - h0, x[e + 1] - h1);
    }
    *(uint2*)(lat_hi + pos * 8 + within) = make_uint2(hw[0], hw[1]);
    *(uint2*)(lat_lo + pos * 8 + within) = make_uint2(lw[0], lw[1]);
  }
  __syncthreads();

  // out[b][h][v] = sum_c lat[b][c] W_UV[h][v][c], 16x16x32 MFMA: D[seq][v],
  // A = lat (row = lane % 16, k = 8 (lane / 16) of each 32-wide step),
  // B = W_UV^T (column v = lane % 16).  Wave w takes 16-column blocks w, w + 8, ...
  const uint16_t* wuv = (const uint16_t*)a.w_uv + (size_t)h * a.d_v * DC;
  const int m16 = lane & 15, q = lane >> 4;
  for (int vb = w; vb * 16 < a.d_v; vb += CNW) {
    asm volatile("" ::: "memory");  // keeps the latent fragment reads inside the loop (registers)
    const uint16_t* wrow = wuv + (size_t)(vb * 16 + m16) * DC + 8 * q;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int KH = DC / 64;  // k-steps per half
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 wf[KH];
#pragma unroll
      for (int k = 0; k < KH; ++k) wf[k] = *(const u32x4*)(wrow + 32 * (KH * half + k));
#pragma unroll
      for (int k = 0; k < KH; ++k) {
        const int ks = KH * half + k;
        const int pos = m16 * (DC / 8) + ((4 * ks + q) ^ m16);
        const u32x4 ah = *(const u32x4*)(lat_hi + pos * 8);
        const u32x4 al = *(const u32x4*)(lat_lo + pos * 8);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(wf[k]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al), as_bf16x8(wf[k]), acc, 0, 0, 0);
      }
    }
    // D: lane holds column v = lane % 16 of sequences 4 (lane / 16) + j
#pragma unroll
    for (int j = 0; j < 4; ++j) o_st[(4 * q + j) * 256 + vb * 16 + m16] = f32_to_bf16(acc[j]);
  }
  __syncthreads();
  // output rows to HBM, 16 bytes per lane
  const int pieces = a.d_v / 8;
  for (int u = tid; u < nb * pieces; u += 64 * CNW) {
    const int bl = u / pieces, pc = u % pieces;
    *(u32x4*)((uint16_t*)a.out + ((size_t)(b0 + bl) * a.H + h) * a.d_v + 8 * pc) =
        *(const u32x4*)(o_st + bl * 256 + 8 * pc);
  }
}


// --------------------------------------------------------------------------
// combine, wide form for d_v = 128: grid (H, ceil(batch / 32)), 1024 threads
// (16 waves), one work-group per CU.  Work-group (h, sequences b0 .. b0+31):
//   - W_UV,h (128 rows x 1 KiB) goes to LDS by direct loads, 8 rows a wave;
//     row r keeps its 16-byte chunk c in slot c ^ (r % 32).
//   - Wave w owns latent columns 32 w .. 32 w + 31, one 32-wide k-step of the
//     16x16x32 product.  Its lane (r, q) = (lane % 16, lane / 16) merges
//     columns 32 w + 8 q .. +7 of sequences r and 16 + r over the items in
//     index order (groups of four items, requested together; a later group
//     rescales the earlier ones).  Those eight columns are its A fragment of
//     each 16-sequence block, and one 16-byte load of a bf16 partial: the
//     four lanes of a sequence read 64 contiguous bytes.  Every partial of
//     the work-group is requested before the first wait; the items' (m, L)
//     pairs come through LDS.
//   - D_w[s][v] = sum over the wave's 32 columns k of lat[s][k] W_UV[h][v][k],
//     lat as bf16 hi + lo (the pair carries the fp32 value to ~2^-17): two
//     16-sequence blocks x eight 16-wide v blocks, 32 MFMAs a wave.
//   - The 16 partial products meet in LDS (over the W_UV buffer), half of v
//     at a time, and each output pair is the sum over w = 0 .. 15 in order.
constexpr int WCB = 32;       // sequences per wide combine work-group
constexpr int WNI = 4;        // items requested per sequence and group
constexpr int WRED_LD = 68;   // floats per reduction row (64 + 4: the four row groups of a D fragment hit other banks)
constexpr int WLDS = 16 * WCB * WRED_LD * 4;  // 139264 bytes: reduction rows; W_UV,h in the first 128 KiB
static_assert(128 * DC * 2 <= WLDS, "W_UV,h fits under the reduction rows");
constexpr int WSCR = RW + 1024;  // floats of scratch for recompute_partial
// buffer resource word 3 for raw 32-bit accesses
constexpr int kRawBufferWord3 = 0x00020000;
__global__ void __launch_bounds__(1024) k_combine_wide(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[WLDS];
  __shared__ __attribute__((aligned(16))) float scr[WSCR];
  __shared__ __attribute__((aligned(16))) f32x2 s_ml[WNI][WCB];  // (m, L) of item j0 + jj of each sequence
  __shared__ int red[16];

  const int h = blockIdx.x, b0 = blockIdx.y * WCB;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int nb = min(WCB, a.batch - b0);
  const float* __restrict__ pml = a.part_ml;

  // items it0[sb] .. it1[sb] - 1 of this lane's sequences b0 + 16 sb + r16 (none past the batch)
  int it0[2], it1[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    it0[sb] = a.plan[b0 + min(16 * sb + r16, nb)];
    it1[sb] = a.plan[b0 + min(16 * sb + r16 + 1, nb)];
  }
  // threads 0 .. 127 fetch the (m, L) pairs: sequence tid / 4, item j0 + tid % 4
  const int mseq = min(tid >> 2, nb);
  int mit0 = a.plan[b0 + mseq], mit1 = a.plan[b0 + min(mseq + 1, nb)];
  // the plan arrives before the direct loads are issued
  asm volatile("" ::"v"(it0[0]), "v"(it1[0]), "v"(it0[1]), "v"(it1[1]), "v"(mit0), "v"(mit1));
  int nmax = max(it1[0] - it0[0], it1[1] - it0[1]);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) nmax = max(nmax, __shfl_xor(nmax, o));
  nmax = __builtin_amdgcn_readfirstlane(nmax);

  // W_UV,h rows 8 w .. 8 w + 7 to LDS: lane l fills slot l of row r from chunk l ^ (r % 32)
  {
    const char* wbase = (const char*)a.w_uv + (size_t)h * 128 * DC * 2;
    const uint32_t lds0 = lds_addr_of(smem);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int r = 8 * w + rr;
      dma16_v(wbase + (size_t)r * DC * 2 + ((lane ^ (r & 31)) << 4), lds0 + r * DC * 2);
    }
  }

  // The partials through buffer resources (32-bit offsets; the host takes this
  // kernel only when both buffers are below 2 GiB): an absent item's loads
  // get an offset past the end and return zeros.
  const __amdgpu_buffer_rsrc_t lat_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.part_lat, (short)0, (int)((size_t)a.max_items * a.H * DC * sizeof(uint16_t)), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t ml_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)pml, (short)0, (int)((size_t)a.max_items * a.H * 2 * sizeof(float)), kRawBufferWord3);
  // merge items it0 + j0 .. +3 (those below it1) of both sequences into the
  // running (v, m, L):
  //   m = max(m, m_i);  v = v 2^(m_old - m) + sum_i 2^(m_i - m) acc_i;  L likewise.
  // FIRST: nothing merged yet (v and L are written, not read).
  auto merge_group = [&](auto first, int j0, f32x4(&v)[2][2], float(&m)[2], float(&l)[2], int& flagged) {
    constexpr bool FIRST = decltype(first)::value;
    u32x4 ai[2][WNI];  // eight bf16 latent sums: columns 32 w + 8 q .. +7
#pragma unroll
    for (int jj = 0; jj < WNI; ++jj)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int i = it0[sb] + j0 + jj;
        const int off_lat = i < it1[sb] ? 2 * (DC * (i * a.H + h) + 32 * w + 8 * q) : (int)0x80000000;
        ai[sb][jj] = __builtin_amdgcn_raw_buffer_load_b128(lat_rs, off_lat, 0, 0);
      }
    // columns 4 u .. 4 u + 3 of the eight as fp32
    auto part = [&](int sb, int jj, int u) {
      const uint32_t x0 = ai[sb][jj][2 * u], x1 = ai[sb][jj][2 * u + 1];
      return f32x4{__uint_as_float(x0 << 16), __uint_as_float(x0 & 0xffff0000u), __uint_as_float(x1 << 16),
                   __uint_as_float(x1 & 0xffff0000u)};
    };
    // (m, L) after the partials: its wait then covers every load of the group
    if (tid < WNI * WCB) {
      const int i = mit0 + j0 + (tid & 3);
      const bool ok = i < mit1;
      const f32x2 ml = __builtin_bit_cast(
          f32x2, __builtin_amdgcn_raw_buffer_load_b64(ml_rs, ok ? 8 * (i * a.H + h) : (int)0x80000000, 0, 0));
      s_ml[tid & 3][tid >> 2] = f32x2{ok ? ml[0] : -INFINITY, ml[1]};
    }
    __syncthreads();
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      float mi[WNI], li[WNI];
#pragma unroll
      for (int jj = 0; jj < WNI; ++jj) {
        const f32x2 ml = s_ml[jj][16 * sb + r16];
        mi[jj] = ml[0];
        li[jj] = ml[1];
      }
      float mn = FIRST ? -INFINITY : m[sb];
#pragma unroll
      for (int jj = 0; jj < WNI; ++jj) {
        flagged |= mi[jj] == INFINITY;
        mn = fmaxf(mn, mi[jj]);
      }
      // weights 2^(m_i - mn): 0 for absent items; all 0 while nothing is merged
      const bool any = mn != -INFINITY;
      float wgt[WNI];
#pragma unroll
      for (int jj = 0; jj < WNI; ++jj) wgt[jj] = any ? exp2f(mi[jj] - mn) : 0.f;
      if constexpr (FIRST) {
#pragma unroll
        for (int u = 0; u < 2; ++u) v[sb][u] = wgt[0] * part(sb, 0, u);
        l[sb] = wgt[0] * li[0];
      } else {
        const float sc = any ? exp2f(m[sb] - mn) : 0.f;  // 0 while m = -inf
#pragma unroll
        for (int u = 0; u < 2; ++u) v[sb][u] = sc * v[sb][u] + wgt[0] * part(sb, 0, u);
        l[sb] = sc * l[sb] + wgt[0] * li[0];
      }
#pragma unroll
      for (int jj = 1; jj < WNI; ++jj) {
#pragma unroll
        for (int u = 0; u < 2; ++u) v[sb][u] += wgt[jj] * part(sb, jj, u);
        l[sb] += wgt[jj] * li[jj];
      }
      m[sb] = mn;
    }
    __syncthreads();  // s_ml is read: the next group may overwrite it
  };
  auto merge_all = [&](f32x4(&v)[2][2], float(&m)[2], float(&l)[2]) {
    int flagged = 0;
    merge_group(std::true_type{}, 0, v, m, l, flagged);
    for (int j0 = WNI; j0 < nmax; j0 += WNI)  // more than four items: later groups in order
      merge_group(std::false_type{}, j0, v, m, l, flagged);
    return flagged;
  };

  f32x4 v[2][2];
  float mrun[2], lrun[2];
  if (__syncthreads_or(merge_all(v, mrun, lrun))) {
    // a flagged partial (m = +inf): recompute it exactly, then merge again
    const int chunk = a.plan[2 * a.batch + 1];
    for (int b = 0; b < nb; ++b) {
      const int i0 = a.plan[b0 + b], i1 = a.plan[b0 + b + 1];
      const int len = a.plan[a.batch + 1 + b0 + b];
      for (int i = i0; i < i1; ++i) {
        const size_t ih = (size_t)i * a.H + h;
        if (pml[ih * 2] != INFINITY) continue;  // same value in every thread
        const int t0 = (i - i0) * chunk;
        const int t1 = min(len, t0 + chunk);
        recompute_partial(a.pool, a.block_table + (size_t)(b0 + b) * a.max_pages_per_seq,
                          (const uint16_t*)a.q_abs + ((size_t)(b0 + b) * a.H + h) * RW, a.part_lat + ih * DC,
                          a.part_ml + ih * 2, a.P, a.scale_log2, t0, t1, scr, red, a.fp8, a.num_pages, a.err);
      }
    }
    __syncthreads();
    // (the load offsets are formed again here rather than kept from the first merge)
    asm volatile("" : "+v"(it0[0]), "+v"(it1[0]), "+v"(it0[1]), "+v"(it1[1]), "+v"(mit0), "+v"(mit1));
    merge_all(v, mrun, lrun);  // recomputed partials are finite
  }

  // lat = v / L as bf16 hi + lo: the A fragments (row = sequence r16 of block
  // sb; its eight k slots hold columns 32 w + 8 q .. +7)
  u32x4 ahi[2], alo[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const float il = lrun[sb] > 0.f ? 1.f / lrun[sb] : 0.f;
    const int seq = 16 * sb + r16;
    if (w == 0 && q == 0 && seq < nb && a.lse)
      a.lse[(size_t)(b0 + seq) * a.H + h] = lrun[sb] > 0.f ? (mrun[sb] + log2f(lrun[sb])) * kLn2 : -INFINITY;
    const f32x4 x0 = v[sb][0] * il, x1 = v[sb][1] * il;
    const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t hp = pack_bf16x2(x[e], x[e + 1]);
      hw[e >> 1] = hp;
      lw[e >> 1] = pack_bf16x2(x[e] - __uint_as_float(hp << 16), x[e + 1] - __uint_as_float(hp & 0xffff0000u));
    }
    ahi[sb] = u32x4{hw[0], hw[1], hw[2], hw[3]};
    alo[sb] = u32x4{lw[0], lw[1], lw[2], lw[3]};
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's W_UV rows have landed
  __syncthreads();                            // and every other wave's

  // D_w: B = W_UV^T fragment (column v = 16 vb + lane % 16, the same eight
  // columns as the A slots): chunk 4 w + q of row 16 vb + lane % 16
  f32x4 acc[2][8];
#pragma unroll
  for (int vb = 0; vb < 8; ++vb) {
    const int row = 16 * vb + r16;
    const u32x4 bw = *(const u32x4*)(smem + row * DC * 2 + (((4 * w + q) ^ (row & 31)) << 4));
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      acc[sb][vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ahi[sb]), as_bf16x8(bw),
                                                            f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      acc[sb][vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(alo[sb]), as_bf16x8(bw), acc[sb][vb], 0, 0, 0);
    }
  }
  __syncthreads();  // W_UV reads done: the buffer takes the partial products

  // D rows: sequence 16 sb + 4 q + j, column v = 16 vb + lane % 16
  float* qs = (float*)smem;  // [w][seq][WRED_LD], v of the current half
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int vl = 0; vl < 4; ++vl)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qs[(w * WCB + 16 * sb + 4 * q + j) * WRED_LD + 16 * vl + r16] = acc[sb][4 * half + vl][j];
    __syncthreads();
    {
      const int seq = tid >> 5, v2 = 2 * (tid & 31);
      f32x2 o = *(const f32x2*)(qs + seq * WRED_LD + v2);
#pragma unroll
      for (int k = 1; k < 16; ++k) o += *(const f32x2*)(qs + (k * WCB + seq) * WRED_LD + v2);
      if (seq < nb)
        *(uint32_t*)((uint16_t*)a.out + ((size_t)(b0 + seq) * a.H + h) * 128 + 64 * half + v2) = pack_bf16x2(o[0], o[1]);
    }
    if (half == 0) __syncthreads();
  }
}

// --------------------------------------------------------------------------
// combine, one work-group per (head, sequence), for launches with few such
// pairs (H * batch <= 2 CUs, d_v = 128; the few-heads shapes): 256 threads.
//   - Each thread requests its half row of W_UV,h at once, straight into
//     registers (row t / 2, columns 256 (t % 2) .. +255: 32 16-byte loads,
//     issued after the partial loads so that the merge waits only for those).
//   - Wave s merges items it0 + s, it0 + s + 4, ... of the sequence in that
//     order; lane l holds latent columns 8 l .. 8 l + 7 (one 16-byte load of
//     a bf16 partial per item) and the running (m, L) of its set.  The four
//     sets then meet in LDS in set order (a fixed order: the result does not
//     depend on page placement).
//   - o[v] = sum_c W_UV[h][v][c] lat[c] in fp32 on the VALU: each thread its
//     half row against the merged latent in LDS, the two halves added by the
//     pair of lanes.  (One sequence per work-group: an MFMA block would be
//     1/16 used.)
constexpr int SNT = 256;  // threads per work-group
__global__ void __launch_bounds__(SNT) k_combine_seq(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float s_v[4][DC];  // per-set partial sums, then the merged latent
  __shared__ float s_m[4], s_l[4];
  __shared__ __attribute__((aligned(16))) float scr[RW + SNT];  // recompute_partial scratch
  __shared__ int red[16];
  const int h = blockIdx.x % a.H, b = blockIdx.x / a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int set = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int it0 = a.plan[b], it1 = a.plan[b + 1];
  const uint16_t* __restrict__ plat = a.part_lat;
  const float* __restrict__ pml = a.part_ml;

  // items i0, i0 + 4, i0 + 8, i0 + 12 of this wave's set (those below it1)
  auto load_group = [&](int i0, u32x4 (&pv)[4], f32x2 (&ml)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = i0 + 4 * k;
      const bool ok = i < it1;
      const size_t ih = (size_t)(ok ? i : it0) * a.H + h;
      pv[k] = ok ? *(const u32x4*)(plat + ih * DC + 8 * lane) : u32x4{0u, 0u, 0u, 0u};
      ml[k] = ok ? *(const f32x2*)(pml + 2 * ih) : f32x2{-INFINITY, 0.f};
    }
  };
  // into the running (v, m, L) in item order; flagged: some m_i = +inf
  auto merge_group = [&](const u32x4 (&pv)[4], const f32x2 (&ml)[4], f32x4 (&v)[2], float& m, float& l) {
    int flagged = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      flagged |= ml[k][0] == INFINITY;
      const float mn = fmaxf(m, ml[k][0]);
      if (mn == -INFINITY) continue;  // nothing merged yet and an absent item
      const float sc = exp2f(m - mn), wg = exp2f(ml[k][0] - mn);  // 0 for m = -inf
      const f32x4 x0 = f32x4{__uint_as_float(pv[k][0] << 16), __uint_as_float(pv[k][0] & 0xffff0000u),
                             __uint_as_float(pv[k][1] << 16), __uint_as_float(pv[k][1] & 0xffff0000u)};
      const f32x4 x1 = f32x4{__uint_as_float(pv[k][2] << 16), __uint_as_float(pv[k][2] & 0xffff0000u),
                             __uint_as_float(pv[k][3] << 16), __uint_as_float(pv[k][3] & 0xffff0000u)};
      v[0] = sc * v[0] + wg * x0;
      v[1] = sc * v[1] + wg * x1;
      l = sc * l + wg * ml[k][1];
      m = mn;
    }
    return flagged;
  };
  auto merge_rest = [&](int first, f32x4 (&v)[2], float& m, float& l) {
    int flagged = 0;
    for (int i0 = first; i0 < it1; i0 += 16) {
      u32x4 pv[4];
      f32x2 ml[4];
      load_group(i0, pv, ml);
      flagged |= merge_group(pv, ml, v, m, l);
    }
    return flagged;
  };

  f32x4 v[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  float m = -INFINITY, l = 0.f;
  u32x4 wrow[32];
  int flagged;
  {
    // the first group of partials, then this thread's W_UV,h half row: the
    // merge of the group waits for its own loads only (in-order counting)
    u32x4 pv[4];
    f32x2 ml[4];
    load_group(it0 + set, pv, ml);
    const uint16_t* wp = (const uint16_t*)a.w_uv + ((size_t)h * 128 + (tid >> 1)) * DC + 256 * (tid & 1);
#pragma unroll
    for (int k = 0; k < 32; ++k) wrow[k] = *(const u32x4*)(wp + 8 * k);
    flagged = merge_group(pv, ml, v, m, l);
    flagged |= merge_rest(it0 + set + 16, v, m, l);
  }
  if (__syncthreads_or(flagged)) {
    // a flagged partial (m = +inf): recompute it exactly, then merge again
    const int chunk = a.plan[2 * a.batch + 1];
    const int len = a.plan[a.batch + 1 + b];
    for (int i = it0; i < it1; ++i) {
      const size_t ih = (size_t)i * a.H + h;
      if (pml[ih * 2] != INFINITY) continue;  // same value in every thread
      const int t0 = (i - it0) * chunk;
      const int t1 = min(len, t0 + chunk);
      recompute_partial(a.pool, a.block_table + (size_t)b * a.max_pages_per_seq,
                        (const uint16_t*)a.q_abs + ((size_t)b * a.H + h) * RW, a.part_lat + ih * DC,
                        a.part_ml + ih * 2, a.P, a.scale_log2, t0, t1, scr, red, a.fp8, a.num_pages, a.err);
    }
    __syncthreads();
    // merge again (recomputed partials are finite)
    v[0] = v[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
    merge_rest(it0 + set, v, m, l);
  }
  *(f32x4*)(&s_v[set][8 * lane]) = v[0];
  *(f32x4*)(&s_v[set][8 * lane + 4]) = v[1];
  if (lane == 0) {
    s_m[set] = m;
    s_l[set] = l;
  }
  __syncthreads();
  // the four sets in order: lat[c] = sum_s 2^(m_s - M) v_s[c] / L
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < 4; ++k) M = fmaxf(M, s_m[k]);
  float wk[4], L = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    wk[k] = M == -INFINITY ? 0.f : exp2f(s_m[k] - M);
    L += wk[k] * s_l[k];
  }
  const float il = L > 0.f ? 1.f / L : 0.f;
  float lat[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = tid + SNT * u;
    float x = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) x += wk[k] * s_v[k][c];
    lat[u] = x * il;
  }
  if (tid == 0 && a.lse) a.lse[(size_t)b * a.H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  __syncthreads();  // every set sum is read: row 0 of s_v takes the merged latent
#pragma unroll
  for (int u = 0; u < 2; ++u) s_v[0][tid + SNT * u] = lat[u];
  __syncthreads();
  const float* lv = &s_v[0][256 * (tid & 1)];
  float o = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const f32x4 l0 = *(const f32x4*)(lv + 8 * k), l1 = *(const f32x4*)(lv + 8 * k + 4);
    const u32x4 wv = wrow[k];
    o += __uint_as_float(wv[0] << 16) * l0[0] + __uint_as_float(wv[0] & 0xffff0000u) * l0[1] +
         __uint_as_float(wv[1] << 16) * l0[2] + __uint_as_float(wv[1] & 0xffff0000u) * l0[3] +
         __uint_as_float(wv[2] << 16) * l1[0] + __uint_as_float(wv[2] & 0xffff0000u) * l1[1] +
         __uint_as_float(wv[3] << 16) * l1[2] + __uint_as_float(wv[3] & 0xffff0000u) * l1[3];
  }
  o += __shfl_xor(o, 1);
  if ((tid & 1) == 0) ((uint16_t*)a.out)[((size_t)b * a.H + h) * 128 + (tid >> 1)] = f32_to_bf16(o);
}

}  // namespace

bool decode_mfma_supported(int H, int d_c, int d_r, int d_v, int P, int batch) {
  return d_c == DC && d_r == DR && H >= 1 && H <= 128 && d_v >= 32 && d_v <= 256 && d_v % 32 == 0 && P >= TT &&
         P % TT == 0 &&
         batch <= kMaxDecodeBatch;
}

// waves per split work-group: 32 heads each, and 16 / NW latent feature
// blocks (1: at most 32 heads; the bf16 path then runs k_split<4, true>, four
// waves that all score the one head block)
static int split_waves(int H) { return H <= 32 ? 1 : (H <= 64 ? 2 : 4); }

int decode_mfma_slots(int H, int cus, bool fp8) {
  // the split kernels hold a CU's whole LDS (one work-group per CU)
  (void)H;
  (void)fp8;
  return cus;
}

int decode_mfma_grid(int slots, int max_items) {
  // rounds per work-group stay <= 64 (one per lane of the descriptor wave)
  return max(slots, (max_items + 63) / 64);
}

hipError_t decode_mfma(const DecodeArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const dim3 g1(decode_mfma_grid(a.slots, a.max_items));
  if (a.fp8) {
    switch (split_waves(a.H)) {
      case 1: hipLaunchKernelGGL(k_split8<1>, g1, dim3(64), 0, s, a); break;
      case 2: hipLaunchKernelGGL(k_split8<2>, g1, dim3(128), 0, s, a); break;
      default: hipLaunchKernelGGL(k_split8<4>, g1, dim3(256), 0, s, a); break;
    }
  } else {
    switch (split_waves(a.H)) {
      case 1:
        if (a.H <= 16) hipLaunchKernelGGL(k_split16, g1, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_split<4, true>), g1, dim3(256), 0, s, a);
        break;
      case 2: hipLaunchKernelGGL(k_split<2>, g1, dim3(128), 0, s, a); break;
      default: hipLaunchKernelGGL(k_split<4>, g1, dim3(256), 0, s, a); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.d_v == 128 && (long long)a.H * ((a.batch + WCB - 1) / WCB) >= a.slots &&
      (long long)a.max_items * a.H * DC * (long long)sizeof(uint16_t) < (1LL << 31))
    hipLaunchKernelGGL(k_combine_wide, dim3(a.H, (a.batch + WCB - 1) / WCB), dim3(1024), 0, s, a);
  else if (a.d_v == 128 && (long long)a.H * a.batch <= 2LL * a.slots)
    hipLaunchKernelGGL(k_combine_seq, dim3(a.H * a.batch), dim3(SNT), 0, s, a);
  else if ((long long)a.H * ((a.batch + 15) / 16) >= 2LL * a.slots)
    hipLaunchKernelGGL((k_combine<16, 2>), dim3(a.H, (a.batch + 15) / 16), dim3(64 * CNW), 0, s, a);
  else
    hipLaunchKernelGGL((k_combine<4, 8>), dim3(a.H, (a.batch + 3) / 4), dim3(64 * CNW), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
