// MFMA kernels of the causal prefill (gfx950, bf16; d_n = d_v = 128, d_R = 64).
//
// Prefill is compute-bound, so it takes the non-absorbed order: the per-head
// keys and values are decompressed from the latent once (yapayzekasozluk.tr
// "Multi-head Latent Attention (MLA) Nedir?", section "MLA nasil calisir?":
// K and V are rebuilt from c_KV), and attention then runs over 192-wide keys
// [K_C | k_R] and 128-wide values, 2 (192 + 128) flops per (query, key, head)
// instead of 2 (576 + 512) in the absorbed order.
//
// 1. k_prefill_proj: K_C[h][n] = W_UK,h c_n and V[h][n] = W_UV,h c_n for every
//    key token (a sequence's cached prefix and its new tokens), a GEMM
//    [tokens x d_c] x [d_c x 128] per head (32x32x16 MFMA).
//    Latent rows come from the paged pool; outputs go to the workspace as
//    bf16, head-major ([H][tokens][128]) so that one head's keys of one
//    sequence are contiguous.
// 2. k_prefill_attn_mfma: causal flash attention per (sequence, head,
//    128-query block of its new tokens; new token j sits at position
//    prefix + j and sees keys 0 .. prefix + j).  Each wave owns 32 queries.  Scores are computed
//    transposed, S^T = K Q^T, so that a lane holds all its scores for one
//    query: the softmax numerators then feed the P.V MFMA straight from
//    registers as its B operand, and the V^T operand comes from LDS transpose
//    reads in the matching key order.  Key tiles of 32 keys (K_C, k_R, V)
//    stream HBM -> LDS by DMA through a 4-stage ring.
#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

__device__ __forceinline__ int seq_of(const int32_t* __restrict__ cu, int num_seqs, int n) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= n) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int PD = 128;  // d_n = d_v
constexpr int PDR = 64;  // d_R

// ---------------------------------------------------------------- up-projection
// One work-group per (128 key tokens, head): K_C and V together, a
// [128 x 512] . [512 x 256] product whose 256 weight rows are W_UK,h then
// W_UV,h, so each latent row fetched serves both.  32-wide k chunks of the 128
// latent rows (gathered through the block table) and the 256 weight rows
// stream into a three-stage LDS ring by direct-to-LDS loads, two chunks
// ahead, one barrier per chunk; two work-groups share a CU.  Wave (wo, wt) =
// (w / 2, w % 2) computes outputs of W block wo (K_C or V) for tokens
// 64 wt .. +63: 4 x 2 MFMA blocks, so a k step reads 6 fragments for 8 MFMAs.
// (One work-group per K_C or V with 32 x 128 wave tiles read 5 fragments per
// 4 MFMAs, and the LDS port, shared with the loads, set its pace: 0.80 ms
// for the V3 prefill's 16,384 keys.)
constexpr int XT = 128;                      // tokens per work-group
constexpr int XW = 2 * PD;                   // weight rows: W_UK,h then W_UV,h
constexpr int XK = 32;                       // latent columns per k-chunk (64-byte rows)
constexpr int XNS = 3;                       // stages
constexpr int XSTAGE = (XT + XW) * XK * 2;   // 24 KiB: 128 latent rows, then 256 weight rows
constexpr int XLPW = (XT + XW) / 16 / 4;     // loads per wave per stage (6)

// LDS stage row r (64 bytes): 16-byte piece c at slot c ^ ((r >> 2) & 3)
// (the 16 rows of a quarter-wave's fragment reads cover all 64 banks).
__device__ __forceinline__ int xslot(int r, int c) { return c ^ ((r >> 2) & 3); }

__global__ void __launch_bounds__(256, 2) k_prefill_proj(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[XNS * XSTAGE];
  const int n0 = blockIdx.x * XT, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int wo = w >> 1, wt = w & 1;
  const int N = a.total_kv, R = a.d_c + a.d_r;  // every key token: cached prefix and new
  const char* __restrict__ Wk = (const char*)a.w_uk + (size_t)h * PD * a.d_c * 2;
  const char* __restrict__ Wv = (const char*)a.w_uv + (size_t)h * PD * a.d_c * 2;
  const uint32_t lds0 = lds_addr_of(smem);

  // loads: instruction k (0..23) of a stage fills LDS bytes [1024 k, +1024):
  // rows 16 k' + lane / 4 (k' = k for the latent block, k < 8; k' = k - 8 of
  // the weight block: W_UK,h rows for k' < 8, W_UV,h rows after), slot
  // lane % 4 holding source piece slot ^ ((row >> 2) & 3).  Wave w issues
  // k = w + 4 i (i < 6): latent rows for i < 2, W_UK,h for i < 4, W_UV,h after.
  const char* crow[2];
  uint32_t cchunk[2], woff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * (w + 4 * i) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const int n = min(n0 + r, N - 1);
    const int s = seq_of(a.cu_kv, a.num_seqs, n);
    // clamped so that the block-table read stays in row s (max_kv_len <= capacity)
    const int t = key_position(n, a.cu_kv[s], a.max_kv_len, a.err);
    const int page = checked_page(a.block_table[(size_t)s * a.max_pages_per_seq + t / a.P], a.num_pages, a.err);
    crow[i] = (const char*)a.pool + ((size_t)page * a.P + t % a.P) * (size_t)R * 2;
    cchunk[i] = 16u * c;
    // weight rows of loads i + 2 and i + 4: row r of W_UK,h, then of W_UV,h
    // (r % 128 = r, (r + 128) >> 2 & 3 = r >> 2 & 3: the same slot)
    woff[i] = (uint32_t)(r * a.d_c * 2 + 16 * c);
  }
  auto issue = [&](int kc, int st) {
    const uint32_t base = lds0 + st * XSTAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16_v(crow[i] + 64 * kc + cchunk[i], base + 1024 * (w + 4 * i));
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16<0>(Wk + 64 * kc, woff[i], base + XT * XK * 2 + 1024 * (w + 4 * i));
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16<0>(Wv + 64 * kc, woff[i], base + XT * XK * 2 + 1024 * (8 + w + 4 * i));
  };

  f32x16 acc[4][2];  // [output block jt][token block tb]
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) acc[jt][tb] = f32x16{};
  const int nk = a.d_c / XK;
#pragma unroll
  for (int c = 0; c < XNS - 1; ++c)
    if (c < nk) issue(c, c);
  for (int kc = 0; kc < nk; ++kc) {
    // chunk kc has landed once at most the next chunk's loads remain
    if (kc + 1 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_vm(XLPW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();  // chunk kc in LDS; chunk kc-1's stage no longer read
    asm volatile("" ::: "memory");
    if (kc + XNS - 1 < nk) issue(kc + XNS - 1, (kc + XNS - 1) % XNS);
    const char* st = smem + (kc % XNS) * XSTAGE;
#pragma unroll
    for (int ks = 0; ks < XK / 16; ++ks) {
      const int c = 2 * ks + g;
      u32x4 bt[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int rt = 64 * wt + 32 * tb + r32;  // B column: token
        bt[tb] = *(const u32x4*)(st + rt * (XK * 2) + 16 * xslot(rt, c));
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int rw = PD * wo + 32 * jt + r32;  // A row: weight row (output)
        const u32x4 aw = *(const u32x4*)(st + XT * XK * 2 + rw * (XK * 2) + 16 * xslot(rw, c));
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[jt][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aw), as_bf16x8(bt[tb]), acc[jt][tb], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave is done with the stages: the epilogue reuses them

  // The products are D^T: lane holds token 64 wt + 32 tb + lane % 32 and
  // outputs j = 32 jt + 8 (e/4) + 4 g + e % 4 of block wo, four consecutive j
  // per e/4, stored as one 8-byte bf16 group.  Staged as bf16
  // [wo][token][128], 16-byte slot (j / 8) ^ (token % 16), then written in
  // whole 256-byte rows.
  uint16_t* ot = (uint16_t*)smem;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int tk = 64 * wt + 32 * tb + r32;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int eg = 0; eg < 4; ++eg) {
        const int j0 = 32 * jt + 8 * eg + 4 * g;
        const u32x2 v = {pack_bf16x2(acc[jt][tb][4 * eg], acc[jt][tb][4 * eg + 1]),
                         pack_bf16x2(acc[jt][tb][4 * eg + 2], acc[jt][tb][4 * eg + 3])};
        *(u32x2*)(ot + (wo * XT + tk) * PD + 8 * ((j0 >> 3) ^ (tk & 15)) + (j0 & 7)) = v;
      }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2 * XT * 16 / 256; ++i) {
    const int u = i * 256 + tid, wb = u / (XT * 16), tk = (u >> 4) % XT, c = u & 15;
    uint16_t* dst = (uint16_t*)(wb ? a.ws_v : a.ws_k) + ((size_t)h * N + n0) * PD;
    if (n0 + tk < N)
      *(u32x4*)(dst + (size_t)tk * PD + 8 * c) = *(const u32x4*)(ot + (wb * XT + tk) * PD + 8 * (c ^ (tk & 15)));
  }
}

// ---------------------------------------------------------------- attention
constexpr int AQ = 128;  // queries per work-group (4 waves x 32)
constexpr int AK = 32;   // keys per tile
constexpr int ST_KC = 0;                   // K_C tile: 32 rows x 256 bytes, slot c ^ (r % 16)
constexpr int ST_KR = AK * PD * 2;         // k_R tile: 32 rows x 128 bytes, slot c ^ ((r >> 1) % 8)
constexpr int ST_V = ST_KR + AK * PDR * 2;  // V tile: 32 rows x 256 bytes, slot c ^ 4 (r % 4)
constexpr int ST_BYTES = ST_V + AK * PD * 2;  // 20480
constexpr int NST = 4;
constexpr int LPT = 5;  // loads per wave per tile (20 wave-wide loads)
constexpr float kLazy = 8.f;     // log2 headroom of the softmax reference maximum
constexpr float kMInit = -1e30f;
constexpr bf16x2 kOnes2 = {(__bf16)1.f, (__bf16)1.f};

__global__ void __launch_bounds__(256, 2) k_prefill_attn_mfma(PrefillArgs a, int nqb) {
  __shared__ __attribute__((aligned(16))) char smem[NST * ST_BYTES];
  // work item: (sequence, head) pair and query block; the query blocks of one
  // pair run on one XCD (work-group i runs on XCD i % 8), heaviest first
  const int id = blockIdx.x;
  const int pairs = a.num_seqs * a.H;
  int pair, qr;
  if ((pairs & 7) == 0) {
    const int slot = id >> 3;
    pair = (slot / nqb) * 8 + (id & 7);
    qr = slot % nqb;
  } else {
    pair = id / nqb;
    qr = id % nqb;
  }
  const int qb = nqb - 1 - qr;
  const int s = pair / a.H, h = pair % a.H;
  // new tokens cu0 .. cu0 + len - 1 of q / out; the sequence's keys (a cached
  // prefix, then the new tokens) are key tokens ck0 .. ck0 + klen - 1 of the
  // workspace and positions 0 .. klen - 1 of the cache
  const PrefillSeq sd = prefill_seq(a.cu_q, a.cu_kv, s, a.total, a.total_kv, a.max_seq_len, a.max_kv_len,
                                    (qr == 0 && h == 0) ? a.err : nullptr);
  const int cu0 = sd.q0, len = sd.q_len;
  const int ck0 = sd.k0, klen = sd.kv_len;
  const int prefix = klen - len;
  const int q0 = qb * AQ;  // query block, in new-token indices
  if (q0 >= len) return;
  const int qend = min(len, q0 + AQ);
  const int n_kt = (prefix + qend + AK - 1) / AK;

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int N = a.total_kv, R = a.d_c + a.d_r;
  const int ql_lane = q0 + 32 * w + r32;  // this lane's query (new-token index)
  const bool qvalid = ql_lane < qend;
  const int qi = prefix + ql_lane;        // its position in the sequence
  const int w_last = prefix + min(qend - 1, q0 + 32 * w + 31);
  const bool w_any = q0 + 32 * w < qend;
  const int kt_last = w_any ? w_last / AK : -1;  // last tile this wave computes
  // tiles before kt_mask hold only keys at or before the wave's first query
  const int kt_mask = w_any ? min(kt_last + 1, (prefix + q0 + 32 * w + 1) / AK) : 0;

  // query fragments (B operand of S^T = K Q^T): query = lane % 32,
  // k = 16 ks + 8 g .. +7; ks < 8: q_C, ks >= 8: RoPE(q_R, qi) rounded to bf16
  u32x4 qf[12];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((size_t)(cu0 + (qvalid ? ql_lane : q0)) * a.H + h) * (PD + PDR) + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) qf[ks] = *(const u32x4*)(qp + 16 * ks);
    // lane l computes theta of pair l % 32 once; the lanes share them
    const double th_l = rope_inv_freq(lane & 31, PDR, a.rope_base);
#pragma unroll
    for (int ks = 8; ks < 12; ++ks) {
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t pr = qf[ks][e];
        const float x0 = __uint_as_float(pr << 16), x1 = __uint_as_float(pr & 0xffff0000u);
        float c, sn;
        rope_cs_theta(qi, __shfl(th_l, (16 * (ks - 8) + 8 * g) / 2 + e), c, sn);
        o[e] = pack_bf16x2(x0 * c - x1 * sn, x0 * sn + x1 * c);
      }
      qf[ks] = u32x4{o[0], o[1], o[2], o[3]};
    }
  }

  // tile loads: wave w issues loads u = w + 4 i (i < 5) of the 20, so the
  // kind of load depends on i alone: i < 2 K_C rows 4 u .. +3 (u = w + 4 i);
  // i = 2 k_R rows 8 w .. +7; i > 2 V rows 4 (w + 4 (i - 3)) .. +3.  The lane
  // offsets are fixed per wave; only the last tile of a sequence can be
  // ragged, and there rows past the end repeat its last key (masked in the
  // scores).
  const char* __restrict__ kc_base = (const char*)a.ws_k + ((size_t)h * N + ck0) * (PD * 2);
  const char* __restrict__ v_base = (const char*)a.ws_v + ((size_t)h * N + ck0) * (PD * 2);
  const int32_t* __restrict__ bt = a.block_table + (size_t)s * a.max_pages_per_seq;
  const uint32_t lds0 = lds_addr_of(smem);
  int lrow[LPT], lcol[LPT];
  uint32_t loff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    if (i < 2) {
      lrow[i] = 4 * (w + 4 * i) + (lane >> 4);
      lcol[i] = 16 * ((lane & 15) ^ (lrow[i] & 15));
    } else if (i == 2) {
      lrow[i] = 8 * w + (lane >> 3);
      lcol[i] = 16 * ((lane & 7) ^ ((lrow[i] >> 1) & 7));
    } else {
      lrow[i] = 4 * (w + 4 * (i - 3)) + (lane >> 4);
      lcol[i] = 16 * ((lane & 15) ^ (4 * (lrow[i] & 3)));
    }
    loff[i] = (uint32_t)(lrow[i] * (i == 2 ? R * 2 : PD * 2) + lcol[i]);
  }
  // the block-table entry of a tile is read one iteration before its loads
  // are issued, so the scalar load never stalls the wave (P % 32 == 0: a
  // tile lies in one page; pages and in-page tiles advance by counting)
  // (through the constant address space: a scalar load, counted by lgkmcnt
  // and not by the vmcnt that tracks the tile loads)
  const __attribute__((address_space(4))) int32_t* bt_c = (const __attribute__((address_space(4))) int32_t*)bt;
  const int tpp = a.P / AK, pg_last = (n_kt - 1) / tpp;
  const uint32_t page_bytes = (uint32_t)(a.P * R * 2), tile_bytes = (uint32_t)(AK * R * 2);
  const char* __restrict__ kr_pool = (const char*)a.pool + a.d_c * 2;
  auto issue = [&](int kt, int page, int in_page) {
    page = checked_page(page, a.num_pages, a.err);
    const int key0 = kt * AK;
    const int maxr = klen - 1 - key0;
    const char* kr_base = kr_pool + (size_t)(uint32_t)page * page_bytes + (uint32_t)in_page * tile_bytes;
    const char* kc_t = kc_base + (size_t)key0 * (PD * 2);
    const char* v_t = v_base + (size_t)key0 * (PD * 2);
    const uint32_t st = lds0 + (kt & (NST - 1)) * ST_BYTES;
    auto loads = [&](auto ragged) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        uint32_t off = loff[i];
        if constexpr (decltype(ragged)::value)
          off = (uint32_t)(min(lrow[i], maxr) * (i == 2 ? R * 2 : PD * 2) + lcol[i]);
        if (i < 2) dma16<0>(kc_t, off, st + ST_KC + 1024 * (w + 4 * i));
        else if (i == 2) dma16<0>(kr_base, off, st + ST_KR + 1024 * w);
        else dma16<0>(v_t, off, st + ST_V + 1024 * (w + 4 * (i - 3)));
      }
    };
    if (maxr >= AK - 1) loads(std::false_type{});
    else loads(std::true_type{});
  };

  // V^T fragment offsets (A operand of O^T += V^T P^T): lane (d = lane % 32, g)
  // needs keys 4 g + 0..3 (lo) and 8 + 4 g + 0..3 (hi) of each 16-key half;
  // the transpose read of a 16-lane group takes 4 rows x 32 bytes.
  const int grp = lane >> 4, jl = lane & 15;
  const int trow = 4 * g + (jl >> 2);          // + 16 kk (+ 8 for hi); trow % 4 = jl >> 2
  const int tch = 2 * (grp & 1) + ((jl & 3) >> 1);  // + 4 dt
  int voff[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) voff[hf] = ST_V + (trow + 8 * hf) * 256 + 8 * (jl & 1);
  // slot swizzle of these rows: the two 16-lane groups that share an LDS
  // cycle read chunk pairs 4 dt + {0, 1} and 4 dt + {2, 3} of rows with
  // r % 4 = 0..3; XOR by 4 (r % 4) spreads them over all 16 chunks (64 banks)
  const int vsw = 4 * (jl >> 2);

  const float sl2 = a.scale * kLog2e;
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  // m: reference maximum of this lane's query (log2 units).  It moves only
  // when a tile's maximum exceeds it by more than kLazy, so numerators stay
  // below 2^kLazy and the accumulator is rescaled on few tiles.  It starts
  // finite so that a fully masked score never meets inf - inf.
  float m = kMInit, l = 0.f;

  // page and in-page tile of the next tile to load (tile 3 after the
  // prologue), and its block-table entry
  int ld_pg = 3 / tpp, ld_in = 3 % tpp;
  int next_page = bt_c[min(ld_pg, pg_last)];
  auto sync = [&](int kt) {
    // tile kt+3's page (read one sync earlier), then the next entry's scalar
    // load, in flight over the wait and the barrier below
    const int page3 = next_page, in3 = ld_in;
    if (++ld_in == tpp) {
      ld_in = 0;
      ++ld_pg;
    }
    next_page = bt_c[min(ld_pg, pg_last)];
    // tile kt has landed once at most the later tiles' loads are in flight
    if (kt + 2 < n_kt) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPT));
    else if (kt + 1 < n_kt) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPT));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();  // tile kt in LDS; tile kt-1's stage no longer read
    // the scalar load is done by now; waiting for it here lets the tile's
    // first score MFMA wait for its own K fragment only (a scalar load in
    // flight forces every LDS wait to count down to zero)
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    if (kt + 3 < n_kt) issue(kt + 3, page3, in3);
  };

  // One key tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  MASKED is
  // the diagonal tile (keys past the query); every earlier tile is full.
  auto tile = [&](int kt, auto masked) {
    const char* st = smem + (kt & (NST - 1)) * ST_BYTES;
    // S^T[key][query], key = lane-row of A: 8 steps over K_C, 4 over k_R
    u32x4 kf[12];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      kf[ks] = *(const u32x4*)(st + ST_KC + r32 * 256 + 16 * ((2 * ks + g) ^ (r32 & 15)));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf[8 + ks] = *(const u32x4*)(st + ST_KR + r32 * 128 + 16 * ((2 * ks + g) ^ ((r32 >> 1) & 7)));
    __builtin_amdgcn_sched_barrier(0);  // all reads in flight before the chain starts
    f32x16 sc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 12; ++ks)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[ks]), as_bf16x8(qf[ks]), sc, 0, 0, 0);
    // V^T fragments of this tile, read while the softmax below runs
    s16x4 vf[2][4][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int sl = (4 * dt + tch) ^ vsw;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          vf[kk][dt][hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + voff[hf] + 16 * kk * 256 + 16 * sl));
      }
    __builtin_amdgcn_sched_barrier(0);
    // sc[j]: key kt*32 + 8 (j/4) + 4 g + j % 4 against query qi
    if constexpr (decltype(masked)::value) {
      const int rel = qi - kt * AK - 4 * g;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (8 * (j >> 2) + (j & 3) > rel) sc[j] = -INFINITY;
    }
    float mt = sc[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mt = fmaxf(mt, sc[j]);
    {
      // lanes l and l + 32 hold the two key halves of one query
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float mts = mt * sl2;  // scale > 0: the maximum commutes with it
    if (__ballot(mts > m + kLazy)) {
      const float mn = fmaxf(m, mts);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
      m = mn;
    }
    const float nm = -m;
    u32x4 pk[2];
    float ls = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t wd[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const f32x2 pf = {__builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * kk + e], sl2, nm)),
                          __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * kk + e + 1], sl2, nm))};
        const bf16x2 pb = __builtin_convertvector(pf, bf16x2);
        ls = __builtin_amdgcn_fdot2_f32_bf16(pb, kOnes2, ls, false);  // the rounded numerators
        wd[e >> 1] = __builtin_bit_cast(uint32_t, pb);
      }
      pk[kk] = u32x4{wd[0], wd[1], wd[2], wd[3]};
    }
    l += ls;
    // O^T[d][query] += V^T[d][keys] P^T[keys][query]
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const s16x4 lo = vf[kk][dt][0], hi = vf[kk][dt][1];
        const s16x8 av = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), as_bf16x8(pk[kk]), acc[dt], 0, 0, 0);
      }
  };

#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (t < n_kt) issue(t, bt_c[t / tpp], t % tpp);
  // every wave takes part in all n_kt barriers and loads; it computes
  // tiles 0 .. kt_last, of which those from kt_mask on meet the diagonal (one
  // tile for a fresh sequence, at most two after a prefix that is not a
  // multiple of 32)
  int kt = 0;
  for (; kt < kt_mask; ++kt) {
    sync(kt);
    tile(kt, std::false_type{});
  }
  for (; kt <= kt_last; ++kt) {
    sync(kt);
    tile(kt, std::true_type{});
  }
  for (; kt < n_kt; ++kt) sync(kt);

  // out[query][h][d] = O^T[d][query] / l: staged as bf16 rows [query][128]
  // (16-byte slot (d / 8) ^ (query % 16)), then written in whole rows
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid && g == 0 && a.lse) a.lse[(size_t)(cu0 + ql_lane) * a.H + h] = (m + log2f(lt)) * kLn2;
  __syncthreads();  // every wave is done with the tile stages
  uint16_t* ot = (uint16_t*)smem;
  const int ql = 32 * w + r32;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      // rows d and d+1 of one lane are e and e + 1 (same 8-aligned group)
      const int d = 32 * dt + 8 * (e >> 2) + 4 * g + (e & 3);
      *(uint32_t*)(ot + ql * PD + 8 * ((d >> 3) ^ (ql & 15)) + (d & 7)) =
          pack_bf16x2(acc[dt][e] * inv, acc[dt][e + 1] * inv);
    }
  __syncthreads();
  uint16_t* out = (uint16_t*)a.out;
#pragma unroll
  for (int i = 0; i < AQ * 16 / 256; ++i) {
    const int u = i * 256 + tid, qq = u >> 4, c = u & 15;
    if (q0 + qq < qend)
      *(u32x4*)(out + ((size_t)(cu0 + q0 + qq) * a.H + h) * PD + 8 * c) = *(const u32x4*)(ot + qq * PD + 8 * (c ^ (qq & 15)));
  }
}

}  // namespace

bool prefill_mfma_supported(int d_n, int d_v, int d_r, int d_c, int P) {
  return d_n == PD && d_v == PD && d_r == PDR && d_c % XK == 0 && d_c >= XK && P % AK == 0;
}

hipError_t prefill_mfma(const PrefillArgs& a, hipStream_t s) {
  if (a.total == 0 || a.num_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prefill_proj, dim3((a.total_kv + XT - 1) / XT, a.H), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (a.max_seq_len + AQ - 1) / AQ;
  if (nqb == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prefill_attn_mfma, dim3(a.num_seqs * a.H * nqb), dim3(256), 0, s, a, nqb);
  return hipGetLastError();
}

}  // namespace mla
