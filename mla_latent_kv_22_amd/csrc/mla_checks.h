// Index checks of MLA_DEBUG builds and the clamps of device-side lengths.
// Plain C++ with no device-only code, so that the same predicates also
// compile for the host (the CPU test suite builds them with g++ and checks
// that every result stays inside the caller's buffers).
#pragma once

#include <stdint.h>

#include "../../include/mla.h"

#if defined(__HIPCC__)
#define MLA_HD __host__ __device__ __forceinline__
#else
#define MLA_HD inline
#endif

namespace mla {

// A library built with MLA_DEBUG checks every device-side index before it
// forms an address from it; a release build compiles the checks out.  A bad
// value sets a bit of the device error word (MLA_DEVERR_*) and is replaced
// by one that stays inside the caller's buffers.  A null err reports nothing.
#ifdef MLA_DEBUG
constexpr bool kChecked = true;
#else
constexpr bool kChecked = false;
#endif

MLA_HD void report_error(int* err, int bit) {
  if (!err) return;
#if defined(__HIP_DEVICE_COMPILE__)
  atomicOr(err, bit);
#else
  *err |= bit;
#endif
}

MLA_HD int clamp_int(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// A block-table entry: outside [0, num_pages) it becomes page 0.
template <bool CHECK = kChecked>
MLA_HD int checked_page(int page, int num_pages, int* err) {
  if (CHECK && (unsigned)page >= (unsigned)num_pages) {
    report_error(err, MLA_DEVERR_PAGE);
    return 0;
  }
  return page;
}

// A slot_mapping entry: outside [-1, num_pages * P) it becomes -1 (skipped).
template <bool CHECK = kChecked>
MLA_HD long long checked_slot(long long slot, int num_pages, int P, int* err) {
  if (CHECK && (slot < -1 || slot >= (long long)num_pages * P)) {
    report_error(err, MLA_DEVERR_SLOT);
    return -1;
  }
  return slot;
}

// v clamped to [lo, hi] (lo <= hi), in every build; MLA_DEBUG builds report
// a change.
template <bool CHECK = kChecked>
MLA_HD int clamp_report(int v, int lo, int hi, int* err) {
  const int c = clamp_int(v, lo, hi);
  if (CHECK && c != v) report_error(err, MLA_DEVERR_LENGTH);
  return c;
}

// One sequence of a prefill: new-token rows [q0, q0 + q_len) and key tokens
// [k0, k0 + kv_len), the device offsets clamped to the host bounds so that
// no row or block-table entry outside the caller's buffers is touched (the
// rule stated for mla_prefill_kv in include/mla.h).  Needs total_q >= 0,
// total_kv >= 0, max_q_len >= 0, max_kv_len >= 0.
struct PrefillSeq {
  int q0, q_len, k0, kv_len;
};
template <bool CHECK = kChecked>
MLA_HD PrefillSeq prefill_seq(const int32_t* cu_q, const int32_t* cu_kv, int s, int total_q, int total_kv,
                              int max_q_len, int max_kv_len, int* err) {
  PrefillSeq r;
  r.q0 = clamp_report<CHECK>(cu_q[s], 0, total_q, err);
  const int qhi = max_q_len < total_q - r.q0 ? max_q_len : total_q - r.q0;
  r.q_len = clamp_report<CHECK>(cu_q[s + 1] - r.q0, 0, qhi, err);
  r.k0 = clamp_report<CHECK>(cu_kv[s], 0, total_kv, err);
  const int khi = max_kv_len < total_kv - r.k0 ? max_kv_len : total_kv - r.k0;
  r.kv_len = clamp_report<CHECK>(cu_kv[s + 1] - r.k0, 0, khi, err);
  r.q_len = clamp_report<CHECK>(r.q_len, 0, r.kv_len, err);
  return r;
}

// Key position t of a key token whose sequence was found by a search over
// cu_kv: clamped to [0, max_kv_len - 1], so that the block-table entry
// t / P stays in the sequence's row (the host checks
// max_kv_len <= max_pages_per_seq * P).  Needs max_kv_len >= 1.
template <bool CHECK = kChecked>
MLA_HD int key_position(int n, int seq_start, int max_kv_len, int* err) {
  return clamp_report<CHECK>(n - seq_start, 0, max_kv_len - 1, err);
}

// Tokens per work item of the decode's split pass.  items(ch) must return
// the item count at chunk ch: the sum over sequences of ceil(len / ch).  Work
// item i runs in round i / slots of its work-group, so a plan costs
//   rounds * (chunk + round_ovh)  +  items * ovh / slots
// in cache-row equivalents: the tokens of the busiest work-group, what a
// round costs besides its tokens (the item's query fragments and pipeline
// fill, which every work-group meets at the same time), and the partial
// results written and merged.
// Candidates:
//   - chunk = total / (k slots) for k = 1, 2, 4 (rounded up to 32): the k = 1
//     plan always fits the partial buffers (items <= slots + batch);
//   - when the best of those leaves the busiest work-group more than 5% (and
//     a tile) above the mean and the batch has at most 2 slots sequences
//     (long contexts, not many short ones), for r = 2 .. 4 rounds the chunk that makes the
//     items fit r * slots: estimated as total / (r slots - batch / 2) (each
//     sequence's last item is on average half a chunk short) and raised at
//     most three times by the ratio of items to r * slots.
// Every chunk is a multiple of 32 in [min_chunk, max_chunk], and no plan with
// more than max_items items is taken.  The result depends only on the
// arguments and items(), so every work-group computes the same plan.
template <class Items>
MLA_HD int choose_chunk(long long total, int batch, int slots, int min_chunk, int max_chunk, int ovh_tokens,
                        int round_ovh, int max_items, Items items) {
  int best_chunk = 0;
  long long best_cost = -1, best_work = 0;
  auto round32 = [&](long long c) {
    c = ((c + 31) / 32) * 32;
    return (int)(c < min_chunk ? min_chunk : (c > max_chunk ? max_chunk : c));
  };
  auto consider = [&](int ch, long long it, bool always) {
    if (!always && it > max_items) return;
    const long long rounds = (it + slots - 1) / slots;
    const long long cost = rounds * (ch + round_ovh) + (it * ovh_tokens) / slots;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_chunk = ch;
      best_work = rounds * ch;
    }
  };
  for (int k = 1; k <= 4; k <<= 1) {
    const int ch = round32((total + (long long)k * slots - 1) / ((long long)k * slots));
    consider(ch, items(ch), k == 1);
  }
  const long long mean = (total + slots - 1) / slots;
  if (best_work > mean + mean / 20 + 32 && batch <= 2 * slots) {
    for (int r = 2; r <= 4; ++r) {
      const long long cap = (long long)r * slots;
      const long long den = cap - batch / 2 > cap / 2 ? cap - batch / 2 : cap / 2;
      int ch = round32((total + den - 1) / den);
      long long it = items(ch);
      for (int t = 0; t < 3 && it > cap && ch < max_chunk; ++t) {
        ch = round32(((long long)ch * it + cap - 1) / cap);
        it = items(ch);
      }
      if (it <= cap) consider(ch, it, false);
    }
  }
  return best_chunk;
}

// Block map of the fused cache write + absorption launch (k_write_absorb).
// Work-group x runs on XCD x % 8.  The S split-K slices of the hidden axis
// are dealt to the XCDs in turn (slice s on XCD s % 8), and the first
// nfb * (slices of XCD c) work-groups of XCD c are the write tiles of its
// slices, so the nfb tiles that read the same h columns share one L2.  Every
// other work-group is an absorption work-group; its rank counts the
// absorption work-groups below it.
MLA_HD int wa_xcd_slices(int c, int S) { return c < S ? (S - 1 - c) / 8 + 1 : 0; }

struct WaRole {
  bool write;
  int fb, s;  // write tile: feature block, slice
  int rank;   // absorption work-group: heads rank, rank + n_ablocks, ...
};
MLA_HD WaRole wa_role(int x, int S, int nfb) {
  WaRole r{false, 0, 0, 0};
  const int c = x & 7, j = x >> 3;
  if (j < nfb * wa_xcd_slices(c, S)) {
    r.write = true;
    r.fb = j % nfb;
    r.s = c + 8 * (j / nfb);
    return r;
  }
  for (int cc = 0; cc < 8; ++cc) {
    const int below = x > cc ? (x - cc + 7) / 8 : 0;  // work-groups x' < x on XCD cc
    const int w = nfb * wa_xcd_slices(cc, S);
    r.rank += below > w ? below - w : 0;
  }
  return r;
}

// Grid of the launch: at least nfb * S write tiles plus n_ablocks (>= 1)
// absorption work-groups, and far enough for the last write tile of every
// XCD (the j-th work-group of XCD c is 8 j + c).  n_ablocks becomes the
// grid's absorption work-group count.
MLA_HD int wa_grid(int S, int nfb, int& n_ablocks) {
  int grid = nfb * S + n_ablocks;
  for (int c = 0; c < 8; ++c) {
    const int tiles = nfb * wa_xcd_slices(c, S);
    if (tiles > 0 && grid < 8 * (tiles - 1) + c + 1) grid = 8 * (tiles - 1) + c + 1;
  }
  n_ablocks = grid - nfb * S;
  return grid;
}

}  // namespace mla
