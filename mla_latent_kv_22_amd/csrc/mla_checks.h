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

}  // namespace mla
