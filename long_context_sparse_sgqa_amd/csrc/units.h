// Per-token and per-pair lists of selected 8-token units, shared by the attention kernels.
//
// A unit u covers tokens 8u .. 8u+7.  A list entry is unit | (mask << 24), mask bit e saying that
// token 8u+e lies in a selected block.  The lists are built by one wavefront from a token's
// ascending block selection.
#pragma once

#include "device_common.h"

namespace sgqa {

// ------------------------------------------------------------------------------------------------
// Unit lists.  An entry is unit | (mask << 24): unit u covers tokens 8u .. 8u+7, mask bit e says
// token 8u+e belongs to a selected block.
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ int lane_lt_count(uint64_t bal, int lane) {
  return __popcll(bal & ((1ull << lane) - 1ull));
}

// Expands one token's selection (NS entries; entries outside [0, o] are ignored) into its sorted
// unit list; returns the entry count.  B is a multiple of 8 or divides 8.
__device__ inline int build_units(const int32_t* __restrict__ selrow, int NS, int B, int64_t o,
                           uint32_t* list, int lane) {
  int running = 0;
  if (B >= 8) {
    const int U = B >> 3;
    for (int base = 0; base < NS; base += 64) {
      const int e = base + lane;
      const int blk = (e < NS) ? selrow[e] : -1;
      const bool valid = blk >= 0 && blk <= o;
      const uint64_t bal = __ballot(valid);
      if (valid) {
        const int pos = running + U * lane_lt_count(bal, lane);
        for (int u = 0; u < U; ++u) list[pos + u] = static_cast<uint32_t>(blk * U + u) | (0xffu << 24);
      }
      running += U * __popcll(bal);
    }
  } else {
    const uint32_t bmask = (1u << B) - 1u;
    for (int base = 0; base < NS; base += 64) {
      const int e = base + lane;
      const int blk = (e < NS) ? selrow[e] : -1;
      const bool valid = blk >= 0 && blk <= o;
      const int unit = (blk * B) >> 3;
      bool head = false;
      uint32_t mask = 0u;
      if (valid) {
        const int prev = (e > 0) ? selrow[e - 1] : -1;
        const bool prev_valid = prev >= 0 && prev <= o;
        head = !(prev_valid && ((prev * B) >> 3) == unit);
        if (head) {
          mask = bmask << ((blk * B) & 7);
          for (int k2 = 1; k2 < 8 && e + k2 < NS; ++k2) {
            const int nb2 = selrow[e + k2];
            if (!(nb2 >= 0 && nb2 <= o) || ((nb2 * B) >> 3) != unit) break;
            mask |= bmask << ((nb2 * B) & 7);
          }
        }
      }
      const uint64_t bal = __ballot(head);
      if (head) list[running + lane_lt_count(bal, lane)] = static_cast<uint32_t>(unit) | (mask << 24);
      running += __popcll(bal);
    }
  }
  return running;
}

// Number of entries of a sorted unit list whose unit is <= last_unit.
__device__ inline int count_units_upto(const uint32_t* list, int n, int64_t last_unit, int lane) {
  int cnt = 0;
  for (int base = 0; base < n; base += 64) {
    const int e = base + lane;
    const bool keep = e < n && static_cast<int64_t>(list[e] & 0xffffffu) <= last_unit;
    cnt += __popcll(__ballot(keep));
  }
  return cnt;
}

__device__ __forceinline__ int lower_bound_units(const uint32_t* list, int n, uint32_t unit) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((list[mid] & 0xffffffu) < unit) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Union of the two sorted unit lists: uunit[] ascending, umask[] = maskA | maskB << 8.
__device__ inline int merge_units(const uint32_t* la, int na, const uint32_t* lb, int nb, int32_t* uunit,
                           uint32_t* umask, int lane) {
  int dups = 0;
  for (int base = 0; base < na; base += 64) {
    const int i = base + lane;
    const uint32_t ea = (i < na) ? la[i] : 0u;
    const uint32_t ua = ea & 0xffffffu;
    const int x = (i < na) ? lower_bound_units(lb, nb, ua) : 0;
    const bool eq = (i < na) && x < nb && (lb[x] & 0xffffffu) == ua;
    const uint64_t bal = __ballot(eq);
    if (i < na) {
      const int pos = i + x - (dups + lane_lt_count(bal, lane));
      uunit[pos] = static_cast<int32_t>(ua);
      umask[pos] = (ea >> 24) | (eq ? ((lb[x] >> 24) << 8) : 0u);
    }
    dups += __popcll(bal);
  }
  int dups_b = 0;
  for (int base = 0; base < nb; base += 64) {
    const int j = base + lane;
    const uint32_t eb = (j < nb) ? lb[j] : 0u;
    const uint32_t ub = eb & 0xffffffu;
    const int x = (j < nb) ? lower_bound_units(la, na, ub) : 0;
    const bool eq = (j < nb) && x < na && (la[x] & 0xffffffu) == ub;
    const uint64_t bal = __ballot(eq);
    if (j < nb && !eq) {
      const int pos = j + x - (dups_b + lane_lt_count(bal, lane));
      uunit[pos] = static_cast<int32_t>(ub);
      umask[pos] = (eb >> 24) << 8;
    }
    dups_b += __popcll(bal);
  }
  return na + nb - dups;
}

// Byte offset, within one (sequence, group) of unit-packed K, of the 16-byte operand that lane
// (lr, lg) feeds to the S^T product of d-slice kc for rows 4h..4h+3 of unit u.  Packed K stores
// k[8u + 4h + r][32kc + 8lg + e] at element ((u * D/32 + kc) * 2 + h) * 128 + (lg * 4 + r) * 8 + e.
__device__ __forceinline__ int kp_offset(int u, int D, int kc, int h, int lg, int lr) {
  return u * D * 16 + (((kc * 2 + h) * 4 + lg) * 4 + (lr & 3)) * 16;
}

// Unit-packed K for the 4-token kernels: k[8u + t][16kc + 8h + e] is stored at element
// ((u * D/16 + kc) * 8 + t) * 16 + h * 8 + e, so the 16 lanes that feed one unit's 8 tokens x 2
// halves of a 16-wide d-slice to v_mfma_f32_32x32x16_bf16 read one contiguous 256-byte block.
__device__ __forceinline__ int kq_offset(int u, int D, int kc, int t, int h) {
  return u * D * 16 + ((kc * 8 + t) * 2 + h) * 16;
}

}  // namespace sgqa
