// Step 4, range-split variant: gated GQA over the selected tokens for groups of 4 adjacent query
// tokens, with each group's selected units split into R contiguous unit ranges that run on
// different XCDs and are merged afterwards.
//
// Same method as attend.hip (Step 5 Preview pages, mo.ai.kr summary, section
// "모델 구조와 학습 안정성": Sparse GQA on Gated GQA attends only over each KV group's selected
// blocks, and batching adjacent tokens, whose selections overlap, raises GPU utilisation).
// Gathering the selected K/V units is what bounds this step.  Two things cut that traffic here:
//   * a wavefront serves 4 adjacent tokens x 8 heads = 32 rows (the M of v_mfma_f32_32x32x16_bf16)
//     and walks the union of their selections, so a unit chosen by several of the 4 tokens is
//     loaded once (the union of 4 tokens is ~0.84x the units that 2 pairs would load);
//   * range r of every group goes to the workgroups numbered r mod R, which the dispatcher deals to
//     XCDs r, r+R, ..., so each XCD's L2 caches only 1/R of a KV group's keys and values.  With
//     fewer groups of 4 tokens than waves per workgroup (decode), a workgroup's waves take one
//     group's R ranges instead, so that no wave idles.
//
// Three kernels:
//   quad_union_kernel  per (sequence, group, 4 tokens): the sorted union of the tokens' selected
//     8-token units, entry = unit | chosen-by-token-t << (27 + t) (B is a multiple of 8, so a unit
//     is wholly selected by a token or not at all), built through LDS bitmaps into an LDS copy
//     of the list that is written out coalesced; every range is padded to a multiple of 4
//     entries and its first entry recorded.  Past 128K tokens (with B = 8 and at most 512
//     selected blocks) quad_union_merge_kernel builds the same list by merging the tokens'
//     ascending selections instead of through bitmaps.
//   attend_range_kernel  one wavefront per (group of 4 tokens, range): the entries inside the
//     range in chunks of 4 units (32 tokens).  S^T = K Q^T on D/16 MFMAs with the K rows permuted
//     so that every lane holds the 16 scores of one row for two units; masks, online softmax in
//     the exp2 domain, O^T += V^T P^T on D/16 MFMAs whose P operand is a lane's own probabilities.
//     K comes from the unit-packed copy laid out for this kernel and V from the unit-packed V,
//     so every 16-lane operand load is one 256-byte run; K is loaded two chunks and V one chunk
//     ahead, list entries arrive by scalar loads, and Q is read from LDS.  The result per row:
//     O / l rounded to bf16 (the wave's tile written out coalesced through its Q slice of LDS),
//     and the running max m and sum l in fp32.
//   merge_ranges_kernel  per row: weight each partial by its sum rescaled to the common max,
//     combine, apply sigmoid(gate), round to bf16.
#include "device_common.h"
#include "sgqa_internal.h"
#include "units.h"

namespace sgqa {
namespace {

constexpr int kRanges = 4;                      // unit ranges per group of tokens
constexpr int kRangeWaves = 4;                  // token groups per workgroup (one per wave)
constexpr int kTok = 4;                         // query tokens per group
constexpr uint32_t kUnitMask = 0x07ffffffu;     // entry bits 0..26: unit; 27..30: chosen bits
constexpr int kChoseShift = 27;
// Entries of one group's list: the union (at most kTok umax) with every range padded to a multiple
// of 4 entries, plus 16 entries the range kernel may read (and discard) past the end of the last
// chunk.
__host__ __device__ constexpr int64_t list_stride(int umax) {
  return (kTok * static_cast<int64_t>(umax) + 4 * kRanges + 16 + 3) / 4 * 4;
}

// Unit ranges of a group: range r covers units [r * u_end / R, (r + 1) * u_end / R) of the
// group's causal unit axis [0, u_end), u_end = the last token's own unit + 1.
__device__ __forceinline__ uint32_t range_start(int r, int64_t u_end) {
  return static_cast<uint32_t>((r * u_end) / kRanges);
}

__device__ __forceinline__ int64_t group_u_end(int64_t pos0, int64_t tok0, int64_t Tq) {
  const int64_t last = (tok0 + kTok - 1 < Tq ? tok0 + kTok - 1 : Tq - 1);
  return ((pos0 + last) >> 3) + 1;
}

// ------------------------------------------------------------------------------------------------
// unions of 4 tokens' selections
// ------------------------------------------------------------------------------------------------
struct UnionArgs {
  const int32_t* sel;
  uint32_t* ulist;         // [Bt * G * ngroups][list_stride(umax)]
  int32_t* bounds;         // [Bt * G * ngroups][kRanges + 1]: first entry of each range, then end
  int64_t Tq, pos0, ngroups, total;
  const int32_t* seq_len;  // per-sequence key counts, or null
  int G, NS, B, umax, words, waves;   // words: bitmap words per token (ceil(NU / 32))
  // ranges of equal entry counts instead of equal unit spans: for launches whose attention waves
  // take a group's ranges in one workgroup (decode), where no L2 locality across groups is to be
  // kept and the slowest range ends the launch
  int balance;
};

// LDS words per wave of the group-list kernel: the four bitmaps and the list, one after the other,
// or overlapping when the bitmaps' words are held in registers.
__host__ __device__ constexpr int64_t union_lds_words(int64_t words, int64_t stride, bool overlap) {
  return overlap ? (kTok * words > stride ? kTok * words : stride) : kTok * words + stride;
}

// Each selected block sets its units' bits in the token's LDS bitmap (units past the token's own
// unit are left out: t <= p); one scan over the words then emits the union in ascending unit order
// with every token's chosen bit.
// kVec4: the bitmap scans read 4 words per token at a time (16-byte LDS reads).  That pays for
// long contexts, where the bitmaps' LDS size leaves few waves per CU to hide each read's latency;
// with short bitmaps and many waves the scalar scans are faster.
// kRegW > 0 (scalar scans, at most 64 kRegW words per token): each lane keeps its words of the four
// bitmaps in registers from the counting pass on, so the list is built in LDS over the bitmaps
// and a wave needs only max(4 words, list stride) words of LDS.
template <bool kVec4, int kRegW>
__global__ void __launch_bounds__(256) quad_union_kernel(UnionArgs a) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gq = static_cast<int64_t>(blockIdx.x) * a.waves + wave;  // (b*G + g)*ngroups + q
  if (gq >= a.total) return;                          // whole wave; no workgroup barriers below
  // this wave's LDS: the 4 tokens' bitmaps, then the list being built (copied out at the end)
  const int64_t stride = list_stride(a.umax);
  uint32_t* bm = lds + static_cast<size_t>(wave) * union_lds_words(a.words, stride, kRegW > 0);
  uint32_t* stg = kRegW > 0 ? bm : bm + kTok * a.words;
  // group indices fit 32 bits (fewer groups than rows, < 2^31): 32-bit divisions, a fraction of
  // a 64-bit division's scalar instructions at one short-lived wave per group of tokens
  const uint32_t gq32 = static_cast<uint32_t>(gq), ng32 = static_cast<uint32_t>(a.ngroups);
  const uint32_t bg32 = gq32 / ng32, b32 = bg32 / static_cast<uint32_t>(a.G);
  const int64_t qi = gq32 - bg32 * ng32;
  const int64_t g = bg32 - b32 * static_cast<uint32_t>(a.G), b = b32;
  const int64_t tok0 = kTok * qi;
  const int64_t pos0 = seq_pos0(a.seq_len, b, a.pos0, a.Tq);
  const int64_t u_end = group_u_end(pos0, tok0, a.Tq);
  const int nw = static_cast<int>((u_end + 31) >> 5);
  const int U = a.B >> 3;                               // units per block
  // The selections of budgets up to 512 blocks are loaded at once (8 entries per lane and token),
  // so the four tokens cost one memory round trip, and the bitmaps are cleared meanwhile.
  constexpr int kPer = 8;
  int blk[kTok][kPer];
  const bool in_regs = a.NS <= 64 * kPer && U == 1;     // B = 8 (a block is one unit)
  if (in_regs) {
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      const int64_t tt = tok0 + t < a.Tq ? tok0 + t : tok0;
      const int32_t* selrow = a.sel + ((b * a.Tq + tt) * a.G + g) * a.NS;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int e = lane + 64 * k;
        blk[t][k] = (e < a.NS && tok0 + t < a.Tq) ? selrow[e] : -1;
      }
    }
  }
  for (int w = lane; w < nw; w += 64) {
#pragma unroll
    for (int t = 0; t < kTok; ++t) bm[t * a.words + w] = 0u;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // each token's own block and last unit, once per token (positions fit 32 bits: NU < 2^31 / 8),
  // so that the unrolled marking below stays a few instructions per selection
  int32_t o_t[kTok], lu_t[kTok];
#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    const int32_t p = static_cast<int32_t>(pos0 + tok0 + t);
    o_t[t] = p / a.B;
    lu_t[t] = p >> 3;
  }
  if (in_regs) {
    // one unit per block: a selected causal block sets its unit's bit (its unit is <= the token's)
#pragma unroll
    for (int t = 0; t < kTok; ++t)
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int bk = blk[t][k];
        if (bk >= 0 && bk <= o_t[t]) atomicOr(&bm[t * a.words + (bk >> 5)], 1u << (bk & 31));
      }
  } else {
#pragma unroll 1
    for (int t = 0; t < kTok; ++t) {
      if (tok0 + t >= a.Tq) break;
      const int32_t* selrow = a.sel + ((b * a.Tq + tok0 + t) * a.G + g) * a.NS;
#pragma unroll 1
      for (int e = lane; e < a.NS; e += 64) {
        const int bk = selrow[e];
        if (bk < 0 || bk > o_t[t]) continue;
        for (int k = 0; k < U; ++k) {                    // units of the block up to the token's own
          const int32_t u = bk * U + k;
          if (u <= lu_t[t]) atomicOr(&bm[t * a.words + (u >> 5)], 1u << (u & 31));
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // each lane owns a contiguous run of words, whole groups of 4 (one 16-byte read per token; a
  // token's bitmap is a multiple of 4 words, and words past the run read as 0: those past nw were
  // never cleared); counts below each range start and in total
  const int per = kVec4 ? ((((nw + 63) >> 6) + 3) & ~3) : ((nw + 63) >> 6);
  const int w0 = lane * per, w1 = min(w0 + per, nw);
  auto read4 = [&](int w, uint32_t (*xt)[4]) {
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      const uint4 v = *reinterpret_cast<const uint4*>(bm + t * a.words + w);
      xt[t][0] = w < w1 ? v.x : 0u;
      xt[t][1] = w + 1 < w1 ? v.y : 0u;
      xt[t][2] = w + 2 < w1 ? v.z : 0u;
      xt[t][3] = w + 3 < w1 ? v.w : 0u;
    }
  };
  uint32_t lo[kRanges];
#pragma unroll
  for (int r = 0; r < kRanges; ++r) lo[r] = range_start(r, u_end);
  int mine = 0;
  int below[kRanges + 1];
#pragma unroll
  for (int r = 0; r <= kRanges; ++r) below[r] = 0;
  auto count_word = [&](int w, uint32_t x) {
    mine += __popc(x);
#pragma unroll
    for (int r = 1; r < kRanges; ++r) {
      const int64_t rel = static_cast<int64_t>(lo[r]) - 32 * w;   // bits of this word below lo[r]
      const uint32_t m = rel >= 32 ? 0xffffffffu : (rel <= 0 ? 0u : ((1u << rel) - 1u));
      below[r] += __popc(x & m);
    }
  };
  uint32_t xr[kTok][kRegW > 0 ? kRegW : 1];
  if constexpr (kVec4) {
    for (int w4 = w0; w4 < w1; w4 += 4) {
      uint32_t xt4[kTok][4];
      read4(w4, xt4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t x = 0u;
#pragma unroll
        for (int t = 0; t < kTok; ++t) x |= xt4[t][k];
        count_word(w4 + k, x);
      }
    }
  } else if constexpr (kRegW > 0) {
#pragma unroll
    for (int k = 0; k < kRegW; ++k) {
      const int w = w0 + k;
      uint32_t x = 0u;
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        xr[t][k] = w < w1 ? bm[t * a.words + w] : 0u;
        x |= xr[t][k];
      }
      count_word(w, x);
    }
    // every lane's words are in registers: the list may now overwrite the bitmaps
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  } else {
    for (int w = w0; w < w1; ++w) {
      uint32_t x = 0u;
#pragma unroll
      for (int t = 0; t < kTok; ++t) x |= bm[t * a.words + w];
      count_word(w, x);
    }
  }
  // exclusive prefix of `mine` over the lanes, and the totals
  const int incl = wave_inclusive_scan(mine);
  const int nu = __builtin_amdgcn_readlane(incl, 63);
  int pos = incl - mine;
#pragma unroll
  for (int r = 1; r < kRanges; ++r) below[r] = a.balance ? (r * nu) / kRanges : wave_total(below[r]);
  below[0] = 0;
  below[kRanges] = nu;
  int start[kRanges + 1];
  start[0] = 0;
#pragma unroll
  for (int r = 0; r < kRanges; ++r) start[r + 1] = start[r] + ((below[r + 1] - below[r] + 3) & ~3);

  uint32_t* out = a.ulist + gq * stride;
  // A lane meets its units in increasing order, so it carries its current range, that range's
  // output shift and the next range's first unit, and updates them only when it crosses a start.
  // Entries go to the LDS copy of the list: a lane's entries are one contiguous run, so stores of
  // them straight to memory would give every entry of a store instruction its own cache line.
  auto shift_of = [&](int r) {
    int v = 0;
#pragma unroll
    for (int q = 0; q < kRanges; ++q) v = q == r ? start[q] - below[q] : v;
    return v;
  };
  auto next_start = [&](int r) {
    uint32_t v = 0xffffffffu;
#pragma unroll
    for (int q = 1; q < kRanges; ++q) v = q == r + 1 ? lo[q] : v;
    return v;
  };
  // Equal entry counts: a range starts at an entry position (below[r]), not at a unit.
  auto next_below = [&](int r) {
    int v = 0x7fffffff;
#pragma unroll
    for (int q = 1; q < kRanges; ++q) v = q == r + 1 ? below[q] : v;
    return v;
  };
  int rcur = 0;
#pragma unroll
  for (int q = 1; q < kRanges; ++q)
    rcur += (a.balance ? pos >= below[q] : static_cast<uint32_t>(32 * w0) >= lo[q]) ? 1 : 0;
  int shift = shift_of(rcur);
  uint32_t nxt = next_start(rcur);
  int nxt_pos = next_below(rcur);
  auto emit_word = [&](int w, const uint32_t* xt) {
    uint32_t x = 0u;
#pragma unroll
    for (int t = 0; t < kTok; ++t) x |= xt[t];
    while (x) {
      const int bit = __builtin_ctz(x);
      x &= x - 1u;
      const uint32_t u = static_cast<uint32_t>(32 * w + bit);
      if (a.balance ? pos >= nxt_pos : u >= nxt) {      // crossed a range start (rare)
        do {
          ++rcur;
          nxt = next_start(rcur);
          nxt_pos = next_below(rcur);
        } while (a.balance ? pos >= nxt_pos : u >= nxt);
        shift = shift_of(rcur);
      }
      uint32_t chose = 0u;
#pragma unroll
      for (int t = 0; t < kTok; ++t) chose |= __builtin_amdgcn_ubfe(xt[t], bit, 1) << t;
      stg[pos + shift] = u | (chose << kChoseShift);
      ++pos;
    }
  };
  if constexpr (kVec4) {
    for (int w4 = w0; w4 < w1; w4 += 4) {
      uint32_t xt4[kTok][4];
      read4(w4, xt4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t xt[kTok];
#pragma unroll
        for (int t = 0; t < kTok; ++t) xt[t] = xt4[t][k];
        emit_word(w4 + k, xt);
      }
    }
  } else if constexpr (kRegW > 0) {
#pragma unroll
    for (int k = 0; k < kRegW; ++k) {
      uint32_t xt[kTok];
#pragma unroll
      for (int t = 0; t < kTok; ++t) xt[t] = xr[t][k];
      if (w0 + k < w1) emit_word(w0 + k, xt);
    }
  } else {
    for (int w = w0; w < w1; ++w) {
      uint32_t xt[kTok];
#pragma unroll
      for (int t = 0; t < kTok; ++t) xt[t] = bm[t * a.words + w];
      emit_word(w, xt);
    }
  }
  if (lane < 4 * kRanges) {                      // padding entries (unit 0, chosen by none)
    const int r = lane >> 2, j = start[r] + (below[r + 1] - below[r]) + (lane & 3);
    if (j < start[r + 1]) stg[j] = 0u;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // the list (a multiple of 4 entries; both copies 16-byte aligned) with consecutive lanes on
  // consecutive 16-byte pieces
  {
    const int n4 = start[kRanges] >> 2;
    const uint4* src = reinterpret_cast<const uint4*>(stg);
    uint4* dst = reinterpret_cast<uint4*>(out);
    for (int j = lane; j < n4; j += 64) dst[j] = src[j];
  }
  int32_t* bnd = a.bounds + gq * (kRanges + 1);
  if (lane <= kRanges) {
    int v = 0;
#pragma unroll
    for (int q = 0; q <= kRanges; ++q) v = q == lane ? start[q] : v;
    bnd[lane] = v;
  }
}

// Long contexts with B = 8 (a block is one unit) and at most 512 selected blocks, ranges of equal
// unit spans: the union by merging the 4 tokens' selections, which arrive in ascending block
// order, instead of through bitmaps (which at 1M tokens take 64 KiB of LDS per group of tokens).
// Lane l owns the units [l u_end / 64, (l + 1) u_end / 64), so lanes 16 r .. 16 r + 15 own range
// r: it finds each selection's run in its span by binary search, counts the distinct units of
// the four runs by a 4-way merge, and after a prefix over the lanes merges them again into the
// LDS copy of the list.  Searches and merges are bounded by the list indices, so any input stays
// in bounds.
constexpr int kMergeSel = 512;                  // selected blocks per token held in LDS
__global__ void __launch_bounds__(256) quad_union_merge_kernel(UnionArgs a) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gq = static_cast<int64_t>(blockIdx.x) * a.waves + wave;
  if (gq >= a.total) return;                          // whole wave; no workgroup barriers below
  const int64_t stride = list_stride(a.umax);
  int32_t* L = reinterpret_cast<int32_t*>(lds + static_cast<size_t>(wave) * (kTok * kMergeSel + stride));
  uint32_t* stg = reinterpret_cast<uint32_t*>(L + kTok * kMergeSel);
  // group indices fit 32 bits (fewer groups than rows, < 2^31): 32-bit divisions, a fraction of
  // a 64-bit division's scalar instructions at one short-lived wave per group of tokens
  const uint32_t gq32 = static_cast<uint32_t>(gq), ng32 = static_cast<uint32_t>(a.ngroups);
  const uint32_t bg32 = gq32 / ng32, b32 = bg32 / static_cast<uint32_t>(a.G);
  const int64_t qi = gq32 - bg32 * ng32;
  const int64_t g = bg32 - b32 * static_cast<uint32_t>(a.G), b = b32;
  const int64_t tok0 = kTok * qi;
  const int64_t pos0 = seq_pos0(a.seq_len, b, a.pos0, a.Tq);
  const int64_t u_end = group_u_end(pos0, tok0, a.Tq);
  // the selections, blocks past a token's own (or of tokens past Tq, or -1 padding) as INT_MAX
#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    const int64_t tt = tok0 + t < a.Tq ? tok0 + t : tok0;
    const int32_t* selrow = a.sel + ((b * a.Tq + tt) * a.G + g) * a.NS;
    const int32_t o_t = static_cast<int32_t>((pos0 + tok0 + t) >> 3);
#pragma unroll
    for (int k = 0; k < kMergeSel / 64; ++k) {
      const int e = lane + 64 * k;
      const int bk = (e < a.NS && tok0 + t < a.Tq) ? selrow[e] : -1;
      L[t * kMergeSel + e] = (bk >= 0 && bk <= o_t) ? bk : 0x7fffffff;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // first index of each selection at or above a unit (binary search over the 512 entries)
  auto lower = [&](int t, int32_t v) {
    int lo = 0, hi = kMergeSel;
#pragma unroll 1
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (L[t * kMergeSel + mid] < v) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  const int32_t c0 = static_cast<int32_t>((lane * u_end) >> 6);
  const int32_t c1 = static_cast<int32_t>(((lane + 1) * u_end) >> 6);
  int p0[kTok], p1[kTok];
#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    p0[t] = lower(t, c0);
    p1[t] = lower(t, c1);
  }
  // 4-way merge of the lane's runs; `visit(unit, chosen bits)` per distinct unit
  auto merge = [&](auto visit) {
    int i[kTok];
    int32_t hd[kTok];
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      i[t] = p0[t];
      hd[t] = i[t] < p1[t] ? L[t * kMergeSel + i[t]] : 0x7fffffff;
    }
#pragma unroll 1
    while (true) {
      int32_t m = hd[0];
#pragma unroll
      for (int t = 1; t < kTok; ++t) m = min(m, hd[t]);
      if (m == 0x7fffffff) break;
      uint32_t chose = 0u;
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        if (hd[t] == m) {
          chose |= 1u << t;
#pragma unroll 1
          while (i[t] < p1[t] && L[t * kMergeSel + i[t]] == m) ++i[t];   // duplicates included
          hd[t] = i[t] < p1[t] ? L[t * kMergeSel + i[t]] : 0x7fffffff;
        }
      }
      visit(static_cast<uint32_t>(m), chose);
    }
  };
  int mine = 0;
  merge([&](uint32_t, uint32_t) { ++mine; });
  // lanes 16 r .. 16 r + 15 are range r: the counts below each range start from the lane prefix
  const int incl = wave_inclusive_scan(mine);
  const int nu = __builtin_amdgcn_readlane(incl, 63);
  int pos = incl - mine;
  int below[kRanges + 1];
  below[0] = 0;
#pragma unroll
  for (int r = 1; r < kRanges; ++r) below[r] = __builtin_amdgcn_readlane(pos, 16 * r);
  below[kRanges] = nu;
  int start[kRanges + 1];
  start[0] = 0;
#pragma unroll
  for (int r = 0; r < kRanges; ++r) start[r + 1] = start[r] + ((below[r + 1] - below[r] + 3) & ~3);
  const int rl = lane >> 4;
  int shift = 0;
#pragma unroll
  for (int q = 0; q < kRanges; ++q) shift = q == rl ? start[q] - below[q] : shift;
  merge([&](uint32_t u, uint32_t chose) {
    stg[pos + shift] = u | (chose << kChoseShift);
    ++pos;
  });
  if (lane < 4 * kRanges) {                      // padding entries (unit 0, chosen by none)
    const int r = lane >> 2, j = start[r] + (below[r + 1] - below[r]) + (lane & 3);
    if (j < start[r + 1]) stg[j] = 0u;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  uint32_t* out = a.ulist + gq * stride;
  {
    const int n4 = start[kRanges] >> 2;
    const uint4* src = reinterpret_cast<const uint4*>(stg);
    uint4* dst = reinterpret_cast<uint4*>(out);
    for (int j = lane; j < n4; j += 64) dst[j] = src[j];
  }
  int32_t* bnd = a.bounds + gq * (kRanges + 1);
  if (lane <= kRanges) {
    int v = 0;
#pragma unroll
    for (int q = 0; q <= kRanges; ++q) v = q == lane ? start[q] : v;
    bnd[lane] = v;
  }
}

// ------------------------------------------------------------------------------------------------
// sliding-window lists: every token of a group attends to the contiguous units of its window
// ------------------------------------------------------------------------------------------------
struct WindowArgs {
  uint32_t* ulist;
  int32_t* bounds;
  int64_t Tq, pos0, ngroups, total;
  int win_m1, umax;
};

// One wave per group of 4 tokens: units from the first token's window start to the last token's
// own unit, all marked as chosen by every token present (the range kernel masks each token's
// window and causal limit per token), split into kRanges equal unit ranges padded to 4 entries.
__global__ void __launch_bounds__(256) window_lists_kernel(WindowArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t gq = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gq >= a.total) return;
  const int64_t qi = gq % a.ngroups;
  const int64_t tok0 = kTok * qi;
  const int64_t p0 = a.pos0 + tok0;
  const int64_t u_lo = (p0 - a.win_m1 > 0 ? p0 - a.win_m1 : 0) >> 3;
  const int64_t u_end = group_u_end(a.pos0, tok0, a.Tq);
  const int64_t n = u_end - u_lo;
  uint32_t bits = 0u;
#pragma unroll
  for (int t = 0; t < kTok; ++t) bits |= (tok0 + t < a.Tq ? 1u : 0u) << (kChoseShift + t);
  uint32_t* out = a.ulist + gq * list_stride(a.umax);
  int start = 0;
#pragma unroll
  for (int r = 0; r < kRanges; ++r) {
    const int64_t lo = u_lo + (r * n) / kRanges, hi = u_lo + ((r + 1) * n) / kRanges;
    const int cnt = static_cast<int>(hi - lo), padded = (cnt + 3) & ~3;
    for (int j = lane; j < padded; j += 64)
      out[start + j] = j < cnt ? (static_cast<uint32_t>(lo + j) | bits) : 0u;
    if (lane == 0) a.bounds[gq * (kRanges + 1) + r] = start;
    start += padded;
  }
  if (lane == 0) a.bounds[gq * (kRanges + 1) + kRanges] = start;
}

// ------------------------------------------------------------------------------------------------
// one unit range of one group of 4 tokens
// ------------------------------------------------------------------------------------------------
struct RangeArgs {
  const bf16_t* q;
  const bf16_t* kp;        // unit-packed K, 4-token layout (kq_offset)
  const bf16_t* vp;        // unit-packed V [.., unit, d, 8 tokens]
  const uint32_t* ulist;
  const int32_t* bounds;
  bf16_t* part_o;          // [gq][R][32 rows][D], normalised by the partial's own sum
  float2* part_ml;         // [gq][R][32 rows]  (running max in the exp2 domain, sum)
  int64_t Tq, Tk, NU, pos0, ngroups, wg_groups;
  int G, umax;
  // fewer groups of tokens than waves per workgroup (decode): one workgroup per group of tokens,
  // its waves the unit ranges, so that no wave is idle (else the waves are kRangeWaves
  // consecutive groups of tokens of one range)
  int wave_ranges;
  float scale_log2e;
  const int32_t* seq_len;      // per-sequence key counts, or null
  // paged cache (kPaged): kp / vp are the page pools, unit u of sequence b lives in page
  // block_table[b * max_pages + (u >> ul2)] at unit u & (2^ul2 - 1)
  const int32_t* block_table;
  int64_t max_pages, num_pages;
  int ul2;
  int win_m1;                  // sliding window: tokens t >= p - win_m1 only (huge: no window)
  float v_scale;               // fp8 K/V: dequantisation scale of V (k_scale is in scale_log2e)
};

// 8 fp8 e4m3 values (two dwords, bytes in element order) as 8 bf16 operand values.  Every e4m3
// value is exactly representable in bf16, so the conversion is exact.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v w = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
  return __builtin_bit_cast(bf16x8_t, w);
}

// K rows of the S^T product, permuted: output r' (0..15) of a lane in half h is C row
// 8 (r'/4) + 4h + r'%4, and should hold token r' % 8 of unit slot (r' < 8 ? h : 2 + h).  So K
// row i (an A operand row, i = lane % 32) is token kq_tok(i) of unit slot kq_slot(i).
__device__ __forceinline__ int kq_slot(int i) {
  const int h = (i >> 2) & 1, j = (i >> 3) * 4 + (i & 3);
  return j < 8 ? h : 2 + h;
}
__device__ __forceinline__ int kq_tok(int i) { return ((i >> 3) * 4 + (i & 3)) & 7; }

template <int D, bool kPaged, bool kFp8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) attend_range_kernel(RangeArgs a) {
  constexpr int H = 8;
  constexpr int kQRow = D * 2 + 16;                      // padded LDS row of Q (bytes)
  __shared__ __attribute__((aligned(16))) unsigned char s_q[kRangeWaves][32 * kQRow];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int c = lane & 31, h = lane >> 5;                // Q row (token c/8, head c%8), lane half
  const int trow = c >> 3, head = c & 7;
  static_assert(kRanges == kRangeWaves, "one wave per range when the waves are the ranges");
  int r;
  int64_t bg, qi;
  if (a.wave_ranges) {
    r = wave;
    bg = blockIdx.x / a.ngroups;
    qi = blockIdx.x - bg * a.ngroups;
  } else {
    // workgroup id: range fastest, so the range decides the XCD
    r = static_cast<int>(blockIdx.x % kRanges);
    const int64_t rest = blockIdx.x / kRanges;
    const int64_t wgq = rest % a.wg_groups;
    bg = rest / a.wg_groups;
    qi = wgq * kRangeWaves + wave;
    if (qi >= a.ngroups) return;                         // whole wave; no workgroup barriers follow
  }
  const int g = static_cast<int>(bg % a.G);
  const int64_t b = bg / a.G;
  const int64_t gq = bg * a.ngroups + qi;
  const int64_t tok0 = kTok * qi;
  const bool rowvalid = tok0 + trow < a.Tq;
  const int64_t pX = seq_pos0(a.seq_len, b, a.pos0, a.Tq) + tok0 + trow;
  // Units holding the group's tokens' own positions (wave-uniform): only there can a row attend to
  // part of a unit (or, with a sliding window, at its start: windowed launches check every chunk).
  const int64_t pfirst = seq_pos0(a.seq_len, b, a.pos0, a.Tq) + tok0;
  const uint32_t own_lo = static_cast<uint32_t>(pfirst >> 3);
  const bool windowed = a.win_m1 < (1 << 29);

  const uint32_t* list = a.ulist + gq * list_stride(a.umax);
  const int32_t* bnd = a.bounds + gq * (kRanges + 1);
  const int e0 = __builtin_amdgcn_readfirstlane(bnd[r]);
  const int e1 = __builtin_amdgcn_readfirstlane(bnd[r + 1]);

  // Q rows of the group into this wave's LDS slice: lane (c, h) copies d in [D/2 h, D/2 (h+1))
  unsigned char* sq = &s_q[wave][0];
  {
    const bf16_t* qrow = a.q + (((b * a.Tq + (rowvalid ? tok0 + trow : tok0)) * a.G + g) * H + head) * D;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
      const int d = (D / 2) * h + 8 * k;
      const uint4 v = rowvalid ? *reinterpret_cast<const uint4*>(qrow + d) : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(sq + c * kQRow + d * 2) = v;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // Q^T operand of d-slice kc: B[8h + e][c] = q[c][16 kc + 8h + e]
  auto q_operand = [&](int kc) -> bf16x8_t {
    return bf16x8_from_u4(*reinterpret_cast<const uint4*>(sq + c * kQRow + (16 * kc + 8 * h) * 2));
  };

  constexpr int64_t kElem = kFp8 ? 1 : 2;                 // bytes per packed K/V element
  const BufRsrc krs = make_rsrc(reinterpret_cast<const char*>(a.kp) + (b * a.G + g) * a.NU * D * 8 * kElem,
                                a.NU * D * 8 * kElem);
  const BufRsrc vrs = make_rsrc(reinterpret_cast<const char*>(a.vp) + (b * a.G + g) * a.NU * D * 8 * kElem,
                                a.NU * D * 8 * kElem);

  // List entries are read with scalar loads (constant address space, wave-uniform, 16-byte aligned
  // because ranges start at multiples of 4): they count against lgkmcnt, so reading them never
  // waits behind the K/V loads in flight.  Entries at or past e1 read as 0 (unit 0, not chosen).
  // On a paged cache the page of each entry's unit is looked up the same way, giving the unit's
  // index in the pools (pu4).
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) u32x4* ConstQuadPtr;
  typedef const __attribute__((address_space(4))) int32_t* ConstIntPtr;
  const int32_t* btrow = kPaged ? a.block_table + b * a.max_pages : nullptr;
  const uint32_t umask_pg = (1u << a.ul2) - 1u;
  auto chunk_entries = [&](int cpos, uint32_t* ent4, uint32_t* pu4) {
    const u32x4 v = *((ConstQuadPtr)(list + cpos));
#pragma unroll
    for (int j = 0; j < 4; ++j) ent4[j] = cpos < e1 ? v[j] : 0u;
    if constexpr (kPaged) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u = ent4[j] & kUnitMask;
        int64_t page = *((ConstIntPtr)(btrow + (u >> a.ul2)));
        page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
        pu4[j] = static_cast<uint32_t>(((page * a.G + g) << a.ul2) | (u & umask_pg));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) pu4[j] = 0u;
    }
  };
  auto pick4 = [](const uint32_t* v, int i) -> uint32_t {
    return i == 0 ? v[0] : (i == 1 ? v[1] : (i == 2 ? v[2] : v[3]));
  };

  // K operands of a chunk: A row c = token kq_tok(c) of unit slot kq_slot(c), d-half h.  With fp8
  // K and V the registers hold the raw bytes (one 16-byte load covers two operands) and are
  // converted to bf16 right before the products.
  const int kslot = kq_slot(c), ktok = kq_tok(c);
  // One register set holds either a chunk's K operands or its V operands (the same size): the
  // pipeline below rotates three sets through both roles.
  struct OpRegs {
    bf16x8_t k[kFp8 ? 1 : D / 16];
    uint4 r[kFp8 ? D / 32 : 1];
  };
  auto load_k = [&](const uint32_t* ent4, const uint32_t* pu4, OpRegs& R) {
    if constexpr (kFp8) {
      // fp8 unit layout: bytes ((m * 8 + t) * 2 + h) * 16 hold d 32m + 8h + [0, 8) then
      // 32m + 16 + 8h + [0, 8) of token t
      const int u = static_cast<int>(pick4(ent4, kslot) & kUnitMask);
#pragma unroll
      for (int m = 0; m < D / 32; ++m)
        R.r[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     krs, u * D * 8 + ((m * 8 + ktok) * 2 + h) * 16, 0, 0));
    } else if constexpr (kPaged) {
      const bf16_t* base = a.kp + static_cast<uint64_t>(pick4(pu4, kslot)) * (D * 8) + (ktok * 2 + h) * 8;
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) R.k[kc] = load_bf16x8(base + kc * 128);
    } else {
      const int u = static_cast<int>(pick4(ent4, kslot) & kUnitMask);
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) R.k[kc] = buffer_load_bf16x8(krs, kq_offset(u, D, kc, ktok, h));
    }
  };
  auto k_op = [&](const OpRegs& K, int kc) -> bf16x8_t {
    if constexpr (kFp8) {
      const uint4 w = K.r[kc >> 1];
      return (kc & 1) ? fp8x8_to_bf16(w.z, w.w) : fp8x8_to_bf16(w.x, w.y);
    } else {
      return K.k[kc];
    }
  };
  // V^T operands of d-tile dt for the units of slot h (first product) and slot 2 + h (second).
  auto load_v = [&](const uint32_t* ent4, const uint32_t* pu4, OpRegs& R) {
    if constexpr (kFp8) {
      // fp8 unit layout: bytes (n * 32 + c) * 16 hold tokens 0..7 of d 64n + c, then of 64n + 32 + c
      const int ua = static_cast<int>(pick4(ent4, h) & kUnitMask);
      const int ub = static_cast<int>(pick4(ent4, 2 + h) & kUnitMask);
#pragma unroll
      for (int n = 0; n < D / 64; ++n) {
        R.r[2 * n] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                         vrs, ua * D * 8 + (n * 32 + c) * 16, 0, 0));
        R.r[2 * n + 1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                             vrs, ub * D * 8 + (n * 32 + c) * 16, 0, 0));
      }
    } else if constexpr (kPaged) {
      const bf16_t* va = a.vp + static_cast<uint64_t>(pick4(pu4, h)) * (D * 8) + c * 8;
      const bf16_t* vb = a.vp + static_cast<uint64_t>(pick4(pu4, 2 + h)) * (D * 8) + c * 8;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        R.k[2 * dt] = load_bf16x8(va + 256 * dt);
        R.k[2 * dt + 1] = load_bf16x8(vb + 256 * dt);
      }
    } else {
      const int ua = static_cast<int>(pick4(ent4, h) & kUnitMask);
      const int ub = static_cast<int>(pick4(ent4, 2 + h) & kUnitMask);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        R.k[2 * dt] = buffer_load_bf16x8(vrs, (ua * D + 32 * dt + c) * 16);
        R.k[2 * dt + 1] = buffer_load_bf16x8(vrs, (ub * D + 32 * dt + c) * 16);
      }
    }
  };
  // operand of d-tile dt, unit slot h (sb = 0) or 2 + h (sb = 1)
  auto v_op = [&](const OpRegs& V, int dt, int sb) -> bf16x8_t {
    if constexpr (kFp8) {
      const uint4 w = V.r[(dt >> 1) * 2 + sb];
      return (dt & 1) ? fp8x8_to_bf16(w.z, w.w) : fp8x8_to_bf16(w.x, w.y);
    } else {
      return V.k[2 * dt + sb];
    }
  };

  f32x16_t acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m_run = -1e30f, l_run = 0.f;

  // valid-token mask (8 bits) of this lane's row for a unit entry
  auto row_mask = [&](uint32_t ent) -> uint32_t {
    const bool chose = (ent >> (kChoseShift + trow)) & 1u;      // 0 past the range (ent = 0)
    const int dlt = static_cast<int>(pX) - static_cast<int>(ent & kUnitMask) * 8;
    const uint32_t causal = dlt >= 7 ? 0xffu : (dlt < 0 ? 0u : ((2u << dlt) - 1u));
    const int lo = dlt - a.win_m1;                               // first token inside the window
    const uint32_t window = lo <= 0 ? 0xffu : (lo >= 8 ? 0u : ((0xffu << lo) & 0xffu));
    return chose ? (causal & window) : 0u;
  };
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  // one chunk: S^T = K Q^T, masks, online softmax, O^T += V^T P^T.  `after_s` runs once S has
  // consumed K and `after_pv` once the P.V products have consumed V, to reuse their registers.  Masked scores become -inf by adding a bias built from the
  // mask bit; the scale enters through one fma in the exp2 argument; the row sum adds the bf16
  // probabilities the product uses, two at a time.
  auto chunk = [&](const OpRegs& K, const OpRegs& V, const uint32_t* ent4, auto after_s, auto after_pv) {
    f32x16_t s = {};
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) s = mfma32x32x16(k_op(K, kc), q_operand(kc), s);
    after_s();
    // Values 0..7 of a lane are the 8 keys of one unit, 8..15 those of another, so each half is
    // wholly attended or wholly masked except for the unit that holds the query's own position
    // (and a sliding window's first unit).  Without such a partial unit anywhere in the wave, a
    // half's mask is a choice of its max and of its exp2 bias (-inf: probability 0); otherwise
    // masked scores become -inf one by one (a sign-extended bit field selects the score or -inf).
    // Whether the chunk can hold a partial unit at all is decided on the scalar unit from the
    // chunk's units: a token chooses no unit past its own, and every unit before it is wholly in
    // its past, so away from the group's own units a half's mask is its token's chosen bit.
    // The chosen bits become lane masks there: lanes 8t .. 8t + 7 of each half are token t's rows,
    // so a unit's 4 chosen bits spread to one byte each (bit t -> byte t) give the half's 32 lanes.
    bool keep_lo, keep_hi, whole;
    uint32_t msk = 0u;                                   // per-score masks (partial chunks only)
    // (no list entry lies past the last token's own unit, and padding entries are unit 0, so the
    // chunk's largest unit decides)
    uint32_t umax4 = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) umax4 = max(umax4, ent4[j] & kUnitMask);
    const bool near_own = windowed || umax4 >= own_lo;
    if (!near_own) {
      auto lanes = [](uint32_t ent) -> uint64_t {
        const uint32_t c4 = (ent >> kChoseShift) & 0xfu;
        return static_cast<uint64_t>(((c4 * 0x00204081u) & 0x01010101u) * 0xffu);
      };
      keep_lo = __builtin_amdgcn_inverse_ballot_w64(lanes(ent4[0]) | (lanes(ent4[1]) << 32));
      keep_hi = __builtin_amdgcn_inverse_ballot_w64(lanes(ent4[2]) | (lanes(ent4[3]) << 32));
      whole = true;
    } else {
      const uint32_t mlo = row_mask(pick4(ent4, h)), mhi = row_mask(pick4(ent4, 2 + h));
      keep_lo = mlo != 0u;
      keep_hi = mhi != 0u;
      msk = mlo | (mhi << 8);
      const bool partial = (mlo != 0u && mlo != 0xffu) || (mhi != 0u && mhi != 0xffu);
      whole = !__ballot(partial);                        // wave-uniform
    }
    float t[16];
    float mx;
    if (whole) {
#pragma unroll
      for (int i = 0; i < 16; ++i) t[i] = s[i];
      float mxa = fmaxf(fmaxf(t[0], t[1]), t[2]), mxb = fmaxf(fmaxf(t[8], t[9]), t[10]);
      mxa = fmaxf(fmaxf(mxa, t[3]), t[4]);
      mxb = fmaxf(fmaxf(mxb, t[11]), t[12]);
      mxa = fmaxf(fmaxf(mxa, t[5]), t[6]);
      mxb = fmaxf(fmaxf(mxb, t[13]), t[14]);
      mxa = fmaxf(mxa, t[7]);
      mxb = fmaxf(mxb, t[15]);
      mx = fmaxf(keep_lo ? mxa : -__builtin_inff(), keep_hi ? mxb : -__builtin_inff());
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t m = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(msk), i, 1));
        t[i] = __uint_as_float((__float_as_uint(s[i]) & m) | (~m & 0xff800000u));
      }
      mx = fmaxf(fmaxf(t[0], t[1]), t[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, t[i]), t[i + 1]);
      mx = fmaxf(mx, t[15]);
    }
    mx = max_with_other_half(mx);
    const float m_new = fmaxf(m_run, mx * a.scale_log2e);
    if (__ballot(m_new > m_run + kLazyRescaleLog2)) {   // a row's max grew by > margin: rescale all
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
      m_run = m_new;
    }
    // exp2 bias of each half: -m_run, or -inf for a masked half on the whole-unit path (the
    // per-score path has already put -inf into the masked scores)
    const float blo = (!whole || keep_lo) ? -m_run : -__builtin_inff();
    const float bhi = (!whole || keep_hi) ? -m_run : -__builtin_inff();
    float pv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(t[i], a.scale_log2e, i < 8 ? blo : bhi));
    const bf16x8_t pa = pack8_bf16(pv), pb = pack8_bf16(pv + 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2_t x = {pa[2 * i], pa[2 * i + 1]};
      const bf16x2_t y = {pb[2 * i], pb[2 * i + 1]};
      l_run = __builtin_amdgcn_fdot2_f32_bf16(x, ones2, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(y, ones2, l_run, false);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      acc[dt] = mfma32x32x16(v_op(V, dt, 0), pa, acc[dt]);
      acc[dt] = mfma32x32x16(v_op(V, dt, 1), pb, acc[dt]);
    }
    after_pv();
  };

  // Software pipeline over chunks of 4 units (past the range's end the loads fetch unit 0 and are
  // masked out).  Three register sets take turns as K and V: in chunk x, once S(x) has consumed
  // K(x) its set receives V(x+1), and once P.V has consumed V(x) that set receives K(x+2).  Every
  // load is thus issued about one chunk before its use, and the compiler's vmcnt waits leave two
  // sets' loads in flight at each product.  The sets' roles repeat every three chunks.
  // On a paged cache the page lookups leave no room for this rotation (it would spill registers):
  // there K is loaded two chunks ahead into two sets and V at the start of its chunk.
  if (kPaged && e0 < e1) {
    uint32_t ec[4], e1c[4], e2c[4], e3c[4];
    uint32_t pc[4], p1c[4], p2c[4], p3c[4];
    chunk_entries(e0, ec, pc);
    chunk_entries(e0 + 4, e1c, p1c);
    chunk_entries(e0 + 8, e2c, p2c);
    OpRegs kA, kB, v0;
    load_k(ec, pc, kA);
    load_k(e1c, p1c, kB);
    int nx = e0 + 12;
    auto step = [&](OpRegs& K) {
      chunk_entries(nx, e3c, p3c);
      nx += 4;
      load_v(ec, pc, v0);
      chunk(K, v0, ec, [&] { load_k(e2c, p2c, K); }, [] {});
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ec[j] = e1c[j];
        e1c[j] = e2c[j];
        e2c[j] = e3c[j];
        pc[j] = p1c[j];
        p1c[j] = p2c[j];
        p2c[j] = p3c[j];
      }
    };
    step(kA);
    int rem = (e1 - e0 - 4) >> 2;
    for (; rem >= 2; rem -= 2) {
      step(kB);
      step(kA);
    }
    if (rem >= 1) step(kB);
  } else if (e0 < e1) {
    uint32_t ec[4], e1c[4], e2c[4], e3c[4];           // entries of chunks x, x+4, x+8, x+12
    uint32_t pc[4], p1c[4], p2c[4], p3c[4];           // their pool units (paged cache)
    chunk_entries(e0, ec, pc);
    chunk_entries(e0 + 4, e1c, p1c);
    chunk_entries(e0 + 8, e2c, p2c);
    OpRegs rA, rB, rC;
    load_k(ec, pc, rA);
    load_v(ec, pc, rB);
    load_k(e1c, p1c, rC);
    int nx = e0 + 12;                                  // next chunk whose entries are read
    // K(x) in Kc, V(x) in Vc (K(x+1) is in the third set)
    auto step = [&](OpRegs& Kc, OpRegs& Vc) {
      chunk_entries(nx, e3c, p3c);                     // entries a chunk ahead of their use
      nx += 4;
      chunk(Kc, Vc, ec, [&] { load_v(e1c, p1c, Kc); }, [&] { load_k(e2c, p2c, Vc); });
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ec[j] = e1c[j];
        e1c[j] = e2c[j];
        e2c[j] = e3c[j];
        pc[j] = p1c[j];
        p1c[j] = p2c[j];
        p2c[j] = p3c[j];
      }
    };
    // the loop body is one period of the rotation, so every trip enters with the same loads in
    // flight; the tail runs outside it
    int rem = (e1 - e0) >> 2;                          // chunks
    for (; rem >= 3; rem -= 3) {
      step(rA, rB);
      step(rC, rA);
      step(rB, rC);
    }
    if (rem >= 1) step(rA, rB);
    if (rem >= 2) step(rC, rA);
  }

  // partial of this range: O / l in bf16 (0 for a row with nothing in the range), and the running
  // max m and sum l per row in fp32.  Lane (c, h) holds d = 32 dt + 8 (i/4) + 4h + i%4 of row c.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? a.v_scale / l_tot : 0.f;
  const int64_t pbase = (gq * kRanges + r) * 32 + c;
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
  // The 32 x D tile is contiguous in memory, but a lane holds pieces of one row: it goes through
  // this wave's Q slice of LDS (Q is no longer read) and out with consecutive lanes on consecutive
  // 16-byte pieces, instead of each store instruction touching 32 rows' cache lines.
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4v v = {acc[dt][4 * i4] * inv, acc[dt][4 * i4 + 1] * inv, acc[dt][4 * i4 + 2] * inv,
                        acc[dt][4 * i4 + 3] * inv};
      *reinterpret_cast<uint2*>(sq + c * kQRow + (32 * dt + 8 * i4 + 4 * h) * 2) =
          __builtin_bit_cast(uint2, __builtin_convertvector(v, bf16x4v));
    }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  {
    unsigned char* tile = reinterpret_cast<unsigned char*>(a.part_o + (pbase - c) * D);
#pragma unroll
    for (int k = 0; k < (32 * D * 2) / 1024; ++k) {
      const int off = 1024 * k + 16 * lane;
      *reinterpret_cast<uint4*>(tile + off) =
          *reinterpret_cast<const uint4*>(sq + (off / (2 * D)) * kQRow + off % (2 * D));
    }
  }
  if (h == 0) a.part_ml[pbase] = make_float2(m_run, l_tot);
}

// ------------------------------------------------------------------------------------------------
// merge of the range partials, gate, bf16 output
// ------------------------------------------------------------------------------------------------
struct MergeArgs {
  const bf16_t* part_o;
  const float2* part_ml;
  const bf16_t* gate;
  bf16_t* out;
  float* lse;              // nullable: per row ln sum_t exp(scale q.k_t) (natural log)
  int64_t Tq, ngroups, total_groups;
  int G, D;
};

// One thread per (row, 8 d): 16-byte loads of each partial and of the gate, one 16-byte store.
__global__ void __launch_bounds__(256) merge_ranges_kernel(MergeArgs a) {
  const int per_row = a.D / 8;                         // 16 (D = 128) or 8 (D = 64) threads per row
  const int64_t gr = static_cast<int64_t>(blockIdx.x) * (256 / per_row) + threadIdx.x / per_row;
  if (gr >= a.total_groups * 32) return;
  const int d0 = static_cast<int>(threadIdx.x % per_row) * 8;
  const int row = static_cast<int>(gr & 31);
  // group indices fit 32 bits (fewer groups than query rows, < 2^31): 32-bit divisions, each a
  // fraction of a 64-bit one; offsets below stay 64-bit
  const uint32_t gq32 = static_cast<uint32_t>(gr >> 5);
  const uint32_t ng32 = static_cast<uint32_t>(a.ngroups), G32 = static_cast<uint32_t>(a.G);
  const uint32_t bg32 = gq32 / ng32;
  const int64_t gq = gq32;
  const int64_t qi = gq32 - bg32 * ng32;
  const int64_t tok = kTok * qi + (row >> 3);
  if (tok >= a.Tq) return;
  const uint32_t b32 = bg32 / G32;
  const int64_t g = bg32 - b32 * G32, b = b32;
  float2 ml[kRanges];
  float mx = -1e30f;
#pragma unroll
  for (int r = 0; r < kRanges; ++r) {
    ml[r] = a.part_ml[(gq * kRanges + r) * 32 + row];
    mx = fmaxf(mx, ml[r].x);
  }
  float L = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < kRanges; ++r) {
    const int64_t pb = (gq * kRanges + r) * 32 + row;
    const float w = ml[r].y * __builtin_amdgcn_exp2f(ml[r].x - mx);   // partial sum at the common max
    L += w;
    // each partial is read exactly once, so it is loaded with the streaming (non-temporal) hint
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 pw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.part_o + pb * a.D + d0));
    const uint32_t pv[4] = {pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] += bf16_to_f32(static_cast<bf16_t>(pv[j] & 0xffffu)) * w;
      o[2 * j + 1] += bf16_to_f32(static_cast<bf16_t>(pv[j] >> 16)) * w;
    }
  }
  const float inv = 1.f / L;
  const int64_t orow = ((b * a.Tq + tok) * a.G + g) * 8 + (row & 7);
  const int64_t obase = orow * a.D + d0;
  // the partials' m are in the exp2 domain of the scaled logits: lse = (m + log2 l) ln 2
  if (a.lse && d0 == 0) a.lse[orow] = (mx + __builtin_amdgcn_logf(L)) * 0.6931471805599453f;
  const uint4 gw = *reinterpret_cast<const uint4*>(a.gate + obase);
  const uint32_t gv[4] = {gw.x, gw.y, gw.z, gw.w};
  uint32_t ov[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float g0 = bf16_to_f32(static_cast<bf16_t>(gv[j] & 0xffffu));
    const float g1 = bf16_to_f32(static_cast<bf16_t>(gv[j] >> 16));
    ov[j] = pack_bf16x2(o[2 * j] * inv / (1.f + __expf(-g0)), o[2 * j + 1] * inv / (1.f + __expf(-g1)));
  }
  *reinterpret_cast<uint4*>(a.out + obase) = make_uint4(ov[0], ov[1], ov[2], ov[3]);
}

// ------------------------------------------------------------------------------------------------
// backward of the gated attention step (fixed selection)
// ------------------------------------------------------------------------------------------------
// Forward statistics for the backward, from the range partials: per row the log-sum-exp in the
// kernel's exp2 domain, lse2 = m + log2(l), the pre-gate output O, and from dout:
// dO = dout * sigmoid(gate) (bf16, the backward's operand), dgate = dout * O * sigmoid'(gate) and
// Dr = dO . O (fp32).  One thread per (row, 4 d); a row's threads are consecutive lanes.
struct StatsArgs {
  const bf16_t* part_o;
  const float2* part_ml;
  const bf16_t* gate;
  const bf16_t* dout;
  bf16_t* d_o;
  bf16_t* dgate;
  float* lse2;
  float* Dr;
  int64_t Tq, ngroups, total_groups;
  int G, D;
};

__global__ void __launch_bounds__(256) merge_stats_kernel(StatsArgs a) {
  const int per_row = a.D / 4;                       // 16 or 32 lanes per row, aligned in a wave
  const int64_t total = a.total_groups * 32 * per_row;
  for (int64_t id = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; id < total;
       id += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int d0 = static_cast<int>(id % per_row) * 4;
    const int64_t gr = id / per_row;
    const int row = static_cast<int>(gr % 32);
    const int64_t gq = gr / 32;
    const int64_t qi = gq % a.ngroups;
    const int64_t bg = gq / a.ngroups;
    const int64_t tok = kTok * qi + (row >> 3);
    if (tok >= a.Tq) continue;                        // whole rows: the lanes of a row agree
    const int64_t g = bg % a.G, b = bg / a.G;
    float mx = -1e30f;
#pragma unroll
    for (int r = 0; r < kRanges; ++r) mx = fmaxf(mx, a.part_ml[(gq * kRanges + r) * 32 + row].x);
    float L = 0.f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < kRanges; ++r) {
      const int64_t pb = (gq * kRanges + r) * 32 + row;
      const float2 ml = a.part_ml[pb];
      const float w = ml.y * __builtin_amdgcn_exp2f(ml.x - mx);
      L += w;
      const uint2 pw = *reinterpret_cast<const uint2*>(a.part_o + pb * a.D + d0);
      o[0] += bf16_to_f32(static_cast<bf16_t>(pw.x & 0xffffu)) * w;
      o[1] += bf16_to_f32(static_cast<bf16_t>(pw.x >> 16)) * w;
      o[2] += bf16_to_f32(static_cast<bf16_t>(pw.y & 0xffffu)) * w;
      o[3] += bf16_to_f32(static_cast<bf16_t>(pw.y >> 16)) * w;
    }
    const float inv = 1.f / L;
    const int64_t rr = ((b * a.Tq + tok) * a.G + g) * 8 + (row & 7);
    const int64_t base = rr * a.D + d0;
    const uint2 gw = *reinterpret_cast<const uint2*>(a.gate + base);
    const uint2 dw = *reinterpret_cast<const uint2*>(a.dout + base);
    const float gv[4] = {bf16_to_f32(static_cast<bf16_t>(gw.x & 0xffffu)), bf16_to_f32(static_cast<bf16_t>(gw.x >> 16)),
                         bf16_to_f32(static_cast<bf16_t>(gw.y & 0xffffu)), bf16_to_f32(static_cast<bf16_t>(gw.y >> 16))};
    const float dv[4] = {bf16_to_f32(static_cast<bf16_t>(dw.x & 0xffffu)), bf16_to_f32(static_cast<bf16_t>(dw.x >> 16)),
                         bf16_to_f32(static_cast<bf16_t>(dw.y & 0xffffu)), bf16_to_f32(static_cast<bf16_t>(dw.y >> 16))};
    float dO[4], dg[4], part = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ov = o[e] * inv;
      const float sg = 1.f / (1.f + __expf(-gv[e]));
      dO[e] = dv[e] * sg;
      dg[e] = dv[e] * ov * sg * (1.f - sg);
      part += dO[e] * ov;
    }
    for (int m = per_row / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
    *reinterpret_cast<uint2*>(a.d_o + base) = make_uint2(pack_bf16x2(dO[0], dO[1]), pack_bf16x2(dO[2], dO[3]));
    *reinterpret_cast<uint2*>(a.dgate + base) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
    if (d0 == 0) {
      a.lse2[rr] = mx + __builtin_amdgcn_logf(L);    // v_log_f32 is log2
      a.Dr[rr] = part;
    }
  }
}

// The same statistics from the forward's saved output and log-sum-exp: with out = sigmoid(gate) O,
// dO . O = dout . out and dgate = dout * out * (1 - sigmoid(gate)); lse2 = lse log2(e).  One
// thread per (row, 4 d); a row's threads are consecutive lanes.
struct SavedStatsArgs {
  const bf16_t* out;
  const float* lse;
  const bf16_t* gate;
  const bf16_t* dout;
  bf16_t* d_o;
  bf16_t* dgate;
  float* lse2;
  float* Dr;
  int64_t rows;
  int D;
};

__global__ void __launch_bounds__(256) saved_stats_kernel(SavedStatsArgs a) {
  const int per_row = a.D / 4;                       // 16 or 32 lanes per row, aligned in a wave
  const int64_t total = a.rows * per_row;
  for (int64_t id = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; id < total;
       id += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int d0 = static_cast<int>(id % per_row) * 4;
    const int64_t rr = id / per_row;
    const int64_t base = rr * a.D + d0;
    const uint2 ow = *reinterpret_cast<const uint2*>(a.out + base);
    const uint2 gw = *reinterpret_cast<const uint2*>(a.gate + base);
    const uint2 dw = *reinterpret_cast<const uint2*>(a.dout + base);
    const uint32_t o2[2] = {ow.x, ow.y}, g2[2] = {gw.x, gw.y}, d2[2] = {dw.x, dw.y};
    float dO[4], dg[4], part = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sh = 16 * (e & 1);
      const float ov = bf16_to_f32(static_cast<bf16_t>((o2[e >> 1] >> sh) & 0xffffu));
      const float gv = bf16_to_f32(static_cast<bf16_t>((g2[e >> 1] >> sh) & 0xffffu));
      const float dv = bf16_to_f32(static_cast<bf16_t>((d2[e >> 1] >> sh) & 0xffffu));
      const float sg = 1.f / (1.f + __expf(-gv));
      dO[e] = dv * sg;
      dg[e] = dv * ov * (1.f - sg);
      part += dv * ov;
    }
    for (int m = per_row / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
    *reinterpret_cast<uint2*>(a.d_o + base) = make_uint2(pack_bf16x2(dO[0], dO[1]), pack_bf16x2(dO[2], dO[3]));
    *reinterpret_cast<uint2*>(a.dgate + base) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
    if (d0 == 0) {
      a.lse2[rr] = a.lse[rr] * 1.4426950408889634f;
      a.Dr[rr] = part;
    }
  }
}

struct BwdArgs {
  const bf16_t* q;
  const bf16_t* d_o;       // dout * sigmoid(gate), bf16, q's layout
  const float* lse2;
  const float* Dr;
  const bf16_t* kq;        // K, 4-token operand layout (kq_offset)
  const bf16_t* vq;        // V, same layout
  const uint32_t* ulist;
  const int32_t* bounds;
  float* dq_part;          // [gq][R][(D/32) * 4 pieces][64 lanes][4], this range's sum
  int64_t Tq, Tk, NU, pos0, ngroups, wg_groups, total;
  int G, umax;
  int wave_ranges;         // fewer groups of tokens than waves per workgroup: waves = ranges
  float scale_log2e, scale;
};

// dQ, query-major, split into the forward's unit ranges: one wave per (group of 4 tokens, range),
// numbered as the forward's range kernel (range fastest, so range r runs on XCDs r and r + 4 and
// each XCD's L2 holds a quarter of a group's K and V), chunks of 4 units as in the forward:
// S^T = K Q^T and dP^T = V dO^T on the same K-row permutation, P = exp2(S scale log2e - lse2)
// under the forward's masks, dS = P (dP - Dr); dQ^T += K^T dS^T in registers (the forward's P V
// product).  The K^T operand (8 keys at one d per lane) is not gathered again: the chunk's K rows,
// already in registers for S^T, go to the wave's LDS, and gfx950's transposing LDS read returns
// them 4 rows of one column per lane.  Two waves per SIMD (240 registers, 8.5 KiB of LDS per
// wave): the Q^T and dO^T operands stay in registers for the whole walk, and one K/V register
// set is refilled with the next chunk as soon as S^T and dP^T have consumed it.  The range's fp32
// sum is stored in the accumulator's lane order (coalesced 1 KB pieces); dq_merge_kernel adds the
// ranges.  dK and dV are accumulated key-major in attend_bwd.hip.
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) attend_bwd_kernel(BwdArgs a) {
  constexpr int H = 8;
  constexpr int kRowB = D * 2 + 16;                      // LDS row of K (bytes)
  __shared__ __attribute__((aligned(16))) unsigned char s_ka[kRangeWaves][32 * kRowB];   // chunk's K
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int trow = c >> 3, head = c & 7;
  int r;
  int64_t bg, qi;
  if (a.wave_ranges) {
    r = wave;
    bg = blockIdx.x / a.ngroups;
    qi = blockIdx.x - bg * a.ngroups;
  } else {
    r = static_cast<int>(blockIdx.x % kRanges);
    const int64_t rest = blockIdx.x / kRanges;
    const int64_t wgq = rest % a.wg_groups;
    bg = rest / a.wg_groups;
    qi = wgq * kRangeWaves + wave;
    if (qi >= a.ngroups) return;                         // whole wave; no workgroup barriers follow
  }
  unsigned char* s_k = s_ka[wave];
  const int64_t gq = bg * a.ngroups + qi;
  const int g = static_cast<int>(bg % a.G);
  const int64_t b = bg / a.G;
  const int64_t tok0 = kTok * qi;
  const bool rowvalid = tok0 + trow < a.Tq;
  const int64_t pX = a.pos0 + tok0 + trow;
  const uint32_t* list = a.ulist + gq * list_stride(a.umax);
  const int e0 = __builtin_amdgcn_readfirstlane(a.bounds[gq * (kRanges + 1) + r]);
  const int e1 = __builtin_amdgcn_readfirstlane(a.bounds[gq * (kRanges + 1) + r + 1]);

  // Q and dO rows into LDS; lane (c, h) copies d in [D/2 h, D/2 (h+1)) of row c
  const int64_t rr = ((b * a.Tq + (rowvalid ? tok0 + trow : tok0)) * a.G + g) * H + head;
  // Q^T and dO^T operands of d-slice kc in registers: lane (c, h) holds row c, d = 16 kc + 8 h .. + 8
  bf16x8_t qop[D / 16], oop[D / 16];
  {
    const bf16_t* qrow = a.q + rr * D;
    const bf16_t* orow = a.d_o + rr * D;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qop[kc] = rowvalid ? load_bf16x8(qrow + 16 * kc + 8 * h) : zero_bf16x8();
      oop[kc] = rowvalid ? load_bf16x8(orow + 16 * kc + 8 * h) : zero_bf16x8();
    }
  }
  const float lse_c = rowvalid ? a.lse2[rr] : 0.f;
  const float D_c = rowvalid ? a.Dr[rr] : 0.f;

  const BufRsrc krs = make_rsrc(a.kq + (b * a.G + g) * a.NU * D * 8, a.NU * D * 16);
  const BufRsrc vrs = make_rsrc(a.vq + (b * a.G + g) * a.NU * D * 8, a.NU * D * 16);

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) u32x4* ConstQuadPtr;
  auto pick4 = [](const uint32_t* v, int i) -> uint32_t {
    return i == 0 ? v[0] : (i == 1 ? v[1] : (i == 2 ? v[2] : v[3]));
  };
  const int kslot = kq_slot(c), ktok = kq_tok(c);
  struct Ops {
    bf16x8_t k[D / 16], v[D / 16];
  };
  auto load_ops = [&](int cpos, uint32_t* ent4, Ops& R) {
    const u32x4 w = *((ConstQuadPtr)(list + cpos));
#pragma unroll
    for (int j = 0; j < 4; ++j) ent4[j] = cpos < e1 ? w[j] : 0u;
    const int u = static_cast<int>(pick4(ent4, kslot) & kUnitMask);
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      R.k[kc] = buffer_load_bf16x8(krs, kq_offset(u, D, kc, ktok, h));
      R.v[kc] = buffer_load_bf16x8(vrs, kq_offset(u, D, kc, ktok, h));
    }
  };
  // K^T operand of unit slot `sl` at d = 32 dt + c: the slot's 8 token rows of one column, as two
  // transposing reads of 4 rows (16-lane group lane i reads row 4 half + i / 4 of the slot at
  // columns 32 dt + 16 ((lane / 16) % 2) + 4 (i % 4) .. + 3, and receives column 32 dt + c)
  const int gi = lane & 15, gh = (lane >> 4) & 1;
  auto kt_operand = [&](int sl, int dt) -> bf16x8_t {
    const unsigned char* p = s_k + (8 * sl + (gi >> 2)) * kRowB + 2 * (32 * dt + 16 * gh + 4 * (gi & 3));
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4* LdsS16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS16x4)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS16x4)(p + 4 * kRowB));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto row_mask = [&](uint32_t ent) -> uint32_t {
    const bool chose = (ent >> (kChoseShift + trow)) & 1u;
    const int dlt = static_cast<int>(pX) - static_cast<int>(ent & kUnitMask) * 8;
    const uint32_t causal = dlt >= 7 ? 0xffu : (dlt < 0 ? 0u : ((2u << dlt) - 1u));
    return chose ? causal : 0u;
  };

  f32x16_t accq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) accq[dt][i] = 0.f;

  // One register set: S^T and dP^T consume the chunk's K and V, its K rows go to LDS, and the
  // next chunk's K and V are loaded into the same registers while dS and dQ^T are computed.
  if (e0 < e1) {
    uint32_t ent[4];
    Ops R;
    load_ops(e0, ent, R);
    for (int cpos = e0; cpos < e1; cpos += 4) {
      f32x16_t s = {}, dp = {};
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        s = mfma32x32x16(R.k[kc], qop[kc], s);
        dp = mfma32x32x16(R.v[kc], oop[kc], dp);
      }
      // the chunk's K rows (lane (c, h): row 8 slot + token of A row c, d = 16 kc + 8 h .. + 8) to
      // LDS; this wave alone reads them, after these writes in program order
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc)
        *reinterpret_cast<bf16x8_t*>(s_k + (8 * kslot + ktok) * kRowB + 2 * (16 * kc + 8 * h)) = R.k[kc];
      const uint32_t msk = row_mask(pick4(ent, h)) | (row_mask(pick4(ent, 2 + h)) << 8);
      if (cpos + 4 < e1) load_ops(cpos + 4, ent, R);
      float dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool on = (msk >> i) & 1u;
        const float p = on ? __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2e, -lse_c)) : 0.f;
        dsv[i] = p * (dp[i] - D_c);
      }
      const bf16x8_t da = pack8_bf16(dsv), db = pack8_bf16(dsv + 8);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        accq[dt] = mfma32x32x16(kt_operand(h, dt), da, accq[dt]);
        accq[dt] = mfma32x32x16(kt_operand(2 + h, dt), db, accq[dt]);
      }
    }
  }

  // this range's dQ^T sum, in the accumulator's lane order: piece (dt, i4) of lane l holds
  // d = 32 dt + 8 i4 + 4 h .. + 4 of row c (0 for a range with no entries)
  float* part = a.dq_part + (gq * kRanges + r) * (32 * D);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      *reinterpret_cast<float4*>(part + ((dt * 4 + i4) * 64 + lane) * 4) =
          make_float4(accq[dt][4 * i4], accq[dt][4 * i4 + 1], accq[dt][4 * i4 + 2], accq[dt][4 * i4 + 3]);
}

// dq = scale * (sum of the ranges' partials), rounded to bf16.  One workgroup per (group of
// tokens, 4 of its D / 8 pieces), wave w taking piece 4 j + w, a lane its (row, 4 d) of the
// partials' layout.  Group indices fit 32 bits (there are fewer groups than query rows): the
// workgroup's indices come from 32-bit divisions on the scalar unit, with no per-lane 64-bit
// division.
struct DqMergeArgs {
  const float* dq_part;
  bf16_t* dq;
  int64_t Tq, ngroups, total;
  int G, D;
  float scale;
};

__global__ void __launch_bounds__(256) dq_merge_kernel(DqMergeArgs a) {
  const uint32_t wgs = static_cast<uint32_t>(a.D / 32);           // workgroups per group of tokens
  const uint32_t gq32 = blockIdx.x / wgs;
  const int piece = static_cast<int>(blockIdx.x - gq32 * wgs) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const uint32_t ng32 = static_cast<uint32_t>(a.ngroups), G32 = static_cast<uint32_t>(a.G);
  const uint32_t bg32 = gq32 / ng32, qi32 = gq32 - bg32 * ng32;
  const int64_t tok = kTok * static_cast<int64_t>(qi32) + (c >> 3);
  if (tok >= a.Tq) return;
  const int64_t gq = gq32;
  // each partial is read exactly once: streaming (non-temporal) loads
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < kRanges; ++r)
    s += __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(
        a.dq_part + (gq * kRanges + r) * (32 * a.D) + (piece * 64 + lane) * 4));
  const int dt = piece >> 2, i4 = piece & 3;
  const uint32_t b32 = bg32 / G32, g32 = bg32 - b32 * G32;
  const int64_t row = ((static_cast<int64_t>(b32) * a.Tq + tok) * a.G + g32) * 8 + (c & 7);
  *reinterpret_cast<uint2*>(a.dq + row * a.D + 32 * dt + 8 * i4 + 4 * h) =
      make_uint2(pack_bf16x2(s[0] * a.scale, s[1] * a.scale), pack_bf16x2(s[2] * a.scale, s[3] * a.scale));
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Token groups whose union bitmaps (kTok x words each) share one workgroup's LDS (0: none fits).
// Bitmap words per token in the group-list kernel: ceil(NU / 32) rounded up to a multiple of 4, so
// that every token's bitmap starts 16-byte aligned.
int64_t union_words(const Dims& d) { return ((d.NU + 31) / 32 + 3) & ~int64_t(3); }

// Bitmap words each lane holds in registers in the group-list kernel (0: the 16-byte scans of
// long contexts, whose bitmaps stay in LDS beside the list).
int union_per_lane(int64_t words) { return words <= 64 * 8 ? 8 : 0; }

int union_waves(const Dims& d) {
  const int64_t words = union_words(d);
  const int64_t per_wave = union_lds_words(words, list_stride(static_cast<int>(units_per_query(d))),
                                           union_per_lane(words) > 0) *
                           static_cast<int64_t>(sizeof(uint32_t));
  const int64_t fit = (160 * 1024) / per_wave;          // waves whose LDS fits one CU
  // up to 4 waves per workgroup, but small enough that two workgroups share a CU
  if (fit >= 8) return 4;
  if (fit >= 2) return static_cast<int>(fit / 2);
  return static_cast<int>(fit);
}

void launch_quad_union(const UnionArgs& ua, int64_t total, hipStream_t s) {
  const int per = union_per_lane(ua.words);
  if (per == 0 && ua.B == 8 && ua.NS <= kMergeSel && !ua.balance) {
    // LDS per wave: the 4 selections and the list; 4 waves per workgroup when 8 fit on a CU
    const int64_t per_wave = (kTok * kMergeSel + list_stride(ua.umax)) * static_cast<int64_t>(sizeof(uint32_t));
    const int64_t fit = (160 * 1024) / per_wave;
    const int waves = fit >= 8 ? 4 : (fit >= 2 ? static_cast<int>(fit / 2) : 1);
    UnionArgs um = ua;
    um.waves = waves;
    const dim3 ugrid(static_cast<unsigned>((total + waves - 1) / waves));
    hipLaunchKernelGGL(quad_union_merge_kernel, ugrid, dim3(64 * waves),
                       static_cast<size_t>(waves * per_wave), s, um);
    return;
  }
  const size_t lds = static_cast<size_t>(ua.waves) *
                     union_lds_words(ua.words, list_stride(ua.umax), per > 0) * sizeof(uint32_t);
  const dim3 ugrid(static_cast<unsigned>((total + ua.waves - 1) / ua.waves));
  if (per == 8)                                         // contexts up to 128K tokens
    hipLaunchKernelGGL((quad_union_kernel<false, 8>), ugrid, dim3(64 * ua.waves), lds, s, ua);
  else if (ua.words >= 2048)                            // contexts of 512K tokens and more
    hipLaunchKernelGGL((quad_union_kernel<true, 0>), ugrid, dim3(64 * ua.waves), lds, s, ua);
  else
    hipLaunchKernelGGL((quad_union_kernel<false, 0>), ugrid, dim3(64 * ua.waves), lds, s, ua);
}

size_t split_bytes_for(const Dims& d, int umax) {
  const int64_t ng = (d.Tq + kTok - 1) / kTok;
  const size_t n = static_cast<size_t>(d.Bt * d.G * ng);
  return align256(n * list_stride(umax) * sizeof(uint32_t)) +
         align256(n * (kRanges + 1) * sizeof(int32_t)) +
         align256(n * kRanges * 32 * d.D * sizeof(bf16_t)) + align256(n * kRanges * 32 * sizeof(float2));
}

// Units a sliding window of `window` tokens covers for a group of 4 tokens, as list entries per
// token (the list stride holds kTok times this).
int window_umax(int64_t window) {
  const int64_t n = (window + kTok - 1 + 7) / 8 + 1;
  return static_cast<int>((n + kTok - 1) / kTok);
}

struct SplitBuffers {
  uint32_t* ulist;
  int32_t* bounds;
  bf16_t* part_o;
  float2* part_ml;
};

SplitBuffers split_buffers(const Dims& d, int umax, void* ws) {
  const int64_t ng = (d.Tq + kTok - 1) / kTok;
  const int64_t total = d.Bt * d.G * ng;
  SplitBuffers sb;
  char* p = static_cast<char*>(ws);
  sb.ulist = reinterpret_cast<uint32_t*>(p);
  p += align256(static_cast<size_t>(total) * list_stride(umax) * sizeof(uint32_t));
  sb.bounds = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(total) * (kRanges + 1) * sizeof(int32_t));
  sb.part_o = reinterpret_cast<bf16_t*>(p);
  p += align256(static_cast<size_t>(total) * kRanges * 32 * d.D * sizeof(bf16_t));
  sb.part_ml = reinterpret_cast<float2*>(p);
  return sb;
}

// The range kernel over prepared lists, then the merge.
hipError_t launch_ranges_and_merge(const Dims& d, const void* q, const void* packed_k,
                                   const void* gate, void* out, const void* packed_v,
                                   const SplitBuffers& sb, int umax, int win_m1, hipStream_t s,
                                   StageMark mark, const PagedKV* paged, const Fp8Scales* fp8,
                                   float* lse = nullptr) {
  const int64_t ng = (d.Tq + kTok - 1) / kTok;
  const int64_t total = d.Bt * d.G * ng;
  RangeArgs a;
  a.q = static_cast<const bf16_t*>(q);
  a.kp = static_cast<const bf16_t*>(packed_k);
  a.vp = static_cast<const bf16_t*>(packed_v);
  a.ulist = sb.ulist;
  a.bounds = sb.bounds;
  a.part_o = sb.part_o;
  a.part_ml = sb.part_ml;
  a.Tq = d.Tq;
  a.Tk = d.Tk;
  a.NU = d.NU;
  a.pos0 = d.pos0;
  a.ngroups = ng;
  a.wg_groups = (ng + kRangeWaves - 1) / kRangeWaves;
  a.wave_ranges = ng < kRangeWaves ? 1 : 0;
  a.G = d.G;
  a.umax = umax;
  a.scale_log2e = d.scale * (fp8 ? fp8->k_scale : 1.0f) * 1.4426950408889634f;
  a.v_scale = fp8 ? fp8->v_scale : 1.0f;
  a.seq_len = d.seq_len;
  a.block_table = nullptr;
  a.max_pages = a.num_pages = 0;
  a.ul2 = 0;
  a.win_m1 = win_m1;
  if (paged) {
    a.kp = static_cast<const bf16_t*>(paged->k);
    a.vp = static_cast<const bf16_t*>(paged->v);
    a.block_table = paged->block_table;
    a.max_pages = paged->max_pages;
    a.num_pages = paged->num_pages;
    a.ul2 = paged->page_units_log2;
  }
  const dim3 grid(static_cast<unsigned>(a.wave_ranges ? d.Bt * d.G * ng : d.Bt * d.G * a.wg_groups * kRanges));
  if (paged) {
    if (d.D == 128)
      hipLaunchKernelGGL((attend_range_kernel<128, true, false>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attend_range_kernel<64, true, false>), grid, dim3(256), 0, s, a);
  } else if (fp8) {
    if (d.D == 128)
      hipLaunchKernelGGL((attend_range_kernel<128, false, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attend_range_kernel<64, false, true>), grid, dim3(256), 0, s, a);
  } else {
    if (d.D == 128)
      hipLaunchKernelGGL((attend_range_kernel<128, false, false>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attend_range_kernel<64, false, false>), grid, dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && mark) e = mark(5, s);
  if (e != hipSuccess) return e;

  MergeArgs m;
  m.part_o = sb.part_o;
  m.part_ml = sb.part_ml;
  m.gate = static_cast<const bf16_t*>(gate);
  m.out = static_cast<bf16_t*>(out);
  m.lse = lse;
  m.Tq = d.Tq;
  m.ngroups = ng;
  m.total_groups = total;
  m.G = d.G;
  m.D = d.D;
  const int64_t rows_per_block = 256 / (d.D / 8);
  const int64_t blocks = (total * 32 + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(merge_ranges_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, m);
  return hipGetLastError();
}

}  // namespace

bool attend_split_supported(const Dims& d) {
  // one token group's union bitmaps must fit in 160 KiB of LDS
  return d.bf16 && d.H == 8 && (d.D == 64 || d.D == 128) && d.B % 8 == 0 &&
         d.NU * 8 * static_cast<int64_t>(d.D) * 2 < (int64_t(1) << 31) &&
         units_per_query(d) <= 1024 && union_waves(d) >= 1;
}

size_t attend_split_bytes(const Dims& d) {
  return split_bytes_for(d, static_cast<int>(units_per_query(d)));
}

hipError_t launch_attend_split(const Dims& d, const void* q, const void* packed_k,
                               const void* gate, const int32_t* sel, void* out,
                               const void* packed_v, void* ws, hipStream_t s, StageMark mark,
                               const PagedKV* paged, const Fp8Scales* fp8, float* lse) {
  const int64_t ng = (d.Tq + kTok - 1) / kTok;
  const int64_t total = d.Bt * d.G * ng;
  const int umax = static_cast<int>(units_per_query(d));
  const SplitBuffers sb = split_buffers(d, umax, ws);

  UnionArgs ua;
  ua.sel = sel;
  ua.ulist = sb.ulist;
  ua.bounds = sb.bounds;
  ua.Tq = d.Tq;
  ua.pos0 = d.pos0;
  ua.seq_len = d.seq_len;
  ua.ngroups = ng;
  ua.total = total;
  ua.G = d.G;
  ua.NS = d.NS;
  ua.B = d.B;
  ua.umax = umax;
  ua.words = static_cast<int>(union_words(d));
  ua.waves = union_waves(d);
  ua.balance = ng < kRangeWaves ? 1 : 0;                // as the attention's wave_ranges
  launch_quad_union(ua, total, s);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && mark) e = mark(4, s);
  if (e != hipSuccess) return e;
  return launch_ranges_and_merge(d, q, packed_k, gate, out, packed_v, sb, umax, 1 << 30, s, mark,
                                 paged, fp8, lse);
}

bool attend_window_supported(const Dims& d) {
  return d.bf16 && d.H == 8 && (d.D == 64 || d.D == 128) &&
         d.NU * 8 * static_cast<int64_t>(d.D) * 2 < (int64_t(1) << 31);
}

size_t attend_window_bytes(const Dims& d, int64_t window) {
  return split_bytes_for(d, window_umax(window));
}

hipError_t launch_attend_window(const Dims& d, int64_t window, const void* q, const void* packed_k,
                                const void* gate, void* out, const void* packed_v, void* ws,
                                hipStream_t s) {
  const int64_t ng = (d.Tq + kTok - 1) / kTok;
  const int64_t total = d.Bt * d.G * ng;
  const int umax = window_umax(window);
  const SplitBuffers sb = split_buffers(d, umax, ws);
  WindowArgs wa;
  wa.ulist = sb.ulist;
  wa.bounds = sb.bounds;
  wa.Tq = d.Tq;
  wa.pos0 = d.pos0;
  wa.ngroups = ng;
  wa.total = total;
  wa.win_m1 = static_cast<int>(window - 1);
  wa.umax = umax;
  hipLaunchKernelGGL(window_lists_kernel, dim3(static_cast<unsigned>((total + 3) / 4)), dim3(256), 0,
                     s, wa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_ranges_and_merge(d, q, packed_k, gate, out, packed_v, sb, umax, wa.win_m1, s,
                                 nullptr, nullptr, nullptr);
}

// fp32 dq partials of the unit ranges: [groups of 4 tokens][R][32 rows x D]
size_t dq_part_bytes(const Dims& d) {
  const int64_t ng = (d.Tq + kTok - 1) / kTok;
  return align256(static_cast<size_t>(d.Bt * d.G * ng) * kRanges * 32 * d.D * sizeof(float));
}

size_t attend_backward_bytes(const Dims& d) {
  const size_t rows = static_cast<size_t>(d.Bt * d.Tq * d.G) * 8;
  return 2 * packed_kv_quad_bytes(d) + attend_split_bytes(d) + 2 * align256(rows * sizeof(float)) +
         align256(rows * d.D * sizeof(bf16_t)) + backward_dkv_bytes(d) + dq_part_bytes(d);
}

// The gradient kernels of the backward, once dO, lse2 and Dr are in place: dk, dv key-major
// (every element written once, no atomics), then dq per unit range and the merge of the ranges.
static hipError_t launch_backward_grads(const Dims& d, const void* q, const void* k, const void* v,
                                        const int32_t* sel, void* dq, float* dk, float* dv,
                                        const bf16_t* d_o, const float* lse2, const float* Dr,
                                        const char* fwd_kv, const char* bwd_kv,
                                        const SplitBuffers& sb, char* dkv_ws, float* dq_part,
                                        hipStream_t s) {
  const int64_t ng = (d.Tq + kTok - 1) / kTok;
  const int64_t total = d.Bt * d.G * ng;
  const int umax = static_cast<int>(units_per_query(d));
  hipError_t e = launch_backward_dkv(d, q, d_o, lse2, Dr, k, v, sel, dk, dv, dkv_ws, s);
  if (e != hipSuccess) return e;
  BwdArgs ba;
  ba.q = static_cast<const bf16_t*>(q);
  ba.d_o = d_o;
  ba.lse2 = lse2;
  ba.Dr = Dr;
  ba.kq = reinterpret_cast<const bf16_t*>(fwd_kv);
  ba.vq = reinterpret_cast<const bf16_t*>(bwd_kv);
  ba.ulist = sb.ulist;
  ba.bounds = sb.bounds;
  ba.dq_part = dq_part;
  ba.Tq = d.Tq;
  ba.Tk = d.Tk;
  ba.NU = d.NU;
  ba.pos0 = d.pos0;
  ba.ngroups = ng;
  ba.wg_groups = (ng + kRangeWaves - 1) / kRangeWaves;
  ba.wave_ranges = ng < kRangeWaves ? 1 : 0;
  ba.total = total;
  ba.G = d.G;
  ba.umax = umax;
  ba.scale_log2e = d.scale * 1.4426950408889634f;
  ba.scale = d.scale;
  const dim3 bgrid(static_cast<unsigned>(ba.wave_ranges ? d.Bt * d.G * ng : d.Bt * d.G * ba.wg_groups * kRanges));
  if (d.D == 128)
    hipLaunchKernelGGL(attend_bwd_kernel<128>, bgrid, dim3(256), 0, s, ba);
  else
    hipLaunchKernelGGL(attend_bwd_kernel<64>, bgrid, dim3(256), 0, s, ba);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  DqMergeArgs dm;
  dm.dq_part = dq_part;
  dm.dq = static_cast<bf16_t*>(dq);
  dm.Tq = d.Tq;
  dm.ngroups = ng;
  dm.total = total;
  dm.G = d.G;
  dm.D = d.D;
  dm.scale = d.scale;
  {
    const int64_t blocks = total * (d.D / 32);
    if (total >= (int64_t(1) << 31) || blocks * 256 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dq_merge_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, dm);
  }
  return hipGetLastError();
}

hipError_t launch_attend_backward(const Dims& d, const void* q, const void* k, const void* v,
                                  const void* gate, const int32_t* sel, const void* dout, void* dq,
                                  float* dk, float* dv, void* dgate, void* ws, hipStream_t s,
                                  const void* saved_out, const float* saved_lse) {
  const int64_t ng = (d.Tq + kTok - 1) / kTok;
  const int64_t total = d.Bt * d.G * ng;
  const int umax = static_cast<int>(units_per_query(d));
  const size_t pkv = packed_kv_quad_bytes(d);
  char* p = static_cast<char*>(ws);
  char* fwd_kv = p;                  // K in the operand layout, V transposed (the forward's copies)
  char* bwd_kv = p + pkv;            // V in the operand layout (and K transposed, unused)
  char* split = bwd_kv + pkv;
  const size_t rows = static_cast<size_t>(d.Bt * d.Tq * d.G) * 8;
  float* lse2 = reinterpret_cast<float*>(split + attend_split_bytes(d));
  float* Dr = reinterpret_cast<float*>(reinterpret_cast<char*>(lse2) + align256(rows * sizeof(float)));
  bf16_t* d_o = reinterpret_cast<bf16_t*>(reinterpret_cast<char*>(Dr) + align256(rows * sizeof(float)));
  char* dkv_ws = reinterpret_cast<char*>(d_o) + align256(rows * d.D * sizeof(bf16_t));
  float* dq_part = reinterpret_cast<float*>(dkv_ws + backward_dkv_bytes(d));

  hipError_t e = launch_pack_kv_quad(d, k, v, fwd_kv, s);
  if (e != hipSuccess) return e;
  e = launch_pack_kv_quad(d, v, k, bwd_kv, s);
  if (e != hipSuccess) return e;
  // forward recompute up to the range partials
  const SplitBuffers sb = split_buffers(d, umax, split);
  UnionArgs ua;
  ua.sel = sel;
  ua.ulist = sb.ulist;
  ua.bounds = sb.bounds;
  ua.Tq = d.Tq;
  ua.pos0 = d.pos0;
  ua.seq_len = nullptr;
  ua.ngroups = ng;
  ua.total = total;
  ua.G = d.G;
  ua.NS = d.NS;
  ua.B = d.B;
  ua.umax = umax;
  ua.words = static_cast<int>(union_words(d));
  ua.waves = union_waves(d);
  ua.balance = ng < kRangeWaves ? 1 : 0;                // as the attention's wave_ranges
  launch_quad_union(ua, total, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (saved_out) {
    // statistics from the forward's output and log-sum-exp: no forward recompute
    SavedStatsArgs st;
    st.out = static_cast<const bf16_t*>(saved_out);
    st.lse = saved_lse;
    st.gate = static_cast<const bf16_t*>(gate);
    st.dout = static_cast<const bf16_t*>(dout);
    st.d_o = d_o;
    st.dgate = static_cast<bf16_t*>(dgate);
    st.lse2 = lse2;
    st.Dr = Dr;
    st.rows = static_cast<int64_t>(rows);
    st.D = d.D;
    const int64_t items = st.rows * (d.D / 4);
    int64_t blocks = (items + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(saved_stats_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_backward_grads(d, q, k, v, sel, dq, dk, dv, d_o, lse2, Dr, fwd_kv, bwd_kv, sb,
                                 dkv_ws, dq_part, s);
  }
  RangeArgs a;
  a.q = static_cast<const bf16_t*>(q);
  a.kp = reinterpret_cast<const bf16_t*>(fwd_kv);
  a.vp = reinterpret_cast<const bf16_t*>(fwd_kv + pkv / 2);
  a.ulist = sb.ulist;
  a.bounds = sb.bounds;
  a.part_o = sb.part_o;
  a.part_ml = sb.part_ml;
  a.Tq = d.Tq;
  a.Tk = d.Tk;
  a.NU = d.NU;
  a.pos0 = d.pos0;
  a.ngroups = ng;
  a.wg_groups = (ng + kRangeWaves - 1) / kRangeWaves;
  a.wave_ranges = ng < kRangeWaves ? 1 : 0;
  a.G = d.G;
  a.umax = umax;
  a.scale_log2e = d.scale * 1.4426950408889634f;
  a.v_scale = 1.0f;
  a.seq_len = nullptr;
  a.block_table = nullptr;
  a.max_pages = a.num_pages = 0;
  a.ul2 = 0;
  a.win_m1 = 1 << 30;
  const dim3 grid(static_cast<unsigned>(a.wave_ranges ? d.Bt * d.G * ng : d.Bt * d.G * a.wg_groups * kRanges));
  if (d.D == 128)
    hipLaunchKernelGGL((attend_range_kernel<128, false, false>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attend_range_kernel<64, false, false>), grid, dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  StatsArgs st;
  st.part_o = sb.part_o;
  st.part_ml = sb.part_ml;
  st.gate = static_cast<const bf16_t*>(gate);
  st.dout = static_cast<const bf16_t*>(dout);
  st.d_o = d_o;
  st.dgate = static_cast<bf16_t*>(dgate);
  st.lse2 = lse2;
  st.Dr = Dr;
  st.Tq = d.Tq;
  st.ngroups = ng;
  st.total_groups = total;
  st.G = d.G;
  st.D = d.D;
  {
    const int64_t items = total * 32 * (d.D / 4);
    int64_t blocks = (items + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(merge_stats_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, st);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_backward_grads(d, q, k, v, sel, dq, dk, dv, d_o, lse2, Dr, fwd_kv, bwd_kv, sb, dkv_ws,
                               dq_part, s);
}

}  // namespace sgqa
