// Steps 2-3 fused for the one-call forward: indexer scores are never stored in full.
//
// Same method as index.hip + topk.hip (Step 5 Preview pages, mo.ai.kr summary, section
// "모델 구조와 학습 안정성": every KV group scores the block-compressed shared index keys and keeps
// its own top-k blocks; B = 8 makes this eight times cheaper than token-level scoring).  Readings:
// raw dot-product scores of the strictly past blocks j < o = p/B, the own block always selected
// and counted in the NS = k/B budget, ties to the lower block index, ascending output.
//
// filter kernel (one workgroup = 4 waves = 64 rows of one sequence; a row = (query, KV group)):
//   1. sample: scores against 384 blocks at a fixed stride (v_mfma_f32_16x16x32_bf16), or 4096
//      through two histogram passes for rows past 32768 blocks; per row the r-th largest sampled
//      score, r chosen so that about twice the budget is expected to pass, is the row's threshold
//      (kept as the top 16 bits of the order-preserving key: any threshold is correct, it only
//      sizes the candidate list);
//   2. filter: every causal score, column tiles of K_blk staged in LDS (double-buffered) and
//      shared by the 4 waves; the products are taken transposed, so a lane holds one row and four
//      consecutive blocks of it, and a passing score's slot is the row's count so far plus the
//      passing scores before it in block order (a cross-lane prefix over the row's 4 lanes, taken
//      for three column steps at once): every row's list is in ascending block order.
// select kernel (one wave per row): the (NS-1)-th largest key tau by a bitwise search over the
//   candidates held in registers, then the keys > tau and the lowest-indexed keys == tau, emitted
//   in block order by a stable compaction of the sorted list (lists appended by several
//   workgroups, as in decode, go through two LDS block bitmaps instead).  Exact whenever at
//   least NS-1 candidates passed (every member of the top set is >= tau >= threshold); rows with
//   too few or too many (> capacity) candidates are queued for the exact fallback in topk.hip,
//   which recomputes the full score row.
// Few rows per sequence (decode) take a threshold kernel and a slab-split filter instead of the
// filter kernel (see below); they share the select kernel and the fallback.
#include "device_common.h"
#include "sgqa_internal.h"

namespace sgqa {
namespace {

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kRows = 64;          // rows per workgroup
constexpr int kSamp = 384;         // sampled blocks per row (a multiple of 64)
// Rows with more causal blocks than this take their threshold from kSampBig samples per row, by
// two histogram passes instead of a stored sample (which would not fit in LDS): with kSamp samples
// only a handful of them lie above a long row's threshold, and its pass count varies too much.
constexpr int64_t kHugeO = 32768;
constexpr int kSampBig = 4096;
// K_blk columns per staged tile: 96 (a tile is 96 x DI/8 16-byte pieces, a whole number of
// 256-thread rounds for DI = 64 and 128); 128 for DI = 32
template <int DI> constexpr int cols_per_tile() { return DI == 32 ? 128 : 96; }

__device__ __forceinline__ uint32_t order_key_f(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;                 // -0.0 and +0.0 are the same score
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The smallest float whose order key is >= thr (thr has its low 16 bits clear): scores pass the
// threshold exactly when score >= that float.  Keys at or below the key of -inf admit everything.
__device__ __forceinline__ float key_threshold_to_float(uint32_t thr) {
  if (thr <= 0x007fffffu) return -__builtin_inff();
  return (thr & 0x80000000u) ? __uint_as_float(thr & 0x7fffffffu) : __uint_as_float(~thr);
}


struct FilterArgs {
  const bf16_t* q_idx;
  const bf16_t* k_blk;
  uint64_t* cand;              // [chunk rows][cap]
  int32_t* cnt;                // [chunk rows]
  int32_t* fail_count;         // zeroed here (block 0) for the select kernel that follows
  int64_t b0, i0, ntok, Tq, pos0, NB, seq_rows, tiles_per_seq;
  int G, B, NS, cap;
};

// 3 workgroups per CU: 53 KB of LDS (384 samples of 64 rows, or two 96-column tiles) and at most
// 168 registers per lane
template <int DI>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) index_filter_kernel(FilterArgs a) {
  constexpr int kCols = cols_per_tile<DI>();
  static_assert((kCols * (DI / 8)) % 256 == 0, "a tile must be whole 256-thread load rounds");
  constexpr int kRowBytes = DI * 2 + 16;                  // padded LDS row of one K_blk block
  constexpr int kTileBytes = kCols * kRowBytes;
  constexpr int kSampBytes = kRows * kSamp * 2;
  constexpr int kLds = (kSampBytes > 2 * kTileBytes) ? kSampBytes : 2 * kTileBytes;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
  __shared__ uint32_t s_thr[kRows];

  if (blockIdx.x == 0 && threadIdx.x == 0) *a.fail_count = 0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  // tiles in reverse order: the last tokens have the most causal blocks, so the longest workgroups
  // are dispatched first and the launch ends on short ones
  const int64_t seq = blockIdx.x / a.tiles_per_seq;
  const int64_t row0 = (a.tiles_per_seq - 1 - (blockIdx.x - seq * a.tiles_per_seq)) * kRows;
  const int64_t rows_here = min<int64_t>(kRows, a.seq_rows - row0);
  const int64_t b = a.b0 + seq;
  const bf16_t* kb = a.k_blk + b * a.NB * DI;

  // o of a local row (rows of the tile hold consecutive tokens, so the last row has the largest)
  auto row_o = [&](int local, int64_t* rr_out) -> int64_t {
    const int64_t rl = row0 + local;
    const int64_t tok = rl / a.G;
    const int64_t i = a.i0 + tok;
    if (rr_out) *rr_out = seq * a.seq_rows + rl;
    return (a.pos0 + i) / a.B;
  };
  const int64_t o_max = row_o(static_cast<int>(rows_here) - 1, nullptr);

  // this wave's 16 rows: A operand (q_idx) for every k-step, plus per-lane row facts for C rows
  const int my_local_a = wave * 16 + lr;                  // A row held by this lane
  const bool a_valid = my_local_a < rows_here;
  bf16x8_t qa[DI / 32];
  {
    const int64_t rl = row0 + (a_valid ? my_local_a : 0);
    const int64_t tok = rl / a.G;
    const int g = static_cast<int>(rl - tok * a.G);
    const bf16_t* qrow = a.q_idx + (((b * a.Tq) + a.i0 + tok) * a.G + g) * DI;
#pragma unroll
    for (int kc = 0; kc < DI / 32; ++kc) qa[kc] = a_valid ? load_bf16x8(qrow + kc * 32 + lg * 8) : zero_bf16x8();
  }
  int64_t c_o[4];
  bool c_valid[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int local = wave * 16 + lg * 4 + e;
    c_valid[e] = local < rows_here;
    c_o[e] = c_valid[e] ? row_o(local, nullptr) : 0;
  }

  const int64_t ntiles = (o_max + kCols - 1) / kCols;
  // staging: 128 blocks x DI bf16 = 128 x (DI/8) 16-byte pieces over 256 threads; the next tile
  // is fetched into registers before the current one is multiplied and written to LDS after it
  constexpr int kPer = kCols * (DI / 8) / 256;
  uint4 pre[kPer];
  // K_blk of this sequence through a buffer descriptor: columns past NB read as zero
  const BufRsrc krs = make_rsrc(kb, a.NB * DI * 2);
  auto load_tile = [&](int64_t t) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int pc = threadIdx.x + k * 256;
      const int row = pc / (DI / 8), part = pc - row * (DI / 8);
      const int col = static_cast<int>(t) * kCols + row;
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(krs, col * (DI * 2) + part * 16, 0, 0);
      pre[k] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* dst = lds + buf * kTileBytes;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int pc = threadIdx.x + k * 256;
      const int row = pc / (DI / 8), part = pc - row * (DI / 8);
      *reinterpret_cast<uint4*>(dst + row * kRowBytes + part * 16) = pre[k];
    }
  };
  // the first tile's loads are issued now: their latency passes under the sampling phase (the LDS
  // they go to is the sample area until the thresholds are taken)
  if (ntiles > 0) load_tile(0);

  // ---------------- phase 1: sampled scores -> per-row threshold ----------------
  const bool sampling = o_max > a.cap;
  if (sampling && o_max > kHugeO) {
    // Long rows: kSampBig samples per row at a fixed stride.  Pass A counts each row's sampled
    // 16-bit keys by their high byte (256 bins per row in LDS); the row's r-th largest key lies in
    // the bin where the count from the top reaches r.  Pass B recomputes the samples and counts,
    // within that bin, the low bytes; the same search gives the exact r-th largest 16-bit key.
    const int64_t stride = (o_max + kSampBig - 1) / kSampBig;
    // [kRows][128] words of two 16-bit bin counts (bin 2w in the low half, 2w + 1 in the high
    // half); a count never exceeds kSampBig < 2^16, so no half carries into the other
    uint32_t* hist = reinterpret_cast<uint32_t*>(lds);
    uint32_t* s_hi = reinterpret_cast<uint32_t*>(s_thr);           // high byte, then the threshold
    __shared__ int s_rank[kRows];                                  // rank left inside the high bin
    auto clear_hist = [&]() {
      for (int i = threadIdx.x; i < kRows * 128; i += 256) hist[i] = 0u;
    };
    auto bump = [&](int row, uint32_t bin) {
      atomicAdd(&hist[row * 128 + (bin >> 1)], 1u << (16u * (bin & 1u)));
    };
    // one pass over the samples; `visit(row, key16)` for every sample inside the row's causal range
    auto sample_pass = [&](auto visit) {
      constexpr int kBatch = 4;
#pragma unroll 1
      for (int n0 = 0; n0 < kSampBig / 16; n0 += kBatch) {
        uint4 bb[kBatch][DI / 32];
        int64_t cols[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          cols[j] = (static_cast<int64_t>(n0 + j) * 16 + lr) * stride;
          const int64_t cc = cols[j] < a.NB ? cols[j] : a.NB - 1;
#pragma unroll
          for (int kc = 0; kc < DI / 32; ++kc)
            bb[j][kc] = *reinterpret_cast<const uint4*>(kb + cc * DI + kc * 32 + lg * 8);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          f32x4_t c = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < DI / 32; ++kc) c = mfma16x16x32(qa[kc], bf16x8_from_u4(bb[j][kc]), c);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c_valid[e] && cols[j] < c_o[e])
              visit(wave * 16 + lg * 4 + e, order_key_f(c[e]) >> 16);
        }
      }
    };
    // the bin of rank `r` counted from the top of a row's 256 bins: lane l holds bins 255 - 4l
    // .. 252 - 4l; returns the bin and the rank left inside it
    auto find_bin = [&](const uint32_t* h, int r, int* left) -> int {
      const uint32_t w_hi = h[127 - 2 * lane], w_lo = h[126 - 2 * lane];
      const uint32_t b0 = w_hi >> 16, b1 = w_hi & 0xffffu, b2 = w_lo >> 16, b3 = w_lo & 0xffffu;
      const int cnt = static_cast<int>(b0 + b1 + b2 + b3);
      const int incl = wave_inclusive_scan(cnt);
      const uint64_t hit = __ballot(incl >= r);
      const int L = hit ? __builtin_ctzll(hit) : 63;
      int acc = __builtin_amdgcn_readlane(incl - cnt, L);
      const uint32_t hb[4] = {static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b0), L)),
                              static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b1), L)),
                              static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b2), L)),
                              static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b3), L))};
      int bin = 252 - 4 * L;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (acc + static_cast<int>(hb[q]) >= r) {
          bin = 255 - 4 * L - q;
          break;
        }
        acc += static_cast<int>(hb[q]);
      }
      *left = r - acc;
      return bin;
    };
    // per-row rank r (about twice the budget passing), or 0 for rows that take every block
    auto row_rank = [&](int local) -> int {
      if (local >= rows_here) return 0;
      const int64_t o = row_o(local, nullptr);
      if (o <= a.cap || o + 1 <= a.NS) return 0;
      const int nvalid = static_cast<int>((o + stride - 1) / stride);
      const int need = a.NS - 1;
      int r = static_cast<int>((2ll * need * nvalid + o - 1) / o);
      return r < 1 ? 1 : (r > nvalid ? nvalid : r);
    };
    clear_hist();
    __syncthreads();
    sample_pass([&](int row, uint32_t k16) { bump(row, k16 >> 8); });
    __syncthreads();
#pragma unroll 1
    for (int rloc = 0; rloc < 16; ++rloc) {
      const int local = wave * 16 + rloc;
      const int r = row_rank(local);
      int left = 0;
      const int bin = r > 0 ? find_bin(hist + local * 128, r, &left) : 0;
      if (lane == 0) {
        s_hi[local] = r > 0 ? static_cast<uint32_t>(bin) : 0xffffffffu;
        s_rank[local] = left;
      }
    }
    __syncthreads();
    clear_hist();
    __syncthreads();
    sample_pass([&](int row, uint32_t k16) {
      if ((k16 >> 8) == s_hi[row]) bump(row, k16 & 255u);
    });
    __syncthreads();
#pragma unroll 1
    for (int rloc = 0; rloc < 16; ++rloc) {
      const int local = wave * 16 + rloc;
      const uint32_t hi = s_hi[local];
      uint32_t thr = 0u;
      if (hi != 0xffffffffu) {
        int left = 0;
        const int lo = find_bin(hist + local * 128, s_rank[local], &left);
        thr = ((hi << 8) | static_cast<uint32_t>(lo)) << 16;
      }
      if (lane == 0) s_thr[local] = thr;
    }
  } else if (sampling) {
    const int64_t stride = (o_max + kSamp - 1) / kSamp;
    uint16_t* samp = reinterpret_cast<uint16_t*>(lds);
    // four column steps per batch: their 16 operand loads are issued before the products (columns
    // past NB load the last block and are zeroed, so no branch splits the batch)
    constexpr int kBatch = 4;
#pragma unroll 1
    for (int n0 = 0; n0 < kSamp / 16; n0 += kBatch) {
      uint4 bb[kBatch][DI / 32];
      bool ok[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t col = (static_cast<int64_t>(n0 + j) * 16 + lr) * stride;
        ok[j] = col < a.NB;
        const int64_t cc = ok[j] ? col : a.NB - 1;
#pragma unroll
        for (int kc = 0; kc < DI / 32; ++kc)
          bb[j][kc] = *reinterpret_cast<const uint4*>(kb + cc * DI + kc * 32 + lg * 8);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        f32x4_t c = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < DI / 32; ++kc) {
          const uint4 u = ok[j] ? bb[j][kc] : make_uint4(0u, 0u, 0u, 0u);
          c = mfma16x16x32(qa[kc], bf16x8_from_u4(u), c);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          samp[(wave * 16 + lg * 4 + e) * kSamp + (n0 + j) * 16 + lr] =
              static_cast<uint16_t>(order_key_f(c[e]) >> 16);
      }
    }
    __syncthreads();
    // per row: the r-th largest sampled key (top 16 bits), one row at a time per wave
#pragma unroll 1
    for (int rloc = 0; rloc < 16; ++rloc) {
      const int local = wave * 16 + rloc;
      uint32_t thr = 0u;
      if (local < rows_here) {
        const int64_t o = row_o(local, nullptr);
        if (o > a.cap && o + 1 > a.NS) {
          const int nvalid = static_cast<int>((o + stride - 1) / stride);
          const int need = a.NS - 1;
          int r = static_cast<int>((2ll * need * nvalid + o - 1) / o);
          r = r < 1 ? 1 : (r > nvalid ? nvalid : r);
          uint32_t kv[kSamp / 64];
#pragma unroll
          for (int e = 0; e < kSamp / 64; ++e) {
            const int s = e * 64 + lane;
            kv[e] = s < nvalid ? samp[local * kSamp + s] : 0u;
          }
          uint32_t prefix = 0u;
#pragma unroll 1
          for (int bit = 15; bit >= 0; --bit) {
            const uint32_t cand = prefix | (1u << bit);
            int c = 0;
#pragma unroll
            for (int e = 0; e < kSamp / 64; ++e) c += __popcll(__ballot(kv[e] >= cand));
            if (c >= r) prefix = cand;
          }
          thr = prefix << 16;
        }
      }
      if (lane == 0) s_thr[local] = thr;
    }
  } else {
    if (threadIdx.x < kRows) s_thr[threadIdx.x] = 0u;
  }
  __syncthreads();
  // Phase 2 takes the products transposed (K_blk tile as the A operand, q_idx as B), so a lane
  // holds one row, the row of its A operand above, and four consecutive blocks of it per column step.
  // Per lane: float threshold (NaN for rows past the tile: never passes), causal limit o as 32 bits.
  const float r_thr = a_valid ? key_threshold_to_float(s_thr[my_local_a]) : __builtin_nanf("");
  int64_t my_rr = 0;
  const int32_t r_o32 = a_valid ? static_cast<int32_t>(row_o(my_local_a, &my_rr)) : 0;

  // ---------------- phase 2: every causal score, filtered, appended ----------------
  // A candidate is (float bits of the score << 32 | block).  A row's 4 lanes (lg = 0 .. 3, 16 lanes
  // apart) hold 16 consecutive blocks of it per step, 4 each in lg order; a passing score's slot is
  // the row's count so far plus the passing scores before it in block order, so every row's list
  // comes out in ascending block order.  The lanes' exclusive prefix comes from the two cross-row
  // swaps (16 lanes: the pair's even and odd row; 32 lanes: the lower and upper half), no LDS.
  // tiles below every row's causal limit need no per-column check
  const int64_t o_min = row_o(0, nullptr);
  const int64_t full_tiles = o_min / kCols;
  if (ntiles > 0) store_tile(0);
  // vmcnt(0): nothing loaded before this point (q_idx rows among it) stays outstanding into the tile
  // loops, so their only memory waits are for the next tile's loads
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // Candidate stores go through a buffer descriptor over this workgroup's rows, each under its
  // lane's pass bit (an exec mask: the selection an out-of-range offset would otherwise need costs
  // a VALU instruction per score, the mask a few scalar ones).
  const BufRsrc crs = make_rsrc(a.cand + (seq * a.seq_rows + row0) * a.cap,
                                static_cast<int64_t>(kRows) * a.cap * 8);
  const int r_off = my_local_a * a.cap * 8;
  int r_count = 0;                       // the row's passing scores so far (same in its 4 lanes)
  // Appends of kGrp consecutive column steps at once.  Each lane's pass counts of the steps are
  // packed one byte per step (at most 4 per lane, 16 per row and step: no byte carries into the
  // next), so one pair of cross-row swaps gives every step's exclusive prefix over the row's 4
  // lanes and its total.  A row whose list would run past the capacity in the group stores none
  // of the group's candidates: it then counts more than `cap` and is recomputed exactly.
  constexpr int kSteps = kCols / 16;
  constexpr int kGrp = kSteps / 2;
  auto append_group = [&](const f32x4_t* c, int32_t cb0, bool check_causal) {
    bool pass[kGrp][4];
    int nn[kGrp];
    uint32_t packed = 0u;
#pragma unroll
    for (int q = 0; q < kGrp; ++q) {
      nn[q] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pass[q][e] = c[q][e] >= r_thr;
        if (check_causal) pass[q][e] = pass[q][e] && cb0 + 16 * q + e < r_o32;
        nn[q] += static_cast<int>(pass[q][e]);
      }
      packed |= static_cast<uint32_t>(nn[q]) << (8 * q);
    }
    const auto p16 = __builtin_amdgcn_permlane16_swap(packed, packed, false, false);
    const uint32_t pair = p16[0] + p16[1];
    const auto p32 = __builtin_amdgcn_permlane32_swap(pair, pair, false, false);
    const uint32_t excl = ((lg & 1) ? p16[0] : 0u) + ((lg & 2) ? p32[0] : 0u);
    const uint32_t tot = p32[0] + p32[1];
    uint32_t all = 0u;
#pragma unroll
    for (int q = 0; q < kGrp; ++q) all += (tot >> (8 * q)) & 0xffu;
    const bool fits = r_count + static_cast<int>(all) <= a.cap;
    int base = r_count;
#pragma unroll
    for (int q = 0; q < kGrp; ++q) {
      int pos = base + static_cast<int>((excl >> (8 * q)) & 0xffu);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32x2_t v = {static_cast<uint32_t>(cb0 + 16 * q + e), __float_as_uint(c[q][e])};
        if (pass[q][e] && fits) __builtin_amdgcn_raw_buffer_store_b64(v, crs, r_off + pos * 8, 0, 0);
        pos += static_cast<int>(pass[q][e]);
      }
      base += static_cast<int>((tot >> (8 * q)) & 0xffu);
    }
    r_count = base;
  };
  // Per tile: all products first (LDS reads and MFMAs only), then the next tile's global loads,
  // then the appends (compares, LDS counters, candidate stores), then the staging of the next tile.
  // The loads are issued for every tile (past the last one they read zeros or unused blocks) and
  // the tiles below every row's causal limit run in a loop of their own, so the staging of the next
  // tile waits for the loads only.
  auto tile = [&](int64_t t, bool check_causal) {
    const int buf = static_cast<int>(t & 1);
    const unsigned char* src = lds + buf * kTileBytes;
    const int32_t col0 = static_cast<int32_t>(t * kCols) + 4 * lg;
    // B operands of step n+1 are read from LDS before the products of step n are issued
    f32x4_t sc[kCols / 16];
    uint4 opb[2][DI / 32];
    auto read_ops = [&](int n, uint4* op) {
#pragma unroll
      for (int kc = 0; kc < DI / 32; ++kc)
        op[kc] = *reinterpret_cast<const uint4*>(src + (n * 16 + lr) * kRowBytes + kc * 64 + lg * 16);
    };
    read_ops(0, opb[0]);
#pragma unroll
    for (int n = 0; n < kCols / 16; ++n) {
      if (n + 1 < kCols / 16) read_ops(n + 1, opb[(n + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);               // keep the reads ahead of the products
      f32x4_t c = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < DI / 32; ++kc) c = mfma16x16x32(bf16x8_from_u4(opb[n & 1][kc]), qa[kc], c);
      sc[n] = c;
    }
    load_tile(t + 1);
#pragma unroll
    for (int n = 0; n < kSteps; n += kGrp) append_group(sc + n, col0 + n * 16, check_causal);
    store_tile(buf ^ 1);   // buf ^ 1 was released by the barrier that ended tile t - 1
    __syncthreads();
  };
  const int64_t t_full = full_tiles < ntiles ? full_tiles : ntiles;
  int64_t t = 0;
#pragma unroll 1
  for (; t < t_full; ++t) tile(t, false);
#pragma unroll 1
  for (; t < ntiles; ++t) tile(t, true);
  if (lg == 0 && a_valid) a.cnt[my_rr] = r_count;
}

// ------------------------------------------------------------------------------------------------
// select: one wave per row over its candidate list
// ------------------------------------------------------------------------------------------------
struct SelectArgs {
  const uint64_t* cand;
  const int32_t* cnt;
  int32_t* sel;
  int32_t* fail_list;
  int32_t* fail_count;
  const int32_t* seq_len;              // per-sequence key counts (nullable: every sequence is full)
  int64_t b0, i0, ntok, Tq, pos0, rows;
  int G, B, NS, cap, words, waves;     // words: bitmap words per row (ceil(NB / 32))
};

constexpr int kSelPer = 32;        // candidates per lane held in registers (cap <= 64 * kSelPer)

// The need-th largest of the wave's keys (slots >= NE are zero), searched bit by bit below `top`
// from the common prefix tau0, down to bit `low`: the result is one of the keys, so its bits below
// the lowest bit set in any key are zero.
template <int NE>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t* key, uint32_t tau0, int top, int low,
                                                int need) {
  uint32_t tau = tau0;
#pragma unroll 1
  for (int bit = top; bit >= low; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int c = 0;                                       // ballots counted on the scalar unit
#pragma unroll
    for (int e = 0; e < NE; ++e) c += __popcll(__ballot(key[e] >= cand));
    if (c >= need) tau = cand;
  }
  return tau;
}

// Each wave owns one row and two LDS bitmaps over the row's candidate blocks: blocks whose key is
// above tau, and blocks whose key equals tau.  Scanning them in block order emits the selection
// ascending, with the lowest-indexed ties taken first.
// kSorted: every list is in ascending block order (the prefill filter), so the selected blocks are
// emitted by a stable compaction of the list; otherwise (decode: lists appended by several
// workgroups) through block bitmaps in LDS.
template <bool kSorted>
__global__ void __launch_bounds__(256) select_candidates_kernel(SelectArgs a) {
  extern __shared__ uint32_t bm_all[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Row indices fit 32 bits (fewer than 2^31 rows), so the row's token, group and sequence come
  // from 32-bit divisions: a 64-bit division is a long scalar routine, and at one wave per row
  // these divisions were about a third of the kernel's scalar instructions.
  const uint32_t rr32 = blockIdx.x * static_cast<uint32_t>(a.waves) + static_cast<uint32_t>(wave);
  if (rr32 >= a.rows) return;                         // whole wave; no workgroup barriers below
  const int64_t rr = rr32;
  const uint32_t G32 = static_cast<uint32_t>(a.G), nt32 = static_cast<uint32_t>(a.ntok);
  const uint32_t tok32 = rr32 / G32;
  const int g = static_cast<int>(rr32 - tok32 * G32);
  const uint32_t sq32 = tok32 / nt32;
  const int64_t bseq = a.b0 + sq32;
  const int64_t i = a.i0 + (tok32 - sq32 * nt32);
  const int64_t p = seq_pos0(a.seq_len, bseq, a.pos0, a.Tq) + i;
  const int64_t o = p <= 0xffffffffll ? static_cast<int64_t>(static_cast<uint32_t>(p) / static_cast<uint32_t>(a.B))
                                      : p / a.B;
  int32_t* out = a.sel + ((bseq * a.Tq + i) * a.G + g) * a.NS;
  if (o + 1 <= a.NS) {
    for (int x = lane; x < a.NS; x += 64) out[x] = (x <= o) ? x : -1;
    return;
  }
  const int need = a.NS - 1;
  // The first 16 slots per lane (the usual list size) are loaded together with the count: they lie
  // inside the row's capacity region whatever the count, and slots past it are discarded below.
  // A row whose count is outside [NS - 1, cap] leaves for the exact fallback only after the keys
  // are reduced, so that no branch stands between these loads and the count.
  const uint64_t* cr = a.cand + rr * a.cap;
  constexpr int kSpec = 16;
  uint64_t spec[kSpec];
#pragma unroll
  for (int e = 0; e < kSpec; ++e) spec[e] = cr[e * 64 + lane];
  const int m_raw = a.cnt[rr];
  const bool fail = m_raw < need || m_raw > a.cap;
  const int m = fail ? 0 : m_raw;
  uint32_t key[kSelPer], col[kSelPer];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < kSelPer; ++e) {
    const int x = e * 64 + lane;
    key[e] = 0u;
    col[e] = 0u;
    if (e < kSpec) {                                  // branch-free use of the loaded slots
      const bool ok = x < m;
      const uint32_t k = order_key_f(__uint_as_float(static_cast<uint32_t>(spec[e] >> 32)));
      key[e] = ok ? k : 0u;
      col[e] = ok ? static_cast<uint32_t>(spec[e]) : 0u;
      kmin = ok ? min(kmin, k) : kmin;
      kmax = ok ? max(kmax, k) : kmax;
    } else if (x < m) {
      const uint64_t v = cr[x];
      key[e] = order_key_f(__uint_as_float(static_cast<uint32_t>(v >> 32)));
      col[e] = static_cast<uint32_t>(v);
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
    }
  }
  kmin = wave_reduce_u32(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
  kmax = wave_reduce_u32(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
  if (fail) {
    if (lane == 0) a.fail_list[atomicAdd(a.fail_count, 1)] = static_cast<int32_t>(rr);
    return;
  }
  // tau = the need-th largest key: the largest v with #(key >= v) >= need.  kmin <= tau <= kmax,
  // so the bits above the highest bit where kmin and kmax differ are those of kmin.  The search
  // counts over the register slots in use only (16, 20, 24 or all 32 per lane).
  const uint32_t diff = kmin ^ kmax;
  const int top = diff ? 31 - __clz(diff) : -1;
  const uint32_t tau0 = top >= 0 ? (kmin & ~((2u << top) - 1u)) : kmin;
  // lowest bit set in any key (integer-valued scores leave the low mantissa bits zero)
  uint32_t kor = 0u;
#pragma unroll
  for (int e = 0; e < kSelPer; ++e) kor |= key[e];
  kor = wave_reduce_u32(kor, [](uint32_t x, uint32_t y) { return x | y; });
  const int low = kor ? __builtin_ctz(kor) : 32;
  const int ne = (m + 63) >> 6;                          // register slots in use per lane
  const uint32_t tau = ne <= 16   ? kth_largest<16>(key, tau0, top, low, need)
                       : ne <= 20 ? kth_largest<20>(key, tau0, top, low, need)
                       : ne <= 24 ? kth_largest<24>(key, tau0, top, low, need)
                                  : kth_largest<kSelPer>(key, tau0, top, low, need);

  if constexpr (kSorted) {
    // Slots x = 64 e + lane are in block order: keys above tau are taken, and of the keys equal to
    // tau the first take_eq in block order; each taking lane writes at the count of takers before
    // it, so consecutive lanes write consecutive entries.
    const int m_u = __builtin_amdgcn_readfirstlane(m);   // the same in every lane
    int n_gt = 0;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e)
      if (e * 64 < m_u) n_gt += __popcll(__ballot(key[e] > tau));
    const int take_eq = need - n_gt;
    int seen_eq = 0, done = 0;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
      if (e * 64 >= m_u) continue;
      const bool eq = key[e] == tau;
      const uint64_t m_eq = __ballot(eq);
      const int eq_rank = seen_eq + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                        static_cast<uint32_t>(m_eq >> 32),
                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m_eq), 0u)));
      const bool take = key[e] > tau || (eq && eq_rank < take_eq);
      const uint64_t m_take = __ballot(take);
      const int before = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
          static_cast<uint32_t>(m_take >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m_take), 0u)));
      if (take) out[done + before] = static_cast<int32_t>(col[e]);
      done += __popcll(m_take);
      seen_eq += __popcll(m_eq);
    }
    if (lane == 0) out[need] = static_cast<int32_t>(o);
    return;
  }
  // bitmaps over blocks 0 .. o-1: above tau, equal to tau; then this wave's copy of the output row
  const int nw = static_cast<int>((o + 31) >> 5);
  uint32_t* bgt = bm_all + static_cast<size_t>(wave) * (2 * a.words + a.NS);
  uint32_t* beq = bgt + a.words;
  int32_t* stg = reinterpret_cast<int32_t*>(beq + a.words);
  for (int w = lane; w < nw; w += 64) {
    bgt[w] = 0u;
    beq[w] = 0u;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  int gt = 0;
#pragma unroll
  for (int e = 0; e < kSelPer; ++e) {
    if (key[e] > tau) {
      atomicOr(&bgt[col[e] >> 5], 1u << (col[e] & 31));
      ++gt;
    } else if (key[e] == tau) {
      atomicOr(&beq[col[e] >> 5], 1u << (col[e] & 31));
    }
  }
  int take_eq = need - wave_total(gt);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // each lane scans a contiguous run of words; ties are taken in block order up to take_eq
  const int per = (nw + 63) >> 6;
  const int w0 = lane * per, w1 = min(w0 + per, nw);
  int n_eq = 0;
  for (int w = w0; w < w1; ++w) n_eq += __popc(beq[w]);
  int eq_before = wave_inclusive_scan(n_eq) - n_eq;     // exclusive prefix over lanes
  int n_sel = 0;
  for (int w = w0; w < w1; ++w) {
    uint32_t e = beq[w];
    uint32_t keep = 0u;
    while (e && eq_before < take_eq) {
      const uint32_t bit = e & (0u - e);
      keep |= bit;
      e ^= bit;
      ++eq_before;
    }
    const uint32_t x = bgt[w] | keep;
    bgt[w] = x;
    n_sel += __popc(x);
  }
  // A lane's selected blocks are one contiguous run of the row: they go to the LDS copy, which is
  // then written with consecutive lanes on consecutive entries (written straight to memory, every
  // entry of a store instruction would take its own cache line).
  int pos = wave_inclusive_scan(n_sel) - n_sel;         // exclusive prefix over lanes
  for (int w = w0; w < w1; ++w) {
    uint32_t x = bgt[w];
    while (x) {
      const int bit = __builtin_ctz(x);
      x &= x - 1u;
      stg[pos++] = 32 * w + bit;
    }
  }
  if (lane == 0) stg[need] = static_cast<int32_t>(o);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  for (int x = lane; x < a.NS; x += 64) out[x] = stg[x];
}

// ------------------------------------------------------------------------------------------------
// few rows per sequence (decode: T_q * G <= 32 rows over long rows)
// ------------------------------------------------------------------------------------------------
// With so few rows, one workgroup per 64 rows would leave most of the GPU idle while it streams the
// sequence's block keys.  The thresholds come first instead (kDecSamp sampled blocks per sequence,
// scored and ranked by four workgroups of 8 rows each), and the filter splits each
// sequence's blocks into slabs of kDecSlab, one workgroup per slab, scoring all 32 rows of the
// sequence at once (v_mfma_f32_32x32x16_bf16: rows are the A operand, 32 blocks per wave and
// step).  Each wave stages
// its passing scores in LDS, per row; when one more step could overflow a row's staging, and at the
// end of the slab, the wave reserves room in each row's list with one global atomic per row and
// copies its staged candidates there (no workgroup barriers).  A row's list is therefore unordered,
// as in the filter above.
constexpr int kDecRows = 32;
constexpr int kDecSamp = 2048;     // sampled blocks per sequence
constexpr int kDecSlab = 1024;     // blocks per filter workgroup: 8 steps of 32 blocks per wave
constexpr int kDecStage = 64;      // staged candidates per wave and row (a step adds at most 32)

struct DecodeArgs {
  const bf16_t* q_idx;
  const bf16_t* k_blk;
  const int32_t* seq_len;      // per-sequence key counts (nullable)
  uint32_t* thr;               // [chunk rows] threshold keys (low 16 bits clear)
  uint64_t* cand;              // [chunk rows][cap]
  int32_t* cnt;                // [chunk rows], zeroed by the threshold kernel
  int32_t* fail_count;         // zeroed by the threshold kernel
  int64_t b0, i0, Tq, pos0, NB, kblk_stride;
  int G, B, NS, cap, seq_rows;
};

// A operand of the 32 rows: row r of a sequence is token i0 + r / G, KV group r % G (all rows of a
// sequence share its length); rows past the sequence's rows load row 0 and are zeroed.
template <int DI>
__device__ __forceinline__ void dec_load_q(const DecodeArgs& a, int64_t b, int c, int h,
                                           bf16x8_t* qa) {
  const bool ok = c < a.seq_rows;
  const int row = ok ? c : 0;
  const bf16_t* qrow = a.q_idx + ((b * a.Tq + a.i0 + row / a.G) * a.G + row % a.G) * DI;
#pragma unroll
  for (int kc = 0; kc < DI / 16; ++kc) {
    const uint4 u = *reinterpret_cast<const uint4*>(qrow + 16 * kc + 8 * h);
    qa[kc] = bf16x8_from_u4(ok ? u : make_uint4(0u, 0u, 0u, 0u));
  }
}

// Row of C register r of a lane in half h of the wave (v_mfma_f32_32x32x16 output layout).
__device__ __forceinline__ int dec_c_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Thresholds: one workgroup per (sequence, group of 8 of its rows), 8 waves.  The group's rows are
// A rows 0-7 of v_mfma_f32_32x32x16_bf16 (the other 24 are zero), so their scores are C registers
// 0-3 of every lane.  kDecSamp blocks at a fixed stride are scored (each wave 8 steps of 32, loaded
// in two batches), their 16-bit keys kept in LDS, and then each wave ranks one row: the threshold is
// the r-th largest of the row's valid samples (sample s is valid for a row with o causal blocks when
// s * stride < o; r is chosen so that about twice the budget is expected to pass, as in the filter
// above).  Rows with at most `cap` causal blocks take every block.  Also clears the rows' candidate
// counts and the failure count.  Positions fit 32 bits on this path (checked on the host).
template <int DI>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_threshold_kernel(DecodeArgs a) {
  __shared__ uint16_t samp[8 * kDecSamp];                // 32 KB
  const int64_t seq = blockIdx.x;
  const int grp = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int64_t b = a.b0 + seq;
  const int64_t rr0 = seq * a.seq_rows;
  const int my_row = 8 * grp + wave;                     // the row this wave ranks
  if (seq == 0 && grp == 0 && threadIdx.x == 0) *a.fail_count = 0;
  if (lane == 0 && my_row < a.seq_rows) a.cnt[rr0 + my_row] = 0;
  if (8 * grp >= a.seq_rows) return;                     // whole workgroup
  const int32_t p0 = static_cast<int32_t>(seq_pos0(a.seq_len, b, a.pos0, a.Tq) + a.i0);
  const int32_t o_max = (p0 + (a.seq_rows - 1) / a.G) / a.B;
  if (o_max <= a.cap) {
    if (lane == 0 && my_row < a.seq_rows) a.thr[rr0 + my_row] = 0u;
    return;
  }
  const int32_t stride = (o_max + kDecSamp - 1) / kDecSamp;
  const bf16_t* kb = a.k_blk + b * a.kblk_stride * DI;
  constexpr int kSteps = kDecSamp / (8 * 32);
  constexpr int kBatch = 4;
  auto load_batch = [&](int s0, uint4 (*kk)[DI / 16]) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int32_t col = ((wave * kSteps + s0 + j) * 32 + c) * stride;
      const int32_t cc = col < a.NB ? col : static_cast<int32_t>(a.NB) - 1;   // never a valid sample
#pragma unroll
      for (int kc = 0; kc < DI / 16; ++kc)
        kk[j][kc] = *reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(cc) * DI + 16 * kc + 8 * h);
    }
  };
  uint4 kk[kBatch][DI / 16];
  load_batch(0, kk);
  bf16x8_t qa[DI / 16];
  {
    const int row = 8 * grp + c;
    const bool ok = c < 8 && row < a.seq_rows;
    const int rq = ok ? row : 0;
    const bf16_t* qrow = a.q_idx + ((b * a.Tq + a.i0 + rq / a.G) * a.G + rq % a.G) * DI;
#pragma unroll
    for (int kc = 0; kc < DI / 16; ++kc) {
      const uint4 u = *reinterpret_cast<const uint4*>(qrow + 16 * kc + 8 * h);
      qa[kc] = bf16x8_from_u4(ok ? u : make_uint4(0u, 0u, 0u, 0u));
    }
  }
#pragma unroll 1
  for (int s0 = 0; s0 < kSteps; s0 += kBatch) {
    __builtin_amdgcn_sched_barrier(0);                    // keep the batch's loads together
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      f32x16_t acc = {};
#pragma unroll
      for (int kc = 0; kc < DI / 16; ++kc) acc = mfma32x32x16(qa[kc], bf16x8_from_u4(kk[j][kc]), acc);
      const int sidx = (wave * kSteps + s0 + j) * 32 + c;
#pragma unroll
      for (int r = 0; r < 4; ++r)                         // C rows 4 h + r = the group's rows
        samp[(4 * h + r) * kDecSamp + sidx] = static_cast<uint16_t>(order_key_f(acc[r]) >> 16);
    }
    if (s0 + kBatch < kSteps) load_batch(s0 + kBatch, kk);
  }
  __syncthreads();
  if (my_row >= a.seq_rows) return;
  const int32_t o = (p0 + my_row / a.G) / a.B;
  uint32_t thr = 0u;
  if (o > a.cap) {
    const int nvalid = (o + stride - 1) / stride;
    const int need = a.NS - 1;
    int r = (2 * need * nvalid + o - 1) / o;
    r = r < 1 ? 1 : (r > nvalid ? nvalid : r);
    uint32_t kv[kDecSamp / 64];
#pragma unroll
    for (int e = 0; e < kDecSamp / 64; ++e) {
      const int sidx = e * 64 + lane;
      kv[e] = sidx < nvalid ? samp[wave * kDecSamp + sidx] : 0u;
    }
    uint32_t prefix = 0u;
#pragma unroll 1
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      int n = 0;
#pragma unroll
      for (int e = 0; e < kDecSamp / 64; ++e) n += __popcll(__ballot(kv[e] >= cand));
      if (n >= r) prefix = cand;
    }
    thr = prefix << 16;
  }
  if (lane == 0) a.thr[rr0 + my_row] = thr;
}

// One workgroup per (slab of kDecSlab blocks, sequence): every causal score of the sequence's rows
// in the slab, compared with the row's threshold; passing ones become candidates.
template <int DI>
__global__ void __launch_bounds__(256) decode_filter_kernel(DecodeArgs a) {
  // [wave][row][slot] staged candidates, then 64 slots per wave that lanes without a candidate
  // write to (so that the staging stores need no branch)
  constexpr int kWaveStage = kDecRows * kDecStage + 64;
  __shared__ uint64_t stage[4 * kWaveStage];             // 66 KB
  __shared__ float s_thr[kDecRows];
  __shared__ int32_t s_o[kDecRows];
  const int64_t seq = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int64_t b = a.b0 + seq;
  const int64_t rr0 = seq * a.seq_rows;
  const int64_t p0 = seq_pos0(a.seq_len, b, a.pos0, a.Tq) + a.i0;
  const int64_t o_max = (p0 + (a.seq_rows - 1) / a.G) / a.B;
  const int64_t c_begin = static_cast<int64_t>(blockIdx.x) * kDecSlab;
  const int64_t c_end = min(c_begin + kDecSlab, o_max);
  if (c_begin >= c_end) return;                          // whole workgroup

  // Lane (c, h) holds the MFMA operand of block c of the step: the k-range [16 kc + 8 h, +8) for
  // kc = 0 .. DI/16 - 1, read through a descriptor over the sequence's block keys (blocks past its
  // NB read 0; such columns are never causal), one step ahead, into two register sets used in turn.
  const BufRsrc krs = make_rsrc(a.k_blk + b * a.kblk_stride * DI, a.NB * DI * 2);
  auto load_keys = [&](int64_t col0, uint4* kk) {
    const int base = static_cast<int>((col0 + c) * (DI * 2)) + 16 * h;   // < 2^31 (checked on the host)
#pragma unroll
    for (int kc = 0; kc < DI / 16; ++kc)
      kk[kc] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, base + 32 * kc, 0, 0));
  };
  int64_t col0 = c_begin + 32 * wave;
  uint4 kA[DI / 16], kB[DI / 16];
  load_keys(col0, kA);
  bf16x8_t qa[DI / 16];
  dec_load_q<DI>(a, b, c, h, qa);
  // per row: the threshold as a float (NaN past the sequence's rows: never passes) and the causal
  // limit (0 past the rows), computed once per row
  if (threadIdx.x < kDecRows) {
    const int row = threadIdx.x;
    const bool ok = row < a.seq_rows;
    s_o[row] = ok ? static_cast<int32_t>((p0 + row / a.G) / a.B) : 0;
    s_thr[row] = ok ? key_threshold_to_float(a.thr[rr0 + row]) : __builtin_nanf("");
  }
  __syncthreads();
  float c_thr[16];
  int32_t o_r[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    c_thr[r] = s_thr[dec_c_row(r, h)];
    o_r[r] = s_o[dec_c_row(r, h)];
  }
  uint64_t* my_stage = stage + wave * kWaveStage;
  int n_lo[16], n_hi[16];           // staged per C register: rows of lanes 0-31 / 32-63 (uniform)
#pragma unroll
  for (int r = 0; r < 16; ++r) n_lo[r] = n_hi[r] = 0;
  // every valid row's causal limit is at least o_min (row 0 has the smallest)
  const int32_t o_min = s_o[0];
  // Staging of one step.  A passing score's slot is its row's staged count plus the passing lanes
  // of its half below it: mbcnt over the 64-bit ballot counts the set bits below the lane, which
  // for the upper half includes the whole lower half (subtracted through the row base).  Lanes
  // without a candidate store to their own dummy slot.
  auto append = [&](const f32x16_t& acc, int32_t col, bool causal) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      bool pass = acc[r] >= c_thr[r];
      if (causal) pass = pass && col < o_r[r];
      const uint64_t m = __ballot(pass);
      const uint32_t lo = static_cast<uint32_t>(m), hi = static_cast<uint32_t>(m >> 32);
      const int plo = __popc(lo);
      const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u)));
      const int row_base = h ? dec_c_row(r, 1) * kDecStage + n_hi[r] - plo
                             : dec_c_row(r, 0) * kDecStage + n_lo[r];
      const int slot = pass ? row_base + below : kDecRows * kDecStage + lane;
      my_stage[slot] = (static_cast<uint64_t>(__float_as_uint(acc[r])) << 32) | static_cast<uint32_t>(col);
      n_lo[r] += plo;
      n_hi[r] += __popc(hi);
    }
  };
  auto step = [&](const uint4* kcur, uint4* knext) {
    load_keys(col0 + 128, knext);
    const int32_t col = static_cast<int32_t>(col0 + c);
    f32x16_t acc = {};
#pragma unroll
    for (int kc = 0; kc < DI / 16; ++kc) acc = mfma32x32x16(qa[kc], bf16x8_from_u4(kcur[kc]), acc);
    if (col0 + 32 <= o_min)
      append(acc, col, false);
    else
      append(acc, col, true);
    col0 += 128;
  };
  // this wave's staged candidates -> the rows' lists: lane l < 32 reserves room for row l, then
  // each row's staged run is copied by the lanes below its count
  auto flush = [&]() {
    int n_mine = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      n_mine = lane == dec_c_row(r, 0) ? n_lo[r] : n_mine;
      n_mine = lane == dec_c_row(r, 1) ? n_hi[r] : n_mine;
    }
    int base = 0;
    if (n_mine > 0) base = atomicAdd(&a.cnt[rr0 + lane], n_mine);   // n_mine = 0 past the rows
#pragma unroll 1
    for (int row = 0; row < kDecRows; ++row) {
      const int n = __builtin_amdgcn_readlane(n_mine, row);
      if (n == 0) continue;
      const int dst = __builtin_amdgcn_readlane(base, row) + lane;
      if (lane < n && dst < a.cap) a.cand[(rr0 + row) * a.cap + dst] = my_stage[row * kDecStage + lane];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) n_lo[r] = n_hi[r] = 0;
  };
  // a step adds at most 32 candidates to a row: flush first when a row could overflow
  auto full = [&]() {
    int m = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) m = max(m, max(n_lo[r], n_hi[r]));
    return m > kDecStage - 32;
  };
  while (col0 < c_end) {
    step(kA, kB);
    if (full()) flush();
    if (col0 >= c_end) break;
    step(kB, kA);
    if (full()) flush();
  }
  flush();
}


// Rows per select workgroup: each needs two bitmaps of ceil(NB / 32) words and its NS output
// entries in LDS (0: none fits).
int select_waves(const Dims& d) {
  const int64_t per_wave = (2 * ((d.NB + 31) / 32) + d.NS) * static_cast<int64_t>(sizeof(uint32_t));
  const int64_t fit = (160 * 1024) / per_wave;
  return static_cast<int>(fit >= 4 ? 4 : fit);
}

}  // namespace

int fused_select_capacity() { return 64 * kSelPer; }

bool fused_select_supported(const Dims& d) {
  // the candidate list holds about twice the budget: budgets up to 512 blocks; the filter addresses
  // one sequence's block keys (and a tile past them) with 32-bit byte offsets
  return d.idx_bf16 && d.NS <= 513 && (d.Di == 32 || d.Di == 64 || d.Di == 128) &&
         (d.NB + 128) * static_cast<int64_t>(d.Di) * 2 < (int64_t(1) << 31);
}

hipError_t launch_index_filter(const Dims& d, const void* q_idx, const void* k_blk, uint64_t* cand,
                               int32_t* cnt, int32_t* fail_count, const Chunk& c, hipStream_t s) {
  // one sequence's K_blk is addressed with 32-bit byte offsets (up to 2^31 / 256 blocks at Di = 128)
  if ((d.NB + 128) * static_cast<int64_t>(d.Di) * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  FilterArgs a;
  a.q_idx = static_cast<const bf16_t*>(q_idx);
  a.k_blk = static_cast<const bf16_t*>(k_blk);
  a.cand = cand;
  a.cnt = cnt;
  a.fail_count = fail_count;
  a.b0 = c.b0;
  a.i0 = c.i0;
  a.ntok = c.ntok;
  a.Tq = d.Tq;
  a.pos0 = d.pos0;
  a.NB = d.NB;
  a.seq_rows = c.ntok * d.G;
  a.tiles_per_seq = (a.seq_rows + kRows - 1) / kRows;
  a.G = d.G;
  a.B = d.B;
  a.NS = d.NS;
  a.cap = fused_select_capacity();
  const dim3 grid(static_cast<unsigned>(a.tiles_per_seq * c.nseq));
  if (d.Di == 128)
    hipLaunchKernelGGL(index_filter_kernel<128>, grid, dim3(256), 0, s, a);
  else if (d.Di == 64)
    hipLaunchKernelGGL(index_filter_kernel<64>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(index_filter_kernel<32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

bool decode_select_supported(const Dims& d, int64_t seq_rows) {
  // the filter addresses a sequence's block keys (and up to two slabs past them) with 32-bit offsets
  // (its lists are appended by several workgroups: the select orders them through LDS bitmaps)
  return fused_select_supported(d) && select_waves(d) >= 1 && seq_rows >= 1 && seq_rows <= kDecRows &&
         (d.NB + 2 * kDecSlab) * d.Di * 2 < (int64_t(1) << 31);
}

hipError_t launch_decode_select(const Dims& d, const void* q_idx, const void* k_blk, uint32_t* thr,
                                uint64_t* cand, int32_t* cnt, int32_t* fail_count, const Chunk& c,
                                hipStream_t s) {
  DecodeArgs a;
  a.q_idx = static_cast<const bf16_t*>(q_idx);
  a.k_blk = static_cast<const bf16_t*>(k_blk);
  a.seq_len = d.seq_len;
  a.thr = thr;
  a.cand = cand;
  a.cnt = cnt;
  a.fail_count = fail_count;
  a.b0 = c.b0;
  a.i0 = c.i0;
  a.Tq = d.Tq;
  a.pos0 = d.pos0;
  a.NB = d.NB;
  a.kblk_stride = d.kblk_stride > 0 ? d.kblk_stride : d.NB;
  a.G = d.G;
  a.B = d.B;
  a.NS = d.NS;
  a.cap = fused_select_capacity();
  a.seq_rows = static_cast<int>(c.ntok * d.G);
  if (c.nseq < 1) return hipSuccess;
  const int64_t max_o = (d.Tk - 1) / d.B;                // no row has more causal blocks
  const unsigned slabs = static_cast<unsigned>(max_o > 0 ? (max_o + kDecSlab - 1) / kDecSlab : 1);
  // blockIdx.x = sequence: a sequence's 4 threshold workgroups are dispatched to the same XCD and
  // share its L2 for the sampled block keys
  const dim3 tgrid(static_cast<unsigned>(c.nseq), kDecRows / 8);
  const dim3 fgrid(slabs, static_cast<unsigned>(c.nseq));
  if (d.Di == 128) {
    hipLaunchKernelGGL(decode_threshold_kernel<128>, tgrid, dim3(512), 0, s, a);
    hipLaunchKernelGGL(decode_filter_kernel<128>, fgrid, dim3(256), 0, s, a);
  } else if (d.Di == 64) {
    hipLaunchKernelGGL(decode_threshold_kernel<64>, tgrid, dim3(512), 0, s, a);
    hipLaunchKernelGGL(decode_filter_kernel<64>, fgrid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(decode_threshold_kernel<32>, tgrid, dim3(512), 0, s, a);
    hipLaunchKernelGGL(decode_filter_kernel<32>, fgrid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_select_candidates(const Dims& d, const uint64_t* cand, const int32_t* cnt,
                                    int32_t* sel, int32_t* fail_list, int32_t* fail_count,
                                    const Chunk& c, bool sorted, hipStream_t s) {
  SelectArgs a;
  a.cand = cand;
  a.cnt = cnt;
  a.sel = sel;
  a.fail_list = fail_list;
  a.fail_count = fail_count;
  a.seq_len = d.seq_len;
  a.b0 = c.b0;
  a.i0 = c.i0;
  a.ntok = c.ntok;
  a.Tq = d.Tq;
  a.pos0 = d.pos0;
  a.rows = c.rows(d.G);
  a.G = d.G;
  a.B = d.B;
  a.NS = d.NS;
  a.cap = fused_select_capacity();
  a.words = static_cast<int>((d.NB + 31) / 32);
  if (sorted) {
    a.waves = 4;
    const dim3 grid(static_cast<unsigned>((a.rows + a.waves - 1) / a.waves));
    hipLaunchKernelGGL(select_candidates_kernel<true>, grid, dim3(64 * a.waves), 0, s, a);
  } else {
    a.waves = select_waves(d);
    if (a.waves < 1) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>((a.rows + a.waves - 1) / a.waves));
    const size_t lds = static_cast<size_t>(a.waves) * (2 * a.words + a.NS) * sizeof(uint32_t);
    hipLaunchKernelGGL(select_candidates_kernel<false>, grid, dim3(64 * a.waves), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace sgqa
