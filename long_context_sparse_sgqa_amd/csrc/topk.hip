// Step 3 -- per-(query, KV group) block selection.
//
// The Step 5 Preview pages (mo.ai.kr summary, section "모델 구조와 학습 안정성"; ai.info article,
// section on Sparse GQA and the 1M context) let every KV group pick its own top-k past blocks, with
// k = 4096 tokens = 512 blocks of 8.  Readings fixed here: the own block o = p/B is always selected
// and counts toward the NS = k/B budget; of the candidates j < o the NS-1 with the highest scores
// are taken, equal scores going to the lower j; when o + 1 <= NS every block 0..o is taken.  The
// output lists the blocks ascending, padded with -1.
//
// One workgroup (256 threads) per row.  Scores become order-preserving 32-bit keys (-0.0 is folded
// into +0.0 first).  The NS-1'th largest key tau is found by an exact 4-pass radix select (8-bit
// digits, LDS histogram); every key > tau is taken, plus the lowest-indexed keys == tau until the
// budget is met.  The emit pass walks candidates in index order with wavefront ballots and prefix
// counts, so the output is ascending without a sort.
//
// Long rows first shrink the candidate set: a strided sample of 1024 scores gives a threshold whose
// expected pass count is about twice the budget; one streaming pass keeps the (key, index) pairs at
// or above it in per-wave LDS segments, in index order.  Every key of the true top NS-1 is >= that
// threshold whenever at least NS-1 candidates pass, so the select then runs on the short list.  If
// too few pass, or a segment overflows, the row is selected directly from the full score row
// instead.  Either way the result is exact.
#include "device_common.h"
#include "sgqa_internal.h"

namespace sgqa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kSegCap = 1024;                 // per-wave candidate capacity
constexpr int kSample = 1024;                 // sampled scores of a long row
constexpr int kDirectMax = 2048;              // rows this short are selected straight from scores
constexpr int kFallbackWorkgroups = 256;      // failed rows handled at once (scratch score rows)
constexpr int kFallbackSlab = 1024;           // blocks per score-recompute workgroup

struct TopkShared {
  uint32_t hist[256];
  int wave_cnt[kWaves];
  int seg_cnt[kWaves];
  int seg_off[kWaves + 1];
  uint32_t pick_digit;
  int pick_above;
  int flag;
  uint32_t key[kWaves * kSegCap];             // candidate keys (also the sample buffer)
  int32_t idx[kWaves * kSegCap];              // candidate block indices
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;                 // -0.0 and +0.0 are the same score
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Exclusive prefix of `flag` over the workgroup in thread order; *total gets the sum.
__device__ __forceinline__ int block_flag_scan(bool flag, int* total, TopkShared& sh) {
  const uint64_t bal = __ballot(flag);
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) sh.wave_cnt[wave] = __popcll(bal);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = sh.wave_cnt[w];
    off += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + in_wave;
}

// Candidate sources: key(x) and index(x) for x in [0, n).
struct RowSource {       // the full score row of one (query, group)
  const float* s;
  __device__ __forceinline__ uint32_t key(int x) const { return order_key(s[x]); }
  __device__ __forceinline__ int32_t index(int x) const { return x; }
};
struct SampleSource {    // sampled keys held in LDS
  const uint32_t* k;
  __device__ __forceinline__ uint32_t key(int x) const { return k[x]; }
  __device__ __forceinline__ int32_t index(int x) const { return x; }
};
struct SegSource {       // per-wave candidate segments, concatenated in wave order
  const TopkShared* sh;
  __device__ __forceinline__ int slot(int x) const {
    int w = 0;
#pragma unroll
    for (int v = 1; v < kWaves; ++v) w += (x >= sh->seg_off[v]) ? 1 : 0;
    return w * kSegCap + (x - sh->seg_off[w]);
  }
  __device__ __forceinline__ uint32_t key(int x) const { return sh->key[slot(x)]; }
  __device__ __forceinline__ int32_t index(int x) const { return sh->idx[slot(x)]; }
};

// The need-th largest key (1-based) of src[0, n): returns tau and *take_eq = how many keys equal
// to tau belong to the top `need` (the others above it are exactly the keys > tau).
template <class Src>
__device__ uint32_t radix_select(const Src& src, int n, int need, int* take_eq, TopkShared& sh) {
  uint32_t prefix = 0u, mask = 0u;
  int rem = need;
  const int t = threadIdx.x;
  for (int shift = 24; shift >= 0; shift -= 8) {
    sh.hist[t] = 0u;                                  // kThreads == 256 bins
    __syncthreads();
    for (int x = t; x < n; x += kThreads) {
      const uint32_t k = src.key(x);
      if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    // inclusive scan over digits from the top: thread t holds digit 255 - t
    const int h = static_cast<int>(sh.hist[255 - t]);
    int incl = wave_inclusive_scan(h);
    if (lane_id() == 63) sh.wave_cnt[t >> 6] = incl;
    __syncthreads();
    for (int w = 0; w < (t >> 6); ++w) incl += sh.wave_cnt[w];
    if (incl >= rem && incl - h < rem) {
      sh.pick_digit = static_cast<uint32_t>(255 - t);
      sh.pick_above = incl - h;
    }
    __syncthreads();
    prefix |= sh.pick_digit << shift;
    mask |= 255u << shift;
    rem -= sh.pick_above;
    __syncthreads();
  }
  *take_eq = rem;
  return prefix;
}

// Writes the selected indices of src[0, n) in index order: keys > tau, then keys == tau while fewer
// than take_eq of them have been taken.  Returns the number written.
template <class Src>
__device__ int emit_selected(const Src& src, int n, uint32_t tau, int take_eq, int need,
                             int32_t* out, TopkShared& sh) {
  int written = 0, eq_seen = 0;
  for (int base = 0; base < n && written < need; base += kThreads) {
    const int x = base + threadIdx.x;
    const uint32_t k = (x < n) ? src.key(x) : 0u;
    const bool gt = (x < n) && k > tau;
    const bool eq = (x < n) && k == tau;
    int eq_total;
    const int eq_rank = eq_seen + block_flag_scan(eq, &eq_total, sh);
    const bool take = gt || (eq && eq_rank < take_eq);
    int take_total;
    const int pos = written + block_flag_scan(take, &take_total, sh);
    if (take) out[pos] = src.index(x);
    written += take_total;
    eq_seen += eq_total;
  }
  return written;
}

// The selection of one row from its stored scores (candidates 0 .. o-1), by the whole workgroup:
// out[0 .. NS-1] ascending, the own block o last, or every causal block when o + 1 <= NS.
__device__ void topk_row(const float* __restrict__ srow, int64_t o, int NS, int32_t* __restrict__ out,
                         TopkShared& sh) {
  const int t = threadIdx.x;
  if (o + 1 <= NS) {                                 // dense: every causal block
    for (int x = t; x < NS; x += kThreads) out[x] = (x <= o) ? x : -1;
    return;
  }
  const int n = static_cast<int>(o);                 // candidates 0..o-1
  const int need = NS - 1;
  const RowSource row{srow};
  int take_eq = 0;
  uint32_t tau;
  bool done = false;

  if (n > kDirectMax) {
    // threshold from a strided sample, aiming at ~2x the budget passing
    for (int s = t; s < kSample; s += kThreads)
      sh.key[s] = row.key(static_cast<int>((static_cast<int64_t>(s) * n) / kSample));
    __syncthreads();
    int rs = static_cast<int>((2ll * need * kSample + n - 1) / n);
    rs = rs < 1 ? 1 : (rs > kSample ? kSample : rs);
    int dummy;
    const uint32_t guess = radix_select(SampleSource{sh.key}, kSample, rs, &dummy, sh);
    __syncthreads();                                 // sample buffer is reused below

    // stream the row once; each wave keeps its contiguous quarter's survivors in order
    const int wave = t >> 6, lane = lane_id();
    const int per_wave = ((n + kWaves - 1) / kWaves + 3) & ~3;   // multiple of 4: aligned quads
    const int lo = wave * per_wave;
    const int hi = min(n, lo + per_wave);
    int cnt = 0;
    // survivors of one 64-lane step in index order (lane l holds the keys x .. x + nq - 1)
    const uint64_t below = (1ull << lane) - 1ull;
    auto keep_step = [&](const uint32_t* kq, int x, int nq) {
      bool keep[4];
      uint64_t bal[4];
      int before = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        keep[q] = q < nq && (x + q < hi) && kq[q] >= guess;
        bal[q] = __ballot(keep[q]);
        before += __popcll(bal[q] & below);
      }
      int mine = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pos = cnt + before + mine;
        if (keep[q] && pos < kSegCap) {
          sh.key[wave * kSegCap + pos] = kq[q];
          sh.idx[wave * kSegCap + pos] = x + q;
        }
        mine += keep[q] ? 1 : 0;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) cnt += __popcll(bal[q]);
    };
    if ((reinterpret_cast<uintptr_t>(row.s) & 15u) == 0u) {
      // 16-byte loads through a descriptor over the candidates (reads past o return 0, and the keep
      // test masks them): lane l of a 256-wide step holds keys 4l .. 4l+3, kUnroll steps in flight.
      // A survivor's slot counts the survivors of lower lanes (all four components) and of its own
      // lane's lower components, so every wave segment stays in index order.
      constexpr int kUnroll = 8;
      const BufRsrc rs = make_rsrc(row.s, static_cast<int64_t>(n) * 4);
      for (int x0 = lo; x0 < hi; x0 += 256 * kUnroll) {
        uint32_t k[kUnroll][4];
#pragma unroll
        for (int e = 0; e < kUnroll; ++e) {
          const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, (x0 + 256 * e + 4 * lane) * 4, 0, 0);
#pragma unroll
          for (int q = 0; q < 4; ++q) k[e][q] = order_key(__uint_as_float(v[q]));
        }
#pragma unroll
        for (int e = 0; e < kUnroll; ++e) keep_step(k[e], x0 + 256 * e + 4 * lane, 4);
      }
    } else {
      // rows not 16-byte aligned: one key per lane and step, kUnroll steps in flight
      constexpr int kUnroll = 8;
      for (int x0 = lo; x0 < hi; x0 += 64 * kUnroll) {
        uint32_t k[kUnroll][4];
#pragma unroll
        for (int e = 0; e < kUnroll; ++e) {
          const int x = x0 + 64 * e + lane;
          k[e][0] = (x < hi) ? row.key(x) : 0u;
        }
#pragma unroll
        for (int e = 0; e < kUnroll; ++e) keep_step(k[e], x0 + 64 * e + lane, 1);
      }
    }
    if (lane == 0) sh.seg_cnt[wave] = cnt;
    __syncthreads();
    if (t == 0) {
      int off = 0, ok = 1;
      for (int w = 0; w < kWaves; ++w) {
        sh.seg_off[w] = off;
        off += sh.seg_cnt[w];
        ok &= (sh.seg_cnt[w] <= kSegCap) ? 1 : 0;
      }
      sh.seg_off[kWaves] = off;
      sh.flag = (ok && off >= need) ? off : -1;
    }
    __syncthreads();
    const int m = sh.flag;
    if (m >= 0) {
      const SegSource seg{&sh};
      tau = radix_select(seg, m, need, &take_eq, sh);
      emit_selected(seg, m, tau, take_eq, need, out, sh);
      done = true;
    }
  }
  if (!done) {
    tau = radix_select(row, n, need, &take_eq, sh);
    emit_selected(row, n, tau, take_eq, need, out, sh);
  }
  if (t == 0) out[need] = static_cast<int32_t>(o);   // the own block, last in ascending order
}

__global__ void __launch_bounds__(kThreads) topk_kernel(const float* __restrict__ scores,
                                                        int32_t* __restrict__ sel, int64_t NB,
                                                        int NS, int B, int G, int64_t Tq,
                                                        int64_t pos0, const int32_t* seq_len,
                                                        int64_t b0, int64_t i0, int64_t ntok) {
  __shared__ TopkShared sh;
  const int64_t rr = blockIdx.x;
  const int64_t tok = rr / G;
  const int g = static_cast<int>(rr - tok * G);
  const int64_t b = b0 + tok / ntok;
  const int64_t i = i0 + tok % ntok;
  const int64_t p = seq_pos0(seq_len, b, pos0, Tq) + i;
  topk_row(scores + rr * NB, p / B, NS, sel + ((b * Tq + i) * G + g) * NS, sh);
}

// Exact selection for rows the fused candidate filter could not settle (too few candidates passed
// the sampled threshold, or more than the candidate capacity).  The full score rows of the first
// kFallbackWorkgroups failed rows are recomputed by fallback_scores_kernel, whose workgroups share
// out (row, kFallbackSlab-block slab) items, so even one failed row is recomputed by many
// workgroups.  select_fallback_kernel then selects each of those rows from its scores as
// topk_kernel does (one workgroup per row), and walks any further failed rows one workgroup per
// row, recomputing their scores itself.  The list length is read from device memory: with no
// failed row both launches exit at once.

// failed row f -> its sequence and position, and its output row
struct FallbackRow {
  int64_t b, i;
  int g;
};
__device__ __forceinline__ FallbackRow fallback_row(int64_t rr, int G, int64_t b0, int64_t i0,
                                                    int64_t ntok) {
  const int64_t tok = rr / G;
  return FallbackRow{b0 + tok / ntok, i0 + tok % ntok, static_cast<int>(rr - tok * G)};
}

__global__ void __launch_bounds__(kThreads) fallback_scores_kernel(
    const bf16_t* __restrict__ q_idx, const bf16_t* __restrict__ k_blk,
    const int32_t* __restrict__ fail_list, const int32_t* __restrict__ fail_count,
    float* __restrict__ scratch, int64_t NB, int64_t kblk_stride, int Di, int B, int G, int64_t Tq,
    int64_t pos0, const int32_t* seq_len, int64_t b0, int64_t i0, int64_t ntok, int64_t slabs) {
  __shared__ float qs[128];
  const int nfail = *fail_count;
  const int64_t rows = nfail < kFallbackWorkgroups ? nfail : kFallbackWorkgroups;
  const int t = threadIdx.x;
  // items in row-major order: consecutive workgroups take consecutive slabs of one row
  for (int64_t item = blockIdx.x; item < rows * slabs; item += gridDim.x) {
    const int f = static_cast<int>(item / slabs);
    const int64_t j0 = (item - f * slabs) * kFallbackSlab;
    const FallbackRow R = fallback_row(fail_list[f], G, b0, i0, ntok);
    const int64_t o = (seq_pos0(seq_len, R.b, pos0, Tq) + R.i) / B;
    if (j0 >= o) continue;                                    // whole workgroup
    const bf16_t* qrow = q_idx + ((R.b * Tq + R.i) * G + R.g) * Di;
    __syncthreads();                                          // qs of the previous item is read
    if (t < Di) qs[t] = bf16_to_f32(qrow[t]);
    __syncthreads();
    const bf16_t* kb = k_blk + R.b * kblk_stride * Di;
    float* srow = scratch + static_cast<int64_t>(f) * NB;
    const int64_t j1 = j0 + kFallbackSlab < o ? j0 + kFallbackSlab : o;
    for (int64_t j = j0 + t; j < j1; j += kThreads) {
      const uint4* kr = reinterpret_cast<const uint4*>(kb + j * Di);
      float acc = 0.f;
      for (int c0 = 0; c0 < Di / 8; ++c0) {
        const uint4 w4 = kr[c0];
        const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc = fmaf(qs[c0 * 8 + 2 * h], __uint_as_float(w[h] << 16), acc);
          acc = fmaf(qs[c0 * 8 + 2 * h + 1], __uint_as_float(w[h] & 0xffff0000u), acc);
        }
      }
      srow[j] = acc;
    }
  }
}

__global__ void __launch_bounds__(kThreads) select_fallback_kernel(
    const bf16_t* __restrict__ q_idx, const bf16_t* __restrict__ k_blk,
    const int32_t* __restrict__ fail_list, const int32_t* __restrict__ fail_count,
    float* __restrict__ scratch, int32_t* __restrict__ sel, int64_t NB, int64_t kblk_stride, int Di,
    int NS, int B, int G, int64_t Tq, int64_t pos0, const int32_t* seq_len, int64_t b0, int64_t i0,
    int64_t ntok, int f0) {
  __shared__ TopkShared sh;
  __shared__ float qs[128];
  const int nfail = *fail_count;
  float* srow = scratch + static_cast<int64_t>(blockIdx.x) * NB;
  const int t = threadIdx.x;
  // this workgroup's row among the first f0, whose scores fallback_scores_kernel has written
  if (static_cast<int>(blockIdx.x) < nfail && static_cast<int>(blockIdx.x) < f0) {
    const FallbackRow R = fallback_row(fail_list[blockIdx.x], G, b0, i0, ntok);
    const int64_t o = (seq_pos0(seq_len, R.b, pos0, Tq) + R.i) / B;
    topk_row(srow, o, NS, sel + ((R.b * Tq + R.i) * G + R.g) * NS, sh);
    __syncthreads();                                          // sh and srow are reused below
  }
  for (int f = f0 + static_cast<int>(blockIdx.x); f < nfail; f += gridDim.x) {
    const int64_t rr = fail_list[f];
    const int64_t tok = rr / G;
    const int g = static_cast<int>(rr - tok * G);
    const int64_t b = b0 + tok / ntok;
    const int64_t i = i0 + tok % ntok;
    const int64_t o = (seq_pos0(seq_len, b, pos0, Tq) + i) / B;
    int32_t* out = sel + ((b * Tq + i) * G + g) * NS;
    const bf16_t* qrow = q_idx + ((b * Tq + i) * G + g) * Di;
    if (t < Di) qs[t] = bf16_to_f32(qrow[t]);
    __syncthreads();
    const bf16_t* kb = k_blk + b * kblk_stride * Di;
    // one block row per thread, 16 bytes (8 index dims) per load; four rows' loads are in flight at
    // once (one workgroup per CU, so registers are plentiful and latency is the cost)
    constexpr int kRowsInFlight = 4;
    for (int64_t j0 = t; j0 < o; j0 += kThreads * kRowsInFlight) {
      float acc[kRowsInFlight];
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) acc[u] = 0.f;
      for (int c0 = 0; c0 < Di / 8; c0 += 4) {
        uint4 w4[kRowsInFlight][4];
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u) {
          const int64_t j = j0 + static_cast<int64_t>(u) * kThreads;
          const uint4* kr = reinterpret_cast<const uint4*>(kb + (j < o ? j : 0) * Di);
#pragma unroll
          for (int q = 0; q < 4; ++q) w4[u][q] = (c0 + q < Di / 8) ? kr[c0 + q] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (c0 + q >= Di / 8) continue;
            const uint32_t w[4] = {w4[u][q].x, w4[u][q].y, w4[u][q].z, w4[u][q].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              acc[u] = fmaf(qs[(c0 + q) * 8 + 2 * h], __uint_as_float(w[h] << 16), acc[u]);
              acc[u] = fmaf(qs[(c0 + q) * 8 + 2 * h + 1], __uint_as_float(w[h] & 0xffff0000u), acc[u]);
            }
          }
      }
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const int64_t j = j0 + static_cast<int64_t>(u) * kThreads;
        if (j < o) srow[j] = acc[u];
      }
    }
    __syncthreads();
    const int need = NS - 1;
    int take_eq = 0;
    const RowSource row{srow};
    const uint32_t tau = radix_select(row, static_cast<int>(o), need, &take_eq, sh);
    emit_selected(row, static_cast<int>(o), tau, take_eq, need, out, sh);
    if (t == 0) out[need] = static_cast<int32_t>(o);
    __syncthreads();
  }
}

}  // namespace

size_t select_fallback_scratch_bytes(const Dims& d) {
  return static_cast<size_t>(kFallbackWorkgroups) * static_cast<size_t>(d.NB) * sizeof(float);
}

hipError_t launch_select_fallback(const Dims& d, const void* q_idx, const void* k_blk,
                                  const int32_t* fail_list, const int32_t* fail_count,
                                  float* scratch, int32_t* sel, const Chunk& c, hipStream_t s) {
  const int64_t kstride = d.kblk_stride > 0 ? d.kblk_stride : d.NB;
  const int64_t max_o = (d.Tk - 1) / d.B;               // no row has more causal blocks
  const unsigned slabs = static_cast<unsigned>(max_o > 0 ? (max_o + kFallbackSlab - 1) / kFallbackSlab : 1);
  hipLaunchKernelGGL(fallback_scores_kernel, dim3(kFallbackWorkgroups), dim3(kThreads), 0, s,
                     static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_blk), fail_list,
                     fail_count, scratch, d.NB, kstride, d.Di, d.B, d.G, d.Tq, d.pos0, d.seq_len, c.b0,
                     c.i0, c.ntok, static_cast<int64_t>(slabs));
  hipLaunchKernelGGL(select_fallback_kernel, dim3(kFallbackWorkgroups), dim3(kThreads), 0, s,
                     static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_blk), fail_list,
                     fail_count, scratch, sel, d.NB, kstride, d.Di, d.NS, d.B, d.G, d.Tq, d.pos0,
                     d.seq_len, c.b0, c.i0, c.ntok, kFallbackWorkgroups);
  return hipGetLastError();
}

hipError_t launch_topk(const Dims& d, const float* scores, int32_t* sel, const Chunk& c,
                       hipStream_t s) {
  const int64_t rows = c.rows(d.G);
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0, s, scores,
                     sel, d.NB, d.NS, d.B, d.G, d.Tq, d.pos0, d.seq_len, c.b0, c.i0, c.ntok);
  return hipGetLastError();
}

}  // namespace sgqa
