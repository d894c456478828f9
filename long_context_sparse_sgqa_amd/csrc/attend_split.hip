// Step 4, range-split variant: gated GQA over the selected tokens, with each query's selected units
// split into R contiguous unit ranges that run on different XCDs and are merged afterwards.
//
// Same method as attend.hip (Step 5 Preview pages, mo.ai.kr summary, section
// "모델 구조와 학습 안정성": Sparse GQA on Gated GQA attends only over each KV group's selected
// blocks).  Gathering the selected K/V units is what bounds this step; most of those gathers are L2
// misses when every XCD serves random units of a whole group.  Here range r of every query goes to
// the workgroups numbered r mod R, which the dispatcher deals to XCDs r, r+R, ..., so each XCD's L2
// caches only 1/R of a group's K/V: the popular part of that range fits, and the hit rate rises.
//
// Three kernels:
//   pair_union_kernel  per (sequence, group, token pair): the sorted union of the two tokens'
//     selected 8-token units, entry = unit | token-A-chose << 30 | token-B-chose << 31 (B is a
//     multiple of 8, so a unit is wholly selected by a token or not at all), built through LDS
//     bitmaps; every range is padded to a multiple of 4 entries and its first entry recorded.
//   attend_range_kernel  one wavefront per (pair, range), 16 rows = 2 tokens x 8 heads: the pair's
//     entries inside the range in chunks of 4 units (S^T = K Q^T and O^T += V^T P^T on
//     v_mfma_f32_16x16x32_bf16, masked online softmax in the exp2 domain), ending in a partial
//     per row: O / l rounded to bf16, and the running max m and sum l in fp32.  K and V come from the unit-packed
//     copies, whose layout makes every 16-lane operand load one 256-byte run; K is loaded two chunks
//     and V one chunk ahead of use, and list entries arrive by scalar loads, so each wave keeps
//     about three chunks of operands in flight.
//   merge_ranges_kernel  per row: weight each partial by its sum rescaled to the common max,
//     combine, apply sigmoid(gate), round to bf16.
#include "device_common.h"
#include "sgqa_internal.h"
#include "units.h"

namespace sgqa {
namespace {

constexpr int kRanges = 4;                      // unit ranges per query
constexpr int kRangeWaves = 4;                  // pairs per workgroup (one per wave)
constexpr uint32_t kUnitMask = 0x3fffffffu;
// Entries of one pair's list: the union (at most 2 umax) with every range padded to a multiple of 4
// entries, plus 16 entries the range kernel may read (and discard) past the end of the last chunk.
__host__ __device__ constexpr int64_t list_stride(int umax) {
  return (2 * static_cast<int64_t>(umax) + 4 * kRanges + 16 + 3) / 4 * 4;
}

// ------------------------------------------------------------------------------------------------
// pair unions
// ------------------------------------------------------------------------------------------------
struct UnionArgs {
  const int32_t* sel;
  uint32_t* ulist;         // [Bt * G * pairs][list_stride(umax)]
  int32_t* bounds;         // [Bt * G * pairs][kRanges + 1]: first entry of each range, then end
  int64_t Tq, pos0, pairs, total;
  int G, NS, B, umax, words;   // words: bitmap words per token (ceil(NU / 32))
};

// Unit ranges of a pair: range r covers units [r * u_end / R, (r + 1) * u_end / R) of the pair's
// causal unit axis [0, u_end), u_end = last token's own unit + 1.
__device__ __forceinline__ uint32_t range_start(int r, int64_t u_end) {
  return static_cast<uint32_t>((r * u_end) / kRanges);
}

// Union through two LDS bitmaps (one bit per unit for each token of the pair): each selected block
// sets its units' bits (units past the token's own unit are left out: t <= p), then one scan over
// the words emits the union in ascending unit order with both tokens' chosen bits, each range
// padded to a multiple of 4 entries.
__global__ void __launch_bounds__(256) pair_union_kernel(UnionArgs a) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gp = static_cast<int64_t>(blockIdx.x) * 4 + wave;   // (b * G + g) * pairs + pair
  if (gp >= a.total) return;                          // whole wave; no workgroup barriers below
  uint32_t* bmA = lds + static_cast<size_t>(wave) * 2 * a.words;
  uint32_t* bmB = bmA + a.words;
  const int64_t pair = gp % a.pairs;
  const int64_t bg = gp / a.pairs;
  const int64_t g = bg % a.G, b = bg / a.G;
  const int64_t tokA = 2 * pair;
  const bool hasB = tokA + 1 < a.Tq;
  const int64_t pA = a.pos0 + tokA;
  const int64_t u_end = ((pA + (hasB ? 1 : 0)) >> 3) + 1;        // units 0 .. u_end-1 can occur
  const int nw = static_cast<int>((u_end + 31) >> 5);
  for (int w = lane; w < nw; w += 64) {
    bmA[w] = 0u;
    bmB[w] = 0u;
  }
  const int U = a.B >> 3;                               // units per block
  auto mark = [&](const int32_t* selrow, int64_t p, uint32_t* bm) {
    const int64_t o = p / a.B, last_unit = p >> 3;
    for (int e = lane; e < a.NS; e += 64) {
      const int blk = selrow[e];
      if (blk < 0 || blk > o) continue;
      for (int k = 0; k < U; ++k) {
        const int64_t u = static_cast<int64_t>(blk) * U + k;
        if (u <= last_unit) atomicOr(&bm[u >> 5], 1u << (u & 31));
      }
    }
  };
  mark(a.sel + ((b * a.Tq + tokA) * a.G + g) * a.NS, pA, bmA);
  if (hasB) mark(a.sel + ((b * a.Tq + tokA + 1) * a.G + g) * a.NS, pA + 1, bmB);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // each lane owns a contiguous run of words; counts below each range start and in total
  const int per = (nw + 63) >> 6;
  const int w0 = lane * per, w1 = min(w0 + per, nw);
  uint32_t lo[kRanges + 1];
#pragma unroll
  for (int r = 0; r <= kRanges; ++r) lo[r] = r < kRanges ? range_start(r, u_end) : static_cast<uint32_t>(u_end);
  int mine = 0;
  int below[kRanges + 1];
#pragma unroll
  for (int r = 0; r <= kRanges; ++r) below[r] = 0;
  for (int w = w0; w < w1; ++w) {
    const uint32_t x = bmA[w] | bmB[w];
    mine += __popc(x);
#pragma unroll
    for (int r = 1; r < kRanges; ++r) {
      const int64_t rel = static_cast<int64_t>(lo[r]) - 32 * w;   // bits of this word below lo[r]
      const uint32_t m = rel >= 32 ? 0xffffffffu : (rel <= 0 ? 0u : ((1u << rel) - 1u));
      below[r] += __popc(x & m);
    }
  }
  // exclusive prefix of `mine` over the lanes, and the totals
  int incl = mine;
#pragma unroll
  for (int o2 = 1; o2 < 64; o2 <<= 1) {
    const int v = __shfl_up(incl, o2, 64);
    if (lane >= o2) incl += v;
  }
  const int nu = __shfl(incl, 63, 64);
  int excl = incl - mine;
#pragma unroll
  for (int r = 1; r < kRanges; ++r) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) below[r] += __shfl_xor(below[r], m, 64);
  }
  below[0] = 0;
  below[kRanges] = nu;
  int start[kRanges + 1];
  start[0] = 0;
#pragma unroll
  for (int r = 0; r < kRanges; ++r) start[r + 1] = start[r] + ((below[r + 1] - below[r] + 3) & ~3);

  uint32_t* out = a.ulist + gp * list_stride(a.umax);
  for (int w = w0; w < w1; ++w) {
    const uint32_t xa = bmA[w], xb = bmB[w];
    uint32_t x = xa | xb;
    while (x) {
      const int bit = __builtin_ctz(x);
      x &= x - 1u;
      const uint32_t u = static_cast<uint32_t>(32 * w + bit);
      int r = 0;
#pragma unroll
      for (int q = 1; q < kRanges; ++q) r += u >= lo[q] ? 1 : 0;
      int shift = 0;
#pragma unroll
      for (int q = 0; q < kRanges; ++q) shift = q == r ? start[q] - below[q] : shift;
      out[excl + shift] = u | (((xa >> bit) & 1u) << 30) | (((xb >> bit) & 1u) << 31);
      ++excl;
    }
  }
  if (lane < 4 * kRanges) {                      // padding entries (unit 0, chosen by neither)
    const int r = lane >> 2, j = start[r] + (below[r + 1] - below[r]) + (lane & 3);
    if (j < start[r + 1]) out[j] = 0u;
  }
  int32_t* bnd = a.bounds + gp * (kRanges + 1);
  if (lane <= kRanges) {
    int v = 0;
#pragma unroll
    for (int q = 0; q <= kRanges; ++q) v = q == lane ? start[q] : v;
    bnd[lane] = v;
  }
}

// ------------------------------------------------------------------------------------------------
// one unit range of one pair
// ------------------------------------------------------------------------------------------------
struct RangeArgs {
  const bf16_t* q;
  const bf16_t* kp;
  const bf16_t* vp;
  const uint32_t* ulist;
  const int32_t* bounds;
  bf16_t* part_o;          // [gp][R][16 rows][D], normalised by the partial's own sum
  float2* part_ml;         // [gp][R][16 rows]  (running max in the exp2 domain, sum)
  int64_t Tq, Tk, NU, pos0, pairs, pair_groups;
  int G, umax;
  float scale_log2e;
};

template <int D>
__global__ void __launch_bounds__(256) attend_range_kernel(RangeArgs a) {
  constexpr int H = 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int lr = lane & 15, lg = lane >> 4;
  const int X = lr >> 3, head = lr & 7;
  // workgroup id: range fastest, so the range decides the XCD
  const int r = static_cast<int>(blockIdx.x % kRanges);
  const int64_t rest = blockIdx.x / kRanges;
  const int64_t pg = rest % a.pair_groups;
  const int64_t bg = rest / a.pair_groups;
  const int g = static_cast<int>(bg % a.G);
  const int64_t b = bg / a.G;
  const int64_t pair = pg * kRangeWaves + wave;
  if (pair >= a.pairs) return;                         // whole wave; no workgroup barriers follow
  const int64_t gp = bg * a.pairs + pair;
  const int64_t tokA = 2 * pair;
  const bool validB = tokA + 1 < a.Tq;
  const bool rowvalid = X ? validB : true;
  const int64_t pX = a.pos0 + tokA + X;

  const uint32_t* list = a.ulist + gp * list_stride(a.umax);
  const int32_t* bnd = a.bounds + gp * (kRanges + 1);
  const int e0 = __builtin_amdgcn_readfirstlane(bnd[r]);
  const int e1 = __builtin_amdgcn_readfirstlane(bnd[r + 1]);

  bf16x8_t qf[D / 32];
  const bf16_t* qrow = a.q + (((b * a.Tq + (rowvalid ? tokA + X : tokA)) * a.G + g) * H + head) * D;
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc)
    qf[kc] = rowvalid ? load_bf16x8(qrow + 32 * kc + 8 * lg) : zero_bf16x8();

  const BufRsrc krs = make_rsrc(a.kp + (b * a.G + g) * a.NU * D * 8, a.NU * D * 16);
  const BufRsrc vrs = make_rsrc(a.vp + (b * a.G + g) * a.NU * D * 8, a.NU * D * 16);

  // List entries are read with scalar loads (constant address space, wave-uniform, 16-byte aligned
  // because ranges start at multiples of 4): they count against lgkmcnt, so reading them never
  // waits behind the K/V loads in flight.  Entries at or past e1 read as 0 (unit 0, not chosen).
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) u32x4* ConstQuadPtr;
  auto chunk_entries = [&](int c, uint32_t* ent4) {
    const u32x4 v = *((ConstQuadPtr)(list + c));
#pragma unroll
    for (int j = 0; j < 4; ++j) ent4[j] = c < e1 ? v[j] : 0u;
  };
  auto pick4 = [](const uint32_t* v, int i) -> uint32_t {
    return i == 0 ? v[0] : (i == 1 ? v[1] : (i == 2 ? v[2] : v[3]));
  };

  // K operands of a chunk (4 units) go to registers: unit slot lr/4, rows lr%4 and lr%4 + 4.
  struct KRegs { bf16x8_t k1[D / 32], k2[D / 32]; };
  auto load_k = [&](const uint32_t* ent4, KRegs& R) {
    const int u = static_cast<int>(pick4(ent4, lr >> 2) & kUnitMask);
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) {
      R.k1[kc] = buffer_load_bf16x8(krs, kp_offset(u, D, kc, 0, lg, lr));
      R.k2[kc] = buffer_load_bf16x8(krs, kp_offset(u, D, kc, 1, lg, lr));
    }
  };
  // V^T operands of a chunk go to registers too: unit slot lg, coalesced 256-byte runs.
  struct VRegs { bf16x8_t v[D / 16]; };
  auto load_v = [&](const uint32_t* ent4, VRegs& R) {
    const int vo = (static_cast<int>(pick4(ent4, lg) & kUnitMask) * D + lr) * 16;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) R.v[t] = buffer_load_bf16x8(vrs, vo + t * 256);
  };

  f32x4_t acc[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;
  const float ninf = -__builtin_inff();

  // one chunk: S^T = K Q^T (tokens 0-3 of each unit slot in s1, 4-7 in s2), masks, online softmax,
  // O^T += V^T P^T.  `refill` runs once S has consumed K, to reuse its registers.
  auto chunk = [&](const KRegs& K, const VRegs& V, const uint32_t* ent4, auto refill) {
    const uint32_t ent = pick4(ent4, lg);
    const int unitS = static_cast<int>(ent & kUnitMask);
    f32x4_t s1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t s2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) {
      s1 = mfma16x16x32(K.k1[kc], qf[kc], s1);
      s2 = mfma16x16x32(K.k2[kc], qf[kc], s2);
    }
    refill();
    const bool chose = X ? (ent >> 31) : ((ent >> 30) & 1u);     // 0 past the range (ent = 0)
    const int64_t dlt = pX - static_cast<int64_t>(unitS) * 8;
    const uint32_t causal = dlt >= 7 ? 0xffu : (dlt < 0 ? 0u : ((2u << dlt) - 1u));
    const uint32_t valid = chose ? causal : 0u;
    float sv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = ((valid >> e) & 1u) ? s1[e] * a.scale_log2e : ninf;
      sv[e + 4] = ((valid >> (e + 4)) & 1u) ? s2[e] * a.scale_log2e : ninf;
    }
    float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run + kLazyRescaleLog2)) {   // a row's max grew by > margin: rescale all
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) acc[t] *= alpha;
      m_run = m_new;
    }
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = __builtin_amdgcn_exp2f(sv[e] - m_run);
      l_run += pv[e];
    }
    const bf16x8_t pf = pack8_bf16(pv);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc[t] = mfma16x16x32(V.v[t], pf, acc[t]);
  };

  // Software pipeline over chunks of 4 units (past the range's end the loads fetch unit 0 and are
  // masked out): K is loaded two chunks ahead and V one chunk ahead, two register sets each.  Per
  // chunk x: V(x+4) is issued first, then K(x+8) once S(x) has freed its set; the compiler's vmcnt
  // waits then leave up to three chunks' worth of K/V in flight.
  if (e0 < e1) {
    uint32_t ec[4], e1c[4], e2c[4], e3c[4];           // entries of chunks x, x+4, x+8, x+12
    chunk_entries(e0, ec);
    chunk_entries(e0 + 4, e1c);
    chunk_entries(e0 + 8, e2c);
    KRegs kA, kB;
    VRegs v0, v1;
    load_k(ec, kA);
    load_k(e1c, kB);
    load_v(ec, v0);
    int nx = e0 + 12;                                  // next chunk whose entries are read
    auto step = [&](KRegs& K, VRegs& Vcur, VRegs& Vnext) {
      chunk_entries(nx, e3c);                          // entries a chunk ahead of their use
      nx += 4;
      load_v(e1c, Vnext);
      chunk(K, Vcur, ec, [&] { load_k(e2c, K); });
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ec[j] = e1c[j];
        e1c[j] = e2c[j];
        e2c[j] = e3c[j];
      }
    };
    // the loop body is one period of the register rotation, so every trip enters with the same
    // loads in flight; the first chunk and the tail run outside it
    step(kA, v0, v1);
    int rem = (e1 - e0 - 4) >> 2;                      // chunks left
    for (; rem >= 2; rem -= 2) {
      step(kB, v1, v0);
      step(kA, v0, v1);
    }
    if (rem >= 1) step(kB, v1, v0);
  }

  // partial of this range: O / l in bf16 (0 for a row with nothing in the range), and the running
  // max m and sum l per row in fp32
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t pbase = (gp * kRanges + r) * 16 + lr;
  bf16_t* po = a.part_o + pbase * D;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    uint2 w;
    w.x = pack_bf16x2(acc[t][0] * inv, acc[t][1] * inv);
    w.y = pack_bf16x2(acc[t][2] * inv, acc[t][3] * inv);
    *reinterpret_cast<uint2*>(po + 16 * t + 4 * lg) = w;
  }
  if (lg == 0) a.part_ml[pbase] = make_float2(m_run, l_tot);
}

// ------------------------------------------------------------------------------------------------
// merge of the range partials, gate, bf16 output
// ------------------------------------------------------------------------------------------------
struct MergeArgs {
  const bf16_t* part_o;
  const float2* part_ml;
  const bf16_t* gate;
  bf16_t* out;
  int64_t Tq, pairs, total_pairs;
  int G, D;
};

__global__ void __launch_bounds__(256) merge_ranges_kernel(MergeArgs a) {
  const int per_row = a.D / 4;
  const int64_t total = a.total_pairs * 16 * per_row;
  for (int64_t id = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; id < total;
       id += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int d0 = static_cast<int>(id % per_row) * 4;
    const int64_t gr = id / per_row;                 // gp * 16 + row
    const int row = static_cast<int>(gr % 16);
    const int64_t gp = gr / 16;
    const int64_t pair = gp % a.pairs;
    const int64_t bg = gp / a.pairs;
    const int64_t tok = 2 * pair + (row >> 3);
    if (tok >= a.Tq) continue;
    const int64_t g = bg % a.G, b = bg / a.G;
    float mx = -1e30f;
#pragma unroll
    for (int r = 0; r < kRanges; ++r) mx = fmaxf(mx, a.part_ml[(gp * kRanges + r) * 16 + row].x);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < kRanges; ++r) {
      const int64_t pb = (gp * kRanges + r) * 16 + row;
      const float2 ml = a.part_ml[pb];
      const float w = ml.y * __builtin_amdgcn_exp2f(ml.x - mx);     // partial sum at the common max
      L += w;
      const uint2 pw = *reinterpret_cast<const uint2*>(a.part_o + pb * a.D + d0);
      o.x += bf16_to_f32(static_cast<bf16_t>(pw.x & 0xffffu)) * w;
      o.y += bf16_to_f32(static_cast<bf16_t>(pw.x >> 16)) * w;
      o.z += bf16_to_f32(static_cast<bf16_t>(pw.y & 0xffffu)) * w;
      o.w += bf16_to_f32(static_cast<bf16_t>(pw.y >> 16)) * w;
    }
    const float inv = 1.f / L;
    const int64_t obase = (((b * a.Tq + tok) * a.G + g) * 8 + (row & 7)) * a.D + d0;
    const uint2 gw = *reinterpret_cast<const uint2*>(a.gate + obase);
    const float g0 = bf16_to_f32(static_cast<bf16_t>(gw.x & 0xffffu));
    const float g1 = bf16_to_f32(static_cast<bf16_t>(gw.x >> 16));
    const float g2 = bf16_to_f32(static_cast<bf16_t>(gw.y & 0xffffu));
    const float g3 = bf16_to_f32(static_cast<bf16_t>(gw.y >> 16));
    uint2 ow;
    ow.x = pack_bf16x2(o.x * inv / (1.f + __expf(-g0)), o.y * inv / (1.f + __expf(-g1)));
    ow.y = pack_bf16x2(o.z * inv / (1.f + __expf(-g2)), o.w * inv / (1.f + __expf(-g3)));
    *reinterpret_cast<uint2*>(a.out + obase) = ow;
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

bool attend_split_supported(const Dims& d) {
  // the pair-union bitmaps of 4 waves (2 x ceil(NU/32) words each) must fit in 160 KiB of LDS
  return d.bf16 && d.H == 8 && (d.D == 64 || d.D == 128) && d.B % 8 == 0 &&
         d.NU * 8 * static_cast<int64_t>(d.D) * 2 < (int64_t(1) << 31) &&
         units_per_query(d) <= 1024 && (d.NU + 31) / 32 <= 5120;
}

size_t attend_split_bytes(const Dims& d) {
  const int64_t pairs = (d.Tq + 1) / 2;
  const size_t n = static_cast<size_t>(d.Bt * d.G * pairs);
  const size_t umax = static_cast<size_t>(units_per_query(d));
  return align256(n * list_stride(static_cast<int>(umax)) * sizeof(uint32_t)) +
         align256(n * (kRanges + 1) * sizeof(int32_t)) +
         align256(n * kRanges * 16 * d.D * sizeof(bf16_t)) + align256(n * kRanges * 16 * sizeof(float2));
}

hipError_t launch_attend_split(const Dims& d, const void* q, const void* packed_k,
                               const void* gate, const int32_t* sel, void* out,
                               const void* packed_v, void* ws, hipStream_t s, StageMark mark) {
  const int64_t pairs = (d.Tq + 1) / 2;
  const int64_t total = d.Bt * d.G * pairs;
  const int umax = static_cast<int>(units_per_query(d));
  char* p = static_cast<char*>(ws);
  uint32_t* ulist = reinterpret_cast<uint32_t*>(p);
  p += align256(static_cast<size_t>(total) * list_stride(umax) * sizeof(uint32_t));
  int32_t* bounds = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(total) * (kRanges + 1) * sizeof(int32_t));
  bf16_t* part_o = reinterpret_cast<bf16_t*>(p);
  p += align256(static_cast<size_t>(total) * kRanges * 16 * d.D * sizeof(bf16_t));
  float2* part_ml = reinterpret_cast<float2*>(p);

  UnionArgs ua;
  ua.sel = sel;
  ua.ulist = ulist;
  ua.bounds = bounds;
  ua.Tq = d.Tq;
  ua.pos0 = d.pos0;
  ua.pairs = pairs;
  ua.total = total;
  ua.G = d.G;
  ua.NS = d.NS;
  ua.B = d.B;
  ua.umax = umax;
  ua.words = static_cast<int>((d.NU + 31) / 32);
  const size_t lds = static_cast<size_t>(4) * 2 * ua.words * sizeof(uint32_t);
  hipLaunchKernelGGL(pair_union_kernel, dim3(static_cast<unsigned>((total + 3) / 4)), dim3(256), lds,
                     s, ua);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && mark) e = mark(4, s);
  if (e != hipSuccess) return e;

  RangeArgs a;
  a.q = static_cast<const bf16_t*>(q);
  a.kp = static_cast<const bf16_t*>(packed_k);
  a.vp = static_cast<const bf16_t*>(packed_v);
  a.ulist = ulist;
  a.bounds = bounds;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.Tq = d.Tq;
  a.Tk = d.Tk;
  a.NU = d.NU;
  a.pos0 = d.pos0;
  a.pairs = pairs;
  a.pair_groups = (pairs + kRangeWaves - 1) / kRangeWaves;
  a.G = d.G;
  a.umax = umax;
  a.scale_log2e = d.scale * 1.4426950408889634f;
  const dim3 grid(static_cast<unsigned>(d.Bt * d.G * a.pair_groups * kRanges));
  if (d.D == 128)
    hipLaunchKernelGGL(attend_range_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attend_range_kernel<64>, grid, dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e == hipSuccess && mark) e = mark(5, s);
  if (e != hipSuccess) return e;

  MergeArgs m;
  m.part_o = part_o;
  m.part_ml = part_ml;
  m.gate = static_cast<const bf16_t*>(gate);
  m.out = static_cast<bf16_t*>(out);
  m.Tq = d.Tq;
  m.pairs = pairs;
  m.total_pairs = total;
  m.G = d.G;
  m.D = d.D;
  const int64_t items = total * 16 * (d.D / 4);
  int64_t blocks = (items + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(merge_ranges_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, m);
  return hipGetLastError();
}

}  // namespace sgqa
