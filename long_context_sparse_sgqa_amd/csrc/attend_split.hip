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
//     multiple of 8, so a unit is wholly selected by a token or not at all).
//   attend_range_kernel  one wavefront per (pair, range), 16 rows = 2 tokens x 8 heads: the pair's
//     entries inside the range in chunks of 4 units, exactly as attend.hip's inner loop
//     (S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16, masked online softmax in the
//     exp2 domain), ending in an unnormalised partial (O, running max m, sum l) per row.
//   merge_ranges_kernel  per row: rescale the R partials to their common max, sum, divide, apply
//     sigmoid(gate), round to bf16.
#include "device_common.h"
#include "sgqa_internal.h"
#include "units.h"

namespace sgqa {
namespace {

constexpr int kRanges = 4;                      // unit ranges per query
constexpr int kRangeWaves = 4;                  // pairs per workgroup (one per wave)
constexpr uint32_t kUnitMask = 0x3fffffffu;

// ------------------------------------------------------------------------------------------------
// pair unions
// ------------------------------------------------------------------------------------------------
struct UnionArgs {
  const int32_t* sel;
  uint32_t* ulist;         // [Bt * G * pairs][2 * umax]
  int32_t* ucount;         // [Bt * G * pairs]
  int64_t Tq, pos0, pairs, total;
  int G, NS, B, umax;
};

__global__ void __launch_bounds__(256) pair_union_kernel(UnionArgs a) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t gp = static_cast<int64_t>(blockIdx.x) * 4 + wave;   // (b * G + g) * pairs + pair
  uint32_t* listA = lds + static_cast<size_t>(wave) * 6 * a.umax;
  uint32_t* listB = listA + a.umax;
  int32_t* uunit = reinterpret_cast<int32_t*>(listB + a.umax);
  uint32_t* umask = reinterpret_cast<uint32_t*>(uunit + 2 * a.umax);
  int na = 0, nb = 0;
  int64_t pair = 0, bg = 0;
  const bool active = gp < a.total;
  if (active) {
    pair = gp % a.pairs;
    bg = gp / a.pairs;
    const int64_t g = bg % a.G, b = bg / a.G;
    const int64_t tokA = 2 * pair;
    const int64_t pA = a.pos0 + tokA;
    na = build_units(a.sel + ((b * a.Tq + tokA) * a.G + g) * a.NS, a.NS, a.B, pA / a.B, listA, lane);
    if (tokA + 1 < a.Tq)
      nb = build_units(a.sel + ((b * a.Tq + tokA + 1) * a.G + g) * a.NS, a.NS, a.B, (pA + 1) / a.B,
                       listB, lane);
  }
  __syncthreads();
  if (active) {
    const int64_t pA = a.pos0 + 2 * pair;
    na = count_units_upto(listA, na, pA >> 3, lane);
    nb = count_units_upto(listB, nb, (pA + 1) >> 3, lane);
  }
  const int nu = merge_units(listA, na, listB, nb, uunit, umask, lane);
  __syncthreads();
  if (!active) return;
  uint32_t* out = a.ulist + gp * 2 * a.umax;
  for (int e = lane; e < nu; e += 64) {
    const uint32_t m = umask[e];
    out[e] = static_cast<uint32_t>(uunit[e]) | ((m & 0xffu) ? (1u << 30) : 0u) |
             ((m >> 8) ? (1u << 31) : 0u);
  }
  if (lane == 0) a.ucount[gp] = nu;
}

// ------------------------------------------------------------------------------------------------
// one unit range of one pair
// ------------------------------------------------------------------------------------------------
struct RangeArgs {
  const bf16_t* q;
  const bf16_t* kp;
  const bf16_t* vp;
  const uint32_t* ulist;
  const int32_t* ucount;
  float* part_o;           // [gp][R][16 rows][D]
  float2* part_ml;         // [gp][R][16 rows]  (running max in the exp2 domain, sum)
  int64_t Tq, Tk, NU, pos0, pairs, pair_groups;
  int G, umax;
  float scale_log2e;
};

// first index of the ascending list whose unit is >= unit (wave-uniform)
__device__ __forceinline__ int list_lower_bound(const uint32_t* list, int n, uint32_t unit) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((list[mid] & kUnitMask) < unit) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <int D>
__global__ void __launch_bounds__(256) attend_range_kernel(RangeArgs a) {
  constexpr int H = 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

  const uint32_t* list = a.ulist + gp * 2 * a.umax;
  const int nu = a.ucount[gp];
  // this range's share of the pair's causal unit axis [0, u_end)
  const int64_t u_end = ((a.pos0 + tokA + (validB ? 1 : 0)) >> 3) + 1;
  const uint32_t lo = static_cast<uint32_t>((r * u_end) / kRanges);
  const uint32_t hi = static_cast<uint32_t>(((r + 1) * u_end) / kRanges);
  const int e0 = list_lower_bound(list, nu, lo);
  const int e1 = list_lower_bound(list, nu, hi);

  bf16x8_t qf[D / 32];
  const bf16_t* qrow = a.q + (((b * a.Tq + (rowvalid ? tokA + X : tokA)) * a.G + g) * H + head) * D;
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc)
    qf[kc] = rowvalid ? load_bf16x8(qrow + 32 * kc + 8 * lg) : zero_bf16x8();

  const BufRsrc krs = make_rsrc(a.kp + (b * a.G + g) * a.NU * D * 8, a.NU * D * 16);
  const BufRsrc vrs = make_rsrc(a.vp + (b * a.G + g) * a.NU * D * 8, a.NU * D * 16);

  // K operands of the chunk at c: unit slot lr/4 of the chunk, rows lr%4 and lr%4 + 4
  bf16x8_t k1[D / 32], k2[D / 32];
  auto load_k = [&](int c) {
    const int e = c + (lr >> 2);
    const int u = (e < e1) ? static_cast<int>(list[e] & kUnitMask) : 0;
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) {
      k1[kc] = buffer_load_bf16x8(krs, kp_offset(u, D, kc, 0, lg, lr));
      k2[kc] = buffer_load_bf16x8(krs, kp_offset(u, D, kc, 1, lg, lr));
    }
  };

  f32x4_t acc[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;
  const float ninf = -__builtin_inff();

  if (e0 < e1) load_k(e0);
  for (int c = e0; c < e1; c += 4) {
    const int eS = c + lg;
    const uint32_t ent = (eS < e1) ? list[eS] : 0u;
    const int unitS = static_cast<int>(ent & kUnitMask);
    // V^T operand rows of this chunk: coalesced 256-byte runs, in flight during S and softmax
    bf16x8_t vf[D / 16];
    const int vo = (unitS * D + lr) * 16;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) vf[t] = buffer_load_bf16x8(vrs, vo + t * 256);

    // S^T = K Q^T: unit slot lr/4, tokens 0-3 (s1) and 4-7 (s2) of each unit
    f32x4_t s1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t s2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) {
      s1 = mfma16x16x32(k1[kc], qf[kc], s1);
      s2 = mfma16x16x32(k2[kc], qf[kc], s2);
    }
    if (c + 4 < e1) load_k(c + 4);                     // prefetch the next chunk's K operands
    const bool chose = (eS < e1) && (X ? (ent >> 31) : ((ent >> 30) & 1u));
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
    if (__ballot(m_new > m_run)) {
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
    for (int t = 0; t < D / 16; ++t) acc[t] = mfma16x16x32(vf[t], pf, acc[t]);
  }

  // partial of this range: unnormalised O, running max m and sum l per row
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const int64_t pbase = (gp * kRanges + r) * 16 + lr;
  float* po = a.part_o + pbase * D;
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    *reinterpret_cast<float4*>(po + 16 * t + 4 * lg) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
  if (lg == 0) a.part_ml[pbase] = make_float2(m_run, l_tot);
}

// ------------------------------------------------------------------------------------------------
// merge of the range partials, gate, bf16 output
// ------------------------------------------------------------------------------------------------
struct MergeArgs {
  const float* part_o;
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
      const float w = __builtin_amdgcn_exp2f(ml.x - mx);
      L += ml.y * w;
      const float4 po = *reinterpret_cast<const float4*>(a.part_o + pb * a.D + d0);
      o.x += po.x * w;
      o.y += po.y * w;
      o.z += po.z * w;
      o.w += po.w * w;
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
  return d.bf16 && d.H == 8 && (d.D == 64 || d.D == 128) && d.B % 8 == 0 &&
         d.NU * 8 * static_cast<int64_t>(d.D) * 2 < (int64_t(1) << 31) &&
         units_per_query(d) <= 1024;
}

size_t attend_split_bytes(const Dims& d) {
  const int64_t pairs = (d.Tq + 1) / 2;
  const size_t n = static_cast<size_t>(d.Bt * d.G * pairs);
  const size_t umax = static_cast<size_t>(units_per_query(d));
  return align256(n * 2 * umax * sizeof(uint32_t)) + align256(n * sizeof(int32_t)) +
         align256(n * kRanges * 16 * d.D * sizeof(float)) + align256(n * kRanges * 16 * sizeof(float2));
}

hipError_t launch_attend_split(const Dims& d, const void* q, const void* packed_k,
                               const void* gate, const int32_t* sel, void* out,
                               const void* packed_v, void* ws, hipStream_t s, StageMark mark) {
  const int64_t pairs = (d.Tq + 1) / 2;
  const int64_t total = d.Bt * d.G * pairs;
  const int umax = static_cast<int>(units_per_query(d));
  char* p = static_cast<char*>(ws);
  uint32_t* ulist = reinterpret_cast<uint32_t*>(p);
  p += align256(static_cast<size_t>(total) * 2 * umax * sizeof(uint32_t));
  int32_t* ucount = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(total) * sizeof(int32_t));
  float* part_o = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(total) * kRanges * 16 * d.D * sizeof(float));
  float2* part_ml = reinterpret_cast<float2*>(p);

  UnionArgs ua;
  ua.sel = sel;
  ua.ulist = ulist;
  ua.ucount = ucount;
  ua.Tq = d.Tq;
  ua.pos0 = d.pos0;
  ua.pairs = pairs;
  ua.total = total;
  ua.G = d.G;
  ua.NS = d.NS;
  ua.B = d.B;
  ua.umax = umax;
  const size_t lds = static_cast<size_t>(4) * 6 * umax * sizeof(uint32_t);
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
  a.ucount = ucount;
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
