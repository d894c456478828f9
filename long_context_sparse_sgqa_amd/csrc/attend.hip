// Step 4 -- gated grouped-query attention over the selected tokens.
//
// The Step 5 Preview pages (mo.ai.kr summary, section "모델 구조와 학습 안정성"; ai.info article,
// section on the 3:1 layer mix) build Sparse GQA on Gated GQA and attend only over the selected
// blocks; the same passage notes that adjacent tokens' selections overlap a lot and that batching
// them raises GPU utilisation.  Readings fixed here: query head j of KV group g attends with group
// g's keys and values; the attended set of a query at position p is every token t <= p of its
// selected blocks; out = sigmoid(gate) * softmax(scale * q.k) v, elementwise in the gate.
//
// Matrix-core path (bf16, 8 heads per group, B dividing 8 or a multiple of 8):
//   * one wavefront owns two adjacent query tokens of one KV group: 2 tokens x 8 heads = 16 rows,
//     the M = 16 of v_mfma_f32_16x16x32_bf16.  The two tokens' selections are expanded into sorted
//     lists of 8-token units (with per-token bitmasks) and merged into their union in LDS, so a unit
//     both tokens chose is loaded and multiplied once (the overlap the pages exploit);
//   * the union is consumed 4 units (32 tokens) at a time: S^T = K Q^T on 2 x D/32 MFMAs, with the
//     K rows permuted so that every lane ends up holding the 8 scores of ONE unit for ONE row;
//     masking (unit not chosen by the row's token, or t > p), an online softmax in the exp2 domain,
//     then O^T += V^T P^T on D/16 MFMAs whose P operand is exactly the lane's 8 probabilities;
//   * V is read from a unit-packed copy [.., unit, d, 8 tokens] so the V^T operand is one 16-byte
//     load per lane;
//   * the epilogue divides by the row sum and multiplies by sigmoid(gate) before a bf16 store.
//   Workgroups are numbered with the token pairs fastest and the KV group next, so the GPU works
//   through one group's K/V at a time (64 MiB at 128K), which stays resident in the Infinity Cache.
// Plain path (fp32, or other head counts): one workgroup per (token, group), 32 lanes per head,
// sequential online softmax over the attended tokens in fp32.
#include "device_common.h"
#include "sgqa_internal.h"
#include "units.h"

namespace sgqa {
namespace {

constexpr int kMfmaWaves = 4;
// Unit-list capacity per token on the matrix-core path (LDS: 4 waves x 24 bytes x units <= 96 KiB).
constexpr int64_t kMaxUnits = 1024;

// ------------------------------------------------------------------------------------------------
// V packing: vp[b, g, u, d, e] = v[b, g, 8u + e, d] (zero past Tk)
// ------------------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) pack_v_kernel(const T* __restrict__ v, T* __restrict__ vp,
                                                     int64_t Tk, int64_t NU, int D, int64_t total) {
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int d = static_cast<int>(id % D);
    const int64_t u = (id / D) % NU;
    const int64_t bg = id / (static_cast<int64_t>(D) * NU);
    const T* src = v + bg * Tk * D + d;
    T vals[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t t = u * 8 + e;
      vals[e] = (t < Tk) ? src[t * D] : T(0);
    }
    T* dst = vp + ((bg * NU + u) * D + d) * 8;
    if constexpr (sizeof(T) == 2) {
      uint4 w;
      w.x = vals[0] | (static_cast<uint32_t>(vals[1]) << 16);
      w.y = vals[2] | (static_cast<uint32_t>(vals[3]) << 16);
      w.z = vals[4] | (static_cast<uint32_t>(vals[5]) << 16);
      w.w = vals[6] | (static_cast<uint32_t>(vals[7]) << 16);
      *reinterpret_cast<uint4*>(dst) = w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = vals[e];
    }
  }
}

// K packing in MFMA operand order (zero past Tk), one of two layouts:
//   pairs  (v_mfma_f32_16x16x32_bf16 kernel, kp_offset): kp[b, g, u, kc, h, lg, r, e] =
//          k[b, g, 8u + 4h + r, 32kc + 8lg + e]: the 16 lanes reading one unit's rows 4h..4h+3 of
//          d 32kc..32kc+31 read 256 contiguous bytes;
//   groups of 4 tokens (v_mfma_f32_32x32x16_bf16 kernel, kq_offset): kp[b, g, u, kc, t, hh, e] =
//          k[b, g, 8u + t, 16kc + 8hh + e]: the 16 lanes reading one unit's 8 tokens of d
//          16kc..16kc+15 read 256 contiguous bytes.
// Either way a wavefront load is 4 such runs: the coalesced pattern, unlike 16 rows x 64 bytes.
__global__ void __launch_bounds__(256) pack_k_kernel(const bf16_t* __restrict__ k, bf16_t* __restrict__ kp,
                                                     int64_t Tk, int64_t NU, int D, int64_t total,
                                                     int quad_layout) {
  // one thread per 16-byte piece: pieces per unit = D (8 rows x D bf16 / 8)
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int q = static_cast<int>(id % D);            // piece within the unit, in packed order
    const int64_t u = (id / D) % NU;
    const int64_t bg = id / (static_cast<int64_t>(D) * NU);
    int row, col;
    if (quad_layout) {
      row = (q >> 1) & 7;
      col = 16 * (q >> 4) + 8 * (q & 1);
    } else {
      row = 4 * ((q >> 4) & 1) + (q & 3);
      col = 32 * (q >> 5) + 8 * ((q >> 2) & 3);
    }
    const int64_t t = u * 8 + row;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (t < Tk) v = *reinterpret_cast<const uint4*>(k + (bg * Tk + t) * D + col);
    *reinterpret_cast<uint4*>(kp + (bg * NU + u) * D * 8 + static_cast<int64_t>(q) * 8) = v;
  }
}

// ------------------------------------------------------------------------------------------------
// Matrix-core kernel: bf16, 8 heads per KV group
// ------------------------------------------------------------------------------------------------
struct MfmaArgs {
  const bf16_t* q;
  const bf16_t* kp;
  const bf16_t* vp;
  const bf16_t* gate;
  const int32_t* sel;
  bf16_t* out;
  int64_t Tq, Tk, NU, pos0, pair_groups;   // pair_groups = ceil(ceil(Tq/2) / waves)
  int G, NS, B, umax;
  float scale_log2e;
};

template <int D>
__global__ void __launch_bounds__(256) attend_mfma_h8_kernel(MfmaArgs a) {
  extern __shared__ uint32_t lds[];
  constexpr int H = 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // group-major order: the whole GPU sweeps one (sequence, KV group) at a time, so the K/V working
  // set is one group's, which the Infinity Cache holds
  const int64_t pg = blockIdx.x % a.pair_groups;
  const int64_t bg = blockIdx.x / a.pair_groups;
  const int g = static_cast<int>(bg % a.G);
  const int64_t b = bg / a.G;
  const int64_t pair = pg * kMfmaWaves + wave;
  const int64_t tokA = 2 * pair;
  const bool validA = tokA < a.Tq;
  const bool validB = tokA + 1 < a.Tq;

  // wave-private LDS: listA[umax], listB[umax], uunit[2 umax], umask[2 umax]
  uint32_t* listA = lds + static_cast<size_t>(wave) * 6 * a.umax;
  uint32_t* listB = listA + a.umax;
  int32_t* uunit = reinterpret_cast<int32_t*>(listB + a.umax);
  uint32_t* umask = reinterpret_cast<uint32_t*>(uunit + 2 * a.umax);

  const int64_t pA = a.pos0 + tokA, pB = pA + 1;
  int na = 0, nb = 0;
  if (validA)
    na = build_units(a.sel + ((b * a.Tq + tokA) * a.G + g) * a.NS, a.NS, a.B, pA / a.B, listA, lane);
  if (validB)
    nb = build_units(a.sel + ((b * a.Tq + tokA + 1) * a.G + g) * a.NS, a.NS, a.B, pB / a.B, listB,
                     lane);
  __syncthreads();
  // drop trailing units that start past the query (only the own block of a B > 8 selection has
  // them); the lists are ascending, so the kept units are a prefix
  na = count_units_upto(listA, na, pA >> 3, lane);
  nb = count_units_upto(listB, nb, pB >> 3, lane);
  const int nu = merge_units(listA, na, listB, nb, uunit, umask, lane);
  __syncthreads();

  const int lr = lane & 15, lg = lane >> 4;
  const int X = lr >> 3;                           // which of the two tokens this lane's row is
  const int head = lr & 7;
  const int64_t tokX = tokA + X;
  const bool rowvalid = X ? validB : validA;
  const int64_t pX = a.pos0 + tokX;

  // Q^T operand: lane holds q[row lr][32 kc + 8 lg .. +8]
  bf16x8_t qf[D / 32];
  const bf16_t* qrow = a.q + (((b * a.Tq + (rowvalid ? tokX : 0)) * a.G + g) * H + head) * D;
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc)
    qf[kc] = rowvalid ? load_bf16x8(qrow + 32 * kc + 8 * lg) : zero_bf16x8();

  // buffer resources of this (sequence, group): 32-bit offsets, out-of-range reads return 0
  const BufRsrc krs = make_rsrc(a.kp + (b * a.G + g) * a.NU * D * 8, a.NU * D * 16);
  const BufRsrc vrs = make_rsrc(a.vp + (b * a.G + g) * a.NU * D * 8, a.NU * D * 16);

  f32x4_t acc[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;
  const float ninf = -__builtin_inff();

  // K rows of a chunk for this lane: unit slot lr/4, tokens (lr%4) and (lr%4)+4 of that unit
  auto k_unit = [&](int c0) -> int {
    const int e = c0 + (lr >> 2);
    return (e < nu) ? uunit[e] : 0;
  };
  bf16x8_t k1[D / 32], k2[D / 32];
  if (nu > 0) {
    const int u = k_unit(0);
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) {
      k1[kc] = buffer_load_bf16x8(krs, kp_offset(u, D, kc, 0, lg, lr));
      k2[kc] = buffer_load_bf16x8(krs, kp_offset(u, D, kc, 1, lg, lr));
    }
  }

  for (int c0 = 0; c0 < nu; c0 += 4) {
    const int eS = c0 + lg;                        // the unit whose scores this lane holds
    int unitS = 0;
    uint32_t msk = 0u;
    if (eS < nu) {
      unitS = uunit[eS];
      msk = umask[eS];
    }
    // V^T operand rows of this chunk (issued early, consumed after the softmax)
    bf16x8_t vf[D / 16];
    const int vo = (unitS * D + lr) * 16;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) vf[t] = buffer_load_bf16x8(vrs, vo + t * 256);

    f32x4_t s1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t s2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) {
      s1 = mfma16x16x32(k1[kc], qf[kc], s1);
      s2 = mfma16x16x32(k2[kc], qf[kc], s2);
    }
    if (c0 + 4 < nu) {                             // prefetch the next chunk's K rows
      const int u = k_unit(c0 + 4);
#pragma unroll
      for (int kc = 0; kc < D / 32; ++kc) {
        k1[kc] = buffer_load_bf16x8(krs, kp_offset(u, D, kc, 0, lg, lr));
        k2[kc] = buffer_load_bf16x8(krs, kp_offset(u, D, kc, 1, lg, lr));
      }
    }

    // valid tokens of the lane's unit for its row: chosen by the row's token and t <= p
    const uint32_t bits = X ? ((msk >> 8) & 0xffu) : (msk & 0xffu);
    const int64_t dlt = pX - static_cast<int64_t>(unitS) * 8;
    const uint32_t causal = dlt >= 7 ? 0xffu : (dlt < 0 ? 0u : ((2u << dlt) - 1u));
    const uint32_t valid = bits & causal;
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
    for (int t = 0; t < D / 16; ++t) acc[t] = mfma16x16x32(vf[t], pf, acc[t]);
  }

  // epilogue: row sum over the 4 lane groups, normalise, gate, store
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (!rowvalid || nu == 0) return;
  const float inv = 1.f / l_tot;
  const int64_t obase = (((b * a.Tq + tokX) * a.G + g) * H + head) * D;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const int d0 = 16 * t + 4 * lg;
    const uint2 gw = *reinterpret_cast<const uint2*>(a.gate + obase + d0);
    const float g0 = bf16_to_f32(static_cast<bf16_t>(gw.x & 0xffffu));
    const float g1 = bf16_to_f32(static_cast<bf16_t>(gw.x >> 16));
    const float g2 = bf16_to_f32(static_cast<bf16_t>(gw.y & 0xffffu));
    const float g3 = bf16_to_f32(static_cast<bf16_t>(gw.y >> 16));
    const float o0 = acc[t][0] * inv / (1.f + __expf(-g0));
    const float o1 = acc[t][1] * inv / (1.f + __expf(-g1));
    const float o2 = acc[t][2] * inv / (1.f + __expf(-g2));
    const float o3 = acc[t][3] * inv / (1.f + __expf(-g3));
    uint2 ow;
    ow.x = pack_bf16x2(o0, o1);
    ow.y = pack_bf16x2(o2, o3);
    *reinterpret_cast<uint2*>(a.out + obase + d0) = ow;
  }
}

// ------------------------------------------------------------------------------------------------
// Plain kernel: any dtype, any head count <= 32.  One workgroup per (b, i, g); 32 lanes per head.
// ------------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(1024) attend_plain_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ gate, const int32_t* __restrict__ sel, T* __restrict__ out, int64_t Tq,
    int64_t Tk, int G, int H, int NS, int B, int64_t pos0, float scale) {
  constexpr int PER = D / 32;
  const int g = static_cast<int>(blockIdx.x % G);
  const int64_t bi = blockIdx.x / G;              // b * Tq + i
  const int64_t i = bi % Tq;
  const int64_t b = bi / Tq;
  const int h = threadIdx.x >> 5;
  const int l32 = threadIdx.x & 31;
  const int64_t p = pos0 + i;
  const int64_t o = p / B;
  const int64_t row = ((bi * G + g) * H + h) * D;
  float qv[PER], acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    qv[j] = Elem<T>::load(q + row + l32 + 32 * j);
    acc[j] = 0.f;
  }
  const T* kg = k + (b * G + g) * Tk * D;
  const T* vg = v + (b * G + g) * Tk * D;
  const int32_t* selrow = sel + (bi * G + g) * NS;
  float m = -__builtin_inff(), l = 0.f;
  for (int e = 0; e < NS; ++e) {
    const int64_t blk = selrow[e];
    if (blk < 0 || blk > o) continue;
    int64_t t_end = blk * B + B;
    if (t_end > p + 1) t_end = p + 1;
    for (int64_t t = blk * B; t < t_end; ++t) {
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < PER; ++j) dot = fmaf(qv[j], Elem<T>::load(kg + t * D + l32 + 32 * j), dot);
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 32);
      const float s = dot * scale;
      const float m_new = fmaxf(m, s);
      const float alpha = expf(m - m_new);
      const float pw = expf(s - m_new);
      l = l * alpha + pw;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        acc[j] = fmaf(pw, Elem<T>::load(vg + t * D + l32 + 32 * j), acc[j] * alpha);
      m = m_new;
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const float gt = Elem<T>::load(gate + row + l32 + 32 * j);
    Elem<T>::store(out + row + l32 + 32 * j, acc[j] / l / (1.f + expf(-gt)));
  }
}

}  // namespace

bool attend_uses_mfma(const Dims& d) {
  const bool block_ok = (d.B % 8 == 0) || (8 % d.B == 0);
  // 32-bit buffer offsets: one (sequence, group) of packed V must stay below 2 GiB
  const bool offsets_ok = d.NU * 8 * static_cast<int64_t>(d.D) * 2 < (int64_t(1) << 31);
  return d.bf16 && d.H == 8 && block_ok && offsets_ok && units_per_query(d) <= kMaxUnits;
}

int64_t units_per_query(const Dims& d) {
  // a query's selection covers at most NS blocks of ceil(B/8) units, and at most the units of
  // blocks 0..o, i.e. NU rounded up to whole blocks
  const int64_t per_blk = d.B >= 8 ? d.B / 8 : 1;
  const int64_t u = static_cast<int64_t>(d.NS) * per_blk;
  const int64_t cap = d.NU + per_blk;
  return u < cap ? u : cap;
}

// Packed K then packed V, each [Bt, G, NU, 8 x D] bf16, on the matrix-core paths.
size_t attend_packed_kv_bytes(const Dims& d) {
  if (!attend_uses_mfma(d) && !attend_split_supported(d)) return 0;
  const size_t one = static_cast<size_t>(d.Bt) * d.G * d.NU * 8 * d.D * 2;
  return 2 * ((one + 255) / 256 * 256);
}

size_t attend_workspace_bytes(const Dims& d) {
  const size_t pkv = attend_packed_kv_bytes(d);
  return pkv + (attend_split_supported(d) ? attend_split_bytes(d) : 0);
}

hipError_t launch_pack_kv(const Dims& d, const void* k, const void* v, void* packed, hipStream_t s) {
  if (attend_packed_kv_bytes(d) == 0) return hipSuccess;
  const int64_t total = d.Bt * d.G * d.NU * d.D;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  bf16_t* kp = static_cast<bf16_t*>(packed);
  bf16_t* vp = kp + attend_packed_kv_bytes(d) / 2 / sizeof(bf16_t);
  hipLaunchKernelGGL(pack_k_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(k), kp, d.Tk, d.NU, d.D, total,
                     attend_split_supported(d) ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_v_kernel<bf16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(v), vp, d.Tk, d.NU, d.D, total);
  return hipGetLastError();
}

hipError_t launch_attend_single(const Dims& d, const void* q, const void* k, const void* v,
                                const void* gate, const int32_t* sel, void* out, const bf16_t* kp,
                                const bf16_t* vp, hipStream_t s);

// fp8 e4m3 packing for the range kernel (zero past Tk).  K: unit byte ((m*8 + t)*2 + h)*16 + kk*8
// + e holds k[8u + t][32m + 16kk + 8h + e], so one 16-byte load gives a lane its operands of two
// consecutive 16-wide d-slices.  V: unit byte (n*32 + c)*16 + kk*8 + t holds v[8u + t][64n +
// 32kk + c], so one 16-byte load gives a lane its 8 tokens for two consecutive 32-wide d-tiles.
// One thread per 16-byte piece (D/2 pieces per unit).
__global__ void __launch_bounds__(256) pack_k_fp8_kernel(const uint8_t* __restrict__ k8,
                                                         uint8_t* __restrict__ kp, int64_t Tk,
                                                         int64_t NU, int D, int64_t total) {
  const int per = D / 2;
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int q = static_cast<int>(id % per);
    const int64_t u = (id / per) % NU;
    const int64_t bg = id / (static_cast<int64_t>(per) * NU);
    const int h = q & 1, t = (q >> 1) & 7, m = q >> 4;
    const int64_t tok = u * 8 + t;
    uint2 lo = make_uint2(0u, 0u), hi = make_uint2(0u, 0u);
    if (tok < Tk) {
      const uint8_t* row = k8 + (bg * Tk + tok) * D + 32 * m + 8 * h;
      lo = *reinterpret_cast<const uint2*>(row);
      hi = *reinterpret_cast<const uint2*>(row + 16);
    }
    *reinterpret_cast<uint4*>(kp + (bg * NU + u) * D * 8 + static_cast<int64_t>(q) * 16) =
        make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

__global__ void __launch_bounds__(256) pack_v_fp8_kernel(const uint8_t* __restrict__ v8,
                                                         uint8_t* __restrict__ vp, int64_t Tk,
                                                         int64_t NU, int D, int64_t total) {
  const int per = D / 2;
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int q = static_cast<int>(id % per);
    const int64_t u = (id / per) % NU;
    const int64_t bg = id / (static_cast<int64_t>(per) * NU);
    const int c = q & 31, n = q >> 5;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int64_t tok = u * 8 + t;
        const uint32_t byte = tok < Tk ? v8[(bg * Tk + tok) * D + 64 * n + 32 * kk + c] : 0u;
        w[(kk * 8 + t) >> 2] |= byte << (8 * (t & 3));
      }
    *reinterpret_cast<uint4*>(vp + (bg * NU + u) * D * 8 + static_cast<int64_t>(q) * 16) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

size_t packed_kv_fp8_bytes(const Dims& d) {
  const size_t one = static_cast<size_t>(d.Bt) * d.G * d.NU * 8 * d.D;
  return 2 * ((one + 255) / 256 * 256);
}

hipError_t launch_pack_kv_fp8(const Dims& d, const void* k8, const void* v8, void* packed,
                              hipStream_t s) {
  const int64_t total = d.Bt * d.G * d.NU * (d.D / 2);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  uint8_t* kp = static_cast<uint8_t*>(packed);
  uint8_t* vp = kp + packed_kv_fp8_bytes(d) / 2;
  hipLaunchKernelGGL(pack_k_fp8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(k8), kp, d.Tk, d.NU, d.D, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_v_fp8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(v8), vp, d.Tk, d.NU, d.D, total);
  return hipGetLastError();
}

size_t packed_kv_quad_bytes(const Dims& d) {
  const size_t one = static_cast<size_t>(d.Bt) * d.G * d.NU * 8 * d.D * 2;
  return 2 * ((one + 255) / 256 * 256);
}

hipError_t launch_pack_kv_quad(const Dims& d, const void* k, const void* v, void* packed,
                               hipStream_t s) {
  const int64_t total = d.Bt * d.G * d.NU * d.D;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  bf16_t* kp = static_cast<bf16_t*>(packed);
  bf16_t* vp = kp + packed_kv_quad_bytes(d) / 2 / sizeof(bf16_t);
  hipLaunchKernelGGL(pack_k_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(k), kp, d.Tk, d.NU, d.D, total, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_v_kernel<bf16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(v), vp, d.Tk, d.NU, d.D, total);
  return hipGetLastError();
}

hipError_t launch_attend_packed(const Dims& d, const void* q, const void* k, const void* v,
                                const void* gate, const int32_t* sel, void* out, void* workspace,
                                hipStream_t s, StageMark mark, float* lse) {
  const bf16_t* kp = static_cast<const bf16_t*>(workspace);
  const bf16_t* vp = kp + attend_packed_kv_bytes(d) / 2 / sizeof(bf16_t);
  if (attend_split_supported(d)) {
    char* rest = static_cast<char*>(workspace) + attend_packed_kv_bytes(d);
    return launch_attend_split(d, q, kp, gate, sel, out, vp, rest, s, mark, nullptr, nullptr, lse);
  }
  if (lse) return hipErrorInvalidValue;
  if (mark) {
    const hipError_t e = mark(4, s);
    if (e != hipSuccess) return e;
  }
  const hipError_t e = launch_attend_single(d, q, k, v, gate, sel, out, kp, vp, s);
  if (e != hipSuccess || !mark) return e;
  return mark(5, s);
}

// One attention kernel for the whole problem: matrix-core pair kernel or the plain kernel.
hipError_t launch_attend_single(const Dims& d, const void* q, const void* k, const void* v,
                                const void* gate, const int32_t* sel, void* out, const bf16_t* kp,
                                const bf16_t* vp, hipStream_t s) {
  if (attend_uses_mfma(d)) {
    MfmaArgs a;
    a.q = static_cast<const bf16_t*>(q);
    a.kp = kp;
    a.vp = vp;
    a.gate = static_cast<const bf16_t*>(gate);
    a.sel = sel;
    a.out = static_cast<bf16_t*>(out);
    a.Tq = d.Tq;
    a.Tk = d.Tk;
    a.NU = d.NU;
    a.pos0 = d.pos0;
    const int64_t pairs = (d.Tq + 1) / 2;
    a.pair_groups = (pairs + kMfmaWaves - 1) / kMfmaWaves;
    a.G = d.G;
    a.NS = d.NS;
    a.B = d.B;
    a.umax = static_cast<int>(units_per_query(d));
    a.scale_log2e = d.scale * 1.4426950408889634f;
    const size_t lds = static_cast<size_t>(kMfmaWaves) * 6 * a.umax * sizeof(uint32_t);
    const int64_t grid = d.Bt * a.pair_groups * d.G;
    if (d.D == 128)
      hipLaunchKernelGGL(attend_mfma_h8_kernel<128>, dim3(static_cast<unsigned>(grid)), dim3(256),
                         lds, s, a);
    else
      hipLaunchKernelGGL(attend_mfma_h8_kernel<64>, dim3(static_cast<unsigned>(grid)), dim3(256),
                         lds, s, a);
    return hipGetLastError();
  }
  const int64_t grid = d.Bt * d.Tq * d.G;
  const dim3 block(32 * d.H);
  if (d.bf16) {
    auto* qq = static_cast<const bf16_t*>(q);
    auto* kk = static_cast<const bf16_t*>(k);
    auto* vv = static_cast<const bf16_t*>(v);
    auto* gg = static_cast<const bf16_t*>(gate);
    auto* oo = static_cast<bf16_t*>(out);
    if (d.D == 128)
      hipLaunchKernelGGL((attend_plain_kernel<bf16_t, 128>), dim3(static_cast<unsigned>(grid)), block,
                         0, s, qq, kk, vv, gg, sel, oo, d.Tq, d.Tk, d.G, d.H, d.NS, d.B, d.pos0,
                         d.scale);
    else
      hipLaunchKernelGGL((attend_plain_kernel<bf16_t, 64>), dim3(static_cast<unsigned>(grid)), block,
                         0, s, qq, kk, vv, gg, sel, oo, d.Tq, d.Tk, d.G, d.H, d.NS, d.B, d.pos0,
                         d.scale);
  } else {
    auto* qq = static_cast<const float*>(q);
    auto* kk = static_cast<const float*>(k);
    auto* vv = static_cast<const float*>(v);
    auto* gg = static_cast<const float*>(gate);
    auto* oo = static_cast<float*>(out);
    if (d.D == 128)
      hipLaunchKernelGGL((attend_plain_kernel<float, 128>), dim3(static_cast<unsigned>(grid)), block,
                         0, s, qq, kk, vv, gg, sel, oo, d.Tq, d.Tk, d.G, d.H, d.NS, d.B, d.pos0,
                         d.scale);
    else
      hipLaunchKernelGGL((attend_plain_kernel<float, 64>), dim3(static_cast<unsigned>(grid)), block,
                         0, s, qq, kk, vv, gg, sel, oo, d.Tq, d.Tk, d.G, d.H, d.NS, d.B, d.pos0,
                         d.scale);
  }
  return hipGetLastError();
}

hipError_t launch_attend(const Dims& d, const void* q, const void* k, const void* v,
                         const void* gate, const int32_t* sel, void* out, void* workspace,
                         hipStream_t s) {
  hipError_t e = launch_pack_kv(d, k, v, workspace, s);
  if (e != hipSuccess) return e;
  return launch_attend_packed(d, q, k, v, gate, sel, out, workspace, s);
}

}  // namespace sgqa
