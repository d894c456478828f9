// Backward of the gated attention step, key-major part: dK and dV without atomics.
//
// Training at long context is the setting of the Step 5 Preview pages (mo.ai.kr summary, section
// "모델 구조와 학습 안정성": Sparse GQA full attention, each KV group attending to its own selected
// blocks).  For a fixed selection, with P = softmax over the attended tokens and dS = P (dP - D):
//   dV_t = sum over query rows r that attend to t of P[r][t] dO[r]
//   dK_t = scale * sum over the same rows of dS[r][t] q[r]
// Accumulating these with atomics from the query side costs one fp32 atomic per (row group, key,
// d) and is bound by the L2's atomic units.  Here each wavefront owns 4 consecutive 8-token units
// (32 keys) of one KV group, keeps their K and V in registers and their dK and dV in accumulators,
// and walks the query tokens that selected any of the 4 units, 4 tokens (32 rows) per step:
//   S = Q K^T and dP = dO V^T     (32 rows x 32 keys, v_mfma_f32_32x32x16_bf16, d as the sum axis)
//   P = exp2(S scale log2e - lse2), dS = P (dP - D), masked to the (token, unit) pairs selected and
//       to keys at or before the token's position
//   dV += P^T dO and dK += dS^T Q (32 keys x d, the 32 rows as the sum axis)
// The rows of the first products are permuted so that each lane's 16 results are exactly the
// operand of the second products: lane l (l mod 32 = key n, l / 32 = h) gets rows of token slots
// h (values 0..7 = heads 0..7) and 2 + h (values 8..15), and the second products take token slot
// 2s + h's 8 heads as sum indices 8h .. 8h + 7 of step s; q and dO are therefore also read in a
// per-token transposed copy ([token][d][8 heads]) so that those 8 heads are one 16-byte load.
// Which tokens selected which unit comes from a bitmap per (sequence, group, unit) over the query
// tokens, built from the selection with atomic ORs (the result does not depend on their order);
// the tokens are walked in increasing order, so dK and dV are the same bits on every run.
#include "device_common.h"
#include "sgqa_internal.h"

namespace sgqa {
namespace {

constexpr int kH = 8;          // heads per group (the split kernels' shape)

// ------------------------------------------------------------------------------------------------
// selection -> per-unit token bitmaps
// ------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) fill_u32x4_zero_kernel(uint4* p, int64_t n4) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// One thread per selection entry: every unit of a selected block gets the query token's bit.
__global__ void __launch_bounds__(256) mark_units_kernel(const int32_t* __restrict__ sel,
                                                         uint32_t* __restrict__ bm, int64_t Tq,
                                                         int64_t NU, int64_t W, int G, int NS,
                                                         int U, int64_t total) {
  for (int64_t id = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; id < total;
       id += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int32_t blk = sel[id];
    if (blk < 0) continue;
    const int64_t row = id / NS;                 // (b, i, g)
    const int g = static_cast<int>(row % G);
    const int64_t bi = row / G;
    const int64_t i = bi % Tq, b = bi / Tq;
    const uint32_t bit = 1u << (i & 31);
    for (int u = 0; u < U; ++u) {
      const int64_t unit = static_cast<int64_t>(blk) * U + u;
      if (unit < NU) atomicOr(bm + ((b * G + g) * NU + unit) * W + (i >> 5), bit);
    }
  }
}

// ------------------------------------------------------------------------------------------------
// q and dO per token transposed: [Bt, G, Tq, D, 8 heads]
// ------------------------------------------------------------------------------------------------
// One thread per (b, i, g, 8 consecutive d): eight 16-byte loads (one per head), an 8 x 8
// transpose in registers, eight 16-byte stores (one per d).
__global__ void __launch_bounds__(256) pack_heads_t_kernel(const bf16_t* __restrict__ q,
                                                           const bf16_t* __restrict__ d_o,
                                                           bf16_t* __restrict__ qt,
                                                           bf16_t* __restrict__ dot, int64_t Tq,
                                                           int G, int D, int64_t total) {
  const int per = D / 8;
  for (int64_t id = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; id < total;
       id += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int j = static_cast<int>(id % per);
    const int64_t row = id / per;                // (b, i, g)
    const int g = static_cast<int>(row % G);
    const int64_t bi = row / G;
    const int64_t i = bi % Tq, b = bi / Tq;
    const int64_t dst = (((b * G + g) * Tq + i) * D + 8 * j) * kH;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const bf16_t* src = (which ? d_o : q) + row * kH * D + 8 * j;
      bf16_t* out = (which ? dot : qt) + dst;
      uint32_t w[kH][4];
#pragma unroll
      for (int hh = 0; hh < kH; ++hh) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + hh * D);
        w[hh][0] = v.x;
        w[hh][1] = v.y;
        w[hh][2] = v.z;
        w[hh][3] = v.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t lo = (w[2 * p][e >> 1] >> (16 * (e & 1))) & 0xffffu;
          const uint32_t hi = (w[2 * p + 1][e >> 1] >> (16 * (e & 1))) & 0xffffu;
          o[p] = lo | (hi << 16);
        }
        *reinterpret_cast<uint4*>(out + e * kH) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// dK, dV per 4-unit chunk
// ------------------------------------------------------------------------------------------------
struct DkvArgs {
  const bf16_t* q;        // [Bt, Tq, G, 8, D]
  const bf16_t* d_o;      // dout * sigmoid(gate), q's layout
  const bf16_t* qt;       // [Bt, G, Tq, D, 8]
  const bf16_t* dot;
  const float* lse2;      // [Bt, Tq, G, 8], exp2 domain
  const float* Dr;        // dO . O per row
  const bf16_t* k;        // [Bt, G, Tk, D]
  const bf16_t* v;
  const uint32_t* bm;     // [Bt, G, NU, W]
  float* dk;              // [Bt, G, Tk, D]
  float* dv;
  int64_t Tq, Tk, NU, pos0, W, nchunks, total;
  int G;
  float scale_log2e, scale;
};

template <int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) dkv_kernel(DkvArgs a) {
  const int64_t wid = blockIdx.x;
  if (wid >= a.total) return;
  const int lane = threadIdx.x;
  const int n = lane & 31, h = lane >> 5;
  const int64_t chunk = wid % a.nchunks;
  const int64_t bg = wid / a.nchunks;
  const int g = static_cast<int>(bg % a.G);
  const int64_t b = bg / a.G;
  const int64_t t = chunk * 32 + n;                      // this lane's key (kv column / dK row n)
  const int un = n >> 3;                                 // its unit inside the chunk

  // K and V of the 32 keys as the B operand of S = Q K^T and dP = dO V^T: lane (n, h) holds
  // key n, d = 16 kc + 8 h .. + 8
  bf16x8_t kb[D / 16], vb[D / 16];
  {
    const bf16_t* kr = a.k + (bg * a.Tk + (t < a.Tk ? t : 0)) * D + 8 * h;
    const bf16_t* vr = a.v + (bg * a.Tk + (t < a.Tk ? t : 0)) * D + 8 * h;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      kb[kc] = t < a.Tk ? load_bf16x8(kr + 16 * kc) : zero_bf16x8();
      vb[kc] = t < a.Tk ? load_bf16x8(vr + 16 * kc) : zero_bf16x8();
    }
  }
  f32x16_t acc_v[D / 32], acc_k[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc_v[dt][r] = 0.f;
      acc_k[dt][r] = 0.f;
    }

  // A-operand row of this lane in the first products: row m = lane % 32 is head
  // 4 ((m / 8) % 2) + m % 4 of token slot 2 (m / 16) + (m / 4) % 2
  const int m = n;
  const int a_slot = 2 * (m >> 4) + ((m >> 2) & 1);
  const int a_head = 4 * ((m >> 3) & 1) + (m & 3);

  // one step: 4 token slots (token index, 4-bit mask of the chunk's units it selected)
  auto step = [&](const int64_t* tok, const uint32_t* msk) {
    auto pick = [&](int s) -> int64_t {
      return s == 0 ? tok[0] : (s == 1 ? tok[1] : (s == 2 ? tok[2] : tok[3]));
    };
    auto pickm = [&](int s) -> uint32_t {
      return s == 0 ? msk[0] : (s == 1 ? msk[1] : (s == 2 ? msk[2] : msk[3]));
    };
    const int64_t ta = pick(a_slot);
    const int64_t arow = ((b * a.Tq + ta) * a.G + g) * kH + a_head;
    bf16x8_t qa[D / 16], oa[D / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qa[kc] = load_bf16x8(a.q + arow * D + 16 * kc + 8 * h);
      oa[kc] = load_bf16x8(a.d_o + arow * D + 16 * kc + 8 * h);
    }
    // rows of this lane's results: slot h (values 0..7) and slot 2 + h (8..15), heads 0..7
    const int64_t t_lo = pick(h), t_hi = pick(2 + h);
    const int64_t r_lo = ((b * a.Tq + t_lo) * a.G + g) * kH;
    const int64_t r_hi = ((b * a.Tq + t_hi) * a.G + g) * kH;
    float lse[16], dr[16];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float4 l0 = *reinterpret_cast<const float4*>(a.lse2 + r_lo + 4 * e);
      const float4 l1 = *reinterpret_cast<const float4*>(a.lse2 + r_hi + 4 * e);
      const float4 d0 = *reinterpret_cast<const float4*>(a.Dr + r_lo + 4 * e);
      const float4 d1 = *reinterpret_cast<const float4*>(a.Dr + r_hi + 4 * e);
      lse[4 * e] = l0.x; lse[4 * e + 1] = l0.y; lse[4 * e + 2] = l0.z; lse[4 * e + 3] = l0.w;
      lse[8 + 4 * e] = l1.x; lse[9 + 4 * e] = l1.y; lse[10 + 4 * e] = l1.z; lse[11 + 4 * e] = l1.w;
      dr[4 * e] = d0.x; dr[4 * e + 1] = d0.y; dr[4 * e + 2] = d0.z; dr[4 * e + 3] = d0.w;
      dr[8 + 4 * e] = d1.x; dr[9 + 4 * e] = d1.y; dr[10 + 4 * e] = d1.z; dr[11 + 4 * e] = d1.w;
    }
    // transposed q / dO of token slot 2 s + h at d = 32 dt + n: the second products' B operand
    bf16x8_t qtb[D / 32][2], otb[D / 32][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t ts = pick(2 * s + h);
      const int64_t base = ((bg * a.Tq + ts) * D + n) * kH;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        qtb[dt][s] = load_bf16x8(a.qt + base + 32 * dt * kH);
        otb[dt][s] = load_bf16x8(a.dot + base + 32 * dt * kH);
      }
    }
    f32x16_t sc = {}, dp = {};
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      sc = mfma32x32x16(qa[kc], kb[kc], sc);
      dp = mfma32x32x16(oa[kc], vb[kc], dp);
    }
    // masks: the token selected this lane's unit, and the key is at or before the token
    const bool on_lo = ((pickm(h) >> un) & 1u) && t <= a.pos0 + t_lo;
    const bool on_hi = ((pickm(2 + h) >> un) & 1u) && t <= a.pos0 + t_hi;
    float pv[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool on = r < 8 ? on_lo : on_hi;
      const float p = on ? __builtin_amdgcn_exp2f(fmaf(sc[r], a.scale_log2e, -lse[r])) : 0.f;
      pv[r] = p;
      ds[r] = p * (dp[r] - dr[r]);
    }
    const bf16x8_t p0 = pack8_bf16(pv), p1 = pack8_bf16(pv + 8);
    const bf16x8_t s0 = pack8_bf16(ds), s1 = pack8_bf16(ds + 8);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      acc_v[dt] = mfma32x32x16(p0, otb[dt][0], acc_v[dt]);
      acc_v[dt] = mfma32x32x16(p1, otb[dt][1], acc_v[dt]);
      acc_k[dt] = mfma32x32x16(s0, qtb[dt][0], acc_k[dt]);
      acc_k[dt] = mfma32x32x16(s1, qtb[dt][1], acc_k[dt]);
    }
  };

  // Query tokens that can select a unit of this chunk have position >= its first key.  The four
  // units' bitmap words are read with scalar loads; the tokens are taken in increasing order.
  typedef const __attribute__((address_space(4))) uint32_t* ConstU32Ptr;
  const int64_t first = chunk * 32 - a.pos0;
  const int64_t w_lo = first > 0 ? (first >> 5) : 0;
  const uint32_t* bmc = a.bm + (bg * a.NU + chunk * 4) * a.W;
  const int nunits = static_cast<int>(a.NU - chunk * 4 < 4 ? a.NU - chunk * 4 : 4);
  int64_t tok[4] = {0, 0, 0, 0};
  uint32_t msk[4] = {0u, 0u, 0u, 0u};
  int fill = 0;
  for (int64_t w = w_lo; w < a.W; ++w) {
    uint32_t wd[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      wd[u] = u < nunits ? *((ConstU32Ptr)(bmc + u * a.W + w)) : 0u;
    uint32_t any = wd[0] | wd[1] | wd[2] | wd[3];
    while (any) {
      const int bit = __builtin_ctz(any);
      any &= any - 1u;
      uint32_t mk = 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u) mk |= ((wd[u] >> bit) & 1u) << u;
      const int64_t ti = w * 32 + bit;
      tok[0] = fill == 0 ? ti : tok[0];
      tok[1] = fill == 1 ? ti : tok[1];
      tok[2] = fill == 2 ? ti : tok[2];
      tok[3] = fill == 3 ? ti : tok[3];
      msk[0] = fill == 0 ? mk : msk[0];
      msk[1] = fill == 1 ? mk : msk[1];
      msk[2] = fill == 2 ? mk : msk[2];
      msk[3] = fill == 3 ? mk : msk[3];
      if (++fill == 4) {
        step(tok, msk);
        fill = 0;
      }
    }
  }
  if (fill > 0) {
    // unused slots repeat a valid token with no unit selected: they add nothing
#pragma unroll
    for (int s = 1; s < 4; ++s) {
      if (s >= fill) {
        tok[s] = tok[0];
        msk[s] = 0u;
      }
    }
    step(tok, msk);
  }

  // dV and dK rows of this chunk: lane (n, h) holds key 8 (r / 4) + 4 h + r % 4, d = 32 dt + n
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t tr = chunk * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (tr >= a.Tk) continue;
    float* dvr = a.dv + (bg * a.Tk + tr) * D + n;
    float* dkr = a.dk + (bg * a.Tk + tr) * D + n;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      dvr[32 * dt] = acc_v[dt][r];
      dkr[32 * dt] = acc_k[dt][r] * a.scale;
    }
  }
}

unsigned grid_for(int64_t total) {
  int64_t blocks = (total + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  return static_cast<unsigned>(blocks);
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t backward_dkv_bytes(const Dims& d) {
  const int64_t W = (d.Tq + 31) / 32;
  const size_t bm = static_cast<size_t>(d.Bt * d.G * d.NU * W) * sizeof(uint32_t);
  const size_t rows = static_cast<size_t>(d.Bt * d.Tq * d.G) * kH;
  return round256(bm) + 2 * round256(rows * d.D * sizeof(bf16_t));
}

hipError_t launch_backward_dkv(const Dims& d, const void* q, const void* d_o, const float* lse2,
                               const float* Dr, const void* k, const void* v, const int32_t* sel,
                               float* dk, float* dv, void* ws, hipStream_t s) {
  const int64_t W = (d.Tq + 31) / 32;
  const size_t bm_bytes = round256(static_cast<size_t>(d.Bt * d.G * d.NU * W) * sizeof(uint32_t));
  const size_t rows = static_cast<size_t>(d.Bt * d.Tq * d.G) * kH;
  char* p = static_cast<char*>(ws);
  uint32_t* bm = reinterpret_cast<uint32_t*>(p);
  bf16_t* qt = reinterpret_cast<bf16_t*>(p + bm_bytes);
  bf16_t* dot = reinterpret_cast<bf16_t*>(p + bm_bytes + round256(rows * d.D * sizeof(bf16_t)));

  const int64_t n4 = static_cast<int64_t>(bm_bytes / 16);
  hipLaunchKernelGGL(fill_u32x4_zero_kernel, dim3(grid_for(n4)), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(bm), n4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t entries = d.Bt * d.Tq * d.G * d.NS;
  hipLaunchKernelGGL(mark_units_kernel, dim3(grid_for(entries)), dim3(256), 0, s, sel, bm, d.Tq,
                     d.NU, W, d.G, d.NS, d.B / 8, entries);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = d.Bt * d.Tq * d.G * (d.D / 8);
  hipLaunchKernelGGL(pack_heads_t_kernel, dim3(grid_for(items)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(d_o), qt, dot, d.Tq,
                     d.G, d.D, items);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  DkvArgs a;
  a.q = static_cast<const bf16_t*>(q);
  a.d_o = static_cast<const bf16_t*>(d_o);
  a.qt = qt;
  a.dot = dot;
  a.lse2 = lse2;
  a.Dr = Dr;
  a.k = static_cast<const bf16_t*>(k);
  a.v = static_cast<const bf16_t*>(v);
  a.bm = bm;
  a.dk = dk;
  a.dv = dv;
  a.Tq = d.Tq;
  a.Tk = d.Tk;
  a.NU = d.NU;
  a.pos0 = d.pos0;
  a.W = W;
  a.nchunks = (d.NU + 3) / 4;
  a.total = d.Bt * d.G * a.nchunks;
  a.G = d.G;
  a.scale_log2e = d.scale * 1.4426950408889634f;
  a.scale = d.scale;
  if (d.D == 128)
    hipLaunchKernelGGL(dkv_kernel<128>, dim3(static_cast<unsigned>(a.total)), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(dkv_kernel<64>, dim3(static_cast<unsigned>(a.total)), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace sgqa
