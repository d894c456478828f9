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
// 2s + h's 8 heads as sum indices 8h .. 8h + 7 of step s.  A step's q and dO rows are read from
// memory once, row-major, into LDS: the first products read them row by row, the second read 4
// heads at one d per lane through gfx950's transposing LDS read.  The next step's rows are loaded
// into registers while the current step is computed, then written to the other LDS buffer.
// Which tokens selected which unit comes from bitmaps over the query tokens, word-major (for each
// 32-token word, one word per unit), built per word in LDS from the 32 tokens' selections (OR
// does not depend on the order) and written out whole; the tokens are walked in increasing
// order, so dK and dV are the same bits on every run.
#include "device_common.h"
#include "sgqa_internal.h"

namespace sgqa {
namespace {

constexpr int kH = 8;          // heads per group (the split kernels' shape)

// ------------------------------------------------------------------------------------------------
// selection -> token bitmaps per unit, word-major: bm[b, g, w, u] has bit i set when query token
// 32 w + i selected a block holding unit u (rows of NU4 = NU rounded up to 4 words)
// ------------------------------------------------------------------------------------------------
constexpr int kMarkTile = 16384;        // units per workgroup: a 64 KiB LDS row of words

// One workgroup per (sequence, group, word w, tile of units): the 32 tokens' selections set bits
// in an LDS copy of the row with LDS atomic ORs (the result does not depend on their order), and
// the row is written out whole, coalesced: no global atomics and no separate zero fill.
__global__ void __launch_bounds__(256) mark_units_kernel(const int32_t* __restrict__ sel,
                                                         uint32_t* __restrict__ bm, int64_t Tq,
                                                         int64_t NU, int64_t NU4, int64_t W, int G,
                                                         int NS, int U, int tiles) {
  __shared__ uint32_t row[kMarkTile];
  const int64_t id = blockIdx.x;
  const int tile = static_cast<int>(id % tiles);
  const int64_t bgw = id / tiles;
  const int64_t w = bgw % W, bg = bgw / W;
  const int g = static_cast<int>(bg % G);
  const int64_t b = bg / G;
  const int64_t u0 = static_cast<int64_t>(tile) * kMarkTile;
  const int n = static_cast<int>(NU4 - u0 < kMarkTile ? NU4 - u0 : kMarkTile);
  for (int x = threadIdx.x; x < n; x += 256) row[x] = 0u;
  __syncthreads();
  // 32 tokens x NS entries; consecutive threads take consecutive entries of one token.  Each
  // thread loads kBatch entries before it marks any, so their loads are in flight together.
  constexpr int kBatch = 8;
  const int n_e = 32 * NS;
  const int32_t* sw = sel + ((b * Tq + 32 * w) * G + g) * NS;   // token 32 w, entry 0
  for (int e0 = 0; e0 < n_e; e0 += 256 * kBatch) {
    int32_t blk[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int e = e0 + 256 * k + threadIdx.x;
      const int i = e / NS;
      const bool ok = e < n_e && 32 * w + i < Tq;
      blk[k] = ok ? sw[static_cast<int64_t>(i) * G * NS + (e - i * NS)] : -1;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (blk[k] < 0) continue;
      const int i = (e0 + 256 * k + threadIdx.x) / NS;
      for (int uu = 0; uu < U; ++uu) {
        const int64_t unit = static_cast<int64_t>(blk[k]) * U + uu - u0;
        if (unit >= 0 && unit < n && unit + u0 < NU) atomicOr(&row[unit], 1u << i);
      }
    }
  }
  __syncthreads();
  uint32_t* dst = bm + (bg * W + w) * NU4 + u0;
  for (int x = threadIdx.x; x < n; x += 256) dst[x] = row[x];
}

// ------------------------------------------------------------------------------------------------
// dK, dV per 4-unit chunk
// ------------------------------------------------------------------------------------------------
struct DkvArgs {
  const bf16_t* q;        // [Bt, Tq, G, 8, D]
  const bf16_t* d_o;      // dout * sigmoid(gate), q's layout
  const float* lse2;      // [Bt, Tq, G, 8], exp2 domain
  const float* Dr;        // dO . O per row
  const bf16_t* k;        // [Bt, G, Tk, D]
  const bf16_t* v;
  const uint32_t* bm;     // [Bt, G, W, NU4] (word-major)
  float* dk;              // [Bt, G, Tk, D]
  float* dv;
  int64_t Tq, Tk, NU, NU4, pos0, W, total;
  int64_t BG;             // Bt * G: wave w takes chunk w / BG of (sequence, group) w % BG
  int G;
  float scale_log2e, scale;
};

// A step's q and dO rows in LDS: 32 rows (4 token slots x 8 heads) of D bf16 each, padded by 16
// bytes (the row-major operand reads of 32 rows then fall in distinct banks), and the rows' lse2
// and Dr; two steps in turn.
template <int D> struct DkvLds {
  static constexpr int kRowBytes = D * 2 + 16;
  static constexpr int kTensorBytes = 32 * kRowBytes;
  static constexpr int kStepBytes = 2 * kTensorBytes + 256;  // q, dO, then 32 lse2 and 32 Dr
  static constexpr int kBytes = 2 * kStepBytes;
  static constexpr int kPieces = D / 64;                    // 16-byte pieces per lane per token row set
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t* LdsS16x4;

// Transposing LDS read (16-bit elements): within each 16-lane group, lane i receives the i & 3-th
// element of the 8 bytes read by group lane 4 j + (i >> 2), j = 0..3.  With group lane a reading
// row base + (a >> 2), columns c + 4 (a & 3) .. + 3 of a row-major matrix, lane i gets rows
// base .. base + 3 of column c + i.
__device__ __forceinline__ s16x4_t lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS16x4)(p));
}

template <int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) dkv_kernel(DkvArgs a) {
  typedef DkvLds<D> L;
  __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBytes];
  const int64_t wid = blockIdx.x;
  if (wid >= a.total) return;
  const int lane = threadIdx.x;
  const int n = lane & 31, h = lane >> 5;
  const int gi = lane & 15, gh = (lane >> 4) & 1;        // lane in its 16-lane group, group's half
  // (sequence, group) fastest: with 8 of them, the XCD that runs a wave (workgroup index mod 8)
  // always serves the same group, and its L2 holds only that group's q and dO rows
  const int64_t chunk = wid / a.BG;
  const int64_t bg = wid - chunk * a.BG;
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
  const int a_row = 8 * (2 * (m >> 4) + ((m >> 2) & 1)) + 4 * ((m >> 3) & 1) + (m & 3);

  // A step's rows go global -> registers -> LDS.  A token's 8 head rows are contiguous (16 D
  // bytes): lane l moves its 16-byte pieces w = 64 p + l of each token slot's rows of q and dO.
  u32x4_t stg_q[4][L::kPieces], stg_o[4][L::kPieces];   // vector types: kept in registers
  float stg_r;                                         // lane l: lse2 (l < 32) or Dr of row l % 32
  auto stage_load = [&](const int32_t* tok) __attribute__((always_inline)) {
    {
      const int row = lane & 31, sl = row >> 3;
      const int32_t tk = sl == 0 ? tok[0] : (sl == 1 ? tok[1] : (sl == 2 ? tok[2] : tok[3]));
      const int64_t r = ((b * a.Tq + tk) * a.G + g) * kH + (row & 7);
      stg_r = lane < 32 ? a.lse2[r] : a.Dr[r];
    }
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int64_t row0 = ((b * a.Tq + tok[sl]) * a.G + g) * kH;
#pragma unroll
      for (int pc = 0; pc < L::kPieces; ++pc) {
        const int w = 64 * pc + lane;
        stg_q[sl][pc] = *reinterpret_cast<const u32x4_t*>(a.q + row0 * D + 8 * w);
        stg_o[sl][pc] = *reinterpret_cast<const u32x4_t*>(a.d_o + row0 * D + 8 * w);
      }
    }
  };
  auto stage_write = [&](int buf) __attribute__((always_inline)) {
    unsigned char* base = lds + buf * L::kStepBytes;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
#pragma unroll
      for (int pc = 0; pc < L::kPieces; ++pc) {
        const int w = 64 * pc + lane;
        const int head = w / (D / 8), piece = w % (D / 8);
        const int off = (8 * sl + head) * L::kRowBytes + 16 * piece;
        *reinterpret_cast<u32x4_t*>(base + off) = stg_q[sl][pc];
        *reinterpret_cast<u32x4_t*>(base + L::kTensorBytes + off) = stg_o[sl][pc];
      }
    }
    reinterpret_cast<float*>(base + 2 * L::kTensorBytes)[lane] = stg_r;
  };
  // one step from LDS buffer `buf`: 4 token slots (token index, 4-bit mask of the chunk's units)
  auto compute = [&](int buf, const int32_t* tok, const uint32_t* msk) __attribute__((always_inline)) {
    const unsigned char* lq = lds + buf * L::kStepBytes;
    const unsigned char* lo = lq + L::kTensorBytes;
    // lse2 and Dr of this lane's result rows: slot h (values 0..7) and slot 2 + h (values 8..15)
    const float* lr = reinterpret_cast<const float*>(lq + 2 * L::kTensorBytes);
    float lse[16], dr[16];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float4 l0 = reinterpret_cast<const float4*>(lr + 8 * h)[e];
      const float4 l1 = reinterpret_cast<const float4*>(lr + 16 + 8 * h)[e];
      const float4 d0 = reinterpret_cast<const float4*>(lr + 32 + 8 * h)[e];
      const float4 d1 = reinterpret_cast<const float4*>(lr + 48 + 8 * h)[e];
      lse[4 * e] = l0.x; lse[4 * e + 1] = l0.y; lse[4 * e + 2] = l0.z; lse[4 * e + 3] = l0.w;
      lse[8 + 4 * e] = l1.x; lse[9 + 4 * e] = l1.y; lse[10 + 4 * e] = l1.z; lse[11 + 4 * e] = l1.w;
      dr[4 * e] = d0.x; dr[4 * e + 1] = d0.y; dr[4 * e + 2] = d0.z; dr[4 * e + 3] = d0.w;
      dr[8 + 4 * e] = d1.x; dr[9 + 4 * e] = d1.y; dr[10 + 4 * e] = d1.z; dr[11 + 4 * e] = d1.w;
    }
    f32x16_t sc = {}, dp = {};
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const int off = a_row * L::kRowBytes + 2 * (16 * kc + 8 * h);
      const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(lq + off);
      const bf16x8_t oa = *reinterpret_cast<const bf16x8_t*>(lo + off);
      sc = mfma32x32x16(qa, kb[kc], sc);
      dp = mfma32x32x16(oa, vb[kc], dp);
    }
    // masks: the token selected this lane's unit, and the key is at or before the token
    const int64_t t_lo = h ? tok[1] : tok[0], t_hi = h ? tok[3] : tok[2];
    const uint32_t m_lo = h ? msk[1] : msk[0], m_hi = h ? msk[3] : msk[2];
    const bool on_lo = ((m_lo >> un) & 1u) && t <= a.pos0 + t_lo;
    const bool on_hi = ((m_hi >> un) & 1u) && t <= a.pos0 + t_hi;
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
    // second products' B operand: token slot 2 s + h's 8 heads (rows) at d = 32 dt + n, read
    // transposed from the row-major rows (two reads of 4 heads each)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const int row = 8 * (2 * sp + h) + (gi >> 2);
        const int off = row * L::kRowBytes + 2 * (32 * dt + 16 * gh + 4 * (gi & 3));
        const s16x4_t q0 = lds_read_tr16(lq + off), q1 = lds_read_tr16(lq + off + 4 * L::kRowBytes);
        const s16x4_t o0 = lds_read_tr16(lo + off), o1 = lds_read_tr16(lo + off + 4 * L::kRowBytes);
        const bf16x8_t qb = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8_t ob = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(o0, o1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc_v[dt] = mfma32x32x16(sp ? p1 : p0, ob, acc_v[dt]);
        acc_k[dt] = mfma32x32x16(sp ? s1 : s0, qb, acc_k[dt]);
      }
    }
  };

  // Query tokens that can select a unit of this chunk have position >= its first key.  The four
  // units' words of each token word are one 16-byte scalar load (units past NU read 0); the
  // tokens are taken in increasing order, four per step (unused slots repeat slot 0's token with
  // no unit selected: they add nothing).
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) u32x4v* ConstU32x4Ptr;
  const int64_t first = chunk * 32 - a.pos0;
  const uint32_t* bmc = a.bm + bg * a.W * a.NU4 + chunk * 4;
  int64_t w_next = first > 0 ? (first >> 5) : 0;      // next bitmap word to read
  int64_t w_cur = 0;                                   // word the bits in `any` belong to
  uint32_t wd[4] = {0u, 0u, 0u, 0u};
  uint32_t any = 0u;
  // the next 4 token words' unit words, loaded together (four independent scalar loads) so that
  // the scan waits for memory once per 4 words rather than once per word
  u32x4v look[4];
  int look_i = 4;
  auto refill = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      look[k] = w_next + k < a.W ? *((ConstU32x4Ptr)(bmc + (w_next + k) * a.NU4)) : u32x4v{0u, 0u, 0u, 0u};
    look_i = 0;
  };
  auto next_step = [&](int32_t* tok, uint32_t* msk) __attribute__((always_inline)) -> int {
    int fill = 0;
    while (fill < 4) {
      while (any == 0u && w_next < a.W) {
        if (look_i == 4) refill();
        const u32x4v q4 = look_i == 0 ? look[0] : (look_i == 1 ? look[1] : (look_i == 2 ? look[2] : look[3]));
        ++look_i;
        wd[0] = q4[0];
        wd[1] = q4[1];
        wd[2] = q4[2];
        wd[3] = q4[3];
        any = wd[0] | wd[1] | wd[2] | wd[3];
        w_cur = w_next++;
      }
      if (any == 0u) break;
      const int bit = __builtin_ctz(any);
      any &= any - 1u;
      uint32_t mk = 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u) mk |= ((wd[u] >> bit) & 1u) << u;
      const int32_t ti = static_cast<int32_t>(w_cur * 32 + bit);
      tok[0] = fill == 0 ? ti : tok[0];
      tok[1] = fill == 1 ? ti : tok[1];
      tok[2] = fill == 2 ? ti : tok[2];
      tok[3] = fill == 3 ? ti : tok[3];
      msk[0] = fill == 0 ? mk : msk[0];
      msk[1] = fill == 1 ? mk : msk[1];
      msk[2] = fill == 2 ? mk : msk[2];
      msk[3] = fill == 3 ? mk : msk[3];
      ++fill;
    }
#pragma unroll
    for (int s = 1; s < 4; ++s) {
      if (s >= fill) {
        tok[s] = tok[0];
        msk[s] = 0u;
      }
    }
    return fill;
  };

  // Software pipeline: step i+1's rows are loaded into registers while step i is computed from
  // LDS, then written to the other LDS buffer.
  int32_t tok_a[4] = {0, 0, 0, 0}, tok_b[4] = {0, 0, 0, 0};
  uint32_t msk_a[4] = {0u, 0u, 0u, 0u}, msk_b[4] = {0u, 0u, 0u, 0u};
  if (next_step(tok_a, msk_a) > 0) {
    stage_load(tok_a);
    stage_write(0);
    int have_b = next_step(tok_b, msk_b);
    int buf = 0;
    while (true) {
      if (have_b > 0) stage_load(tok_b);
      compute(buf, tok_a, msk_a);
      if (have_b == 0) break;
      stage_write(buf ^ 1);
      buf ^= 1;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        tok_a[s] = tok_b[s];
        msk_a[s] = msk_b[s];
      }
      have_b = next_step(tok_b, msk_b);
    }
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

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t backward_dkv_bytes(const Dims& d) {
  const int64_t W = (d.Tq + 31) / 32, NU4 = (d.NU + 3) / 4 * 4;
  const size_t bm = static_cast<size_t>(d.Bt * d.G * W * NU4) * sizeof(uint32_t);
  return round256(bm);
}

hipError_t launch_backward_dkv(const Dims& d, const void* q, const void* d_o, const float* lse2,
                               const float* Dr, const void* k, const void* v, const int32_t* sel,
                               float* dk, float* dv, void* ws, hipStream_t s) {
  const int64_t W = (d.Tq + 31) / 32, NU4 = (d.NU + 3) / 4 * 4;
  uint32_t* bm = static_cast<uint32_t*>(ws);
  const int tiles = static_cast<int>((NU4 + kMarkTile - 1) / kMarkTile);
  const int64_t wgs = d.Bt * d.G * W * tiles;
  if (wgs >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mark_units_kernel, dim3(static_cast<unsigned>(wgs)), dim3(256), 0, s, sel, bm,
                     d.Tq, d.NU, NU4, W, d.G, d.NS, d.B / 8, tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DkvArgs a;
  a.q = static_cast<const bf16_t*>(q);
  a.d_o = static_cast<const bf16_t*>(d_o);
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
  a.NU4 = NU4;
  a.pos0 = d.pos0;
  a.W = W;
  a.BG = d.Bt * d.G;
  a.total = a.BG * ((d.NU + 3) / 4);
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
