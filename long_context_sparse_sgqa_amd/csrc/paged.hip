// Decode over a paged cache: appending new tokens and keeping the block keys current.
//
// The Step 5 Preview summary on mo.ai.kr runs Sparse GQA at contexts up to 1M tokens (section
// "모델 구조와 학습 안정성") and serves the model with MTP-3 heads and a KV cache (section
// "장기 강화학습과 실행 비용"), so new tokens arrive a few at a time.
// The forward path's steps are unchanged; what decode adds is state: each sequence's K, V and
// index keys live in a cache, and the block keys of step 1 are kept per sequence, so a new token
// only recomputes the blocks it falls into (a block key is still the sum of the index keys
// present in the block, accumulated in fp32 in token order and rounded once).
//
// Cache layout (pages of P tokens, P a power of two and a multiple of 8 and of B; page j of
// sequence b is block_table[b * max_pages + j]):
//   K pool     [num_pages][G][P / 8][8 D]  each 8-token unit in the 4-token operand order of the
//                                          attention kernel: k(t, d) at ((d/16) 8 + t) 16 + d % 16
//   V pool     [num_pages][G][P / 8][D][8] each unit transposed: v(t, d) at d 8 + t
//   k_idx pool [num_pages][P][Di]          natural order
//   k_blk      [Bt][max_pages P / B][Di]   block keys per sequence
// Tokens of a sequence's last unit past its length are kept at zero, so the attention kernel,
// which masks them, never multiplies stale data.
#include "device_common.h"
#include "sgqa_internal.h"

namespace sgqa {
namespace {

struct AppendArgs {
  const bf16_t* k_new;        // [Bt][G][n_new][D]
  const bf16_t* v_new;
  const bf16_t* kidx_new;     // [Bt][n_new][Di]
  bf16_t* k_pool;
  bf16_t* v_pool;
  bf16_t* kidx_pool;
  bf16_t* k_blk;
  const int32_t* seq_len;     // lengths after the append
  const int32_t* block_table;
  int64_t n_new, max_len, num_pages, max_pages, kblk_stride;
  int G, D, Di, B, ul2;       // ul2 = log2(P / 8)
  int units_max;              // units one sequence's new tokens can touch
  int blocks_max;             // blocks one sequence's new tokens can touch
};

// Page of logical page j for reading: a bad entry is clamped into the pool, which can only give
// wrong values for sequence b.
__device__ __forceinline__ int64_t page_of(const AppendArgs& a, int64_t b, int64_t j) {
  int64_t pg = a.block_table[b * a.max_pages + j];
  return pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
}

// Page of logical page j for writing, or -1 when the entry is outside [0, num_pages): the append
// then stores nothing there, so a bad entry cannot overwrite a page another sequence owns.
__device__ __forceinline__ int64_t page_for_write(const AppendArgs& a, int64_t b, int64_t j) {
  const int64_t pg = a.block_table[b * a.max_pages + j];
  return (pg < 0 || pg >= a.num_pages) ? -1 : pg;
}

// One thread per (sequence, group, touched unit, 8-wide d piece): the unit's new tokens are
// written into K (one 16-byte run per token) and V (one 16-byte run of 8 tokens per d), tokens
// already cached are kept and tokens past the length are zeroed.
__device__ __forceinline__ void append_kv_one(const AppendArgs& a, int64_t id) {
  const int pieces = a.D / 8;
  {
    const int j = static_cast<int>(id % pieces);
    const int64_t r = id / pieces;
    const int uu = static_cast<int>(r % a.units_max);
    const int64_t bg = r / a.units_max;
    const int g = static_cast<int>(bg % a.G);
    const int64_t b = bg / a.G;
    const int64_t start = seq_pos0(a.seq_len, b, a.max_len - a.n_new, a.n_new);
    const int64_t end = start + a.n_new;                 // exclusive
    const int64_t u = (start >> 3) + uu;
    if (u > ((end - 1) >> 3)) return;
    const int64_t page = page_for_write(a, b, (u * 8) >> (a.ul2 + 3));
    if (page < 0) return;
    const int64_t unit_elem = (((page * a.G + g) << a.ul2) | (u & ((1 << a.ul2) - 1))) * 8 * a.D;
    bf16_t* kdst = a.k_pool + unit_elem;
    bf16_t* vdst = a.v_pool + unit_elem;
    const bf16_t* ksrc = a.k_new + (bg * a.n_new) * a.D + 8 * j;
    const bf16_t* vsrc = a.v_new + (bg * a.n_new) * a.D + 8 * j;
    uint32_t vw[8][4];                                   // v rows of the unit's 8 tokens, d piece j
    uint32_t keepmask = 0u;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int64_t pos = u * 8 + t;
      uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = make_uint4(0u, 0u, 0u, 0u);
      if (pos < start) {
        keepmask |= 1u << t;
      } else {
        if (pos < end) {
          kv = *reinterpret_cast<const uint4*>(ksrc + (pos - start) * a.D);
          vv = *reinterpret_cast<const uint4*>(vsrc + (pos - start) * a.D);
        }
        *reinterpret_cast<uint4*>(kdst + (((j >> 1) * 8 + t) * 2 + (j & 1)) * 8) = kv;
      }
      vw[t][0] = vv.x;
      vw[t][1] = vv.y;
      vw[t][2] = vv.z;
      vw[t][3] = vv.w;
    }
    // V: 8 d rows of 8 tokens; cached tokens of a partly new unit are read back and kept
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t tv[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) tv[t] = static_cast<uint16_t>(vw[t][e >> 1] >> (16 * (e & 1)));
      bf16_t* dst = vdst + (8 * j + e) * 8;
      if (keepmask) {
        const uint4 old = *reinterpret_cast<const uint4*>(dst);
        const uint32_t ow[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if ((keepmask >> t) & 1u) tv[t] = static_cast<uint16_t>(ow[t >> 1] >> (16 * (t & 1)));
      }
      uint4 w;
      w.x = tv[0] | (static_cast<uint32_t>(tv[1]) << 16);
      w.y = tv[2] | (static_cast<uint32_t>(tv[3]) << 16);
      w.z = tv[4] | (static_cast<uint32_t>(tv[5]) << 16);
      w.w = tv[6] | (static_cast<uint32_t>(tv[7]) << 16);
      *reinterpret_cast<uint4*>(dst) = w;
    }
  }
}

// One thread per (sequence, new token, 8-wide index piece): copy into the index-key pool.
__device__ __forceinline__ void append_kidx_one(const AppendArgs& a, int64_t id) {
  const int pieces = a.Di / 8;
  const int64_t ptok = int64_t(8) << a.ul2;
  {
    const int j = static_cast<int>(id % pieces);
    const int64_t r = id / pieces;
    const int64_t t = r % a.n_new;
    const int64_t b = r / a.n_new;
    const int64_t pos = seq_pos0(a.seq_len, b, a.max_len - a.n_new, a.n_new) + t;
    const int64_t page = page_for_write(a, b, pos / ptok);
    if (page < 0) return;
    *reinterpret_cast<uint4*>(a.kidx_pool + (page * ptok + (pos & (ptok - 1))) * a.Di + 8 * j) =
        *reinterpret_cast<const uint4*>(a.kidx_new + r * a.Di + 8 * j);
  }
}

// K/V and index keys in one launch (they write different pools): items below kv_total are K/V
// pieces, the rest index-key pieces.
__global__ void __launch_bounds__(256) append_kv_kidx_kernel(AppendArgs a, int64_t kv_total,
                                                             int64_t ki_total) {
  for (int64_t id = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; id < kv_total + ki_total;
       id += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (id < kv_total)
      append_kv_one(a, id);
    else
      append_kidx_one(a, id - kv_total);
  }
}

// One thread per (sequence, touched block, 8-wide index piece): the block key from the cached
// index keys of the block's tokens below the length, summed in token order in fp32.
__global__ void __launch_bounds__(256) append_kblk_kernel(AppendArgs a, int64_t total) {
  const int pieces = a.Di / 8;
  const int64_t ptok = int64_t(8) << a.ul2;
  for (int64_t id = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; id < total;
       id += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int j = static_cast<int>(id % pieces);
    const int64_t r = id / pieces;
    const int jj = static_cast<int>(r % a.blocks_max);
    const int64_t b = r / a.blocks_max;
    const int64_t start = seq_pos0(a.seq_len, b, a.max_len - a.n_new, a.n_new);
    const int64_t end = start + a.n_new;
    const int64_t blk = start / a.B + jj;
    if (blk > (end - 1) / a.B) continue;
    const int64_t t0 = blk * a.B;
    const int64_t t1 = (t0 + a.B < end) ? t0 + a.B : end;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int64_t t = t0; t < t1; ++t) {
      const int64_t page = page_of(a, b, t / ptok);
      const uint4 u = *reinterpret_cast<const uint4*>(a.kidx_pool + (page * ptok + (t & (ptok - 1))) * a.Di + 8 * j);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_to_f32(static_cast<bf16_t>(w[e] & 0xffffu));
        acc[2 * e + 1] += bf16_to_f32(static_cast<bf16_t>(w[e] >> 16));
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(a.k_blk + (b * a.kblk_stride + blk) * a.Di + 8 * j) = o;
  }
}

unsigned grid_for(int64_t total) {
  int64_t blocks = (total + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  return static_cast<unsigned>(blocks);
}

}  // namespace

hipError_t launch_cache_append(const Dims& d, const PagedKV& pk, int64_t n_new, const void* k_new,
                               const void* v_new, const void* kidx_new, void* kidx_pool,
                               void* k_blk, hipStream_t s) {
  AppendArgs a;
  a.k_new = static_cast<const bf16_t*>(k_new);
  a.v_new = static_cast<const bf16_t*>(v_new);
  a.kidx_new = static_cast<const bf16_t*>(kidx_new);
  a.k_pool = static_cast<bf16_t*>(const_cast<void*>(pk.k));
  a.v_pool = static_cast<bf16_t*>(const_cast<void*>(pk.v));
  a.kidx_pool = static_cast<bf16_t*>(kidx_pool);
  a.k_blk = static_cast<bf16_t*>(k_blk);
  a.seq_len = d.seq_len;
  a.block_table = pk.block_table;
  a.n_new = n_new;
  a.max_len = d.Tk;
  a.num_pages = pk.num_pages;
  a.max_pages = pk.max_pages;
  a.kblk_stride = d.kblk_stride;
  a.G = d.G;
  a.D = d.D;
  a.Di = d.Di;
  a.B = d.B;
  a.ul2 = pk.page_units_log2;
  a.units_max = static_cast<int>((n_new + 14) / 8);
  a.blocks_max = static_cast<int>((n_new + 2 * d.B - 2) / d.B);
  const int64_t kv_total = d.Bt * d.G * a.units_max * (d.D / 8);
  const int64_t ki_total = d.Bt * n_new * (d.Di / 8);
  hipLaunchKernelGGL(append_kv_kidx_kernel, dim3(grid_for(kv_total + ki_total)), dim3(256), 0, s, a,
                     kv_total, ki_total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t kb_total = d.Bt * a.blocks_max * (d.Di / 8);
  hipLaunchKernelGGL(append_kblk_kernel, dim3(grid_for(kb_total)), dim3(256), 0, s, a, kb_total);
  return hipGetLastError();
}

}  // namespace sgqa
