// Step 2 -- the indexer: block scores of every (query token, KV group) row.
//
// The Step 5 Preview pages (mo.ai.kr summary, section "모델 구조와 학습 안정성") score each query
// against the block-compressed shared index keys and note that blocks of 8 make the indexer (and
// the top-k after it) eight times cheaper than token-level scoring.  The score of row (b, i, g)
// against block j is the raw dot product q_idx[b,i,g,:] . k_blk[b,j,:], defined for the strictly
// past blocks j < p/B (the own block is always selected and never scored).
//
// bf16: a GEMM rows x blocks x Di on v_mfma_f32_16x16x32_bf16.  A workgroup of 4 waves owns a
// 128-row x 128-block tile (one sequence), each wave a 64 x 64 sub-tile of 4 x 4 MFMA tiles;
// operands are loaded straight into the MFMA lane layout with 16-byte loads (rows of q_idx and of
// k_blk are contiguous in Di).  Tiles entirely past the causal limit of their last row exit at once;
// partial tiles store only j < p/B.  fp32 accumulation of integer-valued inputs is exact.
// fp32 (the small correctness workload): one thread per (row, block), plain fp32 FMA loop.
#include "device_common.h"
#include "sgqa_internal.h"

namespace sgqa {
namespace {

constexpr int kRowTile = 128;
constexpr int kColTile = 128;

struct RowMap {
  int64_t b0, i0, ntok, Tq, pos0;
  int G, B;
  const int32_t* seq_len;   // per-sequence key counts, or null (every sequence holds Tk keys)
  // causal limit o = p / B of row (b, i)
  __device__ __forceinline__ int64_t own_block(int64_t b, int64_t i) const {
    return (seq_pos0(seq_len, b, pos0, Tq) + i) / B;
  }
  // token coordinates of chunk row rr
  __device__ __forceinline__ void at(int64_t rr, int64_t& b, int64_t& i, int& g) const {
    const int64_t tok = rr / G;
    g = static_cast<int>(rr - tok * G);
    b = b0 + tok / ntok;
    i = i0 + tok % ntok;
  }
};

__global__ void __launch_bounds__(256) index_bf16_kernel(const bf16_t* __restrict__ q_idx,
                                                         const bf16_t* __restrict__ k_blk,
                                                         float* __restrict__ scores, RowMap map,
                                                         int64_t NB, int64_t kblk_stride, int Di,
                                                         int64_t seq_rows, int64_t tiles_per_seq) {
  const int64_t seq = blockIdx.x / tiles_per_seq;
  const int64_t tile = blockIdx.x - seq * tiles_per_seq;
  const int64_t row0 = tile * kRowTile;                        // first row within the sequence
  const int64_t col0 = static_cast<int64_t>(blockIdx.y) * kColTile;
  const int64_t rows_here = min<int64_t>(kRowTile, seq_rows - row0);

  // causal limit of the tile: the last row holds the largest position
  {
    int64_t b, i;
    int g;
    map.at(seq * seq_rows + row0 + rows_here - 1, b, i, g);
    const int64_t o_max = map.own_block(b, i);
    if (col0 >= o_max) return;
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int lr = lane & 15, lk = lane >> 4;

  const int64_t b_seq = map.b0 + seq;
  const bf16_t* kb = k_blk + b_seq * kblk_stride * Di;

  f32x4_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // row pointers of this lane's A rows
  const bf16_t* arow[4];
  bool avalid[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t rl = row0 + wr * 64 + m * 16 + lr;
    avalid[m] = rl < seq_rows;
    int64_t b, i;
    int g;
    map.at(seq * seq_rows + (avalid[m] ? rl : 0), b, i, g);
    arow[m] = q_idx + ((b * map.Tq + i) * map.G + g) * Di;
  }
  const bf16_t* brow[4];
  bool bvalid[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int64_t j = col0 + wc * 64 + n * 16 + lr;
    bvalid[n] = j < NB;                 // NB <= kblk_stride
    brow[n] = kb + (bvalid[n] ? j : 0) * Di;
  }

  for (int kc = 0; kc < Di; kc += 32) {
    bf16x8_t a[4], bb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) a[m] = avalid[m] ? load_bf16x8(arow[m] + kc + lk * 8) : zero_bf16x8();
#pragma unroll
    for (int n = 0; n < 4; ++n) bb[n] = bvalid[n] ? load_bf16x8(brow[n] + kc + lk * 8) : zero_bf16x8();
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = mfma16x16x32(a[m], bb[n], acc[m][n]);
  }

  // store C[row][col] for col < o(row)
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t rl = row0 + wr * 64 + m * 16 + lk * 4 + e;
      if (rl >= seq_rows) continue;
      int64_t b, i;
      int g;
      const int64_t rr = seq * seq_rows + rl;
      map.at(rr, b, i, g);
      const int64_t o = map.own_block(b, i);
      float* dst = scores + rr * NB;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int64_t j = col0 + wc * 64 + n * 16 + lr;
        if (j < o) dst[j] = acc[m][n][e];
      }
    }
  }
}

// Few rows per sequence (decode: 4 new tokens x 8 groups): all of a sequence's rows (<= 32) form
// the M = 32 side of v_mfma_f32_32x32x16_bf16 and a workgroup sweeps a slab of blocks, 32 columns
// per wave per step, so every block key is read once.  Lane (c, h) feeds query row c and block
// col0 + c (index dims 16 kc + 8 h ..), and receives rows 8 (r/4) + 4h + r%4 of column c.
template <int DI>
__global__ void __launch_bounds__(256) index_rows32_kernel(const bf16_t* __restrict__ q_idx,
                                                           const bf16_t* __restrict__ k_blk,
                                                           float* __restrict__ scores, RowMap map,
                                                           int64_t NB, int64_t kblk_stride,
                                                           int64_t seq_rows, int64_t slab_cols) {
  const int64_t seq = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 31, h = lane >> 5;
  // All rows of the workgroup belong to sequence b0 + seq: row r is token i0 + r / G, group r % G,
  // so one load of the sequence's length gives every row's position.
  const int64_t b = map.b0 + seq;
  const int64_t p0 = seq_pos0(map.seq_len, b, map.pos0, map.Tq) + map.i0;   // position of row 0's token
  const int64_t o_max = (p0 + (seq_rows - 1) / map.G) / map.B;
  const int64_t c_begin = static_cast<int64_t>(blockIdx.x) * slab_cols;
  const int64_t c_end = min(c_begin + slab_cols, o_max);
  if (c_begin >= c_end) return;

  bf16x8_t qa[DI / 16];
  {
    const bool ok = c < seq_rows;
    const int row = ok ? c : 0;
    const bf16_t* qrow = q_idx + ((b * map.Tq + map.i0 + row / map.G) * map.G + row % map.G) * DI;
#pragma unroll
    for (int kc = 0; kc < DI / 16; ++kc) qa[kc] = ok ? load_bf16x8(qrow + 16 * kc + 8 * h) : zero_bf16x8();
  }
  // causal limit and score-row offset of each output row of this lane (o = 0 past the sequence's
  // rows).  Scores are written through a buffer descriptor over the sequence's rows with no branch:
  // masked entries take an out-of-range offset, which the hardware drops, so the compiler can count
  // the stores and the next step's loads stay in flight across them.
  int32_t o_r[16];
  int32_t off_r[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + 4 * h + (r & 3);
    const bool ok = row < seq_rows;
    o_r[r] = ok ? static_cast<int32_t>((p0 + row / map.G) / map.B) : 0;
    off_r[r] = static_cast<int32_t>((ok ? row : 0) * NB * 4);
  }
  const BufRsrc srs = make_rsrc(scores + seq * seq_rows * NB, seq_rows * NB * 4);
  const bf16_t* kb = k_blk + b * kblk_stride * DI;
  // The next step's block keys are loaded before this step's products, unconditionally (columns
  // past NB load the last block; their scores are never stored, since every row's causal limit is
  // below NB), so no branch hides the loads from the compiler's wait counting and each step's loads
  // overlap the previous step's products and stores.  Two register sets are used in turn (a copy
  // between them would wait for the loads).
  auto load_keys = [&](int64_t col0, uint4* kk) {
    const int64_t col = col0 + c;
    const int64_t cc = col < NB ? col : NB - 1;
#pragma unroll
    for (int kc = 0; kc < DI / 16; ++kc)
      kk[kc] = *reinterpret_cast<const uint4*>(kb + cc * DI + 16 * kc + 8 * h);
  };
  int64_t col0 = c_begin + 32 * wave;
  uint4 kA[DI / 16], kB[DI / 16];
  load_keys(col0, kA);
  auto step = [&](const uint4* kcur, uint4* knext) {
    load_keys(col0 + 128, knext);
    const int64_t col = col0 + c;
    f32x16_t acc = {};
#pragma unroll
    for (int kc = 0; kc < DI / 16; ++kc) acc = mfma32x32x16(qa[kc], bf16x8_from_u4(kcur[kc]), acc);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[r]), srs,
                                            col < o_r[r] ? off_r[r] + static_cast<int32_t>(col) * 4 : 0x7fffffff,
                                            0, 0);
    col0 += 128;
  };
  while (col0 < c_end) {
    step(kA, kB);
    if (col0 >= c_end) break;
    step(kB, kA);
  }
}

__global__ void __launch_bounds__(256) index_f32_kernel(const float* __restrict__ q_idx,
                                                        const float* __restrict__ k_blk,
                                                        float* __restrict__ scores, RowMap map,
                                                        int64_t NB, int64_t kblk_stride, int Di,
                                                        int64_t rows) {
  const int64_t rr = blockIdx.x;
  if (rr >= rows) return;
  int64_t b, i;
  int g;
  map.at(rr, b, i, g);
  const int64_t o = map.own_block(b, i);
  const float* q = q_idx + ((b * map.Tq + i) * map.G + g) * Di;
  const float* kb = k_blk + b * kblk_stride * Di;
  for (int64_t j = blockIdx.y * (int64_t)blockDim.x + threadIdx.x; j < o;
       j += (int64_t)gridDim.y * blockDim.x) {
    const float* kr = kb + j * Di;
    float s = 0.f;
    for (int c = 0; c < Di; ++c) s = fmaf(q[c], kr[c], s);
    scores[rr * NB + j] = s;
  }
}

}  // namespace

hipError_t launch_index(const Dims& d, const void* q_idx, const void* k_blk, float* scores,
                        const Chunk& c, hipStream_t s) {
  RowMap map{c.b0, c.i0, c.ntok, d.Tq, d.pos0, d.G, d.B, d.seq_len};
  const int64_t kstride = d.kblk_stride > 0 ? d.kblk_stride : d.NB;
  const int64_t rows = c.rows(d.G);
  if (rows == 0) return hipSuccess;
  if (d.idx_bf16 && c.ntok * d.G <= 32) {
    const int64_t seq_rows = c.ntok * d.G;
    const int64_t slab = 1024;
    const int64_t max_o = (d.Tk - 1) / d.B;                  // no query has a past block: no scores
    const dim3 grid(static_cast<unsigned>((max_o + slab - 1) / slab), static_cast<unsigned>(c.nseq));
    if (max_o == 0)
      return hipSuccess;
    else if (d.Di == 128)
      hipLaunchKernelGGL(index_rows32_kernel<128>, grid, dim3(256), 0, s,
                         static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_blk), scores,
                         map, d.NB, kstride, seq_rows, slab);
    else if (d.Di == 64)
      hipLaunchKernelGGL(index_rows32_kernel<64>, grid, dim3(256), 0, s,
                         static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_blk), scores,
                         map, d.NB, kstride, seq_rows, slab);
    else
      hipLaunchKernelGGL(index_rows32_kernel<32>, grid, dim3(256), 0, s,
                         static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_blk), scores,
                         map, d.NB, kstride, seq_rows, slab);
  } else if (d.idx_bf16) {
    const int64_t seq_rows = c.ntok * d.G;
    const int64_t tps = (seq_rows + kRowTile - 1) / kRowTile;
    const int64_t col_tiles = (d.NB + kColTile - 1) / kColTile;
    dim3 grid(static_cast<unsigned>(tps * c.nseq), static_cast<unsigned>(col_tiles));
    hipLaunchKernelGGL(index_bf16_kernel, grid, dim3(256), 0, s,
                       static_cast<const bf16_t*>(q_idx), static_cast<const bf16_t*>(k_blk), scores,
                       map, d.NB, kstride, d.Di, seq_rows, tps);
  } else {
    const int64_t max_o = (d.Tk - 1) / d.B;
    int64_t gy = (max_o + 255) / 256;
    gy = gy < 1 ? 1 : (gy > 1024 ? 1024 : gy);
    dim3 grid(static_cast<unsigned>(rows), static_cast<unsigned>(gy));
    hipLaunchKernelGGL(index_f32_kernel, grid, dim3(256), 0, s, static_cast<const float*>(q_idx),
                       static_cast<const float*>(k_blk), scores, map, d.NB, kstride, d.Di, rows);
  }
  return hipGetLastError();
}

}  // namespace sgqa
