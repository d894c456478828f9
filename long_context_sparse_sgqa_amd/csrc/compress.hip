// Step 1 -- block compression of the shared index keys.
//
// The Step 5 Preview pages (mo.ai.kr summary, section "모델 구조와 학습 안정성"; ai.info article,
// section on Sparse GQA and the 1M context) compress the shared index keys block-wise, B tokens per
// block.  A block key is the sum of its B index keys (a partial last block sums the keys present),
// accumulated in fp32 and rounded once to the index dtype.
//
// HBM streaming pass: each thread owns 16 bytes of one block key (8 bf16 or 4 fp32 dims) and reads
// the matching 16 bytes of the block's B token rows.  Consecutive threads cover consecutive 16-byte
// chunks of a row, so every wavefront load is a contiguous run of one token row.
#include "device_common.h"
#include "sgqa_internal.h"

namespace sgqa {
namespace {

template <typename T, int VEC>
__global__ void __launch_bounds__(256) compress_kernel(const T* __restrict__ k_idx,
                                                       T* __restrict__ k_blk, int64_t Tk,
                                                       int64_t NB, int Di, int B, int64_t total) {
  const int chunks = Di / VEC;
  for (int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * blockDim.x) {
    const int c = static_cast<int>(id % chunks);
    const int64_t bj = id / chunks;          // b * NB + j
    const int64_t j = bj % NB;
    const int64_t b = bj / NB;
    const int64_t t0 = j * B;
    const int64_t t1 = (t0 + B < Tk) ? t0 + B : Tk;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    const T* src = k_idx + (b * Tk) * Di + c * VEC;
    for (int64_t t = t0; t < t1; ++t) {
      const T* row = src + t * Di;
      if constexpr (VEC == 8) {
        uint4 u = *reinterpret_cast<const uint4*>(row);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16_to_f32(static_cast<bf16_t>(w[e] & 0xffffu));
          acc[2 * e + 1] += bf16_to_f32(static_cast<bf16_t>(w[e] >> 16));
        }
      } else {
        float4 f = *reinterpret_cast<const float4*>(row);
        acc[0] += f.x; acc[1] += f.y; acc[2] += f.z; acc[3] += f.w;
      }
    }
    T* dst = k_blk + bj * Di + c * VEC;
    if constexpr (VEC == 8) {
      uint4 u;
      u.x = pack_bf16x2(acc[0], acc[1]);
      u.y = pack_bf16x2(acc[2], acc[3]);
      u.z = pack_bf16x2(acc[4], acc[5]);
      u.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(dst) = u;
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

}  // namespace

hipError_t launch_compress(const Dims& d, const void* k_idx, void* k_blk, hipStream_t s) {
  const int vec = d.idx_bf16 ? 8 : 4;
  const int64_t total = d.Bt * d.NB * (d.Di / vec);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  if (d.idx_bf16) {
    hipLaunchKernelGGL((compress_kernel<bf16_t, 8>), dim3((unsigned)blocks), dim3(threads), 0, s,
                       static_cast<const bf16_t*>(k_idx), static_cast<bf16_t*>(k_blk), d.Tk, d.NB,
                       d.Di, d.B, total);
  } else {
    hipLaunchKernelGGL((compress_kernel<float, 4>), dim3((unsigned)blocks), dim3(threads), 0, s,
                       static_cast<const float*>(k_idx), static_cast<float*>(k_blk), d.Tk, d.NB,
                       d.Di, d.B, total);
  }
  return hipGetLastError();
}

}  // namespace sgqa
