// Device helpers shared by the gfx950 kernels: bf16 storage, vector types, MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgqa {

typedef uint16_t bf16_t;  // bf16 held as its bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Two fp32 -> packed pair of bf16 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float x) { *p = f32_to_bf16(x); }
};

// 16-byte global load as the MFMA bf16x8 operand.
__device__ __forceinline__ bf16x8_t load_bf16x8(const bf16_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ bf16x8_t bf16x8_from_u4(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ bf16x8_t zero_bf16x8() {
  uint4 u = make_uint4(0u, 0u, 0u, 0u);
  return __builtin_bit_cast(bf16x8_t, u);
}

// D = A(16x32) * B(32x16) + C, bf16 inputs, fp32 accumulate (v_mfma_f32_16x16x32_bf16).
// Lane l supplies A[l % 16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l % 16]; it receives
// C[4*(l/16) + i][l % 16] for i = 0..3.
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate (v_mfma_f32_32x32x16_bf16).
// Lane l supplies A[l % 32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l % 32]; it receives
// C[8*(r/4) + 4*(l/32) + r%4][l % 32] for r = 0..15.
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Hardware round-to-nearest-even packing of 8 fp32 into the bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8_t pack8_bf16(const float* v) {
  typedef float f32x8_t __attribute__((ext_vector_type(8)));
  const f32x8_t x = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
  return __builtin_convertvector(x, bf16x8_t);
}

// Raw buffer access: wave-uniform base and size, 32-bit byte offsets, reads past `bytes` give 0.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ BufRsrc make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           0x00020000);
}

__device__ __forceinline__ bf16x8_t buffer_load_bf16x8(BufRsrc r, int byte_offset) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0);
  return __builtin_bit_cast(bf16x8_t, v);
}

// Online softmax with a lazy running max: the accumulators are rescaled only when some row's
// maximum (log2 domain) exceeds the max they are referenced to by more than this margin.  Until
// then probabilities exp2(s - m) may reach 2^margin (256), far inside fp32 and bf16 range, and the
// result is the same softmax: O, l and m stay mutually consistent whatever reference m is used.
constexpr float kLazyRescaleLog2 = 8.0f;

// Position of query 0 of sequence b.  Equal-length sequences: pos0 = Tk - Tq.  With per-sequence
// key counts (decode over a paged cache) the queries are the last Tq of seq_len[b] tokens; the
// count is clamped to [Tq, Tk] so that a bad entry can never index outside the buffers.
__device__ __forceinline__ int64_t seq_pos0(const int32_t* seq_len, int64_t b, int64_t pos0,
                                            int64_t Tq) {
  if (!seq_len) return pos0;
  int64_t L = seq_len[b];
  L = L < Tq ? Tq : (L > pos0 + Tq ? pos0 + Tq : L);
  return L - Tq;
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

// max(v, v of lane ^ 32) without LDS: v_permlane32_swap exchanges the two 32-lane halves of its
// operands, so with both operands = v one result holds v of the other half in lanes 0..31 and the
// other in lanes 32..63.  (A ds_bpermute would count against lgkmcnt, and a wait for it would also
// wait for any scalar load in flight.)
__device__ __forceinline__ float max_with_other_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Wave-wide reductions and scans on DPP (data-parallel primitives on rows of 16 lanes) instead of
// ds_bpermute: no LDS round trip and no lgkmcnt wait per step.  All 64 lanes must be active.
// DPP controls: quad_perm [1,0,3,2] = 0xb1, [2,3,0,1] = 0x4e, row_half_mirror = 0x141,
// row_mirror = 0x140, row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143.
//
// Reduction: after the quad exchanges and the two mirrors every lane holds its row's result;
// the four row results are read into scalars and combined.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xb1, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4e, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x140, 0xf, 0xf, false)));
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
  const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
  const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
  const uint32_t r3 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
  return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ int wave_total(int v) {
  return static_cast<int>(wave_reduce_u32(static_cast<uint32_t>(v),
                                          [](uint32_t x, uint32_t y) { return x + y; }));
}

// Inclusive prefix sum over lanes 0..63: a shift-and-add scan inside each row of 16 lanes (lanes
// shifted in from outside the row read 0), then the last lane of row 0 is added to row 1 and of
// row 2 to row 3, then lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

}  // namespace sgqa
