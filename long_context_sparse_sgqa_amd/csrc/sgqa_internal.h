// Internal host-side interface between the C ABI (sgqa_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace sgqa {

// Validated problem dimensions, all derived once on the host.
struct Dims {
  int64_t Bt, Tq, Tk;    // batch, query tokens, key tokens
  int G, H, D, Di;       // KV groups, heads per group, head dim, index dim
  int B;                 // block size
  int NS;                // selected blocks per (query, group) = topk / B
  int64_t NB;            // number of blocks = ceil(Tk / B)
  int64_t NU;            // number of 8-token units = ceil(Tk / 8)
  int64_t pos0;          // absolute position of query 0 = Tk - Tq
  float scale;           // softmax scale
  bool bf16;             // q/k/v/gate/out are bf16 (else fp32)
  bool idx_bf16;         // q_idx/k_idx/k_blk are bf16 (else fp32)
};

// ---- step 1: block compression -------------------------------------------------------------
hipError_t launch_compress(const Dims& d, const void* k_idx, void* k_blk, hipStream_t s);

// ---- query-row chunks ------------------------------------------------------------------------
// A chunk is a rectangle of query tokens: sequences [b0, b0 + nseq), tokens [i0, i0 + ntok) of each
// (either nseq == 1, or i0 == 0 and ntok == Tq).  Row rr of a chunk is (b, i, g) with
// b = b0 + rr / (ntok * G), i = i0 + (rr / G) % ntok, g = rr % G.
struct Chunk {
  int64_t b0, nseq, i0, ntok;
  int64_t rows(int G) const { return nseq * ntok * G; }
};

// ---- step 2: indexer ----------------------------------------------------------------------------
// Scores of every row of the chunk: scores + rr * NB + j for j < p/B (p = pos0 + i).
hipError_t launch_index(const Dims& d, const void* q_idx, const void* k_blk, float* scores,
                        const Chunk& c, hipStream_t s);

// ---- step 3: selection ---------------------------------------------------------------------------
// Reads the chunk's score rows (laid out as launch_index writes them) and writes
// sel + ((b * Tq + i) * G + g) * NS.
hipError_t launch_topk(const Dims& d, const float* scores, int32_t* sel, const Chunk& c,
                       hipStream_t s);

// ---- step 4: attention ------------------------------------------------------------------------
// Bytes of the unit-packed V copy the matrix-core attention kernel reads (0 when the problem is
// served by the plain kernel, which reads v directly).
size_t attend_packed_v_bytes(const Dims& d);
// True when the problem takes the matrix-core path.
bool attend_uses_mfma(const Dims& d);
// Largest number of 8-token units one (query, group) selection can cover.
int64_t units_per_query(const Dims& d);
hipError_t launch_attend(const Dims& d, const void* q, const void* k, const void* v,
                         const void* gate, const int32_t* sel, void* out, void* packed_v,
                         hipStream_t s);

}  // namespace sgqa
