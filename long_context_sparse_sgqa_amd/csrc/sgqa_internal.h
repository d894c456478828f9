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
  // Decode over a paged cache: per-sequence key counts (device, nullable: all sequences hold Tk
  // keys) and the k_blk row stride in blocks (NB for the contiguous layout).
  const int32_t* seq_len = nullptr;
  int64_t kblk_stride = 0;
};

// Paged K/V cache (decode).  Page p of the pools holds page_tokens consecutive tokens of one
// sequence for every KV group: K as [G][page_tokens / 8] units in the 4-token operand layout
// (kq_offset), V as [G][page_tokens / 8][D][8].  Logical page j of sequence b is
// block_table[b * max_pages + j].
struct PagedKV {
  const void* k;
  const void* v;
  const int32_t* block_table;
  int64_t num_pages, max_pages;
  int page_units_log2;   // log2(page_tokens / 8)
};

// fp8 (e4m3) K and V: k = code * k_scale, v = code * v_scale.
struct Fp8Scales {
  float k_scale, v_scale;
};

// ---- decode: appending to the paged cache ----------------------------------------------------
// Writes n_new tokens per sequence (ending at d.seq_len[b]) into the K/V pools of `pk` and the
// index-key pool, then recomputes the touched block keys in k_blk (row stride d.kblk_stride).
hipError_t launch_cache_append(const Dims& d, const PagedKV& pk, int64_t n_new, const void* k_new,
                               const void* v_new, const void* kidx_new, void* kidx_pool,
                               void* k_blk, hipStream_t s);

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

// ---- steps 2-3 fused (one-call forward) --------------------------------------------------------
// Candidate capacity per row and whether the fused path serves the problem (bf16 index data,
// budgets up to 513 blocks).
int fused_select_capacity();
bool fused_select_supported(const Dims& d);
// Filter: per chunk row, the (score bits << 32 | block) candidates at or above a sampled
// threshold, in ascending block order, into cand + rr * capacity (count in cnt[rr], possibly
// > capacity).  Also zeroes *fail_count.
hipError_t launch_index_filter(const Dims& d, const void* q_idx, const void* k_blk, uint64_t* cand,
                               int32_t* cnt, int32_t* fail_count, const Chunk& c, hipStream_t s);
// Select from the candidates; rows it cannot settle are appended to fail_list.  `sorted`: every
// list is in ascending block order (launch_index_filter's lists; not the decode filter's).
hipError_t launch_select_candidates(const Dims& d, const uint64_t* cand, const int32_t* cnt,
                                    int32_t* sel, int32_t* fail_list, int32_t* fail_count,
                                    const Chunk& c, bool sorted, hipStream_t s);
// Few rows per sequence (chunk tokens * G <= 32, e.g. decode): per-row thresholds from sampled
// blocks (thr, one workgroup per sequence), then the filter split over slabs of each sequence's
// blocks; fills cand / cnt like launch_index_filter (and zeroes *fail_count).
bool decode_select_supported(const Dims& d, int64_t seq_rows);
hipError_t launch_decode_select(const Dims& d, const void* q_idx, const void* k_blk, uint32_t* thr,
                                uint64_t* cand, int32_t* cnt, int32_t* fail_count, const Chunk& c,
                                hipStream_t s);
// Exact selection of the listed rows from recomputed full score rows.
size_t select_fallback_scratch_bytes(const Dims& d);
hipError_t launch_select_fallback(const Dims& d, const void* q_idx, const void* k_blk,
                                  const int32_t* fail_list, const int32_t* fail_count,
                                  float* scratch, int32_t* sel, const Chunk& c, hipStream_t s);

// ---- step 4: attention ------------------------------------------------------------------------
// Bytes of the unit-packed K and V copies the matrix-core attention kernels read (0 when the
// problem is served by the plain kernel, which reads k and v directly).
size_t attend_packed_kv_bytes(const Dims& d);
// True when the problem takes the matrix-core path.
bool attend_uses_mfma(const Dims& d);
// Largest number of 8-token units one (query, group) selection can cover.
int64_t units_per_query(const Dims& d);
// Range-split attention (bf16, 8 heads, B a multiple of 8): pair-union lists and range partials.
bool attend_split_supported(const Dims& d);
size_t attend_split_bytes(const Dims& d);
// Total attention workspace: packed K and V, then (range-split path) lists and partials.
size_t attend_workspace_bytes(const Dims& d);
// K and V packing (matrix-core paths only; no-op otherwise), then the attention kernel(s).
hipError_t launch_pack_kv(const Dims& d, const void* k, const void* v, void* workspace,
                          hipStream_t s);
// Optional profiling marker: called with index 4 once the attention inputs are ready (pair-union
// lists built on the range-split path) and 5 after the main attention kernel.
using StageMark = hipError_t (*)(int index, hipStream_t s);
// lse (nullable): per row ln sum_t exp(scale q.k_t), written on the range-split path only
// (attend_split_supported; hipErrorInvalidValue otherwise).
hipError_t launch_attend_packed(const Dims& d, const void* q, const void* k, const void* v,
                                const void* gate, const int32_t* sel, void* out, void* workspace,
                                hipStream_t s, StageMark mark = nullptr, float* lse = nullptr);
// With `paged`, K and V come from the paged cache (packed_k / packed_v are ignored) and query
// positions follow d.seq_len.  With `fp8`, packed_k / packed_v hold fp8 copies
// (launch_pack_kv_fp8).
hipError_t launch_attend_split(const Dims& d, const void* q, const void* packed_k,
                               const void* gate, const int32_t* sel, void* out,
                               const void* packed_v, void* ws, hipStream_t s, StageMark mark,
                               const PagedKV* paged = nullptr, const Fp8Scales* fp8 = nullptr,
                               float* lse = nullptr);
// fp8 e4m3 K and V ([Bt, G, Tk, D] bytes) packed per 8-token unit for the range kernel: bytes of
// one copy, and the packing of both into `packed` (K copy, then V copy at packed_kv_fp8_bytes / 2).
size_t packed_kv_fp8_bytes(const Dims& d);
hipError_t launch_pack_kv_fp8(const Dims& d, const void* k8, const void* v8, void* packed,
                              hipStream_t s);
// Gated sliding-window attention (the efficient layers): every query attends to the tokens
// t in [p - window + 1, p], with the range kernel over contiguous unit lists; K and V packed as
// for launch_attend_split (launch_pack_kv with quad layout).
bool attend_window_supported(const Dims& d);
size_t attend_window_bytes(const Dims& d, int64_t window);
hipError_t launch_attend_window(const Dims& d, int64_t window, const void* q, const void* packed_k,
                                const void* gate, void* out, const void* packed_v, void* ws,
                                hipStream_t s);
// Packed K and V in the 4-token layout the range kernel reads: bytes, and the packing.
size_t packed_kv_quad_bytes(const Dims& d);
hipError_t launch_pack_kv_quad(const Dims& d, const void* k, const void* v, void* packed,
                               hipStream_t s);
// Backward of the gated attention step for a fixed selection (range-split constraints): dq and
// dgate in q's layout and dtype, dk / dv as fp32 [Bt, G, Tk, D] (zeroed, then accumulated).
size_t attend_backward_bytes(const Dims& d);
// Key-major dK and dV of the gated attention step (attend_bwd.hip): from the selection, dO =
// dout * sigmoid(gate) and the per-row lse2 / Dr statistics; every element of dk and dv written
// once.  Workspace: backward_dkv_bytes(d).
size_t backward_dkv_bytes(const Dims& d);
hipError_t launch_backward_dkv(const Dims& d, const void* q, const void* d_o, const float* lse2,
                               const float* Dr, const void* k, const void* v, const int32_t* sel,
                               float* dk, float* dv, void* ws, hipStream_t s);
// With saved_out / saved_lse (the forward's output and natural-log lse per row, both or neither)
// the softmax statistics come from them instead of a forward recompute.
hipError_t launch_attend_backward(const Dims& d, const void* q, const void* k, const void* v,
                                  const void* gate, const int32_t* sel, const void* dout, void* dq,
                                  float* dk, float* dv, void* dgate, void* ws, hipStream_t s,
                                  const void* saved_out = nullptr, const float* saved_lse = nullptr);
// Both of the above.
hipError_t launch_attend(const Dims& d, const void* q, const void* k, const void* v,
                         const void* gate, const int32_t* sel, void* out, void* workspace,
                         hipStream_t s);

}  // namespace sgqa
