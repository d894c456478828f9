// C ABI of the Sparse GQA forward path: argument validation, sizes, workspace carving, row
// chunking and kernel dispatch.  Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/sgqa.h"
#include "sgqa_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_stage_events[SGQA_STAGE_EVENTS];
thread_local bool g_stage_armed = false;

sgqa_status fail(sgqa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sgqa_status ok() {
  g_last_error.clear();
  return SGQA_OK;
}

sgqa_status hip_fail(hipError_t e, const char* where) {
  return fail(SGQA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// Products of sizes, refusing anything past 2^62.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > (int64_t(1) << 62) / a) return false;
  *out = a * b;
  return true;
}

size_t dtype_size(int32_t dt) { return dt == SGQA_BF16 ? 2 : 4; }

// Query tokens per chunk are bounded by a fixed budget of per-chunk selection state (stored score
// rows on the split path, candidate lists on the fused path).  17 GiB holds the candidate lists of
// a whole 128K-token prefill with 8 groups (16.01 GiB), so it runs as one chunk: one filter launch
// whose row tiles are all dispatched longest first, and one select launch, instead of three of each
// with their launch tails; a small share of a GPU with 288 GB of HBM.
constexpr size_t kForwardChunkBudget = size_t(17) << 30;   // 17 GiB

struct Derived {
  sgqa::Dims d;
  size_t k_blk_bytes, scores_bytes, sel_bytes, attend_ws_bytes;
  size_t score_row_bytes;   // per query token (all groups)
};

sgqa_status derive(const sgqa_problem* p, Derived* out) {
  if (!p) return fail(SGQA_ERR_NULL, "problem descriptor is NULL");
  if (p->batch < 1) return fail(SGQA_ERR_SHAPE, "batch must be >= 1 (got %lld)", (long long)p->batch);
  if (p->t_kv < 1) return fail(SGQA_ERR_SHAPE, "t_kv must be >= 1 (got %lld)", (long long)p->t_kv);
  if (p->t_q < 1 || p->t_q > p->t_kv)
    return fail(SGQA_ERR_SHAPE, "t_q must be in [1, t_kv] (got t_q=%lld, t_kv=%lld)",
                (long long)p->t_q, (long long)p->t_kv);
  if (p->kv_groups < 1) return fail(SGQA_ERR_SHAPE, "kv_groups must be >= 1");
  if (p->heads_per_group < 1) return fail(SGQA_ERR_SHAPE, "heads_per_group must be >= 1");
  if (p->block < 1) return fail(SGQA_ERR_SHAPE, "block must be >= 1 (got %d)", p->block);
  if (p->topk_tokens < p->block || p->topk_tokens % p->block != 0)
    return fail(SGQA_ERR_SHAPE, "topk_tokens must be a positive multiple of block (got k=%d, B=%d)",
                p->topk_tokens, p->block);
  if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f))
    return fail(SGQA_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (p->dtype != SGQA_F32 && p->dtype != SGQA_BF16)
    return fail(SGQA_ERR_UNSUPPORTED, "dtype must be SGQA_F32 or SGQA_BF16 (got %d)", p->dtype);
  if (p->index_dtype != SGQA_F32 && p->index_dtype != SGQA_BF16)
    return fail(SGQA_ERR_UNSUPPORTED, "index_dtype must be SGQA_F32 or SGQA_BF16 (got %d)",
                p->index_dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SGQA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
  if (p->index_dim != 32 && p->index_dim != 64 && p->index_dim != 128)
    return fail(SGQA_ERR_UNSUPPORTED, "index_dim must be 32, 64 or 128 (got %d)", p->index_dim);
  if (p->heads_per_group > 32)
    return fail(SGQA_ERR_UNSUPPORTED, "heads_per_group must be <= 32 (got %d)", p->heads_per_group);
  const int64_t ns = p->topk_tokens / p->block;
  if (ns > 4096) return fail(SGQA_ERR_UNSUPPORTED, "topk_tokens / block must be <= 4096 (got %lld)",
                             (long long)ns);
  if (p->t_kv >= (int64_t(1) << 27))
    return fail(SGQA_ERR_UNSUPPORTED, "t_kv must be < 2^27 (got %lld)", (long long)p->t_kv);

  sgqa::Dims& d = out->d;
  d.Bt = p->batch;
  d.Tq = p->t_q;
  d.Tk = p->t_kv;
  d.G = p->kv_groups;
  d.H = p->heads_per_group;
  d.D = p->head_dim;
  d.Di = p->index_dim;
  d.B = p->block;
  d.NS = static_cast<int>(ns);
  d.NB = (p->t_kv + p->block - 1) / p->block;
  d.NU = (p->t_kv + 7) / 8;
  d.pos0 = p->t_kv - p->t_q;
  d.scale = p->softmax_scale;
  d.bf16 = p->dtype == SGQA_BF16;
  d.idx_bf16 = p->index_dtype == SGQA_BF16;

  int64_t rows, x;
  if (!mul_ok(d.Bt, d.Tq, &rows) || !mul_ok(rows, d.G, &rows) || rows >= (int64_t(1) << 31))
    return fail(SGQA_ERR_UNSUPPORTED, "batch * t_q * kv_groups must be < 2^31");
  if (!mul_ok(d.Bt, d.NB, &x) || !mul_ok(x, d.Di, &x))
    return fail(SGQA_ERR_SHAPE, "k_blk size overflows");
  out->k_blk_bytes = static_cast<size_t>(x) * dtype_size(p->index_dtype);
  if (!mul_ok(rows, d.NB, &x) || !mul_ok(x, 4, &x)) return fail(SGQA_ERR_SHAPE, "scores size overflows");
  out->scores_bytes = static_cast<size_t>(x);
  if (!mul_ok(rows, d.NS, &x) || !mul_ok(x, 4, &x)) return fail(SGQA_ERR_SHAPE, "sel size overflows");
  out->sel_bytes = static_cast<size_t>(x);
  if (!mul_ok(d.Bt * d.G, d.NU, &x) || !mul_ok(x, 8 * d.D, &x))
    return fail(SGQA_ERR_SHAPE, "k/v size overflows");
  out->attend_ws_bytes = sgqa::attend_workspace_bytes(d);
  out->score_row_bytes = static_cast<size_t>(d.G) * static_cast<size_t>(d.NB) * 4;
  return SGQA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Forward workspace layout.
//   fused path : [attention workspace][internal sel][fail count][fallback scratch][cand][cnt][fail list]
//   split path : [attention workspace][internal sel][scores]
// where the last group is sized per query token and repeats for `chunk_tok` tokens.
struct ForwardLayout {
  bool fused;
  size_t off_sel, off_failcnt, off_scratch, off_chunk;
  size_t fixed;           // bytes before the per-chunk area
  size_t per_token;       // per-chunk bytes per query token (all groups)
  size_t cand_bytes, cnt_bytes, fail_bytes;   // per token, fused path
};

ForwardLayout forward_layout(const Derived& dv) {
  ForwardLayout L{};
  const sgqa::Dims& d = dv.d;
  L.fused = sgqa::fused_select_supported(d);
  size_t off = align_up(dv.attend_ws_bytes);
  L.off_sel = off;
  off += align_up(dv.sel_bytes);
  if (L.fused) {
    L.off_failcnt = off;
    off += kAlign;
    L.off_scratch = off;
    off += align_up(sgqa::select_fallback_scratch_bytes(d));
    L.cand_bytes = static_cast<size_t>(d.G) * sgqa::fused_select_capacity() * sizeof(uint64_t);
    L.cnt_bytes = static_cast<size_t>(d.G) * sizeof(int32_t);
    L.fail_bytes = static_cast<size_t>(d.G) * sizeof(int32_t);
    L.per_token = L.cand_bytes + L.cnt_bytes + L.fail_bytes;
  } else {
    L.per_token = dv.score_row_bytes;
  }
  L.off_chunk = off;
  L.fixed = off;
  return L;
}

// Bytes of the per-chunk area for `tok` tokens (each sub-array aligned).
size_t chunk_bytes(const ForwardLayout& L, int64_t tok) {
  const size_t t = static_cast<size_t>(tok);
  if (L.fused) return align_up(t * L.cand_bytes) + align_up(t * L.cnt_bytes) + align_up(t * L.fail_bytes);
  return align_up(t * L.per_token);
}

size_t forward_default_bytes(const Derived& dv) {
  const ForwardLayout L = forward_layout(dv);
  const int64_t tokens = dv.d.Bt * dv.d.Tq;
  int64_t chunk = static_cast<int64_t>(kForwardChunkBudget / L.per_token);
  if (chunk < 1) chunk = 1;
  if (chunk > tokens) chunk = tokens;
  return L.fixed + chunk_bytes(L, chunk);
}

// Largest chunk (in query tokens) the given workspace holds; 0 if not even one token fits.
int64_t forward_chunk_tokens(const Derived& dv, const ForwardLayout& L, size_t ws_bytes) {
  if (ws_bytes < L.fixed) return 0;
  const int64_t tokens = dv.d.Bt * dv.d.Tq;
  int64_t chunk = static_cast<int64_t>((ws_bytes - L.fixed) / L.per_token);
  if (chunk > tokens) chunk = tokens;
  while (chunk > 0 && L.fixed + chunk_bytes(L, chunk) > ws_bytes) --chunk;
  return chunk;
}

sgqa_status check_ptr(const void* p, const char* name, unsigned align = 16) {
  if (!p) return fail(SGQA_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    return fail(SGQA_ERR_ALIGN, "%s is not %u-byte aligned", name, align);
  return SGQA_OK;
}

// Records stage marker `i` when the profiling hook is armed.
sgqa_status mark_stage(int i, hipStream_t s) {
  if (!g_stage_armed) return SGQA_OK;
  hipError_t e = hipEventRecord(g_stage_events[i], s);
  if (e != hipSuccess) return hip_fail(e, "stage marker");
  return SGQA_OK;
}

// The same, in the form the attention launcher calls between its kernels.
hipError_t mark_stage_hip(int i, hipStream_t s) {
  return g_stage_armed ? hipEventRecord(g_stage_events[i], s) : hipSuccess;
}

#define SGQA_CHECK(expr)                \
  do {                                  \
    sgqa_status _st = (expr);           \
    if (_st != SGQA_OK) return _st;     \
  } while (0)

// Query-token rectangles of at most `chunk_tok` tokens covering every sequence.
template <class F>
sgqa_status for_each_chunk(const sgqa::Dims& d, int64_t chunk_tok, F&& fn) {
  for (int64_t b = 0; b < d.Bt;) {
    sgqa::Chunk c;
    if (chunk_tok >= d.Tq) {
      c.b0 = b;
      c.nseq = chunk_tok / d.Tq;
      if (c.nseq > d.Bt - b) c.nseq = d.Bt - b;
      c.i0 = 0;
      c.ntok = d.Tq;
      SGQA_CHECK(fn(c));
      b += c.nseq;
    } else {
      // as many chunks as the workspace requires, of equal size (no short last chunk whose launches
      // would leave most of the GPU idle)
      const int64_t nch = (d.Tq + chunk_tok - 1) / chunk_tok;
      const int64_t per = (d.Tq + nch - 1) / nch;
      for (int64_t i0 = 0; i0 < d.Tq; i0 += per) {
        c.b0 = b;
        c.nseq = 1;
        c.i0 = i0;
        c.ntok = (d.Tq - i0 < per) ? d.Tq - i0 : per;
        SGQA_CHECK(fn(c));
      }
      b += 1;
    }
  }
  return SGQA_OK;
}

// Steps 2-3 of the forward, chunk by chunk, on either path.
sgqa_status select_chunked(const sgqa::Dims& d, const ForwardLayout& L, char* ws, int64_t chunk_tok,
                           const void* q_idx, const void* k_blk, int32_t* sel, hipStream_t s) {
  char* area = ws + L.off_chunk;
  if (!L.fused) {
    float* scores = reinterpret_cast<float*>(area);
    return for_each_chunk(d, chunk_tok, [&](const sgqa::Chunk& c) -> sgqa_status {
      hipError_t e = sgqa::launch_index(d, q_idx, k_blk, scores, c, s);
      if (e != hipSuccess) return hip_fail(e, "indexer launch");
      e = sgqa::launch_topk(d, scores, sel, c, s);
      if (e != hipSuccess) return hip_fail(e, "top-k launch");
      return SGQA_OK;
    });
  }
  const size_t t = static_cast<size_t>(chunk_tok);
  uint64_t* cand = reinterpret_cast<uint64_t*>(area);
  int32_t* cnt = reinterpret_cast<int32_t*>(area + align_up(t * L.cand_bytes));
  int32_t* fail_list = reinterpret_cast<int32_t*>(area + align_up(t * L.cand_bytes) +
                                                  align_up(t * L.cnt_bytes));
  int32_t* fail_count = reinterpret_cast<int32_t*>(ws + L.off_failcnt);
  float* scratch = reinterpret_cast<float*>(ws + L.off_scratch);
  return for_each_chunk(d, chunk_tok, [&](const sgqa::Chunk& c) -> sgqa_status {
    hipError_t e = sgqa::launch_index_filter(d, q_idx, k_blk, cand, cnt, fail_count, c, s);
    if (e != hipSuccess) return hip_fail(e, "index filter launch");
    e = sgqa::launch_select_candidates(d, cand, cnt, sel, fail_list, fail_count, c, true, s);
    if (e != hipSuccess) return hip_fail(e, "candidate select launch");
    e = sgqa::launch_select_fallback(d, q_idx, k_blk, fail_list, fail_count, scratch, sel, c, s);
    if (e != hipSuccess) return hip_fail(e, "select fallback launch");
    return SGQA_OK;
  });
}

// ---- decode over a paged cache ------------------------------------------------------------------
// Decode workspace layout.
//   candidate path : [attention workspace][internal sel][thr][cnt][fail list][fail count]
//                    [fallback scratch][cand]
//   score-row path : [scores][internal sel][attention workspace]
struct DecodeDerived {
  Derived dv;
  sgqa::PagedKV pk;
  size_t scores_bytes, sel_bytes, attend_bytes;
  bool fused;                                   // candidate-list selection (T_q * G <= 32)
  size_t rows_bytes, scratch_bytes, cand_bytes;  // candidate path: per-row arrays, fallback, lists
};

sgqa_status derive_cache(const sgqa_problem* prob, const sgqa_cache* cache, DecodeDerived* out) {
  SGQA_CHECK(derive(prob, &out->dv));
  sgqa::Dims& d = out->dv.d;
  if (!cache) return fail(SGQA_ERR_NULL, "cache descriptor is NULL");
  const int64_t P = cache->page_tokens;
  if (P < 8 || (P & (P - 1)) != 0 || P % d.B != 0)
    return fail(SGQA_ERR_SHAPE, "page_tokens must be a power of two, >= 8 and a multiple of block "
                "(got %lld, block %d)", (long long)P, d.B);
  if (cache->num_pages < 1 || cache->max_pages < 1)
    return fail(SGQA_ERR_SHAPE, "num_pages and max_pages must be >= 1");
  int64_t x;
  if (!mul_ok(cache->max_pages, P, &x) || x < d.Tk)
    return fail(SGQA_ERR_SHAPE, "max_pages * page_tokens (%lld) must cover t_kv (%lld)",
                (long long)x, (long long)d.Tk);
  if (!mul_ok(cache->num_pages, d.G, &x) || !mul_ok(x, P / 8, &x) || x >= (int64_t(1) << 32))
    return fail(SGQA_ERR_UNSUPPORTED, "num_pages * kv_groups * page_tokens / 8 must be < 2^32");
  if (!(d.bf16 && d.idx_bf16))
    return fail(SGQA_ERR_UNSUPPORTED, "the paged cache holds bf16 data (dtype and index_dtype)");
  if (d.B % 8 != 0)
    return fail(SGQA_ERR_UNSUPPORTED, "the paged cache needs block to be a multiple of 8 (got %d)", d.B);
  int l2 = 0;
  while ((int64_t(8) << l2) < P) ++l2;
  out->pk.k = out->pk.v = nullptr;
  out->pk.block_table = nullptr;
  out->pk.num_pages = cache->num_pages;
  out->pk.max_pages = cache->max_pages;
  out->pk.page_units_log2 = l2;
  d.kblk_stride = cache->max_pages * P / d.B;
  return SGQA_OK;
}

sgqa_status derive_decode(const sgqa_problem* prob, const sgqa_cache* cache, DecodeDerived* out) {
  SGQA_CHECK(derive_cache(prob, cache, out));
  const sgqa::Dims& d = out->dv.d;
  if (!sgqa::attend_split_supported(d))
    return fail(SGQA_ERR_UNSUPPORTED, "decode needs heads_per_group == 8, head_dim 64 or 128 and "
                "topk_tokens / block small enough for the grouped attention kernel");
  out->scores_bytes = out->dv.scores_bytes;
  out->sel_bytes = out->dv.sel_bytes;
  out->attend_bytes = sgqa::attend_split_bytes(d);
  out->fused = sgqa::decode_select_supported(d, d.Tq * d.G);
  const size_t rows = static_cast<size_t>(d.Bt * d.Tq * d.G);
  out->rows_bytes = rows * sizeof(int32_t);
  out->scratch_bytes = out->fused ? sgqa::select_fallback_scratch_bytes(d) : 0;
  out->cand_bytes = out->fused ? rows * sgqa::fused_select_capacity() * sizeof(uint64_t) : 0;
  return SGQA_OK;
}

size_t decode_workspace(const DecodeDerived& dd) {
  if (dd.fused)
    return align_up(dd.attend_bytes) + align_up(dd.sel_bytes) + 3 * align_up(dd.rows_bytes) + kAlign +
           align_up(dd.scratch_bytes) + align_up(dd.cand_bytes);
  return align_up(dd.scores_bytes) + align_up(dd.sel_bytes) + align_up(dd.attend_bytes);
}

}  // namespace

extern "C" {

int sgqa_abi_version(void) { return SGQA_ABI_VERSION; }

const char* sgqa_status_string(sgqa_status st) {
  switch (st) {
    case SGQA_OK: return "ok";
    case SGQA_ERR_NULL: return "null pointer";
    case SGQA_ERR_SHAPE: return "invalid shape";
    case SGQA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SGQA_ERR_ALIGN: return "misaligned pointer";
    case SGQA_ERR_WORKSPACE: return "workspace too small";
    case SGQA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* sgqa_last_error(void) { return g_last_error.c_str(); }

sgqa_status sgqa_sizes(const sgqa_problem* prob, sgqa_sizes_t* out) {
  Derived dv;
  SGQA_CHECK(derive(prob, &dv));
  if (!out) return fail(SGQA_ERR_NULL, "output sizes struct is NULL");
  out->num_blocks = dv.d.NB;
  out->n_sel = dv.d.NS;
  out->k_blk_bytes = dv.k_blk_bytes;
  out->scores_bytes = dv.scores_bytes;
  out->sel_bytes = dv.sel_bytes;
  out->attend_workspace_bytes = dv.attend_ws_bytes;
  out->forward_workspace_bytes = forward_default_bytes(dv);
  {
    const ForwardLayout L = forward_layout(dv);
    out->forward_workspace_min_bytes = L.fixed + chunk_bytes(L, 1);
  }
  return ok();
}

sgqa_status sgqa_index(const sgqa_problem* prob, const void* q_idx, const void* k_idx, void* k_blk,
                       float* scores, void* stream) {
  Derived dv;
  SGQA_CHECK(derive(prob, &dv));
  SGQA_CHECK(check_ptr(q_idx, "q_idx"));
  SGQA_CHECK(check_ptr(k_blk, "k_blk"));
  SGQA_CHECK(check_ptr(scores, "scores"));
  if (k_idx) SGQA_CHECK(check_ptr(k_idx, "k_idx"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (k_idx) {
    hipError_t e = sgqa::launch_compress(dv.d, k_idx, k_blk, s);
    if (e != hipSuccess) return hip_fail(e, "compress launch");
  }
  sgqa::Chunk c{0, dv.d.Bt, 0, dv.d.Tq};
  hipError_t e = sgqa::launch_index(dv.d, q_idx, k_blk, scores, c, s);
  if (e != hipSuccess) return hip_fail(e, "indexer launch");
  return ok();
}

sgqa_status sgqa_topk(const sgqa_problem* prob, const float* scores, int32_t* sel, void* stream) {
  Derived dv;
  SGQA_CHECK(derive(prob, &dv));
  SGQA_CHECK(check_ptr(scores, "scores"));
  SGQA_CHECK(check_ptr(sel, "sel"));
  sgqa::Chunk c{0, dv.d.Bt, 0, dv.d.Tq};
  hipError_t e = sgqa::launch_topk(dv.d, scores, sel, c, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return ok();
}

sgqa_status sgqa_attend(const sgqa_problem* prob, const void* q, const void* k, const void* v,
                        const void* gate, const int32_t* sel, void* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Derived dv;
  SGQA_CHECK(derive(prob, &dv));
  SGQA_CHECK(check_ptr(q, "q"));
  SGQA_CHECK(check_ptr(k, "k"));
  SGQA_CHECK(check_ptr(v, "v"));
  SGQA_CHECK(check_ptr(gate, "gate"));
  SGQA_CHECK(check_ptr(sel, "sel"));
  SGQA_CHECK(check_ptr(out, "out"));
  if (dv.attend_ws_bytes > 0) {
    SGQA_CHECK(check_ptr(workspace, "workspace"));
    if (workspace_bytes < dv.attend_ws_bytes)
      return fail(SGQA_ERR_WORKSPACE, "attend workspace needs %zu bytes (got %zu)",
                  dv.attend_ws_bytes, workspace_bytes);
  }
  hipError_t e = sgqa::launch_attend(dv.d, q, k, v, gate, sel, out, workspace,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

}  // extern "C"

namespace {

// sgqa_forward, and with lse_out != NULL its per-row log-sum-exp (range-split path only).
sgqa_status forward_impl(const sgqa_problem* prob, const void* q, const void* k, const void* v,
                         const void* gate, const void* q_idx, const void* k_idx, void* k_blk,
                         int32_t* sel_out, void* out, float* lse_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Derived dv;
  SGQA_CHECK(derive(prob, &dv));
  const sgqa::Dims& d = dv.d;
  if (lse_out) {
    SGQA_CHECK(check_ptr(lse_out, "lse_out", 4));
    if (!sgqa::attend_split_supported(d))
      return fail(SGQA_ERR_UNSUPPORTED,
                  "lse output needs the range-split attention (bf16, H = 8, D in {64, 128}, B a multiple of 8)");
  }
  SGQA_CHECK(check_ptr(q, "q"));
  SGQA_CHECK(check_ptr(k, "k"));
  SGQA_CHECK(check_ptr(v, "v"));
  SGQA_CHECK(check_ptr(gate, "gate"));
  SGQA_CHECK(check_ptr(q_idx, "q_idx"));
  SGQA_CHECK(check_ptr(k_blk, "k_blk"));
  SGQA_CHECK(check_ptr(out, "out"));
  if (k_idx) SGQA_CHECK(check_ptr(k_idx, "k_idx"));
  if (sel_out) SGQA_CHECK(check_ptr(sel_out, "sel_out"));
  SGQA_CHECK(check_ptr(workspace, "workspace"));
  const ForwardLayout L = forward_layout(dv);
  const int64_t chunk_tok = forward_chunk_tokens(dv, L, workspace_bytes);
  if (chunk_tok < 1)
    return fail(SGQA_ERR_WORKSPACE, "forward workspace needs at least %zu bytes (got %zu)",
                L.fixed + chunk_bytes(L, 1), workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  void* attend_ws = dv.attend_ws_bytes ? ws : nullptr;
  int32_t* sel = sel_out ? sel_out : reinterpret_cast<int32_t*>(ws + L.off_sel);

  hipStream_t s = static_cast<hipStream_t>(stream);
  SGQA_CHECK(mark_stage(0, s));
  if (k_idx) {
    hipError_t e = sgqa::launch_compress(d, k_idx, k_blk, s);
    if (e != hipSuccess) return hip_fail(e, "compress launch");
  }
  SGQA_CHECK(mark_stage(1, s));
  SGQA_CHECK(select_chunked(d, L, ws, chunk_tok, q_idx, k_blk, sel, s));
  SGQA_CHECK(mark_stage(2, s));
  hipError_t e = sgqa::launch_pack_kv(d, k, v, attend_ws, s);
  if (e != hipSuccess) return hip_fail(e, "k/v packing launch");
  SGQA_CHECK(mark_stage(3, s));
  e = sgqa::launch_attend_packed(d, q, k, v, gate, sel, out, attend_ws, s,
                                 g_stage_armed ? mark_stage_hip : nullptr, lse_out);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  SGQA_CHECK(mark_stage(6, s));
  return ok();
}

}  // namespace

extern "C" {

sgqa_status sgqa_forward(const sgqa_problem* prob, const void* q, const void* k, const void* v,
                         const void* gate, const void* q_idx, const void* k_idx, void* k_blk,
                         int32_t* sel_out, void* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return forward_impl(prob, q, k, v, gate, q_idx, k_idx, k_blk, sel_out, out, nullptr, workspace,
                      workspace_bytes, stream);
}

sgqa_status sgqa_forward_with_lse(const sgqa_problem* prob, const void* q, const void* k,
                                  const void* v, const void* gate, const void* q_idx,
                                  const void* k_idx, void* k_blk, int32_t* sel_out, void* out,
                                  float* lse_out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (!lse_out) return fail(SGQA_ERR_NULL, "lse_out is NULL");
  return forward_impl(prob, q, k, v, gate, q_idx, k_idx, k_blk, sel_out, out, lse_out, workspace,
                      workspace_bytes, stream);
}

sgqa_status sgqa_cache_append(const sgqa_problem* prob, const sgqa_cache* cache,
                              const int32_t* seq_lens, const int32_t* block_table, int64_t n_new,
                              const void* k_new, const void* v_new, const void* kidx_new,
                              void* k_cache, void* v_cache, void* kidx_cache, void* k_blk,
                              void* stream) {
  DecodeDerived dd;
  SGQA_CHECK(derive_cache(prob, cache, &dd));
  sgqa::Dims d = dd.dv.d;
  if (n_new < 1 || n_new > d.Tk)
    return fail(SGQA_ERR_SHAPE, "n_new must be in [1, t_kv] (got %lld)", (long long)n_new);
  SGQA_CHECK(check_ptr(seq_lens, "seq_lens", 4));
  SGQA_CHECK(check_ptr(block_table, "block_table", 4));
  SGQA_CHECK(check_ptr(k_new, "k_new"));
  SGQA_CHECK(check_ptr(v_new, "v_new"));
  SGQA_CHECK(check_ptr(kidx_new, "kidx_new"));
  SGQA_CHECK(check_ptr(k_cache, "k_cache"));
  SGQA_CHECK(check_ptr(v_cache, "v_cache"));
  SGQA_CHECK(check_ptr(kidx_cache, "kidx_cache"));
  SGQA_CHECK(check_ptr(k_blk, "k_blk"));
  d.seq_len = seq_lens;
  sgqa::PagedKV pk = dd.pk;
  pk.k = k_cache;
  pk.v = v_cache;
  pk.block_table = block_table;
  hipError_t e = sgqa::launch_cache_append(d, pk, n_new, k_new, v_new, kidx_new, kidx_cache, k_blk,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cache append launch");
  return ok();
}

sgqa_status sgqa_decode_workspace_size(const sgqa_problem* prob, const sgqa_cache* cache,
                                       size_t* bytes) {
  DecodeDerived dd;
  SGQA_CHECK(derive_decode(prob, cache, &dd));
  if (!bytes) return fail(SGQA_ERR_NULL, "bytes is NULL");
  *bytes = decode_workspace(dd);
  return ok();
}

namespace {

sgqa_status check_decode_ptrs(const int32_t* seq_lens, const int32_t* block_table, const void* q,
                              const void* gate, const void* q_idx, const void* k_cache,
                              const void* v_cache, const void* k_blk, const int32_t* sel_out,
                              const void* out) {
  SGQA_CHECK(check_ptr(seq_lens, "seq_lens", 4));
  SGQA_CHECK(check_ptr(block_table, "block_table", 4));
  SGQA_CHECK(check_ptr(q, "q"));
  SGQA_CHECK(check_ptr(gate, "gate"));
  SGQA_CHECK(check_ptr(q_idx, "q_idx"));
  SGQA_CHECK(check_ptr(k_cache, "k_cache"));
  SGQA_CHECK(check_ptr(v_cache, "v_cache"));
  SGQA_CHECK(check_ptr(k_blk, "k_blk"));
  SGQA_CHECK(check_ptr(out, "out"));
  if (sel_out) SGQA_CHECK(check_ptr(sel_out, "sel_out"));
  return SGQA_OK;
}

constexpr size_t kNoAllocScratchBytes = SGQA_DECODE_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes % 256 == 0, "scratch size");
constexpr int kMaxDevices = 64;

}  // namespace

// Scratch of sgqa_decode_noalloc: device memory of fixed size in this module, one copy per GPU
// (allocated by the runtime when the module loads on that GPU and held until the process ends).
// In host code `scratch` only names the symbol; its device address on each GPU comes from
// hipGetSymbolAddress, looked up once per device with that device current and kept below.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device `stream` belongs to.
sgqa_status scratch_on_stream_device(hipStream_t stream, void** ptr) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SGQA_ERR_UNSUPPORTED, "device %d is outside the %d devices the scratch table holds",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur) {
      e = hipSetDevice(dev);
      if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) return hip_fail(e2, "hipSetDevice");
    }
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SGQA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SGQA_OK;
}

}  // namespace

sgqa_status sgqa_decode(const sgqa_problem* prob, const sgqa_cache* cache,
                        const int32_t* seq_lens, const int32_t* block_table, const void* q,
                        const void* gate, const void* q_idx, const void* k_cache,
                        const void* v_cache, const void* k_blk, int32_t* sel_out, void* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  DecodeDerived dd;
  SGQA_CHECK(derive_decode(prob, cache, &dd));
  SGQA_CHECK(check_decode_ptrs(seq_lens, block_table, q, gate, q_idx, k_cache, v_cache, k_blk,
                               sel_out, out));
  SGQA_CHECK(check_ptr(workspace, "workspace"));
  const size_t need = decode_workspace(dd);
  if (workspace_bytes < need)
    return fail(SGQA_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu)", need,
                workspace_bytes);
  sgqa::Dims d = dd.dv.d;
  d.seq_len = seq_lens;
  sgqa::PagedKV pk = dd.pk;
  pk.k = k_cache;
  pk.v = v_cache;
  pk.block_table = block_table;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const sgqa::Chunk c{0, d.Bt, 0, d.Tq};
  int32_t* sel;
  void* attend_ws;
  hipError_t e;
  if (dd.fused) {
    size_t off = 0;
    attend_ws = ws;
    off += align_up(dd.attend_bytes);
    sel = sel_out ? sel_out : reinterpret_cast<int32_t*>(ws + off);
    off += align_up(dd.sel_bytes);
    uint32_t* thr = reinterpret_cast<uint32_t*>(ws + off);
    off += align_up(dd.rows_bytes);
    int32_t* cnt = reinterpret_cast<int32_t*>(ws + off);
    off += align_up(dd.rows_bytes);
    int32_t* fail_list = reinterpret_cast<int32_t*>(ws + off);
    off += align_up(dd.rows_bytes);
    int32_t* fail_count = reinterpret_cast<int32_t*>(ws + off);
    off += kAlign;
    float* scratch = reinterpret_cast<float*>(ws + off);
    off += align_up(dd.scratch_bytes);
    uint64_t* cand = reinterpret_cast<uint64_t*>(ws + off);
    SGQA_CHECK(mark_stage(0, s));
    e = sgqa::launch_decode_select(d, q_idx, k_blk, thr, cand, cnt, fail_count, c, s);
    if (e != hipSuccess) return hip_fail(e, "decode filter launch");
    SGQA_CHECK(mark_stage(1, s));
    e = sgqa::launch_select_candidates(d, cand, cnt, sel, fail_list, fail_count, c, false, s);
    if (e != hipSuccess) return hip_fail(e, "candidate select launch");
    e = sgqa::launch_select_fallback(d, q_idx, k_blk, fail_list, fail_count, scratch, sel, c, s);
    if (e != hipSuccess) return hip_fail(e, "select fallback launch");
  } else {
    float* scores = reinterpret_cast<float*>(ws);
    sel = sel_out ? sel_out : reinterpret_cast<int32_t*>(ws + align_up(dd.scores_bytes));
    attend_ws = ws + align_up(dd.scores_bytes) + align_up(dd.sel_bytes);
    SGQA_CHECK(mark_stage(0, s));
    e = sgqa::launch_index(d, q_idx, k_blk, scores, c, s);
    if (e != hipSuccess) return hip_fail(e, "indexer launch");
    SGQA_CHECK(mark_stage(1, s));
    e = sgqa::launch_topk(d, scores, sel, c, s);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
  }
  SGQA_CHECK(mark_stage(2, s));
  SGQA_CHECK(mark_stage(3, s));
  e = sgqa::launch_attend_split(d, q, nullptr, gate, sel, out, nullptr, attend_ws, s,
                                g_stage_armed ? mark_stage_hip : nullptr, &pk);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  SGQA_CHECK(mark_stage(6, s));
  return ok();
}

sgqa_status sgqa_decode_noalloc(const sgqa_problem* prob, const sgqa_cache* cache,
                                const int32_t* seq_lens, const int32_t* block_table, const void* q,
                                const void* gate, const void* q_idx, const void* k_cache,
                                const void* v_cache, const void* k_blk, int32_t* sel_out,
                                void* out, void* stream) {
  DecodeDerived dd;
  SGQA_CHECK(derive_decode(prob, cache, &dd));
  SGQA_CHECK(check_decode_ptrs(seq_lens, block_table, q, gate, q_idx, k_cache, v_cache, k_blk,
                               sel_out, out));
  const size_t need = decode_workspace(dd);
  if (need > kNoAllocScratchBytes)
    return fail(SGQA_ERR_WORKSPACE, "decode needs %zu bytes of scratch; sgqa_decode_noalloc holds "
                "%zu (use sgqa_decode with a workspace)", need, kNoAllocScratchBytes);
  void* ws = nullptr;
  SGQA_CHECK(scratch_on_stream_device(static_cast<hipStream_t>(stream), &ws));
  return sgqa_decode(prob, cache, seq_lens, block_table, q, gate, q_idx, k_cache, v_cache, k_blk,
                     sel_out, out, ws, kNoAllocScratchBytes, stream);
}

sgqa_status derive_swa(const sgqa_problem* prob, int64_t window, Derived* dv, int64_t* w_eff,
                       size_t* bytes) {
  SGQA_CHECK(derive(prob, dv));
  if (window < 1) return fail(SGQA_ERR_SHAPE, "window must be >= 1 (got %lld)", (long long)window);
  if (!sgqa::attend_window_supported(dv->d))
    return fail(SGQA_ERR_UNSUPPORTED, "sliding-window attention needs bf16, heads_per_group == 8 "
                "and head_dim 64 or 128");
  *w_eff = window < dv->d.Tk ? window : dv->d.Tk;      // a window past the context is the context
  *bytes = align_up(sgqa::packed_kv_quad_bytes(dv->d)) + sgqa::attend_window_bytes(dv->d, *w_eff);
  return SGQA_OK;
}

sgqa_status sgqa_swa_workspace_size(const sgqa_problem* prob, int64_t window, size_t* bytes) {
  Derived dv;
  int64_t w;
  size_t need;
  SGQA_CHECK(derive_swa(prob, window, &dv, &w, &need));
  if (!bytes) return fail(SGQA_ERR_NULL, "bytes is NULL");
  *bytes = need;
  return ok();
}

sgqa_status sgqa_swa(const sgqa_problem* prob, int64_t window, const void* q, const void* k,
                     const void* v, const void* gate, void* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  Derived dv;
  int64_t w;
  size_t need;
  SGQA_CHECK(derive_swa(prob, window, &dv, &w, &need));
  SGQA_CHECK(check_ptr(q, "q"));
  SGQA_CHECK(check_ptr(k, "k"));
  SGQA_CHECK(check_ptr(v, "v"));
  SGQA_CHECK(check_ptr(gate, "gate"));
  SGQA_CHECK(check_ptr(out, "out"));
  SGQA_CHECK(check_ptr(workspace, "workspace"));
  if (workspace_bytes < need)
    return fail(SGQA_ERR_WORKSPACE, "sliding-window workspace needs %zu bytes (got %zu)", need,
                workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const size_t pkv = sgqa::packed_kv_quad_bytes(dv.d);
  hipError_t e = sgqa::launch_pack_kv_quad(dv.d, k, v, ws, s);
  if (e != hipSuccess) return hip_fail(e, "k/v packing launch");
  e = sgqa::launch_attend_window(dv.d, w, q, ws, gate, out, ws + pkv / 2, ws + align_up(pkv), s);
  if (e != hipSuccess) return hip_fail(e, "sliding-window attention launch");
  return ok();
}

sgqa_status sgqa_forward_fp8kv(const sgqa_problem* prob, const void* q, const void* k8,
                               const void* v8, float k_scale, float v_scale, const void* gate,
                               const void* q_idx, const void* k_idx, void* k_blk, int32_t* sel_out,
                               void* out, void* workspace, size_t workspace_bytes, void* stream) {
  Derived dv;
  SGQA_CHECK(derive(prob, &dv));
  const sgqa::Dims& d = dv.d;
  if (!sgqa::attend_split_supported(d))
    return fail(SGQA_ERR_UNSUPPORTED, "fp8 K/V needs bf16 q/gate/out, heads_per_group == 8, head_dim "
                "64 or 128, block a multiple of 8 and topk_tokens / block within the grouped kernel");
  if (!(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(SGQA_ERR_SHAPE, "k_scale and v_scale must be finite and > 0");
  SGQA_CHECK(check_ptr(q, "q"));
  SGQA_CHECK(check_ptr(k8, "k"));
  SGQA_CHECK(check_ptr(v8, "v"));
  SGQA_CHECK(check_ptr(gate, "gate"));
  SGQA_CHECK(check_ptr(q_idx, "q_idx"));
  SGQA_CHECK(check_ptr(k_blk, "k_blk"));
  SGQA_CHECK(check_ptr(out, "out"));
  if (k_idx) SGQA_CHECK(check_ptr(k_idx, "k_idx"));
  if (sel_out) SGQA_CHECK(check_ptr(sel_out, "sel_out"));
  SGQA_CHECK(check_ptr(workspace, "workspace"));
  const ForwardLayout L = forward_layout(dv);
  const int64_t chunk_tok = forward_chunk_tokens(dv, L, workspace_bytes);
  if (chunk_tok < 1)
    return fail(SGQA_ERR_WORKSPACE, "forward workspace needs at least %zu bytes (got %zu)",
                L.fixed + chunk_bytes(L, 1), workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  int32_t* sel = sel_out ? sel_out : reinterpret_cast<int32_t*>(ws + L.off_sel);
  hipStream_t s = static_cast<hipStream_t>(stream);
  SGQA_CHECK(mark_stage(0, s));
  if (k_idx) {
    hipError_t e = sgqa::launch_compress(d, k_idx, k_blk, s);
    if (e != hipSuccess) return hip_fail(e, "compress launch");
  }
  SGQA_CHECK(mark_stage(1, s));
  SGQA_CHECK(select_chunked(d, L, ws, chunk_tok, q_idx, k_blk, sel, s));
  SGQA_CHECK(mark_stage(2, s));
  // the fp8 copies fit in the space of the bf16 ones; the range lists follow that space
  hipError_t e = sgqa::launch_pack_kv_fp8(d, k8, v8, ws, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 k/v packing launch");
  SGQA_CHECK(mark_stage(3, s));
  const sgqa::Fp8Scales sc{k_scale, v_scale};
  e = sgqa::launch_attend_split(d, q, ws, gate, sel, out, ws + sgqa::packed_kv_fp8_bytes(d) / 2,
                                ws + sgqa::attend_packed_kv_bytes(d), s,
                                g_stage_armed ? mark_stage_hip : nullptr, nullptr, &sc);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  SGQA_CHECK(mark_stage(6, s));
  return ok();
}

sgqa_status derive_backward(const sgqa_problem* prob, Derived* dv, size_t* bytes) {
  SGQA_CHECK(derive(prob, dv));
  if (!sgqa::attend_split_supported(dv->d))
    return fail(SGQA_ERR_UNSUPPORTED, "the backward needs bf16, heads_per_group == 8, head_dim 64 or "
                "128, block a multiple of 8 and topk_tokens / block within the grouped kernel");
  *bytes = sgqa::attend_backward_bytes(dv->d);
  return SGQA_OK;
}

sgqa_status sgqa_attend_backward_workspace_size(const sgqa_problem* prob, size_t* bytes) {
  Derived dv;
  size_t need;
  SGQA_CHECK(derive_backward(prob, &dv, &need));
  if (!bytes) return fail(SGQA_ERR_NULL, "bytes is NULL");
  *bytes = need;
  return ok();
}

sgqa_status sgqa_attend_backward(const sgqa_problem* prob, const void* q, const void* k,
                                 const void* v, const void* gate, const int32_t* sel,
                                 const void* dout, void* dq, float* dk, float* dv, void* dgate,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  Derived d;
  size_t need;
  SGQA_CHECK(derive_backward(prob, &d, &need));
  SGQA_CHECK(check_ptr(q, "q"));
  SGQA_CHECK(check_ptr(k, "k"));
  SGQA_CHECK(check_ptr(v, "v"));
  SGQA_CHECK(check_ptr(gate, "gate"));
  SGQA_CHECK(check_ptr(sel, "sel"));
  SGQA_CHECK(check_ptr(dout, "dout"));
  SGQA_CHECK(check_ptr(dq, "dq"));
  SGQA_CHECK(check_ptr(dk, "dk"));
  SGQA_CHECK(check_ptr(dv, "dv"));
  SGQA_CHECK(check_ptr(dgate, "dgate"));
  SGQA_CHECK(check_ptr(workspace, "workspace"));
  if (workspace_bytes < need)
    return fail(SGQA_ERR_WORKSPACE, "backward workspace needs %zu bytes (got %zu)", need,
                workspace_bytes);
  hipError_t e = sgqa::launch_attend_backward(d.d, q, k, v, gate, sel, dout, dq, dk, dv, dgate,
                                              workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention backward launch");
  return ok();
}

sgqa_status sgqa_attend_backward_with_lse(const sgqa_problem* prob, const void* q, const void* k,
                                          const void* v, const void* gate, const int32_t* sel,
                                          const void* out, const float* lse, const void* dout,
                                          void* dq, float* dk, float* dv, void* dgate,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  Derived d;
  size_t need;
  SGQA_CHECK(derive_backward(prob, &d, &need));
  SGQA_CHECK(check_ptr(q, "q"));
  SGQA_CHECK(check_ptr(k, "k"));
  SGQA_CHECK(check_ptr(v, "v"));
  SGQA_CHECK(check_ptr(gate, "gate"));
  SGQA_CHECK(check_ptr(sel, "sel"));
  SGQA_CHECK(check_ptr(out, "out"));
  SGQA_CHECK(check_ptr(lse, "lse", 4));
  SGQA_CHECK(check_ptr(dout, "dout"));
  SGQA_CHECK(check_ptr(dq, "dq"));
  SGQA_CHECK(check_ptr(dk, "dk"));
  SGQA_CHECK(check_ptr(dv, "dv"));
  SGQA_CHECK(check_ptr(dgate, "dgate"));
  SGQA_CHECK(check_ptr(workspace, "workspace"));
  if (workspace_bytes < need)
    return fail(SGQA_ERR_WORKSPACE, "backward workspace needs %zu bytes (got %zu)", need,
                workspace_bytes);
  hipError_t e = sgqa::launch_attend_backward(d.d, q, k, v, gate, sel, dout, dq, dk, dv, dgate,
                                              workspace, static_cast<hipStream_t>(stream), out, lse);
  if (e != hipSuccess) return hip_fail(e, "attention backward launch");
  return ok();
}

sgqa_status sgqa_set_stage_events(void* const* events) {
  if (!events) {
    g_stage_armed = false;
    return ok();
  }
  for (int i = 0; i < SGQA_STAGE_EVENTS; ++i) {
    if (!events[i]) {
      g_stage_armed = false;
      return fail(SGQA_ERR_NULL, "stage event %d is NULL", i);
    }
  }
  for (int i = 0; i < SGQA_STAGE_EVENTS; ++i) g_stage_events[i] = static_cast<hipEvent_t>(events[i]);
  g_stage_armed = true;
  return ok();
}

}  // extern "C"
