// C ABI of the Sparse GQA forward path: argument validation, sizes, workspace carving, row
// chunking and kernel dispatch.  Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/sgqa.h"
#include "sgqa_internal.h"

namespace {

thread_local std::string g_last_error;

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

// Query-token rectangle a fixed score budget holds in the forward workspace.
constexpr size_t kForwardScoreBudget = size_t(4) << 30;   // 4 GiB of fp32 scores per chunk

struct Derived {
  sgqa::Dims d;
  size_t k_blk_bytes, scores_bytes, sel_bytes, packed_v_bytes;
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
  out->packed_v_bytes = sgqa::attend_packed_v_bytes(d);
  out->score_row_bytes = static_cast<size_t>(d.G) * static_cast<size_t>(d.NB) * 4;
  return SGQA_OK;
}

bool attend_block_ok(const sgqa::Dims& d) { return (d.B % 8 == 0) || (8 % d.B == 0); }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Forward workspace: [packed v][internal sel][score chunk]; the chunk holds `chunk_tok` tokens.
size_t forward_fixed_bytes(const Derived& dv) {
  return align_up(dv.packed_v_bytes) + align_up(dv.sel_bytes);
}

size_t forward_default_bytes(const Derived& dv) {
  const size_t tokens = static_cast<size_t>(dv.d.Bt * dv.d.Tq);
  size_t chunk = kForwardScoreBudget / dv.score_row_bytes;
  if (chunk < 1) chunk = 1;
  if (chunk > tokens) chunk = tokens;
  return forward_fixed_bytes(dv) + align_up(chunk * dv.score_row_bytes);
}

sgqa_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(SGQA_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(SGQA_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return SGQA_OK;
}

#define SGQA_CHECK(expr)                \
  do {                                  \
    sgqa_status _st = (expr);           \
    if (_st != SGQA_OK) return _st;     \
  } while (0)

// Index + top-k over query-token rectangles of at most `chunk_tok` tokens.
sgqa_status index_topk_chunked(const sgqa::Dims& d, const void* q_idx, const void* k_blk,
                               float* scores, int32_t* sel, int64_t chunk_tok, hipStream_t s) {
  for (int64_t b = 0; b < d.Bt;) {
    sgqa::Chunk c;
    if (chunk_tok >= d.Tq) {
      c.b0 = b;
      c.nseq = chunk_tok / d.Tq;
      if (c.nseq > d.Bt - b) c.nseq = d.Bt - b;
      c.i0 = 0;
      c.ntok = d.Tq;
      hipError_t e = sgqa::launch_index(d, q_idx, k_blk, scores, c, s);
      if (e != hipSuccess) return hip_fail(e, "indexer launch");
      e = sgqa::launch_topk(d, scores, sel, c, s);
      if (e != hipSuccess) return hip_fail(e, "top-k launch");
      b += c.nseq;
    } else {
      for (int64_t i0 = 0; i0 < d.Tq; i0 += chunk_tok) {
        c.b0 = b;
        c.nseq = 1;
        c.i0 = i0;
        c.ntok = (d.Tq - i0 < chunk_tok) ? d.Tq - i0 : chunk_tok;
        hipError_t e = sgqa::launch_index(d, q_idx, k_blk, scores, c, s);
        if (e != hipSuccess) return hip_fail(e, "indexer launch");
        e = sgqa::launch_topk(d, scores, sel, c, s);
        if (e != hipSuccess) return hip_fail(e, "top-k launch");
      }
      b += 1;
    }
  }
  return SGQA_OK;
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
  out->attend_workspace_bytes = dv.packed_v_bytes;
  out->forward_workspace_bytes = forward_default_bytes(dv);
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
  if (!attend_block_ok(dv.d))
    return fail(SGQA_ERR_UNSUPPORTED, "attention needs block dividing 8 or a multiple of 8 (got %d)",
                dv.d.B);
  SGQA_CHECK(check_ptr(q, "q"));
  SGQA_CHECK(check_ptr(k, "k"));
  SGQA_CHECK(check_ptr(v, "v"));
  SGQA_CHECK(check_ptr(gate, "gate"));
  SGQA_CHECK(check_ptr(sel, "sel"));
  SGQA_CHECK(check_ptr(out, "out"));
  if (dv.packed_v_bytes > 0) {
    SGQA_CHECK(check_ptr(workspace, "workspace"));
    if (workspace_bytes < dv.packed_v_bytes)
      return fail(SGQA_ERR_WORKSPACE, "attend workspace needs %zu bytes (got %zu)",
                  dv.packed_v_bytes, workspace_bytes);
  }
  hipError_t e = sgqa::launch_attend(dv.d, q, k, v, gate, sel, out, workspace,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

sgqa_status sgqa_forward(const sgqa_problem* prob, const void* q, const void* k, const void* v,
                         const void* gate, const void* q_idx, const void* k_idx, void* k_blk,
                         int32_t* sel_out, void* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  Derived dv;
  SGQA_CHECK(derive(prob, &dv));
  const sgqa::Dims& d = dv.d;
  if (!attend_block_ok(d))
    return fail(SGQA_ERR_UNSUPPORTED, "attention needs block dividing 8 or a multiple of 8 (got %d)",
                d.B);
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
  const size_t fixed = forward_fixed_bytes(dv);
  if (workspace_bytes < fixed + dv.score_row_bytes)
    return fail(SGQA_ERR_WORKSPACE, "forward workspace needs at least %zu bytes (got %zu)",
                fixed + dv.score_row_bytes, workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  void* packed_v = dv.packed_v_bytes ? ws : nullptr;
  int32_t* sel = sel_out ? sel_out : reinterpret_cast<int32_t*>(ws + align_up(dv.packed_v_bytes));
  float* scores = reinterpret_cast<float*>(ws + fixed);
  int64_t chunk_tok = static_cast<int64_t>((workspace_bytes - fixed) / dv.score_row_bytes);
  if (chunk_tok > d.Bt * d.Tq) chunk_tok = d.Bt * d.Tq;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (k_idx) {
    hipError_t e = sgqa::launch_compress(d, k_idx, k_blk, s);
    if (e != hipSuccess) return hip_fail(e, "compress launch");
  }
  SGQA_CHECK(index_topk_chunked(d, q_idx, k_blk, scores, sel, chunk_tok, s));
  hipError_t e = sgqa::launch_attend(d, q, k, v, gate, sel, out, packed_v, s);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

}  // extern "C"
