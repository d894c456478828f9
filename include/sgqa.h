/*
 * sgqa.h -- C ABI of the MI355X (gfx950) Sparse GQA forward path.
 *
 * Sparse GQA is the full-context attention layer of Step 5 Preview (Step 5 Preview summary on
 * mo.ai.kr, section "모델 구조와 학습 안정성"; ai.info article, section "Sparse GQA punta a un
 * contesto di 1 milione di token").  Per (query token, KV group) it
 *   1. compresses the shared index keys into blocks of B tokens          (sgqa_index, k_idx != NULL)
 *   2. scores the query's index vector against every causal past block   (sgqa_index)
 *   3. keeps the top k/B blocks independently for each KV group          (sgqa_topk)
 *   4. runs sigmoid-gated grouped-query attention over only those tokens (sgqa_attend)
 * and sgqa_forward chains the four steps.
 *
 * Readings fixed where the pages are silent: a block key is the SUM of its B index keys; the score
 * is the raw dot product; the query's own block o = p / B is always selected, counts toward the
 * k/B budget and is causally masked inside (tokens t <= p); among past blocks higher scores win
 * and equal scores go to the lower block index; when o + 1 <= k/B every causal block is taken;
 * out = sigmoid(gate) * attention, elementwise; the softmax scale is an argument; query head j of
 * group g attends with group g's keys and values; the t_q queries are the last t_q positions of
 * the key stream, p = t_kv - t_q + i.
 *
 * Conventions (every call):
 *   - Every tensor pointer is a DEVICE pointer (hipMalloc / torch CUDA memory) of the current
 *     device, contiguous row-major in the layout stated below, aligned to 16 bytes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is enqueued
 *     asynchronously on it; results are valid once the stream has been synchronised.
 *   - The caller owns every buffer, workspaces included; the library allocates no device memory,
 *     keeps no state between calls (apart from the optional stage markers armed by
 *     sgqa_set_stage_events, and the fixed per-GPU scratch of sgqa_decode_noalloc, part of the
 *     library's code object) and never synchronises.  Inputs are read-only; outputs must not
 *     alias inputs.  Concurrent calls need distinct outputs and workspaces.
 *   - Arguments are validated on the host before anything is enqueued.  On any error the call
 *     returns a non-zero sgqa_status, enqueues nothing and touches no output; sgqa_last_error()
 *     then gives a human-readable detail (thread-local).  A failed launch returns SGQA_ERR_HIP.
 *     Nothing aborts the process or throws across this boundary.
 *   - NaN / Inf inputs are not detected and give unspecified results.
 *
 * Layouts (Bt = batch, Tq = t_q, Tk = t_kv, G = kv_groups, H = heads_per_group, D = head_dim,
 * Di = index_dim, NB = ceil(Tk / B), NS = topk_tokens / B):
 *   q, gate, out : [Bt, Tq, G, H, D]      dtype
 *   k, v         : [Bt, G, Tk, D]         dtype
 *   q_idx        : [Bt, Tq, G, Di]        index_dtype   (index query per token and KV group)
 *   k_idx        : [Bt, Tk, Di]           index_dtype   (index key per token, shared by all groups)
 *   k_blk        : [Bt, NB, Di]           index_dtype   (block keys; rounded to index_dtype)
 *   scores       : [Bt, Tq, G, NB]        float32       (entry j valid for j < p / B only)
 *   sel          : [Bt, Tq, G, NS]        int32         (selected blocks ascending, -1 padded)
 */
#ifndef SGQA_H_
#define SGQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGQA_ABI_VERSION 2

typedef enum {
  SGQA_OK = 0,
  SGQA_ERR_NULL = 1,         /* a required pointer is NULL                                   */
  SGQA_ERR_SHAPE = 2,        /* an inconsistent or out-of-range size                          */
  SGQA_ERR_UNSUPPORTED = 3,  /* valid, but outside what the kernels implement                 */
  SGQA_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned                              */
  SGQA_ERR_WORKSPACE = 5,    /* workspace missing or smaller than sgqa_sizes() asks for        */
  SGQA_ERR_HIP = 6           /* the HIP runtime reported an error (detail in sgqa_last_error) */
} sgqa_status;

typedef enum { SGQA_F32 = 0, SGQA_BF16 = 1 } sgqa_dtype;

/* Problem descriptor; passed by const pointer, never retained. */
typedef struct {
  int64_t batch;            /* Bt >= 1                                                   */
  int64_t t_q;              /* 1 <= t_q <= t_kv                                          */
  int64_t t_kv;             /* >= 1                                                      */
  int32_t kv_groups;        /* G >= 1                                                    */
  int32_t heads_per_group;  /* H >= 1 (query heads of KV group g are g*H .. g*H+H-1)      */
  int32_t head_dim;         /* D in {64, 128}                                            */
  int32_t index_dim;        /* Di in {32, 64, 128}                                        */
  int32_t block;            /* B >= 1                                                    */
  int32_t topk_tokens;      /* k >= B, k % B == 0; NS = k / B <= 4096                     */
  float softmax_scale;      /* > 0, finite (1/sqrt(D) in the usual setting)               */
  int32_t dtype;            /* sgqa_dtype of q, k, v, gate, out                          */
  int32_t index_dtype;      /* sgqa_dtype of q_idx, k_idx, k_blk                         */
} sgqa_problem;

/* Derived sizes (bytes unless stated). */
typedef struct {
  int64_t num_blocks;               /* NB                                                  */
  int64_t n_sel;                    /* NS                                                  */
  size_t k_blk_bytes;               /* k_blk buffer                                        */
  size_t scores_bytes;              /* scores buffer for sgqa_index / sgqa_topk            */
  size_t sel_bytes;                 /* sel buffer                                          */
  size_t attend_workspace_bytes;    /* workspace sgqa_attend needs                         */
  size_t forward_workspace_bytes;   /* workspace for sgqa_forward with the default chunking */
  size_t forward_workspace_min_bytes; /* smallest workspace sgqa_forward accepts (one query
                                         token per chunk); any size in between also works   */
} sgqa_sizes_t;

/* ABI version of the loaded library (SGQA_ABI_VERSION when it matches this header). */
int sgqa_abi_version(void);

/* Static text for a status code. */
const char* sgqa_status_string(sgqa_status status);

/* Detail of the last error on the calling thread ("" after a successful call). */
const char* sgqa_last_error(void);

/* Validate `prob` and fill `out` with the derived sizes.  Host only; touches no device. */
sgqa_status sgqa_sizes(const sgqa_problem* prob, sgqa_sizes_t* out);

/*
 * Steps 1-2: block compression and the indexer.  The pages compress the shared index keys block by
 * block and score them with an indexer per KV group (mo.ai.kr summary, section "모델 구조와 학습
 * 안정성"; ai.info article, section "Sparse GQA punta a un contesto di 1 milione di token": blocks of
 * eight tokens, which cut indexer and top-k cost eightfold).
 *   k_idx  : [Bt, Tk, Di] or NULL.  If non-NULL, k_blk is first written as the block sums of k_idx
 *            (fp32 accumulation, rounded to index_dtype).  If NULL, k_blk is an INPUT holding block
 *            keys computed earlier (a decode cache).
 *   k_blk  : [Bt, NB, Di]
 *   q_idx  : [Bt, Tq, G, Di]
 *   scores : [Bt, Tq, G, NB] float32; scores[b,i,g,j] = q_idx[b,i,g,:] . k_blk[b,j,:] for every
 *            j < p_i / B (p_i = Tk - Tq + i), accumulated in fp32.  Entries j >= p_i / B are left
 *            untouched.  Integer-valued index data with |score| < 2^24 gives exact scores.
 */
sgqa_status sgqa_index(const sgqa_problem* prob, const void* q_idx, const void* k_idx,
                       void* k_blk, float* scores, void* stream);

/*
 * Step 3: per-(query, KV group) block selection from stored scores.  Each KV group keeps its own
 * top blocks; k = 4096 tokens is 512 blocks of 8 (mo.ai.kr summary and ai.info article, sections as
 * above).
 *   scores : [Bt, Tq, G, NB] float32 as written by sgqa_index (only j < p/B is read).
 *   sel    : [Bt, Tq, G, NS] int32.  With o = p / B: if o + 1 <= NS, sel = 0..o then -1s;
 *            otherwise sel = {o} plus the NS-1 candidates j < o with the largest scores, equal
 *            scores going to the lower j, listed ascending.  -0.0 and +0.0 are equal scores.
 */
sgqa_status sgqa_topk(const sgqa_problem* prob, const float* scores, int32_t* sel, void* stream);

/*
 * Step 4: gated grouped-query attention over the selected tokens.  The full-attention layers are
 * Sparse GQA built on Gated GQA, each KV group attending to its own selected blocks (mo.ai.kr
 * summary, section "모델 구조와 학습 안정성").
 *   q, gate : [Bt, Tq, G, H, D];  k, v : [Bt, G, Tk, D];  sel : [Bt, Tq, G, NS] (as sgqa_topk).
 *   out     : [Bt, Tq, G, H, D]; for head j of group g, query i at p = Tk - Tq + i:
 *             out = sigmoid(gate) * sum_t softmax_t(scale * q . k_t) v_t over the tokens t <= p
 *             of the selected blocks.  fp32 accumulation; bf16 outputs are rounded to nearest even.
 *   workspace: >= sizes.attend_workspace_bytes of device memory (a block-packed copy of v).
 *   Any B >= 1: blocks that are a multiple of 8 or divide 8 run on the matrix-core kernels;
 *   other block sizes run on the plain kernel (one workgroup per (query, group), every selected
 *   token in turn; much slower, same result up to rounding).
 */
sgqa_status sgqa_attend(const sgqa_problem* prob, const void* q, const void* k, const void* v,
                        const void* gate, const int32_t* sel, void* out, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Steps 1-4 in one call (the pages' Sparse GQA layer: mo.ai.kr summary, section "모델 구조와
 * 학습 안정성").
 *   k_idx   : as in sgqa_index (NULL = k_blk already holds the block keys).
 *   k_blk   : [Bt, NB, Di] (written when k_idx != NULL).
 *   sel_out : [Bt, Tq, G, NS] or NULL (the selection is then not returned).
 *   out     : [Bt, Tq, G, H, D].
 *   workspace: >= sizes.forward_workspace_min_bytes; sizes.forward_workspace_bytes gives the
 *   default chunking.  The workspace holds the packed V, an internal selection buffer and the
 *   selection state of a chunk of query tokens: with bf16 index data and k/B <= 513 that state is
 *   a short candidate list per (query, group) (the full score rows are never stored: candidate
 *   scores at or above a sampled threshold are kept and the exact selection runs on them, falling
 *   back to recomputed full rows when a list is too short or overflows); otherwise the chunk's full
 *   score rows.  Larger workspaces mean fewer, larger chunks.
 * Results equal sgqa_index + sgqa_topk + sgqa_attend on the same inputs (selection bit-exact).
 */
sgqa_status sgqa_forward(const sgqa_problem* prob, const void* q, const void* k, const void* v,
                         const void* gate, const void* q_idx, const void* k_idx, void* k_blk,
                         int32_t* sel_out, void* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * sgqa_forward for training: the same results, plus the softmax normaliser of every attention
 * row, which sgqa_attend_backward_with_lse takes instead of recomputing the forward (training up
 * to 1M tokens is the pages' setting: mo.ai.kr summary, section "모델 구조와 학습 안정성").
 *   lse_out : [Bt, Tq, G, H] float32, caller-owned: ln sum_t exp(scale * q . k_t) over the tokens
 *             the row attends to (fp32, from the kernels' exp2-domain running max and sum).
 * Supported: the range-split configurations (bf16, H == 8, D in {64, 128}, B a multiple of 8);
 * others return SGQA_ERR_UNSUPPORTED.  NULL lse_out: SGQA_ERR_NULL.  Workspace as sgqa_forward.
 */
sgqa_status sgqa_forward_with_lse(const sgqa_problem* prob, const void* q, const void* k,
                                  const void* v, const void* gate, const void* q_idx,
                                  const void* k_idx, void* k_blk, int32_t* sel_out, void* out,
                                  float* lse_out, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Profiling hook: stage markers for sgqa_forward.
 *   events : SGQA_STAGE_EVENTS hipEvent_t handles (passed as void*) created by the caller, or NULL
 *            to disarm.  The handles are copied; the array may be freed after the call.
 * While armed, every sgqa_forward call on the calling thread records, on its stream,
 *   events[0] before the first kernel, events[1] after block compression, events[2] after the
 *   indexer and top-k of every query chunk, events[3] after the K/V packing, events[4] once the
 *   attention work lists are built (the pair-union lists of the range-split path; right after
 *   events[3] when there are none), events[5] after the main attention kernel and events[6]
 *   after the merge of range partials (right after events[5] when there is none),
 * so that hipEventElapsedTime between consecutive markers is the duration of that stage.  Arming
 * costs nothing on the device; recording failures make sgqa_forward return SGQA_ERR_HIP.
 * sgqa_decode records the same markers with events[1] after the indexer, events[2] after the
 * top-k and events[3] right after events[2] (the paged cache needs no packing).
 */
#define SGQA_STAGE_EVENTS 7
sgqa_status sgqa_set_stage_events(void* const* events);

/* ---------------------------------------------------------------------------------------------
 * Decode over a paged cache.
 *
 * The pages run Sparse GQA at contexts up to 1M tokens (Step 5 Preview summary on mo.ai.kr,
 * section "모델 구조와 학습 안정성") and serve the model with MTP-3 heads and a KV cache (same
 * page, section "장기 강화학습과 실행 비용"): new tokens arrive a few at a time.  The method is the forward's: for every new query token,
 * steps 2-4 over the sequence's cached keys, with the block keys of step 1 kept per sequence and
 * recomputed only for the blocks that new tokens fall into.  Sequences may hold different numbers
 * of tokens; every call appends / queries the same number of new tokens per sequence.
 *
 * Cache (all device memory, owned by the caller; P = page_tokens):
 *   k_cache    : [num_pages, G, P/8, 8*D]   bf16.  Token t (0..7) of 8-token unit u of a page holds
 *                k[.., d] at element ((d/16)*8 + t)*16 + d%16 of the unit (the operand order the
 *                attention kernel reads).
 *   v_cache    : [num_pages, G, P/8, D, 8]  bf16.  v[.., d] of token t at element d*8 + t.
 *   kidx_cache : [num_pages, P, Di]         index_dtype (bf16).  Index key of each token.
 *   k_blk      : [Bt, max_pages*P/B, Di]    index_dtype.  Block keys of each sequence.
 *   block_table: [Bt, max_pages] int32: logical page j (tokens j*P .. j*P+P-1) of sequence b is
 *                physical page block_table[b*max_pages + j].  Distinct sequences must not share a
 *                page that either of them appends to.
 *   seq_lens   : [Bt] int32: tokens held by each sequence, including the new ones.
 *   (seq_lens and block_table need 4-byte alignment only; every other pointer 16 bytes.)
 * Only sgqa_cache_append writes the cache; it keeps tokens past a sequence's length inside the
 * sequence's last 8-token unit at zero.  Host-side validation covers every size; device-side
 * values (seq_lens, block_table) are clamped into range where the kernels read, and the append
 * stores nothing for tokens whose block_table entry is outside [0, num_pages), so a bad entry
 * gives wrong results for that sequence but never an out-of-bounds access and never a write into
 * a page the entry does not name.  Required:
 * prob->t_q <= seq_lens[b] <= prob->t_kv <= max_pages * P for sgqa_decode (n_new instead of t_q
 * for sgqa_cache_append), block_table entries in [0, num_pages).
 * --------------------------------------------------------------------------------------------- */
typedef struct {
  int64_t num_pages;        /* pages in each pool                                         */
  int32_t page_tokens;      /* P: a power of two, a multiple of 8 and of the block size   */
  int32_t max_pages;        /* entries per block_table row; max_pages * P >= prob->t_kv    */
} sgqa_cache;

/*
 * Append n_new tokens to every sequence: positions seq_lens[b] - n_new .. seq_lens[b] - 1 of
 * sequence b receive k_new, v_new ([Bt, G, n_new, D], dtype bf16) and kidx_new ([Bt, n_new, Di],
 * index_dtype bf16); then every block those positions fall into is recomputed in k_blk as the sum
 * of the cached index keys of its tokens below seq_lens[b] (fp32, token order, rounded once: the
 * same value step 1 gives for the whole sequence).  prob->t_kv bounds seq_lens; prob->t_q is
 * ignored.  A bulk append (n_new = the whole prompt) fills an empty sequence.
 */
sgqa_status sgqa_cache_append(const sgqa_problem* prob, const sgqa_cache* cache,
                              const int32_t* seq_lens, const int32_t* block_table, int64_t n_new,
                              const void* k_new, const void* v_new, const void* kidx_new,
                              void* k_cache, void* v_cache, void* kidx_cache, void* k_blk,
                              void* stream);

/* Workspace bytes sgqa_decode needs for `prob` (Bt sequences, t_q new tokens each, at most t_kv
 * tokens per sequence).  Host only. */
sgqa_status sgqa_decode_workspace_size(const sgqa_problem* prob, const sgqa_cache* cache,
                                       size_t* bytes);

/*
 * Steps 2-4 for the t_q newest tokens of every sequence, over the paged cache.
 *   q, gate : [Bt, t_q, G, H, D] bf16;  q_idx : [Bt, t_q, G, Di] bf16.
 *   Query i of sequence b sits at position p = seq_lens[b] - t_q + i; its selection and output are
 *   those sgqa_forward gives for a sequence of seq_lens[b] tokens (scores of the strictly past
 *   blocks against k_blk, top NS-1 + own block, gated attention over the selected tokens <= p).
 *   sel_out : [Bt, t_q, G, NS] int32 or NULL.   out : [Bt, t_q, G, H, D] bf16.
 *   Supported: dtype and index_dtype bf16, H == 8, D in {64, 128}, B a multiple of 8.
 * With t_q * G <= 32, index dim 32, 64 or 128 and NS <= 513, the selection keeps short candidate
 * lists in the workspace, not score rows.  Per-row thresholds come from sampled blocks.  The
 * filter splits each sequence's blocks over many workgroups.  The exact selection runs on the
 * candidates, and rows it cannot settle are recomputed in full.  Otherwise the selection runs on
 * stored score rows ([Bt * t_q * G, ceil(t_kv / B)] fp32 in the workspace).  The result is the
 * same either way.
 */
sgqa_status sgqa_decode(const sgqa_problem* prob, const sgqa_cache* cache,
                        const int32_t* seq_lens, const int32_t* block_table, const void* q,
                        const void* gate, const void* q_idx, const void* k_cache,
                        const void* v_cache, const void* k_blk, int32_t* sel_out, void* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * sgqa_decode for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments and results as sgqa_decode
 * without the workspace, which comes from a fixed scratch area inside the library instead.
 *   - The scratch is SGQA_DECODE_NOALLOC_SCRATCH_BYTES (128 MiB) of device memory per GPU, part of
 *     the library's code object: the runtime allocates it when the library's kernels load on a GPU,
 *     and each GPU holds it until the process ends.  The first call on a GPU looks up its address
 *     there (no allocation); no call allocates or frees memory.
 *   - Problems whose sgqa_decode workspace exceeds that size are rejected with SGQA_ERR_WORKSPACE
 *     before anything is enqueued (the 64-sequence, 262 144-token, 4-new-token decode needs about
 *     89 MiB).
 *   - Every call on a GPU uses that GPU's one scratch area, and each call clears what it needs, so
 *     calls in sequence on a stream (or ordered across streams) are safe, but calls that can
 *     overlap on one GPU (different streams without ordering, several host threads) race on the
 *     scratch and give wrong results.  Use sgqa_decode with distinct workspaces for those.
 *   - The scratch belongs to the device of `stream` (the current device for the null stream).
 */
#define SGQA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
sgqa_status sgqa_decode_noalloc(const sgqa_problem* prob, const sgqa_cache* cache,
                                const int32_t* seq_lens, const int32_t* block_table, const void* q,
                                const void* gate, const void* q_idx, const void* k_cache,
                                const void* v_cache, const void* k_blk, int32_t* sel_out,
                                void* out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Backward of step 4 (training at long context; Step 5 Preview summary on mo.ai.kr, section
 * "모델 구조와 학습 안정성").  For a fixed selection `sel` (the indexer is not differentiated) and
 * the output gradient dout ([Bt, Tq, G, H, D], dtype), with s_t = scale q.k_t, P = softmax(s) over
 * the selected tokens t <= p, O = sum_t P_t v_t, out = sigmoid(gate) * O:
 *   dO = dout * sigmoid(gate);  dgate = dout * O * sigmoid(gate) (1 - sigmoid(gate));
 *   dS_t = P_t (dO.v_t - dO.O);  dq = scale sum_t dS_t k_t;  dk_t += scale dS_t q;  dv_t += P_t dO
 *   dq, dgate : [Bt, Tq, G, H, D] dtype (rounded to nearest even)
 *   dk, dv    : [Bt, G, Tk, D] float32, overwritten (contributions of every query head summed)
 * The forward softmax statistics are recomputed.  dk / dv are accumulated key-major (every
 * element written once) and dq from fixed-order sums, so every gradient is the same bits on every
 * run.  Supported: bf16, H == 8, D in {64, 128}, B a multiple of 8, topk_tokens / block within the
 * grouped kernel (as for the range-split forward).
 * --------------------------------------------------------------------------------------------- */
sgqa_status sgqa_attend_backward_workspace_size(const sgqa_problem* prob, size_t* bytes);
sgqa_status sgqa_attend_backward(const sgqa_problem* prob, const void* q, const void* k,
                                 const void* v, const void* gate, const int32_t* sel,
                                 const void* dout, void* dq, float* dk, float* dv, void* dgate,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same gradients from the forward's saved output and normaliser instead of a recompute:
 *   out : [Bt, Tq, G, H, D] dtype, the forward's output (sigmoid(gate) * O);
 *   lse : [Bt, Tq, G, H] float32, sgqa_forward_with_lse's lse_out for the same inputs.
 * With out = sigmoid(gate) O:  dO . O = dout . out  and  dgate = dout * out * (1 - sigmoid(gate)),
 * and P_t = exp(scale q.k_t - lse).  Other arguments, outputs, workspace size and supported
 * configurations as sgqa_attend_backward; out and lse are only read.  Results agree with
 * sgqa_attend_backward up to rounding (dO . O is summed from the bf16 output here).
 */
sgqa_status sgqa_attend_backward_with_lse(const sgqa_problem* prob, const void* q, const void* k,
                                          const void* v, const void* gate, const int32_t* sel,
                                          const void* out, const float* lse, const void* dout,
                                          void* dq, float* dk, float* dv, void* dgate,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Steps 1-4 with K and V stored as fp8.  The pages run the KV cache in FP8 (trained for it: FP8
 * KV QAT; Step 5 Preview summary on mo.ai.kr, section "장기 강화학습과 실행 비용").  Here k8 and v8
 * hold OCP e4m3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, 0x7f /
 * 0xff are NaN) in the layout of k and v ([Bt, G, Tk, D], one byte each), and the values attended
 * to are code * k_scale and code * v_scale (per-tensor scales, finite and > 0).  Everything else
 * is sgqa_forward: same selection, same gate, bf16 q / gate / out, same workspace size
 * (sizes.forward_workspace_*).  Supported: dtype bf16, H == 8, D in {64, 128}, B a multiple of 8.
 * --------------------------------------------------------------------------------------------- */
sgqa_status sgqa_forward_fp8kv(const sgqa_problem* prob, const void* q, const void* k8,
                               const void* v8, float k_scale, float v_scale, const void* gate,
                               const void* q_idx, const void* k_idx, void* k_blk, int32_t* sel_out,
                               void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Gated sliding-window attention: the efficient layers placed three to one with the sparse layer
 * (Step 5 Preview summary on mo.ai.kr, section "모델 구조와 학습 안정성"; ai.info article, section
 * "Perché StepFun ha scelto 92 blocchi transformer").  The pages name the layer (Gated SWA) but no
 * window size, so the window is an argument.  For query i at p = Tk - Tq + i, head j of group g:
 *   out = sigmoid(gate) * sum_t softmax_t(scale * q . k_t) v_t over t in [max(0, p - window + 1), p]
 * with the same layouts, dtypes and rounding as sgqa_attend (k_idx, q_idx and the selection play
 * no part; prob's block / topk fields must still be valid).  Supported: bf16, H == 8, D in
 * {64, 128}.  The workspace holds block-packed K and V and the per-group work lists.
 * --------------------------------------------------------------------------------------------- */
sgqa_status sgqa_swa_workspace_size(const sgqa_problem* prob, int64_t window, size_t* bytes);
sgqa_status sgqa_swa(const sgqa_problem* prob, int64_t window, const void* q, const void* k,
                     const void* v, const void* gate, void* out, void* workspace,
                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* SGQA_H_ */
