"""Plain, slow CPU definition of the Sparse GQA forward path (fp64 / exact) -- test infrastructure.

This file is the oracle the GPU path is checked against.  It is written from the method's description
on the Step 5 Preview pages and nothing else:

* "Step 5 Preview" summary (mo.ai.kr), section "모델 구조와 학습 안정성" (model structure and training
  stability): the full-attention layers use Sparse GQA built on Gated GQA; shared index keys are
  compressed block-wise; every KV group selects its own relevant past context; the block size of 8
  cuts indexer and top-k cost eightfold; the final setting is B = 8 with k = 4096 tokens, i.e. 512
  selected blocks, with a token inclusion rate of 78.06 % against 79.09 % for B = 1, k = 2048.
* "Step 5 Preview" article (ai.info), section "Sparse GQA punta a un contesto di 1 milione di token":
  the same method restated (blocks of eight tokens, top-k of 4096, the 78.06 % / 79.09 % coverage
  comparison).

Where the pages leave a step open, the oracle takes these readings:
  1. block compression is the SUM of the B index keys of the block (a partial last block sums the
     keys that exist);
  2. one index key per token is shared by all KV groups; the index QUERY is per (token, KV group);
  3. the indexer score is the raw dot product q_idx . K_blk (no scale, no activation);
  4. a query at absolute position p owns block o = p // B.  Blocks j < o are candidates; the own
     block is always selected and counts toward the budget of n_sel = k / B blocks; inside the own
     block a causal mask keeps tokens t <= p;
  5. among candidates, higher score wins; equal scores go to the lower block index;
  6. when o + 1 <= n_sel every causal block is selected (the query is dense);
  7. the output gate is elementwise: out = sigmoid(gate) * attention_output;
  8. the softmax scale is an explicit argument (1/sqrt(d) in every workload);
  9. query head j of KV group g uses that group's keys and values (GQA);
 10. queries are the last t_q positions of the key stream (p = t_kv - t_q + i).

Precision: everything is computed in float64.  For integer-valued index data (every workload) the
block sums and scores are exact integers far below 2**53, so the selection is exact.

Parity pins: every function here is checked in tests/ against something other than itself (closed
forms, special cases that reduce to a library routine, brute force on tiny inputs, a hand-worked
example).  The token inclusion rate is pinned by brute force on tiny inputs; its value on the
synthetic workloads is a measured property of those inputs, not a target.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "num_blocks", "n_selected_blocks", "query_positions", "compress", "block_scores",
    "select_blocks", "attended_tokens", "gated_attention", "forward_rows", "forward",
    "scored_candidates", "inclusion_rate", "sequence_rows", "window_rows", "e4m3_decode",
    "attention_backward",
]


# ----------------------------------------------------------------------------------------------
# sizes
# ----------------------------------------------------------------------------------------------
def num_blocks(t_kv: int, block: int) -> int:
    """Number of index-key blocks: ceil(t_kv / B) (blocks of B consecutive tokens)."""
    return -(-int(t_kv) // int(block))


def n_selected_blocks(topk_tokens: int, block: int) -> int:
    """Selected blocks per (query, KV group): k / B (k = 4096, B = 8 gives 512 on the pages)."""
    if topk_tokens % block:
        raise ValueError("the token budget must be a multiple of the block size")
    return int(topk_tokens) // int(block)


def query_positions(t_q: int, t_kv: int) -> np.ndarray:
    """Absolute positions of the queries: the last t_q tokens of the key stream (reading 10)."""
    return np.arange(int(t_kv) - int(t_q), int(t_kv), dtype=np.int64)


def scored_candidates(p: int, block: int) -> int:
    """Blocks the indexer scores for a query at position p: the strictly past blocks 0..p//B - 1."""
    return int(p) // int(block)


# ----------------------------------------------------------------------------------------------
# step 1: block compression of the shared index keys
# ----------------------------------------------------------------------------------------------
def compress(k_idx, block: int) -> np.ndarray:
    """K_blk[b, j, :] = sum of k_idx[b, t, :] over tokens t of block j (reading 1).

    k_idx: [batch, t_kv, d_idx].  Returns float64 [batch, ceil(t_kv/B), d_idx].
    """
    k = np.asarray(k_idx, dtype=np.float64)
    starts = np.arange(0, k.shape[1], int(block))
    return np.add.reduceat(k, starts, axis=1)


# ----------------------------------------------------------------------------------------------
# step 2: the indexer
# ----------------------------------------------------------------------------------------------
def block_scores(q_idx_row, k_blk_seq, o: int) -> np.ndarray:
    """Scores of one (query, KV group) against its candidate blocks j < o (readings 3, 4).

    q_idx_row: [d_idx]; k_blk_seq: [NB, d_idx].  Returns float64 [o].
    """
    q = np.asarray(q_idx_row, dtype=np.float64)
    kb = np.asarray(k_blk_seq, dtype=np.float64)[: int(o)]
    return kb @ q


# ----------------------------------------------------------------------------------------------
# step 3: per-(query, KV group) top-k over blocks
# ----------------------------------------------------------------------------------------------
def select_blocks(scores, o: int, n_sel: int) -> np.ndarray:
    """Selected blocks of one (query, KV group), ascending, padded with -1 to n_sel (readings 4-6).

    scores: the o candidate scores (blocks 0..o-1).  The own block o is always selected.
    A full stable sort of the negated scores orders candidates by (score desc, index asc).
    """
    o = int(o)
    n_sel = int(n_sel)
    if o + 1 <= n_sel:
        chosen = np.arange(o + 1, dtype=np.int64)
    else:
        s = np.asarray(scores, dtype=np.float64)[:o]
        order = np.argsort(-s, kind="stable")
        chosen = np.sort(np.concatenate([order[: n_sel - 1], [o]])).astype(np.int64)
    out = np.full(n_sel, -1, dtype=np.int64)
    out[: chosen.size] = chosen
    return out


def attended_tokens(sel, block: int, p: int, t_kv: int) -> np.ndarray:
    """Tokens a query at position p attends to: every token of every selected block with t <= p."""
    blocks = np.asarray(sel, dtype=np.int64)
    blocks = blocks[blocks >= 0]
    if blocks.size == 0:
        return np.zeros(0, dtype=np.int64)
    toks = (blocks[:, None] * int(block) + np.arange(int(block))[None, :]).reshape(-1)
    toks = toks[(toks <= int(p)) & (toks < int(t_kv))]
    return np.sort(toks)


# ----------------------------------------------------------------------------------------------
# step 4: gated GQA over the gathered tokens
# ----------------------------------------------------------------------------------------------
def gated_attention(q_rows, k_seq, v_seq, gate_rows, tokens, scale: float) -> np.ndarray:
    """sigmoid(gate) * softmax(scale * q k_t^T) v over the given tokens, per head (readings 7-9).

    q_rows, gate_rows: [h, d] (the query heads of one KV group); k_seq, v_seq: [t_kv, d] of that
    group; tokens: attended token indices.  Returns float64 [h, d].
    """
    q = np.asarray(q_rows, dtype=np.float64)
    kk = np.asarray(k_seq, dtype=np.float64)[tokens]
    vv = np.asarray(v_seq, dtype=np.float64)[tokens]
    g = np.asarray(gate_rows, dtype=np.float64)
    logits = float(scale) * (q @ kk.T)                     # [h, n]
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    attn = (w @ vv) / w.sum(axis=1, keepdims=True)         # [h, d]
    return attn / (1.0 + np.exp(-g))


# ----------------------------------------------------------------------------------------------
# the whole path
# ----------------------------------------------------------------------------------------------
def _np64(x):
    """Widen a numpy array or a (CPU or device) torch tensor to a float64 numpy array."""
    if hasattr(x, "detach"):
        import torch  # local: only to widen bf16 tensors, which numpy cannot hold
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _rows64(x, b, g, toks):
    """x[b, g][toks] as float64 (gathers only the rows needed)."""
    if hasattr(x, "detach"):
        import torch
        idx = torch.from_numpy(np.asarray(toks, dtype=np.int64)).to(x.device)
        return _np64(x[b, g].index_select(0, idx))
    return np.asarray(x[b, g][toks], dtype=np.float64)


def forward_rows(inputs, block: int, topk_tokens: int, scale: float, rows, k_blk=None):
    """Run the four steps for the listed query tokens, every KV group.

    inputs: dict with q [Bt,Tq,G,h,d], k, v [Bt,G,Tkv,d], gate [Bt,Tq,G,h,d], q_idx [Bt,Tq,G,di],
            k_idx [Bt,Tkv,di]  (numpy arrays or torch tensors, any float dtype).
    rows: iterable of (b, i) query tokens.
    k_blk: optional precomputed block keys [Bt, NB, di]; otherwise each needed sequence's k_idx is
           compressed here.
    Returns (sel [n, G, n_sel] int64, out [n, G, h, d] float64, {b: K_blk[b]} float64).
    """
    q_idx, q, k, v, gate = (inputs[n] for n in ("q_idx", "q", "k", "v", "gate"))
    t_q, G = q_idx.shape[1], q_idx.shape[2]
    t_kv = k.shape[2]
    n_sel = n_selected_blocks(topk_tokens, block)
    pos = query_positions(t_q, t_kv)
    rows = list(rows)
    h, d = q.shape[3], q.shape[4]
    sel_out = np.full((len(rows), G, n_sel), -1, dtype=np.int64)
    out = np.zeros((len(rows), G, h, d), dtype=np.float64)
    kblk = {}
    for r, (b, i) in enumerate(rows):
        if b not in kblk:
            kblk[b] = (_np64(k_blk[b]) if k_blk is not None
                       else compress(_np64(inputs["k_idx"][b:b + 1]), block)[0])
        p = int(pos[i])
        o = p // block
        qi = _np64(q_idx[b, i])
        qb = _np64(q[b, i])
        gb = _np64(gate[b, i])
        for g in range(G):
            s = block_scores(qi[g], kblk[b], o)
            sel = select_blocks(s, o, n_sel)
            sel_out[r, g] = sel
            toks = attended_tokens(sel, block, p, t_kv)
            kk = _rows64(k, b, g, toks)
            vv = _rows64(v, b, g, toks)
            out[r, g] = gated_attention(qb[g], kk, vv, gb[g], np.arange(toks.size), scale)
    return sel_out, out, kblk


def forward(inputs, block: int, topk_tokens: int, scale: float):
    """Every query token of every sequence (small inputs only).

    Returns (sel [Bt, Tq, G, n_sel], out [Bt, Tq, G, h, d], K_blk [Bt, NB, di])."""
    bt, t_q = inputs["q_idx"].shape[0], inputs["q_idx"].shape[1]
    rows = [(b, i) for b in range(bt) for i in range(t_q)]
    sel, out, kblk = forward_rows(inputs, block, topk_tokens, scale, rows)
    G, n_sel = sel.shape[1], sel.shape[2]
    h, d = out.shape[2], out.shape[3]
    k_blk = np.stack([kblk[b] for b in range(bt)])
    return sel.reshape(bt, t_q, G, n_sel), out.reshape(bt, t_q, G, h, d), k_blk


def sequence_rows(inputs, seq_lens, block: int, topk_tokens: int, scale: float, rows):
    """Rows of sequences that hold different numbers of tokens (decode over a cache).

    Sequence b holds seq_lens[b] tokens: its keys, values and index keys are the first seq_lens[b]
    of inputs' k, v, k_idx (anything past them is not part of the sequence), and its t_q queries
    are the last t_q positions of those tokens (reading 10 applied per sequence).  Each sequence is
    therefore the forward path on its own prefix; the rows (b, i) are computed that way.
    Returns (sel [n, G, n_sel], out [n, G, h, d], {b: K_blk[b]}) like forward_rows.
    """
    rows = list(rows)
    G, n_sel = inputs["q_idx"].shape[2], n_selected_blocks(topk_tokens, block)
    h, d = inputs["q"].shape[3], inputs["q"].shape[4]
    sel_out = np.full((len(rows), G, n_sel), -1, dtype=np.int64)
    out = np.zeros((len(rows), G, h, d), dtype=np.float64)
    kblk = {}
    for b in sorted({b for b, _ in rows}):
        L = int(seq_lens[b])
        seq = {"q": inputs["q"][b:b + 1], "gate": inputs["gate"][b:b + 1],
               "q_idx": inputs["q_idx"][b:b + 1], "k": inputs["k"][b:b + 1, :, :L],
               "v": inputs["v"][b:b + 1, :, :L], "k_idx": inputs["k_idx"][b:b + 1, :L]}
        mine = [r for r, (bb, _) in enumerate(rows) if bb == b]
        s_b, o_b, kb = forward_rows(seq, block, topk_tokens, scale, [(0, rows[r][1]) for r in mine])
        sel_out[mine] = s_b
        out[mine] = o_b
        kblk[b] = kb[0]
    return sel_out, out, kblk


def e4m3_decode(codes) -> np.ndarray:
    """Values of OCP fp8 e4m3 codes (the FP8 KV cache the pages train for: Step 5 Preview summary
    on mo.ai.kr, section "장기 강화학습과 실행 비용").  Bit 7 is the sign, bits 3-6 the exponent
    (bias 7), bits 0-2 the mantissa; exponent 0 is subnormal (m * 2^-9); there are no infinities
    and S.1111.111 is NaN.  Exact in float64."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((e == 15) & ((c & 7) == 7), np.nan, sign * mag)


def attention_backward(inputs, sel, dout, block: int, scale: float):
    """Gradients of the gated attention step for a fixed selection (training at long context is
    the pages' setting: Step 5 Preview summary on mo.ai.kr, section "모델 구조와 학습 안정성").
    The selection comes from the indexer and is not differentiated.  Per query row (b, i, g, head)
    with attended tokens A, s_t = scale q.k_t, P = softmax(s), O = sum_t P_t v_t and
    out = sigmoid(gate) * O, the chain rule gives
        dO = dout * sigmoid(gate),   dgate = dout * O * sigmoid(gate) * (1 - sigmoid(gate)),
        dP_t = dO . v_t,   D = sum_t P_t dP_t (= dO . O),   dS_t = P_t (dP_t - D),
        dq = scale sum_t dS_t k_t,   dk_t += scale dS_t q,   dv_t += P_t dO.
    inputs: q, k, v, gate as for forward_rows; sel [Bt, Tq, G, n_sel]; dout like q.
    Returns float64 (dq, dk, dv, dgate) shaped like q, k, v, gate.  Small inputs only."""
    q, k, v, gate = (_np64(inputs[n]) for n in ("q", "k", "v", "gate"))
    sel = np.asarray(sel)
    dout = _np64(dout)
    bt, t_q, G, h, d = q.shape
    t_kv = k.shape[2]
    pos = query_positions(t_q, t_kv)
    dq, dk, dv, dgate = (np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(gate))
    for b in range(bt):
        for i in range(t_q):
            p = int(pos[i])
            for g in range(G):
                toks = attended_tokens(sel[b, i, g], block, p, t_kv)
                kk, vv = k[b, g, toks], v[b, g, toks]                  # [n, d]
                for j in range(h):
                    s = scale * (kk @ q[b, i, g, j])
                    w = np.exp(s - s.max())
                    P = w / w.sum()
                    O = P @ vv
                    sg = 1.0 / (1.0 + np.exp(-gate[b, i, g, j]))
                    dO = dout[b, i, g, j] * sg
                    dgate[b, i, g, j] = dout[b, i, g, j] * O * sg * (1.0 - sg)
                    dP = vv @ dO
                    dS = P * (dP - P @ dP)
                    dq[b, i, g, j] = scale * (dS @ kk)
                    dk[b, g, toks] += scale * np.outer(dS, q[b, i, g, j])
                    dv[b, g, toks] += np.outer(P, dO)
    return dq, dk, dv, dgate


def attention_lse(inputs, sel, block: int, scale: float, rows):
    """Softmax normaliser of every attention row for the listed query tokens: per (b, i, g, head)
    ln sum_t exp(scale q.k_t) over the attended tokens t (those of the selected blocks at or before
    the query's position), the quantity a training forward keeps for its backward (training at
    long context: Step 5 Preview summary on mo.ai.kr, section "모델 구조와 학습 안정성").
    inputs: q, k as for forward_rows; sel [Bt, Tq, G, n_sel]; rows: query token indices.
    Returns float64 [Bt, len(rows), G, H] (max-shifted sum, so large logits do not overflow)."""
    q, k = inputs["q"], inputs["k"]
    sel = np.asarray(sel)
    bt, t_q, G, h, _ = q.shape
    t_kv = k.shape[2]
    pos = query_positions(t_q, t_kv)
    out = np.zeros((bt, len(rows), G, h))
    for b in range(bt):
        for r, i in enumerate(rows):
            p = int(pos[i])
            for g in range(G):
                toks = attended_tokens(sel[b, i, g], block, p, t_kv)
                kk = _rows64(k, b, g, toks)                            # [n, d]
                qq = _np64(q[b, i, g])                                 # [h, d]
                s = scale * (qq @ kk.T)                                # [h, n]
                m = s.max(axis=1, keepdims=True)
                out[b, r, g] = (m[:, 0] + np.log(np.exp(s - m).sum(axis=1)))
    return out


def window_rows(inputs, window: int, scale: float, rows):
    """Gated sliding-window attention (the efficient layers the pages interleave three to one with
    Sparse GQA; Step 5 Preview summary on mo.ai.kr, section "모델 구조와 학습 안정성").  The pages
    give no window size, so it is an argument: a query at position p attends to the tokens
    t in [max(0, p - window + 1), p], with the same gate, scale and GQA reading as the sparse layer.
    Returns out [n, G, h, d] float64 for the listed (b, i)."""
    q, k, v, gate = (inputs[n] for n in ("q", "k", "v", "gate"))
    t_q, G = q.shape[1], q.shape[2]
    t_kv = k.shape[2]
    pos = query_positions(t_q, t_kv)
    rows = list(rows)
    out = np.zeros((len(rows), G, q.shape[3], q.shape[4]), dtype=np.float64)
    for r, (b, i) in enumerate(rows):
        p = int(pos[i])
        toks = np.arange(max(0, p - window + 1), p + 1)
        qb, gb = _np64(q[b, i]), _np64(gate[b, i])
        for g in range(G):
            out[r, g] = gated_attention(qb[g], _rows64(k, b, g, toks), _rows64(v, b, g, toks),
                                        gb[g], np.arange(toks.size), scale)
    return out


# ----------------------------------------------------------------------------------------------
# token inclusion rate (the pages' selection-quality measure)
# ----------------------------------------------------------------------------------------------
def inclusion_rate(q_idx, k_idx, rows, t_kv: int, cfg_a=(8, 4096), cfg_b=(1, 2048)):
    """Token inclusion of selection A against selection B, per (query, KV group).

    For each listed (b, i) and every group: |A_a & A_b| / |A_b|, where A_x is the set of tokens the
    query attends to under block size / token budget cfg_x.  The pages compare B=8, k=4096 against
    B=1, k=2048 (78.06 % vs 79.09 %) without naming the reference set; this takes the B=1, k=2048
    token set as the reference.  Returns float64 [n_rows, G].  Its value on synthetic data is a
    measured property of those inputs.
    """
    t_q, G = q_idx.shape[1], q_idx.shape[2]
    pos = query_positions(t_q, t_kv)
    (ba, ka), (bb, kb) = cfg_a, cfg_b
    rows = list(rows)
    rate = np.zeros((len(rows), G))
    cache = {}
    for r, (b, i) in enumerate(rows):
        if b not in cache:
            kseq = _np64(k_idx[b:b + 1])
            cache = {b: (compress(kseq, ba)[0], compress(kseq, bb)[0])}
        kblk_a, kblk_b = cache[b]
        qi = _np64(q_idx[b, i])
        p = int(pos[i])
        for g in range(G):
            oa, ob = p // ba, p // bb
            sa = select_blocks(block_scores(qi[g], kblk_a, oa), oa, ka // ba)
            sb = select_blocks(block_scores(qi[g], kblk_b, ob), ob, kb // bb)
            ta = attended_tokens(sa, ba, p, t_kv)
            tb = attended_tokens(sb, bb, p, t_kv)
            rate[r, g] = np.intersect1d(ta, tb).size / tb.size
    return rate
