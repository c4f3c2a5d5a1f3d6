"""fp64 CPU oracle of the Mixtral-style sparse mixture-of-experts layer.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the
benchmark's CPU-baseline leg may use it.  It shares no code with the HIP path.

What it computes is the plain definition of the layer, written out in NumPy
float64 (every input is widened losslessly from its bf16/fp32 storage):

    y = sum_i Softmax(TopK(x . W_g))_i * SwiGLU_i(x)

as given by the layer equation on card 2.1 "Sparse Mixture of Experts" of the
"Mixtral of Experts" study deck (Jiang et al. 2024), with the general
token-choice top-k form from "How Experts Are Chosen (Routing Methods)" in
"Mixtral of Experts? Mixture of Experts? Try to explain Mixtral 8x7B", and the
router walk-through of Part 3, "Pip's token goes to triage" (steps 1-4) in
"Mixture of Experts: Why Mixtral Only Wakes Up Two Specialists".

Readings where the pages leave a step open (each also listed in the design notes):
  * SwiGLU_i(x) = (SiLU(x W1_i) * (x W3_i)) W2_i with SiLU(z) = z * sigmoid(z):
    the pages only name SwiGLU and say an expert expands with d x f matrices,
    applies a simple non-linearity and compresses back (three matrices per
    expert, Part 2 and Part 4 of the explainer).  No biases anywhere.
  * Top-K ties go to the lower expert index; the K kept slots are ordered by
    descending logit (the walk-through lists the larger score first).
  * The softmax runs over the K kept logits only (the others are -inf).
  * Expert indices are 0-based (the equation sums i = 0..n-1); the walk-through
    counts from 1, so its "expert 3 and expert 7" are indices 2 and 6 here.
  * y excludes the residual add that the surrounding block performs.
  * Router statistics (Part 5): f_i counts the T*K assignments once each,
    f_i = counts_i / (T*K), so both shares are 1/N when balanced.
  * Expert-choice routing (named on the first page without details): the
    score is the router's softmax probability over experts; each expert takes
    its C = min(T, ceil(cf * T / n)) best tokens, ties to the lower token
    index; a chosen (t, e) adds S[t][e] * SwiGLU_e(x_t).
  * 4-bit weights (the page sizes the model at 4 bits but gives no format):
    the format is defined with quantize_q4 below; the layer on such weights is
    the plain forward on the dequantised values.
  * Capacity (Part 5, "What happens when an expert is full"): with K
    assignments per token C = ceil(cf * T * K / n); each expert keeps its first
    C assignments in token order, dropped ones add nothing and the kept
    weights are not renormalised.

Pins (tests/test_oracle_pins.py) tie each function to something other than
itself: the walk-through's printed weights, brute force over all expert
subsets, the K = n / K = 1 / n = K = 1 special cases, the parameter arithmetic
printed in Part 4 of the explainer, closed forms of the sigmoid, hand-worked
rows for the top-K margins and for the expert-choice readings, and metamorphic
invariants.  Two limits of those pins:
  * expert_swiglu computes a reading (the pages name SwiGLU without defining
    it and print no expert output); its pins fix that reading (explicit loops,
    closed forms, the gate/up asymmetry), not a number from the pages;
  * the expert-choice, capacity and 4-bit functions implement readings of
    passages that give no worked numbers; their pins are hand-worked examples,
    brute force and limits that reduce to the top-K layer.
"""
from __future__ import annotations

import itertools
import math
from typing import Callable, Union

import numpy as np

ArrayOrGetter = Union[np.ndarray, Callable[[int], np.ndarray]]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _expert(W: ArrayOrGetter, e: int) -> np.ndarray:
    """Expert e's matrix in float64; W is either an [n][..][..] array or a
    callable returning expert e's matrix (lets full-size checks widen one
    expert at a time)."""
    if callable(W):
        return _f64(W(e))
    return _f64(W[e])


# ---------------------------------------------------------------- router ---

def router_logits(x, Wg) -> np.ndarray:
    """Step 1 of the walk-through: a bias-free linear layer scores every expert,
    logits[t][e] = sum_j x[t][j] * W_g[j][e]  (x . W_g in the layer equation)."""
    return _f64(x) @ _f64(Wg)


def topk_select(logits: np.ndarray, K: int):
    """Step 2 of the walk-through: keep the K largest scores and their positions.

    Returns (sel, margin, slot_margin):
      sel[t]        the K kept expert indices, descending logit, ties -> lower index
      margin[t]     gap between the K-th and (K+1)-th sorted logits (+inf if K == n)
      slot_margin[t] smallest gap between consecutive kept logits (+inf if K == 1)
    """
    logits = _f64(logits)
    T, n = logits.shape
    if not 1 <= K <= n:
        raise ValueError("need 1 <= K <= n")
    # a stable sort of the negated scores keeps equal scores in index order
    order = np.argsort(-logits, axis=1, kind="stable")
    sel = order[:, :K].astype(np.int64)
    srt = np.take_along_axis(logits, order, axis=1)
    if K < n:
        margin = srt[:, K - 1] - srt[:, K]
    else:
        margin = np.full(T, np.inf)
    if K > 1:
        slot_margin = np.min(srt[:, :K - 1] - srt[:, 1:K], axis=1)
    else:
        slot_margin = np.full(T, np.inf)
    return sel, margin, slot_margin


def gate_weights(logits: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """Step 3 of the walk-through: softmax over the kept scores only (the
    unselected logits are -inf in the layer equation, so they get weight 0).
    Max-subtracted form; w[t][k] is the weight of expert sel[t][k]."""
    kept = np.take_along_axis(_f64(logits), np.asarray(sel), axis=1)
    z = np.exp(kept - kept.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def route(x, Wg, K: int) -> dict:
    """Steps 1-3 plus the integer dispatch, as one record."""
    logits = router_logits(x, Wg)
    sel, margin, slot_margin = topk_select(logits, K)
    w = gate_weights(logits, sel)
    counts, offsets, perm_token, slot_pos = dispatch(sel, logits.shape[1])
    return dict(logits=logits, sel=sel, w=w, margin=margin, slot_margin=slot_margin,
                counts=counts, offsets=offsets, perm_token=perm_token, slot_pos=slot_pos)


def full_softmax(logits: np.ndarray) -> np.ndarray:
    """The router's probability of every expert for every token: softmax over
    all n logits (max-subtracted), before any expert is dropped."""
    lg = _f64(logits)
    z = np.exp(lg - lg.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def router_stats(logits: np.ndarray, sel: np.ndarray, alpha: float) -> dict:
    """Load-balancing statistics of the Switch design, as Part 5 of "Mixture of
    Experts: Why Mixtral Only Wakes Up Two Specialists" describes them ("The
    favourite expert problem", tool 2), for top-K routing:

      f_i  share of the routed work sent to expert i: the T*K assignments
           count once each, so f_i = counts_i / (T*K) and the shares sum to 1
           (the page calls both shares even at 1/N each);
      P_i  the router's average probability for expert i over the tokens
           (full softmax over all N experts);
      loss = alpha * N * sum_i f_i * P_i.
    """
    lg = _f64(logits)
    T, n = lg.shape
    K = sel.shape[1]
    counts = np.zeros(n, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            counts[sel[t, k]] += 1
    frac = counts / float(T * K)
    prob = full_softmax(lg).mean(axis=0)
    loss = alpha * n * float(np.sum(frac * prob))
    return dict(frac=frac, prob=prob, aux_loss=loss, counts=counts)


def expert_choice_capacity(T: int, n: int, capacity_factor: float) -> int:
    """Tokens each expert takes in expert-choice routing: the batch's tokens
    spread over the experts times a capacity factor (the average number of
    experts per token), at most T."""
    return int(min(T, math.ceil(capacity_factor * T / n)))


def expert_choice_select(logits: np.ndarray, C: int):
    """Expert-based routing ("How Experts Are Chosen (Routing Methods)" in
    "Mixtral of Experts? Mixture of Experts? Try to explain Mixtral 8x7B"): the
    experts choose their tokens, each with a fixed capacity.  The score of
    (token, expert) is the router's probability (softmax over the experts of
    the token's logits); each expert takes its C best-scoring tokens, ties to
    the lower token index.
    Returns chosen [T][n] bool, the scores S [T][n] and, per expert, the gap
    between its C-th and (C+1)-th best scores (inf when C = T)."""
    S = full_softmax(logits)
    T, n = S.shape
    chosen = np.zeros((T, n), dtype=bool)
    margin = np.full(n, np.inf)
    for e in range(n):
        order = np.argsort(-S[:, e], kind="stable")
        chosen[order[:C], e] = True
        if C < T:
            margin[e] = S[order[C - 1], e] - S[order[C], e]
    return chosen, S, margin


def expert_choice_dispatch(chosen: np.ndarray, C: int):
    """Rows of expert e are e*C .. e*C+C-1, its chosen tokens in ascending order.
      perm_token[e*C + j] j-th chosen token of expert e
      slot_pos[t][e]      row of (t, e), -1 if e did not choose t"""
    T, n = chosen.shape
    perm_token = np.empty(n * C, dtype=np.int64)
    slot_pos = np.full((T, n), -1, dtype=np.int64)
    for e in range(n):
        toks = np.nonzero(chosen[:, e])[0]
        perm_token[e * C:e * C + toks.size] = toks
        slot_pos[toks, e] = e * C + np.arange(toks.size)
    return perm_token, slot_pos


def forward_expert_choice(x, Wg, W1: ArrayOrGetter, W3: ArrayOrGetter, W2: ArrayOrGetter,
                          chosen: np.ndarray) -> np.ndarray:
    """y[t] = sum over the experts that chose t of S[t][e] * SwiGLU_e(x[t]); a
    token no expert chose gets y = 0 (it passes on through the residual)."""
    x = _f64(x)
    S = full_softmax(router_logits(x, Wg))
    T, n = S.shape
    y = np.zeros((T, x.shape[1]))
    for e in range(n):
        rows = np.nonzero(chosen[:, e])[0]
        if rows.size == 0:
            continue
        out = expert_swiglu(x[rows], _expert(W1, e), _expert(W3, e), _expert(W2, e))
        y[rows] += S[rows, e][:, None] * out
    return y


def brute_force_topk(logit_row: np.ndarray, K: int) -> tuple:
    """Top-K by exhaustive search over all C(n, K) expert subsets: the subset with
    the largest logit sum; among equal sums the lexicographically smallest
    sorted index tuple.  Returned as a sorted tuple (a set, not slot order)."""
    row = _f64(logit_row)
    best, best_sum = None, -np.inf
    for sub in itertools.combinations(range(row.shape[0]), K):
        s = float(sum(row[i] for i in sub))
        if s > best_sum:  # combinations() runs in lexicographic order
            best, best_sum = sub, s
    return best


# -------------------------------------------------------------- dispatch ---

def dispatch(sel: np.ndarray, n: int):
    """Group the (token, slot) assignments by expert: a counting sort in token order.

    The pages only say that experts with zero gate are not evaluated (Part 3 of
    the explainer, step 2; the sparse-gating passage of "How a mixture-of-experts
    model activates only part of its parameters"); grouping the surviving
    assignments per expert is the plain way to run each expert once on its rows.
      counts[e]      number of assignments to expert e
      offsets[e]     exclusive prefix sum of counts, offsets[n] = T*K
      perm_token[p]  token of position p; expert-contiguous, ascending t per expert
      slot_pos[t][k] position of assignment (t, k)
    """
    sel = np.asarray(sel, dtype=np.int64)
    T, K = sel.shape
    counts = np.zeros(n, dtype=np.int64)
    for e in sel.reshape(-1):
        counts[e] += 1
    offsets = np.zeros(n + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm_token = np.empty(T * K, dtype=np.int64)
    slot_pos = np.empty((T, K), dtype=np.int64)
    for e in range(n):
        hit = sel == e                       # [T][K]; a token holds e at most once
        toks = np.nonzero(hit.any(axis=1))[0]  # ascending token index
        pos = offsets[e] + np.arange(toks.size)
        perm_token[pos] = toks
        k_of = np.argmax(hit[toks], axis=1)
        slot_pos[toks, k_of] = pos
    return counts, offsets, perm_token, slot_pos


# --------------------------------------------------------------- experts ---

def expert_capacity(T: int, n: int, K: int, capacity_factor: float) -> int:
    """Expert capacity of the Switch design (Part 5 of the explainer, "What
    happens when an expert is full"): the batch's tokens divided by the number
    of experts, times a capacity factor.  With K assignments per token the
    work to share is T*K, so C = ceil(capacity_factor * T * K / n)."""
    return int(math.ceil(capacity_factor * T * K / n))


def capacity_dispatch(sel: np.ndarray, n: int, cap: int):
    """Dispatch with a capacity: walking the tokens in order, each expert
    accepts assignments until it holds `cap`; later ones overflow and are
    dropped (no row, no computation).
      kept[t][k]     whether assignment (t, k) got a row
      counts[e]      kept assignments of expert e (<= cap)
      offsets, perm_token over the kept rows (expert-contiguous, ascending t)
      slot_pos[t][k] row of a kept assignment, -1 for a dropped one
    """
    sel = np.asarray(sel, dtype=np.int64)
    T, K = sel.shape
    load = np.zeros(n, dtype=np.int64)
    kept = np.zeros((T, K), dtype=bool)
    for t in range(T):
        for k in range(K):
            e = sel[t, k]
            if load[e] < cap:
                kept[t, k] = True
                load[e] += 1
    counts = load
    offsets = np.zeros(n + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm_token = np.empty(int(offsets[n]), dtype=np.int64)
    slot_pos = np.full((T, K), -1, dtype=np.int64)
    nxt = offsets[:n].copy()
    for t in range(T):
        for k in range(K):
            if kept[t, k]:
                e = sel[t, k]
                perm_token[nxt[e]] = t
                slot_pos[t, k] = nxt[e]
                nxt[e] += 1
    return dict(kept=kept, counts=counts, offsets=offsets, perm_token=perm_token, slot_pos=slot_pos)


def forward_capacity(x, Wg, W1: ArrayOrGetter, W3: ArrayOrGetter, W2: ArrayOrGetter, sel: np.ndarray,
                     cap: int) -> np.ndarray:
    """The layer with dropped assignments: a dropped (t, k) computes nothing and
    adds nothing (the token goes on through the residual connection); the kept
    terms keep the softmax weights of all K selected logits (no renormalisation)."""
    kept = capacity_dispatch(sel, _f64(Wg).shape[1], cap)["kept"]
    return forward_kept(x, Wg, W1, W3, W2, sel, kept)


def forward_kept(x, Wg, W1: ArrayOrGetter, W3: ArrayOrGetter, W2: ArrayOrGetter, sel: np.ndarray,
                 kept: np.ndarray) -> np.ndarray:
    """forward_capacity for a given kept mask (rows of a larger batch can be
    evaluated with the mask the whole batch's dispatch produced)."""
    x = _f64(x)
    logits = router_logits(x, Wg)
    sel = np.asarray(sel, dtype=np.int64)
    w = gate_weights(logits, sel)
    T = x.shape[0]
    y = np.zeros((T, x.shape[1]))
    for e in range(_f64(Wg).shape[1]):
        hit = (sel == e) & kept
        rows = np.nonzero(hit.any(axis=1))[0]
        if rows.size == 0:
            continue
        out = expert_swiglu(x[rows], _expert(W1, e), _expert(W3, e), _expert(W2, e))
        y[rows] += (w[rows] * hit[rows]).sum(axis=1)[:, None] * out
    return y


# ------------------------------------------------- 4-bit expert weights ---
# The explainer (Part 4, "Why total and active both matter") sizes the model at
# 16 bits and at 4 bits per parameter but gives no format.  The format here:
#   groups of Q4_GROUP = 128 consecutive reduction indices r, per column c;
#   scale s[e][g][c] = bf16_rne(max_r |W[e][r][c]| / 7) (fp32 division);
#   code q = clamp(rint(W / s), -7, 7) with the division in fp32 (q = 0 where
#   s = 0); dequantised weight q * s.
# Storage of the codes (nibble u = q + 8), per expert e: group b = r // 128,
# column tile t = c // 16, chunk g = (r % 128) // 32, column c % 16, then 16
# bytes = 4 little-endian 32-bit words; word m holds r = 128b + 32g + 8m + i
# for i = 0..7, element i = 2k in bits 4k..4k+3 and element i = 2k + 1 in bits
# 16+4k..16+4k+3.  (C is a multiple of 16.)  So one group of 16 columns is one
# contiguous kilobyte, and one group of all C columns C*64 contiguous bytes.
Q4_GROUP = 128


def bf16_round(a) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def quantize_q4(W) -> tuple:
    """W [n][R][C] (float32 values) -> codes int8 [n][R][C], scales float32
    [n][R/128][C] (bf16 values).  All arithmetic in float32, as specified."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    n, R, C = W.shape
    G = R // Q4_GROUP
    Wg = W.reshape(n, G, Q4_GROUP, C)
    amax = np.abs(Wg).max(axis=2)
    scale = bf16_round(amax / np.float32(7.0))
    nz = scale > 0
    den = np.where(nz, scale, np.float32(1.0))[:, :, None, :]
    q = np.rint(Wg / den)
    q = np.where(nz[:, :, None, :], q, np.float32(0.0))
    q = np.clip(q, -7, 7).astype(np.int8)
    return q.reshape(n, R, C), scale


def dequantize_q4(codes, scales) -> np.ndarray:
    """codes [n][R][C], scales [n][R/128][C] -> fp64 weights q * s."""
    n, R, C = codes.shape
    q = np.asarray(codes, dtype=np.float64).reshape(n, R // Q4_GROUP, Q4_GROUP, C)
    return (q * np.asarray(scales, dtype=np.float64)[:, :, None, :]).reshape(n, R, C)


def unpack_q4(packed, n: int, R: int, C: int) -> np.ndarray:
    """Packed code bytes (the storage described above) -> codes int8 [n][R][C]."""
    # words[e][b][t][g][c16][m]
    words = np.ascontiguousarray(packed, dtype=np.uint8).view("<u4").reshape(n, R // 128, C // 16, 4, 16, 4)
    codes = np.empty((n, R, C), dtype=np.int8)
    view = codes.reshape(n, R // 128, 4, 4, 8, C // 16, 16)  # [e][b][g][m][i][t][c16]
    for i in range(8):
        shift = 4 * (i // 2) + 16 * (i % 2)
        u = ((words >> np.uint32(shift)) & np.uint32(15)).astype(np.int16) - 8
        # r = 128b + 32g + 8m + i, c = 16t + c16
        view[:, :, :, :, i, :, :] = u.transpose(0, 1, 3, 5, 2, 4)
    return codes


def sigmoid(z) -> np.ndarray:
    z = _f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z) -> np.ndarray:
    """SiLU (Swish with beta = 1): z * sigmoid(z)."""
    z = _f64(z)
    return z * sigmoid(z)


def expert_swiglu(X, W1e, W3e, W2e) -> np.ndarray:
    """One expert on a batch of rows: expand with two d x f matrices, gate one
    with SiLU, multiply, compress with the f x d matrix (the reading of SwiGLU
    stated in the module header)."""
    X = _f64(X)
    a = X @ _f64(W1e)
    b = X @ _f64(W3e)
    return (silu(a) * b) @ _f64(W2e)


# --------------------------------------------------------------- forward ---

def forward_with_selection(x, Wg, W1: ArrayOrGetter, W3: ArrayOrGetter, W2: ArrayOrGetter,
                           sel: np.ndarray) -> np.ndarray:
    """Steps 3-4 of the walk-through for a given selection: weights are the
    softmax over the selected logits, each selected expert runs on the token on
    its own, and the outputs are summed with those weights.  Experts that no
    token selected are never evaluated (so their weights are never read)."""
    x = _f64(x)
    logits = router_logits(x, Wg)
    sel = np.asarray(sel, dtype=np.int64)
    w = gate_weights(logits, sel)
    T = x.shape[0]
    n = _f64(Wg).shape[1]
    y = None
    for e in range(n):
        hit = sel == e
        rows = np.nonzero(hit.any(axis=1))[0]
        if rows.size == 0:
            continue
        out = expert_swiglu(x[rows], _expert(W1, e), _expert(W3, e), _expert(W2, e))
        if y is None:
            y = np.zeros((T, out.shape[1]))
        y[rows] += (w[rows] * hit[rows]).sum(axis=1)[:, None] * out
    if y is None:
        y = np.zeros((T, x.shape[1]))
    return y


def forward(x, Wg, W1: ArrayOrGetter, W3: ArrayOrGetter, W2: ArrayOrGetter, K: int) -> np.ndarray:
    """The layer: route every token (steps 1-3), then run and blend its K experts."""
    sel, _, _ = topk_select(router_logits(x, Wg), K)
    return forward_with_selection(x, Wg, W1, W3, W2, sel)


def forward_mask_form(x, Wg, W1: ArrayOrGetter, W3: ArrayOrGetter, W2: ArrayOrGetter,
                      K: int) -> np.ndarray:
    """The layer equation read literally: logits outside the top K are set to
    -inf, a softmax runs over all n experts, and every expert with a non-zero
    gate contributes gate * expert(x).  Top-K membership is decided here by
    rank counting (a logit is kept when fewer than K logits beat it, a tie
    being beaten by the lower index), independently of topk_select."""
    x = _f64(x)
    logits = router_logits(x, Wg)
    T, n = logits.shape
    keep = np.zeros((T, n), dtype=bool)
    for i in range(n):
        li = logits[:, i:i + 1]
        beats = (logits > li) | ((logits == li) & (np.arange(n)[None, :] < i))
        keep[:, i] = beats.sum(axis=1) < K
    masked = np.where(keep, logits, -np.inf)
    g = np.exp(masked - masked.max(axis=1, keepdims=True))
    g = g / g.sum(axis=1, keepdims=True)
    y = np.zeros_like(x)
    for i in range(n):
        rows = np.nonzero(g[:, i] > 0)[0]
        if rows.size == 0:
            continue
        out = expert_swiglu(x[rows], _expert(W1, i), _expert(W3, i), _expert(W2, i))
        y[rows] += g[rows, i][:, None] * out
    return y


# ------------------------------------------------- parameter arithmetic ---

def mixtral_param_counts(d: int = 4096, f: int = 14336, layers: int = 32, n: int = 8, K: int = 2,
                         vocab: int = 32000, attn_per_layer: int = 42_000_000) -> dict:
    """The parameter count of Part 4 ("Why 8x7B Is Not 56B") of the explainer:
    three d x f matrices per expert, n experts per layer; attention (about 42M
    per layer, taken as printed), two d x vocab embedding tables and a d x n
    router per layer are shared.  Active = shared + K experts per layer."""
    per_expert = 3 * d * f
    experts = per_expert * n * layers
    attention = attn_per_layer * layers
    embeddings = 2 * vocab * d
    routers = d * n * layers
    shared = attention + embeddings + routers
    return dict(per_expert=per_expert, experts=experts, attention=attention,
                embeddings=embeddings, routers=routers, shared=shared,
                total=experts + shared, active=shared + K * per_expert * layers,
                two_experts_all_layers=K * per_expert * layers,
                naive=n * 7_000_000_000)
