"""Plain, slow CPU reference of one MoE layer, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function below is
written from its definition, in float64 unless a precision is stated, with
NumPy matmul / sort / cumsum as the only library steps.

Citations use [MCore-MoE] = the page "Scalable Training of Mixture-of-Experts
Models with Megatron Core", section 2 (Megatron-Core MoE Architecture), whose
four bullets Route / Dispatch / Expert Computation / Combine define the four
stages, and section 5 (Reduced-Precision Training), bullet "Selective
precision" (the router stays in FP32).

Readings where the page is silent (each is also listed in the design notes):
  * Selection key: z = fp32(logit + bias).  Softmax and sigmoid are strictly
    increasing, so the top-k of the probabilities is the top-k of z; ordering
    on z avoids ulp differences of exp between implementations.
  * Ties: equal keys go to the lower expert index; the k slots of a token are
    listed by (key descending, index ascending).
  * Bias: a per-expert constant added to the logits before scoring; it gets
    no gradient.
  * Within an expert's segment, rows are in ascending token order (stable).
  * SwiGLU expert: h = silu(x W1) * (x W3), y = h W2, silu(a) = a * sigmoid(a);
    W13 = [W1 | W3] concatenated along the ffn axis.
  * Shared expert: same SwiGLU form, weight 1, added after the routed sum.
  * Scaling factor on the routed sum: 1.
"""

import math

import numpy as np

SOFTMAX = "softmax"
SIGMOID = "sigmoid"

__all__ = [
    "SOFTMAX", "SIGMOID", "f64", "router_logits", "select_topk", "gates", "dispatch_map",
    "route", "route_replay", "canonical_experts", "capacity_of", "apply_capacity", "aux_loss",
    "sigmoid_spec", "selection_keys", "route_expert_bias", "expert_bias_update", "pad_to_max",
    "route_bwd",
    "router_logits_bwd", "permute", "permute_bwd",
    "grouped_gemm_fwd", "grouped_gemm_dgrad", "grouped_gemm_wgrad", "sigmoid", "silu",
    "swiglu", "swiglu_bwd", "unpermute_combine", "unpermute_combine_bwd",
    "expert_ffn", "expert_ffn_bwd", "layer_forward", "layer_backward",
    "expert_wgrad_columns", "layer_forward_gated", "layer_backward_gated",
]


def f64(a):
    """Exact widening of an fp32/bf16-valued array to float64."""
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Route  ([MCore-MoE] section 2, Route; section 5, Selective precision)
# ---------------------------------------------------------------------------

def router_logits(x, w_r, logit_bias=None):
    """Token hidden states -> expert logits, kept in fp32.

    logits = x @ W_r evaluated in float64 and rounded once to fp32; a bias, if
    given, is then added with one IEEE fp32 addition (round to nearest even).
    The result is the fp32 selection key z of every later step.
    """
    l32 = (f64(x) @ f64(w_r)).astype(np.float32)
    if logit_bias is not None:
        l32 = (l32 + np.asarray(logit_bias, dtype=np.float32)).astype(np.float32)
    return l32


def select_topk(z, k):
    """The k highest-scoring experts of each token.

    Order: key descending, then expert index ascending, so that among equal
    keys the lower expert index wins.  Returns int32 [T, k].
    """
    z = np.asarray(z, dtype=np.float32)
    assert np.all(np.isfinite(z)), "non-finite router logits are a caller error"
    T, E = z.shape
    assert 1 <= k <= E
    idx = np.broadcast_to(np.arange(E), (T, E))
    # lexsort sorts by the last key first: primary -z (descending z), then index.
    # -(+0.0) and -(-0.0) compare equal, so signed zeros tie as they should.
    order = np.lexsort((idx, -z.astype(np.float64)), axis=-1)
    return order[:, :k].astype(np.int32)


def sigmoid(v):
    v = f64(v)
    return 1.0 / (1.0 + np.exp(-v))


def gates(z, topk_idx, score, renorm):
    """Routing weights of the chosen experts (float64).

    softmax, renorm   : softmax over the chosen keys (= full softmax
                        renormalised over the chosen k).
    softmax, no renorm: full softmax over all E experts, read at the chosen.
    sigmoid, renorm   : sigmoid(z_j) / sum over chosen of sigmoid.
    sigmoid, no renorm: sigmoid(z_j).
    """
    z = f64(z)
    zk = np.take_along_axis(z, topk_idx.astype(np.int64), axis=1)
    if score == SOFTMAX:
        if renorm:
            ex = np.exp(zk - zk.max(axis=1, keepdims=True))
            return ex / ex.sum(axis=1, keepdims=True)
        ex = np.exp(z - z.max(axis=1, keepdims=True))
        p = ex / ex.sum(axis=1, keepdims=True)
        return np.take_along_axis(p, topk_idx.astype(np.int64), axis=1)
    if score == SIGMOID:
        s = sigmoid(zk)
        return s / s.sum(axis=1, keepdims=True) if renorm else s
    raise ValueError(score)


def dispatch_map(topk_idx, E):
    """Per-expert counts, segment offsets and the permutation into
    expert-contiguous order ([MCore-MoE] section 2, Dispatch: tokens are
    permuted by destination expert).

    Stable counting sort: experts in ascending order, and inside each
    expert's segment the tokens in ascending order.  Returns
      counts   int64 [E]      number of (token, slot) pairs routed to e
      offsets  int64 [E+1]    offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e]
      dst_row  int32 [T, k]   row of the permuted matrix holding (t, j)
      src_token int32 [T*k]   token held by each permuted row
    """
    T, k = topk_idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for e in topk_idx.ravel():
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    dst_row = np.full((T, k), -1, dtype=np.int32)
    src_token = np.full(T * k, -1, dtype=np.int32)
    r = 0
    for e in range(E):
        ts, js = np.nonzero(topk_idx == e)  # row-major scan: ascending t
        n = len(ts)
        src_token[r:r + n] = ts
        dst_row[ts, js] = r + np.arange(n)
        r += n
    assert r == T * k
    return counts, offsets, dst_row, src_token


def route(z, k, score, renorm):
    """Route stage on fp32 keys z [T, E]: selection, weights and the dispatch
    map.  Dropless: every (token, slot) pair gets a row."""
    z = np.asarray(z, dtype=np.float32)
    idx = select_topk(z, k)
    w = gates(z, idx, score, renorm)
    counts, offsets, dst_row, src_token = dispatch_map(idx, z.shape[1])
    return dict(topk_idx=idx, topk_w=w, counts=counts, offsets=offsets,
                dst_row=dst_row, src_token=src_token)


def canonical_experts(topk_idx, E):
    """Given experts per token, made usable as a routing: a slot whose expert
    is outside [0, E) or repeats an earlier slot of its token is replaced, in
    slot order, by the smallest expert the token does not use yet.  (The pages
    say nothing of replayed routings; this keeps every token's k experts
    distinct, so the dispatch map is a bijection.)  Returns (experts, changed)."""
    idx = np.array(topk_idx, dtype=np.int64, copy=True)
    T, k = idx.shape
    changed = False
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if 0 <= e < E and e not in idx[t, :j]:
                continue
            others = {int(idx[t, s]) for s in range(k) if s != j}
            idx[t, j] = min(c for c in range(E) if c not in others)
            changed = True
    return idx.astype(np.int32), changed


def route_replay(z, topk_idx, score, renorm):
    """Route stage with the experts given (a recorded or forced assignment):
    the routing weights and the dispatch map of ``route`` for those experts,
    in the given slot order (after ``canonical_experts``)."""
    z = np.asarray(z, dtype=np.float32)
    idx, changed = canonical_experts(topk_idx, z.shape[1])
    w = gates(z, idx, score, renorm)
    counts, offsets, dst_row, src_token = dispatch_map(idx, z.shape[1])
    return dict(topk_idx=idx, topk_w=w, counts=counts, offsets=offsets,
                dst_row=dst_row, src_token=src_token, changed=changed)


# ---------------------------------------------------------------------------
# Selection-only expert bias: the auxiliary-loss-free biasing that the page's
# section 7 (Load Balancing) lists among its balancing strategies, without a
# formula.  Reading: a per-expert bias b is added to the sigmoid scores for
# the choice of the top k only; the routing weights stay the unbiased
# sigmoid scores of the chosen experts (renormalised over the k); after each
# step b moves by a fixed rate against each expert's load imbalance.
# ---------------------------------------------------------------------------

# Constants of the specified sigmoid (fp32 values).  ln 2 in two parts: the
# high part has 15 significant bits, so n * LN2_HI is exact for |n| < 2^8.
_SPEC_LOG2E = np.float32(1.44269504)
_SPEC_LN2_HI = np.float32(0.693145751953125)
_SPEC_LN2_LO = np.float32(1.42860677e-06)
_SPEC_CLAMP = np.float32(87.0)
# exp(r) on |r| <= ln2 / 2: Taylor coefficients 1/i!, i = 0..7, in fp32
_SPEC_EXP_C = [np.float32(1.0 / math.factorial(i)) for i in range(8)]


def sigmoid_spec(z):
    """A sigmoid whose every step is one correctly rounded fp32 operation, so
    that two implementations (this one and the GPU's) agree bit for bit --
    the selection keys built from it decide integer results.

      x = clamp(-z, -87, 87)               (keeps exp(x) and the result normal)
      n = round_half_even(x * log2e)        (Cody-Waite reduction)
      r = (x - n * LN2_HI) - n * LN2_LO
      p = Horner(c7 .. c0) at r, each step p = p * r + c (a multiply, then an
          add: no fused multiply-add)
      e = p * 2^n                            (exact: p * 2^n stays normal)
      sigma = 1 / (1 + e)

    fp32 NumPy arithmetic rounds every operation to nearest even, which is
    the specification."""
    z = np.asarray(z, dtype=np.float32)
    x = np.clip(-z, -_SPEC_CLAMP, _SPEC_CLAMP).astype(np.float32)
    n = np.rint(x * _SPEC_LOG2E).astype(np.float32)
    r = ((x - n * _SPEC_LN2_HI) - n * _SPEC_LN2_LO).astype(np.float32)
    p = np.full_like(r, _SPEC_EXP_C[7])
    for c in reversed(_SPEC_EXP_C[:7]):
        p = (p * r).astype(np.float32)
        p = (p + c).astype(np.float32)
    e = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    return (np.float32(1.0) / (np.float32(1.0) + e)).astype(np.float32)


def selection_keys(z, sel_bias):
    """key[t, e] = sigmoid_spec(z[t, e]) + b[e], one fp32 addition."""
    return (sigmoid_spec(z) + np.asarray(sel_bias, dtype=np.float32)).astype(np.float32)


def route_expert_bias(z, sel_bias, k, renorm):
    """Route with a selection-only expert bias on sigmoid scores: the top k
    by ``selection_keys`` (ties and slot order as in ``select_topk``), the
    routing weights from the unbiased scores sigmoid_spec(z) of the chosen
    experts (divided by their sum in float64 when ``renorm``), and the
    dispatch map of ``route``."""
    z = np.asarray(z, dtype=np.float32)
    idx = select_topk(selection_keys(z, sel_bias), k)
    s = f64(np.take_along_axis(sigmoid_spec(z), idx.astype(np.int64), axis=1))
    w = s / s.sum(axis=1, keepdims=True) if renorm else s
    counts, offsets, dst_row, src_token = dispatch_map(idx, z.shape[1])
    return dict(topk_idx=idx, topk_w=w, counts=counts, offsets=offsets,
                dst_row=dst_row, src_token=src_token)


def expert_bias_update(sel_bias, counts, rate):
    """b[e] += rate * sign(mean load - load[e]) (in fp32; one addition of
    +-rate or 0): experts that received more than the mean of the (token,
    slot) pairs become less attractive.  The sign is taken exactly, from the
    integers sum(counts) - E * counts[e]."""
    c = np.asarray(counts, dtype=np.int64)
    sgn = np.sign(c.sum() - c.size * c).astype(np.float32)
    step = (np.float32(rate) * sgn).astype(np.float32)
    return (np.asarray(sel_bias, dtype=np.float32) + step).astype(np.float32)


def capacity_of(capacity_factor, T, k, E):
    """Rows each expert may keep: ceil(capacity_factor * T * k / E) (the
    pages name capacity-limited dropping without a formula; this is the usual
    definition, with the factor as the workload's knob)."""
    return int(math.ceil(capacity_factor * T * k / E))


def apply_capacity(r, capacity):
    """Capacity-limited dropping of a routing ``r`` (a ``route`` or
    ``route_replay`` result): each expert keeps the (token, slot) pairs of its
    ``capacity`` lowest tokens and drops the rest; dropped pairs get no row
    (dst_row -1) and contribute nothing.  The routing weights are unchanged.
    Written as its own scan over tokens, not from the dropless map."""
    idx = r["topk_idx"]
    T, k = idx.shape
    E = len(r["counts"])
    kept = np.zeros(E, dtype=np.int64)
    keep = np.zeros((T, k), dtype=bool)
    for t in range(T):                   # tokens in ascending order
        for j in range(k):
            e = idx[t, j]
            if kept[e] < capacity:
                kept[e] += 1
                keep[t, j] = True
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    dst_row = np.full((T, k), -1, dtype=np.int32)
    src_token = np.full(int(offsets[-1]), -1, dtype=np.int32)
    nxt = offsets[:-1].copy()
    for t in range(T):
        for j in range(k):
            if keep[t, j]:
                e = idx[t, j]
                dst_row[t, j] = nxt[e]
                src_token[nxt[e]] = t
                nxt[e] += 1
    out = dict(r)
    out.update(counts=kept, offsets=offsets, dst_row=dst_row, src_token=src_token,
               capacity=capacity)
    return out


def pad_to_max(r, capacity):
    """Pad-to-max (section 7, Load Balancing: variable expert counts made
    into static shapes): every expert's segment gets the same size C =
    ``capacity``, expert e owning rows e*C .. e*C + C - 1; its kept pairs (the
    first C in token order, as ``apply_capacity``) fill the segment's first
    rows in token order and the rest of the segment is padding (src_token -1,
    zero rows downstream).  Offsets are the static e*C."""
    kept = apply_capacity(r, capacity)
    E = len(kept["counts"])
    offsets = np.arange(E + 1, dtype=np.int64) * capacity
    dst_row = np.full_like(kept["dst_row"], -1)
    src_token = np.full(E * capacity, -1, dtype=np.int32)
    T, k = dst_row.shape
    for t in range(T):
        for j in range(k):
            row = kept["dst_row"][t, j]
            if row < 0:
                continue
            e = int(kept["topk_idx"][t, j])
            rank = row - kept["offsets"][e]
            dst_row[t, j] = e * capacity + rank
            src_token[e * capacity + rank] = t
    out = dict(kept)
    out.update(offsets=offsets, dst_row=dst_row, src_token=src_token, padded_to=capacity)
    return out


def aux_loss(z, counts, k, score, coeff):
    """Auxiliary load-balancing loss (named by the pages among the balancing
    strategies, without a formula; this is the usual form):
      L = coeff * E * sum_e f_e P_e,  f_e = counts_e / (T k),
      P_e = mean over tokens of p[t, e], the router's probabilities: the
      softmax of the keys, or the sigmoid scores normalised over the E experts.
    Returns (L, dL/dz) with f held fixed (the counts come from a discrete
    selection)."""
    z = f64(z)
    T, E = z.shape
    f = f64(counts) / (T * k)
    if score == SOFTMAX:
        ex = np.exp(z - z.max(axis=1, keepdims=True))
        p = ex / ex.sum(axis=1, keepdims=True)
    else:
        s = sigmoid(z)
        p = s / s.sum(axis=1, keepdims=True)
    P = p.mean(axis=0)
    L = coeff * E * float(f @ P)
    g = coeff * E * f / T                    # dL/dp[t, e]
    pg = (p * g).sum(axis=1, keepdims=True)
    if score == SOFTMAX:
        dz = p * (g - pg)
    else:
        dz = s * (1.0 - s) / s.sum(axis=1, keepdims=True) * (g - pg)
    return L, dz


def route_bwd(z, topk_idx, topk_w, d_topk_w, score, renorm):
    """Gradient of the routing weights with respect to the keys z (= logits,
    the bias being constant).  The discrete selection itself carries no
    gradient.  With g = sum over chosen of w_l * dw_l:
      softmax, renorm   : dz_j = w_j (dw_j - g) on chosen, 0 elsewhere
      softmax, no renorm: dz_e = p_e (G_e - g) for every e, G_e = dw_j if
                          e is chosen slot j else 0
      sigmoid, renorm   : dz_j = (dw_j - g) / S * s_j (1 - s_j), S = sum s
      sigmoid, no renorm: dz_j = dw_j * s_j (1 - s_j)
    """
    z = f64(z)
    T, E = z.shape
    idx = topk_idx.astype(np.int64)
    w = f64(topk_w)
    dw = f64(d_topk_w)
    dz = np.zeros((T, E))
    g = (w * dw).sum(axis=1, keepdims=True)
    if score == SOFTMAX:
        if renorm:
            np.put_along_axis(dz, idx, w * (dw - g), axis=1)
        else:
            ex = np.exp(z - z.max(axis=1, keepdims=True))
            p = ex / ex.sum(axis=1, keepdims=True)
            G = np.zeros((T, E))
            np.put_along_axis(G, idx, dw, axis=1)
            dz = p * (G - g)
    elif score == SIGMOID:
        s = sigmoid(np.take_along_axis(z, idx, axis=1))
        if renorm:
            S = s.sum(axis=1, keepdims=True)
            np.put_along_axis(dz, idx, (dw - g) / S * s * (1.0 - s), axis=1)
        else:
            np.put_along_axis(dz, idx, dw * s * (1.0 - s), axis=1)
    else:
        raise ValueError(score)
    return dz


def router_logits_bwd(x, w_r, dz):
    """dW_r = x^T dz and the router's share of dx, dz W_r^T (float64)."""
    return f64(x).T @ f64(dz), f64(dz) @ f64(w_r).T


# ---------------------------------------------------------------------------
# Dispatch ([MCore-MoE] section 2, Dispatch) and Combine (section 2, Combine)
# ---------------------------------------------------------------------------

def permute(x, src_token):
    """Rows in expert-contiguous order: X_perm[r] = x[src_token[r]]."""
    return np.asarray(x)[np.asarray(src_token, dtype=np.int64)]


def permute_bwd(dx_perm, dst_row, addends=()):
    """Adjoint of ``permute``: dx[t] = sum_j dX_perm[dst_row[t, j]] (+ addends)."""
    dx_perm = f64(dx_perm)
    T, k = dst_row.shape
    dx = np.zeros((T, dx_perm.shape[1]))
    for t in range(T):
        for j in range(k):
            dx[t] += dx_perm[dst_row[t, j]]
    for a in addends:
        dx += f64(a)
    return dx


def unpermute_combine(y_perm, topk_w, dst_row, shared_y=None):
    """out[t] = sum_j w[t, j] * Y[dst_row[t, j]] (+ shared expert output):
    tokens return to sequence order weighted by their routing weights."""
    y_perm = f64(y_perm)
    w = f64(topk_w)
    T, k = dst_row.shape
    out = np.zeros((T, y_perm.shape[1]))
    for t in range(T):
        for j in range(k):
            out[t] += w[t, j] * y_perm[dst_row[t, j]]
    if shared_y is not None:
        out += f64(shared_y)
    return out


def unpermute_combine_bwd(dout, y_perm, topk_w, dst_row):
    """Adjoint of ``unpermute_combine``:
    dY[dst_row[t, j]] = w[t, j] * dout[t],  d_w[t, j] = <dout[t], Y[dst_row[t, j]]>.
    (The shared expert's output gradient is dout itself.)"""
    dout = f64(dout)
    y_perm = f64(y_perm)
    w = f64(topk_w)
    T, k = dst_row.shape
    dy = np.zeros_like(y_perm)
    dw = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            r = dst_row[t, j]
            dy[r] = w[t, j] * dout[t]
            dw[t, j] = dout[t] @ y_perm[r]
    return dy, dw


# ---------------------------------------------------------------------------
# Expert computation ([MCore-MoE] section 2, Expert Computation)
# ---------------------------------------------------------------------------

def grouped_gemm_fwd(A, B, offsets):
    """C[rows of g] = A[rows of g] @ B[g]; rows of g = [offsets[g], offsets[g+1])."""
    A = f64(A)
    G = len(offsets) - 1
    C = np.zeros((A.shape[0], B.shape[2]))
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        C[lo:hi] = A[lo:hi] @ f64(B[g])
    return C


def grouped_gemm_dgrad(dC, B, offsets):
    """dA[rows of g] = dC[rows of g] @ B[g]^T."""
    dC = f64(dC)
    G = len(offsets) - 1
    dA = np.zeros((dC.shape[0], B.shape[1]))
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        dA[lo:hi] = dC[lo:hi] @ f64(B[g]).T
    return dA


def grouped_gemm_wgrad(A, dC, offsets):
    """dB[g] = A[rows of g]^T @ dC[rows of g] (zero for an empty group)."""
    A = f64(A)
    dC = f64(dC)
    G = len(offsets) - 1
    dB = np.zeros((G, A.shape[1], dC.shape[1]))
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        dB[g] = A[lo:hi].T @ dC[lo:hi]
    return dB


def silu(a):
    a = f64(a)
    # exp(-a) overflows to inf for a below about -709; a / inf is then the
    # function's limit (-0.0), so the overflow is expected and not reported
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu(ab):
    """H = silu(A) * B with A = ab[:, :f] and B = ab[:, f:]."""
    ab = f64(ab)
    f = ab.shape[1] // 2
    return silu(ab[:, :f]) * ab[:, f:]


def swiglu_bwd(dh, ab):
    """dA = dH * B * s (1 + A (1 - s)),  dB = dH * silu(A),  s = sigmoid(A)."""
    ab = f64(ab)
    dh = f64(dh)
    f = ab.shape[1] // 2
    a, b = ab[:, :f], ab[:, f:]
    s = sigmoid(a)
    return np.concatenate([dh * b * s * (1.0 + a * (1.0 - s)), dh * a * s], axis=1)


def expert_ffn(x_t, w13_e, w2_e):
    """One SwiGLU expert on one token row: returns (a, b, h, y)."""
    x_t = f64(x_t)
    w13_e = f64(w13_e)
    f = w13_e.shape[1] // 2
    a = x_t @ w13_e[:, :f]
    b = x_t @ w13_e[:, f:]
    h = silu(a) * b
    return a, b, h, h @ f64(w2_e)


def expert_ffn_bwd(x_t, w13_e, w2_e, a, b, h, dy):
    """Backward of ``expert_ffn`` for one row: returns (dx_t, dW13_e, dW2_e)."""
    x_t = f64(x_t)
    w13_e = f64(w13_e)
    w2_e = f64(w2_e)
    dh = dy @ w2_e.T
    s = sigmoid(a)
    da = dh * b * s * (1.0 + a * (1.0 - s))
    db = dh * a * s
    dab = np.concatenate([da, db])
    return dab @ w13_e.T, np.outer(x_t, dab), np.outer(h, dy)


def layer_forward(x, w_r, w13, w2, k, score, renorm, logit_bias=None,
                  shared=None, z=None, given_experts=None, capacity=None):
    """The four-stage forward pass as a per-token loop over each token's k
    experts (the one-expert-at-a-time view of [MCore-MoE] section 2, Expert
    Computation).  ``shared`` = (ws13 [d, 2fs], ws2 [fs, d]) or None.
    ``z`` may give the fp32 keys directly; by default they are computed with
    ``router_logits``.  ``given_experts`` [T, k] replays a routing
    (``route_replay``) instead of selecting the top k; ``capacity`` drops
    what exceeds it (``apply_capacity``).  Returns a cache dict consumed by
    ``layer_backward``."""
    x = f64(x)
    T, d = x.shape
    if z is None:
        z = router_logits(x, w_r, logit_bias)
    if given_experts is None:
        r = route(z, k, score, renorm)
    else:
        r = route_replay(z, given_experts, score, renorm)
    if capacity is not None:
        r = apply_capacity(r, capacity)
    idx, w = r["topk_idx"], r["topk_w"]
    out = np.zeros((T, d))
    acts = {}
    for t in range(T):
        for j in range(k):
            if r["dst_row"][t, j] < 0:
                continue  # dropped
            e = int(idx[t, j])
            a, b, h, y = expert_ffn(x[t], w13[e], w2[e])
            acts[(t, j)] = (a, b, h, y)
            out[t] += w[t, j] * y
    shared_acts = None
    if shared is not None:
        shared_acts = []
        for t in range(T):
            a, b, h, y = expert_ffn(x[t], shared[0], shared[1])
            shared_acts.append((a, b, h, y))
            out[t] += y
    return dict(out=out, z=z, route=r, acts=acts, shared_acts=shared_acts,
                x=x, w_r=w_r, w13=w13, w2=w2, k=k, score=score, renorm=renorm,
                shared=shared)


def layer_backward(cache, dout):
    """Backward of ``layer_forward`` by the chain rule, the same per-token
    loop in reverse.  Returns dx, d_logits (= dz), dW_r, dW13, dW2 and, with a
    shared expert, dWs13 and dWs2."""
    dout = f64(dout)
    x, w13, w2 = cache["x"], cache["w13"], cache["w2"]
    r = cache["route"]
    idx, w = r["topk_idx"], r["topk_w"]
    T, k = idx.shape
    dx = np.zeros_like(x)
    dW13 = np.zeros(np.shape(w13))
    dW2 = np.zeros(np.shape(w2))
    dw = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            if (t, j) not in cache["acts"]:
                continue  # dropped: no output, no gradient
            e = int(idx[t, j])
            a, b, h, y = cache["acts"][(t, j)]
            dw[t, j] = dout[t] @ y
            dxt, dw13, dw2 = expert_ffn_bwd(x[t], w13[e], w2[e], a, b, h, w[t, j] * dout[t])
            dx[t] += dxt
            dW13[e] += dw13
            dW2[e] += dw2
    res = {}
    if cache["shared"] is not None:
        ws13, ws2 = cache["shared"]
        dWs13 = np.zeros(np.shape(ws13))
        dWs2 = np.zeros(np.shape(ws2))
        for t in range(T):
            a, b, h, _ = cache["shared_acts"][t]
            dxt, dw13, dw2 = expert_ffn_bwd(x[t], ws13, ws2, a, b, h, dout[t])
            dx[t] += dxt
            dWs13 += dw13
            dWs2 += dw2
        res.update(dWs13=dWs13, dWs2=dWs2)
    dz = route_bwd(cache["z"], idx, w, dw, cache["score"], cache["renorm"])
    dWr, dx_router = router_logits_bwd(x, cache["w_r"], dz)
    dx += dx_router
    res.update(dx=dx, d_logits=dz, dW_r=dWr, dW13=dW13, dW2=dW2, d_topk_w=dw)
    return res


def layer_forward_gated(x, w_r, w13, w2, k, score, renorm, logit_bias=None,
                        shared=None, z=None, given_experts=None, capacity=None):
    """The forward with each routing weight applied inside its expert, before
    W2: y'_tj = (w_tj h_tj) W2 and out_t = sum_j y'_tj (+ shared), an
    unweighted combine.  This is the memory-saving rearrangement of the
    permutation the pages' section 4 (Memory) mentions -- the plain reading:
    by linearity it moves the weight across W2 without extra compute, and the
    backward then needs no Y.  Equal to ``layer_forward`` up to rounding."""
    x = f64(x)
    T, d = x.shape
    if z is None:
        z = router_logits(x, w_r, logit_bias)
    r = (route(z, k, score, renorm) if given_experts is None
         else route_replay(z, given_experts, score, renorm))
    if capacity is not None:
        r = apply_capacity(r, capacity)
    idx, w = r["topk_idx"], r["topk_w"]
    out = np.zeros((T, d))
    acts = {}
    for t in range(T):
        for j in range(k):
            if r["dst_row"][t, j] < 0:
                continue  # dropped
            e = int(idx[t, j])
            f = w13[e].shape[1] // 2
            a = x[t] @ f64(w13[e][:, :f])
            b = x[t] @ f64(w13[e][:, f:])
            h = silu(a) * b
            hg = w[t, j] * h
            out[t] += hg @ f64(w2[e])
            acts[(t, j)] = (a, b, h, hg)
    shared_acts = None
    if shared is not None:
        shared_acts = []
        for t in range(T):
            a, b, h, y = expert_ffn(x[t], shared[0], shared[1])
            shared_acts.append((a, b, h, y))
            out[t] += y
    return dict(out=out, z=z, route=r, acts=acts, shared_acts=shared_acts,
                x=x, w_r=w_r, w13=w13, w2=w2, k=k, score=score, renorm=renorm,
                shared=shared)


def layer_backward_gated(cache, dout):
    """Backward of ``layer_forward_gated``.  For each (t, j): dy' = dout_t
    (the combine is unweighted); dh' = dy' W2^T; the routing-weight gradient
    is <dh', h> over the ffn axis; dh = w dh' goes through SwiGLU' as usual;
    dW2 gets (w h)^T dy'.  Same outputs as ``layer_backward``."""
    dout = f64(dout)
    x, w13, w2 = cache["x"], cache["w13"], cache["w2"]
    r = cache["route"]
    idx, w = r["topk_idx"], r["topk_w"]
    T, k = idx.shape
    dx = np.zeros_like(x)
    dW13 = np.zeros(np.shape(w13))
    dW2 = np.zeros(np.shape(w2))
    dw = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            if (t, j) not in cache["acts"]:
                continue  # dropped
            e = int(idx[t, j])
            f = w13[e].shape[1] // 2
            a, b, h, hg = cache["acts"][(t, j)]
            dhg = f64(w2[e]) @ dout[t]
            dw[t, j] = dhg @ h
            dh = w[t, j] * dhg
            s = sigmoid(a)
            da = dh * b * s * (1.0 + a * (1.0 - s))
            db = dh * a * s
            dW2[e] += np.outer(hg, dout[t])
            dW13[e][:, :f] += np.outer(x[t], da)
            dW13[e][:, f:] += np.outer(x[t], db)
            dx[t] += f64(w13[e][:, :f]) @ da + f64(w13[e][:, f:]) @ db
    res = {}
    if cache["shared"] is not None:
        ws13, ws2 = cache["shared"]
        dWs13 = np.zeros(np.shape(ws13))
        dWs2 = np.zeros(np.shape(ws2))
        for t in range(T):
            a, b, h, _ = cache["shared_acts"][t]
            dxt, dw13, dw2 = expert_ffn_bwd(x[t], ws13, ws2, a, b, h, dout[t])
            dx[t] += dxt
            dWs13 += dw13
            dWs2 += dw2
        res.update(dWs13=dWs13, dWs2=dWs2)
    dz = route_bwd(cache["z"], idx, w, dw, cache["score"], cache["renorm"])
    dWr, dx_router = router_logits_bwd(x, cache["w_r"], dz)
    dx += dx_router
    res.update(dx=dx, d_logits=dz, dW_r=dWr, dW13=dW13, dW2=dW2, d_topk_w=dw)
    return res


def expert_wgrad_columns(x_rows, dy_rows, w13_e, w2_e, cols):
    """Weight gradients of one expert restricted to ffn columns ``cols``.

    x_rows [n, d] are the token rows routed to the expert and dy_rows [n, d]
    their output gradients (routing weight already applied).  Column c of W1
    and W3 and row c of W2 depend only on activation column c, so
      dW1[:, c] = sum_rows x * dA[:, c],  dW3[:, c] = sum_rows x * dB[:, c],
      dW2[c, :] = sum_rows h[:, c] * dy.
    Returns (dW1[:, cols], dW3[:, cols], dW2[cols, :]).
    """
    x_rows = f64(x_rows)
    dy_rows = f64(dy_rows)
    w13_e = f64(w13_e)
    f = w13_e.shape[1] // 2
    cols = np.asarray(cols)
    a = x_rows @ w13_e[:, cols]
    b = x_rows @ w13_e[:, f + cols]
    s = sigmoid(a)
    h = a * s * b
    dh = dy_rows @ f64(w2_e)[cols, :].T
    da = dh * b * s * (1.0 + a * (1.0 - s))
    db = dh * a * s
    return x_rows.T @ da, x_rows.T @ db, h.T @ dy_rows
