"""Plain float64 definition of the MoE expert-MLP layer (routing, dispatch,
expert SwiGLU MLP, combine) and of its backward pass.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Nothing here is
blocked, fused or reordered: each step is the per-expert loop the pages
describe, written out with numpy matmuls as the only library primitive.

Layout conventions (fixed by the library's C-ABI and restated here so the
oracle can be read on its own):
  x      [T, d]        tokens
  logits [T, E]        router scores
  w_gu   [E, 2f, d]    per-expert gate_up weight, rows 0..f-1 gate (W1),
                       rows f..2f-1 up (W3); out_features = 2*intermediate
  w2     [E, d, f]     per-expert down weight (out_features x in_features)
  idx, p [T, k]        chosen experts (descending score, ties -> lower id)
                       and their routing weights
  counts [E], offsets [E+1], pos [T, k], src [T*k]   the dispatch plan
  permuted tensors have one row per (token, slot) pair, rows of expert e
  in [offsets[e], offsets[e+1]), token-ascending inside an expert.

Pinned by tests/test_oracle_pins.py: routing against a pure-Python sort,
softmax against scipy, dispatch against its invariants, the forward against
a dense masked brute force and the E=1,k=1 plain SwiGLU MLP, hand-derived
closed forms (tests/golden/closed_forms.json), the backward against torch
autograd (float64) and central finite differences; the router backward and
the balancing loss (tests/test_oracle_router_pins.py) against torch autograd
of their forward definitions, finite differences and closed forms.
"""

import numpy as np


# --------------------------------------------------------------------------
# Router.  "How MoE Architecture Cuts Costs ...", section "Why Biology Is
# Especially Well-Suited for MoE": the router emits one score per expert and
# only the K best-scoring experts run for a token.
# --------------------------------------------------------------------------

def router_logits(x, w_g, bias=None):
    """Router scores L = x . W_g^T (+ per-expert bias), float64.

    x [T, d], w_g [E, d], bias [E] or None.  Returns [T, E].
    """
    x = np.asarray(x, dtype=np.float64)
    w_g = np.asarray(w_g, dtype=np.float64)
    logits = x @ w_g.T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits


def topk_route(logits, k, renorm=True):
    """Top-k expert choice and routing weights for every token.

    Selection compares the given score values exactly (float32 scores are
    exact in float64): experts are ordered by descending score, equal scores
    by ascending expert id, and the first k are kept.  A NaN score ranks
    below every number (NaNs by ascending id), which is where numpy's sort
    places NaN.  Weights are the
    softmax of the scores; with ``renorm`` they are renormalised over the k
    chosen experts, which equals a softmax over the chosen scores alone.
    Returns idx [T, k] int32 and p [T, k] float64.
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # a stable sort on the negated score keeps the lower id first among ties
    order = np.argsort(-L, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    chosen = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    top = chosen[:, :1]                      # the largest score of the row
    if renorm:
        z = np.exp(chosen - top)
        p = z / z.sum(axis=1, keepdims=True)
    else:
        z_all = np.exp(L - top)
        p = np.exp(chosen - top) / z_all.sum(axis=1, keepdims=True)
    return idx, p


# --------------------------------------------------------------------------
# Dispatch plan.  "Efficient MoE Training ...", Challenge 1: each expert
# gathers the tokens that chose it; GroupedLinear takes the per-expert token
# counts (split_sizes).  Rows are grouped expert by expert, tokens ascending.
# --------------------------------------------------------------------------

def dispatch_plan(idx, E):
    """counts[E], offsets[E+1], pos[T,k], src[T*k] for the expert grouping.

    pos[t, j] is the permuted row of slot j of token t; src[r] is the token
    of permuted row r.  Inside an expert, rows follow ascending token id.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    pos = np.full((T, k), -1, dtype=np.int64)
    src = np.full(T * k, -1, dtype=np.int64)
    row = 0
    for e in range(E):
        offsets[e] = row
        # row-major scan of the [T, k] mask: ascending token, one slot each
        tokens, slots = np.nonzero(idx == e)
        n = tokens.shape[0]
        counts[e] = n
        rows = row + np.arange(n)
        pos[tokens, slots] = rows
        src[rows] = tokens
        row += n
    offsets[E] = row
    return counts, offsets, pos, src


def permute_rows(x, src):
    """Permuted copy of token rows: Xp[r] = x[src[r]]."""
    return np.asarray(x, dtype=np.float64)[np.asarray(src)]


def permuted_weights(p, pos):
    """w_perm[pos[t, j]] = p[t, j]."""
    p = np.asarray(p, dtype=np.float64)
    out = np.zeros(p.size, dtype=np.float64)
    out[np.asarray(pos).reshape(-1)] = p.reshape(-1)
    return out


# --------------------------------------------------------------------------
# Expert MLP.  "Efficient MoE Training ...", Challenge 1 (gate_up projection
# with out_features = 2 * intermediate_size, bias=False) and Challenge 3
# (GroupedLinear(gate_up) -> ScaledSwiGLU -> GroupedLinear(down); the routing
# probabilities are the SwiGLU's scales).
# --------------------------------------------------------------------------

def silu(a):
    """silu(a) = a / (1 + exp(-a))."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def bf16_round(v):
    """Nearest bfloat16 value of v (ties to even), returned as float64.

    "Efficient MoE Training for Biological Foundation Models", Challenge 2:
    BF16 training represents every weight and activation with 16 bits.  With
    ``bf16_act`` the functions below store the activations the path keeps
    (gate/up pre-activations, the SwiGLU output S and its gradient dAB) in
    that format at the points where they are stored."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    binade = np.maximum(ex - 1, -126)     # subnormals share the 2^-126 binade
    spacing = np.ldexp(1.0, binade - 7)   # 7 stored mantissa bits
    return np.copysign(np.rint(a / spacing) * spacing, v)


def _keep(v, bf16_act):
    return bf16_round(v) if bf16_act else v


# One function per step of the expert MLP, each the plain definition.

def gate_up(xp_e, w_gu_e):
    """AB = Xp . W_gu^T: gate pre-activations in columns [0, f), up in
    [f, 2f)."""
    return np.asarray(xp_e, dtype=np.float64) @ \
        np.asarray(w_gu_e, dtype=np.float64).T


def scaled_swiglu(ab_e, w_e):
    """S = w * silu(A_g) * A_u, one routing weight per row."""
    ab_e = np.asarray(ab_e, dtype=np.float64)
    f = ab_e.shape[1] // 2
    return np.asarray(w_e, dtype=np.float64)[:, None] * \
        (silu(ab_e[:, :f]) * ab_e[:, f:])


def down(s_e, w2_e):
    """O = S . W2^T."""
    return np.asarray(s_e, dtype=np.float64) @ \
        np.asarray(w2_e, dtype=np.float64).T


def down_backward(do_e, ab_e, w_e, w2_e):
    """Backward through down and the scaled SwiGLU for one expert's rows:
    dS = dO . W2; dp = <dS, H> per row (H = silu(A_g) A_u); dH = w dS;
    dA_g = dH A_u sig(A_g)(1 + A_g(1 - sig(A_g))); dA_u = dH silu(A_g).
    Returns (dAB, dp)."""
    do_e = np.asarray(do_e, dtype=np.float64)
    ab_e = np.asarray(ab_e, dtype=np.float64)
    f = ab_e.shape[1] // 2
    a_g, a_u = ab_e[:, :f], ab_e[:, f:]
    ds = do_e @ np.asarray(w2_e, dtype=np.float64)
    h = silu(a_g) * a_u
    dp = np.sum(ds * h, axis=1)
    dh = np.asarray(w_e, dtype=np.float64)[:, None] * ds
    sg = sigmoid(a_g)
    dab = np.concatenate([dh * a_u * sg * (1.0 + a_g * (1.0 - sg)),
                          dh * silu(a_g)], axis=1)
    return dab, dp


def gate_up_dgrad(dab_e, w_gu_e):
    """dXp = dAB . W_gu."""
    return np.asarray(dab_e, dtype=np.float64) @ \
        np.asarray(w_gu_e, dtype=np.float64)


def wgrad(a_e, b_e):
    """Weight gradient over an expert's rows: sum_r a[r]^T b[r]."""
    return np.asarray(a_e, dtype=np.float64).T @ \
        np.asarray(b_e, dtype=np.float64)


def expert_forward(xp_e, w_gu_e, w2_e, w_e, bf16_act=False):
    """One expert on its rows: returns (AB, S, O).

    AB = Xp_e . W_gu_e^T  (gate pre-activations first, then up)
    S  = w * silu(A_g) * A_u       (scaled SwiGLU, one weight per row)
    O  = S . W2_e^T
    With bf16_act the returned AB (kept for the backward pass) and S (the
    input of the down projection) are stored as bfloat16; S is formed from
    the unrounded A_g, A_u.
    """
    ab = gate_up(xp_e, w_gu_e)
    s = _keep(scaled_swiglu(ab, w_e), bf16_act)
    o = down(s, w2_e)
    return _keep(ab, bf16_act), s, o


def combine(o_perm, pos, idx):
    """y[t] = sum over the token's k slots, ascending expert id, of O[pos]."""
    pos = np.asarray(pos)
    idx = np.asarray(idx)
    T, k = pos.shape
    y = np.zeros((T, o_perm.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in np.argsort(idx[t], kind="stable"):
            y[t] += o_perm[pos[t, j]]
    return y


def experts_forward(x, idx, p, w_gu, w2, bf16_act=False):
    """The layer forward with routing given (idx, p).  Returns a dict with
    the plan, the permuted intermediates and the output y [T, d]."""
    x = np.asarray(x, dtype=np.float64)
    w_gu = np.asarray(w_gu, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    E = w_gu.shape[0]
    f = w_gu.shape[1] // 2
    d = x.shape[1]
    counts, offsets, pos, src = dispatch_plan(idx, E)
    xp = permute_rows(x, src)
    w_perm = permuted_weights(p, pos)
    Tk = xp.shape[0]
    ab = np.zeros((Tk, 2 * f))
    s = np.zeros((Tk, f))
    o = np.zeros((Tk, d))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        ab[r0:r1], s[r0:r1], o[r0:r1] = expert_forward(
            xp[r0:r1], w_gu[e], w2[e], w_perm[r0:r1], bf16_act)
    y = combine(o, pos, idx)
    return dict(idx=np.asarray(idx), p=np.asarray(p, dtype=np.float64),
                counts=counts, offsets=offsets, pos=pos, src=src,
                xp=xp, w_perm=w_perm, ab=ab, s=s, o=o, y=y)


def moe_forward(x, logits, w_gu, w2, k, renorm=True, bf16_act=False):
    """Route on the given scores, then run the experts and combine."""
    idx, p = topk_route(logits, k, renorm)
    return experts_forward(x, idx, p, w_gu, w2, bf16_act)


def moe_backward(fwd, dy, w_gu, w2, bf16_act=False):
    """Backward of ``experts_forward`` for upstream gradient dy [T, d].

    Routing (idx) is held fixed; the gradient with respect to the routing
    weights is returned as dp [T, k].  Returns dict(dx, dw_gu, dw2, dp,
    dab, do) with dab/do in permuted row order.  Experts that received no
    rows get exactly zero weight gradients.  With bf16_act, fwd must come
    from experts_forward(..., bf16_act=True) and dAB is stored as bfloat16
    before it feeds the two GEMMs that consume it.
    """
    dy = np.asarray(dy, dtype=np.float64)
    w_gu = np.asarray(w_gu, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    E, two_f, d = w_gu.shape
    offsets, pos, src = fwd["offsets"], fwd["pos"], fwd["src"]
    ab, s, xp, w_perm = fwd["ab"], fwd["s"], fwd["xp"], fwd["w_perm"]
    Tk = xp.shape[0]
    do = dy[src]                                  # dO[r] = dY[src[r]]
    dab = np.zeros((Tk, two_f))
    dxp = np.zeros((Tk, d))
    dw_gu = np.zeros_like(w_gu)
    dw2 = np.zeros_like(w2)
    dp_perm = np.zeros(Tk)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        do_e = do[r0:r1]
        dw2[e] = wgrad(do_e, s[r0:r1])                       # dO^T S
        dab_e, dp_perm[r0:r1] = down_backward(do_e, ab[r0:r1],
                                              w_perm[r0:r1], w2[e])
        dab[r0:r1] = _keep(dab_e, bf16_act)
        dw_gu[e] = wgrad(dab[r0:r1], xp[r0:r1])              # dAB^T Xp
        dxp[r0:r1] = gate_up_dgrad(dab[r0:r1], w_gu[e])      # dAB W_gu
    T, k = pos.shape
    dx = np.zeros((T, d))
    dp = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            dx[t] += dxp[pos[t, j]]
            dp[t, j] = dp_perm[pos[t, j]]
    return dict(dx=dx, dw_gu=dw_gu, dw2=dw2, dp=dp, dab=dab, do=do,
                dxp=dxp)


# --------------------------------------------------------------------------
# Sampled evaluation for full-size parity checks: the same definition,
# evaluated for single outputs so that Mixtral-sized layers stay cheap.
# --------------------------------------------------------------------------

def token_forward(x_t, idx_t, p_t, w_gu, w2, bf16_act=False):
    """y[t] for one token: sum over its chosen experts (ascending id) of
    p * (silu(x W1^T) * (x W3^T)) W2^T.  ``w_gu``/``w2`` may be any indexable
    stack of per-expert weights (each item converted to float64 here)."""
    x_t = np.asarray(x_t, dtype=np.float64)
    y = np.zeros(x_t.shape[0])
    for j in np.argsort(np.asarray(idx_t), kind="stable"):
        e = int(idx_t[j])
        wgu = np.asarray(w_gu[e], dtype=np.float64)
        w2e = np.asarray(w2[e], dtype=np.float64)
        _, _, o = expert_forward(x_t[None, :], wgu, w2e,
                                 np.array([float(p_t[j])]), bf16_act)
        y += o[0]
    return y


def row_backward(x_t, dy_t, p_r, w_gu_e, w2_e, bf16_act=False):
    """Backward of one permuted row (one token through one expert).

    Returns (dab_row [2f], dxp_row [d], dp_r scalar, ab_row, s_row).
    """
    x_t = np.asarray(x_t, dtype=np.float64)
    dy_t = np.asarray(dy_t, dtype=np.float64)
    w_gu_e = np.asarray(w_gu_e, dtype=np.float64)
    w2_e = np.asarray(w2_e, dtype=np.float64)
    ab, s, _ = expert_forward(x_t[None, :], w_gu_e, w2_e, np.array([p_r]),
                              bf16_act)
    dab, dp = down_backward(dy_t[None, :], ab, np.array([p_r]), w2_e)
    dab = _keep(dab[0], bf16_act)
    dp_r = float(dp[0])
    dxp = gate_up_dgrad(dab[None, :], w_gu_e)[0]
    return dab, dxp, dp_r, ab[0], s[0]


def dw2_column(xp_e, do_e, w_e, w_gu_e, j, bf16_act=False):
    """Column j of dW2_e = sum over the expert's rows of dO[r] * S[r, j],
    with S[r, j] = w_r * silu(Xp[r] . W1[j]) * (Xp[r] . W3[j]).
    xp_e [n, d], do_e [n, d], w_e [n], w_gu_e [2f, d]."""
    xp_e = np.asarray(xp_e, dtype=np.float64)
    do_e = np.asarray(do_e, dtype=np.float64)
    f = w_gu_e.shape[0] // 2
    g = xp_e @ np.asarray(w_gu_e[j], dtype=np.float64)
    u = xp_e @ np.asarray(w_gu_e[f + j], dtype=np.float64)
    s = _keep(np.asarray(w_e, dtype=np.float64) * silu(g) * u, bf16_act)
    return do_e.T @ s


def dw_gu_row(xp_e, do_e, w_e, w_gu_e, w2_e, i, bf16_act=False):
    """Row i (of 2f) of dW_gu_e = sum over the expert's rows of
    dAB[r, i] * Xp[r]; dAB[:, i] needs only column i mod f of dS, gate and
    up.  xp_e, do_e [n, d]; w_e [n]; w_gu_e [2f, d]; w2_e [d, f]."""
    xp_e = np.asarray(xp_e, dtype=np.float64)
    do_e = np.asarray(do_e, dtype=np.float64)
    f = w_gu_e.shape[0] // 2
    c = i % f
    g = _keep(xp_e @ np.asarray(w_gu_e[c], dtype=np.float64), bf16_act)
    u = _keep(xp_e @ np.asarray(w_gu_e[f + c], dtype=np.float64), bf16_act)
    ds = do_e @ np.asarray(w2_e[:, c], dtype=np.float64)
    dh = np.asarray(w_e, dtype=np.float64) * ds
    if i < f:
        sg = sigmoid(g)
        col = dh * u * sg * (1.0 + g * (1.0 - sg))
    else:
        col = dh * silu(g)
    return _keep(col, bf16_act) @ xp_e


# --------------------------------------------------------------------------
# Router backward and the load-balancing loss.  "How MoE Architecture Cuts
# Costs ...", section "Engineering Challenges of Efficient Training": a
# router that keeps favouring a few experts leaves the others idle, which
# training counters with a balancing term.  The pages give no formula; the
# reading here is the common one: alpha * E * sum_e f_e * P_e, with f_e the
# fraction of routed slots that went to expert e (from the counts, a
# constant) and P_e the mean over tokens of the full softmax probability of
# e.  The selection itself is piecewise constant, so only the chosen
# experts' scores receive the routing-weight gradient.
# --------------------------------------------------------------------------

def routing_weight_backward(logits, idx, p, dp, renorm=True):
    """dL = d(sum_{t,j} dp[t,j] p[t,j]) / dL for fixed choices idx.

    renorm: p is the softmax over the chosen scores, so
      dL[t, idx_j] = p_j (dp_j - sum_i p_i dp_i), 0 for the other experts.
    else:   p_j = P[idx_j] with P the softmax over all E scores, so
      dL[t, e] = P_e (g_e - sum_i p_i dp_i), g_e = dp_j if e = idx_j else 0.
    """
    L = np.asarray(logits, dtype=np.float64)
    idx = np.asarray(idx)
    p = np.asarray(p, dtype=np.float64)
    dp = np.asarray(dp, dtype=np.float64)
    T, E = L.shape
    s = np.sum(p * dp, axis=1, keepdims=True)
    dL = np.zeros((T, E))
    if renorm:
        np.put_along_axis(dL, idx.astype(np.int64), p * (dp - s), axis=1)
        return dL
    P = np.exp(L - L.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    g = np.zeros((T, E))
    np.put_along_axis(g, idx.astype(np.int64), dp, axis=1)
    return P * (g - s)


def aux_loss(logits, counts, alpha):
    """(loss, dL) of the balancing term alpha * E * sum_e f_e * mean_t P_e
    with f_e = counts_e / sum(counts) held constant."""
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    f = np.asarray(counts, dtype=np.float64)
    f = f / f.sum()
    P = np.exp(L - L.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    loss = alpha * E * np.sum(f * P.mean(axis=0))
    # d/dL[t,i] of sum_e f_e P[t,e]  =  P[t,i] (f_i - sum_e f_e P[t,e])
    dL = alpha * E / T * P * (f[None, :] - np.sum(f * P, axis=1,
                                                  keepdims=True))
    return loss, dL


def router_backward(x, w_g, dlogits):
    """Gradients through L = x . W_g^T (+ bias): dW_g = dL^T x [E, d],
    db = sum_t dL [E], and the router's share of dx = dL . W_g [T, d]."""
    x = np.asarray(x, dtype=np.float64)
    w_g = np.asarray(w_g, dtype=np.float64)
    dL = np.asarray(dlogits, dtype=np.float64)
    return dL.T @ x, dL.sum(axis=0), dL @ w_g
