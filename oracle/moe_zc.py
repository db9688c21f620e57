"""Vectorised fp64 oracle of the MoE layer with zero-computation experts.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.

The defining formula is missing from the page that introduces it
(『衝上熱搜！美團大模型，靠「快」火了』, section 零計算專家: the equation was an
image and did not survive).  The layer below is rebuilt from that section's
symbol legend (x_t the t-th token, R a softmax router, b_i the bias of expert
i, K experts per token), from its statement that the N FFN experts are
extended by Z experts that return the input unchanged, and from the statement
that the bias steers routing while staying out of the training objective.
For each token t independently:

    l[t,i]  = x_t . W_r[i]                       router logits, i in [0, E)
    p[t,i]  = softmax_i(l[t,:])                  over all E = N + Z experts
    key     = fl32(fl32(p) + b_i)                selection key only
    TopK_t  = K largest keys, ties to the lower expert index
    g[t,i]  = fl32(p[t,i]) for i in TopK_t       unbiased, not renormalised
    E_i(x)  = W_down_i (silu(W_gate_i x) * (W_up_i x))   i < N   (SwiGLU FFN)
    E_i(x)  = x                                          i >= N  (identity)
    y_t     = r_t + sum over the K chosen slots, in key order, of g * E_i(x_t)

Experts are numbered FFN first (0..N-1), then the zero-computation experts
(N..E-1), following the page's wording that the Z experts extend the pool.

Pins (tests/test_oracle_pins.py with the checks in tests/pins.py, the
fixtures in tests/golden, and tests/test_oracle_mutations.py):
  router_logits   brute-force fsum loops; hand example in tests/golden
  softmax_fp64    sums to 1; brute force with math.exp; hand example
  select_topk     enumeration of all C(E,K) subsets; tie cases by hand
  expert_loads    sum = T*K; brute-force count
  ffn_offsets     monotone, last = S; brute force
  permutation     stable argsort (library); bijection; round trip
  swiglu_ffn      single forced FFN expert equals a dense torch SwiGLU FFN
  combine/forward all-zero-expert closed form (sum g) x + r; K = E closed form
                  (independent of b); brute-force loops; per-token independence
  pid_step        closed-form first and second steps; zero error is a no-op;
                  sum of updates is zero when totals match; sign
  budget_target   closed-form sums (T f FFN slots, T (K - f) identity slots)
  closed_loop     a routing that meets the target is a fixed point; the bias
                  sum is conserved; velocity steps accumulate to the positional
                  form over the recorded loads; integral control of a one-FFN,
                  one-identity layer settles on the target (textbook, monotone
                  plant)
  ffn counts      hypergeometric law of the FFN count under exchangeable logits
PID gains and convergence: parity unpinned (no values on the pages).
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):          # torch tensor (any dtype, CPU)
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def router_logits(x, w_router) -> np.ndarray:
    """l[t,i] = sum_k x[t,k] W_r[i,k], fp64 (router R of section 零計算專家)."""
    return _f64(x) @ _f64(w_router).T


def softmax_fp64(logits32) -> np.ndarray:
    """Softmax over all E experts, evaluated in fp64 from fp32 logits.

    The logits are first taken as fp32 values (the precision the router
    produces them in); max subtraction, exp, sum and division run in fp64.
    """
    l = np.asarray(logits32, dtype=np.float32).astype(np.float64)
    m = l.max(axis=1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=1, keepdims=True)


def selection_keys(p64, bias):
    """p32 = fl32(p); key = fl32(p32 + b): one IEEE fp32 add per expert.

    The bias only enters this selection key (section 零計算專家: the bias
    adjusts routing scores and is kept out of the training objective).
    """
    p32 = np.asarray(p64, dtype=np.float64).astype(np.float32)
    b32 = np.asarray(bias, dtype=np.float32)
    key = np.add(p32, b32[None, :], dtype=np.float32)
    return p32, key


def select_topk(key32, K: int) -> np.ndarray:
    """Indices of the K largest keys per row, ordered by key descending, then
    by expert index ascending (so an exact tie goes to the lower index)."""
    key32 = np.asarray(key32, dtype=np.float32)
    T, E = key32.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)),
                        -key32.astype(np.float64)), axis=-1)
    return order[:, :K].astype(np.int64)


def gates_of(p32, idx) -> np.ndarray:
    """g[t,k] = fl32(p[t, idx[t,k]]): the unbiased router probability."""
    return np.take_along_axis(np.asarray(p32, np.float32), idx, axis=1)


def expert_loads(idx, E: int) -> np.ndarray:
    """Slots routed to each expert (FFN and zero-computation alike)."""
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.int64)


def ffn_offsets(loads, N: int) -> np.ndarray:
    """Exclusive prefix sum over the FFN experts' loads; offsets[N] = S."""
    off = np.zeros(N + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(loads)[:N])
    return off


def permutation(idx, N: int):
    """Expert-major, token-ascending grouping of the FFN slots.

    Returns (perm, pos): perm[s] is the token held in grouped row s; pos[t,k]
    is the grouped row of slot (t,k), or -1 when idx[t,k] is a
    zero-computation expert (those slots are never grouped).
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    pos = np.full((T, K), -1, dtype=np.int64)
    perm = []
    row = 0
    for e in range(N):
        tt, kk = np.nonzero(idx == e)         # row-major: tokens ascending
        for t, k in zip(tt, kk):
            perm.append(t)
            pos[t, k] = row
            row += 1
    return np.asarray(perm, dtype=np.int64), pos


def unpermute(rows, pos, idx, N: int):
    """Inverse of the grouping: out[t,k] = rows[pos[t,k]] for FFN slots."""
    T, K = pos.shape
    out = np.zeros((T, K) + rows.shape[1:], dtype=rows.dtype)
    ffn = np.asarray(idx) < N
    out[ffn] = rows[pos[ffn]]
    return out


def silu(v):
    """silu(v) = v * sigmoid(v) = v / (1 + exp(-v))."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu_ffn(xr, w_gate_e, w_up_e, w_down_e) -> np.ndarray:
    """One FFN expert on rows xr [m, d]: W_down (silu(W_gate x) * (W_up x))."""
    xr = _f64(xr)
    a = xr @ _f64(w_gate_e).T
    u = xr @ _f64(w_up_e).T
    return (silu(a) * u) @ _f64(w_down_e).T


def combine(x, idx, gates, expert_rows, N: int, residual=None) -> np.ndarray:
    """y_t = r_t + sum_k g[t,k] * (FFN output of slot (t,k), or x_t for a
    zero-computation expert), accumulated over k in slot order.

    expert_rows[t][k] holds the FFN output row for FFN slots (ignored for
    zero-computation slots).
    """
    x = _f64(x)
    T, K = np.asarray(idx).shape
    y = np.zeros_like(x) if residual is None else _f64(residual).copy()
    for k in range(K):
        ffn = idx[:, k] < N
        term = np.where(ffn[:, None], expert_rows[:, k, :], x)
        y += gates[:, k].astype(np.float64)[:, None] * term
    return y


def route(logits32, bias, K: int, N: int):
    """Routing from fp32 logits: probabilities, keys, top-K, gates, loads,
    offsets and the grouping permutation."""
    logits32 = np.asarray(logits32, dtype=np.float32)
    E = logits32.shape[1]
    p64 = softmax_fp64(logits32)
    p32, key = selection_keys(p64, bias)
    idx = select_topk(key, K)
    g = gates_of(p32, idx)
    loads = expert_loads(idx, E)
    off = ffn_offsets(loads, N)
    perm, pos = permutation(idx, N)
    return {"p64": p64, "p32": p32, "key": key, "idx": idx, "gate": g,
            "loads": loads, "offsets": off, "perm": perm, "pos": pos,
            "n_rows": int(off[N])}


def _expert_getter(w_gate, w_up, w_down):
    def get(e):
        return w_gate[e], w_up[e], w_down[e]
    return get


def forward_tokens(x_rows, logits32_rows, bias, get_expert, N: int, K: int,
                   residual_rows=None):
    """Layer output for a set of tokens, given their fp32 logits.

    Tokens are independent, so any subset can be evaluated alone.
    get_expert(e) returns (W_gate[e], W_up[e], W_down[e]).
    """
    x = _f64(x_rows)
    rt = route(logits32_rows, bias, K, N)
    idx, g = rt["idx"], rt["gate"]
    T = x.shape[0]
    rows = np.zeros((T, K, x.shape[1]))
    for e in np.unique(idx[idx < N]):
        tt, kk = np.nonzero(idx == e)
        wg, wu, wd = get_expert(int(e))
        rows[tt, kk] = swiglu_ffn(x[tt], wg, wu, wd)
    y = combine(x, idx, g, rows, N, residual_rows)
    return y, rt


def forward(x, w_router, bias, w_gate, w_up, w_down, N: int, Z: int, K: int,
            residual=None, logits32=None):
    """Whole layer.  With ``logits32`` given, routing uses those fp32 logits
    (so that a device result can be compared on the same routing); otherwise
    the oracle's own fp64 logits are rounded once to fp32."""
    l64 = router_logits(x, w_router)
    if logits32 is None:
        logits32 = l64.astype(np.float32)
    y, rt = forward_tokens(x, logits32, bias,
                           _expert_getter(w_gate, w_up, w_down), N, K, residual)
    rt["logits64"] = l64
    rt["y"] = y
    return rt


def ffn_count_per_token(idx, N: int) -> np.ndarray:
    """How many of a token's K chosen experts are FFN experts."""
    return (np.asarray(idx) < N).sum(axis=1)


def pid_step(loads, target, bias, e_prev, e_prev2, kp, ki, kd):
    """One PID update of the expert bias from measured loads.

    The pages say a PID controller from control theory tunes the expert bias
    in real time from recent expert usage (『衝上熱搜！…』, section 零計算專家),
    taking load away from busy experts and giving it to idle ones
    (『美团 LongCat-Flash 这个5600亿参数的懒AI…』).  Reading: the error is the
    normalised load deficit e_i = (target_i - loads_i) / sum(target), one
    controller step per forward, in velocity form

        db_i = kp (e_i - e1_i) + ki e_i + kd (e_i - 2 e1_i + e2_i)

    with histories e1, e2 starting at zero.  Summed over steps this is the
    positional PID b = b0 + kp e + ki sum(e) + kd (e - e1).
    Returns (new_bias, new_e_prev, new_e_prev2) in fp64.
    """
    loads = np.asarray(loads, dtype=np.float64)
    target = np.asarray(target, dtype=np.float64)
    e = (target - loads) / target.sum()
    e1 = np.asarray(e_prev, dtype=np.float64)
    e2 = np.asarray(e_prev2, dtype=np.float64)
    db = kp * (e - e1) + ki * e + kd * (e - 2.0 * e1 + e2)
    return np.asarray(bias, dtype=np.float64) + db, e, e1


def budget_target(T: int, K: int, N: int, Z: int, ffn_per_token: float) -> np.ndarray:
    """Per-expert load target [E] for a chosen number f of FFN experts per token.

    The pages give the controller's purpose as a compute budget: it keeps the
    compute activated per token near a set amount (about 27B of 560B
    parameters, 『美团的 LongCat-Flash：用 27B 激活算力跑起一个 560B 模型』,
    section 关键要点), which comes to about 8 FFN experts per token
    (『美团LongCat-Flash：算力调度新纪元』, Figure 3 caption).  Reading: the T*K
    slots of a batch split into T*f FFN slots and T*(K-f) identity slots, each
    share spread evenly over its experts.  Routing that meets this target
    averages exactly f FFN experts per token.
    """
    if not 0.0 <= ffn_per_token <= K:
        raise ValueError("ffn_per_token outside [0, K]")
    if (N == 0 and ffn_per_token > 0) or (Z == 0 and ffn_per_token < K):
        raise ValueError("budget needs experts of the kind it assigns slots to")
    t = np.zeros(N + Z, dtype=np.float64)
    if N:
        t[:N] = T * ffn_per_token / N
    if Z:
        t[N:] = T * (K - ffn_per_token) / Z
    return t


def closed_loop(logits32_batches, bias0, target, K: int, N: int, kp, ki, kd):
    """The bias controller over a sequence of batches.

    The bias is tuned in real time from recent expert usage
    (『衝上熱搜！美團大模型，靠「快」火了』, section 零計算專家).  Reading: batch s
    is routed with the current bias b_s, its loads drive one pid_step, and
    b_{s+1} routes batch s+1.  Between steps the controller state (bias and the
    two error histories) is held in fp32, as a device stores it; the step
    itself is evaluated in fp64.

    Returns dict: bias [S+1, E] fp32 (bias[0] = bias0), loads [S, E],
    ffn_per_token [S] (mean over the batch's tokens).
    """
    b = np.asarray(bias0, dtype=np.float32).copy()
    E = b.shape[0]
    e1 = np.zeros(E, dtype=np.float32)
    e2 = np.zeros(E, dtype=np.float32)
    tgt = np.asarray(target, dtype=np.float32)
    biases, loads, ffn = [b.copy()], [], []
    for l32 in logits32_batches:
        rt = route(l32, b, K, N)
        loads.append(rt["loads"])
        ffn.append(float(ffn_count_per_token(rt["idx"], N).mean()))
        nb, ne1, ne2 = pid_step(rt["loads"], tgt, b, e1, e2, kp, ki, kd)
        b, e1, e2 = nb.astype(np.float32), ne1.astype(np.float32), ne2.astype(np.float32)
        biases.append(b.copy())
    return {"bias": np.array(biases), "loads": np.array(loads), "ffn_per_token": np.array(ffn)}
