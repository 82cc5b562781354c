"""CPU oracle for one LongCat-2.0-style sparse MoE layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code with the HIP library
(no kernels, headers, helpers or constants) and never imports it.

Plain, slow, obviously correct: NumPy in float64, one step per function, in the
order the method applies them.  Inputs in reduced precision (bf16 weights and
activations) are consumed as the exact values they hold, upcast to float64.

Sources (web pages about LongCat-2.0; cited by page title and section):

* [DS] "LongCat-2.0" model data sheet (archdb), table "Mixture of experts":
  768 routed FFN experts plus 128 identity zero experts scored by one router
  classifier of shape [768+128, d_model], an ``e_score_correction_bias``, 12
  experts per token, expert width 2048, routed scaling factor 9; router score,
  renormalisation and load balancing "not disclosed".  Table "Feed-forward":
  activation "not disclosed".
* [SN] "Meituan lancerer LongCat-2.0: 1,6T MoE-model med million-token
  hukommelse" (snilld.dk), section "MoE i praksis og prisen for fleksibilitet":
  zero-computation experts give trivial tokens a lightweight response, and a
  PID controller adjusts the router bias so that activation stays in range.
* [AS] Ascend deployment article on LongCat-2.0 (10100.com), section
  "底层定制算子深度优化": Dispatch/Combine operators that support
  zero-computation experts; section "MoE专家动态负载均衡": tokens received per
  expert.
* [MD] "2026 Analysis of LongCat-2.0 Technical Principles" (macdate.com),
  section 1: soft-max gated top-k routing.

Readings where the pages are silent (each is listed in the design notes):

* Score function: softmax over all E = N + Z logits jointly ([DS] router
  score undisclosed; [MD] soft-max gated).
* The correction bias is added to the softmax score for *selection only*; the
  gates use the unbiased score and are not renormalised.
* Expert ids 0..N-1 are FFN experts, N..E-1 are identity experts.
* Top-k ties go to the lower expert id; a token's selected set is reported in
  ascending expert id.
* The selection decision is taken in float32: key = fp32(fp32(p) + bias),
  with bias a float32 vector.  This is part of the problem statement adopted
  for this layer (routing scores, correction bias and gates are float32
  quantities in the C interface), not a property of any implementation.
* A zero-computation expert returns its input unchanged; the routed scaling
  factor multiplies every gate, identity experts included.
* SwiGLU expert: H = silu(X Wg^T) * (X Wu^T), Y = H Wd^T, silu(z) = z/(1+e^-z).
* Dispatch order inside an expert is stable by assignment id a = t*k + j.
* PID: incremental form on the FFN experts' bias, error measured in real
  (FFN) experts per token, D = 0 on the first update, no anti-windup clamp.
  The controller is defined in float32 (its state and the bias are float32
  quantities), each multiply and add rounded on its own in the order
  delta = (kp*err + ki*I) + kd*D; ``pid_update_f32`` evaluates exactly that,
  ``pid_update`` the same law in float64 as a cross-check.
* Per-expert load balancing ([AS] section "MoE专家动态负载均衡": dynamic load
  balancing narrows the gap between experts' token loads; method not
  stated): a zero-sum sign step on the FFN experts' correction bias, so it
  evens the load without moving the mean FFN bias the PID controls.
* The same passage read as placement balancing across the expert-parallel
  domain (it names the very large EP domain as the cause of the load
  variance, and an inference deployment cannot change which experts a token
  picks): the N FFN experts occupy S >= N expert slots on D devices; each
  redundant slot replicates the expert with the most tokens per replica, an
  expert's rows are split evenly over its replicas, and slots go to devices
  by longest-processing-time-first with S / D slots per device.  Routing,
  and so the PID's budget, is untouched.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "router_logits",
    "softmax",
    "selection_keys",
    "topk_select",
    "topk_margin",
    "route",
    "dispatch",
    "gather_rows",
    "silu",
    "swiglu_ffn",
    "expert_ffn",
    "combine",
    "PidState",
    "pid_update",
    "pid_update_f32",
    "balance_update",
    "balance_update_f32",
    "eplb_replicas",
    "eplb_slots",
    "eplb_place",
    "eplb_plan",
    "eplb_device_loads",
    "forward",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- router ----

def router_logits(x, w_router, logit_bias=None):
    """Router classifier: l[t, e] = sum_i x[t, i] * W_r[e, i] (+ logit_bias[e]).

    [DS] "Mixture of experts": one classifier of shape [N+Z, d_model] scores
    the FFN experts and the zero experts together.  ``logit_bias`` is a plain
    additive classifier offset (used only to skew synthetic workloads).
    """
    l = _f64(x) @ _f64(w_router).T
    if logit_bias is not None:
        l = l + _f64(logit_bias)[None, :]
    return l


def softmax(logits):
    """Softmax over all E experts of each token (reading of [DS] router score
    "not disclosed" with [MD] section 1 "soft-max gated")."""
    l = _f64(logits)
    m = l.max(axis=1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=1, keepdims=True)


def selection_keys(p, bias):
    """Selection key = score + correction bias, in float32.

    [DS] "Mixture of experts" names an e_score_correction_bias on the router;
    it corrects the score used to *choose* experts.  The layer's problem
    statement makes scores and the bias float32 quantities, so the decision
    is taken in float32: the score is rounded to float32 first and the sum
    is rounded once more.
    """
    p32 = np.asarray(p, dtype=np.float64).astype(np.float32)
    b32 = np.asarray(bias, dtype=np.float32)
    return (p32 + b32[None, :]).astype(np.float32)


def topk_select(keys, k):
    """The k largest keys per row; ties to the lower expert id.

    Returns int32 [T, k] holding each row's selected set in ascending expert
    id ([DS]: 12 experts per token).
    """
    keys = np.asarray(keys)
    T, E = keys.shape
    out = np.empty((T, k), dtype=np.int32)
    ids = np.arange(E)
    for t in range(T):
        # lexsort: last key is primary -> sort by -key, then by id ascending
        order = np.lexsort((ids, -keys[t].astype(np.float64)))
        out[t] = np.sort(order[:k])
    return out


def topk_margin(keys, k):
    """Gap between the k-th and (k+1)-th largest key of each row (inf if k == E).

    Used to decide which tokens have a unique top-k set under small
    perturbations of the keys.
    """
    keys = np.asarray(keys, dtype=np.float64)
    T, E = keys.shape
    if k >= E:
        return np.full(T, np.inf)
    s = -np.sort(-keys, axis=1)
    return s[:, k - 1] - s[:, k]


def route(x, w_router, bias, k, routed_scaling=1.0, logit_bias=None):
    """Router + biased top-k + gates.

    Returns dict(logits, p, keys, topk_idx [T,k] int32, topk_gate [T,k] f64).
    gate[t, j] = s * p[t, idx[t, j]] with the *unbiased* score and no
    renormalisation ([DS] routed scaling factor; renormalise "not disclosed").
    """
    logits = router_logits(x, w_router, logit_bias)
    p = softmax(logits)
    keys = selection_keys(p, bias)
    idx = topk_select(keys, k)
    gate = routed_scaling * np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return dict(logits=logits, p=p, keys=keys, topk_idx=idx, topk_gate=gate)


# -------------------------------------------------------------- dispatch ----

def dispatch(topk_idx, n_experts):
    """Group the T*k assignments by expert ([AS] Dispatch operator).

    Assignment id a = t*k + j.  counts[e] = number of assignments to expert e;
    offsets = exclusive prefix sum with offsets[E] = T*k; perm[p] = the
    assignment at sorted position p, sorted by (expert, a); inv_perm is its
    inverse.  Zero-expert assignments are part of the permutation (they form
    the tail segment [offsets[N], T*k)).
    """
    flat = np.asarray(topk_idx, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=n_experts).astype(np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(perm.size, dtype=np.int32)
    return dict(counts=counts, offsets=offsets, perm=perm, inv_perm=inv_perm)


def gather_rows(x, perm, k, n_rows):
    """x_perm[p] = x[perm[p] // k] for the first n_rows sorted positions."""
    tok = np.asarray(perm[:n_rows], dtype=np.int64) // k
    return np.asarray(x)[tok]


# ------------------------------------------------------------ expert FFN ----

def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(X, w_gate, w_up, w_down):
    """One SwiGLU expert: (silu(X Wg^T) * (X Wu^T)) Wd^T.

    Wg, Wu are [d_ff, d] and Wd is [d, d_ff] (each "Linear" stores
    [out, in]).  [DS] "Mixture of experts": expert width 2048; activation not
    disclosed, read as SwiGLU.
    """
    X = _f64(X)
    h = silu(X @ _f64(w_gate).T) * (X @ _f64(w_up).T)
    return h @ _f64(w_down).T


def expert_ffn(x_perm, offsets, w_gate, w_up, w_down, n_ffn):
    """Run every FFN expert e < N on its contiguous row segment of x_perm.

    Returns y_perm with one row per FFN-expert position (offsets[N] rows).
    Zero experts need no FFN work ([SN]; [AS] zero-computation experts).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    n_rows = int(offsets[n_ffn])
    d = np.asarray(w_down).shape[1]
    y = np.zeros((n_rows, d), dtype=np.float64)
    for e in range(n_ffn):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y[lo:hi] = swiglu_ffn(x_perm[lo:hi], w_gate[e], w_up[e], w_down[e])
    return y


# --------------------------------------------------------------- combine ----

def combine(x, y_perm, topk_idx, topk_gate, inv_perm, n_ffn):
    """y[t] = sum_j gate[t,j] * v[t,j], summed in slot order j = 0..k-1.

    v[t,j] = y_perm[inv_perm[t*k+j]] for an FFN expert, and x[t] itself for a
    zero-computation (identity) expert ([AS] Combine with zero-computation
    experts; [DS] identity zero experts).
    """
    x = _f64(x)
    idx = np.asarray(topk_idx)
    g = _f64(topk_gate)
    T, k = idx.shape
    y = np.zeros_like(x)
    for j in range(k):
        a = np.arange(T) * k + j
        ffn = idx[:, j] < n_ffn
        v = x.copy()
        if ffn.any():
            v[ffn] = _f64(y_perm)[np.asarray(inv_perm)[a[ffn]]]
        y += g[:, j:j + 1] * v
    return y


# ------------------------------------------------------------------- PID ----

class PidState:
    """Controller memory: running integral of the error, previous error and
    the number of updates applied so far."""

    def __init__(self, integral=0.0, prev_err=0.0, step=0):
        self.integral = float(integral)
        self.prev_err = float(prev_err)
        self.step = int(step)

    def copy(self):
        return PidState(self.integral, self.prev_err, self.step)


def pid_update(counts, n_ffn, T, bias, state, setpoint, kp, ki, kd):
    """One PID step on the router bias ([SN]: a PID controller adjusts the
    router bias so the activation stays in the desired range).

    Measured value r = (number of FFN assignments) / T = mean real experts
    per token.  err = setpoint - r; I += err; D = err - prev_err (0 on the
    first update); delta = kp*err + ki*I + kd*D.  Incremental form: every FFN
    expert's bias moves by delta (raising all FFN biases makes FFN experts win
    more selections, which raises r).  Returns (new_bias, new_state, r).
    """
    counts = np.asarray(counts, dtype=np.int64)
    r = float(counts[:n_ffn].sum()) / float(T)
    err = float(setpoint) - r
    st = state.copy()
    st.integral = st.integral + err
    d_term = 0.0 if st.step == 0 else err - st.prev_err
    delta = kp * err + ki * st.integral + kd * d_term
    new_bias = _f64(bias).copy()
    new_bias[:n_ffn] += delta
    st.prev_err = err
    st.step += 1
    return new_bias, st, r


def pid_update_f32(counts, n_ffn, T, bias, state, setpoint, kp, ki, kd):
    """The PID step of ``pid_update`` evaluated in float32, one rounding per
    operation, in this order:

        r     = f32(sum_{e<N} counts[e]) / f32(T)
        err   = setpoint - r
        I     = I + err
        D     = err - prev_err            (0 on the first update)
        delta = (kp*err + ki*I) + kd*D    (three products, then two sums)
        bias[e] = bias[e] + delta         for e < N

    [SN] fixes only that a PID controller moves the router bias; the float32
    evaluation order is the controller's definition in this layer (its state,
    gains and the bias are float32 quantities), so two implementations of it
    can agree bit for bit.  ``state`` holds float32 values; ``bias`` is
    returned as float32.  Returns (new_bias, new_state, r).
    """
    f = np.float32
    counts = np.asarray(counts, dtype=np.int64)
    r = f(counts[:n_ffn].sum()) / f(T)
    err = f(setpoint) - r
    st = state.copy()
    integral = f(st.integral) + err
    d_term = f(0.0) if st.step == 0 else err - f(st.prev_err)
    delta = (f(kp) * err + f(ki) * integral) + f(kd) * d_term
    new_bias = np.asarray(bias, dtype=np.float32).copy()
    new_bias[:n_ffn] = new_bias[:n_ffn] + delta
    st.integral = f(integral)
    st.prev_err = f(err)
    st.step += 1
    return new_bias, st, r


def balance_update(counts, n_ffn, bias, gamma):
    """Per-expert load-balancing step on the FFN experts' bias.

    [AS] "MoE专家动态负载均衡": the token load per expert varies widely and a
    dynamic balancing step narrows the gap.  With mean FFN load
    L = sum_{e<N} counts[e] / N and s_e = sign(L - counts[e]) (over-loaded
    experts get -1), every FFN expert's bias moves by
        delta_e = gamma * (s_e - mean_{e'<N} s_e'),
    a zero-sum step (the mean FFN bias, which sets how many real experts a
    token activates, is unchanged).  Identity experts are untouched.
    Returns the new bias.
    """
    c = np.asarray(counts, dtype=np.int64)[:n_ffn]
    # sign(L - c_e) with L = sum(c)/N, compared exactly as sum(c) vs N*c_e
    s = np.sign(c.sum() - n_ffn * c).astype(np.float64)
    delta = float(gamma) * (s - s.mean())
    new_bias = _f64(bias).copy()
    new_bias[:n_ffn] += delta
    return new_bias


def balance_update_f32(counts, n_ffn, bias, gamma):
    """``balance_update`` in float32, as the layer defines the step: with
    A = sum_{e<N} counts[e], s_e = sign(A - N counts[e]) and S = sum s_e
    (exact integers), every FFN expert's bias becomes
        bias[e] + f32(gamma) * (f32(N s_e - S) / f32(N)),
    one rounding for the quotient, one for the product, one for the sum.
    ``bias`` is returned as float32."""
    f = np.float32
    c = np.asarray(counts, dtype=np.int64)[:n_ffn]
    a = int(c.sum())
    s = np.sign(a - n_ffn * c).astype(np.int64)
    S = int(s.sum())
    frac = (n_ffn * s - S).astype(np.float32) / f(n_ffn)
    step = f(gamma) * frac
    new_bias = np.asarray(bias, dtype=np.float32).copy()
    new_bias[:n_ffn] = new_bias[:n_ffn] + step
    return new_bias


# ------------------------------------------ expert placement balancing ----

def eplb_replicas(counts, n_ffn, n_slots):
    """Replicas per FFN expert for n_slots >= n_ffn expert slots.

    Every expert holds one slot; each of the n_slots - n_ffn redundant slots
    goes, one at a time, to the expert with the most tokens per replica
    (largest c_e / r_e, compared exactly; ties to the lower id).  [AS]
    "MoE专家动态负载均衡": the per-expert token load varies widely across the
    EP domain and dynamic balancing narrows the gap.
    """
    c = [int(v) for v in np.asarray(counts)[:n_ffn]]
    r = [1] * n_ffn
    for _ in range(n_slots - n_ffn):
        best = 0
        for e in range(1, n_ffn):
            if c[e] * r[best] > c[best] * r[e]:   # c_e / r_e > c_best / r_best
                best = e
        r[best] += 1
    return np.array(r, dtype=np.int32)


def eplb_slots(counts, replicas, offsets=None):
    """Slots in expert order (slot s = replica j of expert e, experts
    ascending, replicas ascending).  Replica j of an expert with c rows and
    r replicas takes rows [j*c // r, (j+1)*c // r) of its segment (absolute
    sorted positions when offsets are given).  Returns (expert, begin, end)
    int arrays of length sum(replicas)."""
    ex, beg, end = [], [], []
    for e, r in enumerate(np.asarray(replicas)):
        c = int(counts[e])
        base = 0 if offsets is None else int(offsets[e])
        for j in range(int(r)):
            ex.append(e)
            beg.append(base + (j * c) // int(r))
            end.append(base + ((j + 1) * c) // int(r))
    return (np.array(ex, np.int32), np.array(beg, np.int32), np.array(end, np.int32))


def eplb_place(slot_loads, n_devices):
    """Longest processing time first with equal capacity: slots in order of
    load descending (ties to the lower slot), each to the least-loaded device
    that still has room for one of its len / n_devices slots (ties to the
    lower device).  Returns (device per slot, load per device)."""
    loads = [int(v) for v in slot_loads]
    S = len(loads)
    cap = S // n_devices
    order = sorted(range(S), key=lambda i: (-loads[i], i))
    dev = [0] * S
    dload = [0] * n_devices
    used = [0] * n_devices
    for i in order:
        best = -1
        for d in range(n_devices):
            if used[d] < cap and (best < 0 or dload[d] < dload[best]):
                best = d
        dev[i] = best
        dload[best] += loads[i]
        used[best] += 1
    return np.array(dev, np.int32), np.array(dload, np.int64)


def eplb_plan(counts, offsets, n_ffn, n_slots, n_devices):
    """Replicas, slots and placement of one batch's FFN loads (see above)."""
    rep = eplb_replicas(counts, n_ffn, n_slots)
    ex, beg, end = eplb_slots(counts, rep, offsets)
    dev, dload = eplb_place(end - beg, n_devices)
    return dict(replicas=rep, slot_expert=ex, slot_begin=beg, slot_end=end,
                slot_device=dev, device_load=dload)


def eplb_device_loads(counts, replicas, slot_device, n_devices):
    """Device loads of a placement applied to (possibly other) counts: each
    expert's rows split over its replicas as in eplb_slots."""
    ex, beg, end = eplb_slots(counts, replicas)
    out = np.zeros(n_devices, np.int64)
    np.add.at(out, np.asarray(slot_device), (end - beg).astype(np.int64))
    return out


# --------------------------------------------------------------- forward ----

def forward(x, w_router, bias, w_gate, w_up, w_down, n_ffn, k,
            routed_scaling=1.0, logit_bias=None, topk_idx=None):
    """Whole layer: route -> dispatch -> expert FFN -> combine.

    If ``topk_idx`` is given, those selected sets are used instead of the
    oracle's own selection (gates still come from the oracle's scores), so a
    caller can evaluate the layer on another implementation's routing.
    Returns a dict with every intermediate.
    """
    E = np.asarray(w_router).shape[0]
    r = route(x, w_router, bias, k, routed_scaling, logit_bias)
    if topk_idx is not None:
        idx = np.asarray(topk_idx, dtype=np.int32)
        r["topk_idx"] = idx
        r["topk_gate"] = routed_scaling * np.take_along_axis(
            r["p"], idx.astype(np.int64), axis=1)
    dsp = dispatch(r["topk_idx"], E)
    n_rows = int(dsp["offsets"][n_ffn])
    x_perm = gather_rows(x, dsp["perm"], k, n_rows)
    y_perm = expert_ffn(x_perm, dsp["offsets"], w_gate, w_up, w_down, n_ffn)
    y = combine(x, y_perm, r["topk_idx"], r["topk_gate"], dsp["inv_perm"], n_ffn)
    out = dict(r)
    out.update(dsp)
    out.update(x_perm=x_perm, y_perm=y_perm, y=y)
    return out
