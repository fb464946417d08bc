"""Plain, slow, fp64 CPU oracle for one sparse Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
use it.  It shares no code with the HIP library and imports nothing from it.

Sources (cited by page title and section; every step below names its passage):
  [CH36]  "LLM from scratch", chapter 36 "Mixture-of-Experts models"
          (faketrader.github.io/llm-from-scratch, 27-mixture-experts):
          §36.1 notation / dense and sparse mixture, §36.2 the two weight
          conventions and the tie rule, §36.3 dispatch, capacity and overflow,
          §36.4 load statistics, the worked example and Algorithm 36.1,
          §36.5 parameter and FLOP accounting, §36.6 shared experts.
  [REVIEW] "The real cost of sparse expert models: routing, capacity
          constraints and distributed communication" (auturnal.com review),
          its equation list: y(x), C_e and O, rho_max.
  [ROUTING] "MoE mixture-of-experts models" (blog.vegetog.com, moe-token-routing):
          §2 router and top-k, §3 SwiGLU expert and weighted sum, §6 capacity.
  [SKEWER] "Sizzling MoE skewer analogy" (lzwjava.github.io): the corrected
          forward pass and the DeepSeek-V3 shared-expert formula.

Conventions (readings of the pages, each one justified where it is used):
  * tokens T (the chapter's N), experts E (its E_r), expert width m (its d_f).
  * expert ids are 0-based.
  * weights use the out-features x in-features storage convention:
      router      w_r    [E, d]    (logits = x @ w_r.T + b_r)
      expert gate w_gate [E, m, d], up w_up [E, m, d], down w_down [E, d, m]
    [CH36] §36.8 notes that storing a projection as (out x in) instead of
    (in x out) is only a transpose convention.
  * all arithmetic is fp64, except where a step states a rounding point.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional, Sequence, Tuple, Union

import numpy as np

GATE_RENORM = 0   # renormalise within the selected set ([CH36] §36.2 first convention)
GATE_SWITCH = 1   # keep the full-softmax probability ([CH36] §36.2 second convention)

# Two literal forms of the renormalised weights; equal in exact arithmetic
# ([ROUTING] §2 states the equivalence).
RENORM_FORM_SOFTMAX_THEN_RENORM = "softmax_then_renorm"
RENORM_FORM_TOPK_THEN_SOFTMAX = "topk_then_softmax"


class OracleError(ValueError):
    """Invalid arguments, as Algorithm 36.1 ([CH36] §36.4) checks them."""


class NonFiniteLogit(OracleError):
    """A non-finite router score: Algorithm 36.1 treats it as an input failure."""


# --------------------------------------------------------------------------
# capacity and accounting
# --------------------------------------------------------------------------

def capacity(T: int, k: int, E: int, cf_num: int, cf_den: int) -> int:
    """C = ceil(cf * T * k / E) with cf = cf_num / cf_den, exact integer arithmetic.

    [REVIEW] equation for C_e; [CH36] §36.3 capacity rule (same capacity for
    every expert); [ROUTING] §6 top-1 example C = ceil((T/N) * 1.25).
    """
    if cf_num <= 0 or cf_den <= 0 or E <= 0 or k <= 0 or T < 0:
        raise OracleError("capacity: bad arguments")
    num = cf_num * T * k
    den = cf_den * E
    return -(-num // den)


def expert_params(d: int, m: int) -> int:
    """Parameters of one bias-free gated FFN expert: 3*d*m ([CH36] §36.5;
    [ROUTING] §4 Mixtral accounting)."""
    return 3 * d * m


def router_params(d: int, E: int) -> int:
    """Bias-free router parameters d*E ([ROUTING] §2)."""
    return d * E


# --------------------------------------------------------------------------
# rounding helpers (definitions written out)
# --------------------------------------------------------------------------

def round_to_f32(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest fp32 (IEEE round-to-nearest-even)."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bfloat16 (8 significant bits, fp32 exponent range),
    round-to-nearest, ties to even, returned as fp64.

    Written from the format's definition: v = f * 2**e with f in [0.5, 1);
    a bf16 value has 8 significant bits, so the spacing at v is 2**(e-8);
    below the smallest normal (2**-126) the spacing stays 2**-133.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = (v != 0) & np.isfinite(v)
    f, e = np.frexp(v[nz])
    spacing_exp = np.maximum(e - 8, -133)
    scale = np.ldexp(1.0, spacing_exp)
    # np.round rounds halves to the nearest even integer.
    out[nz] = np.round(v[nz] / scale) * scale
    out[~nz] = v[~nz]
    return out


# --------------------------------------------------------------------------
# router: logits, probabilities, selection, weights
# --------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_r: np.ndarray, b_r: Optional[np.ndarray]):
    """g[t,e] = sum_i x[t,i] * w_r[e,i] + b_r[e].

    [CH36] §36.1 (router scores G = X W_r + b_r, W_r stored here as [E, d]);
    [ROUTING] §2 (a linear map from d to one logit per expert).
    The sum is taken in fp64 from the exact input values; the router's
    outputs are fp32 values, so the result is then rounded to fp32 once.
    Returns (g64, g32), both as fp64 arrays [T, E].
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_r, dtype=np.float64)
    g64 = x @ w.T
    if b_r is not None:
        g64 = g64 + np.asarray(b_r, dtype=np.float64)[None, :]
    g32 = round_to_f32(g64)
    # -0.0 and +0.0 are equal scores: canonicalise so that they tie.
    g32 = g32 + 0.0
    return g64, g32


def check_finite(g32: np.ndarray) -> None:
    """Non-finite scores are an input failure and never enter selection
    (Algorithm 36.1, [CH36] §36.4)."""
    if not np.all(np.isfinite(g32)):
        raise NonFiniteLogit("non-finite router logit")


def softmax_rows(g: np.ndarray) -> np.ndarray:
    """P = softmax(G) along the expert axis, stabilised by subtracting the row
    maximum ([CH36] §36.1 and §36.4 "stable softmax")."""
    g = np.asarray(g, dtype=np.float64)
    z = np.exp(g - g.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def select_topk(g32: np.ndarray, k: int) -> np.ndarray:
    """k distinct expert ids with the highest scores, in rank order (highest
    first); equal scores go to the lower expert id.

    [CH36] §36.1 (top-k = the k highest scores, distinct ids), Algorithm 36.1
    (descending score, ties by ascending expert id).  Selection is made on the
    fp32 logits; softmax preserves their order ([CH36] §36.1), so this is the
    same set as selecting by probability wherever probabilities differ.
    Implemented as k passes of an arg-max (np.argmax returns the first, i.e.
    lowest, index among equal maxima).
    """
    T, E = g32.shape
    work = np.array(g32, dtype=np.float64, copy=True)
    ids = np.empty((T, k), dtype=np.int64)
    for r in range(k):
        pick = np.argmax(work, axis=1)
        ids[:, r] = pick
        work[np.arange(T), pick] = -np.inf
    return ids


def gate_weights(g32: np.ndarray, ids: np.ndarray, mode: int,
                 renorm_form: str = RENORM_FORM_SOFTMAX_THEN_RENORM) -> np.ndarray:
    """Mixing weights a_te for the selected experts, in the order of `ids`.

    mode GATE_RENORM ([CH36] §36.2 eq. (36.5) reading; [ROUTING] §2;
    [SKEWER] corrected forward):
      softmax_then_renorm: a = p_e / sum_{j in S} p_j with p = softmax over all E;
      topk_then_softmax:   a = softmax over the selected logits only.
    mode GATE_SWITCH ([CH36] §36.2 second convention): a = p_e, the
      full-softmax probability; the kept weights sum to at most one.
    """
    rows = np.arange(g32.shape[0])[:, None]
    if mode == GATE_SWITCH:
        return softmax_rows(g32)[rows, ids]
    if mode != GATE_RENORM:
        raise OracleError("unknown gate mode")
    if renorm_form == RENORM_FORM_SOFTMAX_THEN_RENORM:
        p = softmax_rows(g32)[rows, ids]
        return p / p.sum(axis=1, keepdims=True)
    if renorm_form == RENORM_FORM_TOPK_THEN_SOFTMAX:
        return softmax_rows(g32[rows, ids])
    raise OracleError("unknown renormalisation form")


def route_margins(g64: np.ndarray, k: int):
    """Score gaps that decide the selection, from the fp64 logits.

    boundary[t]  = (k-th largest) - ((k+1)-th largest)   (inf when k == E)
    adjacent[t,r] = r-th largest - (r+1)-th largest for r < k-1 (rank order).
    Used only to flag near-ties, where a rounding difference between two
    correct fp32 evaluations may legitimately change the selected set.
    """
    s = -np.sort(-np.asarray(g64, dtype=np.float64), axis=1)
    E = s.shape[1]
    if k < E:
        boundary = s[:, k - 1] - s[:, k]
    else:
        boundary = np.full(s.shape[0], np.inf)
    adjacent = s[:, : k - 1] - s[:, 1:k] if k > 1 else np.zeros((s.shape[0], 0))
    return boundary, adjacent


# --------------------------------------------------------------------------
# dispatch: capacity-limited slot assignment, the serial definition
# --------------------------------------------------------------------------

@dataclass
class Dispatch:
    slot: np.ndarray            # [T, k] slot index c within the expert, or -1 (rejected)
    load: np.ndarray            # [E] requested load L_e (before capacity)
    accepted: np.ndarray        # [E] accepted count min(L_e, C)
    offsets: np.ndarray         # [E+1] exclusive prefix sum of accepted counts
    row_of: np.ndarray          # [T, k] offsets[e] + slot, or -1
    src_token: np.ndarray       # [A] token of each grouped row (expert-major, token order)
    capacity: int
    overflow: int               # O = sum_e max(0, L_e - C)
    max_load: int
    rejected_paths: int
    tokens_affected: int        # tokens with at least one rejected path
    tokens_dropped: int         # tokens with every path rejected
    rho_max: float              # max_e L_e / (T k / E)


def assign_slots(ids: np.ndarray, E: int, C: int) -> Dispatch:
    """Token-order first-come-first-served acceptance with capacity C.

    Algorithm 36.1 ([CH36] §36.4): per-expert slot counters c_e start at 0;
    for each token in order and each of its selected paths, the path takes
    slot c_e if c_e < C, otherwise it is rejected; c_e is incremented for
    every request so that it ends as the requested load n_e ([CH36] §36.3).
    Overflow O and rho_max follow the [REVIEW] equations for O and rho_max;
    rho_max uses the requested (pre-capacity) load ([CH36] §36.4).
    Rejected paths contribute nothing and the other weights are not
    renormalised ([CH36] §36.3 overflow, Algorithm 36.1).
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    if C < 1:
        raise OracleError("capacity must be >= 1")
    counter = [0] * E
    slot = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for r in range(k):
            e = int(ids[t, r])
            if counter[e] < C:
                slot[t, r] = counter[e]
            counter[e] += 1
    return _dispatch_from_slots(ids, slot, np.array(counter, dtype=np.int64), E, C)


def assign_slots_by_gate(ids: np.ndarray, w: np.ndarray, E: int, C: int) -> Dispatch:
    """Acceptance by routing weight instead of arrival order.

    [CH36] §36.3 (acceptance rules): the capacity competition inside a routing
    group may be decided by gate weight, so that low-weight paths are the ones
    that lose compute.  Reading: for each expert, its requests are ranked by
    their routing weight a_{t,e}, larger first, equal weights in token order;
    the first C are accepted.  The accepted paths keep token order inside the
    expert's group of rows (slot = number of accepted earlier tokens of that
    expert), so the grouped layout is the same as under first-come-first-served.
    `w` are the routing weights the decision is taken on (fp32 values).
    """
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(w)
    T, k = ids.shape
    if C < 1:
        raise OracleError("capacity must be >= 1")
    requests = [[] for _ in range(E)]          # (t, r) in token order
    for t in range(T):
        for r in range(k):
            requests[int(ids[t, r])].append((t, r))
    slot = np.full((T, k), -1, dtype=np.int64)
    for e in range(E):
        ranked = sorted(requests[e], key=lambda tr: (-float(w[tr[0], tr[1]]), tr[0]))
        accepted = sorted(ranked[:C])          # back to token order
        for c, (t, r) in enumerate(accepted):
            slot[t, r] = c
    load = np.array([len(q) for q in requests], dtype=np.int64)
    return _dispatch_from_slots(ids, slot, load, E, C)


@dataclass
class Reroute:
    dispatch: Dispatch          # over the 2k columns: k candidates, then k spares
    rerouted: int               # spare paths accepted
    tokens_affected: int        # tokens with at least one candidate rejected in the first pass
    tokens_dropped: int         # tokens left with no accepted path


def assign_slots_reroute(ids2: np.ndarray, k: int, E: int, C: int) -> Reroute:
    """Acceptance with rerouting to the next-choice expert.

    [REVIEW] item 5 (capacity overflow as part of the quality record) names
    rerouting to the next-choice expert as one treatment of a full expert;
    [CH36] §36.3 (routing capacity and overflow) says a reroute calls another
    set of parameters; [ROUTING] §6 lists it among the overflow treatments.
    None of them fixes the rule, so this is a reading (stated where it is used):
      * ids2 [T, 2k]: columns 0..k-1 are the token's selection S_t in rank
        order, columns k..2k-1 its next experts in rank order (the spares;
        -1 where the experts run out);
      * first pass: Algorithm 36.1 ([CH36] §36.4) on the candidates, in token
        order; c_e counts every request and ends as the requested load L_e;
      * second pass, after every first-pass request: the j-th rejected
        candidate of token t (rank order) asks for spare j of token t, in token
        order; it is accepted iff its expert has accepted fewer than C paths,
        and then takes the next slot; otherwise it is dropped (no third try).
    The slots of column k + j are those of the spare requests.
    """
    ids2 = np.asarray(ids2, dtype=np.int64)
    T = ids2.shape[0]
    if C < 1:
        raise OracleError("capacity must be >= 1")
    counter = [0] * E
    slot = np.full((T, 2 * k), -1, dtype=np.int64)
    for t in range(T):                        # first pass: Algorithm 36.1
        for r in range(k):
            e = int(ids2[t, r])
            if counter[e] < C:
                slot[t, r] = counter[e]
            counter[e] += 1
    taken = [min(c, C) for c in counter]      # accepted paths per expert so far
    rerouted = affected = dropped = 0
    for t in range(T):                        # second pass: the rejected candidates, in token order
        rejected = [r for r in range(k) if slot[t, r] < 0]
        affected += bool(rejected)
        for j in range(len(rejected)):
            e = int(ids2[t, k + j])
            if e < 0:                          # no next-choice expert left
                continue
            if taken[e] < C:
                slot[t, k + j] = taken[e]
                taken[e] += 1
                rerouted += 1
        dropped += not (slot[t] >= 0).any()
    disp = _dispatch_from_slots(ids2, slot, np.array(counter, dtype=np.int64), E, C)
    return Reroute(dispatch=disp, rerouted=rerouted, tokens_affected=affected, tokens_dropped=dropped)


def spare_weights(g32: np.ndarray, ids: np.ndarray, spare: np.ndarray, mode: int,
                  renorm_form: str = RENORM_FORM_SOFTMAX_THEN_RENORM) -> np.ndarray:
    """Routing weight of a spare (next-choice) expert: the gate value of the
    expert that would compute the path, with the token's selection normalizer
    (a reading; no renormalisation, as in Algorithm 36.1):
      RENORM  p_e' / sum_{j in S_t} p_j  (both forms of gate_weights);
      SWITCH  p_e', the full-softmax probability.
    Entries of `spare` equal to -1 (no expert left) get weight 0."""
    rows = np.arange(g32.shape[0])[:, None]
    sp = np.maximum(np.asarray(spare, dtype=np.int64), 0)
    if mode == GATE_SWITCH:
        w = softmax_rows(g32)[rows, sp]
    elif mode != GATE_RENORM:
        raise OracleError("unknown gate mode")
    elif renorm_form == RENORM_FORM_SOFTMAX_THEN_RENORM:
        p = softmax_rows(g32)
        w = p[rows, sp] / p[rows, ids].sum(axis=1, keepdims=True)
    elif renorm_form == RENORM_FORM_TOPK_THEN_SOFTMAX:
        gsel = g32[rows, ids]
        top = gsel.max(axis=1, keepdims=True)
        w = np.exp(g32[rows, sp] - top) / np.exp(gsel - top).sum(axis=1, keepdims=True)
    else:
        raise OracleError("unknown renormalisation form")
    return np.where(np.asarray(spare) >= 0, w, 0.0)


def _dispatch_from_slots(ids: np.ndarray, slot: np.ndarray, load: np.ndarray, E: int, C: int) -> Dispatch:
    """Grouped-row offsets, row map and load statistics from per-path slots
    ([REVIEW] equations for C_e, O and rho_max; rho_max on the requested load).
    The rows of expert e are its accepted paths, counted from the slots."""
    T, k = ids.shape
    accepted = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for r in range(k):
            if slot[t, r] >= 0:
                accepted[ids[t, r]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(accepted)
    row_of = np.where(slot >= 0, offsets[np.maximum(ids, 0)] + slot, -1)
    src_token = np.empty(int(offsets[-1]), dtype=np.int64)
    for t in range(T):
        for r in range(k):
            if row_of[t, r] >= 0:
                src_token[row_of[t, r]] = t
    rejected = slot < 0
    mean_load = T * k / E if T > 0 else 0.0
    return Dispatch(
        slot=slot, load=load, accepted=accepted, offsets=offsets, row_of=row_of,
        src_token=src_token, capacity=C,
        overflow=int(np.maximum(load - C, 0).sum()),
        max_load=int(load.max()) if E > 0 else 0,
        rejected_paths=int(rejected.sum()),
        tokens_affected=int(rejected.any(axis=1).sum()) if T > 0 else 0,
        tokens_dropped=int(rejected.all(axis=1).sum()) if T > 0 else 0,
        rho_max=(float(load.max()) / mean_load) if T > 0 else 0.0,
    )


def balance_stats(g32: np.ndarray, ids: np.ndarray, E: int):
    """f_e (pre-capacity assignment share) and p_bar_e (mean router
    probability), each summing to one, and the auxiliary balance value
    E * sum_e f_e * p_bar_e (reading of [CH36] §36.4 eqs. (36.14)-(36.15)
    with lambda = 1; it equals 1 at the uniform reference point)."""
    T, k = ids.shape
    f = np.bincount(np.asarray(ids).ravel(), minlength=E).astype(np.float64) / (T * k)
    p_bar = softmax_rows(g32).mean(axis=0)
    return f, p_bar, float(E * np.dot(f, p_bar))


# --------------------------------------------------------------------------
# experts and combine
# --------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)) ([ROUTING] §3)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(xrows: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
               w_down: np.ndarray, round_h_bf16: bool) -> np.ndarray:
    """E_i(x) = [SiLU(x W_gate,i) (*) (x W_up,i)] W_down,i  ([ROUTING] §3;
    [CH36] §36.1 gated feed-forward expert with W_g, W_u in d x d_f and W_d in
    d_f x d; stored here transposed, as out x in).

    Each row of `xrows` is one token; rows are independent.  With bf16
    operands every GEMM input is bf16, so the intermediate h is rounded to
    bf16 before the down projection (a stated reading: the pages fix no
    rounding point; bf16 inputs with fp32 accumulation imply it).
    """
    x = np.asarray(xrows, dtype=np.float64)
    a = x @ np.asarray(w_gate, dtype=np.float64).T
    b = x @ np.asarray(w_up, dtype=np.float64).T
    h = silu(a) * b
    if round_h_bf16:
        h = round_to_bf16(h)
    return h @ np.asarray(w_down, dtype=np.float64).T


def survivor_weights(row_of: np.ndarray, w: np.ndarray) -> np.ndarray:
    """The overflow variant that renormalises over the surviving paths: each
    accepted weight is divided by the sum of the token's accepted weights
    ([CH36] §36.4 worked example: with its only surviving expert, token 4's
    weight becomes one); rejected paths keep weight 0 and a token with no
    accepted path has no weights."""
    w = np.asarray(w, dtype=np.float64)
    acc = np.asarray(row_of) >= 0
    out = np.zeros_like(w)
    for t in range(w.shape[0]):
        tot = float(w[t][acc[t]].sum())
        if tot > 0:
            out[t][acc[t]] = w[t][acc[t]] / tot
    return out


def combine(T: int, width: int, row_of: np.ndarray, w: np.ndarray,
            path_out: np.ndarray, shared_out: Optional[np.ndarray] = None,
            tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """Y_t = s_t + sum over accepted paths r of a_{t,r} * H[row_of[t,r]].

    Algorithm 36.1 ([CH36] §36.4): every accepted record is added once into
    its token's row; rejected records (row_of == -1) add nothing and the
    remaining weights are not renormalised.  [ROUTING] §3 worked sum;
    [SKEWER] shared expert added unweighted.
    `path_out` is indexed by grouped row; `tokens` restricts the output rows.
    """
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    y = np.zeros((len(tokens), width), dtype=np.float64)
    if shared_out is not None:
        y += np.asarray(shared_out, dtype=np.float64)
    for i, t in enumerate(tokens):
        for r in range(row_of.shape[1]):
            row = int(row_of[t, r])
            if row >= 0:
                y[i] += float(w[t, r]) * np.asarray(path_out[row], dtype=np.float64)
    return y


# --------------------------------------------------------------------------
# whole forward
# --------------------------------------------------------------------------

WeightsArg = Union[Tuple[np.ndarray, np.ndarray, np.ndarray],
                   Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]]


def _expert(weights: WeightsArg, e: int):
    if callable(weights):
        return weights(e)
    wg, wu, wd = weights
    return wg[e], wu[e], wd[e]


@dataclass
class Route:
    g64: np.ndarray
    g32: np.ndarray
    ids: np.ndarray
    w: np.ndarray


def route(x, w_r, b_r, k: int, mode: int,
          renorm_form: str = RENORM_FORM_SOFTMAX_THEN_RENORM) -> Route:
    """Scores, probabilities, top-k and weights (Algorithm 36.1 steps 1-2)."""
    x = np.asarray(x)
    E = np.asarray(w_r).shape[0]
    if not (1 <= k <= E):
        raise OracleError("need 1 <= k <= E")
    g64, g32 = router_logits(x, w_r, b_r)
    check_finite(g32)
    ids = select_topk(g32, k)
    return Route(g64=g64, g32=g32, ids=ids, w=gate_weights(g32, ids, mode, renorm_form))


@dataclass
class ForwardResult:
    y: np.ndarray
    tokens: np.ndarray
    route: Route
    dispatch: Dispatch
    stats: dict = field(default_factory=dict)


def forward(x, w_r, b_r, experts: WeightsArg, k: int, mode: int,
            C: Optional[int] = None, shared: Optional[WeightsArg] = None,
            round_h_bf16: bool = False,
            renorm_form: str = RENORM_FORM_SOFTMAX_THEN_RENORM,
            tokens: Optional[Sequence[int]] = None,
            ids_override: Optional[np.ndarray] = None,
            accept_by_gate: bool = False, renorm_survivors: bool = False,
            accept_weights: Optional[np.ndarray] = None, reroute: bool = False) -> ForwardResult:
    """One sparse MoE layer forward, Algorithm 36.1 ([CH36] §36.4) with the
    conventions above.  The output excludes the residual ([CH36] §36.3: a
    token whose every path is rejected keeps only its residual, which the
    caller adds).

    C=None means no capacity limit (C = T, so nothing can be rejected).
    `tokens` evaluates the expert FFNs and the combine for those output rows
    only; routing and slot assignment always cover the whole routing group,
    because acceptance depends on every earlier token ([CH36] §36.3).
    `ids_override` replaces the selected ids (weights are recomputed for
    them), for staged comparisons where a near-tie flipped a selection.
    `shared` is one expert's (w_gate [m_s,d], w_up [m_s,d], w_down [d,m_s]),
    always applied and unweighted ([CH36] §36.6; [SKEWER] DeepSeek-V3 formula).
    Overflow variants ([CH36] §36.3-§36.4): `accept_by_gate` decides the
    capacity competition by routing weight (assign_slots_by_gate), on
    `accept_weights` if given (the fp32 weights of the run being checked, so
    that both sides take the decision on the same values) else on the weights
    rounded to fp32; `renorm_survivors` renormalises each token's weights over
    its accepted paths (survivor_weights).  `reroute` sends every rejected path
    to the token's next-choice expert (assign_slots_reroute); the routing
    records then have 2k columns, the k selected experts and the k spares
    (ids_override is then [T, 2k] as well), weighted by spare_weights.
    """
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(w_r).shape[0]
    if not (1 <= k <= E):
        raise OracleError("need 1 <= k <= E")
    if C is not None and C < 1:
        raise OracleError("capacity must be >= 1")
    d = x.shape[1]
    if T == 0:
        empty = np.zeros((0, k), dtype=np.int64)
        r = Route(np.zeros((0, E)), np.zeros((0, E)), empty, np.zeros((0, k)))
        disp = assign_slots(empty, E, C if C is not None else 1)
        return ForwardResult(np.zeros((0, d)), np.zeros(0, dtype=np.int64), r, disp)
    rt = route(x, w_r, b_r, k, mode, renorm_form)
    cap = T if C is None else C
    rr = None
    if reroute:
        if accept_by_gate:
            raise OracleError("rerouting is read with acceptance in token order")
        n = min(2 * k, E)
        ids2 = np.full((T, 2 * k), -1, dtype=np.int64)
        ids2[:, :n] = select_topk(rt.g32, n)
        if ids_override is not None:
            ids2 = np.asarray(ids_override, dtype=np.int64)
        w2 = np.zeros((T, 2 * k))
        w2[:, :k] = gate_weights(rt.g32, ids2[:, :k], mode, renorm_form)
        w2[:, k:] = spare_weights(rt.g32, ids2[:, :k], ids2[:, k:], mode, renorm_form)
        rt.ids, rt.w = ids2, w2
        rr = assign_slots_reroute(ids2, k, E, cap)
        disp = rr.dispatch
    else:
        if ids_override is not None:
            rt.ids = np.asarray(ids_override, dtype=np.int64)
            rt.w = gate_weights(rt.g32, rt.ids, mode, renorm_form)
        if accept_by_gate:
            aw = round_to_f32(rt.w) if accept_weights is None else np.asarray(accept_weights)
            disp = assign_slots_by_gate(rt.ids, aw, E, cap)
        else:
            disp = assign_slots(rt.ids, E, cap)
    w_comb = survivor_weights(disp.row_of, rt.w) if renorm_survivors else rt.w
    P = rt.ids.shape[1]   # routing records per token: k, or 2k with rerouting
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)

    # Expert FFN per accepted path of the requested tokens, evaluated expert
    # by expert (rows are independent, so this is the row-wise definition).
    path_out = {}
    for e in range(E):
        sel = [(int(t), r) for t in tok for r in range(P)
               if rt.ids[t, r] == e and disp.slot[t, r] >= 0]
        if not sel:
            continue
        wg, wu, wd = _expert(experts, e)
        z = swiglu_ffn(x[[t for t, _ in sel]].astype(np.float64), wg, wu, wd, round_h_bf16)
        for (t, r), zr in zip(sel, z):
            path_out[int(disp.row_of[t, r])] = zr
    # Every expert maps width d back to width d ([CH36] §36.1).
    d_out = d

    s = None
    if shared is not None:
        sg, su, sd = shared
        s = swiglu_ffn(x[tok].astype(np.float64), sg, su, sd, round_h_bf16)

    y = np.zeros((len(tok), d_out), dtype=np.float64)
    if s is not None:
        y += s
    for i, t in enumerate(tok):
        for r in range(P):
            row = int(disp.row_of[t, r])
            if row >= 0:
                y[i] += float(w_comb[t, r]) * path_out[row]
    stats = dict(load=disp.load, accepted=disp.accepted, overflow=disp.overflow,
                 max_load=disp.max_load, rho_max=disp.rho_max,
                 tokens_dropped=disp.tokens_dropped, tokens_affected=disp.tokens_affected,
                 rejected_paths=disp.rejected_paths)
    if rr is not None:
        stats.update(rerouted=rr.rerouted, tokens_dropped=rr.tokens_dropped, tokens_affected=rr.tokens_affected,
                     rejected_paths=disp.overflow - rr.rerouted)
    return ForwardResult(y=y, tokens=tok, route=rt, dispatch=disp, stats=stats)


def dense_forward(x, w_r, b_r, experts: WeightsArg, round_h_bf16: bool = False) -> np.ndarray:
    """Dense mixture: every expert runs on every token and is weighted by its
    full-softmax probability, y_t = sum_e p_te F_e(x_t) ([CH36] §36.1).
    Written separately from the sparse path (no selection, no dispatch); with
    k = E and no capacity limit the sparse layer must reduce to it."""
    x = np.asarray(x, dtype=np.float64)
    E = np.asarray(w_r).shape[0]
    logits = x @ np.asarray(w_r, dtype=np.float64).T
    if b_r is not None:
        logits = logits + np.asarray(b_r, dtype=np.float64)[None, :]
    logits = round_to_f32(logits)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    y = None
    for e in range(E):
        wg, wu, wd = _expert(experts, e)
        out = p[:, e:e + 1] * swiglu_ffn(x, wg, wu, wd, round_h_bf16)
        y = out if y is None else y + out
    return y
