"""Plain CPU oracle of the LatentMoE layer forward (numpy, float64).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the library path never does.

It computes, slowly and in the most direct way, what the layer is stated to
compute on two pages:
  [QA]  "Nemotron 3 Ultra 架构 QA" (cctoctofx.netlify.app), CH5 Q5.1-Q5.8 and
        CH2 Q2.6 (activation), CH3 Q3.1 (FLOP split);
  [WT]  the Nemotron-3-Labs-Ultra-Math-SFT architecture walkthrough
        (2kiu.com/news/5890699), section "LatentMoE 层".

Layer (QA Q5.1 and Q5.7; WT "LatentMoE 层"):
  out = fc2( sum_{e in topK} g_e * Expert_e( fc1(x) ) ) + Shared(x)
with
  router logits l = x(fp32) . W_r^T in fp32                   (QA Q5.2)
  s = sigmoid(l); choice c = s + e_score_correction_bias       (QA Q5.2, Q5.3)
  top-K experts by c; weights are the unbiased s of the chosen
  experts, normalised to sum 1, then times routed_scaling      (WT "路由与共享专家", QA Q5.8)
  Expert_e(z) = down_e( relu(up_e(z))^2 ), no gate projection  (QA Q2.6, Q5.5, Q5.6)
  the gate multiplies each expert's output before the sum     (QA Q5.5 point 3)
  Shared(x) = sh_down( relu(sh_up(x))^2 ), on the uncompressed x,
  added in parallel                                            (QA Q5.7; WT)

Readings where the pages leave a step open (each listed in the design notes):
  * the router reads the uncompressed x (QA Q5.2 flattens to hidden_size);
  * expert groups: WT "路由与共享专家" says the top-K is taken within groups,
    and QA CH9 Q9.2 has the MoE inherit DeepseekV3MoE's routing, but no page
    gives a group count, how experts are grouped or how a group is scored.
    ``route`` takes n_group / topk_group (default 1 / 1: top-K over all E
    experts, the only setting the pages' workloads use) and, for n_group > 1,
    follows the DeepSeek-V3 rule of that parent, which comes from outside the
    pages: experts form n_group equal contiguous groups, a group scores the sum
    of its two highest choice scores (its one score if it has one expert), the
    topk_group best groups (ties: lower group index) admit their experts, and
    the top-K is taken among those. PARITY UNPINNED for that group ranking: no
    page fixes it, so no test can check it against a fact. The pins check the
    subset search given the ranking, that admitting every group is the plain
    top-K, and that the choice stays inside the admitted groups;
  * dropless: every (token, expert) pair is computed;
  * ties in the choice score go to the lower expert index;
  * a token's K experts are reported in ascending expert order (the sum over
    them is order-free in exact arithmetic);
  * all sums accumulate in float64 here; with ``mirror=True`` values are
    rounded to bf16 where the layer stores a bf16 tensor (z, h, y, the
    combined latent, the shared hidden, out), otherwise nothing is rounded.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, Optional, Tuple

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "round_bf16", "RouteResult", "PermuteResult",
    "route", "permute", "expert_mlp", "forward", "GAP_FLAG",
]

# near-tie band on the K-th / (K+1)-th choice-score gap inside which several
# routings are accepted as correct
GAP_FLAG = 1e-4


# ----------------------------------------------------------------------------
# bf16 <-> float64
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns: a bf16 is the upper 16 bits of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits: a value in [2**(e-1), 2**e) is rounded to a
    multiple of 2**(e-8). Below the smallest normal (2**-126) the spacing stays
    2**-133. Returned as float64 (exactly representable values).
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)                      # a = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    return np.rint(a / q) * q               # np.rint rounds half to even


# ----------------------------------------------------------------------------
# router: logits, sigmoid, biased top-K choice, renormalised gates
# ----------------------------------------------------------------------------

@dataclass
class RouteResult:
    idx: np.ndarray      # [T,K] int32, ascending expert index within a token
    gate: np.ndarray     # [T,K] float32, routed_scaling * s / sum(s) over the chosen set
    gap: np.ndarray      # [T] float64, c_(K) - c_(K+1) in descending order (+inf if K == E)
    logits: np.ndarray   # [T,E] float64
    score: np.ndarray    # [T,E] float64, sigmoid(logits)
    choice: np.ndarray   # [T,E] float64, score + bias


def route(x: np.ndarray, w_router: np.ndarray, corr_bias: np.ndarray, K: int,
          routed_scaling: float, n_group: int = 1, topk_group: int = 1, dtype=np.float64) -> RouteResult:
    """Router of QA Q5.2 / Q5.3 with the gate rule of WT "路由与共享专家" and QA Q5.8.

    x: [T,H] float64 (bf16 values); w_router: [E,H] (fp32 values); corr_bias: [E].
    n_group / topk_group: group-limited selection (module docstring); 1 / 1 is
    the plain top-K over all experts. dtype: the arithmetic type (float64, the
    parity mode; float32 only to time the same code at single precision).

    gap[t] is the smallest margin that decides token t's routing: the K-th
    minus the (K+1)-th choice score among the admitted experts, and, with
    groups, the topk_group-th minus the next group score (inf when nothing
    follows).
    """
    x = np.asarray(x, dtype=dtype)
    wr = np.asarray(w_router, dtype=dtype)
    b = np.asarray(corr_bias, dtype=dtype)
    T = x.shape[0]
    E = wr.shape[0]
    assert np.all(np.isfinite(x)) and np.all(np.isfinite(wr)) and np.all(np.isfinite(b))
    assert n_group >= 1 and E % n_group == 0 and 1 <= topk_group <= n_group
    G = E // n_group
    assert 1 <= K <= topk_group * G
    logits = x @ wr.T                                  # fp32 inputs, exact products in fp64
    score = 1.0 / (1.0 + np.exp(-logits))              # independent per expert (QA Q5.2)
    choice = score + b[None, :]                        # bias steers the choice only (QA Q5.3)
    experts = np.arange(E)
    groups = np.arange(n_group)
    idx = np.empty((T, K), dtype=np.int32)
    gap = np.empty(T, dtype=np.float64)
    for t in range(T):
        c = choice[t]
        # group score: the sum of the group's two highest choice scores
        gs = np.array([np.sort(c[g * G:(g + 1) * G])[::-1][:2].sum() for g in groups])
        gorder = np.lexsort((groups, -gs))             # best groups first, ties -> lower group
        admitted = np.sort(np.concatenate([experts[g * G:(g + 1) * G] for g in gorder[:topk_group]]))
        # descending choice score, equal scores -> lower expert index first
        order = admitted[np.lexsort((admitted, -c[admitted]))]
        chosen = order[:K]
        egap = c[order[K - 1]] - c[order[K]] if K < len(order) else np.inf
        ggap = gs[gorder[topk_group - 1]] - gs[gorder[topk_group]] if topk_group < n_group else np.inf
        gap[t] = min(egap, ggap)
        idx[t] = np.sort(chosen)
    s_sel = np.take_along_axis(score, idx.astype(np.int64), axis=1)
    gate = (routed_scaling * s_sel / s_sel.sum(axis=1, keepdims=True)).astype(np.float32)
    return RouteResult(idx=idx, gate=gate, gap=gap, logits=logits, score=score, choice=choice)


# ----------------------------------------------------------------------------
# permutation: group the T*K (token, slot) pairs by expert, tokens ascending
# ----------------------------------------------------------------------------

@dataclass
class PermuteResult:
    counts: np.ndarray     # [E] int32, tokens per expert
    offsets: np.ndarray    # [E+1] int32, exclusive prefix sum of counts
    row_token: np.ndarray  # [T*K] int32, token of each permuted row
    slot_row: np.ndarray   # [T,K] int32, permuted row of each (token, slot)


def permute(idx: np.ndarray, E: int) -> PermuteResult:
    """Rows of one expert are contiguous, in ascending token order.

    This is the row set that a per-expert loop over the hit experts gathers
    (QA Q5.6 point 3, "for expert_idx in expert_hit"), laid out one expert after
    another.
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    flat_e = idx.reshape(-1)
    flat_t = np.repeat(np.arange(T, dtype=np.int64), K)
    order = np.lexsort((flat_t, flat_e))              # primary key: expert, then token
    counts = np.bincount(flat_e, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    row_token = flat_t[order].astype(np.int32)
    slot_row = np.empty(T * K, dtype=np.int32)
    slot_row[order] = np.arange(T * K, dtype=np.int32)
    return PermuteResult(counts=counts, offsets=offsets, row_token=row_token,
                         slot_row=slot_row.reshape(T, K))


# ----------------------------------------------------------------------------
# MLPs and the whole layer
# ----------------------------------------------------------------------------

def _relu2(a: np.ndarray) -> np.ndarray:
    """relu(a)**2, the "relu2" hidden activation (QA Q2.6)."""
    r = np.maximum(a, 0.0)
    return r * r


def expert_mlp(z: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, rnd: Callable) -> Tuple[np.ndarray, np.ndarray]:
    """Non-gated MLP down(relu(up(z))^2) with [out,in] weights (QA Q2.6, Q5.5, Q5.6)."""
    h = rnd(_relu2(z @ w_up.T))
    y = rnd(h @ w_down.T)
    return h, y


def _identity(a):
    return a


def forward(x_bits: np.ndarray, w_router: np.ndarray, corr_bias: np.ndarray,
            w_fc1_bits: np.ndarray, w_fc2_bits: np.ndarray,
            w_sh_up_bits: np.ndarray, w_sh_down_bits: np.ndarray,
            expert: Callable[[int], Tuple[np.ndarray, np.ndarray]],
            K: int, routed_scaling: float, mirror: bool = True,
            idx_override: Optional[np.ndarray] = None,
            keep: bool = False, n_group: int = 1, topk_group: int = 1,
            dtype=np.float64) -> Dict[str, np.ndarray]:
    """One forward of the layer on the tokens in ``x_bits`` (tokens are independent).

    x_bits [T,H] and the *_bits weights are bf16 bit patterns (uint16);
    w_router [E,H] and corr_bias [E] are float32. ``expert(e)`` returns the bf16
    bit patterns (W_up[e] [I,L], W_down[e] [L,I]) of expert e, so large layers
    can be fed one expert at a time.

    ``idx_override`` replaces the chosen expert sets (the gates still follow the
    stated rule on the unbiased scores of those experts); it is used to follow
    another party's choice on near-tie tokens.

    ``dtype`` is the arithmetic type: float64 is the parity mode; float32 runs
    the same steps at single precision (used only to time the oracle at that
    precision; every parity comparison uses float64).

    Returns out [T,H] (float64; bf16 values when mirror) plus the route and
    permutation results; with ``keep`` also z, h, y, y_lat, hs.
    """
    if mirror:
        def rnd(a):
            return round_bf16(a).astype(dtype)
    else:
        rnd = _identity

    def dec(bits):
        return bf16_bits_to_f64(bits).astype(dtype)

    x = dec(x_bits)
    T, H = x.shape
    E = np.asarray(w_router).shape[0]
    r = route(x, w_router, corr_bias, K, routed_scaling, n_group, topk_group, dtype=dtype)
    if idx_override is not None:
        idx = np.sort(np.asarray(idx_override, dtype=np.int64), axis=1).astype(np.int32)
        assert idx.shape == (T, K)
        for t in range(T):
            assert len(np.unique(idx[t])) == K
        s_sel = np.take_along_axis(r.score, idx.astype(np.int64), axis=1)
        r.idx = idx
        r.gate = (routed_scaling * s_sel / s_sel.sum(axis=1, keepdims=True)).astype(np.float32)
    p = permute(r.idx, E)

    # fc1_latent_proj: compress to the latent (QA Q5.1)
    z = rnd(x @ dec(w_fc1_bits).T)
    L = z.shape[1]

    # routed experts over the latent, one expert's rows at a time
    y = np.zeros((T * K, L), dtype=dtype)
    hs_list = {}
    for e in range(E):
        a, b = int(p.offsets[e]), int(p.offsets[e + 1])
        if a == b:
            continue
        wu_bits, wd_bits = expert(e)
        h_e, y_e = expert_mlp(z[p.row_token[a:b]], dec(wu_bits), dec(wd_bits), rnd)
        y[a:b] = y_e
        if keep:
            hs_list[e] = h_e

    # gate each expert output, then sum in the latent (QA Q5.5 point 3)
    gate64 = r.gate.astype(dtype)
    y_lat = np.zeros((T, L), dtype=dtype)
    for j in range(K):
        y_lat += gate64[:, j:j + 1] * y[p.slot_row[:, j]]
    y_lat = rnd(y_lat)

    # shared expert on the uncompressed input (QA Q5.7)
    hs = rnd(_relu2(x @ dec(w_sh_up_bits).T))

    # fc2_latent_proj plus the shared expert, one rounding at the end (QA Q5.1)
    out = rnd(y_lat @ dec(w_fc2_bits).T + hs @ dec(w_sh_down_bits).T)

    res = dict(out=out, idx=r.idx, gate=r.gate, gap=r.gap, counts=p.counts,
               offsets=p.offsets, row_token=p.row_token, slot_row=p.slot_row)
    if keep:
        h = None
        if hs_list:
            I = next(iter(hs_list.values())).shape[1]
            h = np.zeros((T * K, I), dtype=dtype)
            for e, h_e in hs_list.items():
                h[p.offsets[e]:p.offsets[e + 1]] = h_e
        res.update(z=z, h=h, y=y, y_lat=y_lat, hs=hs, logits=r.logits, score=r.score,
                   choice=r.choice)
    return res
