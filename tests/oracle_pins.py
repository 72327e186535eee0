"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes an oracle module (the real one, or a mutant built by the
mutation test) and raises AssertionError if the oracle disagrees with:
  * brute force (all C(E,K) expert subsets; Python loops for the permutation),
  * a library routine (torch's bf16 conversion, torch float64 linear algebra
    for special cases that reduce to a dense MLP chain),
  * closed forms (identity experts, zero routed path, forced routing),
  * invariants (gates sum to routed_scaling, K distinct experts per token,
    token-permutation equivariance, expert-relabel invariance, scale
    linearity, token independence).
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch

import workloads as W

TOL64 = 1e-12


# ----------------------------------------------------------------------------
# small inputs
# ----------------------------------------------------------------------------

def case(name="tiny", **over):
    """Seeded small inputs as numpy arrays (bf16 as uint16 bit patterns)."""
    if name in W.CONFIGS:
        cfg = W.get_config(name, **over)
    else:
        base = dict(T=24, H=96, L=32, E=12, I=48, K=3, Is=80, bias_halfwidth=0.1, seed=7,
                    weight_key="custom")
        base.update(over)
        cfg = W.MoEConfig(name, **base)
    d = W.make_inputs(cfg)
    u = W.bf16_tensor_to_u16_numpy
    return dict(cfg=cfg, x=u(d["x"]), wr=d["w_router"].numpy().copy(),
                b=d["corr_bias"].numpy().copy(), fc1=u(d["w_fc1"]), fc2=u(d["w_fc2"]),
                su=u(d["w_sh_up"]), sd=u(d["w_sh_down"]), up=u(d["w_up"]), down=u(d["w_down"]))


def run(O, c, mirror=True, scale=None, keep=False, **over):
    cc = dict(c)
    cc.update(over)
    cfg = cc["cfg"]
    up, down = cc["up"], cc["down"]
    return O.forward(cc["x"], cc["wr"], cc["b"], cc["fc1"], cc["fc2"], cc["su"], cc["sd"],
                     lambda e: (up[e], down[e]), cfg.K,
                     cfg.routed_scaling if scale is None else scale, mirror=mirror, keep=keep)


def f64(bits):
    """bf16 bits -> float64 through torch (independent of the oracle's decoder)."""
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64)


def choice_scores(c):
    x = f64(c["x"])
    l = x @ torch.from_numpy(c["wr"]).to(torch.float64).T
    s = torch.sigmoid(l)
    return l.numpy(), s.numpy(), (s + torch.from_numpy(c["b"]).to(torch.float64)).numpy()


def relerr(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def to_bits(a):
    """float64 array of bf16-representable values -> bf16 bit patterns via torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(torch.float32).to(torch.bfloat16)
    assert torch.equal(t.to(torch.float64), torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)))
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# ----------------------------------------------------------------------------
# bf16 conversions
# ----------------------------------------------------------------------------

def pin_bf16_conversions(O):
    v = W.gen_normal_f32(5, 5, (20000,), 3.0).numpy()
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40A08000, 0x3F80FFFF, 0x3F807FFF,
                     0x00018000, 0x7F7F0000], dtype=np.uint32).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.float32([0.0, 1.0, -2.5, 1e-30, 3e38])])
    got = O.round_bf16(v.astype(np.float64))
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, want), "round_bf16 differs from torch's RNE on float32 inputs"
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                 # finite values only
    dec = O.bf16_bits_to_f64(bits)
    assert np.array_equal(dec, f64(bits).numpy())


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------

def pin_route_bruteforce(O):
    for name, over in (("tiny", {}), ("r2", dict(E=10, K=3, T=40, H=64, bias_halfwidth=0.3))):
        c = case(name, **over)
        cfg = c["cfg"]
        _, s, ch = choice_scores(c)
        r = O.route(O.bf16_bits_to_f64(c["x"]), c["wr"], c["b"], cfg.K, cfg.routed_scaling)
        combos = np.array(list(itertools.combinations(range(cfg.E), cfg.K)))
        sums = ch[:, combos].sum(-1)                          # [T, C(E,K)]
        best = combos[np.argmax(sums, axis=1)]
        srt = -np.sort(-ch, axis=1)
        gap = srt[:, cfg.K - 1] - srt[:, cfg.K]
        assert np.all(gap > 1e-9), "case chosen to have no exact ties"
        assert np.array_equal(np.sort(best, 1), r.idx), "top-K set differs from brute force"
        assert np.allclose(r.gap, gap, rtol=0, atol=1e-12), "gap differs from sorted scores"


def pin_route_bias_zero(O):
    c = case("r3", E=20, K=5, T=50, bias_halfwidth=0.0)
    cfg = c["cfg"]
    l, _, _ = choice_scores(c)
    r = O.route(O.bf16_bits_to_f64(c["x"]), c["wr"], c["b"], cfg.K, cfg.routed_scaling)
    want = np.sort(np.argsort(-l, axis=1, kind="stable")[:, :cfg.K], axis=1)
    assert np.array_equal(r.idx, want), "zero bias: sigmoid is monotone, top-K must follow the logits"


def pin_route_forced_and_gates(O):
    c = case("tiny")
    cfg = c["cfg"]
    forced = np.array([1, 5, 9, 14])
    b = np.zeros(cfg.E, np.float32)
    b[forced] = 2.0                       # s in (0,1): +2 beats any unbiased score
    c2 = dict(c, b=b)
    _, s, _ = choice_scores(c2)
    r = O.route(O.bf16_bits_to_f64(c["x"]), c["wr"], b, cfg.K, cfg.routed_scaling)
    assert np.array_equal(r.idx, np.tile(forced, (cfg.T, 1)))
    want = cfg.routed_scaling * s[:, forced] / s[:, forced].sum(1, keepdims=True)
    assert relerr(r.gate, want) < 1e-6, "gates must be the unbiased scores, renormalised and scaled"
    assert np.all(np.abs(r.gap - (2.0 + s[:, forced].min(1) - np.max(np.delete(s, forced, 1), 1))) < 1e-9)


def pin_route_invariants(O):
    for name, over in (("tiny", {}), ("r4", dict(E=40, K=7, T=30, bias_halfwidth=0.05)),
                       ("r5", dict(E=6, K=6, T=10))):
        c = case(name, **over)
        cfg = c["cfg"]
        _, s, _ = choice_scores(c)
        r = O.route(O.bf16_bits_to_f64(c["x"]), c["wr"], c["b"], cfg.K, cfg.routed_scaling)
        assert r.idx.shape == (cfg.T, cfg.K) and r.idx.dtype == np.int32
        assert np.all(np.diff(r.idx, axis=1) > 0), "K distinct experts, ascending"
        assert np.all((r.idx >= 0) & (r.idx < cfg.E))
        assert np.all(np.abs(r.gate.astype(np.float64).sum(1) - cfg.routed_scaling) <= 1e-5)
        ssel = np.take_along_axis(s, r.idx.astype(np.int64), 1)
        ratio = r.gate / ssel
        assert np.all(np.abs(ratio / ratio[:, :1] - 1) < 1e-6), "gates proportional to scores"
        if cfg.K == cfg.E:
            assert np.all(np.isinf(r.gap))
        else:
            assert np.all(r.gap >= 0)


def pin_route_ties(O):
    c = case("r6", E=12, K=4, T=20, bias_halfwidth=0.0)
    wr = c["wr"].copy()
    wr[11] = wr[3]                        # experts 3 and 11 get identical logits
    b = np.zeros(12, np.float32)
    b[[0, 1, 2]] = 2.0
    b[[3, 11]] = 1.0                      # exactly one of {3, 11} fits
    r = O.route(O.bf16_bits_to_f64(c["x"]), wr, b, 4, 5.0)
    assert np.array_equal(r.idx, np.tile([0, 1, 2, 3], (20, 1))), "equal scores: lower index wins"
    assert np.all(r.gap == 0.0)


# ----------------------------------------------------------------------------
# group-limited router (n_group equal contiguous groups, group score = sum of
# the group's two highest choice scores, topk_group groups admitted)
# ----------------------------------------------------------------------------

def _group_brute(ch_t, E, K, n_group, topk_group):
    """Expected (set, gap) for one token by plain Python ranking and subset enumeration."""
    G = E // n_group
    gs = [sum(sorted(ch_t[g * G:(g + 1) * G].tolist())[-2:]) for g in range(n_group)]
    granked = sorted(range(n_group), key=lambda g: (-gs[g], g))
    admitted = [e for g in granked[:topk_group] for e in range(g * G, (g + 1) * G)]
    best, best_sum = None, -math.inf
    for comb in itertools.combinations(admitted, K):
        v = sum(ch_t[list(comb)])
        if v > best_sum:
            best, best_sum = comb, v
    vals = sorted(ch_t[admitted].tolist(), reverse=True)
    egap = vals[K - 1] - vals[K] if K < len(vals) else math.inf
    ggap = gs[granked[topk_group - 1]] - gs[granked[topk_group]] if topk_group < n_group else math.inf
    return sorted(best), min(egap, ggap)


def pin_group_bruteforce(O):
    for name, over, ng, tg in (("tiny", {}, 4, 2),
                               ("g2", dict(E=24, K=5, T=40, H=64, bias_halfwidth=0.2), 6, 3),
                               ("g3", dict(E=12, K=2, T=30, H=64, bias_halfwidth=0.2), 12, 3)):
        c = case(name, **over)
        cfg = c["cfg"]
        _, s, ch = choice_scores(c)
        r = O.route(O.bf16_bits_to_f64(c["x"]), c["wr"], c["b"], cfg.K, cfg.routed_scaling,
                    n_group=ng, topk_group=tg)
        for t in range(cfg.T):
            want, gap = _group_brute(ch[t], cfg.E, cfg.K, ng, tg)
            assert gap > 1e-9, "case chosen to have no exact ties"
            assert list(r.idx[t]) == want, f"token {t}: group-limited set differs from brute force"
            assert abs(r.gap[t] - gap) <= 1e-12, f"token {t}: gap differs"
        ssel = np.take_along_axis(s, r.idx.astype(np.int64), 1)
        want_g = cfg.routed_scaling * ssel / ssel.sum(1, keepdims=True)
        assert relerr(r.gate, want_g) < 1e-6, "gates: unbiased scores of the chosen set, renormalised"


def pin_group_all_admitted_is_plain(O):
    """With every group admitted the rule is the plain top-K over all experts."""
    c = case("tiny")
    cfg = c["cfg"]
    _, _, ch = choice_scores(c)
    combos = np.array(list(itertools.combinations(range(cfg.E), cfg.K)))
    best = np.sort(combos[np.argmax(ch[:, combos].sum(-1), axis=1)], 1)
    for ng in (1, 2, 4, 8):
        r = O.route(O.bf16_bits_to_f64(c["x"]), c["wr"], c["b"], cfg.K, cfg.routed_scaling,
                    n_group=ng, topk_group=ng)
        assert np.array_equal(r.idx, best), f"n_group={ng}, all admitted: must equal the plain top-K"


def pin_group_confinement(O):
    c = case("g4", E=32, K=6, T=60, H=64, bias_halfwidth=0.3)
    cfg = c["cfg"]
    for ng, tg in ((8, 2), (4, 2), (16, 3)):
        G = cfg.E // ng
        r = O.route(O.bf16_bits_to_f64(c["x"]), c["wr"], c["b"], cfg.K, cfg.routed_scaling,
                    n_group=ng, topk_group=tg)
        groups = r.idx // G
        assert all(len(set(row.tolist())) <= tg for row in groups), "experts from more groups than admitted"
        assert np.all(np.diff(r.idx, axis=1) > 0) and np.all(r.gap >= 0)


def pin_group_tie(O):
    """Two groups with exactly equal scores: the lower group is admitted, gap 0."""
    c = case("g5", E=8, K=2, T=16, H=64, bias_halfwidth=0.0)
    wr = c["wr"].copy()
    wr[6], wr[7] = wr[2], wr[3]           # group 3 mirrors group 1
    b = np.zeros(8, np.float32)
    b[[2, 3, 6, 7]] = 1.0
    r = O.route(O.bf16_bits_to_f64(c["x"]), wr, b, 2, 5.0, n_group=4, topk_group=1)
    assert np.array_equal(r.idx, np.tile([2, 3], (16, 1))), "equal group scores: lower group wins"
    assert np.all(r.gap == 0.0)


# ----------------------------------------------------------------------------
# permutation
# ----------------------------------------------------------------------------

def _perm_brute(idx, E):
    T, K = idx.shape
    rows, offsets = [], [0]
    for e in range(E):
        for t in range(T):
            if e in idx[t]:
                rows.append(t)
        offsets.append(len(rows))
    slot_row = np.full((T, K), -1, np.int64)
    for e in range(E):
        seg = rows[offsets[e]:offsets[e + 1]]
        for k, t in enumerate(seg):
            j = list(idx[t]).index(e)
            slot_row[t, j] = offsets[e] + k
    return np.array(rows), np.array(offsets), slot_row


def pin_permute_bruteforce(O):
    rng = np.random.default_rng(3)
    cases = []
    for T, E, K in ((64, 16, 4), (9, 30, 5), (50, 5, 5), (1, 8, 2), (33, 3, 1)):
        idx = np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]).astype(np.int32)
        cases.append((idx, E))
    # a skewed one with idle experts
    idx = np.stack([np.sort(np.array([0, 1, 2 + (t % 3)])) for t in range(40)]).astype(np.int32)
    cases.append((idx, 9))
    for idx, E in cases:
        p = O.permute(idx, E)
        rows, offs, slot = _perm_brute(idx, E)
        T, K = idx.shape
        assert np.array_equal(p.row_token, rows)
        assert np.array_equal(p.offsets, offs)
        assert np.array_equal(p.counts, np.diff(offs))
        assert np.array_equal(p.slot_row, slot)
        assert p.counts.sum() == T * K
        assert np.array_equal(np.sort(p.slot_row.reshape(-1)), np.arange(T * K))
        assert np.array_equal(p.row_token[p.slot_row], np.repeat(np.arange(T)[:, None], K, 1))


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def _relu2(a):
    return torch.relu(a) ** 2


def _mlp(v, up, down):
    F = torch.nn.functional
    return F.linear(_relu2(F.linear(v, up)), down)


def pin_dense_masked(O):
    """Sum over ALL experts with a 0/1 mask and the gate, no permutation, torch fp64."""
    for name, over in (("tiny", {}), ("r7", dict(E=9, K=3, T=21))):
        c = case(name, **over)
        cfg = c["cfg"]
        res = run(O, c, mirror=False)
        F = torch.nn.functional
        x = f64(c["x"])
        z = F.linear(x, f64(c["fc1"]))
        ylat = torch.zeros(cfg.T, cfg.L, dtype=torch.float64)
        gate = torch.from_numpy(res["gate"].astype(np.float64))
        for e in range(cfg.E):
            mask = torch.from_numpy((res["idx"] == e).astype(np.float64))      # [T,K]
            g = (mask * gate).sum(1, keepdim=True)                             # 0 if not chosen
            ylat += g * _mlp(z, f64(c["up"][e]), f64(c["down"][e]))
        out = F.linear(ylat, f64(c["fc2"])) + _mlp(x, f64(c["su"]), f64(c["sd"]))
        assert relerr(res["out"], out.numpy()) < TOL64


def pin_dense_e1k1(O):
    """E=1, K=1: the gate is exactly routed_scaling and the layer is a dense MLP chain."""
    c = case("e1", E=1, K=1, T=16, H=64, L=32, I=48, Is=40)
    F = torch.nn.functional
    x = f64(c["x"])
    up, down = f64(c["up"][0]), f64(c["down"][0])
    for mirror in (False, True):
        res = run(O, c, mirror=mirror)
        assert np.all(res["gate"] == np.float32(5.0))
        R = (lambda a: torch.from_numpy(O.round_bf16(a.numpy()))) if mirror else (lambda a: a)
        z = R(F.linear(x, f64(c["fc1"])))
        y = R(F.linear(R(_relu2(F.linear(z, up))), down))
        ylat = R(5.0 * y)
        hs = R(_relu2(F.linear(x, f64(c["su"]))))
        out = R(F.linear(ylat, f64(c["fc2"])) + F.linear(hs, f64(c["sd"])))
        if mirror:
            # BLAS summation order may move a value across a bf16 rounding boundary
            assert relerr(res["out"], out.numpy()) < 1e-2
            assert np.mean(res["out"] == out.numpy()) > 0.97
        else:
            assert relerr(res["out"], out.numpy()) < TOL64


def pin_identity_expert(O):
    """Identity experts on binary latents: out[:, :L] = routed_scaling * x[:, :L] exactly."""
    T, H, L, E, I, K, Is = 20, 96, 32, 8, 64, 3, 48
    c = case("ident", T=T, H=H, L=L, E=E, I=I, K=K, Is=Is)
    rng = np.random.default_rng(1)
    xb = rng.integers(0, 2, size=(T, H)).astype(np.float64)
    eye = np.eye(L)
    fc1 = np.zeros((L, H)); fc1[:, :L] = eye
    up = np.zeros((E, I, L)); up[:, :L, :] = eye
    down = np.zeros((E, L, I)); down[:, :, :L] = eye
    fc2 = np.zeros((H, L)); fc2[:L, :] = eye
    c2 = dict(c, x=to_bits(xb), fc1=to_bits(fc1), up=to_bits(up), down=to_bits(down),
              fc2=to_bits(fc2), su=to_bits(np.zeros((Is, H))), sd=to_bits(np.zeros((H, Is))))
    res = run(O, c2, mirror=True, keep=True)
    assert np.array_equal(res["y"], res["z"][res["row_token"]]), "each expert returns its input"
    assert np.array_equal(res["out"][:, :L], 5.0 * xb[:, :L])
    assert np.all(res["out"][:, L:] == 0)


def pin_zero_routed_path(O):
    """W_down = 0 (or W_fc2 = 0): only the shared expert remains, computed here with torch."""
    c = case("tiny")
    F = torch.nn.functional
    x = f64(c["x"])
    R = lambda a: torch.from_numpy(O.round_bf16(a.numpy()))
    hs = R(_relu2(F.linear(x, f64(c["su"]))))
    want = R(F.linear(hs, f64(c["sd"]))).numpy()
    for over in (dict(down=np.zeros_like(c["down"])), dict(fc2=np.zeros_like(c["fc2"]))):
        res = run(O, dict(c, **over), mirror=True)
        d = np.abs(res["out"] - want)
        ulp = np.abs(want) * 2.0 ** -7 + 1e-30
        assert np.all(d <= ulp), "a zero routed path must leave exactly the shared output"
        assert np.mean(d == 0) > 0.99


def pin_scale_linearity(O):
    c = case("tiny")
    shared = run(O, dict(c, fc2=np.zeros_like(c["fc2"])), mirror=False)["out"]
    o5 = run(O, c, mirror=False, scale=5.0)["out"]
    o1 = run(O, c, mirror=False, scale=1.0)["out"]
    # the gates are stored in fp32, so the two sides differ by fp32 rounding of the gates
    assert relerr(o5 - shared, 5.0 * (o1 - shared)) < 1e-6


def pin_token_equivariance_and_subset(O):
    c = case("tiny")
    full = run(O, c, mirror=False)
    perm = np.random.default_rng(4).permutation(c["cfg"].T)
    pr = run(O, dict(c, x=c["x"][perm]), mirror=False)
    assert np.array_equal(pr["idx"], full["idx"][perm])
    assert relerr(pr["out"], full["out"][perm]) < TOL64
    sub = run(O, dict(c, x=c["x"][5:20], cfg=W.get_config("tiny", T=15)), mirror=False)
    assert np.array_equal(sub["idx"], full["idx"][5:20])
    assert relerr(sub["out"], full["out"][5:20]) < TOL64


def pin_expert_relabel(O):
    c = case("tiny")
    E = c["cfg"].E
    pi = np.random.default_rng(5).permutation(E)            # new expert k is old expert pi[k]
    c2 = dict(c, wr=c["wr"][pi], b=c["b"][pi], up=c["up"][pi], down=c["down"][pi])
    a = run(O, c, mirror=False)
    b = run(O, c2, mirror=False)
    inv = np.argsort(pi)
    assert np.array_equal(np.sort(pi[b["idx"]], 1), a["idx"])
    assert np.array_equal(np.sort(inv[a["idx"]], 1), b["idx"])
    assert relerr(b["out"], a["out"]) < TOL64


def pin_mirror_grid(O):
    """With mirror=True every stored tensor lies on the bf16 grid (checked with torch)."""
    c = case("tiny")
    res = run(O, c, mirror=True, keep=True)
    for k in ("z", "h", "y", "y_lat", "hs", "out"):
        v = res[k]
        back = torch.from_numpy(v).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(v, back), k
    # fraction of relu2 zeros ~ 1/2 for zero-mean pre-activations (QA Q2.6)
    assert 0.45 < np.mean(res["h"] == 0) < 0.55


def pin_fp32_mode(O):
    """The float32 timing mode runs the same steps at single precision: on tiny
    (no token near a tie) it routes exactly as the pinned float64 mode and its
    output agrees with it to the bf16 rounding of the stored tensors."""
    c = case("tiny")
    cfg = c["cfg"]
    up, down = c["up"], c["down"]
    res = {dt: O.forward(c["x"], c["wr"], c["b"], c["fc1"], c["fc2"], c["su"], c["sd"],
                         lambda e: (up[e], down[e]), cfg.K, cfg.routed_scaling, dtype=dt)
           for dt in (np.float64, np.float32)}
    a, b = res[np.float64], res[np.float32]
    assert np.all(a["gap"] > 1e-4)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.max(np.abs(a["gate"] - b["gate"]) / a["gate"]) < 1e-5
    assert relerr(b["out"], a["out"]) < 1e-2
    assert b["out"].dtype == np.float32


ALL_PINS = [
    pin_group_bruteforce, pin_group_all_admitted_is_plain, pin_group_confinement, pin_group_tie,
    pin_bf16_conversions, pin_route_bruteforce, pin_route_bias_zero, pin_route_forced_and_gates,
    pin_route_invariants, pin_route_ties, pin_permute_bruteforce, pin_dense_masked,
    pin_dense_e1k1, pin_identity_expert, pin_zero_routed_path, pin_scale_linearity,
    pin_token_equivariance_and_subset, pin_expert_relabel, pin_mirror_grid, pin_fp32_mode,
]
