"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these checks re-types the oracle's own formulas: each compares the
oracle (plain C loops) with a different route to the same number -- the gate
values the pages print, numpy/scipy/torch library routines in float64, a
brute-force dense mixture that runs every expert on every token, full stable
sorts, and closed forms.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as TF

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _ref_act(name, z):
    z = torch.from_numpy(z)
    if name == "relu":
        return TF.relu(z).numpy()
    if name == "gelu":
        return TF.gelu(z, approximate="none").numpy()
    raise ValueError(name)


def _ref_expert(act, X, w1, w3, w2, b1=None, b2=None):
    """Expert FFN via float64 numpy matmuls and torch's activation routines."""
    X, w1, w2 = (np.asarray(a, np.float64) for a in (X, w1, w2))
    a = X @ w1.T
    if act == "swiglu":
        u = X @ np.asarray(w3, np.float64).T
        h = TF.silu(torch.from_numpy(a)).numpy() * u
    else:
        if b1 is not None:
            a = a + np.asarray(b1, np.float64)
        h = _ref_act(act, a)
    y = h @ w2.T
    if act != "swiglu" and b2 is not None:
        y = y + np.asarray(b2, np.float64)
    return y


def _np_inputs(spec, inp):
    return {k: (None if v is None else v.float().numpy()) for k, v in inp.items()}


def _ref_shared(x, ws1, ws3, ws2):
    """Shared experts via float64 numpy: one (2-D weights) or the sum of S ([S, ...] weights)."""
    if ws1.ndim == 2:
        return _ref_expert("swiglu", x, ws1, ws3, ws2)
    return sum(_ref_expert("swiglu", x, ws1[s], ws3[s], ws2[s]) for s in range(ws1.shape[0]))


# ---------------------------------------------------------------------------
# logits
# ---------------------------------------------------------------------------

def test_logits_match_float64_matmul():
    r = _rng(1)
    x = r.standard_normal((37, 70)).astype(np.float32)
    wg = r.standard_normal((9, 70)).astype(np.float32)
    b = r.standard_normal(9).astype(np.float32)
    got = oracle.logits(x, wg, b)
    ref = (x.astype(np.float64) @ wg.astype(np.float64).T + b).astype(np.float32)
    ulp = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
    # the bias must enter, and the operands must not be transposed
    assert not np.allclose(oracle.logits(x, wg, None), got)


# ---------------------------------------------------------------------------
# gating
# ---------------------------------------------------------------------------

def _stable_rank(lg):
    """Experts of each row by (logit desc, index asc) via numpy's stable lexsort."""
    T, E = lg.shape
    out = np.empty((T, E), np.int64)
    for t in range(T):
        out[t] = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))
    return out


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("E,k", [(8, 2), (16, 1), (64, 8), (5, 5)])
def test_topk_selection_is_stable_sort_prefix(E, k, ties):
    lg = workloads.random_logits(300, E, seed=11 + E + k, ties=ties).numpy()
    idx, _ = oracle.route_topk(lg, k, "topk_softmax")
    assert np.array_equal(idx, _stable_rank(lg)[:, :k])


def test_negative_zero_ties_positive_zero():
    lg = np.array([[-0.0, 0.0, -1.0, 0.0]], np.float32)
    idx, w = oracle.route_topk(lg, 2, "topk_softmax")
    assert idx.tolist() == [[0, 1]]
    assert np.allclose(w, 0.5)
    lg = np.array([[0.0, -0.0, -0.0, -1.0]], np.float32)
    idx, _ = oracle.route_topk(lg, 3, "topk_softmax")
    assert idx.tolist() == [[0, 1, 2]]


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (7, 3)])
def test_topk_softmax_weights_match_scipy(E, k):
    lg = workloads.random_logits(200, E, seed=5).numpy()
    idx, w = oracle.route_topk(lg, k, "topk_softmax")
    sel = np.take_along_axis(lg.astype(np.float64), idx, axis=1)
    ref = scipy.special.softmax(sel, axis=1)
    assert np.allclose(w, ref, rtol=2e-7, atol=0)
    # each token's gates sum to 1
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    # slot order is descending weight
    assert np.all(np.diff(w, axis=1) <= 0)


def test_softmax_then_topk_renormalised_equals_topk_then_softmax():
    """[yj-ja] TopKGating renormalises softmax probabilities; [yj-zh] takes softmax of
    the top-k logits.  Implemented literally in float64 the two agree."""
    E, k = 16, 4
    lg = workloads.random_logits(400, E, seed=21).numpy()
    idx, w = oracle.route_topk(lg, k, "topk_softmax")
    probs = scipy.special.softmax(lg.astype(np.float64), axis=1)
    order = np.argsort(-probs, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(probs, order, axis=1)
    ren = top / top.sum(1, keepdims=True)
    assert np.array_equal(order, idx)
    assert np.allclose(ren, w, rtol=1e-6, atol=0)


def test_softmax_topk_weights_are_full_softmax_entries():
    """[yj-ja] gating formula: softmax over all experts, zero outside the top-k."""
    E, k = 8, 2
    lg = workloads.random_logits(150, E, seed=8).numpy()
    idx, w = oracle.route_topk(lg, k, "softmax_topk")
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(full, idx, axis=1), rtol=2e-7, atol=0)
    assert np.all(w.astype(np.float64).sum(1) < 1.0)


def test_switch_gate_is_max_softmax_probability():
    """[yj-zh] SwitchRouter: probs = softmax(logits); gate, expert = probs.max(-1)."""
    E = 16
    lg = workloads.random_logits(500, E, seed=3).numpy()
    idx, w = oracle.route_topk(lg, 1, "switch")
    probs = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.array_equal(idx[:, 0], np.argmax(lg, axis=1))
    assert np.allclose(w[:, 0], probs.max(1), rtol=2e-7, atol=0)


def test_all_ties_pick_lowest_experts_with_equal_weights():
    lg = np.zeros((4, 8), np.float32)
    idx, w = oracle.route_topk(lg, 3, "topk_softmax")
    assert idx.tolist() == [[0, 1, 2]] * 4
    assert np.allclose(w, 1.0 / 3.0)
    idx, w = oracle.route_topk(lg, 1, "switch")
    assert idx[:, 0].tolist() == [0] * 4
    assert np.allclose(w, 1.0 / 8.0)


def _golden_gates():
    rows = []
    with open(os.path.join(GOLDEN, "gate_worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, E, k, lg, ids, gates = [c.strip() for c in line.split("|")]
            rows.append((name, int(E), int(k), [float(v) for v in lg.split(",")],
                         [int(v) for v in ids.split(",")], [float(v) for v in gates.split(",")]))
    return rows


@pytest.mark.parametrize("row", _golden_gates(), ids=lambda r: r[0])
def test_worked_gate_examples(row):
    name, E, k, lg, ids, gates = row
    lg = np.array([lg], np.float32)
    assert lg.shape[1] == E
    idx, w = oracle.route_topk(lg, k, "topk_softmax")
    assert idx[0].tolist() == ids
    assert np.allclose(w[0], gates, atol=1e-6)


def test_capacity_truncates():
    assert oracle.capacity(1.25, 1024, 16) == 80     # Switch layer, per sequence row
    assert oracle.capacity(1.0, 8192, 64) == 128     # expert-choice layer
    assert oracle.capacity(1.25, 100, 16) == 7       # int(7.8125)
    assert oracle.capacity(1.0, 10, 4) == 2          # int(2.5)


# ---------------------------------------------------------------------------
# counts, capacity, permutation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (16, 1)])
def test_permutation_structure(E, k):
    T = 777
    idx = workloads.random_topk_idx(T, E, k, seed=E + k, skew=1.1).numpy()
    p = oracle.permute(idx, E)
    assert p["counts"].sum() == T * k
    assert np.array_equal(p["counts"], np.bincount(idx.ravel(), minlength=E))
    assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(p["counts"])]))
    rt, sr = p["row_token"], p["slot_row"]
    for e in range(E):
        seg = rt[p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)  # ascending tokens inside each expert
        assert np.array_equal(seg, np.nonzero((idx == e).any(1))[0])
    tt = np.repeat(np.arange(T), k).reshape(T, k)
    assert np.array_equal(rt[sr], tt)
    expert_of_row = np.repeat(np.arange(E), p["counts"])
    assert np.array_equal(expert_of_row[sr], idx)


def _literal_switch_keep(idx, E, cap, group):
    """[yj-zh] SwitchRouter, literally: per expert, the positions where the expert
    was chosen, in order; all but the first `cap` are cleared.  Applied per group."""
    T = idx.shape[0]
    keep = np.zeros(T, bool)
    G = group if group > 0 else T
    for g0 in range(0, T, G):
        sel = idx[g0:g0 + G, 0]
        for e in range(E):
            pos = np.nonzero(sel == e)[0]
            keep[g0 + pos[:cap]] = True
    return keep


@pytest.mark.parametrize("group", [320, 0])
def test_switch_capacity_drops_in_token_order(group):
    E, T = 16, 640
    lg = workloads.random_logits(T, E, seed=4).numpy() + np.linspace(-2, 2, E, dtype=np.float32)
    idx, _ = oracle.route_topk(lg, 1, "switch")
    cap = oracle.capacity(1.25, group if group else T, E)
    p = oracle.permute(idx, E, cap, group)
    keep = _literal_switch_keep(idx, E, cap, group)
    assert np.array_equal(p["slot_row"][:, 0] >= 0, keep)
    assert keep.sum() < T  # the skew makes some experts overflow
    # kept per (group, expert) = min(count, C)
    G = group if group else T
    want = sum(min(int((idx[g0:g0 + G, 0] == e).sum()), cap) for g0 in range(0, T, G) for e in range(E))
    assert p["kept"] == want


# ---------------------------------------------------------------------------
# expert choice
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ties", [False, True])
def test_expert_choice_selection_and_scores(ties):
    T, E = 300, 12
    cap = oracle.capacity(1.0, T, E)
    lg = workloads.random_logits(T, E, seed=9, ties=ties).numpy()
    ec_idx, ec_score = oracle.route_expert_choice(lg, cap)
    probs = scipy.special.softmax(lg.astype(np.float64), axis=0)  # over tokens
    for e in range(E):
        order = np.lexsort((np.arange(T), -lg[:, e].astype(np.float64)))[:cap]
        assert np.array_equal(ec_idx[e], order)
        assert len(set(ec_idx[e].tolist())) == cap  # every expert fills its capacity exactly
        assert np.allclose(ec_score[e], probs[order, e], rtol=2e-7, atol=1e-30)


# ---------------------------------------------------------------------------
# expert FFNs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu"])
def test_expert_ffn_matches_numpy(act):
    r = _rng(2)
    n, d, F = 9, 24, 40
    X = r.standard_normal((n, d)).astype(np.float32)
    w1 = (r.standard_normal((F, d)) / 5).astype(np.float32)
    w3 = (r.standard_normal((F, d)) / 5).astype(np.float32)
    w2 = (r.standard_normal((d, F)) / 6).astype(np.float32)
    b1 = r.standard_normal(F).astype(np.float32)
    b2 = r.standard_normal(d).astype(np.float32)
    kw = dict(b1=b1, b2=b2) if act != "swiglu" else {}
    got = oracle.expert_ffn(act, X, w1, w3 if act == "swiglu" else None, w2, **kw)
    ref = _ref_expert(act, X, w1, w3, w2, **kw)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def _dense_gates(spec, out):
    """Dense gate matrix G [T, E] from the oracle's routing (0 outside the selection)."""
    T, E = spec.T, spec.E
    G = np.zeros((T, E), np.float64)
    if spec.gating == "expert_choice":
        for e in range(E):
            G[out["ec_idx"][e], e] = out["ec_score"][e]
        return G
    for t in range(T):
        for j in range(spec.k):
            if out["slot_row"][t, j] >= 0:
                G[t, out["topk_idx"][t, j]] = out["topk_w"][t, j]
    return G


def _dense_mixture(spec, inp, G):
    """Brute force: every expert on every token, mixed with G (zero where unselected).
    The pages note this gives the sparse layer's result while wasting the work
    ([lecture] "Token Routing"; [yj-ja] gating formula y = sum_i G(x)_i E_i(x))."""
    x = inp["x"].astype(np.float64)
    y = np.zeros((spec.T, spec.d))
    for e in range(spec.E):
        Ye = _ref_expert(spec.act, x, inp["w1"][e], None if inp["w3"] is None else inp["w3"][e],
                         inp["w2"][e], None if inp["b1"] is None else inp["b1"][e],
                         None if inp["b2"] is None else inp["b2"][e])
        y += G[:, e:e + 1] * Ye
    if spec.F_shared:
        y += _ref_shared(x, inp["ws1"], inp["ws3"], inp["ws2"])
    return y


TINY = [
    workloads.BASIC_TOP2_F32.replace(name="tiny_basic", T=40, d=16, F=24),
    workloads.SWITCH_TOP1_BF16.replace(name="tiny_switch", T=3 * 20, d=16, E=4, F=24,
                                       capacity_group=20),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="tiny_mixtral", T=33, d=32, F=48),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="tiny_deepseek", T=50, d=32, E=16, k=4, F=16,
                                           F_shared=24),
    workloads.EXPERT_CHOICE_BF16.replace(name="tiny_ec", T=64, d=32, E=8, F=24),
    workloads.MIXTRAL_PREFILL_BF16.replace(name="tiny_softmax_topk", T=30, d=16, F=24,
                                           gating="softmax_topk"),
    workloads.DEEPSEEK_SHARED_BF16.replace(name="tiny_deepseek_3_shared", T=40, d=32, E=16, k=4, F=16,
                                           F_shared=24, num_shared=3),
]


@pytest.mark.parametrize("spec", TINY, ids=lambda s: s.name)
def test_sparse_layer_equals_dense_masked_mixture(spec):
    inp = workloads.make_inputs(spec)
    out = oracle.forward(spec, inp)
    npi = _np_inputs(spec, inp)
    ref = _dense_mixture(spec, npi, _dense_gates(spec, out))
    assert np.allclose(out["y64"], ref, rtol=1e-11, atol=1e-11)
    if spec.gating == "switch":
        assert (out["slot_row"] < 0).any()  # the skew drops some tokens in this case


def test_all_experts_selected_equals_full_softmax_mixture():
    """k = E with softmax gating is the dense softmax mixture sum_i softmax(l)_i E_i(x)."""
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="k_eq_E", T=25, d=16, E=6, k=6, F=20)
    inp = workloads.make_inputs(spec)
    out = oracle.forward(spec, inp)
    npi = _np_inputs(spec, inp)
    lg = (npi["x"].astype(np.float64) @ npi["wg"].astype(np.float64).T)
    G = scipy.special.softmax(lg, axis=1)
    ref = _dense_mixture(spec, npi, G)
    assert np.allclose(out["y64"], ref, rtol=1e-6, atol=1e-7)


def _identical_experts(spec, inp):
    inp = dict(inp)
    for key in ("w1", "w3", "w2", "b1", "b2"):
        if inp.get(key) is not None:
            inp[key] = inp[key][:1].expand_as(inp[key]).contiguous()
    return inp


@pytest.mark.parametrize("spec", TINY[:5], ids=lambda s: s.name)
def test_identical_experts_closed_form(spec):
    """With every expert equal to one FFN E: renormalised top-k gives y = E(x);
    Switch gives g*E(x) for kept tokens and 0 for dropped ones; expert choice gives
    (sum_e D[e,t]) * E(x)."""
    inp = _identical_experts(spec, workloads.make_inputs(spec))
    out = oracle.forward(spec, inp)
    npi = _np_inputs(spec, inp)
    one = _ref_expert(spec.act, npi["x"], npi["w1"][0], None if npi["w3"] is None else npi["w3"][0],
                      npi["w2"][0], None if npi["b1"] is None else npi["b1"][0],
                      None if npi["b2"] is None else npi["b2"][0])
    shared = 0.0
    if spec.F_shared:
        shared = _ref_shared(npi["x"], npi["ws1"], npi["ws3"], npi["ws2"])
    if spec.gating == "topk_softmax":
        scale = np.ones((spec.T, 1))
    elif spec.gating == "switch":
        scale = np.where(out["slot_row"][:, :1] >= 0, out["topk_w"][:, :1].astype(np.float64), 0.0)
    else:
        D = np.zeros((spec.E, spec.T))
        for e in range(spec.E):
            D[e, out["ec_idx"][e]] = out["ec_score"][e]
        scale = D.sum(0)[:, None]
        assert (scale[:, 0] == 0).any()  # some tokens are chosen by no expert -> 0
    assert np.allclose(out["y64"], scale * one + shared, rtol=1e-6, atol=1e-7)


def test_single_expert_is_plain_ffn():
    """E = 1, k = 1: the layer reduces to one two-layer FFN with gate 1."""
    spec = workloads.BASIC_TOP2_F32.replace(name="single", T=31, d=12, E=1, k=1, F=20)
    inp = workloads.make_inputs(spec)
    out = oracle.forward(spec, inp)
    npi = _np_inputs(spec, inp)
    ref = _ref_expert("relu", npi["x"], npi["w1"][0], None, npi["w2"][0], npi["b1"][0], npi["b2"][0])
    assert np.allclose(out["y64"], ref, rtol=1e-12, atol=1e-12)


def test_several_shared_experts_equal_one_wide_expert():
    """S shared SwiGLU experts of width Fs summed ([yj-zh] DeepSeekMoELayer)
    equal one SwiGLU expert of width S*Fs whose gate and up rows are the S
    experts' rows stacked and whose down projection is theirs concatenated
    along the hidden axis: the hidden units split into S groups and the
    down projection sums over all of them."""
    spec = workloads.DEEPSEEK_SHARED_BF16.replace(name="shared_stack", T=23, d=32, E=4, F=16, F_shared=24,
                                                  num_shared=3)
    npi = _np_inputs(spec, workloads.make_inputs(spec))
    ws1, ws3, ws2 = npi["ws1"], npi["ws3"], npi["ws2"]
    S, Fs, d = ws1.shape
    got = oracle.shared_ffn(npi["x"], ws1, ws3, ws2)
    wide = oracle.expert_ffn("swiglu", npi["x"], ws1.reshape(S * Fs, d), ws3.reshape(S * Fs, d),
                             np.concatenate(list(ws2), axis=1))
    assert np.allclose(got, wide, rtol=1e-12, atol=1e-13)
    assert not np.allclose(got, oracle.expert_ffn("swiglu", npi["x"], ws1[0], ws3[0], ws2[0]), rtol=1e-3)


def test_identical_shared_experts_add_up():
    """S identical shared experts give S times one expert's output."""
    spec = workloads.DEEPSEEK_SHARED_BF16.replace(name="shared_same", T=19, d=32, E=4, F=16, F_shared=24,
                                                  num_shared=4)
    npi = _np_inputs(spec, workloads.make_inputs(spec))
    same = {k: np.broadcast_to(npi[k][:1], npi[k].shape).copy() for k in ("ws1", "ws3", "ws2")}
    got = oracle.shared_ffn(npi["x"], same["ws1"], same["ws3"], same["ws2"])
    one = _ref_expert("swiglu", npi["x"], npi["ws1"][0], npi["ws3"][0], npi["ws2"][0])
    assert np.allclose(got, 4.0 * one, rtol=1e-12, atol=1e-13)


def test_shared_expert_only_when_routed_experts_vanish():
    spec = TINY[3]
    inp = workloads.make_inputs(spec)
    inp["w2"] = torch.zeros_like(inp["w2"])
    out = oracle.forward(spec, inp)
    npi = _np_inputs(spec, inp)
    ref = _ref_expert("swiglu", npi["x"], npi["ws1"], npi["ws3"], npi["ws2"])
    assert np.allclose(out["y64"], ref, rtol=1e-12, atol=1e-12)
    spec3 = [s for s in TINY if s.num_shared == 3][0]
    inp = workloads.make_inputs(spec3)
    inp["w2"] = torch.zeros_like(inp["w2"])
    out = oracle.forward(spec3, inp)
    npi = _np_inputs(spec3, inp)
    ref = sum(_ref_expert("swiglu", npi["x"], npi["ws1"][s], npi["ws3"][s], npi["ws2"][s]) for s in range(3))
    assert np.allclose(out["y64"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("spec", TINY[:5], ids=lambda s: s.name)
def test_forward_tokens_matches_forward(spec):
    """The sampled-token path used at full sizes equals the all-token path."""
    inp = workloads.make_inputs(spec)
    full = oracle.forward(spec, inp)
    toks = np.array([0, 3, spec.T // 2, spec.T - 1])
    part = oracle.forward_tokens(spec, inp, toks)
    assert np.allclose(part["y64"], full["y64"][toks], rtol=1e-12, atol=1e-12)


def test_integer_inputs_make_router_exact():
    """The integer recipe gives logits that float32 holds exactly (so any summation
    order yields the same bits)."""
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="int", T=64, d=256, inputs="integer")
    inp = workloads.make_inputs(spec, experts=False)
    lg = oracle.logits(inp["x"], inp["wg"])
    ref = inp["x"].double().numpy() @ inp["wg"].double().numpy().T
    assert np.array_equal(lg.astype(np.float64), ref)
    assert np.all(ref * 8 == np.round(ref * 8))


# ---------------------------------------------------------------------------
# router side outputs, top-k capacity, noisy router
# ---------------------------------------------------------------------------

def test_router_losses_closed_forms():
    """Uniform probabilities and a balanced selection give aux = 1 and, with zero
    logits, z = (ln E)^2 ([yj-ja] compute_load_balancing_loss: minimal when balanced)."""
    T, E, k = 64, 8, 2
    lg = np.zeros((T, E), np.float32)
    idx = (np.arange(T * k).reshape(T, k) % E).astype(np.int32)
    aux, z, P = oracle.router_losses(lg, idx)
    assert abs(aux - 1.0) < 1e-12
    assert abs(z - math.log(E) ** 2) < 1e-12
    assert np.allclose(P, 1.0 / E)
    # everything on expert 3 with probability ~1: aux -> E
    lg2 = np.zeros((T, E), np.float32)
    lg2[:, 3] = 60.0
    idx2 = np.full((T, 1), 3, np.int32)
    aux2, _, _ = oracle.router_losses(lg2, idx2)
    assert abs(aux2 - E) < 1e-9


def test_router_losses_match_scipy():
    T, E, k = 300, 16, 4
    lg = workloads.random_logits(T, E, seed=31).numpy()
    idx, _ = oracle.route_topk(lg, k, "topk_softmax")
    aux, z, P = oracle.router_losses(lg, idx)
    lg64 = lg.astype(np.float64)
    Pref = scipy.special.softmax(lg64, axis=1).mean(0)
    f = np.bincount(idx.ravel(), minlength=E) / (T * k)
    assert np.allclose(P, Pref, rtol=1e-12)
    assert abs(aux - E * float((f * Pref).sum())) < 1e-12
    assert abs(z - float((scipy.special.logsumexp(lg64, axis=1) ** 2).mean())) < 1e-9


def test_topk_capacity_formula():
    # [devtips] capacity example: (batch * seq * top_k / experts) * capacity_factor
    assert oracle.capacity_topk(1.25, 8 * 512, 2, 8) == 1280
    assert oracle.capacity_topk(1.25, 1024, 1, 16) == 80  # k = 1 is the Switch capacity
    assert oracle.capacity_topk(1.25, 10, 2, 64, 4) == 4  # min_capacity floor ([yj-zh] DeepSpeed example)


def _literal_topk_keep(idx, E, cap, group):
    """Flatten-order keep rule: visit (token, slot) in order; keep while the expert
    has fewer than cap kept assignments in the current group."""
    T, k = idx.shape
    G = group if group > 0 else T
    keep = np.zeros((T, k), bool)
    for g0 in range(0, T, G):
        used = np.zeros(E, int)
        for t in range(g0, min(T, g0 + G)):
            for j in range(k):
                e = idx[t, j]
                if used[e] < cap:
                    keep[t, j] = True
                    used[e] += 1
    return keep


@pytest.mark.parametrize("group", [0, 128])
def test_topk_capacity_drops(group):
    T, E, k = 512, 16, 2
    idx = workloads.random_topk_idx(T, E, k, seed=77, skew=1.2).numpy()
    cap = oracle.capacity_topk(1.0, group if group else T, k, E)
    p = oracle.permute(idx, E, cap, group)
    keep = _literal_topk_keep(idx, E, cap, group)
    assert np.array_equal(p["slot_row"] >= 0, keep)
    assert (~keep).any() and p["counts"].max() <= cap * (T // (group or T))


def test_noisy_logits_reduce_to_closed_forms():
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="noisy", T=50, d=64, E=8, noisy=True, router_bias="normal")
    inp = workloads.make_inputs(spec, experts=False)
    base = oracle.logits(inp["x"], inp["wg"], inp["bg"])
    zero = torch.zeros_like(inp["noise"])
    assert np.array_equal(oracle.logits_noisy(inp["x"], inp["wg"], inp["bg"], inp["wn"], zero), base)
    # Wn = 0: softplus(0) = ln 2
    got = oracle.logits_noisy(inp["x"], inp["wg"], inp["bg"], torch.zeros_like(inp["wn"]), inp["noise"])
    ref = base.astype(np.float64) + math.log(2.0) * inp["noise"].double().numpy()
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-6)


def test_noisy_logits_match_torch_softplus():
    spec = workloads.MIXTRAL_PREFILL_BF16.replace(name="noisy2", T=40, d=32, E=6, noisy=True)
    inp = workloads.make_inputs(spec, experts=False)
    x, wg, wn, n = (inp[k].double() for k in ("x", "wg", "wn", "noise"))
    ref = (x @ wg.T + TF.softplus(x @ wn.T) * n).numpy()
    got = oracle.logits_noisy(inp["x"], inp["wg"], None, inp["wn"], inp["noise"])
    assert np.allclose(got, ref, rtol=2e-7, atol=1e-6)
