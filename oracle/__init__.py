"""CPU oracle for the sparse MoE layer forward pass.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers.  The product path (the
HIP library and its binding) never imports this package, and this package
imports nothing from the product path.

The arithmetic lives in ``moe_oracle.c`` (plain loops, double precision),
loaded through ctypes.  This module only marshals numpy arrays and chains the
steps in the order the pages give them:

    logits -> gating -> counts / capacity / permutation -> experts -> combine

Every function takes float32 arrays (bf16 workloads pass their bf16-rounded
values, which float32 holds exactly) and returns float32 for final results
and float64 for expert outputs, which stay unrounded until the combine.

Page keys used in citations:
  [devtips]  devtips.kr, "MoE (Mixture of Experts) 아키텍처 완전 정복"
  [garden]   ricepunchb.github.io obsidian garden, "Mixture of Experts (MoE)"
  [yj-zh]    youngju.dev, "Mixture of Experts（MoE）架构深度解析：从 Switch Transformer 到 Mixtral"
  [yj-ja]    youngju.dev, "Sparse Mixture of Experts（MoE）アーキテクチャ深層分析"
  [lecture]  study-site lecture-03, "Mixture of Experts"

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against values and properties the pages and the mathematics fix (worked
gate examples, a brute-force dense mixture, closed forms, library routines).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GATING = {"topk_softmax": 0, "softmax_topk": 1, "switch": 2}
ACT = {"relu": 0, "gelu": 1, "swiglu": 2}

_lib = None


def build_sanitized(out: str) -> str:
    """Compile moe_oracle.c with gcc's AddressSanitizer and UndefinedBehaviorSanitizer
    into `out` (load it through ORACLE_LIB with gcc's libasan and libubsan preloaded)."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           _SRC, "-o", out, "-lm"]
    subprocess.check_call(cmd)
    return out


def build(force: bool = False) -> str:
    """Compile moe_oracle.c into liboracle.so with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Werror",
               _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # ORACLE_LIB points at another build of moe_oracle.c (the mutation tests use it
    # to load copies with a planted mistake and check that the pins catch it).
    path = os.environ.get("ORACLE_LIB") or build()
    lib = ctypes.CDLL(path)
    i32, i64, f64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.oracle_logits.argtypes = [i64, i32, i32, p, p, p, p]
    lib.oracle_logits.restype = None
    lib.oracle_route_topk.argtypes = [i64, i32, i32, i32, p, p, p]
    lib.oracle_route_topk.restype = ctypes.c_int
    lib.oracle_capacity.argtypes = [f64, i64, i32]
    lib.oracle_capacity.restype = i32
    lib.oracle_permute.argtypes = [i64, i32, i32, p, i32, i64, p, p, p, p]
    lib.oracle_permute.restype = i64
    lib.oracle_route_expert_choice.argtypes = [i64, i32, i32, p, p, p]
    lib.oracle_route_expert_choice.restype = ctypes.c_int
    lib.oracle_expert_ffn.argtypes = [i32, i32, i32, i64, p, p, p, p, p, p, p]
    lib.oracle_expert_ffn.restype = ctypes.c_int
    lib.oracle_combine_topk.argtypes = [i64, i32, i32, p, p, p, p, p]
    lib.oracle_combine_topk.restype = None
    lib.oracle_combine_expert_choice.argtypes = [i64, i32, i32, i32, p, p, p, p, p]
    lib.oracle_combine_expert_choice.restype = None
    lib.oracle_capacity_topk.argtypes = [f64, i64, i32, i32, i32]
    lib.oracle_capacity_topk.restype = i32
    lib.oracle_router_losses.argtypes = [i64, i32, i32, p, p, p, p, p]
    lib.oracle_router_losses.restype = ctypes.c_int
    lib.oracle_logits_noisy.argtypes = [i64, i32, i32, p, p, p, p, p, p]
    lib.oracle_logits_noisy.restype = None
    _lib = lib
    return lib


def _f32(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: exact widening of bf16 to float32
        a = a.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data


# ----------------------------------------------------------------------------
# individual steps
# ----------------------------------------------------------------------------

def logits(x, wg, bias=None) -> np.ndarray:
    """Router logits l = x Wg^T + b, double sums rounded once to float32.
    [devtips] MoELayer gate; [yj-zh] GatingNetwork; [yj-ja] gating formula."""
    x, wg, bias = _f32(x), _f32(wg), _f32(bias)
    T, d = x.shape
    E = wg.shape[0]
    assert wg.shape == (E, d)
    out = np.empty((T, E), np.float32)
    _load().oracle_logits(T, d, E, _ptr(x), _ptr(wg), _ptr(bias), _ptr(out))
    return out


def route_topk(lg, k: int, gating: str = "topk_softmax"):
    """Token-choice gating on given float32 logits -> (idx int32 [T,k], w float32 [T,k]).
    Slot j holds the expert of rank j (larger logit first, lower index first on ties).
    [devtips] MoELayer; [yj-zh] GatingNetwork, SwitchRouter, MixtralMoELayer;
    [yj-ja] TopKGating and gating formula."""
    lg = _f32(lg)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = _load().oracle_route_topk(T, E, k, GATING[gating], _ptr(lg), _ptr(idx), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_route_topk: bad arguments")
    return idx, w


def capacity(capacity_factor: float, tokens: int, num_experts: int) -> int:
    """int(cf * tokens / E), truncated toward zero ([yj-zh] SwitchRouter)."""
    return int(_load().oracle_capacity(float(capacity_factor), int(tokens), int(num_experts)))


def capacity_topk(capacity_factor: float, tokens: int, k: int, num_experts: int, min_capacity: int = 0) -> int:
    """max(min_capacity, int(cf * tokens * k / E)) ([devtips] capacity example; k = 1 is Switch)."""
    return int(_load().oracle_capacity_topk(float(capacity_factor), int(tokens), int(k), int(num_experts),
                                            int(min_capacity)))


def router_losses(lg, idx):
    """(aux, z_loss, mean_probs): E * sum f_e P_e and mean logsumexp^2 ([yj-ja]
    compute_load_balancing_loss, router_z_loss)."""
    lg, idx = _f32(lg), _i32(idx)
    T, E = lg.shape
    k = idx.shape[1]
    aux, z = ctypes.c_double(), ctypes.c_double()
    P = np.empty(E, np.float64)
    rc = _load().oracle_router_losses(T, E, k, _ptr(lg), _ptr(idx), ctypes.addressof(aux), ctypes.addressof(z),
                                      _ptr(P))
    if rc != 0:
        raise ValueError("oracle_router_losses: bad arguments")
    return aux.value, z.value, P


def logits_noisy(x, wg, bias, wn, noise) -> np.ndarray:
    """Noisy router logits x Wg^T + b + softplus(x Wn^T) * noise ([yj-ja] TopKGating)."""
    x, wg, bias, wn, noise = _f32(x), _f32(wg), _f32(bias), _f32(wn), _f32(noise)
    T, d = x.shape
    E = wg.shape[0]
    out = np.empty((T, E), np.float32)
    _load().oracle_logits_noisy(T, d, E, _ptr(x), _ptr(wg), _ptr(bias), _ptr(wn), _ptr(noise), _ptr(out))
    return out


def permute(idx, num_experts: int, cap: int = 0, group: int = 0):
    """Counts, capacity drops and the expert-contiguous row order.
    Returns dict(counts, offsets, row_token, slot_row, kept)."""
    idx = _i32(idx)
    T, k = idx.shape
    counts = np.empty(num_experts, np.int32)
    offsets = np.empty(num_experts + 1, np.int32)
    row_token = np.empty(max(T * k, 1), np.int32)
    slot_row = np.empty((T, k), np.int32)
    kept = _load().oracle_permute(T, num_experts, k, _ptr(idx), int(cap), int(group), _ptr(counts),
                                  _ptr(offsets), _ptr(row_token), _ptr(slot_row))
    if kept < 0:
        raise ValueError("oracle_permute: bad arguments")
    return dict(counts=counts, offsets=offsets, row_token=row_token[:kept].copy(),
                slot_row=slot_row, kept=int(kept))


def route_expert_choice(lg, cap: int):
    """Expert choice on given float32 logits -> (ec_idx int32 [E,C], ec_score float32 [E,C]).
    [yj-zh] ExpertChoiceRouter; [yj-ja] ExpertChoiceGating."""
    lg = _f32(lg)
    T, E = lg.shape
    ec_idx = np.empty((E, cap), np.int32)
    ec_score = np.empty((E, cap), np.float32)
    rc = _load().oracle_route_expert_choice(T, E, cap, _ptr(lg), _ptr(ec_idx), _ptr(ec_score))
    if rc != 0:
        raise ValueError("oracle_route_expert_choice: bad arguments")
    return ec_idx, ec_score


def expert_ffn(act: str, X, w1, w3, w2, b1=None, b2=None) -> np.ndarray:
    """One expert on rows X [n, d] -> float64 [n, d].
    [devtips] ReLU FFN with biases; [yj-zh] GELU FFN and SwiGLUExpert; [yj-ja] SwiGLUExpert."""
    X, w1, w3, w2, b1, b2 = (_f32(a) for a in (X, w1, w3, w2, b1, b2))
    n, d = X.shape
    F = w1.shape[0]
    assert w1.shape == (F, d) and w2.shape == (d, F)
    Y = np.empty((n, d), np.float64)
    if n == 0:
        return Y
    rc = _load().oracle_expert_ffn(ACT[act], d, F, n, _ptr(X), _ptr(w1), _ptr(w3), _ptr(w2),
                                   _ptr(b1), _ptr(b2), _ptr(Y))
    if rc != 0:
        raise ValueError("oracle_expert_ffn: bad arguments")
    return Y


def combine_topk(w, slot_row, Y, Ys=None) -> np.ndarray:
    """y[t] = sum_j w[t,j] Y[slot_row[t,j]] (+ Ys[t]); float64 [T, d]."""
    w = _f32(w)
    slot_row = _i32(slot_row)
    Y = np.ascontiguousarray(Y, np.float64)
    Ys = None if Ys is None else np.ascontiguousarray(Ys, np.float64)
    T, k = w.shape
    d = Y.shape[1] if Y.ndim == 2 and Y.shape[0] > 0 else (Ys.shape[1] if Ys is not None else 0)
    if Y.shape[0] == 0:
        Y = np.zeros((1, d), np.float64)
    y = np.empty((T, d), np.float64)
    _load().oracle_combine_topk(T, k, d, _ptr(w), _ptr(slot_row), _ptr(Y), _ptr(Ys), _ptr(y))
    return y


def combine_expert_choice(ec_idx, ec_score, Y, T: int, Ys=None) -> np.ndarray:
    """y[t] = sum_e D[e,t] Y[row(e,t)] (+ Ys[t]); float64 [T, d]."""
    ec_idx, ec_score = _i32(ec_idx), _f32(ec_score)
    E, C = ec_idx.shape
    Y = np.ascontiguousarray(Y, np.float64)
    Ys = None if Ys is None else np.ascontiguousarray(Ys, np.float64)
    d = Y.shape[1]
    y = np.empty((T, d), np.float64)
    _load().oracle_combine_expert_choice(T, E, C, d, _ptr(ec_idx), _ptr(ec_score), _ptr(Y),
                                         _ptr(Ys), _ptr(y))
    return y


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def _spec_capacity(spec) -> int:
    min_cap = getattr(spec, "min_capacity", 0)
    if spec.gating == "switch" or (spec.gating in ("topk_softmax", "softmax_topk") and spec.capacity_factor > 0):
        group = spec.capacity_group if spec.capacity_group > 0 else spec.T
        return capacity_topk(spec.capacity_factor, group, spec.k, spec.E, min_cap)
    if spec.gating == "expert_choice":
        return capacity(spec.capacity_factor, spec.T, spec.E)
    return 0


def _router_logits(spec, inp, x):
    if getattr(spec, "noisy", False):
        return logits_noisy(x, inp["wg"], inp.get("bg"), inp["wn"], inp["noise"])
    return logits(x, inp["wg"], inp.get("bg"))


def _experts_rows(spec, inp, X, expert_of_row):
    """Run each row of X through its expert; rows of one expert are batched."""
    n = X.shape[0]
    Y = np.zeros((n, spec.d), np.float64)
    for e in np.unique(expert_of_row):
        rows = np.nonzero(expert_of_row == e)[0]
        Y[rows] = expert_ffn(spec.act, X[rows], inp["w1"][e],
                             None if inp.get("w3") is None else inp["w3"][e], inp["w2"][e],
                             None if inp.get("b1") is None else inp["b1"][e],
                             None if inp.get("b2") is None else inp["b2"][e])
    return Y


def shared_ffn(X, ws1, ws3, ws2) -> np.ndarray:
    """Always-on shared SwiGLU experts on rows X -> float64 [n, d]: one expert
    (ws1, ws3 [Fs, d], ws2 [d, Fs]) or the sum of S of them (ws1, ws3
    [S, Fs, d], ws2 [S, d, Fs]), added in expert order ([yj-zh]
    DeepSeekMoELayer sums its shared experts; [devtips] DeepSeekMoE)."""
    ws1, ws3, ws2 = _f32(ws1), _f32(ws3), _f32(ws2)
    if ws1.ndim == 2:
        return expert_ffn("swiglu", X, ws1, ws3, ws2)
    out = expert_ffn("swiglu", X, ws1[0], ws3[0], ws2[0])
    for s in range(1, ws1.shape[0]):
        out = out + expert_ffn("swiglu", X, ws1[s], ws3[s], ws2[s])
    return out


def _shared(spec, inp, X):
    if not spec.F_shared:
        return None
    return shared_ffn(X, inp["ws1"], inp["ws3"], inp["ws2"])


def forward(spec, inp, lg=None) -> dict:
    """The whole layer on every token; returns every intermediate.

    ``spec`` has the attributes T, d, E, k, F, gating, act, capacity_factor,
    capacity_group, F_shared.  ``inp`` maps x, wg, bg, w1, w3, w2, b1, b2,
    ws1, ws3, ws2 to arrays (missing or None where a layer has none).
    ``lg`` replaces the router product with given float32 logits (used to
    pin gating on logits that both sides receive as an input).
    """
    x = _f32(inp["x"])
    if lg is None:
        lg = _router_logits(spec, inp, x)
    lg = _f32(lg)
    out = dict(logits=lg)
    cap = _spec_capacity(spec)
    if spec.gating == "expert_choice":
        ec_idx, ec_score = route_expert_choice(lg, cap)
        E, C = ec_idx.shape
        rows_tok = ec_idx.reshape(-1)
        X = x[rows_tok]
        expert_of_row = np.repeat(np.arange(E, dtype=np.int32), C)
        inpf = {kk: (_f32(v) if v is not None else None) for kk, v in inp.items()}
        Y = _experts_rows(spec, inpf, X, expert_of_row)
        Ys = _shared(spec, inpf, x)
        y = combine_expert_choice(ec_idx, ec_score, Y, spec.T, Ys)
        out.update(ec_idx=ec_idx, ec_score=ec_score, capacity=cap,
                   counts=np.full(E, C, np.int32), offsets=np.arange(E + 1, dtype=np.int32) * C,
                   row_token=rows_tok.copy(), y_rows=Y, y_shared=Ys, y=y.astype(np.float32), y64=y)
        return out
    idx, w = route_topk(lg, spec.k, spec.gating)
    group = spec.capacity_group if cap > 0 else 0
    perm = permute(idx, spec.E, cap, group)
    inpf = {kk: (_f32(v) if v is not None else None) for kk, v in inp.items()}
    rt = perm["row_token"]
    X = x[rt]
    expert_of_row = np.repeat(np.arange(spec.E, dtype=np.int32), perm["counts"])
    Y = _experts_rows(spec, inpf, X, expert_of_row)
    Ys = _shared(spec, inpf, x)
    y = combine_topk(w, perm["slot_row"], Y, Ys)
    out.update(topk_idx=idx, topk_w=w, capacity=cap, y_rows=Y, y_shared=Ys,
               y=y.astype(np.float32), y64=y, **perm)
    return out


def forward_tokens(spec, inp, tokens, lg=None) -> dict:
    """The layer's output for the listed tokens only.

    Used at full sizes, where running every token through the oracle would take
    too long.  Routing is computed for every token whenever a token's result
    depends on others (Switch capacity, expert choice); the expert FFNs run only
    on the listed tokens' rows, one expert at a time.  Returns dict(y [n, d]
    float32, y64, and the listed tokens' routing).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    x = inp["x"]
    xs = _f32(x[_index_like(x, tokens)])
    need_all = spec.gating in ("switch", "expert_choice") or spec.capacity_factor > 0
    if lg is None and (need_all or getattr(spec, "noisy", False)):
        lg = _router_logits(spec, inp, _f32(x))
    if lg is not None:
        lg = _f32(lg)
        lg_sel = lg[tokens]
    else:
        lg_sel = logits(xs, inp["wg"], inp.get("bg"))
    cap = _spec_capacity(spec)
    n = len(tokens)
    res = dict(tokens=tokens, logits_sel=lg_sel)
    # (sampled row i, gate weight, expert e) triples
    terms = []
    if spec.gating == "expert_choice":
        ec_idx, ec_score = route_expert_choice(lg, cap)
        res.update(ec_idx=ec_idx, ec_score=ec_score)
        pos = {int(t): i for i, t in enumerate(tokens)}
        for e in range(spec.E):
            for j in range(cap):
                i = pos.get(int(ec_idx[e, j]))
                if i is not None:
                    terms.append((i, float(ec_score[e, j]), e))
    else:
        if cap > 0:
            idx_all, w_all = route_topk(lg, spec.k, spec.gating)
            perm = permute(idx_all, spec.E, cap, spec.capacity_group)
            idx, w, kept = idx_all[tokens], w_all[tokens], perm["slot_row"][tokens] >= 0
        else:
            idx, w = route_topk(lg_sel, spec.k, spec.gating)
            kept = np.ones_like(idx, dtype=bool)  # no capacity: every slot is kept
        res.update(topk_idx=idx, topk_w=w, kept=kept)
        for i in range(n):
            for j in range(spec.k):
                if kept[i, j]:
                    terms.append((i, float(w[i, j]), int(idx[i, j])))
    y = np.zeros((n, spec.d), np.float64)
    for e in sorted({t[2] for t in terms}):
        mine = [(i, g) for (i, g, ee) in terms if ee == e]
        rows = np.array([i for i, _ in mine], dtype=np.int64)
        Ye = expert_ffn(spec.act, xs[rows], _f32(inp["w1"][e]),
                        None if inp.get("w3") is None else _f32(inp["w3"][e]), _f32(inp["w2"][e]),
                        None if inp.get("b1") is None else _f32(inp["b1"][e]),
                        None if inp.get("b2") is None else _f32(inp["b2"][e]))
        for r, (i, g) in enumerate(mine):
            y[i] += g * Ye[r]
    if spec.F_shared:
        y += shared_ffn(xs, inp["ws1"], inp["ws3"], inp["ws2"])
    res["y"] = y.astype(np.float32)
    res["y64"] = y
    return res


def _index_like(x, tokens):
    if hasattr(x, "index_select"):
        import torch  # only reached when the caller passes torch tensors
        return torch.as_tensor(tokens, dtype=torch.long, device=x.device)
    return tokens
