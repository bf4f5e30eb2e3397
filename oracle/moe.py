"""Oracle for the sparse MoE FFN layer: route -> permute -> grouped FFN -> combine.

TEST INFRASTRUCTURE ONLY.  A plain, slow CPU implementation used to check the
GPU library.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; it shares no code with the GPU library and
the GPU library never calls it.

Sources (page titles with the section or table each step follows):
  [P1] "How DeepSeek inference works": sparse mixture-of-experts, a learned
       router activating a small subset of experts per token; worked example
       of 256 experts with 8 active per token.
  [P2] "DeepSeek V3/R1 Inference Efficiency (2)": section 2.3.1 (routed expert
       GEMM "up & gate" [7168, 4096] = [H, 2I] and "down" [2048, 7168];
       shared expert GEMMs; the "Gate: router gate", "Expert: prepare routed
       GEMM", "Expert: SwiGLU" and "Expert: combine reduce" operators).

Floating point: fp64 everywhere except where the method fixes a precision:
  * router logits are fp32 fused-multiply-add chains (router_chain.c), because
    the top-k decision must be taken in the same precision as the GPU's;
  * fp8 quantisation (activations and h) is fp32 arithmetic with fp32 scales;
    MX quantisation (MXFP8 activations and h of MXFP4 layers, mx.py) is exact
    from the fp32 value (power-of-two scales);
  * h is rounded to bf16 for bf16 layers, and outputs to their storage type.
Every reading of a point the pages leave open is listed in the design notes.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import codecs, mx
from .build import LIB as _ROUTER_LIB, build as _build_router

_lib = None


def _router_lib():
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_ORACLE_ROUTER_LIB")   # another build of router_chain.c (sanitizer runs)
        if not path:
            path = _ROUTER_LIB
            if not os.path.exists(path):
                _build_router(force=True)
        _lib = ctypes.CDLL(path)
        _lib.oracle_router_logits.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_void_p]
        _lib.oracle_router_logits.restype = None
    return _lib


# ---------------------------------------------------------------- routing [P1], [P2] "Gate"

def router_logits(x32: np.ndarray, wr: np.ndarray, bias) -> np.ndarray:
    """l[t][e] = (fp32 FMA chain over h ascending of x[t][h] * Wr[h][e]) + b[e]."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    T, H = x32.shape
    H2, E = wr.shape
    assert H == H2
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, E), dtype=np.float32)
    _router_lib().oracle_router_logits(x32.ctypes.data, T, H, wr.ctypes.data,
                                       None if b is None else b.ctypes.data, E, out.ctypes.data)
    return out


def select_topk(l: np.ndarray, k: int) -> np.ndarray:
    """For each token, the k experts with the largest logit, in descending
    logit order; equal logits are ordered by ascending expert index (a stable
    sort on the negated logit)."""
    order = np.argsort(-l, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def route_weights(l_sel: np.ndarray, score: str) -> np.ndarray:
    """Weights of the selected experts, renormalised to sum to one over the k
    chosen (computed in fp64, stored as fp32).

    softmax: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)  (the full softmax
             over all experts restricted to the chosen k and renormalised;
             l_0 is the largest logit);
    sigmoid: s_j = 1 / (1 + exp(-l_j)),  w_j = s_j / sum_i s_i.
    """
    l = l_sel.astype(np.float64)
    if score == "softmax":
        z = np.exp(l - l[:, :1])
        w = z / z.sum(axis=1, keepdims=True)
    elif score == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-l))
        w = s / s.sum(axis=1, keepdims=True)
    else:
        raise ValueError(score)
    return w.astype(np.float32)


def route(x32, wr, bias, k: int, score: str):
    l = router_logits(x32, wr, bias)
    ids = select_topk(l, k)
    w = route_weights(np.take_along_axis(l, ids, axis=1), score)
    return ids, w, l


# ------------------------------------------------------- permute [P2] "prepare routed GEMM"

def permute(ids: np.ndarray, E: int):
    """Group the T*k assignments by expert.

    counts[e]  = number of assignments (t, j) with ids[t][j] = e
    offsets    = exclusive prefix sum of counts (length E + 1)
    src[p]     = flat index f = t*k + j of the assignment at permuted position
                 p; within one expert the flat indices ascend (stable)
    dest[f]    = the permuted position of assignment f (dest[src[p]] = p)
    """
    flat = ids.reshape(-1).astype(np.int64)
    R = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:-1].copy()
    src = np.empty(R, dtype=np.int64)
    dest = np.empty(R, dtype=np.int64)
    for f in range(R):
        e = flat[f]
        src[fill[e]] = f
        dest[f] = fill[e]
        fill[e] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            src.astype(np.int32), dest.astype(np.int32))


# ------------------------------------------------------------- expert FFN [P2] 2.3.1

_E4M3_TABLE = codecs.e4m3_decode(np.arange(256))


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def bank_expert_f64(bank, e: int):
    """Expert e of a bank (synth.Bank, torch tensors) as fp64 numpy matrices
    Wg [I][H], Wu [I][H], Wd [H][I] (storage is output-major)."""
    if bank.dt in ("f32", "bf16"):
        f = lambda t: t[e].float().cpu().numpy().astype(np.float64)
        return f(bank.w_gate), f(bank.w_up), f(bank.w_down)
    if bank.dt == "mxfp4":
        f = lambda w, s: mx.mxfp4_matrix(w[e].cpu().numpy(), s[e].cpu().numpy())
        return f(bank.w_gate, bank.s_gate), f(bank.w_up, bank.s_up), f(bank.w_down, bank.s_down)
    assert bank.dt == "e4m3"

    def dq(q, s):
        qn = q[e].cpu().numpy()
        sn = s[e].cpu().numpy().astype(np.float64)
        R, C = qn.shape
        return (_E4M3_TABLE[qn].reshape(R // 128, 128, C // 128, 128)
                * sn[:, None, :, None]).reshape(R, C)
    return dq(bank.w_gate, bank.s_gate), dq(bank.w_up, bank.s_up), dq(bank.w_down, bank.s_down)


def expert_ffn(a: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, h_mode: str,
               return_h: bool = False):
    """y = (silu(a Wg) * (a Wu)) Wd for the rows a [m][H] (fp64).

    The [H, 2I] "up & gate" product is two [H, I] products here (gate and up
    columns kept apart); SwiGLU is silu(gate) times up.  The intermediate h is
    taken at the precision the down-projection consumes it in:
      'f32'  : unrounded;
      'bf16' : rounded to bf16 (nearest even);
      'e4m3' : fl32(h), then quantised per row and 128-column block exactly as
               the activations are (quant_e4m3_1x128) and dequantised;
      'mxfp8': fl32(h), then MXFP8 per row and 32-column block (mx.py), as
               the activations of an MXFP4 layer are.
    """
    g = a @ wg.T
    u = a @ wu.T
    h = silu(g) * u
    if h_mode == "bf16":
        h = codecs.bf16_rne(h)
    elif h_mode == "e4m3":
        q, s = codecs.quant_e4m3_1x128(h.astype(np.float32))
        h = codecs.dequant_e4m3_1x128(q, s)
    elif h_mode == "mxfp8":
        h = mx.mxfp8_round_trip(h.astype(np.float32))
    elif h_mode != "f32":
        raise ValueError(h_mode)
    y = h @ wd.T
    return (y, h) if return_h else y


def round_to(v: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f32":
        return v.astype(np.float32).astype(np.float64)
    if dt == "bf16":
        return codecs.bf16_rne(v)
    raise ValueError(dt)


def round_y(v: np.ndarray, y_dt: str) -> np.ndarray:
    """Expert outputs as the combine receives them: rounded to fp32 / bf16,
    or, for the FP8 combine ([P2] section 2: FP8 for the combine payload is
    the lever from 3300 to 5000 tokens/s per GPU), each row quantised per
    128-column block by the same rule as the activations (O6) from its fp32
    value, then dequantised (exact)."""
    if y_dt == "e4m3":
        q, s = codecs.quant_e4m3_1x128(np.asarray(v, dtype=np.float64).astype(np.float32))
        return codecs.dequant_e4m3_1x128(q, s)
    return round_to(v, y_dt)


def h_mode_for(w_dt: str) -> str:
    return {"f32": "f32", "bf16": "bf16", "e4m3": "e4m3", "mxfp4": "mxfp8"}[w_dt]


# ---------------------------------------------------------- combine [P2] "combine reduce"

def combine(y_perm: np.ndarray, y_sh, dest: np.ndarray, w: np.ndarray, k: int) -> np.ndarray:
    """out[t] = y_sh[t] + sum_{j=0}^{k-1} w[t][j] * y_perm[dest[t*k + j]]
    (y_sh = 0 without a shared expert), accumulated in fp64 in this order."""
    T = w.shape[0]
    H = y_perm.shape[1]
    out = np.zeros((T, H)) if y_sh is None else y_sh.astype(np.float64).copy()
    for t in range(T):
        for j in range(k):
            out[t] += np.float64(w[t, j]) * y_perm[dest[t * k + j]]
    return out


# --------------------------------------------------------------------- inputs

def layer_inputs(wl):
    """x as float32 numpy (exact widening of bf16) and the router arrays."""
    x32 = wl.x.float().cpu().numpy()
    wr = wl.w_router.float().cpu().numpy()
    b = None if wl.bias is None else wl.bias.float().cpu().numpy()
    return x32, wr, b


def activation_rows(wl, x32: np.ndarray) -> np.ndarray:
    """The rows the experts consume, fp64: the input itself for f32/bf16
    layers; for e4m3 layers the per-1x128 quantised-and-dequantised input,
    for MXFP4 layers the MXFP8 (per-32) one (the quantisation is done once
    per token and shared by its k copies)."""
    if wl.w_dt == "e4m3":
        q, s = codecs.quant_e4m3_1x128(x32)
        return codecs.dequant_e4m3_1x128(q, s)
    if wl.w_dt == "mxfp4":
        return mx.mxfp8_round_trip(x32)
    return x32.astype(np.float64)


# ------------------------------------------------------------------ full layer

def moe_layer(wl, want_intermediates: bool = False) -> dict:
    """The whole layer on every token: route, permute, per-expert FFN over
    each expert's segment in permuted order, shared expert, combine."""
    x32, wr, b = layer_inputs(wl)
    ids, w, l = route(x32, wr, b, wl.k, wl.score)
    counts, offsets, src, dest = permute(ids, wl.E)
    a = activation_rows(wl, x32)
    hm = h_mode_for(wl.w_dt)
    y_dt = "bf16" if wl.out_dt == "bf16" else "f32"
    yr_dt = wl.y_dt or y_dt           # routed outputs (FP8 combine: 'e4m3')
    R = wl.T * wl.k
    y_perm = np.zeros((R, wl.H))
    for e in range(wl.E):
        p0, p1 = offsets[e], offsets[e + 1]
        if p1 == p0:
            continue
        rows = src[p0:p1] // wl.k
        wg, wu, wd = bank_expert_f64(wl.routed, e)
        y_perm[p0:p1] = round_y(expert_ffn(a[rows], wg, wu, wd, hm), yr_dt)
    y_sh = None
    if wl.shared is not None:
        wg, wu, wd = bank_expert_f64(wl.shared, 0)
        y_sh = round_to(expert_ffn(a, wg, wu, wd, hm), y_dt)
    out = round_to(combine(y_perm, y_sh, dest, w, wl.k), wl.out_dt)
    res = dict(ids=ids, w=w, counts=counts, offsets=offsets, src=src, dest=dest, out=out)
    if want_intermediates:
        res.update(logits=l, y_perm=y_perm, y_sh=y_sh, a=a)
    return res


def moe_layer_tokens(wl, tokens, procs: int = 1) -> dict:
    """Outputs for a subset of tokens only.  A token's routing and output
    depend on that token alone (the permutation only reorders work), so each
    sampled output is computed directly: out[t] = y_sh(x_t) +
    sum_j w[t][j] y_{ids[t][j]}(x_t).  Experts are visited one at a time
    (only one expert's weights are held on the host at once).

    procs > 1 spreads the experts (and the shared expert) over that many
    single-threaded worker processes (fork, no exec); every expert's rows are
    computed by the same code either way, and the combine below is the same,
    so the result does not depend on procs.  The banks are copied to host
    memory first (the workers never touch a device)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    x32, wr, b = layer_inputs(wl)
    xs = x32[tokens]
    ids, w, _ = route(xs, wr, b, wl.k, wl.score)
    a = activation_rows(wl, xs)
    hm = h_mode_for(wl.w_dt)
    y_dt = "bf16" if wl.out_dt == "bf16" else "f32"
    yr_dt = wl.y_dt or y_dt
    # tasks: (key, bank, expert, token rows, output rounding)
    tasks = []
    if wl.shared is not None:
        tasks.append(("shared", "shared", 0, np.arange(len(tokens)), y_dt))
    for e in sorted(set(int(e) for e in ids.reshape(-1))):
        rows_t, rows_j = np.nonzero(ids == e)
        tasks.append(((e, rows_t, rows_j), "routed", e, rows_t, yr_dt))
    banks = {"routed": wl.routed, "shared": wl.shared}
    if procs > 1:
        results = _map_experts(banks, a, hm, tasks, procs)
    else:
        results = [_expert_task(banks, a, hm, t) for t in tasks]
    out = np.zeros((len(tokens), wl.H))
    ys = {}
    for (key, _, _, _, _), y in zip(tasks, results):
        if key == "shared":
            out += y
        else:
            _, rows_t, rows_j = key
            for r, (t, j) in enumerate(zip(rows_t, rows_j)):
                ys[(t, j)] = y[r]
    for t in range(len(tokens)):          # combine in slot order j = 0 .. k-1
        for j in range(wl.k):
            out[t] += np.float64(w[t, j]) * ys[(t, j)]
    return dict(tokens=tokens, ids=ids, w=w, out=round_to(out, wl.out_dt))


def _expert_task(banks, a, hm, task):
    """One expert's FFN on its token rows, rounded as the combine receives
    it (routed: round_y; shared: round_to)."""
    key, which, e, rows, rdt = task
    y = expert_ffn(a[rows], *bank_expert_f64(banks[which], e), hm)
    return round_to(y, rdt) if key == "shared" else round_y(y, rdt)


_FORKED = {}   # state the forked workers inherit


def _forked_task(i):
    from threadpoolctl import threadpool_limits
    st = _FORKED
    with threadpool_limits(limits=1):
        return _expert_task(st["banks"], st["a"], st["hm"], st["tasks"][i])


def _map_experts(banks, a, hm, tasks, procs):
    """_expert_task over tasks in `procs` forked processes (largest first).
    The experts the tasks use are copied to host memory first, one bank of
    one expert each, which the workers then read as expert 0."""
    import multiprocessing as mp
    host = {}
    local = []
    for key, which, e, rows, rdt in tasks:
        if (which, e) not in host:
            host[(which, e)] = banks[which].expert(e).to("cpu")
        local.append((key, (which, e), 0, rows, rdt))
    _FORKED.update(banks=host, a=a, hm=hm, tasks=local)
    order = sorted(range(len(tasks)), key=lambda i: -len(tasks[i][3]))
    try:
        with mp.get_context("fork").Pool(procs) as pool:
            done = dict(zip(order, pool.map(_forked_task, order, chunksize=1)))
    finally:
        _FORKED.clear()
    return [done[i] for i in range(len(tasks))]


# ----------------------------------------------------------- pre-routed groups

def prerouted_rows(wl):
    """The activation rows of a pre-routed grouped workload as the experts
    consume them: a function of row indices giving fp64 rows [len][H].
    e4m3 rows are codes with one fp32 scale per row and 128 columns, value =
    e4m3(code) * scale[row][col / 128]; MXFP4 layers receive bf16 rows and
    consume them as MXFP8 (quantised per 32 columns); bf16 / fp32 rows are
    taken as they are."""
    H = wl.H
    if wl.w_dt == "e4m3":
        qa = wl.a_q.cpu().numpy()
        sa = wl.a_s.cpu().numpy().astype(np.float64)

        def rows_of(idx):
            idx = np.asarray(idx)
            return (_E4M3_TABLE[qa[idx]].reshape(len(idx), H // 128, 128) * sa[idx][:, :, None]).reshape(len(idx), H)
    elif wl.w_dt == "mxfp4":
        xa = wl.x.float().cpu().numpy()

        def rows_of(idx):
            return mx.mxfp8_round_trip(xa[np.asarray(idx)])
    else:
        xa = wl.x.float().cpu().numpy()

        def rows_of(idx):
            return xa[np.asarray(idx)].astype(np.float64)
    return rows_of


def grouped_ffn(wl, group_sample=None) -> dict:
    """Pre-routed grouped FFN (no routing, no combine): each routed group g
    runs expert g on its contiguous rows, the shared expert on the last
    segment; outputs unweighted, rounded to wl.out_dt (routed groups: to
    wl.y_dt when set, see round_y).  `group_sample` maps a
    group index (or 'shared') to the row indices within that group to
    evaluate (all rows when absent).  Returns {group: (rows, y)}."""
    H = wl.H
    G = len(wl.group_m)
    starts = np.concatenate([[0], np.cumsum(wl.group_m)]).astype(np.int64)
    rows_of = prerouted_rows(wl)
    res = {}
    segs = [(g, starts[g], wl.group_m[g]) for g in range(G)]
    if wl.shared_m:
        segs.append(("shared", starts[G], wl.shared_m))
    for g, r0, m in segs:
        sel = np.arange(m) if (group_sample is None or g not in group_sample) else np.asarray(group_sample[g])
        if len(sel) == 0:
            res[g] = (sel, np.zeros((0, H)))
            continue
        bank, e = (wl.shared, 0) if g == "shared" else (wl.routed, g)
        y = expert_ffn(rows_of(r0 + sel), *bank_expert_f64(bank, e), h_mode_for(wl.w_dt))
        res[g] = (sel, round_to(y, wl.out_dt) if g == "shared" else round_y(y, wl.y_dt or wl.out_dt))
    return res


# --------------------------------------------------------------- brute force

def dense_moe(wl, ids: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Brute force: run EVERY routed expert on EVERY token, weight each
    output by the token's routing weight for that expert (zero when the
    expert was not chosen) and add the shared expert.  Uses torch float64
    library routines (matmul, silu), not the oracle's own FFN.  No
    intermediate rounding: compare against the oracle with its rounding
    points disabled, or with a tolerance."""
    import torch
    x32, _, _ = layer_inputs(wl)
    xa = torch.from_numpy(activation_rows(wl, x32))
    T = xa.shape[0]
    gate = torch.zeros(T, wl.E, dtype=torch.float64)
    for t in range(T):
        for j in range(wl.k):
            gate[t, ids[t, j]] += float(w[t, j])
    out = torch.zeros(T, wl.H, dtype=torch.float64)
    for e in range(wl.E):
        wg, wu, wd = (torch.from_numpy(m) for m in bank_expert_f64(wl.routed, e))
        ye = torch.nn.functional.silu(xa @ wg.T) * (xa @ wu.T) @ wd.T
        out += gate[:, e:e + 1] * ye
    if wl.shared is not None:
        wg, wu, wd = (torch.from_numpy(m) for m in bank_expert_f64(wl.shared, 0))
        out += torch.nn.functional.silu(xa @ wg.T) * (xa @ wu.T) @ wd.T
    return out.numpy()
