"""Seeded synthetic inputs for the sparse MoE FFN layer.

This module only draws numbers: tokens, router weights, expert weights, the
skewed-popularity logit bias and pre-routed group sizes.  It contains none of
the layer's own arithmetic (no routing, no permutation, no FFN, no combine),
so both the GPU library's tests and the CPU oracle can take their inputs from
here without sharing any of the method.

Random numbers come from a counter-based generator: element i of the tensor
stream (seed, stream) is a pure function of (seed, stream, i), built from the
SplitMix64 finaliser (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014) and the Box-Muller transform in double precision.  It
is written with torch integer ops so the same code runs on the CPU (small
cases) and on the GPU (the multi-gigabyte expert banks), and any slice of a
tensor can be regenerated on its own.  Values drawn on the two devices agree up
to the last bit of the double-precision log/cos, which is far below the
storage rounding.

Shapes follow the pages' DeepSeek-V3 layer: hidden 7168, expert intermediate
2048, 256 routed experts plus one shared expert, top-8 ("DeepSeek V3/R1
Inference Efficiency (2)", section 2.3.1, the routed and shared expert GEMM
shapes; "How DeepSeek inference works", the worked example of 256 experts
with 8 active per token).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from statistics import NormalDist
from typing import Optional

import torch

_MASK64 = (1 << 64) - 1


def _s64(v: int) -> int:
    """Map an unsigned 64-bit constant onto torch's signed int64."""
    v &= _MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


_GAMMA = _s64(0x9E3779B97F4A7C15)
_M1 = _s64(0xBF58476D1CE4E5B9)
_M2 = _s64(0x94D049BB133111EB)


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 (torch's >> is arithmetic)."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _M1
    z = (z ^ _srl(z, 27)) * _M2
    return z ^ _srl(z, 31)


def _mix_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    return _mix_int(_mix_int(seed * 0x9E3779B97F4A7C15 + 0x632BE59BD9B4E019) ^ (stream * 0xD1B54A32D192ED03))


def uniform64(seed: int, stream: int, start: int, n: int, device) -> torch.Tensor:
    """Raw 64-bit draws (as int64) for counters start .. start+n-1."""
    key = _s64(stream_key(seed, stream))
    i = torch.arange(start, start + n, dtype=torch.int64, device=device)
    return _mix(key + i * _GAMMA)


def normal_(out: torch.Tensor, seed: int, stream: int, std: float = 1.0,
            start: int = 0, chunk: int = 1 << 25) -> torch.Tensor:
    """Fill `out` (any dtype, contiguous) with N(0, std^2) draws.

    Element j of `out` is draw number start + j of stream (seed, stream): two
    counters per draw, one Box-Muller cosine branch, computed in float64 and
    rounded once to out.dtype.
    """
    assert out.is_contiguous()
    flat = out.view(-1)
    n = flat.numel()
    key = _s64(stream_key(seed, stream))
    two_pi = 2.0 * math.pi
    for c0 in range(0, n, chunk):
        m = min(chunk, n - c0)
        i = torch.arange(2 * (start + c0), 2 * (start + c0 + m), dtype=torch.int64, device=out.device)
        z = _mix(key + i * _GAMMA).view(m, 2)
        u1 = (_srl(z[:, 0], 11) + 1).to(torch.float64) * (2.0 ** -53)
        u2 = _srl(z[:, 1], 11).to(torch.float64) * (2.0 ** -53)
        v = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(two_pi * u2)
        if std != 1.0:
            v = v * std
        flat[c0:c0 + m] = v.to(out.dtype)
        del z, u1, u2, v, i
    return out


def normal(shape, seed: int, stream: int, std: float = 1.0, dtype=torch.float32,
           device="cpu", start: int = 0) -> torch.Tensor:
    return normal_(torch.empty(shape, dtype=dtype, device=device), seed, stream, std, start)


def randint_list(seed: int, stream: int, n: int, lo: int, hi: int) -> list[int]:
    """n integers uniform on {lo..hi} (multiply-shift on the top 32 bits)."""
    key = stream_key(seed, stream)
    span = hi - lo + 1
    out = []
    for i in range(n):
        z = _mix_int(key + i * 0x9E3779B97F4A7C15)
        out.append(lo + (((z >> 32) * span) >> 32))
    return out


def permutation(seed: int, stream: int, n: int) -> list[int]:
    """Seeded Fisher-Yates shuffle of range(n)."""
    key = stream_key(seed, stream)
    p = list(range(n))
    for i in range(n - 1, 0, -1):
        z = _mix_int(key + (n - 1 - i) * 0x9E3779B97F4A7C15)
        j = ((z >> 32) * (i + 1)) >> 32
        p[i], p[j] = p[j], p[i]
    return p


# --------------------------------------------------------------------------
# Block-scaled e4m3 storage of weights and pre-quantised activations.
# The codes are produced with torch's float8_e4m3fn cast (a library codec);
# the scale of a block is its largest magnitude over 448, in fp32.
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def block_quant_e4m3(w: torch.Tensor, br: int, bc: int):
    """w [..., R, C] fp32 -> (codes uint8 [..., R, C], scales fp32 [..., R/br, C/bc])."""
    *lead, R, C = w.shape
    assert R % br == 0 and C % bc == 0
    wb = w.reshape(*lead, R // br, br, C // bc, bc)
    amax = wb.abs().amax(dim=(-3, -1))
    s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (wb / s[..., :, None, :, None]).to(torch.float8_e4m3fn)
    return q.reshape(*lead, R, C).view(torch.uint8), s.to(torch.float32)


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
# stream ids (one counter space per tensor; experts of a bank share one)
ST_X, ST_ROUTER, ST_ORDER, ST_GROUPS = 1, 2, 3, 4
ST_RG, ST_RU, ST_RD = 10, 11, 12      # routed bank gate / up / down
ST_SG, ST_SU, ST_SD = 20, 21, 22      # shared expert gate / up / down


@dataclass
class Bank:
    """A bank of n experts; weights stored output-major (K contiguous):
    w_gate, w_up [n][I][H] (element (h, i) of W_gate at [e][i][h]);
    w_down [n][H][I].  dt is 'f32', 'bf16' or 'e4m3' (uint8 codes);
    e4m3 banks carry scales s_gate, s_up [n][I/128][H/128], s_down [n][H/128][I/128].
    'mxfp4' banks hold two E2M1 codes per byte along the reduction index
    (w_gate, w_up [n][I][H/2], w_down [n][H][I/2], lower index in the low
    nibble) and one E8M0 scale byte per 32 (s_gate, s_up [n][I][H/32],
    s_down [n][H][I/32])."""
    n: int
    H: int
    I: int
    dt: str
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    s_gate: Optional[torch.Tensor] = None
    s_up: Optional[torch.Tensor] = None
    s_down: Optional[torch.Tensor] = None

    def to(self, device):
        f = lambda t: None if t is None else t.to(device)
        return Bank(self.n, self.H, self.I, self.dt, f(self.w_gate), f(self.w_up), f(self.w_down),
                    f(self.s_gate), f(self.s_up), f(self.s_down))

    def expert(self, e: int) -> "Bank":
        f = lambda t: None if t is None else t[e:e + 1]
        return Bank(1, self.H, self.I, self.dt, f(self.w_gate), f(self.w_up), f(self.w_down),
                    f(self.s_gate), f(self.s_up), f(self.s_down))


@dataclass
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    x_dt: str            # 'f32' | 'bf16' | 'e4m3' (pre-quantised, pre-routed)
    w_dt: str
    out_dt: str          # 'f32' | 'bf16'
    score: str           # 'softmax' | 'sigmoid'
    x: Optional[torch.Tensor] = None
    w_router: Optional[torch.Tensor] = None   # [H][E] fp32
    bias: Optional[torch.Tensor] = None       # [E] fp32
    routed: Optional[Bank] = None
    shared: Optional[Bank] = None
    # pre-routed grouped input (the expert-parallel prefill share)
    group_m: Optional[list] = None            # rows per routed group
    shared_m: int = 0
    a_q: Optional[torch.Tensor] = None        # [sum m][H] uint8 (routed groups, then shared)
    a_s: Optional[torch.Tensor] = None        # [sum m][H/128] fp32
    meta: dict = field(default_factory=dict)
    # routed expert outputs before the combine: None = out_dt precision,
    # 'e4m3' = per-1x128 fp8 (the FP8 combine)
    y_dt: Optional[str] = None


def _mx_codes_(out: torch.Tensor, seed: int, stream: int, start: int, chunk: int = 1 << 24):
    """Fill a uint8 tensor with uniform bytes (the low byte of each draw)."""
    flat = out.view(-1)
    for c0 in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - c0)
        flat[c0:c0 + n] = (uniform64(seed, stream, start + c0, n, out.device) & 255).to(torch.uint8)
    return out


def _mx_scales_(out: torch.Tensor, seed: int, stream: int, start: int, e_lo: int, chunk: int = 1 << 24):
    """Fill a uint8 tensor with E8M0 exponents drawn uniformly from {e_lo, e_lo + 1}."""
    flat = out.view(-1)
    for c0 in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - c0)
        flat[c0:c0 + n] = (e_lo + (_srl(uniform64(seed, stream, start + c0, n, out.device), 40) & 1)).to(torch.uint8)
    return out


# E8M0 exponents of the synthetic MXFP4 banks: scales 2^-8 and 2^-7 with codes
# uniform over all 16 E2M1 values (mean square 8.5625) give weights of rms
# about 0.018, the scale of the N(0, 0.02^2) banks of the other dtypes.
MX_E_LO = 119
ST_MX_SCALE = 100                     # scale streams: code stream + 100


def _bank_mxfp4(idx, H, I, seed, streams, device) -> Bank:
    """Random MXFP4 experts: uniform E2M1 codes and E8M0 scales drawn
    directly (no quantisation of real-valued weights)."""
    sg, su, sd = streams
    per_w, per_s = H * I // 2, H * I // 32
    w = [torch.empty((len(idx), I, H // 2), dtype=torch.uint8, device=device) for _ in range(2)]
    w.append(torch.empty((len(idx), H, I // 2), dtype=torch.uint8, device=device))
    sc = [torch.empty((len(idx), I, H // 32), dtype=torch.uint8, device=device) for _ in range(2)]
    sc.append(torch.empty((len(idx), H, I // 32), dtype=torch.uint8, device=device))
    for j, e in enumerate(idx):
        for t, st in enumerate((sg, su, sd)):
            _mx_codes_(w[t][j], seed, st, e * per_w)
            _mx_scales_(sc[t][j], seed, st + ST_MX_SCALE, e * per_s, MX_E_LO)
    return Bank(len(idx), H, I, "mxfp4", w[0], w[1], w[2], sc[0], sc[1], sc[2])


def _bank(n, H, I, dt, seed, streams, std, device, experts=None) -> Bank:
    """Draw a bank of n experts.  `experts` optionally selects a subset of
    expert indices of the full counter space (regeneration of a slice)."""
    idx = list(range(n)) if experts is None else list(experts)
    if dt == "mxfp4":
        return _bank_mxfp4(idx, H, I, seed, streams, device)
    sg, su, sd = streams
    per = H * I
    tgt = torch.float32 if dt in ("f32", "e4m3") else torch.bfloat16
    wg = torch.empty((len(idx), I, H), dtype=tgt, device=device)
    wu = torch.empty((len(idx), I, H), dtype=tgt, device=device)
    wd = torch.empty((len(idx), H, I), dtype=tgt, device=device)
    for j, e in enumerate(idx):
        normal_(wg[j], seed, sg, std, start=e * per)
        normal_(wu[j], seed, su, std, start=e * per)
        normal_(wd[j], seed, sd, std, start=e * per)
    if dt != "e4m3":
        return Bank(len(idx), H, I, dt, wg, wu, wd)
    qg, s_g = block_quant_e4m3(wg, 128, 128)
    del wg
    qu, s_u = block_quant_e4m3(wu, 128, 128)
    del wu
    qd, s_d = block_quant_e4m3(wd, 128, 128)
    del wd
    return Bank(len(idx), H, I, dt, qg, qu, qd, s_g, s_u, s_d)


def zipf_bias(E: int, k: int, s: float, seed: int) -> tuple[torch.Tensor, list[float]]:
    """Additive logit bias whose expected inclusion probabilities follow a
    capped Zipf(s) law over a seeded expert order.

    Target inclusion of the expert at popularity rank r: pi_r = min(1, c r^-s),
    with c chosen so that sum_r pi_r = k (plain Zipf cannot hold: its top
    expert would need probability above 1).  With unit-variance logits and a
    selection threshold near 0, P(selected) ~ Phi(b), so b = Phi^-1(pi).
    """
    def total(c):
        return sum(min(1.0, c * r ** (-s)) for r in range(1, E + 1))
    lo, hi = 0.0, float(k)
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if total(mid) < k:
            lo = mid
        else:
            hi = mid
    c = 0.5 * (lo + hi)
    order = permutation(seed, ST_ORDER, E)
    nd = NormalDist()
    b = [0.0] * E
    pis = [0.0] * E
    for r in range(1, E + 1):
        pi = min(1.0, c * r ** (-s))
        e = order[r - 1]
        pis[e] = pi
        b[e] = nd.inv_cdf(min(max(pi, 1e-6), 1.0 - 1e-4))
    return torch.tensor(b, dtype=torch.float32), pis


CONFIG_NAMES = {
    1: "tiny-fp32-T64-H256-E8-top2",
    2: "dsv3-decode-bf16-T128-H7168-E256+1-top8",
    3: "dsv3-skew-bf16-T4096-H7168-E256+1-top8-zipf1.2",
    4: "ep-prefill-share-fp8-9+1groups-H7168-I2048",
    5: "dsv3-prefill-fp8-T16384-H7168-E256+1-top8",
}


def make_layer(T, H, E, k, I, *, x_dt="bf16", w_dt="bf16", out_dt="f32", score="sigmoid",
               shared=True, bias=None, seed=0, layer_seed=None, x_seed=None, device="cpu",
               w_std=0.02, name="custom") -> Workload:
    """A routed MoE layer: tokens, router, routed bank, optional shared expert."""
    ls = seed if layer_seed is None else layer_seed
    xs = seed if x_seed is None else x_seed
    xdt = torch.float32 if x_dt == "f32" else torch.bfloat16
    x = normal((T, H), xs, ST_X, 1.0, xdt, device)
    wr = normal((H, E), ls, ST_ROUTER, 1.0 / math.sqrt(H), torch.float32, device)
    routed = _bank(E, H, I, w_dt, ls, (ST_RG, ST_RU, ST_RD), w_std, device)
    sh = _bank(1, H, I, w_dt, ls, (ST_SG, ST_SU, ST_SD), w_std, device) if shared else None
    b = None if bias is None else bias.to(device)
    return Workload(name, T, H, E, k, I, x_dt, w_dt, out_dt, score, x, wr, b, routed, sh)


def make_grouped(group_m, shared_m, H, I, *, dt="e4m3", seed=4, device="cpu", w_std=0.02,
                 y_dt="bf16", name="custom-grouped") -> Workload:
    """Pre-routed grouped input: len(group_m) routed experts (group g owns the
    g-th contiguous run of rows) plus one shared expert on the last shared_m
    rows; rows x ~ N(0,1).  dt 'e4m3': rows stored as e4m3 codes with
    per-1x128 fp32 scales (a_q, a_s); 'bf16'/'f32': rows stored in x."""
    G = len(group_m)
    rows = sum(group_m) + shared_m
    routed = _bank(G, H, I, dt, seed, (ST_RG, ST_RU, ST_RD), w_std, device)
    sh = _bank(1, H, I, dt, seed, (ST_SG, ST_SU, ST_SD), w_std, device) if shared_m > 0 else None
    wl = Workload(name, 0, H, G, 8, I, dt, dt, y_dt, "none", routed=routed, shared=sh,
                  group_m=list(group_m), shared_m=shared_m)
    if dt == "e4m3":
        xa = normal((rows, H), seed, ST_X, 1.0, torch.float32, device)
        wl.a_q, wl.a_s = block_quant_e4m3(xa, 1, 128)
        del xa
    else:
        wl.x = normal((rows, H), seed, ST_X, 1.0, torch.float32 if dt == "f32" else torch.bfloat16, device)
    if dt == "mxfp4":
        wl.x_dt = "bf16"
    return wl


def routing_inputs(cid: int, device="cpu") -> dict:
    """The draws of layer workload cid that decide its routing (tokens,
    router, bias) and its shape, without the expert banks: the same values
    config(cid) holds."""
    if cid == 1:
        T, H, E, k, I, seed_l, seed_x = 64, 256, 8, 2, 512, 1, 1
        shape = dict(x_dt="f32", w_dt="f32", out_dt="f32", score="softmax", shared=False)
        bias = None
    elif cid == 2:
        T, H, E, k, I, seed_l, seed_x = 128, 7168, 256, 8, 2048, 2, 2
        shape = dict(x_dt="bf16", w_dt="bf16", out_dt="f32", score="sigmoid", shared=True)
        bias = None
    elif cid == 3:
        T, H, E, k, I, seed_l, seed_x = 4096, 7168, 256, 8, 2048, 2, 3
        shape = dict(x_dt="bf16", w_dt="bf16", out_dt="f32", score="sigmoid", shared=True)
        bias, _ = zipf_bias(256, 8, 1.2, seed=3)
    elif cid == 5:
        T, H, E, k, I, seed_l, seed_x = 16384, 7168, 256, 8, 2048, 2, 5
        shape = dict(x_dt="bf16", w_dt="e4m3", out_dt="bf16", score="sigmoid", shared=True)
        bias = None
    else:
        raise ValueError(cid)
    xdt = torch.float32 if shape["x_dt"] == "f32" else torch.bfloat16
    x = normal((T, H), seed_x, ST_X, 1.0, xdt, device)
    wr = normal((H, E), seed_l, ST_ROUTER, 1.0 / math.sqrt(H), torch.float32, device)
    return dict(T=T, H=H, E=E, k=k, I=I, x=x, w_router=wr, bias=None if bias is None else bias.to(device), **shape)


def config(cid: int, device="cpu", T: Optional[int] = None) -> Workload:
    """The five seeded workloads.  `T` overrides the token count (the layer
    and every other draw stay the same), for sampled or shrunken runs."""
    name = CONFIG_NAMES[cid]
    if cid == 1:
        return make_layer(T or 64, 256, 8, 2, 512, x_dt="f32", w_dt="f32", out_dt="f32",
                          score="softmax", shared=False, seed=1, device=device, name=name)
    if cid == 2:
        return make_layer(T or 128, 7168, 256, 8, 2048, x_dt="bf16", w_dt="bf16", out_dt="f32",
                          score="sigmoid", shared=True, seed=2, device=device, name=name)
    if cid == 3:
        b, pis = zipf_bias(256, 8, 1.2, seed=3)
        wl = make_layer(T or 4096, 7168, 256, 8, 2048, x_dt="bf16", w_dt="bf16", out_dt="f32",
                        score="sigmoid", shared=True, bias=b, layer_seed=2, x_seed=3,
                        device=device, name=name)
        wl.meta["target_inclusion"] = pis
        return wl
    if cid == 4:
        gm = randint_list(4, ST_GROUPS, 10, 256, 4096)
        return make_grouped(gm[:9], gm[9], 7168, 2048, seed=4, device=device, name=name)
    if cid == 5:
        return make_layer(T or 16384, 7168, 256, 8, 2048, x_dt="bf16", w_dt="e4m3", out_dt="bf16",
                          score="sigmoid", shared=True, layer_seed=2, x_seed=5, device=device, name=name)
    raise ValueError(cid)


def mxfp4_name(cid: int) -> str:
    """Name of layer workload cid with MXFP4 expert weights."""
    return CONFIG_NAMES[cid].replace("-bf16-", "-mxfp4-").replace("-fp8-", "-mxfp4-")


def config_mxfp4(cid: int, device="cpu", T: Optional[int] = None) -> Workload:
    """Layer workload cid (2, 3 or 5) with MXFP4 expert weights in place of
    its bf16 / e4m3 ones: the same tokens, router, bias and so the same
    routing; random MXFP4 banks (see _bank_mxfp4); x arrives in bf16 and is
    quantised to MXFP8 in-layer."""
    if cid not in (2, 3, 5):
        raise ValueError(f"MXFP4 variants exist for the layer workloads 2, 3 and 5, not {cid}")
    r = routing_inputs(cid, device="cpu")
    T = T or r["T"]
    ls = 2
    wl = make_layer(T, r["H"], r["E"], r["k"], r["I"], x_dt="bf16", w_dt="mxfp4", out_dt=r["out_dt"],
                    score=r["score"], shared=r["shared"], bias=r["bias"], layer_seed=ls,
                    x_seed={2: 2, 3: 3, 5: 5}[cid], device=device, name=mxfp4_name(cid))
    return wl
