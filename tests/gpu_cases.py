"""Shared helpers for the GPU parity tests: seeded cases on both sides and comparisons.

The oracle quantizes its own copy of every weight; the GPU path quantizes with
the library.  Inputs come from seeded numpy draws (or workloads.gen); the
calibrated global scales of a random case come from the oracle's calibration
(an input to both sides).  Nothing flows from the GPU path into the oracle.
"""

from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np
import torch

from oracle import moe as omoe
from oracle import nvfp4 as onv
from oracle import routing as oroute
from workloads import gen

NEAR_TIE = 1e-9


def say(msg: str) -> None:
    """Name the case on stdout before a GPU step, so a fault can be attributed."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def pair_rows(pair_out: torch.Tensor, pair_scale: torch.Tensor) -> np.ndarray:
    """FP64 pair rows from the FP16 values and their power-of-two row scales (exact)."""
    return to_np(pair_out).astype(np.float64) * to_np(pair_scale).astype(np.float64)[:, None]


def expected_pair_scale(topk_w: np.ndarray, ids: np.ndarray, I: int, h_gs: np.ndarray, w2_gs: np.ndarray) -> np.ndarray:
    """The row scales the library's pair-row format states: 2^E, E = floor(log2(B)) - 14 clamped to [-126, 113],
    B = |w_p| * (I * 2688^2) * (1 / (h_gs[e] * w2_gs[e])) in FP32 operations in that order."""
    f32 = np.float32
    w = np.abs(np.asarray(topk_w, f32).reshape(-1))
    e = np.asarray(ids).reshape(-1)
    alpha = f32(1.0) / (np.asarray(h_gs, f32)[e] * np.asarray(w2_gs, f32)[e])
    with np.errstate(over="ignore", invalid="ignore"):
        bound = (w * f32(f32(I) * f32(7225344.0))) * alpha
    bits = bound.view(np.uint32)
    eb = ((bits >> 23) & 255).astype(np.int64) - 127
    E = np.clip(eb - 14, -126, 113)
    return np.ldexp(np.float32(1.0), E).astype(np.float32)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def bf16_round(a: np.ndarray) -> np.ndarray:
    return gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(np.asarray(a, np.float32))).astype(np.float64)


@dataclass
class Case:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    rsf: float
    x: np.ndarray  # [T, H] bf16 bits
    wr: np.ndarray  # [E, H] bf16 bits
    bias: np.ndarray  # [E] f32
    gate: list  # per expert [I, H] bf16 bits
    up: list
    down: list  # per expert [H, I] bf16 bits
    gs_x: np.float32
    gs_h: np.ndarray  # [E] f32
    experts_q: list  # oracle ExpertQ per expert

    def w13_bf16(self, device="cuda") -> torch.Tensor:
        w = np.stack([np.concatenate([g, u], axis=0) for g, u in zip(self.gate, self.up)])
        return dev_bf16(w, device)

    def w2_bf16(self, device="cuda") -> torch.Tensor:
        return dev_bf16(np.stack(self.down), device)


def random_case(name, seed, T, H, I, E, k, rsf=2.5, wscale=0.02, xscale=1.0, bias_range=0.1, n_cal=64,
                tiny_rows: float = 0.0) -> Case:
    """A seeded random layer.  tiny_rows > 0 shrinks that fraction of weight rows by
    2^-10..2^-14 so their E4M3 block scales fall in the subnormal range."""
    rng = np.random.default_rng(seed)
    bf = lambda a: gen.f32_to_bf16_bits(np.asarray(a, np.float32))  # noqa: E731

    def w(shape):
        a = rng.standard_normal(shape) * wscale
        if tiny_rows:
            sel = rng.random(shape[0]) < tiny_rows
            a[sel] *= np.exp2(-rng.uniform(10, 14, (int(sel.sum()), 1)))
        return bf(a)

    x = bf(rng.standard_normal((T, H)) * xscale)
    wr = bf(rng.standard_normal((E, H)) * 0.02)
    bias = rng.uniform(-bias_range, bias_range, E).astype(np.float32)
    gate = [w((I, H)) for _ in range(E)]
    up = [w((I, H)) for _ in range(E)]
    down = [w((H, I)) for _ in range(E)]
    f32 = gen.bf16_bits_to_f32
    experts_q = [omoe.quantize_expert(f32(g), f32(u), f32(d)) for g, u, d in zip(gate, up, down)]
    x_cal = bf(rng.standard_normal((n_cal, H)) * xscale)
    gs_x, gs_h = omoe.calibrate(x_cal, experts_q, E)
    return Case(name, T, H, I, E, k, rsf, x, wr, bias, gate, up, down, gs_x, gs_h, experts_q)


def config_case(cfg, T=None, experts=None) -> Case:
    """A workload config's inputs (optionally fewer tokens) with oracle-quantized experts (lazily: only `experts`)."""
    ws = cfg.weights
    x = gen.tokens(cfg, T)
    gs_x, gs_h = gen.global_scales(ws)
    gate, up, down, q = [None] * ws.E, [None] * ws.E, [None] * ws.E, [None] * ws.E
    for e, g, u, d in gen.iter_experts_bf16(ws, experts):
        gate[e], up[e], down[e] = g, u, d
        f32 = gen.bf16_bits_to_f32
        q[e] = omoe.quantize_expert(f32(g), f32(u), f32(d))
    return Case(cfg.name, x.shape[0], ws.H, ws.I, ws.E, cfg.k, cfg.rsf, x, gen.router_weight(ws),
                gen.router_bias(cfg), gate, up, down, gs_x, gs_h, q)


def gpu_layer(case: Case, device="cuda"):
    from nvfp4_w4a4_mixture_amd.layer import NVFP4MoELayer

    return NVFP4MoELayer.from_bf16(dev_bf16(case.wr, device), torch.from_numpy(case.bias).to(device), case.k,
                                   case.rsf, torch.tensor([case.gs_x], dtype=torch.float32, device=device),
                                   torch.from_numpy(case.gs_h).to(device), case.w13_bf16(device),
                                   case.w2_bf16(device))


def oracle_layer(case: Case, tokens=None, with_pairs=False) -> dict:
    return omoe.moe_layer(case.x, case.wr, case.bias, case.k, case.rsf, case.gs_x, case.experts_q, case.gs_h,
                          tokens=tokens, with_pairs=with_pairs)


def check_routing(ids_gpu, w_gpu, ref: dict, rsf: float, E: int, x_bf16=None, wr_bf16=None, bias=None) -> int:
    """Routing parity; returns the number of near-tie tokens.

    Tokens whose oracle top-k margin (score_(k) - score_(k+1)) is >= NEAR_TIE:
    the GPU ids equal the oracle's bitwise and topk_w is within 1e-6 * rsf of
    the oracle's FP64 weights.  Near-tie tokens (an exact tie included) may
    legitimately pick another top-k when the two sides round a score
    differently, so for them the GPU choice is checked for validity against
    the oracle's FP64 scores, recomputed for those tokens from x, the router
    and the bias: k distinct ids in [0, E); slots in descending score (each
    within NEAR_TIE of the next); every chosen score >= every unchosen score -
    NEAR_TIE; and topk_w = rsf * s_j / sum(s) over the GPU's own chosen set,
    within 1e-6 * rsf."""
    ids_ref, gap = ref["ids"], ref["gap"]
    ids_gpu = np.asarray(ids_gpu)
    w_gpu = np.asarray(w_gpu)
    k = ids_gpu.shape[1]
    clear = gap >= NEAR_TIE
    assert np.array_equal(ids_gpu[clear], ids_ref[clear]), "top-k ids differ"
    assert np.all(np.abs(w_gpu[clear].astype(np.float64) - ref["weights64"][clear]) <= 1e-6 * rsf), "topk_w differ"
    near = np.nonzero(~clear)[0]
    if len(near) == 0:
        return 0
    if x_bf16 is None or wr_bf16 is None or bias is None:
        raise AssertionError(f"{len(near)} near-tie tokens and no x/router/bias to validate them")
    s = oroute.sigmoid(oroute.router_logits(np.asarray(x_bf16)[near], wr_bf16))
    score = s + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    for n, t in enumerate(near):
        sel = ids_gpu[t].astype(np.int64)
        assert np.all((sel >= 0) & (sel < E)) and len(set(sel.tolist())) == k, f"token {t}: invalid ids {sel}"
        sc = score[n, sel]
        assert np.all(sc[:-1] >= sc[1:] - NEAR_TIE), f"token {t}: slots not in descending score"
        rest = np.setdiff1d(np.arange(E), sel)
        if len(rest):
            assert sc.min() >= score[n, rest].max() - NEAR_TIE, f"token {t}: not a top-k"
        w_want = rsf * s[n, sel] / np.sum(s[n, sel])
        assert np.all(np.abs(w_gpu[t].astype(np.float64) - w_want) <= 1e-6 * rsf), f"token {t}: topk_w"
    return int(len(near))


def untile_weight_scales(s) -> np.ndarray:
    """Tiled weight scales [..., R/16, K/128, 16, 8] -> row-major [..., R, K/16].

    The tiled layout is an index permutation of the row-major one: scale (r, b)
    sits at [r // 16, b // 8, r % 16, b % 8]."""
    s = np.asarray(s)
    *lead, rt, kt, r16, q8 = s.shape
    return np.swapaxes(s, -3, -2).reshape(*lead, rt * r16, kt * q8)


def oracle_codes(case: Case):
    """Oracle quantization of x: (packed codes [T, H/2], scales [T, H/16])."""
    c, s = onv.quantize(gen.bf16_bits_to_f32(case.x), case.gs_x)
    return onv.pack_codes(c), s


def oracle_perm(ids: np.ndarray, E: int):
    return oroute.permute(ids, E)
