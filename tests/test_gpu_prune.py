"""GPU parity of the REAP pruning step (reap_prune_select, moe_gather_experts,
NVFP4MoELayer.prune) against the oracle in oracle/reap.py.

Bit-exact: the kept expert ids and every gathered byte.  The pruned layer's
output is held to the layer bar (routing bit-exact, y rel-L2 <= 2e-3) against
the oracle's layer built from the oracle-sliced router, bias and experts.
"""

import zlib

import numpy as np
import pytest
import torch

from gpu_cases import check_routing, dev_bf16, gpu_layer, random_case, rel_l2, say, to_np
from oracle import moe as omoe
from oracle import reap as oreap

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3
SAL_TOL = 1e-3


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from nvfp4_w4a4_mixture_amd import ops as _ops

    return _ops


def _saliency(kind: str, E: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        return rng.random(E).astype(np.float32)
    if kind == "ties":  # few distinct values, zeros and negative zeros among them
        s = rng.integers(0, 4, E).astype(np.float32) * np.float32(0.25)
        s[rng.random(E) < 0.2] = np.float32(-0.0)
        return s
    if kind == "equal":
        return np.full(E, 0.5, np.float32)
    if kind == "unrouted":  # a tail of never-routed experts (saliency exactly 0)
        s = rng.lognormal(0.0, 1.0, E).astype(np.float32)
        s[rng.choice(E, E // 3, replace=False)] = 0.0
        return s
    raise ValueError(kind)


@pytest.mark.parametrize("E", [1, 8, 80, 128, 200, 256])
@pytest.mark.parametrize("kind", ["uniform", "ties", "equal", "unrouted"])
def test_prune_select_bitexact(ops, E, kind):
    s = _saliency(kind, E, zlib.crc32(f"{kind}{E}".encode()))
    dev = torch.from_numpy(s).cuda()
    for n in sorted({1, max(1, E // 2), max(1, E - 1), E, (E * 5) // 8 or 1}):
        say(f"prune_select E={E} kind={kind} n_keep={n}")
        got = to_np(ops.reap_prune_select(dev, n))
        assert np.array_equal(got, oreap.keep_ids(s, n)), (E, kind, n)


def test_prune_select_nan_still_gives_a_valid_set(ops):
    s = _saliency("uniform", 80, 5)
    s[[3, 17, 40]] = np.nan
    say("prune_select with NaN saliencies")
    got = to_np(ops.reap_prune_select(torch.from_numpy(s).cuda(), 50))
    assert got.shape == (50,) and np.all(np.diff(got) > 0) and got.min() >= 0 and got.max() < 80
    finite = np.setdiff1d(np.arange(80), [3, 17, 40])
    # among the finite experts, the kept ones still outrank the dropped ones
    kept_f = np.intersect1d(got, finite)
    drop_f = np.setdiff1d(finite, got)
    assert s[kept_f].min() >= s[drop_f].max()


@pytest.mark.parametrize("block,offset", [(1, 0), (3, 1), (4, 0), (12, 4), (16, 0), (48, 16), (16400, 0),
                                          (65539, 1), (262144, 0)])
def test_gather_experts_bytes(ops, block, offset):
    rng = np.random.default_rng(block)
    E_src, n = 37, 23
    src_np = rng.integers(0, 256, E_src * block, dtype=np.uint8)
    buf = torch.zeros(E_src * block + offset, dtype=torch.uint8, device="cuda")
    buf[offset:] = torch.from_numpy(src_np).cuda()
    src = buf[offset:].view(E_src, block)  # offset 1: unaligned, byte path; 4: 4-byte path
    ids_np = rng.choice(E_src, n, replace=True).astype(np.int32)  # repeats allowed
    say(f"gather block={block} offset={offset}")
    out = ops.moe_gather_experts(src, torch.from_numpy(ids_np).cuda())
    assert np.array_equal(to_np(out), src_np.reshape(E_src, block)[ids_np])


def test_gather_out_of_range_id_leaves_block_unwritten(ops):
    src = torch.arange(8 * 64, dtype=torch.int32, device="cuda").view(8, 64)
    ids = torch.tensor([2, 8, -1, 7], dtype=torch.int32, device="cuda")
    out = torch.full((4, 64), -5, dtype=torch.int32, device="cuda")
    say("gather with out-of-range ids")
    ops.moe_gather_experts(src, ids, out=out)
    o = to_np(out)
    s = to_np(src)
    assert np.array_equal(o[0], s[2]) and np.array_equal(o[3], s[7])
    assert np.all(o[1] == -5) and np.all(o[2] == -5)


def _pruned_check(ops, case, sal: np.ndarray, n_keep: int):
    """GPU layer.prune(sal) against the oracle layer over oreap-sliced inputs."""
    layer = gpu_layer(case)
    say(f"pruned layer {case.name} T={case.T} E={case.E} -> {n_keep}")
    pl = layer.prune(torch.from_numpy(sal).cuda(), n_keep)
    keep = oreap.keep_ids(sal, n_keep)
    assert np.array_equal(to_np(pl.keep_ids), keep)
    assert pl.E == n_keep
    # every gathered tensor equals the unpruned one's kept slices, bitwise
    full = [layer.w_router, layer.bias, layer.h_gs, *layer.w13, *layer.w2]
    pruned = [pl.w_router, pl.bias, pl.h_gs, *pl.w13, *pl.w2]
    for a, b in zip(full, pruned):
        assert torch.equal(a.cpu()[torch.from_numpy(keep).long()], b.cpu())
    wr_k, b_k = oreap.slice_router(case.wr, case.bias, keep)
    out = pl(dev_bf16(case.x), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = omoe.moe_layer(case.x, wr_k, b_k, case.k, case.rsf, case.gs_x, oreap.slice_experts(case.experts_q, keep),
                         case.gs_h[keep])
    check_routing(to_np(out.route.topk_ids), to_np(out.route.topk_w), ref, case.rsf, n_keep, case.x, wr_k, b_k)
    err = rel_l2(to_np(out.y), ref["y"])
    print(f"  pruned rel-L2 y={err:.3e}", flush=True)
    assert err <= Y_TOL
    return layer, pl


@pytest.mark.parametrize("name,T,H,I,E,k,n_keep", [
    ("prune_tiled", 200, 512, 256, 16, 4, 10),
    ("prune_small", 9, 512, 256, 12, 4, 5),
    ("prune_to_k", 40, 256, 128, 8, 2, 2),
])
def test_pruned_layer_parity(ops, name, T, H, I, E, k, n_keep):
    case = random_case(name, zlib.crc32(name.encode()) % 1000, T, H, I, E, k)
    _pruned_check(ops, case, _saliency("ties", E, 3), n_keep)


def test_reap_flow_keeps_the_oracles_clear_experts(ops):
    """Saliency from the layer on the GPU, then pruning: every expert whose oracle
    saliency is clearly above (below) the keep threshold is kept (dropped)."""
    case = random_case("reap_flow", 77, 300, 256, 128, 24, 4, bias_range=0.3)
    layer = gpu_layer(case)
    say("reap flow: layer with saliency, then prune 24 -> 15")
    out = layer(dev_bf16(case.x), out_dtype=torch.float32, reap=True)
    pl = layer.prune(out.saliency, 15)
    torch.cuda.synchronize()
    ref = omoe.moe_layer(case.x, case.wr, case.bias, case.k, case.rsf, case.gs_x, case.experts_q, case.gs_h)
    s_ref = ref["saliency"]
    thr = np.sort(s_ref)[::-1][14:16].mean()  # between the 15th and 16th largest
    margin = 2.5 * SAL_TOL * thr
    keep = set(to_np(pl.keep_ids).tolist())
    clear_in = np.nonzero(s_ref > thr + margin)[0]
    clear_out = np.nonzero(s_ref < thr - margin)[0]
    assert len(clear_in) + len(clear_out) >= 20
    assert set(clear_in.tolist()) <= keep and not (set(clear_out.tolist()) & keep)
