"""GPU parity of the router top-k (softmax of FP32 logits, the k largest)
against the FP64 oracle.

The expert ids are chosen on the logits on both sides (the order of the exact
probabilities), so they must match exactly, ties (equal logits) included.
The weights are FP32 softmax values: the kernel's exp of the FP32 difference
l - max (rounded: at most 2^-24 |l - max|, about 6e-7 relative for the
workload's |l - max| < 10), an exp within a couple of ulps, a sum of E
positive terms (relative error at most (E-1) 2^-24, 3.8e-6 for E = 64) and one
division: a relative bound of 1e-5, and 2e-5 for E = 1000 logits of the same
spread (sum error up to 6e-5 in the worst order; the tested draws sit far
below it).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_precision_tn_amd as mg
    mg.load()
    yield


def route(lg, k):
    import block_scaled_precision_tn_amd as mg
    ids, w = mg.mgemm_moe_route_topk(torch.from_numpy(np.ascontiguousarray(lg)).cuda(), k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("T,E,k,rtol", [(4096, 64, 8, 1e-5), (37, 1000, 13, 2e-5),
                                        (130, 256, 1, 1e-5), (5, 64, 64, 1e-5),
                                        (9, 7, 3, 1e-5), (3, 1, 1, 1e-5)])
def test_route_matches_oracle(T, E, k, rtol):
    lg = synth.moe_logits(T, E, seed=T + E)
    ids, w = route(lg, k)
    ids0, w0 = oracle.topk_softmax(lg, k)
    assert np.array_equal(ids, ids0)
    np.testing.assert_allclose(w, w0, rtol=rtol, atol=0)


def test_route_ties_go_to_the_lower_id():
    lg = np.zeros((6, 64), np.float32)
    lg[1, [5, 9, 40]] = 1.0                    # three equal maxima
    lg[2] = np.repeat(np.arange(16, dtype=np.float32), 4)   # runs of four equal logits
    lg[3, ::2] = -1.0
    ids, w = route(lg, 8)
    ids0, w0 = oracle.topk_softmax(lg, 8)
    assert np.array_equal(ids, ids0)
    assert ids[0].tolist() == list(range(8)) and ids[1, :3].tolist() == [5, 9, 40]
    np.testing.assert_allclose(w, w0, rtol=1e-5)


def test_route_repeat_bit_identical():
    lg = synth.moe_logits(512, 64, seed=1)
    a = route(lg, 8)
    b = route(lg, 8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


# ------------------------------------------ the router fused into route prep
def _moe_both_ways(T, H, I, E, topk, seed):
    """The MXFP8 MoE routed from logits in one call, and the unfused path:
    the standalone router, then the MoE on its ids / weights."""
    import block_scaled_precision_tn_amd as mg
    from gpu_cases import dev
    inp = synth.moe(T, H, I, E, topk, seed=seed)
    lg = synth.moe_logits(T, E, seed=seed)
    args = [dev(inp[k]) for k in ("xq", "xs")]
    wts = [dev(inp[k]) for k in ("w13q", "w13s", "w2q", "w2s")]
    lgd = dev(lg)
    dbg_f = torch.zeros(T * topk * (I + I // 32), dtype=torch.uint8, device="cuda")
    out_f = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    _, ids_f, w_f = mg.mgemm_moe_mxfp8_glu_logits(*args, lgd, topk, *wts, out_f, dbg_h=dbg_f)
    ids_u, w_u = mg.mgemm_moe_route_topk(lgd, topk)
    dbg_u = torch.zeros_like(dbg_f)
    out_u = torch.empty_like(out_f)
    mg.mgemm_moe_mxfp8_glu(*args, ids_u, w_u, *wts, out_u, dbg_h=dbg_u)
    torch.cuda.synchronize()
    return lg, (ids_f, w_f, out_f, dbg_f), (ids_u, w_u, out_u, dbg_u)


@pytest.mark.parametrize("T,H,I,E,topk", [(1, 256, 128, 64, 8),      # one-workgroup routing
                                          (29, 128, 256, 300, 5),    # E > 256 (16 logits per lane)
                                          (333, 128, 128, 64, 8),    # the four-kernel routing
                                          (70, 64, 64, 7, 3)])       # a ragged last workgroup
def test_fused_routing_matches_unfused(T, H, I, E, topk):
    lg, f, u = _moe_both_ways(T, H, I, E, topk, seed=T + E)
    ids0, w0 = oracle.topk_softmax(lg, topk)
    assert np.array_equal(f[0].cpu().numpy(), ids0)
    np.testing.assert_allclose(f[1].cpu().numpy(), w0, rtol=2e-5, atol=0)
    for a, b in zip(f, u):    # ids, weights, output and re-quantised h: bit for bit
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_fused_routing_full_size():
    """T = 4096, H = 4096, I = 1536, E = 64, top 8 (the MoE workload) and
    T = 1 on its weights."""
    for T in (4096, 1):
        lg, f, u = _moe_both_ways(T, 4096, 1536, 64, 8, seed=0)
        ids0, _ = oracle.topk_softmax(lg, 8)
        assert np.array_equal(f[0].cpu().numpy(), ids0)
        for a, b in zip(f, u):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
