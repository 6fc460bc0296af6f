"""Per-entry-point parity on the GPU: router top-k, permute, grouped SwiGLU
GEMM and combine, each called through the C ABI and compared with the
oracle element by element on seeded inputs that span several tiles and a
ragged tail."""
import numpy as np
import pytest

import moe_inputs
from oracle import moe_oracle as mo
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    torch, moe = gh.torch_and_lib()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, moe


# ------------------------------------------------------------ router ----

@pytest.mark.parametrize("T,H,E,k,rsf", [
    (1, 8, 1, 1, 1.0),          # degenerate: one token, one expert
    (100, 136, 8, 2, 1.0),      # ragged T, H not a multiple of the K step
    (333, 512, 64, 8, 2.5),     # several token tiles, scaled weights
    (70, 256, 200, 16, 1.0),    # k at its bound, E not a multiple of 64
    (65, 128, 1024, 16, 1.0),   # E at its bound
    (64, 64, 16, 16, 1.0),      # k == E
])
def test_router_topk_parity(tl, T, H, E, k, rsf):
    torch, moe = tl
    gh.note(f"router T={T} H={H} E={E} k={k}")
    rng = np.random.default_rng(T + E)
    x = moe_inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    p = moe.make_params(T, H, E, k, 8, 0, rsf, 7.0)
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(p, gh.dev_bf16(torch, x), gh.dev_f32(torch, wr), gh.dev_f32(torch, b),
                        ids, w, ws)
    torch.cuda.synchronize()
    ids_g, w_g = ids.cpu().numpy(), w.cpu().numpy()
    logits_g = ws[: T * E * 4].view(torch.float32).cpu().numpy().reshape(T, E)
    rep = gh.check_router(x, wr, b, k, rsf, logits_g, ids_g, w_g)
    rep.pop("route")
    gh.note(f"  {rep}")


@pytest.mark.parametrize("T,H,E", [(64, 4096, 64), (700, 4096, 256), (37, 520, 24)])
def test_router_logits_one_hot_exact(tl, T, H, E):
    """With one-hot activations (one entry +-2^j per token) each logit is a
    single product, and the three bf16 pieces of an fp32 router weight add
    up to it exactly in fp32 (8 + 8 + 8 significant bits): the GPU must
    return +-2^j * W_r[e, i_t] bit for bit, whatever the K slicing and
    summation order.  A piece left out of the split -- the lowest carries
    bits 17..24 of each weight -- changes these bits, which the forward-error
    bound of the general test is too wide to see."""
    torch, moe = tl
    gh.note(f"router one-hot T={T} H={H} E={E}")
    rng = np.random.default_rng(T * 7 + E)
    pos = rng.integers(0, H, T)
    val = rng.choice([-1.0, 1.0], T) * np.ldexp(1.0, rng.integers(-3, 4, T))
    xv = np.zeros((T, H), np.float32)
    xv[np.arange(T), pos] = val
    x = moe_inputs.f32_to_bf16_bits(xv)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    k = min(8, E)
    p = moe.make_params(T, H, E, k, 8, 0, 1.0, 7.0)
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(p, gh.dev_bf16(torch, x), gh.dev_f32(torch, wr), None, ids, w, ws)
    torch.cuda.synchronize()
    logits_g = ws[: T * E * 4].view(torch.float32).cpu().numpy().reshape(T, E)
    want = (val[:, None] * wr[:, pos].T.astype(np.float64)).astype(np.float32)
    assert np.array_equal(want.astype(np.float64), val[:, None] * wr[:, pos].T.astype(np.float64))
    bad = np.argwhere(logits_g.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, f"{len(bad)} logits differ, first {bad[:4]}"


def test_router_ties_nan_and_no_bias(tl):
    """Exact ties (identical router rows) go to the lower id; a NaN logit
    ranks last; NULL bias means zeros."""
    torch, moe = tl
    T, H, E, k = 40, 64, 12, 3
    rng = np.random.default_rng(0)
    x = moe_inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    wr[5] = wr[2]
    wr[9] = wr[2]           # experts 2, 5, 9 always tie
    wr[7] = np.nan          # expert 7's logit is NaN for every token
    p = moe.make_params(T, H, E, k, 8, 0, 1.0, 7.0)
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(p, gh.dev_bf16(torch, x), gh.dev_f32(torch, wr), None, ids, w, ws)
    torch.cuda.synchronize()
    r = mo.topk_route(mo.router_logits(x, wr), None, k, 1.0)
    np.testing.assert_array_equal(ids.cpu().numpy(), r["ids"])
    assert not np.any(ids.cpu().numpy() == 7)
    logits_g = ws[: T * E * 4].view(torch.float32).cpu().numpy().reshape(T, E)
    assert np.all(logits_g[:, 2] == logits_g[:, 5]) and np.all(logits_g[:, 2] == logits_g[:, 9])
    assert np.all(np.isnan(logits_g[:, 7]))


TIED = [3, 20, 40, 50, 63, 64, 70, 77, 90, 99]


@pytest.mark.parametrize("case", ["nan_majority", "all_equal", "ties_across_halves"])
def test_router_selection_edges(tl, case):
    """Selections decided at the k-th score: more NaN logits than E - k (the
    threshold falls to NaN, whose experts then go by lowest id), every
    expert tied (ids 0..k-1), and ties at the k-th score that span both
    halves of a 100-expert lane layout; against the oracle's selection, with
    the separate top-k kernel and the fused decode routing."""
    torch, moe = tl
    rng = np.random.default_rng(11)
    T, H = 24, 64
    E, k = (12, 5) if case == "nan_majority" else (100, 8)
    x = moe_inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    bias = (rng.uniform(-0.1, 0.1, E)).astype(np.float32)
    if case == "nan_majority":
        wr[[0, 1, 3, 4, 6, 7, 8, 10, 11]] = np.nan   # 3 finite experts, k = 5
    elif case == "all_equal":
        wr[:] = wr[0]
        bias[:] = 0.0
    else:
        # ten experts share the best row and bias: the picks are the eight
        # lowest ids among them, across both 64-expert halves
        for e in TIED:
            wr[e] = wr[3]
            bias[e] = 0.5
    r = mo.topk_route(mo.router_logits(x, wr), bias, k, 1.0)
    p = moe.make_params(T, H, E, k, 8, 0, 1.0, 7.0)
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(p, gh.dev_bf16(torch, x), gh.dev_f32(torch, wr), gh.dev_f32(torch, bias),
                        ids, w, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), r["ids"])
    if case == "all_equal":
        np.testing.assert_array_equal(r["ids"], np.tile(np.arange(k), (T, 1)))
    if case == "nan_majority":
        assert np.all(np.isin([2, 5, 9], r["ids"]))
    if case == "ties_across_halves":
        np.testing.assert_array_equal(r["ids"], np.tile(TIED[:k], (T, 1)))
    # the fused decode routing (top-k and permutation in one launch)
    d = gh.Device(moe_inputs.Workload("edge", T=T, H=H, E=E, k=k, I=128, I_s=0),
                  dict(x=x, w_router=wr, corr_bias=bias, w_gate_up=np.zeros((E, 256, H), np.uint16),
                       w_down=np.zeros((E, H, 128), np.uint16), gamma_pre=None, gamma_post=None,
                       x_cur=None, ws_gate_up=None, ws_down=None))
    d.run()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d.result()["ids"], r["ids"])


@pytest.mark.parametrize("T,H,E,k", [
    (32, 4096, 64, 8),     # the decode workload's routing
    (64, 128, 8, 2),       # tiny
    (64, 256, 256, 8),     # T * E at the LDS bound, four experts per lane
    (16, 520, 1024, 16),   # E and k at their bounds, ragged K
    (1, 64, 3, 3),         # one token, k == E
])
def test_fused_routing_matches_separate_calls(tl, T, H, E, k):
    """moe_forward routes decode-sized batches with one kernel after the
    router GEMM (partials summed into LDS, wave top-k over the LDS logits,
    permutation, GEMM schedule); its ids, weights, logits and permutation
    equal those of moe_router_topk followed by moe_permute bit for bit."""
    torch, moe = tl
    gh.note(f"fused routing T={T} H={H} E={E} k={k}")
    wl = moe_inputs.Workload("route", T=T, H=H, E=E, k=k, I=64, I_s=0, rsf=1.5)
    inp = moe_inputs.generate(wl, seed=T + E)
    d = gh.Device(wl, inp)
    d.canary()
    d.run()
    g = d.result()
    p = d.params
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(p, d.x, d.w_router, d.corr_bias, ids, w, ws)
    logits = ws[: T * E * 4].view(torch.float32).clone()
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    st = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ip = torch.empty(T * k, dtype=torch.int32, device="cuda")
    moe.moe_permute(p, ids, offs, st, ip, ws)
    torch.cuda.synchronize()
    assert np.array_equal(g["ids"], ids.cpu().numpy())
    assert np.array_equal(g["w"].view(np.uint32), w.cpu().numpy().view(np.uint32))
    assert np.array_equal(g["logits"].view(np.uint32),
                          logits.cpu().numpy().reshape(T, E).view(np.uint32))
    assert np.array_equal(g["offsets"], offs.cpu().numpy())
    assert np.array_equal(g["sorted_token"], st.cpu().numpy())
    assert np.array_equal(g["inv_pos"], ip.cpu().numpy())


# ----------------------------------------------------------- permute ----

@pytest.mark.parametrize("T,E,k,skew", [
    (1, 1, 1, 0.0),
    (37, 8, 2, 0.0),
    (1500, 64, 8, 0.0),       # 12000 pairs: three permute tiles
    (600, 1024, 16, 0.0),     # E and k at their bounds
    (5000, 256, 8, 3.0),      # heavy skew: few experts take most pairs
    (700, 100, 4, 50.0),      # extreme skew: most experts empty
])
def test_permute_parity(tl, T, E, k, skew):
    torch, moe = tl
    gh.note(f"permute T={T} E={E} k={k}")
    rng = np.random.default_rng(T * 3 + E)
    prob = np.exp(-skew * np.arange(E) / E)
    prob /= prob.sum()
    ids = np.stack([np.sort(rng.choice(E, size=k, replace=False, p=prob)) for _ in range(T)]).astype(np.int32)
    H = 24 if T > 1000 else 136   # the optional gather: ragged row widths (16-byte chunks)
    p = moe.make_params(T, H, E, k, 8, 0, 1.0, 7.0)
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda")
    off = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
    st = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
    inv = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
    x = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
    xp = torch.full((T * k, H), -1, dtype=torch.int16, device="cuda")
    moe.moe_permute(p, torch.from_numpy(ids).cuda(), off, st, inv, ws, x=gh.dev_bf16(torch, x),
                    x_perm=xp)
    torch.cuda.synchronize()
    ref = mo.permute(ids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(st.cpu().numpy(), ref["sorted_token"])
    np.testing.assert_array_equal(inv.cpu().numpy(), ref["inv_pos"])
    # gathered rows are byte copies of the oracle's permuted rows
    np.testing.assert_array_equal(gh.to_bits(xp), x[ref["sorted_token"]])
    # without x / x_perm nothing is gathered (and the sort is the same)
    st.fill_(-1)
    moe.moe_permute(p, torch.from_numpy(ids).cuda(), off, st, inv, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.cpu().numpy(), ref["sorted_token"])


# ------------------------------------------------------ grouped GEMM ----

@pytest.mark.parametrize("counts,H,I,std", [
    ([3], 64, 8, 0.05),                                  # one tiny group
    ([0, 5, 0, 1, 130, 0, 7], 136, 264, 0.05),          # empty groups, ragged M/N/K
    ([257, 128, 1, 300], 520, 136, 0.05),               # several m-tiles per group
    ([40] * 12, 256, 384, 0.3),                          # clamp stress: |g|,|u| past L
    ([2, 3, 4, 1] * 16, 512, 1408, 0.02),                # short groups (weight streaming tiles)
])
def test_grouped_swiglu_gemm_parity(tl, counts, H, I, std):
    check_grouped_gemm(tl, counts, H, I, std)


@pytest.mark.parametrize("counts,H,I", [
    # the 256-row ping-pong tile with every kind of last m-tile: exactly 128
    # rows and 1 row (half-height), 129 and 256 rows (full), 384 = 256 + 128
    # and 640 = 2 x 256 + 128 (full tiles, then a half-height one), an empty
    # group; K = 512 / 384 (both >= 256), down N = 512 (two column tiles)
    ([128, 129, 1, 384, 0, 640, 256, 513], 512, 384),
    # K = 256 in down (the shortest the tile takes)
    ([130, 100, 700], 288, 256),
    # K = 256 in gate_up, and a ragged gate_up N (288: a last column tile
    # with 32 of its 128 columns)
    ([130, 100, 700], 256, 288),
])
def test_grouped_gemm_pingpong_tiles(tl, counts, H, I, monkeypatch):
    """The ping-pong tile forced on groups whose last m-tiles are full or
    half-height (at most 128 rows), against the same forward-error bounds."""
    monkeypatch.setenv("MOE_GEMM_VARIANT", "pingpong")
    check_grouped_gemm(tl, counts, H, I, 0.05)


def check_grouped_gemm(tl, counts, H, I, std):
    torch, moe = tl
    gh.note(f"grouped gemm counts={counts[:8]} H={H} I={I}")
    rng = np.random.default_rng(sum(counts) + H + I)
    G = len(counts)
    M = int(sum(counts))
    rows_a = max(M // 2, 1) + 3
    a = moe_inputs.f32_to_bf16_bits(rng.standard_normal((rows_a, H)).astype(np.float32))
    row_index = rng.integers(0, rows_a, M).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    wgu = moe_inputs.f32_to_bf16_bits((rng.standard_normal((G, 2 * I, H)) * std).astype(np.float32))
    wd = moe_inputs.f32_to_bf16_bits((rng.standard_normal((G, H, I)) * std).astype(np.float32))
    L = 7.0
    h = torch.full((M, I), 0x7FC0, dtype=torch.int16, device="cuda")
    y = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_grouped_gemm_workspace_size(G, M, H, I), dtype=torch.uint8, device="cuda")
    moe.moe_grouped_swiglu_gemm(G, M, H, I, L, gh.dev_bf16(torch, a), torch.from_numpy(row_index).cuda(),
                                torch.from_numpy(offsets).cuda(), gh.dev_bf16(torch, wgu),
                                gh.dev_bf16(torch, wd), h, y, ws)
    torch.cuda.synchronize()
    h_g = mo.bf16_to_f64(gh.to_bits(h))
    y_g = y.cpu().numpy().astype(np.float64)
    u32 = 2.0 ** -24
    for g in range(G):
        sl = slice(offsets[g], offsets[g + 1])
        if offsets[g] == offsets[g + 1]:
            continue
        A = mo.bf16_to_f64(a[row_index[sl]])
        Wg_, Wu_ = mo.bf16_to_f64(wgu[g][:I]), mo.bf16_to_f64(wgu[g][I:])
        gg, uu = A @ Wg_.T, A @ Wu_.T
        gc, uc = np.minimum(gg, L), np.clip(uu, -L, L)
        h_ref = gc / (1 + np.exp(-gc)) * uc
        # forward-error bound: fp32 sums of H products, |silu'| <= 1.1, then
        # one bf16 rounding (half an ulp is at most 2^-8 of the value)
        eg = H * u32 * (np.abs(A) @ np.abs(Wg_).T)
        eu = H * u32 * (np.abs(A) @ np.abs(Wu_).T)
        bound = 1.1 * np.abs(uc) * eg + np.abs(gc / (1 + np.exp(-gc))) * eu
        # (+ a few fp32 ulps for evaluating silu and the product)
        bound = bound + 2.0 ** -8 * (np.abs(h_ref) + bound) + 1e-6 * np.abs(h_ref) + 1e-30
        assert np.all(np.abs(h_g[sl] - h_ref) <= bound), f"group {g}: h"
        # y from the GPU's own h: fp32 sums of I products
        Wd_ = mo.bf16_to_f64(wd[g])
        y_ref = h_g[sl] @ Wd_.T
        ey = I * u32 * (np.abs(h_g[sl]) @ np.abs(Wd_).T) + 1e-30
        assert np.all(np.abs(y_g[sl] - y_ref) <= ey), f"group {g}: y"
    if std >= 0.3:   # the clamp stress case really hit both clamps
        A = mo.bf16_to_f64(a[row_index])
        gg = A[: offsets[1]] @ mo.bf16_to_f64(wgu[0][:I]).T
        assert (gg > L).any() and (gg < -L).any()


# ----------------------------------------------------------- combine ----

@pytest.mark.parametrize("T,H,k,shared,post", [
    (1, 8, 1, False, False),
    (77, 136, 3, True, False),
    (300, 1024, 8, True, False),
    (50, 520, 4, True, True),        # ScMoE post-norm
    (20, 8192, 16, False, True),     # post-norm at its H bound
])
def test_combine_parity(tl, T, H, k, shared, post):
    torch, moe = tl
    gh.note(f"combine T={T} H={H} k={k} shared={shared} post={post}")
    rng = np.random.default_rng(T + H)
    N = T * k
    y = (rng.standard_normal((N, H)) * 3).astype(np.float32)
    w = rng.uniform(0, 2.5, (T, k)).astype(np.float32)
    inv = rng.permutation(N).astype(np.int32)
    ys = (rng.standard_normal((T, H)) * 2).astype(np.float32) if shared else None
    gamma = rng.uniform(0.9, 1.1, H).astype(np.float32) if post else None
    p = moe.make_params(T, H, 16, k, 8, 8 if shared else 0, 1.0, 7.0, scmoe=post, norm_eps=1e-6)
    out = torch.full((T, H), 0x7FC0, dtype=torch.int16, device="cuda")
    moe.moe_combine(p, gh.dev_f32(torch, y), gh.dev_f32(torch, w), torch.from_numpy(inv).cuda(),
                    None if ys is None else gh.dev_f32(torch, ys),
                    None if gamma is None else gh.dev_f32(torch, gamma), out)
    torch.cuda.synchronize()
    z = mo.combine(y.astype(np.float64), w, inv, None if ys is None else ys.astype(np.float64))
    ref = mo.bf16_to_f64(mo.bf16_round(mo.rmsnorm_f64(z, gamma, 1e-6) if post else z))
    got = mo.bf16_to_f64(gh.to_bits(out))
    d = np.abs(got - ref) / (gh.OUT_TOL * np.maximum(1, np.abs(ref)))
    assert d.max() <= 1.0
    # fp32 accumulation of at most 17 terms: almost every element rounds the same
    assert np.mean(got == ref) > 0.99


@pytest.mark.parametrize("post,in_place,c0,c1", [(False, False, 1.0, 1.0), (True, False, 0.6, 0.8),
                                                  (True, True, 1.0, 1.0), (False, True, 0.25, 1.5)])
def test_combine_finish_bits(tl, post, in_place, c0, c1):
    """moe_combine_finish = the finish of moe_combine's own output, bit for
    bit (the same kernel arithmetic, then S8), also in place."""
    torch, moe = tl
    T, H, k = 37, 1032, 5
    gh.note(f"combine_finish post={post} in_place={in_place} c=({c0},{c1})")
    rng = np.random.default_rng(41)
    N = T * k
    y = gh.dev_f32(torch, (rng.standard_normal((N, H)) * 3).astype(np.float32))
    w = gh.dev_f32(torch, rng.uniform(0, 2.5, (T, k)).astype(np.float32))
    inv = torch.from_numpy(rng.permutation(N).astype(np.int32)).cuda()
    ys = gh.dev_f32(torch, (rng.standard_normal((T, H)) * 2).astype(np.float32))
    gamma = gh.dev_f32(torch, rng.uniform(0.9, 1.1, H).astype(np.float32))
    res = moe_inputs.f32_to_bf16_bits((rng.standard_normal((T, H)) * 4).astype(np.float32))
    p_plain = moe.make_params(T, H, 16, k, 8, 8, 1.0, 7.0, scmoe=False, norm_eps=1e-6)
    p_o = moe.make_params(T, H, 16, k, 8, 8, 1.0, 7.0, scmoe=post, norm_eps=1e-6)
    o = torch.full((T, H), 0x7FC0, dtype=torch.int16, device="cuda")
    moe.moe_combine(p_o, y, w, inv, ys, gamma, o)
    r_dev = gh.dev_bf16(torch, res)
    out = r_dev if in_place else torch.full((T, H), 0x7FC0, dtype=torch.int16, device="cuda")
    moe.moe_combine_finish(p_plain, y, w, inv, ys, gamma, moe.make_finish(r_dev, c0, c1, post), out)
    torch.cuda.synchronize()
    want = mo.finish(gh.to_bits(o), res, c0, c1)
    assert np.array_equal(gh.to_bits(out), want)


# ------------------------------------------------- W4A16 dequantisation ----

@pytest.mark.parametrize("G,R,K,ts", [
    (3, 70, 384, None),     # no tensor scale: the exact expansion
    (2, 33, 256, "pow2"),   # power-of-two tensor scales: exact as well
    (2, 40, 256, "fp32"),   # arbitrary fp32 tensor scales: one rounding per weight
    (1, 1, 128, None),      # one row, one group
])
def test_w4_dequantize_bits(tl, G, R, K, ts):
    """moe_w4_dequantize = bf16 of the oracle's exact dequantisation (round to
    nearest even) over every E4M3 scale byte but the NaNs, bit for bit
    except the sign of zero weights (u = 8 under a negative scale: the
    oracle's 0 * (-s) is -0, the kernel's (128 + u) s - 136 s is +0);
    nothing is written past the output."""
    torch, moe = tl
    gh.note(f"w4_dequantize G={G} R={R} K={K} tscale={ts}")
    rng = np.random.default_rng(K + R)
    q = rng.integers(0, 256, size=(G, R, K // 2), dtype=np.uint8)
    sc = rng.integers(0, 254, size=(G, K // 128, R)).astype(np.uint8)
    sc = np.where(sc >= 0x7F, sc + 1, sc).astype(np.uint8)     # no NaN codes
    tsv = None
    if ts == "pow2":
        tsv = np.ldexp(1.0, rng.integers(-12, 3, size=G)).astype(np.float32)
    elif ts == "fp32":
        tsv = rng.uniform(1e-3, 3e-3, size=G).astype(np.float32)
    want = np.stack([mo.bf16_round(mo.dequant_w4(q[g], sc[g], 1.0 if tsv is None else tsv[g]))
                     for g in range(G)])
    q_d = torch.from_numpy(q).cuda()
    sc_d = torch.from_numpy(sc).cuda()
    ts_d = None if tsv is None else gh.dev_f32(torch, tsv)
    pad = 1024
    buf = torch.full((G * R * K + pad,), 0x7FC0, dtype=torch.int16, device="cuda")
    moe.moe_w4_dequantize(q_d, sc_d, buf, G, R, K, tscale=ts_d)
    torch.cuda.synchronize()
    got = gh.to_bits(buf)
    got_w = got[:G * R * K].reshape(G, R, K)
    assert np.array_equal(mo.bf16_to_f64(got_w), mo.bf16_to_f64(want))
    nz = mo.bf16_to_f64(want) != 0
    assert np.array_equal(got_w[nz], want[nz]) and np.all(got_w[~nz] == 0)
    assert np.all(got[G * R * K:] == 0x7FC0)
