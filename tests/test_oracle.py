"""Pins for the CPU oracle, checked against things other than the oracle itself.

Each test ties one part of the oracle to an independent fact: a library routine in a special
case (dense attention = torch's scaled_dot_product_attention in float64 with autograd), float64
finite differences of the forward, closed forms, invariants of the softmax gradient, exact zeros
that the FastVideo backward test page requires, and small hand-worked metadata fixtures.
"""
import dataclasses
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import workloads
from oracle import vsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BLOCK = 64


def _case(nb=4, topk=2, H=1, B=1, seed=0, vbs=None, kv_pool=None, scale=1.0):
    return workloads.make_case(B, H, nb, topk, seed=seed, vbs=vbs, kv_pool=kv_pool, scale=scale)


def _mask_torch(c):
    """Boolean [B,H,S,S] keep mask built with torch ops, independently of the oracle: a
    block-level selection table, expanded to tokens, and a key-column mask from vbs."""
    B, H, nb = c.B, c.H, c.nb
    blk = torch.zeros(B, H, nb, nb, dtype=torch.bool)
    for b, h, qb in itertools.product(range(B), range(H), range(nb)):
        for t in range(int(c.q2k_num[b, h, qb])):
            blk[b, h, qb, int(c.q2k_idx[b, h, qb, t])] = True
    tok = blk.repeat_interleave(BLOCK, dim=2).repeat_interleave(BLOCK, dim=3)
    col_ok = (torch.arange(nb * BLOCK) % BLOCK) < c.vbs.long().repeat_interleave(BLOCK)
    return tok & col_ok.view(1, 1, 1, -1)


def _sdpa_grads(c, mask=None):
    q, k, v = (t.to(torch.float64).requires_grad_(True) for t in (c.q, c.k, c.v))
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                           scale=c.sm_scale)
    loss = (out * c.do.to(torch.float64)).sum()
    dq, dk, dv = torch.autograd.grad(loss, (q, k, v))
    return out.detach().numpy(), dq.numpy(), dk.numpy(), dv.numpy()


def _close(a, b, tol=1e-10):
    scale = max(np.abs(b).max(), 1e-30)
    assert np.abs(a - b).max() <= tol * scale, (np.abs(a - b).max(), scale)


# ---------------------------------------------------------------------------------------------
# forward and backward against a library routine
# ---------------------------------------------------------------------------------------------

def test_dense_special_case_matches_sdpa():
    """All kv blocks selected, all blocks full: block-sparse attention is dense attention."""
    c = _case(nb=4, topk=4, H=2, seed=3)
    o, lse = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    ref_o, ref_dq, ref_dk, ref_dv = _sdpa_grads(c)
    _close(o, ref_o)
    s = c.sm_scale * np.einsum("bhid,bhjd->bhij", O.f64(c.q), O.f64(c.k))
    _close(lse, scipy.special.logsumexp(s, axis=-1) * O.LOG2E)
    dq, dk, dv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    _close(dq, ref_dq)
    _close(dk, ref_dk)
    _close(dv, ref_dv)


@pytest.mark.parametrize("seed", [0, 1])
def test_masked_ragged_matches_sdpa_with_mask(seed):
    """Partial selection, an unselected kv block and ragged vbs, against SDPA with a boolean
    mask built by torch ops (not by the oracle)."""
    vbs = [64, 37, 64, 50, 64, 1]
    c = _case(nb=6, topk=3, H=2, B=2, seed=seed, vbs=vbs, kv_pool=[0, 1, 2, 3, 5])
    mask = _mask_torch(c)
    o, lse = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    ref_o, ref_dq, ref_dk, ref_dv = _sdpa_grads(c, mask)
    _close(o, ref_o)
    dq, dk, dv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    _close(dq, ref_dq)
    _close(dk, ref_dk)
    _close(dv, ref_dv)
    # the literal dense mask of the page's reference agrees with the torch-built one
    assert np.array_equal(O.dense_keep_mask(c.q2k_idx, c.q2k_num, c.vbs, c.S), mask.numpy())


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 0.3])
def test_masked_ragged_any_scale_matches_sdpa(scale):
    """The masked ragged case at a negative, a zero and a large positive sm_scale (the scales the
    GPU tests use) against SDPA with the same scale and mask; lse against scipy's logsumexp of
    the masked scores."""
    c = _case(nb=6, topk=3, H=2, seed=5, vbs=[64, 37, 64, 50, 64, 1], kv_pool=[0, 1, 2, 3, 5])
    c = dataclasses.replace(c, sm_scale=scale)
    mask = _mask_torch(c)
    o, lse = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    ref_o, ref_dq, ref_dk, ref_dv = _sdpa_grads(c, mask)
    _close(o, ref_o)
    s = scale * np.einsum("bhid,bhjd->bhij", O.f64(c.q), O.f64(c.k))
    s = np.where(mask.numpy(), s, -np.inf)
    _close(lse, scipy.special.logsumexp(s, axis=-1) * O.LOG2E)
    dq, dk, dv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    _close(dv, ref_dv)
    if scale == 0.0:  # dq and dk carry the scale
        assert not dq.any() and not dk.any()
    else:
        _close(dq, ref_dq)
        _close(dk, ref_dk)


# ---------------------------------------------------------------------------------------------
# finite differences of the oracle's own forward (pins the gradient formulas)
# ---------------------------------------------------------------------------------------------

def _loss(c, q, k, v):
    o, _ = O.forward(q, k, v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    return float(np.sum(o * O.f64(c.do)))


def test_gradient_matches_central_differences():
    c = _case(nb=4, topk=2, seed=5, vbs=[64, 45, 64, 30])
    q, k, v = O.f64(c.q), O.f64(c.k), O.f64(c.v)
    dq, dk, dv = O.backward(q, k, v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    rng = np.random.default_rng(0)
    eps = 1e-4
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        gmax = np.abs(g).max()
        for _ in range(48):
            i = tuple(rng.integers(0, n) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args = {"q": q, "k": k, "v": v}
            fp = _loss(c, **{**args, name: xp})
            fm = _loss(c, **{**args, name: xm})
            fd = (fp - fm) / (2 * eps)
            assert abs(fd - g[i]) <= 1e-7 * gmax, (name, i, fd, g[i])
    # directional derivative along a random direction of all three inputs
    dirs = [rng.standard_normal(x.shape) for x in (q, k, v)]
    eps = 1e-5
    fp = _loss(c, q + eps * dirs[0], k + eps * dirs[1], v + eps * dirs[2])
    fm = _loss(c, q - eps * dirs[0], k - eps * dirs[1], v - eps * dirs[2])
    fd = (fp - fm) / (2 * eps)
    an = sum(np.sum(d * g) for d, g in zip(dirs, (dq, dk, dv)))
    assert abs(fd - an) <= 1e-7 * abs(an)


# ---------------------------------------------------------------------------------------------
# closed forms and special cases
# ---------------------------------------------------------------------------------------------

def test_zero_queries_give_uniform_attention():
    """q = 0: every kept key scores 0, so lse = log2(n) and o = the mean of the kept v rows."""
    vbs = [64, 20, 64, 7]
    c = _case(nb=4, topk=2, H=2, seed=7, vbs=vbs)
    q = torch.zeros_like(c.q)
    o, lse = O.forward(q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    V = O.f64(c.v)
    for h, qb in itertools.product(range(2), range(4)):
        blocks = sorted(set(int(x) for x in c.q2k_idx[0, h, qb, :int(c.q2k_num[0, h, qb])]))
        rows = np.concatenate([V[0, h, kb * 64:kb * 64 + vbs[kb]] for kb in blocks])
        n = rows.shape[0]
        assert np.allclose(lse[0, h, qb * 64:(qb + 1) * 64], np.log2(n), atol=1e-13)
        assert np.allclose(o[0, h, qb * 64:(qb + 1) * 64], rows.mean(axis=0)[None], atol=1e-13)


def test_single_valid_key_special_case():
    """vbs = 1 and top-k 1: each q row sees one key, so P = 1: o = that v row, dq = dk = 0,
    and dv of the key = sum of dO over the rows that see it."""
    c = _case(nb=4, topk=1, H=1, seed=2, vbs=[1, 1, 1, 1])
    o, lse = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    dq, dk, dv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    V, DO, Q, K = O.f64(c.v), O.f64(c.do), O.f64(c.q), O.f64(c.k)
    expect_dv = np.zeros_like(V)
    for qb in range(4):
        kb = int(c.q2k_idx[0, 0, qb, 0])
        assert np.array_equal(o[0, 0, qb * 64:(qb + 1) * 64], np.repeat(V[0, 0, kb * 64][None], 64, 0))
        s = c.sm_scale * Q[0, 0, qb * 64:(qb + 1) * 64] @ K[0, 0, kb * 64]
        assert np.allclose(lse[0, 0, qb * 64:(qb + 1) * 64], s * O.LOG2E, rtol=0, atol=1e-13)
        expect_dv[0, 0, kb * 64] += DO[0, 0, qb * 64:(qb + 1) * 64].sum(axis=0)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13
    assert np.allclose(dv, expect_dv, atol=1e-12)


def test_lse_bounds():
    """max_j s_ij log2e <= lse_i <= max_j s_ij log2e + log2(n_i)."""
    c = _case(nb=4, topk=3, H=1, seed=11, vbs=[64, 33, 64, 64])
    _, lse = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    Q, K = O.f64(c.q), O.f64(c.k)
    for qb in range(4):
        keys = O.kept_keys(c.q2k_idx, c.q2k_num, c.vbs, 0, 0, qb)
        s = c.sm_scale * Q[0, 0, qb * 64:(qb + 1) * 64] @ K[0, 0, keys].T * O.LOG2E
        m = s.max(axis=1)
        li = lse[0, 0, qb * 64:(qb + 1) * 64]
        assert np.all(li >= m - 1e-12) and np.all(li <= m + np.log2(keys.size) + 1e-12)


def test_gradient_invariants_and_exact_zeros():
    """dS rows sum to 0 (exact Delta), so per head sum_j dK_j = 0 and sum_j dV_j = sum of dO
    over rows that have keys; unselected kv blocks and padded kv rows get exactly 0
    (the page's zero-count and padded-row tests)."""
    c = workloads.config(2)
    dq, dk, dv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    DO = O.f64(c.do)
    for b, h in itertools.product(range(2), range(2)):
        assert np.abs(dk[b, h].sum(axis=0)).max() <= 1e-12 * max(1.0, np.abs(dk[b, h]).max())
        assert np.allclose(dv[b, h].sum(axis=0), DO[b, h].sum(axis=0), atol=1e-10)
    for kb in (4, 11):
        assert np.all(dk[:, :, kb * 64:(kb + 1) * 64] == 0)
        assert np.all(dv[:, :, kb * 64:(kb + 1) * 64] == 0)
    for kb, n in ((7, 50), (15, 37)):
        assert np.all(dk[:, :, kb * 64 + n:(kb + 1) * 64] == 0)
        assert np.all(dv[:, :, kb * 64 + n:(kb + 1) * 64] == 0)
        assert np.abs(dk[:, :, kb * 64:kb * 64 + n]).max() > 0


def test_empty_rows_reading():
    """A q block with no selection: o = 0, lse = -inf, dq = 0 (no key depends on it)."""
    c = _case(nb=4, topk=2, H=1, seed=4)
    c.q2k_num[0, 0, 2] = 0
    o, lse = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    dq, dk, dv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    assert np.all(o[0, 0, 128:192] == 0) and np.all(np.isneginf(lse[0, 0, 128:192]))
    assert np.all(dq[0, 0, 128:192] == 0)
    # removing the empty block's rows changes nothing else: compare with a case whose dO rows
    # there are zero (the loss then does not see them either)
    do2 = c.do.clone()
    do2[0, 0, 128:192] = 0
    _, dk2, dv2 = O.backward(c.q, c.k, c.v, do2, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def test_sampled_backward_matches_full():
    c = workloads.config(2)
    dq, dk, dv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    qbs = [(0, 0, 3), (1, 1, 15)]
    kbs = [(0, 1, 7), (1, 0, 15), (0, 0, 4)]
    sdq, sdkv = O.backward_sampled(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale,
                                   qblocks=qbs, kvblocks=kbs)
    for b, h, qb in qbs:
        _close(sdq[(b, h, qb)], dq[b, h, qb * 64:(qb + 1) * 64], 1e-13)
    for b, h, kb in kbs:
        assert np.allclose(sdkv[(b, h, kb)][0], dk[b, h, kb * 64:(kb + 1) * 64], atol=1e-13)
        assert np.allclose(sdkv[(b, h, kb)][1], dv[b, h, kb * 64:(kb + 1) * 64], atol=1e-13)


@pytest.mark.parametrize("precision,tol", [("float64", 1e-13), ("float32", 1e-5)])
def test_kvblock_backward_matches_full(precision, tol):
    """The per-kv-block gradient (used at sizes where the full backward is out of reach) equals
    the full backward's rows: ragged blocks, an unselected block, a block sharing q blocks with
    another requested one, in both precisions."""
    c = workloads.config(2)
    dq, dk, dv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    kbs = [(0, 1, 7), (1, 0, 15), (0, 0, 4), (1, 1, 0), (0, 1, 15), (0, 1, 3)]
    got = O.kvblock_backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale, kbs,
                             precision)
    assert sorted(got) == sorted(kbs)
    for (b, h, kb), (gk, gv) in got.items():
        rows = slice(kb * 64, (kb + 1) * 64)
        _close(gk, dk[b, h, rows], tol * np.abs(dk[b, h]).max() / max(np.abs(dk[b, h, rows]).max(), 1e-30))
        _close(gv, dv[b, h, rows], tol * np.abs(dv[b, h]).max() / max(np.abs(dv[b, h, rows]).max(), 1e-30))
    assert not got[(0, 0, 4)][0].any() and not got[(0, 0, 4)][1].any()   # selected by nobody
    assert not got[(1, 0, 15)][0][37:].any()                              # padded rows


# ---------------------------------------------------------------------------------------------
# rounding helper
# ---------------------------------------------------------------------------------------------

def test_bf16_rne_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 3e38, -3.4e38]])
    x32 = x.astype(np.float32).astype(np.float64)       # float32-representable inputs
    ref = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_rne(x32)
    assert np.array_equal(got, ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert O.bf16_rne(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert O.bf16_rne(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2 * 2.0 ** -7


# ---------------------------------------------------------------------------------------------
# metadata
# ---------------------------------------------------------------------------------------------

def test_invert_matches_hand_worked_fixture():
    with open(os.path.join(GOLDEN, "invert_tiny.json")) as f:
        g = json.load(f)
    idx, num = O.invert_indices(np.array(g["q2k_idx"]), np.array(g["q2k_num"]), g["nkv"])
    assert idx.tolist() == g["k2q_idx"] and num.tolist() == g["k2q_num"]


def _invert_by_scanning_rows(q2k_idx, q2k_num, nkv):
    """A second construction of the inversion, from the definition of a k2q row: walk the q
    blocks of each (b, h) in increasing order and append each one to the list of every kv block
    its counted q2k entries name, unless that list already ends with it (a repeated id). Lists
    built this way are ascending without any sorting; they are then written out zero-padded."""
    idx = np.asarray(q2k_idx, dtype=np.int64)
    num = np.asarray(q2k_num, dtype=np.int64)
    B, H, nq, _ = idx.shape
    out_idx = np.zeros((B, H, nkv, nq), dtype=np.int32)
    out_num = np.zeros((B, H, nkv), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            lists = {}
            for qb in range(nq):
                for kb in idx[b, h, qb, :num[b, h, qb]].tolist():
                    lst = lists.setdefault(kb, [])
                    if not lst or lst[-1] != qb:
                        lst.append(qb)
            for kb, lst in lists.items():
                out_num[b, h, kb] = len(lst)
                out_idx[b, h, kb, :len(lst)] = lst
    return out_idx, out_num


@pytest.mark.parametrize("n", [1, 2])
def test_invert_matches_row_scan_construction_and_invariants(n):
    c = workloads.config(n)
    idx, num = O.invert_indices(c.q2k_idx, c.q2k_num, c.nb)
    ridx, rnum = _invert_by_scanning_rows(c.q2k_idx, c.q2k_num, c.nb)
    assert np.array_equal(idx, ridx) and np.array_equal(num, rnum)
    assert int(num.sum()) == int(c.q2k_num.sum())
    B, H = c.B, c.H
    for b, h, qb in itertools.product(range(B), range(H), range(c.nb)):
        for t in range(int(c.q2k_num[b, h, qb])):
            kb = int(c.q2k_idx[b, h, qb, t])
            listed = idx[b, h, kb, :num[b, h, kb]].tolist()
            assert listed.count(qb) == 1 and listed == sorted(listed)
    if n == 2:
        assert np.all(num[:, :, 4] == 0) and np.all(num[:, :, 11] == 0)


def test_invert_row_scan_with_duplicates_and_rectangular_shape():
    """Repeated kv ids in a q2k row, counts below the row width (entries past a count are never
    read) and nq != nkv: both constructions agree."""
    g = torch.Generator().manual_seed(9)
    B, H, nq, nkv, K = 2, 3, 40, 70, 9
    idx = torch.randint(0, nkv, (B, H, nq, K), generator=g, dtype=torch.int32)
    idx[..., 1] = idx[..., 0]
    num = torch.randint(0, K + 1, (B, H, nq), generator=g, dtype=torch.int32)
    got = O.invert_indices(idx, num, nkv)
    want = _invert_by_scanning_rows(idx.numpy(), num.numpy(), nkv)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_delta_is_the_p_weighted_mean_of_dp():
    """Delta_i = rowsum(o_i * dO_i) equals sum_j P_ij dP_ij with dP = dO V^T, because o = P V.
    P here is torch's softmax of the masked scores (mask built by torch ops), o comes from
    SDPA; the oracle's delta() only sees o and dO. Ragged blocks, an unselected kv block."""
    c = _case(nb=6, topk=3, H=2, B=2, seed=13, vbs=[64, 37, 64, 50, 64, 1],
              kv_pool=[0, 1, 2, 3, 5])
    mask = _mask_torch(c)
    q, k, v, do = (t.to(torch.float64) for t in (c.q, c.k, c.v, c.do))
    s = c.sm_scale * q @ k.transpose(-1, -2)
    p = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1)
    dp = do @ v.transpose(-1, -2)
    want = (p * dp).sum(-1).numpy()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                         scale=c.sm_scale)
    got = O.delta(o, c.do)
    _close(got, want, 1e-12)
    # and it is what the oracle's own gradient subtracts: the dS row sums vanish with it
    ds = p * (dp - torch.from_numpy(got)[..., None])
    assert ds.sum(-1).abs().max().item() <= 1e-12 * max(1.0, ds.abs().max().item())


def test_gradient_with_delta_from_a_rounded_o():
    """The reference the GPU tests use where Delta comes from the bf16 o the backward is given: the
    exact gradient shifted by delta_i = rowsum((bf16(o) - o) * dO)_i, dq_i by -sm_scale delta_i
    (P K)_i and dk_j by -sm_scale (P^T (delta * q))_j (from oracle calls: a forward with v := k, a
    backward with dO := delta * q), equals the gradient computed directly with that Delta from
    torch's softmax of the masked scores. Scores 64x larger than N(0,1) make the rows nearly
    one-hot, where the shift is largest."""
    c = _case(nb=6, topk=3, H=2, B=1, seed=17, vbs=[64, 37, 64, 50, 64, 1],
              kv_pool=[0, 1, 2, 3, 5])
    c.q = (c.q.float() * 8).to(torch.bfloat16)
    c.k = (c.k.float() * 8).to(torch.bfloat16)
    ro, _ = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    o16 = O.bf16_rne(ro)
    rdq, rdk, rdv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    do = c.do.double().numpy()
    delta = ((o16 - ro) * do).sum(-1, keepdims=True)
    pk, _ = O.forward(c.q, c.k, c.k, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    _, _, ptdq = O.backward(c.q, c.k, c.v, torch.from_numpy(delta * c.q.double().numpy()),
                            c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    got_dq = rdq - c.sm_scale * delta * pk
    got_dk = rdk - c.sm_scale * ptdq
    mask = _mask_torch(c)
    q, k, v, dO = (t.to(torch.float64) for t in (c.q, c.k, c.v, c.do))
    s_ = c.sm_scale * q @ k.transpose(-1, -2)
    p = torch.softmax(s_.masked_fill(~mask, float("-inf")), dim=-1)
    dp = dO @ v.transpose(-1, -2)
    d16 = (torch.from_numpy(o16) * dO).sum(-1, keepdim=True)
    ds = p * (dp - d16)
    want_dq = (c.sm_scale * ds @ k).numpy()
    want_dk = (c.sm_scale * ds.transpose(-1, -2) @ q).numpy()
    _close(got_dq, want_dq, 1e-12)
    _close(got_dk, want_dk, 1e-12)
    # the shift is not negligible here (so the test can see a wrong sign or a dropped term)
    assert np.abs(want_dq - rdq).max() > 1e-4 * np.abs(rdq).max()


def test_work_order_matches_hand_worked_fixture_and_invariants():
    with open(os.path.join(GOLDEN, "order_tiny.json")) as f:
        g = json.load(f)
    got = O.work_order(np.array(g["k2q_num"]), g["bin_width"])
    assert got.tolist() == g["order"]
    rng = np.random.default_rng(3)
    num = rng.integers(0, 200, size=(2, 3, 1024))
    order = O.work_order(num, 8)
    nb = 1024
    for bh in range(6):
        seg = order[bh * nb:(bh + 1) * nb] - bh * nb
        assert sorted(seg.tolist()) == list(range(nb))                 # a permutation of its head
        bins = num.reshape(6, nb)[bh][seg] // 8
        assert np.all(np.diff(bins) <= 0)                               # longest bin first
        same = np.diff(bins) == 0
        assert np.all(np.diff(seg)[same] > 0)                           # ascending kv in a bin


def test_workloads_are_reproducible_and_shaped():
    a, b = workloads.config(2), workloads.config(2)
    for x, y in ((a.q, b.q), (a.q2k_idx, b.q2k_idx), (a.q2k_num, b.q2k_num)):
        assert torch.equal(x, y)
    assert a.q.dtype == torch.bfloat16 and a.q.shape == (2, 2, 1024, 128)
    assert set(a.q2k_num.unique().tolist()) <= {1, 2, 3, 5, 7}
    assert a.vbs[7] == 50 and a.vbs[15] == 37
    sel = O.selection(a.q2k_idx, a.q2k_num, 16)
    assert not sel[..., 4].any() and not sel[..., 11].any()
    # distinct selections per row
    for b, h, qb in itertools.product(range(2), range(2), range(16)):
        row = a.q2k_idx[b, h, qb, :int(a.q2k_num[b, h, qb])].tolist()
        assert len(set(row)) == len(row) and row == sorted(row)
