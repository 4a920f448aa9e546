"""GPU parity tests: the HIP path through the C ABI against the float64 CPU oracle.

Gates (per tensor):
  * index metadata (k2q lists and counts, work order): bit-exact;
  * gradients and o: max|gpu - ref| / max|ref| <= 1e-2, and mean|gpu - ref| <= 1e-3 * mean|ref|
    beyond the irreducible rounding of the bf16 outputs, i.e.
    mean|gpu - ref| <= 1e-3 * mean|ref| + mean|bf16(ref) - ref|  (ref = unrounded oracle);
    the absolute mean of the FastVideo test page (mean|diff| <= 1e-3) is reported too;
  * o (the forward's output): the same two bounds;
  * lse: max|gpu - ref| <= 1e-4 (absolute, base-2 units);
  * exact zeros where the method defines them (unselected kv blocks, padded kv rows, empty q rows).
Small workloads are compared in full; the 32k and 65k-token workloads on sampled blocks, each
computed by the oracle one block at a time, plus invariants that hold at any size.
"""
import dataclasses
import itertools
import copy
import json

import numpy as np
import pytest
import torch

import block_sparse_attention_attn_amd as V
import workloads
from oracle import vsa_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

REL_MAX_TOL = 1e-2
MEAN_REL_TOL = 1e-3
LSE_ABS_TOL = 1e-4


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert V.is_built(), "libvsa.so must be built before the GPU tests"
    V.lib()


def to_dev(c):
    return {n: getattr(c, n).to(DEV) for n in ("q", "k", "v", "do", "q2k_idx", "q2k_num", "vbs")}


def nan_like(t):
    out = torch.empty_like(t)
    if out.dtype.is_floating_point:
        out.fill_(float("nan"))
    else:
        out.fill_(-7)
    return out


def check_close(name, got, ref, report=None):
    """got: GPU tensor (any float dtype); ref: float64 numpy array of the same shape.

    Three gates on every tensor: max|diff|/max|ref| <= 1e-2; mean|diff| <= 1e-3 mean|ref| plus
    the mean error of rounding the exact result to bf16 (which no bf16 output can avoid); and the
    strict form of the mean bound, measured against the bf16-rounded exact result:
    mean|got - bf16(ref)| <= 1e-3 mean|ref|.
    """
    g = got.detach().to("cpu", torch.float64).numpy()
    assert g.shape == ref.shape, f"{name}: shape {g.shape} vs {ref.shape}"
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    diff = np.abs(g - ref)
    max_ref = max(np.abs(ref).max(), 1e-30)
    mean_ref = np.abs(ref).mean()
    rel_max = diff.max() / max_ref
    mean_abs = diff.mean()
    rounded = O.bf16_rne(ref)
    rounding = np.abs(rounded - ref).mean()
    strict = np.abs(g - rounded).mean()
    line = dict(tensor=name, rel_max=float(rel_max), mean_abs=float(mean_abs),
                mean_ref=float(mean_ref), mean_rel=float(mean_abs / max(mean_ref, 1e-30)),
                mean_rel_vs_bf16_ref=float(strict / max(mean_ref, 1e-30)),
                page_abs_mean_ok=bool(mean_abs <= 1e-3))
    say("  " + json.dumps(line))
    if report is not None:
        report.append(line)
    assert rel_max <= REL_MAX_TOL, f"{name}: max|diff|/max|ref| = {rel_max:.3e}"
    assert mean_abs <= MEAN_REL_TOL * mean_ref + rounding, (
        f"{name}: mean|diff| = {mean_abs:.3e} > 1e-3*mean|ref| ({mean_ref:.3e}) + bf16 rounding "
        f"{rounding:.3e}")
    assert strict <= MEAN_REL_TOL * mean_ref, (
        f"{name}: mean|got - bf16(ref)| = {strict:.3e} > 1e-3*mean|ref| ({mean_ref:.3e})")


# -----------------------------------------------------------------------------------------------
# invert_indices (bit-exact)
# -----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_invert_bit_exact(n):
    c = workloads.config(n)
    say(f"[invert] config {n}")
    d = to_dev(c)
    out = (nan_like(torch.empty(c.B, c.H, c.nb, c.nb, dtype=torch.int32, device=DEV)),
           nan_like(torch.empty(c.B, c.H, c.nb, dtype=torch.int32, device=DEV)))
    k2q_idx, k2q_num = V.invert_indices(d["q2k_idx"], d["q2k_num"], c.nb, out=out)
    torch.cuda.synchronize()
    ridx, rnum = O.invert_indices(c.q2k_idx, c.q2k_num, c.nb)
    assert np.array_equal(k2q_num.cpu().numpy(), rnum)
    assert np.array_equal(k2q_idx.cpu().numpy(), ridx)


def test_invert_duplicates_counts_and_rectangular():
    """Duplicate kv ids count once; counts below the row width; nq != nkv."""
    g = torch.Generator().manual_seed(9)
    B, H, nq, nkv, K = 2, 3, 40, 70, 9
    idx = torch.randint(0, nkv, (B, H, nq, K), generator=g, dtype=torch.int32)
    idx[..., 1] = idx[..., 0]  # duplicates
    num = torch.randint(0, K + 1, (B, H, nq), generator=g, dtype=torch.int32)
    say("[invert] duplicates / rectangular")
    k2q_idx, k2q_num = V.invert_indices(idx.to(DEV), num.to(DEV), nkv)
    torch.cuda.synchronize()
    ridx, rnum = O.invert_indices(idx, num, nkv)
    assert np.array_equal(k2q_num.cpu().numpy(), rnum)
    assert np.array_equal(k2q_idx.cpu().numpy(), ridx)


@pytest.mark.parametrize("B,H,nq,nkv,K", [(1, 2, 3000, 50, 20), (1, 1, 70, 16384, 9),
                                         (1, 2, 40, 20000, 6)])
def test_invert_wide_shapes(B, H, nq, nkv, K):
    """Rows of more than 64 bitmap words (nq = 3000: the compaction takes its words in several
    passes), the largest LDS column (nkv = 16384: 64 KiB), and more kv blocks than one LDS column
    holds (nkv = 20000: the bitmap is set with global atomics instead)."""
    g = torch.Generator().manual_seed(nq + nkv)
    idx = torch.randint(0, nkv, (B, H, nq, K), generator=g, dtype=torch.int32)
    num = torch.randint(0, K + 1, (B, H, nq), generator=g, dtype=torch.int32)
    say(f"[invert] nq={nq} nkv={nkv}")
    k2q_idx, k2q_num = V.invert_indices(idx.to(DEV), num.to(DEV), nkv)
    torch.cuda.synchronize()
    ridx, rnum = O.invert_indices(idx, num, nkv)
    assert np.array_equal(k2q_num.cpu().numpy(), rnum)
    assert np.array_equal(k2q_idx.cpu().numpy(), ridx)


# -----------------------------------------------------------------------------------------------
# work order (bit-exact)
# -----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,H,nb,bw", [(1, 8, 1024, 8), (2, 3, 3000, 12), (1, 2, 16384, 8),
                                       (1, 1, 5, 8)])
def test_order_bit_exact(B, H, nb, bw):
    g = torch.Generator().manual_seed(nb)
    num = torch.randint(0, 300, (B, H, nb), generator=g, dtype=torch.int32)
    say(f"[order] B={B} H={H} nb={nb} bin={bw}")
    got = V.bwd_order(num.to(DEV), bw)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), O.work_order(num, bw))


# -----------------------------------------------------------------------------------------------
# forward
# -----------------------------------------------------------------------------------------------

def _fwd_compare(c, d, o, lse, qblocks=None):
    ro, rl = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale, qblocks=qblocks)
    if qblocks is None:
        check_close("o", o, ro)
        got_l = lse.cpu().double().numpy()
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(got_l), fin)
        assert np.all(got_l[~fin] == rl[~fin])
        assert np.abs(got_l[fin] - rl[fin]).max() <= LSE_ABS_TOL
    else:
        for b, h, qb in qblocks:
            rows = slice(qb * 64, (qb + 1) * 64)
            check_close(f"o[{b},{h},{qb}]", o[b, h, rows], ro[b, h, rows])
            assert np.abs(lse[b, h, rows].cpu().double().numpy() - rl[b, h, rows]).max() <= LSE_ABS_TOL


@pytest.mark.parametrize("n", [1, 2])
def test_forward_parity(n):
    c = workloads.config(n)
    d = to_dev(c)
    say(f"[forward] config {n}")
    o = nan_like(d["q"])
    lse = nan_like(torch.empty(c.B, c.H, c.S, dtype=torch.float32, device=DEV))
    V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"], out=(o, lse))
    torch.cuda.synchronize()
    _fwd_compare(c, d, o, lse)


@pytest.mark.parametrize("case,chunk,shuffle", [(2, 3, False), (2, 1, False), (2, 5, True),
                                                ("odd_blocks_ragged", 2, False),
                                                ("empty_q_blocks", 4, True),
                                                ("pool_excludes_three", 5, False)])
def test_forward_kv_range_chunks(case, chunk, shuffle):
    """The forward in kv-range chunks (kv_chunk_blocks): each wave's running O, max and sum pass
    from launch to launch in fp32, and each launch takes a contiguous run of list positions, so o
    and lse are bit-identical to one launch, also for lists in no particular order (shuffled)."""
    if case == 2:
        c = workloads.config(2)
    else:
        B, H, nb, topk, vbs, pool, empty = EDGE_CASES[case]
        c = workloads.make_case(B, H, nb, topk, seed=17, vbs=vbs, kv_pool=pool, name=case)
        for b, h, qb in empty:
            c.q2k_num[b, h, qb] = 0
    d = to_dev(c)
    idx = d["q2k_idx"]
    if shuffle:
        g = torch.Generator().manual_seed(3)
        perm = torch.stack([torch.randperm(idx.shape[-1], generator=g)
                            for _ in range(idx.numel() // idx.shape[-1])])
        rows = c.q2k_idx.reshape(-1, idx.shape[-1])
        nums = c.q2k_num.reshape(-1)
        sh = rows.clone()
        for i in range(rows.shape[0]):  # permute the valid prefix of each row
            k = int(nums[i])
            sh[i, :k] = rows[i, :k][perm[i][perm[i] < k]]
        idx = sh.reshape(idx.shape).to(DEV)
    say(f"[forward] {case}, kv-range chunks of {chunk} kv blocks, shuffled {shuffle}")
    one = V.forward(d["q"], d["k"], d["v"], idx, d["q2k_num"], d["vbs"], kv_chunk_blocks=-1)
    assert V.fwd_workspace_bytes(c.B, c.H, c.S, chunk) > 0
    o, lse = V.forward(d["q"], d["k"], d["v"], idx, d["q2k_num"], d["vbs"], kv_chunk_blocks=chunk,
                       out=(nan_like(d["q"]), nan_like(one[1])))
    torch.cuda.synchronize()
    assert torch.equal(o, one[0]) and torch.equal(lse, one[1])
    if not shuffle:
        _fwd_compare(c, d, o, lse)


def test_forward_chunk_work_orders():
    """kv-range chunks with the library's per-chunk work order (96 kv blocks, chunks of 16): o and
    lse are bitwise those of one launch and match the oracle; the workspace's order (the last
    chunk's) equals the oracle's work order over the lengths of the lists' parts in that chunk."""
    c = workloads.make_case(1, 2, 96, None, topk_choices=[3, 8, 13, 21], seed=75,
                            vbs=[64] * 95 + [29], name="forward chunk orders")
    d = to_dev(c)
    say("[forward] per-chunk work orders")
    one = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"],
                    kv_chunk_blocks=-1)
    R = 16
    nbytes = V.fwd_workspace_bytes(c.B, c.H, c.S, R)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"],
                       kv_chunk_blocks=R, workspace=ws, out=(nan_like(d["q"]), nan_like(one[1])))
    torch.cuda.synchronize()
    assert torch.equal(o, one[0]) and torch.equal(lse, one[1])
    # the order is the workspace's last region: [B*H*nb] int32, 256-byte aligned
    n = c.B * c.H * c.nb
    tail = -(-n * 4 // 256) * 256
    order = ws[nbytes - tail:].view(torch.int32)[:n].cpu().numpy()
    idx, num = c.q2k_idx.numpy(), c.q2k_num.numpy()
    last = -(-c.nb // R) - 1
    pos = np.arange(idx.shape[-1])
    part = ((idx >= last * R) & (pos < num[..., None])).sum(-1).astype(np.int32)
    assert np.array_equal(order, O.work_order(torch.from_numpy(part), V.ORDER_BIN_WIDTH))
    _fwd_compare(c, d, o, lse)
    # lists in no particular order: the chunks partition them by position, the order bins the
    # parts, and o, lse stay bitwise those of one launch over the same lists
    g = torch.Generator().manual_seed(5)
    rows = c.q2k_idx.reshape(-1, c.q2k_idx.shape[-1]).clone()
    for i, k_ in enumerate(c.q2k_num.reshape(-1).tolist()):
        rows[i, :k_] = rows[i, :k_][torch.randperm(k_, generator=g)]
    shuf = rows.reshape(c.q2k_idx.shape).to(DEV)
    one = V.forward(d["q"], d["k"], d["v"], shuf, d["q2k_num"], d["vbs"], kv_chunk_blocks=-1)
    o2, lse2 = V.forward(d["q"], d["k"], d["v"], shuf, d["q2k_num"], d["vbs"], kv_chunk_blocks=R,
                         out=(nan_like(d["q"]), nan_like(one[1])))
    torch.cuda.synchronize()
    assert torch.equal(o2, one[0]) and torch.equal(lse2, one[1])


def test_forward_v_magnitudes_per_head():
    """The P V product runs on an fp16 copy of v scaled per head by a power of two: heads whose
    v is tiny (3e-30), huge (1e30), all zero, or has one large outlier, all against the oracle on
    the ragged workload (o scales with v; lse does not depend on it)."""
    c = workloads.config(2)
    v = c.v.to(torch.float32).clone()
    v[0, 0] *= 3e-30
    v[0, 1] *= 1e30
    v[1, 0] = 0
    v[1, 1, 5, 7] = 3e4   # one outlier sets the head's scale
    c = dataclasses.replace(c, v=v.to(torch.bfloat16).contiguous())
    d = to_dev(c)
    say("[forward] per-head v magnitudes")
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"],
                       out=(nan_like(d["q"]), nan_like(torch.empty(c.B, c.H, c.S,
                                                                   dtype=torch.float32, device=DEV))))
    torch.cuda.synchronize()
    ro, rl = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    for b, h in ((0, 0), (0, 1), (1, 1)):
        check_close(f"o[{b},{h}]", o[b, h], ro[b, h])
    assert torch.all(o[1, 0] == 0)
    assert np.abs(lse.cpu().double().numpy() - rl).max() <= LSE_ABS_TOL


def test_forward_ignores_out_of_range_kv_ids():
    """kv ids outside [0, nb) in a q2k list (a caller-contract violation) contribute nothing and
    fault nothing: the forward with such ids inserted in the middle of the lists gives the same
    bits as without them."""
    c = workloads.make_case(1, 2, 8, 3, seed=23, vbs=[64, 64, 64, 64, 64, 64, 64, 29])
    d = to_dev(c)
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
    # lists of width 5: the three valid ids with -1 and nb spliced in after the first one
    bad = torch.empty(1, 2, 8, 5, dtype=torch.int32)
    bad[..., 0] = c.q2k_idx[..., 0]
    bad[..., 1] = -1
    bad[..., 2] = c.q2k_idx[..., 1]
    bad[..., 3] = c.nb
    bad[..., 4] = c.q2k_idx[..., 2]
    num = torch.full((1, 2, 8), 5, dtype=torch.int32)
    say("[forward] lists with out-of-range kv ids")
    o2, lse2 = V.forward(d["q"], d["k"], d["v"], bad.to(DEV), num.to(DEV), d["vbs"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    assert torch.equal(lse, lse2)


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 0.3])
def test_forward_scale_sign_and_zero(scale):
    """The forward with a negative, a zero and a large positive sm_scale (the kernel keeps its
    scores unscaled and needs a positive factor: a negative one moves into Q, a zero one becomes
    the least normal float) against the oracle at that scale, on the ragged config with empty kv
    blocks. At zero every valid key weighs the same: lse = log2(#valid keys)."""
    c = dataclasses.replace(workloads.config(2), sm_scale=scale)
    d = to_dev(c)
    say(f"[forward] sm_scale {scale}")
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"], sm_scale=scale,
                       out=(nan_like(d["q"]), nan_like(torch.empty(c.B, c.H, c.S, dtype=torch.float32,
                                                                   device=DEV))))
    torch.cuda.synchronize()
    _fwd_compare(c, d, o, lse)


# -----------------------------------------------------------------------------------------------
# backward on small workloads, o and lse from the oracle (as the FastVideo test does)
# -----------------------------------------------------------------------------------------------

MODES = {"recompute": V.DQ_RECOMPUTE, "spill": V.DQ_SPILL}


def _bwd_small(c, label, mode=V.DQ_RECOMPUTE):
    d = to_dev(c)
    ro, rl = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    o = torch.from_numpy(O.bf16_rne(ro)).to(torch.bfloat16).to(DEV)
    lse = torch.from_numpy(rl).to(torch.float32).to(DEV)
    ridx, rnum = O.invert_indices(c.q2k_idx, c.q2k_num, c.nb)
    k2q_idx = torch.from_numpy(ridx).to(DEV)
    k2q_num = torch.from_numpy(rnum).to(DEV)
    ws = torch.full((V.bwd_workspace_bytes(c.B, c.H, c.S, 0, mode),), 0xFF, dtype=torch.uint8,
                    device=DEV)
    out = (nan_like(d["q"]), nan_like(d["k"]), nan_like(d["v"]))
    say(f"[backward] {label} (q2k derived from k2q, dq mode {mode})")
    plan = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                     sm_scale=c.sm_scale, workspace=ws, out=out, dq_mode=mode)
    dq, dk, dv = plan.run()
    torch.cuda.synchronize()
    # the same call with the forward's q2k lists given: bit-identical results
    say(f"[backward] {label} (q2k given)")
    given = V.backward_from_k2q(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num,
                                d["vbs"], sm_scale=c.sm_scale, q2k_idx=d["q2k_idx"],
                                q2k_num=d["q2k_num"], dq_mode=mode)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), given):
        assert torch.equal(a, b)
    if mode == V.DQ_SPILL:
        # dk, dv come from the same kernel arithmetic in both modes: identical bits
        other = V.backward_from_k2q(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num,
                                    d["vbs"], sm_scale=c.sm_scale, dq_mode=V.DQ_RECOMPUTE)
        torch.cuda.synchronize()
        assert torch.equal(dk, other[1]) and torch.equal(dv, other[2])
    rdq, rdk, rdv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert got.dtype == torch.bfloat16
        check_close(name, got, ref)
    sc = _check_scales(c, plan, o)
    # Delta from the preprocess (the records hold -Delta 2^-(eo + ev)), on the bf16 o it was given
    rdelta = O.delta(o.cpu(), c.do)
    shift = 2.0 ** (sc[..., V.SC_EO] + sc[..., V.SC_EV]).double().numpy()[..., None]
    gd = -plan.lse_delta()[:, :, :, 1, :].reshape(c.B, c.H, c.S).cpu().double().numpy() * shift
    assert np.abs(gd - rdelta).max() <= 1e-5 * max(1.0, np.abs(rdelta).max())
    # the records also carry (pp - lse) / c, subtracted and divided in IEEE fp32 (torch rounds
    # the same way)
    glse = plan.lse_delta()[:, :, :, 0, :].reshape(c.B, c.H, c.S)
    pp = sc[..., V.SC_PP].float()[..., None]
    cc = sc[..., V.SC_C].contiguous().view(torch.float32)[..., None]
    assert torch.equal(glse.cpu(), (pp - lse.cpu()) / cc)
    return dq, dk, dv, rdq, rdk, rdv


def _check_scales(c, plan, o):
    """The preprocess's per-head exponents against the inputs (vsa.h, VSA_WS_SCALES): q, k
    copies with max |.| in [2^14, 2^15), v, dO in [1, 2), c = fp32(sm_scale log2 e) 2^(eq + ek),
    es = pp - eo - ev, and pp the largest exponent <= 15 with 2^pp times the bound on
    |dP - Delta| (row norms, largest |Delta|, margin 1.0625) in the scaled units at most 2^15."""
    sc = plan.scales().cpu()
    q, k, v, do = (t.double().numpy() for t in (c.q, c.k, c.v, c.do))
    delta = O.delta(o.cpu(), c.do)
    c2 = (torch.tensor(c.sm_scale, dtype=torch.float32)
          * torch.tensor(1.4426950408889634, dtype=torch.float32))
    for b in range(c.B):
        for h in range(c.H):
            w = [int(x) for x in sc[b, h]]
            eq, ek, ev, eo, pp, es = w[:6]
            for x, e, lo in ((q, eq, 2.0 ** 14), (k, ek, 2.0 ** 14), (v, ev, 1.0), (do, eo, 1.0)):
                m = np.abs(x[b, h]).max() * 2.0 ** -e
                assert lo <= m < 2 * lo, (b, h, w)
            assert es == pp - eo - ev
            assert sc[b, h, V.SC_C:V.SC_C + 1].view(torch.float32).item() == (
                c2 * 2.0 ** (eq + ek)).item()
            nv = np.sqrt((v[b, h] ** 2).sum(-1)).max() * 2.0 ** -ev
            no = np.sqrt((do[b, h] ** 2).sum(-1)).max() * 2.0 ** -eo
            bound = 1.0625 * (no * nv + np.abs(delta[b, h]).max() * 2.0 ** -(eo + ev))
            assert 2.0 ** pp * bound <= 2.0 ** 15 * (1 + 1e-5), (b, h, w, bound)
            assert pp == 15 or 2.0 ** (pp + 1) * bound > 2.0 ** 15 * (1 - 1e-5), (b, h, w, bound)
    return sc


# input magnitudes far from N(0,1), each tensor scaled by the factor (then rounded to bf16)
SCALE_CASES = {
    "tiny_dO": dict(do=2.0 ** -20),             # gradients of training-loss size
    "large_v_small_dO": dict(v=1000.0, do=1e-3),
    "peaked_scores": dict(q=8.0, k=8.0),        # scores 64x larger: nearly one-hot rows
    "flat_scores": dict(q=1e-3),                # nearly uniform rows
    "tiny_v_large_dO": dict(v=1e-8, do=1e4),
}


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("case", sorted(SCALE_CASES))
def test_backward_operand_scales(case, mode):
    """The per-head power-of-two scales of the fp16 operands at input magnitudes far from N(0,1):
    the exponents against the inputs (_check_scales) and all three gates on every gradient
    (config 2: ragged blocks, unselected kv blocks).

    The reference is the oracle's gradient with Delta taken from the bf16 o the backward is given
    (the pages' preprocess): the exact gradient moved by the rounding of o, which is linear in
    delta_i = rowsum((bf16(o) - o) * dO)_i: dq_i changes by -sm_scale delta_i (P K)_i and dk_j by
    -sm_scale (P^T (delta * q))_j, both from oracle calls (a forward with v := k, a backward with
    dO := delta * q). With nearly one-hot rows dP - Delta is small and that shift reaches ~1 % of
    dq, far above the gates; at N(0,1) inputs it is negligible."""
    c = copy.copy(workloads.config(2))
    for name, f in SCALE_CASES[case].items():
        setattr(c, name, (getattr(c, name).float() * f).to(torch.bfloat16))
    mode = MODES[mode]
    d = to_dev(c)
    ro, rl = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    o16 = O.bf16_rne(ro)
    o = torch.from_numpy(o16).to(torch.bfloat16).to(DEV)
    lse = torch.from_numpy(rl).to(torch.float32).to(DEV)
    ridx, rnum = O.invert_indices(c.q2k_idx, c.q2k_num, c.nb)
    k2q_idx, k2q_num = torch.from_numpy(ridx).to(DEV), torch.from_numpy(rnum).to(DEV)
    say(f"[backward] operand scales {case}, dq mode {mode}")
    plan = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                     sm_scale=c.sm_scale, out=(nan_like(d["q"]), nan_like(d["k"]), nan_like(d["v"])),
                     dq_mode=mode)
    dq, dk, dv = plan.run()
    torch.cuda.synchronize()
    _check_scales(c, plan, o)
    rdq, rdk, rdv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    delta = ((o16 - ro) * c.do.double().numpy()).sum(-1, keepdims=True)  # [B, H, S, 1]
    pk, _ = O.forward(c.q, c.k, c.k, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    _, _, ptdq = O.backward(c.q, c.k, c.v, torch.from_numpy(delta * c.q.double().numpy()),
                            c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    rdq = rdq - c.sm_scale * delta * pk
    rdk = rdk - c.sm_scale * ptdq
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        check_close(name, got, ref)


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("n", [1, 2])
def test_backward_parity(n, mode):
    c = workloads.config(n)
    dq, dk, dv, *_ = _bwd_small(c, f"config {n}", MODES[mode])
    if n == 2:
        dk, dv = dk.float().cpu(), dv.float().cpu()
        for kb in (4, 11):  # selected by no q block
            assert torch.all(dk[:, :, kb * 64:(kb + 1) * 64] == 0)
            assert torch.all(dv[:, :, kb * 64:(kb + 1) * 64] == 0)
        for kb, nvalid in ((7, 50), (15, 37)):  # padded kv rows
            assert torch.all(dk[:, :, kb * 64 + nvalid:(kb + 1) * 64] == 0)
            assert torch.all(dv[:, :, kb * 64 + nvalid:(kb + 1) * 64] == 0)


EDGE_CASES = {
    # name: (B, H, nb, topk, vbs, kv_pool, empty_q_blocks)
    "odd_blocks_ragged": (2, 3, 5, 3, [64, 17, 64, 40, 1], None, ()),
    "dense_all_selected": (1, 2, 8, 8, None, None, ()),
    "single_block": (1, 1, 1, 1, [29], None, ()),
    "zero_valid_block": (1, 2, 6, 3, [64, 0, 64, 64, 33, 64], None, ()),
    "empty_q_blocks": (2, 2, 6, 2, [64, 64, 50, 64, 64, 64], None, ((0, 1, 2), (1, 0, 5))),
    "topk_7_ragged_tail": (1, 2, 8, 7, [64, 64, 64, 64, 64, 64, 64, 23], None, ()),
    "pool_excludes_three": (1, 2, 12, 4, None, [0, 1, 2, 4, 5, 7, 8, 10, 11], ()),
}


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("name", sorted(EDGE_CASES))
def test_backward_edge_cases(name, mode):
    B, H, nb, topk, vbs, pool, empty = EDGE_CASES[name]
    c = workloads.make_case(B, H, nb, topk, seed=17, vbs=vbs, kv_pool=pool, name=name)
    for b, h, qb in empty:
        c.q2k_num[b, h, qb] = 0
    # forward first: also the GPU forward's o/lse on these shapes
    d = to_dev(c)
    say(f"[forward] edge case {name}")
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
    torch.cuda.synchronize()
    _fwd_compare(c, d, o, lse)
    dq, dk, dv, rdq, rdk, rdv = _bwd_small(c, f"edge case {name}", MODES[mode])
    # exact zeros wherever the oracle is exactly zero (unselected, padded, empty rows)
    for got, ref in ((dq, rdq), (dk, rdk), (dv, rdv)):
        zero = ref == 0
        assert np.all(got.float().cpu().numpy()[zero] == 0)


@pytest.mark.parametrize("seed", range(8))
def test_backward_random_shapes(seed):
    """Seeded random shapes and options: B, H, nb, per-row top-k, ragged vbs (0 to 64), a kv pool,
    empty q rows, the dQ mode, q-range chunks and whether the q2k lists are given. GPU forward
    and backward against the oracle (all gates on o, lse and the three gradients)."""
    rng = np.random.default_rng(1000 + seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    nb = int(rng.integers(1, 14))
    pool = sorted(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False).tolist())
    choices = sorted({int(x) for x in rng.integers(1, len(pool) + 1, size=3)})
    vbs = [int(x) if rng.random() < 0.35 else 64 for x in rng.integers(0, 65, size=nb)]
    mode = V.DQ_SPILL if rng.random() < 0.5 else V.DQ_RECOMPUTE
    chunk = int(rng.integers(1, nb + 1)) if rng.random() < 0.5 else 0
    give = bool(rng.random() < 0.5)
    c = workloads.make_case(B, H, nb, None, seed=2000 + seed, vbs=vbs, kv_pool=pool,
                            topk_choices=choices, name=f"random{seed}")
    for _ in range(int(rng.integers(0, 3))):  # a few empty q rows
        c.q2k_num[int(rng.integers(0, B)), int(rng.integers(0, H)), int(rng.integers(0, nb))] = 0
    say(f"[backward] random shape {seed}: B={B} H={H} nb={nb} pool={pool} top-k {choices} "
        f"vbs={vbs} mode={mode} chunk={chunk} q2k {'given' if give else 'derived'}")
    d = to_dev(c)
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
    k2q_idx, k2q_num = V.invert_indices(d["q2k_idx"], d["q2k_num"], nb)
    extra = dict(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"]) if give else {}
    dq, dk, dv = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                           out=(nan_like(d["q"]), nan_like(d["k"]), nan_like(d["v"])),
                           dq_mode=mode, chunk_blocks=chunk, **extra).run()
    torch.cuda.synchronize()
    ro, rl = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    check_close("o", o, ro)
    finite = np.isfinite(rl)
    got_lse = lse.cpu().double().numpy()
    assert np.array_equal(np.isfinite(got_lse), finite)
    assert np.abs(got_lse[finite] - rl[finite]).max(initial=0.0) <= LSE_ABS_TOL
    rdq, rdk, rdv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        if np.abs(ref).max() == 0:  # nothing selected anywhere: exact zeros
            assert torch.all(got == 0), name
            continue
        check_close(name, got, ref)
        assert np.all(got.float().cpu().numpy()[ref == 0] == 0), name


@pytest.mark.parametrize("mode", sorted(MODES))
def test_backward_negative_scale(mode):
    """The backward with a negative sm_scale (the records hold lse / scale_log2, negative here)
    against the oracle at that scale, on the ragged config with empty kv blocks."""
    c = dataclasses.replace(workloads.config(2), sm_scale=-0.0883883)
    _bwd_small(c, "negative sm_scale", MODES[mode])


@pytest.mark.parametrize("mode", sorted(MODES))
def test_rows_without_valid_keys(mode):
    """q blocks whose every selected kv block is fully padded (vbs 0): their rows have no valid
    key, so the forward gives o = 0 and lse = -inf, and the backward (given that lse) gives their
    dq rows exactly 0 and no NaN anywhere, although the kv-major kernel's P of such a row is not
    finite (the padded kv rows of dK/dV and the padded slots of dS never reach an output)."""
    c = workloads.make_case(1, 2, 6, 3, seed=29, vbs=[64, 0, 64, 0, 40, 64], name="no_valid_keys")
    c.q2k_idx[0, 0, 2] = torch.tensor([1, 0, 0], dtype=torch.int32)  # only kv block 1
    c.q2k_num[0, 0, 2] = 1
    c.q2k_idx[0, 1, 5] = torch.tensor([3, 1, 0], dtype=torch.int32)  # kv blocks 3 and 1
    c.q2k_num[0, 1, 5] = 2
    d = to_dev(c)
    say("[forward] rows without valid keys")
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
    torch.cuda.synchronize()
    _fwd_compare(c, d, o, lse)
    for h, qb in ((0, 2), (1, 5)):
        rows = slice(qb * 64, (qb + 1) * 64)
        assert torch.all(o[0, h, rows] == 0)
        assert torch.all(lse[0, h, rows] == -float("inf"))
    dq, dk, dv, rdq, rdk, rdv = _bwd_small(c, "rows without valid keys", MODES[mode])
    for got, ref in ((dq, rdq), (dk, rdk), (dv, rdv)):
        g = got.float().cpu().numpy()
        assert np.all(np.isfinite(g))
        assert np.all(g[ref == 0] == 0)
    assert torch.all(dq[0, 0, 128:192] == 0) and torch.all(dq[0, 1, 320:384] == 0)


@pytest.mark.parametrize("mode", sorted(MODES))
def test_backward_very_negative_lse(mode):
    """Every valid score below -88 (lse < -128 in base 2) with ragged kv blocks: a padded kv row
    (zero K row, score 0) then has P = exp2(-lse) = inf in fp32, and nothing of it may reach an
    output (inf times a zero K row, or times dP - Delta = 0, is NaN). Scores that negative come
    from a key direction u shared by all keys that q opposes (q = -14 u + noise). With V = 0
    the gradient is exact and simple: o = 0, so Delta = 0 and dP = 0, every dS is 0 and dq, dk
    are exactly zero, while dv = P^T dO is compared with the oracle."""
    c = workloads.make_case(1, 2, 6, 3, seed=41, vbs=[64, 40, 64, 17, 64, 64], name="neg_lse")
    g = torch.Generator().manual_seed(5)
    u = torch.randn(c.H, 1, 128, generator=g)
    k = u + torch.randn(c.H, c.S, 128, generator=g)
    q = -14.0 * u + torch.randn(c.H, c.S, 128, generator=g)
    c = dataclasses.replace(c, q=q[None].to(torch.bfloat16).contiguous(),
                            k=k[None].to(torch.bfloat16).contiguous(),
                            v=torch.zeros_like(c.v))
    _, rl = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    assert rl.max() < -128
    say(f"[backward] lse below -128 (max {rl.max():.1f}), V = 0, dq mode {mode}")
    d = to_dev(c)
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    assert np.abs(lse.cpu().double().numpy() - rl).max() <= LSE_ABS_TOL
    ridx, rnum = O.invert_indices(c.q2k_idx, c.q2k_num, c.nb)
    k2q_idx, k2q_num = torch.from_numpy(ridx).to(DEV), torch.from_numpy(rnum).to(DEV)
    for give in (False, True):
        extra = dict(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"]) if give else {}
        dq, dk, dv = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num,
                               d["vbs"], out=(nan_like(d["q"]), nan_like(d["k"]), nan_like(d["v"])),
                               dq_mode=MODES[mode], **extra).run()
        torch.cuda.synchronize()
        assert torch.all(dq == 0) and torch.all(dk == 0)
        _, _, rdv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
        check_close("dv", dv, rdv)
        assert np.all(dv.float().cpu().numpy()[rdv == 0] == 0)


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("case,chunk", [(2, 3), (2, 1), ("odd_blocks_ragged", 2),
                                        ("empty_q_blocks", 4), ("pool_excludes_three", 5)])
def test_backward_q_range_chunks(case, chunk, mode):
    """The main kernels in chunks (chunk_blocks): the chunk bounds bit-exact (positions of the
    chunk starts in each ascending k2q row and, in recompute mode, q2k row, from numpy's
    searchsorted), all three gradients within the oracle's tolerance, equal to the one-launch
    results up to the fp32 summation order (dq bit-identical in spill mode, whose q-major kernel
    runs as one launch), and exactly zero wherever the oracle is (unselected kv blocks, padded
    rows, empty q rows)."""
    if case == 2:
        c = workloads.config(2)
    else:
        B, H, nb, topk, vbs, pool, empty = EDGE_CASES[case]
        c = workloads.make_case(B, H, nb, topk, seed=17, vbs=vbs, kv_pool=pool, name=case)
        for b, h, qb in empty:
            c.q2k_num[b, h, qb] = 0
    d = to_dev(c)
    ro, rl = O.forward(c.q, c.k, c.v, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    o = torch.from_numpy(O.bf16_rne(ro)).to(torch.bfloat16).to(DEV)
    lse = torch.from_numpy(rl).to(torch.float32).to(DEV)
    ridx, rnum = O.invert_indices(c.q2k_idx, c.q2k_num, c.nb)
    k2q_idx, k2q_num = torch.from_numpy(ridx).to(DEV), torch.from_numpy(rnum).to(DEV)
    say(f"[backward] {case}, q-range chunks of {chunk} q blocks, dq mode {mode}")
    runs = {}
    for qc in (-1, chunk):
        plan = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                         out=(nan_like(d["q"]), nan_like(d["k"]), nan_like(d["v"])),
                         dq_mode=MODES[mode], chunk_blocks=qc)
        runs[qc] = plan.run()
        torch.cuda.synchronize()
    nch = -(-c.nb // chunk)

    def want_bounds(idx, num):
        rows, nums = idx.reshape(-1, idx.shape[-1]), num.reshape(-1)
        w = np.stack([np.searchsorted(rows[i, :nums[i]], np.arange(nch + 1) * chunk)
                      for i in range(rows.shape[0])])
        w[:, nch] = nums
        return w
    n_items = c.B * c.H * c.nb
    bounds = plan.region(V.WS_CHUNK_BOUNDS, n_items * (nch + 1)).cpu().numpy()
    assert np.array_equal(bounds.reshape(-1, nch + 1), want_bounds(ridx, rnum))
    (dq1, dk1, dv1), (dq, dk, dv) = runs[-1], runs[chunk]
    if MODES[mode] == V.DQ_SPILL:
        assert torch.equal(dq, dq1)
    else:  # the q2k lists derived on the device: ascending, as the oracle's
        qb = plan.region(V.WS_DQ_BOUNDS, n_items * (nch + 1)).cpu().numpy()
        qidx, qnum = O.invert_indices(ridx, rnum, c.nb)
        assert np.array_equal(qb.reshape(-1, nch + 1), want_bounds(qidx, qnum))
    rdq, rdk, rdv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    for name, got, one, ref in (("dq", dq, dq1, rdq), ("dk", dk, dk1, rdk), ("dv", dv, dv1, rdv)):
        check_close(name, got, ref)
        g, g1 = got.float(), one.float()
        assert (g - g1).abs().max().item() <= 1e-2 * g1.abs().max().item() + 1e-30
        assert np.all(got.float().cpu().numpy()[ref == 0] == 0)


@pytest.mark.parametrize("chunk", [-1, 3])
@pytest.mark.parametrize("give_q2k", [False, True])
@pytest.mark.parametrize("n", [2, "odd_blocks_ragged"])
def test_spill_slot_tables_bit_exact(n, give_q2k, chunk):
    """The dS slot tables of the spill mode (index work: bit-exact). Expected values from their
    definition in include/vsa.h, on the oracle's k2q: kbase = exclusive prefix sum of the k2q
    counts inside each head; qent = (kbase[kv] + position of q in kv's ascending k2q row) |
    kv << 32 | vbs[kv] << 48 for every q2k entry. With chunks of R q blocks (a chunked spill) the
    same per chunk: kbase[c] counts each kv block's q blocks in [cR, (c+1)R), and the slot of q is
    kbase[q // R][kv] + its position - the position of the chunk's first entry."""
    if n == 2:
        c = workloads.config(2)
    else:
        B, H, nb, topk, vbs, pool, _ = EDGE_CASES[n]
        c = workloads.make_case(B, H, nb, topk, seed=17, vbs=vbs, kv_pool=pool, name=n)
    d = to_dev(c)
    ridx, rnum = O.invert_indices(c.q2k_idx, c.q2k_num, c.nb)
    k2q_idx, k2q_num = torch.from_numpy(ridx).to(DEV), torch.from_numpy(rnum).to(DEV)
    o = torch.zeros_like(d["q"])
    lse = torch.zeros(c.B, c.H, c.S, dtype=torch.float32, device=DEV)
    extra = dict(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"]) if give_q2k else {}
    plan = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                     dq_mode=V.DQ_SPILL, chunk_blocks=chunk, **extra)
    say(f"[slot tables] {n}, q2k {'given' if give_q2k else 'derived'}, chunks {chunk}")
    plan.stage(plan.PREPROCESS)
    plan.stage(plan.INDEX)
    torch.cuda.synchronize()
    BH, nb = c.B * c.H, c.nb
    kq = c.q2k_idx.shape[-1] if give_q2k else nb
    kidx = ridx.reshape(BH, nb, -1)
    num = rnum.reshape(BH, nb).astype(np.int64)
    R = chunk if chunk > 0 else nb
    nch = -(-nb // R)
    # first[c][bh, kv]: position in kv's k2q row of its first q block >= cR
    first = np.zeros((nch + 1, BH, nb), np.int64)
    for bh in range(BH):
        for kv in range(nb):
            row = kidx[bh, kv, :num[bh, kv]]
            first[:, bh, kv] = np.searchsorted(row, np.arange(nch + 1) * R)
    first[nch] = num
    kbase = np.zeros((nch, BH, nb), np.int64)
    kbase[:, :, 1:] = np.cumsum(first[1:] - first[:-1], axis=2)[:, :, :-1]
    got_kb = plan.region(V.WS_KBASE, nch * BH * nb).cpu().numpy().reshape(nch, BH, nb)
    assert np.array_equal(got_kb, kbase)
    got = plan.region(V.WS_QENT, BH * nb * kq, torch.int64).cpu().numpy().reshape(BH, nb, kq)
    # the q2k lists the library walks: the given ones, or the inverse of k2q (ascending)
    if give_q2k:
        qidx = c.q2k_idx.numpy().reshape(BH, nb, -1)
        qnum = c.q2k_num.numpy().reshape(BH, nb)
    else:
        di, dn = O.invert_indices(ridx, rnum, nb)
        qidx, qnum = di.reshape(BH, nb, -1), dn.reshape(BH, nb)
    vbs = c.vbs.numpy()
    for bh in range(BH):
        for q in range(nb):
            ch = q // R
            for s_ in range(int(qnum[bh, q])):
                kv = int(qidx[bh, q, s_])
                row = list(kidx[bh, kv, :num[bh, kv]])
                slot = int(kbase[ch, bh, kv]) + row.index(q) - int(first[ch, bh, kv])
                want = slot | (kv << 32) | (int(vbs[kv]) << 48)
                assert int(got[bh, q, s_]) == want, (bh, q, s_)


@pytest.mark.parametrize("mode", sorted(MODES))
def test_backward_any_order_gives_identical_bits(mode):
    """Any kv work order: the same dq, dk, dv bits (fixed per-item summation order, no atomics)."""
    c = workloads.config(2)
    d = to_dev(c)
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
    k2q_idx, k2q_num = V.invert_indices(d["q2k_idx"], d["q2k_num"], c.nb)
    say(f"[backward] identity vs reversed order ({mode})")
    a = V.backward_from_k2q(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                            dq_mode=MODES[mode])
    rev = torch.arange(c.B * c.H * c.nb - 1, -1, -1, dtype=torch.int32, device=DEV)
    b = V.backward_from_k2q(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                            order=rev, dq_mode=MODES[mode])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("mode", ["recompute", "spill"])
def test_chunk_work_orders(mode):
    """With q-range chunks and the library's work order (96 kv blocks, chunks of 16 q blocks) the
    kv-major items are ordered per chunk, by the length of their list's part in the chunk: the
    workspace holds the last chunk's order, equal to the oracle's work order over those lengths;
    every output is bitwise that of the same call under a caller-given identity order, and
    matches the oracle."""
    c = workloads.make_case(1, 2, 96, None, topk_choices=[3, 8, 13, 21], seed=71,
                            vbs=[64] * 95 + [29], name="chunk orders")
    d = to_dev(c)
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
    k2q_idx, k2q_num = V.invert_indices(d["q2k_idx"], d["q2k_num"], c.nb)
    R = 16
    extra = dict(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"]) if mode == "spill" else {}
    say(f"[backward] per-chunk work orders ({mode})")
    plan = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                     out=(nan_like(d["q"]), nan_like(d["k"]), nan_like(d["v"])),
                     dq_mode=MODES[mode], chunk_blocks=R, **extra)
    got = plan.run()
    ident = torch.arange(c.B * c.H * c.nb, dtype=torch.int32, device=DEV)
    other = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                      order=ident, dq_mode=MODES[mode], chunk_blocks=R, **extra).run()
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv"), got, other):
        assert torch.equal(x, y), name
    # the last chunk's part of each k2q list: its q blocks >= (C - 1) * R
    idx, num = k2q_idx.cpu().numpy(), k2q_num.cpu().numpy()
    last = (c.nb + R - 1) // R - 1
    pos = np.arange(idx.shape[-1])
    part = ((idx >= last * R) & (pos < num[..., None])).sum(-1).astype(np.int32)
    n = c.B * c.H * c.nb
    assert np.array_equal(plan.region(V.WS_KV_ORDER, n).cpu().numpy(),
                          O.work_order(torch.from_numpy(part), V.ORDER_BIN_WIDTH))
    rdq, rdk, rdv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    check_close("dq", got[0], rdq)
    check_close("dk", got[1], rdk)
    check_close("dv", got[2], rdv)


@pytest.mark.parametrize("mode", ["recompute", "spill"])
@pytest.mark.parametrize("chunk", [0, 24])
def test_stages_match_one_call(mode, chunk):
    """The four stages enqueued one at a time (the path the benchmark times) give the bits of the
    one-call backward, with and without chunks (80 kv blocks: the library's work orders run)."""
    c = workloads.make_case(1, 2, 80, None, topk_choices=[5, 9, 16], seed=73,
                            vbs=[64] * 79 + [45], name="stages")
    d = to_dev(c)
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
    k2q_idx, k2q_num = V.invert_indices(d["q2k_idx"], d["q2k_num"], c.nb)
    extra = dict(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"]) if mode == "spill" else {}
    say(f"[stages] {mode}, chunks {chunk}")

    def plan():
        return V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                         out=(nan_like(d["q"]), nan_like(d["k"]), nan_like(d["v"])),
                         dq_mode=MODES[mode], chunk_blocks=chunk, **extra)

    first = plan()
    one = first.run()
    staged = plan()
    for s_ in (staged.PREPROCESS, staged.INDEX, staged.DKDV, staged.DQ):
        staged.stage(s_)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv"), one, (staged.dq, staged.dk, staged.dv)):
        assert torch.equal(x, y), name
    rdq, rdk, rdv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    check_close("dq", one[0], rdq)
    check_close("dk", one[1], rdk)
    check_close("dv", one[2], rdv)


def test_nondefault_stream():
    c = workloads.config(1)
    d = to_dev(c)
    s = torch.cuda.Stream()
    say("[stream] side stream")
    with torch.cuda.stream(s):
        o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
        dq, dk, dv = V.backward(d["do"], d["q"], d["k"], d["v"], o, lse, d["q2k_idx"],
                                d["q2k_num"], d["vbs"], dq_mode=V.DQ_SPILL)
    s.synchronize()
    rdq, rdk, rdv = O.backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale)
    check_close("dq", dq, rdq)
    check_close("dk", dk, rdk)
    check_close("dv", dv, rdv)


# -----------------------------------------------------------------------------------------------
# full-size workloads: sampled blocks + invariants
# -----------------------------------------------------------------------------------------------

def _end_to_end(c, mode=V.DQ_RECOMPUTE, give_q2k=False):
    """GPU forward -> GPU invert -> GPU backward, outputs and workspace NaN-prefilled."""
    d = to_dev(c)
    o = nan_like(d["q"])
    lse = nan_like(torch.empty(c.B, c.H, c.S, dtype=torch.float32, device=DEV))
    V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"], out=(o, lse))
    k2q_idx, k2q_num = V.invert_indices(d["q2k_idx"], d["q2k_num"], c.nb)
    kq = d["q2k_idx"].shape[-1] if give_q2k else 0
    ws = torch.full((V.bwd_workspace_bytes(c.B, c.H, c.S, kq, mode),), 0xFF, dtype=torch.uint8,
                    device=DEV)
    out = (nan_like(d["q"]), nan_like(d["k"]), nan_like(d["v"]))
    extra = dict(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"]) if give_q2k else {}
    plan = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                     workspace=ws, out=out, dq_mode=mode, **extra)
    dq, dk, dv = plan.run()
    torch.cuda.synchronize()
    return d, o, lse, (k2q_idx, k2q_num), plan, (dq, dk, dv)


def _sampled_checks(c, o, lse, grads, qblocks, kvblocks, precision="float64"):
    """o, lse and dq of the q blocks, dk and dv of the kv blocks, each against the oracle
    computed for that block alone (a kv block sums the contributions of every q block that
    selects it, each with its full softmax)."""
    dq, dk, dv = grads
    if qblocks:
        _fwd_compare(c, None, o, lse, qblocks=qblocks)
        sdq, _ = O.backward_sampled(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs,
                                    c.sm_scale, qblocks=qblocks, kvblocks=())
        for (b, h, qb), ref in sdq.items():
            check_close(f"dq[{b},{h},{qb}]", dq[b, h, qb * 64:(qb + 1) * 64], ref)
    if kvblocks:
        say(f"  oracle for {len(kvblocks)} kv blocks ({precision})")
        sdkv = O.kvblock_backward(c.q, c.k, c.v, c.do, c.q2k_idx, c.q2k_num, c.vbs, c.sm_scale,
                                  kvblocks, precision,
                                  progress=lambda i, n: say(f"    q block {i} of {n}"))
        for (b, h, kb), (rk, rv) in sorted(sdkv.items()):
            check_close(f"dk[{b},{h},{kb}]", dk[b, h, kb * 64:(kb + 1) * 64], rk)
            check_close(f"dv[{b},{h},{kb}]", dv[b, h, kb * 64:(kb + 1) * 64], rv)


def _spread(c, n, seed):
    """n (b, h, block) samples spread over the heads: the first and last block of the first
    and last head, the rest drawn at random (seeded)."""
    g = np.random.default_rng(seed)
    heads = [(b, h) for b in range(c.B) for h in range(c.H)]
    out = [(*heads[0], 0), (*heads[-1], c.nb - 1), (*heads[0], c.nb - 1), (*heads[-1], 0)]
    while len(out) < n:
        b, h = heads[len(out) % len(heads)]
        blk = int(g.integers(1, c.nb - 1))
        if (b, h, blk) not in out:
            out.append((b, h, blk))
    return out


def _invariants(c, grads):
    """dS rows sum to zero: per head sum_j dk_j = 0 and sum_j dv_j = sum_i dO_i (every q row here
    has keys). Checked column-wise against the column's absolute mass."""
    dq, dk, dv = grads
    for g in grads:
        assert torch.isfinite(g.float()).all()
    dk64 = dk.double()
    colsum = dk64.sum(dim=2).abs()
    mass = dk64.abs().sum(dim=2)
    assert (colsum <= 2e-3 * mass + 1e-6).all(), float((colsum / mass).max())
    dvs = dv.double().sum(dim=2)
    dos = c.do.to(DEV).double().sum(dim=2)
    mass = dv.double().abs().sum(dim=2)
    assert ((dvs - dos).abs() <= 2e-3 * mass + 1e-6).all()


@pytest.mark.timeout(900)
def test_config3_32k_end_to_end_sampled():
    c = workloads.config(3)
    say("[end-to-end] config 3 (B=1 H=8 S=32768, 25%, dS spill, q2k given)")
    d, o, lse, (k2q_idx, k2q_num), plan, grads = _end_to_end(c, V.DQ_SPILL, give_q2k=True)
    # 512 kv blocks: the library computed the length-binned kv-major order into the workspace
    n = c.B * c.H * c.nb
    assert np.array_equal(plan.region(V.WS_KV_ORDER, n).cpu().numpy(),
                          O.work_order(k2q_num.cpu(), V.ORDER_BIN_WIDTH))
    _invariants(c, grads)
    _sampled_checks(c, o, lse, grads, qblocks=_spread(c, 8, 31), kvblocks=_spread(c, 8, 37))


@pytest.mark.timeout(900)
def test_config4_65k_order_stability_sampled():
    c = workloads.config(4)
    say("[end-to-end] config 4 (B=1 H=8 S=65536, 12.5%, device work order)")
    d, o, lse, (k2q_idx, k2q_num), plan, grads = _end_to_end(c)
    # the library computed the length-binned orders (kv-major from k2q counts, q-major from the
    # derived q2k counts) and the q2k lists into the workspace; all match the oracle's
    n = c.B * c.H * c.nb
    ridx, rnum = O.invert_indices(k2q_idx.cpu(), k2q_num.cpu(), c.nb)
    assert np.array_equal(plan.region(V.WS_Q2K_NUM, n).cpu().numpy().reshape(rnum.shape), rnum)
    assert np.array_equal(plan.region(V.WS_Q2K_IDX, n * c.nb).cpu().numpy().reshape(ridx.shape), ridx)
    bw = V.ORDER_BIN_WIDTH
    assert np.array_equal(plan.region(V.WS_KV_ORDER, n).cpu().numpy(), O.work_order(k2q_num.cpu(), bw))
    assert np.array_equal(plan.region(V.WS_Q_ORDER, n).cpu().numpy(), O.work_order(rnum, bw))
    _invariants(c, grads)
    # run-to-run: every output bitwise equal (no atomics anywhere)
    grads = tuple(t.clone() for t in grads)
    again = plan.run()
    torch.cuda.synchronize()
    for x, y in zip(grads, again):
        assert torch.equal(x, y)
    dq, dk, dv = grads
    _sampled_checks(c, o, lse, grads, qblocks=_spread(c, 8, 41), kvblocks=_spread(c, 8, 43))
    del plan, again
    # the dS spill with the forward's q2k lists: the same dk, dv bits, dq on samples, and
    # run-to-run identical
    say("[end-to-end] config 4, dS spill")
    sp = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                   q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"], dq_mode=V.DQ_SPILL)
    g2 = tuple(t.clone() for t in sp.run())
    torch.cuda.synchronize()
    assert torch.equal(g2[1], dk) and torch.equal(g2[2], dv)
    g3 = sp.run()
    torch.cuda.synchronize()
    for x, y in zip(g2, g3):
        assert torch.equal(x, y)
    _sampled_checks(c, o, lse, g2, qblocks=_spread(c, 8, 41), kvblocks=[])


def _head(c, h):
    """Head h of a case as a one-head case (the oracle then converts one head, not eight)."""
    import dataclasses
    sl = slice(h, h + 1)
    return dataclasses.replace(c, H=1, q=c.q[:, sl], k=c.k[:, sl], v=c.v[:, sl], do=c.do[:, sl],
                               q2k_idx=c.q2k_idx[:, sl], q2k_num=c.q2k_num[:, sl])


@pytest.fixture(scope="module")
def c5_run():
    """524288 tokens, 8192 kv blocks, top-k 2048, inputs x0.5, last kv block 40 valid tokens:
    GPU forward -> invert -> backward on the library's defaults for this shape with the q2k rows
    given (the chunked dS spill: chunks of SPILL_CHUNK_BLOCKS q blocks), run once for the tests
    below."""
    c = workloads.config(5)
    mode = V.default_dq_mode(c.B, c.H, c.S, c.q2k_idx.shape[-1], device=DEV)
    assert mode == V.DQ_SPILL  # 72 GiB of workspace, within a third of the device's memory
    say("[end-to-end] config 5 (B=1 H=8 S=524288, 25%, ragged last block), chunked spill")
    d, o, lse, (k2q_idx, k2q_num), plan, grads = _end_to_end(c, mode, give_q2k=True)
    yield c, d, o, lse, (k2q_idx, k2q_num), plan, grads
    del d, o, lse, k2q_idx, k2q_num, plan, grads
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_config5_524k_invert_bit_exact(c5_run):
    """The 2 GiB k2q of the 524288-token workload, bit-exact against the oracle's inversion."""
    c, _, _, _, (k2q_idx, k2q_num), _, _ = c5_run
    say("  k2q vs oracle")
    ridx, rnum = O.invert_indices(c.q2k_idx, c.q2k_num, c.nb)
    assert np.array_equal(k2q_num.cpu().numpy(), rnum)
    for h in range(c.H):  # one head (256 MiB) at a time
        assert np.array_equal(k2q_idx[:, h].cpu().numpy(), ridx[:, h]), h


@pytest.mark.timeout(900)
def test_config5_524k_end_to_end_sampled(c5_run):
    """o, lse and dq on sampled q blocks against the oracle (each one q block of one head);
    the invariants and the exact zeros of the ragged block; the default chunked path against one
    launch per kernel in recompute mode: dk and dv within the fp32 reordering bound, dq within the
    same bound (the two dQ kernels round dS alike but sum in another arrangement)."""
    c, d, o, lse, (k2q_idx, k2q_num), plan, grads = c5_run
    dq, dk, dv = grads
    _invariants(c, grads)
    last = (c.nb - 1) * 64
    assert torch.all(dk[:, :, last + 40:] == 0) and torch.all(dv[:, :, last + 40:] == 0)
    assert torch.any(dk[:, :, last:last + 40] != 0)
    for h, qb in ((0, 0), (4, 4096), (7, c.nb - 1)):
        ch = _head(c, h)
        sub = (o[:, h:h + 1], lse[:, h:h + 1], (dq[:, h:h + 1], dk[:, h:h + 1], dv[:, h:h + 1]))
        say(f"  sampled q block (h={h}, qb={qb})")
        _sampled_checks(ch, sub[0], sub[1], sub[2], qblocks=[(0, 0, qb)], kvblocks=[])
    # the reported time of the whole backward chain at this size
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    plan.run()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    say(f"  backward chain {ms:.1f} ms, {c.pairs * 5 * 2 * 64 * 64 * 128 / ms / 1e9:.1f} TFLOPS "
        f"on selected blocks")
    # the same backward as one launch per kernel, recompute mode: dk, dv equal up to the fp32
    # summation order of the chunk partial sums; dq from the other dQ kernel
    say("  one-launch recompute backward for comparison")
    one = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                    dq_mode=V.DQ_RECOMPUTE, chunk_blocks=-1).run()
    torch.cuda.synchronize()
    for name, g1, g in (("dq", one[0], dq), ("dk", one[1], dk), ("dv", one[2], dv)):
        diff = (g.float() - g1.float()).abs()
        say(f"  {name}: chunked vs one launch max|diff| {diff.max().item():.3e}, "
            f"mean {diff.mean().item():.3e}, mean|one| {g1.float().abs().mean().item():.3e}")
        assert diff.max().item() <= 1e-2 * g1.float().abs().max().item()
        assert diff.mean().item() <= 1e-3 * g1.float().abs().mean().item()
    del one


@pytest.mark.timeout(900)
def test_config5_524k_kv_blocks_vs_oracle(c5_run):
    """dk and dv of the default chunked dK/dV path at full size against the oracle: the ragged
    last kv block (40 valid tokens) and an interior kv block of one head. Each kv block sums the
    contributions of the ~2048 q blocks that select it, each with its softmax over 131072 keys:
    the oracle runs those full-key-set products in float32 (every product with the sampled kv
    blocks in float64), a few minutes of CPU."""
    c, _, _, _, _, _, grads = c5_run
    dq, dk, dv = grads
    h = 5
    ch = _head(c, h)
    sub = (dq[:, h:h + 1], dk[:, h:h + 1], dv[:, h:h + 1])
    say(f"  kv blocks {c.nb - 1} (ragged) and 2900 of head {h}")
    _sampled_checks(ch, None, None, sub, qblocks=[], kvblocks=[(0, 0, c.nb - 1), (0, 0, 2900)],
                    precision="float32")


def test_binding_rejects_bad_outputs_and_workspaces():
    """Caller-supplied outputs and workspaces go to the kernels as raw pointers, so the binding
    refuses any of the wrong dtype, shape, device or layout before anything is launched."""
    c = workloads.config(1)
    d = to_dev(c)
    say("[binding] bad outputs / workspaces")
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
    k2q_idx, k2q_num = V.invert_indices(d["q2k_idx"], d["q2k_num"], c.nb)
    torch.cuda.synchronize()
    fwd_bad = [
        (torch.empty_like(d["q"], dtype=torch.float32), lse),               # o dtype
        (d["q"].new_empty(c.B, c.H, c.S, 64), lse),                          # o shape
        (torch.empty_like(d["q"]).transpose(2, 3).contiguous().transpose(2, 3), lse),  # layout
        (torch.empty_like(c.q), lse),                                        # o on the host
        (torch.empty_like(d["q"]), lse.to(torch.float64)),                   # lse dtype
        (torch.empty_like(d["q"]), lse[..., :-1]),                           # lse shape
    ]
    for out in fwd_bad:
        with pytest.raises(RuntimeError):
            V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"], out=out)
    with pytest.raises(RuntimeError):  # a workspace on the host
        V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"],
                  kv_chunk_blocks=1, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(RuntimeError):  # a workspace too small
        V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"],
                  kv_chunk_blocks=1, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    for out in ((k2q_idx.to(torch.int64), k2q_num), (k2q_idx[..., :-1], k2q_num),
                (k2q_idx, k2q_num.cpu())):
        with pytest.raises(RuntimeError):
            V.invert_indices(d["q2k_idx"], d["q2k_num"], c.nb, out=out)
    with pytest.raises(RuntimeError):
        V.invert_indices(d["q2k_idx"], d["q2k_num"], c.nb,
                         workspace=torch.empty(64, dtype=torch.float32, device=DEV))
    args = (d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"])
    good = (torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]))
    for i, bad in enumerate((good[0].float(), good[1][:, :, :-64], torch.empty_like(c.v))):
        out = list(good)
        out[i] = bad
        with pytest.raises(RuntimeError):
            V.BwdPlan(*args, out=tuple(out), dq_mode=V.DQ_SPILL)
    for ws in (torch.empty(1 << 20, dtype=torch.uint8),
               torch.empty(1 << 20, dtype=torch.int32, device=DEV),
               torch.empty(8, dtype=torch.uint8, device=DEV)):
        with pytest.raises(RuntimeError):
            V.BwdPlan(*args, workspace=ws, dq_mode=V.DQ_SPILL)
    # the same call with valid buffers runs, and the default dq mode is the dS spill here
    plan = V.BwdPlan(*args, out=good)
    assert plan.dq_mode == V.DQ_SPILL
    plan.run()
    torch.cuda.synchronize()
