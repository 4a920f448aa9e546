"""CPU oracle for 64-token block-sparse (VSA) attention: forward, backward, k2q inversion and
work order, in float64 with plain numpy.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this module. The HIP library never calls it, and it shares no code with the library:
inputs come from the seeded generator in ``workloads.py``, nothing else is common.

Sources (web pages of the FastVideo project; cited below by tag):
  [bwd-test]   compare page main...vsa_bwd_fix, file tests/test_block_sparse_bwd_sm100a.py:
               the fp32 masked-dense autograd ``reference`` (keys of selected blocks at or past
               ``variable_block_sizes`` masked to -inf, loss = sum(out * grad_o), lse =
               logsumexp * log2e, o rounded to bf16) and ``invert_indices_torch`` (k2q rows
               ascending, padded with 0).
  [bwd-args]   same compare page, csrc/attention/block_sparse_bwd_launch_sm100a.cuh, the
               argument struct: lse "M form" max(qk * sm_scale * log2e) + log2(l), [B, H, S]
               fp32; k2q_idx rows of LOCAL q block ids with stride max_q_blocks; k2q_num counts
               (0 allowed); variable_block_sizes masks kv rows at or past the count; dq and dk
               carry sm_scale, dv does not; work order length-binned from 1024 kv blocks.
  [bwd-module] file view of python/fastvideo_kernel/block_sparse_attn_bwd_sm100a.py: module
               docstring (the same lse form and scaling), sm_scale = 1/sqrt(head_dim).

Everything here is the plain definition of the result. Block-sparse attention equals dense
attention with a boolean key mask (a masked key contributes exp(-inf) = 0 exactly), so the
oracle gathers, per q block, exactly the keys that the mask keeps and runs textbook softmax
attention and its textbook gradient on them in float64. Nothing is blocked, fused or reordered
beyond that gather.

Readings of points the pages leave open (each also listed in the design notes):
  * A q row with no valid key (q2k_num = 0, or every selected block has 0 valid tokens): o = 0,
    lse = -inf (logsumexp of an empty set), dq = 0, and it contributes nothing to dk, dv.
  * Duplicate kv ids in one q2k row count once (the mask is boolean).
  * k2q padding value 0; the work order is a stable counting sort by list length in bins of
    width ``bin_width``, longest bin first, ascending kv id inside a bin.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64
LOG2E = 1.4426950408889634
ORDER_MIN_KV_BLOCKS = 1024


# --------------------------------------------------------------------------------------------
# conversions
# --------------------------------------------------------------------------------------------

def f64(t) -> np.ndarray:
    """A torch tensor (bf16, fp32, int) or array as float64; bf16 -> fp64 is exact."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def i64(t) -> np.ndarray:
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu", torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.int64)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range: x = m * 2**e with
    0.5 <= |m| < 1 rounds to rint(m * 256) / 256 * 2**e, with the spacing floored at the
    smallest subnormal 2**-133; magnitudes past the largest finite value become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    m, e = np.frexp(x[finite])
    step_exp = np.maximum(e - 8, -133)
    r = np.rint(x[finite] / np.ldexp(1.0, step_exp)) * np.ldexp(1.0, step_exp)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


# --------------------------------------------------------------------------------------------
# metadata
# --------------------------------------------------------------------------------------------

def selection(q2k_idx, q2k_num, nkv: int) -> np.ndarray:
    """Boolean relation sel[b, h, qb, kb]: q block qb selects kv block kb.

    Only the first q2k_num[b, h, qb] entries of a q2k row count [bwd-test, make_case/reference].
    """
    idx = i64(q2k_idx)
    num = i64(q2k_num)
    B, H, nq, K = idx.shape
    sel = np.zeros((B, H, nq, nkv), dtype=bool)
    rows = np.broadcast_to(np.arange(nq)[:, None], (nq, K))
    for b in range(B):
        for h in range(H):
            counted = np.arange(K)[None, :] < num[b, h][:, None]   # [nq, K]
            sel[b, h, rows[counted], idx[b, h][counted]] = True
    return sel


def invert_indices(q2k_idx, q2k_num, nkv: int):
    """k2q metadata from q2k metadata [bwd-test, invert_indices_torch; bwd-args, k2q fields].

    k2q_num[b, h, kb] = number of q blocks whose (counted) q2k entries contain kb;
    k2q_idx[b, h, kb, :k2q_num] = those q block ids in ascending order; the rest of the row
    (row length = number of q blocks) is 0. Returns int32 arrays.
    """
    sel = selection(q2k_idx, q2k_num, nkv)          # [B, H, nq, nkv]
    B, H, nq, _ = sel.shape
    k2q_num = np.zeros((B, H, nkv), dtype=np.int32)
    k2q_idx = np.zeros((B, H, nkv, nq), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            rel = np.ascontiguousarray(sel[b, h].T)   # [nkv, nq]: row kb lists its q blocks
            for kb in range(nkv):
                qbs = np.flatnonzero(rel[kb])         # ascending by construction
                k2q_num[b, h, kb] = qbs.size
                k2q_idx[b, h, kb, :qbs.size] = qbs
    return k2q_idx, k2q_num


def work_order(k2q_num, bin_width: int = 8) -> np.ndarray:
    """Work-item order for the backward [bwd-args, order workspace; reading in module header].

    Items are (b, h, kv) with global id (b*H + h)*nb + kv. Within each (b, h) the items are
    ranked by bin = k2q_num // bin_width, largest bin first, ties by ascending kv id; the
    result lists global item ids, (b, h) segments in order. Returns int32 [B*H*nb].
    """
    num = i64(k2q_num)
    B, H, nb = num.shape
    out = np.empty(B * H * nb, dtype=np.int32)
    for bh in range(B * H):
        bins = num.reshape(B * H, nb)[bh] // bin_width
        # a stable sort on -bin keeps ascending kv id inside a bin
        rank = np.argsort(-bins, kind="stable")
        out[bh * nb:(bh + 1) * nb] = bh * nb + rank
    return out


def kept_keys(q2k_idx, q2k_num, vbs, b: int, h: int, qb: int) -> np.ndarray:
    """Key token ids (ascending) that q block qb attends to [bwd-test, reference mask]:
    token j is kept iff its block j // 64 is among the row's counted selections and
    j % 64 < vbs[j // 64]. Duplicated selections count once."""
    idx = i64(q2k_idx)
    num = i64(q2k_num)
    vb = i64(vbs)
    blocks = np.unique(idx[b, h, qb, :num[b, h, qb]])
    if blocks.size == 0:
        return np.zeros(0, dtype=np.int64)
    toks = [kb * BLOCK + np.arange(int(vb[kb])) for kb in blocks]
    return np.concatenate(toks).astype(np.int64)


def dense_keep_mask(q2k_idx, q2k_num, vbs, S: int) -> np.ndarray:
    """The literal [B, H, S, S] boolean mask of [bwd-test, reference] (small sizes only)."""
    idx = i64(q2k_idx)
    B, H, nq, _ = idx.shape
    keep = np.zeros((B, H, S, S), dtype=bool)
    for b in range(B):
        for h in range(H):
            for qb in range(nq):
                keep[b, h, qb * BLOCK:(qb + 1) * BLOCK, kept_keys(q2k_idx, q2k_num, vbs, b, h, qb)] = True
    return keep


# --------------------------------------------------------------------------------------------
# attention on one q block's kept keys
# --------------------------------------------------------------------------------------------

def qblock_forward(qi: np.ndarray, kk: np.ndarray, vk: np.ndarray, sm_scale: float):
    """Softmax attention of the rows qi [r, D] over keys kk, values vk [n, D], float64.

    s = sm_scale * qi kk^T; P = softmax_row(s); o = P vk; lse in M form =
    log2e * logsumexp(s) = max(s * log2e) + log2(sum exp(s - max)) [bwd-args, lse field].
    With no keys: o = 0, lse = -inf. Returns (o, lse, P).
    """
    r = qi.shape[0]
    if kk.shape[0] == 0:
        return np.zeros_like(qi), np.full(r, -np.inf), np.zeros((r, 0))
    s = sm_scale * (qi @ kk.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ vk
    lse = LOG2E * (m[:, 0] + np.log(l[:, 0]))
    return o, lse, p


def qblock_backward(qi, doi, kk, vk, sm_scale: float):
    """Gradient of L = sum(o * dO) for one q block's rows over its kept keys, float64.

    The textbook softmax-attention gradient [bwd-test, reference: autograd of that loss]:
      dV = P^T dO;  dP = dO V^T;  Delta = rowsum(o * dO) = rowsum(P * dP);
      dS = P * (dP - Delta);  dQ = sm_scale * dS K;  dK = sm_scale * dS^T Q.
    Returns (o, lse, dq_rows [r, D], dk_keys [n, D], dv_keys [n, D]).
    """
    o, lse, p = qblock_forward(qi, kk, vk, sm_scale)
    if kk.shape[0] == 0:
        return o, lse, np.zeros_like(qi), np.zeros_like(kk), np.zeros_like(vk)
    dv = p.T @ doi
    dp = doi @ vk.T
    delta = np.sum(o * doi, axis=1, keepdims=True)
    ds = p * (dp - delta)
    dq = sm_scale * (ds @ kk)
    dk = sm_scale * (ds.T @ qi)
    return o, lse, dq, dk, dv


# --------------------------------------------------------------------------------------------
# whole tensors
# --------------------------------------------------------------------------------------------

def _rows(x, b, h, blk):
    return x[b, h, blk * BLOCK:(blk + 1) * BLOCK]


def forward(q, k, v, q2k_idx, q2k_num, vbs, sm_scale: float, qblocks=None):
    """Block-sparse attention forward [bwd-test, reference; bwd-args, lse field].

    Returns (o [B,H,S,D] float64, unrounded; lse [B,H,S] float64, M form). With ``qblocks``
    (a list of (b, h, qb)) only those q blocks are computed; the rest stay NaN.
    """
    Q, K, V = f64(q), f64(k), f64(v)
    B, H, S, D = Q.shape
    o = np.full((B, H, S, D), np.nan)
    lse = np.full((B, H, S), np.nan)
    todo = qblocks if qblocks is not None else [(b, h, qb) for b in range(B) for h in range(H)
                                                 for qb in range(S // BLOCK)]
    for b, h, qb in todo:
        keys = kept_keys(q2k_idx, q2k_num, vbs, b, h, qb)
        oi, li, _ = qblock_forward(_rows(Q, b, h, qb), K[b, h, keys], V[b, h, keys], sm_scale)
        o[b, h, qb * BLOCK:(qb + 1) * BLOCK] = oi
        lse[b, h, qb * BLOCK:(qb + 1) * BLOCK] = li
    return o, lse


def backward(q, k, v, do, q2k_idx, q2k_num, vbs, sm_scale: float):
    """Block-sparse attention backward: (dq, dk, dv) float64, unrounded, [B,H,S,D] each.

    dq and dk carry sm_scale, dv does not [bwd-args; bwd-module]. Accumulates every q block's
    contributions to its kept keys; keys nobody keeps get exactly 0.
    """
    Q, K, V, DO = f64(q), f64(k), f64(v), f64(do)
    B, H, S, D = Q.shape
    dq = np.zeros_like(Q)
    dk = np.zeros_like(K)
    dv = np.zeros_like(V)
    for b in range(B):
        for h in range(H):
            for qb in range(S // BLOCK):
                keys = kept_keys(q2k_idx, q2k_num, vbs, b, h, qb)
                _, _, dqi, dkk, dvk = qblock_backward(_rows(Q, b, h, qb), _rows(DO, b, h, qb),
                                                      K[b, h, keys], V[b, h, keys], sm_scale)
                dq[b, h, qb * BLOCK:(qb + 1) * BLOCK] = dqi
                np.add.at(dk[b, h], keys, dkk)
                np.add.at(dv[b, h], keys, dvk)
    return dq, dk, dv


def backward_sampled(q, k, v, do, q2k_idx, q2k_num, vbs, sm_scale: float,
                     qblocks=(), kvblocks=()):
    """The same gradient, for chosen blocks only (large sizes).

    ``qblocks``: (b, h, qb) -> dq rows of that q block (needs only its own row).
    ``kvblocks``: (b, h, kb) -> dk, dv rows of that kv block: the sum over every q block that
    keeps a key of kb of its contribution (each such q block's softmax needs its full key set).
    Returns dicts keyed like the inputs: dq[(b,h,qb)] -> [64, D]; dkv[(b,h,kb)] -> (dk, dv).
    """
    Q, K, V, DO = f64(q), f64(k), f64(v), f64(do)
    dq_out = {}
    for b, h, qb in qblocks:
        keys = kept_keys(q2k_idx, q2k_num, vbs, b, h, qb)
        _, _, dqi, _, _ = qblock_backward(_rows(Q, b, h, qb), _rows(DO, b, h, qb),
                                          K[b, h, keys], V[b, h, keys], sm_scale)
        dq_out[(b, h, qb)] = dqi
    idx = i64(q2k_idx)
    num = i64(q2k_num)
    dkv_out = {}
    for b, h, kb in kvblocks:
        dkb = np.zeros((BLOCK, Q.shape[-1]))
        dvb = np.zeros((BLOCK, Q.shape[-1]))
        for qb in range(idx.shape[2]):
            if kb not in idx[b, h, qb, :num[b, h, qb]]:
                continue
            keys = kept_keys(q2k_idx, q2k_num, vbs, b, h, qb)
            _, _, _, dkk, dvk = qblock_backward(_rows(Q, b, h, qb), _rows(DO, b, h, qb),
                                                K[b, h, keys], V[b, h, keys], sm_scale)
            inblk = (keys // BLOCK) == kb
            dkb[keys[inblk] % BLOCK] += dkk[inblk]
            dvb[keys[inblk] % BLOCK] += dvk[inblk]
        dkv_out[(b, h, kb)] = (dkb, dvb)
    return dq_out, dkv_out


def delta(o, do) -> np.ndarray:
    """Delta[b, h, i] = sum_d o[b,h,i,d] * dO[b,h,i,d] for the o given (the backward's
    preprocess row sum, taken on whatever o the caller holds), float64."""
    return np.sum(f64(o) * f64(do), axis=-1)


def kvblock_backward(q, k, v, do, q2k_idx, q2k_num, vbs, sm_scale: float, kvblocks,
                     precision: str = "float64", progress=None):
    """dk and dv rows of chosen kv blocks, straight from their definition [bwd-test, reference:
    the gradient of sum(o * grad_o)]:

        dV_j = sum_i P_ij^T dO_i,   dK_j = sm_scale * sum_i dS_ij^T Q_i,
        dS_ij = P_ij * (dP_ij - Delta_i),  dP_ij = dO_i V_j^T,  Delta_i = rowsum(o_i * dO_i),

    summed over every q block i whose counted q2k entries name block j, where P_ij is the
    block-j columns of q block i's softmax over its full key set. Only those columns of the
    gradient are formed, so a kv block costs the softmax statistics and o of the q blocks that
    select it; q blocks selecting several of the chosen kv blocks are computed once.

    The softmax of q block i runs over the whole 64-row tiles of its selected kv blocks, with the
    scores of padded rows (at or past vbs) set to -inf: the masked-dense form of [bwd-test].

    ``precision``: "float64", or "float32" for the work over a q block's full key set (its scores,
    exp(s - max), their row sum and o = P V), as the largest workloads need (about 2e-7
    relative); every product with the chosen kv blocks stays float64. ``progress``: called with
    (done, total) q blocks now and then. Works on torch CPU tensors (threaded).
    Returns {(b, h, kb): (dk [64, D], dv [64, D])}.
    """
    import torch

    def t64(x):
        return x.detach().to("cpu", torch.float64) if isinstance(x, torch.Tensor) \
            else torch.from_numpy(np.asarray(x, dtype=np.float64))

    wd = torch.float64 if precision == "float64" else torch.float32
    idx, num, vb = i64(q2k_idx), i64(q2k_num), i64(vbs)
    nb = vb.shape[0]
    counted = np.arange(idx.shape[-1])[None, :] < num[..., None]     # [B, H, nq, K]
    out = {}
    heads = sorted({(b, h) for b, h, _ in kvblocks})
    for b, h in heads:
        want = sorted({kb for bb, hh, kb in kvblocks if (bb, hh) == (b, h)})
        Q, K, V, DO = (t64(x[b, h]) for x in (q, k, v, do))
        D = Q.shape[-1]
        Kb = K.to(wd).reshape(nb, BLOCK, D)
        Vb = V.to(wd).reshape(nb, BLOCK, D)
        acc = {kb: (torch.zeros(BLOCK, D, dtype=torch.float64),
                    torch.zeros(BLOCK, D, dtype=torch.float64)) for kb in want}
        sel_rows = counted[b, h] & np.isin(idx[b, h], want)
        qblocks = np.flatnonzero(sel_rows.any(axis=1)).tolist()
        for n_done, qb in enumerate(qblocks):
            if progress is not None and n_done % 200 == 0:
                progress(n_done, len(qblocks))
            blocks = np.unique(idx[b, h, qb, :num[b, h, qb]])
            blocks_t = torch.from_numpy(blocks)
            qi = Q[qb * BLOCK:(qb + 1) * BLOCK]
            doi = DO[qb * BLOCK:(qb + 1) * BLOCK]
            # scores of every row of the selected tiles, (K q^T)^T: one tall product
            s = sm_scale * (torch.index_select(Kb, 0, blocks_t).reshape(-1, D) @ qi.to(wd).T).T
            if (vb[blocks] < BLOCK).any():
                rows_ok = torch.from_numpy(
                    (np.arange(BLOCK)[None, :] < vb[blocks][:, None]).reshape(-1))
                s = s.masked_fill(~rows_ok[None, :], float("-inf"))
            m = s.max(dim=1, keepdim=True).values
            e = torch.exp(s - m)
            l = e.sum(dim=1, keepdim=True).to(torch.float64)
            o = (e @ torch.index_select(Vb, 0, blocks_t).reshape(-1, D)).to(torch.float64) / l
            delta_i = (o * doi).sum(dim=1, keepdim=True)
            for pos in np.flatnonzero(np.isin(blocks, want)).tolist():
                kb = int(blocks[pos])
                nvalid = int(vb[kb])
                if nvalid <= 0:
                    continue
                pj = e[:, pos * BLOCK:pos * BLOCK + nvalid].to(torch.float64) / l
                vj = V[kb * BLOCK:kb * BLOCK + nvalid]
                dsj = pj * (doi @ vj.T - delta_i)
                dk_acc, dv_acc = acc[kb]
                dk_acc[:nvalid] += sm_scale * (dsj.T @ qi)
                dv_acc[:nvalid] += pj.T @ doi
        for kb in want:
            out[(b, h, kb)] = (acc[kb][0].numpy(), acc[kb][1].numpy())
    return out
