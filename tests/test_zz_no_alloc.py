"""vsa_bwd_noalloc (the backward with its workspace in the library's static scratch) against
vsa_bwd with a caller workspace: the same kernels, so every output is bitwise identical. Two
calls in a row, the second on a smaller problem (the scratch keeps the first call's contents),
in both dQ modes, with the q2k lists given and derived; a call whose workspace would not fit
the scratch is refused before anything runs; and a call captured into a HIP graph replays to the
same bits."""
import pytest
import torch

import block_sparse_attention_attn_amd as V
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def _inputs(c):
    d = {n: getattr(c, n).to(DEV) for n in ("q", "k", "v", "do", "q2k_idx", "q2k_num", "vbs")}
    o, lse = V.forward(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"], d["vbs"])
    k2q_idx, k2q_num = V.invert_indices(d["q2k_idx"], d["q2k_num"], c.nb)
    return d, o, lse, k2q_idx, k2q_num


def _nan_out(d):
    return tuple(torch.full_like(d[n], float("nan")) for n in ("q", "k", "v"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    V.lib()


@pytest.mark.parametrize("mode", [V.DQ_RECOMPUTE, V.DQ_SPILL])
@pytest.mark.parametrize("give_q2k", [False, True])
def test_noalloc_matches_workspace_call(mode, give_q2k):
    # 72 kv blocks: the length-binned work orders run too
    big = workloads.make_case(1, 1, 72, 8, seed=61, vbs=[64] * 71 + [23], name="big")
    small = workloads.make_case(1, 2, 6, 3, seed=62, vbs=[64, 17, 64, 64, 0, 50], name="small")
    for c in (big, small):  # the second call is smaller: stale scratch from the first
        d, o, lse, k2q_idx, k2q_num = _inputs(c)
        extra = dict(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"]) if give_q2k else {}
        say(f"[noalloc] {c.name} mode {mode} q2k {'given' if give_q2k else 'derived'}")
        want = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                         out=_nan_out(d), dq_mode=mode, **extra).run()
        got = V.backward_noalloc(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num,
                                 d["vbs"], _nan_out(d), dq_mode=mode, **extra)
        torch.cuda.synchronize()
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(g, w), name


def test_noalloc_large_recompute_call():
    """A call that fills most of the scratch: 8 heads of 16384 tokens, recompute mode, q2k given
    (about 130 MiB of workspace), against the workspace call."""
    c = workloads.make_case(1, 8, 256, 32, seed=66, name="large")
    need = V.bwd_workspace_bytes(c.B, c.H, c.S, c.q2k_idx.shape[-1], V.DQ_RECOMPUTE)
    assert V.NOALLOC_SCRATCH_BYTES // 8 < need <= V.NOALLOC_SCRATCH_BYTES
    d, o, lse, k2q_idx, k2q_num = _inputs(c)
    extra = dict(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"])
    say(f"[noalloc] large recompute call, {need >> 20} MiB of workspace")
    want = V.BwdPlan(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                     out=_nan_out(d), dq_mode=V.DQ_RECOMPUTE, **extra).run()
    got = V.backward_noalloc(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num, d["vbs"],
                             _nan_out(d), dq_mode=V.DQ_RECOMPUTE, **extra)
    torch.cuda.synchronize()
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        assert torch.equal(g, w), name


def test_noalloc_refuses_a_call_beyond_the_scratch():
    # 32768 tokens, top-k 128, dS spill: 4 GiB of workspace
    B, H, S = 1, 8, 32768
    need = V.bwd_workspace_bytes(B, H, S, 128, V.DQ_SPILL)
    assert need > V.NOALLOC_SCRATCH_BYTES
    c = workloads.make_case(1, 1, 4, 2, seed=63)
    d, o, lse, k2q_idx, k2q_num = _inputs(c)
    big = torch.empty(B, H, S, 128, dtype=torch.bfloat16, device=DEV)
    lse_big = torch.empty(B, H, S, dtype=torch.float32, device=DEV)
    idx = torch.zeros(B, H, S // 64, S // 64, dtype=torch.int32, device=DEV)
    num = torch.zeros(B, H, S // 64, dtype=torch.int32, device=DEV)
    q2k = torch.zeros(B, H, S // 64, 128, dtype=torch.int32, device=DEV)
    vbs = torch.full((S // 64,), 64, dtype=torch.int32, device=DEV)
    say("[noalloc] refusal")
    with pytest.raises(RuntimeError, match="static scratch"):
        V.backward_noalloc(big, big, big, big, big, lse_big, idx, num, vbs, (big, big, big),
                           q2k_idx=q2k, q2k_num=num, dq_mode=V.DQ_SPILL)


@pytest.mark.parametrize("mode", [V.DQ_RECOMPUTE, V.DQ_SPILL])
def test_noalloc_replays_under_graph_capture(mode):
    """The callers the entry is for include code under HIP graph capture: the call is captured
    (its kernels launch on the capturing stream; nothing is allocated or cleared with a memset),
    then the graph is replayed three times, each after eager work on another problem through the
    same scratch and with the outputs refilled with NaN; every replay gives the eager call's bits."""
    c = workloads.make_case(1, 2, 12, 4, seed=64, vbs=[64] * 11 + [30], name="graph")
    other = workloads.make_case(1, 1, 9, 3, seed=65, vbs=[64] * 8 + [41], name="other")
    d, o, lse, k2q_idx, k2q_num = _inputs(c)
    d2, o2, lse2, k2q_idx2, k2q_num2 = _inputs(other)
    extra = dict(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"])

    def call(out):
        return V.backward_noalloc(d["do"], d["q"], d["k"], d["v"], o, lse, k2q_idx, k2q_num,
                                  d["vbs"], out, dq_mode=mode, **extra)

    say(f"[noalloc] graph capture, mode {mode}")
    want = [t.clone() for t in call(_nan_out(d))]  # eager; also resolves the scratch address
    torch.cuda.synchronize()
    out = _nan_out(d)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up call on the capturing stream, as torch advises
        call(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    torch.cuda.synchronize()
    for rep in range(3):
        V.backward_noalloc(d2["do"], d2["q"], d2["k"], d2["v"], o2, lse2, k2q_idx2, k2q_num2,
                           d2["vbs"], _nan_out(d2), dq_mode=mode)
        for t in out:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for name, g, w in zip(("dq", "dk", "dv"), out, want):
            assert torch.equal(g, w), (rep, name)
