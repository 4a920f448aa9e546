"""Host-side tests of the C ABI (no GPU needed): the library loads, exports every entry point
the public header declares, sizes workspaces as documented, and rejects bad arguments with the
right status before anything is launched (validation never touches the device)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import block_sparse_attention_attn_amd as V

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")

VSA_OK, VSA_EINVAL, VSA_EUNSUPPORTED, VSA_ELAUNCH = 0, 1, 2, 3

pytestmark = pytest.mark.skipif(not V.is_built(), reason="libvsa.so not built (run build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert "vsa_bwd" in names and "vsa_invert_indices" in names and "vsa_fwd" in names
    handle = ctypes.CDLL(V.library_path())
    for n in names:
        assert hasattr(handle, n), f"libvsa.so does not export {n}"
    # and the binding declares exactly those
    assert sorted(V._SIGNATURES) == names


@pytest.mark.skipif(shutil.which("nm") is None, reason="nm not available")
def test_library_exports_no_unprefixed_c_symbols():
    """Every function the library exports under a plain C name is part of the declared API
    (vsa_*): the host-side helpers have internal linkage, so no generic name (run_stage, ...)
    can clash with a caller's symbols. C++ names are mangled into the vsa namespace."""
    out = subprocess.run(["nm", "-D", "--defined-only", V.library_path()], check=True,
                         capture_output=True, text=True).stdout
    plain = [f[2] for f in (l.split() for l in out.splitlines())
             if len(f) == 3 and f[1] == "T" and not f[2].startswith("_Z")]
    assert plain and all(n.startswith("vsa_") for n in plain), plain
    assert sorted(plain) == _declared_functions()


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    for name, value in (("VSA_ORDER_MIN_KV_BLOCKS", V.ORDER_MIN_KV_BLOCKS),
                        ("VSA_ORDER_BIN_WIDTH", V.ORDER_BIN_WIDTH),
                        ("VSA_CHUNK_MIN_KV_BLOCKS", V.CHUNK_MIN_KV_BLOCKS),
                        ("VSA_CHUNK_BLOCKS", V.CHUNK_BLOCKS),
                        ("VSA_SPILL_CHUNK_BLOCKS", V.SPILL_CHUNK_BLOCKS),
                        ("VSA_FWD_CHUNK_KV_BLOCKS", V.FWD_CHUNK_KV_BLOCKS),
                        ("VSA_FWD_CHUNK_MIN_KV_BLOCKS", V.FWD_CHUNK_MIN_KV_BLOCKS)):
        m = re.search(r"#define\s+" + name + r"\s+(\d+)", text)
        assert m and int(m.group(1)) == value, name
    m = re.search(r"#define\s+VSA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == V.NOALLOC_SCRATCH_BYTES


def test_status_strings():
    L = V.lib()
    for st, word in ((0, b"OK"), (1, b"EINVAL"), (2, b"EUNSUPPORTED"), (3, b"ELAUNCH")):
        assert word in L.vsa_status_string(st)
    assert b"unknown" in L.vsa_status_string(42)


def _a256(x):
    return (x + 255) // 256 * 256


def _tail(B, H, S, spill):
    """Bytes of the regions every backward uses after the mode- and chunk-dependent ones: block
    statistics, head scales, the fp16 copies of q, k, dO (and v in recompute mode)."""
    copy = _a256(B * H * S * 128 * 2)
    return _a256(B * H * (S // 64) * 8 * 4) + _a256(B * H * 8 * 4) + (3 if spill else 4) * copy


def test_workspace_sizes_and_layout():
    B, H, S = 1, 8, 32768
    nb = S // 64
    # derived q2k, recompute mode
    offs = [V.bwd_workspace_offset(B, H, S, r) for r in range(V.WS_END + 1)]
    assert offs[V.WS_LSE_DELTA] == 0
    assert offs[V.WS_KV_ORDER] == B * H * S * 2 * 4
    assert offs[V.WS_Q_ORDER] == offs[V.WS_KV_ORDER] + B * H * nb * 4
    assert offs[V.WS_Q2K_NUM] == offs[V.WS_Q_ORDER] + B * H * nb * 4
    assert offs[V.WS_Q2K_IDX] == offs[V.WS_Q2K_NUM] + B * H * nb * 4
    assert offs[V.WS_BITMAP] == offs[V.WS_Q2K_IDX] + B * H * nb * nb * 4
    assert offs[V.WS_KBASE] == offs[V.WS_BITMAP] + B * H * nb * ((nb + 31) // 32) * 4
    assert offs[V.WS_KBASE] == offs[V.WS_QENT] == offs[V.WS_DS] == offs[V.WS_STATS]
    assert offs[V.WS_SCALES] == offs[V.WS_STATS] + B * H * nb * 8 * 4
    assert offs[V.WS_Q16] == offs[V.WS_SCALES] + 256
    assert offs[V.WS_K16] == offs[V.WS_Q16] + B * H * S * 128 * 2
    assert offs[V.WS_DO16] == offs[V.WS_K16] + B * H * S * 128 * 2
    assert offs[V.WS_V16] == offs[V.WS_DO16] + B * H * S * 128 * 2
    assert offs[V.WS_END] == offs[V.WS_V16] + B * H * S * 128 * 2
    assert offs[V.WS_END] - offs[V.WS_STATS] == _tail(B, H, S, False)
    assert V.bwd_workspace_bytes(B, H, S) == offs[V.WS_END]
    # given q2k lists (row width 128): no derivation regions
    given = [V.bwd_workspace_offset(B, H, S, r, 128) for r in range(V.WS_END + 1)]
    assert given[V.WS_Q2K_NUM] == given[V.WS_STATS] == offs[V.WS_Q2K_NUM]
    assert V.bwd_workspace_bytes(B, H, S, 128) == offs[V.WS_Q2K_NUM] + _tail(B, H, S, False)
    # spill mode: slot bases, the slot table and one 8 KiB dS tile per possible pair
    sp = [V.bwd_workspace_offset(B, H, S, r, 128, V.DQ_SPILL) for r in range(V.WS_END + 1)]
    assert sp[V.WS_KBASE] == offs[V.WS_Q2K_NUM]
    assert sp[V.WS_QENT] == sp[V.WS_KBASE] + B * H * nb * 4
    assert sp[V.WS_DS] == sp[V.WS_QENT] + B * H * nb * 128 * 8
    assert sp[V.WS_STATS] == sp[V.WS_DS] + B * H * nb * 128 * 64 * 64 * 2
    assert sp[V.WS_END] - sp[V.WS_STATS] == _tail(B, H, S, True)  # no fp16 copy of v
    assert sp[V.WS_V16] == sp[V.WS_END]
    # derived q2k in spill mode: row width nb for the slot table and tiles
    spd = [V.bwd_workspace_offset(1, 2, 64 * 5, r, 0, V.DQ_SPILL) for r in range(V.WS_END + 1)]
    assert spd[V.WS_STATS] - spd[V.WS_DS] == 2 * 5 * 5 * 8192
    # every region starts on a 256-byte boundary, also for odd sizes
    for kq in (0, 3):
        for mode in (V.DQ_RECOMPUTE, V.DQ_SPILL):
            assert all(V.bwd_workspace_offset(1, 3, 64 * 5, r, kq, mode) % 256 == 0
                       for r in range(V.WS_END + 1))
    assert V.bwd_workspace_bytes(0, 1, 64) == 0
    assert V.bwd_workspace_bytes(1, 1, 64, 0, 7) == 0  # unknown mode


def test_workspace_chunk_regions():
    def offs(B, H, S, kq, chunk):
        return [V.bwd_workspace_offset(B, H, S, r, kq, V.DQ_RECOMPUTE, chunk)
                for r in range(V.WS_END + 1)]
    a256 = lambda x: (x + 255) // 256 * 256
    # below the default threshold: no chunk regions
    o = offs(1, 8, 64 * 512, 128, 0)
    assert o[V.WS_CHUNK_BOUNDS] == o[V.WS_DKV_PART] == o[V.WS_STATS] == o[V.WS_DS]
    # from the threshold on, chunks of CHUNK_BLOCKS q blocks for the kv-major kernel: bounds and
    # fp32 dV/dK sums; the q-major kernel's chunks only on request
    nb = V.CHUNK_MIN_KV_BLOCKS
    o = offs(1, 2, 64 * nb, 128, 0)
    c = -(-nb // V.CHUNK_BLOCKS)
    assert o[V.WS_DKV_PART] - o[V.WS_CHUNK_BOUNDS] == a256(2 * nb * (c + 1) * 4)
    assert o[V.WS_STATS] == o[V.WS_DQ_BOUNDS] == o[V.WS_DKV_PART] + 2 * nb * 2 * 64 * 128 * 4
    assert V.bwd_workspace_bytes(1, 2, 64 * nb, 128, V.DQ_RECOMPUTE, -1) == (
        o[V.WS_CHUNK_BOUNDS] + _tail(1, 2, 64 * nb, False))
    o = offs(1, 2, 64 * nb, 128, V.CHUNK_BLOCKS)  # requested: both kernels
    assert o[V.WS_DQ_PART] - o[V.WS_DQ_BOUNDS] == a256(2 * nb * (c + 1) * 4)
    assert o[V.WS_STATS] - o[V.WS_DQ_PART] == 2 * nb * 64 * 128 * 4
    # spill mode: no dQ chunk regions (the dS-reading q-major kernel runs once per chunk), and a
    # chunked spill: C rows of slot bases, one chunk's tiles (R x K' per head)
    sp = [V.bwd_workspace_offset(1, 2, 64 * nb, r, 128, V.DQ_SPILL, 0) for r in range(V.WS_END + 1)]
    cs = -(-nb // V.SPILL_CHUNK_BLOCKS)  # the library's chunks are narrower with the spill
    assert sp[V.WS_DKV_PART] - sp[V.WS_CHUNK_BOUNDS] == a256(2 * nb * (cs + 1) * 4)
    assert sp[V.WS_DQ_BOUNDS] == sp[V.WS_STATS] == sp[V.WS_DKV_PART] + 2 * nb * 2 * 64 * 128 * 4
    assert sp[V.WS_QENT] - sp[V.WS_KBASE] == a256(cs * 2 * nb * 4)
    assert sp[V.WS_CHUNK_BOUNDS] - sp[V.WS_DS] == 2 * V.SPILL_CHUNK_BLOCKS * 128 * 8192
    un = [V.bwd_workspace_offset(1, 2, 64 * nb, r, 128, V.DQ_SPILL, -1) for r in range(V.WS_END + 1)]
    assert un[V.WS_QENT] - un[V.WS_KBASE] == a256(2 * nb * 4)
    assert un[V.WS_CHUNK_BOUNDS] - un[V.WS_DS] == 2 * nb * 128 * 8192
    # a forced width at a small size: ceil(10 / 3) = 4 chunks, tiles for 3 q blocks x 7 per head
    sp = [V.bwd_workspace_offset(1, 2, 64 * 10, r, 7, V.DQ_SPILL, 3) for r in range(V.WS_END + 1)]
    assert sp[V.WS_QENT] - sp[V.WS_KBASE] == a256(4 * 2 * 10 * 4)
    assert sp[V.WS_CHUNK_BOUNDS] - sp[V.WS_DS] == a256(2 * 3 * 7 * 8192)
    # a forced chunk size at any size; one chunk covering every block is no chunk
    o = offs(1, 1, 64 * 10, 0, 3)
    assert o[V.WS_DKV_PART] - o[V.WS_CHUNK_BOUNDS] == a256(10 * 5 * 4)
    assert o[V.WS_DQ_BOUNDS] - o[V.WS_DKV_PART] == 10 * 2 * 64 * 128 * 4
    assert o[V.WS_STATS] - o[V.WS_DQ_PART] == 10 * 64 * 128 * 4
    o = offs(1, 1, 64 * 10, 0, 10)
    assert o[V.WS_STATS] == o[V.WS_CHUNK_BOUNDS]
    # the forward: per-head max |v| bits and the fp16 copy of v, then with kv-range chunks the
    # bounds, per-wave state of 66 x 64 floats and the work order
    def v16(bh, S):
        return a256(bh * 4) + a256(bh * (S // 64) * 4) + a256(bh * S * 128 * 2)
    nbf = V.FWD_CHUNK_MIN_KV_BLOCKS
    cf = -(-nbf // V.FWD_CHUNK_KV_BLOCKS)
    # (from VSA_ORDER_MIN_KV_BLOCKS kv blocks on, the chunks' int32 work order follows)
    assert V.fwd_workspace_bytes(1, 2, 64 * nbf) == (v16(2, 64 * nbf) + a256(2 * nbf * (cf + 1) * 4)
                                                     + 2 * nbf * 4 * 66 * 64 * 4 + a256(2 * nbf * 4))
    assert V.fwd_workspace_bytes(1, 2, 64 * nbf, -1) == v16(2, 64 * nbf)
    assert V.fwd_workspace_bytes(1, 2, 64 * (nbf - 1)) == v16(2, 64 * (nbf - 1))
    assert V.fwd_workspace_bytes(1, 1, 64 * 10, 4) == (v16(1, 640) + a256(10 * 4 * 4)
                                                       + 10 * 4 * 66 * 64 * 4)
    assert V.fwd_workspace_bytes(1, 1, 64 * 80, 16) == (v16(1, 64 * 80) + a256(80 * 6 * 4)
                                                        + 80 * 4 * 66 * 64 * 4 + a256(80 * 4))
    assert V.fwd_workspace_bytes(1, 1, 63) == 0
    assert V.invert_workspace_bytes(2, 3, 100, 50) == ((2 * 3 * 50 * 4 * 4 + 255) // 256) * 256
    assert V.invert_workspace_bytes(1, 1, 0, 1) == 0


def _bwd_args(**over):
    fake = 0x10000  # never dereferenced: validation fails or we do not launch
    a = dict(q=fake, k=fake, v=fake, o=fake, dout=fake, lse=fake, k2q_idx=fake, k2q_num=fake,
             q2k_idx=None, q2k_num=None, vbs=fake, order=None, dq=fake, dk=fake, dv=fake,
             workspace=fake, workspace_bytes=V.bwd_workspace_bytes(1, 2, 256), batch=1,
             heads=2, seqlen=256, head_dim=128, num_kv_blocks=4, max_q_blocks=4, q2k_stride=0,
             sm_scale=0.088, dq_mode=V.DQ_RECOMPUTE)
    a.update(over)
    return V._BwdArgs(**a)


def _check(args):
    return V.lib().vsa_bwd_check(ctypes.byref(args))


def test_bwd_check_accepts_a_valid_call():
    assert _check(_bwd_args()) == VSA_OK
    # odd block counts are fine
    assert _check(_bwd_args(num_kv_blocks=3, seqlen=192,
                            workspace_bytes=V.bwd_workspace_bytes(1, 2, 192))) == VSA_OK
    # given q2k lists need less workspace
    small = V.bwd_workspace_bytes(1, 2, 256, 2)
    assert _check(_bwd_args(q2k_idx=0x10000, q2k_num=0x10000, q2k_stride=2,
                            workspace_bytes=small)) == VSA_OK
    assert _check(_bwd_args(workspace_bytes=small)) == VSA_EINVAL
    # the dS spill needs its tiles' room
    spill = V.bwd_workspace_bytes(1, 2, 256, 2, V.DQ_SPILL)
    assert _check(_bwd_args(q2k_idx=0x10000, q2k_num=0x10000, q2k_stride=2, workspace_bytes=spill,
                            dq_mode=V.DQ_SPILL)) == VSA_OK
    assert _check(_bwd_args(q2k_idx=0x10000, q2k_num=0x10000, q2k_stride=2, workspace_bytes=small,
                            dq_mode=V.DQ_SPILL)) == VSA_EINVAL
    assert _check(_bwd_args(dq_mode=2)) == VSA_EINVAL


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=64), VSA_EUNSUPPORTED),
    (dict(seqlen=250), VSA_EINVAL),
    (dict(num_kv_blocks=0, seqlen=0), VSA_EINVAL),
    (dict(batch=0), VSA_EINVAL),
    (dict(heads=-1), VSA_EINVAL),
    (dict(max_q_blocks=0), VSA_EINVAL),
    (dict(sm_scale=float("nan")), VSA_EINVAL),
    (dict(sm_scale=float("inf")), VSA_EINVAL),
    (dict(sm_scale=0.0), VSA_EINVAL),
    (dict(sm_scale=-1e-37), VSA_EINVAL),
    (dict(q=None), VSA_EINVAL),
    (dict(lse=None), VSA_EINVAL),
    (dict(k2q_idx=None), VSA_EINVAL),
    (dict(vbs=None), VSA_EINVAL),
    (dict(dv=None), VSA_EINVAL),
    (dict(workspace=None), VSA_EINVAL),
    (dict(workspace_bytes=1024), VSA_EINVAL),
    (dict(q2k_idx=0x10000), VSA_EINVAL),
    (dict(q2k_idx=0x10000, q2k_num=0x10000, q2k_stride=0), VSA_EINVAL),
])
def test_bwd_check_rejects(over, status):
    assert _check(_bwd_args(**over)) == status
    assert V.lib().vsa_last_error() != b""


def test_bwd_and_stage_fail_before_launch_on_bad_args():
    L = V.lib()
    a = _bwd_args(head_dim=96)
    assert L.vsa_bwd(ctypes.byref(a), None) == VSA_EUNSUPPORTED
    assert L.vsa_bwd_stage(ctypes.byref(a), 2, None) == VSA_EUNSUPPORTED
    assert L.vsa_bwd_stage(ctypes.byref(_bwd_args()), 4, None) == VSA_EINVAL
    assert L.vsa_bwd_stage(ctypes.byref(_bwd_args()), -1, None) == VSA_EINVAL


def test_fwd_check():
    fake = 0x10000
    need = V.fwd_workspace_bytes(1, 1, 256)
    base = dict(q=fake, k=fake, v=fake, q2k_idx=fake, q2k_num=fake, vbs=fake, o=fake, lse=fake,
                batch=1, heads=1, seqlen=256, head_dim=128, num_kv_blocks=4, q2k_stride=2,
                sm_scale=0.088, workspace=fake, workspace_bytes=need)
    L = V.lib()
    assert L.vsa_fwd_check(ctypes.byref(V._FwdArgs(**base))) == VSA_OK
    for over, st in ((dict(head_dim=256), VSA_EUNSUPPORTED), (dict(q2k_stride=0), VSA_EINVAL),
                     (dict(o=None), VSA_EINVAL), (dict(seqlen=255), VSA_EINVAL),
                     (dict(workspace=None), VSA_EINVAL), (dict(workspace_bytes=need - 1), VSA_EINVAL)):
        assert L.vsa_fwd_check(ctypes.byref(V._FwdArgs(**{**base, **over}))) == st
        assert L.vsa_fwd(ctypes.byref(V._FwdArgs(**{**base, **over})), None) == st


def test_invert_and_order_validation():
    L = V.lib()
    fake = 0x10000
    assert L.vsa_invert_indices(fake, fake, 1, 1, 0, 2, 4, fake, fake, fake, 1 << 20, None) == VSA_EINVAL
    assert L.vsa_invert_indices(None, fake, 1, 1, 4, 2, 4, fake, fake, fake, 1 << 20, None) == VSA_EINVAL
    assert L.vsa_invert_indices(fake, fake, 1, 1, 4, 2, 4, fake, fake, fake, 0, None) == VSA_EINVAL
    assert L.vsa_bwd_order(fake, 1, 1, 20000, 8, fake, None) == VSA_EUNSUPPORTED
    assert L.vsa_bwd_order(fake, 1, 1, 1024, 0, fake, None) == VSA_EINVAL
    assert L.vsa_bwd_order(None, 1, 1, 1024, 8, fake, None) == VSA_EINVAL


def test_python_layer_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16)
    vbs = torch.full((1,), 64, dtype=torch.int32)
    assert not V.is_supported(q, vbs)
    with pytest.raises(RuntimeError, match="GPU"):
        V.forward(q, q, q, torch.zeros(1, 1, 1, 1, dtype=torch.int32),
                  torch.ones(1, 1, 1, dtype=torch.int32), vbs)
