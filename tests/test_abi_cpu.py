"""The C-ABI library loads without a GPU, exports every entry point the header
declares, and its CPU-side argument checks reject bad input."""
import ctypes
import os
import re

import pytest

from communication_overlap_gemm_amd import _abi as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sync_overlap.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sync_[a-z_]+)\s*\(", text)))


def test_header_declares_the_bound_names():
    assert sorted(A.EXPORTED_SYMBOLS) == _declared()


@pytest.mark.parametrize("name", _declared())
def test_library_exports_symbol(name):
    lib = ctypes.CDLL(A.LIB_PATH)
    assert hasattr(lib, name)


@pytest.mark.parametrize("bad,msg", [
    (dict(m=10, world=4), "divisible"),
    (dict(split=0), "split"),
    (dict(split=99), "split"),
    (dict(rank=-1), "rank"),
    (dict(ring_dir=2), "ring_dir"),
    (dict(op=7), "op"),
    (dict(tile_order=9), "tile_order"),
    (dict(b_layout=3), "b_layout"),
    (dict(pattern=1, explicit_order=[0, 1, 1, 2]), "permutation"),
    (dict(pattern=1), "explicit_order"),
    (dict(m=0), "positive"),              # empty problems are rejected, not run as no-ops
    (dict(n=0), "positive"),
    (dict(k=0), "positive"),
    (dict(n=-8), "positive"),
    (dict(world=0), "world"),
    (dict(tile_m=0), "tile_m"),
])
def test_plan_rejects(bad, msg):
    kw = dict(op=1, m=8, n=8, k=64, world=4, tile_m=2, tile_n=2)
    kw.update(bad)
    with pytest.raises(A.SyncError) as ei:
        A.sync_plan(A.make_desc(**kw))
    assert ei.value.code == A.SYNC_EINVAL and msg in ei.value.message


def test_reserved_must_be_zero():
    d = A.make_desc(1, 8, 8, 64, 4, tile_m=2, tile_n=2)
    d.reserved[0] = 5
    with pytest.raises(A.SyncError):
        A.sync_plan(d)


def test_null_arguments():
    lib = A.lib()
    assert lib.sync_plan(None, None) == A.SYNC_EINVAL
    assert lib.sync_plan_get_info(None, None) == A.SYNC_EINVAL
    assert lib.sync_workspace_size(None) == 0
    assert lib.sync_ag_gemm(None, None, None, None, None, None, 0, None, None, None) == A.SYNC_EINVAL
    assert lib.sync_gemm_rs(None, None, None, None, None, 0, None, None, None, None) == A.SYNC_EINVAL
    assert "plan" in A.sync_last_error()


def test_wrong_op_for_plan():
    p = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, 8, 8, 64, 4, tile_m=2, tile_n=2))
    rc = A.lib().sync_ag_gemm(p.handle, None, None, None, None, None, 0, 256, None, None)
    assert rc == A.SYNC_EINVAL and "different op" in A.sync_last_error()


def test_workspace_size_scales_with_chunks():
    p1 = A.sync_plan(A.make_desc(1, 64, 8, 64, 4, split=1, tile_m=2, tile_n=2))
    p2 = A.sync_plan(A.make_desc(1, 4096, 8, 64, 4, split=256, tile_m=2, tile_n=2))
    # header + four uint32[C] arrays + uint32[C][16], the K-sliced copy's two
    # uint32[C][8] and uint32[C][8][16], then the trace: uint64[T][4] and
    # uint64[C][2]; each array padded to 256 bytes
    assert A.sync_workspace_size(p1) == 256 + 4 * 256 + 256 + 2 * 256 + 2048 + 128 * 32 + 256
    assert A.sync_workspace_size(p2) == (256 + 4 * 4096 + 1024 * 64 + 2 * 1024 * 32 + 1024 * 512 + 8192 * 32
                                         + 1024 * 16)


def test_withhold_and_trace_validation():
    p = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, 64, 8, 64, 4, split=1, tile_m=128, tile_n=128))
    bad = A.make_cfg(A.SYNC_COPY_CU, copy_cus=8, flags=A.SYNC_RUN_WITHHOLD, withhold_chunk=9)
    rc = A.lib().sync_ag_gemm(p.handle, ctypes.byref(bad), None, None, None, None, 0, 256, None, None)
    assert rc == A.SYNC_EINVAL and "withhold_chunk" in A.sync_last_error()
    sdma = A.make_cfg(A.SYNC_COPY_SDMA, flags=A.SYNC_RUN_WITHHOLD, withhold_chunk=1)
    rc = A.lib().sync_ag_gemm(p.handle, ctypes.byref(sdma), None, None, None, None, 0, 256, None, None)
    assert rc == A.SYNC_EINVAL and "WITHHOLD" in A.sync_last_error()
    pa = A.sync_plan(A.make_desc(A.SYNC_OP_RING_ATTN, 64, 16, 128, 4, heads_q=4, heads_kv=1))
    tr = A.make_cfg(A.SYNC_COPY_CU, copy_cus=8, flags=A.SYNC_RUN_TRACE)
    rc = A.lib().sync_ring_attn_step(pa.handle, ctypes.byref(tr), *([None] * 9), 1.0, 0, 256, None, None)
    assert rc == A.SYNC_EINVAL and "TRACE" in A.sync_last_error()


def test_kslices_validation():
    """copy_kslices is checked before any device work: range, op, backend, and
    at least four 64-deep K steps per slice."""
    def rc_of(plan, cfg):
        return A.lib().sync_ag_gemm(plan.handle, ctypes.byref(cfg), None, None, None, None, 0, 256, None, None)
    nk = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, 1024, 256, 1024, 4, tile_m=256, tile_n=256, b_layout=A.SYNC_B_NK))
    assert rc_of(nk, A.make_cfg(A.SYNC_COPY_CU, 8, copy_kslices=9)) == A.SYNC_EINVAL
    assert "[0, 8]" in A.sync_last_error()
    assert rc_of(nk, A.make_cfg(A.SYNC_COPY_CU, 8, copy_kslices=-1)) == A.SYNC_EINVAL
    assert rc_of(nk, A.make_cfg(A.SYNC_COPY_CU, 8, copy_kslices=5)) == A.SYNC_EINVAL  # 1024/64 = 16 < 20
    assert "K/64" in A.sync_last_error()
    assert rc_of(nk, A.make_cfg(A.SYNC_COPY_SDMA, copy_kslices=2)) == A.SYNC_EINVAL
    assert "COLOCATED" in A.sync_last_error()
    rs = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, 1024, 256, 1024, 4, tile_m=256, tile_n=256, b_layout=A.SYNC_B_NK))
    rc = A.lib().sync_gemm_rs(rs.handle, ctypes.byref(A.make_cfg(A.SYNC_COPY_CU, 8, copy_kslices=2)), None, None,
                              None, 0, None, 256, None, None)
    assert rc == A.SYNC_EINVAL and "AG-GEMM" in A.sync_last_error()


def test_link_pacing_validation():
    """copy_link_gbps: 0 or within [1, 10000], and only for the CU backend."""
    def rc_of(plan, cfg):
        return A.lib().sync_ag_gemm(plan.handle, ctypes.byref(cfg), None, None, None, None, 0, 256, None, None)
    p = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, 1024, 256, 1024, 4, tile_m=256, tile_n=256, b_layout=A.SYNC_B_NK))
    for bad in (0.5, -3.0, 20000.0, float("nan")):
        assert rc_of(p, A.make_cfg(A.SYNC_COPY_CU, 8, copy_link_gbps=bad)) == A.SYNC_EINVAL
        assert "copy_link_gbps" in A.sync_last_error()
    assert rc_of(p, A.make_cfg(A.SYNC_COPY_COLOCATED, copy_link_gbps=100.0)) == A.SYNC_EINVAL
    assert "CU backend" in A.sync_last_error()


def test_epilogue_backend_is_for_gemm_rs():
    p = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, 1024, 256, 1024, 4, tile_m=256, tile_n=256, b_layout=A.SYNC_B_NK))
    rc = A.lib().sync_ag_gemm(p.handle, ctypes.byref(A.make_cfg(A.SYNC_COPY_EPILOGUE)), None, None, None, None, 0,
                              256, None, None)
    assert rc == A.SYNC_EUNSUPPORTED and "EPILOGUE" in A.sync_last_error()


def test_host_gated_backend_is_withdrawn():
    """HOST_GATED is rejected before any device work, for every launch call."""
    p = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, 1024, 256, 1024, 4, tile_m=256, tile_n=256))
    cfg = A.make_cfg(A.SYNC_COPY_HOST_GATED)
    rc = A.lib().sync_ag_gemm(p.handle, ctypes.byref(cfg), None, None, None, None, 0, 256, None, None)
    assert rc == A.SYNC_EUNSUPPORTED and "withdrawn" in A.sync_last_error()
    rs = A.sync_plan(A.make_desc(A.SYNC_OP_GEMM_RS, 1024, 256, 1024, 4, tile_m=256, tile_n=256))
    rc = A.lib().sync_gemm_rs(rs.handle, ctypes.byref(cfg), None, None, None, 0, None, 256, None, None)
    assert rc == A.SYNC_EUNSUPPORTED and "withdrawn" in A.sync_last_error()


def test_binding_checks_tensor_sizes():
    """The binding refuses tensors that are not on a GPU, not contiguous, of
    the wrong element size or too small for the plan, before the library sees
    them (a short tensor would otherwise be read or written past its end)."""
    torch = pytest.importorskip("torch")
    p = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, 256, 128, 64, 4, tile_m=128, tile_n=128))
    host = torch.zeros(256 * 64, dtype=torch.int16)
    with pytest.raises(A.SyncError) as ei:
        A.sync_ag_gemm(p, None, host, 0x1000, 0x1000, 0x1000, A.SYNC_DTYPE_F32, 0x1000)
    assert ei.value.code == A.SYNC_EINVAL and "device tensor" in ei.value.message

    class FakeDev:  # the attributes the checks read, without a GPU
        is_cuda = True

        def __init__(self, n, elem, contiguous=True):
            self.n, self.elem, self.contig = n, elem, contiguous

        def data_ptr(self):
            return 0x1000

        def is_contiguous(self):
            return self.contig

        def element_size(self):
            return self.elem

        def numel(self):
            return self.n

    for bad, msg in ((FakeDev(256 * 64 - 1, 2), "elements"), (FakeDev(256 * 64, 4), "2-byte"),
                     (FakeDev(256 * 64, 2, contiguous=False), "contiguous")):
        with pytest.raises(A.SyncError) as ei:
            A.sync_ag_gemm(p, None, None, bad, 0x1000, 0x1000, A.SYNC_DTYPE_F32, 0x1000)
        assert ei.value.code == A.SYNC_EINVAL and msg in ei.value.message
    with pytest.raises(A.SyncError) as ei:  # fp32 C needs 4-byte elements
        A.sync_ag_gemm(p, None, None, 0x1000, 0x1000, FakeDev(256 * 128, 2), A.SYNC_DTYPE_F32, 0x1000)
    assert "c must have 4-byte" in ei.value.message


def test_lead_slice_validation():
    """copy_lead_slice: 0 or in [1, copy_kslices] with copy_kslices > 1, and
    only for AG-GEMM with the CU backend and no pacing."""
    def rc_of(plan, cfg):
        return A.lib().sync_ag_gemm(plan.handle, ctypes.byref(cfg), None, None, None, None, 0, 256, None, None)
    p = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, 1024, 256, 1024, 4, tile_m=256, tile_n=256, b_layout=A.SYNC_B_NK))
    for bad in (A.make_cfg(A.SYNC_COPY_CU, 8, copy_kslices=2, copy_lead_slice=3),
                A.make_cfg(A.SYNC_COPY_CU, 8, copy_kslices=1, copy_lead_slice=1),
                A.make_cfg(A.SYNC_COPY_CU, 8, copy_kslices=4, copy_lead_slice=-1),
                A.make_cfg(A.SYNC_COPY_CU, 8, copy_lead_slice=1),
                A.make_cfg(A.SYNC_COPY_COLOCATED, copy_kslices=2, copy_lead_slice=1),
                A.make_cfg(A.SYNC_COPY_CU, 8, copy_kslices=2, copy_lead_slice=1, copy_link_gbps=100.0)):
        assert rc_of(p, bad) == A.SYNC_EINVAL
        assert "copy_lead_slice" in A.sync_last_error()


def test_split_baseline_validation():
    """sync_gemm_split: a GEMM plan, a copy stream, a runtime-copy backend and
    no run flags; checked before any device work."""
    lib = A.lib()
    ag = A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, 1024, 256, 1024, 4, tile_m=256, tile_n=256))
    at = A.sync_plan(A.make_desc(A.SYNC_OP_RING_ATTN, 64, 16, 128, 4, heads_q=4, heads_kv=1))
    args = (0x1000, 0x1000, 0x1000, 0x1000, 0, None, 256)
    assert lib.sync_gemm_split(None, None, *args, None, 0x10) == A.SYNC_EINVAL
    assert lib.sync_gemm_split(at.handle, None, *args, None, 0x10) == A.SYNC_EINVAL
    assert "GEMM plan" in A.sync_last_error()
    assert lib.sync_gemm_split(ag.handle, None, *args, None, None) == A.SYNC_EINVAL
    assert "copy stream" in A.sync_last_error()
    for bad in (A.make_cfg(A.SYNC_COPY_COLOCATED), A.make_cfg(A.SYNC_COPY_CU, 16, flags=A.SYNC_RUN_TIMED)):
        assert lib.sync_gemm_split(ag.handle, ctypes.byref(bad), *args, None, 0x10) == A.SYNC_EINVAL


def test_head_attn_validation():
    """sync_head_attn: a HEAD_ATTN plan whose queries are every token, no
    trace mode; checked before any device work."""
    lib = A.lib()
    with pytest.raises(A.SyncError) as ei:
        A.sync_plan(A.make_desc(A.SYNC_OP_HEAD_ATTN, 48, 16, 128, 4, tile_m=64, heads_q=4, heads_kv=1))
    assert ei.value.code == A.SYNC_EINVAL and "every token" in ei.value.message
    hp = A.sync_plan(A.make_desc(A.SYNC_OP_HEAD_ATTN, 64, 16, 128, 4, tile_m=64, heads_q=4, heads_kv=1))
    at = A.sync_plan(A.make_desc(A.SYNC_OP_RING_ATTN, 64, 16, 128, 4, heads_q=4, heads_kv=1))
    args = [0x1000] * 8
    assert lib.sync_head_attn(at.handle, None, *args, 1.0, 256, None, None) == A.SYNC_EINVAL
    assert "different op" in A.sync_last_error()
    tr = A.make_cfg(A.SYNC_COPY_CU, copy_cus=8, flags=A.SYNC_RUN_TRACE)
    assert lib.sync_head_attn(hp.handle, ctypes.byref(tr), *args, 1.0, 256, None, None) == A.SYNC_EINVAL
    assert "TRACE" in A.sync_last_error()
    info = A.sync_plan_get_info(hp)
    assert info.num_chunks == 4 and info.num_tiles == 4


def test_attn_query_block():
    """The query rows of one attention work item: a multiple of 32 that
    halves as the query heads per item double (up to 4), 0 for groupings the
    kernel has no variant for.  Plans of op HEAD_ATTN must use it as tile_m."""
    qb = A.sync_attn_query_block
    base = qb(4, 1)
    assert base > 0 and base % 32 == 0
    assert qb(8, 2) == qb(16, 1) == qb(32, 8) == base
    assert qb(2, 1) == qb(4, 2) == 2 * base and qb(1, 1) == qb(8, 8) == 4 * base
    for hq, hkv in ((3, 1), (6, 1), (4, 3), (0, 1), (4, 0), (-4, 1)):
        assert qb(hq, hkv) == 0
