"""Autotuner host logic (no GPU): space validation and the workspace bound."""
import ctypes

import pytest

from communication_overlap_gemm_amd import _abi as A


def base(op=A.SYNC_OP_AG_GEMM, m=8192, n=1792, k=4096, world=8):
    return A.make_desc(op, m, n, k, world)


def test_tune_workspace_fits_every_candidate():
    b = base()
    space = A.make_tune_space(splits=(1, 2, 4), tiles=((256, 256), (128, 128)))
    need = A.sync_tune_workspace_size(b, space)
    sizes = []
    for s in (1, 2, 4):
        for tm, tn in ((256, 256), (128, 128)):
            sizes.append(A.sync_workspace_size(A.sync_plan(A.make_desc(A.SYNC_OP_AG_GEMM, 8192, 1792, 4096, 8,
                                                                       split=s, tile_m=tm, tile_n=tn))))
    assert need == max(sizes)


@pytest.mark.parametrize("field", ["splits", "tiles", "orders", "copy_cus"])
def test_empty_list_is_rejected(field):
    kw = {"splits": (1,), "tiles": ((256, 256),), "orders": (A.SYNC_ORDER_CHUNK_MAJOR,), "copy_cus": (16,)}
    kw[field] = ()
    sp, keep = A.make_tune_space(**kw)
    assert A.sync_tune_workspace_size(base(), (sp, keep)) == 0
    res = A.sync_tune_result()
    bufs = A.sync_tune_buffers()
    bufs.ws = 256
    rc = A.lib().sync_autotune(ctypes.byref(base()), ctypes.byref(sp), ctypes.byref(bufs), ctypes.byref(res))
    msg = "copy-CU counts or a list of copy agents" if field == "copy_cus" else "at least one entry"
    assert rc == A.SYNC_EINVAL and msg in A.sync_last_error()


def test_attention_is_not_tuned():
    b = A.make_desc(A.SYNC_OP_RING_ATTN, 64, 16, 128, 4, heads_q=4, heads_kv=1)
    sp, keep = A.make_tune_space()
    res, bufs = A.sync_tune_result(), A.sync_tune_buffers()
    bufs.ws = 256
    rc = A.lib().sync_autotune(ctypes.byref(b), ctypes.byref(sp), ctypes.byref(bufs), ctypes.byref(res))
    assert rc == A.SYNC_EINVAL and "GEMM ops" in A.sync_last_error()


def test_unaligned_workspace_is_rejected():
    sp, keep = A.make_tune_space()
    res, bufs = A.sync_tune_result(), A.sync_tune_buffers()
    bufs.ws = 257
    rc = A.lib().sync_autotune(ctypes.byref(base()), ctypes.byref(sp), ctypes.byref(bufs), ctypes.byref(res))
    assert rc == A.SYNC_EINVAL and "256-byte" in A.sync_last_error()


def test_copy_agents_replace_the_copy_cu_list():
    """With agents the copy_cus list may be empty; agents take no run flags,
    no host gates, and only the SDMA, CU, COLOCATED or EPILOGUE backends."""
    ok = (A.make_cfg(A.SYNC_COPY_SDMA, copy_teams=7), A.make_cfg(A.SYNC_COPY_CU, 32, copy_teams=7, copy_kslices=4))
    sp = A.make_tune_space(splits=(1,), tiles=((256, 256),), copy_cus=(), agents=ok)
    assert A.sync_tune_workspace_size(base(), sp) > 0
    for bad in (A.make_cfg(A.SYNC_COPY_HOST_GATED), A.make_cfg(A.SYNC_COPY_PRESET),
                A.make_cfg(A.SYNC_COPY_CU, 16, flags=A.SYNC_RUN_TIMED)):
        sp, keep = A.make_tune_space(splits=(1,), tiles=((256, 256),), copy_cus=(), agents=(bad,))
        res, bufs = A.sync_tune_result(), A.sync_tune_buffers()
        bufs.ws = 256
        rc = A.lib().sync_autotune(ctypes.byref(base()), ctypes.byref(sp), ctypes.byref(bufs), ctypes.byref(res))
        assert rc == A.SYNC_EINVAL and "agents" in A.sync_last_error()
