"""The C-ABI library loads, exports every call include/psd.h declares, and rejects bad
arguments on the host before launching anything (no GPU needed for these paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "psd.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(psd_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def native():
    from page_selected_sparse_amd import _native
    return _native


def test_exports_every_declared_symbol(native):
    lib = native.lib()
    names = _declared()
    assert set(names) == set(native.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(native):
    lib = native.lib()
    assert lib.psd_version() >= 100
    for code in native.STATUS:
        assert lib.psd_status_string(code)
    assert lib.psd_status_string(-4) == b"selection capacity (b_max) exceeded"


def _shape(native, **kw):
    base = dict(batch=2, num_q_heads=32, num_kv_heads=8, head_dim=128, head_dim_v=128,
                page_size=16, num_blocks=100, max_pages_per_seq=50, dtype=1, reserved=0,
                k_block_stride=16 * 8 * 128, k_token_stride=8 * 128, k_head_stride=128,
                v_block_stride=16 * 8 * 128, v_token_stride=8 * 128, v_head_stride=128)
    base.update(kw)
    return native.PsdShape(**base)


def test_workspace_queries(native):
    lib = native.lib()
    sh = _shape(native)
    assert lib.psd_select_workspace_bytes(ctypes.byref(sh), 10) > 0
    assert lib.psd_decode_workspace_bytes(ctypes.byref(sh), 10) > 0
    assert lib.psd_select_workspace_bytes(ctypes.byref(sh), 1) == 0  # b_max < 2
    bad = _shape(native, head_dim=96, head_dim_v=96)
    assert lib.psd_select_workspace_bytes(ctypes.byref(bad), 10) == 0
    # 1M tokens, b_max 128: the two-level plan must fit
    long = _shape(native, batch=1, max_pages_per_seq=65536, num_blocks=65536)
    assert lib.psd_select_workspace_bytes(ctypes.byref(long), 128) > 0
    # a capacity no plan can hold
    assert lib.psd_select_workspace_bytes(ctypes.byref(long), 60000) == 0


@pytest.mark.parametrize("field,value,code", [
    ("page_size", 32, -1), ("num_q_heads", 30, -1), ("head_dim_v", 64, -2),
    ("num_q_heads", 8 * 20, -2), ("dtype", 7, -1), ("reserved", 1, -1),
    ("head_dim_v", 256, -1), ("batch", 0, -1)])
def test_bad_shapes_rejected(native, field, value, code):
    lib = native.lib()
    sh = _shape(native, **{field: value})
    fake = ctypes.c_void_p(16)  # never dereferenced: the checks fail first
    st = lib.psd_select_pages(ctypes.byref(sh), fake, fake, fake, fake, fake, 10, fake, fake,
                              fake, 1 << 30, None)
    assert st == code


def test_null_and_workspace_errors(native):
    lib = native.lib()
    sh = _shape(native)
    f = ctypes.c_void_p(16)
    assert lib.psd_select_pages(None, f, f, f, f, f, 10, f, f, f, 1 << 30, None) == -1
    assert lib.psd_select_pages(ctypes.byref(sh), None, f, f, f, f, 10, f, f, f, 1 << 30,
                                None) == -1
    assert lib.psd_select_pages(ctypes.byref(sh), f, f, f, f, f, 1, f, f, f, 1 << 30, None) == -1
    assert lib.psd_select_pages(ctypes.byref(sh), f, f, f, f, f, 10, f, f, f, 8, None) == -3
    assert lib.psd_select_pages(ctypes.byref(sh), f, f, f, f, f, 10, f, f, None, 1 << 30,
                                None) == -3
    long = _shape(native, batch=1, max_pages_per_seq=65536, num_blocks=65536)
    assert lib.psd_select_pages(ctypes.byref(long), f, f, f, f, f, 60000, f, f, f, 1 << 40,
                                None) == -4
    # the two selection stages check the same way
    assert lib.psd_select_score(ctypes.byref(sh), f, f, f, f, f, 10, f, f, f, 8, None) == -3
    assert lib.psd_select_score(ctypes.byref(sh), f, f, f, f, f, 1, f, f, f, 1 << 30, None) == -1
    assert lib.psd_select_score(ctypes.byref(sh), f, None, f, f, f, 10, f, f, f, 1 << 30,
                                None) == -1
    assert lib.psd_select_merge(ctypes.byref(sh), f, f, f, f, f, 10, f, f, 8, None) == -3
    assert lib.psd_select_merge(ctypes.byref(sh), f, f, f, None, f, 10, f, f, 1 << 30,
                                None) == -1
    assert lib.psd_select_merge(ctypes.byref(sh), None, f, f, f, f, 10, f, f, 1 << 30,
                                None) == -1
    assert lib.psd_select_merge(ctypes.byref(long), f, f, f, f, f, 60000, f, f, 1 << 40,
                                None) == -4
    # misaligned pointer
    assert lib.psd_page_meta_update(ctypes.byref(sh), ctypes.c_void_p(18), f, f, f, None,
                                    None) == -1
    # strides that overlap heads
    bad = _shape(native, k_head_stride=64)
    assert lib.psd_page_meta_update(ctypes.byref(bad), f, f, f, f, None, None) == -1
    # decode: bad scale, small workspace
    assert lib.psd_dense_decode(ctypes.byref(sh), f, f, f, f, f, 0.0, f, f, 1 << 30, None) == -1
    assert lib.psd_dense_decode(ctypes.byref(sh), f, f, f, f, f, 0.1, f, f, 4, None) == -3
    assert lib.psd_sparse_decode(ctypes.byref(sh), f, f, f, f, f, None, f, 10, 0.1, f, f,
                                 1 << 30, None) == -1


def test_one_call_step_checks(native):
    """psd_select_sparse_decode: workspace covers both stages; the checks of the two calls
    it stands for apply before anything launches."""
    lib = native.lib()
    sh = _shape(native)
    f = ctypes.c_void_p(16)
    ws = lib.psd_select_sparse_decode_workspace_bytes(ctypes.byref(sh), 10)
    assert ws >= lib.psd_select_workspace_bytes(ctypes.byref(sh), 10)
    # past 256 pages per sequence the attention of a two-unit batch takes split partials
    # (whose size both decode plans share at 10 pages): the workspace holds them too
    mid = _shape(native, max_pages_per_seq=512, num_blocks=1100)
    ws_mid = lib.psd_select_sparse_decode_workspace_bytes(ctypes.byref(mid), 10)
    assert ws_mid >= lib.psd_select_workspace_bytes(ctypes.byref(mid), 10)
    assert ws_mid >= lib.psd_decode_workspace_bytes(ctypes.byref(mid), 10)
    assert lib.psd_select_sparse_decode_workspace_bytes(ctypes.byref(sh), 1) == 0
    long = _shape(native, batch=1, max_pages_per_seq=65536, num_blocks=65536)
    assert lib.psd_select_sparse_decode_workspace_bytes(ctypes.byref(long), 60000) == 0
    call = lambda shp, q, k, b_max, scale, out, nbytes: lib.psd_select_sparse_decode(
        shp, q, f, k, f, f, f, f, b_max, scale, f, f, out, f, nbytes, None)
    big = 1 << 30
    assert call(None, f, f, 10, 0.1, f, big) == -1
    assert call(ctypes.byref(sh), None, f, 10, 0.1, f, big) == -1
    assert call(ctypes.byref(sh), f, None, 10, 0.1, f, big) == -1
    assert call(ctypes.byref(sh), f, f, 10, 0.1, None, big) == -1
    assert call(ctypes.byref(sh), f, f, 1, 0.1, f, big) == -1
    assert call(ctypes.byref(sh), f, f, 10, 0.0, f, big) == -1
    assert call(ctypes.byref(sh), f, f, 10, 0.1, f, 8) == -3
    assert call(ctypes.byref(long), f, f, 60000, 0.1, f, 1 << 40) == -4
    assert call(ctypes.byref(_shape(native, head_dim=96, head_dim_v=96)), f, f, 10, 0.1, f,
                big) == -2
    step = lambda shp, meta, b_max, nbytes: lib.psd_decode_step(
        shp, f, meta, f, f, f, f, f, b_max, 0.1, f, f, f, f, nbytes, None)
    assert step(ctypes.byref(sh), None, 10, big) == -1
    assert step(ctypes.byref(sh), ctypes.c_void_p(24), 10, big) == -1  # misaligned
    assert step(ctypes.byref(sh), f, 10, 8) == -3
    assert step(ctypes.byref(long), f, 60000, 1 << 40) == -4


def test_plans_follow_the_batch_shape(native):
    """Host planning, through the workspace queries: whole-unit scoring needs no candidate
    area; small batches keep chunk candidates and split partials; many-head bf16 groups
    keep the certified planes."""
    lib = native.lib()
    q = lambda sh, b: (lib.psd_select_workspace_bytes(ctypes.byref(sh), b),
                       lib.psd_decode_workspace_bytes(ctypes.byref(sh), b))
    ragged = _shape(native, batch=32, max_pages_per_seq=2048, num_blocks=65536)
    sel, dec = q(ragged, 102)
    assert 0 < sel <= 256 * 4 + 512  # 256 units: one scoring workgroup each, no candidates
    assert dec > 0  # sized for the dense walk too (split partials)
    one = _shape(native, batch=1, max_pages_per_seq=2048, num_blocks=2048)
    sel, dec = q(one, 102)
    assert sel >= 8 * 2046 * 12  # every page of the 8 units is a candidate
    assert dec >= 32 * 2 * 128 * 4  # at least two splits of fp32 partials per head
    mla = _shape(native, batch=16, num_q_heads=128, num_kv_heads=1, head_dim=576,
                 head_dim_v=512, max_pages_per_seq=4096, num_blocks=65536,
                 k_block_stride=16 * 576, k_token_stride=576, k_head_stride=576,
                 v_block_stride=16 * 576, v_token_stride=576, v_head_stride=576)
    sel, dec = q(mla, 205)
    assert sel >= 4 * 16 * 4094 * 4  # approximate score, maxima, runner-up, leading tile
    assert dec > 0
    # a wider budget never needs a smaller workspace
    for sh in (one, mla):
        assert q(sh, 400)[0] >= q(sh, 100)[0]


def test_whole_unit_attention_needs_no_partials(native):
    """With 256 units, or rows of at most 256 pages, whole-unit attention (bf16 and fp32,
    D = 64 and 128) keeps no split partials, so the one-call workspace stays small; at 64
    units of longer rows split-K holds them."""
    lib = native.lib()
    one_call = lambda sh: lib.psd_select_sparse_decode_workspace_bytes(ctypes.byref(sh), 102)
    d64 = dict(head_dim=64, head_dim_v=64, k_block_stride=16 * 8 * 64, k_token_stride=8 * 64,
               k_head_stride=64, v_block_stride=16 * 8 * 64, v_token_stride=8 * 64,
               v_head_stride=64)
    for dtype in (0, 1):
        for extra in ({}, d64):
            sh = _shape(native, batch=32, max_pages_per_seq=2048, num_blocks=65536, dtype=dtype,
                        **extra)
            assert 0 < one_call(sh) < 64 * 1024
        few = _shape(native, batch=8, max_pages_per_seq=2048, num_blocks=65536, dtype=dtype)
        assert one_call(few) >= 8 * 32 * 2 * 128 * 4  # B x H_q x (2+ splits) x D_v fp32
        # rows of at most 256 pages take the whole-unit plans at any batch size; one
        # page more and the small batch is back on chunks and split partials
        for b in (1, 8):
            short = _shape(native, batch=b, max_pages_per_seq=256, num_blocks=65536,
                           dtype=dtype)
            assert 0 < one_call(short) < 64 * 1024
            longer = _shape(native, batch=b, max_pages_per_seq=257, num_blocks=65536,
                            dtype=dtype)
            assert one_call(longer) >= b * 32 * 2 * 128 * 4


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU and says so when asked for more."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_unpinned_host_tensors_refused():
    """A host tensor reaches the library only when pinned (mapped for the device)."""
    import torch

    from page_selected_sparse_amd import api

    with pytest.raises(api.PsdError):
        api._ptr(torch.zeros(4))


def test_coverage_selection_checks(native):
    lib = native.lib()
    sh = _shape(native)
    f = ctypes.c_void_p(16)
    need = lib.psd_select_coverage_workspace_bytes(ctypes.byref(sh))
    assert need == 2 * 4 * sh.batch * sh.num_q_heads * sh.max_pages_per_seq
    call = lib.psd_select_pages_coverage
    assert call(None, f, f, f, f, 0.95, 0.1, 10, f, f, f, need, None) == -1
    assert call(ctypes.byref(sh), None, f, f, f, 0.95, 0.1, 10, f, f, f, need, None) == -1
    assert call(ctypes.byref(sh), f, f, f, f, 0.0, 0.1, 10, f, f, f, need, None) == -1
    assert call(ctypes.byref(sh), f, f, f, f, float("nan"), 0.1, 10, f, f, f, need, None) == -1
    assert call(ctypes.byref(sh), f, f, f, f, 0.95, 0.0, 10, f, f, f, need, None) == -1
    assert call(ctypes.byref(sh), f, f, f, f, 0.95, 0.1, 1, f, f, f, need, None) == -1
    assert call(ctypes.byref(sh), f, f, f, f, 0.95, 0.1, 10, f, f, f, need - 4, None) == -3
    assert call(ctypes.byref(sh), f, f, f, f, 0.95, 0.1, 10, f, f, None, need, None) == -3
    # groups of more than 8 query heads, more than 4096 pages, and the latent shape
    for kw in (dict(num_q_heads=sh.num_kv_heads * 16), dict(max_pages_per_seq=4097)):
        big = _shape(native, **kw)
        assert lib.psd_select_coverage_workspace_bytes(ctypes.byref(big)) == 0
        assert call(ctypes.byref(big), f, f, f, f, 0.95, 0.1, 10, f, f, f, 1 << 40, None) == -2


def test_noalloc_step_rejects_oversize_before_touching_the_device(native):
    """psd_decode_step_noalloc checks the step's workspace against its static scratch
    (PSD_SCRATCH_BYTES) first: a step that needs more returns PSD_ERR_SCRATCH without
    launching or even looking the scratch up (no GPU needed)."""
    lib = native.lib()
    sh = _shape(native, batch=128, num_q_heads=128, num_kv_heads=1, head_dim=576,
                head_dim_v=512, num_blocks=65536, max_pages_per_seq=4096,
                k_block_stride=16 * 576, k_token_stride=576, k_head_stride=576,
                v_block_stride=16 * 576, v_token_stride=576, v_head_stride=576)
    assert lib.psd_select_sparse_decode_workspace_bytes(ctypes.byref(sh), 2048) > native.SCRATCH_BYTES
    f = ctypes.c_void_p(16)
    st = lib.psd_decode_step_noalloc(ctypes.byref(sh), f, f, f, f, f, f, f, 2048, 0.04, f, f, f,
                                     None)
    assert st == -6
    assert b"scratch" in lib.psd_status_string(-6)
    # shape errors come back as for the other calls
    bad = _shape(native, page_size=32)
    assert lib.psd_decode_step_noalloc(ctypes.byref(bad), f, f, f, f, f, f, f, 10, 0.1, f, f, f,
                                       None) == -1
    assert lib.psd_decode_step_noalloc(ctypes.byref(_shape(native)), f, f, f, f, f, f, f, 1,
                                       0.1, f, f, f, None) == -1


def test_diag_walk_checks(native):
    """The diagnostic walk refuses bad kinds, missing pointers and shapes it has no build
    for on the host."""
    lib = native.lib()
    sh = _shape(native, batch=2, num_blocks=100)
    f = ctypes.c_void_p(4096)
    walk = lambda shape, kind, k, v, meta, sel, cnt, checksum: lib.psd_diag_walk(
        ctypes.byref(shape), kind, k, v, meta, f, f, sel, cnt, 12, checksum, None)
    assert walk(sh, 2, f, f, f, f, f, f) == -1
    assert walk(sh, 0, f, f, f, f, f, None) == -1
    assert walk(sh, 0, None, f, f, f, f, f) == -1
    assert walk(sh, 0, f, f, f, None, f, f) == -1
    assert walk(sh, 1, f, f, None, f, f, f) == -1
    odd = _shape(native, head_dim=96, head_dim_v=96, k_block_stride=16 * 8 * 96,
                 k_token_stride=8 * 96, k_head_stride=96, v_block_stride=16 * 8 * 96,
                 v_token_stride=8 * 96, v_head_stride=96)
    assert walk(odd, 0, f, f, f, f, f, f) in (-1, -2)


def test_value_tier_queries_and_checks(native):
    """Value tier: state and workspace sizes follow the layout the calls document (page map
    of num_blocks x H_kv words, owner and last-step words per slot; per-entry miss and copy
    lists, a free list per slot); unsupported shapes and bad arguments are refused on the
    host."""
    lib = native.lib()
    al = lambda x: (x + 255) // 256 * 256
    sh = _shape(native, batch=2, num_blocks=100)
    keys = 100 * 8
    assert lib.psd_value_tier_state_bytes(ctypes.byref(sh), 10) == al(keys * 4) + 2 * al(40)
    assert lib.psd_value_tier_state_bytes(ctypes.byref(sh), 0) == al(keys * 4)
    assert lib.psd_value_tier_state_bytes(ctypes.byref(sh), -1) == 0
    entries = 2 * 8 * 12
    assert (lib.psd_value_tier_workspace_bytes(ctypes.byref(sh), 12, 10)
            == 2 * al(entries * 4) + al(40) + 256)
    assert lib.psd_value_tier_workspace_bytes(ctypes.byref(sh), 0, 10) == 0
    latent = _shape(native, num_q_heads=16, num_kv_heads=1, head_dim=576, head_dim_v=512,
                    k_block_stride=16 * 576, k_token_stride=576, k_head_stride=576,
                    v_block_stride=16 * 576, v_token_stride=576, v_head_stride=576)
    assert lib.psd_value_tier_state_bytes(ctypes.byref(latent), 10) == 0
    f = ctypes.c_void_p(4096)
    assert lib.psd_value_tier_reset(ctypes.byref(latent), 10, f, None) == -2
    assert lib.psd_value_tier_reset(ctypes.byref(sh), -1, f, None) == -1
    assert lib.psd_value_tier_reset(ctypes.byref(sh), 10, None, None) == -1
    stage = lambda hot, slots, ws, nbytes: lib.psd_value_tier_stage(
        ctypes.byref(sh), f, hot, f, slots, 1, f, f, f, f, 12, f, f, ws, nbytes, None)
    need = lib.psd_value_tier_workspace_bytes(ctypes.byref(sh), 12, 10)
    assert stage(None, 10, f, need) == -1  # slots without a hot buffer
    assert stage(f, 10, None, need) == -3
    assert stage(f, 10, f, need - 1) == -3
    assert lib.psd_value_tier_stage(ctypes.byref(latent), f, f, f, 10, 1, f, f, f, f, 12, f, f,
                                    f, 1 << 30, None) == -2
    dec = lambda vslot, nbytes: lib.psd_sparse_decode_tiered(
        ctypes.byref(sh), f, f, f, f, vslot, f, f, f, f, 12, 0.1, f, f, nbytes, None)
    assert dec(None, 1 << 30) == -1
    assert dec(f, 8) == -3
    # the KV tier: K pool required, a K hot buffer beside the V one whenever slots exist
    kvstage = lambda k, hot_k, hot_v, slots, ws, nbytes: lib.psd_kv_tier_stage(
        ctypes.byref(sh), k, f, hot_k, hot_v, f, slots, 1, f, f, f, f, 12, f, f, ws, nbytes,
        None)
    assert kvstage(None, f, f, 10, f, need) == -1
    assert kvstage(f, None, f, 10, f, need) == -1
    assert kvstage(f, f, None, 10, f, need) == -1
    assert kvstage(f, f, f, 10, None, need) == -3
    assert kvstage(f, f, f, 10, f, need - 1) == -3
    assert lib.psd_kv_tier_stage(ctypes.byref(latent), f, f, f, f, f, 10, 1, f, f, f, f, 12, f,
                                 f, f, 1 << 30, None) == -2
    kvdec = lambda k, hot_k, hot_v, nbytes: lib.psd_sparse_decode_kv_tiered(
        ctypes.byref(sh), f, k, f, hot_k, hot_v, f, f, f, f, f, 12, 0.1, f, f, nbytes, None)
    assert kvdec(None, f, f, 1 << 30) == -1
    assert kvdec(f, f, None, 1 << 30) == -1  # both hot buffers or neither
    assert kvdec(f, None, f, 1 << 30) == -1
    assert kvdec(f, f, f, 8) == -3
