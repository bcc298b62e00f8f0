"""The C-ABI library loads on a machine without a GPU, exports every entry
point the header declares, and rejects bad arguments on the host before any
HIP call."""
import ctypes
import os
import re

import pytest

import block_sparse_long_pooled_amd as bslp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(bslp.LIB_PATH),
                                reason="libbslp.so not built")


def header_functions():
    text = open(os.path.join(ROOT, "include", "bslp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bslp_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = bslp.load_library()
    names = header_functions()
    assert set(names) == set(bslp.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None


def _problem(**kw):
    args = dict(dtype="bf16", hq=8, hkv=2, head_dim=128, block_size=128, seqlens=[1000, 300])
    args.update(kw)
    return bslp.make_problem(**args)


def test_sizes_match_the_layout():
    p = _problem()
    s = bslp.get_sizes(p)
    N = [8, 3]
    assert s.total_tokens == 1300
    assert s.pooled_rows == sum(N)
    assert s.num_segments == 2 * sum(N)
    assert s.score_elems == 2 * sum(n * (n + 1) // 2 for n in N)
    # bf16 copies of the pooled keys and values for the correction steps, then
    # the work-unit list (an int32 per segment x row block: g*B = 512 rows, 2
    # row blocks of 256) and its 12 queue words
    assert s.workspace_bytes == 3 * s.pooled_rows * 2 * 128 * 2 + (s.num_segments * 2 + 12) * 4


def _status(fn):
    with pytest.raises(bslp.BslpError) as e:
        fn()
    return e.value.status, e.value.detail


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 1),
    (dict(hq=6, hkv=4), 1),
    (dict(hq=0), 1),
    (dict(hq=34, hkv=2), 2),
    (dict(head_dim=96), 2),
    (dict(block_size=32), 2),
    (dict(softmax_scale=float("nan")), 1),
    (dict(softmax_scale=-1.0), 1),
    (dict(q_scale=2.0), 1),
    (dict(dtype="fp8", k_scale=0.0), 1),
    (dict(seqlens=[]), 1),
    (dict(seqlens=[5] * 65), 2),
    (dict(seqlens=[10, -1]), 1),
    (dict(seqlens=[128 * 16385]), 2),
])
def test_problem_validation(kw, status):
    st, detail = _status(lambda: bslp.get_sizes(_problem(**kw)))
    assert st == status and detail


class FakeTensor:
    """Stands in for a device tensor: a pointer that is never dereferenced."""

    def __init__(self, shape=(4, 4), nbytes=16, ptr=0x1000):
        self.shape = shape
        self.nbytes = nbytes
        self.ptr = ptr

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return self.ptr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def test_page_table_validation():
    pt = FakeTensor((2, 4))
    st, _ = _status(lambda: bslp.get_sizes(_problem(page_table=pt, page_size=96)))
    assert st == 1
    st, _ = _status(lambda: bslp.get_sizes(_problem(page_table=pt, page_size=64)))
    assert st == 1  # 1000 tokens need 16 pages of 64 > 4
    assert bslp.get_sizes(_problem(page_table=pt, page_size=256)).total_tokens == 1300


def test_v_layout_validation():
    # d-major V (fp8 only, pages of at least 64 tokens); other values refused
    fp8 = dict(dtype="fp8", q_scale=0.5, k_scale=0.5, v_scale=0.5)
    assert bslp.get_sizes(_problem(v_dmajor=True, **fp8)).kv_tokens == 1300
    st, _ = _status(lambda: bslp.get_sizes(_problem(v_dmajor=True)))
    assert st == 2  # bf16
    pt = FakeTensor((2, 64))
    st, _ = _status(lambda: bslp.get_sizes(_problem(v_dmajor=True, page_table=pt, page_size=16,
                                                    **fp8)))
    assert st == 2
    assert bslp.get_sizes(_problem(v_dmajor=True, page_table=pt, page_size=64, **fp8)).kv_tokens == 1300
    p = _problem(**fp8)
    p.v_layout = 7
    st, _ = _status(lambda: bslp.get_sizes(p))
    assert st == 1


@pytest.mark.parametrize("kw", [dict(alpha=-0.1), dict(alpha=float("inf")), dict(sink=-1),
                                dict(correction=2)])
def test_params_validation(kw):
    args = dict(alpha=0.05, sink=1, window=2, recent=1, correction=True)
    args.update(kw)
    params = bslp.make_params(**args)
    if kw.get("correction") == 2:
        params.mean_correction = 2
    t = FakeTensor()
    st, _ = _status(lambda: bslp.select_blocks(_problem(), params, t, t, t, t, t, t, stream=0))
    assert st == 1


def test_null_pointers_rejected_before_launch():
    p = _problem()
    params = bslp.make_params(0.05)
    t = FakeTensor()
    st, d = _status(lambda: bslp.block_scores(p, t, t, None, t, t, t, stream=0))
    assert st == 1 and "NULL" in d
    st, _ = _status(lambda: bslp.select_blocks(p, params, t, t, t, t, None, t, stream=0))
    st2, _ = _status(lambda: bslp.select_blocks(p, params, None, t, t, t, t, t, stream=0))
    assert st2 == 1
    assert st == 1
    st, _ = _status(lambda: bslp.sparse_prefill_attn(p, params, t, t, t, t, t, t, None, t,
                                                     stream=0))
    assert st == 1
    st, _ = _status(lambda: bslp.sparse_prefill_attn(None or _problem(head_dim=80), params,
                                                     t, t, t, t, t, t, t, t, stream=0))
    assert st == 2


def test_empty_problem_enqueues_nothing():
    p = _problem(seqlens=[0, 0])
    s = bslp.get_sizes(p)
    assert s.total_tokens == 0 and s.num_segments == 0
    bslp.block_scores(p, None, None, None, None, None, None, stream=0)
    bslp.sparse_prefill_attn(p, bslp.make_params(0.1), None, None, None, None, None, None,
                             None, None, stream=0)


def test_status_strings():
    lib = bslp.load_library()
    assert lib.bslp_status_string(0) == b"ok"
    assert lib.bslp_status_string(2) == b"unsupported"
    assert isinstance(lib.bslp_last_error(), bytes)


def test_attention_workspace_validated_before_launch():
    # NULL, short and misaligned workspaces are BSLP_ERR_WORKSPACE (4)
    p = _problem()
    need = bslp.get_sizes(p).workspace_bytes
    assert bslp.workspace_bytes(p) == need > 0
    params = bslp.make_params(0.05)
    t = FakeTensor()
    st, d = _status(lambda: bslp.sparse_prefill_attn(p, params, t, t, t, t, t, t, t, t, t,
                                                     workspace=FakeTensor(nbytes=need - 1),
                                                     stream=0))
    assert st == 4 and "workspace" in d
    st, d = _status(lambda: bslp.sparse_prefill_attn(p, params, t, t, t, t, t, t, t, t, t,
                                                     workspace=None, stream=0))
    assert st == 4 and "workspace" in d
    st, d = _status(lambda: bslp.sparse_prefill_attn(
        p, params, t, t, t, t, t, t, t, t, t,
        workspace=FakeTensor(nbytes=need, ptr=0x1008), stream=0))
    assert st == 4 and "aligned" in d
    assert bslp.load_library().bslp_status_string(4) == b"workspace"


def test_workspace_bytes_of_an_invalid_problem_is_zero():
    p = _problem(head_dim=80)
    assert bslp.workspace_bytes(p) == 0
    assert b"head_dim" in bslp.load_library().bslp_last_error()


def test_dense_attention_validated_before_launch():
    t = FakeTensor()
    st, d = _status(lambda: bslp.dense_prefill_attn(_problem(), t, None, t, t, stream=0))
    assert st == 1 and "NULL" in d
    st, _ = _status(lambda: bslp.dense_prefill_attn(_problem(head_dim=80), t, t, t, t,
                                                    stream=0))
    assert st == 2
    # nothing to do for an empty problem, so NULL pointers are fine
    bslp.dense_prefill_attn(_problem(seqlens=[0]), None, None, None, None, stream=0)


def test_kv_splits_validated_and_sized():
    st, d = _status(lambda: bslp.get_sizes(_problem(kv_splits=17)))
    assert st == 1 and "kv_splits" in d
    st, _ = _status(lambda: bslp.get_sizes(_problem(kv_splits=-1)))
    assert st == 1
    base = bslp.get_sizes(_problem(kv_splits=1))
    assert base.workspace_bytes == bslp.get_sizes(_problem()).workspace_bytes  # small: no split
    pooled = 3 * base.pooled_rows * 2 * 128 * 2
    assert base.workspace_bytes == pooled + (base.num_segments * 2 + 12) * 4
    for u in (2, 5):
        s = bslp.get_sizes(_problem(kv_splits=u))
        # per split: float32 O [T*Hq, d] and (m, l) [T*Hq, 2] after the pooled
        # copies, then the work list (an int32 per segment x row block x split)
        # and its queue words
        items = s.num_segments * 2 * u + 12  # g*B = 512 rows: 2 row blocks of 256
        assert s.workspace_bytes == pooled + u * s.total_tokens * 8 * (128 + 2) * 4 + items * 4
    # float32 never splits
    f = bslp.get_sizes(_problem(dtype="f32", kv_splits=4))
    assert f.workspace_bytes == bslp.get_sizes(_problem(dtype="f32", kv_splits=1)).workspace_bytes


def test_automatic_kv_splits_only_for_small_launches():
    # 16K tokens, one KV head of four query heads: 128 tiles x 2 row blocks
    small = bslp.get_sizes(_problem(hq=4, hkv=1, seqlens=[16384]))
    none = bslp.get_sizes(_problem(hq=4, hkv=1, seqlens=[16384], kv_splits=1))
    assert small.workspace_bytes == (none.workspace_bytes + 2 * 16384 * 4 * 130 * 4
                                     + small.num_segments * 2 * (2 - 1) * 4)
    # 64K tokens x 8 KV heads: thousands of units, no split
    big = bslp.get_sizes(_problem(hq=32, hkv=8, seqlens=[65536]))
    assert big.workspace_bytes == bslp.get_sizes(
        _problem(hq=32, hkv=8, seqlens=[65536], kv_splits=1)).workspace_bytes


def test_quantize_and_device_scales_validated_before_launch():
    lib = bslp.load_library()
    # bad dtype, negative n, NULL and misaligned pointers
    assert lib.bslp_quantize_e4m3(2, 0x1000, 8, 0x2000, 0x3000, None) == 1
    assert lib.bslp_quantize_e4m3(1, 0x1000, -1, 0x2000, 0x3000, None) == 1
    assert lib.bslp_quantize_e4m3(1, None, 8, 0x2000, 0x3000, None) == 1
    assert lib.bslp_quantize_e4m3(1, 0x1008, 8, 0x2000, 0x3000, None) == 1
    assert b"aligned" in lib.bslp_last_error()
    # device scales are for fp8 only, and aligned
    t = FakeTensor(ptr=0x4000)
    st, d = _status(lambda: bslp.get_sizes(_problem(dtype="bf16", scales_dev=t)))
    assert st == 1 and "fp8" in d
    st, d = _status(lambda: bslp.get_sizes(_problem(dtype="fp8", scales_dev=FakeTensor(ptr=0x4002))))
    assert st == 1 and "aligned" in d
    assert bslp.get_sizes(_problem(dtype="fp8", scales_dev=t)).total_tokens == 1300


def test_noalloc_limits_checked_before_launch():
    params = bslp.make_params(0.05)
    t = FakeTensor()
    # pooled copies alone: 6 * pooled_rows * Hkv * d bytes above 32 MiB
    p = _problem(hq=8, hkv=8, head_dim=128, block_size=64, seqlens=[5462 * 64], kv_splits=1)
    assert 6 * 5462 * 8 * 128 > bslp.NOALLOC_SCRATCH_BYTES
    st, d = _status(lambda: bslp.sparse_prefill_attn_noalloc(p, params, t, t, t, t, t, t, t, t,
                                                             stream=0))
    assert st == 2 and "scratch" in d
    # a requested split count whose partial results do not fit is refused too
    p = _problem(hq=32, hkv=8, seqlens=[65536], kv_splits=4)
    st, d = _status(lambda: bslp.sparse_prefill_attn_noalloc(p, params, t, t, t, t, t, t, t, t,
                                                             stream=0))
    assert st == 2 and "scratch" in d
    # NULL tensors and bad problems are rejected as by the workspace entry point
    st, _ = _status(lambda: bslp.sparse_prefill_attn_noalloc(_problem(), params, t, None, t, t,
                                                             t, t, t, t, stream=0))
    assert st == 1
    st, _ = _status(lambda: bslp.sparse_prefill_attn_noalloc(_problem(head_dim=80), params, t,
                                                             t, t, t, t, t, t, t, stream=0))
    assert st == 2
    # nothing to do for an empty problem: no scratch is touched
    bslp.sparse_prefill_attn_noalloc(_problem(seqlens=[0]), params, None, None, None, None,
                                     None, None, None, None, stream=0)
