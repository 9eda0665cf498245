"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds_indexer.h")


@pytest.fixture(scope="module")
def ix():
    from sparse_attention_kv_ds_amd import indexer
    return indexer


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ds_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(["ds_indexer_create", "ds_indexer_score_topk",
                                           "ds_indexer_destroy", "ds_indexer_scores",
                                           "ds_indexer_status_str", "ds_indexer_timing",
                                           "ds_indexer_timing_read", "ds_sparse_attention",
                                           "ds_sparse_attention_all",
                                           "ds_indexer_score_topk_batch", "ds_indexer_project_q",
                                           "ds_indexer_project_score_topk",
                                           "ds_indexer_score_topk_noalloc",
                                           "ds_indexer_stamps_read",
                                           "ds_indexed_sparse_attention"])


def test_every_declared_symbol_is_exported(ix):
    lib = ctypes.CDLL(ix.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    dyn = subprocess.run(["nm", "-D", "--defined-only", ix.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ds_[a-z_]+)\b", dyn))
    assert exported == set(declared_functions())


def test_binding_names_match_the_header(ix):
    for name in declared_functions():
        assert callable(getattr(ix, name)), name
    assert set(ix.EXPORTS) == set(declared_functions())


def test_stamps_only_in_the_stamps_build(ix):
    """The product build records no timestamps: the reader refuses without
    touching the device.  The stamps build exports the same entry points."""
    if os.path.basename(ix.LIB_PATH) != "libds_indexer.so":
        pytest.skip("another build selected through DS_INDEXER_LIB")
    buf = ctypes.create_string_buffer(64)
    assert ix.ds_indexer_stamps_read(0, ctypes.addressof(buf), 64) == ix.DS_ERR_UNSUPPORTED
    stamps = os.path.join(os.path.dirname(ix.LIB_PATH), "libds_indexer_stamps.so")
    assert os.path.exists(stamps), "build() also builds the stamps library"
    dyn = subprocess.run(["nm", "-D", "--defined-only", stamps], capture_output=True, text=True,
                         check=True).stdout
    assert set(re.findall(r"\bT (ds_[a-z_]+)\b", dyn)) == set(declared_functions())


def test_status_strings(ix):
    for code in (0, -1, -2, -3, -4, -5):
        s = ix.ds_indexer_status_str(code)
        assert s and s != "unknown status"
    assert ix.ds_indexer_status_str(12345) == "unknown status"


def test_header_constants_match_binding(ix):
    text = open(HEADER).read()
    for name in ("DS_F16", "DS_BF16", "DS_OK", "DS_ERR_INVALID_ARG", "DS_ERR_UNSUPPORTED",
                 "DS_ERR_CAPACITY", "DS_ERR_HIP", "DS_ERR_OOM", "DS_KERNEL_SCORE",
                 "DS_KERNEL_SELECT", "DS_KERNEL_DECODE_SCORE", "DS_KERNEL_DECODE_SELECT",
                 "DS_KERNEL_PROJECT", "DS_KERNEL_CLASSES", "DS_STAMPS_DECODE_SCORE",
                 "DS_STAMPS_TOPK", "DS_STAMPS_MERGE", "DS_STAMPS_ATTENTION"):
        m = re.search(rf"\b{name}\s*=\s*(-?\d+)", text)
        assert m and int(m.group(1)) == getattr(ix, name), name


@pytest.mark.parametrize("args,want", [
    ((0, 64, 128, 1, 0, 16, 16), -1),          # max_topk < 1
    ((0, 64, 128, 1, 4096, 16, 16), -1),       # max_topk too large
    ((0, 64, 128, 1, 512, 0, 16), -1),         # max_tokens < 1
    ((0, 64, 128, 1, 512, 16, 0), -1),         # max_rows < 1
    ((-1, 64, 128, 1, 512, 16, 16), -1),       # device < 0
    ((0, 48, 128, 1, 512, 16, 16), -2),        # head count not compiled
    ((0, 64, 96, 1, 512, 16, 16), -2),         # head dim not compiled
    ((0, 64, 128, 3, 512, 16, 16), -2),        # dtype
])
def test_create_rejects_bad_arguments_on_host(ix, args, want):
    st, h = ix.ds_indexer_create(*args)
    assert st == want and h is None


def test_create_null_out_pointer(ix):
    lib = ix.library()
    assert lib.ds_indexer_create(None, 0, 64, 128, 1, 512, 16, 16) == ix.DS_ERR_INVALID_ARG


def test_calls_on_null_handle(ix):
    assert ix.ds_indexer_score_topk(None, 16, 16, 16, 16, 1, 1, 4, 1, 16, None) == -1
    assert ix.ds_indexer_score_topk_batch(None, 16, 16, 16, 16, 2, 1, 4, 1, 16, None) == -1
    assert ix.ds_indexer_project_q(None, 16, 16, 1, 64, 16, None) == -1
    assert ix.ds_indexer_project_score_topk(None, 16, 16, 16, 16, 16, 1, 1, 64, 4, 1, 16,
                                            None) == -1
    assert ix.ds_indexer_scores(None, 16, 16, 16, 16, 1, 1, 4, 16, None) == -1
    ix.ds_indexer_destroy(None)  # accepted and ignored
    assert ix.ds_indexer_timing(None, 1) == -1
    assert ix.ds_indexer_timing_read(None)[0] == -1


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "sparse_attention_kv_ds_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b|liboracle|oracle_score",
                                     text, flags=re.M), f"{f} reaches into the oracle"


def test_sparse_attention_rejects_bad_arguments_on_the_host(ix):
    """Every rejection happens before any device call (no GPU is used here)."""
    fake = 0x1000  # never dereferenced: each call below returns before any launch
    def call(**kw):
        a = dict(q=fake, k_pool=fake, v_pool=fake, k_local=fake, v_local=fake, idx=fake,
                 pos=fake, T=4, N=8, L=8, n_heads=64, head_dim=128, dtype=ix.DS_BF16, topk=4,
                 window=2, scale=0.1, out=fake, stream=None)
        a.update(kw)
        return ix.ds_sparse_attention(*a.values())
    assert call(T=-1) == ix.DS_ERR_INVALID_ARG
    assert call(window=-1) == ix.DS_ERR_INVALID_ARG
    assert call(scale=float("nan")) == ix.DS_ERR_INVALID_ARG
    assert call(scale=float("inf")) == ix.DS_ERR_INVALID_ARG
    assert call(scale=0.0) == ix.DS_ERR_INVALID_ARG
    assert call(scale=-0.1) == ix.DS_ERR_INVALID_ARG
    assert call(n_heads=48) == ix.DS_ERR_UNSUPPORTED
    assert call(head_dim=96) == ix.DS_ERR_UNSUPPORTED
    assert call(dtype=7) == ix.DS_ERR_UNSUPPORTED
    assert call(topk=2049) == ix.DS_ERR_UNSUPPORTED
    assert call(q=None) == ix.DS_ERR_INVALID_ARG
    assert call(idx=None) == ix.DS_ERR_INVALID_ARG
    assert call(out=fake + 4) == ix.DS_ERR_INVALID_ARG  # misaligned
    assert call(T=0, q=None, out=None) == ix.DS_OK      # nothing to do


def test_sparse_attention_all_rejects_bad_arguments_on_the_host(ix):
    """The all-visible form: same checks, plus ratio >= 1 and at most 2048 pooled
    rows (the length of its implicit list); no index list is needed."""
    fake = 0x1000  # never dereferenced: each call below returns before any launch
    def call(**kw):
        a = dict(q=fake, k_pool=fake, v_pool=fake, k_local=fake, v_local=fake, pos=fake, T=4,
                 N=8, L=8, n_heads=64, head_dim=128, dtype=ix.DS_BF16, ratio=128, window=2,
                 scale=0.1, out=fake, stream=None)
        a.update(kw)
        return ix.ds_sparse_attention_all(*a.values())
    assert call(ratio=0) == ix.DS_ERR_INVALID_ARG
    assert call(ratio=-4) == ix.DS_ERR_INVALID_ARG
    assert call(N=2049) == ix.DS_ERR_UNSUPPORTED
    assert call(T=-1) == ix.DS_ERR_INVALID_ARG
    assert call(scale=0.0) == ix.DS_ERR_INVALID_ARG
    assert call(n_heads=16) == ix.DS_ERR_UNSUPPORTED
    assert call(pos=None) == ix.DS_ERR_INVALID_ARG
    assert call(k_pool=None) == ix.DS_ERR_INVALID_ARG
    assert call(v_local=fake + 8) == ix.DS_ERR_INVALID_ARG  # misaligned
    assert call(T=0, q=None, out=None) == ix.DS_OK
