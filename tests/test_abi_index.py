"""Host-side checks of the token indexer's C-ABI calls (no GPU): argument
validation, the length limits of each path, and the workspace sizes."""

import ctypes

import pytest

import dynamic_block_sparse_dsa_amd as dsa

P = ctypes.c_void_p(16)  # never dereferenced: every call below returns before a launch


@pytest.fixture(scope="module")
def lib():
    return dsa.load()


def ishape(**kw):
    a = dict(batch=1, n_q_heads=4, n_kv_heads=2, seq_len=1000, head_dim=128, n_index_heads=16, index_dim=128,
             topk=64, flags=3)
    a.update(kw)
    return dsa.make_index_shape(**a)


def a256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("B,N,topk,want", [
    (1, 2048, 64, 0),                                    # one chunk of keys: no lists
    (1, 2049, 64, a256(2049 * 2 * (8 * 64 + 4))),       # two chunks of at least 32 key tiles
    (1, 4096, 64, a256(4096 * 2 * (8 * 64 + 4))),
    (1, 4097, 64, a256(4097 * 2 * (8 * 64 + 4))),       # two chunks of 64 key tiles
    (1, 8192, 64, a256(8192 * 2 * (8 * 64 + 4))),
    (2, 32768, 64, a256(2 * 32768 * 2 * (8 * 64 + 4))),  # two chunks of 256 tiles
    (1, 131072, 128, a256(131072 * 2 * (8 * 128 + 4))),
    (1, 3000, 129, a256(3000 * 3000 * 4)),               # kmax 129: the scores array
])
def test_index_workspace_bytes(lib, B, N, topk, want):
    s = ishape(batch=B, seq_len=N, topk=topk)
    assert lib.dsa_index_workspace_bytes(ctypes.byref(s)) == want


def test_index_topk_limits(lib):
    s = ishape(topk=129)
    assert lib.dsa_index_topk(ctypes.byref(s), P, P, P, P, P, P, 1 << 40, None) == dsa.DSA_ERR_UNSUPPORTED
    assert b"kept tokens" in lib.dsa_last_error()
    # no length limit on the fused path; the workspace is checked
    s = ishape(seq_len=100000)
    need = lib.dsa_index_workspace_bytes(ctypes.byref(s))
    assert need > 0
    assert lib.dsa_index_topk(ctypes.byref(s), P, P, P, P, P, P, need - 1, None) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_index_topk(ctypes.byref(s), P, P, P, P, P, None, need, None) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_index_prefill(ctypes.byref(s), P, P, P, P, P, P, P, None, P, P, P, need - 1,
                                 None) == dsa.DSA_ERR_WORKSPACE


def test_scores_array_path_limits(lib):
    s = ishape(seq_len=8193)
    assert lib.dsa_select_tokens(ctypes.byref(s), P, P, P, None) == dsa.DSA_ERR_UNSUPPORTED
    s = ishape(seq_len=8193, topk=200)
    assert lib.dsa_index_prefill(ctypes.byref(s), P, P, P, P, P, P, P, None, P, P, P, 1 << 40,
                                 None) == dsa.DSA_ERR_UNSUPPORTED
    s = ishape(seq_len=8192)
    assert lib.dsa_select_tokens(ctypes.byref(s), None, P, P, None) == dsa.DSA_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(n_index_heads=8), dsa.DSA_ERR_UNSUPPORTED),
    (dict(index_dim=96), dsa.DSA_ERR_UNSUPPORTED),
    (dict(head_dim=96), dsa.DSA_ERR_UNSUPPORTED),
    (dict(n_q_heads=6, n_kv_heads=2), dsa.DSA_ERR_UNSUPPORTED),
    (dict(n_q_heads=5, n_kv_heads=2), dsa.DSA_ERR_SHAPE),
    (dict(topk=0), dsa.DSA_ERR_SHAPE),
    (dict(flags=4), dsa.DSA_ERR_SHAPE),
    (dict(seq_len=-1), dsa.DSA_ERR_SHAPE),
])
def test_bad_index_shapes(lib, kw, code):
    s = ishape(**kw)
    out = ctypes.c_int32()
    assert lib.dsa_index_kmax(ctypes.byref(s), ctypes.byref(out)) == code
    assert lib.dsa_index_topk(ctypes.byref(s), P, P, P, P, P, P, 1 << 40, None) == code
    assert lib.dsa_index_scores(ctypes.byref(s), P, P, P, P, None) == code
    assert lib.dsa_index_prefill(ctypes.byref(s), P, P, P, P, P, P, P, None, P, P, P, 1 << 40, None) == code
    assert lib.dsa_index_workspace_bytes(ctypes.byref(s)) == 0


def test_index_null_and_empty(lib):
    s = ishape()
    assert lib.dsa_index_topk(ctypes.byref(s), P, P, None, P, P, P, 1 << 40, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_index_topk(ctypes.byref(s), P, P, P, None, P, P, 1 << 40, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_index_topk(None, P, P, P, P, P, P, 1 << 40, None) == dsa.DSA_ERR_NULL
    for e in (ishape(batch=0), ishape(seq_len=0)):
        assert lib.dsa_index_topk(ctypes.byref(e), P, P, P, P, P, None, 0, None) == 0
        assert lib.dsa_index_prefill(ctypes.byref(e), P, P, P, P, P, P, P, None, P, P, None, 0, None) == 0
    # short sequences need no workspace
    s = ishape(seq_len=2048)
    assert lib.dsa_index_workspace_bytes(ctypes.byref(s)) == 0
