"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""

import ctypes
import os
import re
import subprocess

import pytest

import oracle as O
import dynamic_block_sparse_dsa_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIB_PATH):
        pytest.fail("libdsa.so is not built (run __graft_entry__.build())")
    return dsa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(dsa.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dsa_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


# The boundary's core calls: name, return type and parameter types in order
# (parameter names are free).  dsa_decode also takes a nullable LSE output
# after o, for callers that merge decodes.
BOUNDARY = {
    "dsa_kmax": ("int32_t", ["const dsa_shape*"]),
    "dsa_block_scores": ("int", ["const dsa_shape*", "const void*", "const void*", "float*", "void*"]),
    "dsa_select_topk": ("int", ["const dsa_shape*", "const float*", "int32_t*", "int32_t*", "void*"]),
    "dsa_sparse_attn_fwd": ("int", ["const dsa_shape*", "const void*", "const void*", "const void*", "const int32_t*",
                                    "const int32_t*", "void*", "float*", "void*"]),
    "dsa_prefill_workspace_bytes": ("size_t", ["const dsa_shape*"]),
    "dsa_prefill": ("int", ["const dsa_shape*", "const void*", "const void*", "const void*", "void*", "float*",
                            "int32_t*", "int32_t*", "void*", "size_t", "void*"]),
    "dsa_kv_block_means": ("int", ["const dsa_shape*", "const void*", "float*", "void*"]),
    "dsa_decode_workspace_bytes": ("size_t", ["const dsa_shape*"]),
    "dsa_decode": ("int", ["const dsa_shape*", "const void*", "const void*", "const void*", "const float*", "void*",
                           "float*", "int32_t*", "void*", "size_t", "void*"]),
    "dsa_status_str": ("const char*", ["int"]),
    "dsa_last_error": ("const char*", ["void"]),
}


def prototypes():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"([A-Za-z_][\w \t*]*?)\b(dsa_\w+)\s*\(([^)]*)\)\s*;", text):
        ret = " ".join(m.group(1).split())
        params = []
        for par in m.group(3).split(","):
            par = " ".join(par.replace("*", " * ").split())
            toks = par.split(" ")
            if len(toks) > 1 and toks[-1] not in ("*",) and toks[-1] != "void" and not toks[-1].endswith("_t") \
                    and toks[-1] not in ("int", "float", "dsa_shape"):
                toks = toks[:-1]  # drop the parameter name
            params.append(" ".join(toks).replace(" *", "*"))
        out[m.group(2)] = (ret.replace(" *", "*"), params)
    return out


def test_boundary_calls_have_the_specified_signatures():
    protos = prototypes()
    for name, want in BOUNDARY.items():
        assert name in protos, name
        assert protos[name] == want, (name, protos[name], want)


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.dsa_status_str(code)
    assert lib.dsa_status_str(17) == b"unknown status"


def shape(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, seq_len=1024, head_dim=128, block=64, topk=4, topk_num=0,
                topk_den=1, flags=3)
    base.update(kw)
    return dsa.Shape(**base)


BAD = [
    (dict(head_dim=96), dsa.DSA_ERR_UNSUPPORTED),
    (dict(block=32), dsa.DSA_ERR_UNSUPPORTED),
    (dict(n_q_heads=5, n_kv_heads=2), dsa.DSA_ERR_SHAPE),
    (dict(n_kv_heads=0), dsa.DSA_ERR_SHAPE),
    (dict(batch=-1), dsa.DSA_ERR_SHAPE),
    (dict(seq_len=-5), dsa.DSA_ERR_SHAPE),
    (dict(topk=-1), dsa.DSA_ERR_SHAPE),
    (dict(topk=0, topk_num=1, topk_den=0), dsa.DSA_ERR_SHAPE),
    (dict(topk=0, topk_num=-1, topk_den=3), dsa.DSA_ERR_SHAPE),
    (dict(topk=0, topk_num=0, flags=0), dsa.DSA_ERR_SHAPE),
    (dict(flags=8), dsa.DSA_ERR_SHAPE),
    (dict(seq_len=64 * 4096 + 1), dsa.DSA_ERR_UNSUPPORTED),
    (dict(select_mode=3), dsa.DSA_ERR_SHAPE),
    (dict(n_anchor=-1), dsa.DSA_ERR_SHAPE),
    (dict(window=-2), dsa.DSA_ERR_SHAPE),
    (dict(select_mode=1, threshold=0.0), dsa.DSA_ERR_SHAPE),
    (dict(select_mode=1, threshold=1.5), dsa.DSA_ERR_SHAPE),
    (dict(select_mode=1, threshold=float("nan")), dsa.DSA_ERR_SHAPE),
    (dict(select_mode=1, threshold=0.1, flags=0), dsa.DSA_ERR_SHAPE),
    (dict(select_mode=2, k_min=0, k_max=4), dsa.DSA_ERR_SHAPE),
    (dict(select_mode=2, k_min=5, k_max=4), dsa.DSA_ERR_SHAPE),
]


@pytest.mark.parametrize("kw,code", BAD)
def test_bad_shapes_are_rejected_everywhere(lib, kw, code):
    s = shape(**kw)
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    out = ctypes.c_int32()
    calls = [
        lambda: lib.dsa_kmax(ctypes.byref(s)),
        lambda: lib.dsa_prefill_kmax(ctypes.byref(s), ctypes.byref(out)),
        lambda: lib.dsa_block_means(ctypes.byref(s), 2, p, p, None),
        lambda: lib.dsa_block_scores(ctypes.byref(s), p, p, p, None),
        lambda: lib.dsa_block_scores_from_means(ctypes.byref(s), p, p, p, None),
        lambda: lib.dsa_select_topk(ctypes.byref(s), p, p, p, None),
        lambda: lib.dsa_sparse_attn_fwd(ctypes.byref(s), p, p, p, p, p, p, None, None),
        lambda: lib.dsa_prefill(ctypes.byref(s), p, p, p, p, None, p, p, p, 1 << 40, None),
        lambda: lib.dsa_decode(ctypes.byref(s), p, p, p, p, p, None, p, p, 1 << 40, None),
        lambda: lib.dsa_decode_noalloc(ctypes.byref(s), p, p, p, p, p, None, p, None),
    ]
    for c in calls:
        assert c() == code
        assert lib.dsa_last_error()
    assert lib.dsa_prefill_workspace_bytes(ctypes.byref(s)) == 0


def test_null_arguments(lib):
    s = shape()
    p = ctypes.c_void_p(16)
    assert lib.dsa_prefill_kmax(None, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_prefill_kmax(ctypes.byref(s), None) == dsa.DSA_ERR_NULL
    assert lib.dsa_block_means(ctypes.byref(s), 4, None, p, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_block_scores(ctypes.byref(s), p, None, p, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_block_scores(ctypes.byref(s), p, p, None, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_block_scores_from_means(ctypes.byref(s), p, None, p, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_kmax(None) == dsa.DSA_ERR_NULL
    assert lib.dsa_select_topk(ctypes.byref(s), p, p, None, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_sparse_attn_fwd(ctypes.byref(s), p, p, None, p, p, p, None, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_prefill(ctypes.byref(s), p, p, p, None, None, p, p, p, 1 << 40, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_decode(ctypes.byref(s), p, p, p, None, p, None, p, p, 1 << 40, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_decode_noalloc(ctypes.byref(s), p, p, p, None, p, None, p, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_decode_noalloc(ctypes.byref(s), p, p, p, p, p, None, None, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_block_means(ctypes.byref(s), 0, p, p, None) == dsa.DSA_ERR_SHAPE


def test_workspace_too_small(lib):
    s = shape()
    p = ctypes.c_void_p(16)
    need = lib.dsa_prefill_workspace_bytes(ctypes.byref(s))
    nb = 1024 // 64
    a256 = lambda x: (x + 255) // 256 * 256
    assert need == a256(4 * nb * 128 * 4) + a256(2 * nb * 128 * 4) + a256(2 * nb * nb * 4)
    assert lib.dsa_prefill(ctypes.byref(s), p, p, p, p, None, p, p, p, need - 1, None) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_prefill(ctypes.byref(s), p, p, p, p, None, p, p, None, need, None) == dsa.DSA_ERR_WORKSPACE
    d = shape(batch=3, seq_len=1000)
    dneed = lib.dsa_decode_workspace_bytes(ctypes.byref(d))
    assert dneed > 0
    assert lib.dsa_decode(ctypes.byref(d), p, p, p, p, p, None, p, p, dneed - 1, None) == dsa.DSA_ERR_WORKSPACE


def test_decode_specific_checks(lib):
    p = ctypes.c_void_p(16)
    s = shape(n_q_heads=24, n_kv_heads=2)  # group of 12: prefill yes, decode no
    out = ctypes.c_int32()
    assert lib.dsa_prefill_kmax(ctypes.byref(s), ctypes.byref(out)) == 0
    assert lib.dsa_decode_kmax(ctypes.byref(s), ctypes.byref(out)) == dsa.DSA_ERR_UNSUPPORTED
    z = shape(seq_len=0)
    assert lib.dsa_decode(ctypes.byref(z), p, p, p, p, p, None, p, p, 1 << 40, None) == dsa.DSA_ERR_SHAPE


def test_noalloc_decode_scratch_covers_every_split_shape(lib):
    """The split partials of every decode shape the library takes fit the
    library-owned scratch of dsa_decode_noalloc (the fused path, >= 256
    units, needs none): the largest split workspace over group sizes, head
    dims, unit counts and budgets stays within DSA_DECODE_NOALLOC_MAX_BYTES."""
    worst = 0
    for G in (1, 2, 4, 8):
        for d in (64, 128):
            for S, Hkv in ((1, 1), (1, 8), (3, 7), (31, 8), (255, 1), (127, 2), (300, 1)):
                for topk, L in ((1, 64), (4, 4096), (32, 65536), (4096, 64 * 4096), (700, 64 * 1000)):
                    s = shape(batch=S, n_q_heads=Hkv * G, n_kv_heads=Hkv, seq_len=L, head_dim=d, topk=topk)
                    worst = max(worst, lib.dsa_decode_workspace_bytes(ctypes.byref(s)))
    assert 0 < worst <= 8 << 20


def test_decode_takes_top_k_only(lib):
    """Threshold and entropy budgets vary per row; the decode kernels keep the
    same count in every unit, so they refuse those modes (anchors and a window
    are fine)."""
    out = ctypes.c_int32()
    for kw in (dict(select_mode=1, threshold=0.1), dict(select_mode=2, k_min=2, k_max=8)):
        s = shape(**kw)
        assert lib.dsa_prefill_kmax(ctypes.byref(s), ctypes.byref(out)) == 0
        assert lib.dsa_decode_kmax(ctypes.byref(s), ctypes.byref(out)) == dsa.DSA_ERR_UNSUPPORTED
    s = shape(n_anchor=3, window=4)
    assert lib.dsa_decode_kmax(ctypes.byref(s), ctypes.byref(out)) == 0 and out.value == 7


def test_bitmap_argument_checks(lib):
    p = ctypes.c_void_p(16)
    f = lib.dsa_indices_to_bitmap
    assert f(p, None, -1, 4, 16, p, None) == dsa.DSA_ERR_SHAPE
    assert f(p, None, 4, 0, 16, p, None) == dsa.DSA_ERR_SHAPE
    assert f(p, None, 4, 4, 0, p, None) == dsa.DSA_ERR_SHAPE
    assert f(p, None, 4, 4, 4097, p, None) == dsa.DSA_ERR_SHAPE
    assert f(None, None, 4, 4, 16, p, None) == dsa.DSA_ERR_NULL
    assert f(p, None, 4, 4, 16, None, None) == dsa.DSA_ERR_NULL
    assert f(None, None, 0, 4, 16, None, None) == 0  # empty: nothing enqueued


def test_empty_problems_are_no_ops(lib):
    """B == 0 or N == 0 returns OK without touching the (invalid) pointers."""
    p = ctypes.c_void_p(16)
    for s in (shape(batch=0), shape(seq_len=0)):
        assert lib.dsa_prefill(ctypes.byref(s), p, p, p, p, None, p, p, None, 0, None) == 0
        assert lib.dsa_sparse_attn_fwd(ctypes.byref(s), p, p, p, p, p, p, None, None) == 0
        assert lib.dsa_block_means(ctypes.byref(s), 4, p, p, None) == 0
    d = shape(batch=0)
    assert lib.dsa_decode(ctypes.byref(d), p, p, p, p, p, None, p, None, 0, None) == 0
    assert lib.dsa_decode_noalloc(ctypes.byref(d), p, p, p, p, p, None, p, None) == 0


@pytest.mark.parametrize("N,b,topk,num,den,flags", [
    (1024, 64, 4, 0, 1, 3), (8192, 64, 16, 0, 1, 3), (32768, 64, 0, 15, 100, 3), (131072, 128, 64, 0, 1, 3),
    (100, 64, 4, 0, 1, 3), (1000, 64, 1, 0, 1, 0), (5000, 128, 0, 1, 3, 1), (640, 64, 50, 0, 1, 2)])
def test_kmax_matches_the_oracle(lib, N, b, topk, num, den, flags):
    s = shape(seq_len=N, block=b, topk=topk, topk_num=num, topk_den=den, flags=flags)
    nb = -(-N // b)
    assert dsa.dsa_prefill_kmax(s) == O.kmax(nb, topk, num, den, flags, True, nb)
    assert dsa.dsa_decode_kmax(s) == O.kmax(1, topk, num, den, flags, False, nb)
    assert dsa.dsa_kmax(s) == dsa.dsa_prefill_kmax(s) == dsa.dsa_decode_kmax(s)


VARIANTS = [
    dict(n_anchor=3, window=2), dict(n_anchor=5, window=1, flags=1), dict(window=7, flags=2, topk=3),
    dict(select_mode=1, threshold=0.1), dict(select_mode=1, threshold=0.05, n_anchor=2, window=2),
    dict(select_mode=1, threshold=0.25, flags=1), dict(select_mode=1, threshold=1.0),
    dict(select_mode=2, k_min=2, k_max=32), dict(select_mode=2, k_min=1, k_max=1, n_anchor=2, window=3),
    dict(select_mode=2, k_min=4, k_max=4000),
]


@pytest.mark.parametrize("N", [100, 1024, 20000])
@pytest.mark.parametrize("kw", VARIANTS, ids=[str(v) for v in VARIANTS])
def test_kmax_of_selection_variants_matches_the_oracle(lib, N, kw):
    s = shape(seq_len=N, **kw)
    nb = -(-N // 64)
    spec = O.SelectSpec(mode=kw.get("select_mode", 0), anchors=max(1, kw.get("n_anchor", 0)),
                        window=max(1, kw.get("window", 0)), threshold=kw.get("threshold", 0.0),
                        k_min=kw.get("k_min", 0), k_max=kw.get("k_max", 0))
    flags, topk = kw.get("flags", 3), kw.get("topk", 4)
    assert dsa.dsa_prefill_kmax(s) == O.kmax(nb, topk, 0, 1, flags, True, nb, spec)
    assert dsa.dsa_kmax(s) == dsa.dsa_prefill_kmax(s)
    if kw.get("select_mode", 0) == 0:
        assert dsa.dsa_decode_kmax(s) == O.kmax(1, topk, 0, 1, flags, False, nb, spec)


def test_binding_rejects_host_tensors():
    import torch
    s = shape(batch=1, n_q_heads=2, n_kv_heads=2, seq_len=128, head_dim=64)
    x = torch.zeros((1, 2, 128, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dsa.dsa_block_means(s, 2, x, torch.zeros((1, 2, 2, 64)), stream=0)


def test_decode_workspace_is_zero_on_the_one_launch_path(lib):
    """From 256 (sequence, KV head) units on a decode step is one launch with
    no partials: its workspace is 0 bytes and dsa_decode takes a NULL
    workspace there (it still refuses one below that)."""
    p = ctypes.c_void_p(16)
    for S, Hkv in ((64, 4), (256, 1), (32, 8), (300, 1)):
        s = shape(batch=S, n_q_heads=Hkv * 4, n_kv_heads=Hkv, seq_len=4096, topk=16)
        assert lib.dsa_decode_workspace_bytes(ctypes.byref(s)) == 0
    s = shape(batch=63, n_q_heads=16, n_kv_heads=4, seq_len=4096, topk=16)  # 252 units: split path
    assert lib.dsa_decode_workspace_bytes(ctypes.byref(s)) > 0
    assert lib.dsa_decode(ctypes.byref(s), p, p, p, p, p, None, p, None, 0, None) == dsa.DSA_ERR_WORKSPACE


def test_deterministic_flag_is_a_shape_flag(lib):
    """DSA_DETERMINISTIC is accepted next to the forcing flags (prefill and
    decode shapes), does not count as a forced block, and the index shape,
    whose calls are deterministic anyway, does not take it."""
    out = ctypes.c_int32()
    for fl in (dsa.DETERMINISTIC, 3 | dsa.DETERMINISTIC, 1 | dsa.DETERMINISTIC):
        s = shape(flags=fl)
        assert lib.dsa_prefill_kmax(ctypes.byref(s), ctypes.byref(out)) == 0
        assert lib.dsa_decode_kmax(ctypes.byref(s), ctypes.byref(out)) == 0
    # the flag forces nothing: a fraction of 0 with no forcing flag keeps no block
    s = shape(topk=0, topk_num=0, topk_den=1, flags=dsa.DETERMINISTIC)
    assert lib.dsa_prefill_kmax(ctypes.byref(s), ctypes.byref(out)) == dsa.DSA_ERR_SHAPE
    s = shape(select_mode=1, threshold=0.1, flags=dsa.DETERMINISTIC)  # threshold needs a forced block
    assert lib.dsa_prefill_kmax(ctypes.byref(s), ctypes.byref(out)) == dsa.DSA_ERR_SHAPE
    i = dsa.make_index_shape(1, 4, 2, 1024, 128, 16, 128, 64, flags=3 | dsa.DETERMINISTIC)
    assert lib.dsa_index_kmax(ctypes.byref(i), ctypes.byref(out)) == dsa.DSA_ERR_SHAPE
