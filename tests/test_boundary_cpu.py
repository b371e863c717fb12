"""The C-ABI boundary on the CPU: the library loads, exports every entry
point the public header declares, and rejects bad arguments before anything
reaches a GPU (no call here launches a kernel)."""
import ctypes
import os
import re

import pytest

import mla_attention_kv_amd as mla
from mla_attention_kv_amd import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmlaprolog.h")

V2 = Dims(H=2048, nh=16)
R1 = Dims(H=7168, nh=128)


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", src)))


def test_exports_match_header():
    L = mla.lib()
    names = header_functions()
    assert set(names) == set(mla.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        s = mla.mla_status_string(code)
        assert s.startswith("MLA_")
    assert "unknown" in mla.mla_status_string(42)


def test_workspace_sizes():
    assert mla.mla_kv_prolog_workspace_size(0, V2) == 0
    assert mla.mla_kv_prolog_workspace_size(-1, V2) == 0
    assert mla.mla_kv_prolog_workspace_size(1 << 23, V2) == 0
    assert mla.mla_kv_prolog_workspace_size(64, V2, 7) == 0  # bad dtype
    prev = 0
    for T in (1, 16, 64, 65, 1000, 4096, 20000):
        b = mla.mla_kv_prolog_workspace_size(T, V2)
        assert b > 0 and b % 256 == 0
        assert mla.mla_kv_prolog_w8a8_workspace_size(T, R1) > 0
        prev = b
    assert prev > 0
    assert mla.mla_kv_prolog_workspace_size(64, Dims(H=2048, nh=16, r=256)) == 0
    assert mla.mla_kv_prolog_w8a8_workspace_size(4, Dims(H=64, nh=1)) == 0  # H % 128


def test_dispatcher_and_force_hook():
    assert mla.mla_kv_prolog_selected_path(1, V2) == 0
    assert mla.mla_kv_prolog_selected_path(64, V2) == 0
    assert mla.mla_kv_prolog_selected_path(65, V2) == 1
    assert mla.mla_kv_prolog_selected_path(4096, V2) == 1
    try:
        assert mla.mla_kv_prolog_force_path(1) == -1
        assert mla.mla_kv_prolog_selected_path(1, V2) == 1
        assert mla.mla_kv_prolog_force_path(0) == 1
        assert mla.mla_kv_prolog_selected_path(4096, V2) == 0
    finally:
        mla.mla_kv_prolog_force_path(-1)
    assert mla.mla_kv_prolog_selected_path(1, V2) == 0


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation


def call_fp(T=4, d=V2, dt=1, eps=1e-6, theta=1e4, ptrs=None, ws=FAKE, wsb=1 << 40):
    p = [FAKE] * 9 if ptrs is None else ptrs
    return mla.lib().mla_kv_prolog(p[0], p[1], p[2], p[3], p[4], T, d.c(), dt, eps, theta,
                                   p[5], p[6], p[7], p[8], ws, wsb, None)


@pytest.mark.parametrize("i", range(9))
def test_null_pointer_rejected(i):
    p = [FAKE] * 9
    p[i] = None
    assert call_fp(ptrs=p) == mla.MLA_ERR_INVALID_ARG


@pytest.mark.parametrize("i", range(9))
def test_misaligned_pointer_rejected(i):
    p = [FAKE] * 9
    p[i] = FAKE + 2
    assert call_fp(ptrs=p) == mla.MLA_ERR_MISALIGNED


def test_argument_errors():
    assert call_fp(T=-1) == mla.MLA_ERR_INVALID_ARG
    assert call_fp(T=(1 << 22) + 1) == mla.MLA_ERR_INVALID_ARG
    assert call_fp(dt=3) == mla.MLA_ERR_INVALID_ARG
    assert call_fp(eps=float("nan")) == mla.MLA_ERR_INVALID_ARG
    assert call_fp(eps=-1.0) == mla.MLA_ERR_INVALID_ARG
    assert call_fp(theta=0.0) == mla.MLA_ERR_INVALID_ARG
    assert call_fp(theta=float("inf")) == mla.MLA_ERR_INVALID_ARG
    for bad in (Dims(H=2048, nh=16, r=256), Dims(H=2048, nh=16, dr=32),
                Dims(H=2048, nh=16, dn=64), Dims(H=2048, nh=16, dv=64),
                Dims(H=2000, nh=16), Dims(H=0, nh=16), Dims(H=2048, nh=0),
                Dims(H=2048, nh=2048), Dims(H=1 << 17, nh=1)):
        assert call_fp(d=bad) == mla.MLA_ERR_UNSUPPORTED, bad
    assert call_fp(ws=None) == mla.MLA_ERR_WORKSPACE
    assert call_fp(ws=FAKE + 4) == mla.MLA_ERR_MISALIGNED
    assert call_fp(wsb=0) == mla.MLA_ERR_WORKSPACE
    need = mla.mla_kv_prolog_workspace_size(4, V2)
    assert call_fp(wsb=need - 1) == mla.MLA_ERR_WORKSPACE


def test_zero_tokens_ok_without_pointers():
    assert call_fp(T=0, ptrs=[None] * 9, ws=None, wsb=0) == mla.MLA_OK
    # unsupported dims are still reported at T == 0
    assert call_fp(T=0, d=Dims(H=100, nh=1)) == mla.MLA_ERR_UNSUPPORTED


def call_w8(T=4, d=R1, ptrs=None, dbg=(None, None, 0, 0), ws=FAKE, wsb=1 << 40):
    p = [FAKE] * 11 if ptrs is None else ptrs
    return mla.lib().mla_kv_prolog_w8a8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], T, d.c(),
                                        1e-6, 1e4, p[7], p[8], p[9], p[10], dbg[0], dbg[1],
                                        dbg[2], dbg[3], ws, wsb, None)


def test_w8a8_argument_errors():
    for i in range(11):
        p = [FAKE] * 11
        p[i] = None
        assert call_w8(ptrs=p) == mla.MLA_ERR_INVALID_ARG
        p[i] = FAKE + 8
        assert call_w8(ptrs=p) == mla.MLA_ERR_MISALIGNED
    assert call_w8(d=Dims(H=64, nh=1)) == mla.MLA_ERR_UNSUPPORTED
    assert call_w8(dbg=(FAKE, None, 2, 3)) == mla.MLA_ERR_INVALID_ARG   # rows past T
    assert call_w8(dbg=(FAKE, None, -1, 1)) == mla.MLA_ERR_INVALID_ARG
    assert call_w8(dbg=(None, FAKE + 4, 0, 1)) == mla.MLA_ERR_MISALIGNED
    assert call_w8(wsb=16) == mla.MLA_ERR_WORKSPACE
    assert call_w8(T=0, ptrs=[None] * 11, ws=None, wsb=0) == mla.MLA_OK


def test_python_binding_checks_tensors():
    torch = pytest.importorskip("torch")
    X = torch.zeros(2, 64, dtype=torch.float32)
    with pytest.raises(ValueError):
        mla.mla_kv_prolog(X, X, X, X, X)


def call_cache(T=4, d=V2, dt=1, ptrs=None, slots=1024, q8=False):
    p = [FAKE] * 5 if ptrs is None else ptrs
    if q8:
        return mla.lib().mla_kv_cache_append_int8(p[0], p[1], p[2], T, d.c(), dt, p[3], p[4],
                                                  slots, None)
    return mla.lib().mla_kv_cache_append(p[0], p[1], p[2], T, d.c(), dt, p[3], slots, None)


@pytest.mark.parametrize("q8", [False, True])
def test_cache_append_argument_errors(q8):
    n = 5 if q8 else 4
    for i in range(n):
        p = [FAKE] * 5
        p[i] = None
        assert call_cache(ptrs=p, q8=q8) == mla.MLA_ERR_INVALID_ARG, i
    # 16-byte rows and caches, 8-byte slot mapping, 4-byte scales (only
    # misalignments: a valid call would launch)
    for i, off in ((0, 8), (1, 8), (2, 4), (3, 8)):
        p = [FAKE] * 5
        p[i] = FAKE + off
        assert call_cache(ptrs=p, q8=q8) == mla.MLA_ERR_MISALIGNED, (i, off)
    if q8:
        p = [FAKE] * 5
        p[4] = FAKE + 2
        assert call_cache(ptrs=p, q8=True) == mla.MLA_ERR_MISALIGNED
    assert call_cache(T=-1, q8=q8) == mla.MLA_ERR_INVALID_ARG
    assert call_cache(T=(1 << 22) + 1, q8=q8) == mla.MLA_ERR_INVALID_ARG
    assert call_cache(slots=-1, q8=q8) == mla.MLA_ERR_INVALID_ARG
    assert call_cache(dt=0, q8=q8) == mla.MLA_ERR_INVALID_ARG
    assert call_cache(d=Dims(H=2048, nh=16, r=256), q8=q8) == mla.MLA_ERR_UNSUPPORTED
    assert call_cache(d=Dims(H=2048, nh=16, dr=32), q8=q8) == mla.MLA_ERR_UNSUPPORTED
    # nothing to do: no pointer is needed and nothing is launched
    assert call_cache(T=0, ptrs=[None] * 5, q8=q8) == mla.MLA_OK
    assert call_cache(slots=0, ptrs=[FAKE, FAKE, FAKE, None, None], q8=q8) == mla.MLA_OK


def call_fp_cached(T=4, ptrs=None, slots_ptr=FAKE, cache=FAKE, slots=1024, ws=FAKE,
                   wsb=1 << 40):
    p = [FAKE] * 9 if ptrs is None else ptrs
    return mla.lib().mla_kv_prolog_cached(p[0], p[1], p[2], p[3], p[4], T, V2.c(), 1, 1e-6,
                                          1e4, p[5], p[6], p[7], p[8], slots_ptr, cache, slots,
                                          ws, wsb, None)


def test_prolog_cached_argument_errors():
    # the prolog's own checks still apply
    for i in range(9):
        p = [FAKE] * 9
        p[i] = None
        assert call_fp_cached(ptrs=p) == mla.MLA_ERR_INVALID_ARG, i
        p[i] = FAKE + 2
        assert call_fp_cached(ptrs=p) == mla.MLA_ERR_MISALIGNED, i
    assert call_fp_cached(wsb=0) == mla.MLA_ERR_WORKSPACE
    # and the cache's
    assert call_fp_cached(slots=-1) == mla.MLA_ERR_INVALID_ARG
    assert call_fp_cached(slots_ptr=None) == mla.MLA_ERR_INVALID_ARG
    assert call_fp_cached(cache=None) == mla.MLA_ERR_INVALID_ARG
    assert call_fp_cached(slots_ptr=FAKE + 4) == mla.MLA_ERR_MISALIGNED
    assert call_fp_cached(cache=FAKE + 8) == mla.MLA_ERR_MISALIGNED
    # without slots the cache pointers are not needed (the call then fails
    # only on the prolog's workspace check, so nothing launches)
    assert call_fp_cached(slots=0, slots_ptr=None, cache=None, wsb=0) == mla.MLA_ERR_WORKSPACE
    assert call_fp_cached(T=0, ptrs=[None] * 9, slots_ptr=None, cache=None, ws=None,
                          wsb=0) == mla.MLA_OK


def test_python_prolog_cached_checks_tensors():
    torch = pytest.importorskip("torch")
    T, H = 3, 64
    X = torch.zeros(T, H, dtype=torch.float16)
    Wa = torch.zeros(H, 576, dtype=torch.float16)
    g = torch.zeros(512, dtype=torch.float16)
    Wb = torch.zeros(512, 256, dtype=torch.float16)
    pos = torch.zeros(T, dtype=torch.int32)
    with pytest.raises(ValueError):  # int32 slot mapping
        mla.mla_kv_prolog_cached(X, Wa, g, Wb, pos, torch.zeros(T, dtype=torch.int32),
                                 torch.zeros(8, 576, dtype=torch.float16))
    with pytest.raises(ValueError):  # cache of another dtype
        mla.mla_kv_prolog_cached(X, Wa, g, Wb, pos, torch.zeros(T, dtype=torch.int64),
                                 torch.zeros(8, 576, dtype=torch.bfloat16))


def call_w8_cached(T=4, slots_ptr=FAKE, cache=None, q=FAKE, sc=FAKE, slots=1024, wsb=1 << 40):
    p = [FAKE] * 11
    return mla.lib().mla_kv_prolog_w8a8_cached(p[0], p[1], p[2], p[3], p[4], p[5], p[6], T,
                                               R1.c(), 1e-6, 1e4, p[7], p[8], p[9], p[10],
                                               slots_ptr, cache, q, sc, slots, FAKE, wsb, None)


def test_prolog_w8a8_cached_argument_errors():
    assert call_w8_cached(slots=-1) == mla.MLA_ERR_INVALID_ARG
    assert call_w8_cached(slots_ptr=None) == mla.MLA_ERR_INVALID_ARG
    # exactly one cache
    assert call_w8_cached(cache=FAKE) == mla.MLA_ERR_INVALID_ARG
    assert call_w8_cached(q=None, sc=None) == mla.MLA_ERR_INVALID_ARG
    assert call_w8_cached(sc=None) == mla.MLA_ERR_INVALID_ARG
    assert call_w8_cached(q=None) == mla.MLA_ERR_INVALID_ARG
    assert call_w8_cached(slots_ptr=FAKE + 4) == mla.MLA_ERR_MISALIGNED
    assert call_w8_cached(q=FAKE + 8) == mla.MLA_ERR_MISALIGNED
    assert call_w8_cached(sc=FAKE + 2) == mla.MLA_ERR_MISALIGNED
    assert call_w8_cached(cache=FAKE + 8, q=None, sc=None) == mla.MLA_ERR_MISALIGNED
    # valid cache arguments: the prolog's own checks still apply
    assert call_w8_cached(wsb=16) == mla.MLA_ERR_WORKSPACE
    assert call_w8_cached(cache=FAKE, q=None, sc=None, wsb=16) == mla.MLA_ERR_WORKSPACE
    assert call_w8_cached(slots=0, slots_ptr=None, q=None, sc=None, wsb=16) == \
        mla.MLA_ERR_WORKSPACE


def test_rms_norm_and_rope_argument_errors():
    L = mla.lib()
    rms = lambda rows=4, n=512, dt=1, eps=1e-6, p=(FAKE, FAKE, FAKE): L.mla_rms_norm(  # noqa: E731
        p[0], p[1], rows, n, dt, eps, p[2], None)
    for i in range(3):
        p = [FAKE] * 3
        p[i] = None
        assert rms(p=p) == mla.MLA_ERR_INVALID_ARG, i
        p[i] = FAKE + 8
        assert rms(p=p) == mla.MLA_ERR_MISALIGNED, i
    assert rms(rows=-1) == mla.MLA_ERR_INVALID_ARG
    assert rms(dt=0) == mla.MLA_ERR_INVALID_ARG
    assert rms(eps=-1.0) == mla.MLA_ERR_INVALID_ARG
    assert rms(eps=float("nan")) == mla.MLA_ERR_INVALID_ARG
    for n in (0, 4, 12, 8200, 16384):
        assert rms(n=n) == mla.MLA_ERR_UNSUPPORTED, n
    assert rms(rows=0, p=(None, None, None)) == mla.MLA_OK

    rope = lambda T=4, heads=2, dr=64, dt=2, theta=1e4, p=(FAKE, FAKE, FAKE): L.mla_rope(  # noqa: E731
        p[0], p[1], T, heads, dr, dt, theta, p[2], None)
    for i in range(3):
        p = [FAKE] * 3
        p[i] = None
        assert rope(p=p) == mla.MLA_ERR_INVALID_ARG, i
        p[i] = FAKE + (2 if i == 1 else 8)
        assert rope(p=p) == mla.MLA_ERR_MISALIGNED, i
    assert rope(T=-1) == mla.MLA_ERR_INVALID_ARG
    assert rope(T=(1 << 22) + 1) == mla.MLA_ERR_INVALID_ARG
    assert rope(heads=0) == mla.MLA_ERR_INVALID_ARG
    assert rope(heads=1025) == mla.MLA_ERR_INVALID_ARG
    assert rope(dt=5) == mla.MLA_ERR_INVALID_ARG
    assert rope(theta=0.0) == mla.MLA_ERR_INVALID_ARG
    assert rope(dr=128) == mla.MLA_ERR_UNSUPPORTED
    assert rope(T=0, p=(None, None, None)) == mla.MLA_OK


def graph_desc(**kw):
    d = dict(w8a8=0, d=V2.c(), dt=mla.MLA_F16, eps=1e-6, theta=1e4, W_kv_a=FAKE, s_kv_a=None,
             gamma=FAKE, W_kv_b=FAKE, s_kv_b=None, hidden=FAKE, positions=FAKE, k_nope=FAKE,
             value=FAKE, k_pe=FAKE, compressed_kv=FAKE, slot_mapping=None, kv_cache=None,
             kv_cache_q=None, kv_scale=None, num_slots=0, workspace=FAKE,
             workspace_bytes=1 << 40)
    d.update(kw)
    return mla.mla_prolog_graph_desc_t(**d)


def create(desc, buckets):
    out = ctypes.c_void_p(None)
    arr = (ctypes.c_int64 * max(1, len(buckets)))(*buckets)
    st = mla.lib().mla_prolog_graphs_create(ctypes.byref(desc) if desc is not None else None,
                                            arr if buckets else None, len(buckets),
                                            ctypes.byref(out))
    return st, out.value


def test_graph_set_argument_errors():
    L = mla.lib()
    bad = mla.MLA_ERR_INVALID_ARG
    # bucket lists: empty, zero, unsorted, repeated, too many, above the limit
    for b in ([], [0], [4, 2], [2, 2], list(range(1, 66)), [mla.MLA_MAX_TOKENS + 1]):
        assert create(graph_desc(), b) == (bad, None), b
    assert create(None, [1]) == (bad, None)
    assert L.mla_prolog_graphs_create(ctypes.byref(graph_desc()),
                                      (ctypes.c_int64 * 1)(1), 1, None) == bad
    # every check of the recorded call, for every bucket, before any capture
    assert create(graph_desc(hidden=None), [1, 64])[0] == bad
    assert create(graph_desc(k_pe=FAKE + 8), [1])[0] == mla.MLA_ERR_MISALIGNED
    assert create(graph_desc(dt=7), [1])[0] == bad
    assert create(graph_desc(eps=float("nan")), [1])[0] == bad
    assert create(graph_desc(d=Dims(H=2048, nh=16, r=256).c()), [1])[0] == \
        mla.MLA_ERR_UNSUPPORTED
    assert create(graph_desc(w8a8=2), [1])[0] == bad
    # a workspace that fits the small bucket but not the large one
    small = mla.mla_kv_prolog_workspace_size(1, V2)
    assert small < mla.mla_kv_prolog_workspace_size(4096, V2)
    assert create(graph_desc(workspace_bytes=small), [1, 4096])[0] == mla.MLA_ERR_WORKSPACE
    assert create(graph_desc(workspace=None), [1])[0] == mla.MLA_ERR_WORKSPACE
    # a cache needs its slot mapping; W8A8 needs its scales and H % 128 == 0
    assert create(graph_desc(num_slots=8, kv_cache=FAKE), [1])[0] == bad
    w8 = dict(w8a8=1, s_kv_a=FAKE, s_kv_b=FAKE)
    assert create(graph_desc(**dict(w8, s_kv_b=None)), [1])[0] == bad
    assert create(graph_desc(**dict(w8, d=Dims(H=64, nh=1).c())), [1])[0] == \
        mla.MLA_ERR_UNSUPPORTED
    # handles: NULL is rejected or ignored
    used = ctypes.c_int64(5)
    assert L.mla_prolog_graphs_launch(None, 1, None, ctypes.byref(used)) == bad
    assert used.value == 0
    assert L.mla_prolog_graphs_bucket(None, 1) == 0
    assert L.mla_prolog_graphs_update(None, ctypes.byref(graph_desc())) == bad
    L.mla_prolog_graphs_destroy(None)


def test_graph_set_checks_pass_before_capture():
    # with arguments that pass every check, create reaches the runtime: on a
    # machine without a GPU that is MLA_ERR_HIP, and nothing is returned
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present: capture would run")
    st, h = create(graph_desc(), [1, 2, 64, 128])
    assert st == mla.MLA_ERR_HIP and h is None
    st, h = create(graph_desc(w8a8=1, s_kv_a=FAKE, s_kv_b=FAKE, d=R1.c()), [4])
    assert st == mla.MLA_ERR_HIP and h is None


def test_python_graph_set_checks_buckets():
    import torch

    w = torch.zeros((2048, 576), dtype=torch.float16)
    g = torch.zeros(512, dtype=torch.float16)
    wb = torch.zeros((512, 4096), dtype=torch.float16)
    for b in ((), (4, 2), (2, 2)):
        with pytest.raises(ValueError):
            mla.PrologGraphs((w, g, wb), b)


def test_handoff_spin_hook_round_trip():
    # setting the bound needs no GPU; the default reads back as -1
    prev = mla.mla_debug_set_handoff_spin(5)
    try:
        assert mla.mla_debug_set_handoff_spin(0) == 5
        assert mla.mla_debug_set_handoff_spin(-7) == 0
        assert mla.mla_debug_set_handoff_spin(-1) == -1
    finally:
        mla.mla_debug_set_handoff_spin(prev)


def test_prefill_fusion_hook_round_trip():
    # needs no GPU; out-of-range modes mean the dispatcher's choice (-1)
    prev = mla.mla_debug_set_prefill_fusion(1)
    try:
        assert mla.mla_debug_set_prefill_fusion(0) == 1
        assert mla.mla_debug_set_prefill_fusion(7) == 0
        assert mla.mla_debug_set_prefill_fusion(-1) == -1
    finally:
        mla.mla_debug_set_prefill_fusion(prev)


def test_launch_event_hook_records_nothing_for_rejected_calls():
    # a call that fails validation launches nothing, so it records none of
    # the registered events (the handles are never touched)
    L = mla.lib()
    evs = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    assert L.mla_debug_set_launch_events(evs, 4) == 0
    try:
        assert call_fp(T=4, dt=7) != 0
        assert call_w8(T=4, d=Dims(H=100, nh=16)) != 0
    finally:
        assert L.mla_debug_set_launch_events(None, 0) == 0
    assert L.mla_debug_set_launch_events(None, -3) == 0


def call_noalloc(T=4, d=V2, ptrs=None, dt=1, eps=1e-6, theta=1e4):
    p = [FAKE] * 9 if ptrs is None else ptrs
    return mla.lib().mla_kv_prolog_noalloc(p[0], p[1], p[2], p[3], p[4], T, d.c(), dt, eps,
                                           theta, p[5], p[6], p[7], p[8], None)


def test_noalloc_argument_errors():
    # every check runs before the library looks up its scratch array (which
    # needs a GPU), so each error is reported here as it is on a GPU machine
    for i in range(9):
        p = [FAKE] * 9
        p[i] = None
        assert call_noalloc(ptrs=p) == mla.MLA_ERR_INVALID_ARG, i
        p[i] = FAKE + 8
        assert call_noalloc(ptrs=p) == mla.MLA_ERR_MISALIGNED, i
    assert call_noalloc(T=-1) == mla.MLA_ERR_INVALID_ARG
    assert call_noalloc(dt=9) == mla.MLA_ERR_INVALID_ARG
    assert call_noalloc(eps=-1.0) == mla.MLA_ERR_INVALID_ARG
    assert call_noalloc(d=Dims(H=2048, nh=16, r=256)) == mla.MLA_ERR_UNSUPPORTED
    assert call_noalloc(T=0, ptrs=[None] * 9) == mla.MLA_OK


def test_noalloc_rejects_token_counts_beyond_its_array():
    # the largest V2-Lite token count whose workspace fits is accepted by the
    # size check; the next token count that does not fit is rejected with
    # MLA_ERR_WORKSPACE before anything else (no launch)
    lim = mla.MLA_NOALLOC_SCRATCH_BYTES
    T = 40000
    assert mla.mla_kv_prolog_workspace_size(T, V2) > lim
    assert call_noalloc(T=T) == mla.MLA_ERR_WORKSPACE
    assert call_noalloc(T=T, ptrs=[None] * 9) == mla.MLA_ERR_WORKSPACE
    fits = max(t for t in range(1, 30000, 97) if mla.mla_kv_prolog_workspace_size(t, V2) <= lim)
    # a fitting size passes every host check (the bad pointer below is then
    # what stops it, before any launch)
    p = [FAKE] * 9
    p[0] = None
    assert call_noalloc(T=fits, ptrs=p) == mla.MLA_ERR_INVALID_ARG


def test_multi_layer_graph_set_argument_errors():
    L = mla.lib()
    bad = mla.MLA_ERR_INVALID_ARG

    def create_layers(descs, buckets=(1, 64)):
        out = ctypes.c_void_p(None)
        arr = (mla.mla_prolog_graph_desc_t * max(1, len(descs)))(*descs)
        b = (ctypes.c_int64 * len(buckets))(*buckets)
        st = L.mla_prolog_graphs_create_layers(arr if descs else None, len(descs), b,
                                               len(buckets), ctypes.byref(out))
        return st, out.value

    assert create_layers([]) == (bad, None)
    assert create_layers([graph_desc()] * 257) == (bad, None)
    # the layers must record the same kind of call
    assert create_layers([graph_desc(), graph_desc(d=Dims(H=1024, nh=16).c())])[0] == bad
    assert create_layers([graph_desc(), graph_desc(dt=2)])[0] == bad
    assert create_layers([graph_desc(), graph_desc(w8a8=1, s_kv_a=FAKE, s_kv_b=FAKE)])[0] == bad
    # every layer's checks run before any capture
    assert create_layers([graph_desc(), graph_desc(hidden=None)])[0] == bad
    assert create_layers([graph_desc(), graph_desc(k_pe=FAKE + 8)])[0] == mla.MLA_ERR_MISALIGNED
    assert L.mla_prolog_graphs_layers(None) == 0
    arr = (mla.mla_prolog_graph_desc_t * 2)(graph_desc(), graph_desc())
    assert L.mla_prolog_graphs_update_layers(None, arr, 2) == bad
