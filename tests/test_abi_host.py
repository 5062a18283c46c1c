"""Host-side checks of the C ABI that need no GPU: the library loads, every
function include/ep.h declares is exported, host-only queries return the
documented sizes, and bad arguments are rejected before anything is enqueued
(these calls return before any HIP call, so they run without a device)."""
import ctypes

import pytest
from hypothesis import event, given, settings, strategies as st

import combine_get_dispatch_amd as ep


def test_library_exports_every_declared_function():
    names = ep.header_functions()
    assert set(names) >= {"ep_get_dispatch_layout", "ep_dispatch", "ep_combine"}
    L = ep.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in ep.h but not exported"


def test_status_strings():
    L = ep.lib()
    for code in range(7):
        assert L.ep_status_string(code) != b"unknown status"
    assert L.ep_status_string(99) == b"unknown status"


def test_capacity_and_workspace_queries():
    cfg = ep.ep_config_t(4096, 7168, 8, 256, 8, 1)
    assert ep.ep_recv_capacity_rows(cfg) == 4096 * 8
    cfg4 = ep.ep_config_t(4, 8, 2, 4, 2, 4)
    assert ep.ep_recv_capacity_rows(cfg4) == 4 * 2 + 4 * 3
    n = ep.ep_layout_workspace_bytes(cfg)
    # header + tile histogram + tile rank counts + counts + in-tile ranks
    assert n >= 4 * (16 + 16 * 256 + 16 * 8 + 256 + 4096 * 8) and n % 256 == 0


@pytest.mark.parametrize("bad", [
    (4, 8, 2, 6, 4, 1),     # E % R != 0
    (4, 12, 2, 4, 2, 1),    # H % 8 != 0
    (4, 8, 5, 4, 2, 1),     # k > E
    (4, 8, 33, 64, 2, 1),   # k > EP_MAX_TOPK
    (4, 8, 2, 2048, 2, 1),  # E > EP_MAX_EXPERTS
    (4, 8, 2, 128, 128, 1), # R > EP_MAX_RANKS
    (4, 8, 2, 4, 2, 0),     # A < 1
    (-1, 8, 2, 4, 2, 1),    # T < 0
    (1 << 28, 8, 8, 4, 2, 1),  # T*k overflows int32 rows
])
def test_bad_config_rejected(bad):
    with pytest.raises(ep.EpError) as e:
        ep.ep_recv_capacity_rows(ep.ep_config_t(*bad))
    assert e.value.status == ep.EP_ERR_INVALID_ARG
    assert ep.lib().ep_last_error_string()
    # the short name is the same function
    assert ep.lib().ep_last_error() == ep.lib().ep_last_error_string()


def _fake(n):
    return ctypes.c_void_p(0x100000 * n)  # never dereferenced: rejected first


def test_dispatch_rejections_happen_before_launch():
    L = ep.lib()
    cfg = ep.ep_config_t(16, 200, 2, 4, 2, 1)  # H % 128 != 0
    h = ep.ep_handle_t()
    st = L.ep_dispatch(ctypes.byref(cfg), ep.EP_DTYPE_FP8_E4M3, _fake(1), _fake(2), None,
                       _fake(3), _fake(4), 1 << 20, 32, 1, _fake(5), _fake(6), None, _fake(7),
                       _fake(8), _fake(9), ctypes.byref(h), None)
    assert st == ep.EP_ERR_INVALID_ARG and b"128" in L.ep_last_error()
    cfg = ep.ep_config_t(16, 256, 2, 4, 2, 1)
    st = L.ep_dispatch(ctypes.byref(cfg), 7, _fake(1), _fake(2), None, _fake(3), _fake(4),
                       1 << 20, 32, 1, _fake(5), _fake(6), None, _fake(7), _fake(8), _fake(9),
                       None, None)
    assert st == ep.EP_ERR_INVALID_ARG  # unknown dtype
    st = L.ep_dispatch(ctypes.byref(cfg), ep.EP_DTYPE_BF16, _fake(1), _fake(2), None,
                       _fake(3), _fake(4), 16, 32, 1, _fake(5), None, None, _fake(7), _fake(8),
                       _fake(9), None, None)
    assert st == ep.EP_ERR_INVALID_ARG and b"workspace" in L.ep_last_error()
    st = L.ep_dispatch(ctypes.byref(cfg), ep.EP_DTYPE_BF16, None, _fake(2), None,
                       _fake(3), _fake(4), 1 << 20, 32, 1, _fake(5), None, None, _fake(7),
                       _fake(8), _fake(9), None, None)
    assert st == ep.EP_ERR_INVALID_ARG  # NULL x
    st = L.ep_dispatch(ctypes.byref(cfg), ep.EP_DTYPE_BF16, ctypes.c_void_p(0x100008),
                       _fake(2), None, _fake(3), _fake(4), 1 << 20, 32, 1, _fake(5), None, None,
                       _fake(7), _fake(8), _fake(9), None, None)
    assert st == ep.EP_ERR_INVALID_ARG and b"aligned" in L.ep_last_error()


def test_layout_and_combine_rejections():
    L = ep.lib()
    cfg = ep.ep_config_t(16, 256, 2, 4, 2, 1)
    st = L.ep_get_dispatch_layout(ctypes.byref(cfg), _fake(1), _fake(2), _fake(3), _fake(4),
                                  _fake(5), _fake(6), _fake(7), 8, _fake(8), None, None)
    assert st == ep.EP_ERR_INVALID_ARG and b"workspace" in L.ep_last_error()
    st = L.ep_get_dispatch_layout(ctypes.byref(cfg), _fake(1), _fake(2), _fake(3), _fake(4),
                                  _fake(5), _fake(6), ctypes.c_void_p(0x100010), 1 << 20,
                                  _fake(8), None, None)
    assert st == ep.EP_ERR_INVALID_ARG and b"aligned" in L.ep_last_error()
    assert L.ep_combine(None, _fake(1), None, _fake(2), None) == ep.EP_ERR_INVALID_ARG
    h = ep.ep_handle_t()
    h.config = ep.ep_config_t(16, 256, 2, 4, 2, 1)
    h.capacity = -1
    assert L.ep_combine(ctypes.byref(h), _fake(1), None, _fake(2), None) == ep.EP_ERR_INVALID_ARG
    h.capacity = 32
    h.tok_slot_row = None
    assert L.ep_combine(ctypes.byref(h), _fake(1), None, _fake(2), None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_read_status(None, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_workspace_init(None, 1024, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_workspace_init(ctypes.c_void_p(0x100010), 1024, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_workspace_init(_fake(1), 64, None) == ep.EP_ERR_INVALID_ARG


def test_probe_rejects_bad_arguments_before_launch():
    """The HBM probe checks kind, workgroup count, size and pointers before
    any HIP call (include/ep_probe.h)."""
    L = ep.lib()
    buf = ctypes.c_void_p(256)  # never dereferenced: every call below is rejected first
    cases = [(7, 1, 1024, buf, buf, 4096),       # unknown kind
             (ep.EP_PROBE_COPY, 1, 0, buf, buf, 4096),       # no workgroups
             (ep.EP_PROBE_COPY, 1, 1024, buf, buf, 100),     # not a multiple of 16
             (ep.EP_PROBE_COPY, 1, 1024, None, buf, 4096),   # copy needs a source
             (ep.EP_PROBE_WRITE, 1, 1024, None, ctypes.c_void_p(264), 4096)]  # misaligned
    for kind, nt, wgs, src, dst, nbytes in cases:
        st = L.ep_hbm_probe(kind, nt, wgs, src, dst, nbytes, None)
        assert st == ep.EP_ERR_INVALID_ARG
        assert L.ep_last_error().decode().startswith("probe")


def test_layout_dispatch_rejects_bad_arguments_before_launch():
    """ep_layout_dispatch takes any batch size; a bad argument is rejected
    before anything is enqueued, on either side of the one-launch bound."""
    L = ep.lib()
    P = ctypes.c_void_p(256)
    for T in (256, 257, 4096):
        cfg = ep.ep_config_t(T, 256, 8, 256, 8, 1)
        st = L.ep_layout_dispatch(ctypes.byref(cfg), ep.EP_DTYPE_BF16, P, P, P, P, P, P, P, P, P,
                                  16, T * 8, 1, P, P, P, P, P, P, None, None)
        assert st == ep.EP_ERR_INVALID_ARG and "workspace" in L.ep_last_error().decode()
        st = L.ep_layout_dispatch(ctypes.byref(cfg), ep.EP_DTYPE_BF16, ctypes.c_void_p(264), P,
                                  P, P, P, P, P, P, P, 1 << 24, T * 8, 1, P, P, P, P, P, P,
                                  None, None)
        assert st == ep.EP_ERR_INVALID_ARG and "aligned" in L.ep_last_error().decode()


def test_combine_ranked_rejects_item_overflow_before_launch():
    """The ranked combine runs one 64-lane wave per (row, 512-column chunk)
    item, and one launch holds fewer than 2^32 lanes; a handle with more
    items than that is rejected before anything is enqueued (2^22 tokens,
    top-8 over 8 ranks, hidden 7168: a valid config, but 2^25 rows x 14
    chunks)."""
    L = ep.lib()
    h = ep.ep_ranked_handle_t()
    h.config = ep.ep_config_t(1 << 22, 7168, 8, 32, 8, 1)
    h.capacity = (1 << 22) * 8
    h.ranked_capacity = (1 << 22) * 8
    for i, name in enumerate(("rank_token_offsets", "tok_rank_row", "tok_slot_row",
                              "ne_topk_idx", "ne_topk_weights", "ne_src")):
        setattr(h, name, 0x100000 * (i + 1))
    P = ctypes.c_void_p(256)
    st = L.ep_combine_ranked(ctypes.byref(h), P, 1, P, P, None)
    assert st == ep.EP_ERR_INVALID_ARG
    assert "too large" in L.ep_last_error().decode()
    h.ranked_capacity = ((1 << 26) - 4) // 14 + 1
    assert L.ep_combine_ranked(ctypes.byref(h), P, 1, P, P, None) == ep.EP_ERR_INVALID_ARG
    assert "too large" in L.ep_last_error().decode()


def test_combine_backward_rejects_too_many_tokens_before_launch():
    """Combine backward runs one 256-lane workgroup per token, so at most
    2^24 - 1 tokens fit one launch (hidden 8 keeps the config itself valid)."""
    L = ep.lib()
    h = ep.ep_handle_t()
    h.config = ep.ep_config_t(1 << 24, 8, 1, 1, 1, 1)
    h.capacity = 1 << 24
    h.tok_slot_row = 256
    P = ctypes.c_void_p(256)
    st = L.ep_combine_backward(ctypes.byref(h), P, None, P, P, None, None)
    assert st == ep.EP_ERR_INVALID_ARG
    assert "too large" in L.ep_last_error().decode()


def test_missing_library_fails_loudly():
    """Without libep.so every call raises: there is no CPU fallback on the
    product path.  Run in a child process so this process keeps its library."""
    import subprocess
    import sys
    import textwrap

    code = textwrap.dedent("""
        import combine_get_dispatch_amd as ep
        ep.LIB_PATH = "/nonexistent/libep.so"
        ep._lib = None
        for call in (ep.lib, lambda: ep.ep_recv_capacity_rows(ep.ep_config_t(4, 8, 1, 2, 1, 1))):
            try:
                call()
            except RuntimeError as err:
                assert "not built" in str(err), err
            else:
                raise SystemExit("a call succeeded without the library")
        print("raised")
    """)
    root = __import__("os").path.dirname(__import__("os").path.dirname(__file__))
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0 and "raised" in res.stdout, res.stderr


def _config_is_valid(T, H, k, E, R, A):
    """The rules include/ep.h states for ep_config_t, written out."""
    int32_max = 2**31 - 1
    return (T >= 0 and H >= 8 and H % 8 == 0 and 1 <= E <= 1024 and 1 <= k <= min(E, 32)
            and 1 <= R <= 64 and E % R == 0 and A >= 1
            and T * k + E * (A - 1) < int32_max
            and T * -(-H // 512) <= 2**26 - 4)


@st.composite
def _configs(draw):
    """Configurations on both sides of every rule: a valid one is built,
    then some fields are moved across (or near) their limits."""
    R = draw(st.sampled_from([1, 2, 4, 8, 16, 64]))
    E = R * draw(st.integers(1, 1024 // R))
    k = draw(st.integers(1, min(E, 32)))
    H = 8 * draw(st.integers(1, 2048))
    A = draw(st.sampled_from([1, 2, 4, 128]))
    T = draw(st.one_of(st.integers(0, 5000), st.sampled_from([
        (2**31 - 1 - E * (A - 1)) // k, (2**31 - 1 - E * (A - 1)) // k + 1,
        (2**26 - 4) // -(-H // 512), (2**26 - 4) // -(-H // 512) + 1])))
    f = [T, H, k, E, R, A]
    edits = {0: [-1, 2**31 - 1], 1: [0, 4, H + 4, 12], 2: [0, E + 1, 33], 3: [0, 1025, E + 1],
             4: [0, 65, 3, E + 1], 5: [0, -1, 2**30]}
    for i in draw(st.sets(st.integers(0, 5), max_size=2)):
        f[i] = draw(st.sampled_from(edits[i]))
    return tuple(max(-(2**31), min(v, 2**31 - 1)) for v in f)


@settings(max_examples=3000, derandomize=True, deadline=None)
@given(_configs())
def test_config_accepted_exactly_when_the_stated_rules_hold(config):
    """Every host entry point validates the config first; the size query
    accepts exactly the configurations include/ep.h allows and then returns
    T*k + E*(A-1) rows and a 256-byte multiple of workspace."""
    T, H, k, E, R, A = config
    cfg = ep.ep_config_t(T, H, k, E, R, A)
    valid = _config_is_valid(T, H, k, E, R, A)
    event("valid" if valid else "invalid")
    if valid:
        assert ep.ep_recv_capacity_rows(cfg) == T * k + E * (A - 1)
        n = ep.ep_layout_workspace_bytes(cfg)
        assert n % 256 == 0 and n >= 4 * T * k
    else:
        with pytest.raises(ep.EpError) as e:
            ep.ep_recv_capacity_rows(cfg)
        assert e.value.status == ep.EP_ERR_INVALID_ARG


def test_last_error_is_per_thread():
    """ep_last_error describes the last failure of the calling thread: a
    rejection in one thread leaves another thread's message untouched."""
    import threading

    L = ep.lib()
    seen = {}

    def fail():
        st = L.ep_recv_capacity_rows(ctypes.byref(ep.ep_config_t(4, 8, 5, 4, 2, 1)),
                                     ctypes.byref(ctypes.c_int64()))
        seen["fail"] = (st, L.ep_last_error())

    def quiet():
        seen["quiet_before"] = L.ep_last_error()
        th = threading.Thread(target=fail)
        th.start()
        th.join()
        seen["quiet_after"] = L.ep_last_error()

    th = threading.Thread(target=quiet)
    th.start()
    th.join()
    assert seen["fail"][0] == ep.EP_ERR_INVALID_ARG and seen["fail"][1]
    assert seen["quiet_before"] == b"" and seen["quiet_after"] == b""
