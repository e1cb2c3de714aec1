"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, and its host-side validation and workspace queries behave.  None of
these calls reaches a HIP API (every invalid call returns before enqueueing)."""
import ctypes

import pytest

import gemm_exl3_linear_amd as X


def _w(k=256, n=256, bits=4, cb=X.CODEBOOK_MUL1, ptr=16):
    return X._Weight(ptr, ptr, ptr, 0, k, n, bits, cb)


def test_library_exports_every_header_function():
    L = X.lib()
    names = X.header_functions()
    assert {"exl3_linear", "exl3_grouped_experts", "exl3_hadamard", "exl3_reconstruct"} <= set(names)
    for nm in names:
        assert hasattr(L, nm), nm


def test_abi_version_and_status_strings():
    assert X.abi_version() == 1
    for s in range(5):
        assert X.status_str(s)
    assert "unknown" in X.status_str(99)


def test_workspace_queries_are_host_only():
    L = X.lib()
    w = _w(5120, 17408, 4)
    for m in (1, 4, 16):
        ws = L.exl3_linear_workspace_size(ctypes.byref(w), m)
        assert ws > 0 and ws % 4 == 0
    assert L.exl3_linear_workspace_size(ctypes.byref(w), 4096) == 4096 * 5120 * 2
    assert L.exl3_linear_workspace_size(ctypes.byref(_w(bits=9)), 1) == 0
    assert L.exl3_linear_workspace_size(ctypes.byref(_w(k=200)), 1) == 0
    gu = X._Arena(16, 16, 16, 256, 2, 2048, 512, 3, X.CODEBOOK_MUL1)
    dn = X._Arena(16, 16, 16, 256, 1, 512, 2048, 3, X.CODEBOOK_MUL1)
    assert L.exl3_grouped_experts_workspace_size(ctypes.byref(gu), ctypes.byref(dn), 1, 8) > 0
    assert L.exl3_grouped_experts_workspace_size(ctypes.byref(gu), ctypes.byref(dn), 4096, 8) > 0
    bad = X._Arena(16, 16, 16, 256, 1, 2048, 512, 3, X.CODEBOOK_MUL1)
    assert L.exl3_grouped_experts_workspace_size(ctypes.byref(bad), ctypes.byref(dn), 1, 8) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(bits=0), X.EXL3_E_INVALID),
    (dict(bits=9), X.EXL3_E_INVALID),
    (dict(cb=1), X.EXL3_E_UNSUPPORTED),
    (dict(cb=3), X.EXL3_E_UNSUPPORTED),
    (dict(k=200), X.EXL3_E_INVALID),
    (dict(n=100), X.EXL3_E_INVALID),
    (dict(ptr=0), X.EXL3_E_INVALID),
    (dict(ptr=18), X.EXL3_E_INVALID),
])
def test_linear_rejects_before_enqueue(kw, expect):
    L = X.lib()
    w = _w(**kw)
    st = L.exl3_linear(ctypes.byref(w), 16, 1, w.k, 16, w.n, X.EXL3_F16, 0, 0, 0)
    assert st == expect


def test_linear_other_argument_errors():
    L = X.lib()
    w = _w()
    assert L.exl3_linear(ctypes.byref(w), 16, 1, 255, 16, 256, X.EXL3_F16, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_linear(ctypes.byref(w), 16, 1, 256, 16, 256, 7, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_linear(ctypes.byref(w), 16, -1, 256, 16, 256, X.EXL3_F16, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_linear(ctypes.byref(w), 0, 1, 256, 16, 256, X.EXL3_F16, 0, 0, 0) == X.EXL3_E_INVALID
    # valid shapes but no workspace: refused with the workspace status
    assert L.exl3_linear(ctypes.byref(w), 16, 1, 256, 16, 256, X.EXL3_F16, 0, 0, 0) == X.EXL3_E_WORKSPACE
    need = L.exl3_linear_workspace_size(ctypes.byref(w), 1)
    assert L.exl3_linear(ctypes.byref(w), 16, 1, 256, 16, 256, X.EXL3_F16, 16, need - 4, 0) == X.EXL3_E_WORKSPACE
    # m == 0 is a no-op
    assert L.exl3_linear(ctypes.byref(w), 0, 0, 256, 0, 256, X.EXL3_F16, 0, 0, 0) == X.EXL3_OK
    assert L.exl3_linear(None, 16, 1, 256, 16, 256, X.EXL3_F16, 0, 0, 0) == X.EXL3_E_INVALID


def test_reconstruct_and_hadamard_rejects():
    L = X.lib()
    assert L.exl3_reconstruct(ctypes.byref(_w(bits=0)), 16, 0) == X.EXL3_E_INVALID
    assert L.exl3_reconstruct(ctypes.byref(_w(cb=1)), 16, 0) == X.EXL3_E_UNSUPPORTED
    assert L.exl3_reconstruct(ctypes.byref(_w(k=24)), 16, 0) == X.EXL3_E_INVALID
    assert L.exl3_reconstruct(ctypes.byref(_w()), 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_hadamard(16, 16, 0, 4, 100, 128, 128, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_hadamard(16, 16, 2, 4, 128, 128, 128, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_hadamard(16, 16, 0, 4, 128, 120, 128, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_hadamard(0, 16, 0, 4, 128, 128, 128, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_hadamard(16, 16, 0, 4, 128, 128, 136, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_hadamard(0, 0, 0, 0, 128, 128, 128, 0, 0, 0) == X.EXL3_OK


def test_grouped_rejects():
    L = X.lib()
    gu = X._Arena(16, 16, 16, 8, 2, 256, 128, 3, X.CODEBOOK_MUL1)
    dn = X._Arena(16, 16, 16, 8, 1, 128, 256, 3, X.CODEBOOK_MUL1)
    args = lambda g, d, t, k, ws=0, n=0: L.exl3_grouped_experts(ctypes.byref(g), ctypes.byref(d), 16, 16, 16,
                                                                   t, k, 16, ws, n, 0)
    assert args(gu, dn, 1, 0) == X.EXL3_E_INVALID
    assert args(gu, dn, 1, 17) == X.EXL3_E_INVALID
    assert args(gu, dn, 1, 2) == X.EXL3_E_WORKSPACE
    assert args(gu, dn, 0, 2) == X.EXL3_OK
    dn_bad = X._Arena(16, 16, 16, 7, 1, 128, 256, 3, X.CODEBOOK_MUL1)
    assert args(gu, dn_bad, 1, 2) == X.EXL3_E_INVALID
    gu_cb = X._Arena(16, 16, 16, 8, 2, 256, 128, 3, 1)
    assert args(gu_cb, dn, 1, 2) == X.EXL3_E_UNSUPPORTED


def test_grouped_mixed_widths_validation_host_only():
    # widths are read from the host array; the device pointers only need to
    # be present and aligned for the checks (no call here reaches a kernel)
    L = X.lib()
    E = 8
    host = (ctypes.c_int32 * E)(2, 3, 4, 3, 2, 6, 8, 1)
    wgu = X._Widths(ctypes.addressof(host), 16, 16)
    wdn = X._Widths(ctypes.addressof(host), 16, 16)
    gu = X._Arena(16, 16, 16, E, 2, 256, 128, 0, X.CODEBOOK_MUL1)
    dn = X._Arena(16, 16, 16, E, 1, 128, 256, 0, X.CODEBOOK_MUL1)
    size = lambda g, wg, d, wd, t, k: L.exl3_grouped_experts_mixed_workspace_size(
        ctypes.byref(g), ctypes.byref(wg), ctypes.byref(d), ctypes.byref(wd), t, k)
    call = lambda g, wg, d, wd, t, k, ws=0, n=0: L.exl3_grouped_experts_mixed(
        ctypes.byref(g), ctypes.byref(wg), ctypes.byref(d), ctypes.byref(wd), 16, 16, 16, t, k, 16, ws, n, 0)
    # the workspace does not depend on the widths: same as a uniform arena of these shapes
    gu_u = X._Arena(16, 16, 16, E, 2, 256, 128, 3, X.CODEBOOK_MUL1)
    dn_u = X._Arena(16, 16, 16, E, 1, 128, 256, 3, X.CODEBOOK_MUL1)
    for t in (1, 3, 48, 200):
        want = L.exl3_grouped_experts_workspace_size(ctypes.byref(gu_u), ctypes.byref(dn_u), t, 2)
        assert want > 0 and size(gu, wgu, dn, wdn, t, 2) == want
    assert call(gu, wgu, dn, wdn, 1, 2) == X.EXL3_E_WORKSPACE
    assert call(gu, wgu, dn, wdn, 0, 2) == X.EXL3_OK
    assert call(gu, wgu, dn, wdn, 1, 0) == X.EXL3_E_INVALID
    # a uniform record (bits != 0) is not a mixed arena
    assert call(gu_u, wgu, dn, wdn, 1, 2) == X.EXL3_E_INVALID
    assert size(gu_u, wgu, dn, wdn, 1, 2) == 0
    # a width outside 1..8 anywhere in the host array
    for bad in (0, 9, -1):
        host[5] = bad
        assert call(gu, wgu, dn, wdn, 1, 2) == X.EXL3_E_INVALID
        assert size(gu, wgu, dn, wdn, 1, 2) == 0
    host[5] = 6
    # missing or misaligned width arrays
    for w in (X._Widths(0, 16, 16), X._Widths(ctypes.addressof(host), 0, 16),
              X._Widths(ctypes.addressof(host), 16, 0), X._Widths(ctypes.addressof(host), 18, 16),
              X._Widths(ctypes.addressof(host), 16, 20)):
        assert call(gu, w, dn, wdn, 1, 2) == X.EXL3_E_INVALID
        assert call(gu, wgu, dn, w, 1, 2) == X.EXL3_E_INVALID
    # shapes and codebook as for uniform arenas
    dn_bad = X._Arena(16, 16, 16, E - 1, 1, 128, 256, 0, X.CODEBOOK_MUL1)
    assert call(gu, wgu, dn_bad, wdn, 1, 2) == X.EXL3_E_INVALID
    gu_cb = X._Arena(16, 16, 16, E, 2, 256, 128, 0, 1)
    assert call(gu_cb, wgu, dn, wdn, 1, 2) == X.EXL3_E_UNSUPPORTED


def _multi(ws):
    recs = list(ws)
    arr = (ctypes.POINTER(X._Weight) * len(recs))(*[ctypes.pointer(r) for r in recs])
    return arr, recs


def test_linear_multi_workspace_and_rejects():
    # host-only checks: nothing reaches a device for any of these
    L = X.lib()
    q, k_, v = _w(5120, 5120, 7), _w(5120, 1024, 2), _w(5120, 1024, 3)
    arr, _r = _multi([q, k_, v])
    ws1 = L.exl3_linear_multi_workspace_size(arr, 3, 1)
    assert ws1 > 0 and ws1 % 256 == 0
    # m >= 2: the largest single-tensor workspace (tensors run one after another)
    ws4 = L.exl3_linear_multi_workspace_size(arr, 3, 4)
    assert ws4 == max(L.exl3_linear_workspace_size(ctypes.byref(w), 4) for w in (q, k_, v))
    y = (ctypes.c_void_p * 3)(16, 16, 16)
    ld = (ctypes.c_int64 * 3)(5120, 1024, 1024)
    f16 = X.EXL3_F16
    assert L.exl3_linear_multi(arr, 0, 16, 1, 5120, y, ld, f16, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_linear_multi(arr, X.MAX_MULTI + 1, 16, 1, 5120, y, ld, f16, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_linear_multi(None, 3, 16, 1, 5120, y, ld, f16, 0, 0, 0) == X.EXL3_E_INVALID
    # a tensor with another k, an unsupported codebook, a too-small ldy
    arr2, _r2 = _multi([q, _w(1024, 1024, 2)])
    assert L.exl3_linear_multi(arr2, 2, 16, 1, 5120, y, ld, f16, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_linear_multi_workspace_size(arr2, 2, 1) == 0
    arr3, _r3 = _multi([q, _w(5120, 1024, 3, cb=1)])
    assert L.exl3_linear_multi(arr3, 2, 16, 1, 5120, y, ld, f16, 0, 0, 0) == X.EXL3_E_UNSUPPORTED
    ld_bad = (ctypes.c_int64 * 3)(5120, 1000, 1024)
    assert L.exl3_linear_multi(arr, 3, 16, 1, 5120, y, ld_bad, f16, 0, 0, 0) == X.EXL3_E_INVALID
    # missing workspace, then the empty call
    assert L.exl3_linear_multi(arr, 3, 16, 1, 5120, y, ld, f16, 0, 0, 0) == X.EXL3_E_WORKSPACE
    assert L.exl3_linear_multi(arr, 3, 16, 0, 5120, y, ld, f16, 0, 0, 0) == X.EXL3_OK


def test_linear_int8_validation_host_only():
    L = X.lib()
    w = _w(512, 256, 4)
    ws = L.exl3_linear_int8_workspace_size(ctypes.byref(w), 300)
    assert ws >= 300 * 512 + 300 * 4 and ws % 256 == 0
    assert L.exl3_linear_int8_workspace_size(ctypes.byref(w), 0) == 0
    assert L.exl3_linear_int8_workspace_size(ctypes.byref(_w(bits=9)), 4) == 0
    f16 = X.EXL3_F16
    call = lambda ww, m, ws_=0, n=0, ldx=512, ldy=256, dt=f16: L.exl3_linear_int8(
        ctypes.byref(ww), 16, m, ldx, 16, ldy, dt, ws_, n, 0)
    assert call(_w(512, 256, 0), 4) == X.EXL3_E_INVALID
    assert call(_w(512, 256, 4, cb=1), 4) == X.EXL3_E_UNSUPPORTED
    assert call(_w(200, 256, 4), 4, ldx=200) == X.EXL3_E_INVALID
    assert call(w, 4, ldx=500) == X.EXL3_E_INVALID
    assert call(w, 4, dt=7) == X.EXL3_E_INVALID
    assert call(w, -1) == X.EXL3_E_INVALID
    assert call(w, 4) == X.EXL3_E_WORKSPACE
    need = L.exl3_linear_int8_workspace_size(ctypes.byref(w), 4)
    assert call(w, 4, 16, need - 16) == X.EXL3_E_WORKSPACE
    assert call(w, 0) == X.EXL3_OK
    assert L.exl3_reconstruct_int8(ctypes.byref(_w(bits=0)), 16, 0) == X.EXL3_E_INVALID
    assert L.exl3_reconstruct_int8(ctypes.byref(_w(cb=1)), 16, 0) == X.EXL3_E_UNSUPPORTED
    assert L.exl3_reconstruct_int8(ctypes.byref(_w()), 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_reconstruct_int8(ctypes.byref(_w()), 17, 0) == X.EXL3_E_INVALID


def test_row_count_limits_in_workspace_queries():
    # m above 2^24 rows is refused everywhere, queries included (they return 0
    # instead of planning with a truncated row count)
    L = X.lib()
    w = _w(5120, 17408, 4)
    assert L.exl3_linear_workspace_size(ctypes.byref(w), 1 << 24) > 0
    for m in ((1 << 24) + 1, 1 << 31, 1 << 40):
        assert L.exl3_linear_workspace_size(ctypes.byref(w), m) == 0
        assert L.exl3_linear_int8_workspace_size(ctypes.byref(w), m) == 0
        arr = (ctypes.POINTER(X._Weight) * 1)(ctypes.pointer(w))
        assert L.exl3_linear_multi_workspace_size(arr, 1, m) == 0
    big = 1 << 25
    assert L.exl3_linear(ctypes.byref(w), 16, big, 5120, 16, 17408, X.EXL3_F16, 16, 1 << 40, 0) == X.EXL3_E_INVALID


def test_prefill_grids_must_fit_one_launch():
    # 2^24 rows: the GEMM over 32768 columns would need 65536 row tiles x 256
    # column blocks = 2^24 workgroups, and the input transform of k = 5120
    # 2^20 x 40 of them; both past the launch limit, refused before any work
    L = X.lib()
    m = 1 << 24
    wide = _w(128, 32768, 1)
    deep = _w(5120, 128, 1)
    for w in (wide, deep):
        st = L.exl3_linear(ctypes.byref(w), 16, m, w.k, 16, w.n, X.EXL3_F16, 16, 1 << 50, 0)
        assert st == X.EXL3_E_INVALID
    st = L.exl3_linear_int8(ctypes.byref(wide), 16, m, wide.k, 16, wide.n, X.EXL3_F16, 16, 1 << 50, 0)
    assert st == X.EXL3_E_INVALID
    # one row group less keeps the GEMM grid below the limit: the call goes on
    # to its workspace check
    ok = L.exl3_linear(ctypes.byref(wide), 16, m - 256, wide.k, 16, wide.n, X.EXL3_F16, 0, 0, 0)
    assert ok == X.EXL3_E_WORKSPACE


def test_reconstruct_and_hadamard_grid_limits():
    L = X.lib()
    # (k/16)(n/16) = 2^29 tiles is below the 2^31 tile limit but 8 threads
    # per tile would need 2^24 workgroups
    w = _w(1 << 19, 1 << 18, 1)
    assert L.exl3_reconstruct(ctypes.byref(w), 16, 0) == X.EXL3_E_INVALID
    assert L.exl3_reconstruct_int8(ctypes.byref(w), 16, 0) == X.EXL3_E_INVALID
    assert L.exl3_hadamard(16, 16, 0, 1 << 26, 128, 128, 128, 0, 0, 0) == X.EXL3_E_INVALID
    assert L.exl3_hadamard(16, 16, 0, 1 << 25, 256, 256, 256, 0, 0, 0) == X.EXL3_E_INVALID


def test_arena_tensor_size_limits():
    # one (expert, slot) tensor of 4 GiB (65536 x 65536 at 8 bits) is refused,
    # also for an arena with a width per expert (checked at width 8 whatever
    # the host widths say)
    L = X.lib()
    big_gu = X._Arena(16, 16, 16, 2, 2, 65536, 65536, 8, X.CODEBOOK_MUL1)
    big_dn = X._Arena(16, 16, 16, 2, 1, 65536, 65536, 8, X.CODEBOOK_MUL1)
    ok_gu = X._Arena(16, 16, 16, 2, 2, 65536, 32768, 8, X.CODEBOOK_MUL1)
    ok_dn = X._Arena(16, 16, 16, 2, 1, 32768, 65536, 8, X.CODEBOOK_MUL1)
    size = lambda g, d: L.exl3_grouped_experts_workspace_size(ctypes.byref(g), ctypes.byref(d), 1, 2)
    assert size(ok_gu, ok_dn) > 0
    assert size(big_gu, big_dn) == 0
    call = lambda g, d: L.exl3_grouped_experts(ctypes.byref(g), ctypes.byref(d), 16, 16, 16, 1, 2, 16, 0, 0, 0)
    assert call(big_gu, big_dn) == X.EXL3_E_INVALID
    assert call(ok_gu, ok_dn) == X.EXL3_E_WORKSPACE
    host = (ctypes.c_int32 * 2)(2, 2)
    wd = X._Widths(ctypes.addressof(host), 16, 16)
    mgu = X._Arena(16, 16, 16, 2, 2, 65536, 65536, 0, X.CODEBOOK_MUL1)
    mdn = X._Arena(16, 16, 16, 2, 1, 65536, 65536, 0, X.CODEBOOK_MUL1)
    st = L.exl3_grouped_experts_mixed(ctypes.byref(mgu), ctypes.byref(wd), ctypes.byref(mdn), ctypes.byref(wd),
                                      16, 16, 16, 1, 2, 16, 0, 0, 0)
    assert st == X.EXL3_E_INVALID


def test_no_workspace_entry_point_host_checks():
    # exl3_linear_no_workspace validates like exl3_linear and refuses, before
    # any HIP call, a call whose workspace would exceed the library's array
    L = X.lib()
    w = _w(5120, 17408, 4)
    need = L.exl3_linear_workspace_size(ctypes.byref(w), 4096)
    assert need > X.SCRATCH_BYTES
    assert L.exl3_linear_no_workspace(ctypes.byref(w), 16, 4096, 5120, 16, 17408, X.EXL3_F16, 0) == X.EXL3_E_WORKSPACE
    assert L.exl3_linear_no_workspace(ctypes.byref(_w(bits=9)), 16, 1, 256, 16, 256, X.EXL3_F16, 0) == X.EXL3_E_INVALID
    assert L.exl3_linear_no_workspace(ctypes.byref(_w(cb=1)), 16, 1, 256, 16, 256, X.EXL3_F16, 0) == X.EXL3_E_UNSUPPORTED
    assert L.exl3_linear_no_workspace(ctypes.byref(w), 16, 1, 5119, 16, 17408, X.EXL3_F16, 0) == X.EXL3_E_INVALID
    assert L.exl3_linear_no_workspace(ctypes.byref(w), 16, 0, 5120, 16, 17408, X.EXL3_F16, 0) == X.EXL3_OK
    # every decode call of the largest workload tensors fits
    for k, n in ((5120, 17408), (17408, 5120)):
        for m in range(1, 17):
            assert L.exl3_linear_workspace_size(ctypes.byref(_w(k, n, 8)), m) <= X.SCRATCH_BYTES
