"""The C ABI on the CPU: the built library loads and exports every function
include/em.h declares; host-only calls and argument checks behave as the
header states.  Nothing here launches GPU work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "em.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(em_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from merge_front_coded_amd import binding
    return binding.load_library()


def test_header_declares_the_calls():
    names = _declared()
    for n in ("em_partition", "em_merge_keep", "em_collision_rank", "em_fc_lengths", "em_scan",
              "em_emit", "em_workspace_bytes", "em_payload_bound_bits", "em_rank512_probe",
              "em_strerror", "em_last_hip_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, f"libem.so lacks {missing}"


def test_binding_wraps_every_declared_symbol():
    from merge_front_coded_amd import binding
    missing = [n for n in _declared() if n not in ("em_strerror", "em_last_hip_error")
               and not hasattr(binding, n)]
    assert not missing


def test_strerror_and_last_error(lib):
    assert lib.em_strerror(0) == b"success"
    assert b"capacity" in lib.em_strerror(-3)
    assert lib.em_strerror(-99) == b"unknown error code"
    assert lib.em_last_hip_error() == 0


def _side(n=0, key_bytes=0, val_bytes=0, ptr=0x1000):
    from merge_front_coded_amd.binding import em_side_t
    return em_side_t(ptr, ptr, ptr, ptr, None, n, key_bytes, val_bytes)


def test_payload_bound(lib):
    A, B = _side(10, 100, 50), _side(5, 40, 0)
    out = ctypes.c_uint64()
    assert lib.em_payload_bound_bits(ctypes.byref(A), ctypes.byref(B), ctypes.byref(out)) == 0
    assert out.value == 8 * (100 + 50 + 40) + 15 * 184
    big = _side(1 << 24, 0, 0)
    assert lib.em_payload_bound_bits(ctypes.byref(big), ctypes.byref(B), ctypes.byref(out)) == -2
    assert lib.em_payload_bound_bits(None, ctypes.byref(B), ctypes.byref(out)) == -1


def test_workspace_sizes_grow_with_inputs(lib):
    small = lib.em_workspace_bytes(1000, 1000, 2048)
    large = lib.em_workspace_bytes(8_000_000, 8_000_000, 2048)
    assert 0 < small < large and large % 256 == 0
    assert lib.em_workspace_bytes(8_000_000, 8_000_000, 1) > large  # one descriptor per output
    assert lib.em_rank512_workspace_bytes(0) > 0


def test_argument_errors_before_any_launch(lib):
    A, B = _side(), _side()
    buf = ctypes.c_void_p(0x100000)
    # null splits, zero or oversized partition sizes
    assert lib.em_partition(ctypes.byref(A), ctypes.byref(B), 16, None, None, 0, None) == -1
    assert lib.em_partition(ctypes.byref(A), ctypes.byref(B), 0, buf, None, 0, None) == -1
    # merge tiles hold at most EM_MAX_ITEMS_PER_PART outputs; em_merge_fc's 2048
    assert lib.em_merge_keep(ctypes.byref(A), ctypes.byref(B), buf, 4097, buf, None, None, buf,
                             ctypes.c_void_p(0x100000), 1 << 20, None) == -1
    for items, coarse in ((0, 256), (2049, 4098), (64, 100), (64, 0)):
        assert lib.em_merge_fc(ctypes.byref(A), ctypes.byref(B), buf, coarse, items, buf, 1 << 20, buf,
                               buf, None, None, None, None, None, None, ctypes.c_void_p(0x100000),
                               1 << 20, None) == -1
    # the two halves of em_merge_fc check the same way
    assert lib.em_merge_lengths(ctypes.byref(A), ctypes.byref(B), buf, 64, 0, buf, buf, None, None, None, None,
                                None, ctypes.c_void_p(0x100000), 1 << 20, None) == -1
    assert lib.em_merge_lengths(ctypes.byref(A), ctypes.byref(B), None, 64, 64, buf, buf, None, None, None,
                                None, None, ctypes.c_void_p(0x100000), 1 << 20, None) == -1
    assert lib.em_emit_merged(ctypes.byref(A), ctypes.byref(B), 64, ctypes.c_void_p(0x100008), 1 << 20, buf,
                              buf, None, None, None, ctypes.c_void_p(0x100000), 1 << 20, None) == -1
    assert lib.em_emit_merged(ctypes.byref(A), ctypes.byref(B), 64, buf, 1 << 20, buf, buf, None, None, None,
                              ctypes.c_void_p(0x100000), 0, None) == -3
    # misaligned arena
    bad = _side(ptr=0x1001)
    assert lib.em_partition(ctypes.byref(bad), ctypes.byref(B), 16, buf, None, 0, None) == -1
    # record cap
    big = _side(n=(1 << 24) - 1)
    one = _side(n=1)
    assert lib.em_partition(ctypes.byref(big), ctypes.byref(one), 16, buf, None, 0, None) == -2
    # workspace too small
    A5 = _side(n=5, key_bytes=5, val_bytes=0)
    assert lib.em_merge_keep(ctypes.byref(A5), ctypes.byref(B), buf, 4, buf, None, None, buf,
                             ctypes.c_void_p(0x100000), 0, None) == -3
    assert lib.em_scan(buf, 10, buf, ctypes.c_void_p(0x100000), 0, None) == -3
    # emit: S and T must agree on emptiness; payload capacity
    assert lib.em_emit(ctypes.byref(A5), ctypes.byref(B), buf, None, 0, buf, 5, buf, 1, buf, 0,
                       None) == -1
    assert lib.em_emit(ctypes.byref(A5), ctypes.byref(B), buf, None, 2, buf, 100, buf, 3, buf, 0,
                       None) == -3
    assert lib.em_rank512_probe(None, 5, None, 0, None, ctypes.c_void_p(0x100000), 1 << 20, None) == -1
    assert lib.em_rank2048_probe(None, 5, None, 0, None, ctypes.c_void_p(0x100000), 1 << 20, None) == -1
    assert lib.em_rank2048_probe(buf, 5, None, 0, None, ctypes.c_void_p(0x100000), 0, None) == -3
    # collision modes: an unknown mode, and each mode's own workspace size
    assert lib.em_collision_rank_mode(ctypes.byref(A5), ctypes.byref(B), 4, buf, None, None, buf,
                                      ctypes.c_void_p(0x100000), 1 << 20, None) == -1
    compact = lib.em_collision_workspace_bytes(1000, 10, 3)
    assert compact >= lib.em_collision_workspace_bytes(1000, 10, 2) + 4000
    assert lib.em_collision_rank_mode(ctypes.byref(A5), ctypes.byref(B), 3, buf, None, None, buf,
                                      ctypes.c_void_p(0x100000), lib.em_collision_workspace_bytes(5, 0, 2),
                                      None) == -3


def test_byte_profile_argument_errors(lib):
    A5, B = _side(n=5, key_bytes=5, val_bytes=0), _side()
    buf = ctypes.c_void_p(0x100000)
    ws = ctypes.c_void_p(0x100000)
    assert lib.em_bp_workspace_bytes(5) >= 16
    # more survivors than records; no width output; misaligned or small workspace
    assert lib.em_bp_lengths(ctypes.byref(A5), ctypes.byref(B), buf, buf, 6, buf, buf, ws, 256, None) == -1
    assert lib.em_bp_lengths(ctypes.byref(A5), ctypes.byref(B), buf, buf, 5, buf, None, ws, 256, None) == -1
    assert lib.em_bp_lengths(ctypes.byref(A5), ctypes.byref(B), buf, buf, 5, buf, buf,
                             ctypes.c_void_p(0x100008), 256, None) == -1
    assert lib.em_bp_lengths(ctypes.byref(A5), ctypes.byref(B), buf, buf, 5, buf, buf, ws, 0, None) == -3
    # emit: S and T agree on emptiness; payload capacity; overflow flag required
    assert lib.em_bp_emit(ctypes.byref(A5), ctypes.byref(B), buf, buf, 0, buf, 5, buf, buf, 10, buf, None) == -1
    assert lib.em_bp_emit(ctypes.byref(A5), ctypes.byref(B), buf, buf, 5, buf, 50, buf, buf, 49, buf, None) == -3
    assert lib.em_bp_emit(ctypes.byref(A5), ctypes.byref(B), buf, buf, 5, buf, 50, buf, buf, 64, None, None) == -1
    # navigation over byte offsets: the width comes from the device; record cap
    assert lib.em_bp_navigation(buf, 5, 50, None, buf, 8, buf, 8, buf, 8, buf, 8, buf, ws, 1 << 20, None) == -1
    assert lib.em_bp_navigation(buf, 1 << 24, 50, buf, buf, 8, buf, 8, buf, 8, buf, 8, buf, ws, 1 << 20,
                                None) == -2


def test_onepass_argument_errors(lib):
    A, B = _side(), _side()
    buf = ctypes.c_void_p(0x100000)
    ws = ctypes.c_void_p(0x100000)
    # partition sizes, coarse splits that are not a multiple, a misaligned payload, no splits
    for items, coarse in ((0, 256), (1025, 2050), (64, 100)):
        assert lib.em_merge_fc_onepass(ctypes.byref(A), ctypes.byref(B), buf, coarse, items, buf, 1 << 20, buf,
                                       buf, None, None, None, None, None, None, ws, 1 << 20, None) == -1
    assert lib.em_merge_fc_onepass(ctypes.byref(A), ctypes.byref(B), buf, 64, 64, ctypes.c_void_p(0x100008),
                                   1 << 20, buf, buf, None, None, None, None, None, None, ws, 1 << 20, None) == -1
    assert lib.em_merge_fc_onepass(ctypes.byref(A), ctypes.byref(B), None, 64, 64, buf, 1 << 20, buf, buf, None,
                                   None, None, None, None, None, ws, 1 << 20, None) == -1
    # workspace too small
    A5 = _side(n=5, key_bytes=5, val_bytes=0)
    assert lib.em_merge_fc_onepass(ctypes.byref(A5), ctypes.byref(B), buf, 64, 64, buf, 1 << 20, buf, buf, None,
                                   None, None, None, None, None, ws, 0, None) == -3


def test_fcin_prefix8_argument_errors(lib):
    buf = ctypes.c_void_p(0x100000)
    need = lib.em_fcin_workspace_bytes(5)
    assert lib.em_fcin_prefix8(buf, 4, 5, buf, None, need, None) == -1  # no workspace
    assert lib.em_fcin_prefix8(buf, 4, 5, buf, ctypes.c_void_p(0x100008), need, None) == -1  # misaligned
    assert lib.em_fcin_prefix8(None, 4, 5, buf, buf, need, None) == -1  # no payload
    assert lib.em_fcin_prefix8(buf, 4, 5, None, buf, need, None) == -1  # no output
    assert lib.em_fcin_prefix8(buf, 4, 1 << 24, buf, buf, 1 << 40, None) == -2  # record cap
    assert lib.em_fcin_prefix8(buf, 4, 5, buf, buf, need - 1, None) == -3  # workspace too small
    assert lib.em_fcin_prefix8(None, 0, 0, None, buf, lib.em_fcin_workspace_bytes(0), None) == 0  # nothing to do


def test_fcin_compare_argument_errors(lib):
    buf = ctypes.c_void_p(0x100000)
    mis = ctypes.c_void_p(0x100008)
    need = lib.em_fcin_workspace_bytes(5)

    def call(pa=buf, Sa=5, wa=buf, na=need, pb=buf, Sb=5, wb=buf, nb=need, n=3, ia=buf, jb=buf, lcp=buf, cmp=buf):
        return lib.em_fcin_compare(pa, 4, Sa, wa, na, pb, 4, Sb, wb, nb, n, ia, jb, 0, lcp, cmp, None)

    assert call(wa=None) == -1 and call(wb=mis) == -1  # no or misaligned workspace
    assert call(pa=None) == -1 and call(pb=None) == -1  # no payload with records
    assert call(ia=None) == -1 and call(jb=None) == -1  # no indices
    assert call(lcp=None, cmp=None) == -1  # no output
    assert call(Sa=1 << 24, na=1 << 40) == -2 and call(Sb=1 << 24, nb=1 << 40) == -2  # record cap
    assert call(na=need - 1) == -3 and call(nb=need - 1) == -3  # workspace too small
    assert call(n=0, ia=None, jb=None, lcp=None, cmp=None) == 0  # nothing to do
    assert call(pa=None, Sa=0, na=lib.em_fcin_workspace_bytes(0), n=0) == 0


def test_missing_library_fails_loudly(tmp_path):
    """Without the HIP library the binding raises; there is no CPU fallback."""
    from merge_front_coded_amd import binding
    with pytest.raises(ImportError):
        binding.load_library(str(tmp_path / "libem.so"))
