"""The C ABI library loads, exports what include/*.h declares, and validates
arguments on the host (every call below fails validation before any HIP call,
so these tests need no GPU)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(nvfp4_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import quantized_kv_decode_amd as qk
    if not os.path.exists(qk.LIB_PATH):
        pytest.fail("libnvfp4kv.so not built (run __graft_entry__.build())")
    return qk.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("nvfp4_kv_calibrate", "nvfp4_kv_append", "nvfp4_decode_attn_workspace_bytes", "nvfp4_decode_attn",
              "nvfp4_decode_step", "nvfp4_decode_step_dev_len", "nvfp4_decode_attn_partial",
              "nvfp4_decode_attn_combine", "nvfp4_hbm_read_probe", "nvfp4_last_error"):
        assert f in names


def test_binding_symbol_list_matches_header():
    import quantized_kv_decode_amd as qk
    assert sorted(qk.SYMBOLS) == declared_functions()


def test_read_probe_validation_codes(lib):
    import quantized_kv_decode_amd as qk
    a, sink = 0x100000, 0x200000
    assert lib.nvfp4_hbm_read_probe(0, 1024, sink, 4, None) == qk.EINVAL
    assert lib.nvfp4_hbm_read_probe(a + 8, 1024, sink, 4, None) == qk.EINVAL
    assert lib.nvfp4_hbm_read_probe(a, 1000, sink, 4, None) == qk.EINVAL      # not a multiple of 16
    assert lib.nvfp4_hbm_read_probe(a, 0, sink, 4, None) == qk.EINVAL
    assert lib.nvfp4_hbm_read_probe(a, 1024, 0, 4, None) == qk.EINVAL
    assert lib.nvfp4_hbm_read_probe(a, 1024, sink + 2, 4, None) == qk.EINVAL
    assert lib.nvfp4_hbm_read_probe(a, 1024, sink, 0, None) == qk.EINVAL
    assert lib.nvfp4_hbm_read_probe(a, 1024, sink, 65537, None) == qk.EINVAL


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names
    for f in names:
        assert hasattr(lib, f), f


class _FakeTensor:
    """Stands in for a device tensor: only an aligned address is needed for validation."""
    def __init__(self, addr, n=0):
        self._a, self._n = addr, n

    def data_ptr(self):
        return self._a

    def numel(self):
        return self._n


def _desc(qk, H=4, D=256, cap=1000, addr=0x100000):
    return qk.CacheDesc(addr, addr + 0x10000, addr + 0x20000, addr + 0x30000, H, D, cap)


def _call_decode(qk, lib, d, B=1, lens=(100,), base=(0,), n_q=1, Hq=24, ws=1 << 30, out_dtype=0, q=0x200000,
                 out=0x300000, g=0x400000, wsp=0x500000, sm=0.0625):
    return lib.nvfp4_decode_attn(ctypes.byref(d) if d is not None else None, g, q, out, out_dtype, B, qk._i64(base),
                                 qk._i64(lens), n_q, Hq, sm, wsp, ws, None)


def test_decode_validation_codes(lib):
    import quantized_kv_decode_amd as qk
    d = _desc(qk)
    assert _call_decode(qk, lib, None) == qk.EINVAL
    assert "null" in lib.nvfp4_last_error().decode()
    assert _call_decode(qk, lib, _desc(qk, D=64)) == qk.EUNSUPPORTED
    # one head's code plane must stay below 2^31 bytes (32-bit kernel offsets)
    assert _call_decode(qk, lib, _desc(qk, cap=(2 ** 31 - 1) // 128 + 1)) == qk.EUNSUPPORTED
    assert "capacity" in lib.nvfp4_last_error().decode()
    assert _call_decode(qk, lib, _desc(qk, D=128, cap=(2 ** 31 - 1) // 64 + 1)) == qk.EUNSUPPORTED
    assert _call_decode(qk, lib, _desc(qk, H=0)) == qk.EINVAL
    assert _call_decode(qk, lib, _desc(qk, addr=0x100008)) == qk.EINVAL          # unaligned plane
    assert _call_decode(qk, lib, d, Hq=25) == qk.EUNSUPPORTED                      # Hq % Hkv
    assert _call_decode(qk, lib, d, n_q=1400) == qk.EUNSUPPORTED                   # 6 x 1400 rows > 8192
    assert _call_decode(qk, lib, d, n_q=0) == qk.EINVAL
    assert _call_decode(qk, lib, d, B=0) == qk.EINVAL
    assert _call_decode(qk, lib, d, B=9, lens=[10] * 9, base=[0] * 9) == qk.EUNSUPPORTED
    assert _call_decode(qk, lib, d, lens=(0,)) == qk.ERANGE                        # shorter than n_q
    assert _call_decode(qk, lib, d, lens=(1001,)) == qk.ERANGE                     # past capacity
    assert _call_decode(qk, lib, d, base=(950,)) == qk.ERANGE                      # slots past capacity
    assert _call_decode(qk, lib, d, ws=16) == qk.EWORKSPACE
    assert _call_decode(qk, lib, d, out_dtype=7) == qk.EINVAL
    assert _call_decode(qk, lib, d, q=0) == qk.EINVAL
    assert _call_decode(qk, lib, d, q=0x200004) == qk.EINVAL
    assert _call_decode(qk, lib, d, g=0) == qk.EINVAL
    assert _call_decode(qk, lib, d, sm=float("nan")) == qk.EINVAL


def test_append_and_calibrate_validation_codes(lib):
    import quantized_kv_decode_amd as qk
    d = _desc(qk)
    i64 = qk._i64
    a = 0x600000
    # empty append is a no-op success, with or without row pointers
    assert lib.nvfp4_kv_append(ctypes.byref(d), None, None, a, 1, i64([0]), i64([0]), i64([0]), None) == qk.OK
    assert lib.nvfp4_kv_append(ctypes.byref(d), a, a, a, 1, i64([0]), i64([990]), i64([11]), None) == qk.ERANGE
    assert lib.nvfp4_kv_append(ctypes.byref(d), a, a, a, 1, i64([0]), i64([-1]), i64([1]), None) == qk.ERANGE
    assert lib.nvfp4_kv_append(ctypes.byref(d), a, a, a, 1, i64([0]), i64([0]), i64([-1]), None) == qk.EINVAL
    assert lib.nvfp4_kv_append(ctypes.byref(d), a, a, 0, 1, i64([0]), i64([0]), i64([1]), None) == qk.EINVAL
    assert lib.nvfp4_kv_append(ctypes.byref(d), a + 2, a, a, 1, i64([0]), i64([0]), i64([1]), None) == qk.EINVAL
    assert lib.nvfp4_kv_append(ctypes.byref(d), a, a, a, 9, i64([0] * 9), i64([0] * 9), i64([1] * 9),
                               None) == qk.EUNSUPPORTED
    assert lib.nvfp4_kv_append(ctypes.byref(_desc(qk, D=192)), a, a, a, 1, i64([0]), i64([0]), i64([1]),
                               None) == qk.EUNSUPPORTED
    assert lib.nvfp4_kv_calibrate(ctypes.byref(d), a, a, 1, i64([-1]), a, None) == qk.EINVAL
    assert lib.nvfp4_kv_calibrate(ctypes.byref(d), a, a, 0, i64([1]), a, None) == qk.EINVAL
    assert lib.nvfp4_kv_calibrate(ctypes.byref(d), a, a, 1, i64([1]), 0, None) == qk.EINVAL
    assert lib.nvfp4_kv_calibrate(ctypes.byref(d), 0, a, 1, i64([1]), a, None) == qk.EINVAL


def test_workspace_query(lib):
    import quantized_kv_decode_amd as qk
    d = _desc(qk, cap=10 ** 6)
    ws = lambda lens, n_q=1, Hq=24: lib.nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), len(lens), qk._i64(lens),
                                                                          n_q, Hq)
    assert ws([0]) == 0                                  # invalid arguments -> 0
    assert ws([100], Hq=25) == 0
    small, big = ws([100]), ws([400000])
    assert 0 < small <= big
    # one split per (sequence, head) at minimum: R x (D + 2) floats each
    assert small >= 4 * 6 * (256 + 2) * 4
    # a long sequence is cut into at most two workgroups per CU for one row tile
    assert big <= 2 * 256 * 6 * (256 + 2) * 4 + 3 * 256


def test_decode_step_validation_codes(lib):
    import quantized_kv_decode_amd as qk
    d = _desc(qk)
    a = 0x600000

    def call(k=a, v=a, q=0x200000, out=0x300000, lens=(100,), base=(0,), n_q=1, ws=1 << 30):
        return lib.nvfp4_decode_step(ctypes.byref(d), 0x400000, k, v, q, out, 0, 1, qk._i64(base), qk._i64(lens),
                                     n_q, 24, 0.0625, 0x500000, ws, None)
    assert call(k=0) == qk.EINVAL
    assert call(v=a + 8) == qk.EINVAL
    assert call(q=0) == qk.EINVAL
    assert call(lens=(0,)) == qk.ERANGE
    assert call(base=(950,)) == qk.ERANGE
    assert call(ws=16) == qk.EWORKSPACE


def test_decode_step_dev_len_validation_codes(lib):
    import quantized_kv_decode_amd as qk
    d = _desc(qk)
    a = 0x600000

    def call(k=a, v=a, q=0x200000, out=0x300000, max_len=(100,), base=(0,), lens_dev=0x700000, n_q=1,
             ws=1 << 30):
        return lib.nvfp4_decode_step_dev_len(ctypes.byref(d), 0x400000, k, v, q, out, 0, 1, qk._i64(base),
                                             qk._i64(max_len), lens_dev, n_q, 24, 0.0625, 0x500000, ws, None)
    assert call(lens_dev=0) == qk.EINVAL                  # device lengths required
    assert call(lens_dev=0x700004) == qk.EINVAL           # 8-byte alignment
    assert call(k=0) == qk.EINVAL                         # only one of k_new / v_new
    assert call(q=0) == qk.EINVAL
    assert call(max_len=(0,)) == qk.ERANGE                # the bound must hold n_q tokens
    assert call(base=(950,)) == qk.ERANGE                 # bound past capacity
    assert call(ws=16) == qk.EWORKSPACE
    assert lib.nvfp4_decode_step_dev_len(ctypes.byref(d), 0x400000, a, a, 0x200000, 0x300000, 0, 1, qk._i64([0]),
                                         None, 0x700000, 1, 24, 0.0625, 0x500000, 1 << 30, None) == qk.EINVAL
    # above 128 rows per KV head the device-length step does not store rows itself
    assert call(max_len=(800,), n_q=30) == qk.EUNSUPPORTED


def test_wide_row_counts_plan_like_their_chunks(lib):
    """65..128 rows per KV head run as 32-row chunks side by side (grid y) over one split
    plan: 96 rows (n_q = 16, G = 6) and 72 rows (32 + 32 + 8) are three chunks, so of the
    256 workgroup slots (one 8-wave workgroup per CU at two row tiles) each chunk gets
    256 // 3 = 85, i.e. 21 splits of the sequence for each of the 4 KV heads; the workspace
    holds every row of every unit."""
    import quantized_kv_decode_amd as qk
    d = _desc(qk, cap=10 ** 6)
    al = lambda x: (x + 255) // 256 * 256
    ws = lambda L, n_q: lib.nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), 1, qk._i64([L]), n_q, 24)
    units = 4 * ((256 // 3) // 4)
    assert units == 84
    for n_q in (16, 12):
        R = 6 * n_q
        assert ws(400000, n_q) == al(units * R * 256 * 4) + 2 * al(units * R * 4)


def test_prefill_rows_plan_fewer_units(lib):
    """Row chunks run side by side (grid y), so the planner makes proportionally fewer
    units: 1024 query tokens at G = 6 are 6144 rows = 192 chunks of 32, and 256 / 192 = 1
    unit slot falls below one unit per (sequence, KV head): 4 units."""
    import quantized_kv_decode_amd as qk
    d = _desc(qk, cap=10 ** 6)
    al = lambda x: (x + 255) // 256 * 256
    R = 6 * 1024
    got = lib.nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), 1, qk._i64([30000]), 1024, 24)
    assert got == al(4 * R * 256 * 4) + 2 * al(4 * R * 4)
    # past the 32768-token unit cap each head's sequence takes two units
    got = lib.nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), 1, qk._i64([40000]), 1024, 24)
    assert got == al(8 * R * 256 * 4) + 2 * al(8 * R * 4)


def test_split_plan_last_unit_holds_new_rows(lib):
    """A decode step appends its n_q rows in the workgroup of the sequence's last unit, so
    a remainder shorter than n_q joins the unit before it. L = 4003 at 4 KV heads is cut
    into units of 160 tokens (31 wanted, at least 128 tokens each): 25 full units and a
    3-token remainder. The workspace size (units x R x (D + 2) floats, parts 256-byte
    aligned) shows the unit count."""
    import quantized_kv_decode_amd as qk
    d = _desc(qk, cap=10 ** 6)
    al = lambda x: (x + 255) // 256 * 256

    def expected(units, R, D=256):
        return al(units * R * D * 4) + 2 * al(units * R * 4)
    ws = lambda L, n_q: lib.nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), 1, qk._i64([L]), n_q, 24)
    assert ws(4003, 3) == expected(26 * 4, 6 * 3)        # remainder 3 >= n_q: its own unit
    assert ws(4003, 4) == expected(25 * 4, 6 * 4)        # remainder 3 < n_q: merged
    assert ws(4003, 6) == expected(25 * 4, 6 * 6)


def test_split_plan_caps_unit_length(lib):
    """No unit is longer than 32768 tokens, even when that takes more units than the 256
    workgroup slots of a one-row-tile launch: with 8 sequences x 32 KV heads (one unit per
    (sequence, head) fills the slots) at 200000 tokens each, every (sequence, head) is cut
    into ceil(200000 / 32768) = 7 units of 28576 tokens (a multiple of 32)."""
    import quantized_kv_decode_amd as qk
    d = _desc(qk, H=32, D=128, cap=8 * 200000)
    al = lambda x: (x + 255) // 256 * 256
    lens = [200000] * 8
    got = lib.nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), 8, qk._i64(lens), 1, 32)
    units = 8 * 32 * 7
    assert got == al(units * 1 * 128 * 4) + 2 * al(units * 1 * 4)
    # at or below the cap nothing changes: one unit per (sequence, head)
    got = lib.nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), 8, qk._i64([32768] * 8), 1, 32)
    assert got == al(256 * 128 * 4) + 2 * al(256 * 4)


def test_kv_format_validation(lib):
    """kv_format must be NVFP4 (0) or K8V4 (1); a K8V4 pool's K code plane (head_dim bytes
    a row) must also stay below 2^31 bytes per head."""
    import quantized_kv_decode_amd as qk
    d = _desc(qk)
    d.kv_format = 2
    assert _call_decode(qk, lib, d) == qk.EINVAL
    assert "kv_format" in lib.nvfp4_last_error().decode()
    d = _desc(qk, cap=(2 ** 31 - 1) // 256 + 1)                 # fine for NVFP4 (128 B rows) ...
    d.kv_format = 1
    assert _call_decode(qk, lib, d) == qk.EUNSUPPORTED          # ... too large for FP8 K (256 B rows)
    d.kv_format = 0
    assert lib.nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), 1, qk._i64([100]), 1, 24) > 0
    d = _desc(qk)
    d.kv_format = 1
    assert lib.nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), 1, qk._i64([100]), 1, 24) > 0
