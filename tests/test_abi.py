"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ace_moe.h")


def _lib():
    import token_adaptive_expert_amd as m
    try:
        return m, m.load()
    except ImportError as e:
        pytest.fail(f"HIP library not built: {e}")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:ace_status|int|size_t|const char\*)\s+(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_calls():
    fns = header_functions()
    for f in ("moe_route_skip", "moe_dispatch", "moe_expert_forward", "moe_combine"):
        assert f in fns


def test_library_exports_every_declared_symbol():
    m, lib = _lib()
    for f in header_functions():
        assert hasattr(lib, f), f
    assert set(header_functions()) <= set(m._lib.EXPORTS)
    version = re.search(r"#define ACE_MOE_ABI_VERSION (\d+)", open(HEADER).read())
    assert m.moe_abi_version() == int(version.group(1)) == m._lib.ABI_VERSION


def test_desc_layout_matches_header():
    m, _ = _lib()
    # twelve 4-byte fields, no padding
    assert ctypes.sizeof(m.MoeDesc) == 48


@pytest.mark.parametrize("kw,status,needle", [
    (dict(k=0), 1, "k=0"),
    (dict(k=17, E=32), 2, "k=17"),
    (dict(k=9, E=8), 2, "k=9"),
    (dict(E=300), 2, "E=300"),
    (dict(H=200), 2, "H=200"),
    (dict(I=96), 2, "I=96"),
    (dict(T=-1), 1, "T=-1"),
    (dict(dtype=7), 1, "dtype=7"),
    (dict(fusion=9), 1, "fusion=9"),
    (dict(norm_topk=2), 1, "norm_topk=2"),
    (dict(weight_layout=3), 1, "weight_layout=3"),
    (dict(router_layout=2), 1, "router_layout=2"),
    (dict(router_layout=1, dtype=0), 2, "router_layout=PACKED"),
    (dict(expert_pool=-1), 1, "expert_pool=-1"),
    (dict(expert_pool=4, T=2049), 2, "expert_pool needs T*k <= 8192"),
])
def test_bad_descriptors_are_rejected_before_launch(kw, status, needle):
    m, lib = _lib()
    base = dict(T=8, H=256, E=16, I=128, k=4, dtype=1, norm_topk=1, fusion=0, rms_eps=1e-6, weight_layout=0,
                router_layout=0, expert_pool=0)
    base.update(kw)
    d = m.MoeDesc(**base)
    fake = 0x1000  # never dereferenced: validation fails first
    st = lib.moe_route_skip(ctypes.byref(d), fake, fake, fake, None, None, fake, fake, fake, 0.0, 0.0, fake, fake,
                            fake, fake, None)
    assert st == status
    assert needle in lib.moe_last_error().decode()
    assert lib.moe_workspace_bytes(ctypes.byref(d)) == 0


def test_null_pointers_named():
    m, lib = _lib()
    d = m.make_desc(8, 256, 16, 128, 4, "bf16")
    st = lib.moe_route_skip(ctypes.byref(d), None, 0x1000, 0x1000, None, None, 0x1000, 0x1000, 0x1000, 0.0, 0.0,
                            0x1000, 0x1000, 0x1000, 0x1000, None)
    assert st == 1 and "x is NULL" in lib.moe_last_error().decode()
    st = lib.moe_route_skip(ctypes.byref(d), 0x1000, 0x1000, 0x1000, None, None, None, 0x1000, 0x1000, 0.0, 0.0,
                            0x1000, 0x1000, 0x1000, 0x1000, None)
    assert st == 1 and "logits_out is NULL" in lib.moe_last_error().decode()
    st = lib.moe_route_skip(ctypes.byref(d), 0x1000, 0x1000, 0x1000, None, 0x2000, 0x2000, 0x1000, 0x1000, 0.0, 0.0,
                            0x1000, 0x1000, 0x1000, 0x1000, None)
    assert st == 1 and "alias" in lib.moe_last_error().decode()
    st = lib.moe_combine(ctypes.byref(d), 0x1000, None, None, 0x1000, None)
    assert st == 1 and "slot_out is NULL" in lib.moe_last_error().decode()
    st = lib.moe_route_skip(ctypes.byref(d), 0x1000, 0x1000, 0x1000, None, None, 0x1000, 0x1000, 0x1000, -1.0, 0.0,
                            0x1000, 0x1000, 0x1000, 0x1000, None)
    assert st == 1 and "thresholds" in lib.moe_last_error().decode()
    assert lib.moe_route_skip(None, *([0x1000] * 8), 0.0, 0.0, *([0x1000] * 4), None) == 1


def test_workspace_too_small():
    m, lib = _lib()
    d = m.make_desc(1024, 2048, 128, 768, 8, "bf16")
    need = lib.moe_workspace_bytes(ctypes.byref(d))
    assert need > 0
    st = lib.moe_dispatch(ctypes.byref(d), *([0x1000] * 7), 0x1000, need - 1, None)
    assert st == 3 and str(need) in lib.moe_last_error().decode()
    # more than 32768 slots: per-block counts and row bases, 8 bytes per expert per 4096 slots
    d = m.make_desc(8192, 4096, 128, 1408, 8, "bf16")
    need = lib.moe_workspace_bytes(ctypes.byref(d))
    assert need >= 8 * 128 * 16
    st = lib.moe_dispatch(ctypes.byref(d), *([0x1000] * 7), 0x1000, need - 1, None)
    assert st == 3 and str(need) in lib.moe_last_error().decode()


def test_empty_batch_is_a_no_op():
    m, lib = _lib()
    d = m.make_desc(0, 256, 16, 128, 4, "f32")
    f = 0x1000
    assert lib.moe_route_skip(ctypes.byref(d), f, f, f, None, None, f, f, f, 0.0, 0.0, f, f, f, f, None) == 0
    assert lib.moe_dispatch(ctypes.byref(d), f, f, f, f, f, f, f, f, 1 << 20, None) == 0
    assert lib.moe_expert_forward(ctypes.byref(d), 0, f, f, f, f, f, f, f, f, f, f, 1 << 20, None) == 0
    assert lib.moe_combine(ctypes.byref(d), f, f, None, f, None) == 0
    assert lib.moe_last_error().decode() == ""


def test_bad_path_and_events():
    m, lib = _lib()
    d = m.make_desc(4, 256, 16, 128, 4, "f32")
    f = 0x1000
    assert lib.moe_expert_forward(ctypes.byref(d), 5, f, f, f, f, f, f, f, f, f, f, 1 << 20, None) == 1
    assert lib.moe_expert_forward(ctypes.byref(d), 0, f, f, f, f, f, f, f, f, f, None, 1 << 20, None) == 1
    assert "workspace" in lib.moe_last_error().decode()
    assert lib.moe_expert_forward(ctypes.byref(d), 0, f, f, f, f, f, f, f, f, f, f, 16, None) == 3
    assert lib.moe_set_kernel_events(f, None) == 1
    assert lib.moe_set_kernel_events(None, None) == 0


def test_pack_rejects_overlap_and_bad_kind():
    m, lib = _lib()
    d = m.make_desc(8, 256, 16, 128, 4, "bf16")
    assert lib.moe_pack_weights(ctypes.byref(d), 2, 0x1000, 0x100000000, None) == 1
    assert lib.moe_pack_weights(ctypes.byref(d), 0, 0x1000, 0x1000 + 64, None) == 1
    assert "overlap" in lib.moe_last_error().decode()


def test_build_tables_validation():
    m, lib = _lib()
    f = 0x1000
    d = m.make_desc(1, 2048, 128, 768, 8, "bf16")
    pref = lib.moe_tables_workspace_bytes(ctypes.byref(d))
    # transposed w_down for every expert (3 MiB each) fits under the 512 MiB cap
    assert pref >= 128 * 768 * 2048 * 2
    args = [f] * 7
    assert lib.moe_build_tables(ctypes.byref(d), 1e-6, *args, None, 1 << 30, None) == 1
    assert "workspace is NULL" in lib.moe_last_error().decode()
    assert lib.moe_build_tables(ctypes.byref(d), 1e-6, None, *args[1:], f, 1 << 30, None) == 1
    assert "gamma is NULL" in lib.moe_last_error().decode()
    assert lib.moe_build_tables(ctypes.byref(d), -1.0, *args, f, 1 << 30, None) == 1
    # the minimum is one expert's transposed w_down plus the per-expert partials
    assert lib.moe_build_tables(ctypes.byref(d), 1e-6, *args, f, 768 * 2048 * 2, None) == 3
    assert "batches of one expert" in lib.moe_last_error().decode()
    dp = m.make_desc(1, 2048, 128, 768, 8, "bf16", weight_layout=1)
    assert lib.moe_build_tables(ctypes.byref(dp), 1e-6, *args, f, pref, None) == 2
    assert "LINEAR" in lib.moe_last_error().decode()
    big = m.make_desc(1, 4096, 128, 1408, 8, "bf16")
    assert lib.moe_tables_workspace_bytes(ctypes.byref(big)) < (512 + 64) << 20


def test_misaligned_pointers_rejected():
    m, lib = _lib()
    d = m.make_desc(8, 256, 16, 128, 4, "bf16")
    f = 0x1000
    st = lib.moe_route_skip(ctypes.byref(d), f + 4, f, f, None, None, f, f, f, 0.0, 0.0, f, f, f, f, None)
    assert st == 1 and "x is not 16-byte aligned" in lib.moe_last_error().decode()
    st = lib.moe_route_skip(ctypes.byref(d), f, f, f, f + 8, None, f, f, f, 0.0, 0.0, f, f, f, f, None)
    assert st == 1 and "router_bias is not 16-byte aligned" in lib.moe_last_error().decode()
    st = lib.moe_dispatch(ctypes.byref(d), f, f, f + 1, f, f, f, f, f, 1 << 20, None)
    assert st == 1 and "keep is not 16-byte aligned" in lib.moe_last_error().decode()
    st = lib.moe_combine(ctypes.byref(d), f, f, f + 2, f, None)
    assert st == 1 and "residual is not 16-byte aligned" in lib.moe_last_error().decode()


def test_forward_validates_before_launch():
    m, lib = _lib()
    d = m.make_desc(4, 256, 16, 128, 4, "bf16")
    f = 0x1000
    args = [f] * 6 + [f, f]  # x..a_rcr (logits_in NULL handled below)
    # y NULL
    st = lib.moe_forward(ctypes.byref(d), 0, f, f, f, None, None, f, f, f, 0.0, 0.0, f, f, f, None, f, f, f, f, f, f,
                         f, f, f, f, None, f, 1 << 20, None)
    assert st == 1 and "y is NULL" in lib.moe_last_error().decode()
    st = lib.moe_forward(ctypes.byref(d), 7, f, f, f, None, None, f, f, f, 0.0, 0.0, f, f, f, None, f, f, f, f, f, f,
                         f, f, f, f, f, f, 1 << 20, None)
    assert st == 1 and "path=7" in lib.moe_last_error().decode()
    st = lib.moe_forward(ctypes.byref(d), 0, f, f, f, None, None, f, f, f, 0.0, 0.0, f, f, f, None, f, f, f, f, f, f,
                         f, f, f, f, f, f, 16, None)
    assert st == 3
    d0 = m.make_desc(0, 256, 16, 128, 4, "bf16")
    assert lib.moe_forward(ctypes.byref(d0), 0, f, f, f, None, None, f, f, f, 0.0, 0.0, f, f, f, None, f, f, f, f, f,
                           f, f, f, f, f, f, f, 1 << 20, None) == 0


def test_forward_static_validates_and_bounds_its_scratch():
    """moe_forward_static checks every argument and its scratch bound on the
    host, before it looks up or touches the static device buffer."""
    m, lib = _lib()
    f = 0x1000
    d = m.make_desc(4, 256, 16, 128, 4, "bf16")
    st = lib.moe_forward_static(ctypes.byref(d), 0, f, f, f, None, None, f, f, f, 0.0, 0.0, f, f, f, None, f, f, f, f,
                                f, f, f, f, None, None)
    assert st == 1 and "y is NULL" in lib.moe_last_error().decode()
    st = lib.moe_forward_static(ctypes.byref(d), 9, f, f, f, None, None, f, f, f, 0.0, 0.0, f, f, f, None, f, f, f, f,
                                f, f, f, f, f, None)
    assert st == 1 and "path=9" in lib.moe_last_error().decode()
    # T = 1024 of the Qwen3-30B-A3B shape fits the 80 MiB buffer; T = 2048 does not
    d = m.make_desc(2048, 2048, 128, 768, 8, "bf16")
    st = lib.moe_forward_static(ctypes.byref(d), 0, f, f, f, None, None, f, f, f, 0.0, 0.0, f, f, f, None, f, f, f, f,
                                f, f, f, f, f, None)
    assert st == 2 and "static buffer" in lib.moe_last_error().decode()
    hdr = re.search(r"#define ACE_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m.ACE_STATIC_SCRATCH_BYTES == int(hdr.group(1)) << int(hdr.group(2)) == 80 << 20
    need_1024 = 8192 * 768 * 2 + 8192 * 2048 * 4 + 256
    assert need_1024 <= m.ACE_STATIC_SCRATCH_BYTES < 2 * 8192 * 2048 * 4
    d0 = m.make_desc(0, 256, 16, 128, 4, "bf16")
    assert lib.moe_forward_static(ctypes.byref(d0), 0, f, f, f, None, None, f, f, f, 0.0, 0.0, f, f, f, None, f, f, f,
                                  f, f, f, f, f, f, None) == 0


def test_probe_arguments_validated_before_launch():
    m, lib = _lib()
    f = 0x1000
    mib2 = 2 << 20
    # moe_l2_load_probe(buf, bytes, rounds, loads, mfma_per_load, stride_mode, sink, workgroups, stream)
    for args, needle in (((f, 3 << 20, 8, 6, 0, 0, f, 8, None), "bytes="),
                         ((f, 1 << 20, 8, 6, 0, 0, f, 8, None), "bytes="),
                         ((f, mib2, 8, 7, 0, 0, f, 8, None), "loads=7"),
                         ((f, mib2, 8, 6, 2, 0, f, 8, None), "mfma_per_load=2"),
                         ((f, mib2, 8, 6, 4, 2, f, 8, None), "stride_mode=2"),
                         ((f, mib2, 0, 6, 4, 0, f, 8, None), "rounds=0"),
                         ((f, mib2, 8, 6, 4, 0, f, 0, None), "workgroups=0"),
                         ((None, mib2, 8, 6, 4, 0, f, 8, None), "buf is NULL"),
                         ((f, mib2, 8, 6, 4, 0, None, 8, None), "sink is NULL")):
        assert lib.moe_l2_load_probe(*args) == 1, args
        assert needle in lib.moe_last_error().decode(), (needle, lib.moe_last_error())
    assert lib.moe_hbm_read_probe(f, 24, f, 4, None) == 1
    assert lib.moe_hbm_read_probe(f, 32, f, 0, None) == 1
