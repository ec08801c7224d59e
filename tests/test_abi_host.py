"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything.

No call here reaches a kernel launch (validation fails first), so these run
without a GPU.  Device pointers are fake addresses: validation never
dereferences them.
"""
import ctypes
import os
import re

import pytest

from rank_gradient_sketching_logra_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "logra.h")


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LOGRA_API\s+[\w\s\*]+?\b(logra_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        import rank_gradient_sketching_logra_amd.build as build
        build.build(verbose=False)
    return B.lib()


def test_exports_every_declared_symbol(lib):
    syms = header_symbols()
    assert len(syms) >= 15
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(B.SIGNATURES), "binding and header disagree"


def test_version_and_sizes(lib):
    assert "gfx950" in B.version()
    assert B.sketch_bytes(4096, 64) == 1 << 20          # 1 MiB, paper §2.2
    assert lib.logra_sketch_bytes(-1, 3) == -1
    # packed XAt (hi, lo bf16: 4 bytes per padded token x rank) + fp32 partials
    # (512-column groups x padded ranks x 1024-token groups)
    assert B.accumulate_ws_bytes(4096, 3584, 64) == 64 * 4096 * 4
    assert B.accumulate_ws_bytes(1000, 300, 33) == 64 * 1008 * 4
    assert B.accumulate_ws_bytes(4096, 100, 100) == 128 * 4096 * 4
    # ranks pad to 1, 2, 4 or 8 blocks of 32: r = 160 and 192 take 256
    assert B.accumulate_ws_bytes(4096, 100, 160) == 256 * 4096 * 4
    assert B.accumulate_ws_bytes(16, 100, 192) == 256 * 16 * 4
    assert B.accumulate_ws_bytes(16, 100, 32) == 32 * 16 * 4
    assert B.accumulate_ws_bytes(0, 8, 8) == 0
    assert B.accumulate_ws_bytes(8, 0, 8) == 0
    assert B.rowadam_ws_bytes(0) == 0
    assert B.predicted_kl_q_ws_bytes(64, 152064) > 0


def test_step_alpha_host(lib):
    assert B.step_alpha(8e-3, 2e-3, 4.0) == pytest.approx(0.5, rel=1e-15)
    assert B.step_alpha(0.0, 2e-3, 4.0) == 4.0
    assert B.step_alpha(1e-9, 2e-3, 4.0) == 4.0
    for q, dl, am in ((-1.0, 1e-3, 1.0), (float("nan"), 1e-3, 1.0), (1.0, 0.0, 1.0), (1.0, 1e-3, -1.0)):
        with pytest.raises(B.LograError) as e:
            B.step_alpha(q, dl, am)
        assert e.value.status == B.ERR_DOMAIN


A = 0x10000          # fake, 16-byte aligned device addresses
Bp = 0x4000000
C = 0x8000000
Dp = 0xC000000


PIN = 128 * 64 * 4        # packed projected input of T = 128 tokens at r = 64
PUP = 64 * 64 * 4         # packed update of d = 64 rows at r = 64 (or fewer ranks)


def key():
    return B.Key(1, 0, 0)


def err(fn, *args):
    st = fn(*args)
    assert st != B.OK
    return st


def test_regen_validation(lib):
    assert err(lib.logra_regen_A, None, 8, 16, B.I8, A, None) == B.ERR_NULL
    assert err(lib.logra_regen_A, ctypes.byref(key()), 0, 16, B.I8, A, None) == B.ERR_SHAPE
    assert err(lib.logra_regen_A, ctypes.byref(key()), 257, 16, B.I8, A, None) == B.ERR_SHAPE
    assert err(lib.logra_regen_A, ctypes.byref(key()), 8, 16, B.BF16, A, None) == B.ERR_DTYPE
    assert "regen_A" in lib.logra_last_error().decode()


def test_project_validation(lib):
    k = ctypes.byref(key())
    f = lib.logra_project_input
    assert err(f, k, 16, 64, 8, None, B.BF16, 64, Bp, None) == B.ERR_NULL
    assert err(f, k, 0, 64, 8, A, B.BF16, 64, Bp, None) == B.ERR_SHAPE
    assert err(f, k, 16, 64, 8, A, B.BF16, 32, Bp, None) == B.ERR_SHAPE        # ldx < k
    assert err(f, k, 16, 64, 8, A, B.I8, 64, Bp, None) == B.ERR_DTYPE
    assert err(f, k, 16, 64, 8, A + 2, B.BF16, 64, Bp, None) == B.ERR_ALIGN
    assert err(f, k, 16, 60, 8, A, B.BF16, 60, Bp, None) == B.ERR_ALIGN      # 120-byte rows
    assert err(f, k, 16, 64, 8, A, B.BF16, 64, A + 64, None) == B.ERR_ALIAS


def test_accumulate_validation(lib):
    f = lib.logra_sketch_accumulate
    ws = B.accumulate_ws_bytes(128, 64, 64)
    assert err(f, 128, 64, 64, None, B.BF16, 64, Bp, C, Dp, ws, None) == B.ERR_NULL
    assert err(f, 128, 64, 300, A, B.BF16, 64, Bp, C, Dp, ws, None) == B.ERR_SHAPE
    assert err(f, 0, 64, 64, A, B.BF16, 64, Bp, C, Dp, ws, None) == B.ERR_SHAPE
    assert err(f, 128, 64, 64, A, B.BF16, 64, Bp, C, None, 0, None) == B.ERR_WORKSPACE
    assert err(f, 128, 64, 64, A, B.BF16, 64, Bp, C, Dp, ws - 1, None) == B.ERR_WORKSPACE
    assert err(f, 128, 64, 64, A, B.BF16, 64, Bp, A + 128, Dp, ws, None) == B.ERR_ALIAS   # S in D
    assert err(f, 128, 64, 64, A, B.BF16, 64, Bp, C, C + 256, ws, None) == B.ERR_ALIAS    # ws in S
    assert err(f, 128, 64, 64, A, B.BF16, 64, Bp + 4, C, Dp, ws, None) == B.ERR_ALIGN


def test_grouped_validation(lib):
    f = lib.logra_sketch_accumulate_grouped
    ws = 2 * B.accumulate_ws_bytes(128, 64, 64)
    descs = (B.AccDesc * 2)(B.AccDesc(A, Bp, C, 64, 64), B.AccDesc(A + 65536, Bp + 65536, C + 64, 64, 64))
    assert err(f, 128, 64, B.BF16, descs, 2, Dp, ws, None) == B.ERR_ALIAS     # sketches overlap
    assert err(f, 128, 64, B.BF16, descs, 0, Dp, ws, None) == B.ERR_SHAPE
    assert err(f, 128, 64, B.BF16, descs, 17, Dp, ws, None) == B.ERR_SHAPE
    assert err(f, 128, 64, B.BF16, descs, 2, Dp, ws // 2, None) == B.ERR_WORKSPACE
    assert err(f, 128, 64, B.BF16, None, 2, Dp, ws, None) == B.ERR_NULL


def test_packed_sizes_and_validation(lib):
    assert B.packed_input_bytes(4096, 64) == 64 * 4096 * 4
    assert B.packed_input_bytes(1000, 33) == 64 * 1008 * 4
    assert B.packed_input_bytes(4096, 256) == 256 * 4096 * 4
    assert B.packed_input_bytes(0, 64) == 0 and B.packed_input_bytes(16, 0) == 0
    k = ctypes.byref(key())
    f = lib.logra_project_input_packed
    nb = B.packed_input_bytes(16, 8)
    assert err(f, k, 16, 64, 8, A, B.BF16, 64, None, None, nb, None) == B.ERR_NULL
    assert err(f, k, 16, 64, 8, A, B.F32, 64, None, Bp, nb, None) == B.ERR_DTYPE
    assert err(f, k, 16, 64, 8, A, B.BF16, 64, None, Bp, nb - 1, None) == B.ERR_WORKSPACE
    assert err(f, k, 16, 64, 8, A, B.BF16, 64, None, Bp + 8, nb, None) == B.ERR_ALIGN
    assert err(f, k, 16, 64, 8, A, B.BF16, 64, None, A + 256, nb, None) == B.ERR_ALIAS     # planes in X
    assert err(f, k, 16, 64, 8, A, B.BF16, 64, Bp + 16, Bp, nb, None) == B.ERR_ALIAS       # XAt in planes
    g = lib.logra_sketch_accumulate_grouped_packed
    d2 = (B.AccPackedDesc * 2)(B.AccPackedDesc(A, Bp, C, 64, 64, PIN), B.AccPackedDesc(A + 65536, Bp, C + 64, 64, 64, PIN))
    assert err(g, 128, 64, d2, 2, None) == B.ERR_ALIAS                                     # sketches overlap
    assert err(g, 128, 64, d2, 0, None) == B.ERR_SHAPE
    assert err(g, 128, 300, d2, 1, None) == B.ERR_SHAPE
    assert err(g, 128, 64, None, 1, None) == B.ERR_NULL
    d1 = (B.AccPackedDesc * 1)(B.AccPackedDesc(A, Bp, Bp + 64, 64, 64, PIN))
    assert err(g, 128, 64, d1, 1, None) == B.ERR_ALIAS                                     # S in planes
    d1 = (B.AccPackedDesc * 1)(B.AccPackedDesc(A, Bp + 4, C, 64, 64, PIN))
    assert err(g, 128, 64, d1, 1, None) == B.ERR_ALIGN


def test_merge_grouped_validation(lib):
    f = lib.logra_merge_grouped
    d2 = (B.MergeDesc * 2)(B.MergeDesc(key(), A, 64, 64, 64, Bp, 0), B.MergeDesc(key(), A + 4096, 64, 64, 64, C, 0))
    assert err(f, 64, d2, 2, 1.0, None, 0, 0, None) == B.ERR_ALIAS        # W overlap
    assert err(f, 64, d2, 0, 1.0, None, 0, 0, None) == B.ERR_SHAPE
    assert err(f, 64, d2, 17, 1.0, None, 0, 0, None) == B.ERR_SHAPE
    assert err(f, 300, d2, 1, 1.0, None, 0, 0, None) == B.ERR_SHAPE
    assert err(f, 64, d2, 1, float("inf"), None, 0, 0, None) == B.ERR_DOMAIN
    assert err(f, 64, d2, 1, 1.0, None, 5, 0, None) == B.ERR_DOMAIN
    assert err(f, 64, None, 1, 1.0, None, 0, 0, None) == B.ERR_NULL
    d1 = (B.MergeDesc * 1)(B.MergeDesc(key(), A, 64, 64, 64, A + 512, 0))
    assert err(f, 64, d1, 1, 1.0, None, 0, 0, None) == B.ERR_ALIAS        # U inside W
    d1 = (B.MergeDesc * 1)(B.MergeDesc(key(), A, 64, 64, 64, Bp + 8, 0))
    assert err(f, 64, d1, 1, 1.0, None, 0, 0, None) == B.ERR_ALIGN
    d2 = (B.MergeDesc * 2)(B.MergeDesc(key(), A, 64, 64, 64, Bp, 0), B.MergeDesc(key(), C, 64, 64, 64, A + 256, 0))
    assert err(f, 64, d2, 2, 1.0, None, 0, 0, None) == B.ERR_ALIAS        # U of 1 inside W of 0


def test_rowadam_validation(lib):
    f = lib.logra_rowadam
    ws = B.rowadam_ws_bytes(64)
    assert err(f, 64, 8, None, Bp, 1, 0.95, 1e-8, C, Dp, ws, None) == B.ERR_NULL
    assert err(f, 64, 8, A, Bp, 0, 0.95, 1e-8, C, Dp, ws, None) == B.ERR_DOMAIN       # t < 1
    assert err(f, 64, 8, A, Bp, 1, 1.0, 1e-8, C, Dp, ws, None) == B.ERR_DOMAIN        # beta
    assert err(f, 64, 8, A, Bp, 1, 0.95, -1.0, C, Dp, ws, None) == B.ERR_DOMAIN       # eps
    assert err(f, 64, 8, A, Bp, 1, 0.95, 1e-8, C, Dp, ws - 8, None) == B.ERR_WORKSPACE
    assert err(f, 64, 8, A, Bp, 1, 0.95, 1e-8, A + 16, Dp, ws, None) == B.ERR_ALIAS    # partial overlap
    assert err(f, 64, 8, A, A + 64, 1, 0.95, 1e-8, C, Dp, ws, None) == B.ERR_ALIAS     # v inside S


def test_rowadam_grouped_validation(lib):
    f = lib.logra_rowadam_packed_grouped
    r = 64
    pb = B.packed_update_bytes(64, r)
    E = 0x10000000

    def descs(*rows):
        arr = (B.RowAdamDesc * len(rows))()
        for i, row in enumerate(rows):
            arr[i] = B.RowAdamDesc(*row)
        return arr

    good = [(A, Bp, C, pb, 64), (A + 64 * r * 4, Bp + 256, C + pb, pb, 64)]
    ws = B.rowadam_grouped_ws_bytes(2, 128)
    assert ws > 0 and B.rowadam_grouped_ws_bytes(0, 10) == 0 and B.rowadam_grouped_ws_bytes(3, 2) == 0
    assert err(f, r, None, 2, 1, 0.95, 1e-8, E, ws, None) == B.ERR_NULL
    assert err(f, r, descs(*good), 0, 1, 0.95, 1e-8, E, ws, None) == B.ERR_SHAPE
    assert err(f, 300, descs(*good), 2, 1, 0.95, 1e-8, E, ws, None) == B.ERR_SHAPE      # r above the maximum
    assert err(f, r, descs(*good), 2, 0, 0.95, 1e-8, E, ws, None) == B.ERR_DOMAIN       # t < 1
    assert err(f, r, descs(*good), 2, 1, 1.0, 1e-8, E, ws, None) == B.ERR_DOMAIN        # beta
    assert err(f, r, descs(*good), 2, 1, 0.95, 1e-8, E, ws - 8, None) == B.ERR_WORKSPACE
    assert err(f, r, descs(good[0], (A, Bp + 256, C + pb, pb - 16, 64)), 2, 1, 0.95, 1e-8, E, ws,
               None) == B.ERR_WORKSPACE                                                  # packed bytes
    assert err(f, r, descs(good[0], (A, Bp + 8, C + pb, pb, 64)), 2, 1, 0.95, 1e-8, E, ws,
               None) == B.ERR_ALIGN
    assert err(f, r, descs(good[0], (A, Bp + 128, C + pb, pb, 64)), 2, 1, 0.95, 1e-8, E, ws,
               None) == B.ERR_ALIAS                                                      # two v overlap
    assert err(f, r, descs(good[0], (A + 64 * r * 4, Bp + 256, A + 1024, pb, 64)), 2, 1, 0.95, 1e-8,
               E, ws, None) == B.ERR_ALIAS                                               # output in a sketch
    assert err(f, r, descs(*good), 2, 1, 0.95, 1e-8, C + 64, ws, None) == B.ERR_ALIAS    # workspace


def test_predicted_kl_validation(lib):
    f = lib.logra_predicted_kl_q
    ws = B.predicted_kl_q_ws_bytes(4, 512)
    assert err(f, 4, 512, None, Bp, B.BF16, 1.0, C, Dp, ws, None) == B.ERR_NULL
    assert err(f, 0, 512, A, Bp, B.BF16, 1.0, C, Dp, ws, None) == B.ERR_SHAPE
    assert err(f, 4, 512, A, Bp, B.I8, 1.0, C, Dp, ws, None) == B.ERR_DTYPE
    assert err(f, 4, 512, A, Bp, B.BF16, 0.0, C, Dp, ws, None) == B.ERR_DOMAIN
    assert err(f, 4, 512, A, Bp, B.BF16, float("inf"), C, Dp, ws, None) == B.ERR_DOMAIN
    assert err(f, 4, 512, A, Bp, B.BF16, 1.0, C, Dp, 0, None) == B.ERR_WORKSPACE
    assert err(lib.logra_step_alpha_dev, None, 1e-3, 4.0, C, None) == B.ERR_NULL
    assert err(lib.logra_step_alpha_dev, A, 0.0, 4.0, C, None) == B.ERR_DOMAIN


def test_merge_validation(lib):
    f = lib.logra_merge
    k = ctypes.byref(key())
    assert err(f, None, 64, 64, 8, A, B.BF16, 64, Bp, 1.0, None, 0, 0, 0, None) == B.ERR_NULL
    assert err(f, k, 64, 64, 8, A, B.BF16, 64, Bp, 1.0, None, 0, 0, -1, None) == B.ERR_SHAPE
    assert err(f, k, 64, 64, 0, A, B.BF16, 64, Bp, 1.0, None, 0, 0, 0, None) == B.ERR_SHAPE
    assert err(f, k, 64, 64, 8, A, B.F32, 64, Bp, 1.0, None, 1, 0, 0, None) == B.ERR_DTYPE   # SR on fp32
    assert err(f, k, 64, 64, 8, A, B.BF16, 64, Bp, float("nan"), None, 0, 0, 0, None) == B.ERR_DOMAIN
    assert err(f, k, 64, 64, 8, A, B.BF16, 64, Bp, 1.0, None, 7, 0, 0, None) == B.ERR_DOMAIN
    assert err(f, k, 64, 64, 8, A, B.BF16, 64, A + 1024, 1.0, None, 0, 0, 0, None) == B.ERR_ALIAS
    assert err(f, k, 64, 64, 8, A, B.BF16, 64, Bp + 8, 1.0, None, 0, 0, 0, None) == B.ERR_ALIGN


def test_packed_update_sizes_and_validation(lib):
    # rows padded to 32, ranks to 16-rank steps padded to 1, 2, 4, 8 or 16; 4 bytes per element
    assert B.packed_update_bytes(4096, 64) == 4096 * 64 * 4
    assert B.packed_update_bytes(100, 33) == 128 * 64 * 4
    assert B.packed_update_bytes(1, 1) == 32 * 16 * 4
    assert B.packed_update_bytes(17408, 160) == 17408 * 256 * 4
    assert B.packed_update_bytes(0, 8) == 0 and B.packed_update_bytes(8, 257) == 0
    nb = B.packed_update_bytes(64, 8)
    f = lib.logra_pack_update
    assert err(f, 64, 8, None, Bp, nb, None) == B.ERR_NULL
    assert err(f, 64, 300, A, Bp, nb, None) == B.ERR_SHAPE
    assert err(f, 64, 8, A, Bp, nb - 1, None) == B.ERR_WORKSPACE
    assert err(f, 64, 8, A, Bp + 8, nb, None) == B.ERR_ALIGN
    assert err(f, 64, 8, A, A + 256, nb, None) == B.ERR_ALIAS            # packed inside U
    g = lib.logra_rowadam_packed
    ws = B.rowadam_ws_bytes(64)
    assert err(g, 64, 8, A, Bp, 1, 0.95, 1e-8, None, nb, Dp, ws, None) == B.ERR_NULL
    assert err(g, 64, 8, A, Bp, 1, 0.95, 1e-8, C, nb - 16, Dp, ws, None) == B.ERR_WORKSPACE
    assert err(g, 64, 8, A, Bp, 1, 0.95, 1e-8, A + 64, nb, Dp, ws, None) == B.ERR_ALIAS    # packed in S
    assert err(g, 64, 300, A, Bp, 1, 0.95, 1e-8, C, nb, Dp, ws, None) == B.ERR_SHAPE
    m = lib.logra_merge_grouped_packed
    d2 = (B.MergePackedDesc * 2)(B.MergePackedDesc(key(), A, 64, 64, 64, Bp, 0, PUP),
                                 B.MergePackedDesc(key(), A + 4096, 64, 64, 64, C, 0, PUP))
    assert err(m, 64, d2, 2, 1.0, None, 0, 0, None) == B.ERR_ALIAS        # W overlap
    assert err(m, 64, None, 1, 1.0, None, 0, 0, None) == B.ERR_NULL
    assert err(m, 300, d2, 1, 1.0, None, 0, 0, None) == B.ERR_SHAPE
    d1 = (B.MergePackedDesc * 1)(B.MergePackedDesc(key(), A, 64, 64, 64, A + 512, 0, PUP))
    assert err(m, 64, d1, 1, 1.0, None, 0, 0, None) == B.ERR_ALIAS        # packed U inside W
    d1 = (B.MergePackedDesc * 1)(B.MergePackedDesc(key(), Bp, 64, 64, 64, Bp - 16, 0, PUP))
    assert err(m, 64, d1, 1, 1.0, None, 0, 0, None) == B.ERR_ALIAS        # packed U runs into W
    d1 = (B.MergePackedDesc * 1)(B.MergePackedDesc(key(), A, 64, 64, 64, Bp + 8, 0, PUP))
    assert err(m, 64, d1, 1, 1.0, None, 0, 0, None) == B.ERR_ALIGN


def test_reconstruction_cosine_sizes_and_validation(lib):
    assert B.reconstruction_cosine_ws_bytes(1000, 1536, 64) >= 1000 * 64 * 4 + 64 * 64 * 8
    assert B.reconstruction_cosine_ws_bytes(0, 8, 8) == 0 and B.reconstruction_cosine_ws_bytes(8, 8, 300) == 0
    f = lib.logra_reconstruction_cosine
    k = ctypes.byref(key())
    ws = B.reconstruction_cosine_ws_bytes(64, 64, 8)
    assert err(f, k, 64, 64, 8, None, B.BF16, 64, C, Dp, ws, None) == B.ERR_NULL
    assert err(f, k, 64, 64, 300, A, B.BF16, 64, C, Dp, ws, None) == B.ERR_SHAPE
    assert err(f, k, 64, 64, 8, A, 7, 64, C, Dp, ws, None) == B.ERR_DTYPE
    assert err(f, k, 64, 64, 8, A, B.BF16, 60, C, Dp, ws, None) == B.ERR_SHAPE        # ldg < k
    assert err(f, k, 64, 64, 8, A, B.BF16, 64, C, Dp, ws - 8, None) == B.ERR_WORKSPACE
    assert err(f, k, 64, 64, 8, A, B.BF16, 64, C + 4, Dp, ws, None) == B.ERR_ALIGN     # output
    assert err(f, k, 64, 64, 8, A, B.BF16, 64, C, A + 512, ws, None) == B.ERR_ALIAS    # workspace in G


def test_sync_payload_validation(lib):
    f = lib.logra_sync_pack
    k = ctypes.byref(key())
    nb = B.packed_update_bytes(64, 8)
    h = B.SyncHeader()
    assert err(f, k, 64, 128, 8, A, 1e-3, None, 0, 0, 0, None, Bp, nb, None) == B.ERR_NULL
    assert err(f, k, 64, 128, 300, A, 1e-3, None, 0, 0, 0, ctypes.byref(h), Bp, nb, None) == B.ERR_SHAPE
    assert err(f, k, 64, 128, 8, A, 1e-3, None, 0, 0, -1, ctypes.byref(h), Bp, nb, None) == B.ERR_SHAPE
    assert err(f, k, 64, 128, 8, A, 1e-3, None, 3, 0, 0, ctypes.byref(h), Bp, nb, None) == B.ERR_DOMAIN
    assert err(f, k, 64, 128, 8, A, float("nan"), None, 0, 0, 0, ctypes.byref(h), Bp, nb, None) == B.ERR_DOMAIN
    assert err(f, k, 64, 128, 8, A, 1e-3, None, 0, 0, 0, ctypes.byref(h), Bp, nb - 1, None) == B.ERR_WORKSPACE
    assert err(f, k, 64, 128, 8, A, 1e-3, None, 0, 0, 0, ctypes.byref(h), Bp + 8, nb, None) == B.ERR_ALIGN
    assert err(f, k, 64, 128, 8, A, 1e-3, None, 0, 0, 0, ctypes.byref(h), A + 64, nb, None) == B.ERR_ALIAS
    assert h.magic == 0                                   # no header written on failure

    def header(d=64, kk=128, r=8, mode=0, seed=0, magic=0x4C475253, version=1, nbytes=None):
        return B.SyncHeader(magic, version, key(), d, kk, r, mode, 0, seed, 0,
                            B.packed_update_bytes(d, r) if nbytes is None else nbytes)
    g = lib.logra_sync_apply

    def descs(*hs):
        arr = (B.SyncDesc * len(hs))()
        for i, hh in enumerate(hs):
            arr[i] = B.SyncDesc(ctypes.pointer(hh), Bp + 0x100000 * i, C + 0x100000 * i, hh.k)
        return arr
    h1, h2 = header(), header(magic=7)
    assert err(g, descs(h1, h2), 2, None) == B.ERR_DOMAIN           # bad magic
    assert err(g, descs(header(version=2)), 1, None) == B.ERR_DOMAIN
    assert err(g, descs(header(nbytes=16)), 1, None) == B.ERR_DOMAIN  # sizes disagree
    assert err(g, descs(header(), header(r=16)), 2, None) == B.ERR_SHAPE
    assert err(g, descs(header(), header(mode=1)), 2, None) == B.ERR_SHAPE
    assert err(g, descs(header()), 0, None) == B.ERR_SHAPE
    assert err(g, None, 1, None) == B.ERR_NULL


def test_exact_kl_validation(lib):
    f = lib.logra_exact_kl
    ws = B.exact_kl_ws_bytes(4)
    assert ws == 4 * 8 and B.exact_kl_ws_bytes(0) == 0
    assert err(f, 4, 512, None, Bp, B.BF16, 0.1, 1.0, C, Dp, ws, None) == B.ERR_NULL
    assert err(f, 0, 512, A, Bp, B.BF16, 0.1, 1.0, C, Dp, ws, None) == B.ERR_SHAPE
    assert err(f, 4, 512, A, Bp, 9, 0.1, 1.0, C, Dp, ws, None) == B.ERR_DTYPE
    assert err(f, 4, 512, A, Bp, B.BF16, 0.1, 0.0, C, Dp, ws, None) == B.ERR_DOMAIN
    assert err(f, 4, 512, A, Bp, B.BF16, float("inf"), 1.0, C, Dp, ws, None) == B.ERR_DOMAIN
    assert err(f, 4, 512, A, Bp, B.BF16, 0.1, 1.0, C, Dp, ws - 1, None) == B.ERR_WORKSPACE
    assert err(f, 4, 512, A, Bp, B.BF16, 0.1, 1.0, C + 4, Dp, ws, None) == B.ERR_ALIGN


def test_gaussian_projection_validation(lib):
    k = ctypes.byref(key())
    assert err(lib.logra_regen_A_gaussian, k, 8, 64, None, None) == B.ERR_NULL
    assert err(lib.logra_regen_A_gaussian, k, 300, 64, A, None) == B.ERR_SHAPE
    assert err(lib.logra_regen_A_gaussian, k, 8, 64, A + 4, None) == B.ERR_ALIGN
    # 256-column blocks x 8 steps x 16-rank blocks (padded to 1, 2, 4, 6, 8, 12, 16) x 2 KiB
    assert B.projection_packed_bytes(64, 3584) == 14 * 8 * 4 * 2048
    assert B.projection_packed_bytes(100, 300) == 2 * 8 * 8 * 2048
    assert B.projection_packed_bytes(0, 8) == 0
    nb = B.projection_packed_bytes(8, 64)
    f = lib.logra_pack_projection
    assert err(f, 8, 64, None, Bp, nb, None) == B.ERR_NULL
    assert err(f, 8, 64, A, Bp, nb - 1, None) == B.ERR_WORKSPACE
    assert err(f, 8, 64, A, A + 64, nb, None) == B.ERR_ALIAS
    g = lib.logra_project_input_explicit
    assert err(g, 16, 64, 8, A, B.BF16, 64, Bp, nb, None, None, 0, None) == B.ERR_NULL        # no output
    assert err(g, 16, 64, 8, A, B.F32, 64, Bp, nb, C, None, 0, None) == B.ERR_DTYPE
    assert err(g, 16, 64, 8, A, B.BF16, 64, Bp, nb - 16, C, None, 0, None) == B.ERR_WORKSPACE
    assert err(g, 16, 64, 8, A, B.BF16, 64, Bp, nb, Bp + 64, None, 0, None) == B.ERR_ALIAS     # XAt in A
    h = lib.logra_reconstruction_cosine_explicit
    ws = B.reconstruction_cosine_ws_bytes(64, 64, 8)
    assert err(h, 64, 64, 8, A, B.BF16, 64, None, Bp, nb, C, Dp, ws, None) == B.ERR_NULL
    assert err(h, 64, 64, 8, A, B.F32, 64, C, Bp, nb, C + 0x100000, Dp, ws, None) == B.ERR_DTYPE
    assert err(h, 64, 64, 8, A, B.BF16, 64, C, Bp, nb - 1, C + 0x100000, Dp, ws, None) == B.ERR_WORKSPACE


def test_merge_explicit_validation(lib):
    assert B.merge_projection_packed_bytes(64, 3584) == 7 * 8 * 2 * 4 * 2048     # BC = 512, E = 2, KS = 4
    assert B.merge_projection_packed_bytes(256, 5120) == 20 * 8 * 1 * 16 * 2048  # BC = 256, E = 1, KS = 16
    assert B.merge_projection_packed_bytes(8, 0) == 0
    nb = B.merge_projection_packed_bytes(8, 64)
    assert err(lib.logra_pack_merge_projection, 8, 64, A, Bp, nb - 1, None) == B.ERR_WORKSPACE
    assert err(lib.logra_pack_merge_projection, 8, 64, None, Bp, nb, None) == B.ERR_NULL
    f = lib.logra_merge_grouped_explicit
    d1 = (B.MergeExplicitDesc * 1)(B.MergeExplicitDesc(key(), A, 64, 64, 64, Bp, None, 0, PUP, 1 << 20))
    assert err(f, 8, d1, 1, 1.0, None, 0, 0, None) == B.ERR_NULL
    d1 = (B.MergeExplicitDesc * 1)(B.MergeExplicitDesc(key(), A, 64, 64, 64, Bp, C + 8, 0, PUP, 1 << 20))
    assert err(f, 8, d1, 1, 1.0, None, 0, 0, None) == B.ERR_ALIGN
    d1 = (B.MergeExplicitDesc * 1)(B.MergeExplicitDesc(key(), A, 64, 64, 64, Bp, A + 256, 0, PUP, 1 << 20))
    assert err(f, 8, d1, 1, 1.0, None, 0, 0, None) == B.ERR_ALIAS       # projection inside W


def test_accumulate_table_validation(lib):
    assert B.sketch_accumulate_table_ws_bytes(196) >= 198 * 48 and B.sketch_accumulate_table_ws_bytes(0) == 0
    f = lib.logra_sketch_accumulate_table
    ws = B.sketch_accumulate_table_ws_bytes(2)
    W = 0x20000000
    d2 = (B.AccPackedDesc * 2)(B.AccPackedDesc(A, Bp, C, 64, 64, PIN), B.AccPackedDesc(A + 65536, Bp, C + 64, 64, 64, PIN))
    assert err(f, 128, 64, d2, 2, W, ws, None) == B.ERR_ALIAS            # sketches overlap
    assert err(f, 128, 64, d2, 0, W, ws, None) == B.ERR_SHAPE
    assert err(f, 128, 64, d2, 2, W, ws - 1, None) == B.ERR_WORKSPACE
    assert err(f, 128, 64, d2, 2, None, ws, None) == B.ERR_NULL
    assert err(f, 128, 300, d2, 1, W, ws, None) == B.ERR_SHAPE
    d2 = (B.AccPackedDesc * 2)(B.AccPackedDesc(A, Bp, C, 64, 64, PIN), B.AccPackedDesc(C + 1024, Bp, Dp, 64, 64, PIN))
    assert err(f, 128, 64, d2, 2, W, ws, None) == B.ERR_ALIAS            # sketch 0 inside D of 1
    d1 = (B.AccPackedDesc * 1)(B.AccPackedDesc(A, Bp, C, 64, 64, PIN))
    assert err(f, 128, 64, d1, 1, C + 64, ws, None) == B.ERR_ALIAS       # workspace inside S


def test_project_table_validation(lib):
    """Host-side checks of the table projection; nothing is launched."""
    assert B.project_input_table_ws_bytes(196) >= 198 * 64
    assert B.project_input_table_ws_bytes(0) == 0 and B.project_input_table_ws_bytes(1025) == 0
    f = lib.logra_project_input_table
    ws = B.project_input_table_ws_bytes(2)
    W = 0x20000000
    k0 = B.key(1, 2, 3)
    P = B.packed_input_bytes(64, 64)

    def descs(*rows):
        return (B.ProjectDesc * len(rows))(*[B.ProjectDesc(k0, *row, P) for row in rows])

    good = descs((A, 256, 256, None, C), (A, 256, 256, None, C + P))       # one X shared
    assert err(f, 64, 64, good, 2, W, ws - 1, None) == B.ERR_WORKSPACE
    assert err(f, 64, 64, good, 0, W, ws, None) == B.ERR_SHAPE
    assert err(f, 64, 64, good, 1025, W, ws, None) == B.ERR_SHAPE
    assert err(f, 64, 300, good, 2, W, ws, None) == B.ERR_SHAPE
    assert err(f, 64, 64, good, 2, None, ws, None) == B.ERR_NULL
    assert err(f, 64, 64, descs((A, 256, 256, None, None)), 1, W, ws, None) == B.ERR_NULL  # no output
    assert err(f, 64, 64, descs((0, 256, 256, None, C)), 1, W, ws, None) == B.ERR_NULL
    assert err(f, 64, 64, descs((A, 256, 200, None, C)), 1, W, ws, None) == B.ERR_SHAPE    # ldx < k
    assert err(f, 64, 64, descs((A, 256, 256, None, C + 8)), 1, W, ws, None) == B.ERR_ALIGN
    assert err(f, 64, 64, descs((A + 8, 256, 256, None, C)), 1, W, ws, None) == B.ERR_ALIGN
    overl = descs((A, 256, 256, None, C), (A, 256, 256, None, C + P - 256))
    assert err(f, 64, 64, overl, 2, W, ws, None) == B.ERR_ALIAS                # planes overlap
    xat = descs((A, 256, 256, C, C + 64 * 64 * 4 - 16))
    assert err(f, 64, 64, xat, 1, W, ws, None) == B.ERR_ALIAS                  # XAt meets planes
    into_x = descs((A, 256, 256, None, C), (C + 2 * P, 256, 256, None, A + 4096))
    assert err(f, 64, 64, into_x, 2, W, ws, None) == B.ERR_ALIAS               # planes inside X of 0
    assert err(f, 64, 64, good, 2, A + 1024, ws, None) == B.ERR_ALIAS          # workspace inside X
    assert err(f, 64, 64, good, 2, C + 16, ws, None) == B.ERR_ALIAS            # workspace meets planes


def test_packed_buffer_sizes_are_checked(lib):
    """Every descriptor that points at a packed buffer carries its size, and a buffer smaller
    than the layout needs is rejected before anything is launched (a short buffer would be
    read past its end)."""
    W = 0x20000000
    # accumulate: table and grouped packed, planes one 16-byte chunk short
    f = lib.logra_sketch_accumulate_table
    ws = B.sketch_accumulate_table_ws_bytes(1)
    for pb, want in ((PIN - 16, B.ERR_WORKSPACE), (0, B.ERR_WORKSPACE)):
        d1 = (B.AccPackedDesc * 1)(B.AccPackedDesc(A, Bp, C, 64, 64, pb))
        assert err(f, 128, 64, d1, 1, W, ws, None) == want
        assert err(lib.logra_sketch_accumulate_grouped_packed, 128, 64, d1, 1, None) == want
        assert "packed input" in lib.logra_last_error().decode()
    # planes sized for fewer tokens or a lower rank than the call's
    small_T = B.packed_input_bytes(64, 64)
    small_r = B.packed_input_bytes(128, 32)
    for pb in (small_T, small_r):
        d1 = (B.AccPackedDesc * 1)(B.AccPackedDesc(A, Bp, C, 64, 64, pb))
        assert err(f, 128, 64, d1, 1, W, ws, None) == B.ERR_WORKSPACE
    # table projection: planes too small for T x r
    g = lib.logra_project_input_table
    pws = B.project_input_table_ws_bytes(1)
    d = (B.ProjectDesc * 1)(B.ProjectDesc(B.key(1, 2, 3), A, 256, 256, None, C, B.packed_input_bytes(64, 64) - 16))
    assert err(g, 64, 64, d, 1, W, pws, None) == B.ERR_WORKSPACE
    # merges: packed update and explicit projection too small
    m = lib.logra_merge_grouped_packed
    d1 = (B.MergePackedDesc * 1)(B.MergePackedDesc(key(), A, 64, 64, 64, Bp, 0, PUP - 16))
    assert err(m, 64, d1, 1, 1.0, None, 0, 0, None) == B.ERR_WORKSPACE
    x = lib.logra_merge_grouped_explicit
    need = B.merge_projection_packed_bytes(8, 64)
    d1 = (B.MergeExplicitDesc * 1)(B.MergeExplicitDesc(key(), A, 64, 64, 64, Bp, C, 0, PUP, need - 16))
    assert err(x, 8, d1, 1, 1.0, None, 0, 0, None) == B.ERR_WORKSPACE
    d1 = (B.MergeExplicitDesc * 1)(B.MergeExplicitDesc(key(), A, 64, 64, 64, Bp, C, 0, 16, need))
    assert err(x, 8, d1, 1, 1.0, None, 0, 0, None) == B.ERR_WORKSPACE


def test_bandwidth_probe_validation(lib):
    f = lib.logra_bandwidth_probe
    assert err(f, 0, None, Bp, 1 << 20, 4, None) == B.ERR_NULL
    assert err(f, 2, A, Bp, 1 << 20, 4, None) == B.ERR_DOMAIN             # unknown mode
    assert err(f, 0, A, Bp, 0, 4, None) == B.ERR_SHAPE
    assert err(f, 0, A, Bp, 1000, 4, None) == B.ERR_SHAPE                 # not a multiple of 16
    assert err(f, 0, A, Bp, 1 << 20, 0, None) == B.ERR_SHAPE
    assert err(f, 0, A, Bp, 1 << 20, 33, None) == B.ERR_SHAPE
    assert err(f, 1, A + 8, Bp, 1 << 20, 4, None) == B.ERR_ALIGN
    assert err(f, 1, A, A + (1 << 19), 1 << 20, 4, None) == B.ERR_ALIAS   # copy onto itself
    assert err(f, 0, A, A + 4096, 1 << 20, 4, None) == B.ERR_ALIAS        # fold slots inside src


def test_predicted_kl_noalloc_validation(lib):
    """The allocation-free q takes no workspace and rejects more contexts than its scratch holds."""
    f = lib.logra_predicted_kl_q_noalloc
    assert err(f, 4, 512, None, Bp, B.BF16, 1.0, C, None) == B.ERR_NULL
    assert err(f, 0, 512, A, Bp, B.BF16, 1.0, C, None) == B.ERR_SHAPE
    assert err(f, B.NOALLOC_MAX_CONTEXTS + 1, 8, A, Bp, B.BF16, 1.0, C, None) == B.ERR_SHAPE
    assert err(f, 4, 512, A, Bp, B.I8, 1.0, C, None) == B.ERR_DTYPE
    assert err(f, 4, 512, A, Bp, B.BF16, 0.0, C, None) == B.ERR_DOMAIN
    assert err(f, 4, 512, A + 8, Bp, B.BF16, 1.0, C, None) == B.ERR_ALIGN
    assert "contexts" in (lib.logra_predicted_kl_q_noalloc(B.NOALLOC_MAX_CONTEXTS + 1, 8, A, Bp, B.BF16, 1.0, C,
                                                           None) and lib.logra_last_error().decode())
