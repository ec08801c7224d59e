"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Tolerances (the contract): S and U relative Frobenius error <= 2e-3; q and
alpha <= 1e-4 relative; merged W within 1 bf16 ulp of the oracle on >= 99.99%
of elements; A bit-exact; repeated merges bit-identical.  Tighter bounds
derived from the arithmetic are asserted as well, so that a dropped term
(e.g. the lo half of the bf16 split, worth ~1.7e-3) cannot hide under the
contract's 2e-3:
  - XAt from bf16 X: exact products, fp32 accumulation -> <= 1e-5;
  - S from bf16 D: XAt carried as bf16 hi + lo (~2^-17 relative) and fp32
    accumulation -> <= 5e-5;
  - U from the same S: fp64 reductions -> <= 1e-6.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import philox
from rank_gradient_sketching_logra_amd import binding as B
from rank_gradient_sketching_logra_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the parity tests need an MI355X")
    B.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def relfro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def bf16_inputs(shape, std, words):
    bits = synth.normal(shape, std, words, "bf16")
    return bits, oracle.bf16_bits_to_f64(bits)


# ------------------------------------------------------------ regen A


@pytest.mark.parametrize("r,k", [(1, 1), (8, 256), (64, 3584), (33, 700), (256, 5120), (7, 1000)])
def test_regen_A_bit_exact(r, k):
    say(f"regen_A r={r} k={k}")
    kk = B.key(0x1234ABCD, 17, 3)
    A8 = B.regen_A(kk, r, k, torch.int8, DEV).cpu().numpy()
    A32 = B.regen_A(kk, r, k, torch.float32, DEV).cpu().numpy()
    assert np.array_equal(A8, oracle.regen_A(0x1234ABCD, 17, 3, r, k, kind="i8"))
    assert np.array_equal(A32.view(np.uint32), oracle.regen_A(0x1234ABCD, 17, 3, r, k, kind="f32").view(np.uint32))


# ------------------------------------------------------------ project


@pytest.mark.parametrize("T,k,r,ldx", [(64, 256, 64, 256), (1000, 712, 33, 720), (96, 3584, 256, 3584),
                                       (37, 40, 1, 48), (512, 1536, 64, 1536), (50, 1001, 64, 1008),
                                       (20, 259, 96, 264), (1, 300, 64, 304), (3, 5120, 256, 5120)])
def test_project_bf16(T, k, r, ldx):
    say(f"project bf16 T={T} k={k} r={r} ldx={ldx}")
    bits, X = bf16_inputs((T, ldx), 1.0, (9, T, k, r, 0))
    Xd = bf16_dev(bits)[:, :k]
    kk = B.key(5, 2, 1)
    XAt = B.project_input(kk, Xd, r).cpu().numpy()
    want = oracle.project(X[:, :k], oracle.regen_A(5, 2, 1, r, k))
    assert relfro(XAt, want) <= 1e-5


def test_project_identity_gives_projection_transpose():
    """X = I_k (bf16, exact) gives X A^T = A^T bit for bit against regen_A's fp32 A."""
    k, r = 512, 64
    say("project identity")
    Xd = torch.eye(k, dtype=torch.bfloat16, device=DEV)
    kk = B.key(11, 4, 9)
    XAt = B.project_input(kk, Xd, r).cpu().numpy()
    A32 = B.regen_A(kk, r, k, torch.float32, DEV).cpu().numpy()
    assert np.array_equal(XAt.view(np.uint32), A32.T.copy().view(np.uint32))


@pytest.mark.parametrize("T,k,r", [(512, 256, 8), (33, 300, 5)])
def test_project_f32(T, k, r):
    say(f"project f32 T={T} k={k} r={r}")
    X = synth.normal((T, k), 1.0, (10, T, k, r, 0), "f32")
    kk = B.key(1, 0, 0)
    XAt = B.project_input(kk, torch.from_numpy(X).to(DEV), r).cpu().numpy()
    want = oracle.project(X.astype(np.float64), oracle.regen_A(1, 0, 0, r, k))
    assert relfro(XAt, want) <= 1e-6


# ------------------------------------------------------------ accumulate


@pytest.mark.parametrize("T,d,r,ldd", [(1000, 300, 64, 304), (512, 256, 8, 256), (4096, 512, 64, 512),
                                       (300, 1000, 256, 1000), (77, 24, 33, 24), (2048, 1536, 100, 1536),
                                       (16, 8, 1, 8), (4500, 700, 40, 704), (32, 300, 64, 304),
                                       (1000, 1280, 256, 1280), (777, 768, 128, 768), (520, 600, 160, 608),
                                       (40, 520, 96, 520), (2, 257, 256, 264)])
def test_accumulate_bf16(T, d, r, ldd):
    say(f"accumulate bf16 T={T} d={d} r={r} ldd={ldd}")
    S0 = synth.fp32_matrix((d, r), 0.1, (12, d, r, 0, 5))
    S = torch.from_numpy(S0.copy()).to(DEV)
    want = S0.astype(np.float64)
    for mb in range(2):
        bits, Dm = bf16_inputs((T, ldd), 1e-3, (12, T, d, mb, 1))
        XAt = synth.fp32_matrix((T, r), 3.0, (12, T, r, mb, 0))
        B.sketch_accumulate(bf16_dev(bits)[:, :d], torch.from_numpy(XAt).to(DEV), S)
        want = oracle.accumulate(want, Dm[:, :d], XAt.astype(np.float64))
    got = S.cpu().numpy()
    err = relfro(got, want)
    say(f"  rel-Fro {err:.3e}")
    assert err <= 5e-5


@pytest.mark.parametrize("T,d,r", [(512, 256, 8), (100, 37, 3)])
def test_accumulate_f32(T, d, r):
    say(f"accumulate f32 T={T} d={d} r={r}")
    ld = (d + 3) // 4 * 4
    D = synth.normal((T, ld), 1e-3, (13, T, d, 0, 1), "f32")
    XAt = synth.fp32_matrix((T, r), 2.0, (13, T, r, 0, 0))
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    B.sketch_accumulate(torch.from_numpy(D).to(DEV)[:, :d], torch.from_numpy(XAt).to(DEV), S)
    want = oracle.accumulate(np.zeros((d, r)), D[:, :d].astype(np.float64), XAt.astype(np.float64))
    assert relfro(S.cpu().numpy(), want) <= 1e-6


@pytest.mark.parametrize("T,r", [(1024, 64), (4200, 64), (1000, 256), (520, 128)])
def test_accumulate_grouped_is_bit_identical_to_single_calls(T, r):
    shapes = [(3584, 0), (512, 1), (512, 2), (1000, 3), (2048, 4)]
    say(f"accumulate grouped vs single T={T} r={r}")
    items, singles, xat = [], [], {}
    for d, i in shapes:
        bits, _ = bf16_inputs((T, d), 1e-3, (14, d, i, 0, 1))
        D = bf16_dev(bits)
        # items 0-2 read one projected input (one tensor), as q, k and v do
        if i <= 2 and 0 in xat:
            XAt = xat[0]
        else:
            XAt = xat[i] = torch.from_numpy(synth.fp32_matrix((T, r), 3.0, (14, d, i, 0, 0))).to(DEV)
        S1 = torch.from_numpy(synth.fp32_matrix((d, r), 0.1, (14, d, i, 0, 5))).to(DEV)
        S2 = S1.clone()
        items.append((D, XAt, S1))
        singles.append((D, XAt, S2))
    B.sketch_accumulate_grouped(items)
    for D, XAt, S2 in singles:
        B.sketch_accumulate(D, XAt, S2)
    for (_, _, S1), (_, _, S2) in zip(items, singles):
        assert torch.equal(S1.view(torch.int32), S2.view(torch.int32))


@pytest.mark.parametrize("T,r", [(1000, 64), (4096, 33), (520, 256), (777, 100)])
def test_accumulate_table_equals_grouped_calls(T, r):
    """One persistent launch over a table of many matrices (three 'layers' of mixed widths,
    including a ragged edge tile) gives the bits of the per-layer grouped packed launches, and
    matches the oracle."""
    shapes = [(640, 0), (256, 1), (1000, 2), (2048, 3), (512, 4), (300, 5), (768, 6), (256, 7), (1536, 8)]
    say(f"accumulate table T={T} r={r}")
    planes = []
    for g in range(3):
        xb = synth.normal((T, 64), 1.0, (33, T, g, 0, 9), "bf16")
        planes.append(B.project_input_packed(B.key(2, g, 1), bf16_dev(xb), r))
    items_t, items_g, host = [], [], []
    for d, i in shapes:
        ld = (d + 7) // 8 * 8
        db, Dm = bf16_inputs((T, ld), 1e-3, (33, T, d, i, 1))
        D = bf16_dev(db)[:, :d]
        S0 = synth.fp32_matrix((d, r), 0.1, (33, d, r, i, 5))
        P = planes[i // 3]
        items_t.append((D, P, torch.from_numpy(S0.copy()).to(DEV)))
        items_g.append((D, P, torch.from_numpy(S0.copy()).to(DEV)))
        host.append((Dm[:, :d], S0))
    B.sketch_accumulate_table(items_t, r)
    for g in range(3):
        B.sketch_accumulate_grouped_packed(items_g[3 * g:3 * g + 3], r)
    for (_, _, St), (_, _, Sg) in zip(items_t, items_g):
        assert torch.equal(St.view(torch.int32), Sg.view(torch.int32))
    # the oracle, through the projection the packed planes hold
    for g in range(3):
        X = oracle.bf16_bits_to_f64(synth.normal((T, 64), 1.0, (33, T, g, 0, 9), "bf16"))
        XAt = oracle.project(X, oracle.regen_A(2, g, 1, r, 64))
        for (_, _, St), (Dm, S0) in list(zip(items_t, host))[3 * g:3 * g + 3]:
            assert relfro(St.cpu().numpy(), S0 + Dm.T @ XAt) <= 5e-5


@pytest.mark.parametrize("T,r", [(48, 64), (200, 256)])
def test_accumulate_table_many_tiles_per_block(T, r):
    """A table of more tiles than the grid has blocks, so every block claims several tiles in
    turn from its XCD's range: twice in a row on one workspace (the counters start again from
    zero), the same bits as one grouped launch per matrix, and the oracle on two matrices."""
    widths = [4096 + 256 * (i % 5) - 37 * (i % 3) for i in range(24)]  # 16..20 tiles each
    say(f"accumulate table, many tiles T={T} r={r} tiles={sum((d + 255) // 256 for d in widths)}")
    xb = synth.normal((T, 64), 1.0, (34, T, r, 0, 9), "bf16")
    P = B.project_input_packed(B.key(2, 5, 1), bf16_dev(xb), r)
    items_t, items_g, host = [], [], []
    for i, d in enumerate(widths):
        ld = (d + 7) // 8 * 8
        db, Dm = bf16_inputs((T, ld), 1e-3, (34, T, d, i, 1))
        D = bf16_dev(db)[:, :d]
        S0 = synth.fp32_matrix((d, r), 0.1, (34, d, r, i, 5))
        items_t.append((D, P, torch.from_numpy(S0.copy()).to(DEV)))
        items_g.append((D, P, torch.from_numpy(S0.copy()).to(DEV)))
        host.append((Dm[:, :d], S0))
    ws = B.workspace(B.sketch_accumulate_table_ws_bytes(len(widths)), DEV)
    for _ in range(2):
        B.sketch_accumulate_table(items_t, r, ws=ws)
        for it in items_g:
            B.sketch_accumulate_grouped_packed([it], r)
    for (_, _, St), (_, _, Sg) in zip(items_t, items_g):
        assert torch.equal(St.view(torch.int32), Sg.view(torch.int32))
    X = oracle.bf16_bits_to_f64(xb)
    XAt = oracle.project(X, oracle.regen_A(2, 5, 1, r, 64))
    for i in (0, len(widths) - 1):
        Dm, S0 = host[i]
        assert relfro(items_t[i][2].cpu().numpy(), S0 + 2.0 * (Dm.T @ XAt)) <= 5e-5


@pytest.mark.parametrize("T,r", [(1000, 64), (4096, 33), (48, 256)])
def test_packed_projection_feeds_accumulate(T, r):
    """project_input_packed + accumulate_grouped_packed: the same XAt bits as project_input,
    the same S bits as the unpacked grouped accumulate, and S within tolerance of the oracle's
    (D^T X) A^T."""
    k, ds = 320, [640, 300, 256]
    say(f"packed projection T={T} r={r}")
    kk = B.key(3, 7, 1)
    xb, X = bf16_inputs((T, k), 1.0, (17, T, r, 0, 0))
    Xd = bf16_dev(xb)
    XAt_ref = B.project_input(kk, Xd, r)
    XAt = torch.empty_like(XAt_ref)
    planes = B.project_input_packed(kk, Xd, r, out=XAt)
    assert torch.equal(XAt.view(torch.int32), XAt_ref.view(torch.int32))
    items_p, items_u, wants = [], [], []
    A = oracle.regen_A(3, 7, 1, r, k)
    for i, d in enumerate(ds):
        ld = (d + 7) // 8 * 8
        db, Dm = bf16_inputs((T, ld), 1e-3, (17, T, d, i, 1))
        D = bf16_dev(db)[:, :d]
        S0 = synth.fp32_matrix((d, r), 0.1, (17, d, r, i, 5))
        items_p.append((D, planes, torch.from_numpy(S0.copy()).to(DEV)))
        items_u.append((D, XAt_ref, torch.from_numpy(S0.copy()).to(DEV)))
        wants.append(S0.astype(np.float64) + oracle.dense_gradient(Dm[:, :d], X) @ A.T)
    B.sketch_accumulate_grouped_packed(items_p, r)
    B.sketch_accumulate_grouped(items_u)
    for (_, _, Sp), (_, _, Su), want in zip(items_p, items_u, wants):
        assert torch.equal(Sp.view(torch.int32), Su.view(torch.int32))
        assert relfro(Sp.cpu().numpy(), want) <= 5e-5


@pytest.mark.parametrize("T,k,r", [(777, 64, 100), (48, 312, 256), (777, 312, 8), (1000, 64, 33)])
def test_packed_planes_layout_against_oracle(T, k, r):
    """The packed projected input decoded by its documented layout (per 16-token step and
    32-rank block a hi operand then a lo operand; lane l holding tokens 8(l >> 5) + i of rank
    32b + (l & 31)): hi + lo is the oracle's X A^T, and the padding (ranks past r, tokens past
    T) is exactly zero.  Run twice, on a fresh output and on one filled with NaN, so no part
    of the output may be left unwritten."""
    say(f"packed planes layout T={T} k={k} r={r}")
    xb, X = bf16_inputs((T, k), 1.0, (35, T, k, r, 0))
    want = oracle.project(X, oracle.regen_A(4, 2, 1, r, k))
    nrb = {1: 1, 2: 2}.get((r + 31) // 32, 4 if (r + 31) // 32 <= 4 else 8)
    nsteps = (T + 15) // 16
    pad = np.zeros((16 * nsteps, 32 * nrb))
    pad[:T, :r] = want
    full = np.zeros((nsteps, nrb, 64, 8))
    for lane in range(64):
        for i in range(8):
            full[:, :, lane, i] = pad[8 * (lane >> 5) + i::16, :].reshape(nsteps, nrb, 32)[:, :, lane & 31]
    for fill in (None, float("nan")):
        planes = None
        if fill is not None:
            planes = torch.full((B.packed_input_bytes(T, r) // 2,), fill, dtype=torch.bfloat16, device=DEV).view(torch.uint8)
        planes = B.project_input_packed(B.key(4, 2, 1), bf16_dev(xb), r, planes=planes)
        u = planes.cpu().numpy().view(np.uint16)[: nsteps * nrb * 1024].reshape(nsteps, nrb, 2, 64, 8)
        dec = (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        got = dec[:, :, 0] + dec[:, :, 1]
        assert np.isfinite(got).all()
        live = np.zeros_like(full, dtype=bool)
        live_pad = np.zeros_like(pad, dtype=bool)
        live_pad[:T, :r] = True
        for lane in range(64):
            for i in range(8):
                live[:, :, lane, i] = live_pad[8 * (lane >> 5) + i::16, :].reshape(nsteps, nrb, 32)[:, :, lane & 31]
        assert np.all(dec[:, :, 0][~live] == 0) and np.all(dec[:, :, 1][~live] == 0)
        assert relfro(got, full) <= 2e-5
        # hi is the nearest bf16 of the sum: |lo| at most half an ulp of hi
        hi = dec[:, :, 0]
        assert np.all(np.abs(dec[:, :, 1]) <= np.abs(hi) * 2.0 ** -8 + 1e-30)


@pytest.mark.parametrize("T,r", [(1000, 64), (48, 256), (200, 33), (1, 64), (5, 256)])
def test_project_table(T, r):
    """One table launch over projections of mixed widths (ragged k, padded rows, one X shared by
    two projections, entries with only XAt or only planes): XAt within 1e-5 of the oracle and
    within fp32 rounding of the single-call projection; the planes give the S bits of the
    table's own XAt through the unpacked accumulate, and S within tolerance of the oracle; a
    second call on the same workspace gives the same bits."""
    widths = [(256, 256), (712, 720), (1001, 1008), (3584, 3584), (40, 48)]
    say(f"project table T={T} r={r}")
    xs = []
    for i, (k, ld) in enumerate(widths):
        xb, X = bf16_inputs((T, ld), 1.0, (35, T, k, i, 0))
        xs.append((bf16_dev(xb)[:, :k], X[:, :k]))
    # (input, matrix id, XAt wanted, planes wanted); input 0 is shared by two projections
    spec = [(0, 1, True, True), (1, 2, True, True), (2, 3, True, False), (3, 4, True, True),
            (4, 5, True, True), (0, 6, False, True)]
    nb = B.packed_input_bytes(T, r)

    def outputs():
        return [(torch.full((T, r), float("nan"), device=DEV) if want_x else None,
                 torch.zeros((nb,), dtype=torch.uint8, device=DEV) if want_p else None)
                for (_, _, want_x, want_p) in spec]

    ws = B.workspace(B.project_input_table_ws_bytes(len(spec)), DEV)
    runs = []
    for _ in range(2):
        outs = outputs()
        B.project_input_table([(B.key(8, mid, 2), xs[xi][0], xo, po)
                               for (xi, mid, _, _), (xo, po) in zip(spec, outs)], r, ws=ws)
        runs.append(outs)
    for (xa, pa), (xb_, pb) in zip(*runs):
        if xa is not None:
            assert torch.equal(xa.view(torch.int32), xb_.view(torch.int32))
        if pa is not None:
            assert torch.equal(pa, pb)
    d = 300
    db, Dm = bf16_inputs((T, 304), 1e-3, (35, T, d, 0, 1))
    D = bf16_dev(db)[:, :d]
    S0 = synth.fp32_matrix((d, r), 0.1, (35, d, r, 0, 5))
    for (xi, mid, _, _), (xo, po) in zip(spec, runs[0]):
        Xd, X = xs[xi]
        A = oracle.regen_A(8, mid, 2, r, X.shape[1])
        if xo is not None:
            assert relfro(xo.cpu().numpy(), oracle.project(X, A)) <= 1e-5
            assert relfro(xo.cpu().numpy(), B.project_input(B.key(8, mid, 2), Xd, r).cpu().numpy()) <= 1e-6
        if po is not None:
            Sp = torch.from_numpy(S0.copy()).to(DEV)
            B.sketch_accumulate_grouped_packed([(D, po, Sp)], r)
            assert relfro(Sp.cpu().numpy(), S0 + oracle.dense_gradient(Dm[:, :d], X) @ A.T) <= 5e-5
            if xo is not None:
                Su = torch.from_numpy(S0.copy()).to(DEV)
                B.sketch_accumulate_grouped([(D, xo, Su)])
                assert torch.equal(Sp.view(torch.int32), Su.view(torch.int32))


@pytest.mark.parametrize("T,r", [(1000, 64), (777, 33), (200, 100)])
def test_project_table_fused_inputs(T, r):
    """Consecutive projections of one input (q, k, v; gate, up; four in a row, one more than an
    entry holds) are projected together, reading the input once: the same XAt and packed bits
    as the same table with every input a distinct copy, and within 1e-5 of the oracle."""
    say(f"project table fused T={T} r={r}")
    widths = [(512, 512), (300, 304), (3584, 3584)]
    xs = []
    for i, (k, ld) in enumerate(widths):
        xb, X = bf16_inputs((T, ld), 1.0, (37, T, k, i, 0))
        xs.append((bf16_dev(xb), X[:, :k], k))
    order = [0, 0, 0, 1, 2, 2, 1, 0, 0, 0, 0, 2]   # input of each projection, in table order
    nb = B.packed_input_bytes(T, r)

    def run(inputs):
        outs = [(torch.full((T, r), float("nan"), device=DEV),
                 torch.full((nb // 2,), float("nan"), dtype=torch.bfloat16, device=DEV).view(torch.uint8))
                for _ in order]
        B.project_input_table([(B.key(10, j, 3), inputs[j], xo, po)
                               for j, (xo, po) in enumerate(outs)], r)
        return outs

    fused = run([xs[i][0][:, :xs[i][2]] for i in order])
    # distinct copies (padded rows kept): nothing to share
    alone = run([xs[i][0].clone()[:, :xs[i][2]] for i in order])
    for (xf, pf), (xa, pa) in zip(fused, alone):
        assert torch.equal(xf.view(torch.int32), xa.view(torch.int32))
        assert torch.equal(pf, pa)
    for j in (0, 2, 5, 10):
        X = xs[order[j]][1]
        want = oracle.project(X, oracle.regen_A(10, j, 3, r, X.shape[1]))
        assert relfro(fused[j][0].cpu().numpy(), want) <= 1e-5


@pytest.mark.parametrize("T,r", [(1000, 64), (777, 33), (40, 8)])
def test_project_table_sixteen_byte_inputs(T, r):
    """Up to 64 ranks, a table whose every k is a multiple of 8 loads its inputs 16 bytes at a
    time and rearranges the sign words to match (k from 8 to 3584, one input shared by
    consecutive projections, ragged T): XAt within 1e-5 of the oracle and within fp32 rounding
    of the single-call projection, and the planes give the S bits of the table's own XAt
    through the unpacked accumulate."""
    say(f"project table, 16-byte inputs T={T} r={r}")
    widths = [(512, 512), (3584, 3584), (40, 48), (1000, 1000), (8, 8)]
    xs = []
    for i, (k, ld) in enumerate(widths):
        xb, X = bf16_inputs((T, ld), 1.0, (39, T, k, i, 0))
        xs.append((bf16_dev(xb)[:, :k], X[:, :k]))
    order = [0, 0, 0, 1, 2, 3, 3, 4]   # input of each projection, in table order
    nb = B.packed_input_bytes(T, r)
    outs = [(torch.full((T, r), float("nan"), device=DEV), torch.zeros((nb,), dtype=torch.uint8, device=DEV))
            for _ in order]
    B.project_input_table([(B.key(11, j, 4), xs[xi][0], xo, po)
                           for j, (xi, (xo, po)) in enumerate(zip(order, outs))], r)
    d = 200
    db, _ = bf16_inputs((T, d), 1e-3, (39, T, d, 0, 1))
    D = bf16_dev(db)
    S0 = synth.fp32_matrix((d, r), 0.1, (39, d, r, 0, 5))
    for j, xi in enumerate(order):
        Xd, X = xs[xi]
        xo, po = outs[j]
        assert relfro(xo.cpu().numpy(), oracle.project(X, oracle.regen_A(11, j, 4, r, X.shape[1]))) <= 1e-5
        assert relfro(xo.cpu().numpy(), B.project_input(B.key(11, j, 4), Xd, r).cpu().numpy()) <= 1e-6
        Sp = torch.from_numpy(S0.copy()).to(DEV)
        B.sketch_accumulate_grouped_packed([(D, po, Sp)], r)
        Su = torch.from_numpy(S0.copy()).to(DEV)
        B.sketch_accumulate_grouped([(D, xo, Su)])
        assert torch.equal(Sp.view(torch.int32), Su.view(torch.int32))


def test_project_table_many_items_per_wave():
    """More work items (two 16-token steps each) than the grid has waves, so every wave claims
    several in turn: every XAt within fp32 rounding of the single-call projection, two against
    the oracle."""
    T, r = 4096, 64
    ks = [256, 512, 300] * 12
    say(f"project table, many items: {len(ks) * T // 32} items")
    xs = []
    for i, k in enumerate(ks):
        ld = (k + 7) // 8 * 8
        xb, X = bf16_inputs((T, ld), 1.0, (36, T, k, i, 0))
        xs.append((bf16_dev(xb)[:, :k], X[:, :k]))
    outs = [torch.full((T, r), float("nan"), device=DEV) for _ in ks]
    B.project_input_table([(B.key(9, i, 1), xs[i][0], outs[i], None) for i in range(len(ks))], r)
    for i in range(len(ks)):
        single = B.project_input(B.key(9, i, 1), xs[i][0], r)
        assert relfro(outs[i].cpu().numpy(), single.cpu().numpy()) <= 1e-6
    for i in (0, len(ks) - 1):
        want = oracle.project(xs[i][1], oracle.regen_A(9, i, 1, r, ks[i]))
        assert relfro(outs[i].cpu().numpy(), want) <= 1e-5


@pytest.mark.parametrize("r", [64, 256])
def test_accumulate_nan_in_d_stays_in_its_row(r):
    """A NaN in D at (token t, column c) makes row c of S NaN, as D^T X A^T does, and leaves
    every other row within tolerance of the oracle: through the table projection's packed
    planes and the table accumulate the benchmark times."""
    T, k, d = 300, 256, 512
    say(f"accumulate with a NaN in D r={r}")
    xb, X = bf16_inputs((T, k), 1.0, (47, T, k, r, 0))
    db, Dm = bf16_inputs((T, d), 1e-3, (47, T, d, r, 1))
    db = db.copy()
    db[5, 7] = 0x7FC0
    db[200, 300] = 0xFFC0
    kk = B.key(6, 3, 1)
    P = torch.zeros((B.packed_input_bytes(T, r),), dtype=torch.uint8, device=DEV)
    B.project_input_table([(kk, bf16_dev(xb), None, P)], r)
    S0 = synth.fp32_matrix((d, r), 0.1, (47, d, r, 0, 5))
    S = torch.from_numpy(S0.copy()).to(DEV)
    B.sketch_accumulate_table([(bf16_dev(db), P, S)], r)
    got = S.cpu().numpy()
    bad = np.zeros(d, bool)
    bad[[7, 300]] = True
    assert np.isnan(got[bad]).all()
    assert np.isfinite(got[~bad]).all()
    want = S0.astype(np.float64) + oracle.dense_gradient(Dm, X) @ oracle.regen_A(6, 3, 1, r, k).T
    assert relfro(got[~bad], want[~bad]) <= 5e-5


def test_accumulate_deterministic_and_zero_d_is_noop():
    T, d, r = 2048, 2000, 64
    say("accumulate determinism")
    bits, _ = bf16_inputs((T, d), 1e-3, (15, 0, 0, 0, 1))
    D = bf16_dev(bits)
    XAt = torch.from_numpy(synth.fp32_matrix((T, r), 3.0, (15, 0, 0, 0, 0))).to(DEV)
    S0 = torch.from_numpy(synth.fp32_matrix((d, r), 0.1, (15, 0, 0, 0, 5))).to(DEV)
    a, b = S0.clone(), S0.clone()
    B.sketch_accumulate(D, XAt, a)
    B.sketch_accumulate(D, XAt, b)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    c = S0.clone()
    B.sketch_accumulate(torch.zeros_like(D), XAt, c)
    assert torch.equal(c.view(torch.int32), S0.view(torch.int32))


def test_project_then_accumulate_equals_dense_gradient_projection():
    """End to end on the smallest workload's shapes with bf16 data: S from the
    library vs (D^T X) A^T from the oracle's dense gradient."""
    T, d, k, r = 512, 256, 256, 8
    say("project+accumulate vs dense gradient")
    kk = B.key(1, 0, 0)
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    G = np.zeros((d, k))
    for mb in range(2):
        xb, X = bf16_inputs((T, k), 1.0, (16, mb, 0, 0, 0))
        db, Dm = bf16_inputs((T, d), 1e-3, (16, mb, 0, 0, 1))
        XAt = B.project_input(kk, bf16_dev(xb), r)
        B.sketch_accumulate(bf16_dev(db), XAt, S)
        G += oracle.dense_gradient(Dm, X)
    want = G @ oracle.regen_A(1, 0, 0, r, k).T
    assert relfro(S.cpu().numpy(), want) <= 5e-5


# ------------------------------------------------------------ RowAdam


@pytest.mark.parametrize("d,r,t,beta", [(4096, 64, 1, 0.999), (18944, 64, 3, 0.95), (300, 7, 2, 0.9),
                                        (1, 1, 1, 0.95), (513, 256, 5, 0.0)])
def test_rowadam(d, r, t, beta):
    say(f"rowadam d={d} r={r} t={t} beta={beta}")
    S0 = synth.fp32_matrix((d, r), 0.5, (17, d, r, t, 5))
    S0 *= synth.fp32_matrix((d, 1), 1.0, (17, d, r, t, 6)) ** 2 + np.float32(0.05)
    if d > 10:
        S0[5] = 0
    v0 = np.abs(synth.fp32_matrix((d,), 0.2, (17, d, r, t, 7))) if t > 1 else np.zeros(d, np.float32)
    S = torch.from_numpy(S0).to(DEV)
    v = torch.from_numpy(v0.copy()).to(DEV)
    U = B.rowadam(S, v, t, beta, 1e-8)
    Uw, vw = oracle.rowadam(S0.astype(np.float64), v0.astype(np.float64), t, beta, 1e-8)
    assert relfro(U.cpu().numpy(), Uw) <= 1e-6
    assert relfro(v.cpu().numpy(), vw) <= 1e-6
    nu, ns = np.linalg.norm(U.cpu().numpy().astype(np.float64)), np.linalg.norm(S0.astype(np.float64))
    assert abs(nu - ns) <= 1e-6 * ns


def test_rowadam_in_place_and_zero():
    d, r = 1000, 64
    say("rowadam in place / zero")
    S0 = synth.fp32_matrix((d, r), 1.0, (18, 0, 0, 0, 5))
    v0 = np.zeros(d, np.float32)
    S = torch.from_numpy(S0.copy()).to(DEV)
    v = torch.from_numpy(v0.copy()).to(DEV)
    B.rowadam(S, v, 1, 0.95, 1e-8, U=S)
    Uw, _ = oracle.rowadam(S0.astype(np.float64), v0.astype(np.float64), 1, 0.95, 1e-8)
    assert relfro(S.cpu().numpy(), Uw) <= 1e-6
    Z = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    U = B.rowadam(Z, torch.ones(d, device=DEV), 4, 0.95, 1e-8)
    assert torch.count_nonzero(U).item() == 0


# ------------------------------------------------------------ predicted KL


@pytest.mark.parametrize("P,V,dtype,tau", [(4, 512, "f32", 1.0), (64, 152064, "bf16", 1.0), (3, 1000, "bf16", 0.7),
                                           (1, 7, "f32", 2.0), (128, 4099, "bf16", 1.0)])
def test_predicted_kl_q(P, V, dtype, tau):
    say(f"predicted_kl_q P={P} V={V} {dtype} tau={tau}")
    z = synth.normal((P, V), 4.0, (19, P, V, 0, 3), dtype)
    zd = synth.normal((P, V), 1.0, (19, P, V, 0, 4), dtype)
    if dtype == "bf16":
        zt, zdt = bf16_dev(z), bf16_dev(zd)
        z64, zd64 = oracle.bf16_bits_to_f64(z), oracle.bf16_bits_to_f64(zd)
    else:
        zt, zdt = torch.from_numpy(z).to(DEV), torch.from_numpy(zd).to(DEV)
        z64, zd64 = z.astype(np.float64), zd.astype(np.float64)
    q = B.predicted_kl_q(zt, zdt, tau).item()
    qw = oracle.predicted_kl_q(z64, zd64, tau)
    assert abs(q - qw) <= 1e-4 * qw
    a = B.step_alpha_dev(torch.tensor([q], device=DEV), 2e-3, 4.0).item()
    aw = oracle.step_alpha(qw, 2e-3, 4.0)
    assert abs(a - aw) <= 1e-4 * aw


@pytest.mark.parametrize("P,V,dtype,tau", [(4, 512, "f32", 1.0), (64, 152064, "bf16", 1.0), (3, 1000, "bf16", 0.7)])
def test_exact_kl_probe(P, V, dtype, tau):
    """The finite-difference check: the mean exact KL of a step against the oracle's
    (log-softmax difference in fp64), over small and large steps, and alpha^2 q -> KL as the
    step shrinks, with q and the KL both from the GPU ([paper] §2.3 Eq. 5, App. A.1)."""
    say(f"exact KL P={P} V={V} {dtype} tau={tau}")
    zb = synth.normal((P, V), 4.0, (30, P, V, 0, 3), dtype)
    zdb = synth.normal((P, V), 1.0, (30, P, V, 0, 4), dtype)
    if dtype == "bf16":
        z, zd = bf16_dev(zb), bf16_dev(zdb)
        zh, zdh = oracle.bf16_bits_to_f64(zb), oracle.bf16_bits_to_f64(zdb)
    else:
        z, zd = torch.from_numpy(zb).to(DEV), torch.from_numpy(zdb).to(DEV)
        zh, zdh = zb.astype(np.float64), zdb.astype(np.float64)
    for a in (1e-3, 0.05, 1.0, 4.0):
        got = float(B.exact_kl(z, zd, a, tau).item())
        want = oracle.exact_kl_mean(zh, zdh, a, tau)
        assert got == pytest.approx(want, rel=1e-6), a
    q = float(B.predicted_kl_q(z, zd, tau).item())
    a = 1e-3
    assert float(B.exact_kl(z, zd, a, tau).item()) == pytest.approx(a * a * q, rel=2e-2)


def test_predicted_kl_special_cases():
    say("predicted_kl_q special cases")
    P, V = 5, 3000
    z = torch.from_numpy(synth.normal((P, V), 4.0, (20, 0, 0, 0, 3), "f32")).to(DEV)
    q0 = B.predicted_kl_q(z, torch.full((P, V), 3.25, device=DEV), 1.0).item()
    assert abs(q0) <= 1e-7
    zd = synth.normal((1, V), 1.0, (20, 0, 0, 0, 4), "f32")
    qu = B.predicted_kl_q(torch.zeros((1, V), device=DEV), torch.from_numpy(zd).to(DEV), 2.0).item()
    assert abs(qu - zd.astype(np.float64).var() / 8.0) <= 1e-5 * qu


@pytest.mark.parametrize("kind", ["first", "common", "scattered"])
def test_predicted_kl_zdot_offsets(kind):
    """q is a variance, so it must not lose precision when zdot carries a large offset: on the
    first entry of each context, on every entry, or on a few scattered entries.  q within 1e-5
    of the oracle in each case."""
    P, V = 8, 20000
    say(f"predicted_kl_q with zdot offsets ({kind})")
    z = synth.normal((P, V), 4.0, (22, P, V, 0, 3), "f32")
    zd = synth.normal((P, V), 1.0, (22, P, V, 0, 4), "f32").copy()
    if kind == "first":
        zd[:, 0] += 1000.0
    elif kind == "common":
        zd += 10000.0
    else:
        zd[:, ::997] += 300.0
    want = oracle.predicted_kl_q(z.astype(np.float64), zd.astype(np.float64), 1.0)
    got = B.predicted_kl_q(torch.from_numpy(z).to(DEV), torch.from_numpy(zd).to(DEV), 1.0).item()
    assert got == pytest.approx(want, rel=1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_predicted_kl_masked_vocabulary(dtype):
    """Masked vocabulary entries (logit -inf, so probability 0): scattered, a whole leading range
    (several chunks with no finite logit, the case that must not become NaN), and a context with
    a single finite logit (variance 0).  q matches the oracle, through the workspace call and the
    allocation-free one, and so does the exact KL of two steps."""
    P, V = 6, 5000
    say(f"predicted_kl_q masked vocabulary {dtype}")
    z = synth.normal((P, V), 4.0, (21, P, V, 0, 3), "f32").copy()
    zd = synth.normal((P, V), 1.0, (21, P, V, 0, 4), "f32")
    rs = np.random.default_rng(5)
    z[0, rs.random(V) < 0.3] = -np.inf
    z[1, :1800] = -np.inf
    z[2, :] = -np.inf
    z[2, 1234] = 1.5
    z[3, V - 700:] = -np.inf
    if dtype == "bf16":
        zb = torch.from_numpy(z).to(torch.bfloat16)
        zdb = torch.from_numpy(zd).to(torch.bfloat16)
        zh, zdh = zb.float().numpy(), zdb.float().numpy()
        zdev, zddev = zb.to(DEV), zdb.to(DEV)
    else:
        zh, zdh = z, zd
        zdev, zddev = torch.from_numpy(z).to(DEV), torch.from_numpy(zd).to(DEV)
    want = oracle.predicted_kl_q(zh.astype(np.float64), zdh.astype(np.float64), 1.0)
    got = B.predicted_kl_q(zdev, zddev, 1.0).item()
    assert math.isfinite(got) and got == pytest.approx(want, rel=1e-4)
    q = torch.empty((1,), dtype=torch.float32, device=DEV)
    B.predicted_kl_q_noalloc(zdev, zddev, 1.0, q)
    assert q.item() == got
    for a in (1e-3, 0.5):
        kl = float(B.exact_kl(zdev, zddev, a, 1.0).item())
        assert math.isfinite(kl)
        assert kl == pytest.approx(oracle.exact_kl_mean(zh.astype(np.float64), zdh.astype(np.float64), a, 1.0),
                                   rel=1e-6)


def test_step_alpha_device_edges():
    say("step_alpha_dev edges")
    q = torch.tensor([0.0, 8e-3, -1.0], device=DEV)
    assert B.step_alpha_dev(q[0:1], 2e-3, 4.0).item() == 4.0
    assert B.step_alpha_dev(q[1:2], 2e-3, 4.0).item() == pytest.approx(0.5, rel=1e-6)
    assert math.isnan(B.step_alpha_dev(q[2:3], 2e-3, 4.0).item())


# ------------------------------------------------------------ merge


def merge_case(d, k, r, mode, scale, seed_words, ldw=None, row0=0, sr_seed=2, mid=3, step=1):
    ldw = ldw or k
    wbits = synth.normal((d, ldw), 0.02, seed_words + (2,), "bf16")
    U = synth.fp32_matrix((d, r), 1.0, seed_words + (7,))
    W = bf16_dev(wbits)[:, :k]
    Ut = torch.from_numpy(U).to(DEV)
    kk = B.key(1, mid, step)
    B.merge(kk, W, Ut, scale, mode=mode, sr_seed=sr_seed, row0=row0)
    got = bf16_host(W)
    A = oracle.regen_A(1, mid, step, r, k)
    u = philox.sr_draws(sr_seed, mid, step, d, k, row0=row0) if mode == "stochastic" else None
    want = oracle.merge(oracle.bf16_bits_to_f64(wbits[:, :k]), U.astype(np.float64), A, scale,
                        w_dtype="bf16", mode=mode, u_draws=u)
    return got, want, wbits


def ulp_check(got_bits, want_bits):
    g = oracle.bf16_bits_to_f64(got_bits)
    w = oracle.bf16_bits_to_f64(want_bits)
    within = np.abs(g - w) <= oracle.ulp_bf16(w)
    return within.mean(), (got_bits == want_bits).mean()


@pytest.mark.parametrize("d,k,r,mode,ldw", [(256, 256, 8, "nearest", 256), (300, 712, 64, "nearest", 712),
                                            (300, 712, 64, "stochastic", 712), (1000, 3584, 64, "stochastic", 3584),
                                            (130, 5120, 256, "stochastic", 5120), (64, 100, 33, "nearest", 104),
                                            (64, 100, 33, "stochastic", 104), (17, 37 * 8, 1, "stochastic", 296)])
def test_merge_bf16(d, k, r, mode, ldw):
    say(f"merge bf16 d={d} k={k} r={r} {mode} ldw={ldw}")
    # scale chosen so the update is a few bf16 ulps of W (W ~ 0.02, ulp ~ 1e-4)
    got, want, _ = merge_case(d, k, r, mode, 2e-4, (21, d, k, r), ldw=ldw)
    frac, exact = ulp_check(got, want)
    say(f"  within 1 ulp {frac:.6f}, identical {exact:.6f}")
    assert frac >= 0.9999
    assert exact >= 0.999


@pytest.mark.parametrize("r,mode,k", [(64, "nearest", 512), (64, "stochastic", 512), (64, "stochastic", 520),
                                      (256, "nearest", 1024), (256, "stochastic", 1024)])
def test_merge_special_values(r, mode, k):
    """NaN (quiet and signalling, both signs) and infinities in W through the packed merge the
    benchmark times and the fp32-U merge: a NaN becomes the quiet NaN of its sign and an
    infinity stays itself, bit for bit as the oracle rounds them, and every other element meets
    the merge bar.  k = 520 takes the stochastic path for k not a multiple of 16; 256 ranks the
    path whose draws are generated inside the MFMA chain."""
    d = 96
    say(f"merge special values r={r} {mode} k={k}")
    wbits = synth.normal((d, k), 0.02, (41, d, k, r, 2), "bf16").copy()
    specials = np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x7F81, 0xFFA5], np.uint16)
    ii, jj = np.nonzero((np.arange(d)[:, None] * 7 + np.arange(k)[None, :] * 13) % 89 == 0)
    wbits[ii, jj] = specials[np.arange(len(ii)) % len(specials)]
    special = np.zeros((d, k), bool)
    special[ii, jj] = True
    U = synth.fp32_matrix((d, r), 1.0, (41, d, r, 0, 7))
    kk = B.key(2, 9, 1)
    A = oracle.regen_A(2, 9, 1, r, k)
    u = philox.sr_draws(4, 9, 1, d, k) if mode == "stochastic" else None
    want = oracle.merge(oracle.bf16_bits_to_f64(wbits), U.astype(np.float64), A, 3e-4, w_dtype="bf16",
                        mode=mode, u_draws=u)
    W1, W2 = bf16_dev(wbits), bf16_dev(wbits)
    Ud = torch.from_numpy(U).to(DEV)
    B.merge_grouped_packed([(kk, W1, B.pack_update(Ud))], r, 3e-4, mode=mode, sr_seed=4)
    B.merge(kk, W2, Ud, 3e-4, mode=mode, sr_seed=4)
    assert torch.equal(W1.view(torch.int16), W2.view(torch.int16))
    got = bf16_host(W1)
    assert np.array_equal(got[special], want[special])
    frac, exact = ulp_check(got[~special], want[~special])
    assert frac >= 0.9999 and exact >= 0.999


@pytest.mark.parametrize("r,mode", [(64, "nearest"), (64, "stochastic"), (256, "stochastic")])
def test_merge_overflow(r, mode):
    """Weights near the largest finite bf16 and an update of the same size: values past the
    largest finite bf16 go to the infinity of their sign (stochastically: with the probability
    of their fraction of the last gap), as the oracle rounds them; the finite results meet the
    merge bar."""
    d, k = 64, 512
    say(f"merge overflow r={r} {mode}")
    sign = np.where(synth.normal((d, k), 1.0, (45, d, k, r, 1), "f32") < 0, -1.0, 1.0)
    W64 = sign * 3.0e38
    wbits = oracle.f64_to_bf16_rne(W64)
    U = synth.fp32_matrix((d, r), 1.0, (45, d, r, 0, 7))
    kk = B.key(3, 11, 1)
    A = oracle.regen_A(3, 11, 1, r, k)
    u = philox.sr_draws(4, 11, 1, d, k) if mode == "stochastic" else None
    want = oracle.merge(oracle.bf16_bits_to_f64(wbits), U.astype(np.float64), A, 1e38, w_dtype="bf16",
                        mode=mode, u_draws=u)
    W = bf16_dev(wbits)
    B.merge_grouped_packed([(kk, W, B.pack_update(torch.from_numpy(U).to(DEV)))], r, 1e38, mode=mode,
                           sr_seed=4)
    got = bf16_host(W)
    inf = np.isinf(oracle.bf16_bits_to_f64(want))
    say(f"  {inf.mean():.3f} of the results overflow")
    assert 0.05 < inf.mean() < 0.95
    # where the oracle overflows: the same infinity, but for the rare element whose fp32 update
    # (rounded once before the bf16 rounding) falls on the other side of the last decision
    assert (got[inf] == want[inf]).mean() >= 0.999
    frac, exact = ulp_check(got[~inf], want[~inf])
    assert frac >= 0.9999 and exact >= 0.999


@pytest.mark.parametrize("r,mode", [(64, "nearest"), (64, "stochastic"), (33, "nearest"), (256, "stochastic")])
def test_merge_grouped_equals_single_merges(r, mode):
    """One grouped launch over matrices of mixed shapes (full, ragged column and row edges, small)
    gives the bits of separate merges, and each matches the oracle to the merge bar."""
    shapes = [(320, 1024), (100, 712), (64, 3584), (96, 512)]
    say(f"merge grouped r={r} {mode}")
    items, singles, wants = [], [], []
    for i, (d, k) in enumerate(shapes):
        wb, W64 = bf16_inputs((d, k), 0.02, (19, d, k, i, 2))
        U = synth.fp32_matrix((d, r), 1.0, (19, d, r, i, 7))
        kk = B.key(11, 40 + i, 3)
        W1 = bf16_dev(wb)
        W2 = W1.clone()
        Ud = torch.from_numpy(U).to(DEV)
        items.append((kk, W1, Ud))
        singles.append((kk, W2, Ud))
        A = oracle.regen_A(11, 40 + i, 3, r, k)
        u = philox.sr_draws(5, 40 + i, 3, d, k) if mode == "stochastic" else None
        wants.append(oracle.merge(W64, U.astype(np.float64), A, 2e-4, w_dtype="bf16", mode=mode,
                                  u_draws=u))
    B.merge_grouped(items, 2e-4, mode=mode, sr_seed=5)
    for kk, W2, Ud in singles:
        B.merge(kk, W2, Ud, 2e-4, mode=mode, sr_seed=5)
    for (_, W1, _), (_, W2, _), want in zip(items, singles, wants):
        assert torch.equal(W1.view(torch.int16), W2.view(torch.int16))
        frac, exact = ulp_check(bf16_host(W1), want)
        assert frac >= 0.9999 and exact >= 0.999


def packed_update_reference(U: np.ndarray, r: int) -> np.ndarray:
    """The documented packed-update layout built on the host: per 32-row band and 16-rank
    step (steps padded to a power of two), a hi slab then a lo slab of 64 lanes x 8 bf16,
    lane l holding row 32g + (l & 31), ranks 16s + 8(l >> 5) + i."""
    d = U.shape[0]
    ks = 1
    while 16 * ks < r:
        ks *= 2
    nb = (d + 31) // 32
    Up = np.zeros((nb * 32, 16 * ks), np.float32)
    Up[:d, :r] = U
    hi = torch.from_numpy(Up).to(torch.bfloat16)
    lo = (torch.from_numpy(Up) - hi.float()).to(torch.bfloat16)
    out = []
    for t in (hi, lo):
        bits = t.view(torch.int16).numpy().view(np.uint16).reshape(nb, 32, ks, 2, 8)
        # [band, row, step, half, i] -> [band, step, half, row, i]
        out.append(bits.transpose(0, 2, 3, 1, 4).reshape(nb, ks, 64, 8))
    return np.stack(out, axis=2).reshape(-1)          # [band, step, hi/lo, lane, i]


@pytest.mark.parametrize("d,r", [(100, 33), (64, 64), (1000, 256), (7, 1), (300, 130)])
def test_pack_update_layout_and_rowadam_packed(d, r):
    """pack_update writes the documented operand layout; rowadam_packed writes the packed form of
    the U that rowadam computes (same v as well)."""
    say(f"packed update d={d} r={r}")
    U = synth.fp32_matrix((d, r), 1.0, (26, d, r, 0, 7))
    P = B.pack_update(torch.from_numpy(U).to(DEV))
    assert np.array_equal(P.cpu().numpy().view(np.uint16), packed_update_reference(U, r))
    S = torch.from_numpy(synth.fp32_matrix((d, r), 0.3, (26, d, r, 0, 5))).to(DEV)
    v0 = torch.from_numpy(np.abs(synth.fp32_matrix((d, 1), 0.1, (26, d, 0, 0, 6)))[:, 0].copy()).to(DEV)
    v1, v2 = v0.clone(), v0.clone()
    Uf = B.rowadam(S, v1, 3, 0.95, 1e-8)
    Pk = B.rowadam_packed(S, v2, 3, 0.95, 1e-8)
    assert torch.equal(v1.view(torch.int32), v2.view(torch.int32))
    assert torch.equal(Pk, B.pack_update(Uf))


@pytest.mark.parametrize("r", [64, 100, 256])
def test_rowadam_packed_grouped_equals_single_calls(r):
    """One grouped RowAdam over sketches of mixed heights gives every sketch the v and packed
    update bits of its own rowadam_packed call, and U within 1e-6 of the oracle."""
    ds = [3584, 512, 17, 1000, 33, 18944]
    say(f"rowadam grouped r={r}")
    t, beta, eps = 3, 0.95, 1e-8
    items, singles, host = [], [], []
    for i, d in enumerate(ds):
        S = torch.from_numpy(synth.fp32_matrix((d, r), 0.1, (38, d, r, i, 0))).to(DEV)
        v0 = np.abs(synth.fp32_matrix((d, 1), 0.01, (38, d, r, i, 1)))[:, 0].astype(np.float32)
        nb = B.packed_update_bytes(d, r)
        P1 = torch.full((nb // 4,), float("nan"), device=DEV).view(torch.uint8)
        P2 = torch.full((nb // 4,), float("nan"), device=DEV).view(torch.uint8)
        v1, v2 = torch.from_numpy(v0.copy()).to(DEV), torch.from_numpy(v0.copy()).to(DEV)
        items.append((S, v1, P1))
        singles.append((S, v2, P2))
        host.append((S.cpu().numpy(), v0))
    B.rowadam_packed_grouped(items, r, t, beta, eps)
    for S, v2, P2 in singles:
        B.rowadam_packed(S, v2, t, beta, eps, out=P2)
    for (_, v1, P1), (_, v2, P2) in zip(items, singles):
        assert torch.equal(v1.view(torch.int32), v2.view(torch.int32))
        assert torch.equal(P1, P2)
    # the oracle, through the fp32 U of a single call on the first and last sketch
    for i in (0, len(ds) - 1):
        S_h, v0 = host[i]
        U = torch.empty((ds[i], r), dtype=torch.float32, device=DEV)
        B.rowadam(torch.from_numpy(S_h).to(DEV), torch.from_numpy(v0.copy()).to(DEV), t, beta, eps, U=U)
        want, _ = oracle.rowadam(S_h.astype(np.float64), v0.astype(np.float64), t, beta, eps)
        assert relfro(U.cpu().numpy(), want) <= 1e-6
        assert torch.equal(items[i][2], B.pack_update(U))


@pytest.mark.parametrize("r,mode", [(64, "nearest"), (64, "stochastic"), (33, "stochastic"), (8, "nearest"),
                                    (8, "stochastic"), (20, "stochastic"), (100, "nearest"),
                                    (128, "stochastic"), (256, "stochastic"), (256, "nearest")])
def test_merge_grouped_packed_equals_fp32_update(r, mode):
    """The merge from a packed update gives the bits of the merge from the fp32 U it was packed
    from, over full, ragged-row, ragged-column and small matrices in one grouped launch."""
    shapes = [(320, 1024), (100, 712), (64, 3584), (96, 512), (1000, 1280)]
    say(f"merge grouped packed r={r} {mode}")
    items_p, items_u = [], []
    for i, (d, k) in enumerate(shapes):
        wb, _ = bf16_inputs((d, k), 0.02, (27, d, k, i, 2))
        U = torch.from_numpy(synth.fp32_matrix((d, r), 1.0, (27, d, r, i, 7))).to(DEV)
        kk = B.key(13, 50 + i, 2)
        W1 = bf16_dev(wb)
        items_u.append((kk, W1, U))
        items_p.append((kk, W1.clone(), B.pack_update(U)))
    alpha = torch.tensor([0.75], dtype=torch.float32, device=DEV)
    B.merge_grouped(items_u, 3e-4, scale_dev=alpha, mode=mode, sr_seed=9)
    B.merge_grouped_packed(items_p, r, 3e-4, scale_dev=alpha, mode=mode, sr_seed=9)
    for (_, W1, _), (_, W2, _) in zip(items_u, items_p):
        assert torch.equal(W1.view(torch.int16), W2.view(torch.int16))


@pytest.mark.parametrize("r,mode", [(64, "stochastic"), (33, "nearest"), (100, "stochastic"),
                                    (256, "stochastic"), (16, "stochastic"), (32, "stochastic")])
def test_sync_payload_trainer_and_rollout_agree(r, mode):
    """Policy sync ([paper] §2.2): the trainer packs fl32(alpha eta U) once; its own merge from the
    payload and the rollout side's sync_apply give identical weights, and both match the oracle's
    merge with the same update to the merge bar."""
    shapes = [(320, 1024), (100, 712), (64, 512)]
    say(f"sync payload r={r} {mode}")
    alpha = torch.tensor([0.6], dtype=torch.float32, device=DEV)
    trainer, rollout, host = [], [], []
    for i, (d, k) in enumerate(shapes):
        wb, W64 = bf16_inputs((d, k), 0.02, (29, d, k, i, 2))
        U = synth.fp32_matrix((d, r), 1.0, (29, d, r, i, 7))
        kk = B.key(17, 60 + i, 4)
        h, P = B.sync_pack(kk, (d, k), torch.from_numpy(U).to(DEV), 5e-4, scale_dev=alpha, mode=mode,
                           sr_seed=3)
        assert (h.magic, h.version, h.d, h.k, h.r, h.payload_bytes) == (0x4C475253, 1, d, k, r,
                                                                        B.packed_update_bytes(d, r))
        trainer.append((kk, bf16_dev(wb), P))
        rollout.append((h, P, bf16_dev(wb)))
        host.append((i, d, k, W64, U))
    B.merge_grouped_packed(trainer, r, 1.0, mode=mode, sr_seed=3)
    B.sync_apply(rollout)
    for (_, W1, _), (_, _, W2), (i, d, k, W64, U) in zip(trainer, rollout, host):
        assert torch.equal(W1.view(torch.int16), W2.view(torch.int16))
        A = oracle.regen_A(17, 60 + i, 4, r, k)
        u = philox.sr_draws(3, 60 + i, 4, d, k) if mode == "stochastic" else None
        want = oracle.merge(W64, U.astype(np.float64), A, 5e-4 * 0.6, w_dtype="bf16", mode=mode, u_draws=u)
        frac, exact = ulp_check(bf16_host(W2), want)
        assert frac >= 0.9999 and exact >= 0.999


def test_merge_rollout_sync_invariant_and_row_blocks():
    """Two merges of equal W with equal (U, key, scale, mode, sr_seed) are bit-identical;
    merging a row block with its global row offset equals the same rows of the whole merge."""
    d, k, r = 700, 1024, 64
    say("merge determinism / row blocks")
    wbits = synth.normal((d, k), 0.02, (22, 0, 0, 0, 2), "bf16")
    U = torch.from_numpy(synth.fp32_matrix((d, r), 1.0, (22, 0, 0, 0, 7))).to(DEV)
    kk = B.key(9, 5, 2)
    outs = []
    for mode in ("nearest", "stochastic"):
        W1, W2 = bf16_dev(wbits), bf16_dev(wbits)
        B.merge(kk, W1, U, 3e-4, mode=mode, sr_seed=77)
        B.merge(kk, W2, U, 3e-4, mode=mode, sr_seed=77)
        assert torch.equal(W1.view(torch.int16), W2.view(torch.int16))
        W3 = bf16_dev(wbits)
        for a, b in ((0, 100), (100, 333), (333, 700)):
            B.merge(kk, W3[a:b], U[a:b], 3e-4, mode=mode, sr_seed=77, row0=a)
        assert torch.equal(W1.view(torch.int16), W3.view(torch.int16))
        outs.append(W1)
    assert not torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_merge_zero_update_and_device_scale():
    d, k, r = 200, 512, 64
    say("merge zero update / device scale")
    wbits = synth.normal((d, k), 0.02, (23, 0, 0, 0, 2), "bf16")
    kk = B.key(3, 1, 0)
    for mode in ("nearest", "stochastic"):
        W = bf16_dev(wbits)
        B.merge(kk, W, torch.zeros((d, r), device=DEV), 1.0, mode=mode, sr_seed=5)
        assert np.array_equal(bf16_host(W), wbits)
        W = bf16_dev(wbits)
        B.merge(kk, W, torch.ones((d, r), device=DEV), 0.0, mode=mode, sr_seed=5)
        assert np.array_equal(bf16_host(W), wbits)
    U = torch.from_numpy(synth.fp32_matrix((d, r), 1.0, (23, 0, 0, 0, 7))).to(DEV)
    W1, W2 = bf16_dev(wbits), bf16_dev(wbits)
    B.merge(kk, W1, U, 2.5e-4, mode="stochastic", sr_seed=5)
    B.merge(kk, W2, U, 1e-3, scale_dev=torch.tensor([0.25], device=DEV), mode="stochastic", sr_seed=5)
    assert torch.equal(W1.view(torch.int16), W2.view(torch.int16))


def test_merge_fp32_unit_factor_and_values():
    """fp32 W: U = e_i e_j^T, scale = -1 on W = 0 writes row j of A into row i;
    general values match the oracle's fp32 rounding."""
    d, k, r = 6, 600, 8
    say("merge fp32")
    kk = B.key(5, 9, 2)
    A32 = B.regen_A(kk, r, k, torch.float32, DEV)
    for i, j in ((0, 0), (4, 7), (5, 3)):
        W = torch.zeros((d, k), dtype=torch.float32, device=DEV)
        U = torch.zeros((d, r), dtype=torch.float32, device=DEV)
        U[i, j] = 1.0
        B.merge(kk, W, U, -1.0)
        assert torch.equal(W[i].view(torch.int32), A32[j].view(torch.int32))
        assert torch.count_nonzero(W).item() == torch.count_nonzero(A32[j]).item()
    d, k, r = 256, 256, 8
    W0 = synth.normal((d, k), 0.02, (24, 0, 0, 0, 2), "f32")
    U0 = synth.fp32_matrix((d, r), 1.0, (24, 0, 0, 0, 7))
    W = torch.from_numpy(W0.copy()).to(DEV)
    B.merge(B.key(1, 0, 0), W, torch.from_numpy(U0).to(DEV), 1e-3)
    want = oracle.merge(W0.astype(np.float64), U0.astype(np.float64), oracle.regen_A(1, 0, 0, r, k), 1e-3,
                        w_dtype="f32")
    got = W.cpu().numpy()
    assert (got == want).mean() >= 0.999
    assert np.max(np.abs(got.astype(np.float64) - want) / np.spacing(np.abs(want))) <= 1.0


def test_merge_fp32_special_values():
    """fp32 W with NaN (quiet and signalling, both signs) and infinities: each infinity stays
    itself, each NaN stays a NaN of its sign, and every other element matches the oracle's fp32
    rounding as in the test above."""
    d, k, r = 96, 512, 8
    say("merge fp32 special values")
    W0 = synth.normal((d, k), 0.02, (25, 0, 0, 0, 2), "f32").copy()
    specials = np.array([0x7FC00000, 0xFFC00000, 0x7F800000, 0xFF800000, 0x7F800123, 0xFFA00001],
                        np.uint32).view(np.float32)
    ii, jj = np.nonzero((np.arange(d)[:, None] * 7 + np.arange(k)[None, :] * 13) % 89 == 0)
    W0[ii, jj] = specials[np.arange(len(ii)) % len(specials)]
    special = np.zeros((d, k), bool)
    special[ii, jj] = True
    U0 = synth.fp32_matrix((d, r), 1.0, (25, 0, 0, 0, 7))
    W = torch.from_numpy(W0.copy()).to(DEV)
    B.merge(B.key(1, 0, 0), W, torch.from_numpy(U0).to(DEV), 1e-3)
    with np.errstate(invalid="ignore"):
        want = oracle.merge(W0.astype(np.float64), U0.astype(np.float64), oracle.regen_A(1, 0, 0, r, k), 1e-3,
                            w_dtype="f32")
    got = W.cpu().numpy()
    nan = special & np.isnan(W0)
    assert np.all(np.isnan(got[nan])) and np.array_equal(np.signbit(got[nan]), np.signbit(W0[nan]))
    inf = special & np.isinf(W0)
    assert np.array_equal(got[inf], W0[inf])
    rest = ~special
    assert (got[rest] == want[rest]).mean() >= 0.999
    assert np.max(np.abs(got[rest].astype(np.float64) - want[rest]) / np.spacing(np.abs(want[rest]))) <= 1.0


# ------------------------------------------------ reconstruction cosine


@pytest.mark.parametrize("d,k,r,dtype,ld", [(64, 256, 8, "bf16", 256), (300, 712, 33, "bf16", 720),
                                            (1000, 1536, 64, "bf16", 1536), (517, 1536, 256, "bf16", 1536),
                                            (40, 300, 5, "f32", 304), (18944, 3584, 64, "bf16", 3584)])
def test_reconstruction_cosine(d, k, r, dtype, ld):
    """cos(G, (G A^T) A) and its parts against the oracle's direct definition ([paper] App. D.3);
    the last case is a 7B gate-projection gradient at full size."""
    say(f"reconstruction cosine d={d} k={k} r={r} {dtype}")
    bits_or_x = synth.normal((d, ld), 0.01, (28, d, k, r, 1), dtype)
    if dtype == "bf16":
        G = bf16_dev(bits_or_x)[:, :k]
        Gh = oracle.bf16_bits_to_f64(bits_or_x)[:, :k]
    else:
        G = torch.from_numpy(bits_or_x).to(DEV)[:, :k]
        Gh = bits_or_x[:, :k].astype(np.float64)
    out = B.reconstruction_cosine(B.key(4, 9, 1), G, r).cpu().numpy()
    A = oracle.regen_A(4, 9, 1, r, k)
    want = oracle.reconstruction_cosine(Gh, A)
    S = Gh @ A.T
    say(f"  cos {out[0]:.6f} oracle {want:.6f}")
    assert out[0] == pytest.approx(want, rel=1e-5)
    assert out[1] == pytest.approx((Gh * Gh).sum(), rel=1e-12)
    assert out[2] == pytest.approx((S * S).sum(), rel=1e-5)
    assert out[3] == pytest.approx(((S @ A) ** 2).sum(), rel=1e-5)


# ------------------------------------------------ Gaussian projection variant


@pytest.mark.parametrize("r,k", [(64, 3584), (33, 700), (256, 1536), (5, 40)])
def test_gaussian_projection(r, k):
    """The Gaussian variant: A from Box-Muller on the Philox stream against the oracle's (device
    and host libm may differ in the last fp64 bit, so fp32 A is compared within one ulp); the
    projection with the packed explicit A against the oracle's X A^T; its packed output feeding
    the accumulate; and the reconstruction cosine with Gaussian A against the oracle's."""
    say(f"gaussian projection r={r} k={k}")
    kk = B.key(6, 11, 2)
    A = B.regen_A_gaussian(kk, r, k, DEV)
    Ah = A.cpu().numpy()
    want = oracle.gaussian_A(6, 11, 2, r, k, kind="f32")
    assert np.all(np.abs(Ah.astype(np.float64) - want) <= np.spacing(np.abs(want)))
    assert (Ah == want).mean() >= 0.999
    A64 = oracle.gaussian_A(6, 11, 2, r, k)
    Ap = B.pack_projection(A)
    T, ld = 1000, (k + 7) // 8 * 8
    xb, X = bf16_inputs((T, ld), 1.0, (31, T, k, r, 0))
    planes = torch.empty((B.packed_input_bytes(T, r),), dtype=torch.uint8, device=DEV)
    XAt, _ = B.project_input_explicit(bf16_dev(xb)[:, :k], Ap, r, planes=planes)
    want_x = oracle.project(X[:, :k], A64)
    assert relfro(XAt.cpu().numpy(), want_x) <= 1e-5
    d, ldd = 300, 304
    db, Dm = bf16_inputs((T, ldd), 1e-3, (31, T, d, r, 1))
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    B.sketch_accumulate_grouped_packed([(bf16_dev(db)[:, :d], planes, S)], r)
    assert relfro(S.cpu().numpy(), Dm[:, :d].T @ want_x) <= 5e-5
    gb, Gh = bf16_inputs((512, ld), 0.01, (31, 512, k, r, 2))
    out = B.reconstruction_cosine_explicit(bf16_dev(gb)[:, :k], A, Ap).cpu().numpy()
    assert out[0] == pytest.approx(oracle.reconstruction_cosine(Gh[:, :k], A64), rel=1e-5)


@pytest.mark.parametrize("r,mode", [(64, "nearest"), (64, "stochastic"), (33, "nearest"), (256, "stochastic")])
def test_gaussian_merge(r, mode):
    """The merge with the Gaussian projection (explicit A in the merge's operand order) against the
    oracle's W - s U A with the same A, over full, ragged-row and ragged-column matrices."""
    shapes = [(320, 1024), (100, 712), (64, 3584)]
    say(f"gaussian merge r={r} {mode}")
    items, host = [], []
    for i, (d, k) in enumerate(shapes):
        wb, W64 = bf16_inputs((d, k), 0.02, (32, d, k, i, 2))
        U = synth.fp32_matrix((d, r), 1.0, (32, d, r, i, 7))
        kk = B.key(8, 70 + i, 1)
        A = B.regen_A_gaussian(kk, r, k, DEV)
        items.append((kk, bf16_dev(wb), B.pack_update(torch.from_numpy(U).to(DEV)), B.pack_merge_projection(A)))
        host.append((i, d, k, W64, U))
    B.merge_grouped_explicit(items, r, 3e-4, mode=mode, sr_seed=4)
    for (_, W, _, _), (i, d, k, W64, U) in zip(items, host):
        A64 = oracle.gaussian_A(8, 70 + i, 1, r, k)
        u = philox.sr_draws(4, 70 + i, 1, d, k) if mode == "stochastic" else None
        want = oracle.merge(W64, U.astype(np.float64), A64, 3e-4, w_dtype="bf16", mode=mode, u_draws=u)
        frac, exact = ulp_check(bf16_host(W), want)
        assert frac >= 0.9999 and exact >= 0.999


@pytest.mark.parametrize("mode", ["nearest", "stochastic"])
def test_gaussian_merge_special_values(mode):
    """NaN and infinities in W through the merge with an explicit (Gaussian) projection: a NaN
    becomes the quiet NaN of its sign and an infinity stays itself, bit for bit as the oracle
    rounds them; every other element meets the merge bar."""
    d, k, r = 96, 512, 64
    say(f"gaussian merge special values {mode}")
    wbits = synth.normal((d, k), 0.02, (43, d, k, r, 2), "bf16").copy()
    specials = np.array([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x7F81, 0xFFA5], np.uint16)
    ii, jj = np.nonzero((np.arange(d)[:, None] * 5 + np.arange(k)[None, :] * 11) % 83 == 0)
    wbits[ii, jj] = specials[np.arange(len(ii)) % len(specials)]
    special = np.zeros((d, k), bool)
    special[ii, jj] = True
    U = synth.fp32_matrix((d, r), 1.0, (43, d, r, 0, 7))
    kk = B.key(8, 77, 1)
    A = B.regen_A_gaussian(kk, r, k, DEV)
    W = bf16_dev(wbits)
    B.merge_grouped_explicit([(kk, W, B.pack_update(torch.from_numpy(U).to(DEV)), B.pack_merge_projection(A))],
                             r, 3e-4, mode=mode, sr_seed=4)
    u = philox.sr_draws(4, 77, 1, d, k) if mode == "stochastic" else None
    want = oracle.merge(oracle.bf16_bits_to_f64(wbits), U.astype(np.float64), oracle.gaussian_A(8, 77, 1, r, k),
                        3e-4, w_dtype="bf16", mode=mode, u_draws=u)
    got = bf16_host(W)
    assert np.array_equal(got[special], want[special])
    frac, exact = ulp_check(got[~special], want[~special])
    assert frac >= 0.9999 and exact >= 0.999


# ------------------------------------------------------ whole update


@pytest.mark.parametrize("workload", ["single-256-r8-fp32", "single-4096-r64"])
def test_whole_update_matches_oracle(workload):
    """One whole update of a small workload, every step on the GPU through the C ABI: the
    projection of each microbatch's input, the sketch over all microbatches, the optimiser
    (SGD U = S, or RowAdam from v = 0 at t = 1), q and alpha where the workload has contexts,
    and the merge -- against the oracle's chain on the same inputs ([paper] §2.1-2.3)."""
    w = synth.BY_NAME[workload]
    (layer, kind, mid, d, k) = w.matrices()[0]
    T, r = w.T, w.r
    bf16 = w.dtype == "bf16"
    say(f"whole update of {workload}")
    kk = B.key(w.seed, mid, w.step)
    A = oracle.regen_A(w.seed, mid, w.step, r, k)
    S = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    S_h = np.zeros((d, r))
    for mb in range(w.microbatches):
        xb = synth.layer_input(w, layer, kind, mb)
        db = synth.output_grad(w, layer, kind, mb)
        if bf16:
            X, D = bf16_dev(xb), bf16_dev(db)
            Xh, Dh = oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(db)
        else:
            X, D = torch.from_numpy(xb).to(DEV), torch.from_numpy(db).to(DEV)
            Xh, Dh = xb.astype(np.float64), db.astype(np.float64)
        B.sketch_accumulate(D, B.project_input(kk, X, r), S)
        S_h = oracle.accumulate(S_h, Dh, oracle.project(Xh, A))
    assert relfro(S.cpu().numpy(), S_h) <= (5e-5 if bf16 else 1e-5)
    if w.optimizer == "sgd":
        U, U_h = S, S_h
    else:
        v = torch.zeros((d,), dtype=torch.float32, device=DEV)
        U = B.rowadam(S, v, 1, w.beta, w.eps)
        U_h, _ = oracle.rowadam(S_h, np.zeros(d), 1, w.beta, w.eps)
        assert relfro(U.cpu().numpy(), U_h) <= 5e-5
    alpha = w.alpha
    if w.P:
        zb, zdb = synth.kl_inputs(w)
        zt = torch.from_numpy(zb).to(DEV) if not bf16 else bf16_dev(zb)
        zdt = torch.from_numpy(zdb).to(DEV) if not bf16 else bf16_dev(zdb)
        q = float(B.predicted_kl_q(zt, zdt, w.tau).item())
        zh = zb.astype(np.float64) if not bf16 else oracle.bf16_bits_to_f64(zb)
        zdh = zdb.astype(np.float64) if not bf16 else oracle.bf16_bits_to_f64(zdb)
        q_h = oracle.predicted_kl_q(zh, zdh, w.tau)
        assert q == pytest.approx(q_h, rel=1e-4)
        assert B.step_alpha(q, w.delta, w.alpha_max) == pytest.approx(
            oracle.step_alpha(q_h, w.delta, w.alpha_max), rel=1e-4)
        if alpha is None:
            alpha = oracle.step_alpha(q_h, w.delta, w.alpha_max)
    wb = synth.weight(w, layer, kind)
    W = bf16_dev(wb) if bf16 else torch.from_numpy(wb).to(DEV)
    B.merge(kk, W, U, w.eta * alpha, mode=w.rounding, sr_seed=w.sr_seed)
    Wh = oracle.bf16_bits_to_f64(wb) if bf16 else wb.astype(np.float64)
    u = philox.sr_draws(w.sr_seed, mid, w.step, d, k) if w.rounding == "stochastic" else None
    want = oracle.merge(Wh, U_h, A, w.eta * alpha, w_dtype=w.dtype, mode=w.rounding, u_draws=u)
    if bf16:
        frac, exact = ulp_check(bf16_host(W), want)
        assert frac >= 0.9999 and exact >= 0.999
    else:
        # the chain: the applied update W' - W against the oracle's, relative Frobenius (the
        # oracle's U is fp64, the GPU's fp32, so W' may differ by an ulp where the two round apart)
        got = W.cpu().numpy().astype(np.float64)
        assert relfro(got - Wh, want - Wh) <= 1e-5
        # the merge alone: from the GPU's own U the oracle's W matches bit for bit
        want_u = oracle.merge(Wh, U.cpu().numpy().astype(np.float64), A, w.eta * alpha, w_dtype="f32",
                              mode="nearest")
        assert (got == want_u).mean() >= 0.999


# --------------------------------------------- full-size shapes (sampled)


@pytest.mark.parametrize("workload,layer", [("qwen2.5-7b-set-r64", 0), ("qwen2.5-7b-set-r64", 27),
                                            ("qwen2.5-1.5b-set-r64", 14), ("dense-27b-set-r256", 0),
                                            ("dense-27b-set-r256", 63)])
def test_full_size_layer_sampled(workload, layer):
    """One full-size layer (q, k, v, o, gate, up, down; 1.5B and 7B shapes at r = 64, 27B
    shapes at r = 256; T = 4096; first, middle or last layer, so each matrix has its own key)
    through the single-layer entry points: projections straight into packed operands, one
    grouped packed accumulate, one grouped merge from packed updates with the step size on
    the device.  (The table launches the benchmark times are checked at full size in
    test_gpu_layerset.py.)  S is checked on sampled rows of every matrix against the
    oracle's X A^T and D^T (X A^T); W on sampled rows of every matrix."""
    w = synth.BY_NAME[workload]
    T, r = w.T, w.r
    say(f"full-size layer {layer} of {workload}, sampled (bench configuration)")
    rs = np.random.default_rng(25 + layer)
    items, host = [], []
    for (layer, kind, mid, d, k) in w.matrices(layers=[layer]):
        xb = synth.layer_input(w, layer, kind, 0)
        db = synth.output_grad(w, layer, kind, 0)
        S0 = synth.fp32_matrix((d, r), 0.3, (25, mid, 0, 0, 5))
        kk = B.key(w.seed, mid, w.step)
        planes = B.project_input_packed(kk, bf16_dev(xb), r)
        A = oracle.regen_A(w.seed, mid, w.step, r, k)
        XAt = oracle.project(oracle.bf16_bits_to_f64(xb), A)
        items.append((bf16_dev(db), planes, torch.from_numpy(S0.copy()).to(DEV)))
        host.append((db, XAt, S0, d))
    B.sketch_accumulate_grouped_packed(items, r)
    for (db, XAt, S0, d), (_, _, S) in zip(host, items):
        rows = np.unique(np.concatenate([[0, d - 1], rs.integers(0, d, 48)]))
        Dc = oracle.bf16_bits_to_f64(db[:, rows])
        want = S0[rows].astype(np.float64) + Dc.T @ XAt
        assert relfro(S.cpu().numpy()[rows], want) <= 5e-5
    del items
    # the layer's grouped merge, step size on the device
    alpha = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    mitems, mhost = [], []
    for (layer, kind, mid, d, k) in w.matrices(layers=[layer]):
        wbits = synth.weight(w, layer, kind)
        U = synth.fp32_matrix((d, r), 1.0, (25, mid, 0, 0, 7))
        mitems.append((B.key(w.seed, mid, w.step), bf16_dev(wbits), torch.from_numpy(U).to(DEV)))
        mhost.append((mid, d, k, wbits, U))
    packed = [B.pack_update(U) for (_, _, U) in mitems]
    for mode in ("nearest", "stochastic"):
        Ws = [W.clone() for (_, W, _) in mitems]
        B.merge_grouped_packed([(kk, W2, P) for (kk, _, _), W2, P in zip(mitems, Ws, packed)], r, 1e-3,
                               scale_dev=alpha, mode=mode, sr_seed=w.sr_seed)
        for (mid, d, k, wbits, U), W2 in zip(mhost, Ws):
            rows = np.unique(np.concatenate([[0, d - 1], rs.integers(0, d, 16)]))
            A = oracle.regen_A(w.seed, mid, w.step, r, k)
            u = (np.concatenate([philox.sr_draws(w.sr_seed, mid, w.step, 1, k, row0=int(i)) for i in rows])
                 if mode == "stochastic" else None)
            want = oracle.merge(oracle.bf16_bits_to_f64(wbits[rows]), U[rows].astype(np.float64), A, 5e-4,
                                w_dtype="bf16", mode=mode, u_draws=u)
            frac, exact = ulp_check(bf16_host(W2)[rows], want)
            assert frac >= 0.9999 and exact >= 0.999
