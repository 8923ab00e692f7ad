"""GPU parity of the launches that keep partial sums in a workspace against
the CPU oracle: stream-K (tiles flagged TILE_STREAMK, asked for with
FLAG_STREAMK) and split-K of the few-rows skinny tiles; and the workspace
cache itself (streams, growth, release, graph capture).

Stream-K cuts the k-steps of the last waves' tiles into 256 equal runs; a
tile touched by several runs is summed by a second launch from partial sums.
The shapes below make every case of that split happen: all tiles split (few
tiles), whole waves before the split ones (more than 512 tiles), a tile cut
into hundreds of one-step pieces, K under one step (nothing split), and
M, N, K that are not tile multiples (each stays a multiple of 4: stream-K
takes operands whose stored rows allow 16-byte loads).  Integer-valued
inputs must match the oracle bit for bit (every partial sum is exact in
fp32, so the split cannot change them); random inputs are held to the
tolerance in parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest

import fp32_sgemm_02_amd as sg
import workloads
from parity import epilogue_err_ratio, max_err_ratio, sample_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32 = np.float32
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def sk_tiles(trans_a):
    out = []
    for t in range(sg.tile_count(sg.VARIANT_MFMA)):
        d = sg.tile_info(sg.VARIANT_MFMA, t)
        if d["flags"] & sg.TILE_STREAMK and bool(d["flags"] & sg.TILE_TRANS_A) == trans_a:
            out.append(t)
    return out


def stored(A, B, trans_a, trans_b):
    return (np.ascontiguousarray(A.T) if trans_a else A,
            np.ascontiguousarray(B.T) if trans_b else B)


def run(As, Bs, C0, alpha, beta, ta, tb, tile, rows=None, **kw):
    M = As.shape[1] if ta else As.shape[0]
    N = Bs.shape[0] if tb else Bs.shape[1]
    C = dev(C0) if C0 is not None else torch.full((M, N), float("nan"), device=DEV)
    sg.gemm(dev(As), dev(Bs), C, alpha, beta, trans_a=ta, trans_b=tb, variant=sg.VARIANT_MFMA,
            tile=tile, flags=sg.FLAG_STREAMK, **kw)
    torch.cuda.synchronize()
    out = C.cpu().numpy()
    return out if rows is None else out[rows]


def oracle_rows(oracle_mod, As, Bs, C0, alpha, beta, ta, tb, rows, **kw):
    Ar = np.ascontiguousarray(As[:, rows] if ta else As[rows])
    Cr = None if C0 is None else np.ascontiguousarray(C0[rows])
    return oracle_mod.sgemm(Ar, Bs, Cr, alpha, beta if C0 is not None else 0.0, trans_a=ta,
                            trans_b=tb, **kw)


def shapes_for(tile):
    d = sg.tile_info(sg.VARIANT_MFMA, tile)
    bm, bn, bk = d["bm"], d["bn"], d["bk"]
    return bk, [
        (3 * bm + 4, 2 * bn - 4, 3004),        # 6 tiles, each cut into ~43 pieces
        (bm, bn, 250 * bk),                    # one tile, 250 one-step pieces
        (5 * bm - 8, 3 * bn + 12, 40 * bk + 4),  # ragged, a few pieces a tile
        (2 * bm, 2 * bn, 4),                   # K under one step: no tile is split
        (17 * bm, 16 * bn + 8, 64),            # 289 tiles: one split wave of 289
        (24 * bm, 24 * bn, 2 * bk + 4),        # 576 tiles: 256 whole, 320 split
    ]


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("trans_a", [False, True])
def test_streamk_tiles(trans_a, trans_b, oracle_mod):
    """Every stream-K tile, B either way (A as the tile serves it): random
    inputs with alpha/beta and beta = 0 over a NaN C within tolerance,
    integer inputs bit-exact; large shapes on sampled rows."""
    tiles = sk_tiles(trans_a)
    if not tiles:
        pytest.skip("no stream-K tile for this A")
    for tile in tiles:
        bk, shapes = shapes_for(tile)
        for i, (M, N, K) in enumerate(shapes):
            lab = f"sk t{tile} ta={trans_a} tb={trans_b} {(M, N, K)}"
            print(lab, flush=True)
            rows = sample_rows(M, 40) if M * N > 2_000_000 else np.arange(M)
            A, B, C0 = workloads.draw(M, N, K, "uniform", 2100 + i, True)
            As, Bs = stored(A, B, trans_a, trans_b)
            got = run(As, Bs, C0, 0.5, -1.25, trans_a, trans_b, tile, rows)
            ref = oracle_rows(oracle_mod, As, Bs, C0, 0.5, -1.25, trans_a, trans_b, rows)
            r = max_err_ratio(got, ref, K, 0.5, -1.25, As, Bs, C0[rows])
            assert r <= 1.0, f"{lab}: max err/tol = {r}"
            got = run(As, Bs, None, 1.0, 0.0, trans_a, trans_b, tile, rows)
            ref = oracle_rows(oracle_mod, As, Bs, None, 1.0, 0.0, trans_a, trans_b, rows)
            r = max_err_ratio(got, ref, K, 1.0, 0.0, As, Bs, None)
            assert r <= 1.0, f"{lab} b0: max err/tol = {r}"
            Ai, Bi, Ci = workloads.draw(M, N, K, "int4", 2200 + i, True)
            Ai, Bi = stored(Ai, Bi, trans_a, trans_b)
            got = run(Ai, Bi, Ci, 0.5, -1.25, trans_a, trans_b, tile, rows)
            ref = oracle_rows(oracle_mod, Ai, Bi, Ci, 0.5, -1.25, trans_a, trans_b, rows)
            assert np.array_equal(got, ref), f"{lab} int: not bit-exact"


def test_streamk_repeatable_and_epilogue(oracle_mod):
    """Two stream-K calls give the same bits; bias + GELU after stream-K (the
    elementwise pass) within the epilogue tolerance."""
    tiles = sk_tiles(False)
    if not tiles:
        pytest.skip("no stream-K tile")
    tile = tiles[0]
    M, N, K = 700, 900, 4004
    A, B, C0 = workloads.draw(M, N, K, "uniform", 2300, True)
    c1 = run(A, B, C0, 1.0, 0.5, False, False, tile)
    c2 = run(A, B, C0, 1.0, 0.5, False, False, tile)
    assert np.array_equal(c1, c2), "stream-K results differ between calls"
    bias = np.random.default_rng(2301).uniform(-1, 1, N).astype(F32)
    Bs = np.ascontiguousarray(B.T)
    got = run(A, Bs, C0, 1.0, 0.5, False, True, tile, bias=dev(bias), act=sg.ACT_GELU_ERF)
    ref = oracle_mod.sgemm(A, Bs, C0.copy(), 1.0, 0.5, trans_b=True, bias=bias,
                           act=sg.ACT_GELU_ERF)
    x = oracle_mod.sgemm(A, Bs, C0.copy(), 1.0, 0.5, trans_b=True, bias=bias)
    r = epilogue_err_ratio(got, ref, x, K, 1.0, 0.5, A, Bs, C0, bias, sg.ACT_GELU_ERF)
    assert r <= 1.0, f"stream-K + GELU: max err/tol = {r}"


def test_streamk_rejected_configs():
    """FLAG_STREAMK without a stream-K tile, with 4-byte I/O, or for A rows
    that cannot take 16-byte loads is an invalid configuration (-13)."""
    tiles = sk_tiles(False)
    if not tiles:
        pytest.skip("no stream-K tile")
    plain = [t for t in range(sg.tile_count(sg.VARIANT_MFMA))
             if not sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_STREAMK]
    A = torch.zeros((256, 258), device=DEV)
    B = torch.zeros((258, 256), device=DEV)
    C = torch.zeros((256, 256), device=DEV)
    for tile, flags, a in ((plain[0], sg.FLAG_STREAMK, A[:, :256]),
                           (tiles[0], sg.FLAG_STREAMK | sg.FLAG_SCALAR_IO, A[:, :256]),
                           (tiles[0], sg.FLAG_STREAMK, A[:, :255])):
        K = a.shape[1]
        with pytest.raises(sg.SgemmError) as e:
            sg.gemm(a, B[:K], C, variant=sg.VARIANT_MFMA, tile=tile, flags=flags)
        assert e.value.status == -13
    with pytest.raises(sg.SgemmError):
        sg.gemm(A[:, :256], B[:256], C, flags=sg.FLAG_STREAMK)   # no explicit tile


@pytest.mark.parametrize("ta,tb,shape", [(False, False, (1536, 1536, 8192)),
                                         (False, True, (768, 768, 65536)),
                                         (True, False, (3000, 3000, 3000))])
def test_streamk_automatic(ta, tb, shape, oracle_mod):
    """Shapes whose automatic plan is stream-K: the plan reports it, and
    integer inputs match the oracle bit for bit on sampled rows."""
    M, N, K = shape
    cfg = sg.plan(M, N, K, trans_a=ta, trans_b=tb)[0]
    assert cfg.flags & sg.FLAG_STREAMK, f"plan for {shape} is not stream-K"
    A, B, C0 = workloads.draw(M, N, K, "int4", 2400, True)
    As, Bs = stored(A, B, ta, tb)
    dC = dev(C0)
    sg.gemm(dev(As), dev(Bs), dC, 0.5, -1.25, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    rows = sample_rows(M, 24)
    ref = oracle_rows(oracle_mod, As, Bs, C0, 0.5, -1.25, ta, tb, rows)
    assert np.array_equal(dC.cpu().numpy()[rows], ref), f"automatic stream-K {shape}"


def test_streamk_graph_capture():
    """Stream-K calls captured in a HIP graph (workspace taken and returned by
    stream-ordered allocation inside the graph): every replay, with eager
    work and synchronisation between replays, gives the eager call's bits."""
    tiles = sk_tiles(False)
    if not tiles:
        pytest.skip("no stream-K tile")
    M, N, K = 512, 512, 8192
    A, B, C0 = workloads.draw(M, N, K, "uniform", 2500, True)
    dA, dB = dev(A), dev(B)
    cfg = sg.plan(M, N, K)[0]
    assert cfg.flags & sg.FLAG_STREAMK, "plan for 512x512x8192 is not stream-K"
    eager = torch.empty((M, N), device=DEV)
    sg.gemm(dA, dB, eager)
    torch.cuda.synchronize()
    want = eager.cpu().numpy()
    C = torch.empty((M, N), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sg.gemm(dA, dB, C)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        C.fill_(float("nan"))
        sg.gemm(dA, dB, C)
    for r in range(3):
        C.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), want), f"replay {r} differs from the eager call"
        sg.gemm(dA, dB, eager, 1.0, 0.0)   # eager work between replays
        torch.cuda.synchronize()
    del g


def test_workspace_streams_grow_and_release():
    """The cached workspaces: stream-K and split-K calls on two streams at
    once (each stream its own workspace), a larger call after a smaller one
    on the same stream (the workspace grows while earlier work may still
    use the old one), and calls after workspace_release; every result
    matches a call made alone on the default stream, bit for bit."""
    tiles = sk_tiles(False)
    if not tiles:
        pytest.skip("no stream-K tile")
    rng = np.random.default_rng(2600)
    cases = [(512, 512, 8192, dict(variant=sg.VARIANT_MFMA, tile=tiles[0], flags=sg.FLAG_STREAMK)),
             (768, 640, 16384, dict(variant=sg.VARIANT_MFMA, tile=tiles[0], flags=sg.FLAG_STREAMK)),
             (4, 1024, 8192, dict(variant=sg.VARIANT_SKINNY, tile=0, group_m=8)),
             (16, 2048, 16384, dict(variant=sg.VARIANT_SKINNY, tile=2, group_m=16))]
    ops = []
    for M, N, K, kw in cases:
        A = dev(rng.uniform(-1, 1, (M, K)).astype(F32))
        B = dev(rng.uniform(-1, 1, (K, N)).astype(F32))
        ref = torch.empty((M, N), device=DEV)
        sg.gemm(A, B, ref, **kw)
        ops.append((A, B, ref, kw))
    torch.cuda.synchronize()
    want = [r.cpu().numpy() for _, _, r, _ in ops]
    for rnd in range(2):
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        outs = [[torch.full_like(r, float("nan")) for _, _, r, _ in ops] for _ in streams]
        for rep in range(3):
            for si, st in enumerate(streams):
                with torch.cuda.stream(st):
                    # small before large on each stream: the workspace grows in order
                    for (A, B, _, kw), C in zip(ops, outs[si]):
                        sg.gemm(A, B, C, **kw)
        torch.cuda.synchronize()
        for si in range(len(streams)):
            for j, C in enumerate(outs[si]):
                assert np.array_equal(C.cpu().numpy(), want[j]), \
                    f"round {rnd} stream {si} case {cases[j][:3]} differs"
        sg.workspace_release()


SPLIT_CASES = [(1, 1000, 3001, 5), (7, 77, 4097, 0), (16, 2000, 8192, 7), (3, 300, 16384, 0),
               (1, 64, 1024, 3), (2, 4100, 999, 64)]


def rows_tiles():
    return [t for t in range(sg.tile_count(sg.VARIANT_SKINNY))
            if sg.tile_info(sg.VARIANT_SKINNY, t)["tm"] == 0]


def test_workspace_per_thread_default_stream(oracle_mod):
    """Two host threads running split-K plans on the per-thread default stream
    (hipStreamPerThread: one handle value, a different stream on each host
    thread) at the same time, with different workspace sizes: each thread
    keeps its own workspace, and every result matches the oracle bit for bit."""
    import threading

    per_thread = 2   # the handle value of hipStreamPerThread
    cases = [(1, 4096, 4096, 31), (3, 2048, 8192, 32)]
    data = []
    for M, N, K, seed in cases:
        assert sg.plan(M, N, K)[0].group_m > 1, f"{(M, N, K)} is no longer split"
        A, B, _ = workloads.draw(M, N, K, "int4", seed, False)
        data.append((dev(A), dev(B), torch.full((M, N), float("nan"), device=DEV),
                     oracle_mod.sgemm(A, B)))
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            torch.cuda.set_device(0)
            dA, dB, C, _ = data[i]
            for _ in range(20):
                sg.gemm(dA, dB, C, stream=per_thread)
        except Exception as ex:   # reported by the main thread
            errors.append(ex)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(data))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (M, N, K, _), (_, _, C, ref) in zip(cases, data):
        assert np.array_equal(C.cpu().numpy(), ref), f"{(M, N, K)} per-thread stream"


@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False)])
@pytest.mark.parametrize("tile", range(6))
def test_skinny_split_k(tile, ta, tb, oracle_mod):
    """The few-rows tiles split over K (group_m slices, 0: the library's
    choice; partial sums in a workspace, added in slice order by the last
    workgroup of each strip): random inputs with alpha/beta and with bias +
    GELU within tolerance, 4-byte loads, integer inputs bit-exact, and two
    calls give the same bits."""
    if tile >= len(rows_tiles()):
        pytest.skip("tile not compiled")
    tile = rows_tiles()[tile]
    for i, (M, N, K, slices) in enumerate(SPLIT_CASES):
        kw = dict(variant=sg.VARIANT_SKINNY, tile=tile, group_m=slices)
        lab = f"split t{tile} s{slices} ta={ta} tb={tb} {(M, N, K)}"
        print(lab, flush=True)
        A, B, C0 = workloads.draw(M, N, K, "uniform", 2700 + i, True)
        As, Bs = stored(A, B, ta, tb)
        for flags in (0, sg.FLAG_SCALAR_IO):
            C = dev(C0)
            sg.gemm(dev(As), dev(Bs), C, 0.5, -1.25, trans_a=ta, trans_b=tb, flags=flags, **kw)
            torch.cuda.synchronize()
            got = C.cpu().numpy()
            ref = oracle_mod.sgemm(As, Bs, C0.copy(), 0.5, -1.25, trans_a=ta, trans_b=tb)
            r = max_err_ratio(got, ref, K, 0.5, -1.25, As, Bs, C0)
            assert r <= 1.0, f"{lab} flags {flags}: max err/tol = {r}"
        C2 = dev(C0)
        sg.gemm(dev(As), dev(Bs), C2, 0.5, -1.25, trans_a=ta, trans_b=tb, **kw)
        C3 = dev(C0)
        sg.gemm(dev(As), dev(Bs), C3, 0.5, -1.25, trans_a=ta, trans_b=tb, **kw)
        torch.cuda.synchronize()
        assert torch.equal(C2, C3), f"{lab}: two calls differ"
        bias = np.random.default_rng(2750 + i).uniform(-1, 1, N).astype(F32)
        C = dev(C0)
        sg.gemm(dev(As), dev(Bs), C, 1.0, 0.5, trans_a=ta, trans_b=tb, bias=dev(bias),
                act=sg.ACT_GELU_ERF, **kw)
        torch.cuda.synchronize()
        ref = oracle_mod.sgemm(As, Bs, C0.copy(), 1.0, 0.5, trans_a=ta, trans_b=tb, bias=bias,
                               act=sg.ACT_GELU_ERF)
        x = oracle_mod.sgemm(As, Bs, C0.copy(), 1.0, 0.5, trans_a=ta, trans_b=tb, bias=bias)
        r = epilogue_err_ratio(C.cpu().numpy(), ref, x, K, 1.0, 0.5, As, Bs, C0, bias,
                               sg.ACT_GELU_ERF)
        assert r <= 1.0, f"{lab} GELU: max err/tol = {r}"
        Ai, Bi, Ci = workloads.draw(M, N, K, "int4", 2800 + i, True)
        Ai, Bi = stored(Ai, Bi, ta, tb)
        C = dev(Ci)
        sg.gemm(dev(Ai), dev(Bi), C, 0.5, -1.25, trans_a=ta, trans_b=tb, **kw)
        torch.cuda.synchronize()
        ref = oracle_mod.sgemm(Ai, Bi, Ci.copy(), 0.5, -1.25, trans_a=ta, trans_b=tb)
        assert np.array_equal(C.cpu().numpy(), ref), f"{lab} int: not bit-exact"


def test_skinny_split_repeated_bit_exact(oracle_mod):
    """Many-slice splits, repeated: each slice's partial sums are read back by
    whichever workgroup of the strip arrives last, so a partial sum that was
    not yet visible would show as a wrong cell.  Integer inputs make every
    order exact: 40 calls per case must all equal the oracle bit for bit."""
    cases = [(1, 4096, 4096, 0, 32), (4, 1000, 3001, 1, 16), (16, 2048, 4096, 2, 8),
             (3, 700, 8192, 3, 64), (16, 14336, 4096, 4, 3)]
    for M, N, K, tile, slices in cases:
        A, B, C0 = workloads.draw(M, N, K, "int4", 3100 + M + K, True)
        ref = oracle_mod.sgemm(A, B, C0.copy(), 0.5, -1.25)
        dA, dB = dev(A), dev(B)
        outs = [dev(C0) for _ in range(40)]
        for C in outs:
            sg.gemm(dA, dB, C, 0.5, -1.25, variant=sg.VARIANT_SKINNY, tile=tile, group_m=slices)
        torch.cuda.synchronize()
        for n, C in enumerate(outs):
            assert np.array_equal(C.cpu().numpy(), ref), \
                f"call {n} of {(M, N, K)} tile {tile} slices {slices} is not bit-exact"


@pytest.mark.parametrize("tb", [False, True])
def test_persistent_batched(tb, oracle_mod):
    """A batch through the stream-K launchers (persistent workgroups over the
    whole tiles of every entry): ragged entries, more tiles than workgroups,
    a shared B (stride 0); integers bit-exact, random inputs within
    tolerance, the same bits as one workgroup per tile."""
    tiles = sk_tiles(False)
    if not tiles:
        pytest.skip("no stream-K tile")
    rng = np.random.default_rng(2900)
    for tile in tiles:
        d = sg.tile_info(sg.VARIANT_MFMA, tile)
        for batch, M, N, K, shared_b in ((5, d["bm"] + 4, 3 * d["bn"] - 8, 68, False),
                                        (40, 2 * d["bm"], 2 * d["bn"], 128, False),
                                        (3, 300, 520, 36, True)):
            lab = f"persistent t{tile} tb={tb} {(batch, M, N, K)} shared_b={shared_b}"
            print(lab, flush=True)
            for dist in ("int4", "uniform"):
                if dist == "int4":
                    A = rng.integers(-4, 5, (batch, M, K)).astype(F32)
                    B = rng.integers(-4, 5, (1 if shared_b else batch, N if tb else K,
                                             K if tb else N)).astype(F32)
                    C0 = rng.integers(-4, 5, (batch, M, N)).astype(F32)
                else:
                    A = rng.uniform(-1, 1, (batch, M, K)).astype(F32)
                    B = rng.uniform(-1, 1, (1 if shared_b else batch, N if tb else K,
                                            K if tb else N)).astype(F32)
                    C0 = rng.uniform(-1, 1, (batch, M, N)).astype(F32)
                dA, dB = dev(A), dev(B[0] if shared_b else B)
                C = dev(C0)
                sg.gemm_batched(dA, dB, C, 0.5, -1.25, trans_b=tb, variant=sg.VARIANT_MFMA,
                                tile=tile, flags=sg.FLAG_STREAMK)
                C1 = dev(C0)
                sg.gemm_batched(dA, dB, C1, 0.5, -1.25, trans_b=tb, variant=sg.VARIANT_MFMA,
                                tile=tile)
                torch.cuda.synchronize()
                got = C.cpu().numpy()
                assert np.array_equal(got, C1.cpu().numpy()), f"{lab} {dist}: differs from plain"
                Bb = np.broadcast_to(B, (batch,) + B.shape[1:]) if shared_b else B
                ref = oracle_mod.sgemm_batched(A, np.ascontiguousarray(Bb), C0.copy(), 0.5, -1.25,
                                               trans_b=tb)
                if dist == "int4":
                    assert np.array_equal(got, ref), f"{lab}: not bit-exact"
                else:
                    for b in range(batch):
                        r = max_err_ratio(got[b], ref[b], K, 0.5, -1.25, A[b], Bb[b], C0[b])
                        assert r <= 1.0, f"{lab} entry {b}: max err/tol = {r}"
