"""The stream-K form of the MFMA rung on the GPU: the split of tiles over
workgroups, the two-pass deterministic reduction, and the two ways to
provide its workspace (the library's per-stream buffer and the caller's).
Results are checked against the CPU oracle (exact on integer patterns,
1e-5 * sum |A_ik B_kj| on floating point)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import tiling_roofline_analysis_amd as tra
from tiling_roofline_analysis_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tra.load()


def dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def check_tol(C, ref, what):
    err = np.abs(C.astype(np.float64) - ref.c64)
    assert np.all(err <= TOL * ref.s64), f"{what}: max |diff|/S = {np.max(err / ref.s64):.3e}"


# Shapes whose tiles do not fill whole waves, for both forms of the split:
# parts (the split tiles cut into equal K runs that share the main launch
# with the data-parallel tiles) and stream-K runs (a launch of their own,
# runs crossing tiles).  The form each shape gets on MI355X is asserted.
SPLIT_SHAPES = [
    (300, 500, 203, "parts"),     # all 40 tiles in 6 parts of 2-3 slices
    (257, 129, 1000, "parts"),    # all 15 tiles in 8 parts
    (3000, 2049, 1531, "parts"),  # the ragged shape: its last 15 tiles in 8 parts
    (4000, 4200, 1027, "parts"),   # 528 tiles of 256 x 128: the last 16 in 8 parts
    (1500, 1500, 77, "runs"),     # 576 tiles of 64 x 64 in under a wave, 5 slices each
    (1152, 1152, 8192, "runs"),   # 324 tiles: 2 parts each would leave CUs uneven
    (4608, 4608, 4096, "runs"),   # 648 tiles of 256 x 128: the last 136, over half a wave
    (4000, 60, 3000, "parts"),    # narrower than a tile (float4 edge loads), 63 tiles in 8 parts
    (8200, 61, 3000, "runs"),     # narrower, N odd (element edge loads), 129 tiles
]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s[:3])))
def test_split_shapes_match_oracle(shape):
    import torch
    M, N, K, form = shape
    d = tra.tra_gemm_describe(tra.MFMA_STREAMK, M, N, K)
    print(f"[case] split ({form}) {M}x{N}x{K} ({d})", flush=True)
    assert "stream_k_tiles=0" not in d and f"split={form} " in d, d
    A = inputs.uniform(M, K, 31)
    B = inputs.uniform(K, N, 32)
    C = tra.matmul(dev(A), dev(B), variant=tra.MFMA_STREAMK)
    torch.cuda.synchronize()
    C = C.cpu().numpy()
    # every element against the oracle's full product (4608^2 x 4096: about
    # 25 s on 16 cores), and a direct sample of rows, columns and entries
    check_tol(C, oracle.gemm(A, B), f"{M}x{N}x{K}")
    rng = np.random.default_rng(M)
    rows = np.concatenate([rng.integers(0, M, 2000), np.arange(M), np.full(N, M - 1)])
    cols = np.concatenate([rng.integers(0, N, 2000), np.full(M, N - 1), np.arange(N)])
    ref = oracle.gemm_entries(A, B, rows, cols)
    err = np.abs(C[rows, cols].astype(np.float64) - ref.c64)
    assert np.all(err <= TOL * ref.s64)
    # integer patterns: exact whatever the split
    Ai, Bi = inputs.int_pattern_a(M, K), inputs.int_pattern_b(K, N)
    Ci = tra.matmul(dev(Ai), dev(Bi), variant=tra.MFMA_STREAMK)
    torch.cuda.synchronize()
    ii, jj = np.meshgrid(np.arange(min(13, M)), np.arange(min(7, N)), indexing="ij")
    per = oracle.gemm_entries(Ai, Bi, ii.ravel(), jj.ravel()).c32.reshape(ii.shape)
    exp = per[np.arange(M)[:, None] % 13, np.arange(N)[None, :] % 7]
    assert np.array_equal(Ci.cpu().numpy(), exp)


def test_split_is_deterministic():
    import torch
    M, N, K = 1500, 1500, 77
    A, B = dev(inputs.uniform(M, K, 3)), dev(inputs.uniform(K, N, 4))
    first = tra.matmul(A, B, variant=tra.MFMA_STREAMK).clone()
    for _ in range(5):
        again = tra.matmul(A, B, variant=tra.MFMA_STREAMK)
        torch.cuda.synchronize()
        assert torch.equal(first, again)


def test_caller_workspace_matches_library_workspace():
    import torch
    M, N, K = 3000, 2049, 1531
    A, B = dev(inputs.uniform(M, K, 5)), dev(inputs.uniform(K, N, 6))
    need = tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, M, N, K)
    assert need > 0
    ws = torch.full((need // 4,), float("nan"), device="cuda:0")
    C1 = tra.matmul(A, B, variant=tra.MFMA_STREAMK, workspace=ws)
    C2 = tra.matmul(A, B, variant=tra.MFMA_STREAMK)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    # a workspace one byte short is refused before anything runs
    with pytest.raises(tra.TraError):
        tra.matmul(A, B, variant=tra.MFMA_STREAMK, workspace=torch.empty(need // 4 - 1,
                                                                          device="cuda:0"))


def test_library_workspace_grows_and_serves_several_streams():
    import torch
    small, large = (300, 500, 203), (4000, 4200, 1027)
    assert (tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, *small)
            < tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, *large))
    cases = {}
    for M, N, K in (small, large):
        A, B = inputs.int_pattern_a(M, K), inputs.int_pattern_b(K, N)
        rows = np.arange(0, M, 7)
        cols = np.arange(0, N, 5)
        rr, cc = np.meshgrid(rows, cols, indexing="ij")
        ref = oracle.gemm_entries(A, B, rr.ravel(), cc.ravel()).c32.reshape(rr.shape)
        cases[(M, N, K)] = (dev(A), dev(B), rows, cols, ref)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    # small then large on one stream (the buffer grows), then both streams
    for shape, stream in ((small, s1), (large, s1), (large, s2), (small, s2), (small, s1)):
        A, B, rows, cols, ref = cases[shape]
        with torch.cuda.stream(stream):
            C = tra.matmul(A, B, variant=tra.MFMA_STREAMK)
        stream.synchronize()
        assert np.array_equal(C.cpu().numpy()[np.ix_(rows, cols)], ref), shape


def test_auto_uses_the_split_where_it_pays():
    import torch
    M, N, K = 3000, 2049, 1531
    assert "rung=mfma_streamk" in tra.tra_gemm_describe(tra.AUTO, M, N, K)
    A, B = dev(inputs.uniform(M, K, 5)), dev(inputs.uniform(K, N, 6))
    C1 = tra.matmul(A, B)
    C2 = tra.matmul(A, B, variant=tra.MFMA_STREAMK)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


def test_threads_on_their_own_streams_share_the_library_safely():
    # four threads, each on its own stream, alternate a split in parts and
    # one in stream-K runs (with a larger workspace) without synchronising,
    # so the library's per-stream workspaces are created and grown while the
    # other threads launch; every result must equal the single-threaded one
    # bit for bit (the split's reduction order is fixed)
    import threading
    import torch
    shapes = [(4000, 4200, 1027), (1500, 1500, 77)]
    assert (tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, *shapes[0])
            < tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, *shapes[1]))
    operands, expect = {}, {}
    for M, N, K in shapes:
        A, B = dev(inputs.uniform(M, K, M + 1)), dev(inputs.uniform(K, N, N + 2))
        operands[(M, N, K)] = (A, B)
        expect[(M, N, K)] = tra.matmul(A, B, variant=tra.MFMA_STREAMK)
    streams = [torch.cuda.Stream() for _ in range(4)]
    plan = {(t, i): shapes[(t + i) % 2] for t in range(4) for i in range(6)}
    outs = {key: torch.full((s[0], s[1]), float("nan"), device="cuda:0")
            for key, s in plan.items()}
    torch.cuda.synchronize()
    failures = []

    def work(t):
        for i in range(6):
            M, N, K = plan[(t, i)]
            A, B = operands[(M, N, K)]
            st = tra.gemm_f32_variant(tra.MFMA_STREAMK, M, N, K, A.data_ptr(), K, B.data_ptr(),
                                      N, outs[(t, i)].data_ptr(), N, streams[t].cuda_stream)
            if st != tra.TRA_OK:
                failures.append((t, i, tra.tra_status_string(st)))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not failures, failures
    for key, C in outs.items():
        assert torch.equal(C, expect[plan[key]]), key


def _hip_runtime():
    """The process's HIP runtime (the copy torch loaded), for stream calls
    torch does not expose: creating and destroying raw streams."""
    import ctypes
    import torch  # noqa: F401  (loads the runtime first)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    hip.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    return hip


def _int_case(M, N, K):
    A, B = inputs.int_pattern_a(M, K), inputs.int_pattern_b(K, N)
    ii, jj = np.meshgrid(np.arange(min(13, M)), np.arange(min(7, N)), indexing="ij")
    per = oracle.gemm_entries(A, B, ii.ravel(), jj.ravel()).c32.reshape(ii.shape)
    exp = per[np.arange(M)[:, None] % 13, np.arange(N)[None, :] % 7]
    return dev(A), dev(B), exp


def test_streams_destroyed_and_recreated_between_split_calls():
    # raw streams created and destroyed around each split call (synchronised
    # first, as the header asks); handles of destroyed streams are commonly
    # handed out again, and the buffer of a handle must then grow in stream
    # order on the new stream
    import ctypes
    import torch
    hip = _hip_runtime()
    small, large = (300, 500, 203), (4000, 4200, 1027)
    cases = {s: _int_case(*s) for s in (small, large)}
    handles = []
    for i, shape in enumerate((small, large, small, large, large, small)):
        h = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(h)) == 0
        handles.append(h.value)
        A, B, exp = cases[shape]
        M, N, K = shape
        C = torch.full((M, N), float("nan"), device="cuda:0")
        torch.cuda.synchronize()
        st = tra.gemm_f32_variant(tra.MFMA_STREAMK, M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                  C.data_ptr(), N, h.value)
        assert st == tra.TRA_OK, tra.tra_status_string(st)
        assert hip.hipStreamSynchronize(h) == 0
        assert hip.hipStreamDestroy(h) == 0
        assert np.array_equal(C.cpu().numpy(), exp), (i, shape)
    print(f"[case] stream handles used: {len(set(handles))} distinct of {len(handles)}",
          flush=True)


def test_per_thread_default_stream_keeps_one_workspace_per_thread():
    # hipStreamPerThread is one handle naming a different stream in each
    # thread: each thread must get its own buffer.  Four threads alternate
    # a small and a large split on it without synchronising in between.
    import threading
    import torch
    hip = _hip_runtime()
    per_thread = 2   # hipStreamPerThread
    shapes = [(300, 500, 203), (4000, 4200, 1027)]
    cases = {s: _int_case(*s) for s in shapes}
    outs = {(t, i): torch.full(shapes[(t + i) % 2][:2], float("nan"), device="cuda:0")
            for t in range(4) for i in range(4)}
    torch.cuda.synchronize()
    failures = []

    def work(t):
        for i in range(4):
            M, N, K = shapes[(t + i) % 2]
            A, B, _ = cases[(M, N, K)]
            st = tra.gemm_f32_variant(tra.MFMA_STREAMK, M, N, K, A.data_ptr(), K,
                                      B.data_ptr(), N, outs[(t, i)].data_ptr(), N, per_thread)
            if st != tra.TRA_OK:
                failures.append((t, i, tra.tra_status_string(st)))
        if hip.hipStreamSynchronize(per_thread) != 0:
            failures.append((t, "sync"))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not failures, failures
    for (t, i), C in outs.items():
        assert np.array_equal(C.cpu().numpy(), cases[shapes[(t + i) % 2]][2]), (t, i)


def test_graph_capture_takes_the_caller_workspace():
    # while a stream is captured, the library's own scratch is refused (it
    # would be allocated into the graph); the caller's workspace, the entry
    # point that allocates nothing and an unsplit direct-load launch are
    # captured, and every replay -- with eager work and synchronisation in
    # between -- equals the eager result
    import torch
    M, N, K = 3000, 2049, 1531
    A, B = dev(inputs.uniform(M, K, 7)), dev(inputs.uniform(K, N, 8))
    need = tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, M, N, K)
    ws = torch.empty(need // 4, device="cuda:0")
    eager = tra.matmul(A, B, variant=tra.MFMA_STREAMK, workspace=ws).clone()
    C = torch.full((M, N), float("nan"), device="cuda:0")
    # the entry point that allocates nothing, warmed by one eager call (its
    # first call on a device looks up the address of its scratch array)
    C2 = torch.full((M, N), float("nan"), device="cuda:0")
    h0 = torch.cuda.current_stream().cuda_stream
    assert tra.gemm_f32_variant_noalloc(tra.MFMA_STREAMK, M, N, K, A.data_ptr(), K, B.data_ptr(),
                                        N, C2.data_ptr(), N, h0) == tra.TRA_OK
    torch.cuda.synchronize()
    assert torch.equal(C2, eager)
    other = torch.empty((M, N), device="cuda:0")
    # and an unsplit launch that stages its slices with direct loads into LDS
    Md = Nd = Kd = 1024
    Ad, Bd = dev(inputs.uniform(Md, Kd, 9)), dev(inputs.uniform(Kd, Nd, 10))
    assert "LDS stages" in tra.tra_gemm_describe(tra.MFMA, Md, Nd, Kd)
    eager_d = tra.matmul(Ad, Bd, variant=tra.MFMA).clone()
    Cd = torch.full((Md, Nd), float("nan"), device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        refused = tra.gemm_f32_variant(tra.MFMA_STREAMK, M, N, K, A.data_ptr(), K, B.data_ptr(),
                                       N, C.data_ptr(), N, s.cuda_stream)
        st = tra.gemm_f32_variant_ws(tra.MFMA_STREAMK, M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                     C.data_ptr(), N, ws.data_ptr(), need, s.cuda_stream)
        st2 = tra.gemm_f32_variant_noalloc(tra.MFMA_STREAMK, M, N, K, A.data_ptr(), K,
                                           B.data_ptr(), N, C2.data_ptr(), N, s.cuda_stream)
        st3 = tra.gemm_f32_variant(tra.MFMA, Md, Nd, Kd, Ad.data_ptr(), Kd, Bd.data_ptr(), Nd,
                                   Cd.data_ptr(), Nd, s.cuda_stream)
    assert refused == tra.TRA_ERR_UNSUPPORTED
    assert st == tra.TRA_OK and st2 == tra.TRA_OK and st3 == tra.TRA_OK
    for r in range(3):
        C.fill_(float("nan"))
        C2.fill_(float("nan"))
        Cd.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, eager), r
        assert torch.equal(C2, eager), r
        assert torch.equal(Cd, eager_d), r
        tra.matmul(A, B, other)   # eager work between replays (library workspace)
        torch.cuda.synchronize()
