"""q4k_gemm_batch_noalloc (scratch in the library's static device array, no
allocation) against q4k_gemm_batch with a caller workspace, called through the
C ABI: bit-identical outputs on two calls in a row, the second with a smaller
input, and the oracle on sampled rows."""
import ctypes

import numpy as np
import pytest

import q4k_inputs as qi
from _helpers import assert_close, to_dev

pytestmark = pytest.mark.gpu


def _problems(q4k, ws, ys, Ns):
    P = q4k._lib.GemmProblem
    return (P * len(Ns))(*[P(w.data_ptr(), y.data_ptr(), N) for w, y, N in zip(ws, ys, Ns)])


def test_gemm_batch_noalloc_matches_workspace_entry(oracle_lib):
    import torch
    import gemm_q4_super_amd as q4k
    L = q4k.lib()
    ws_buf = torch.zeros(int(L.q4k_gemm_workspace_bytes()), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    # a 512-row prefill batch ({q, k, v}-shaped, tiles split across workgroups),
    # then a smaller ragged one
    for M, K, Ns, seed in ((512, 2560, [4096, 1024, 1024], 9300), (77, 1024, [700, 33], 9400)):
        wts = [to_dev(qi.make_q4k_bytes(N, K, seed + i)) for i, N in enumerate(Ns)]
        codes, scales, sums = oracle_lib.quantize_act(qi.make_act(M, K, seed + 50))
        dc, ds, dsu = to_dev(codes), to_dev(scales), to_dev(sums)
        y_a = [torch.full((M, N), np.nan, dtype=torch.float32, device="cuda") for N in Ns]
        y_b = [torch.full((M, N), np.nan, dtype=torch.float32, device="cuda") for N in Ns]
        st = L.q4k_gemm_batch_noalloc(_problems(q4k, wts, y_a, Ns), len(Ns), K, dc.data_ptr(),
                                      ds.data_ptr(), dsu.data_ptr(), M, stream)
        assert st == 0, q4k.q4k_status_string(st)
        st = L.q4k_gemm_batch(_problems(q4k, wts, y_b, Ns), len(Ns), K, dc.data_ptr(),
                              ds.data_ptr(), dsu.data_ptr(), M, ws_buf.data_ptr(), ws_buf.numel(),
                              stream)
        assert st == 0, q4k.q4k_status_string(st)
        torch.cuda.synchronize()
        for i, (N, a, b) in enumerate(zip(Ns, y_a, y_b)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), "M=%d product %d" % (M, i)
            rows = np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, 16)])
            ref = oracle_lib.matvec(wts[i].cpu().numpy(), N, K, codes, scales, rows=rows,
                                    parallel=True)
            assert_close(a.cpu().numpy()[:, rows], ref, "noalloc M=%d product %d" % (M, i))


def test_gemm_batch_noalloc_argument_checks():
    import gemm_q4_super_amd as q4k
    L = q4k.lib()
    P = q4k._lib.GemmProblem
    A = 0x10000
    arr = (P * 1)(P(A, A, 16))
    assert L.q4k_gemm_batch_noalloc(None, 1, 512, A, A, A, 1, None) == -1
    assert L.q4k_gemm_batch_noalloc(arr, 0, 512, A, A, A, 1, None) == -3
    assert L.q4k_gemm_batch_noalloc(arr, 1, 500, A, A, A, 1, None) == -3
    assert L.q4k_gemm_batch_noalloc(arr, 1, 512, A + 4, A, A, 1, None) == -2
