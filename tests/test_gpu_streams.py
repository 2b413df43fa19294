"""One handle used from two HIP streams: the calls share the handle's
workspace, so a call on a new stream must not start before the previous
stream's call has finished with it (oz2_set_stream orders the switch).
Results are checked against the CPU oracle, bitwise."""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import check_float_parity, from_dev, to_dev

pytestmark = pytest.mark.gpu


def test_alternating_streams_share_workspace_in_order():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import complex_gemm_emulation_amd as oz2
    big, small, s = 2048, 384, 16
    A1 = workloads.real_matrix(big, big, workloads.seed(30, 0), "phi", 1.0)
    B1 = workloads.real_matrix(big, big, workloads.seed(30, 1), "phi", 1.0)
    A2 = workloads.real_matrix(small, small, workloads.seed(30, 2), "phi", 1.0)
    B2 = workloads.real_matrix(small, small, workloads.seed(30, 3), "phi", 1.0)
    dA1, dB1, dA2, dB2 = to_dev(A1), to_dev(B1), to_dev(A2), to_dev(B2)
    outs1 = [torch.zeros(big * big, dtype=torch.float64, device="cuda") for _ in range(3)]
    outs2 = [torch.zeros(small * small, dtype=torch.float64, device="cuda") for _ in range(3)]
    torch.cuda.synchronize()
    st1, st2 = torch.cuda.Stream(), torch.cuda.Stream()
    print(f"[streams] {big}^3 on one stream, {small}^3 on another, s={s}, three rounds", flush=True)
    sys.stdout.flush()
    with oz2.Handle() as h:
        for r in range(3):
            # the small product goes first on a fresh handle's first round, so the
            # big one grows the workspace while the small one may still run
            with torch.cuda.stream(st2):
                h.dgemm("N", "N", small, small, small, 1.0, dA2, small, dB2, small, 0.0, outs2[r], small, s)
            with torch.cuda.stream(st1):
                h.dgemm("N", "N", big, big, big, 1.0, dA1, big, dB1, big, 0.0, outs1[r], big, s)
            with torch.cuda.stream(st2):
                h.dgemm("N", "N", small, small, small, 1.0, dA2, small, dB2, small, 0.0, outs2[r], small, s)
        torch.cuda.synchronize()
    want2 = oracle.gemm_entries(False, "N", "N", small, small, small, 1.0, A2, small, B2, small, 0.0,
                                None, small, s, chat_ints=False)["out"]
    rng = np.random.default_rng(30)
    rows = np.concatenate([[0, big - 1], rng.integers(0, big, 126)])
    cols = np.concatenate([[0, big - 1], rng.integers(0, big, 126)])
    want1 = oracle.gemm_entries(False, "N", "N", big, big, big, 1.0, A1, big, B1, big, 0.0, None, big, s,
                                rows=rows, cols=cols, chat_ints=False)["out"]
    for r in range(3):
        assert check_float_parity(from_dev(outs2[r]), want2, f"small, round {r}") == 0
        g1 = from_dev(outs1[r]).reshape(big, big).T
        assert check_float_parity(g1[rows, cols], want1, f"big, round {r}") == 0
