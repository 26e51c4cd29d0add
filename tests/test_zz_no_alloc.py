"""GPU: wq_gemm_noalloc (the WNA16 layer on the library's static per-GPU
scratch, no allocation) against wq_gemm (caller's workspace) on the same
inputs.  Both run the same kernels and plans, so the outputs must agree bit
for bit; each is also held to the oracle's bound
|y - y_ref| <= 4e-3 sum|a w| + 1e-3 ("vLLM Can Run INT5-7", section 2).
Every case makes two calls in a row, the second on a smaller input, so the
second call runs on the scratch the first one left behind: a K split across
workgroups at decode batch sizes (tickets and partials in the scratch), a K
split in prefill (partials), the prefill split of a last round's tiles
(partials), and the one-row decode kernel (no scratch)."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_wq_amd as wq
from weight_only_bit_wq_amd import synth
from gpu_util import Layer, assert_wna16, dev_bf16, host_bf16_bits

pytestmark = pytest.mark.gpu


def _workload(M, N, K, b, seed):
    rng = np.random.default_rng(seed)
    return synth.Workload(synth.draw_act(rng, M, K), synth.draw_codes(rng, N, K, b),
                          synth.draw_scales_halfnormal_signed(rng, N, K // 128), b)


def _pair(w, layout):
    L = Layer(w, layout)
    A = dev_bf16(w.A)
    Y0 = wq.wq_gemm(A, L.W_d, layout, L.S_d, w.N, w.b)
    Y1 = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    wq.wq_gemm_noalloc(A, L.W_d, layout, L.S_d, w.N, w.b, Y=Y1)
    torch.cuda.synchronize()
    return host_bf16_bits(Y0), host_bf16_bits(Y1)


def _check(w, layout, what):
    y0, y1 = _pair(w, layout)
    np.testing.assert_array_equal(y1, y0, err_msg=what + ": noalloc != wq_gemm")
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, w.b), w.scales, w.b)
    assert_wna16(y1, y_ref, mag, what)


# (first, second): M, N, K of two calls in a row; b.
CASES = {
    "decode_split_k": [((4, 4096, 5120), (2, 1024, 2560)), 6],
    "decode_split_k_m16": [((16, 2048, 17408), (9, 512, 5120)), 5],
    "prefill_split_k": [((300, 256, 5120), (100, 256, 2560)), 6],
    "prefill_tail_split": [((800, 16590, 4096), (790, 16420, 4096)), 6],
    "one_row": [((1, 4352, 5120), (1, 640, 1280)), 7],
}


@pytest.mark.parametrize("layout", [wq.WQ_LAYOUT_TILED, wq.WQ_LAYOUT_DENSE],
                         ids=["tiled", "dense"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_matches_wq_gemm(case, layout):
    shapes, b = CASES[case]
    for i, (M, N, K) in enumerate(shapes):
        need = wq.wq_workspace_bytes(wq.WQ_OP_GEMM, M, N, K, b)
        assert 0 <= need <= wq.WQ_NOALLOC_SCRATCH_BYTES
        if case != "one_row" and i == 0:
            assert need > 0, "case must use the scratch"
        w = _workload(M, N, K, b, seed=7000 + 31 * i + len(case))
        _check(w, layout, "%s call %d (M=%d N=%d K=%d b=%d)" % (case, i, M, N, K, b))

