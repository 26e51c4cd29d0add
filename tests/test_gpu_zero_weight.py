"""GPU parity on zero and near-zero weights with one-signed, large activations.

A symmetric group stores the signed weight c - 2^(b-1) ("Qwen3.8-27B-INT6-
Mixed-AutoRound", Findings: symmetric above four bits), so the midpoint code
is the weight 0, and the layer is the dequantize-then-F.linear definition
("vLLM Can Run INT5-7", section 2), whose per-element tolerance is
4e-3 * sum|a*w| + 1e-3.  Rows and groups of midpoint codes (sum|a*w| = 0)
and codes within one step of the midpoint, against activations that are all
of one sign and large (|N(0,1)| * 50, |N(0,3)|), are where a kernel whose
error grows with sum|a| (an offset carried through the accumulation) rather
than with sum|a*w| leaves the bound.  Every path is covered: one-row decode
(vector ALU), 4- and 16-row decode (matrix cores), K split across
workgroups, 64- and 256-row prefill tiles with and without a K split, both
layouts and the grouped layer.  Rows of midpoint codes must come out exactly
0."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_wq_amd as wq
from weight_only_bit_wq_amd import synth
from gpu_util import Layer, assert_wna16, bf16_values, dev_bf16, host_bf16_bits

pytestmark = pytest.mark.gpu


def _edge_workload(M, N, K, b, seed, act="half50", smin=0.02, smax=1.0):
    """Row classes by n % 4: 0 all midpoint codes; 1 midpoint +- 1;
    2 alternate groups of midpoint and uniform codes; 3 uniform codes.
    Scales |s| log-uniform in [smin, smax] with a random sign.  Activations
    one-signed: |N(0,1)| * 50 ("half50") or |N(0,3)| ("half3"); rows with odd
    m are negated (all negative)."""
    rng = np.random.default_rng(seed)
    h = 1 << (b - 1)
    codes = np.full((N, K), h, dtype=np.uint8)
    cls = np.arange(N) % 4
    near = rng.integers(-1, 2, size=(N, K))
    codes[cls == 1] = (h + near[cls == 1]).astype(np.uint8)
    uni = synth.draw_codes(rng, N, K, b)
    gmask = ((np.arange(K) // 128) % 2 == 1)[None, :] & (cls == 2)[:, None]
    codes[gmask] = uni[gmask]
    codes[cls == 3] = uni[cls == 3]
    mag = np.exp(rng.uniform(np.log(smin), np.log(smax), size=(N, K // 128)))
    sign = np.where(rng.random((N, K // 128)) < 0.5, -1.0, 1.0)
    scales = synth.f32_to_bf16_bits((mag * sign).astype(np.float32))
    if act == "half50":
        a = np.abs(rng.standard_normal((M, K))) * 50.0
    else:
        a = np.abs(rng.normal(0.0, 3.0, size=(M, K)))
    a[1::2] *= -1.0
    A = synth.f32_to_bf16_bits(a.astype(np.float32))
    return synth.Workload(A, codes, scales, b)


def _check(w, Y_bits, what):
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, w.b), w.scales, w.b)
    assert_wna16(Y_bits, y_ref, mag, what)
    zero_rows = np.arange(w.N) % 4 == 0
    y = bf16_values(Y_bits)
    assert np.all(y[:, zero_rows] == 0.0), "%s: midpoint rows not exactly 0" % what


@pytest.mark.parametrize("act", ["half50", "half3"])
@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("b", [2, 5, 6, 7, 8])
def test_decode_zero_weights(b, M, act):
    # 136 groups over 4 row blocks: the default plan splits K 8 ways (one
    # row) or 16 ways (matrix-core row tiles) across workgroups.
    w = _edge_workload(M, 256, 17408, b, seed=2000 + 10 * b + M, act=act,
                       smax=0.02 if act == "half50" else 1.0)
    _check(w, Layer(w, wq.WQ_LAYOUT_TILED).gemm(), "decode b=%d M=%d %s" % (b, M, act))


@pytest.mark.parametrize("rows", [4, 8])
@pytest.mark.parametrize("b", [2, 6, 7, 8])
def test_decode_row_kernel_zero_weights(b, rows, monkeypatch):
    # The one-row kernel without a K split (the default for large layers),
    # forced onto the edge-case layer.
    monkeypatch.setenv("WQ_DECODE_ROWS", str(rows))
    w = _edge_workload(1, 256, 17408, b, seed=2050 + 10 * b + rows, act="half50")
    _check(w, Layer(w, wq.WQ_LAYOUT_TILED).gemm(), "row kernel b=%d rows=%d" % (b, rows))


@pytest.mark.parametrize("M,N,K", [(40, 256, 5120), (100, 256, 5120), (300, 256, 5120),
                                   (600, 2048, 1024)])
@pytest.mark.parametrize("b", [2, 6, 8])
def test_prefill_zero_weights(b, M, N, K):
    # 64-row tiles (M = 40, 100) and 256-row tiles (300, 600); the first
    # three shapes split K 5 ways, the last does not.
    w = _edge_workload(M, N, K, b, seed=2100 + 10 * b + M)
    _check(w, Layer(w, wq.WQ_LAYOUT_TILED).gemm(), "prefill b=%d M=%d" % (b, M))


@pytest.mark.parametrize("M", [1, 40])
def test_zero_weights_dense_layout(M):
    w = _edge_workload(M, 192, 2048, 6, seed=2200 + M, act="half3")
    _check(w, Layer(w, wq.WQ_LAYOUT_DENSE).gemm(), "dense M=%d" % M)


def test_grouped_zero_weights():
    # One decode-sized and two prefill-sized experts sharing the edge-case
    # weights (one blob repeated per expert).
    b, N, K = 6, 256, 5120
    w = _edge_workload(8 + 70 + 260, N, K, b, seed=2300, act="half3")
    L = Layer(w, wq.WQ_LAYOUT_TILED)
    eb = L.W_d.numel()
    W3 = L.W_d.repeat(3)
    off = np.array([0, 8, 78, 338], dtype=np.int64)
    Y = wq.wq_gemm_grouped(dev_bf16(w.A), W3, eb, off, N, b)
    torch.cuda.synchronize()
    _check(w, host_bf16_bits(Y), "grouped")


def test_grouped_decode_split_after_many_prefill_tiles():
    # More than one prefill table (over 240 tiles), then a decode expert
    # whose K is split: sizes [300] + [64] * 239 + [10], K = 5120.  The
    # decode partials and the prefill tiles use the workspace and the
    # launch tables in turn; every expert's rows are checked that the
    # oracle reaches (expert 0, three 64-row experts, the decode expert).
    b, N, K = 6, 256, 5120
    sizes = [300] + [64] * 239 + [10]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    M = int(off[-1])
    rng = np.random.default_rng(2400)
    wts = [synth.Workload(np.zeros((1, K), np.uint16), synth.draw_codes(rng, N, K, b),
                          synth.draw_scales_halfnormal_signed(rng, N, K // 128), b)
           for _ in range(3)]
    blobs = [Layer(wt, wq.WQ_LAYOUT_TILED).W_d for wt in wts]
    eb = blobs[0].numel()
    which = [0] + [1] * 239 + [2]
    Wall = torch.cat([blobs[i] for i in which])
    A = synth.draw_act(rng, M, K)
    assert wq.wq_grouped_workspace_bytes(off, N, K, b) > wq.WORKSPACE_ZERO_BYTES
    Y = host_bf16_bits(wq.wq_gemm_grouped(dev_bf16(A), Wall, eb, off, N, b))
    for e in (0, 1, 120, 239, 240):
        r0, r1 = int(off[e]), int(off[e + 1])
        wt = wts[which[e]]
        y_ref, mag = oracle.wna16(A[r0:r1], oracle.pack(wt.codes, b), wt.scales, b)
        assert_wna16(Y[r0:r1], y_ref, mag, "grouped expert %d" % e)


def test_non_default_stream_split_k(monkeypatch):
    # The binding allocates the output and the zeroed workspace on the
    # stream the call runs on; a one-row decode with its K split (the
    # split-K kernel forced) runs on a fresh stream, twice, against the
    # oracle and bit for bit.
    monkeypatch.setenv("WQ_DECODE_ROWS", "0")
    w = synth.decode(M=1, b=6, N=4096, K=5120)
    L = Layer(w, wq.WQ_LAYOUT_TILED)
    assert wq.wq_workspace_bytes(wq.WQ_OP_GEMM, 1, w.N, w.K, 6) > 0
    A = dev_bf16(w.A)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    Y0 = wq.wq_gemm(A, L.W_d, L.layout, None, w.N, 6, stream=s)
    Y1 = wq.wq_gemm(A, L.W_d, L.layout, None, w.N, 6, stream=s)
    s.synchronize()
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, 6), w.scales, 6)
    assert_wna16(host_bf16_bits(Y0), y_ref, mag, "stream")
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
