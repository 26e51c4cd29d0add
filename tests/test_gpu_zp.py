"""GPU parity with zero points (b = 4 and 8) and per-channel scales (group = K)
against the CPU oracle, through the C ABI: the WNA16 layer on every kernel
(decode row tiles 1/4/8/16, the split-K hand-off, prefill on both tile
sizes) in both layouts, the int8-activation path (b = 4) and the
embedding gather (bit-exact).  Pages: model card
"Qwen3.8-27B-INT6-Mixed-AutoRound", Findings (the asymmetric form exists for
4 and 8 bits); "vLLM Quantization", online shorthands (INT8, one scale per
channel)."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_wq_amd as wq
from weight_only_bit_wq_amd import synth
from gpu_util import assert_a8, assert_wna16, dev_bf16, dev_words, host_bf16_bits, sample_points

pytestmark = pytest.mark.gpu

LAYOUTS = [wq.WQ_LAYOUT_DENSE, wq.WQ_LAYOUT_TILED]
LNAME = {wq.WQ_LAYOUT_DENSE: "dense", wq.WQ_LAYOUT_TILED: "tiled"}


def _zp_workload(M, N, K, b, seed):
    rng = np.random.default_rng(seed)
    codes = synth.draw_codes(rng, N, K, b)
    scales = synth.draw_scales_halfnormal_signed(rng, N, K // 128)
    zeros = rng.integers(0, 1 << b, size=(N, K // 128), dtype=np.uint8)
    A = synth.draw_act(rng, M, K)
    return A, codes, scales, zeros


def _weights(codes, scales, b, layout, group=128):
    K = codes.shape[1]
    packed = wq.wq_pack(codes, b)
    if layout == wq.WQ_LAYOUT_TILED:
        return wq.wq_repack(dev_words(packed), dev_bf16(scales), K, b, group=group), None, packed
    return dev_words(packed), dev_bf16(scales), packed


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("M", [1, 3, 4, 8, 16, 33, 300])
@pytest.mark.parametrize("b", [4, 8])
def test_gemm_zero_points(b, M, layout):
    N, K = 200, 1024
    A, codes, scales, zeros = _zp_workload(M, N, K, b, 2000 + 10 * M + b)
    print("zp gemm b=%d M=%d %s" % (b, M, LNAME[layout]), flush=True)
    W_d, S_d, packed = _weights(codes, scales, b, layout)
    Y = wq.wq_gemm(dev_bf16(A), W_d, layout, S_d, N, b, zeros=torch.from_numpy(zeros).cuda())
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16(A, packed, scales, b, zeros=zeros)
    assert_wna16(host_bf16_bits(Y), y_ref, mag, "zp b=%d M=%d" % (b, M))


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("b", [4, 8])
def test_gemm_zero_points_split_k_forced(b, M, monkeypatch):
    # The decode hand-off with zero points, K forced into 4 splits.
    monkeypatch.setenv("WQ_DECODE_ROWS", "0")  # M = 1 would take the row kernel
    monkeypatch.setenv("WQ_DECODE_WAVES", "8")
    monkeypatch.setenv("WQ_DECODE_SPLITS", "4")
    N, K = 200, 1536
    A, codes, scales, zeros = _zp_workload(M, N, K, b, 2100 + M + b)
    W_d, _, packed = _weights(codes, scales, b, wq.WQ_LAYOUT_TILED)
    ws = torch.zeros(8 << 20, dtype=torch.uint8, device="cuda")
    Y = wq.wq_gemm(dev_bf16(A), W_d, wq.WQ_LAYOUT_TILED, None, N, b, ws=ws,
                   zeros=torch.from_numpy(zeros).cuda())
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16(A, packed, scales, b, zeros=zeros)
    assert_wna16(host_bf16_bits(Y), y_ref, mag, "zp split-K b=%d M=%d" % (b, M))
    assert not ws[:wq.WORKSPACE_ZERO_BYTES].any()


@pytest.mark.parametrize("b", [4, 8])
def test_gemm_zero_points_integer_exact(b):
    # Integer activations, unit scales: the layer is the integer product
    # A . (c - z)^T, exact (|sums| < 2^24), on the decode and prefill paths.
    rng = np.random.default_rng(2200 + b)
    N, K = 96, 512
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    zeros = rng.integers(0, 1 << b, size=(N, K // 128), dtype=np.uint8)
    scales = np.full((N, K // 128), 0x3F80, dtype=np.uint16)
    W_d, _, _ = _weights(codes, scales, b, wq.WQ_LAYOUT_TILED)
    q = codes.astype(np.int64) - np.repeat(zeros.astype(np.int64), 128, axis=1)
    for M in (1, 4, 40):
        A_int = rng.integers(-8, 9, size=(M, K))
        Y = wq.wq_gemm(dev_bf16(synth.f32_to_bf16_bits(A_int.astype(np.float32))), W_d,
                       wq.WQ_LAYOUT_TILED, None, N, b, zeros=torch.from_numpy(zeros).cuda())
        torch.cuda.synchronize()
        ref = (A_int @ q.T).astype(np.float32)
        np.testing.assert_array_equal(synth.bf16_bits_to_f32(host_bf16_bits(Y)),
                                      synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(ref)))


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("b,zp", [(4, True), (4, False), (8, True)])
def test_gemm_extreme_codes_integer_exact(b, zp, layout):
    # Codes and zero points only at the ends of their range (0 and 2^b - 1),
    # so c - z spans its extremes (-(2^b - 1) .. 2^b - 1, or -2^(b-1) and
    # 2^(b-1) - 1 without zero points): the b = 4 operands are built four
    # bytes at a time, and a borrow between bytes would show here.  Integer
    # activations and unit scales make the layer an exact integer product,
    # on the decode row kernel (M = 1), the split-K row tiles (4, 16) and
    # both prefill tiles (40, 300); the oracle is checked against it too.
    rng = np.random.default_rng(2300 + 10 * b + zp)
    N, K = 96, 512
    top = (1 << b) - 1
    codes = (rng.integers(0, 2, size=(N, K)) * top).astype(np.uint8)
    zeros = (rng.integers(0, 2, size=(N, K // 128)) * top).astype(np.uint8) if zp else None
    scales = np.full((N, K // 128), 0x3F80, dtype=np.uint16)
    W_d, S_d, packed = _weights(codes, scales, b, layout)
    zcol = (np.repeat(zeros.astype(np.int64), 128, axis=1) if zp
            else np.full((N, K), 1 << (b - 1), dtype=np.int64))
    q = codes.astype(np.int64) - zcol
    Z = torch.from_numpy(zeros).cuda() if zp else None
    for M in (1, 4, 16, 40, 300):
        A_int = rng.integers(-8, 9, size=(M, K))
        A = synth.f32_to_bf16_bits(A_int.astype(np.float32))
        Y = wq.wq_gemm(dev_bf16(A), W_d, layout, S_d, N, b, zeros=Z)
        torch.cuda.synchronize()
        ref = synth.f32_to_bf16_bits((A_int @ q.T).astype(np.float32))
        np.testing.assert_array_equal(host_bf16_bits(Y), ref, err_msg="M=%d" % M)
        y_ref, _ = oracle.wna16(A, packed, scales, b, zeros=zeros)
        np.testing.assert_array_equal(synth.f32_to_bf16_bits(y_ref.astype(np.float32)), ref,
                                      err_msg="oracle M=%d" % M)


@pytest.mark.parametrize("M", [1, 4, 16, 40, 300])
@pytest.mark.parametrize("b", [4, 6, 8])
def test_gemm_per_channel_scales(b, M):
    # One scale per row (group = K), expanded into the tiled blob by wq_repack.
    N, K = 200, 1024
    rng = np.random.default_rng(2300 + M + b)
    codes = synth.draw_codes(rng, N, K, b)
    scales = synth.draw_scales_halfnormal_signed(rng, N, 1)
    A = synth.draw_act(rng, M, K)
    W_d, _, packed = _weights(codes, scales, b, wq.WQ_LAYOUT_TILED, group=K)
    Y = wq.wq_gemm(dev_bf16(A), W_d, wq.WQ_LAYOUT_TILED, None, N, b, group=K)
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16(A, packed, scales, b, group=K)
    assert_wna16(host_bf16_bits(Y), y_ref, mag, "per-channel b=%d M=%d" % (b, M))


def test_gemm_zero_points_decode_full_shape():
    # b = 4 with zero points at the decode layer's full size, M = 1 and 4.
    N, K, b = 17408, 5120, 4
    for M in (1, 4):
        A, codes, scales, zeros = _zp_workload(M, N, K, b, 2400 + M)
        W_d, _, packed = _weights(codes, scales, b, wq.WQ_LAYOUT_TILED)
        Y = wq.wq_gemm(dev_bf16(A), W_d, wq.WQ_LAYOUT_TILED, None, N, b,
                       zeros=torch.from_numpy(zeros).cuda())
        torch.cuda.synchronize()
        y_ref, mag = oracle.wna16(A, packed, scales, b, zeros=zeros)
        assert_wna16(host_bf16_bits(Y), y_ref, mag, "zp full decode M=%d" % M)


def test_gemm_zero_points_prefill_shape_sampled():
    N, K, b, M = 5120, 5120, 4, 1024
    A, codes, scales, zeros = _zp_workload(M, N, K, b, 2500)
    W_d, _, packed = _weights(codes, scales, b, wq.WQ_LAYOUT_TILED)
    Y = host_bf16_bits(wq.wq_gemm(dev_bf16(A), W_d, wq.WQ_LAYOUT_TILED, None, N, b,
                                  zeros=torch.from_numpy(zeros).cuda()))
    mi, ni = sample_points(M, N, 2000, seed=25)
    y_ref, mag = oracle.wna16_points(A, packed, scales, b, mi, ni, zeros=zeros)
    assert_wna16(Y[mi, ni], y_ref, mag, "zp prefill sampled")


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("M,N,K", [(37, 200, 640), (256, 512, 1024)])
def test_gemm_a8_zero_points(M, N, K, layout):
    w = synth.w4a8(M=M, N=N, K=K, seed=2600 + M)
    zeros = np.random.default_rng(2601 + M).integers(0, 16, size=(N, K // 128), dtype=np.uint8)
    W_d, S_d, packed = _weights(w.codes, w.scales, 4, layout)
    y_ref, mag, _, _ = oracle.w4a8(w.A, packed, w.scales, zeros=zeros)
    Z = torch.from_numpy(zeros).cuda()
    Y = wq.wq_gemm_a8(dev_bf16(w.A), W_d, layout, S_d, N, 4, out_dtype=wq.WQ_OUT_F32, zeros=Z)
    torch.cuda.synchronize()
    assert_a8(Y.cpu().numpy().astype(np.float64), y_ref, mag, False, "a8 zp %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("b", [4, 8])
def test_embed_zero_points_and_per_channel(b):
    V, K = 300, 640
    rng = np.random.default_rng(2700 + b)
    codes = synth.draw_codes(rng, V, K, b)
    zeros = rng.integers(0, 1 << b, size=(V, K // 128), dtype=np.uint8)
    sg = synth.draw_scales_halfnormal_signed(rng, V, K // 128)
    s1 = synth.draw_scales_halfnormal_signed(rng, V, 1)
    packed = wq.wq_pack(codes, b)
    ids = np.concatenate([rng.integers(0, V, size=30), [-1, V, 0, V - 1]])
    ids_d = torch.from_numpy(ids).cuda()
    Z = torch.from_numpy(zeros).cuda()
    Y = wq.wq_embed(ids_d, dev_words(packed), dev_bf16(sg), K, b, zeros=Z)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bf16_bits(Y), oracle.embed(packed, sg, K, b, ids, zeros=zeros))
    Y = wq.wq_embed(ids_d, dev_words(packed), dev_bf16(s1), K, b, group=K, zeros=Z)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bf16_bits(Y),
                                  oracle.embed(packed, s1, K, b, ids, group=K, zeros=zeros))


def test_zero_points_refused_for_other_widths():
    A, codes, scales, zeros = _zp_workload(2, 64, 256, 6, 2800)
    W_d, _, _ = _weights(codes, scales, 6, wq.WQ_LAYOUT_TILED)
    with pytest.raises(wq.WQError) as e:
        wq.wq_gemm(dev_bf16(A), W_d, wq.WQ_LAYOUT_TILED, None, 64, 6,
                   zeros=torch.zeros((64, 2), dtype=torch.uint8, device="cuda"))
    assert e.value.status == wq.WQ_ERR_ZERO_POINTS


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("rows", [4, 8])
@pytest.mark.parametrize("b", [4, 8])
def test_gemm_zero_points_row_kernel(b, rows, layout, monkeypatch):
    # The one-row kernel without a K split, forced, with zero points.
    monkeypatch.setenv("WQ_DECODE_ROWS", str(rows))
    N, K = 333, 1920
    A, codes, scales, zeros = _zp_workload(1, N, K, b, 2500 + 10 * rows + b)
    W_d, S_d, packed = _weights(codes, scales, b, layout)
    Y = wq.wq_gemm(dev_bf16(A), W_d, layout, S_d, N, b, zeros=torch.from_numpy(zeros).cuda())
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16(A, packed, scales, b, zeros=zeros)
    assert_wna16(host_bf16_bits(Y), y_ref, mag, "zp row kernel b=%d rows=%d" % (b, rows))
