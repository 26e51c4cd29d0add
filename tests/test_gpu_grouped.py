"""GPU parity of the grouped (mixture-of-experts) WNA16 layer (wq_gemm_grouped,
through the C ABI) against the CPU oracle: experts with no rows, decode-sized
and prefill-sized row blocks in one call, with and without zero points.
Page: model card "Qwen3.8-27B-INT6-Mixed-AutoRound", Findings (the dense
format has no fused MoE path)."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_wq_amd as wq
from weight_only_bit_wq_amd import synth
from gpu_util import assert_wna16, dev_bf16, dev_words, host_bf16_bits

pytestmark = pytest.mark.gpu


def _experts(E, N, K, b, seed, zp=False):
    rng = np.random.default_rng(seed)
    codes = synth.draw_codes(rng, E * N, K, b)
    scales = synth.draw_scales_halfnormal_signed(rng, E * N, K // 128)
    zeros = rng.integers(0, 1 << b, size=(E * N, K // 128), dtype=np.uint8) if zp else None
    packed = wq.wq_pack(codes, b)
    eb = wq.wq_repacked_bytes(wq.WQ_LAYOUT_TILED, N, K, b)
    W = torch.empty(E * eb, dtype=torch.uint8, device="cuda")
    for e in range(E):
        wq.wq_repack(dev_words(packed[e * N:(e + 1) * N]), dev_bf16(scales[e * N:(e + 1) * N]),
                     K, b, out=W[e * eb:(e + 1) * eb])
    return packed, scales, zeros, W, eb


@pytest.mark.parametrize("b,zp", [(4, False), (4, True), (6, False), (8, True)])
def test_grouped_mixed_sizes(b, zp):
    E, N, K = 7, 200, 1024
    sizes = [3, 0, 1, 40, 16, 0, 17]   # empty, decode row tiles, prefill
    off = np.concatenate([[0], np.cumsum(sizes)])
    packed, scales, zeros, W, eb = _experts(E, N, K, b, 3000 + b + 10 * zp, zp)
    A = synth.draw_act(np.random.default_rng(3001 + b), int(off[-1]), K)
    print("grouped b=%d zp=%d rows=%s" % (b, zp, sizes), flush=True)
    Z = torch.from_numpy(zeros).cuda() if zp else None
    Y = wq.wq_gemm_grouped(dev_bf16(A), W, eb, off, N, b, zeros=Z)
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16_grouped(A, packed, scales, b, off, zeros=zeros)
    assert_wna16(host_bf16_bits(Y), y_ref, mag, "grouped b=%d zp=%d" % (b, zp))


@pytest.mark.parametrize("b,zp", [(3, False), (6, False), (4, True), (8, True)])
def test_grouped_tile_boundaries(b, zp):
    # Expert sizes on both sides of every tile boundary: 64-row tiles below
    # 192 remaining rows (64, 65, 191, 17, 128), 256-row tiles from 192 (192,
    # 257 = 256 + a 1-row small tile, 449 = 256 + 193); K = 6144 (48
    # groups), N = 136 (a ragged n-tile).
    E, N, K = 10, 136, 6144
    sizes = [64, 65, 191, 192, 257, 449, 17, 128, 0, 5]
    off = np.concatenate([[0], np.cumsum(sizes)])
    packed, scales, zeros, W, eb = _experts(E, N, K, b, 3050 + b + 10 * zp, zp)
    A = synth.draw_act(np.random.default_rng(3051 + b), int(off[-1]), K)
    print("grouped tiles b=%d zp=%d rows=%s" % (b, zp, sizes), flush=True)
    Z = torch.from_numpy(zeros).cuda() if zp else None
    Y = wq.wq_gemm_grouped(dev_bf16(A), W, eb, off, N, b, zeros=Z)
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16_grouped(A, packed, scales, b, off, zeros=zeros)
    assert_wna16(host_bf16_bits(Y), y_ref, mag, "grouped tiles b=%d zp=%d" % (b, zp))


def test_grouped_decode_routing():
    # One token routed to 4 of 16 experts (rows sorted by expert), b = 4.
    E, N, K, b = 16, 512, 2048, 4
    packed, scales, _, W, eb = _experts(E, N, K, b, 3100)
    active = [2, 5, 11, 14]
    sizes = [1 if e in active else 0 for e in range(E)]
    off = np.concatenate([[0], np.cumsum(sizes)])
    A = np.repeat(synth.draw_act(np.random.default_rng(3101), 1, K), 4, axis=0)
    Y = wq.wq_gemm_grouped(dev_bf16(A), W, eb, off, N, b)
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16_grouped(A, packed, scales, b, off)
    assert_wna16(host_bf16_bits(Y), y_ref, mag, "grouped decode routing")
    # each output row is that expert's dense layer on the token
    for i, e in enumerate(active):
        blob = W[e * eb:(e + 1) * eb]
        Ye = wq.wq_gemm(dev_bf16(A[i:i + 1]), blob, wq.WQ_LAYOUT_TILED, None, N, b)
        torch.cuda.synchronize()
        assert torch.equal(Ye.view(torch.int16), Y[i:i + 1].view(torch.int16))


@pytest.mark.parametrize("b", [4, 6])
def test_grouped_many_experts_ragged(b):
    # 40 experts with a ragged N (not a multiple of 64), most with decode-
    # sized row blocks, a few with prefill-sized ones (300 rows: a 256-row
    # and a 64-row tile; 20 rows: a 64-row tile).
    E, N, K = 40, 200, 640
    rng = np.random.default_rng(3200 + b)
    sizes = rng.integers(0, 6, size=E)
    sizes[[3, 17]] = [300, 20]
    sizes[[5, 6, 30]] = 0
    off = np.concatenate([[0], np.cumsum(sizes)])
    packed, scales, _, W, eb = _experts(E, N, K, b, 3210 + b)
    A = synth.draw_act(rng, int(off[-1]), K)
    ws = torch.zeros(wq.wq_grouped_workspace_bytes(off, N, K, b) + 256, dtype=torch.uint8,
                     device="cuda")
    Y0 = wq.wq_gemm_grouped(dev_bf16(A), W, eb, off, N, b, ws=ws)
    Y1 = wq.wq_gemm_grouped(dev_bf16(A), W, eb, off, N, b, ws=ws)
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16_grouped(A, packed, scales, b, off)
    assert_wna16(host_bf16_bits(Y0), y_ref, mag, "grouped many b=%d" % b)
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
    assert not ws[:wq.WORKSPACE_ZERO_BYTES].any()


def test_grouped_table_overflow():
    # 260 experts of 17..40 rows: more 64-row tiles than one launch's table
    # holds (240 entries), so the call spans two prefill launches.
    E, N, K, b = 260, 64, 256, 5
    rng = np.random.default_rng(3300)
    sizes = rng.integers(17, 41, size=E)
    off = np.concatenate([[0], np.cumsum(sizes)])
    packed, scales, _, W, eb = _experts(E, N, K, b, 3301)
    A = synth.draw_act(rng, int(off[-1]), K)
    print("grouped overflow E=%d rows=%d" % (E, off[-1]), flush=True)
    Y = wq.wq_gemm_grouped(dev_bf16(A), W, eb, off, N, b)
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16_grouped(A, packed, scales, b, off)
    assert_wna16(host_bf16_bits(Y), y_ref, mag, "grouped overflow")


def test_grouped_overflow_with_split_decode_expert():
    # A 300-row expert first, then 239 prefill-sized experts (more 64-row
    # tiles than one table holds, so prefill launches come before and after
    # the decode table) and a 3-row expert whose decode table splits K: its
    # partials live in the workspace while prefill tiles of the first
    # expert are still pending.  Every prefill launch must be unaffected.
    E, N, K, b = 241, 64, 2048, 5
    sizes = [300] + [20] * 239 + [3]
    off = np.concatenate([[0], np.cumsum(sizes)])
    need = wq.wq_grouped_workspace_bytes(off, N, K, b)
    assert need > wq.WORKSPACE_ZERO_BYTES  # the decode table is split
    packed, scales, _, W, eb = _experts(E, N, K, b, 3400)
    A = synth.draw_act(np.random.default_rng(3401), int(off[-1]), K)
    print("grouped overflow + split decode rows=%d ws=%d" % (off[-1], need), flush=True)
    Y = wq.wq_gemm_grouped(dev_bf16(A), W, eb, off, N, b)
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16_grouped(A, packed, scales, b, off)
    assert_wna16(host_bf16_bits(Y), y_ref, mag, "grouped overflow + split decode")
