"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Unpacking is bit-exact; WNA16 outputs meet
|y - y_ref| <= 4e-3 sum|a w| + 1e-3; W4A8 activation codes are bit-exact and
its fp32 output is within 1e-5 of the oracle's magnitude sum."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_bit_wq_amd as wq
from weight_only_bit_wq_amd import synth
from gpu_util import (Layer, assert_a8, assert_wna16, bf16_values, dev_bf16, dev_words,
                      host_bf16_bits, sample_points)

pytestmark = pytest.mark.gpu

LAYOUTS = [wq.WQ_LAYOUT_DENSE, wq.WQ_LAYOUT_TILED]
LNAME = {wq.WQ_LAYOUT_DENSE: "dense", wq.WQ_LAYOUT_TILED: "tiled"}
BITS = [2, 3, 4, 5, 6, 7, 8]


def _workload(M, N, K, b, seed, scales="halfnormal"):
    rng = np.random.default_rng(seed)
    codes = synth.draw_codes(rng, N, K, b)
    if scales == "uniform":
        sc = synth.draw_scales_uniform(rng, N, K // 128)
    else:
        sc = synth.draw_scales_halfnormal_signed(rng, N, K // 128)
    A = synth.draw_act(rng, M, K)
    return synth.Workload(A, codes, sc, b)


def test_device_is_gfx950():
    assert torch.cuda.is_available()
    assert wq.wq_device_supported(torch.cuda.current_device())


# --- unpacker / repack ------------------------------------------------------------

@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("b", BITS)
def test_unpack_dev_bit_exact(b, layout):
    w = _workload(1, 200, 384, b, seed=200 + b)  # N ragged w.r.t. 64-row tiles
    packed = wq.wq_pack(w.codes, b)
    ref = oracle.unpack(oracle.pack(w.codes, b), w.K, b)
    np.testing.assert_array_equal(packed, oracle.pack(w.codes, b))
    L = Layer(w, layout, packed)
    codes = wq.wq_unpack_dev(L.W_d, layout, w.N, w.K, b)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref)


@pytest.mark.parametrize("b", [5, 6, 7])
def test_unpack_dev_decode_shape(b):
    w = synth.decode(M=1, b=b)
    L = Layer(w, wq.WQ_LAYOUT_TILED)
    codes = wq.wq_unpack_dev(L.W_d, wq.WQ_LAYOUT_TILED, w.N, w.K, b).cpu().numpy()
    rows = np.r_[0:64, w.N - 64:w.N]
    np.testing.assert_array_equal(codes[rows], oracle.unpack(oracle.pack(w.codes[rows], b), w.K, b))
    np.testing.assert_array_equal(codes, w.codes)


def _arranged_group_stream(c, b):
    """The 16b bytes of one row's group stream for b = 5, 6, 7 in the tiled
    layout, built from the 128 codes c by the rule wq.h states: v = c XOR
    2^(b-1), 4 runs of 32 values; byte k < 4b of a run holds u_k in its top b
    bits, the low 8 - b bits hold the bits of u_(4b) .. u_31 as listed."""
    out = np.zeros(16 * b, dtype=np.uint8)
    v = [int(x) ^ (1 << (b - 1)) for x in c]
    for q in range(4):
        u = v[32 * q:32 * q + 32]
        run = [(u[k] << (8 - b)) & 0xFF for k in range(4 * b)]

        def put(byte, bit, val):
            run[byte] |= val << bit
        for e in range(4):
            if b == 7:
                for i in range(7):
                    put(4 * i + e, 0, (u[28 + e] >> i) & 1)
            elif b == 6:
                for s in range(2):
                    x = u[24 + 4 * s + e]
                    put(12 * s + e, 0, (x >> 4) & 3)
                    put(12 * s + 4 + e, 0, (x >> 2) & 3)
                    put(12 * s + 8 + e, 0, x & 3)
            else:
                for s in range(2):
                    x = u[20 + 4 * s + e]
                    put(4 * s + e, 0, (x >> 2) & 7)
                    put(12 + 4 * s + e, 0, x & 3)
                x = u[28 + e]
                put(8 + e, 0, (x >> 2) & 7)
                put(12 + e, 2, (x >> 1) & 1)
                put(16 + e, 2, x & 1)
        out[4 * b * q:4 * b * (q + 1)] = run
    return out


@pytest.mark.parametrize("b", BITS)
def test_repack_matches_documented_tile_layout(b):
    w = _workload(1, 130, 256, b, seed=300 + b)
    L = Layer(w, wq.WQ_LAYOUT_TILED)
    blob = L.W_d.cpu().numpy()
    G = w.K // 128
    tb = 1024 * b + 128
    assert blob.size == 3 * G * tb
    dense = L.packed.view(np.uint8).reshape(w.N, -1)
    for n in (0, 63, 64, 129):
        for g in range(G):
            if b in (5, 6, 7):
                stream = _arranged_group_stream(w.codes[n, 128 * g:128 * (g + 1)], b)
            else:
                stream = dense[n, g * 16 * b:(g + 1) * 16 * b]
            tile = blob[((n // 64) * G + g) * tb:((n // 64) * G + g + 1) * tb]
            for j in range(b):
                got = tile[j * 1024 + (n % 64) * 16:j * 1024 + (n % 64) * 16 + 16]
                np.testing.assert_array_equal(got, stream[16 * j:16 * j + 16])
            s = tile[b * 1024:].view(np.uint16)
            assert s[n % 64] == w.scales[n, g]
    # padded rows 130..191 are zero
    last = blob[(2 * G) * tb:(2 * G + 1) * tb]
    assert not last[2 * 16:1024].any()


# --- WNA16 GEMM -----------------------------------------------------------------------

@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
def test_gemm_tiny_workload(layout):
    w = synth.tiny(0)
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, w.b), w.scales, w.b)
    assert_wna16(Layer(w, layout).gemm(), y_ref, mag, "tiny")


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 8, 13, 16])
@pytest.mark.parametrize("b", BITS)
def test_gemm_decode_path(b, M, layout):
    w = _workload(M, 300, 1280, b, seed=400 + 10 * b + M)
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, b), w.scales, b)
    assert_wna16(Layer(w, layout).gemm(), y_ref, mag, "decode b=%d M=%d" % (b, M))


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("M", [17, 100, 128, 130, 257])
@pytest.mark.parametrize("b", BITS)
def test_gemm_prefill_path(b, M, layout):
    # 64-row m-tiles up to M = 128 (100: a ragged second tile), 256-row above.
    w = _workload(M, 200, 640, b, seed=500 + 10 * b + M)
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, b), w.scales, b)
    assert_wna16(Layer(w, layout).gemm(), y_ref, mag, "prefill b=%d M=%d" % (b, M))


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("b", [5, 6, 7])
def test_gemm_decode_sweep_full_shape(b, M):
    w = synth.decode(M=M, b=b)
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, b), w.scales, b)
    assert_wna16(Layer(w, wq.WQ_LAYOUT_TILED).gemm(), y_ref, mag, "decode sweep b=%d M=%d" % (b, M))


@pytest.mark.parametrize("N,K,b", [(6437, 3840, 6), (4352, 5120, 5), (3200, 17408, 7),
                                   (2560, 10240, 8)])
def test_gemm_decode_m1_shapes(N, K, b):
    # M = 1 at shapes between the parity and the full sweep sizes (ragged N,
    # 30 to 136 groups, K split 1 to 5 ways); full outputs against the oracle.
    w = _workload(1, N, K, b, seed=900 + b)
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, b), w.scales, b)
    assert_wna16(Layer(w, wq.WQ_LAYOUT_TILED).gemm(), y_ref, mag, "decode M=1 N=%d K=%d b=%d" % (N, K, b))


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("M,N,K,b", [(300, 700, 5120, 6), (130, 1000, 3072, 3),
                                     (100, 700, 6144, 6), (40, 1000, 17408, 4)])
def test_gemm_prefill_k_split(M, N, K, b, layout):
    # Few output tiles: the prefill kernel splits K across workgroups (5, 3,
    # 6 and 17 splits here; the last two on 64-row tiles) and a reduce pass
    # adds the fp32 partials; full outputs.
    w = _workload(M, N, K, b, seed=950 + b)
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, b), w.scales, b)
    Y = Layer(w, layout).gemm()
    assert_wna16(Y, y_ref, mag, "prefill split M=%d b=%d" % (M, b))
    np.testing.assert_array_equal(Layer(w, layout).gemm(), Y)


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("M,N,K,b,bn0", [(800, 16590, 4096, 3, 122), (556, 16334, 8192, 6, 0)],
                         ids=["4parts", "2parts"])
def test_gemm_prefill_tail_split(M, N, K, b, bn0, layout):
    # Tiles of 256 x 128 with both edges ragged: 4 x 130 = 520 tiles, whose
    # last round of 8 (row tile 3, column tiles 122 .. 129) runs as 4 K parts
    # of 8 groups, or 3 x 128 = 384 tiles, whose last round is the whole last
    # row of tiles, as 2 parts of 32 groups.  Every output of the split tiles
    # (of the first and last three of that row), and a sample of the others,
    # against the oracle; a bitwise repeat.
    w = _workload(M, N, K, b, seed=980 + b)
    packed = oracle.pack(w.codes, b)
    m0 = (M - 1) // 256 * 256
    cols = np.arange(bn0 * 128, N)
    if len(cols) > 2048:  # the first three and the last three column tiles
        cols = np.concatenate([cols[:384], cols[-(N - (N - 1) // 128 * 128) - 256:]])
    tm, tn = np.meshgrid(np.arange(m0, M), cols, indexing="ij")
    si, sj = sample_points(M, N, 2000, seed=17 + b)
    mi = np.concatenate([tm.ravel(), si])
    ni = np.concatenate([tn.ravel(), sj])
    y_ref, mag = oracle.wna16_points(w.A, packed, w.scales, b, mi, ni)
    Y = Layer(w, layout).gemm()
    assert_wna16(Y[mi, ni], y_ref, mag, "prefill tail split M=%d b=%d" % (M, b))
    np.testing.assert_array_equal(Layer(w, layout).gemm(), Y)


@pytest.mark.parametrize("shape", [(5120, 17408), (17408, 5120)], ids=["up", "down"])
def test_gemm_prefill_full_shape_sampled(shape):
    K, N = shape
    w = synth.prefill(M=4096, N=N, K=K, b=6)
    L = Layer(w, wq.WQ_LAYOUT_TILED)
    Y = L.gemm()
    packed = oracle.pack(w.codes, 6)
    mi, ni = sample_points(w.M, w.N, 3000, seed=7)
    y_ref, mag = oracle.wna16_points(w.A, packed, w.scales, 6, mi, ni)
    assert_wna16(Y[mi, ni], y_ref, mag, "prefill %dx%dx%d" % (w.M, N, K))
    # whole rows and columns at the tile edges
    for m in (0, 127, 128, 4095):
        yr, mg = oracle.wna16_points(w.A, packed, w.scales, 6, np.full(N, m), np.arange(N))
        assert_wna16(Y[m], yr, mg, "prefill row %d" % m)


@pytest.mark.parametrize("shape", [(5120, 2176), (2176, 5120)], ids=["up_N2176", "down_K2176"])
def test_gemm_shard_shapes(shape):
    # One GPU's shard of the decode layer under an 8-way split (column-
    # parallel up projection N / 8, row-parallel down projection K / 8, whose
    # partial sums an all-reduce would add): the shapes bench.py times.
    # Decode rows in full, prefill M = 4096 on sampled points and edge rows.
    K, N = shape
    for M in (1, 4, 16):
        w = synth.decode(M=M, b=6, N=N, K=K)
        y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, 6), w.scales, 6)
        assert_wna16(Layer(w, wq.WQ_LAYOUT_TILED).gemm(), y_ref, mag,
                     "shard decode M=%d N=%d K=%d" % (M, N, K))
    w = synth.prefill(M=4096, N=N, K=K, b=6)
    Y = Layer(w, wq.WQ_LAYOUT_TILED).gemm()
    packed = oracle.pack(w.codes, 6)
    mi, ni = sample_points(w.M, w.N, 3000, seed=8)
    y_ref, mag = oracle.wna16_points(w.A, packed, w.scales, 6, mi, ni)
    assert_wna16(Y[mi, ni], y_ref, mag, "shard prefill %dx%dx%d" % (w.M, N, K))
    for m in (0, 255, 256, 4095):
        yr, mg = oracle.wna16_points(w.A, packed, w.scales, 6, np.full(N, m), np.arange(N))
        assert_wna16(Y[m], yr, mg, "shard prefill row %d" % m)


@pytest.mark.parametrize("M", [2, 20])
@pytest.mark.parametrize("b", BITS)
def test_hand_computed_example_exact(b, M):
    # The 2x3x128 example with a closed form (see tests/golden/hand_2x3x128.txt),
    # rows repeated to reach the decode (M=2) and prefill (M=20) paths.
    rows = [r for r in open(__file__.replace("test_gpu_parity.py", "golden/hand_2x3x128.txt"))
            if r.strip() and not r.startswith("#")]
    expect = {int(r.split()[0]): np.array([float(v) for v in r.split()[1:]]).reshape(2, 3)
              for r in rows}[b]
    K = 128
    A = np.stack([np.ones(K), (-1.0) ** np.arange(K)]).astype(np.float32)
    A = np.tile(A, (M // 2, 1))
    codes = np.stack([np.full(K, (1 << (b - 1)) + 1), np.arange(K) % (1 << b),
                      np.zeros(K)]).astype(np.uint8)
    scales = synth.f32_to_bf16_bits(np.array([[1.0], [-0.5], [2.0 ** -7]], dtype=np.float32))
    w = synth.Workload(synth.f32_to_bf16_bits(A), codes, scales, b)
    for layout in LAYOUTS:
        Y = bf16_values(Layer(w, layout).gemm())
        np.testing.assert_array_equal(Y, np.tile(expect, (M // 2, 1)))


@pytest.mark.parametrize("M", [3, 33])
def test_integer_invariant_b8(M):
    rng = np.random.default_rng(600 + M)
    N, K = 96, 512
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    A_int = rng.integers(-16, 17, size=(M, K))
    w = synth.Workload(synth.f32_to_bf16_bits(A_int.astype(np.float32)), codes,
                       np.full((N, K // 128), 0x3F80, dtype=np.uint16), 8)
    ref = (A_int @ (codes.astype(np.int64) - 128).T).astype(np.float32)
    for layout in LAYOUTS:
        np.testing.assert_array_equal(Layer(w, layout).gemm(), synth.f32_to_bf16_bits(ref))


@pytest.mark.parametrize("M", [1, 5, 16, 40, 300])
def test_negated_scales_negate_output_bitwise(M):
    # Every path keeps the scales out of the products: they enter once per
    # group in an fp32 multiply-add (tot += s * P) whose round-to-nearest-even
    # is sign-symmetric, as are the split-K sums and the bf16 rounding; so
    # negating every scale negates every output bit for bit, on the decode
    # kernel (M <= 16) and on the prefill kernel (64-row tiles at M = 40,
    # 256-row tiles with a K split at M = 300).
    w = _workload(M, 256, 1024, 6, seed=700 + M)
    Y1 = Layer(w, wq.WQ_LAYOUT_TILED).gemm()
    w2 = synth.Workload(w.A, w.codes, w.scales ^ np.uint16(0x8000), 6)
    Y2 = Layer(w2, wq.WQ_LAYOUT_TILED).gemm()
    np.testing.assert_array_equal(Y2, Y1 ^ np.uint16(0x8000))
    y_ref, mag = oracle.wna16(w2.A, oracle.pack(w2.codes, 6), w2.scales, 6)
    assert_wna16(Y2, y_ref, mag, "negated scales M=%d" % M)


@pytest.mark.parametrize("M", [1, 16, 64])
def test_deterministic(M):
    w = _workload(M, 17408 // 4, 5120, 6, seed=800 + M)
    L = Layer(w, wq.WQ_LAYOUT_TILED)
    np.testing.assert_array_equal(L.gemm(), L.gemm())


def test_empty_batch_is_noop():
    w = _workload(1, 64, 128, 6, seed=900)
    L = Layer(w, wq.WQ_LAYOUT_TILED)
    A = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    Y = wq.wq_gemm(A, L.W_d, L.layout, None, 64, 6)
    assert Y.shape == (0, 64)


def test_dense_and_tiled_agree_bitwise():
    w = _workload(8, 1000, 2048, 7, seed=901)
    np.testing.assert_array_equal(Layer(w, wq.WQ_LAYOUT_DENSE).gemm(),
                                  Layer(w, wq.WQ_LAYOUT_TILED).gemm())


# --- W4A8 ------------------------------------------------------------------------------

@pytest.mark.parametrize("M,K", [(1, 128), (7, 5120), (64, 1024), (300, 5120)])
def test_quant_act_bit_exact(M, K):
    w = synth.w4a8(M=M, N=8, K=K, seed=3)
    Aq, sa = wq.wq_quant_act_i8(dev_bf16(w.A))
    Aq_ref, sa_ref = oracle.quant_act_i8(w.A)
    np.testing.assert_array_equal(sa.cpu().numpy(), sa_ref)
    np.testing.assert_array_equal(Aq.cpu().numpy(), Aq_ref)


def test_quant_act_zero_row_and_ties():
    row = np.zeros(256, dtype=np.float32)
    row[:7] = [127.0, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5]
    A = synth.f32_to_bf16_bits(np.stack([row, np.zeros(256, dtype=np.float32)]))
    Aq, sa = wq.wq_quant_act_i8(dev_bf16(A))
    Aq_ref, sa_ref = oracle.quant_act_i8(A)
    np.testing.assert_array_equal(sa.cpu().numpy(), sa_ref)
    np.testing.assert_array_equal(Aq.cpu().numpy(), Aq_ref)


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (37, 200, 640), (256, 512, 1024), (130, 96, 5120)])
def test_gemm_a8_fp32(M, N, K, layout):
    w = synth.w4a8(M=M, N=N, K=K, seed=1000 + M)
    y_ref, mag, _, _ = oracle.w4a8(w.A, oracle.pack(w.codes, 4), w.scales)
    L = Layer(w, layout)
    assert_a8(L.gemm_a8(wq.WQ_OUT_F32), y_ref, mag, False, "a8 f32 %dx%dx%d" % (M, N, K))
    assert_a8(L.gemm_a8(wq.WQ_OUT_BF16), y_ref, mag, True, "a8 bf16 %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("M,N,K", [(37, 200, 640), (130, 96, 5120)])
@pytest.mark.parametrize("b", [2, 3, 5, 6, 7, 8])
def test_gemm_a8_other_widths(b, M, N, K, layout):
    # Int8 activations on b-bit codes (b = 8: W8A8): the same activations as
    # the W4A8 workload, codes of width b.
    w4 = synth.w4a8(M=M, N=N, K=K, seed=1300 + M + b)
    codes = synth.draw_codes(np.random.default_rng(1310 + b), N, K, b)
    w = synth.Workload(w4.A, codes, w4.scales, b)
    y_ref, mag, _, _ = oracle.w4a8(w.A, oracle.pack(codes, b), w.scales, b=b)
    L = Layer(w, layout)
    assert_a8(L.gemm_a8(wq.WQ_OUT_F32), y_ref, mag, False, "a8 b=%d f32 %dx%dx%d" % (b, M, N, K))
    assert_a8(L.gemm_a8(wq.WQ_OUT_BF16), y_ref, mag, True, "a8 b=%d bf16 %dx%dx%d" % (b, M, N, K))


@pytest.mark.parametrize("b", [2, 3, 5, 6, 7, 8])
def test_gemm_a8_on_grid_integer_exact_other_widths(b):
    rng = np.random.default_rng(1400 + b)
    M, N, K = 40, 64, 512
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    A_int = rng.integers(-127, 128, size=(M, K))
    A_int[:, 3] = 127
    w = synth.Workload(synth.f32_to_bf16_bits(A_int.astype(np.float32)), codes,
                       np.full((N, K // 128), 0x3F80, dtype=np.uint16), b)
    ref = (A_int @ (codes.astype(np.int64) - (1 << (b - 1))).T).astype(np.float64)
    for layout in LAYOUTS:
        np.testing.assert_array_equal(Layer(w, layout).gemm_a8(wq.WQ_OUT_F32), ref)


def test_gemm_a8_w8a8_full_shape_sampled():
    # W8A8 (8-bit codes, int8 activations) at the W4A8 prefill shape.
    w4 = synth.w4a8(M=2048)
    codes = synth.draw_codes(np.random.default_rng(1500), w4.N, w4.K, 8)
    w = synth.Workload(w4.A, codes, w4.scales, 8)
    Y = Layer(w, wq.WQ_LAYOUT_TILED).gemm_a8(wq.WQ_OUT_F32)
    Aq, sa = oracle.quant_act_i8(w.A)
    mi, ni = sample_points(w.M, w.N, 3000, seed=12)
    y_ref, mag = oracle.w4a8_points(Aq, sa, oracle.pack(codes, 8), w.scales, mi, ni, b=8)
    assert_a8(Y[mi, ni], y_ref, mag, False, "w8a8 full shape")


def test_gemm_a8_on_grid_integer_exact():
    rng = np.random.default_rng(1100)
    M, N, K = 40, 64, 512
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    A_int = rng.integers(-127, 128, size=(M, K))
    A_int[:, 3] = 127
    w = synth.Workload(synth.f32_to_bf16_bits(A_int.astype(np.float32)), codes,
                       np.full((N, K // 128), 0x3F80, dtype=np.uint16), 4)
    ref = (A_int @ (codes.astype(np.int64) - 8).T).astype(np.float64)
    np.testing.assert_array_equal(Layer(w, wq.WQ_LAYOUT_TILED).gemm_a8(wq.WQ_OUT_F32), ref)


@pytest.mark.parametrize("M", [2048, 8192])
def test_gemm_a8_full_shape_sampled(M):
    w = synth.w4a8(M=M)
    L = Layer(w, wq.WQ_LAYOUT_TILED)
    Y = L.gemm_a8(wq.WQ_OUT_F32)
    Aq, sa = oracle.quant_act_i8(w.A)
    mi, ni = sample_points(w.M, w.N, 3000, seed=11)
    y_ref, mag = oracle.w4a8_points(Aq, sa, oracle.pack(w.codes, 4), w.scales, mi, ni)
    assert_a8(Y[mi, ni], y_ref, mag, False, "a8 full shape")


@pytest.mark.parametrize("b,layout", [(4, wq.WQ_LAYOUT_TILED), (4, wq.WQ_LAYOUT_DENSE),
                                      (6, wq.WQ_LAYOUT_TILED)], ids=["b4-tiled", "b4-dense", "b6-tiled"])
def test_gemm_a8_tail_split(b, layout):
    # 258 tiles of 256 x 128 (M 300 and N 16500: both edges ragged), K 2048:
    # the last round's 2 tiles (row tile 1, column tiles 127 and 128) run as
    # 4 K parts of 4 groups each, added by the second kernel.  Every output
    # of those tiles, and a sample of the others, against the oracle, in
    # both output types.
    M, N, K = 300, 16500, 2048
    w4 = synth.w4a8(M=M, N=N, K=K, seed=1500 + b)
    codes = w4.codes if b == 4 else synth.draw_codes(np.random.default_rng(1510 + b), N, K, b)
    w = synth.Workload(w4.A, codes, w4.scales, b)
    L = Layer(w, layout)
    Aq, sa = oracle.quant_act_i8(w.A)
    tm, tn = np.meshgrid(np.arange(256, M), np.arange(127 * 128, N), indexing="ij")
    si, sj = sample_points(M, N, 2000, seed=15 + b)
    mi = np.concatenate([tm.ravel(), si])
    ni = np.concatenate([tn.ravel(), sj])
    y_ref, mag = oracle.w4a8_points(Aq, sa, oracle.pack(codes, b), w.scales, mi, ni, b=b)
    Y = L.gemm_a8(wq.WQ_OUT_F32)
    assert_a8(Y[mi, ni], y_ref, mag, False, "a8 tail split b=%d f32" % b)
    Yb = L.gemm_a8(wq.WQ_OUT_BF16)
    assert_a8(Yb[mi, ni], y_ref, mag, True, "a8 tail split b=%d bf16" % b)


def test_gemm_a8_negated_scales():
    w = synth.w4a8(M=64, N=128, K=1024, seed=1200)
    Y1 = Layer(w, wq.WQ_LAYOUT_TILED).gemm_a8(wq.WQ_OUT_F32)
    w2 = synth.Workload(w.A, w.codes, w.scales ^ np.uint16(0x8000), 4)
    Y2 = Layer(w2, wq.WQ_LAYOUT_TILED).gemm_a8(wq.WQ_OUT_F32)
    np.testing.assert_array_equal(Y2, -Y1)


def test_workspace_reused_across_shapes_and_ops():
    # One workspace for a sequence of calls with different split layouts and
    # a W4A8 call in between: the counter region must stay valid throughout.
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    cases = [(16, 6, 1000, 1280), (1, 3, 300, 1280), (4, 7, 520, 2560), (1, 5, 64, 384)]
    for M, b, N, K in cases:
        w = _workload(M, N, K, b, seed=1300 + M + b)
        L = Layer(w, wq.WQ_LAYOUT_TILED)
        Y = wq.wq_gemm(dev_bf16(w.A), L.W_d, L.layout, None, N, b, ws=ws)
        torch.cuda.synchronize()
        y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, b), w.scales, b)
        assert_wna16(host_bf16_bits(Y), y_ref, mag, "ws reuse b=%d M=%d" % (b, M))
        w4 = synth.w4a8(M=20, N=64, K=256, seed=1400 + M)
        L4 = Layer(w4, wq.WQ_LAYOUT_TILED)
        wq.wq_gemm_a8(dev_bf16(w4.A), L4.W_d, L4.layout, None, 64, 4, ws=ws)
    torch.cuda.synchronize()
    assert not ws[:wq.WORKSPACE_ZERO_BYTES].any()


@pytest.mark.parametrize("b,M,K,N", [(6, 1, 5120, 17408), (6, 4, 17408, 5120), (5, 16, 5120, 17408)])
def test_split_k_handoff_repeated(b, M, K, N):
    # The split-K partial sums cross workgroups (and XCDs) through device-scope
    # atomics; 30 back-to-back calls must all equal the first, which matches
    # the oracle.
    w = synth.decode(M=M, b=b, N=N, K=K)
    L = Layer(w, wq.WQ_LAYOUT_TILED)
    A = dev_bf16(w.A)
    Y0 = wq.wq_gemm(A, L.W_d, L.layout, None, N, b)
    outs = [wq.wq_gemm(A, L.W_d, L.layout, None, N, b) for _ in range(30)]
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, b), w.scales, b)
    assert_wna16(host_bf16_bits(Y0), y_ref, mag, "split-K b=%d M=%d" % (b, M))
    for Y in outs:
        assert torch.equal(Y.view(torch.int16), Y0.view(torch.int16))



@pytest.mark.parametrize("reduce", [0, 1], ids=["handoff", "reduce"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("waves", [4, 8, 16])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 6, 8, 13, 16])
def test_decode_split_k_forced(M, waves, layout, reduce, monkeypatch):
    # The lane-per-row decode kernel's split-K sum at every row tile and
    # wave count it supports, either handed off inside the kernel (one
    # ticket per row block and storing wave, the other waves leaving after
    # the LDS sum) or by the second kernel that adds the stored partials, on
    # a small ragged layer with K forced into 4 splits of 3 groups (the
    # default plan would not split it): full outputs against the oracle, a
    # bitwise repeat, the counter region left zero, and (second kernel) the
    # same bits as the hand-off, which adds in the same order.  Row tiles
    # above 1 take the 4x4x4 matrix-core form.
    mt = 1 if M <= 1 else 4 if M <= 4 else 8 if M <= 8 else 16
    if waves == 16 and mt > 4:
        pytest.skip("wave count not offered for this row tile")
    monkeypatch.setenv("WQ_DECODE_ROWS", "0")  # M = 1 would take the row kernel
    monkeypatch.setenv("WQ_DECODE_WAVES", str(waves))
    monkeypatch.setenv("WQ_DECODE_SPLITS", "4")
    monkeypatch.setenv("WQ_DECODE_REDUCE", str(reduce))
    b, N, K = 6, 200, 1536
    w = _workload(M, N, K, b, seed=1600 + 17 * M + waves)
    L = Layer(w, layout)
    ws = torch.zeros(8 << 20, dtype=torch.uint8, device="cuda")
    A = dev_bf16(w.A)
    Y0 = wq.wq_gemm(A, L.W_d, L.layout, L.S_d, N, b, ws=ws)
    Y1 = wq.wq_gemm(A, L.W_d, L.layout, L.S_d, N, b, ws=ws)
    torch.cuda.synchronize()
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, b), w.scales, b)
    assert_wna16(host_bf16_bits(Y0), y_ref, mag,
                 "forced split-K M=%d waves=%d reduce=%d" % (M, waves, reduce))
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
    assert not ws[:wq.WORKSPACE_ZERO_BYTES].any()
    if reduce:
        monkeypatch.setenv("WQ_DECODE_REDUCE", "0")
        Yh = wq.wq_gemm(A, L.W_d, L.layout, L.S_d, N, b, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(Y0.view(torch.int16), Yh.view(torch.int16))
        assert not ws[:wq.WORKSPACE_ZERO_BYTES].any()


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: LNAME[l])
@pytest.mark.parametrize("share", [1, 2, 4])
@pytest.mark.parametrize("rows", [4, 8])
@pytest.mark.parametrize("N,K", [(300, 128), (777, 640), (200, 5120), (130, 17408)])
@pytest.mark.parametrize("b", BITS)
def test_decode_row_kernel_forced(b, N, K, rows, share, layout, monkeypatch):
    # The one-row kernel without a cross-workgroup K split (a wave owns 8 or
    # 4 rows, 8 or 16 lanes per row take every 8th or 16th group, 1, 2 or 4
    # waves of a workgroup share a row set's groups; the lanes' sums meet by
    # DPP, the waves' in LDS), forced onto small ragged layers: 1 to 136
    # groups, groups per lane not a whole number, waves with no group at
    # all, rows past N in the last wave; full outputs against the oracle and
    # a bitwise repeat.
    monkeypatch.setenv("WQ_DECODE_ROWS", str(rows))
    monkeypatch.setenv("WQ_DECODE_ROW_WAVES", str(share))
    w = _workload(1, N, K, b, seed=3000 + 7 * b + N + K)
    assert wq.wq_workspace_bytes(wq.WQ_OP_GEMM, 1, N, K, b) == 0
    L = Layer(w, layout)
    y_ref, mag = oracle.wna16(w.A, oracle.pack(w.codes, b), w.scales, b)
    Y = L.gemm()
    assert_wna16(Y, y_ref, mag, "row kernel b=%d N=%d K=%d rows=%d" % (b, N, K, rows))
    np.testing.assert_array_equal(L.gemm(), Y)
