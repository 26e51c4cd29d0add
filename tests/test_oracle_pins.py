"""Pins for the CPU oracle: each test ties the oracle to something other than
itself (a worked example or figure printed on the pages, a closed form, an
invariant, a library routine on a special case, or exact brute force).

Pages cited by title and section:
  [card]  model card "Qwen3.8-27B-INT6-Mixed-AutoRound"
  [int57] "vLLM Can Run INT5-7" (minamism.com)
  [w4a8]  club-3090 discussion #733 on int8 activations (W4A8)
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from weight_only_bit_wq_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BF16_ONE = 0x3F80


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _stream_words(codes_row, b):
    """Dense LSB-first stream of one row as a Python big integer, cut into
    32-bit words: an independent definition of the packed layout."""
    acc = 0
    for k, c in enumerate(codes_row):
        acc |= int(c) << (k * b)
    nwords = (len(codes_row) * b + 31) // 32
    return [(acc >> (32 * j)) & 0xFFFFFFFF for j in range(nwords)]


# --- packing -----------------------------------------------------------------

def test_packed_row_length_worked_example():
    # [card] Findings: 5120 codes at 6 bits -> 960 words (legacy formula 1024).
    (K, b, dense, legacy), = [tuple(int(v) for v in r) for r in _golden_rows("packed_shape.txt")]
    assert oracle.words_per_row(K, b) == dense
    assert K // (32 // b) == legacy
    codes = np.zeros((2, K), dtype=np.uint8)
    assert oracle.pack(codes, b).shape == (2, dense)


@pytest.mark.parametrize("b", [4, 5, 6, 7, 8])
@pytest.mark.parametrize("K", [5120, 17408])
def test_packed_shape_at_exported_widths(b, K):
    # [card] "Reproducing this model": export shapes match ceil(in * bits / 32).
    codes = np.zeros((1, K), dtype=np.uint8)
    assert oracle.pack(codes, b).shape == (1, math.ceil(K * b / 32))


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 7, 8])
def test_legacy_per_word_formula_agrees_only_when_b_divides_32(b):
    # [card] Findings: the per-word formula (packed_idx = col // PF,
    # shift = (col % PF) * bits, PF = 32 // bits) reads the dense layout only
    # for widths that divide 32.  This pins the LSB-first bit order for 2/4/8.
    rng = np.random.default_rng(10 + b)
    K = 5120
    codes = rng.integers(0, 1 << b, size=(3, K), dtype=np.uint8)
    packed = oracle.pack(codes, b)
    pf = 32 // b
    legacy_words = -(-K // pf)
    if 32 % b == 0:
        assert legacy_words == packed.shape[1]
        col = np.arange(K)
        got = (packed[:, col // pf] >> ((col % pf) * b).astype(np.uint32)) & ((1 << b) - 1)
        np.testing.assert_array_equal(got.astype(np.uint8), codes)
    else:
        assert legacy_words != packed.shape[1]


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 7, 8])
def test_pack_equals_big_integer_stream(b):
    rng = np.random.default_rng(20 + b)
    codes = rng.integers(0, 1 << b, size=(3, 256), dtype=np.uint8)
    packed = oracle.pack(codes, b)
    for n in range(3):
        assert [int(w) for w in packed[n]] == _stream_words(codes[n], b)


def test_pack_literal_words_for_nibbles_and_bytes():
    # For b = 4 and 8 the dense stream is the familiar nibble / byte order.
    k = np.arange(32, dtype=np.uint8)
    p4 = oracle.pack((k % 16)[None, :], 4)
    assert [int(w) for w in p4[0, :2]] == [0x76543210, 0xFEDCBA98]
    p8 = oracle.pack(k[None, :], 8)
    assert int(p8[0, 0]) == 0x03020100 and int(p8[0, 7]) == 0x1F1E1D1C


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 7, 8])
def test_roundtrip_every_code_value(b):
    # Every code value at every position modulo the word period.
    K = 128 * 4
    n_vals = 1 << b
    codes = np.stack([(np.arange(K) + r) % n_vals for r in range(n_vals)]).astype(np.uint8)
    np.testing.assert_array_equal(oracle.unpack(oracle.pack(codes, b), K, b), codes)


@pytest.mark.parametrize("b", [2, 5, 6, 7])
def test_row_padding_is_zero(b):
    # A row whose bit count is not a multiple of 32 is zero-padded.
    codes = np.full((2, 7), (1 << b) - 1, dtype=np.uint8)
    packed = oracle.pack(codes, b)
    used = 7 * b
    last = int(packed[0, -1])
    assert last >> (used - 32 * (packed.shape[1] - 1)) == 0
    np.testing.assert_array_equal(oracle.unpack(packed, 7, b), codes)


def test_pack_rejects_out_of_range_code():
    codes = np.zeros((1, 128), dtype=np.uint8)
    codes[0, 5] = 64
    with pytest.raises(ValueError):
        oracle.pack(codes, 6)


def test_vocab_int8_frees_233_gib():
    # [int57] section 3: vocabulary layers in INT8 instead of BF16 free 2.33 GiB.
    (V, H, per_layer, freed), = [r for r in _golden_rows("vocab_int8_freed.txt")]
    V, H, per_layer, freed = int(V), int(H), float(per_layer), float(freed)
    gib = float(1 << 30)
    bf16 = V * H * 2 / gib
    packed8 = V * oracle.words_per_row(H, 8) * 4 / gib
    scales = V * (H // 128) * 2 / gib
    assert round(bf16, 2) == per_layer
    assert round(2 * (bf16 - packed8 - scales), 2) == freed


# --- WNA16 arithmetic ----------------------------------------------------------

def _hand_inputs(b):
    K = 128
    A = np.stack([np.ones(K), (-1.0) ** np.arange(K)]).astype(np.float32)
    codes = np.stack([np.full(K, (1 << (b - 1)) + 1),
                      np.arange(K) % (1 << b),
                      np.zeros(K)]).astype(np.uint8)
    scales = _bf16(np.array([[1.0], [-0.5], [2.0 ** -7]]))
    return _bf16(A), codes, scales


@pytest.mark.parametrize("row", _golden_rows("hand_2x3x128.txt"), ids=lambda r: "b%s" % r[0])
def test_hand_computed_example(row):
    b = int(row[0])
    expect = np.array([float(v) for v in row[1:]]).reshape(2, 3)
    A, codes, scales = _hand_inputs(b)
    y, mag = oracle.wna16(A, oracle.pack(codes, b), scales, b)
    np.testing.assert_array_equal(y, expect)
    assert np.all(mag >= np.abs(y))


def test_integer_invariant_b8_unit_scale():
    # b = 8, every scale 1: the layer is the integer product A . (c - 128)^T.
    rng = np.random.default_rng(5)
    M, N, K = 5, 33, 384
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    A_int = rng.integers(-16, 17, size=(M, K))
    A = _bf16(A_int.astype(np.float32))
    scales = np.full((N, K // 128), BF16_ONE, dtype=np.uint16)
    y, _ = oracle.wna16(A, oracle.pack(codes, 8), scales, 8)
    ref = A_int.astype(np.int64) @ (codes.astype(np.int64) - 128).T
    np.testing.assert_array_equal(y, ref.astype(np.float64))


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 7, 8])
def test_power_of_two_scales_match_bf16_dequant_and_linear(b):
    # Special case where dequantizing to bf16 is exact (scale a power of two,
    # |q| <= 128): the layer equals torch's F.linear on the bf16 weights, the
    # pages' own definition of the result ([int57] section 2).
    rng = np.random.default_rng(30 + b)
    M, N, K = 3, 17, 512
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    e = rng.integers(-9, -3, size=(N, K // 128))
    sgn = np.where(rng.integers(0, 2, size=e.shape) == 1, -1.0, 1.0)
    s = (sgn * np.exp2(e)).astype(np.float32)
    scales = _bf16(s)
    A = _bf16(rng.normal(size=(M, K)).astype(np.float32))
    y, mag = oracle.wna16(A, oracle.pack(codes, b), scales, b)
    q = codes.astype(np.float32) - (1 << (b - 1))
    w_bf16 = torch.from_numpy(np.repeat(s, 128, axis=1) * q).to(torch.bfloat16)
    assert torch.equal(w_bf16.float(), torch.from_numpy(np.repeat(s, 128, axis=1) * q))
    a = torch.from_numpy(synth.bf16_bits_to_f32(A)).double()
    ref = torch.nn.functional.linear(a, w_bf16.double()).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * mag.max())


@pytest.mark.parametrize("b", [3, 5, 6, 7])
def test_exact_rational_brute_force(b):
    # Tiny case in exact rational arithmetic, codes read from the big-integer
    # stream definition (not from the oracle's unpacker).
    rng = np.random.default_rng(40 + b)
    M, N, K = 2, 3, 256
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    scales = synth.draw_scales_uniform(rng, N, K // 128)
    A = _bf16(rng.normal(size=(M, K)).astype(np.float32))
    packed = oracle.pack(codes, b)
    y, mag = oracle.wna16(A, packed, scales, b)
    a = synth.bf16_bits_to_f32(A)
    s = synth.bf16_bits_to_f32(scales)
    for n in range(N):
        stream = 0
        for j, wd in enumerate(packed[n]):
            stream |= int(wd) << (32 * j)
        c = [(stream >> (k * b)) & ((1 << b) - 1) for k in range(K)]
        for m in range(M):
            exact = sum(Fraction(float(a[m, k])) * Fraction(float(s[n, k // 128])) *
                        (c[k] - (1 << (b - 1))) for k in range(K))
            exact_mag = sum(abs(Fraction(float(a[m, k])) * Fraction(float(s[n, k // 128])) *
                                (c[k] - (1 << (b - 1)))) for k in range(K))
            bound = K * 2.0 ** -52 * float(exact_mag)
            assert abs(y[m, n] - float(exact)) <= bound
            assert abs(mag[m, n] - float(exact_mag)) <= bound


def test_negated_scales_negate_output():
    w = synth.tiny(0)
    packed = oracle.pack(w.codes, w.b)
    y, mag = oracle.wna16(w.A, packed, w.scales, w.b)
    y2, mag2 = oracle.wna16(w.A, packed, w.scales ^ np.uint16(0x8000), w.b)
    np.testing.assert_array_equal(y2, -y)
    np.testing.assert_array_equal(mag2, mag)


def test_group_scales_act_on_their_own_128_columns():
    # Zeroing the scale of group g removes exactly the contribution of input
    # columns [128 g, 128 g + 128); checked against the layer with those
    # activation columns zeroed instead.
    w = synth.tiny(0)
    packed = oracle.pack(w.codes, w.b)
    for g in range(w.K // 128):
        sc = w.scales.copy()
        sc[:, g] = 0
        A0 = w.A.copy()
        A0[:, 128 * g:128 * (g + 1)] = 0
        y1, _ = oracle.wna16(w.A, packed, sc, w.b)
        y2, _ = oracle.wna16(A0, packed, w.scales, w.b)
        np.testing.assert_allclose(y1, y2, rtol=0, atol=1e-15)


def test_points_equal_full_layer():
    w = synth.tiny(0)
    packed = oracle.pack(w.codes, w.b)
    y, mag = oracle.wna16(w.A, packed, w.scales, w.b)
    rng = np.random.default_rng(0)
    mi = rng.integers(0, w.M, 50)
    ni = rng.integers(0, w.N, 50)
    yp, magp = oracle.wna16_points(w.A, packed, w.scales, w.b, mi, ni)
    np.testing.assert_array_equal(yp, y[mi, ni])
    np.testing.assert_array_equal(magp, mag[mi, ni])


# --- W4A8 ---------------------------------------------------------------------

def test_int4_widening_is_lossless():
    # [w4a8] "Under the hood": int4 weights widen to int8 without loss.
    c = np.arange(16)
    q = c - 8
    assert q.min() == -8 and q.max() == 7
    np.testing.assert_array_equal(q.astype(np.int8).astype(np.int64), q)


def test_quant_act_on_grid_rows_are_exact():
    rng = np.random.default_rng(6)
    A_int = rng.integers(-127, 128, size=(4, 256))
    A_int[:, 3] = 127
    A_int[1, 3] = -127
    Aq, sa = oracle.quant_act_i8(_bf16(A_int.astype(np.float32)))
    np.testing.assert_array_equal(sa, np.ones(4, dtype=np.float32))
    np.testing.assert_array_equal(Aq.astype(np.int64), A_int)


def test_quant_act_rounds_half_to_even_and_zero_row():
    row = np.zeros(128, dtype=np.float32)
    row[:7] = [127.0, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5]
    A = _bf16(np.stack([row, np.zeros(128, dtype=np.float32)]))
    Aq, sa = oracle.quant_act_i8(A)
    assert sa[0] == 1.0 and sa[1] == 0.0
    assert list(Aq[0, :7]) == [127, 2, 4, -2, 0, 0, 2]
    assert not np.any(Aq[1])


def test_quant_act_error_bound_and_full_range():
    w = synth.w4a8(M=16, N=8, K=512, seed=3)
    Aq, sa = oracle.quant_act_i8(w.A)
    a = synth.bf16_bits_to_f32(w.A).astype(np.float64)
    amax = np.abs(a).max(axis=1)
    assert np.all(np.abs(Aq).max(axis=1) == 127)
    np.testing.assert_allclose(sa.astype(np.float64), amax / 127, rtol=2 ** -23)
    err = np.abs(a - sa[:, None].astype(np.float64) * Aq)
    assert np.all(err <= sa[:, None] * (0.5 + 1e-6))


def test_quant_act_matches_fp32_numpy_convention():
    # The fp32 convention (IEEE division, ties-to-even rint, clamp 127) is a
    # reading; this only checks the C code follows it in fp32 throughout.
    w = synth.w4a8(M=32, N=8, K=1024, seed=7)
    Aq, sa = oracle.quant_act_i8(w.A)
    a = synth.bf16_bits_to_f32(w.A)
    s = (np.abs(a).max(axis=1) / np.float32(127)).astype(np.float32)
    q = np.clip(np.rint(a / s[:, None]), -127, 127).astype(np.int8)
    np.testing.assert_array_equal(sa, s)
    np.testing.assert_array_equal(Aq, q)


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 7, 8])
def test_w4a8_on_grid_integer_product(b):
    # Activations already on the int8 grid (a 127 in every row, so s_a = 1)
    # and unit scales: the layer is the integer product A . (c - 2^(b-1))^T.
    rng = np.random.default_rng(8 + 100 * b)
    M, N, K = 6, 40, 512
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    A_int = rng.integers(-127, 128, size=(M, K))
    A_int[:, 0] = 127
    scales = np.full((N, K // 128), BF16_ONE, dtype=np.uint16)
    y, mag, Aq, sa = oracle.w4a8(_bf16(A_int.astype(np.float32)), oracle.pack(codes, b), scales,
                                 b=b)
    ref = A_int.astype(np.int64) @ (codes.astype(np.int64) - (1 << (b - 1))).T
    np.testing.assert_array_equal(y, ref.astype(np.float64))


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 7, 8])
def test_w4a8_equals_wna16_b4_for_on_grid_activations(b):
    rng = np.random.default_rng(9 + 100 * b)
    M, N, K = 4, 24, 768
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    A_int = rng.integers(-127, 128, size=(M, K))
    A_int[:, 5] = -127
    A = _bf16(A_int.astype(np.float32))
    scales = synth.draw_scales_halfnormal_signed(rng, N, K // 128)
    packed = oracle.pack(codes, b)
    y8, mag8, _, _ = oracle.w4a8(A, packed, scales, b=b)
    y16, mag16 = oracle.wna16(A, packed, scales, b)
    np.testing.assert_allclose(y8, y16, rtol=0, atol=1e-12 * mag16.max())
    np.testing.assert_allclose(mag8 >= np.abs(y8), True)


@pytest.mark.parametrize("b", [4, 6])
def test_w4a8_exact_rational_brute_force(b):
    # y and its tolerance denominator mag = |s_a| * sum_g |s_g * acc_g| in
    # exact rational arithmetic, from codes read off the big-integer stream
    # and activation codes from the fp32 numpy convention (not the oracle's
    # own unpacker or quantizer).  The absolute value sits outside each
    # group's integer sum [w4a8 Under the hood: group scales applied to the
    # int products]; moving it inside (a looser bound) must fail here, so
    # the case is checked to tell the two apart.
    rng = np.random.default_rng(70 + b)
    M, N, K = 2, 3, 384
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    scales = synth.draw_scales_halfnormal_signed(rng, N, K // 128)
    A = _bf16(rng.normal(size=(M, K)).astype(np.float32))
    packed = oracle.pack(codes, b)
    y, mag, Aq, sa = oracle.w4a8(A, packed, scales, b=b)
    a = synth.bf16_bits_to_f32(A)
    s_a = (np.abs(a).max(axis=1) / np.float32(127)).astype(np.float32)
    q_a = np.clip(np.rint(a / s_a[:, None]), -127, 127).astype(np.int64)
    np.testing.assert_array_equal(sa, s_a)
    np.testing.assert_array_equal(Aq, q_a)
    s = synth.bf16_bits_to_f32(scales)
    for n in range(N):
        stream = 0
        for j, wd in enumerate(packed[n]):
            stream |= int(wd) << (32 * j)
        qw = [((stream >> (k * b)) & ((1 << b) - 1)) - (1 << (b - 1)) for k in range(K)]
        for m in range(M):
            acc = [sum(int(q_a[m, k]) * qw[k] for k in range(g * 128, (g + 1) * 128))
                   for g in range(K // 128)]
            exact = Fraction(float(s_a[m])) * sum(Fraction(float(s[n, g])) * acc[g]
                                                  for g in range(K // 128))
            exact_mag = abs(Fraction(float(s_a[m]))) * sum(abs(Fraction(float(s[n, g])) * acc[g])
                                                           for g in range(K // 128))
            loose = abs(Fraction(float(s_a[m]))) * sum(
                abs(Fraction(float(s[n, k // 128])) * int(q_a[m, k]) * qw[k]) for k in range(K))
            assert loose > exact_mag * Fraction(11, 10)  # the case separates the two readings
            bound = 8 * 2.0 ** -52 * float(exact_mag)
            assert abs(y[m, n] - float(exact)) <= bound
            assert abs(mag[m, n] - float(exact_mag)) <= bound


def test_w4a8_negative_scales_negate_output():
    w = synth.w4a8(M=8, N=32, K=512, seed=11)
    packed = oracle.pack(w.codes, 4)
    y, mag, _, _ = oracle.w4a8(w.A, packed, w.scales)
    y2, mag2, _, _ = oracle.w4a8(w.A, packed, w.scales ^ np.uint16(0x8000))
    np.testing.assert_array_equal(y2, -y)
    np.testing.assert_array_equal(mag2, mag)


def test_w4a8_points_equal_full_layer():
    w = synth.w4a8(M=8, N=32, K=512, seed=12)
    packed = oracle.pack(w.codes, 4)
    y, mag, Aq, sa = oracle.w4a8(w.A, packed, w.scales)
    mi = np.array([0, 7, 3, 5])
    ni = np.array([31, 0, 16, 2])
    yp, magp = oracle.w4a8_points(Aq, sa, packed, w.scales, mi, ni)
    np.testing.assert_array_equal(yp, y[mi, ni])
    np.testing.assert_array_equal(magp, mag[mi, ni])


# --- the input generator --------------------------------------------------------

def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).normal(size=10000).astype(np.float32) * 1e3
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_workload_shapes_and_sign_mix():
    w = synth.tiny(0)
    assert (w.M, w.N, w.K, w.b) == (4, 256, 512, 6)
    assert w.codes.max() < 64
    neg = np.mean(synth.bf16_bits_to_f32(w.scales) < 0)
    assert 0.4 < neg < 0.6
    assert [synth.layer_bits(i) for i in (0, 9, 10, 11, 53, 54, 63)] == [7, 7, 5, 6, 6, 7, 7]


@pytest.mark.parametrize("b", [4, 8])
def test_w4a8_power_of_two_activation_scale(b):
    # On-grid activations times 2^-3: s_a = 2^-3 exactly, Aq = the integers,
    # and the layer is 2^-3 * A_int . (c - 2^(b-1))^T exactly.
    rng = np.random.default_rng(13 + 100 * b)
    M, N, K = 5, 24, 512
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    A_int = rng.integers(-127, 128, size=(M, K))
    A_int[:, 9] = 127
    A = _bf16((A_int * 2.0 ** -3).astype(np.float32))
    scales = np.full((N, K // 128), BF16_ONE, dtype=np.uint16)
    y, _, Aq, sa = oracle.w4a8(A, oracle.pack(codes, b), scales, b=b)
    np.testing.assert_array_equal(sa, np.full(M, 2.0 ** -3, dtype=np.float32))
    np.testing.assert_array_equal(Aq.astype(np.int64), A_int)
    ref = (A_int.astype(np.int64) @ (codes.astype(np.int64) - (1 << (b - 1))).T) * 2.0 ** -3
    np.testing.assert_array_equal(y, ref)


@pytest.mark.parametrize("b", [3, 4, 6, 8])
def test_w4a8_within_activation_rounding_of_wna16(b):
    # For any activations the int8 layer differs from the bf16-activation
    # layer only by the activation rounding: |y8 - y16| <= (s_a / 2) * sum_k |w|.
    w = synth.w4a8(M=8, N=48, K=1024, seed=14)
    codes = synth.draw_codes(np.random.default_rng(15 + b), 48, 1024, b)
    packed = oracle.pack(codes, b)
    y8, _, Aq, sa = oracle.w4a8(w.A, packed, w.scales, b=b)
    y16, _ = oracle.wna16(w.A, packed, w.scales, b)
    s = np.repeat(synth.bf16_bits_to_f32(w.scales).astype(np.float64), 128, axis=1)
    wsum = np.abs(s * (codes.astype(np.float64) - (1 << (b - 1)))).sum(axis=1)
    bound = 0.5 * sa.astype(np.float64)[:, None] * wsum[None, :] * (1 + 1e-6)
    assert np.all(np.abs(y8 - y16) <= bound)
    # and the bound is not vacuous: the difference is well below |y16| scale
    assert np.median(np.abs(y8 - y16)) < 0.1 * np.median(np.abs(y16))


# --- quantized embedding gather ([card] Findings; [int57] section 3) -------------

def test_bf16_rne_closed_forms():
    # Ties go to the even neighbour (bf16 keeps 7 fraction bits, so 2^-8 is
    # half a step at 1.0); the sign of zero is kept; the subnormal step is
    # 2^-133; past the largest finite value (2 - 2^-7) 2^127 the result is
    # infinity once the rounding carries over.
    cases = [(1.0, 0x3F80), (1 + 2.0 ** -8, 0x3F80), (1 + 3 * 2.0 ** -8, 0x3F82),
             (-(1 + 2.0 ** -8 + 2.0 ** -30), 0xBF81), (-0.0, 0x8000), (0.0, 0x0000),
             (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (3 * 2.0 ** -134, 0x0002),
             ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F), ((2 - 2.0 ** -9) * 2.0 ** 127, 0x7F80),
             (-96.0, 0xC2C0)]
    got = oracle.bf16_rne([c[0] for c in cases])
    assert [int(v) for v in got] == [c[1] for c in cases]


def test_bf16_rne_matches_torch_on_fp32_values():
    # torch's float32 -> bfloat16 conversion rounds to nearest even; on values
    # that are exact in float32 (so no double rounding) the oracle must agree,
    # ties included (constructed with the low 16 bits exactly 0x8000).
    rng = np.random.default_rng(41)
    x = (rng.normal(size=3000) * np.exp2(rng.integers(-30, 30, size=3000))).astype(np.float32)
    ties = (x.view(np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, ties.astype(np.uint32).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_rne(x.astype(np.float64)), ref)


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 7, 8])
def test_embed_hand_computed_rows(b):
    # The three weight rows of the hand-computed example, gathered in a mixed
    # order with ids outside the table; closed forms: row 0 is q = 1 at scale
    # 1 (1.0 everywhere), row 1 is q = (k mod 2^b) - 2^(b-1) at scale -1/2,
    # row 2 is q = -2^(b-1) at scale 2^-7, ids -1 and 3 give zeros.
    _, codes, scales = _hand_inputs(b)
    K = 128
    ids = np.array([2, 0, -1, 1, 3, 1])
    out = oracle.embed(oracle.pack(codes, b), scales, K, b, ids)
    k = np.arange(K)
    row1 = -0.5 * ((k % (1 << b)) - (1 << (b - 1)))
    expect = np.stack([np.full(K, -2.0 ** (b - 1 - 7)), np.ones(K), np.zeros(K), row1,
                       np.zeros(K), row1])
    got = synth.bf16_bits_to_f32(out).astype(np.float64)
    np.testing.assert_array_equal(got, expect)
    # -0.5 * 0 is -0: the product's sign is kept (row 1 where the code is 2^(b-1)).
    assert np.all(out[3][(k % (1 << b)) == (1 << (b - 1))] == 0x8000)
    assert np.all(out[2] == 0) and np.all(out[4] == 0)


def test_embed_b8_unit_scale_is_integer():
    # b = 8 with scale 1: the gathered row is the integer c - 128.
    rng = np.random.default_rng(42)
    V, K = 50, 384
    codes = rng.integers(0, 256, size=(V, K), dtype=np.uint8)
    scales = np.full((V, K // 128), BF16_ONE, dtype=np.uint16)
    ids = rng.integers(0, V, size=20)
    out = oracle.embed(oracle.pack(codes, 8), scales, K, 8, ids)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(out),
                                  (codes[ids].astype(np.float32) - 128))


@pytest.mark.parametrize("b", [3, 5, 6, 7])
def test_embed_equals_layer_on_one_hot_rows(b):
    # Embedding row id, column k, is the layer's output for the one-hot
    # activation row e_k at output id (y = A . dequant(W)^T with A = I):
    # the gather must give the nearest bf16 of the layer's exact fp64 value.
    # (The layer's sum starts from +0, so a weight of -0 comes out +0 there;
    # zeros are compared without their sign, which the hand-computed rows pin.)
    rng = np.random.default_rng(43 + b)
    V, K = 40, 256
    codes = rng.integers(0, 1 << b, size=(V, K), dtype=np.uint8)
    scales = synth.draw_scales_halfnormal_signed(rng, V, K // 128)
    packed = oracle.pack(codes, b)
    eye = np.where(np.eye(K, dtype=bool), BF16_ONE, 0).astype(np.uint16)
    y, _ = oracle.wna16(eye, packed, scales, b)          # y[k, n] = w[n, k]
    ids = rng.integers(0, V, size=12)
    out = oracle.embed(packed, scales, K, b, ids)
    unsigned_zero = lambda bits: np.where(bits == 0x8000, 0, bits)
    np.testing.assert_array_equal(unsigned_zero(out), unsigned_zero(oracle.bf16_rne(y[:, ids].T)))


# --- zero points (b = 4, 8) and per-channel scales ([card] Findings; vLLM Quantization,
#     online shorthands) ---------------------------------------------------------

@pytest.mark.parametrize("b", [4, 8])
def test_zero_points_integer_product(b):
    # Integer activations, unit scales, zero points z[n, g]: the layer is the
    # integer product sum_k a[m,k] (c[n,k] - z[n, k/128]).
    rng = np.random.default_rng(60 + b)
    M, N, K = 5, 33, 384
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    zeros = rng.integers(0, 1 << b, size=(N, K // 128), dtype=np.uint8)
    A_int = rng.integers(-16, 17, size=(M, K))
    scales = np.full((N, K // 128), BF16_ONE, dtype=np.uint16)
    y, _ = oracle.wna16(_bf16(A_int.astype(np.float32)), oracle.pack(codes, b), scales, b,
                        zeros=zeros)
    q = codes.astype(np.int64) - np.repeat(zeros.astype(np.int64), 128, axis=1)
    np.testing.assert_array_equal(y, (A_int.astype(np.int64) @ q.T).astype(np.float64))


@pytest.mark.parametrize("b", [4, 8])
def test_midpoint_zero_points_are_the_symmetric_layer(b):
    # z = 2^(b-1) everywhere is the symmetric form: identical fp64 results.
    w = synth.decode(M=3, b=b, N=40, K=512)
    packed = oracle.pack(w.codes, b)
    zeros = np.full((40, 4), 1 << (b - 1), dtype=np.uint8)
    y0, m0 = oracle.wna16(w.A, packed, w.scales, b)
    y1, m1 = oracle.wna16(w.A, packed, w.scales, b, zeros=zeros)
    np.testing.assert_array_equal(y1, y0)
    np.testing.assert_array_equal(m1, m0)


@pytest.mark.parametrize("b", [4, 6, 8])
def test_per_channel_scale_is_the_replicated_group_scale(b):
    # group = K (one scale per row) equals group 128 with that scale in every
    # group: each dequantized weight is the same exact fp64 product.
    rng = np.random.default_rng(70 + b)
    M, N, K = 4, 24, 640
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    s1 = synth.draw_scales_halfnormal_signed(rng, N, 1)
    A = synth.draw_act(rng, M, K)
    packed = oracle.pack(codes, b)
    y_pc, mag_pc = oracle.wna16(A, packed, s1, b, group=K)
    y_g, mag_g = oracle.wna16(A, packed, np.repeat(s1, K // 128, axis=1), b)
    np.testing.assert_array_equal(y_pc, y_g)
    np.testing.assert_array_equal(mag_pc, mag_g)
    if b in (4, 8):  # zero points stay per 128 codes under a per-channel scale
        z = rng.integers(0, 1 << b, size=(N, K // 128), dtype=np.uint8)
        y_pc, _ = oracle.wna16(A, packed, s1, b, group=K, zeros=z)
        y_g, _ = oracle.wna16(A, packed, np.repeat(s1, K // 128, axis=1), b, zeros=z)
        np.testing.assert_array_equal(y_pc, y_g)


def test_embed_zero_points_and_per_channel_closed_form():
    # b = 4: row r has codes k mod 16, zero point r mod 16 in every group and
    # scale 2^-(r mod 4): w = 2^-(r mod 4) * ((k mod 16) - (r mod 16)).
    V, K, b = 20, 256, 4
    k = np.arange(K)
    codes = np.tile(k % 16, (V, 1)).astype(np.uint8)
    r = np.arange(V)
    zeros = np.repeat((r % 16)[:, None], K // 128, axis=1).astype(np.uint8)
    s = _bf16(2.0 ** -(r % 4).astype(np.float32))[:, None]
    ids = np.array([3, 17, 0, 19])
    packed = oracle.pack(codes, b)
    # group-128 scales (the row's scale in each group) with the zero points
    out = oracle.embed(packed, np.repeat(s, K // 128, axis=1), K, b, ids, zeros=zeros)
    expect = np.stack([2.0 ** -(i % 4) * ((k % 16) - (i % 16)) for i in ids])
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(out).astype(np.float64), expect)
    # per-channel scales (group = K), symmetric: w = s * (c - 8)
    out_pc = oracle.embed(packed, s, K, b, ids, group=K)
    expect_sym = np.stack([2.0 ** -(i % 4) * ((k % 16) - 8) for i in ids])
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(out_pc).astype(np.float64), expect_sym)


def test_w4a8_zero_points_integer_product():
    # On-grid activations, unit scales, b = 4 with zero points: the int8 path
    # is the integer product A . (c - z)^T.
    rng = np.random.default_rng(80)
    M, N, K = 6, 40, 512
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(N, K // 128), dtype=np.uint8)
    A_int = rng.integers(-127, 128, size=(M, K))
    A_int[:, 0] = 127
    scales = np.full((N, K // 128), BF16_ONE, dtype=np.uint16)
    y, _, _, _ = oracle.w4a8(_bf16(A_int.astype(np.float32)), oracle.pack(codes, 4), scales,
                             zeros=zeros)
    q = codes.astype(np.int64) - np.repeat(zeros.astype(np.int64), 128, axis=1)
    np.testing.assert_array_equal(y, (A_int.astype(np.int64) @ q.T).astype(np.float64))


# --- grouped (mixture-of-experts) layer ([card] Findings) ------------------------

@pytest.mark.parametrize("b", [4, 6])
def test_grouped_constant_experts_closed_form(b):
    # Expert e has every weight q = e + 1 at scale 1 (codes 2^(b-1) + e + 1):
    # a row of expert e gives (e + 1) * sum_k a[m,k] in every column.
    E, N, K = 3, 16, 256
    off = np.array([0, 2, 2, 7])  # expert 1 has no rows
    rng = np.random.default_rng(90 + b)
    A_int = rng.integers(-8, 9, size=(7, K))
    codes = np.concatenate([np.full((N, K), (1 << (b - 1)) + e + 1) for e in range(E)]).astype(np.uint8)
    scales = np.full((E * N, K // 128), BF16_ONE, dtype=np.uint16)
    y, mag = oracle.wna16_grouped(_bf16(A_int.astype(np.float32)), oracle.pack(codes, b), scales,
                                  b, off)
    expert = np.repeat(np.arange(E), np.diff(off))
    expect = ((expert + 1) * A_int.sum(axis=1))[:, None] * np.ones((1, N))
    np.testing.assert_array_equal(y, expect)


def test_grouped_is_invariant_under_expert_order():
    # Reordering the experts, and their row blocks with them, permutes the
    # output rows the same way.
    E, N, K, b = 4, 24, 384, 5
    rng = np.random.default_rng(95)
    off = np.array([0, 3, 3, 9, 10])
    A = synth.draw_act(rng, 10, K)
    codes = synth.draw_codes(rng, E * N, K, b)
    scales = synth.draw_scales_halfnormal_signed(rng, E * N, K // 128)
    y, _ = oracle.wna16_grouped(A, oracle.pack(codes, b), scales, b, off)
    perm = [2, 0, 3, 1]
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in perm])
    off2 = np.concatenate([[0], np.cumsum([off[e + 1] - off[e] for e in perm])])
    wrows = np.concatenate([np.arange(e * N, (e + 1) * N) for e in perm])
    y2, _ = oracle.wna16_grouped(A[rows], oracle.pack(codes[wrows], b), scales[wrows], b, off2)
    np.testing.assert_array_equal(y2, y[rows])
