"""Property tests on small random shapes (CPU only, hypothesis): the C ABI's
host packer, size queries and argument refusals, and the oracle against exact
rational arithmetic, on shapes and values hypothesis draws (derandomized, so
every run checks the same cases).

Pages cited by title and section:
  [card]  model card "Qwen3.8-27B-INT6-Mixed-AutoRound", Reproducing this model
          (a packed row holds ceil(in * bits / 32) words) and Findings
          (unsupported widths are refused, not mis-computed)
  [int57] "vLLM Can Run INT5-7", section 2 (dequantize the codes, then the
          linear layer)
  [w4a8]  club-3090 discussion #733, Under the hood (int8 activations, group
          scales applied to the integer products)
"""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import weight_only_bit_wq_amd as wq
from weight_only_bit_wq_amd import synth

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True)
seeds = st.integers(0, 2 ** 32 - 1)
bits = st.integers(2, 8)


def _stream_codes(packed_row, K, b):
    """Codes of one packed row read off the row as one LSB-first big integer
    (an independent definition of the layout [card])."""
    stream = 0
    for j, wd in enumerate(packed_row):
        stream |= int(wd) << (32 * j)
    return [(stream >> (k * b)) & ((1 << b) - 1) for k in range(K)]


def _stream_words(codes_row, b):
    acc = 0
    for k, c in enumerate(codes_row):
        acc |= int(c) << (k * b)
    return [(acc >> (32 * j)) & 0xFFFFFFFF for j in range((len(codes_row) * b + 31) // 32)]


# --- host packer and size queries of the C ABI ---------------------------------

@SETTINGS
@given(K=st.integers(0, 1 << 40), b=st.integers(-2, 12))
def test_words_per_row_is_the_ceiling(K, b):
    w = wq.wq_packed_words_per_row(K, b)
    if 1 <= b <= 8:
        assert w * 32 >= K * b > (w - 1) * 32 or (K == 0 and w == 0)  # [card]
    else:
        assert w == -1


@SETTINGS
@given(b=bits, N=st.integers(1, 5), G=st.integers(1, 4), mid=st.booleans(), seed=seeds)
def test_host_pack_is_the_lsb_first_stream(b, N, G, mid, seed):
    rng = np.random.default_rng(seed)
    K = 128 * G
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    if mid:  # rows of the midpoint code (zero weights) pack like any other
        codes[rng.integers(0, N)] = 1 << (b - 1)
    packed = wq.wq_pack(codes, b)
    assert packed.shape == (N, wq.wq_packed_words_per_row(K, b))
    for n in range(N):
        assert packed[n].tolist() == _stream_words(codes[n], b)
    np.testing.assert_array_equal(wq.wq_unpack(packed, K, b), codes)
    np.testing.assert_array_equal(oracle.unpack(packed, K, b), codes)


@SETTINGS
@given(b=bits, N=st.integers(1, 4), K=st.integers(1, 300), seed=seeds)
def test_oracle_pack_any_length_is_the_stream(b, N, K, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    packed = oracle.pack(codes, b)
    for n in range(N):
        assert packed[n].tolist() == _stream_words(codes[n], b)
        assert _stream_codes(packed[n], K, b) == codes[n].tolist()


@SETTINGS
@given(b=st.integers(2, 7), k=st.integers(0, 255), extra=st.integers(0, 255), seed=seeds)
def test_host_pack_refuses_any_code_beyond_b_bits(b, k, extra, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << b, size=(2, 256), dtype=np.uint8)
    codes[1, k] = min(255, (1 << b) + extra)
    with pytest.raises(wq.WQError) as e:
        wq.wq_pack(codes, b)
    assert e.value.status == wq.WQ_ERR_CODE_RANGE


@SETTINGS
@given(b=st.sampled_from([-1, 0, 1, 9, 12, 16]), seed=seeds)
def test_unsupported_widths_are_refused(b, seed):  # [card] Findings
    codes = np.random.default_rng(seed).integers(0, 2, size=(2, 128), dtype=np.uint8)
    with pytest.raises(wq.WQError) as e:
        wq.wq_pack(codes, b)
    assert e.value.status == wq.WQ_ERR_UNSUPPORTED_BITS
    for layout in (wq.WQ_LAYOUT_DENSE, wq.WQ_LAYOUT_TILED):
        assert wq.wq_repacked_bytes(layout, 64, 128, b) == -1
    for op in (wq.WQ_OP_GEMM, wq.WQ_OP_GEMM_A8):
        assert wq.wq_workspace_bytes(op, 1, 64, 128, b) == -1


@SETTINGS
@given(b=bits, N=st.integers(1, 1 << 20), G=st.integers(1, 256))
def test_repacked_sizes_hold_every_code_and_scale(b, N, G):
    K = 128 * G
    payload = N * K * b // 8 + 2 * N * G  # codes + bf16 scales
    dense = wq.wq_repacked_bytes(wq.WQ_LAYOUT_DENSE, N, K, b)
    tiled = wq.wq_repacked_bytes(wq.WQ_LAYOUT_TILED, N, K, b)
    assert dense == 4 * N * wq.wq_packed_words_per_row(K, b)
    # The tiled blob holds every code and scale, pads rows to whole 64-row
    # tiles and no more, and keeps 16-byte alignment between experts.
    assert payload <= tiled <= payload + 63 * (K * b // 8 + 2 * G)
    assert tiled % 16 == 0
    assert wq.wq_repacked_bytes(wq.WQ_LAYOUT_TILED, N + 1, K, b) >= tiled
    assert wq.wq_repacked_bytes(wq.WQ_LAYOUT_TILED, N, K + 1, b) == -1  # K % 128 != 0


@SETTINGS
@given(op=st.sampled_from(["gemm", "a8"]), M=st.integers(0, 1 << 16), N=st.integers(1, 1 << 17),
       G=st.integers(1, 160), b=bits)
def test_workspace_sizes_are_zero_or_cover_the_counters(op, M, N, G, b):
    code = wq.WQ_OP_GEMM if op == "gemm" else wq.WQ_OP_GEMM_A8
    K = 128 * G
    w = wq.wq_workspace_bytes(code, M, N, K, b)
    assert w == 0 or w >= wq.WORKSPACE_ZERO_BYTES
    assert w % 16 == 0
    assert wq.wq_workspace_bytes(code, -1 - M, N, K, b) == -1
    assert wq.wq_workspace_bytes(code, M, N, K + 64, b) == -1


# --- the oracle against exact rational arithmetic ------------------------------

@SETTINGS
@given(b=bits, M=st.integers(1, 2), N=st.integers(1, 3), G=st.integers(1, 2),
       zp=st.booleans(), mid=st.sampled_from([0.0, 0.5, 1.0]), seed=seeds)
def test_oracle_wna16_is_exact_dequantize_then_linear(b, M, N, G, zp, mid, seed):
    # [int57] section 2: y = sum_k a[m,k] * s[n,g(k)] * (c[n,k] - z), z the
    # zero point (b = 4, 8) or 2^(b-1); mag = sum_k |a * s * (c - z)|.  A
    # fraction `mid` of the codes is the midpoint (zero weight), with
    # one-signed activations: an all-midpoint row must give exactly 0.
    rng = np.random.default_rng(seed)
    K = 128 * G
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    codes[rng.random(size=(N, K)) < mid] = 1 << (b - 1)
    zeros = None
    if zp and b in (4, 8):
        zeros = rng.integers(0, 1 << b, size=(N, G), dtype=np.uint8)
    scales = synth.draw_scales_halfnormal_signed(rng, N, G)
    A = synth.f32_to_bf16_bits(np.abs(rng.normal(size=(M, K)) * 50).astype(np.float32))
    packed = oracle.pack(codes, b)
    y, mag = oracle.wna16(A, packed, scales, b, zeros=zeros)
    a = synth.bf16_bits_to_f32(A)
    s = synth.bf16_bits_to_f32(scales)
    for n in range(N):
        c = _stream_codes(packed[n], K, b)
        z = [int(zeros[n, k // 128]) if zeros is not None else 1 << (b - 1) for k in range(K)]
        for m in range(M):
            terms = [Fraction(float(a[m, k])) * Fraction(float(s[n, k // 128])) * (c[k] - z[k])
                     for k in range(K)]
            exact, exact_mag = sum(terms), sum(abs(t) for t in terms)
            bound = K * 2.0 ** -52 * float(exact_mag)
            assert abs(y[m, n] - float(exact)) <= bound
            assert abs(mag[m, n] - float(exact_mag)) <= bound


@SETTINGS
@given(b=bits, M=st.integers(1, 2), N=st.integers(1, 3), G=st.integers(1, 3), seed=seeds)
def test_oracle_w4a8_is_the_rescaled_integer_product(b, M, N, G, seed):
    # [w4a8] Under the hood: per-row int8 activations q_a with scale s_a
    # (|q_a| <= 127, the row's largest |a| maps to 127, q_a the nearest
    # integer to a / s_a), then y = s_a * sum_g s_g * (integer sum of q_a * q_w
    # over the group), mag = |s_a| * sum_g |s_g * group sum|.
    rng = np.random.default_rng(seed)
    K = 128 * G
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    scales = synth.draw_scales_halfnormal_signed(rng, N, G)
    A = synth.draw_act(rng, M, K)
    packed = oracle.pack(codes, b)
    y, mag, Aq, sa = oracle.w4a8(A, packed, scales, b=b)
    a = synth.bf16_bits_to_f32(A).astype(np.float64)
    q_a = Aq.astype(np.int64)
    assert np.abs(q_a).max() <= 127
    for m in range(M):
        if np.abs(a[m]).max() > 0:
            assert np.abs(q_a[m]).max() == 127
            # nearest integer to a / s_a, up to the fp32 rounding of the quotient
            assert np.all(np.abs(a[m] / float(sa[m]) - q_a[m]) <= 0.5 + 1e-5)
    s = synth.bf16_bits_to_f32(scales)
    for n in range(N):
        qw = [c - (1 << (b - 1)) for c in _stream_codes(packed[n], K, b)]
        for m in range(M):
            acc = [sum(int(q_a[m, k]) * qw[k] for k in range(g * 128, (g + 1) * 128))
                   for g in range(G)]
            exact = Fraction(float(sa[m])) * sum(Fraction(float(s[n, g])) * acc[g]
                                                 for g in range(G))
            exact_mag = abs(Fraction(float(sa[m]))) * sum(abs(Fraction(float(s[n, g])) * acc[g])
                                                          for g in range(G))
            bound = 8 * 2.0 ** -52 * float(exact_mag)
            assert abs(y[m, n] - float(exact)) <= bound
            assert abs(mag[m, n] - float(exact_mag)) <= bound
