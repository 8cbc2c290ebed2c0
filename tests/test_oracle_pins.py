"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test ties one oracle function to something independent of its code: a
value printed on the pages, the byte order of memory, a library routine
(numpy integer/fp64 matmul, numpy/torch dtype converters), a closed form, an
invariant, or a special case that reduces to a textbook computation.  They are
chosen so that a plausible slip (a dropped term, a wrong shift or group index,
a transposed operand, a sign error, round-half-up instead of half-even) fails
at least one of them.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- converters

def test_bf16_widen_matches_torch():
    r = np.random.default_rng(1)
    bits = r.integers(0, 2**16, size=4096, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.to_f64(bits, "bf16"), ref)


def test_f16_widen_matches_numpy_including_subnormals():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 10) & 0x1F) != 0x1F]
    ref = bits.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(oracle.to_f64(bits, "f16"), ref)


def test_f64_to_f16_rounding_matches_numpy():
    r = np.random.default_rng(2)
    v = np.concatenate([
        r.standard_normal(20000) * 10.0 ** r.integers(-9, 5, 20000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
         2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1e9],
    ])
    # ties-to-even cases at several binades
    for e in range(-20, 15):
        v = np.append(v, [(1024 + 0.5) * 2.0 ** (e - 10), (1025 + 0.5) * 2.0 ** (e - 10)])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.f64_to_f16(v), ref)


def test_f32_to_bf16_rounding_matches_torch():
    r = np.random.default_rng(3)
    u = r.integers(0, 2**32, size=50000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]
    # exact ties: low 16 bits = 0x8000 with both parities of the kept part
    ties = (np.arange(1, 200, dtype=np.uint32) << 16) | np.uint32(0x8000)
    v = np.concatenate([u, ties]).view(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16(v), ref)


# ---------------------------------------------------------------- O1 unpack

def test_unpack_8bit_low_byte_is_lowest_column():
    # mlx_int8.rs "Layout": four unsigned bytes per word, low byte = lowest column.
    # Little-endian memory puts byte j of the stream in bits [8j, 8j+8) of the word.
    stream = np.array([1, 2, 3, 4, 250, 0, 17, 255], dtype=np.uint8)
    words = stream.view(np.uint32)
    assert words[0] == 0x04030201
    np.testing.assert_array_equal(oracle.unpack_affine(words[None, :], 1, 8, 8)[0], stream)


def test_unpack_4bit_and_2bit_closed_forms():
    np.testing.assert_array_equal(
        oracle.unpack_affine(np.array([[0x76543210]], dtype=np.uint32), 1, 8, 4)[0], np.arange(8))
    np.testing.assert_array_equal(
        oracle.unpack_affine(np.array([[0xFEDCBA98]], dtype=np.uint32), 1, 8, 4)[0], np.arange(8, 16))
    # 2-bit codes 0,1,2,3 repeating: byte = 0b11100100 = 0xE4
    np.testing.assert_array_equal(
        oracle.unpack_affine(np.array([[0xE4E4E4E4]], dtype=np.uint32), 1, 16, 2)[0], np.tile(np.arange(4), 4))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_unpack_every_code_at_every_position(bits):
    per = 32 // bits
    vals = np.arange(2 ** bits, dtype=np.uint32)
    for pos in range(per):
        words = (vals << np.uint32(bits * pos)).astype(np.uint32)[:, None]
        codes = oracle.unpack_affine(words, len(vals), per, bits)
        expect = np.zeros((len(vals), per), dtype=np.uint8)
        expect[:, pos] = vals
        np.testing.assert_array_equal(codes, expect)


def _codes_by_memory_order(packed: np.ndarray, bits: int) -> np.ndarray:
    """Independent decode: walk the bytes of the words in memory order and split
    each byte low bits first."""
    by = np.ascontiguousarray(packed).view(np.uint8)
    per_byte = 8 // bits
    parts = [(by >> np.uint8(bits * j)) & np.uint8(2 ** bits - 1) for j in range(per_byte)]
    return np.stack(parts, axis=-1).reshape(packed.shape[0], -1)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_unpack_random_words_matches_memory_order(bits):
    r = np.random.default_rng(bits)
    packed = r.integers(0, 2**32, size=(5, 12), dtype=np.uint64).astype(np.uint32)
    K = 12 * 32 // bits
    np.testing.assert_array_equal(oracle.unpack_affine(packed, 5, K, bits), _codes_by_memory_order(packed, bits))


# ---------------------------------------------------------------- O2/O3 affine

def _const(shape, value, dtype="bf16"):
    return si.store(np.full(shape, value, dtype=np.float32), dtype)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_affine_unit_scale_zero_bias_is_integer_matmul(bits):
    # scale 1, bias 0, integer x: y = x . Q^T exactly (numpy int64 matmul on codes
    # decoded by memory order).  Catches a transposed operand or a wrong row stride.
    M, N, K, G = 3, 7, 128, 32
    r = np.random.default_rng(10 + bits)
    packed = r.integers(0, 2**32, size=(N, K * bits // 32), dtype=np.uint64).astype(np.uint32)
    xi = r.integers(-20, 21, size=(M, K))
    x = si.bf16_bits(xi.astype(np.float32))
    y = oracle.qmm_affine(x, "bf16", packed, _const((N, K // G), 1.0), _const((N, K // G), 0.0), "bf16",
                          M, N, K, G, bits)
    Q = _codes_by_memory_order(packed, bits).astype(np.int64)
    np.testing.assert_array_equal(y, (xi @ Q.T).astype(np.float64))


@pytest.mark.parametrize("sb", ["bf16", "f16", "f32"])
def test_affine_zero_codes_leave_only_group_bias(sb):
    # codes 0 => w[n,k] = bias[n, k/G]; y = x . repeat(bias)^T (numpy fp64 matmul).
    M, N, K, G = 4, 6, 256, 64
    r = np.random.default_rng(20)
    b = si.store(r.standard_normal((N, K // G)).astype(np.float32), sb)
    s = si.store(r.uniform(0.1, 1, (N, K // G)).astype(np.float32), sb)
    x = si.activations(M, K, seed=(21,))
    y = oracle.qmm_affine(x, "bf16", np.zeros((N, K * 4 // 32), np.uint32), s, b, sb, M, N, K, G, 4)
    W = np.repeat(oracle.to_f64(b, sb), G, axis=1)
    ref = oracle.to_f64(x, "bf16") @ W.T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("G", [32, 64, 128])
def test_affine_constant_codes_scale_by_group(G):
    # all codes = c, bias 0: w[n,k] = c*scale[n, k/G]; checks the group index k/G.
    M, N, K, c = 2, 5, 512, 11
    r = np.random.default_rng(G)
    s = si.bf16_bits(r.uniform(0.01, 0.1, (N, K // G)).astype(np.float32))
    word = np.uint32(sum(c << (4 * j) for j in range(8)))
    packed = np.full((N, K // 8), word, dtype=np.uint32)
    x = si.activations(M, K, seed=(G, 1))
    y = oracle.qmm_affine(x, "bf16", packed, s, _const((N, K // G), 0.0), "bf16", M, N, K, G, 4)
    W = c * np.repeat(oracle.to_f64(s, "bf16"), G, axis=1)
    np.testing.assert_allclose(y, oracle.to_f64(x, "bf16") @ W.T, rtol=1e-12, atol=1e-12)


def test_affine_linear_in_x_and_in_scale_bias():
    M, N, K, G = 3, 9, 256, 64
    case = si.affine_case(M, N, K, G, 4, seed=(30,))
    r = np.random.default_rng(31)
    x1, x2 = r.integers(-8, 9, (M, K)), r.integers(-8, 9, (M, K))
    f = lambda xi: oracle.qmm_affine(si.bf16_bits(xi.astype(np.float32)), "bf16", case.packed, case.scales,
                                     case.biases, "bf16", M, N, K, G, 4)
    np.testing.assert_allclose(f(x1 + x2), f(x1) + f(x2), rtol=1e-13, atol=1e-12)
    # doubling scale and bias doubles y (exact: powers of two)
    s2 = si.bf16_bits(2 * si.bits_to_f32(case.scales, "bf16"))
    b2 = si.bf16_bits(2 * si.bits_to_f32(case.biases, "bf16"))
    y1 = oracle.qmm_affine(case.x, "bf16", case.packed, case.scales, case.biases, "bf16", M, N, K, G, 4)
    y2 = oracle.qmm_affine(case.x, "bf16", case.packed, s2, b2, "bf16", M, N, K, G, 4)
    np.testing.assert_array_equal(y2, 2 * y1)


def test_affine_group_permutation_invariance():
    # Moving whole groups (x columns, code words, scale/bias columns together) leaves y.
    M, N, K, G, bits = 2, 6, 512, 64, 4
    case = si.affine_case(M, N, K, G, bits, seed=(40,))
    r = np.random.default_rng(41)
    pg = r.permutation(K // G)
    kcols = (pg[:, None] * G + np.arange(G)).ravel()
    wpg = G * bits // 32
    wcols = (pg[:, None] * wpg + np.arange(wpg)).ravel()
    y = oracle.qmm_affine_case(case)
    y2 = oracle.qmm_affine(case.x[:, kcols], "bf16", case.packed[:, wcols], case.scales[:, pg], case.biases[:, pg],
                           "bf16", M, N, K, G, bits)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-12)


def test_affine_k_perm_reads_x_through_permutation():
    M, N, K, G = 2, 5, 256, 64
    case = si.affine_case(M, N, K, G, 4, seed=(50,))
    kp = np.random.default_rng(51).permutation(K).astype(np.int32)
    y_perm = oracle.qmm_affine(case.x, "bf16", case.packed, case.scales, case.biases, "bf16", M, N, K, G, 4, k_perm=kp)
    y_ref = oracle.qmm_affine(case.x[:, kp], "bf16", case.packed, case.scales, case.biases, "bf16", M, N, K, G, 4)
    np.testing.assert_array_equal(y_perm, y_ref)
    with pytest.raises(ValueError):
        bad = kp.copy()
        bad[3] = K
        oracle.qmm_affine(case.x, "bf16", case.packed, case.scales, case.biases, "bf16", M, N, K, G, 4, k_perm=bad)


def test_affine_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.qmm_affine(np.zeros((1, 96), np.uint16), "bf16", np.zeros((1, 12), np.uint32),
                          np.zeros((1, 2), np.uint16), np.zeros((1, 2), np.uint16), "bf16", 1, 1, 96, 64, 4)
    with pytest.raises(ValueError):
        oracle.qmm_affine(np.zeros((1, 64), np.uint16), "bf16", np.zeros((1, 8), np.uint32),
                          np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16), "bf16", 1, 1, 64, 64, 3)


# ---------------------------------------------------------------- G1/G2 GPTQ

def _golden_values(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return np.array([float(l) for l in f if l.strip() and not l.startswith("#")])


def test_gptq_worked_example_row0():
    # TinyGPT "GPTQReader" smoke test: codes 0..15, scale 1, stored zero 0 -> [-1 .. 14]
    K, N, G = 16, 8, 16
    codes = np.zeros((K, N), dtype=np.uint32)
    codes[:, 0] = np.arange(16)
    qweight = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(K):                      # nibble i%8 of word (i/8) along IN
        qweight[i // 8] |= codes[i] << np.uint32(4 * (i % 8))
    assert qweight[0, 0] == 0x76543210 and qweight[1, 0] == 0xFEDCBA98
    scales = si.f16_bits(np.ones((1, N), np.float32))
    qzeros = np.zeros((1, N // 8), dtype=np.int32)
    W = oracle.dequant_gptq(qweight.view(np.int32), qzeros, scales, None, K, N, G)
    np.testing.assert_array_equal(W[0], _golden_values("gptq_row0.txt"))


def test_gptq_zero_nibble_along_out_axis():
    # qzeros packs 8 zero points along OUT: column o uses nibble o%8 of word o/8.
    K, N, G = 8, 16, 8
    qweight = np.zeros((1, N), dtype=np.int32)           # codes 0
    zs = np.arange(N, dtype=np.uint32) % 16               # stored zero per column
    qzeros = si.pack_nibbles_along_last(zs[None, :]).view(np.int32)
    scales = si.f16_bits(np.ones((1, N), np.float32))
    W = oracle.dequant_gptq(qweight, qzeros, scales, None, K, N, G)
    np.testing.assert_array_equal(W[:, 0], -(zs.astype(np.float64) + 1))


def test_gptq_top_nibble_is_unsigned():
    # an int32 word with the sign bit set still holds code 15 in its top nibble
    K, N, G = 8, 8, 8
    qweight = np.full((1, N), 0xF0000000, dtype=np.uint32).view(np.int32)
    assert qweight[0, 0] < 0
    W = oracle.dequant_gptq(qweight, np.zeros((1, 1), np.int32), si.f16_bits(np.ones((1, N), np.float32)),
                            None, K, N, G)
    np.testing.assert_array_equal(W[0], [-1.0] * 7 + [14.0])


def _gptq_codes_by_memory_order(qweight: np.ndarray) -> np.ndarray:
    """[K/8, N] words -> [K, N] codes: code i sits in nibble i%8 of word i/8."""
    w = np.ascontiguousarray(qweight).view(np.uint32)
    parts = [(w >> np.uint32(4 * j)) & np.uint32(0xF) for j in range(8)]
    return np.stack(parts, axis=1).reshape(-1, w.shape[1])


@pytest.mark.parametrize("bias_dtype", ["f32", "f16"])
def test_gptq_repack_equals_gptq_dequant(bias_dtype):
    # bias_aff = -scale*(zero+1):  code*scale + bias == scale*(code - zero) term by term.
    case = si.gptq_case(2, 512, 64, 128, seed=(60,))
    packed, s_aff, b_aff, kp = oracle.gptq_to_affine_repack(case.qweight, case.qzeros, case.scales, case.g_idx,
                                                            case.K, case.N, case.G, bias_dtype)
    assert sorted(kp.tolist()) == list(range(case.K))
    assert np.all(np.diff(case.g_idx[kp]) >= 0)                      # grouped
    for g in range(case.K // case.G):                                 # stable inside a group
        assert np.all(np.diff(kp[g * case.G:(g + 1) * case.G]) > 0)
    W_aff = oracle.dequant_affine(packed, s_aff, b_aff, "f16", case.N, case.K, case.G, 4, bias_dtype=bias_dtype)
    W_g = oracle.dequant_gptq(case.qweight, case.qzeros, case.scales, case.g_idx, case.K, case.N, case.G)
    if bias_dtype == "f32":
        np.testing.assert_array_equal(W_aff, W_g[:, kp])               # bit-exact
    else:
        assert np.max(np.abs(W_aff - W_g[:, kp])) <= 2.0 ** -11 * np.max(np.abs(W_g)) + 1e-12
    # and the repacked layer computes the same y through k_perm
    y_g = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, 2, case.K, case.N, case.G)
    y_a = oracle.qmm_affine(case.x, "f16", packed, s_aff, b_aff, "f16", 2, case.N, case.K, case.G, 4, k_perm=kp,
                            bias_dtype=bias_dtype)
    if bias_dtype == "f32":
        np.testing.assert_allclose(y_a, y_g, rtol=1e-12, atol=1e-12)
    else:                                    # f16 bias is rounded: within the float bar
        assert oracle.affine_tolerance_report(y_a, y_g)["ok"]


def test_gptq_gidx_permutation_invariance():
    # Permuting K consistently in x, qweight codes and g_idx leaves y unchanged.
    case = si.gptq_case(3, 256, 16, 64, seed=(70,))
    r = np.random.default_rng(71)
    p = r.permutation(case.K)
    codes = _gptq_codes_by_memory_order(case.qweight)[p]              # [K, N]
    qw2 = np.zeros_like(case.qweight.view(np.uint32))
    for i in range(case.K):
        qw2[i // 8] |= codes[i].astype(np.uint32) << np.uint32(4 * (i % 8))
    y1 = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, 3, case.K, case.N, case.G)
    y2 = oracle.qmm_gptq(case.x[:, p], qw2.view(np.int32), case.qzeros, case.scales, case.g_idx[p], 3,
                         case.K, case.N, case.G)
    np.testing.assert_allclose(y2, y1, rtol=1e-12, atol=1e-12)


def test_gptq_trivial_gidx_equals_affine_on_transposed_packing():
    case = si.gptq_case(2, 256, 16, 64, seed=(80,), act_order=False)
    y_none = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, None, 2, case.K, case.N, case.G)
    y_expl = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, 2, case.K, case.N, case.G)
    np.testing.assert_array_equal(y_none, y_expl)
    # same layer in the affine format, built with numpy only
    codes = _gptq_codes_by_memory_order(case.qweight).T                # [N, K]
    packed = si.pack_nibbles_along_last(codes)
    s = case.scales.T.copy()                                           # [N, K/G] f16 patterns
    zeros = case.zeros.T.astype(np.float64)                            # drawn zero points (z_stored+1)
    b = (-oracle.to_f64(s, "f16") * zeros).astype(np.float32)
    W = codes.astype(np.float64) * np.repeat(oracle.to_f64(s, "f16"), case.G, 1) + np.repeat(b.astype(np.float64), case.G, 1)
    y_aff = oracle.to_f64(case.x, "f16") @ W.T
    np.testing.assert_allclose(y_none, y_aff, rtol=1e-12, atol=1e-12)


def test_gptq_repack_rejects_uneven_groups():
    case = si.gptq_case(1, 256, 8, 64, seed=(90,))
    g = case.g_idx.copy()
    i0 = int(np.flatnonzero(case.g_idx == 0)[0])
    g[i0] = 1                                   # group 0 now has G-1 members, group 1 has G+1
    with pytest.raises(ValueError):
        oracle.gptq_to_affine_repack(case.qweight, case.qzeros, case.scales, g, case.K, case.N, case.G)


# ---------------------------------------------------------------- W4A8

def _s4_by_memory_order(w_q4: np.ndarray) -> np.ndarray:
    by = np.ascontiguousarray(w_q4).view(np.uint8)
    lo = (by << np.uint8(4)).view(np.int8) >> 4     # arithmetic shift sign-extends
    hi = by.view(np.int8) >> 4
    return np.stack([lo, hi], axis=-1).reshape(w_q4.shape[0], -1).astype(np.int64)


def test_w4a8_acc_matches_integer_matmul_all_nibbles():
    # every nibble value -8..7 present in every row; numpy int64 matmul is the reference
    M, N, K = 8, 8, 64
    r = np.random.default_rng(100)
    codes = np.stack([r.permutation(np.tile(np.arange(-8, 8), K // 16)) for _ in range(N)])
    w_q4 = si.pack_nibbles_along_last(codes & 0xF)
    np.testing.assert_array_equal(_s4_by_memory_order(w_q4), codes)
    q = r.integers(-127, 128, size=(M, K)).astype(np.int8)
    acc = oracle.w4a8_acc(q, w_q4, M, N, K)
    np.testing.assert_array_equal(acc, q.astype(np.int64) @ codes.T)


def test_w4a8_quantize_ties_and_extremes():
    # amax = 127 * 2^-3 makes s_x = 2^-3 exactly, so x = (j + 1/2) * 2^-3 is an exact tie
    e = 2.0 ** -3
    row = [127 * e, 0.5 * e, 1.5 * e, 2.5 * e, 3.5 * e, -0.5 * e, -1.5 * e, -2.5 * e, 126.5 * e, -127 * e,
           0.0, 10 * e, 10.25 * e, 10.75 * e, 64.5 * e, 65.5 * e]
    x = si.f16_bits(np.array([row], dtype=np.float32))
    assert np.array_equal(si.bits_to_f32(x, "f16")[0], np.array(row, dtype=np.float32))   # all exact in f16
    q, s = oracle.w4a8_quantize_act(x, 1, len(row))
    assert s[0] == np.float32(e)
    expect = [127, 0, 2, 2, 4, 0, -2, -2, 126, -127, 0, 10, 10, 11, 64, 66]   # half to even
    np.testing.assert_array_equal(q[0], expect)


def test_w4a8_quantize_properties_and_zero_row():
    case = si.w4a8_case(6, 8, 256, seed=(110,))
    x = case.x.copy()
    x[3] = 0                                                  # an all-zero row
    q, s = oracle.w4a8_quantize_act(x, 6, 256)
    xf = si.bits_to_f32(x, "f16")
    assert s[3] == 0 and not q[3].any()
    for m in (0, 1, 2, 4, 5):
        assert s[m] == np.float32(np.abs(xf[m]).max()) / np.float32(127)
        k = int(np.abs(xf[m]).argmax())
        assert abs(int(q[m, k])) == 127 and np.sign(q[m, k]) == np.sign(xf[m, k])
        # each code is within half a step of x/s (plus float slack)
        assert np.all(np.abs(q[m].astype(np.float64) - xf[m] / s[m]) <= 0.5 + 1e-5)
    assert np.abs(q.astype(int)).max() <= 127
    _, _, acc, y = oracle.w4a8(x, case.w_q4, case.s_w, 6, 8, 256)
    assert not y[3].any() and not acc[3].any()


def test_w4a8_y_is_acc_times_scales():
    case = si.w4a8_case(4, 16, 128, seed=(120,))
    q, s, acc, y = oracle.w4a8(case.x, case.w_q4, case.s_w, 4, 16, 128)
    np.testing.assert_array_equal(acc, q.astype(np.int64) @ _s4_by_memory_order(case.w_q4).T)
    ref = acc.astype(np.float64) * s.astype(np.float64)[:, None] * oracle.to_f64(case.s_w, "f16")[None, :]
    np.testing.assert_array_equal(y, ref)


# ---------------------------------------------------------------- quantize_pack

@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("sb", ["bf16", "f16", "f32"])
def test_quantize_pack_recovers_grid_aligned_weights(bits, sb):
    # w = q*s + b with s = 2^-6, b = -0.25 (exact everywhere) and both 0 and
    # 2^bits-1 present in each group must come back unchanged.
    N, K, G = 4, 256, 64
    r = np.random.default_rng(bits)
    qmax = 2 ** bits - 1
    q = r.integers(0, qmax + 1, size=(N, K))
    q[:, ::G] = 0
    q[:, 1::G] = qmax
    s, b = 2.0 ** -6, -0.25
    w = (q * s + b).astype(np.float32)
    packed, S, B = oracle.quantize_pack_affine(w, "f32", N, K, G, bits, sb)
    np.testing.assert_array_equal(_codes_by_memory_order(packed, bits), q)
    np.testing.assert_array_equal(oracle.to_f64(S, sb), np.full((N, K // G), s))
    np.testing.assert_array_equal(oracle.to_f64(B, sb), np.full((N, K // G), b))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_quantize_pack_reconstruction_error_bound(bits):
    N, K, G = 8, 512, 64
    w = si.dense_weights(N, K, seed=(130, bits), dtype="bf16")
    packed, S, B = oracle.quantize_pack_affine(w, "bf16", N, K, G, bits, "bf16")
    Wd = oracle.dequant_affine(packed, S, B, "bf16", N, K, G, bits)
    wf = oracle.to_f64(w, "bf16")
    s = np.repeat(oracle.to_f64(S, "bf16"), G, axis=1)
    # half a step, plus the bf16 rounding of scale and bias stretched over 2^bits steps
    slack = 0.5 * s + (2 ** bits) * s * 2.0 ** -8 + np.abs(np.repeat(oracle.to_f64(B, "bf16"), G, 1)) * 2.0 ** -8
    assert np.all(np.abs(Wd - wf) <= slack + 1e-12)
    codes = _codes_by_memory_order(packed, bits)
    assert codes.min() == 0 and codes.max() <= 2 ** bits - 1


def test_quantize_pack_constant_group_gives_zero_scale():
    N, K, G = 2, 64, 32
    w = np.full((N, K), 0.375, dtype=np.float32)
    packed, S, B = oracle.quantize_pack_affine(w, "f32", N, K, G, 4, "bf16")
    assert not packed.any()
    np.testing.assert_array_equal(oracle.to_f64(S, "bf16"), 0.0)
    np.testing.assert_array_equal(oracle.to_f64(B, "bf16"), 0.375)


# ---------------------------------------------------------------- dequant to a storage type

def _bf16_nearest_brute(v: float) -> int:
    """The bf16 pattern nearest to v by exact rational comparison over all
    finite positive patterns (ties to the even pattern): no rounding formula."""
    from fractions import Fraction
    fv = Fraction(abs(v))
    pats = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (pats << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    i = int(np.searchsorted(vals, abs(v)))
    cands = [j for j in (i - 1, i) if 0 <= j < len(vals)]
    best = None
    for j in cands:
        d = abs(Fraction(vals[j]) - fv)
        if best is None or d < best[0] or (d == best[0] and (pats[j] & 1) == 0):
            best = (d, int(pats[j]))
    sign = 0x8000 if np.signbit(v) else 0
    return sign | best[1]


def test_f64_to_bf16_equals_brute_force_nearest():
    r = np.random.default_rng(70)
    v = np.concatenate([r.standard_normal(300) * 10.0 ** r.integers(-30, 30, 300),
                        # double-rounding traps: just above a bf16 tie, where
                        # rounding through fp32 first would land on the tie
                        [1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -8 - 2.0 ** -30, -(3.0 + 2.0 ** -7 + 2.0 ** -40),
                         2.0 ** -130 * (1 + 2.0 ** -5), 2.0 ** -133 * 0.5, 2.0 ** -133 * 0.75, 1.0 + 2.0 ** -8]])
    got = oracle.f64_to_bf16(v)
    want = np.array([_bf16_nearest_brute(float(t)) for t in v], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)
    assert got[300] == 0x3F81 and got[306] == 0x3F80  # above the tie rounds up; the tie itself to even


def test_f64_to_bf16_agrees_with_f32_path_on_f32_values():
    # a value that is already an fp32 is rounded once either way
    r = np.random.default_rng(71)
    f = (r.standard_normal(5000) * 10.0 ** r.integers(-35, 35, 5000)).astype(np.float32)
    np.testing.assert_array_equal(oracle.f64_to_bf16(f.astype(np.float64)), oracle.f32_to_bf16(f))


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_dequant_to_rounds_the_exact_weight_once(out, bits):
    N, K, G = 6, 256, 64
    packed, s, b = si.affine_weights(N, K, G, bits, seed=(72, bits), scale_range=(0.003, 0.03), bias_mode="noise")
    exact = oracle.dequant_affine(packed, s, b, "bf16", N, K, G, bits)
    got = oracle.dequant_affine_to(packed, s, b, "bf16", N, K, G, bits, out)
    if out == "f32":
        np.testing.assert_array_equal(got, exact.astype(np.float32))   # numpy's fp64->fp32 is one rounding
    elif out == "f16":
        np.testing.assert_array_equal(got.view(np.float16), exact.astype(np.float16))
    else:
        want = np.array([_bf16_nearest_brute(float(t)) for t in exact.ravel()[:300]], dtype=np.uint16)
        np.testing.assert_array_equal(got.ravel()[:300], want)


def test_dequant_to_codes_with_unit_scale_are_the_codes():
    N, K, G, bits = 3, 64, 32, 8
    codes = np.random.default_rng(73).integers(0, 256, size=(N, K))
    packed = np.zeros((N, K // 4), dtype=np.uint32)
    for k in range(K):
        packed[:, k // 4] |= (codes[:, k].astype(np.uint32) << (8 * (k % 4)))
    one = np.full((N, K // G), 0x3F80, dtype=np.uint16)        # bf16 1.0
    zero = np.zeros((N, K // G), dtype=np.uint16)
    got = oracle.dequant_affine_to(packed, one, zero, "bf16", N, K, G, bits, "f32")
    np.testing.assert_array_equal(got, codes.astype(np.float32))


# ---------------------------------------------------------------- SiLU-gated GEMV

def test_silu_closed_forms():
    t = np.concatenate([np.linspace(-30, 30, 601), [0.0, 1e-8, -1e-8, 700.0, -700.0]])
    got = oracle.silu(t)
    # t * sigmoid(t) with scipy's logistic function (a library routine)
    from scipy.special import expit
    np.testing.assert_allclose(got, t * expit(t), rtol=1e-13, atol=1e-300)
    # and with tanh where that formula is stable (t >= 0)
    pos = t >= 0
    np.testing.assert_allclose(got[pos], 0.5 * t[pos] * (1.0 + np.tanh(0.5 * t[pos])), rtol=1e-13)
    assert got[601] == 0.0
    np.testing.assert_allclose(got - oracle.silu(-t), t, rtol=1e-12, atol=1e-12)  # silu(t) - silu(-t) = t
    assert abs(got[604] - 700.0) < 1e-12 and got[605] <= 0.0 and got[605] > -1e-200


@pytest.mark.parametrize("bits", [4, 8])
def test_silu_gate_equals_affine_on_the_gated_input(bits):
    M, N, K, G = 3, 40, 256, 64
    c = si.affine_case(M, N, K, G, bits, seed=(74, bits))
    gate = c.x
    up = si.activations(M, K, seed=(74, bits, 9))
    h = oracle.silu(oracle.to_f64(gate, "bf16")) * oracle.to_f64(up, "bf16")
    # the plain affine oracle on h, through fp64 weights and numpy's matmul
    w = oracle.dequant_affine(c.packed, c.scales, c.biases, "bf16", N, K, G, bits)
    want = h @ w.T
    got = oracle.qmm_affine_silu_gate(gate, up, None, "bf16", c.packed, c.scales, c.biases, "bf16", M, N, K, G, bits)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_silu_gate_residual_is_added_once():
    M, N, K, G = 2, 24, 128, 32
    c = si.affine_case(M, N, K, G, 4, seed=(75,), act_dtype="f16")
    up = si.activations(M, K, seed=(75, 9), dtype="f16")
    resid = si.activations(M, N, seed=(75, 10), dtype="f16")
    y0 = oracle.qmm_affine_silu_gate(c.x, up, None, "f16", c.packed, c.scales, c.biases, "bf16", M, N, K, G, 4)
    y1 = oracle.qmm_affine_silu_gate(c.x, up, resid, "f16", c.packed, c.scales, c.biases, "bf16", M, N, K, G, 4)
    np.testing.assert_allclose(y1 - y0, resid.view(np.float16).astype(np.float64), rtol=0, atol=1e-12)
    # up = 0 leaves exactly the residual
    zero = np.zeros_like(up)
    y2 = oracle.qmm_affine_silu_gate(c.x, zero, resid, "f16", c.packed, c.scales, c.biases, "bf16", M, N, K, G, 4)
    np.testing.assert_array_equal(y2, resid.view(np.float16).astype(np.float64))


# ---------------------------------------------------------------- SmoothQuant ahead of W4A8

def test_smooth_factors_hand_values():
    w = np.array([[1.0, -4.0, 0.0], [0.5, 2.0, 0.0]], dtype=np.float32)   # column max |w|: 1, 4, 0
    a = np.array([4.0, 1.0, 3.0], dtype=np.float32)
    s = oracle.smooth_factors(a, w, "f32", 2, 3, 0.5)
    np.testing.assert_array_equal(s, np.array([2.0, 0.5, 1.0], dtype=np.float32))   # sqrt(4/1), sqrt(1/4), zero column
    np.testing.assert_array_equal(oracle.smooth_factors(a, w, "f32", 2, 3, 1.0), np.array([4.0, 1.0, 1.0], np.float32))
    np.testing.assert_array_equal(oracle.smooth_factors(a, w, "f32", 2, 3, 0.0), np.array([1.0, 0.25, 1.0], np.float32))
    a0 = np.array([0.0, 1.0, 3.0], dtype=np.float32)
    assert oracle.smooth_factors(a0, w, "f32", 2, 3, 0.5)[0] == 1.0


def test_smoothing_is_the_identity_for_the_dense_product():
    # (x / s) . (W diag(s))^T == x . W^T up to fp64 rounding, for the oracle's s
    r = np.random.default_rng(76)
    M, N, K = 5, 7, 64
    x = r.standard_normal((M, K))
    x[:, 3] *= 50.0                                   # an outlier channel
    w = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    s = oracle.smooth_factors(np.abs(x).max(0).astype(np.float32), w, "f32", N, K, 0.5).astype(np.float64)
    lhs = (x / s) @ (w.astype(np.float64) * s).T
    np.testing.assert_allclose(lhs, x @ w.astype(np.float64).T, rtol=1e-12, atol=1e-14)
    assert (np.abs(x / s).max(0).max() < np.abs(x).max(0).max() / 3)   # the outlier range shrinks


def test_w4a8_weight_quantization_recovers_grid_weights():
    r = np.random.default_rng(77)
    N, K = 6, 64
    codes = r.integers(-7, 8, size=(N, K))
    codes[:, 5] = 7                                   # the row maximum is +7 steps
    sw = np.float16(r.uniform(0.001, 0.01, size=N)).astype(np.float32)
    w = codes * sw[:, None]                           # exact in fp32
    wq, sw_out = oracle.w4a8_quantize_weights(w.astype(np.float32), "f32", None, N, K)
    np.testing.assert_array_equal(sw_out.view(np.float16).astype(np.float32), sw)
    nib = np.stack([(wq >> (4 * j)) & 0xF for j in range(8)], axis=-1).reshape(N, K).astype(np.int64)
    np.testing.assert_array_equal(np.where(nib >= 8, nib - 16, nib), codes)
    # smoothing by ones changes nothing; by a power of two per channel it
    # quantizes the exactly scaled weights
    wq1, sw1 = oracle.w4a8_quantize_weights(w.astype(np.float32), "f32", np.ones(K, np.float32), N, K)
    np.testing.assert_array_equal(wq1, wq)
    np.testing.assert_array_equal(sw1, sw_out)
    p2 = (2.0 ** r.integers(-2, 3, size=K)).astype(np.float32)
    wq2, sw2 = oracle.w4a8_quantize_weights(w.astype(np.float32), "f32", p2, N, K)
    wq3, sw3 = oracle.w4a8_quantize_weights((w * p2).astype(np.float32), "f32", None, N, K)
    np.testing.assert_array_equal(wq2, wq3)
    np.testing.assert_array_equal(sw2, sw3)


def test_w4a8_smooth_reduces_to_plain_w4a8():
    c = si.w4a8_case(4, 16, 128, seed=(78,))
    ones = np.ones(c.K, np.float32)
    q0, s0, a0, y0 = oracle.w4a8(c.x, c.w_q4, c.s_w, c.M, c.N, c.K)
    q1, s1, a1, y1 = oracle.w4a8_smooth(c.x, ones, c.w_q4, c.s_w, c.M, c.N, c.K)
    np.testing.assert_array_equal(q1, q0)
    np.testing.assert_array_equal(s1, s0)
    np.testing.assert_array_equal(a1, a0)
    # a power-of-two divisor is exact: the same as dividing x beforehand
    p2 = (2.0 ** np.random.default_rng(79).integers(-3, 4, size=c.K)).astype(np.float32)
    xd = (c.x.view(np.float16).astype(np.float32) / p2).astype(np.float16)
    assert np.array_equal(xd.astype(np.float32) * p2, c.x.view(np.float16).astype(np.float32))  # no rounding in x/p2
    q2, s2, a2, _ = oracle.w4a8_smooth(c.x, p2, c.w_q4, c.s_w, c.M, c.N, c.K)
    q3, s3, a3, _ = oracle.w4a8(xd.view(np.uint16), c.w_q4, c.s_w, c.M, c.N, c.K)
    np.testing.assert_array_equal(q2, q3)
    np.testing.assert_array_equal(s2, s3)
    np.testing.assert_array_equal(a2, a3)


# ---------------------------------------------------------------- decode chain

def _np_dequant4(packed, scales, biases, N, K, G, dt):
    # numpy only: codes by shifts of the words, low nibble = lowest column
    words = packed.astype(np.uint64)
    q = np.stack([(words >> (4 * i)) & 15 for i in range(8)], axis=-1).reshape(N, K).astype(np.float64)
    s = si.bits_to_f32(scales, dt).astype(np.float64)
    b = si.bits_to_f32(biases, dt).astype(np.float64)
    return q * np.repeat(s, G, axis=1) + np.repeat(b, G, axis=1)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_chain_matches_numpy_composition(dt):
    # three stages: a, b from x0; c = W (silu(a) * b) + x0; d = W c.  The
    # reference dequantizes and multiplies with numpy, stores every output
    # with the pinned rounding, and feeds the stored values on: wrong
    # routing, a missing residual, or unrounded values passed on all show.
    G = 32
    x0 = si.activations(1, 64, seed=(70, 1), dtype=dt).reshape(64)
    shapes = {"a": (96, 64), "b": (96, 64), "c": (64, 96), "d": (32, 64)}
    W = {}
    lins = []
    for i, (name, (N, K)) in enumerate(shapes.items()):
        p, s, b = si.affine_weights(N, K, G, 4, seed=(70, 2, i), scale_range=(0.01, 0.05), bias_mode="noise",
                                    sb_dtype=dt)
        W[name] = _np_dequant4(p, s, b, N, K, G, dt)
        lins.append(dict(name=name, packed=p, scales=s, biases=b, N=N, K=K, x=None, gate=None, resid=None))
    lins[0]["x"] = lins[1]["x"] = "x0"
    lins[2].update(x="b", gate="a", resid="x0")
    lins[3]["x"] = "c"
    buffers = {"x0": x0}
    got = oracle.qgemv_affine_chain(lins, buffers, dt, G)
    rnd = oracle.f64_to_f16 if dt == "f16" else oracle.f64_to_bf16
    f = lambda bits: oracle.to_f64(bits, dt)
    ra = W["a"] @ f(x0)
    rb = W["b"] @ f(x0)
    a_s, b_s = rnd(ra), rnd(rb)
    h = f(a_s) / (1.0 + np.exp(-f(a_s))) * f(b_s)
    rc = W["c"] @ h + f(x0)
    c_s = rnd(rc)
    rd = W["d"] @ f(c_s)
    for name, ref in (("a", ra), ("b", rb), ("c", rc), ("d", rd)):
        np.testing.assert_allclose(got[name], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(buffers["d"], rnd(rd))
