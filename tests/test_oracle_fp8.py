"""Pins of the E4M3 KV oracle (``oracle/fp8.py``): the byte decoder against the OCP "FN"
format's closed-form values and torch's own float8_e4m3fn conversion, and the per-tensor
scales against invariants of attention."""
import math

import numpy as np
import pytest

import workloads as I
from oracle import attention as A
from oracle import fp8


@pytest.mark.parametrize("byte,value", [
    (0x00, 0.0), (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x30, 0.5), (0xB8, -1.0),
    (0x77, 240.0), (0x0F, 1.875 * 2.0 ** -6),
])
def test_closed_form_values(byte, value):
    assert fp8.e4m3_to_float([byte])[0] == value


def test_signed_zero_and_nan_patterns():
    v = fp8.e4m3_to_float(np.arange(256))
    assert math.copysign(1.0, v[0x80]) == -1.0 and v[0x80] == 0.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert int(np.isnan(v).sum()) == 2  # no infinity, one NaN pattern per sign
    assert np.nanmax(np.abs(v)) == 448.0


def test_matches_torch_float8_e4m3fn_exhaustively():
    torch = pytest.importorskip("torch")
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    v = fp8.e4m3_to_float(b)
    assert np.array_equal(np.isnan(ref), np.isnan(v))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], v[ok])


def test_positive_codes_increase_strictly():
    v = fp8.e4m3_to_float(np.arange(0x7F))
    assert np.all(np.diff(v) > 0)


def _batch(seed=0):
    b = I.make_paged_batch(seed, [37, 1, 200, 0, 65], None, page_size=16, num_qo_heads=8, num_kv_heads=2,
                           head_dim=64, num_pages=30)
    return b, I.to_e4m3(b)


def _run(e, k_scale, v_scale, sm=0.125):
    b = e.base
    return fp8.paged_decode_e4m3(b.q_f32, e.k_bytes, e.v_bytes, k_scale, v_scale, b.kv_indptr, b.kv_indices,
                                 b.last_page_len, b.page_size, b.num_qo_heads, b.num_kv_heads, sm)


def test_unit_scales_equal_plain_attention_on_the_decoded_values():
    b, e = _batch()
    o, l = _run(e, 1.0, 1.0)
    kd = fp8.e4m3_to_float(e.k_bytes)
    vd = fp8.e4m3_to_float(e.v_bytes)
    ro, rl = A.batch_attention(b.q_f32, kd, vd, b.kv_indptr, b.kv_indices, b.last_page_len, b.page_size,
                               b.num_qo_heads, b.num_kv_heads, 0.125)
    assert np.array_equal(np.isneginf(l), np.isneginf(rl))
    assert np.allclose(o, ro, atol=1e-12) and np.allclose(l[np.isfinite(l)], rl[np.isfinite(rl)], atol=1e-12)
    assert np.all(np.isfinite(o))  # NaN bytes in the unused slots are never read


def test_v_scale_scales_the_output_and_not_the_lse():
    _, e = _batch(1)
    o1, l1 = _run(e, 1.0, 1.0)
    o3, l3 = _run(e, 1.0, 3.0)
    assert np.allclose(o3, 3.0 * o1, atol=1e-12)
    assert np.array_equal(l1, l3)


def test_k_scale_acts_as_the_score_scale():
    _, e = _batch(2)
    o_a, l_a = _run(e, 2.5, 1.0, sm=0.1)
    o_b, l_b = _run(e, 1.0, 1.0, sm=0.25)
    assert np.allclose(o_a, o_b, atol=1e-12)
    fin = np.isfinite(l_a)
    assert np.array_equal(fin, np.isfinite(l_b)) and np.allclose(l_a[fin], l_b[fin], atol=1e-12)


def test_quantised_inputs_stay_close_to_the_source_values():
    b, e = _batch(3)
    m = np.isfinite(b.k_f32)
    dk = fp8.e4m3_to_float(e.k_bytes)[m] * e.k_scale
    # three mantissa bits: relative error at most 2^-4 for normal values
    big = np.abs(b.k_f32[m]) > 448 * e.k_scale * 2.0 ** -6 * 1.01
    assert np.all(np.abs(dk[big] - b.k_f32[m][big]) <= 2.0 ** -4 * np.abs(b.k_f32[m][big]))
    assert np.all(e.k_bytes[~m] == 0x7F)
