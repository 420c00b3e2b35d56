"""Pins of the oracle's cache-building steps: oracle.calibrate (which rows define each
global scale g[b][h][K|V]) and oracle.append (which slot each quantised row lands in).

Expected values are written down from the readings, not recomputed by the functions
under test:
  * global scale (a stated reading; gzenz/ninfer page, "Context and model", NVFP4 KV
    cache bullet, gives only the group format): one fp32 per (sequence, KV head) for K and
    one for V, g = amax / (6 * 448) over that sequence's rows of that head. A planted
    maximum of 2688 * 2^k in one slice makes that slice's g exactly 2^k;
  * append: row r of sequence b lands at slot seq_base[b] + write_pos[b] + r of every head
    plane, quantised with g[b][h][0] (K) or g[b][h][1] (V); every other slot is untouched.
    The per-row bytes come from quantize_rows, which has its own pins (hand-worked
    groups, brute force, invariants).
"""
import numpy as np
import torch

import oracle
import workloads


def _bf16(x):
    return workloads.as_u16(torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def _rows(rng, n, H, D, scale):
    """bf16 rows [n][H][D] with magnitudes below scale (strictly: |x| <= scale / 2)."""
    return _bf16(rng.uniform(-0.5, 0.5, size=(n, H, D)) * scale).reshape(n, H, D)


def test_calibrate_planted_maxima():
    rng = np.random.default_rng(11)
    H, D = 2, 128
    lens = [5, 0, 3, 7]                       # sequence 1 has no rows: g = 0 for both heads
    n = sum(lens)
    k = _rows(rng, n, H, D, 1.0)
    v = _rows(rng, n, H, D, 1.0)
    # one exponent per (b, h, K|V) slice, all different; the planted value has |x| = 2688 * 2^e
    expected = np.zeros((len(lens), H, 2), np.float32)
    base = 0
    for b, L in enumerate(lens):
        for h in range(H):
            for kv, arr in ((0, k), (1, v)):
                if L == 0:
                    continue
                e = 4 * b + 2 * h + kv - 6          # -6 .. 9: distinct per slice
                row = base + (3 * b + h + kv) % L
                col = (17 * b + 5 * h + 3 * kv) % D
                sign = -1.0 if (b + h + kv) % 2 else 1.0
                arr[row, h, col] = _bf16([sign * 2688.0 * 2.0 ** e])[0]
                expected[b, h, kv] = np.float32(2.0 ** e)
                # every other value of the slice stays below the planted magnitude
                assert 2.0 ** e * 2688.0 > 0.5
        base += L
    g = oracle.calibrate(k, v, lens)
    assert g.dtype == np.float32 and g.shape == (len(lens), H, 2)
    np.testing.assert_array_equal(g, expected)


def test_calibrate_is_per_sequence_not_per_batch():
    """Two sequences with very different maxima: each gets its own g (a batch-wide amax
    would give both the larger one)."""
    H, D = 1, 128
    k = np.zeros((4, H, D), np.uint16)
    v = np.zeros((4, H, D), np.uint16)
    k[0, 0, 0] = _bf16([2688.0 * 8])[0]         # sequence 0 (rows 0, 1): K amax 21504
    k[3, 0, 1] = _bf16([-2688.0 / 4])[0]        # sequence 1 (rows 2, 3): K amax 672
    v[1, 0, 2] = _bf16([2688.0])[0]
    v[2, 0, 3] = _bf16([2688.0 * 2])[0]
    g = oracle.calibrate(k, v, [2, 2])
    np.testing.assert_array_equal(g[:, 0, 0], np.float32([8.0, 0.25]))
    np.testing.assert_array_equal(g[:, 0, 1], np.float32([1.0, 2.0]))


def test_calibrate_non_power_of_two_rounds_to_nearest_fp32():
    """amax = 1.0: g = fp32(1 / 2688). 1/2688 = 2^-7 / 21 in binary is periodic; the fp32
    nearest to it is written out from its exact rational value."""
    from fractions import Fraction
    x = np.zeros((1, 1, 128), np.uint16)
    x[0, 0, 9] = _bf16([1.0])[0]
    g = oracle.calibrate(x, x, [1])
    exact = Fraction(1, 2688)
    f = float(g[0, 0, 0])
    lo = np.nextafter(np.float32(f), np.float32(0))
    hi = np.nextafter(np.float32(f), np.float32(1))
    assert abs(Fraction(f) - exact) <= abs(Fraction(float(lo)) - exact)
    assert abs(Fraction(f) - exact) <= abs(Fraction(float(hi)) - exact)
    assert g[0, 0, 1] == g[0, 0, 0]


def test_append_places_rows_at_their_slots():
    rng = np.random.default_rng(12)
    H, D, cap = 2, 128, 64
    n_new = [3, 0, 4]
    seq_base = [5, 20, 40]
    write_pos = [2, 7, 9]                      # rows of seq b go to seq_base + write_pos + r
    rows = sum(n_new)
    k = _rows(rng, rows, H, D, 8.0)
    v = _rows(rng, rows, H, D, 0.5)
    # a different g for every (b, h, K|V) so a wrong scale index changes the bytes
    g = np.array([[[0.01, 0.002], [0.03, 0.0007]],
                  [[1.0, 1.0], [1.0, 1.0]],
                  [[0.005, 0.0001], [0.02, 0.0003]]], np.float32)
    cache = oracle.Cache(H, D, cap)
    oracle.append(cache, k, v, g, seq_base, write_pos, n_new)

    exp_kc = np.zeros((H, cap, D // 2), np.uint8)
    exp_ks = np.zeros((H, cap, D // 16), np.uint8)
    exp_vc = np.zeros_like(exp_kc)
    exp_vs = np.zeros_like(exp_ks)
    r = 0
    for b in range(len(n_new)):
        for j in range(n_new[b]):
            slot = seq_base[b] + write_pos[b] + j
            for h in range(H):
                kc, ks = oracle.quantize_rows(k[r, h][None], g[b, h, 0])
                vc, vs = oracle.quantize_rows(v[r, h][None], g[b, h, 1])
                exp_kc[h, slot], exp_ks[h, slot] = kc[0], ks[0]
                exp_vc[h, slot], exp_vs[h, slot] = vc[0], vs[0]
            r += 1
    for name, exp in (("k_codes", exp_kc), ("k_scales", exp_ks), ("v_codes", exp_vc), ("v_scales", exp_vs)):
        np.testing.assert_array_equal(getattr(cache, name), exp, err_msg=name)
    # untouched slots are still zero; written slots are exactly the expected ones
    written = {seq_base[b] + write_pos[b] + j for b in range(len(n_new)) for j in range(n_new[b])}
    assert written == {7, 8, 9, 49, 50, 51, 52}
    untouched = [s for s in range(cap) if s not in written]
    assert not cache.k_codes[:, untouched].any() and not cache.v_scales[:, untouched].any()
    # K and V are not swapped: their scale codes differ for these inputs
    assert not np.array_equal(exp_ks[:, sorted(written)], exp_vs[:, sorted(written)])


def test_append_keeps_existing_slots():
    """A second append into a partly filled cache changes only its own slots."""
    rng = np.random.default_rng(13)
    H, D, cap = 1, 128, 16
    a = _rows(rng, 6, H, D, 1.0)
    b = _rows(rng, 2, H, D, 1.0)
    g = np.array([[[0.001, 0.001]]], np.float32)
    cache = oracle.Cache(H, D, cap)
    oracle.append(cache, a, a, g, [4], [0], [6])
    before = cache.k_codes.copy()
    oracle.append(cache, b, b, g, [4], [6], [2])          # slots 10, 11
    np.testing.assert_array_equal(cache.k_codes[:, :10], before[:, :10])
    np.testing.assert_array_equal(cache.k_codes[:, 12:], before[:, 12:])
    kc, _ = oracle.quantize_rows(b[:, 0], 0.001)
    np.testing.assert_array_equal(cache.k_codes[0, 10:12], kc)
