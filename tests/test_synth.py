"""The seeded input generator: published SplitMix64 outputs, distribution sanity,
storage rounding, int8 format and the paged layout (bit-exact through the page table)."""
import numpy as np

import synth


def test_splitmix64_published_outputs():
    # Seed 0: the first outputs of SplitMix64 as published with the algorithm
    # (Steele, Lea and Flood, "Fast splittable pseudorandom number generators").
    z = synth.splitmix64(0, 0, 3)
    assert [int(x) for x in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_slices_agree():
    a = synth.splitmix64(77, 0, 1000)
    b = synth.splitmix64(77, 400, 100)
    assert np.array_equal(a[400:500], b)
    n = synth.normal_f32_stream(5, 0, 1001)
    assert np.array_equal(n[:1000], synth.normal_f32_stream(5, 0, 1000))
    assert np.array_equal(n[301:700], synth.normal_f32_stream(5, 301, 399))


def test_c_loop_matches_numpy_definition():
    a = synth.normal_f32_stream(42, 0, 200_001)
    b = synth.normal_numpy(42, 200_001)
    # same uniforms and formula; libm and numpy may differ in the last f64 ulp only
    np.testing.assert_allclose(a, b.astype(np.float32), rtol=1e-6, atol=1e-7)
    assert np.mean(a == b.astype(np.float32)) > 0.999


def test_normals_look_normal():
    x = synth.normal_f32_stream(12345, 0, 400_000).astype(np.float64)
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - 1.0) < 0.01
    assert abs(np.mean(np.abs(x) < 1.0) - 0.6827) < 0.005


def test_f16_storage_is_round_to_nearest_even():
    x = synth.normal_f16(3, (1000,))
    assert x.dtype == np.float16
    f32 = synth.normal_f32(3, (1000,))
    assert np.array_equal(x, f32.astype(np.float16))
    # RNE tie: 1 + 2^-11 is exactly half-way between 1 and the next f16; rounds to even (1.0)
    assert np.float32(1 + 2 ** -11).astype(np.float16) == np.float16(1.0)


def test_quantize_i8_format():
    x = synth.normal_f32(8, (100, 8, 128))
    x[0, 0] = 0.0
    q, s = synth.quantize_i8(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert s[0, 0] == 1.0 and np.all(q[0, 0] == 0)
    assert q.min() >= -127 and q.max() <= 127
    # every nonzero row hits +-127 at its max-abs element
    amax = np.abs(q.astype(np.int32)).max(axis=-1)
    assert np.all(amax[1:] == 127)


def test_paged_layout_round_trips_and_is_poisoned():
    kv_lens = np.array([37, 16, 1, 50], np.int32)
    d = synth.paged_inputs(20261299, 4, 8, 2, 16, kv_lens, n_poison=5)
    kp, vp, ks, vs, tab = d["k_pages"], d["v_pages"], d["k_scales"], d["v_scales"], d["page_table"]
    n_live = [(int(L) + 15) // 16 for L in kv_lens]
    assert kp.shape[0] == sum(n_live) + 5
    used = set()
    for b, L in enumerate(kv_lens):
        for t in range(int(L)):
            ph = tab[b, t >> 4]
            sl = t & 15
            assert np.array_equal(kp[ph, :, sl], d["k_q"][b][t])
            assert np.array_equal(vp[ph, :, sl], d["v_q"][b][t])
            assert np.array_equal(ks[ph, :, sl], d["k_s"][b][t])
            assert np.array_equal(vs[ph, :, sl], d["v_s"][b][t])
        for lp in range(n_live[b]):
            used.add(int(tab[b, lp]))
        assert np.all(tab[b, n_live[b]:] == -1)
        rem = int(L) % 16
        if rem:
            last = tab[b, n_live[b] - 1]
            assert np.all(kp[last, :, rem:] == -128) and np.all(np.isnan(ks[last, :, rem:]))
    assert len(used) == sum(n_live)
    poison = sorted(set(range(kp.shape[0])) - used)
    assert len(poison) == 5
    assert np.all(kp[poison] == -128) and np.all(np.isnan(vs[poison]))


def test_alternative_permutation_moves_pages_not_data():
    kv_lens = np.array([40, 33], np.int32)
    a = synth.paged_inputs(20261298, 2, 4, 1, 8, kv_lens, n_poison=3)
    b = synth.paged_inputs(20261298, 2, 4, 1, 8, kv_lens, n_poison=3, alt_perm=True)
    assert not np.array_equal(a["page_table"], b["page_table"])
    for x, y in zip(a["k_q"], b["k_q"]):
        assert np.array_equal(x, y)


def test_kv_lens_in_range():
    L = synth.paged_kv_lens(synth.seed_of(5), 1000, 16384, 32768)
    assert L.min() >= 16384 and L.max() <= 32768
    assert L.std() > 3000


def test_tiered_inputs_place_the_hot_tier_in_the_ring():
    """Hot position p (cold_len <= p < cold_len + hot_len) sits at ring row
    (hot_start + p - cold_len) % hot_window; rows holding no position are NaN; the cold tier
    is the paged layout of one sequence, and an empty cold tier is one poison page."""
    t = synth.tiered_inputs(20261297, 4, 2, 16, 40, 13, 16, 9, n_poison=2)
    assert t["ring_k"].shape == (2, 16, 16) and t["hot_k"].shape == (13, 2, 16)
    for i in range(13):
        r = (9 + i) % 16
        assert np.array_equal(t["ring_k"][:, r], t["hot_k"][i])
        assert np.array_equal(t["ring_v"][:, r], t["hot_v"][i])
    used = {(9 + i) % 16 for i in range(13)}
    for r in set(range(16)) - used:
        assert np.all(np.isnan(t["ring_k"][:, r].astype(np.float32)))
    c = t["cold"]
    assert c["k_q"][0].shape == (40, 2, 16) and c["page_table"].shape == (1, 3)
    assert c["k_scales"].shape == (c["k_pages"].shape[0], 2, 16)
    e = synth.tiered_inputs(20261297, 4, 2, 16, 0, 5, 8, 0)
    assert e["cold"]["k_pages"].shape == (1, 2, 16, 16) and np.all(np.isnan(e["cold"]["k_scales"]))
    # the query is the same stream whether or not there is a cold tier
    assert np.array_equal(e["q"], t["q"])
