"""Host logic of the benchmark's shader-clock figure: samples are paired per compute unit only."""
import bench


def _sample(pairs, slots):
    """Counter buffer of one sample: pairs maps slot -> (s_memtime, s_memrealtime)."""
    v = [0] * (2 * slots)
    for u, (t, r) in pairs.items():
        v[2 * u], v[2 * u + 1] = t, r
    return v


def test_unit_clocks_pair_each_unit_with_itself():
    slots = 4
    # unit 0: 2.3 GHz over 1 ms; unit 2: 2.1 GHz over 1 ms, its counter offset far from unit 0's;
    # unit 1 written only by the second sample; unit 3 never written
    before = _sample({0: (10_000, 500), 2: (9_000_000_000, 500)}, slots)
    after = _sample({0: (10_000 + 2_300_000, 100_500), 1: (5, 100_500), 2: (9_000_000_000 + 2_100_000, 100_500)},
                    slots)
    units = bench.unit_clocks(before + after, slots)
    assert [round(m, 6) for m, _ in units] == [2300.0, 2100.0]
    assert all(abs(ms - 1.0) < 1e-12 for _, ms in units)


def test_clock_summary_median_and_percentiles():
    units = [(2000.0 + 10 * i, 1.0) for i in range(11)]   # 2000 .. 2100 MHz
    s = bench.clock_summary(units)
    assert s["gfx_mhz_avg"] == 2050.0 and s["units"] == 11
    assert s["gfx_mhz_p10_p90"] == [2010.0, 2090.0]
    assert bench.clock_summary([])["error"]
