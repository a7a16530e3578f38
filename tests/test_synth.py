"""The seeded input generator gives bit-identical values on the host (numpy) and through torch, and follows the
published workload shapes."""
import numpy as np
import torch

import kpool_synth as ks


def test_hash_numpy_equals_torch():
    idx = np.arange(0, 1 << 40, (1 << 40) // 50021, dtype=np.int64)
    a = ks.hash32(ks.stream_key(7, "lat"), idx)
    b = ks.hash32(ks.stream_key(7, "lat"), torch.from_numpy(idx)).numpy()
    np.testing.assert_array_equal(a, b)
    assert a.min() >= 0 and a.max() < 2 ** 32


def test_mixer_against_python_ints():
    for x in [0, 1, 12345, 2 ** 31, 2 ** 32 - 1]:
        assert int(ks._mix32(np.int64(x))) == ks._mix32_int(x)


def test_value_ranges():
    u = ks.uniform_int(3, np.arange(200000), -4, 4)
    assert u.min() == -4 and u.max() == 4
    counts = np.bincount(u + 4)
    assert counts.min() > 0.9 * counts.mean()
    t = ks.normal_table("bf16")
    assert abs(t.mean()) < 1e-6 and abs(t.std() - 1) < 1e-3
    # every table value is a bf16 value
    assert (t.view(np.uint32) & 0xFFFF).max() == 0


def test_device_fill_matches_host_rows():
    """The paged caches filled through torch hold the same rows the host generator gives."""
    wl = ks.scaled(ks.workloads()["batch64"], ctx=[300, 77, 129], new_from=[299, 76, 128],
                   q_seq=np.arange(3, dtype=np.int32), q_pos=np.array([299, 76, 128], np.int32))
    lat, pooled = ks.device_caches(wl, "cpu", chunk_pages=2)
    bt = wl.block_table()
    for s, t in [(0, 5), (1, 70), (2, 128), (0, 299)]:
        row = lat[bt[s, t // 64], t % 64].float().numpy()
        np.testing.assert_array_equal(row, ks.host_latent(wl, s, np.array([t]))[0])
    for s, p in [(0, 3), (1, 18), (2, 31)]:
        row = pooled[bt[s, p // 16], p % 16].float().numpy()
        want = ks.host_pool_keys(wl, s, np.array([p]))[0] if p < wl.new_from[s] // 4 else 0 * row
        np.testing.assert_array_equal(row, want)


def test_device_fill_fp8_latent_codes():
    """An fp8 latent cache filled through torch holds the host generator's E4M3 codes; codes stay finite with
    magnitudes in [0.125, 1.875] and the rotary columns hold code 0."""
    import oracle as O
    wl = ks.scaled(ks.workloads()["batch64"], ctx=[300, 77], new_from=[299, 76], q_seq=np.arange(2, dtype=np.int32),
                   q_pos=np.array([299, 76], np.int32), latent_fp8=True, kv_scale=0.5)
    lat, _ = ks.device_caches(wl, "cpu", chunk_pages=2)
    assert lat.dtype == torch.uint8
    bt = wl.block_table()
    for s, t in [(0, 5), (1, 70), (0, 299)]:
        row = lat[bt[s, t // 64], t % 64].numpy()
        np.testing.assert_array_equal(row, ks.host_latent_codes(wl, s, np.array([t]))[0])
    codes = ks.host_latent_codes(wl, 0, np.arange(300))
    v = O.fp8_e4m3_decode(codes)
    assert not np.isnan(v).any() and (v[:, wl.V:] == 0).all()
    assert np.abs(v[:, :wl.V]).min() == 0.125 and np.abs(v[:, :wl.V]).max() == 1.875


def test_batch64_contexts():
    t = ks.cfg3_contexts()
    assert int(t.sum()) == 4151643 and int(t.min()) == 8375 and int(t.max()) == 127811
