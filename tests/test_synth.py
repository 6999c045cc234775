"""The seeded input generator: Philox known answers, distribution shape, and
host/device agreement (device part marked gpu)."""
import numpy as np
import pytest

import synth


def test_philox4x32_10_known_answers():
    # Known-answer vectors published with the Random123 library for
    # philox4x32 with 10 rounds.
    assert synth.philox([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    f = 0xFFFFFFFF
    assert synth.philox([f, f, f, f], [f, f]) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert synth.philox([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344],
                        [0xA4093822, 0x299F31D0]) == [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_keys_distinct():
    ks = {synth.key(w, k, r, m, s) for w in ("flat1m", "llama8b") for k in synth.KIND
          for r in range(3) for m in range(2) for s in range(3)}
    assert len(ks) == 2 * len(synth.KIND) * 3 * 2 * 3


@pytest.mark.parametrize("dist,scale", [("normal", 1e-3), ("absnormal", 1e-6),
                                        ("student_t3", 1e-3), ("normal_zeros", 1e-3)])
def test_distribution_shape(dist, scale):
    n = 400_000
    x = synth.fill_host(n, synth.OUT_F32, [(0, 12345, n, 0)], synth.key("flat1m", "grad", 1),
                        dist, scale).astype(np.float64)
    if dist == "absnormal":
        assert (x >= 0).all()
        assert abs(x.mean() / scale - np.sqrt(2 / np.pi)) < 0.01
    elif dist == "student_t3":
        # t_3: variance 3; heavy tails
        assert abs(np.median(x)) < 0.01 * scale
        assert 2.0 < x.var() / scale ** 2 < 4.5
        assert (np.abs(x) > 10 * scale).mean() > 1e-3
    else:
        z = x[x != 0] if dist == "normal_zeros" else x
        assert abs(z.mean()) < 0.01 * scale and abs(z.std() / scale - 1) < 0.01
        if dist == "normal_zeros":
            assert abs((x == 0).mean() - 0.01) < 0.001


def test_fill_host_matches_values_at_and_pads():
    segs = [(0, 100, 50, 6), (56, 5000, 10, 0), (66, 7, 0, 4)]
    k = synth.key("gpt2s", "master")
    out = synth.fill_host(70, synth.OUT_BF16, segs, k, "normal", 0.02)
    xs = np.concatenate([np.arange(100, 150), -np.ones(6, np.int64), np.arange(5000, 5010),
                         -np.ones(4, np.int64)])
    assert np.array_equal(out, synth.values_at(xs, k, "normal", 0.02, synth.OUT_BF16))
    assert not out[50:56].any() and not out[66:].any()
    f = synth.values_at(xs, k, "normal", 0.02, synth.OUT_F32)
    # bf16 bits are the truncated upper half of the binary32 sample
    assert np.array_equal(out, (f.view(np.uint32) >> 16).astype(np.uint16))


@pytest.mark.gpu
@pytest.mark.parametrize("dist,scale", [("normal", 1e-3), ("absnormal", 1e-6),
                                        ("student_t3", 1e-3), ("normal_zeros", 1e-3)])
def test_device_fill_matches_host(dist, scale):
    import torch
    n = 3_000_001
    segs = [(0, 7, 1_000_000, 3), (1_000_003, 10 ** 10, 1_999_990, 8)]
    k = synth.key("llama70b", "grad", 5, 0, 1001)
    for out_type, dt in ((synth.OUT_BF16, torch.int16), (synth.OUT_F32, torch.float32)):
        dev = torch.full((n,), -1, dtype=dt, device="cuda")
        synth.fill_device(dev, segs, k, dist, scale)
        torch.cuda.synchronize()
        host = synth.fill_host(n, out_type, segs, k, dist, scale)
        got = dev.cpu().numpy().view(host.dtype)
        assert np.array_equal(got.view(np.uint8), host.view(np.uint8))
