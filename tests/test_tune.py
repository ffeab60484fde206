"""The per-shape tiling sweep tool (weight_only_quantized_fp8_amd.tune)."""
import pytest


def test_candidates_respect_the_kernel_limits():
    from weight_only_quantized_fp8_amd import tune
    for fmt in ("fp8", "lut3", "lut3d"):
        for gemv in ((False, True) if fmt == "fp8" else (False,)):
            c = tune.candidates(fmt, gemv)
            assert c and len(set(c)) == len(c)
            assert set(tune.candidates(fmt, gemv, kp=3)) <= set(c)
            for nt, sn, split in c:
                assert 1 <= sn <= 8 and split % sn == 0 and split // sn <= 4
                assert nt in ((1,) if gemv else (1, 2))
                assert split <= 8 or gemv or (fmt != "fp8" and nt == 1 and sn >= 4)


@pytest.mark.gpu
@pytest.mark.parametrize("args", [
    ["--fmt", "fp8", "--N", "384", "--K", "1152", "--M", "16", "--top", "3"],
    ["--fmt", "fp8", "--N", "384", "--K", "1152", "--M", "2", "--path", "gemv", "--top", "3"],
    ["--fmt", "lut3", "--N", "272", "--K", "1152", "--M", "24", "--top", "3"],
    ["--fmt", "lut3d", "--N", "272", "--K", "1152", "--M", "7", "--top", "3"],
    ["--fmt", "fp8", "--N", "384", "--K", "1152", "--M", "20", "--kparts", "1,3,9", "--top", "3"],
    ["--fmt", "lut3", "--N", "272", "--K", "2048", "--M", "16", "--kparts", "2", "--top", "3"],
], ids=["fp8-mfma", "fp8-gemv", "lut3-m24", "lut3d-m7", "fp8-kparts", "lut3-kparts"])
def test_every_candidate_passes_the_exactness_gate(args, capsys):
    from weight_only_quantized_fp8_amd import tune
    assert tune.main(args) == 0
    out = capsys.readouterr().out
    assert "0 rejected" in out and "table row (" in out
