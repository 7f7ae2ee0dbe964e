"""Host checks of the diagnostic tool (no GPU): the LDS microbenchmark's
pattern families."""

from tiled_movement_amd import lds_bankbench as LB


def test_subword_patterns_cover_both_widths_and_directions():
    pats = LB.patterns({"subword"})
    widths = {(p["width"], p["write"]) for p in pats}
    assert widths == {(1, 0), (1, 1), (2, 0), (2, 1)}
    for p in pats:
        assert len(p["addrs"]) == 64 and all(0 <= a < 96 * 1024 for a in p["addrs"])
        active = [l for l in range(64) if (p["mask"] >> l) & 1]
        assert active, p["name"]
    # the same-word pairs put lanes 0 and j on two parts of one 4-byte word
    for p in pats:
        if "/sameword/" in p["name"]:
            j = int(p["name"].rsplit("/", 1)[1])
            assert p["addrs"][0] // 4 == p["addrs"][j] // 4 and p["addrs"][0] != p["addrs"][j]


def test_kernel_patterns_include_the_small_element_narrow_kinds():
    names = {p["name"].split("/")[1] for p in LB.patterns({"kernel"})}
    assert {"hnarrow8", "bnarrow16", "scalar_col", "mfma"} <= names
