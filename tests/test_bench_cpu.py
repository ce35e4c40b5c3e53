"""bench.py's byte accounting against the per-workload figures worked out from the definitions
(algorithmic bytes: what the method must move, no zero padding), and its one-GPU guard. CPU only."""

import subprocess
import sys

import pytest

import bench
from conftest import ROOT
from workloads import WORKLOADS

# (layout, pack, combine) bytes per launch with every entry valid (N = S*K) and C = min(S, 128)
EXPECTED = {
    1: (12_968, 790_528, 788_480),
    2: (224_264, 16_531_456, 16_523_264),
    3: (432_200, 529_006_592, 528_744_448),
    4: (432_200, 294_256_640, 528_744_448),
    5: (1_772_552, 1_058_013_184, 1_057_488_896),
}


@pytest.mark.parametrize("cfg", sorted(EXPECTED))
def test_algorithmic_bytes(cfg):
    w = WORKLOADS[cfg]
    got = bench.algorithmic_bytes(w, w.C, w.S * w.K)
    assert (got["layout"], got["dispatch"], got["combine"]) == EXPECTED[cfg]


def test_per_token_bytes_at_h7168():
    w = WORKLOADS[3]
    b = bench.algorithmic_bytes(w, w.C, w.S * w.K)
    assert b["dispatch"] == 129_152 * w.S and b["combine"] == 129_088 * w.S


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr


def test_code_digest_ignores_comments_only(tmp_path, monkeypatch):
    """The PMC traffic entries are tied to the kernel code, not to its comments."""
    import bench

    csrc = tmp_path / "combine_moe_layout_02_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (csrc / "k.hip").write_text("// header\nint f() { return 1; }  // trailing\n/* block\n comment */\n")
    a = bench.code_digest(["k.hip"])
    (csrc / "k.hip").write_text("// a different header\n\nint f() { return 1; }\n")
    assert bench.code_digest(["k.hip"]) == a
    (csrc / "k.hip").write_text("int f() { return 2; }\n")
    assert bench.code_digest(["k.hip"]) != a


def test_cpu_baseline_fields():
    """The oracle leg of the bench on the tiny workload: one full step, its stages timed apart."""
    from workloads import make_inputs

    w = WORKLOADS[1]
    inp = make_inputs(w)
    n_valid = int(((inp["topk_idx"] >= 0) & (inp["topk_idx"] < w.E)).sum())
    cb = bench.cpu_baseline(w, w.C, inp, inp["expert_out"], n_valid, min_seconds=0.0, max_reps=1)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["cores"] >= 1 and cb["value"] > 0
    assert set(cb["stage_ms"]) == {"layout", "dispatch", "combine"}
    assert all(v >= 0 for v in cb["stage_ms"].values())
    assert cb["sample"].startswith("1 full steps")


@pytest.mark.parametrize("cfg", sorted(EXPECTED))
def test_read_write_split_adds_up(cfg):
    """The read/write split behind the pattern ceilings covers exactly the algorithmic bytes."""
    w = WORKLOADS[cfg]
    nb = bench.algorithmic_bytes(w, w.C, w.S * w.K)
    split = bench.rw_split(w, w.C, w.S * w.K)
    for k in ("layout", "dispatch", "combine"):
        assert sum(split[k]) == nb[k], k


def test_pattern_ceiling():
    ceil = {"read": 7000.0, "fill": 6000.0}
    assert bench.pattern_ceiling(ceil, 1, 0) == pytest.approx(7000.0)
    assert bench.pattern_ceiling(ceil, 0, 1) == pytest.approx(6000.0)
    # equal bytes each way: the harmonic mean of the two rates
    assert bench.pattern_ceiling(ceil, 5, 5) == pytest.approx(2 / (1 / 7000 + 1 / 6000))
    assert bench.pattern_ceiling(None, 1, 1) is None
