"""Host-side checks of the benchmark's contract (no GPU): more than one GPU
is refused with a JSON message, and the rocprofv3 counter summarizer takes
the median per dispatch of every counter of the named kernel."""

import json
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_counter_summary_median_per_dispatch(tmp_path):
    sys.path.insert(0, str(ROOT))
    import bench
    d = tmp_path / "pmc"
    d.mkdir()
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    for disp, v in ((1, 10), (2, 30), (3, 20)):
        rows.append(f'{disp},"void cam::k_proj_direct<false>(cam::Proj)",SQ_LDS_BANK_CONFLICT,{v}')
        rows.append(f'{disp},"void cam::k_proj_direct<false>(cam::Proj)",SQ_INSTS_LDS,{v * 100}')
    rows.append('4,"void cam::k_pack<16>(cam::Pack)",SQ_LDS_BANK_CONFLICT,999')
    (d / "pmc_counter_collection.csv").write_text("\n".join(rows) + "\n")
    out = tmp_path / "summary.txt"
    bench.summarize_counters(str(d), "k_proj_direct", str(out), "command: example")
    text = out.read_text()
    assert text.startswith("command: example\n")
    lines = {ln.split()[0]: ln.split() for ln in text.splitlines() if ln.startswith("  SQ_")}
    assert lines["SQ_LDS_BANK_CONFLICT"][1] == "20" and lines["SQ_LDS_BANK_CONFLICT"][2] == "dispatches=3"
    assert lines["SQ_INSTS_LDS"][1] == "2000"
    assert "k_pack" not in text


def test_ab_verdict_rule():
    """Paired A/B decision: faster or slower only beyond twice the null
    control's largest per-pair difference and with every pair agreeing."""
    sys.path.insert(0, str(ROOT))
    import bench
    null = [(100.0, 101.0), (100.0, 99.5), (100.0, 100.2)]           # floor 1%
    faster = [(100.0, 97.0), (100.0, 96.5), (100.0, 97.5)]           # -3%, all pairs
    assert bench.ab_verdict(null, faster)["verdict"] == "B faster"
    assert bench.ab_verdict(null, faster)["noise_floor_pct"] == 1.0
    assert bench.ab_verdict(null, [(100.0, 98.5), (100.0, 98.6), (100.0, 98.4)])["verdict"] == "neutral"  # < 2%
    mixed = [(100.0, 96.0), (100.0, 101.0), (100.0, 96.0)]
    assert bench.ab_verdict(null, mixed)["verdict"] == "neutral"     # a pair disagrees
    slower = [(100.0, 104.0), (100.0, 103.0), (100.0, 105.0)]
    assert bench.ab_verdict(null, slower)["verdict"] == "B slower"


def test_kernel_source_hash_covers_every_library_source():
    """Every source compiled into libcam.so takes part in the hash that keys
    the stored hardware counters, so a change to any of them retires them."""
    import bench
    from context_attention_movement_amd import build as cam_build
    headers = {p.name for p in cam_build.CSRC.glob("*.h")}
    assert set(cam_build.SOURCES) | headers <= set(bench.KERNEL_SOURCES)
