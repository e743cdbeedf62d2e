"""The benchmark's host logic, on the CPU: kernel-name parsing, the
algorithmic byte counts every bandwidth figure divides by, the rocprofv3
summaries (kernel statistics and the calibrated HBM byte counters) on
synthetic CSV files with known answers, and the refusal of more than one
GPU. The byte counts need the library (for the layout), not a GPU."""

import csv
import dataclasses
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from fsdp_sharded_mixed_zero_amd import synth, zero  # noqa: E402

needs_lib = pytest.mark.skipif(not os.path.exists(zero.LIB_PATH), reason="libzero_mi355x.so not built")


def test_kernel_name():
    cases = {
        "void (anonymous namespace)::copy_pieces_kernel<true>((anonymous namespace)::CopyPieces, double*)":
            "copy_pieces_kernel<true>",
        "(anonymous namespace)::sqnorm_final_kernel(double const*, long, double*, int)": "sqnorm_final_kernel",
        "void (anonymous namespace)::adamw_vec_kernel<unsigned short>((anonymous namespace)::AdamWArgs)":
            "adamw_vec_kernel<unsigned short>",
        "accumulate_kernel": "accumulate_kernel",
    }
    for raw, short in cases.items():
        assert bench.kernel_name(raw) == short


@needs_lib
def test_algorithmic_bytes_modes():
    wl = synth.WORKLOADS["tiny"]
    S = 262_144
    s, real, b = bench.algorithmic_bytes(wl)
    assert (s, real) == (S, S)
    # default: the norm fused into pack, the unpack fused into AdamW (2 more bytes)
    assert b == {"copy_pieces_kernel<true>": 4 * S, "adamw_unpack_vec_kernel<unsigned short>": 30 * S}
    _, _, b = bench.algorithmic_bytes(wl, separate_unpack=True)
    assert b == {"copy_pieces_kernel<false>": 4 * S, "copy_pieces_kernel<true>": 4 * S,
                 "adamw_vec_kernel<unsigned short>": 28 * S}
    _, _, b = bench.algorithmic_bytes(wl, separate_norm=True, separate_unpack=True)
    assert b == {"copy_pieces_kernel<false>": 8 * S, "sqnorm_partial_kernel": 2 * S,
                 "adamw_vec_kernel<unsigned short>": 28 * S}
    _, _, b = bench.algorithmic_bytes(wl, separate_norm=True)
    assert b == {"copy_pieces_kernel<false>": 4 * S, "sqnorm_partial_kernel": 2 * S,
                 "adamw_unpack_vec_kernel<unsigned short>": 30 * S}
    _, _, b = bench.algorithmic_bytes(wl, accum=4)
    assert b == {"copy_pieces_kernel<false>": 4 * 4 * S, "accumulate_kernel": (6 + 30) * S,
                 "sqnorm_f32_partial_kernel": 4 * S, "adamw_unpack_vec_kernel<float>": 32 * S}
    _, _, b = bench.algorithmic_bytes(wl, accum=4, separate_unpack=True)
    assert b == {"copy_pieces_kernel<false>": 4 * S + 4 * 4 * S, "accumulate_kernel": (6 + 30) * S,
                 "sqnorm_f32_partial_kernel": 4 * S, "adamw_vec_kernel<float>": 30 * S}
    _, _, b = bench.algorithmic_bytes(wl, flat=True)
    assert b == {"sqnorm_partial_kernel": 2 * S, "adamw_vec_kernel<unsigned short>": 28 * S}
    # three state arrays: the unpack is its own pass
    _, _, b = bench.algorithmic_bytes(wl, state_arrays=True)
    assert b == {"copy_pieces_kernel<false>": 4 * S, "copy_pieces_kernel<true>": 4 * S,
                 "adamw_arrays_vec_kernel<unsigned short>": 28 * S}
    assert bench.update_kernel(state_arrays=True) == "adamw_arrays_vec_kernel<unsigned short>"


@needs_lib
def test_algorithmic_bytes_with_padding():
    # GPT-2 1.5B's last rank holds 7,488 padding elements: pack writes 2 bytes
    # there and reads nothing, unpack moves nothing
    wl = dataclasses.replace(synth.WORKLOADS["gpt2-1.5b"], rank=63)
    S, real, b = bench.algorithmic_bytes(wl)
    assert S - real == 7_488
    assert b["copy_pieces_kernel<true>"] == 4 * real + 2 * (S - real)
    assert b["adamw_unpack_vec_kernel<unsigned short>"] == 28 * S + 2 * real   # no tensor writes on padding
    _, _, b = bench.algorithmic_bytes(wl, separate_unpack=True)
    assert b["copy_pieces_kernel<false>"] == 4 * real
    assert b["adamw_vec_kernel<unsigned short>"] == 28 * S


def _write_csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


NS = "(anonymous namespace)::"
FINAL = f"{NS}sqnorm_final_kernel(double const*, long, double*, int)"
PARTIAL = f"{NS}sqnorm_partial_kernel(unsigned short const*, long, long, double*)"


def _setup_launches(wl):
    """The trace rows of the set-up launches (the other ranks' partial sums,
    one partial and one final kernel each) that precede the first step."""
    n = bench.setup_sqnorm_launches(wl)
    rows = []
    for j in range(n):
        rows += [{"Kernel_Name": PARTIAL, "Start_Timestamp": 10 * j, "End_Timestamp": 10 * j + 4},
                 {"Kernel_Name": FINAL, "Start_Timestamp": 10 * j + 5, "End_Timestamp": 10 * j + 9}]
    return n, rows


@needs_lib
def test_setup_launch_count():
    """The tiny model's rank 1 of 4 holds tensors 2 and 3: the six others are
    each in one other rank's shard."""
    assert bench.setup_sqnorm_launches(synth.WORKLOADS["tiny"]) == 6


@needs_lib
def test_stats_summary_table(tmp_path):
    wl = synth.WORKLOADS["tiny"]
    S = 262_144
    names = {"adamw": f"void {NS}adamw_vec_kernel<unsigned short>({NS}AdamWArgs)",
             "pack": f"void {NS}copy_pieces_kernel<true>({NS}CopyPieces, double*)",
             "unpack": f"void {NS}copy_pieces_kernel<false>({NS}CopyPieces, double*)",
             "final": FINAL}
    # the set-up launches, then 12 steps: AdamW 2 us per launch (1.9 to 2.1),
    # pack and unpack 1 us, the final sum 3 us
    n_setup, trace = _setup_launches(wl)
    dur = {"adamw": 2000, "pack": 1000, "unpack": 1000, "final": 3000}
    t = 1_000_000
    for k in range(12):
        for key, d in dur.items():
            d = d + (100 if k == 0 else -100 if k == 1 else 0) if key == "adamw" else d
            trace.append({"Kernel_Name": names[key], "Start_Timestamp": t, "End_Timestamp": t + d})
            t += d + 500
    _write_csv(str(tmp_path / "prof" / "x" / "bench_kernel_trace.csv"),
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    md = bench.stats_summary(str(tmp_path / "prof"), wl, steps=10, warmup=2, separate_unpack=True)
    assert "--steps 10 --warmup 2 --separate-unpack --no-cpu-baseline --no-copy-ceiling" in md
    assert "12 steps traced" in md and f"The {n_setup} launches" in md
    table = {line.split("|")[1].strip(): [c.strip() for c in line.split("|")[2:-1]]
             for line in md.splitlines() if line.startswith("| ") and not line.startswith("| kernel |")}
    adamw = table["adamw_vec_kernel<unsigned short>"]
    assert adamw[0] == "12" and adamw[1] == "1.00" and adamw[2] == "2.0"
    assert adamw[3] == "1.9" and adamw[4] == "2.1"
    assert int(adamw[5]) == 28 * S
    assert float(adamw[6]) == pytest.approx(28 * S / 2e-6 / 1e9, abs=0.1)
    assert float(adamw[7]) == pytest.approx(100 * 28 * S / 2e-6 / 1e9 / 8000, abs=0.1)
    assert float(adamw[8]) == pytest.approx(2.0)                        # busy us per step
    assert int(table["copy_pieces_kernel<false>"][5]) == 4 * S
    final = table["sqnorm_final_kernel"]
    assert final[0] == "12" and final[2] == "3.0" and final[5] == "-"   # the set-up launches left out


def test_stats_summary_busy_time_is_the_union_of_launches(tmp_path):
    """Launches on two streams overlap: the busy time per step is the union
    of the launch intervals, and the rate over it counts each byte once."""
    wl = synth.WORKLOADS["tiny"]
    S = 262_144
    adamw = f"void {NS}adamw_vec_kernel<unsigned short>({NS}AdamWArgs)"
    final = FINAL
    # the set-up launches, then two steps; in each, two 2 us launches
    # overlapping by 1 us (3 us busy)
    _, trace = _setup_launches(wl)
    for t0 in (1_000_000, 1_010_000):
        trace += [{"Kernel_Name": adamw, "Start_Timestamp": t0, "End_Timestamp": t0 + 2000},
                  {"Kernel_Name": adamw, "Start_Timestamp": t0 + 1000, "End_Timestamp": t0 + 3000},
                  {"Kernel_Name": final, "Start_Timestamp": t0 + 5000, "End_Timestamp": t0 + 5100}]
    _write_csv(str(tmp_path / "prof" / "x" / "bench_kernel_trace.csv"),
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    md = bench.stats_summary(str(tmp_path / "prof"), wl, steps=2, warmup=0, flat=True)
    row = [line for line in md.splitlines() if line.startswith("| adamw_vec_kernel")][0]
    cells = [c.strip() for c in row.split("|")[1:-1]]
    assert float(cells[9]) == pytest.approx(3.0)                        # busy us per step
    assert float(cells[10]) == pytest.approx(28 * S / 3e-6 / 1e9, abs=0.1)


def _counter_csvs(tmp_path, raw, wl, small_copy=None):
    """Counter rows: the set-up launches first (the other ranks' partial sums:
    counter values that must not count), then 5 dispatches of each kernel in
    ``raw`` (grid 1000), the final sum once per step (the step count); with
    ``small_copy`` (fetch, write), 5 more copy dispatches on a smaller grid
    (the copy ceiling's copy of the pack's size)."""
    n_setup = bench.setup_sqnorm_launches(wl)
    for counter, k in (("FETCH_SIZE", 0), ("WRITE_SIZE", 1)):
        rows, d = [], 0
        for _ in range(n_setup):
            for name in ("sqnorm_partial_kernel", "sqnorm_final_kernel"):
                rows.append({"Dispatch_Id": d, "Grid_Size": 64, "Kernel_Name": f"void {NS}{name}(x)",
                             "Counter_Name": counter, "Counter_Value": 1e9})
                d += 1
        for name, vals in dict(raw, sqnorm_final_kernel=(1.0, 0.0)).items():
            for _ in range(5):
                rows.append({"Dispatch_Id": d, "Grid_Size": 1000, "Kernel_Name": f"void {NS}{name}(x)",
                             "Counter_Name": counter, "Counter_Value": vals[k]})
                d += 1
        if small_copy:
            for _ in range(5):
                rows.append({"Dispatch_Id": d, "Grid_Size": 10, "Kernel_Name": f"void {NS}copy_pieces_kernel<false>(x)",
                             "Counter_Name": counter, "Counter_Value": small_copy[k]})
                d += 1
        _write_csv(str(tmp_path / counter / "y" / "bench_counter_collection.csv"),
                   ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    return str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE")


@needs_lib
def test_pmc_summary_calibration_from_the_copy_ceiling(tmp_path):
    """Default mode: the copy ceiling's plain copy (4 bytes per element of its
    buffers, sized from the update's bytes per launch) calibrates the
    counters; FETCH_SIZE reading half the bytes and WRITE_SIZE all of them (as
    measured on MI355X) give factors 2 and 1, and the fused update whose raw
    counters match its 30 bytes per element comes out at 1.0."""
    wl = synth.WORKLOADS["tiny"]
    S = 262_144
    copy, update = "copy_pieces_kernel<false>", "adamw_unpack_vec_kernel<unsigned short>"
    n = bench.ceiling_elems(30 * S)
    assert n == 30 * S // 4
    raw = {copy: (2 * n / 1024 / 2, 2 * n / 1024), update: (14 * S / 1024 / 2, 16 * S / 1024),
           "copy_pieces_kernel<true>": (2 * S / 1024 / 2, 2 * S / 1024)}
    out = bench.pmc_summary(*_counter_csvs(tmp_path, raw, wl, small_copy=(7.0, 3.0)), wl, steps=3, warmup=2)
    assert out["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert out["calibration"]["write_factor"] == pytest.approx(1.0)
    assert out["kernels"][update]["algorithmic_bytes"] == 30 * S
    assert out["kernels"][update]["traffic_over_algorithmic"] == pytest.approx(1.0)
    assert out["kernels"]["copy_pieces_kernel<true>"]["traffic_over_algorithmic"] == pytest.approx(1.0)
    assert "--no-copy-ceiling" not in out["commands"][1] and "TMPDIR" in out["commands"][0]


@needs_lib
def test_pmc_summary_calibration(tmp_path):
    """--separate-unpack: the unpack calibrates the counters (factors 2 and
    1), and a kernel whose raw counters match its algorithmic bytes comes out
    at 1.0."""
    wl = synth.WORKLOADS["tiny"]
    S = 262_144
    copy, adamw = "copy_pieces_kernel<false>", "adamw_vec_kernel<unsigned short>"
    raw = {copy: (2 * S / 1024 / 2, 2 * S / 1024), adamw: (14 * S / 1024 / 2, 14 * S / 1024 * 1.01)}
    out = bench.pmc_summary(*_counter_csvs(tmp_path, raw, wl), wl, steps=3, warmup=2, separate_unpack=True)
    assert out["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert out["calibration"]["write_factor"] == pytest.approx(1.0)
    assert out["kernels"][copy]["traffic_over_algorithmic"] == pytest.approx(1.0)
    a = out["kernels"][adamw]
    assert a["algorithmic_bytes"] == 28 * S
    assert a["traffic_bytes"] == pytest.approx(14 * S + 14 * S * 1.01, rel=1e-6)
    assert a["traffic_over_algorithmic"] == pytest.approx(1.005, abs=1e-4)
    assert "--steps 3 --warmup 2" in out["commands"][1]
    json.dumps(out)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_single_launch_calls():
    """Which workloads' update calls are one kernel launch (the roofline is
    then per launch): the 7.5B shard and the 70B buckets are, the 7B shard
    (1.68 G elements) is not, and 100 tensors in one call are not for the
    fused update."""
    import types

    from fsdp_sharded_mixed_zero_amd import synth, zero

    def fake(sizes, n_d, rank, align, bucket):
        lay = zero.zero_layout(sizes, n_d, rank, align)
        S = lay.info["shard"]
        pieces = [(0, S)] if bucket <= 0 else [(b, min(bucket, S - b)) for b in range(0, S, bucket)]
        return types.SimpleNamespace(pieces=lambda: pieces, segments=lay.segments)

    W = synth.WORKLOADS
    for name, want in (("gpt-7.5b", True), ("gpt2-1.5b", True), ("llama-70b", True), ("llama-7b", False)):
        wl = W[name]
        assert bench.single_launch_calls(fake(wl.sizes, wl.n_d, wl.rank, wl.align, wl.bucket), True) == want, name
    many = fake([10] * 100, 1, 0, 1, 0)
    assert not bench.single_launch_calls(many, True) and bench.single_launch_calls(many, False)


def test_code_hash_ignores_comments_not_code():
    src = 'int f(int x) { // a comment\n  return x + 1; /* block\n comment */ }\nconst char* s = "a // b /* c";\n'
    same = 'int f(int x) {\n  return x + 1;   }\n// other words\nconst char* s = "a // b /* c";'
    other = 'int f(int x) { return x + 2; }\nconst char* s = "a // b /* c";'
    assert bench.code_text(src) == bench.code_text(same)
    assert bench.code_text(src) != bench.code_text(other)
    assert '"a // b /* c"' in bench.code_text(src)
    assert len(bench.source_hash()) == 64
