"""Host logic of bench.py, on the CPU: kernel names as the counter summaries key
them, the calibration of FETCH_SIZE / WRITE_SIZE by the copy kernel, the
source-hash guard on stored traffic, the routing statistics, the bytes the
combine reads for the second GEMM's cut tiles, and the refusal
of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("symbol,key", [
    ("void moe::(anonymous namespace)::ffn_gemm_bf16<256, 1, false, 0>(unsigned short const*)",
     "ffn_gemm_bf16_up"),
    ("void moe::(anonymous namespace)::ffn_gemm_bf16<256, 2, true, 0>(unsigned short const*)",
     "ffn_gemm_bf16_up"),
    ("void moe::(anonymous namespace)::ffn_gemm_bf16<128, 0, false, 3>(unsigned short const*)",
     "ffn_gemm_bf16_down"),
    ("ffn_gemm_bf16<64, 0, false, 0>", "ffn_gemm_bf16_down"),
    ("void moe::(anonymous namespace)::route_bf16<1, 16, 256, 3, 8, false>(int)", "route_bf16"),
    ("void moe::(anonymous namespace)::combine_rows<true, 256>(float const*)", "combine_rows"),
    ("void moe::(anonymous namespace)::ffn_gemm_fixup<256, 1, 0>(int const*)", "ffn_gemm_fixup"),
    ("scan_columns", "scan_columns"),
])
def test_kernel_key(symbol, key):
    assert bench.kernel_key(symbol) == key


def _pmc_dir(tmp_path, name, counter, rows):
    d = tmp_path / name / "host" / "pid"
    d.mkdir(parents=True)
    with open(d / "p_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for kname, grid, value in rows:
            w.writerow({"Kernel_Name": kname, "Grid_Size": grid, "Counter_Name": counter,
                        "Counter_Value": value})
        # a row of another counter in the same file is ignored
        w.writerow({"Kernel_Name": "combine_rows<true, 256>", "Grid_Size": 1,
                    "Counter_Name": "GRBM_COUNT", "Counter_Value": 1e9})
    return str(tmp_path / name)


def test_summarize_pmc_calibrates_by_the_largest_copy(tmp_path):
    up = "void moe::(anonymous namespace)::ffn_gemm_bf16<256, 1, false, 0>(x)"
    dn = "void moe::(anonymous namespace)::ffn_gemm_bf16<256, 0, false, 0>(x)"
    kib = 256 * 1024.0
    fetch = _pmc_dir(tmp_path, "fetch", "FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", 1024, 0.1 * kib),        # a small copy: not the calibration
        ("__amd_rocclr_copyBuffer", 1 << 20, 0.5 * kib),     # the 256 MiB copy: factor 0.5
        ("fill_kernel", 4096, 123.0),                        # fills are skipped
        (up, 7448, 1000.0), (up, 7448, 3000.0),              # mean 2000 KiB
        (dn, 2128, 500.0)])
    write = _pmc_dir(tmp_path, "write", "WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", 1 << 20, 1.0 * kib),     # factor 1.0
        (up, 7448, 400.0), (up, 7448, 600.0)])               # mean 500 KiB; down writes none
    out, lines = bench.summarize_pmc(fetch, write, "wl", 256)
    assert out["workload"] == "wl" and out["source_hash"] == bench.kernel_source_hash()
    assert out["fetch_factor"] == pytest.approx(0.5) and out["write_factor"] == pytest.approx(1.0)
    assert set(out["kernels"]) == {"ffn_gemm_bf16_up", "ffn_gemm_bf16_down"}
    u, d = out["kernels"]["ffn_gemm_bf16_up"], out["kernels"]["ffn_gemm_bf16_down"]
    assert u["fetch_kib"] == pytest.approx(2000.0) and u["write_kib"] == pytest.approx(500.0)
    assert u["hbm_bytes"] == pytest.approx((2000.0 / 0.5 + 500.0 / 1.0) * 1024.0)
    assert d["write_kib"] is None and d["hbm_bytes"] == pytest.approx(500.0 / 0.5 * 1024.0)
    # the table lists the larger fetch first
    assert lines[2].startswith("| ffn_gemm_bf16_up |") and len(lines) == 4


def test_summarize_pmc_needs_the_calibration_copy(tmp_path):
    fetch = _pmc_dir(tmp_path, "fetch", "FETCH_SIZE", [("combine_rows<true, 256>", 1, 5.0)])
    write = _pmc_dir(tmp_path, "write", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 9, 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(fetch, write, "wl", 256)


def test_traffic_is_reported_only_for_the_same_sources_and_workload(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"source_hash": bench.kernel_source_hash(), "workload": "wl",
           "kernels": {"ffn_gemm_bf16_up": {"hbm_bytes": 1.5e9}}}
    with open(tmp_path / "traffic_wl.json", "w") as fh:
        json.dump(rec, fh)
    assert bench.traffic_for("ffn_gemm_bf16_up", "wl") == 1.5e9
    assert bench.traffic_for("combine_rows", "wl") is None          # not measured
    assert bench.traffic_for("ffn_gemm_bf16_up", "other") is None   # no file
    rec["source_hash"] = "0" * 16                                   # other sources
    with open(tmp_path / "traffic_wl.json", "w") as fh:
        json.dump(rec, fh)
    assert bench.traffic_for("ffn_gemm_bf16_up", "wl") is None
    rec["source_hash"], rec["workload"] = bench.kernel_source_hash(), "other"
    with open(tmp_path / "traffic_wl.json", "w") as fh:
        json.dump(rec, fh)
    assert bench.traffic_for("ffn_gemm_bf16_up", "wl") is None


def test_source_hash_follows_every_library_source(tmp_path, monkeypatch):
    csrc = tmp_path / "sparse_mixture_experts_21_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("kernel a\n")
    (csrc / "b.h").write_text("header b\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    assert h0 == bench.kernel_source_hash() and len(h0) == 16
    (csrc / "b.h").write_text("header b changed\n")
    h1 = bench.kernel_source_hash()
    (csrc / "c.cpp").write_text("")
    h2 = bench.kernel_source_hash()
    assert len({h0, h1, h2}) == 3


def test_routing_stats():
    # E = 4, T = 6, k = 2: loads 5, 4, 3, 0 before capacity 4
    counts = [5, 4, 3, 0]
    offsets = np.cumsum([0, 4, 4, 3, 0])
    s = bench.routing_stats(4, counts, offsets, 4, 6, 2)
    assert s == {"load_max": 5, "load_min": 0, "kept_max": 4, "kept_min": 0,
                 "experts_empty": 1, "capacity": 4, "dropped_pairs": 1,
                 "drop_fraction": pytest.approx(1 / 12)}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


# ---------------------------------------------------------------- combine bytes
def _library_dense_coords(grids, tmp_path):
    """dense_coords exactly as the library's gemm_common.h writes it, compiled
    for the host, printing (mt, nt) for every position of each grid."""
    src = open(os.path.join(ROOT, "sparse_mixture_experts_21_amd", "csrc", "gemm_common.h")).read()
    i = src.index("__device__ __forceinline__ void dense_coords(")
    j = src.index("{", i)
    depth = 0
    for end in range(j, len(src)):
        depth += {"{": 1, "}": -1}.get(src[end], 0)
        if depth == 0:
            break
    fn = src[i:end + 1].replace("__device__ __forceinline__", "static inline")
    lines = "\n".join(f"    run({rm}, {nt}, {sbn});" for rm, nt, sbn in grids)
    prog = ("#include <cstdio>\n" + fn + "\nstatic void run(int rm, int Nt, int SBN) {\n"
            "    for (int p = 0; p < rm * Nt; ++p) { int mt, nt; dense_coords(p, rm, Nt, SBN, mt, nt);"
            " printf(\"%d %d\\n\", mt, nt); }\n}\nint main() {\n" + lines + "\n    return 0;\n}\n")
    c = tmp_path / "dc.cpp"
    c.write_text(prog)
    exe = tmp_path / "dc"
    subprocess.run(["g++", "-O1", "-o", str(exe), str(c)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    return [(int(a), int(b)) for a, b in zip(out[0::2], out[1::2])]


def test_dense_coords_restatement_matches_library(tmp_path):
    grids = [(rm, nt, sbn) for sbn in (4, 8, 16) for nt in (1, 3, 4, 8, 16, 24, 56)
             for rm in (1, 5, 17, 33, 64, 133)]
    want = _library_dense_coords(grids, tmp_path)
    got = [bench._dense_coords(p, rm, nt, sbn) for rm, nt, sbn in grids for p in range(rm * nt)]
    assert got == want


def test_combine_cut_extra_bytes_decode():
    # one token to experts 0 and 1: 2 one-row tiles x 16 column tiles, all cut
    # into min(256 // 32, 448 k-tiles // 4 stages) = 8 slices
    extra = bench.combine_cut_extra_bytes(1, 2, 8, 4096, 14336, 0.0, [1, 1, 0, 0, 0, 0, 0, 0], 256)
    assert extra == 2 * 16 * 1 * 256 * (4 * 8 - 2)


def test_combine_cut_extra_bytes_hand_case():
    # Two experts of 300 rows: 256-row tiles (mean load 300), 2 row tiles each
    # (256 and 44 rows), 3 column tiles (H = 768): 12 tiles, all in the ragged
    # last round of 256 CUs, cut into min(256 // 12, 64 k-tiles // 2 stages) =
    # 21 slices; each cut row reads 21 fp32 slices instead of one bf16 value.
    extra = bench.combine_cut_extra_bytes(300, 2, 2, 768, 4096, 0.0, [300, 300], 256)
    assert extra == 3 * 2 * (256 + 44) * 256 * (4 * 21 - 2)


def test_combine_cut_extra_bytes_no_cut():
    # a whole round has no tail; a tail above half a round is not cut
    assert bench.combine_cut_extra_bytes(8192, 2, 8, 1024, 4096, 0.0, [2048] * 8, 256) == 0
    # 73 row tiles x 16 column tiles = 1168 = 4 rounds + 144 > 128
    assert bench.combine_cut_extra_bytes(18688, 1, 1, 4096, 4096, 0.0, [18688], 256) == 0
    # one more row tile on one expert: 65 x 16 = 1040 = 4 rounds + 16, cut into 16
    assert bench.combine_cut_extra_bytes(8192, 2, 8, 4096, 4096, 0.0,
                                         [2048] * 7 + [2049], 256) > 0
