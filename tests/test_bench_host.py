"""Host-side pieces of bench.py (no GPU): the single-GPU guard, the
algorithmic work count behind the roofline, the kernel-name decoding of the
trace summaries and the counter arithmetic of the traffic and counter
summaries."""
from __future__ import annotations

import importlib.util
import json
import os
import sqlite3
import subprocess
import sys
import types

import numpy as np
import pytest

import oracle
from tree_verify_mla_kdt_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout


@pytest.mark.parametrize("name", ["max_budget", "ragged_deep", "tiny_fp32"])
def test_visible_pairs_count_the_masks(name):
    """The roofline's work count: H x (q x L_b + set bits of every mask row),
    checked against the oracle's masks."""
    bench = _bench()
    cfg = synth.CONFIGS[name]
    rng = synth.rng_for(77)
    parents = np.stack([synth.make_tree(rng, cfg.tree, cfg.q_len) for _ in range(3)]).astype(np.int32)
    prefix_lens = np.asarray([0, 5, 1000], np.int32)
    vis, _ = oracle.build_visibility(parents)
    bits = sum(bin(int(w)).count("1") for w in vis.reshape(-1))
    want = cfg.H * (cfg.q_len * int(prefix_lens.sum()) + bits)
    assert bench.visible_pairs(parents, prefix_lens, cfg.H) == want


def test_kernel_names_decode():
    bench = _bench()
    assert (bench.short_kernel_name("_ZN3kdt19verify_split_kernelIDF16bLi512ELi64ELb0ELi4ELb0EEEvNS_10VerifyArgsE")
            == "verify_split_kernel<bf16, R=512, P=64, partials, layout 4>")
    assert (bench.short_kernel_name("_ZN3kdt19verify_split_kernelIfLi64ELi16ELb1ELi1ELb0EEEvNS_10VerifyArgsE")
            == "verify_split_kernel<f32, R=64, P=16, direct, layout 1>")
    assert (bench.short_kernel_name("_ZN3kdt19verify_split_kernelIDF16bLi512ELi64ELb0ELi1ELb1EEEvNS_10VerifyArgsE")
            == "verify_split_kernel<bf16, R=512, P=64, partials, layout 1, balanced>")
    assert (bench.short_kernel_name("_ZN3kdt12merge_kernelIDF16bDF16bLb1ELb0ELi16EEEvPKT0_PKfiiiiiiPKiiiPT_lllPf")
            == "merge_kernel<out bf16, partials bf16, wide>")
    assert (bench.short_kernel_name("_ZN3kdt12merge_kernelIDF16bfLb0ELb1ELi4EEEvPKT0_PKfiiiiiiPKiiiPT_lllPf")
            == "merge_kernel<out bf16, partials f32, gated>")
    assert bench.short_kernel_name("_ZN3kdt18absorb_gemm_kernelILi8ELi2EEEvNS_6RowSrcE") == "absorb_gemm_kernel<8, 2>"
    assert bench.short_kernel_name("void kdt::append_kernel(int*, int)") == "kdt::append_kernel"


def _pmc_db(path, events):
    """A counter database with the two tables the summaries read: kernels
    (dispatch_id, name) and pmc_events (counter_name, dispatch_id,
    counter_value), one row per counter instance."""
    con = sqlite3.connect(path)
    con.execute("create table kernels (dispatch_id integer, name text)")
    con.execute("create table pmc_events (counter_name text, dispatch_id integer, counter_value real)")
    names = {}
    for did, name, counter, values in events:
        names[did] = name
        con.executemany("insert into pmc_events values (?, ?, ?)", [(counter, did, v) for v in values])
    con.executemany("insert into kernels values (?, ?)", list(names.items()))
    con.commit()
    con.close()


def test_counter_means_per_dispatch(tmp_path):
    bench = _bench()
    db = str(tmp_path / "pmc.db")
    split = "_ZN3kdt19verify_split_kernelIDF16bLi512ELi64ELb0ELi4ELb0EEEvNS_10VerifyArgsE"
    _pmc_db(db, [(1, split, "FETCH_SIZE", [100.0, 300.0]),          # instances of one dispatch add up
                 (2, split, "FETCH_SIZE", [500.0, 100.0]),
                 (3, "kdt::merge_kernel", "FETCH_SIZE", [9999.0]),   # another kernel: ignored
                 (1, split, "SQ_WAVES", [952.0]),
                 (2, split, "SQ_WAVES", [952.0])])
    assert bench.pmc_kib_per_dispatch(db, "FETCH_SIZE", "verify_split_kernel") == pytest.approx(500.0)
    means = bench.pmc_means(db, "verify_split_kernel")
    assert means == {"FETCH_SIZE": pytest.approx(500.0), "SQ_WAVES": pytest.approx(952.0)}
    with pytest.raises(SystemExit):
        bench.pmc_kib_per_dispatch(db, "WRITE_SIZE", "verify_split_kernel")


def test_traffic_is_scaled_by_the_copy_calibration(tmp_path, monkeypatch):
    """Bytes per launch = counter KiB x 1024 x (copy bytes / what the same
    counter reads for the copy)."""
    bench = _bench()
    split = "_ZN3kdt19verify_split_kernelIDF16bLi512ELi64ELb0ELi4ELb0EEEvNS_10VerifyArgsE"
    copy = "__amd_rocclr_copyBuffer"
    n_mb = 4
    dbs = {}
    for key, counter, name, kib in (("f", "FETCH_SIZE", split, 1000.0), ("w", "WRITE_SIZE", split, 250.0),
                                    ("cf", "FETCH_SIZE", copy, 2.0 * (n_mb << 10)),   # the copy reads 2x
                                    ("cw", "WRITE_SIZE", copy, 1.0 * (n_mb << 10))):
        dbs[key] = str(tmp_path / f"{key}.db")
        _pmc_db(dbs[key], [(1, name, counter, [kib]), (2, name, counter, [kib])])
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda: "test")
    args = types.SimpleNamespace(write_traffic=[dbs["f"], dbs["w"], dbs["cf"], dbs["cw"]], calibration_mb=n_mb,
                                 workload="unit")
    bench.write_traffic(args)
    rec = json.load(open(tmp_path / "profiles" / "traffic_verify_split_unit.json"))
    assert rec["fetch_calibration"] == pytest.approx(0.5) and rec["write_calibration"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == pytest.approx(1000.0 * 1024 * 0.5)
    assert rec["write_bytes_per_launch"] == pytest.approx(250.0 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx(1000.0 * 512 + 250.0 * 1024)
