"""Host-side checks of bench.py's measurement plumbing (no GPU): the refusal
of multi-GPU runs, and the rocprofv3 summaries, computed from small databases
that have the tables and columns rocprofv3 writes and numbers chosen so that
every figure is known in advance."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

GEMM = "vbq::(anonymous namespace)::k_gemm(vbq::(anonymous namespace)::GemmArgs)"
GEMV = "void vbq::k_gemv<1, 8, false>(vbq::GemvLaunch)"


def _pmc_db(path, dispatches):
    """dispatches: (dispatch_id, kernel, start_ns, end_ns, {counter: [value per instance]})."""
    c = sqlite3.connect(path)
    c.execute("create table rocpd_info_pmc (id integer, guid text, name text)")
    c.execute("create table rocpd_pmc_event (id integer, guid text, event_id integer, pmc_id integer, value real)")
    c.execute("create table rocpd_kernel_dispatch (event_id integer, guid text, dispatch_id integer, "
              "start integer, end integer)")
    c.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
              "value real, grid_size integer, workgroup_size integer)")
    names = sorted({n for d in dispatches for n in d[4]})
    for i, n in enumerate(names):
        c.execute("insert into rocpd_info_pmc values (?, 'g', ?)", (i, n))
    ev = 0
    for did, kernel, start, end, counters in dispatches:
        ev += 1
        c.execute("insert into rocpd_kernel_dispatch values (?, 'g', ?, ?, ?)", (ev, did, start, end))
        for n, values in counters.items():
            for v in values:
                c.execute("insert into rocpd_pmc_event (guid, event_id, pmc_id, value) values ('g', ?, ?, ?)",
                          (ev, names.index(n), v))
                c.execute("insert into counters_collection values (?, ?, ?, ?, ?, 512)",
                          (did, kernel, n, v, 512 * (729 if did % 2 else 498)))
    c.commit()
    c.close()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_summarize_mfma(tmp_path):
    gui = 200.0                                  # busiest XCD; the others read less
    busy = 1024 * gui * 0.25                     # a quarter of all SIMD cycles
    flops = 2.0 * 256 * 14336 * 4096
    gemm = {"GRBM_GUI_ACTIVE": [120.0, gui, 150.0],
            "SQ_VALU_MFMA_BUSY_CYCLES": [busy / 2, busy / 2],
            "SQ_INSTS_VALU_MFMA_MOPS_BF16": [flops / 512 / 2, flops / 512 / 2],
            "SQ_VALU_MFMA_COEXEC_CYCLES": [busy * 0.5],
            "SQ_INSTS_MFMA": [1000.0],
            "SQ_INSTS_VALU": [5000.0],
            "SQ_BUSY_CU_CYCLES": [256 * gui * 0.8]}
    other = {"GRBM_GUI_ACTIVE": [9e9], "SQ_VALU_MFMA_BUSY_CYCLES": [9e9]}
    _pmc_db(str(tmp_path / "m_results.db"),
            [(1, "vbq::k_pack_tiles(...)", 0, 10, other), (2, GEMM, 1000, 1100, gemm), (3, GEMM, 2000, 2100, gemm)])
    text = bench.summarize_mfma(str(tmp_path), "the command", flops)
    assert "| k_gemm dispatches | 2 |" in text
    assert "(2.00 GHz over the duration)" in text      # 200 cycles in 100 ns
    assert "**25.0 %**" in text
    assert "| SQ_VALU_MFMA_COEXEC_CYCLES / busy | 50.0 % |" in text
    assert "CUs holding work | 80.0 % |" in text
    assert f"{flops:.4g} flop (2 M N K = {flops:.4g})" in text
    assert "the command" in text


def test_summarize_pmc(tmp_path):
    cal = bench.COPY_CAL_BYTES / 1024.0          # KiB one calibration copy moves each way
    _pmc_db(str(tmp_path / "f_results.db"),
            [(1, "at::native::neg_kernel", 0, 1, {"FETCH_SIZE": [cal / 4, cal / 4]}),
             (2, GEMV, 0, 1, {"FETCH_SIZE": [600.0, 400.0]}),
             (3, GEMV, 0, 1, {"FETCH_SIZE": [1000.0]})])
    _pmc_db(str(tmp_path / "w_results.db"),
            [(1, "at::native::neg_kernel", 0, 1, {"WRITE_SIZE": [cal]}),
             (2, GEMV, 0, 1, {"WRITE_SIZE": [10.0]})])
    res = bench.summarize_pmc(str(tmp_path / "f_results.db"), str(tmp_path / "w_results.db"))
    f, w = res["FETCH_SIZE"], res["WRITE_SIZE"]
    assert f["copy_factor"] == pytest.approx(2.0) and w["copy_factor"] == pytest.approx(1.0)
    assert f["gemv_dispatches"] == 2 and f["kib_per_gemv_dispatch"] == pytest.approx(1000.0)
    assert f["bytes_per_gemv_dispatch"] == pytest.approx(1000.0 * 1024 * 2)
    assert w["bytes_per_gemv_dispatch"] == pytest.approx(10.0 * 1024)


def test_summarize_pmc_needs_the_calibration(tmp_path):
    _pmc_db(str(tmp_path / "f_results.db"), [(2, GEMV, 0, 1, {"FETCH_SIZE": [1.0]})])
    _pmc_db(str(tmp_path / "w_results.db"), [(2, GEMV, 0, 1, {"WRITE_SIZE": [1.0]})])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(tmp_path / "f_results.db"), str(tmp_path / "w_results.db"))


def test_summarize_trace(tmp_path):
    c = sqlite3.connect(str(tmp_path / "kt_results.db"))
    c.execute("create table kernels (name text, duration integer, grid_x integer, workgroup_x integer, "
              "lds_size integer, vgpr_count integer, sgpr_count integer)")
    rows = [(GEMV, 26000, 498 * 512, 512, 79616, 52, 112), (GEMV, 28000, 498 * 512, 512, 79616, 52, 112),
            (GEMV, 45000, 729 * 512, 512, 81664, 52, 112), (GEMM, 55000, 224 * 512, 512, 150528, 112, 112)]
    c.executemany("insert into kernels values (?, ?, ?, ?, ?, ?, ?)", rows)
    c.commit()
    c.close()
    text = bench.summarize_trace(str(tmp_path), "cmd")
    assert "| `vbq::k_gemv<1, 8, false>` | 498 | 512 | 79616 | 52 | 112 | 2 | 27.00 | 26.00 | 28.00 | 54.0 |" in text
    assert "| `vbq::k_gemv<1, 8, false>` | 729 |" in text
    assert "| `vbq::k_gemm` | various |" in text          # anonymous namespace dropped from the name
    assert "All `k_gemv` dispatches: 3 calls, average 33.00 us." in text


def test_read_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    p = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(p))
    assert bench.read_traffic(32, 1) is None                       # no summary
    doc = dict(kernel_source_sha=bench.kernel_source_sha(), layers=32, batch=1, bytes_per_launch=123.0)
    p.write_text(json.dumps(doc))
    assert bench.read_traffic(32, 1) == 123.0
    assert bench.read_traffic(8, 1) is None                        # another workload
    p.write_text(json.dumps(dict(doc, kernel_source_sha="0" * 16)))
    assert bench.read_traffic(32, 1) is None                       # counters of other kernel sources


def test_summarize_counters(tmp_path):
    _pmc_db(str(tmp_path / "g_results.db"),
            [(1, GEMV, 0, 10, {"SQ_INSTS_VALU": [100.0, 300.0], "GRBM_GUI_ACTIVE": [50.0, 70.0]}),
             (2, GEMV, 0, 10, {"SQ_INSTS_VALU": [500.0], "GRBM_GUI_ACTIVE": [90.0, 80.0]}),
             (4, GEMV, 0, 10, {"SQ_INSTS_VALU": [700.0], "GRBM_GUI_ACTIVE": [110.0]}),
             (3, "at::native::other", 0, 10, {"SQ_INSTS_VALU": [1e9], "GRBM_GUI_ACTIVE": [1e9]})])
    text = bench.summarize_counters(str(tmp_path), "k_gemv", "cmd")
    assert "Launches of 498 workgroups (2 dispatches)" in text     # dispatches 2 and 4
    assert "Launches of 729 workgroups (1 dispatches)" in text     # dispatch 1
    part498 = text.split("Launches of 498")[1].split("Launches of 729")[0]
    assert "| SQ_INSTS_VALU | 600 |" in part498                      # (500 + 700) / 2
    assert "| GRBM_GUI_ACTIVE | 100 |" in part498                    # busiest XCD: (90 + 110) / 2
    assert "| SQ_INSTS_VALU | 400 |" in text.split("Launches of 729")[1]


def test_workload_parity_recomputes_every_kind():
    """bench.workload_parity regenerates each workload's rows from the seeded
    draws and compares them with the given outputs: outputs equal to the
    oracle's (here computed by the oracle itself, then perturbed by a known
    relative 1e-6 or 1e-2) give that rel-L2 for every kind of output (GEMV at
    one and four rows, fp16 and compact in-cell residuals, levels, GEMM), and
    a sampled matrix is compared on its sampled rows only."""
    import numpy as np

    import oracle
    import synth
    outs = []
    cases = [("gemv", 0, 0, synth.C0.projs[0], 1), ("gemv", 1, 1, synth.C1.projs[1], 4),
             ("resid16", 2, 0, synth.C2.projs[0], 1), ("cell8", 2, 0, synth.C2.projs[0], 1),
             ("levels", 2, 0, synth.C2.projs[0], 1), ("gemm", 4, 0, synth.C4.projs[0], 8)]
    for i, (kind, cid, pi, proj, B) in enumerate(cases):
        p = synth.Proj(proj.name, 96, proj.k, proj.mix)
        key = synth.proj_key(cid, 0, pi)
        W = synth.weights(synth.SEED, key, p.n, p.k)
        q, s, o = oracle.quantize_matrix(W, synth.widths(synth.SEED, key, p.n, p.k // 64, p.mix))
        if kind == "gemm":
            y = oracle.gemm_bf16_weights(q, s, o, synth.x_bf16(synth.SEED, key, B, p.k))
        elif kind == "levels":
            lv, _ = oracle.rrq_levels(W, 4)
            y = oracle.rrq_gemv(lv, synth.x_f16(synth.SEED, key, 1, p.k))
        else:
            x = synth.x_f16(synth.SEED, key, B, p.k)
            f = synth.cell_f(synth.SEED, key, p.n, p.k)
            y = (oracle.gemv(q, s, o, x) if kind == "gemv" else
                 oracle.gemv(q, s, o, x, resid=oracle.cell8_decode(f, s)) if kind == "resid16" else
                 oracle.gemv_cell8(q, s, o, x, f))
        eps = 1e-2 if i == 2 else 1e-6
        outs.append(dict(name=f"{kind}{i}", kind=kind, cid=cid, layer=0, pi=pi, proj=p, B=B, y=y * (1 + eps)))
    res = bench.workload_parity(outs, max_rows=40)
    for i, (kind, *_rest) in enumerate(cases):
        r = res["outputs"][f"{kind}{i}"]
        assert r["rows"] == 40
        assert abs(r["rel_l2"] - (1e-2 if i == 2 else 1e-6)) < 1e-9
    assert abs(res["max_rel_l2"] - 1e-2) < 1e-9
