"""bench.py's host side, on the CPU: a request for more than one GPU exits with a message; the
algorithmic byte counts are the sums of what one step must touch; the committed traffic summary is
used only while it matches the kernel source; the trace and MFMA summarisers read rocprofv3 tables."""
import hashlib
import os
import shutil
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from compressed_sparse_attention_03_amd import inputs as gen  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""                       # no JSON line for a configuration not measured


def test_algorithmic_bytes_of_the_decode_steps():
    # 1M CSA decode, B = 4, MXFP4 keys (64 B of e2m1 codes + 4 scale bytes per entry)
    keys = 262_144 * (64 + 4)
    query = 64 * 128 * 2 + 64 * 4                       # bf16 indexer query and its fp32 head weights
    assert bench.index_score_bytes(gen.CSA_DECODE_1M) == 4 * (keys + query) == 71_369_728
    rows = (1024 + 128) * 512 * 2                       # selected entries + window rows, bf16
    q_out = 2 * 64 * 512 * 2                            # attention query in, output out
    sel = 1024 * 4 * 2                                  # top-k indices written, then read
    assert 4 * bench.csa_query_bytes(gen.CSA_DECODE_1M) == 4 * (keys + rows + q_out + query + sel)
    # 128K CSA decode, B = 16, fp8 keys (128 B of e4m3 codes + a 4-byte scale per entry)
    keys = 32_768 * (128 + 4)
    assert 16 * bench.csa_query_bytes(gen.CSA_DECODE_128K) == 16 * (keys + rows + q_out + query + sel)
    # HCA 1M decode, B = 8: every entry and the window, bf16, plus query and output
    assert 8 * bench.hca_query_bytes(gen.HCA_DECODE_1M) == 8 * ((8_192 + 128) * 512 * 2 + q_out)


def test_traffic_summary_follows_the_kernel_source(tmp_path, monkeypatch):
    # a summary taken on the current kernel source is used; the same summary beside a source that
    # differs from the one it was taken on is ignored
    name = "index_score_csa_decode_1m_b4_mxfp4_pmc.txt"
    src = open(os.path.join(ROOT, "compressed_sparse_attention_03_amd", "csrc", "indexer.hip")).read()
    sha = hashlib.sha256(src.encode()).hexdigest()[:16]
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / name).write_text(
        f"kernel = index_score_kernel\nsource = indexer.hip\nsource_sha256_16 = {sha}\n"
        "traffic_bytes_per_dispatch = 72306425\n")
    csrc = tmp_path / "compressed_sparse_attention_03_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "indexer.hip").write_text(src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profile_traffic("index_score", "csa_decode_1m_b4_mxfp4") == 72306425.0
    (csrc / "indexer.hip").write_text(src + "\n// changed\n")
    assert bench.profile_traffic("index_score", "csa_decode_1m_b4_mxfp4") is None


def test_summarize_trace_reads_a_kernel_table(tmp_path):
    db = tmp_path / "trace.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, grid_x int, grid_y int, workgroup_x int, duration int, "
                "start int)")
    rows = [("void csa::(anonymous namespace)::k<1>(csa::Args)", 64, 1, 64, d, s)
            for s, d in ((0, 1000), (5000, 2000), (9000, 3000))]
    rows.append(("void other(int)", 8, 1, 8, 500, 20000))              # fewer than three launches
    con.executemany("insert into kernels values (?, ?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()
    out = bench.summarize_trace(str(db)).splitlines()
    assert out[2] == "| k<1> | 64x1 | 64 | 3 | 2.00 | 1.00 | 3.00 |"
    assert len(out) == 3


def test_summarize_mfma_sums_shader_engines_per_dispatch(tmp_path):
    db = tmp_path / "pmc.db"
    con = sqlite3.connect(db)
    con.execute("create table pmc_events (name text, dispatch_id int, counter_name text, counter_value real)")
    rows = []
    for d in (1, 2):                                    # two dispatches, 32 shader-engine rows each
        rows.append(("k<1>", d, "MfmaUtil", 20.0 + d))
        rows += [("k<1>", d, "SQ_INSTS_VALU_MFMA_MOPS_F8", 1e6 / 32) for _ in range(32)]
        rows += [("k<1>", d, c, 0.0) for c in ("SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_INSTS_VALU_MFMA_MOPS_BF16")]
    con.executemany("insert into pmc_events values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()
    out = bench.summarize_mfma(str(db), ["k<1>"]).splitlines()
    assert out[2] == "| k<1> | 2 | 21.5 | 0.5 | 0.0 | 0.0 |"      # 1e6 x 512 ops = 0.512 GFLOP


def test_summarize_counters_sums_instances_and_forms_ratios(tmp_path):
    # two databases (counter sets of separate runs), two dispatches, two instances per counter
    a, b = tmp_path / "a.db", tmp_path / "b.db"
    for db, rows in ((a, [("SQ_WAVE_CYCLES", 100.0), ("SQ_WAIT_INST_ANY", 30.0)]),
                     (b, [("TCC_HIT_sum", 3.0), ("TCC_MISS_sum", 1.0)])):
        con = sqlite3.connect(db)
        con.execute("create table pmc_events (name text, dispatch_id int, counter_name text, counter_value real)")
        for d in (1, 2):
            for c, v in rows:
                con.executemany("insert into pmc_events values (?, ?, ?, ?)",
                                [("void csa::attend_split_kernel<512, false>(...)", d, c, v / 2)] * 2)
        con.commit()
        con.close()
    out = bench.summarize_counters([str(a), str(b)], ["attend_split_kernel"])
    assert "attend_split_kernel (2 dispatches)" in out
    assert "SQ_WAVE_CYCLES = 100" in out and "SQ_WAIT_INST_ANY = 30" in out
    assert "[wave cycles waiting on a dependency] = 0.300" in out
    assert "[L2 hit rate] = 0.750" in out
