"""Host logic of bench.py on the CPU: the algorithmic byte and FLOP counts
behind the roofline figures (pinned on hand-counted cases), the rocprofv3
counter summary and its calibration, the stale-profile rule, and the refusal
of more than one GPU."""

import os
import subprocess
import sys
from dataclasses import replace

import numpy as np
import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402


def test_pcg_bytes_resident_and_streamed():
    # ss=2, kp=3: n=6, S and Pinv 6*6 floats each = 288 B together; vectors
    # x, b read and x written 3*6*4 = 72 B plus the 4-byte count.
    w = replace(workloads.WORKLOADS[0], ss=2, kp=3, dtype=np.float32)
    it = np.array([4, 0])
    assert bench.algorithmic_bytes_pcg(w, it, resident=True) == 2 * (288 + 76)
    # streamed: S and Pinv once per pass, iterations + 1 passes
    assert bench.algorithmic_bytes_pcg(w, it, resident=False) == (5 * 288 + 76) + (1 * 288 + 76)
    # only Pinv's D blocks: S 6*6*4 = 144 B plus Pinv 6*2*4 = 48 B
    assert bench.algorithmic_bytes_pcg(w, it, resident=True, pinv_diag=True) == 2 * (192 + 76)
    # S on chip (144 B once), Pinv (144 B) once per pass
    assert bench.algorithmic_bytes_pcg(w, it, resident="S") == \
        (144 + 5 * 144 + 76) + (144 + 1 * 144 + 76)
    # Pinv rows as the placement reads them (24 B each): all 6 at pass 0,
    # 4 at odd passes and 3 at even ones; 4 iterations are passes 1-4 (two
    # odd, two even), none after the first for the solve that stops at 0.
    assert bench.algorithmic_bytes_pcg(w, it, resident="S", pass_rows=(6, 4, 3)) == \
        (144 + (6 + 2 * 4 + 2 * 3) * 24 + 76) + (144 + 6 * 24 + 76)
    it3 = np.array([3])  # passes 1, 2, 3: two odd, one even
    assert bench.algorithmic_bytes_pcg(w, it3, resident="S", pass_rows=(6, 4, 3)) == \
        144 + (6 + 2 * 4 + 3) * 24 + 76


def test_bdmv_bytes():
    # ss=2, kp=3, float32: strip 6*6*4 = 144 B, padded input (kp+2)*ss*4 = 40 B,
    # output 6*4 = 24 B, per problem.
    w = replace(workloads.WORKLOADS[1], ss=2, kp=3, dtype=np.float32)
    assert bench.algorithmic_bytes_bdmv(w, 5) == 5 * (144 + 40 + 24)


def test_bdsv_flops_hand_counted():
    # ss=1, kp=2: each block-row factors a 1x1 pivot (2/3) and solves for two
    # columns (2*1*2 = 4); the second block-row's update costs 2*1*2 = 4 and
    # the back substitution 2*1 = 2.
    w = replace(workloads.WORKLOADS[2], ss=1, kp=2)
    assert bench.algorithmic_flops_bdsv(w) == pytest.approx(2 * (2 / 3 + 4) + 4 + 2)
    # ss=14, kp=32 (the direct-solve workload): 441,130.67 per problem
    w = replace(workloads.WORKLOADS[2], ss=14, kp=32)
    assert bench.algorithmic_flops_bdsv(w) == pytest.approx(441130.6667, rel=1e-9)


def test_roofline_fields():
    r = bench.roofline(8e9, 1.0, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(8000.0) and r["frac"] == pytest.approx(1.0)
    a = bench.roofline_alu(7.86e10, 1e9, 1.0, 123.0, np.float32)
    assert a["bound"] == "alu" and a["unit"] == "TFLOP/s" and a["peak"] == 78.6
    assert a["frac"] == pytest.approx(1.0) and a["traffic"] == 123.0
    assert a["hbm_achieved_gbs"] == pytest.approx(1000.0)
    assert bench.roofline_alu(1e9, 0, 1.0, None, np.float64)["peak"] == 78.6


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for did, name, val in rows:
            f.write('%d,"%s","%s",%r\n' % (did, name, counter, val))


def test_summarize_pmc_calibrates_and_reads_back(tmp_path):
    neg = "void at::native::neg_kernel_cuda(...)"
    pcg3 = "void glass::pcg_batched_kernel<float, 21, 3, 7>(glass::PcgArgs<float>)"
    # Counter instances of one dispatch are summed (two rows for dispatch 2).
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(1, neg, 524288.0), (2, pcg3, 1000.0), (2, pcg3, 24.0), (3, pcg3, 1024.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(1, neg, 1048576.0), (2, pcg3, 10.0), (3, pcg3, 10.0)])
    out = tmp_path / "traffic.md"
    # Over all workloads the ss=21 kernel serves two of them: no row.
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "cmd f", "cmd w",
                        out=str(out))
    assert "pcg3" not in bench.read_traffic(str(out))
    sel = [k for k in bench.KERNEL_OF if k != "pcg3_unaligned"]
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "cmd f", "cmd w",
                        out=str(out), workloads=sel)
    text = out.read_text()
    # 1 GiB read as 524288 KiB of FETCH_SIZE -> factor 2; writes factor 1.
    assert "x 2.0000" in text and "x 1.0000" in text
    got = bench.read_traffic(str(out))
    assert got == {"pcg3": pytest.approx(1024 * 1024 * 2.0 + 10 * 1024 * 1.0)}
    # A profile taken from other sources is not used.
    out.write_text(text.replace(bench.kernel_source_hash(), "0" * 64))
    assert bench.read_traffic(str(out)) == {}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_compulsory_bytes_and_fraction():
    # ss=2, kp=3, float32, 2 problems: S and Pinv once (288 B), vectors 76 B
    w = replace(workloads.WORKLOADS[0], ss=2, kp=3, dtype=np.float32)
    assert bench.compulsory_bytes_pcg(w, 2) == 2 * (288 + 76)
    assert bench.compulsory_bytes_pcg(w, 2, pinv_diag=True) == 2 * (192 + 76)
    r = bench.roofline(16e9, 1.0, None, compulsory=4e9, served_by="hbm+infinity-cache")
    assert r["frac"] == pytest.approx(2.0) and r["frac_compulsory"] == pytest.approx(0.5)
    assert r["served_by"] == "hbm+infinity-cache"


def test_alu_roofline_uses_the_unpacked_fp32_peak():
    r = bench.roofline_alu(78.6e9, 1e9, 1.0, None, np.float32)
    assert r["peak"] == pytest.approx(78.6) and r["frac"] == pytest.approx(1.0)
    assert r["frac_of_packed_peak"] == pytest.approx(78.6 / 157.3)


def test_code_without_comments():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "// not a comment";\nchar c = \'/\'; /**/x'
    got = bench.code_without_comments(src)
    assert "note" not in got and "block" not in got
    assert '"// not a comment"' in got and "'/'" in got
    assert got.replace(" ", "").replace("\n", "") == 'inta=1;constchar*s="//notacomment";charc=\'/\';x'
    # comments alone do not change the code text; code does
    assert bench.code_without_comments("x = 1; // a\n") == bench.code_without_comments("x = 1; // b\n")
    # a comment that takes more lines does not change it either
    assert (bench.code_without_comments("x = 1;\n// a\ny = 2;\n") ==
            bench.code_without_comments("x = 1;\n// a\n// b\n\ny = 2;   \n"))
    assert bench.code_without_comments("x = 1;\n") != bench.code_without_comments("x = 2;\n")
