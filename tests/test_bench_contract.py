"""CPU checks of bench.py's contract that need no GPU: more than one GPU is
refused with a message (the path has no collective; every GPU runs its own
tokens), the algorithmic byte counts match their stated formulas, and the CPU
baseline record is complete."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_byte_counts():
    import bench
    # query: 256H q + 4H weights + 8 position + 256 cos/sin + 64H codes + 64J scales + 4H weights_out
    assert bench.q_bytes_per_token(64) == 16384 + 256 + 8 + 256 + 4096 + 256 + 256
    assert bench.k_bytes_per_token() == 256 + 8 + 64 + 4
    assert bench.step_bytes_per_token(64) == 21844
    assert bench.step_bytes_per_token(64) * 131072 == 2863136768
    assert bench.q_bytes_per_token(48) == 256 * 48 + 4 * 48 + 8 + 256 + 64 * 48 + 64 * 4 + 4 * 48
    assert bench.sglang_q_bytes_per_token(64) == 21000
    assert bench.fp8_q_bytes_per_token(64) == 25224


def test_cpu_baseline_record():
    """The oracle baseline record carries the contract's keys plus the host's
    CPU model and counts, timed as a median of 3 runs."""
    import bench
    from pack_token_amd import workloads

    wl = workloads.RECIPES["tiny"]()
    rec = bench.cpu_baseline(wl, wl.T, 2)
    for key in ("value", "unit", "cores", "kind", "sample", "cpu_model", "host_cpu_count",
                "usable_cpus", "single_thread_value", "single_thread_sample"):
        assert key in rec, key
    assert rec["kind"] == "oracle" and rec["cores"] == 2 and rec["value"] > 0
    assert rec["host_cpu_count"] == os.cpu_count()
    assert "median of 3" in rec["sample"]


def test_traffic_hash_ignores_comments_only():
    """A traffic record stays valid across comment and whitespace edits of the
    kernel sources and is dropped when the code changes."""
    import bench

    base = 'int f(int x) {\n  return x + 1;  // one\n}\nconst char* s = "a // b";\n'
    same = '/* header */\nint f(int x)   {\n  return x + 1;\n}\n// note\nconst char* s = "a // b";\n'
    assert bench.code_text(base) == bench.code_text(same)
    assert bench.code_text(base) != bench.code_text(base.replace("x + 1", "x + 2"))
    assert bench.code_text(base) != bench.code_text(base.replace('"a // b"', '"a // c"'))


def test_alu_op_count():
    """Hadamard path, per token at H = 64 with key RMSNorm: 65 rows of 128 x
    (RoPE 3 on 64 elements + FWHT 7 + scale 1 + quantizer scaling 1 per element)
    + 3 per element for the RMSNorm; peak = MI355X's fp32 vector 157.3 TFLOP/s
    with a fused multiply-add counted as two flops: 78.65 T lane operations/s."""
    import bench

    row = 64 * 3 + 128 * (7 + 1 + 1)
    assert bench.alu_ops_per_token(64, True, True) == 65 * row + 384 == 87744
    assert bench.alu_ops_per_token(64, True, False) == 65 * row
    assert abs(bench.VALU_PEAK_GOPS - 78650.0) < 1e-6
