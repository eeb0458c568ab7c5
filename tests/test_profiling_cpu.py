"""The rocprofv3 summary helper on a synthetic kernel trace (no GPU): per-step kernel
time from the first step's first kernel on, step count from the cross-entropy kernel,
and the time some kernel is running (the union of the dispatch intervals, which two
overlapping streams keep below the summed kernel time)."""
import re

from gpt_pretraining_step_train_amd import profiling

TRACE = """Kernel_Name,Start_Timestamp,End_Timestamp
"fill_normal_kernel(unsigned long)",0,5000000
"(anonymous namespace)::embed_gather_kernel(int const*)",10000000,11000000
"(anonymous namespace)::gemm_a(GemmArgs)",11000000,15000000
"(anonymous namespace)::gemm_b(GemmArgs)",12000000,16000000
"(anonymous namespace)::ce_stream_kernel<unsigned short>(float const*)",16000000,17000000
"(anonymous namespace)::embed_gather_kernel(int const*)",20000000,21000000
"(anonymous namespace)::gemm_a(GemmArgs)",21000000,23000000
"(anonymous namespace)::ce_kernel<unsigned short, 32>(float const*)",23000000,24000000
"""


def test_step_table_counts_steps_and_busy_time(tmp_path):
    (tmp_path / "x_kernel_trace.csv").write_text(TRACE)
    out = profiling.step_table(str(tmp_path), "cmd")
    assert "over 2 steps" in out                       # two cross-entropy dispatches
    assert "fill_normal_kernel" not in out             # set-up kernel before the first step
    # busy: [10, 17] + [20, 24] ms = 11 ms over 2 steps; summed: (1+4+4+1 + 1+2+1) / 2 = 7
    assert re.search(r"running 5\.5 ms per step", out)
    assert re.search(r"\| \(all kernels\) \| \| \| 7\.0 \| 100% \|", out)
    row = next(l for l in out.splitlines() if "`gemm_a`" in l)
    assert "| 1 | 3000.0 | 3.00 |" in row              # one launch per step, 3 ms on average
