"""Host-side checks of the rocprofv3 summary helpers (no GPU): the warm / after-flush
split of a kernel's dispatches in a --kernel-trace CSV."""
import csv

from normalisation_dilated_conv1d_amd import profiling

FIELDS = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]


def write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, start, dur) in enumerate(rows):
            w.writerow({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": i + 1, "Kernel_Name": name,
                        "Start_Timestamp": start, "End_Timestamp": start + dur})


def test_warm_split_counts_a_flush_before_the_prep_kernel(tmp_path):
    conv = "void dconv1d::conv_f32_kernel<128, 4, true, 0, float>(dconv1d::ConvF32Args)"
    prep = "dconv1d::prep_f32_kernel(float const*, ...)"
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>"
    red = "void at::native::reduce_kernel<512, 1, at::native::ReduceOp<float, ...>>"
    rows = [  # (name, start ns, duration ns), deliberately out of order in the file
        (conv, 3_000, 400_000),      # warm
        (prep, 1_000, 1_000),
        (fill, 500_000, 70_000),     # flush ...
        (prep, 580_000, 1_000),      # ... then the block's own prep kernel ...
        (conv, 590_000, 450_000),    # ... so this conv dispatch is cold
        (prep, 1_100_000, 1_000),
        (conv, 1_102_000, 410_000),  # warm again
        (red, 1_600_000, 140_000),   # a read flush (reduction over the scratch) ...
        (prep, 1_750_000, 1_000),
        (conv, 1_752_000, 430_000),  # ... so this one is cold too
    ]
    path = tmp_path / "t_kernel_trace.csv"
    write_trace(path, rows)
    warm, cold = profiling.warm_split(str(path), "conv_f32_kernel")
    assert warm == [400.0, 410.0]
    assert cold == [450.0, 430.0]
    text = profiling.warm_markdown(str(path), "conv_f32_kernel")
    assert "2 warm, average 405.00 us" in text and "2 after a cache flush, average 440.00" in text
