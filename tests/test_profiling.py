"""Host logic of the profile tooling: the code hash that ties a stored
counter reading to the kernel source it was taken with."""
from roofline_driven_optimisation_amd.profiling import code_hash, source_hash


def test_code_hash_ignores_comments_and_blank_lines():
    a = "int f(int x) {\n    return x + 1;\n}\n"
    b = ("// header comment\n/* block\n   comment */\nint f(int x) {  // trailing\n\n"
         "    return x + 1;   \n}\n")
    assert code_hash(a) == code_hash(b)


def test_code_hash_sees_code_changes():
    assert code_hash("int f(int x) { return x + 1; }") != code_hash("int f(int x) { return x + 2; }")
    assert code_hash("a = b / c;") != code_hash("a = b;")


def test_source_hash_known_families():
    for fam in ("bf16_q4", "bf16_pp", "bf16_mfma", "f32_mfma", "f32_dma", "skinny", "naive"):
        h = source_hash(fam)
        assert len(h) == 16 and int(h, 16) >= 0
    assert source_hash("bf16_q4") == source_hash("bf16_pp")  # one source file
    assert source_hash("unknown_kernel") == ""
    assert source_hash("fp8_q4") == source_hash("bf16_q4")
    assert len(source_hash("reduce")) == 16


def _trace_csv(path, dispatches):
    """A minimal kernel-trace CSV: (name, grid, workgroup, start ns, end ns)."""
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp",
                    "End_Timestamp"])
        for d in dispatches:
            w.writerow(d)


def test_dispatch_stats_splits_runs_of_one_kernel(tmp_path):
    """Two workloads that launch the same kernel on the same grid, with a copy
    between them, come out as two rows in time order; --last keeps the tail
    of each long run and drops short runs."""
    from roofline_driven_optimisation_amd.profiling import dispatch_stats
    k = "void gemm_kernel<true>(float*) [clone .kd]"
    rows, t = [], 0
    for us in [9.0] * 2 + [4.0] * 5:  # warm-up then steady state, workload 1
        rows.append((k, 65536, 256, t, t + int(us * 1000))); t += 20000
    rows.append(("__amd_rocclr_copyBuffer", 1024, 512, t, t + 1000)); t += 20000
    for us in [8.0] * 5:             # workload 2, same kernel and grid
        rows.append((k, 65536, 256, t, t + int(us * 1000))); t += 20000
    rows.sort(key=lambda r: -r[3])  # the file's own order does not matter
    path = tmp_path / "t_kernel_trace.csv"
    _trace_csv(path, rows)
    all_runs = dispatch_stats(str(path))
    assert [r["calls"] for r in all_runs] == [7, 1, 5]
    steady = dispatch_stats(str(path), last=5)
    assert [r["calls"] for r in steady] == [5, 5]
    assert [r["avg_us"] for r in steady] == [4.0, 8.0]
    assert steady[0]["kernel"] == steady[1]["kernel"] == "gemm_kernel<true> [256 workgroups x 256]"


def test_counter_runs_label_consecutive_runs(tmp_path):
    """Counter passes: two workloads on the same kernel and grid, with
    another kernel between them, get their own medians, matched to the
    labels in time order; short runs (warm-up copies) are skipped."""
    import csv
    from roofline_driven_optimisation_amd.profiling import counter_runs
    path = tmp_path / "p_counter_collection.csv"
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Start_Timestamp",
                    "End_Timestamp", "Counter_Name", "Counter_Value"])
        t, d = 0, 0
        for kernel, grid, value, n in (("bf16_q4_kernel<false>", 65536, 10.0, 6),
                                       ("fp8_q4_kernel<false, 0>", 65536, 20.0, 6),
                                       ("bf16_q4_kernel<false>", 65536, 30.0, 6),
                                       ("bf16_q4_kernel<false>", 1024, 99.0, 2)):
            for i in range(n):
                d += 1
                for se in range(2):  # per-SE rows are summed
                    w.writerow([d, kernel, grid, 256, t, t + 5000, "SQ_WAVES", value / 2])
                t += 10000
    runs = counter_runs([str(path)], ["a", "b", "c"], last=4)
    assert list(runs) == ["a", "b", "c"]
    assert [runs[k]["SQ_WAVES"] for k in "abc"] == [10.0, 20.0, 30.0]
    assert runs["a"]["us"] == 5.0


def test_lds_probe_rows_groups_by_stride(tmp_path):
    """The LDS probe's dispatches are one group per stride (warm-up first);
    the extra cycles per conflict-free one are conflict / (active - conflict)."""
    import csv
    from roofline_driven_optimisation_amd.profiling import lds_probe_rows
    path = tmp_path / "p_counter_collection.csv"
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
                    "Counter_Name", "Counter_Value"])
        d, t = 0, 0
        for st in (1, 2, 4):
            for i in range(5):  # 2 warm-up + 3 timed
                d += 1
                conflict = 0 if i < 2 else 100 * (st - 1)
                w.writerow([d, "lds_probe_kernel(int, int, unsigned int*)", t, t + 1000 * st,
                            "SQ_LDS_IDX_ACTIVE", 100 * st])
                w.writerow([d, "lds_probe_kernel(int, int, unsigned int*)", t, t + 1000 * st,
                            "SQ_LDS_BANK_CONFLICT", conflict])
                t += 10000
    rows = lds_probe_rows(str(path), [1, 2, 4], skip=2)
    assert [r["stride"] for r in rows] == [1, 2, 4]
    assert [r["extra_per_cycle"] for r in rows] == [0.0, 1.0, 3.0]
    assert [r["us"] for r in rows] == [1.0, 2.0, 4.0]


def test_dispatch_stats_timed_runs_between_markers(tmp_path):
    """bench.py's phase markers (a one-workgroup K = 0 launch before, a
    two-workgroup one after each timed loop): --timed keeps exactly the
    enclosed runs, whole, not the warm-ups or what follows a loop."""
    from roofline_driven_optimisation_amd.profiling import dispatch_stats
    k = "void gemm_kernel<true>(float*) [clone .kd]"
    mark = "void mgemm::(anonymous namespace)::scale_kernel<false>(unsigned long, int, float, float*)"
    close = mark + " "  # the same kernel; the marker after a timed loop has two workgroups
    seq = ([(k, 9.0)] * 30 + [(mark, 1.0)] + [(k, 4.0)] * 20 + [(close, 1.0)] + [(k, 6.0)] * 40
           + [(mark, 1.0)] + [(k, 5.0)] * 10 + [(close, 1.0)])
    rows, t = [], 0
    for name, us in seq:
        grid = {mark: 256, close: 512}.get(name, 65536)
        rows.append((name, grid, 256, t, t + int(us * 1000)))
        t += 20000
    path = tmp_path / "t_kernel_trace.csv"
    _trace_csv(path, rows)
    timed = dispatch_stats(str(path), timed=True)
    # the 40 launches after the first closing marker are the next warm-up:
    # a closing marker before them, not an opening one
    assert [(r["calls"], r["avg_us"]) for r in timed] == [(20, 4.0), (10, 5.0)]
    assert [r["calls"] for r in dispatch_stats(str(path))] == [30, 1, 20, 1, 40, 1, 10, 1]
