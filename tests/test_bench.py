"""Host logic of bench.py (no GPU): the single-GPU guard, the kernel-symbol
table, and the counter summary that turns rocprofv3 byte counters into the
HBM traffic bench.py reports (scaled by a plain 1 GiB copy)."""
import csv
import os
import subprocess
import sys


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_kernel_symbols_belong_to_their_source_group():
    for name, (_, group) in bench.KERNEL_SYMBOLS.items():
        assert group in bench.SOURCE_GROUPS, name
        forms = bench.kernel_forms(name)
        assert forms and all(isinstance(f, tuple) and f for f in forms), name
        for form in forms:
            for sym in form:
                assert bench.symbol_group(sym) == group, (name, sym)


def test_short_kernel_names():
    mangled = "_ZN12_GLOBAL__N_116attn_dkdv_kernelIDF16bLi64EfLi8ELi64EEEvPKT_"
    assert bench.short_kernel_name(mangled) == "attn_dkdv_kernel"
    assert bench.short_kernel_name("void pool_kernel<float, false>(float const*)") == "pool_kernel"


def _write(path, rows, fields):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_summary_scales_by_the_copy(tmp_path, capsys):
    """Two counter passes and a kernel trace, synthetic: the copy reads 1 GiB
    but FETCH_SIZE reports half of it (as measured on this GPU), writes are
    reported in full.  A kernel with FETCH 1000 KiB and
    WRITE 500 KiB per dispatch then moved (1000 x 2 + 500) KiB, and its rate
    is taken over the trace's average duration."""
    copy = "__amd_rocclr_copyBuffer"
    mangled = "_ZN12_GLOBAL__N_111pool_kernelIDF16bLb0EEEvPKT_"
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(str(tmp_path / "fetch" / "f_counter_collection.csv"),
           [{"Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 524288},
            {"Kernel_Name": mangled, "Counter_Name": "FETCH_SIZE", "Counter_Value": 900},
            {"Kernel_Name": mangled, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1100}], fields)
    _write(str(tmp_path / "write" / "w_counter_collection.csv"),
           [{"Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1048576},
            {"Kernel_Name": mangled, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500},
            {"Kernel_Name": mangled, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500}], fields)
    _write(str(tmp_path / "trace" / "t_kernel_stats.csv"),
           [{"Name": mangled, "Calls": 2, "TotalDurationNs": 2000, "AverageNs": 1000, "MinNs": 900, "MaxNs": 1100}],
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
    bench.pmc_summary([str(tmp_path / "trace"), str(tmp_path / "fetch"), str(tmp_path / "write")])
    out = capsys.readouterr().out
    expected = (1000 * 2 + 500) * 1024
    assert f"- hbm_bytes_per_launch.pool_kernel: `{expected}`" in out
    # 2.56 MB over 1 us: 2560 GB/s, 32.0% of the 8 TB/s peak
    assert "| pool_kernel | 2.6 | 1.0 | 2560 | 32.0% |" in out
    assert "- sources_sha256.select: `" in out


def test_cpu_baseline_parity_verdict():
    """The parity verdict of the oracle leg: outputs equal to the oracle's (as
    stored in the dtype) pass; a changed slot or a perturbed gradient fails."""
    import numpy as np
    import torch
    from long_context_pretraining_amd import inputs
    from oracle import lighthouse_oracle as orc

    w = inputs.Workload("bench_parity", 1, 2, 1024, 64, "bf16", 4, 3, 16, 21, True)
    q, k, v = inputs.make_qkv(w)
    dout = inputs.make_dout(w)
    gidx, outs = [], {n: [] for n in ("o", "dq", "dk", "dv")}
    for h in range(w.H):
        f = lambda t: t[0, h].float().numpy().astype(np.float64)
        st = orc.head_forward(f(q), f(k), f(v), w.p, w.L, w.k, w.dtype)
        bw = orc.head_backward(st, f(dout))
        gidx.append(torch.from_numpy(np.asarray(st["gidx"], np.int32)))
        for n, x in (("o", st["O"]), ("dq", bw["dq"]), ("dk", bw["dk"]), ("dv", bw["dv"])):
            outs[n].append(torch.from_numpy(x).to(torch.bfloat16))
    gpu = {"gidx": torch.stack(gidx)[None]}
    gpu.update({n: torch.stack(x)[None] for n, x in outs.items()})
    r = bench.cpu_baseline(w, q, k, v, dout, nheads=2, gpu=gpu)["parity"]
    assert r["pass"] and r["selection_bit_exact"] and r["heads"] == 2
    assert max(r["err_over_bound"].values()) <= 0.5   # one bf16 rounding of the oracle's values
    gpu["gidx"] = gpu["gidx"].clone()
    gpu["gidx"][0, 1, 0] += 1
    gpu["dk"] = gpu["dk"].clone()
    gpu["dk"][0, 0, 5, 3] += 1.0
    r = bench.cpu_baseline(w, q, k, v, dout, nheads=2, gpu=gpu)["parity"]
    assert not r["pass"] and not r["selection_bit_exact"] and r["err_over_bound"]["dk"] > 1.0
