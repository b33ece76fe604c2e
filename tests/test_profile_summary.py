"""Host checks of the rocprofv3 summariser's step anatomy (profile_summary
chain) on a hand-made kernel trace whose spans, busy and idle times are
known."""
import csv
import os

from optimizer_muon_step_amd import profile_summary as ps

FIELDS = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]


def _write_trace(d, launches):
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, b, e) in enumerate(launches):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Start_Timestamp": b, "End_Timestamp": e})


def _step(t0, gap):
    """momentum, norm, cast, one NS iteration, apply: 6 kernels of 1000 ns,
    `gap` ns apart; returns the launches and the step's end."""
    names = ["muon::momentum_kernel(x)", "muon::norm_finalize_kernel(x)", "void muon::cast_kernel<false>(x)",
             "void muon::ns_gemm_kernel<0, 256>(x)", "void muon::ns_gemm_kernel<2, 192>(x)", "muon::apply_kernel(x)"]
    out, t = [], t0
    for n in names:
        out.append((n, t, t + 1000))
        t += 1000 + gap
    return out, t - gap


def test_chain_splits_steps_and_groups(tmp_path):
    launches = [("void at::native::fill(x)", 0, 500)]  # not part of any step
    t = 1000
    for k in range(5):  # group a: 1 skipped + 2 steps, gap 100 ns
        st, t = _step(t, 100)
        launches += st
        t += 10_000
    for k in range(3):  # group b: 3 steps, gap 300 ns
        st, t = _step(t, 300)
        launches += st
        t += 20_000
    _write_trace(str(tmp_path), launches)
    out = tmp_path / "chain.md"

    class A:
        dir = str(tmp_path)
        group = ["a:1:2", "b:2:3"]
        command = "cmd"
        title = "t"
        note = ""
    A.out = str(out)
    ps.cmd_chain(A)
    text = out.read_text()
    # group a: span 6*1000 + 5*100 = 6500 ns, busy 6000, idle 500, period 6500 + 10000
    assert "| a | 2 | 6.0 | 6.5 | 6.0 | 0.5 | 0.10 | 16.5 |" in text
    # group b skips the last 2 steps of the 5 of group a's run, then takes the 3 with 300 ns gaps
    assert "| b | 3 | 6.0 | 7.5 | 6.0 | 1.5 | 0.30 | 27.5 |" in text
    assert "| ns_update | 1.0 | 1.00 | 1.0 |" in text


def test_chain_refuses_short_traces(tmp_path):
    st, _ = _step(0, 0)
    _write_trace(str(tmp_path), st)

    class A:
        dir = str(tmp_path)
        group = ["a:0:2"]
        command = "cmd"
        title = "t"
        note = ""
        out = str(tmp_path / "x.md")
    try:
        ps.cmd_chain(A)
    except SystemExit as e:
        assert "only 1 steps" in str(e)
    else:
        raise AssertionError("a group longer than the trace was accepted")
