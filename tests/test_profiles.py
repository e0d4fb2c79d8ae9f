"""The rocprofv3 summaries behind profiles/: only dispatches after the canvas
set-up are counted (the prefill launches the same kernels on 2,048 causal
rows first), GRBM_GUI_ACTIVE is taken per XCD, and byte counters are scaled
by the copy probe. Synthetic CSVs in rocprofv3's column layout; no GPU."""
import csv

import pytest

from block_discrete_diffusion_dg_amd import profiles as P

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Dispatch_Id", "Kernel_Name", "Correlation_Id",
              "Start_Timestamp", "End_Timestamp"]
PMC_COLS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
            "Start_Timestamp", "End_Timestamp"]


def _write(path, cols, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _trace_row(did, name, dur_ns, t0=0):
    return {"Kind": "KERNEL_DISPATCH", "Agent_Id": 1, "Queue_Id": 1, "Dispatch_Id": did, "Kernel_Name": name,
            "Correlation_Id": did, "Start_Timestamp": t0 + 1000 * did, "End_Timestamp": t0 + 1000 * did + dur_ns}


def test_stats_count_only_the_steps(tmp_path):
    rows = [_trace_row(1, "void moe_experts_kernel<8, false>(MoeArgs)", 900_000),    # prefill
            _trace_row(2, "attn_kernel<128>(...)", 400_000),                          # prefill
            _trace_row(3, "init_canvas_kernel(int*)", 2_000),
            _trace_row(4, "void moe_experts_kernel<8, false>(MoeArgs)", 130_000),
            _trace_row(5, "attn_kernel<128>(...)", 20_000),
            _trace_row(6, "void moe_experts_kernel<8, false>(MoeArgs)", 132_000),
            _trace_row(7, "at::native::vectorized_elementwise_kernel(...)", 5_000)]
    src, out = tmp_path / "t.csv", tmp_path / "s.md"
    _write(src, TRACE_COLS, rows)
    res = P.summarize_stats(str(src), str(out), "cmd")
    assert res["moe_experts_kernel<8, false>"] == {"calls": 2, "avg_us": 131.0}
    assert res["attn_kernel<128>"]["calls"] == 1 and res["attn_kernel<128>"]["avg_us"] == 20.0
    assert not any("native" in k for k in res)
    text = out.read_text()
    assert "after the first `init_canvas_kernel`" in text and "| 2 | 131.00 |" in text


def test_stats_without_marker_keep_everything(tmp_path):
    src, out = tmp_path / "t.csv", tmp_path / "s.md"
    _write(src, TRACE_COLS, [_trace_row(1, "router_kernel(...)", 20_000), _trace_row(2, "router_kernel(...)", 30_000)])
    res = P.summarize_stats(str(src), str(out), "cmd")
    assert res["router_kernel"] == {"calls": 2, "avg_us": 25.0}
    assert "every dispatch" in out.read_text()


def _pmc(did, name, counter, value):
    return {"Correlation_Id": did, "Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
            "Counter_Value": value, "Start_Timestamp": 0, "End_Timestamp": 0}


def test_traffic_scales_by_the_copy_probe_after_the_marker(tmp_path, monkeypatch):
    monkeypatch.setattr(P, "source_hash", lambda k: "h")
    moe = "moe_experts_kernel<8, false>(MoeArgs)"
    fetch = [_pmc(1, moe, "FETCH_SIZE", 9e9), _pmc(2, "init_canvas_kernel", "FETCH_SIZE", 1),
             _pmc(3, moe, "FETCH_SIZE", 300_000.0), _pmc(4, moe, "FETCH_SIZE", 310_000.0),
             _pmc(5, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524_288.0)]
    write = [_pmc(1, moe, "WRITE_SIZE", 9e9), _pmc(2, "init_canvas_kernel", "WRITE_SIZE", 1),
             _pmc(3, moe, "WRITE_SIZE", 10_000.0), _pmc(4, moe, "WRITE_SIZE", 10_000.0),
             _pmc(5, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1_048_576.0)]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(fp, PMC_COLS, fetch)
    _write(wp, PMC_COLS, write)
    rec = P.summarize_traffic(str(fp), str(wp), str(tmp_path / "moe"), "moe_experts", "moe_experts_kernel",
                              1 << 30, "cf", "cw")
    assert rec["dispatches"] == {"fetch": 2, "write": 2}
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(305_000 * 1024 * 2 + 10_000 * 1024)
    assert rec["after_marker"] == "init_canvas_kernel"


def test_mfma_active_time_is_per_xcd(tmp_path):
    rows = []
    for did, name, util, mops, active in [(1, "attn_kernel<128>", 50.0, 1e9, 8e9),       # prefill, dropped
                                          (2, "init_canvas_kernel", 0.0, 0.0, 1.0),
                                          (3, "attn_kernel<128>", 4.0, 5e9, 8 * 48_000.0),
                                          (4, "attn_kernel<128>", 6.0, 5e9, 8 * 48_000.0)]:
        rows += [_pmc(did, name, "MfmaUtil", util), _pmc(did, name, "MfmaFlopsBF16", mops),
                 _pmc(did, name, "GRBM_GUI_ACTIVE", active)]
    src = tmp_path / "m.csv"
    _write(src, PMC_COLS, rows)
    out = P.summarize_mfma(str(src), str(tmp_path / "m.md"), "cmd")
    a = out["attention (attn_kernel)"]
    assert a["dispatches"] == 2 and a["mfma_util_pct"] == pytest.approx(5.0)
    assert a["active_us"] == pytest.approx(20.0)  # 48,000 cycles per XCD at 2.4 GHz
    assert a["tflops"] == pytest.approx(5e9 / 20e-6 / 1e12)


def test_counter_means_and_wave_state_ratios(tmp_path):
    rows = []
    for did, name, wave, wait, lds, conf in [(1, "attn_kernel<128>", 1.0, 1.0, 1.0, 1.0),   # prefill, dropped
                                             (2, "init_canvas_kernel", 5.0, 5.0, 5.0, 5.0),
                                             (3, "attn_kernel<128>", 1000.0, 400.0, 100.0, 10.0),
                                             (4, "attn_kernel<128>", 3000.0, 1600.0, 300.0, 50.0),
                                             (5, "router_kernel<8>", 9e9, 9e9, 9e9, 9e9)]:  # other kernel
        rows += [_pmc(did, name, "SQ_WAVE_CYCLES", wave), _pmc(did, name, "SQ_WAIT_ANY", wait),
                 _pmc(did, name, "SQ_ACTIVE_INST_LDS", lds), _pmc(did, name, "SQ_LDS_BANK_CONFLICT", conf)]
    src = tmp_path / "c.csv"
    _write(src, PMC_COLS, rows)
    out = P.summarize_counters(str(src), str(tmp_path / "c.md"), "attn_kernel", "cmd")
    assert out["means"]["SQ_WAVE_CYCLES"] == pytest.approx(2000.0)
    assert out["ratios"]["waiting (any)"] == pytest.approx(1000.0 / 2000.0)
    assert out["ratios"]["issuing LDS instructions"] == pytest.approx(200.0 / 2000.0)
    assert out["ratios"]["LDS bank-conflict cycles per LDS issue cycle"] == pytest.approx(30.0 / 200.0)
    assert "waiting for an instruction to issue" not in out["ratios"]  # its counter was not collected
    assert "| SQ_WAIT_ANY | 2 |" in (tmp_path / "c.md").read_text()
