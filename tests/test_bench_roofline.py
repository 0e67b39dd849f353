"""bench.py's roofline objects on the CPU: the algorithmic bytes and flops of
the dominant stage, achieved / peak, and the counter traffic of the committed
profiles, which is not reported once taken on other kernel sources."""
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_decode_step_roofline_counts_selection_and_attention_bytes(bench):
    cfg = bench.CONFIGS["decode"]
    res = {"stages_us_eager": {"decode_step": 40.0}}
    roof = bench.decode_roofline(res, cfg, 19)
    # per (sequence, group): every visible K^C1 row (8191 at 131072 keys), Q,
    # the appended kernel's 32 keys and its row; the 19 selected blocks' K and
    # V, Q and O -- bf16, d = 128, 16 heads per group
    n_c1, qo = 8191, 16 * 128 * 2
    per = n_c1 * 128 * 2 + qo + 32 * 128 * 2 + 128 * 2 + 19 * 64 * 128 * 2 * 2 + 2 * qo
    want = 16 * 2 * per
    assert roof["kernel"] == "decode_step" and roof["bound"] == "hbm"
    assert roof["per_launch_algorithmic"] == pytest.approx(want)
    assert roof["achieved"] == pytest.approx(want / 40e-6 / 1e9)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 8000.0)
    assert "attn_split_select_kernel" in roof["launches"]


def test_prefill_roofline_takes_the_dominant_stage(bench):
    res = {"stages_ms": {"compress_k": 0.02, "block_scores": 0.6, "topk_select": 0.07,
                         "sparse_attn": 1.6},
           "sel_flops_2pass": 5.49e11, "attn_flops": 6.24e11}
    roof = bench.prefill_roofline(res, "prefill32k")
    assert roof["kernel"] == "sparse_attn" and roof["bound"] == "mfma"
    assert roof["achieved"] == pytest.approx(6.24e11 / 1.6e-3 / 1e12)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 2500.0)


def test_traffic_of_other_sources_is_not_reported(bench, tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        tr = json.load(f)
    key = "prefill32k/attn_prefill_seq_kernel<2>"
    assert key in tr
    tr[key]["source_hash"] = "0" * 16          # as if taken on other sources
    fake = tmp_path / "traffic.json"
    fake.write_text(json.dumps(tr))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(fake))
    assert bench.stage_traffic("prefill32k", bench.STAGE_KERNELS["sparse_attn"]) == (None, [])
