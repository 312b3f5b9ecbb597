"""Host logic of bench.py (no GPU): the algorithmic work it divides by, the
gating of the recorded HBM traffic on the attention sources, and the
rocprofv3 CSV summaries it writes into profiles/."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402
from oracle import mask as omask  # noqa: E402


@pytest.mark.parametrize("name", ["policy_bf16", "t2v480p_bf16", "t2v480p_long_bf16"])
def test_attention_pairs_equal_the_mask_count(name):
    wl = W.BY_NAME[name]
    n, n_ar = wl.n_tokens, W.region_counts(wl.segments)[0]
    assert bench.attention_pairs(n, n_ar) == omask.count_pairs(n, n, 0, W.AR_CAUSAL_DM_FULL, n_ar=n_ar)


def test_profile_work_text_names_the_launchs_flops():
    assert bench.attention_work_text("t2v480p_bf16") == \
        "7.815 TFLOP per launch (635,963,395 allowed pairs x 24 heads x 512 flop)"
    # the streaming chunk: 1,440 rows x 13,218 keys
    assert bench.attention_work_text("stream_chunk_bf16").startswith("0.234 TFLOP per launch (19,033,920 ")


def test_480p_flops_per_launch():
    wl = W.BY_NAME["t2v480p_bf16"]
    n, n_ar = wl.n_tokens, W.region_counts(wl.segments)[0]
    pairs = bench.attention_pairs(n, n_ar)
    assert pairs == 635_963_395
    assert abs(4.0 * wl.head_dim * wl.n_heads * pairs - 7.815e12) < 1e9


def _recorded_hash(workload):
    path = os.path.join(ROOT, "profiles", "%s_%s_hbm_traffic.txt" % (bench.ATTN_KERNEL, workload))
    for line in open(path):
        if line.startswith("attention_kernel_hash:"):
            return line.split(":", 1)[1].strip()
    return None


def test_traffic_is_read_only_for_the_profiled_kernels(monkeypatch):
    h = _recorded_hash("t2v480p_bf16")
    assert h is not None and len(h) == 16
    monkeypatch.setattr(bench, "attention_kernel_hash", lambda: h)
    rec = bench.traffic_from_profile("t2v480p_bf16")
    assert rec is not None and rec > 0.6e9  # at least Q, K, V read and O written once
    monkeypatch.setattr(bench, "attention_kernel_hash", lambda: "0" * 16)
    assert bench.traffic_from_profile("t2v480p_bf16") is None
    monkeypatch.setattr(bench, "attention_kernel_hash", lambda: None)
    assert bench.traffic_from_profile("t2v480p_bf16") is None
    assert bench.traffic_from_profile("no_such_workload") is None


def test_kernel_hash_tracks_the_attention_machine_code(tmp_path):
    so = open(bench.LIB_PATH, "rb").read()
    spans = bench.attention_kernel_spans(so)
    names = {n for n, _, _ in spans}
    # bf16 kernel at D = 128, 80 and 64, with and without Q rotation, and descriptors
    assert len(spans) == 12 and sum(n.endswith(b".kd") for n in names) == 6
    assert all(size > 0 for _, _, size in spans)
    h0 = bench.attention_kernel_hash()
    assert h0 is not None and len(h0) == 16

    def flipped(off):
        b = bytearray(so)
        b[off] ^= 0x01
        p = tmp_path / ("lib_%d.so" % off)
        p.write_bytes(bytes(b))
        return bench.attention_kernel_hash(str(p))

    # a bit inside the first attention kernel changes the hash
    _, off, size = sorted(spans)[0]
    assert flipped(off + size // 2) != h0
    # a bit of host code (the ELF .text of the library) does not, nor the
    # code-entry offset of a descriptor (where the kernel sits)
    text = next(x for x in bench._elf_sections(so) if x["name"] == ".text")
    assert flipped(text["off"] + text["size"] // 2) == h0
    _, kd_off, _ = next(s for s in sorted(spans) if s[0].endswith(b".kd"))
    assert flipped(kd_off + 17) == h0
    assert flipped(kd_off + 24) != h0
    # an unreadable library gives no hash
    (tmp_path / "junk.so").write_bytes(b"not an elf")
    assert bench.attention_kernel_hash(str(tmp_path / "junk.so")) is None
    assert bench.attention_kernel_hash(str(tmp_path / "missing.so")) is None


def test_rocprof_summaries_parse_csv(tmp_path):
    (tmp_path / "x_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void mot::attn_fwd_mfma<128, 4, true>(mot::AttnParams)",2,200,100.0,75.0,90,110,10\n')
    (tmp_path / "x_counter_collection.csv").write_text(
        '"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n'
        '1,"void mot::attn_fwd_mfma<128, 4, true>(mot::AttnParams)","FETCH_SIZE",10\n'
        '1,"void mot::attn_fwd_mfma<128, 4, true>(mot::AttnParams)","FETCH_SIZE",5\n'
        '2,"void mot::attn_fwd_mfma<128, 4, true>(mot::AttnParams)","FETCH_SIZE",25\n')
    text = bench.rocprof_summary(str(tmp_path))
    assert "attn_fwd_mfma" in text and "100" in text
    mean, n = bench._counter_mean(str(tmp_path), "attn_fwd_mfma", "FETCH_SIZE")
    assert n == 2 and mean == 20.0  # per dispatch: 15 and 25


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_reports_a_bounded_oracle_sample():
    wl = W.BY_NAME["tiny_fp32"]
    cb = bench.cpu_baseline(wl, budget_s=0.5)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["cores"] >= 1
    assert cb["value"] > 0 and cb["single_core_value"] > 0
    n_ar = W.region_counts(wl.segments)[0]
    # every DM row of every head, as the tiny workload fits the budget
    assert "%d DM query rows" % ((wl.n_tokens - n_ar) * wl.n_heads) in cb["sample"]


def test_cpu_baseline_reports_the_fields_of_the_line():
    """The oracle leg of the bench line (host only): a bounded sample of the
    480p attention, with the fields the line carries."""
    b = bench.cpu_baseline(W.BY_NAME["t2v480p_bf16"], budget_s=0.5)
    assert b["kind"] == "oracle" and b["unit"] == "TFLOP/s"
    assert b["value"] > 0 and b["single_core_value"] > 0
    assert isinstance(b["cores"], int) and b["cores"] >= 1
    assert "rows" in b["sample"] and b["projected_full_workload_s"] > 0
