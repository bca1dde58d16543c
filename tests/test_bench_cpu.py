"""Host logic of bench.py: the algorithmic byte and flop counts of the
roofline, and which counter record may be attached to a bench line."""
import json

import pytest

import bench


def test_prefill_bytes_per_token_head():
    # q, k (bf16, d_k), v (bf16, d_v), g (fp32, d_k), beta (fp32), o (bf16,
    # d_v): 768 + 512 + 4 + 256 = 1540 B per token-head at d = 128
    assert bench.prefill_bytes(1, 1, 128, 128, 0, False) == 1540
    # S_T written per (sequence, head); S0 read as well when given
    st = 128 * 128 * 4
    assert bench.prefill_bytes(0, 2, 128, 128, 3, False) == 6 * st
    assert bench.prefill_bytes(0, 2, 128, 128, 3, True) == 12 * st
    # the bench workload: 4 x 4096 tokens, H = 32, S0 = 0
    assert bench.prefill_bytes(16384, 32, 128, 128, 4, False) == 815792128


def test_prefill_flops_per_token_head():
    assert bench.prefill_flops(1, 1, 128, 128) == 6 * 128 * 128 + 16 * (3 * 128 + 2 * 128)
    assert bench.prefill_flops(1, 1, 128, 128) == 108544


def test_decode_bytes():
    state, total = bench.decode_bytes(256, 64, 128, 128)
    assert state == 256 * 64 * 128 * 128 * 4 * 2
    assert total - state == 256 * 64 * 1540


def test_gated_and_spec_bytes():
    # q, k, z (bf16, d_k), v, o (bf16, d_v), b (bf16): 1282 B per token-head
    assert bench.gated_prefill_bytes(1, 1, 128, 128, 0) == 1282 + 4
    state, total = bench.spec_bytes(2, 3, 128, 128, 4, 4)
    assert state == 2 * 3 * 128 * 128 * 8
    assert total - state == 2 * 4 * 3 * (2 * 128 + 2 * 128 + 4 * 128 + 4) + \
        2 * 4 * 3 * 1540 + 4 * 2


@pytest.fixture
def record(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    import profile_summary

    def write(file_workload="prefill", prefill_hash=None, **kw):
        h = profile_summary.source_hash
        rec = {"workload": file_workload,
               "kernels": {"prefill": {"source_sha256_16": prefill_hash or h("prefill"),
                                       "hbm_bytes_per_dispatch": 123.0, "mfma_busy_pct": 30.0,
                                       "valu_busy_pct": 40.0},
                           "decode": {"source_sha256_16": h("decode"),
                                      "hbm_bytes_per_dispatch": 7.0}}}
        rec.update(kw)
        (tmp_path / f"pmc_{file_workload}.json").write_text(json.dumps(rec))
    return write


def test_counters_only_for_matching_source_workload_and_kernel(record):
    record()
    r = bench.attach_counters({}, "prefill", "prefill")
    assert r["traffic"] == 123.0 and r["counters"]["mfma_busy_pct"] == 30.0
    assert bench.attach_counters({}, "prefill", "decode") == {"traffic": 7.0}
    assert bench.attach_counters({}, "prefill", "spec") == {"traffic": None}
    # counters taken on the prefill workload say nothing about other workloads
    assert bench.attach_counters({}, "long_prefill", "prefill") == {"traffic": None}
    # a kernel's figures taken on other sources of that kernel are stale;
    # the other kernels' figures in the same record still count
    record(prefill_hash="0" * 16)
    assert bench.attach_counters({}, "prefill", "prefill") == {"traffic": None}
    assert bench.attach_counters({}, "prefill", "decode") == {"traffic": 7.0}
    # a record filed under another workload's name is not trusted
    record(workload="varlen")
    assert bench.counter_record("prefill", "prefill") is None


def test_summed_counters_need_every_kernel(record):
    record()
    r = bench.attach_counters_sum({}, "prefill", ("prefill", "decode"))
    assert r == {"traffic": 130.0, "traffic_by_kernel": {"prefill": 123.0, "decode": 7.0}}
    # one kernel without a current record leaves the sum unknown
    assert bench.attach_counters_sum({}, "prefill", ("prefill", "spec")) == {"traffic": None}
    record(prefill_hash="0" * 16)
    assert bench.attach_counters_sum({}, "prefill", ("prefill", "decode")) == {"traffic": None}


def test_counters_missing_record(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.counter_record("prefill", "prefill") is None


def test_kernel_classes():
    import profile_summary as ps
    # every class has a defining source, and its hash depends on that file only
    for cls in ps.KERNEL_SOURCE:
        assert len(ps.source_hash(cls)) == 16
    assert ps.source_hash("prefill") == ps.source_hash("seg_scan")
    assert ps.source_hash("prefill") != ps.source_hash("bwd_sweep")
    assert ps.kernel_class("_ZN3kda18kda_prefill_kernelIDF16bDF16bLi128ELi128ELi4ELi3ELb0ELb0EEEvNS_6"
                           "ParamsIT_T0_EE") == "prefill"
    assert ps.kernel_class("_ZN3kda18kda_prefill_kernelIDF16bDF16bLi128ELi128ELi4ELi3ELb1ELb0EEEvNS_6"
                           "ParamsIT_T0_EE") == "prefill_gated"
    assert ps.kernel_class("_ZN3kda18kda_prefill_kernelIDF16bDF16bLi128ELi128ELi4ELi3ELb0ELb1EEEvNS_6"
                           "ParamsIT_T0_EE") == "prefill_ckpt"
    assert ps.kernel_class("void kda::kda_seg_scan_kernel<128, 128>(float const*)") == "seg_scan"
    assert ps.kernel_class("__amd_rocclr_copyBuffer") == "copy"
    assert ps.kernel_class("void kda::kda_bwd_sweep<__hip_bfloat16, 128, 128, 64>(kda::SweepArgs)") == "bwd_sweep"
    assert ps.kernel_class("void kda::kda_bwd_sweep_mfma<128, 128, 4>(kda::bwdm::SweepParams)") == "bwd_sweep_mfma"
    assert ps.kernel_class("void kda::kda_bwd_chunk<128, 128>(kda::bwdm::ChunkParams)") == "bwd_chunk"
    assert ps.kernel_class("void kda::kda_bwd_finish<__hip_bfloat16, 128, 128>(kda::FinishArgs)") == "bwd_finish"
