"""Host logic of the counter parsers behind the reported HBM traffic and
utilisation figures, on synthetic rocprofv3 counter-collection files."""
import csv

import pytest

from bit_mla_kv_decode_amd import measure as M

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


COPY = "(anonymous namespace)::k_copy(unsigned char const*, unsigned char*, long)"
DECODE = "void mla::k_decode_flat<0, 1>(mla::DecodeArgs)"
OTHER = "void at::native::elementwise_kernel<128, 4>(int, float)"  # a torch kernel in the same trace


def test_kernel_name_matching():
    assert M._is_kernel(COPY, "k_copy")
    assert M._is_kernel(DECODE, "k_decode_flat")
    assert M._is_kernel("_ZN3mla13k_decode_flatILi0ELi1EEEvNS_10DecodeArgsE", "k_decode_flat")
    assert not M._is_kernel(DECODE, "k_decode")       # a prefix of another kernel's name
    assert not M._is_kernel(OTHER, "k_copy")


def test_traffic_scales_each_counter_by_the_copy(tmp_path):
    # the copy moves 1 GiB each way: FETCH_SIZE reads 2048 bytes per unit, WRITE_SIZE 1024
    fetch = [(COPY, "FETCH_SIZE", 524288.0)] * 3 + [(OTHER, "FETCH_SIZE", 7.0)]
    fetch += [(DECODE, "FETCH_SIZE", v) for v in (1000.0, 1010.0, 990.0)]
    write = [(COPY, "WRITE_SIZE", 1048576.0)] * 3 + [(DECODE, "WRITE_SIZE", v) for v in (400.0, 420.0, 410.0)]
    _write(tmp_path / "f.csv", fetch)
    _write(tmp_path / "w.csv", write)
    r = M.parse_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), packed_bytes=2048 * 1000)
    assert r["fetch_scale_bytes_per_unit"] == 2048.0 and r["write_scale_bytes_per_unit"] == 1024.0
    assert r["decode_read_bytes"] == 1000 * 2048          # median of the three decode dispatches
    assert r["decode_write_bytes"] == 410 * 1024
    assert r["decode_traffic_bytes"] == 1000 * 2048 + 410 * 1024
    assert r["read_over_packed"] == 1.0


def test_traffic_needs_both_kernels(tmp_path):
    _write(tmp_path / "f.csv", [(DECODE, "FETCH_SIZE", 1.0)])
    _write(tmp_path / "w.csv", [(COPY, "WRITE_SIZE", 1.0), (DECODE, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        M.parse_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))


def test_pmc_ratios(tmp_path):
    # one pass: median over the decode dispatches, other kernels ignored
    rows = []
    for scale in (0.9, 1.0, 1.1):
        rows += [(DECODE, "GRBM_GUI_ACTIVE", 8000.0 * scale),
                 (DECODE, "SQ_VALU_MFMA_BUSY_CYCLES", M.SIMDS * 500.0 * scale),
                 (DECODE, "SQ_VALU_MFMA_COEXEC_CYCLES", M.SIMDS * 125.0 * scale),
                 (DECODE, "SQ_INSTS_MFMA", 100.0 * scale),
                 (DECODE, "SQ_INSTS_VALU", 500.0 * scale),
                 (DECODE, "SQ_INSTS_LDS", 125.0 * scale),
                 (DECODE, "TCC_HIT_sum", 30.0 * scale),
                 (DECODE, "TCC_MISS_sum", 70.0 * scale)]
    rows += [(OTHER, "SQ_INSTS_MFMA", 1e9)]
    _write(tmp_path / "a.csv", rows)
    d = M.parse_pmc([str(tmp_path / "a.csv")])
    assert d["counters"]["SQ_INSTS_MFMA"] == 100.0
    assert d["gpu_active_cycles"] == 1000                  # GRBM_GUI_ACTIVE summed over the 8 XCDs
    assert d["mfma_busy_share"] == 0.5                     # busy cycles over SIMDs x active cycles
    assert d["coexec_share_of_mfma_busy"] == 0.25
    assert d["valu_per_mfma"] == 5.0 and d["lds_per_mfma"] == 1.25
    assert d["l2_hit_rate"] == 0.3
