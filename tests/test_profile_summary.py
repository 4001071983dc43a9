"""The counter summary's traffic is used only while the kernel sources are
unchanged (digest match)."""
import json

from sparse_moe_ffn_02_amd import profile_summary as ps


def test_traffic_digest_gate(tmp_path):
    good = tmp_path / "good.md"
    stale = tmp_path / "stale.md"
    data = {"kernels": {"gateup_split": {"read_bytes": 10, "write_bytes": 2}}}
    good.write_text("# x\n\ntraffic-json: " + json.dumps({"digest": ps.source_digest(), **data}) + "\n")
    stale.write_text("traffic-json: " + json.dumps({"digest": "0" * 16, **data}) + "\n")
    assert ps.load_traffic(str(good))["kernels"]["gateup_split"]["read_bytes"] == 10
    assert ps.load_traffic(str(stale)) is None
    assert ps.load_traffic(str(tmp_path / "absent.md")) is None


def test_short_names():
    assert ps.short_name("moe::k_gateup_split(moe::FfnArgs)") == "gateup_split"
    assert ps.short_name("moe::k_front(moe::RouteArgs, moe::FfnArgs, int)") == "front"
    assert ps.short_name("void moe::k_router_logits<4>(moe::RouteArgs)") == "router_logits"
    assert ps.is_library_kernel("void moe::k_quant_rows<unsigned short>(unsigned short const*)")
    assert not ps.is_library_kernel("__amd_rocclr_copyBuffer")


def test_mfma_summary_fraction(tmp_path):
    """busy fraction = MFMA busy cycles / (GUI active cycles x 1024 SIMDs)."""
    d = tmp_path / "run"
    d.mkdir()
    rows = ["Kernel_Name,Counter_Name,Counter_Value"]
    for v in (1000, 3000):
        rows.append(f"moe::k_gateup_tiled(moe::FfnArgs),GRBM_GUI_ACTIVE,{v}")
    for v in (1024 * 250, 1024 * 750):
        rows.append(f"moe::k_gateup_tiled(moe::FfnArgs),SQ_VALU_MFMA_BUSY_CYCLES,{v}")
    rows.append("__amd_rocclr_copyBuffer,GRBM_GUI_ACTIVE,5")
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    out = tmp_path / "mfma.md"
    ps.mfma_summary(str(d), str(out), "cmd")
    data = ps.load_mfma(str(out))
    k = data["kernels"]["gateup_tiled"]
    assert abs(k["busy_frac"] - 0.25) < 1e-9
    assert "copyBuffer" not in out.read_text()
    stale = tmp_path / "stale.md"
    stale.write_text(out.read_text().replace(ps.source_digest(), "0" * 16))
    assert ps.load_mfma(str(stale)) is None


def test_mfma_summary_prefers_derived_metric(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    rows = ["Kernel_Name,Counter_Name,Counter_Value",
            "moe::k_down_tiled(moe::FfnArgs),MfmaUtil,40.0",
            "moe::k_down_tiled(moe::FfnArgs),SQ_INSTS_VALU_MFMA_MOPS_F8,1000"]
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    out = tmp_path / "m.md"
    ps.mfma_summary(str(d), str(out), "cmd")
    k = ps.load_mfma(str(out))["kernels"]["down_tiled"]
    assert abs(k["busy_frac"] - 0.4) < 1e-12 and k["SQ_INSTS_VALU_MFMA_MOPS_F8"] == 1000
