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
