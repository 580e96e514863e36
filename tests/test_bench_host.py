"""Host-side logic of bench.py (CPU only): the rocprofv3 counter summary and the
hash gate that drops counter-derived traffic once a kernel source changes."""
import json
import os

import bench


def test_counter_summary_means_per_kernel(tmp_path, capsys):
    d = tmp_path / "pmc" / "host"
    d.mkdir(parents=True)
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    for i, (k, v) in enumerate([("a", 10.0), ("a", 30.0), ("b", 7.0)]):
        rows.append(f"{i},{k},FETCH_SIZE,{v}")
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.counter_summary(str(tmp_path))
    out = [json.loads(l) for l in capsys.readouterr().out.splitlines()]
    assert out[0] == {"kernel": "a", "dispatches": 2, "mean": {"FETCH_SIZE": 20.0}}
    assert out[1] == {"kernel": "b", "dispatches": 1, "mean": {"FETCH_SIZE": 7.0}}


def test_counter_traffic_tracks_the_sources(tmp_path, monkeypatch):
    """The committed counter files match the committed sources; a copy of the
    tree whose source differs reports no traffic."""
    assert bench.gemm_traffic() is not None
    hk = bench.hbm_kernel_traffic()
    assert set(hk) == {"adaln1", "adaln2", "quant_o", "quant_g"}
    # counters within a few percent of the algorithmic bytes of these kernels
    alg = bench.hbm_bytes(4352, 4096, 16384)
    for site, b in hk.items():
        assert 1.0 <= b / alg[site] < 1.05
    csrc = tmp_path / "diffusion_transformer_text_qwen_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    for name in ("gemm_w8a8_1024px_traffic.json", "hbm_kernels_1024px_traffic.json"):
        (tmp_path / "profiles" / name).write_text(open(os.path.join(bench.ROOT, "profiles", name)).read())
    (csrc / "gemm.hip").write_text("// changed\n")
    (csrc / "elementwise.hip").write_text("// changed\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.gemm_traffic() is None
    assert bench.hbm_kernel_traffic() == {}
