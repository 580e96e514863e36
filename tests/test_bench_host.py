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


def _tree(tmp_path, sources):
    csrc = tmp_path / "diffusion_transformer_text_qwen_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    for name in ("gemm_w8a8_1024px_traffic.json", "hbm_kernels_1024px_traffic.json"):
        (tmp_path / "profiles" / name).write_text(open(os.path.join(bench.ROOT, "profiles", name)).read())
    for name, text in sources.items():
        (csrc / name).write_bytes(text)
    return str(tmp_path)


def test_counter_traffic_tracks_the_sources(tmp_path, monkeypatch):
    """Counter bytes are reported only for the source they were taken with: a
    tree whose sources hash as recorded reports them, any other reports none."""
    gt = json.load(open(os.path.join(bench.ROOT, "profiles", "gemm_w8a8_1024px_traffic.json")))
    ht = json.load(open(os.path.join(bench.ROOT, "profiles", "hbm_kernels_1024px_traffic.json")))
    # the HBM-bound kernels' counters lie within a few percent of their algorithmic bytes
    alg = bench.hbm_bytes(4352, 4096, 16384)
    site = {"adaln": "adaln1", "quant_o": "quant_o", "quant_g": "quant_g"}
    for k, v in ht["kernels"].items():
        assert 1.0 <= (v["bytes_read"] + v["bytes_written"]) / alg[site[k]] < 1.05
    # a source that does not hash as recorded: no traffic
    monkeypatch.setattr(bench, "ROOT", _tree(tmp_path / "a", {"gemm.hip": b"// changed\n",
                                                              "elementwise.hip": b"// changed\n"}))
    assert bench.gemm_traffic() is None
    assert bench.hbm_kernel_traffic() == {}
    # sources that hash as recorded (stand-ins with the recorded digests patched in)
    real_sha = bench.hashlib.sha256
    digests = {b"G": gt["gemm_source_sha256"], b"E": ht["elementwise_source_sha256"]}

    class _Fake:
        def __init__(self, data):
            self.d = digests.get(data)
            self.r = real_sha(data)

        def hexdigest(self):
            return self.d or self.r.hexdigest()
    monkeypatch.setattr(bench.hashlib, "sha256", _Fake)
    monkeypatch.setattr(bench, "ROOT", _tree(tmp_path / "b", {"gemm.hip": b"G", "elementwise.hip": b"E"}))
    want = gt["fetch_kib_per_launch"] * 1024 / gt["copy_fetch_per_byte"] + \
        gt["write_kib_per_launch"] * 1024 / gt["copy_write_per_byte"]
    assert bench.gemm_traffic() == int(want)
    hk = bench.hbm_kernel_traffic()
    assert set(hk) == {"adaln1", "adaln2", "quant_o", "quant_g"}
    assert hk["quant_g"] == ht["kernels"]["quant_g"]["bytes_read"] + ht["kernels"]["quant_g"]["bytes_written"]
