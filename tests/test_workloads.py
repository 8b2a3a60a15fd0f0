"""The seeded input generators: deterministic, right shapes and dtypes."""

import torch

import workloads


def test_configs_shapes_and_determinism():
    for name, w in workloads.CONFIGS.items():
        s = w.with_(B=1, H=2, Nq=min(w.Nq, 64), Nk=min(w.Nk, 80))
        a = workloads.make_inputs(s)
        b = workloads.make_inputs(s)
        for key in ("q", "k", "v"):
            assert a[key].shape == (1, 2, s.Nq if key == "q" else s.Nk, s.d)
            assert a[key].dtype == (torch.float32 if w.dtype == "f32" else torch.bfloat16)
            assert torch.equal(a[key], b[key])
        c = workloads.make_inputs(s, seed=100 + w.seed)
        assert not torch.equal(a["q"], c["q"])
        if w.bias_std is not None:
            assert a["bias"].shape == (1, 2, s.Nq, s.Nk) and a["bias"].dtype == torch.float32
        if w.kv_len_range is not None:
            lo, hi = w.kv_len_range
            assert a["kv_len"].dtype == torch.int32
            assert int(a["kv_len"].min()) >= lo and int(a["kv_len"].max()) <= hi
        assert a["scale"] == float(torch.tensor(w.softmax_scale, dtype=torch.float32))


def test_long_context_row_factor_range():
    w = workloads.CONFIGS["c4_bf16_d128_long_causal"].with_(H=1, Nq=512, Nk=512)
    x = workloads.make_inputs(w)
    g = torch.Generator().manual_seed(w.seed)
    z = torch.randn((1, 1, 512, 128), generator=g)
    ratio = x["q"].float() / (0.5 * z).to(torch.bfloat16).float()
    r = ratio[(z.abs() > 0.5)]
    assert float(r.min()) > 0.95 and float(r.max()) < 4.05


def test_flops():
    w = workloads.CONFIGS["c3_bf16_d128"]
    assert w.flops() == 4.0 * 2 * 32 * 4096 * 4096 * 128
    assert workloads.CONFIGS["c3_bf16_d128_causal"].flops() == w.flops() / 2
