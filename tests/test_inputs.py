"""The seeded input generator: deterministic, in range, and bf16-exact."""
import torch

import fa_inputs


def test_prefill_inputs_deterministic_and_bf16():
    a = fa_inputs.prefill_inputs(2, 4, 2, 16, 16, 64, seed=3, len_range=(4, 16))
    b = fa_inputs.prefill_inputs(2, 4, 2, 16, 16, 64, seed=3, len_range=(4, 16))
    for key in ("q", "k", "v"):
        assert a[key].dtype == torch.bfloat16
        assert torch.equal(a[key], b[key])
    assert torch.equal(a["seqlens_cpu"], b["seqlens_cpu"])
    assert a["q"].shape == (2, 4, 16, 64) and a["k"].shape == (2, 2, 16, 64)
    c = fa_inputs.prefill_inputs(2, 4, 2, 16, 16, 64, seed=4)
    assert not torch.equal(a["q"], c["q"])


def test_lengths_inclusive_range():
    lens = fa_inputs.draw_lengths(5000, 3, 7, seed=1)
    assert lens.dtype == torch.int32
    assert int(lens.min()) == 3 and int(lens.max()) == 7


def test_f32_io_and_oracle_view():
    x = fa_inputs.prefill_inputs(1, 1, 1, 8, 8, 64, seed=1, io="f32")
    assert x["q"].dtype == torch.float32
    q64 = fa_inputs.as_oracle_f64(x["q"])
    # The oracle sees exactly the bf16-rounded (RNE) values.
    assert (torch.from_numpy(q64) == x["q"].to(torch.bfloat16).double()).all()


def test_decode_inputs_shapes():
    x = fa_inputs.decode_inputs(3, 8, 2, 32, 64, seed=5, len_range=(4, 32))
    assert x["q"].shape == (3, 8, 64) and x["k_cache"].shape == (3, 2, 32, 64)
    assert x["ctx_lens"].dtype == torch.int32
    assert int(x["ctx_lens"].min()) >= 4 and int(x["ctx_lens"].max()) <= 32


def test_named_workloads():
    names = list(fa_inputs.WORKLOADS)
    assert len(names) == 5
    w = fa_inputs.WORKLOADS["causal_prefill_B1_H32_L16384_d128"]
    assert (w.B, w.H, w.L, w.d, w.causal) == (1, 32, 16384, 128, True)
