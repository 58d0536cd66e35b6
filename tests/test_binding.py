"""The Python binding's argument checks, on the CPU: every tensor the kernels
read or write must have the shape, dtype, layout and device that include/kda.h
describes, or the call raises ValueError before reaching the C ABI (a wrong
shape or dtype there would let a kernel write past a buffer)."""
import pytest

torch = pytest.importorskip("torch")

import gated_delta_rule_63_amd as kda  # noqa: E402


def inputs(B=1, T=40, H=2, dtype=torch.bfloat16):
    q = torch.zeros((B, T, H, 128), dtype=dtype)
    return dict(q=q, k=q.clone(), v=q.clone(), g=torch.zeros((B, T, H, 128)), beta=torch.zeros((B, T, H)))


def check(t, cu=None, scalar_gate=False):
    kda._check_inputs(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, scalar_gate=scalar_gate, _device=False)


def test_good_inputs_pass():
    check(inputs())
    check(inputs(dtype=torch.float32))
    t = inputs()
    t["g"] = torch.zeros((1, 40, 2))
    check(t, scalar_gate=True)
    check(inputs(), cu=torch.tensor([0, 10, 40], dtype=torch.int32))


def test_cpu_tensors_rejected_for_the_device_path():
    t = inputs()
    with pytest.raises(ValueError, match="device"):
        kda._check_inputs(t["q"], t["k"], t["v"], t["g"], t["beta"], None)


@pytest.mark.parametrize("name,bad", [
    ("k", lambda t: t["k"].float()),                                   # dtype differs from q
    ("v", lambda t: t["v"][:, :20]),                                    # shape
    ("g", lambda t: t["g"].to(torch.bfloat16)),                         # g must be fp32
    ("g", lambda t: t["g"][..., :64]),
    ("beta", lambda t: t["beta"].double()),
    ("beta", lambda t: t["beta"][..., None]),
    ("q", lambda t: t["q"].transpose(1, 2).contiguous().transpose(1, 2)),   # not contiguous
    ("q", lambda t: t["q"][..., :64]),                                  # head size 64
])
def test_bad_inputs_rejected(name, bad):
    t = inputs()
    t[name] = bad(t)
    with pytest.raises(ValueError):
        check(t)


def test_bad_cu_seqlens_rejected():
    for cu in (torch.tensor([0, 40], dtype=torch.int64), torch.tensor([[0, 40]], dtype=torch.int32),
               torch.zeros(0, dtype=torch.int32)):
        with pytest.raises(ValueError, match="cu_seqlens"):
            check(inputs(), cu=cu)
    with pytest.raises(ValueError, match="batch"):
        check(inputs(B=2), cu=torch.tensor([0, 40], dtype=torch.int32))


@pytest.mark.parametrize("fn,name", [(kda._check_state, "initial_state"), (kda._check_out, "final_state")])
def test_state_tensors(fn, name):
    shape = (3, 2, 128, 128)
    good = torch.zeros(shape)
    fn(name, good, shape, good.device)
    for bad in (torch.zeros((3, 2, 128, 64)), torch.zeros(shape, dtype=torch.bfloat16),
                torch.zeros((3, 2, 128, 128 * 2))[..., ::2], torch.zeros((2, 2, 128, 128))):
        with pytest.raises(ValueError, match=name):
            fn(name, bad, shape, good.device)
    with pytest.raises(ValueError):
        fn(name, good, shape, torch.device("meta"))                    # another device
    kda._check_state(name, None, shape, good.device)                    # no initial state: allowed


def test_out_tensor():
    shape = (1, 40, 2, 128)
    kda._check_out("out", torch.zeros(shape), shape, torch.device("cpu"))
    for bad in (torch.zeros((1, 39, 2, 128)), torch.zeros(shape, dtype=torch.bfloat16),
                torch.zeros((1, 40, 2, 256))[..., ::2]):
        with pytest.raises(ValueError, match="out"):
            kda._check_out("out", bad, shape, torch.device("cpu"))
