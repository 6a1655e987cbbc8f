"""GPU checks of the measurement export bfo_stream_mix: it must move exactly
the update's bytes and leave its buffers as documented (bit-XOR with the key,
params = grads ^ key), so the ceiling it measures is a real one."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def bfo():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from bf16_numerics_amd import binding
    torch.cuda.set_device(0)
    return binding


def _bits(rs, count, dtype):
    info = np.iinfo(dtype)
    return rs.integers(info.min, info.max, size=count, dtype=dtype, endpoint=True)


@pytest.mark.parametrize("master", [True, False])
@pytest.mark.parametrize("count,key", [(3 * 4096 + 13, 0x9E3779B9), (4096 * 2, 0), (7, 0x12345678)])
def test_stream_mix_moves_and_xors_every_element(bfo, count, key, master):
    rs = np.random.default_rng(count)
    guard = 64
    host = {name: _bits(rs, count + guard, np.int32) for name in ("M", "m", "v")}
    host["G"] = _bits(rs, count + guard, np.int16)
    host["P"] = _bits(rs, count + guard, np.int16)
    d = {k: torch.from_numpy(a).to(DEV) for k, a in host.items()}
    f32 = {k: d[k].view(torch.float32) for k in ("M", "m", "v")}
    bf = {k: d[k].view(torch.bfloat16) for k in ("G", "P")}
    bfo.stream_mix(bf["P"][:count], bf["G"][:count], f32["M"][:count] if master else None, f32["m"][:count],
                   f32["v"][:count], key)
    torch.cuda.synchronize()
    k32 = np.array(key, dtype=np.uint32).view(np.int32)
    k16 = np.array(key & 0xFFFF, dtype=np.uint16).view(np.int16)
    for name in ("M", "m", "v"):
        out = d[name].cpu().numpy()
        want = host[name][:count] ^ k32 if (master or name != "M") else host[name][:count]
        np.testing.assert_array_equal(out[:count], want, err_msg=name)
        np.testing.assert_array_equal(out[count:], host[name][count:], err_msg=name + " guard")
    out = d["P"].cpu().numpy()
    want = host["G"][:count] ^ k16 if master else host["P"][:count] ^ host["G"][:count] ^ k16
    np.testing.assert_array_equal(out[:count], want, err_msg="P")
    np.testing.assert_array_equal(out[count:], host["P"][count:], err_msg="P guard")
    np.testing.assert_array_equal(d["G"].cpu().numpy(), host["G"], err_msg="G is read-only")
