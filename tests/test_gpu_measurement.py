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


@pytest.mark.parametrize("master", [True, False])
@pytest.mark.parametrize("count", [3 * 4096 + 13, 4096 * 2, 7])
def test_stream_mix_reads_change_nothing_and_writes_read_nothing(bfo, count, master):
    # READS: the update's loads alone -- every buffer keeps its bits.
    # WRITES: the update's stores alone -- the result depends only on the key
    # and the index (two different starting states give the same bits), every
    # element is written, the guards and the grads are untouched.
    guard = 64
    outs = []
    for seed in (1, 2):
        rs = np.random.default_rng(seed)
        host = {name: _bits(rs, count + guard, np.int32) for name in ("M", "m", "v")}
        host["G"] = _bits(rs, count + guard, np.int16)
        host["P"] = _bits(rs, count + guard, np.int16)
        d = {k: torch.from_numpy(a).to(DEV) for k, a in host.items()}
        f32 = {k: d[k].view(torch.float32) for k in ("M", "m", "v")}
        bf = {k: d[k].view(torch.bfloat16) for k in ("G", "P")}
        args = (bf["P"][:count], bf["G"][:count], f32["M"][:count] if master else None, f32["m"][:count],
                f32["v"][:count])
        bfo.stream_mix(*args, key=0x2545F491, mode=bfo.MIX_READS)
        torch.cuda.synchronize()
        for k, a in host.items():
            np.testing.assert_array_equal(d[k].cpu().numpy(), a, err_msg=f"READS changed {k}")
        bfo.stream_mix(*args, key=0x2545F491, mode=bfo.MIX_WRITES)
        torch.cuda.synchronize()
        got = {k: d[k].cpu().numpy() for k in host}
        for k in host:
            np.testing.assert_array_equal(got[k][count:], host[k][count:], err_msg=f"{k} guard")
        np.testing.assert_array_equal(got["G"], host["G"], err_msg="G is read-only")
        written = ("P", "m", "v") + (("M",) if master else ())
        for k in written:
            assert (got[k][:count] != host[k][:count]).mean() > 0.99, k
        if not master:
            np.testing.assert_array_equal(got["M"], host["M"], err_msg="no master: M untouched")
        outs.append({k: got[k][:count] for k in written})
    for k in outs[0]:
        np.testing.assert_array_equal(outs[0][k], outs[1][k], err_msg=f"WRITES depends on the old {k}")
    with pytest.raises(bfo.BfoError):
        bfo.stream_mix(*args, mode=3)
