"""The scheduled step (lr, bias corrections and seed read on the device) and
its replay from a HIP graph.

adamw_sr_step_scheduled must give the by-value step's results bit for bit,
and a graph recorded once from grad_global_norm, the scheduled step and the
cursor advance must reproduce the eager run step after step: every replay
is compared with the eager state of the same step, with the program's own
eager work (the next grads) and a synchronisation between replays.  The
eager run itself is the one the parity tests pin to the oracle; the d=32
model's graph run is also compared with the oracle directly.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as o
from bf16_numerics_amd import workloads as W
from gpu_harness import assert_state_parity, host_copy, oracle_step, step_seed

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
STEPS = 5


@pytest.fixture(scope="module")
def bfo():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from bf16_numerics_amd import binding
    torch.cuda.set_device(0)
    return binding


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def padded_tiny():
    """The d=32 model plus a 13-element 1-D tensor: a ragged end mid-vector."""
    w = W.tiny()
    w.tensors = list(w.tensors) + [("pad", (13,))]
    return w


def lr_of(bfo, t):
    """A schedule that changes every step: 2 warm-up steps, then cosine."""
    return bfo.lr_at(bfo.LR_COSINE, t - 1, 2, STEPS, 1e-3, 0.1)


def with_lr(bfo, hp, lr):
    return bfo.AdamwHParams(lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, 1 if hp.bias_correction else 0)


def bits(st):
    return {k: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).clone()
            for k, t in st.items() if t is not None}


def assert_same_bits(a, b, what):
    for k in a:
        assert torch.equal(a[k], b[k]), f"{what}: {k} differs"


def fresh_state(w, master):
    P, M, m, v = W.init_state(torch, w, 0, w.n, DEV, master=master)
    return {"P": P, "M": M, "m": m, "v": v}


def clone_state(st):
    return {k: (t.clone() if t is not None else None) for k, t in st.items()}


@pytest.mark.parametrize("make", [W.tiny, padded_tiny, W.gpt2_124m])
@pytest.mark.parametrize("master,rounding", [(True, o.ROUND_SR), (False, o.ROUND_SR), (True, o.ROUND_RNE),
                                             (False, o.ROUND_RNE)])
def test_scheduled_step_equals_by_value_step(bfo, make, master, rounding):
    w = make()
    T = bfo.Table(w.entries())
    a = fresh_state(w, master)
    b = clone_state(a)
    G = torch.empty(w.n, dtype=torch.bfloat16, device=DEV)
    res = bfo.new_norm_result(DEV)
    sched = bfo.step_schedule(w.hparams, [(t, lr_of(bfo, t), step_seed(t)) for t in range(1, STEPS + 1)], DEV)
    cursor = torch.zeros(1, dtype=torch.int64, device=DEV)
    for t in range(1, STEPS + 1):
        W.fill_grads(torch, w, G, 0, t)
        bfo.grad_global_norm(T, G, res, w.hparams.max_norm)
        bfo.adamw_sr_step(T, a["P"], G, a["M"], a["m"], a["v"], with_lr(bfo, w.hparams, lr_of(bfo, t)), t,
                          step_seed(t), scale=res, rounding=rounding)
        bfo.adamw_sr_step_scheduled(T, b["P"], G, b["M"], b["m"], b["v"], w.hparams, sched, cursor, scale=res,
                                    rounding=rounding)
        bfo.cursor_advance(cursor)
        assert_same_bits(bits(a), bits(b), f"{w.name} t={t}")
    assert int(cursor.item()) == STEPS


def test_cursor_selects_the_step_and_past_the_end_changes_nothing(bfo):
    w = W.tiny()
    T = bfo.Table(w.entries())
    st = fresh_state(w, True)
    G = torch.empty(w.n, dtype=torch.bfloat16, device=DEV)
    W.fill_grads(torch, w, G, 0, 1)
    sched = bfo.step_schedule(w.hparams, [(1, 1e-3, step_seed(1)), (7, 3e-4, step_seed(7))], DEV)
    before = bits(st)
    cursor = torch.full((1,), 2, dtype=torch.int64, device=DEV)
    bfo.adamw_sr_step_scheduled(T, st["P"], G, st["M"], st["m"], st["v"], w.hparams, sched, cursor)
    torch.cuda.synchronize()
    assert_same_bits(bits(st), before, "cursor past the schedule")
    # cursor 1 is step 7 with lr 3e-4 and step 7's seed
    ref = clone_state(st)
    cursor.fill_(1)
    bfo.adamw_sr_step_scheduled(T, st["P"], G, st["M"], st["m"], st["v"], w.hparams, sched, cursor)
    bfo.adamw_sr_step(T, ref["P"], G, ref["M"], ref["m"], ref["v"], with_lr(bfo, w.hparams, 3e-4), 7,
                      step_seed(7))
    assert_same_bits(bits(st), bits(ref), "cursor 1")


def test_scheduled_step_rejects_overlaps_and_bad_schedules(bfo):
    w = W.tiny()
    T = bfo.Table(w.entries())
    st = fresh_state(w, True)
    G = torch.zeros(w.n, dtype=torch.bfloat16, device=DEV)
    sched = bfo.step_schedule(w.hparams, [(1, 1e-3, 1)], DEV)
    cursor = torch.zeros(1, dtype=torch.int64, device=DEV)
    lib, stream = bfo.library(), ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    hp = bfo.AdamwHParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    # the schedule inside m, the cursor inside v
    assert lib.adamw_sr_step_scheduled(T.handle, ptr(st["P"]), ptr(G), ptr(st["M"]), ptr(st["m"]), ptr(st["v"]),
                                       ctypes.byref(hp), ptr(st["m"]), 1, ptr(cursor), None, None, 0,
                                       stream) == bfo.EINVAL
    assert lib.adamw_sr_step_scheduled(T.handle, ptr(st["P"]), ptr(G), ptr(st["M"]), ptr(st["m"]), ptr(st["v"]),
                                       ctypes.byref(hp), ptr(sched), 1, ptr(st["v"]), None, None, 0,
                                       stream) == bfo.EINVAL
    with pytest.raises(ValueError):
        bfo.adamw_sr_step_scheduled(T, st["P"], G, st["M"], st["m"], st["v"], w.hparams, sched[:31], cursor)


@pytest.mark.parametrize("make", [W.tiny, padded_tiny, W.gpt2_124m])
@pytest.mark.parametrize("master", [True, False])
def test_graph_replay_matches_the_eager_step(bfo, make, master):
    w = make()
    T = bfo.Table(w.entries())
    eager = fresh_state(w, master)
    graph = clone_state(eager)
    G = torch.empty(w.n, dtype=torch.bfloat16, device=DEV)      # the graph's grads buffer, refilled per step
    res_e, res_g = bfo.new_norm_result(DEV), bfo.new_norm_result(DEV)
    sched = bfo.step_schedule(w.hparams, [(t, lr_of(bfo, t), step_seed(t)) for t in range(1, STEPS + 1)], DEV)
    cursor = torch.zeros(1, dtype=torch.int64, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bfo.grad_global_norm(T, G, res_g, w.hparams.max_norm)
        bfo.adamw_sr_step_scheduled(T, graph["P"], G, graph["M"], graph["m"], graph["v"], w.hparams, sched,
                                    cursor, scale=res_g)
        bfo.cursor_advance(cursor)
    torch.cuda.synchronize()
    assert int(cursor.item()) == 0, "capture must not run the step"
    tbl = o.table(w.entries())
    h = host_copy({**eager, "G": G}) if w.n < 100_000 else None
    for t in range(1, STEPS + 1):
        W.fill_grads(torch, w, G, 0, t)
        if h is not None:
            h["G"] = host_copy({"G": G})["G"]
        bfo.grad_global_norm(T, G, res_e, w.hparams.max_norm)
        bfo.adamw_sr_step(T, eager["P"], G, eager["M"], eager["m"], eager["v"],
                          with_lr(bfo, w.hparams, lr_of(bfo, t)), t, step_seed(t), scale=res_e)
        g.replay()
        torch.cuda.synchronize()
        assert int(cursor.item()) == t
        assert torch.equal(res_g, res_e), f"norm result differs at t={t}"
        assert_same_bits(bits(graph), bits(eager), f"{w.name} master={master} replay {t}")
        if h is not None:
            scale = bfo.read_norm_result(res_g)[2]
            o.adamw_step(tbl, 0, h["P"], h["G"], h["M"], h["m"], h["v"],
                         o.hparams(lr_of(bfo, t), w.hparams.beta1, w.hparams.beta2, w.hparams.eps,
                                   w.hparams.weight_decay, w.hparams.bias_correction),
                         scale, t, step_seed(t))
            assert_state_parity(host_copy(graph), h, f"{w.name} graph replay {t} vs oracle")
    del g
