"""Overlapped context projection: the projection forked onto an aux stream ahead of a simulated
sample/accept window on the main stream, joined before the store (TensorRT-LLM PR #20550 "fuse the
decode-step drafter bookkeeping into Triton kernels", section TLLM_DFLASH_OVERLAP_CONTEXT_PROJECTION).

The overlapped step must give the same bits as dfkv_step, eagerly and from a captured graph; a
negative control shows that without the join the store reads kv_out before the projection wrote it."""
import numpy as np
import pytest

from dfkv_workloads import make_workload
from gpu_helpers import compare_bookkeeping, oracle_bookkeeping

pytestmark = pytest.mark.gpu


def _event(stream):
    """A torch event whose HIP event exists (created on its first record)."""
    import torch
    e = torch.cuda.Event()
    e.record(stream)
    return e


def _pair(cfg):
    from store_dfkv_project_amd.step import DeviceStep
    wl = make_workload(cfg)
    return wl, DeviceStep(wl, pool_seed=7), DeviceStep(wl, pool_seed=7)


def _same(a, b):
    import torch
    assert torch.equal(a.kv_out, b.kv_out), "kv_out"
    assert torch.equal(a.pool_t, b.pool_t), "pool"
    ga, gb = a.outputs_host(), b.outputs_host()
    for k in ga:
        assert np.array_equal(ga[k], gb[k]), k


def _overlapped(a, main, aux, fork, join, window, recorded):
    """One overlapped step on `main`: the projection forked at the call, ahead of the window, or
    (recorded) at a fork point the caller records before the window, the projection queued after it."""
    import torch
    from store_dfkv_project_amd import dfkv
    with torch.cuda.stream(main):
        if recorded:
            fork.record(main)
            torch.cuda._sleep(window)
            a.project_fork(main, aux, fork.cuda_event, join.cuda_event,
                           flags=dfkv.DFKV_FUSE_NORM_ROPE | dfkv.DFKV_FORK_RECORDED)
        else:
            a.project_fork(main, aux, fork.cuda_event, join.cuda_event)
            torch.cuda._sleep(window)            # the sample/accept window on main
        dfkv.dfkv_join(main, join.cuda_event)
        a.store_advance(stream=main)


@pytest.mark.parametrize("recorded", [False, True])
@pytest.mark.parametrize("cfg", [0, 1])
def test_fork_join_equals_step(orc, cfg, recorded):
    import torch
    wl, a, b = _pair(cfg)
    print(f"[overlap] fork/join config {cfg} fork recorded by the caller {recorded}", flush=True)
    main, aux = torch.cuda.Stream(), torch.cuda.Stream()
    fork, join = _event(main), _event(aux)
    torch.cuda.synchronize()
    _overlapped(a, main, aux, fork, join, 2_000_000, recorded)
    b.step()
    torch.cuda.synchronize()
    _same(a, b)
    compare_bookkeeping(a.outputs_host(), oracle_bookkeeping(orc, wl), f"overlap config {cfg}")


@pytest.mark.parametrize("recorded", [False, True])
def test_fork_join_graph_replays(recorded):
    """The overlapped step (fork, window, join, store) captured into one graph on `main`: every replay,
    with eager work and synchronisations between replays, gives the eager bits."""
    import torch
    wl, a, b = _pair(1)
    print(f"[overlap] graph capture, fork recorded by the caller {recorded}", flush=True)
    main, aux = torch.cuda.Stream(), torch.cuda.Stream()
    fork, join = _event(main), _event(aux)
    b.step()
    torch.cuda.synchronize()
    pool0 = a.pool_t.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=main):
        _overlapped(a, main, aux, fork, join, 200_000, recorded)
    torch.cuda.synchronize()
    for rep in range(3):
        a.pool_t.copy_(pool0)
        a.kv_out.zero_()
        a.block_slot.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(a, b)
        b.step()                                  # eager work between replays
        torch.cuda.synchronize()


def test_missing_join_negative_control():
    """Without dfkv_join the store on `main` does not wait for the projection on `aux`: with the aux stream
    held back, the pool receives kv_out's stale contents.  With the join it receives the projection."""
    import time
    import torch
    from store_dfkv_project_amd import dfkv
    wl, a, b = _pair(1)
    print("[overlap] negative control", flush=True)
    b.step()
    torch.cuda.synchronize()
    main, aux = torch.cuda.Stream(), torch.cuda.Stream()
    fork, join, main_done, aux_done = _event(main), _event(aux), torch.cuda.Event(), torch.cuda.Event()
    sentinel = 0x1234
    a.kv_out.fill_(sentinel)
    torch.cuda.synchronize()
    with torch.cuda.stream(aux):
        torch.cuda._sleep(100_000_000)            # hold the aux stream back (tens of ms)
    a.project_fork(main, aux, fork.cuda_event, join.cuda_event)
    aux_done.record(aux)
    with torch.cuda.stream(main):
        a.store_advance(stream=main)              # no dfkv_join: nothing orders it after the projection
    main_done.record(main)
    t0 = time.time()
    while not main_done.query() and time.time() - t0 < 5.0:
        time.sleep(0.0005)
    raced = main_done.query() and not aux_done.query()
    torch.cuda.synchronize()
    if not raced:
        pytest.skip("the two streams did not run concurrently here: the race could not be shown")
    want = b.outputs_host()
    rows = np.nonzero(want["write_mask"])[0]
    assert len(rows) > 0
    # the written rows carry the stale kv_out (sentinel) instead of the projection
    slot = want["slot"][rows[0]]
    view = a.pool_slot_view(0, 0)
    assert int(view[slot, 0].item()) == sentinel
    assert not torch.equal(a.pool_t, b.pool_t)
