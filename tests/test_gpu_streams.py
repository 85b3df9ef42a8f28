"""GPU test of the library's thread safety and stream ordering: host threads
calling kda_chunk_fwd and kda_recurrent_step at the same time, each on its
own stream with its own buffers, get bit for bit what the same calls give one
after another on one stream."""
import dataclasses
import threading

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as kda
    kda.load_library()


def _job(kind, seed):
    """Inputs of one thread's work: a few-pair batch (split design), a packed
    many-pair call (pair mode) or a decode step run four times in place."""
    if kind == "batch":
        return W.make_prefill(dataclasses.replace(W.WORKLOADS["prefill_8k"], seed=seed), "cuda", T=700, H=8)
    if kind == "packed":
        w = dataclasses.replace(W.WORKLOADS["varlen_64"], seed=seed)
        lens = torch.randint(1, 150, (64,), generator=torch.Generator().manual_seed(seed))
        return W.make_prefill(w, "cuda", H=2, lengths=lens)
    return W.make_decode(dataclasses.replace(W.WORKLOADS["decode_512"], seed=seed), device="cuda", N=16, H=4,
                         steps=4)


def _run(kind, inp, stream):
    """The job's calls on `stream`; returns its outputs (new tensors)."""
    import gated_delta_rule_20_amd as kda
    with torch.cuda.stream(stream):
        if kind == "decode":
            state = inp["state"].clone()
            outs = [kda.recurrent_step(st["q"], st["k"], st["v"], st["z"], st["beta"], state, A_log=inp["A_log"],
                                       stream=stream) for st in inp["steps"]]
            return outs + [state]
        outs = []
        for _ in range(3):  # repeated calls on the same inputs give the same bits
            o, hT = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["z"], inp["beta"], A_log=inp["A_log"],
                                  g_min=inp["g_min"], cu_seqlens=inp.get("cu_seqlens"),
                                  initial_state=inp["h0"], stream=stream)
            outs += [o, hT]
        return outs


def test_concurrent_threads_match_sequential_calls():
    kinds = ["batch", "packed", "decode", "batch", "packed", "decode"]
    jobs = [(k, _job(k, 400 + i)) for i, k in enumerate(kinds)]
    main = torch.cuda.current_stream()
    ref = [_run(k, inp, main) for k, inp in jobs]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in jobs]
    got = [None] * len(jobs)
    errors = []

    def worker(i):
        try:
            k, inp = jobs[i]
            streams[i].wait_stream(main)
            got[i] = _run(k, inp, streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported below, in the test's own thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (k, _) in enumerate(jobs):
        assert len(got[i]) == len(ref[i])
        for j, (a, b) in enumerate(zip(got[i], ref[i])):
            bad = (a.view(torch.uint8) != b.view(torch.uint8)).sum().item()
            assert bad == 0, f"job {i} ({k}), output {j}: {bad} bytes differ from the sequential run"
