"""Entry points are reentrant: two host threads, each with its own stream,
buffers and workspaces, run the decode path and the prefill path at the same
time; every output equals, bit for bit, the one of the same call run alone."""
import threading

import pytest
import torch

import trainable_block_sparse_amd as tbs
from synth import CONFIGS, make_inputs

from parity import problems

pytestmark = pytest.mark.gpu


def _decode_case():
    cfg = CONFIGS["decode"]
    x = make_inputs(cfg, n_kv=20000, batch=4, seed=401)
    lp, _ = problems(cfg, n_kv=20000, batch=4)
    return lp, x


def _prefill_case():
    cfg = CONFIGS["prefill32k"]
    x = make_inputs(cfg, n_kv=3000, batch=1, seed=402)
    lp, _ = problems(cfg, n_kv=3000, batch=1)
    return lp, x


def _run(lp, x, stream, reps):
    dev = torch.device("cuda:0")
    with torch.cuda.stream(stream):
        Q, K, V = (x[k].to(dev, non_blocking=False) for k in ("q", "k", "v"))
        outs = []
        for _ in range(reps):
            Kc1 = tbs.compress_k(lp, K, stream=stream)
            idx, n_sel = tbs.select_blocks(lp, Q, Kc1, stream=stream)
            O, lse = tbs.sparse_attn(lp, Q, K, V, idx, n_sel, stream=stream)
            outs.append((idx, n_sel, O, lse))
    stream.synchronize()
    return [tuple(t.cpu() for t in o) for o in outs]


def test_two_threads_two_streams_match_the_calls_run_alone():
    cases = [_decode_case(), _prefill_case()]
    print("case: concurrent decode and prefill on two streams", flush=True)
    alone = [_run(lp, x, torch.cuda.Stream(), 1)[0] for lp, x in cases]
    results = [None, None]

    def worker(i):
        lp, x = cases[i]
        results[i] = _run(lp, x, torch.cuda.Stream(), 6)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i in range(2):
        assert results[i] is not None
        for rep in results[i]:
            for got, want in zip(rep, alone[i]):
                assert torch.equal(got, want)
