"""Concurrent use: the library keeps no state besides a thread-local last
error, so gathers and sums issued from several host threads, each on its own
stream (default priority), run side by side on the GPU and each result
matches the oracle."""
from __future__ import annotations

import threading

import numpy as np
import pytest
import torch

from deterministic_collective_movement_amd import rog
from deterministic_collective_movement_amd import workloads as wl
from oracle import oracle

pytestmark = pytest.mark.gpu


def test_threads_and_streams(gpu):
    n_threads, rounds = 4, 6
    jobs = []
    for t in range(n_threads):
        W, S = 3 + t, 200_000 + 17 * t
        payloads = [wl.random_bytes(wl.case_seed(27, t), r, S) for r in range(W)]
        want_g = np.empty(W * S, np.uint8)
        oracle.gather_c(payloads, want_g)
        rp = wl.reduce_payloads(wl.case_seed(28, t), W, 150_001, "bf16")
        want_r = np.empty(150_001, np.uint16)
        oracle.reduce_c(rp, want_r, "bf16")
        jobs.append({"W": W, "S": S, "payloads": payloads, "want_g": want_g, "want_r": want_r,
                     "gsrcs": [torch.from_numpy(p).to(gpu) for p in payloads],
                     "rsrcs": [torch.from_numpy(p.view(np.int16)).to(gpu).view(torch.bfloat16) for p in rp],
                     "gout": torch.empty(W * S, dtype=torch.uint8, device=gpu),
                     "rout": torch.empty(150_001, dtype=torch.bfloat16, device=gpu),
                     "stream": torch.cuda.Stream(device=gpu)})
    torch.cuda.synchronize()
    errors = []

    def work(job):
        try:
            for _ in range(rounds):
                rog.rog_gather(job["gsrcs"], job["gout"], stream=job["stream"])
                rog.rog_reduce(job["rsrcs"], job["rout"], stream=job["stream"])
            job["stream"].synchronize()
        except Exception as e:      # pragma: no cover - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for j in jobs:
        assert np.array_equal(j["gout"].cpu().numpy(), j["want_g"]), (j["W"], j["S"])
        assert np.array_equal(j["rout"].view(torch.int16).cpu().numpy().view(np.uint16), j["want_r"]), j["W"]
    assert rog.rog_last_hip_error() == 0
