"""The README's Python example runs as written and its results match the oracle."""
from __future__ import annotations

import os
import re

import numpy as np
import pytest
import torch

from oracle import oracle

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def _python_example():
    text = open(README).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert blocks, "README has no python example"
    return blocks[0]


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_readme_python_example(gpu):
    ns = {}
    exec(compile(_python_example(), "README.md", "exec"), ns)
    torch.cuda.synchronize()
    srcs = ns["srcs"]
    host = [s.view(torch.uint8).cpu().numpy() for s in srcs]
    assert np.array_equal(ns["out"].view(torch.uint8).cpu().numpy(), np.concatenate(host))
    payloads = [_bits(s) for s in srcs]
    want = np.empty(payloads[0].shape[0], np.uint16)
    oracle.reduce_c(payloads, want, "bf16")
    assert np.array_equal(_bits(ns["total"]), want)
    n = want.shape[0] // len(srcs)
    assert np.array_equal(_bits(ns["share"]), want[3 * n:4 * n])
    a, b = ns["outs"]
    assert np.array_equal(a.view(torch.uint8).cpu().numpy(), np.concatenate(host[:4]))
    assert np.array_equal(b.view(torch.uint8).cpu().numpy(), np.concatenate(host[4:]))
