"""The C ABI is reentrant: several host threads call it at once, each on its own
stream.  The calls run in a fresh child process, so the threads' first calls
into the library (which set per-kernel launch attributes) race as well.  Every
thread's gate scores, attention output and LSE must equal, bit for bit, those
of the same calls made one after another."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, threading
sys.path.insert(0, ROOT)
import numpy as np, torch
import workloads
from learned_token_pruning_05_amd import _lib as tg

tg.load()
dev = "cuda:0"
w = workloads.by_name("16k")
g = w.gate_inputs(with_bias=True)
x, w1, b1, w2 = (g[k].to(dev) for k in ("x", "w1", "b1", "w2"))
ck = tg.tg_kept_counts(w.cu_seqlens, w.doc_begin, w.doc_end, w.k_doc_arr)
m, mx = int(ck[-1]), int(np.diff(ck).max())
q, k, v = (t.to(dev) for t in w.qkv(m))
gain, tau = w.attn_params()
gain = torch.from_numpy(gain).to(dev)
sk = torch.from_numpy(np.random.default_rng(3).standard_normal(m).astype(np.float32)).to(dev)
pos = torch.cat([torch.arange(int(ck[i + 1] - ck[i]), dtype=torch.int32) for i in range(len(ck) - 1)]).to(dev)
ckd = torch.from_numpy(ck).to(dev)
torch.cuda.synchronize()

N = 4
streams = [torch.cuda.Stream() for _ in range(N)]
start = threading.Barrier(N)
res = [None] * N
err = []


def run(i):
    try:
        with torch.cuda.stream(streams[i]):
            start.wait()
            s = tg.tg_gate_score(x, w1, b1, w2, g["b2"])
            o, l = tg.tg_keybias_attn_prefill(q, k, v, sk, gain, tau, pos, ckd, mx, 1e6)
        streams[i].synchronize()
        res[i] = (s.cpu(), o.cpu(), l.cpu())
    except Exception as e:  # reported below, after every thread has joined
        err.append(f"thread {i}: {e!r}")


threads = [threading.Thread(target=run, args=(i,)) for i in range(N)]
for t in threads:
    t.start()
for t in threads:
    t.join()
assert not err, err
s0 = tg.tg_gate_score(x, w1, b1, w2, g["b2"])
o0, l0 = tg.tg_keybias_attn_prefill(q, k, v, sk, gain, tau, pos, ckd, mx, 1e6)
torch.cuda.synchronize()
ref = (s0.cpu(), o0.cpu(), l0.cpu())
for i, r in enumerate(res):
    for a, b, name in zip(r, ref, ("scores", "out", "lse")):
        assert torch.equal(a, b), f"thread {i}: {name} differs from the sequential call"
print("threads ok", flush=True)
"""


def test_threads_first_calls_race():
    print("\n>> case: 4 threads, first calls racing, own streams (16k gate + attention)", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD.replace("ROOT", repr(ROOT))], capture_output=True, text=True,
                       timeout=110)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "threads ok" in r.stdout
