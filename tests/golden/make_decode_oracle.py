"""Writes the oracle's 16-step greedy decode of the full-size synthetic models.

Runs only the fp64 oracle (oracle/) on the seeded inputs of synth/: nothing
here touches the HIP library.  For each model it stores, per step and
sequence, the greedy token, the oracle's top-2 margin, and the oracle logits
at a sample of vocabulary indices (the 8 largest plus 24 fixed seeded ones);
for the first and the last step it also stores every logit of the vocabulary
(fp32, ``<name>_logits_sNN.npy``), so the GPU test compares the whole
vocabulary there without re-running a multi-minute fp64 decode on every test
run.

Usage:  python tests/golden/make_decode_oracle.py [decode_qwen3_4b] [decode_gemma4_31b]
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from synth import workloads as wl  # noqa: E402

N_TOP = 8
N_FIXED = 24


def full_logit_steps(m):
    return [0, m.steps - 1]


def logits_path(name, step):
    return os.path.join(HERE, f"{name}_logits_s{step:02d}.npy")


def run(m):
    t0 = time.time()
    weights = wl.model_weights(m)
    caches = [(wl.prefilled_cache(m, l, "k"), wl.prefilled_cache(m, l, "v"))
              for l in range(m.n_layers)]
    print(f"{m.name}: inputs in {time.time() - t0:.0f} s, {oracle.num_threads()} oracle threads",
          flush=True)
    om = oracle.Model(wl.oracle_spec(m, weights, caches))
    fixed = synth.tokens(m.seed, "logit_sample", N_FIXED, m.vocab).astype(np.int64)
    tok = wl.start_tokens(m)
    out = dict(workload=m.name, seed=m.seed, start_pos=m.start_pos, steps=m.steps,
               batch=m.batch, vocab=m.vocab, start_tokens=tok.tolist(),
               tokens=[], margins=[], sample_idx=[], sample_logits=[], logits_sq_sum=[],
               full_logit_steps=full_logit_steps(m))
    for s in range(m.steps):
        t1 = time.time()
        nxt, lg, mg = om.step(m.start_pos + s, tok, want_logits=True)
        idx = []
        vals = []
        for b in range(m.batch):
            top = np.argsort(-lg[b], kind="stable")[:N_TOP]
            ib = [int(i) for i in top] + [int(i) for i in fixed if int(i) not in set(top.tolist())]
            idx.append(ib)
            vals.append([float(lg[b, i]) for i in ib])
        out["tokens"].append(nxt.tolist())
        out["margins"].append(mg.tolist())
        out["sample_idx"].append(idx)
        out["sample_logits"].append(vals)
        out["logits_sq_sum"].append([float((lg[b] ** 2).sum()) for b in range(m.batch)])
        if s in out["full_logit_steps"]:
            np.save(logits_path(m.name, s), lg.astype(np.float32))
        print(f"  step {s}: {time.time() - t1:.1f} s tokens {nxt.tolist()} "
              f"min margin {mg.min():.4f}", flush=True)
        tok = nxt
    return out


def main():
    names = sys.argv[1:] or ["decode_qwen3_4b", "decode_gemma4_31b"]
    shapes = {wl.QWEN3_4B.name: wl.QWEN3_4B, wl.GEMMA4_31B.name: wl.GEMMA4_31B}
    for name in names:
        out = run(shapes[name])
        path = os.path.join(HERE, f"{name}_oracle.json")
        with open(path, "w") as f:
            json.dump(out, f)
        print(f"wrote {path}", flush=True)


if __name__ == "__main__":
    main()
