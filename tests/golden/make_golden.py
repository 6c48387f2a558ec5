"""Writes the stored expected values of the GPU tests by running the oracle only.

llama1b_greedy256.json: 256 free-running greedy decode steps of the
Llama-3.2-1B-shaped decoder (synthetic weights seed 1, KV-cache prefill seed 2,
first token seed 3), batch 1, context 1024 -> positions 1024..1279, KV cache of
2048 slots.  Stores every chosen token and the oracle's top-2 logit gap at that
step (a gap below the GPU's logit error marks a near-tie).

Usage: python tests/golden/make_golden.py
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def llama1b_greedy(steps=256, P0=1024, C=2048):
    cfg = synth.configs.LLAMA_1B
    w = synth.make_weights(cfg)
    kc, vc = synth.make_kv(cfg, 1, C)
    tok = synth.make_tokens(cfg, 1)
    t0 = time.time()
    r = oracle.greedy(cfg, w, tok, [P0], kc, vc, steps)
    return dict(config=cfg.name, seeds=dict(weights=synth.SEED_WEIGHTS, kv=synth.SEED_KV, tokens=synth.SEED_TOKENS),
                first_token=int(tok[0]), first_position=P0, max_ctx=C, steps=steps,
                tokens=[int(t) for t in r["tokens"][:, 0]], top2_gaps=[float(g) for g in r["gaps"][:, 0]],
                oracle_seconds=round(time.time() - t0, 1))


if __name__ == "__main__":
    out = llama1b_greedy()
    with open(os.path.join(HERE, "llama1b_greedy256.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print("min top-2 gap", min(out["top2_gaps"]), "oracle seconds", out["oracle_seconds"])
