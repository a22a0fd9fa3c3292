"""Write verify_drafts_7b.json: the drafted tokens of the 7B fp16 verify workload, from the oracle alone.

The workload: 8 sequences, each with 1023 positions of synthetic K/V (content id
= sequence index), a random token at position 1023, then one verify pass of
K = 5 drafted tokens at positions 1024..1028.

Drafts follow the greedy-verify reading of [KV Cache] section 08 and
[Spending the Idle] section 12.4: the target's own greedy token is the one a
perfect draft would propose, and a draft is right with probability alpha =
0.7, independently per position. Per sequence:

  g0      = the oracle's greedy token after the K = 1 step at position 1023;
  d_j     = g_{j-1} with probability 0.7, else a uniform token (j = 1..5);
  g_j     = the oracle's greedy token after a K = 1 step that feeds d_j at
            position 1023 + j (j = 1..4), continuing the same cache.

The coin flips and replacement tokens come from the drafts stream of the
seeded generator (seed 4005). Only oracle/ and synth/ are called; run from the
repository root:  python tests/golden/make_verify_drafts.py
"""
from __future__ import annotations

import json
import os
import sys
import time

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from synth import workloads as W  # noqa: E402

WL = 4
SEED_W, SEED_KV, SEED_TOK, SEED_DR = 1000 * WL + 1, 1000 * WL + 2, 1000 * WL + 3, 1000 * WL + 5
B, CTX, K, ALPHA = 8, 1024, 5, 0.7
OUT = os.path.join(HERE, "verify_drafts_7b.json")


def draws(b: int):
    coin = synth.uniform(synth.key(SEED_DR, W.STREAM_DRAFTS, b), 0, K)
    alt = synth.uniform_int(synth.key(SEED_DR, W.STREAM_DRAFTS, 100 + b), 0, K, 0, W.LLAMA7B.vocab)
    return [float(c) for c in coin], [int(a) for a in alt]


def main():
    dims = W.LLAMA7B
    t0 = time.time()
    w = W.make_weights(dims, SEED_W)
    print(f"weights {time.time() - t0:.0f}s", flush=True)
    seqs = []
    t_last = []
    for b in range(B):
        kv = torch.zeros(dims.n_layers, 2, CTX + K, dims.n_kv_heads, dims.head_dim, dtype=dims.torch_dtype)
        kv[:, :, :CTX - 1] = W.kv_block(dims, SEED_KV, b, 0, CTX - 1)
        tok = W.token_ids(SEED_TOK, b, 1, dims.vocab)[0]
        t_last.append(tok)
        seqs.append(oracle.SeqState(kv, CTX - 1, [tok]))
    res = oracle.decode_step(dims, w, seqs)
    g0 = list(res.argmax)
    g0_gap = list(res.gap)
    print(f"g0 {g0}  {time.time() - t0:.0f}s", flush=True)
    drafts = [[0] * K for _ in range(B)]
    chain = [[] for _ in range(B)]
    chain_gap = [[] for _ in range(B)]
    coins = [draws(b) for b in range(B)]
    prev = list(g0)
    for j in range(1, K + 1):
        for b in range(B):
            coin, alt = coins[b]
            drafts[b][j - 1] = prev[b] if coin[j - 1] < ALPHA else alt[j - 1]
        if j == K:
            break
        for b in range(B):
            seqs[b].ctx += 1
            seqs[b].tokens = [drafts[b][j - 1]]
        res = oracle.decode_step(dims, w, seqs)
        for b in range(B):
            chain[b].append(int(res.argmax[b]))
            chain_gap[b].append(float(res.gap[b]))
        prev = [int(a) for a in res.argmax]
        print(f"step {j}: {prev}  {time.time() - t0:.0f}s", flush=True)
    data = {
        "what": "7B fp16 verify workload: 8 sequences, context 1024 (1023 synthetic positions + one K=1 step), "
                "K=5 drafts, each the oracle's greedy token with probability 0.7",
        "written_by": "tests/golden/make_verify_drafts.py (oracle and synth only)",
        "seeds": {"weights": SEED_W, "kv": SEED_KV, "tokens": SEED_TOK, "drafts": SEED_DR},
        "B": B, "ctx": CTX, "K": K, "alpha": ALPHA,
        "token_at_1023": t_last,
        "g0": g0,
        "g0_gap": g0_gap,
        "drafts": drafts,
        "greedy_chain_g1_to_g4": chain,
        "greedy_chain_gaps": chain_gap,
    }
    with open(OUT, "w") as f:
        json.dump(data, f, indent=1)
    print("wrote", OUT, flush=True)


if __name__ == "__main__":
    main()
