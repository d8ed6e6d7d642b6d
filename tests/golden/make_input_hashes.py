"""Writes SHA-256 hashes of the tiny workload's seeded inputs (tiny_4k_input_sha256.json).

The hashes pin the input recipe (seeded generators, shapes, dtypes, value ranges), not any
result of the layer: no oracle or library call is involved.  torch draws different streams
on the CPU and on the GPU, so each device kind has its own entry; run once per kind:

    python tests/golden/make_input_hashes.py cpu
    python tests/golden/make_input_hashes.py cuda
"""

import hashlib
import json
import os
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from long_context_sparse_index_amd import inputs as I  # noqa: E402
from long_context_sparse_index_amd import workloads as W  # noqa: E402

OUT = os.path.join(HERE, "tiny_4k_input_sha256.json")


def tensor_sha256(t: torch.Tensor) -> str:
    b = t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()
    return hashlib.sha256(b).hexdigest()


def tiny_input_hashes(device) -> dict:
    wl = W.WORKLOADS["tiny_4k"]
    q_i, k_i, w = I.index_inputs(wl, device)
    q, kv, v = I.attn_inputs(wl, device, separate_v=True)
    d_o = I.grad_output(wl, device)
    named = {"q_idx": q_i, "k_idx": k_i, "w": w, "q": q, "kv": kv, "v": v, "d_o": d_o}
    return {n: {"shape": list(t.shape), "dtype": str(t.dtype).replace("torch.", ""),
                "sha256": tensor_sha256(t)} for n, t in named.items()}


def main(kind: str):
    device = torch.device("cuda:0" if kind == "cuda" else "cpu")
    rec = {}
    if os.path.exists(OUT):
        with open(OUT) as fh:
            rec = json.load(fh)
    rec[kind] = tiny_input_hashes(device)
    with open(OUT, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print("wrote", kind, "hashes to", OUT)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "cpu")
