"""Child process of the decode split-size test: runs the decode workload once with the chunk size
the environment variable FA_DECODE_CHUNK selects (read once per process by the library) and saves
O (as fp32) and lse to the .npz file named by argv[1]. Not a test module: pytest does not collect it."""

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import io_aware_exact_23_amd as fa  # noqa: E402
from io_aware_exact_23_amd import configs, inputs  # noqa: E402


def main(out_path: str) -> None:
    print(f"decode chunk child: FA_DECODE_CHUNK={os.environ.get('FA_DECODE_CHUNK')}", flush=True)
    fa.load_library()
    w = configs.DECODE_SPLIT_KV
    q, k, v, lt = inputs.make(w, "cuda")
    o, lse = fa.attention(q, k, v, scale=w.scale, causal=w.causal, kv_seqlens=lt)
    torch.cuda.synchronize()
    np.savez(out_path, o=o.float().cpu().numpy(), lse=lse.cpu().numpy())


if __name__ == "__main__":
    main(sys.argv[1])
