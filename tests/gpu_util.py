"""Device upload helpers for the GPU tests (test infrastructure)."""

import numpy as np
import torch

DEV = torch.device("cuda:0")


def up(a):
    """numpy array -> device tensor of the same bits (bf16 bits become bfloat16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def down_bits(t):
    """device tensor -> numpy array of its stored bits (bf16 -> uint16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def down_f64(t):
    return t.detach().cpu().float().numpy().astype(np.float64)


class Paged:
    """Device copies of a PagedDecodeInputs."""

    def __init__(self, inp):
        self.inp = inp
        self.q = up(inp.q)
        self.k_cache = up(inp.k_pool)
        self.v_cache = up(inp.v_pool)
        self.k_new = up(inp.k_new)
        self.v_new = up(inp.v_new)
        self.table = up(inp.block_table)
        self.seq = up(inp.seq_lens)


def log(msg):
    print(msg, flush=True)
