"""Test-side helpers: dtype plumbing and an independent packer for the pool format.

The packer writes token vectors into pools with numpy reshapes of the
documented storage format; it shares no code with the oracle (C index
arithmetic) or with the kernels.
"""
import numpy as np
import torch

import oracle

TORCH_DTYPE = {oracle.F32: torch.float32, oracle.F16: torch.float16, oracle.BF16: torch.bfloat16}
CODE = {v: k for k, v in TORCH_DTYPE.items()}


def raw(t: torch.Tensor) -> np.ndarray:
    """numpy view of a CPU tensor's element bits, as the oracle takes them."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def empty_pools(NB, Hkv, D, B, dtype, x, fill=float("nan")):
    k = torch.full((NB, Hkv, D // x, B, x), fill, dtype=dtype)
    v = torch.full((NB, Hkv, D, B), fill, dtype=dtype)
    return k, v


def put_token(k_pool, v_pool, block, offset, k_tok, v_tok):
    """Store one token ([Hkv, D] each) at (block, offset) of the pools."""
    NB, Hkv, DX, B, X = k_pool.shape
    k_pool[block, :, :, offset, :] = k_tok.reshape(Hkv, DX, X)
    v_pool[block, :, :, offset] = v_tok


def get_token(k_pool, v_pool, block, offset):
    NB, Hkv, DX, B, X = k_pool.shape
    return (k_pool[block, :, :, offset, :].reshape(Hkv, DX * X), v_pool[block, :, :, offset])


def sdpa64(q, k, v, scale, group):
    """Textbook softmax attention in float64 through torch.

    q [Hq, D], k/v [n, Hkv, D] (float64) -> [Hq, D].  Query head h uses kv
    head h // group (k and v repeated along heads).
    """
    n = k.shape[0]
    Hq, D = q.shape
    if n == 0:
        return torch.zeros(Hq, D, dtype=torch.float64)
    kk = k.permute(1, 0, 2).repeat_interleave(group, dim=0).contiguous()  # [Hq, n, D]
    vv = v.permute(1, 0, 2).repeat_interleave(group, dim=0).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(
        q[None, :, None, :], kk[None], vv[None], scale=scale)
    return out[0, :, 0, :]
