"""Unsharded, per-tensor block-wise 8-bit AdamW in numpy -- TEST INFRASTRUCTURE.

This is the same step as ``ve_oracle.c`` written against the *tensor*, with
no bucket, no ranks and no shard coordinates: every quantisation block is the
natural 2-D slice ``W[p*br:(p+1)*br, j*bc:(j+1)*bc]``.  Because shard
boundaries coincide with block boundaries, running the sharded oracle on
every rank and reassembling must reproduce this bit for bit (sync-free
block-wise quantisation; veScale-FSDP talk notes, "1. RaggedShard").  It
exists to pin the sharded oracle's layout logic, and runs on small tensors
only.
"""

from __future__ import annotations

import numpy as np


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16).copy()


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def step_tensor(grad_bits, master, m_q, v_q, m_scale, v_scale, block_rows, block_cols, hp, t):
    """One step on one whole tensor.

    grad_bits: uint16[R, C] bf16 gradient; master: float32[R, C];
    m_q, v_q: int8[R, C]; m_scale, v_scale: float32[P, J] with P row panels
    and J = C / block_cols tiles per panel.  Returns new
    (master, m_q, v_q, m_scale, v_scale, param_bits) without touching inputs.
    """
    f = lambda key: float(np.float32(hp[key]))
    lr, b1, b2, eps, wd = f("lr"), f("beta1"), f("beta2"), f("eps"), f("weight_decay")
    bc1 = 1.0 - b1 ** t
    bc2 = 1.0 - b2 ** t
    R, Cc = master.shape
    P = -(-R // block_rows)
    J = Cc // block_cols
    master_o = master.copy()
    mq_o, vq_o = m_q.copy(), v_q.copy()
    ms_o, vs_o = m_scale.copy(), v_scale.copy()
    for p in range(P):
        rs = slice(p * block_rows, min((p + 1) * block_rows, R))
        for j in range(J):
            cs = slice(j * block_cols, (j + 1) * block_cols)
            g = _bf16_to_f64(grad_bits[rs, cs])
            m0 = m_q[rs, cs].astype(np.float64) * float(m_scale[p, j])
            v0 = v_q[rs, cs].astype(np.float64) * float(v_scale[p, j])
            m1 = b1 * m0 + (1.0 - b1) * g
            v1 = b2 * v0 + (1.0 - b2) * g * g
            w = master[rs, cs].astype(np.float64)
            w = w * (1.0 - lr * wd) - (lr / bc1) * m1 / (np.sqrt(v1) / np.sqrt(bc2) + eps)
            master_o[rs, cs] = w.astype(np.float32)
            m1f, v1f = m1.astype(np.float32), v1.astype(np.float32)
            am, av = np.float32(np.abs(m1f).max()), np.float32(v1f.max())
            ms_o[p, j] = np.float32(np.float64(am) / 127.0)
            vs_o[p, j] = np.float32(np.float64(av) / 127.0)
            im = np.float32(127.0 / np.float64(am)) if am > 0 else np.float32(0)
            iv = np.float32(127.0 / np.float64(av)) if av > 0 else np.float32(0)
            xm = np.rint((m1f.astype(np.float64) * np.float64(im)).astype(np.float32))
            xv = np.rint((v1f.astype(np.float64) * np.float64(iv)).astype(np.float32))
            mq_o[rs, cs] = np.clip(xm, -127, 127).astype(np.int8)
            vq_o[rs, cs] = np.clip(xv, -127, 127).astype(np.int8)
    return master_o, mq_o, vq_o, ms_o, vs_o, _bf16_bits(master_o)
