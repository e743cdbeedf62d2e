"""Small helpers shared by the GPU tests: the bf16 bits of a device tensor on
the host, and the library's hyperparameters from the oracle's."""

import numpy as np


def u16(t):
    """The bit patterns of a bf16 (or int16) device tensor, as a host uint16 array."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def hp_of(ohp, step):
    """zero.hparams from the oracle's AdamWHParams at step ``step``."""
    from fsdp_sharded_mixed_zero_amd import zero
    return zero.hparams(lr=ohp.lr, beta1=ohp.beta1, beta2=ohp.beta2, eps=ohp.eps,
                        weight_decay=ohp.weight_decay, max_norm=ohp.max_norm,
                        clip_eps=ohp.clip_eps, step=step)
