"""Move seeded synthetic inputs (numpy, from ``synth``) onto a GPU as torch tensors (torch is
imported by the caller; this module only converts)."""
from types import SimpleNamespace

import numpy as np
import torch


def tensor(a, device="cuda"):
    if a is None:
        return None
    arr = np.ascontiguousarray(a)
    if arr.dtype == np.uint16:                      # bfloat16 bit patterns
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr).to(device)


def layer(inp, device="cuda"):
    return SimpleNamespace(
        x=tensor(inp.x, device), x_scale=tensor(inp.x_scale, device),
        w_gate=tensor(inp.w_gate, device), w_up=tensor(inp.w_up, device),
        w_down=tensor(inp.w_down, device), wg_scale=tensor(inp.wg_scale, device),
        wu_scale=tensor(inp.wu_scale, device), wd_scale=tensor(inp.wd_scale, device),
        expert_ids=tensor(inp.expert_ids, device), probs=tensor(inp.probs, device))


def forward(mel, d, head_m_size=0, workspace=None, separate_permute=False):
    if d.x.dtype == torch.uint8:
        return mel.expert_forward_mx(d.x, d.x_scale, d.w_gate, d.wg_scale, d.w_up, d.wu_scale,
                                     d.w_down, d.wd_scale, d.expert_ids, d.probs,
                                     head_m_size=head_m_size, workspace=workspace,
                                     separate_permute=separate_permute)
    return mel.expert_forward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs,
                              head_m_size=head_m_size, workspace=workspace,
                              separate_permute=separate_permute)


def host(t):
    """Device tensor -> numpy (bfloat16 widened exactly to float32)."""
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()
