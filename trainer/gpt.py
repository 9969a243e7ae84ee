"""Learned-position GPT with the gpt-11m tensor list.

Vocabulary 12,096 (tied embedding and head), 1,024 positions, 10 blocks of
width 256 with 4 heads, GELU MLP of width 1,024, pre-LayerNorm, final
LayerNorm: 124 tensors, 11,256,832 parameters, all FP32.  The page gives the
real model only as "a lean learned-position GPT" of 11,637,760 parameters
(Packed AdamW Reference README, What is included; project page header);
the head count and block layout are readings.
"""
import math

import torch
import torch.nn as nn
import torch.nn.functional as F


class Block(nn.Module):
    def __init__(self, d, heads):
        super().__init__()
        self.heads = heads
        self.ln1 = nn.LayerNorm(d)
        self.qkv = nn.Linear(d, 3 * d)
        self.proj = nn.Linear(d, d)
        self.ln2 = nn.LayerNorm(d)
        self.fc = nn.Linear(d, 4 * d)
        self.fc2 = nn.Linear(4 * d, d)

    def forward(self, x):
        b, t, d = x.shape
        q, k, v = self.qkv(self.ln1(x)).split(d, dim=2)
        shape = (b, t, self.heads, d // self.heads)
        q, k, v = (z.view(shape).transpose(1, 2) for z in (q, k, v))
        y = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        x = x + self.proj(y.transpose(1, 2).reshape(b, t, d))
        return x + self.fc2(F.gelu(self.fc(self.ln2(x))))


class GPT(nn.Module):
    def __init__(self, vocab=12096, ctx=1024, d=256, layers=10, heads=4):
        super().__init__()
        self.wte = nn.Embedding(vocab, d)
        self.wpe = nn.Embedding(ctx, d)
        self.blocks = nn.ModuleList([Block(d, heads) for _ in range(layers)])
        self.lnf = nn.LayerNorm(d)
        self.reset(seed=0)

    @torch.no_grad()
    def reset(self, seed):
        g = torch.Generator().manual_seed(seed)
        for name, p in self.named_parameters():
            is_norm = name.startswith("lnf") or ".ln" in name
            if name.endswith("bias"):
                p.zero_()                                    # every bias, norms included
            elif is_norm:
                p.fill_(1.0)                                 # LayerNorm gains
            else:
                p.copy_(torch.randn(p.shape, generator=g) * 0.02)

    def forward(self, idx, targets=None):
        t = idx.shape[1]
        pos = torch.arange(t, device=idx.device)
        x = self.wte(idx) + self.wpe(pos)[None]
        for blk in self.blocks:
            x = blk(x)
        logits = self.lnf(x) @ self.wte.weight.t()
        if targets is None:
            return logits
        return F.cross_entropy(logits.view(-1, logits.shape[-1]), targets.reshape(-1))


def count_params(model):
    return sum(p.numel() for p in model.parameters())


def lr_at(step, base_lr, warmup, total):
    """Linear warm-up then linear decay (the reference config's schedule shape)."""
    if step <= warmup:
        return base_lr * step / max(1, warmup)
    return base_lr * max(0.0, (total - step) / max(1, total - warmup))


assert math.isclose(lr_at(5, 1.0, 10, 20), 0.5)
