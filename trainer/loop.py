"""Synthetic-tape training loop, checkpoints and the one-update smoke gates.

Tapes (Packed AdamW Reference README, Training on prepared tapes): a
little-endian uint32 token tape and an optional aligned little-endian uint16
tape of each token's length in bytes, memory-mapped from files, or seeded
synthetic tokens below the vocabulary size; either is read sequentially and
never wraps.  With byte lengths, evaluation reports bits per byte: the
summed cross-entropy of the predicted tokens in bits over their bytes.
Smoke gates (same README, One-update smoke test): finite train and
validation loss, zero optimizer non-finite count, a one-word state ledger,
and a checkpoint that round-trips.
"""
import math
import time

import numpy as np
import torch

from .gpt import GPT, count_params, lr_at


class Tape:
    def __init__(self, tokens, batch, seq, byte_lengths=None):
        if byte_lengths is not None and len(byte_lengths) != len(tokens):
            raise ValueError("the byte-length tape must hold one length per token")
        self.tokens = tokens
        self.byte_lengths = byte_lengths
        self.batch, self.seq = batch, seq
        self.cursor = 0

    @staticmethod
    def synthetic(n_tokens, vocab, seed):
        r = np.random.Generator(np.random.PCG64(seed))
        return Tape(r.integers(0, vocab, n_tokens, dtype=np.int64), 1, 1)

    @staticmethod
    def from_files(tokens_path, batch, seq, byte_lengths_path=None):
        """Memory-map a little-endian uint32 token tape and, optionally, its
        aligned little-endian uint16 byte-length tape."""
        tokens = np.memmap(tokens_path, dtype="<u4", mode="r")
        lengths = None if byte_lengths_path is None else np.memmap(byte_lengths_path, dtype="<u2", mode="r")
        return Tape(tokens, batch, seq, lengths)

    def _take(self):
        need = self.batch * self.seq + 1
        if self.cursor + need > len(self.tokens):
            raise RuntimeError("token tape exhausted (the trainer does not wrap)")
        a = self.cursor
        self.cursor += self.batch * self.seq
        return a, need

    def next(self, device):
        x, y, _ = self.next_with_bytes(device)
        return x, y

    def next_with_bytes(self, device):
        """The next window; the third value is the byte count of its predicted
        tokens (None without a byte-length tape)."""
        a, need = self._take()
        chunk = torch.from_numpy(np.asarray(self.tokens[a:a + need], dtype=np.int64))
        x = chunk[:-1].view(self.batch, self.seq)
        y = chunk[1:].view(self.batch, self.seq)
        nbytes = None
        if self.byte_lengths is not None:
            nbytes = int(np.asarray(self.byte_lengths[a + 1:a + need], dtype=np.int64).sum())
        return x.to(device), y.to(device), nbytes


def bits_per_byte(nats, nbytes):
    """Cross-entropy summed over predicted tokens (nats), in bits per byte."""
    return nats / (math.log(2.0) * nbytes)


@torch.no_grad()
def evaluate(model, tape, batches, device):
    """Mean cross-entropy per token over `batches` windows, and bits per byte
    when the tape carries byte lengths."""
    nats, tokens, nbytes = 0.0, 0, 0
    for _ in range(batches):
        x, y, b = tape.next_with_bytes(device)
        loss = float(model(x, y))
        nats += loss * y.numel()
        tokens += y.numel()
        if b is not None:
            nbytes += b
    mean = nats / max(1, tokens)
    return mean, (bits_per_byte(nats, nbytes) if tape.byte_lengths is not None and nbytes > 0 else None)


def make_optimizer(model, kind, lr, weight_decay=0.01):
    if kind in ("e4", "fp16", "fp32"):
        from adamw_step_amd.optim import PackedAdamW
        return PackedAdamW(model.parameters(), lr=lr, weight_decay=weight_decay, mode=kind)
    if kind == "turbo":
        from adamw_step_amd.optim import TurboAdam
        return TurboAdam(model.parameters(), lr=lr, weight_decay=weight_decay)
    if kind == "torch-fused":
        return torch.optim.AdamW(model.parameters(), lr=lr, weight_decay=weight_decay, fused=True)
    raise ValueError(kind)


def save_checkpoint(path, model, opt, step, cursor):
    torch.save({"model": model.state_dict(), "opt": opt.state_dict(), "step": step, "cursor": cursor}, path)


def load_checkpoint(path, model, opt):
    ck = torch.load(path, map_location="cpu", weights_only=True)
    model.load_state_dict(ck["model"])
    opt.load_state_dict(ck["opt"])
    return ck["step"], ck["cursor"]


def train(model, opt, tape, steps, base_lr, warmup, device, timer=None):
    """Run `steps` updates; returns the list of losses."""
    losses = []
    for s in range(1, steps + 1):
        for g in opt.param_groups:
            g["lr"] = lr_at(s, base_lr, warmup, steps)
        x, y = tape.next(device)
        loss = model(x, y)
        model.zero_grad(set_to_none=False)
        loss.backward()
        if timer is not None:
            timer.before_opt()
        opt.step()
        if timer is not None:
            timer.after_opt()
        losses.append(loss.detach())
    return [float(l) for l in losses]


def smoke(device="cuda:0", layers=2, seq=128, tmpdir="/tmp"):
    """One synthetic update through the whole loop; raises if a gate fails."""
    import os
    torch.manual_seed(0)
    model = GPT(layers=layers).to(device)
    opt = make_optimizer(model, "e4", lr=1e-3)
    tape = Tape.synthetic(4 * seq + 1, 12096, seed=7)
    tape.batch, tape.seq = 1, seq
    losses = train(model, opt, tape, 1, 1e-3, 0, device)
    with torch.no_grad():
        xv, yv = tape.next(device)
        val = float(model(xv, yv))
    gates = {"finite_train_loss": all(np.isfinite(losses)), "finite_val_loss": bool(np.isfinite(val)),
             "zero_nonfinite": opt.nonfinite_count() == 0,
             "one_word_ledger": opt.state_bytes() == 4 * count_params(model)}
    path = os.path.join(tmpdir, f"pa_smoke_{os.getpid()}.pt")
    save_checkpoint(path, model, opt, 1, tape.cursor)
    model2 = GPT(layers=layers).to(device)
    opt2 = make_optimizer(model2, "e4", lr=1e-3)
    load_checkpoint(path, model2, opt2)
    os.remove(path)
    same = all(torch.equal(a, b) for a, b in zip(model.parameters(), model2.parameters()))
    same &= all(torch.equal(opt.state[a]["words"], opt2.state[b]["words"])
                for a, b in zip(model.parameters(), model2.parameters()))
    gates["checkpoint_round_trip"] = bool(same)
    if not all(gates.values()):
        raise AssertionError(f"smoke gates failed: {gates}")
    return gates, losses, val


class OptTimer:
    """HIP events around each optimizer step, on torch's current stream."""

    def __init__(self):
        self.pairs = []

    def before_opt(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append([e, None])

    def after_opt(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[-1][1] = e

    def mean_ms(self, skip=0):
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) for a, b in self.pairs[skip:]]
        return sum(t) / max(1, len(t))


def measure(kind, steps=30, warmup=5, batch=4, seq=1024, device="cuda:0"):
    """Mean ms of a whole training step and of its optimizer step alone."""
    torch.manual_seed(0)
    model = GPT().to(device)
    opt = make_optimizer(model, kind, lr=1e-3)
    tape = Tape.synthetic((steps + warmup) * batch * seq + 1, 12096, seed=11)
    tape.batch, tape.seq = batch, seq
    timer = OptTimer()
    train(model, opt, tape, warmup, 1e-3, 0, device, timer)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    train(model, opt, tape, steps, 1e-3, 0, device, timer)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"optimizer": kind, "step_ms": round(step_ms, 4), "opt_ms": round(timer.mean_ms(skip=warmup), 4),
            "params": count_params(model), "batch": batch, "seq": seq}
