"""Token tapes from files (Packed AdamW Reference README, Training on prepared
tapes): a little-endian uint32 token tape and an aligned little-endian
uint16 byte-length tape, read sequentially without wrapping, and bits per
byte against its closed form for a model that predicts every token with
probability 1/V."""
import math
import struct

import numpy as np
import pytest
import torch

from trainer.loop import Tape, bits_per_byte, evaluate


def _write(tmp_path, tokens, lengths):
    tp, bp = tmp_path / "t.tokens.u32", tmp_path / "t.byte-lengths.u16"
    tp.write_bytes(b"".join(struct.pack("<I", int(t)) for t in tokens))
    bp.write_bytes(b"".join(struct.pack("<H", int(b)) for b in lengths))
    return str(tp), str(bp)


def test_tapes_read_little_endian_in_order_and_never_wrap(tmp_path):
    tokens = [0, 1, 70000, 4294967295, 5, 6, 7, 8, 9, 10, 11]
    lengths = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 65535]
    tp, bp = _write(tmp_path, tokens, lengths)
    tape = Tape.from_files(tp, batch=1, seq=4, byte_lengths_path=bp)
    x, y, b = tape.next_with_bytes("cpu")
    assert x.tolist() == [[0, 1, 70000, 4294967295]] and y.tolist() == [[1, 70000, 4294967295, 5]]
    assert b == 2 + 3 + 4 + 5                      # the predicted tokens' bytes
    x, y, b = tape.next_with_bytes("cpu")
    assert x.tolist() == [[5, 6, 7, 8]] and b == 6 + 7 + 8 + 9
    with pytest.raises(RuntimeError):
        tape.next("cpu")                             # 3 tokens left, 5 needed: no wrap
    assert tape.cursor == 8


def test_misaligned_byte_tape_is_refused(tmp_path):
    tp, bp = _write(tmp_path, range(10), range(9))
    with pytest.raises(ValueError):
        Tape.from_files(tp, 1, 4, bp)


def test_bits_per_byte_closed_form(tmp_path):
    """Uniform logits over V classes cost ln V nats per token, so the bits per
    byte are T log2(V) / B for T predicted tokens of B bytes."""
    V, seq, batches = 96, 8, 3
    r = np.random.default_rng(3)
    tokens = r.integers(0, V, seq * batches + 1)
    lengths = r.integers(1, 7, tokens.size)
    tp, bp = _write(tmp_path, tokens, lengths)

    class Uniform(torch.nn.Module):
        def forward(self, x, y):
            logits = torch.zeros(x.shape + (V,), dtype=torch.float64)
            return torch.nn.functional.cross_entropy(logits.view(-1, V), y.reshape(-1))

    mean, bpb = evaluate(Uniform(), Tape.from_files(tp, 1, seq, bp), batches, "cpu")
    T, B = seq * batches, int(lengths[1:seq * batches + 1].sum())
    assert abs(mean - math.log(V)) < 1e-12
    assert abs(bpb - T * math.log2(V) / B) < 1e-12
    assert bits_per_byte(math.log(2.0) * 10, 5) == pytest.approx(2.0)
    mean2, none = evaluate(Uniform(), Tape.from_files(tp, 1, seq), 1, "cpu")
    assert none is None and abs(mean2 - math.log(V)) < 1e-12
