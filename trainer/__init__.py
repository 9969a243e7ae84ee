"""A small learned-position GPT trained on synthetic token tapes with the
packed-AdamW step: the steps on either side of the optimizer update
(ordinary PyTorch forward and backward, checkpoints), used to exercise the
optimizer end to end and to measure its share of a training step.

There is no real data here: tokens come from a seeded generator, so losses
say nothing about learning (Packed AdamW Reference README, one-update smoke
test: synthetic loss is not a learning benchmark).
"""
