"""The reference decoder against its pins (CPU only)."""

import pytest

from oracle import decoder

from . import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(decoder)


def test_generate_matches_teacher_forced_steps():
    """generate() feeds its own greedy tokens back: replaying them step by step gives the same logits."""
    import numpy as np

    shape = oracle_pins.MICRO_GQA
    w = oracle_pins.micro_weights(shape, seed=31)
    prompt = [3, 1, 4, 1, 5]
    o = decoder.Oracle(shape, w, batch=1, max_seq=12)
    toks, logits = o.generate(prompt, 6)
    assert toks.shape == (6,) and logits.shape == (6, shape.vocab)
    o2 = decoder.Oracle(shape, w, batch=1, max_seq=12)
    feed = list(prompt) + list(toks[:-1])
    replay = [o2.step_one(0, int(t), p) for p, t in enumerate(feed)]
    for i in range(6):
        assert np.array_equal(replay[len(prompt) - 1 + i], logits[i])
        assert decoder.greedy_token(replay[len(prompt) - 1 + i][None])[0] == toks[i]


def test_step_rejects_bad_inputs():
    shape = oracle_pins.MICRO_GQA
    w = oracle_pins.micro_weights(shape)
    o = decoder.Oracle(shape, w, batch=1, max_seq=4)
    with pytest.raises(ValueError):
        o.step_one(0, shape.vocab, 0)
    with pytest.raises(ValueError):
        o.step_one(0, 0, 4)
    with pytest.raises(ValueError):
        decoder.greedy_token([[float("nan"), 1.0]])
