"""Tail policy of the prompt-tail driver ([cactus] "Fix": tails of up to 8 tokens stay
token by token, padding from 9; a kill switch forces token by token).  Host logic only."""
import pytest


@pytest.fixture
def path(monkeypatch):
    monkeypatch.delenv("CP_DISABLE_PREFILL_TAIL_PAD", raising=False)
    from chunked_prefill_attention_rope_amd import path as mod
    return mod


def test_pad_from_nine(path):
    assert path.PAD_FROM == 9
    assert [path.pad_tail(n) for n in (1, 7, 8)] == [False, False, False]
    assert [path.pad_tail(n) for n in (9, 10, 127)] == [True, True, True]


def test_threshold_is_a_parameter(path):
    assert path.pad_tail(2, pad_from=2) and not path.pad_tail(1, pad_from=2)


@pytest.mark.parametrize("val,forced", [("1", True), ("yes", True), ("0", False), ("", False)])
def test_kill_switch(path, monkeypatch, val, forced):
    monkeypatch.setenv("CP_DISABLE_PREFILL_TAIL_PAD", val)
    assert path.pad_tail(100) is (not forced)
