"""Tail policy of the prompt-tail driver ([cactus] "Fix": short tails stay token by token,
longer ones run as one padded chunk, from the hardware's measured breakeven -- 9 tokens on
the page's M4 Pro, 2 on MI355X; a kill switch forces token by token).  Host logic only."""
import pytest


@pytest.fixture
def path(monkeypatch):
    monkeypatch.delenv("CP_DISABLE_PREFILL_TAIL_PAD", raising=False)
    from chunked_prefill_attention_rope_amd import path as mod
    return mod


def test_default_is_the_mi355x_breakeven(path):
    assert path.PAD_FROM == 2
    assert not path.pad_tail(1)
    assert [path.pad_tail(n) for n in (2, 3, 8, 9, 127)] == [True] * 5


def test_pages_threshold(path):
    # [cactus] review: tails of up to 8 tokens stay token by token on the M4 Pro
    assert path.PAGES_PAD_FROM == 9
    assert [path.pad_tail(n, pad_from=path.PAGES_PAD_FROM) for n in (1, 7, 8)] == [False] * 3
    assert [path.pad_tail(n, pad_from=path.PAGES_PAD_FROM) for n in (9, 10, 127)] == [True] * 3


def test_threshold_is_a_parameter(path):
    assert path.pad_tail(2, pad_from=2) and not path.pad_tail(1, pad_from=2)


@pytest.mark.parametrize("val,forced", [("1", True), ("yes", True), ("0", False), ("", False)])
def test_kill_switch(path, monkeypatch, val, forced):
    monkeypatch.setenv("CP_DISABLE_PREFILL_TAIL_PAD", val)
    assert path.pad_tail(100) is (not forced)


def test_choose_chunk_minimises_total_time(path):
    table = {32: 20.0, 64: 24.0, 128: 30.0, 256: 55.0}
    # 1023 tokens: 32 chunks x 20 = 640, 16 x 24 = 384, 8 x 30 = 240, 4 x 55 = 220
    assert path.choose_chunk(1023, table) == 256
    # 100 tokens: 4 x 20 = 80, 2 x 24 = 48, 1 x 30 = 30, 1 x 55 = 55
    assert path.choose_chunk(100, table) == 128
    # ties go to the smaller chunk
    assert path.choose_chunk(64, {32: 10.0, 64: 20.0}) == 32
    with pytest.raises(ValueError):
        path.choose_chunk(0, table)


def test_balance_policy():
    """Balanced key splits for a batch whose longest past exceeds 1.5x the mean (the
    Llama-8B-like batch), not for equal pasts, one sequence or an empty batch."""
    from chunked_prefill_attention_rope_amd import cp, inputs as I, path
    assert path.attn_flags_for(I.config("c4").seen) == cp.ATTN_BALANCE
    assert path.attn_flags_for(I.config("c5", 5).seen) == 0
    assert path.attn_flags_for([800]) == 0
    assert path.attn_flags_for([]) == 0
    assert path.attn_flags_for([0, 0, 0]) == 0
    assert path.attn_flags_for([100, 100, 100, 140]) == 0     # longest 1.27x the mean
    assert path.attn_flags_for([100, 100, 100, 400]) == cp.ATTN_BALANCE  # 2.29x
    assert path.attn_flags_for([10, 10, 10, 1000]) == cp.ATTN_BALANCE
