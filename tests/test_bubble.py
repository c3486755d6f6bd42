"""The pipeline-bubble arithmetic behind the LAMB batch argument, pinned to
an event-by-event replay of the 1F1B and interleaved-1F1B schedules (the
closed form (p - 1) / (v m) is not used by the replay), plus the pages'
printed comparison of 4 steps at 1x against 1 step at 4x."""
import pytest

from transformer_block_lamb_amd import bubble as Bb


@pytest.mark.parametrize("p,m,v", [(2, 2, 1), (4, 4, 1), (4, 9, 1), (8, 16, 1), (8, 64, 1),
                                   (2, 4, 2), (4, 8, 2), (8, 16, 2), (8, 32, 4), (4, 12, 3)])
@pytest.mark.parametrize("f,b", [(1.0, 2.0), (1.0, 1.0)])
def test_replay_matches_closed_form(p, m, v, f, b):
    r = Bb.simulate_1f1b(p, m, v, f, b)
    t = f + b
    for idle in r["idle"]:
        assert idle == pytest.approx(Bb.bubble_time(p, v, t), abs=1e-9)
    assert r["makespan"] == pytest.approx(m * t + Bb.bubble_time(p, v, t), abs=1e-9)
    assert (r["makespan"] - m * t) / (m * t) == pytest.approx(Bb.bubble_fraction(p, m, v))


def test_single_stage_has_no_bubble():
    assert Bb.simulate_1f1b(1, 5)["idle"] == [0.0]
    assert Bb.bubble_fraction(1, 5) == 0.0


def test_interleaving_needs_whole_groups():
    with pytest.raises(ValueError):
        Bb.simulate_1f1b(4, 6, 2)


def test_page_comparison_readings():
    """p = 8 (the 175B pipeline depth on the pages): one step at 4x against
    four at 1x.  Same tokens: 1/4 of the idle time.  The pages' printed pair
    4/v (p-1)/m against 1/v (p-1)/(4m): 1/16 (93.75 % fewer), not the quoted
    87.5 %; the production 3x batch gives 1/9 under the same reading."""
    for v in (1, 2, 3):
        r4 = Bb.lamb_batch_comparison(8, v, 16, 4)
        assert r4["same_tokens_time"] == pytest.approx(0.25)
        assert r4["fraction"] == pytest.approx(0.25)
        assert r4["literal_page"] == pytest.approx(1 / 16)
        assert r4["literal_page_reduction"] == pytest.approx(0.9375)
        r3 = Bb.lamb_batch_comparison(8, v, 16, 3)
        assert r3["literal_page"] == pytest.approx(1 / 9)
