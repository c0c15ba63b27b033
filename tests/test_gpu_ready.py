"""GPU tests of the readiness words and the wait kernel.

With publishing on, the fused kernel runs its tiles destination by destination
and releases each destination's stores before counting them in that
destination's readiness word; a consumer stream that waits on the word may read
the destination's receive slot while the producer is still running.  The
results must not change (parity with the oracle), the words must reach the
values the session expects, work ordered only by a wait must see complete
data, and a wait that cannot be satisfied must end by counting a timeout.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import check_fp, to_bits
from test_gpu_fused import (SMALL, Inputs, check_coverage, check_full, check_whole_slots,
                            make_session, run, sample_tokens)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_publishing_keeps_results(gpu_lib, wl):
    """Whole slots with publishing on (destination-major tile order where the
    band is a whole number of tiles, the plain order otherwise)."""
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    sess.set_publish(True)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_full(views, inp, wl.rank, wl.name + ":publish")
    words, timeouts = sess.ready_state()
    assert words == sess.ready_expected() and timeouts == 0
    assert '"publish": true' in sess.describe()


def test_words_accumulate_over_calls(gpu_lib):
    wl = SMALL[0]
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    sess.set_publish(True)
    per_call = ((wl.tokens + 255) // 256) * 6 * wl.local_heads
    for call in range(3):
        run(sess, inp)
        torch.cuda.synchronize()
        words, _ = sess.ready_state()
        assert words == [per_call * (call + 1)] * wl.world
    sess.set_publish(False)                      # a plain call leaves the words alone
    run(sess, inp)
    torch.cuda.synchronize()
    assert sess.ready_state()[0] == [per_call * 3] * wl.world


def test_full_size_publishing_whole_slots(gpu_lib):
    """The publishing launch at full size (destination-major tile order over
    248 compute units, claimed per XCD): every element of every destination's
    slot against the oracle, the other ranks' rows untouched, and the words at
    their expected values."""
    wl = W.WORKLOADS["h56_u4"]
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    sess.set_publish(True)
    sess.poison_receive_slots()
    views = run(sess, inp)
    torch.cuda.synchronize()
    check_coverage(views, wl, wl.rank, "h56_u4:publish")
    check_whole_slots(views, inp, wl.rank, "h56_u4:publish")
    assert sess.ready_state() == (sess.ready_expected(), 0)


def test_consumer_streams_see_complete_destinations(gpu_lib):
    """The producer runs on one stream; each destination's consumer stream
    waits on its readiness word only (no event joins the streams) and then
    copies that destination's q, k and v rows of this rank.  Every copy must
    equal the oracle's values: a consumer that ran early would read the poison
    pattern the slots start with."""
    wl = W.WORKLOADS["h56_u4"]
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    sess.set_publish(True)
    sess.poison_receive_slots()
    torch.cuda.synchronize()
    producer = torch.cuda.Stream()
    consumers = [torch.cuda.Stream() for _ in range(wl.world)]
    r0, r1 = wl.rank * wl.s_local, (wl.rank + 1) * wl.s_local
    with torch.cuda.stream(producer):
        views = run(sess, inp)
    copies = []
    for d, cs in enumerate(consumers):
        sess.wait_ready(d, stream=cs)
        with torch.cuda.stream(cs):
            copies.append([views[d][p][:, r0:r1].clone() for p in range(3)])
    torch.cuda.synchronize()
    assert sess.ready_state()[1] == 0, "a wait timed out"
    tokens = sample_tokens(wl, n=16)
    vals = O.front_end_rows(inp.x.reshape(wl.tokens, wl.hidden)[tokens], inp.w, inp.wq,
                            inp.wk, inp.cs[wl.rank * wl.s_local + tokens % wl.s_local],
                            wl.heads)
    hl = wl.local_heads
    for d in range(wl.world):
        for p in range(3):
            got = to_bits(copies[d][p])                          # [B, S_local, hl, 128]
            assert not np.any(got == O.POISON_BITS), f"dest {d} part {p}: unwritten rows"
            g = got.reshape(wl.tokens, hl, 128)[tokens]
            check_fp(g, vals[:, p, d * hl:(d + 1) * hl], f"consumer d{d} p{p}")


def test_wait_word_times_out_and_returns(gpu_lib):
    """A wait that cannot be satisfied (the word stays 0) ends after its spin
    limit and counts one timeout; a satisfied one counts none."""
    word = torch.zeros(1, dtype=torch.int64, device="cuda")
    timeouts = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.qkvx_wait_word(word, 1, timeouts, spin_limit=4)
    torch.cuda.synchronize()
    assert int(timeouts.item()) == 1
    word.fill_(5)
    gpu_lib.qkvx_wait_word(word, 5, timeouts, spin_limit=0)
    gpu_lib.qkvx_wait_word(word, 3, timeouts, spin_limit=0)
    torch.cuda.synchronize()
    assert int(timeouts.item()) == 1


def test_wait_ready_needs_a_publishing_call(gpu_lib):
    wl = SMALL[0]
    inp = Inputs(wl)
    sess = make_session(gpu_lib, wl)
    run(sess, inp)
    with pytest.raises(ValueError):
        sess.wait_ready(0)
    sess.set_publish(True)
    run(sess, inp)
    with pytest.raises(ValueError):
        sess.wait_ready(wl.world)
    sess.wait_ready(wl.world - 1)
    torch.cuda.synchronize()
    assert sess.ready_state()[1] == 0
