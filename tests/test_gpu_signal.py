"""GPU test of the inter-partition signal probe (moe_signal_probe): every hand-off
completes within its wait budget; with agent-scope release/acquire no consumer ever reads
a stale payload word, on one XCD or across XCDs; with the L2-local hand-off the same holds
for partners that share an XCD.  Latencies are printed (the bench's --signal-latency mode
reports them)."""
import sys

import pytest

from mixture_experts_layer_histogram_amd import moe

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cross,scope,words", [(0, 0, 16384), (0, 0, 1024), (0, 1, 16384), (0, 1, 1024),
                                               (1, 1, 16384), (1, 0, 16384)],
                         ids=["same-xcd-l2", "same-xcd-l2-4KiB", "same-xcd-agent", "same-xcd-agent-4KiB",
                              "cross-xcd-agent", "cross-xcd-l2"])
def test_signal_probe(cross, scope, words):
    """A 4 KiB payload stays in the consumer CU's L1 from one round to the next, so it
    catches an acquire that does not invalidate the L1 (a 64 KiB payload evicts itself)."""
    import torch
    rounds = 200
    _say(f"[signal] cross_xcd={cross} scope={scope} payload={words * 4} B rounds={rounds}")
    scratch = torch.empty(moe.moe_signal_probe_bytes(words), dtype=torch.uint8, device="cuda:0")
    rc, us, stale, tmo, same = moe.moe_signal_probe(cross, scope, words, rounds, scratch, check=False)
    _say(f"  rc={rc} {us:.2f} us/round, stale words {stale}, timeouts {tmo}, pairs on one XCD {same}/128")
    assert rc == 0 and tmo == 0
    assert us > 0
    if scope == 1:
        assert stale == 0
    if scope == 0 and same == 128:
        assert stale == 0


def test_signal_probe_consumer_l1():
    """Same-XCD hand-off of a 4 KiB payload, which stays in the consumer CU's L1 between
    rounds: a workgroup-scope invalidate (buffer_inv sc0) leaves it there and the consumer
    reads stale words; device-coherent sc1 loads without any invalidate read none (the
    persistent kernel's form)."""
    import torch
    words, rounds = 1024, 200
    scratch = torch.empty(moe.moe_signal_probe_bytes(words), dtype=torch.uint8, device="cuda:0")
    res = {}
    for scope in (2, 3):
        rc, us, stale, tmo, same = moe.moe_signal_probe(0, scope, words, rounds, scratch, check=False)
        _say(f"[signal] 4 KiB same XCD, consumer form {scope}: {us:.2f} us/round, stale words {stale}")
        assert rc == 0 and tmo == 0 and same == 128
        res[scope] = stale
    assert res[2] > 0
    assert res[3] == 0


def test_signal_probe_without_payload():
    import torch
    scratch = torch.empty(moe.moe_signal_probe_bytes(0), dtype=torch.uint8, device="cuda:0")
    for cross in (0, 1):
        rc, us, stale, tmo, same = moe.moe_signal_probe(cross, 1, 0, 500, scratch, check=False)
        _say(f"[signal] flag only, cross_xcd={cross}: {us:.2f} us/round")
        assert rc == 0 and tmo == 0 and stale == 0
