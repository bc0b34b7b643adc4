"""Cross-XCD message passing with the handshake every role uses (write-through payload, then a
relaxed agent-scope flag; the consumer polls the flag, then reads).  64 producer/consumer pairs
on different XCDs exchange thousands of payloads.

* fresh payload addresses + ordinary loads (what the kernels do: each payload is written once per
  launch and never read before its flag) must never mismatch;
* reused addresses + device-coherent loads must never mismatch;
* reused addresses + ordinary loads is only reported: another XCD's L2 may keep a stale copy of a
  rewritten line, which is why no kernel re-reads an address rewritten within the launch;
* fresh addresses over the load paths the kernels take must never mismatch: the compute role's
  buffer loads straight into LDS, the copy role's non-temporal loads into LDS followed by
  write-through stores, and the MoE counter handshake (atomic increment, count wait).
"""
import pytest

pytestmark = pytest.mark.gpu


def _mk():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import communication_gemm_role_amd as mk
    return mk


def test_fresh_addresses_plain_loads():
    mk = _mk()
    mismatches, timeouts = mk.mk_selftest_flags(0, mode=0, pairs=64, rounds=4096)
    assert timeouts == 0 and mismatches == 0


def test_reused_addresses_coherent_loads():
    mk = _mk()
    mismatches, timeouts = mk.mk_selftest_flags(0, mode=1, pairs=64, rounds=20000)
    assert timeouts == 0 and mismatches == 0


@pytest.mark.parametrize("mode,what", [(3, "consumer reads by buffer load into LDS (compute role operands)"),
                                       (4, "producer lands by non-temporal DMA + write-through stores (copy role)"),
                                       (5, "counter increment and count wait, then LDS load (MoE m-tiles)")])
def test_fresh_addresses_kernel_load_paths(mode, what):
    mk = _mk()
    mismatches, timeouts = mk.mk_selftest_flags(0, mode=mode, pairs=64, rounds=2048)
    assert timeouts == 0 and mismatches == 0, what


def test_reused_addresses_plain_loads_is_reported(capsys):
    mk = _mk()
    mismatches, timeouts = mk.mk_selftest_flags(0, mode=2, pairs=64, rounds=4096)
    assert timeouts == 0
    print(f"reused addresses with ordinary loads: {mismatches} stale payload words (diagnostic)")


def test_selftest_rejects_bad_arguments():
    mk = _mk()
    for kw in (dict(mode=6), dict(mode=-1), dict(pairs=0), dict(pairs=129), dict(rounds=0),
               dict(mode=0, pairs=128, rounds=4096), dict(mode=4, pairs=128, rounds=2048)):
        with pytest.raises(mk.MkError):
            mk.mk_selftest_flags(0, **kw)
