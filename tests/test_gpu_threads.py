"""Host threads calling the library at once, each on its own stream (default
priority), with plans shared across threads: results equal single-threaded
calls bitwise.  The library's host state is per-call apart from per-device
caches guarded by a mutex and a thread-local error string."""
import threading

import pytest
import torch

from gpu_util import device_qkv, say

pytestmark = pytest.mark.gpu

import block_sparse_attention_lcsa_amd as lcsa  # noqa: E402  (fails loudly if not built)


def test_threads_on_separate_streams():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say("[gpu] start threads on separate streams")
    cases = {}
    for name in ("small_edges", "tiny", "small_16x8"):
        desc, q, k, v = device_qkv(name)
        plan = lcsa.Plan.from_desc(desc)
        rp, ci = lcsa.select(plan, q, k)
        o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
        cases[name] = (plan, q, k, v, ci.clone(), o.clone(), lse.clone())
    torch.cuda.synchronize()

    errors = []

    def worker(name, reps=15):
        plan, q, k, v, ci_ref, o_ref, lse_ref = cases[name]
        stream = torch.cuda.Stream()
        try:
            with torch.cuda.stream(stream):
                for _ in range(reps):
                    rp, ci = lcsa.select(plan, q, k)
                    o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
                    stream.synchronize()
                    if not (torch.equal(ci, ci_ref) and torch.equal(o, o_ref) and torch.equal(lse, lse_ref)):
                        errors.append(f"{name}: result differs")
                        return
        except Exception as e:  # noqa: BLE001
            errors.append(f"{name}: {e!r}")

    threads = [threading.Thread(target=worker, args=(n,)) for n in list(cases) * 2]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    say("[gpu] done  threads on separate streams: 6 threads x 15 calls, bitwise equal")
