"""pa_forward_noalloc, the entry point for callers that cannot allocate:
through the C ABI, its output against pa_forward's on the same inputs, to
the 2e-3 max-abs bar, on two calls in a row, the second with a smaller input
(the scratch array still holds the first call's partials and work list)."""
import numpy as np
import pytest

from paged_kv_cache_append_amd import workloads as wl

from pa_harness import TOL, attn_for, gpu_append, max_err

pytestmark = pytest.mark.gpu


def _both(w):
    """(pa_forward output, pa_forward_noalloc output) on the same appended pools."""
    import torch
    import paged_kv_cache_append_amd as pa
    dev = wl.to_device(w)
    gpu_append(w, dev)
    a = attn_for(w)
    args = (dev["query"], dev["key_cache"], dev["value_cache"], dev["block_table"], dev["cum"],
            dev["past"], dev["cos"], dev["sin"])
    ref = pa.forward(a, *args)
    out = torch.full_like(ref, float("nan"))
    pa.forward_noalloc(a, *args, out=out)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


def test_noalloc_matches_forward_on_two_calls_the_second_smaller():
    first = wl.scaled_down("llama3_8b_mixed")            # decode splits beside prefill tiles
    second = wl.scaled_down("long_context_decode_rope")   # fewer tokens, rotary, more splits
    assert second.token_count < first.token_count
    for w in (first, second):
        print(f"\n[noalloc] {w.name} T={w.token_count} B={w.batch_size}", flush=True)
        ref, out = _both(w)
        err = max_err(out, ref.astype(np.float64))
        same = out.tobytes() == ref.tobytes()
        print(f"[noalloc] max_abs_err vs pa_forward={err:.3e} bit-identical={same}", flush=True)
        assert err <= TOL, err
