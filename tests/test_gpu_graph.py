"""A whole step (append + forward) captured into a HIP graph replays to the
eager result, bit for bit, on a mixed prefill + decode batch and on a
prefill-only batch: the step records no memsets and reads nothing back to the
host, and the second stream that runs the prefill beside the decode joins the
capture through its fork event.  Each replay follows eager work and a
synchronisation, and every replay is checked."""
import numpy as np
import pytest

from paged_kv_cache_append_amd import workloads as wl

from pa_harness import TOL, attn_for, max_err, oracle_append, oracle_forward

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["llama3_8b_mixed", "gemma2_prefill_window", "long_context_decode_rope"])
def test_graph_replay_matches_eager(name):
    import torch

    import paged_kv_cache_append_amd as pa
    w = wl.scaled_down(name)
    print(f"\n[case] graph {w.name} B={w.batch_size} T={w.token_count} D={w.head_size}", flush=True)
    dev = wl.to_device(w)
    a = attn_for(w)
    T, HD = w.token_count, w.num_heads * w.head_size
    args = (dev["key_cache"], dev["value_cache"], dev["block_table"], dev["cum"], dev["past"])
    need = pa.forward_workspace_bytes(a, *args, T)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def step(out):
        pa.append_kv(a, dev["key"], dev["value"], *args, dev["cos"], dev["sin"])
        pa.forward(a, dev["query"], *args, dev["cos"], dev["sin"], workspace=ws, out=out)

    out_e = torch.empty((T, HD), dtype=torch.float16, device="cuda")
    step(out_e)
    torch.cuda.synchronize()
    eager = out_e.cpu().numpy()
    nk, nv = oracle_append(w)
    assert max_err(eager, oracle_forward(w, nk, nv)) <= TOL

    out_g = torch.empty_like(out_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out_g)   # warm-up on the capturing stream's kind of stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out_g)
    for rep in range(3):
        out_g.fill_(float("nan"))            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_g.cpu().numpy()
        print(f"[case] replay {rep}", flush=True)
        assert got.tobytes() == eager.tobytes(), f"replay {rep} differs from the eager step"
    assert dev["key_cache"].cpu().numpy().tobytes() == nk.tobytes()
    assert dev["value_cache"].cpu().numpy().tobytes() == nv.tobytes()
