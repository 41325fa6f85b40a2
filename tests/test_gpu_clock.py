"""The diagnostic shader-clock probe (lilicorr_clock_probe): a plausible clock
with the GPU idle, and a reading taken beside a running linear that overlaps it.
Not part of the reranking path; bench.py --clock-probe reports the same readings."""
import pytest
import torch

import draft_block_candidate_amd as L

pytestmark = pytest.mark.gpu


def _ghz(out):
    v = out.cpu().tolist()
    assert v[0] > 0 and v[1] > 0
    return 0.1 * v[1] / v[0]


def test_clock_probe_idle_window():
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    L.clock_probe(out, 1000)
    torch.cuda.synchronize()
    v = out.cpu().tolist()
    # the window is counted on the 100 MHz constant counter: at least 1,000 us
    assert 100_000 <= v[0] < 100_000 + 50_000
    assert 0.3 < _ghz(out) < 3.0


def test_clock_probe_beside_a_linear():
    dev = torch.device("cuda")
    m, kd, n = 16384, 1024, 4096
    g = torch.Generator(device=dev).manual_seed(1)
    A = (torch.randn((m, kd), device=dev, generator=g) * 0.5).to(torch.bfloat16)
    W = (torch.randn((n, kd), device=dev, generator=g) * 0.03).to(torch.bfloat16)
    L.linear(A, W, None, L.EPI_BF16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    out = torch.zeros(2, dtype=torch.int64, device=dev)
    main = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    ep = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(main)
    side.wait_stream(main)
    with torch.cuda.stream(side):
        L.clock_probe(out, 2000, side)
        ep.record(side)
    for _ in range(60):
        L.linear(A, W, None, L.EPI_BF16)
    e1.record(main)
    torch.cuda.synchronize()
    print(f"[clock] beside linear {m}x{kd}x{n}: {_ghz(out):.3f} GHz; probe ended at "
          f"{e0.elapsed_time(ep):.2f} ms of {e0.elapsed_time(e1):.2f} ms", flush=True)
    assert e0.elapsed_time(ep) < e0.elapsed_time(e1)   # the window lies inside the linears
    assert 0.3 < _ghz(out) < 3.0


def test_clock_probe_rejects_bad_window():
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    with pytest.raises(L.LilicorrError):
        L.clock_probe(out, 0)
    with pytest.raises(L.LilicorrError):
        L.clock_probe(out, 2_000_000)
