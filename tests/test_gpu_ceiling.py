"""spkv_hbm_read, the streaming-read kernel behind the measured bandwidth
ceiling: every access order and hint runs to completion on a small buffer and
leaves the sink word alone (the loads are folded, nothing is written)."""
import pytest
import torch

from learned_kv_cache_sp_amd import spkv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("runs", [False, True])
@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("grid", [1, 7, 2048])
def test_hbm_read_runs(runs, nt, grid):
    x = torch.arange((3 << 20) // 4, dtype=torch.int32, device="cuda")   # 3 MiB: 192 blocks of 16 KB
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    spkv.spkv_hbm_read(x, sink, nontemporal=nt, runs=runs, grid=grid)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    assert int(x[-1].item()) == x.numel() - 1
