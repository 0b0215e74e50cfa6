"""The measurement kernels (include/fp4idx_ceiling.h) move the traffic they are
said to move: the 1:1 stream copies its source, the mixed stream writes each
write unit once with data it read, the read-only stream leaves its destination
alone, and the paged gather writes exactly the in-context entries of every
logit row (keys s < ctx of each sequence) and nothing past them."""
import numpy as np
import pytest

from pack_token_amd import workloads
from harness import say

pytestmark = pytest.mark.gpu


def test_stream_copy_read_only_and_mix():
    import torch

    from pack_token_amd import fp4idx

    dev = "cuda:0"
    n = 3 << 20
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev)
    say("case ceiling stream: copy, read-only, 3:1 mix")
    dst = torch.zeros(n, dtype=torch.uint8, device=dev)
    fp4idx.ceiling_stream(src, n, dst, n)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    dst = torch.full((4096,), 7, dtype=torch.uint8, device=dev)
    fp4idx.ceiling_stream(src, n, dst, 0)
    torch.cuda.synchronize()
    assert (dst == 7).all()
    w = n // 4
    dst = torch.zeros(w + 1024, dtype=torch.uint8, device=dev)
    fp4idx.ceiling_stream(src, n, dst, w)
    torch.cuda.synchronize()
    # every written 1 KB unit holds some 1 KB unit of the source; nothing past w
    units = src.view(-1, 1024).cpu().numpy()
    got = dst[:w].view(-1, 1024).cpu().numpy()
    known = {u.tobytes() for u in units}
    assert all(g.tobytes() in known for g in got)
    assert (dst[w:] == 0).all()


@pytest.mark.parametrize("stride_pad", [0, 3])
def test_paged_gather_writes_in_context_entries_only(stride_pad):
    import torch

    from pack_token_amd import fp4idx

    dev = "cuda:0"
    sc = workloads.scorer_case(31, 70, 4, 32, 0, 3000)
    sc.block_table[3, 1] = -1                                 # an invalid entry
    stride = sc.max_blocks * 64 + stride_pad
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    logits = torch.full((70 * 4, stride), -7.0, dtype=torch.float32, device=dev)
    say(f"case ceiling paged gather stride={stride}")
    fp4idx.ceiling_paged_gather(t(sc.kv_cache), t(sc.kv_cache_scale), t(sc.block_table),
                                t(sc.context_lens), 4, logits)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    for b in range(70):
        ctx = int(sc.context_lens[b])
        rows = got[4 * b:4 * b + 4]
        assert (rows[:, :ctx] >= 0).all() and np.isfinite(rows[:, :ctx]).all()
        assert (rows[:, ctx:] == -7.0).all()


def _valu_expected(kind, workgroups, iterations):
    """Per-thread results of the fp32 add / max chains (numpy fp32, one rounding
    per operation, as the kernel computes them)."""
    tid = np.arange(workgroups * 256, dtype=np.int64)
    y = np.float32(1.0001)
    r = np.zeros(tid.size, np.uint32)
    for i in range(8):
        f = (tid & 1023).astype(np.float32) * np.float32(0.001) + np.float32(i)
        for _ in range(iterations):
            f = (f + y) if kind == "fp32_add" else np.maximum(f, y)
        u = (tid.astype(np.uint64) * 2654435761 + 0x3F803F80 * i).astype(np.uint32)
        r ^= u ^ f.astype(np.float32).view(np.uint32)
    return r


def test_valu_issue_kernel_runs_its_chains():
    """The issue-rate kernel computes what it claims: the fp32 add and max
    chains match a numpy evaluation, every kind is deterministic, and nothing
    past workgroups * 256 elements is written."""
    import torch

    from pack_token_amd import fp4idx

    wg, it = 4, 37
    for kind in fp4idx.VALU_KINDS:
        say(f"case ceiling valu kind={kind}")
        outs = []
        for _ in range(2):
            out = torch.full((wg * 256 + 64,), -5, dtype=torch.int32, device="cuda:0")
            fp4idx.ceiling_valu(kind, wg, it, out)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
        assert np.array_equal(outs[0], outs[1])
        assert (outs[0][wg * 256:] == -5).all()
        if kind in ("fp32_add", "fp32_max"):
            assert np.array_equal(outs[0][:wg * 256].view(np.uint32), _valu_expected(kind, wg, it))
