"""Run as a script (by tests/test_gpu_graph_first.py, in a process of its own):
the process's very first few-row (16) and tiled (128) MLP calls go straight
into HIP graph capture, with nothing run on the GPU by the library before.
Each captured graph is replayed three times, its output cleared and other
work queued between replays, and every replay must equal an eager call made
afterwards bit for bit and meet the oracle bar.  Prints one line per case and
exits 0 only if all pass."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import torch  # noqa: E402

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_cases import TOL, from_device, generic_case, to_device  # noqa: E402


def main():
    import quantized_decode_mlp_amd as qdm
    torch.cuda.set_device(0)
    ok = True
    # 16 rows: the down projection splits K on the matrix cores; 128 rows: the
    # tiled kernels split K in both projections (few output tiles at this shape)
    for m, bits, group in ((16, 4, 64), (128, 4, 64), (16, 8, 128), (128, 8, 32)):
        d, ffn = 1024, 2048
        ow, (gu, dn) = generic_case((77, m, bits, group), d, ffn, bits, group)
        x = W.generic_act((77, m, 1), (m, d), "bf16")
        r = W.generic_act((77, m, 2), (m, d), "bf16")
        xd, rd = to_device(x), to_device(r)
        ws = torch.empty(qdm.mlp_workspace_bytes(m, qdm.QDM_BF16, gu, dn), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(rd)
        torch.cuda.synchronize()
        print(f"case m={m} bits={bits} group={group} workspace {ws.numel()} B: capturing the first call",
              flush=True)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            qdm.mlp_decode(xd, rd, gu, dn, workspace=ws, out=out)
        replays = []
        for i in range(3):
            out.zero_()
            junk = torch.randn(1 << 20, device="cuda").sum()   # other work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            replays.append(out.clone())
            del junk
        eager = qdm.mlp_decode(xd, rd, gu, dn, workspace=torch.empty_like(ws))
        torch.cuda.synchronize()
        same = all(torch.equal(rp, eager) for rp in replays)
        _, y_ref = oracle.mlp_decode(x.values, r.values, ow.wg, ow.wu, ow.wd)
        err = oracle.scaled_error(from_device(replays[0]), y_ref)
        good = same and err <= TOL["bf16"]
        print(f"  replays bitwise equal to eager: {same}; error vs oracle {err:.3e}: {'ok' if good else 'FAIL'}",
              flush=True)
        ok = ok and good
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
