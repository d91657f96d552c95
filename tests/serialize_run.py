"""Child process of tests/test_gpu_serialize.py: runs a fixed sequence of
paged-layer steps whose streams could race (host-driven decode on three
streams, a host-driven stack with lookahead, a device-resolved stack with
lookahead on a copy stream) and saves every output, plan and table state to
an .npz file. The test runs it twice, once with the HIP runtime serialising
every kernel and copy, and compares the two files."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import expert_weight_paging_amd as ewp  # noqa: E402
import workloads as W  # noqa: E402
from workloads import gen  # noqa: E402
from stack_check import StackPair  # noqa: E402


def main(path):
    res = {}
    cfg = W.CONFIGS[2]
    rec = ewp.record_bytes(cfg.fmt, cfg.H, cfg.I)
    host = ewp.HostStore(cfg.E, rec)
    gen.expert_store(cfg, out=host.array)
    s = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
    slots, state = ewp.alloc_layer_buffers(cfg.E, cfg.K, rec, "cuda")
    L = ewp.Layer(cfg.E, cfg.top_k, cfg.H, cfg.I, cfg.K, cfg.fmt, host, slots, state, *s)
    P = ewp.Plan(L, 1)
    logits, x = gen.decode_inputs(cfg, 1, steps=12)
    lg = torch.from_numpy(logits).cuda()
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    out = torch.empty(1, cfg.H, dtype=torch.float32, device="cuda")
    for t in range(12):
        L.step(P, lg[t], xd[t], out)
        torch.cuda.synchronize()
        res["decode_out_%d" % t] = out.cpu().numpy()
        for n, v in zip(("ids", "w", "sid", "wave"), P.read()):
            res["decode_%s_%d" % (n, t)] = v
        for n, v in zip(("se", "es", "st", "clk"), L.get_state()):
            res["decode_%s_%d" % (n, t)] = np.asarray(v)
    P.close()
    L.close()
    host.free()
    cfg = W.CONFIGS[4]
    for mode in ("host", "device"):
        c = torch.cuda.Stream()
        A = StackPair(cfg, 4, 1, False, (c, torch.cuda.Stream(), c if mode == "device" else torch.cuda.Stream()),
                      keep_refs=False)
        lgs, x0 = gen.stack_inputs(cfg, steps=6)
        for t in range(6):
            xx = torch.from_numpy(np.ascontiguousarray(x0[t]).view(np.int16)).cuda()
            o = torch.empty(1, cfg.H, dtype=torch.float32, device="cuda")
            lgt = torch.from_numpy(np.ascontiguousarray(lgs[t][:4])).cuda()
            torch.cuda.synchronize()
            if mode == "host":
                ewp.stack_forward(A.layers, A.plans, lgt, xx, o, lookahead=True)
            else:
                ewp.stack_forward_device(A.layers, A.plans, lgt, xx, o, lookahead=True)
            torch.cuda.synchronize()
            res["%s_x_%d" % (mode, t)] = xx.cpu().numpy()
            res["%s_out_%d" % (mode, t)] = o.cpu().numpy()
            for l in range(4):
                for n, v in zip(("ids", "w", "sid", "wave"), A.plans[l].read()):
                    res["%s_%s_%d_%d" % (mode, n, t, l)] = v
                for n, v in zip(("se", "es", "st", "clk"), A.layers[l].get_state()):
                    res["%s_%s_%d_%d" % (mode, n, t, l)] = np.asarray(v)
        A.close()
    np.savez(path, **res)
    print("saved %d arrays" % len(res), flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
