"""Child process of test_gpu_threads.py: four threads make their first library
calls at once, each stepping its own tensors on its own stream; then the same
steps run one after another; prints "same" when every result matches bit for bit."""
import os
import sys
import threading

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import matrix_optimizer_muon_amd as mm  # noqa: E402
from matrix_optimizer_muon_amd.workloads import make_custom  # noqa: E402


def inputs(k):
    tds = [make_custom((600, 1000), "bf16", seed=(93, 2 * k), scale=1e-3),
           make_custom((2, 520, 300), "f32", seed=(93, 2 * k + 1))]
    out = []
    for td in tds:
        g = (torch.from_numpy(td.grad_bits.view(np.int16).copy()).view(torch.bfloat16)
             if td.grad_bits is not None else torch.from_numpy(td.grad.copy()))
        out.append((g.cuda(), torch.from_numpy(td.momentum.copy()).cuda(), torch.from_numpy(td.master.copy()).cuda(),
                    torch.empty(td.grad.shape, dtype=torch.float32, device="cuda")))
    return out


def run(devs, precision, stream):
    mm.muon_step([d[0] for d in devs], [d[1] for d in devs], [d[2] for d in devs], ns_outs=[d[3] for d in devs],
                 precision=precision, stream=stream)


def main():
    torch.cuda.init()
    precisions = ["bf16", "f32", "bf16", "f32"]
    sets = [inputs(k) for k in range(4)]
    streams = [torch.cuda.Stream() for _ in range(4)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    start = threading.Barrier(4)
    errors = []

    def worker(k):
        try:
            start.wait()
            run(sets[k], precisions[k], streams[k])
        except Exception as exc:          # reported by the parent
            errors.append(repr(exc))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    if errors:
        print("errors", errors)
        return 1
    for k in range(4):
        ref = inputs(k)
        run(ref, precisions[k], torch.cuda.current_stream())
        torch.cuda.synchronize()
        for d, r in zip(sets[k], ref):
            for i in (1, 2, 3):
                if not torch.equal(d[i], r[i]):
                    print("differs", k, i)
                    return 1
    print("same")
    return 0


if __name__ == "__main__":
    sys.exit(main())
