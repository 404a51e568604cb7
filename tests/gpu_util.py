"""Helpers shared by the GPU tests: build a case on the device, run the HIP
path through the C ABI, and copy what the oracle needs back to the host."""
import sys

import numpy as np
import torch

import kv_cache_quantization_kvarn_amd as kv
import oracle
from synth.cases import WORKLOADS, make_case


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch.device("cuda:0")


def workload(name, **over):
    w = dict(WORKLOADS[name])
    w.update(over)
    return w


def gpu_case(w, **kw):
    return make_case(w, device=device(), **kw)


def alloc_records(case):
    lay = case["layout"]
    L = kv.layout_from_dict(lay)
    nq = max(case["n_qpages"], 1)
    H = lay["H"]
    krec = torch.zeros((nq, H, kv.record_bytes(L, 0)), dtype=torch.uint8, device=device())
    vrec = None if lay["mla"] else torch.zeros((nq, H, kv.record_bytes(L, 1)), dtype=torch.uint8,
                                               device=device())
    return L, krec, vrec


def run_quantize(case):
    L, krec, vrec = alloc_records(case)
    kv.quantize(L, case["k16"], case["v16"], krec, vrec, case["src"], case["dst"])
    torch.cuda.synchronize()
    return L, krec, vrec


def run_decode(case, L, krec, vrec):
    out = kv.decode_attn(L, krec, vrec, case["k16"], case["v16"], case["block_table"], case["seq_lens"],
                         case["q"], case["sm_scale"])
    torch.cuda.synchronize()
    return out


def host_u16(t):
    return None if t is None else t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_q(q):
    """Queries for the oracle: bfloat16 bits, or float32 (fp16 queries are
    widened to float32, which holds every fp16 value exactly)."""
    if q.dtype == torch.bfloat16:
        return q.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return q.cpu().float().numpy()


def oracle_decode(case, krec, vrec, pairs=None, k16=None, v16=None):
    k16 = host_u16(case["k16"]) if k16 is None else k16
    v16 = host_u16(case["v16"]) if v16 is None else v16
    kr = krec.cpu().numpy()
    vr = None if vrec is None else vrec.cpu().numpy()
    return oracle.decode(case["layout"], kr, vr, k16, v16, case["block_table"].cpu().numpy(),
                         case["seq_lens"].cpu().numpy(), host_q(case["q"]), case["Hq"], case["sm_scale"],
                         pairs=pairs)
