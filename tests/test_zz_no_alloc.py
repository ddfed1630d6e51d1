"""The allocation-free forward scan, mssm_selective_scan_fwd_noalloc, through
the C ABI: its outputs against those of the caller-workspace forward,
mssm_selective_scan_fwd_ws, on the same inputs, for two calls in a row (the
second smaller), to the parity bar -- and bit for bit, since both run the same
kernels on the same work split."""
import ctypes

import pytest
import torch

import workloads as W
from tests.gpu_common import DEV, check_out, check_state, np64

pytestmark = pytest.mark.gpu


def _run(entry, d, s, io):
    from selective_state_space_52_amd import _lib
    import selective_state_space_52_amd as m
    L = _lib.lib()
    dims = _lib.Dims(s.batch, s.dim, s.dstate, s.seqlen, io, 0, 0, 1)
    out = torch.full_like(d["u"], float("nan"))
    last = torch.full((s.batch, s.dim, s.dstate), float("nan"), device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    args = [d["u"].data_ptr(), d["delta"].data_ptr(), d["A"].data_ptr(), d["B"].data_ptr(),
            d["C"].data_ptr(), d["D"].data_ptr(), d["z"].data_ptr(),
            d["delta_bias"].data_ptr(), 1, out.data_ptr(), last.data_ptr()]
    if entry == "noalloc":
        rc = L.mssm_selective_scan_fwd_noalloc(*args, ctypes.byref(dims), st)
    else:
        need = m.workspace_size(_lib.MSSM_OP_SCAN_FWD, dims)
        ws = torch.empty(need + 256, dtype=torch.uint8, device=DEV)
        p = ws.data_ptr() + (-ws.data_ptr()) % 256
        rc = L.mssm_selective_scan_fwd_ws(*args, p if need else None, need,
                                          ctypes.byref(dims), st)
    torch.cuda.synchronize()
    assert rc == 0, (entry, rc, L.mssm_last_error().decode())
    return out.cpu(), last.cpu()


# first a shape whose plan cuts rows in time (260 channel
# groups on 256 CUs), then a smaller one on the element-load path
CASES = [("bf16", 5, 3328, 16, 1024), ("f32", 2, 96, 16, 300)]


def test_noalloc_matches_workspace_entry_twice():
    import selective_state_space_52_amd as m
    for io, batch, dim, N, L in CASES:
        print("noalloc case %s batch %d dim %d N %d L %d plan %s" % (
            io, batch, dim, N, L, m.scan_plan(batch, dim, N, L,
                                              torch.bfloat16 if io == "bf16" else torch.float32)),
              flush=True)
        s = W.spec("mamba130m_layer", io=io, batch=batch, dim=dim, dstate=N, seqlen=L,
                   seed=37 + L)
        inp = W.make_scan_inputs(s)
        d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        code = 1 if io == "bf16" else 0
        o_ref, l_ref = _run("ws", d, s, code)
        o_na, l_na = _run("noalloc", d, s, code)
        check_out(o_na, np64(o_ref), io, "noalloc out vs workspace entry",
                  ref_rounded=(io == "bf16"))
        check_state(l_na, np64(l_ref), "noalloc last_state vs workspace entry")
        assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref), "not bit-identical"
