"""The entry point that allocates nothing (ocq_mlp_forward_noalloc) against
the workspace entry point (ocq_mlp_forward), through the C ABI.

Both run the same kernels; the no-allocation call takes its workspace from
the library's fixed per-device scratch array, so its outputs (y and every
tap) must equal the workspace call's bit for bit.  Two calls in a row reuse
the array, the second with fewer rows (what the first left in the array
must not leak into the second).  A call whose workspace would exceed the
array is rejected before any launch.
"""

import numpy as np
import pytest

from oracle import mlp as O
from quantized_memory_bound_amd import inputs as I
from quantized_memory_bound_amd import ocq
from parity import check_y

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ocq.lib()


def _taps(M, H, Iw, prec):
    return {"x_codes": torch.empty((M, H), dtype=torch.uint8, device="cuda"),
            "x_scales": torch.empty(M, dtype=torch.float32, device="cuda"),
            "h_out": torch.empty((M, Iw), dtype=torch.int16 if prec == O.PREC_FP8_DOWN_BF16 else torch.uint8,
                                 device="cuda"),
            "h_scales": torch.empty(M, dtype=torch.float32, device="cuda")}


def _host(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("H,Iw,n,prec", [(2048, 6144, 208, 0), (512, 1024, 420, 1), (4096, 12288, 52, 2)])
def test_noalloc_matches_workspace_entry_point(H, Iw, n, prec):
    print("case noalloc hidden=%d inter=%d M=%d then 13 prec=%d" % (H, Iw, n, prec), flush=True)
    d = I.make_inputs(H, Iw, n, x_outliers=True, w_std=0.02, seed=H + n + prec)
    blob = ocq.pack_weights(d["w_gate"], d["w_up"], d["w_down"], prec)
    for M in (n, 13):                                  # second call with fewer rows
        xb = np.ascontiguousarray(d["x_bits"][:M])
        x = torch.from_numpy(xb.view(np.int16)).to("cuda").view(torch.bfloat16)
        t_ref, t_na = _taps(M, H, Iw, prec), _taps(M, H, Iw, prec)
        y_ref = ocq.mlp_forward(blob, x, H, Iw, prec, taps=t_ref)
        y_na = ocq.mlp_forward_noalloc(blob, x, H, Iw, prec, taps=t_na)
        torch.cuda.synchronize()
        assert np.array_equal(_host(y_na), _host(y_ref)), "y differs (M=%d)" % M
        for k in t_ref:
            if prec == O.PREC_FP8_DOWN_BF16 and k == "h_scales":
                continue                               # untouched in the BF16-down mode
            assert np.array_equal(_host(t_na[k]), _host(t_ref[k])), "%s differs (M=%d)" % (k, M)
        if M == 13:
            r = O.block_reference(xb, d["w_gate"], d["w_up"], d["w_down"], prec)
            check_y(_host(y_na).view(np.uint16), r["y"], "noalloc y against the oracle")


def test_noalloc_rejects_oversize_call():
    H, Iw, M = 4096, 12288, 8192
    assert ocq.workspace_bytes(M, H, Iw, 1) > ocq.noalloc_scratch_bytes()
    x = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    blob = torch.zeros(ocq.packed_bytes(H, Iw, 1), dtype=torch.uint8, device="cuda")
    with pytest.raises(ocq.OcqError) as e:
        ocq.mlp_forward_noalloc(blob, x, H, Iw, 1)
    assert e.value.status == ocq.ERR_BUFFER_TOO_SMALL and "no-allocation" in str(e.value)
