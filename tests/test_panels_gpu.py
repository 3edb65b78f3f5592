"""The 16-row panel copies of the projection weights (m2_pack_panels through the C ABI):
every byte of the packed copy against the layout the header defines, rebuilt here with
numpy index arithmetic, for bf16 and int8 matrices whose rows and K are not multiples of
the 16-row panel or the 32-wide k-step."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def expected_panels(w: np.ndarray) -> np.ndarray:
    """Panel p, k-step s, fragment l holds row 16p + l%16, columns 32s + 8(l//16) .. +7, zero
    past the matrix; fragments in (p, s, l) order."""
    rows, k = w.shape
    npan, nks = -(-rows // 16), -(-k // 32)
    pad = np.zeros((npan * 16, nks * 32), w.dtype)
    pad[:rows, :k] = w
    out = np.empty((npan, nks, 64, 8), w.dtype)
    for lane in range(64):
        r = lane % 16
        c = 8 * (lane // 16)
        for s in range(nks):
            out[:, s, lane, :] = pad[r::16, 32 * s + c: 32 * s + c + 8]
    return out.reshape(-1)


@pytest.mark.parametrize("wtype,rows,k", [("bf16", 37, 100), ("bf16", 16, 32), ("bf16", 130, 4480),
                                           ("int8g", 37, 100), ("int8g", 908, 384)])
def test_pack_panels_layout(wtype, rows, k):
    import torch
    from full_duplex_speech_mamba2_amd import m2
    rng = np.random.default_rng(rows * 7 + k)
    if wtype == "bf16":
        w = rng.integers(0, 1 << 16, size=(rows, k), dtype=np.uint16)
        wd = torch.from_numpy(w.view(np.int16)).cuda()
    else:
        w = rng.integers(-127, 128, size=(rows, k), dtype=np.int8)
        wd = torch.from_numpy(w).cuda()
    assert m2.panels_bytes(wtype, rows, k) == expected_panels(w).nbytes
    out = m2.pack_panels(wtype, wd, rows, k)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(w.dtype)
    print("[panels] %s %dx%d: %d bytes" % (wtype, rows, k, got.nbytes), flush=True)
    assert np.array_equal(got, expected_panels(w))
