"""Hardware assumptions that the kernels' performance rests on, checked on the GPU through the C
ABI. A failure here means a schedule tuned for one placement now runs on another: results stay
correct, only the timing model no longer holds.

The forward kernel with independent wavefronts paces wavefronts w and w ^ 4 of its 8-wavefront
workgroups against each other (the one behind takes the higher issue priority) on the
assumption that they share a SIMD, i.e. that a workgroup's wavefronts go to the SIMDs of its
compute unit in turn."""
import pytest
import torch

import selective_state_space_24_amd as ssm

pytestmark = pytest.mark.gpu


def test_partner_wavefronts_share_a_simd():
    n = 512  # two rounds of workgroups over the chip
    out = torch.full((n, 8), -1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    assert ssm.wave_simd_ids_raw(out.data_ptr(), n, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    ids = out.cpu()
    assert int(ids.min()) >= 0 and int(ids.max()) <= 3
    for w in range(4):
        assert torch.equal(ids[:, w], ids[:, w + 4]), f"wavefronts {w} and {w + 4}"
    # the four pairs of a workgroup take the four SIMDs of its compute unit
    assert all(len(set(row[:4].tolist())) == 4 for row in ids)


def test_wave_simd_ids_rejects_bad_arguments():
    assert ssm.wave_simd_ids_raw(None, 1, None) == -1  # SSM_ERR_NULL_ARG
    out = torch.zeros(8, dtype=torch.int32, device="cuda")
    assert ssm.wave_simd_ids_raw(out.data_ptr(), -1, None) != 0
    assert ssm.wave_simd_ids_raw(out.data_ptr(), 0, None) == 0
