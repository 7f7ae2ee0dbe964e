"""Host checks of the Python binding's buffer validation (no GPU): every
wrapper rejects, before calling the library, a tensor that is not on a CUDA
device, not contiguous, on another device than the call's other buffers, or
too small for the bytes the call reads or writes there, or on a device
other than the current one."""

import pytest
import torch

import tiled_movement_amd as T


class FakeCuda:
    """Stands in for a CUDA tensor of `nbytes` bytes (these tests never let a
    call through to the library, so no device memory is needed)."""

    is_cuda = True

    def __init__(self, nbytes, device="cuda:0", contiguous=True, esz=4):
        self.nbytes, self.device, self._contig, self.esz = nbytes, torch.device(device), contiguous, esz

    def is_contiguous(self):
        return self._contig

    def numel(self):
        return self.nbytes // self.esz

    def element_size(self):
        return self.esz

    def data_ptr(self):  # pragma: no cover - reaching here would be a failure of the check
        raise AssertionError("the call reached the library")


def test_host_tensors_are_rejected():
    a = torch.zeros(64, 64, dtype=torch.int32)
    with pytest.raises(ValueError, match="CUDA tensor"):
        T.swz_transpose(a, torch.empty_like(a), 64, 64, 4)


@pytest.mark.parametrize("call", [
    lambda s, d: T.swz_transpose(s, d, 64, 64, 4),
    lambda s, d: T.swz_convert_layout(s, d, 2, 64, 32, 4),
    lambda s, d: T.swz_stage_operand(s, d, 64, 64),
    lambda s, d: T.swz_map(s, d, 4096, (5, 0, 5)),
    lambda s, d: T.swz_map_batch(s, d, 2048, [(5, 0, 5), (3, 3, 4)]),
    lambda s, d: T.swz_copy(s, d, 16384),
])
def test_undersized_destination_is_rejected(call):
    # every call above moves 16 KiB (transposes: 64 x 64 x 4, staging: 64 x 64 x 2 + ...)
    src = FakeCuda(1 << 20)
    with pytest.raises(ValueError, match="holds"):
        call(src, FakeCuda(1024))


def test_fp16_storage_too_small_for_4_byte_elements():
    """The advisor's case: fp16 storage of rows x cols elements given to a
    4-byte transpose holds half the bytes the kernel would write."""
    src = FakeCuda(64 * 64 * 4)
    dst = FakeCuda(64 * 64 * 2, esz=2)
    with pytest.raises(ValueError, match="dst holds 8192 bytes, the call needs 16384"):
        T.swz_transpose(src, dst, 64, 64, 4)


def test_strided_views_and_mixed_devices_are_rejected():
    with pytest.raises(ValueError, match="contiguous"):
        T.swz_transpose(FakeCuda(16384, contiguous=False), FakeCuda(16384), 64, 64, 4)
    with pytest.raises(ValueError, match="cuda:1"):
        T.swz_transpose(FakeCuda(16384), FakeCuda(16384, device="cuda:1"), 64, 64, 4)


def test_gemm_buffers_are_sized_from_m_n_k_and_the_result_type():
    a, bt = FakeCuda(2 * 64 * 32), FakeCuda(2 * 48 * 32)
    with pytest.raises(ValueError, match="c holds"):
        T.swz_gemm(a, bt, FakeCuda(4 * 64 * 48 - 4), 64, 48, 32)
    with pytest.raises(ValueError, match="c holds"):
        T.swz_gemm_ex(a, bt, FakeCuda(2 * 64 * 48 - 2, esz=2), 64, 48, 32, c_type=T.C_BF16)
    with pytest.raises(ValueError, match="fb holds"):
        T.swz_gemm_frag(FakeCuda(2 * 64 * 32), FakeCuda(10), FakeCuda(4 * 64 * 48), 64, 48, 32)


def test_buffers_off_the_current_device_are_rejected(monkeypatch):
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    with pytest.raises(ValueError, match="current device is cuda:0"):
        T.swz_transpose(FakeCuda(16384, device="cuda:1"), FakeCuda(16384, device="cuda:1"), 64, 64, 4)
