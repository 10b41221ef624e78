"""The opt-in DCN_VALIDATE input check of the Python binding (host side)."""
import math

import pytest
import torch

import modulated_deformable_convolution_dcn_amd as dcn


def test_off_by_default(monkeypatch):
    monkeypatch.delenv("DCN_VALIDATE", raising=False)
    assert not dcn.validation_enabled()
    dcn._validate(offset=torch.tensor([math.nan]))  # no check, no error
    monkeypatch.setenv("DCN_VALIDATE", "0")
    assert not dcn.validation_enabled()


@pytest.mark.parametrize("bad", [math.nan, math.inf, -math.inf])
def test_rejects_non_finite(monkeypatch, bad):
    monkeypatch.setenv("DCN_VALIDATE", "1")
    assert dcn.validation_enabled()
    dcn._validate(offset=torch.zeros(3), mask=None)
    with pytest.raises(ValueError, match="offset"):
        dcn._validate(offset=torch.tensor([0.0, bad]))
    with pytest.raises(ValueError, match="mask"):
        dcn._validate(offset=torch.zeros(2), mask=torch.tensor([bad]))
