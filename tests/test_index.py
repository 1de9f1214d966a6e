"""Variable-length helpers: bit-exact against independent integer definitions
(CPU only; the helpers are host code in libgdr.so)."""
import json
import os

import numpy as np
import pytest
import torch

import gated_delta_rule_66_amd as gdr
from gated_delta_rule_66_amd._lib import GdrError

HERE = os.path.dirname(os.path.abspath(__file__))


def ref_lens(cu):
    return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]


def ref_chunk_indices(cu, bt):
    rows = []
    for n in range(len(cu) - 1):
        L = cu[n + 1] - cu[n]
        j = 0
        while j * bt < L:
            rows.append([n, j])
            j += 1
    return rows


def ref_chunk_offsets(cu, bt):
    offs = [0]
    for n in range(len(cu) - 1):
        L = cu[n + 1] - cu[n]
        offs.append(offs[-1] + (L + bt - 1) // bt)
    return offs, offs[-1]


def test_prepare_lens_worked_example():
    with open(os.path.join(HERE, "golden", "prepare_lens.json")) as f:
        g = json.load(f)
    out = gdr.prepare_lens(torch.tensor(g["cu_seqlens"], dtype=torch.long))
    assert out.tolist() == g["lens"]
    assert out.dtype == torch.long


def test_chunk_helpers_documented_inputs():
    cu = torch.tensor([0, 4, 8], dtype=torch.long)
    assert gdr.prepare_chunk_indices(cu, 2).tolist() == [[0, 0], [0, 1], [1, 0], [1, 1]]
    offs, total = gdr.prepare_chunk_offsets(cu, 2)
    assert offs.tolist() == [0, 2, 4] and total == 4
    assert offs.shape == cu.shape


LENS = [[5], [0], [1, 63, 64, 65], [64, 0, 0, 3], [129, 1, 200, 4097, 7], [0, 0]]


@pytest.mark.parametrize("lens", LENS, ids=str)
@pytest.mark.parametrize("bt", [1, 2, 3, 64])
@pytest.mark.parametrize("dtype", [torch.int32, torch.int64])
def test_helpers_bit_exact(lens, bt, dtype):
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    t = torch.tensor(cu, dtype=dtype)
    assert gdr.prepare_lens(t).tolist() == ref_lens(cu)
    assert gdr.prepare_lens(t).dtype == dtype
    idx = gdr.prepare_chunk_indices(t, bt)
    assert idx.tolist() == ref_chunk_indices(cu, bt) or (idx.numel() == 0 and not ref_chunk_indices(cu, bt))
    offs, total = gdr.prepare_chunk_offsets(t, bt)
    r_offs, r_total = ref_chunk_offsets(cu, bt)
    assert offs.tolist() == r_offs and total == r_total


def test_token_starts_reading():
    import ctypes
    from gated_delta_rule_66_amd._lib import lib
    cu = np.array([0, 4, 8, 9], dtype=np.int64)
    n = ctypes.c_int64(0)
    out = np.zeros((8, 2), dtype=np.int64)
    st = lib.gdr_prepare_chunk_token_starts_i64(cu.ctypes.data_as(ctypes.c_void_p), 4, 2,
                                                out.ctypes.data_as(ctypes.c_void_p),
                                                ctypes.byref(n))
    assert st == 0 and n.value == 5
    assert out[:5].tolist() == [[0, 0], [2, 1], [4, 2], [6, 3], [8, 4]]


@pytest.mark.parametrize("cu", [[1, 4], [0, 4, 3]])
def test_malformed_cu_seqlens_rejected(cu):
    with pytest.raises(GdrError) as e:
        gdr.prepare_lens(torch.tensor(cu))
    assert e.value.name == "GDR_ERR_VARLEN"


def test_bad_chunk_size_rejected():
    with pytest.raises(GdrError) as e:
        gdr.prepare_chunk_offsets(torch.tensor([0, 4]), 0)
    assert e.value.name == "GDR_ERR_ARG"
