"""The C ABI's host-only functions: the library loads and exports every
function the header declares with the ABI version the binding expects, the
status strings, the timing hook's argument checks and the shard split.  No
call here takes a device address, so the module runs anywhere."""
import ctypes
import os
import re

import pytest

import megatron_tensor_transformer_fwd_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_shard.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tp.LIB_PATH), reason="libtpshard.so not built")

OK, E_NULL, E_DIM, E_DIVIS, E_DTYPE, E_ALIGN, E_ALIAS, E_WS, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree_and_library_exports_all():
    names = _declared_functions()
    assert set(names) == set(tp.EXPORTS), (names, sorted(tp.EXPORTS))
    L = tp.lib()
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strerror():
    hdr = open(HEADER).read()
    declared = int(re.search(r"#define TP_ABI_VERSION (\d+)", hdr).group(1))
    assert tp.tp_abi_version() == declared == tp.ABI_VERSION
    L = tp.lib()
    for code in (OK, E_NULL, E_DIM, E_DIVIS, E_DTYPE, E_ALIGN, E_ALIAS, E_WS, E_HIP):
        assert L.tp_strerror(code) and L.tp_strerror(code) != b"unknown status"
    assert L.tp_strerror(-99) == b"unknown status"


def test_profile_hook_arguments():
    """The timing hook's host-side contract: bad arrays or capacities are
    refused, a label filter can be set and lifted, and ending an armed hook
    that launched nothing reports zero kernels and an empty label."""
    import ctypes
    L = tp.lib()
    ev = (ctypes.c_void_p * 4)()
    assert L.tp_profile_begin(None, ev, 4) == E_NULL
    assert L.tp_profile_begin(ev, ev, 0) == E_DIM
    assert L.tp_profile_begin(ev, ev, 4) == OK
    assert L.tp_profile_only(b"mlp_bwd.dyw2t_dgelu") == OK
    assert L.tp_profile_only(None) == OK
    assert L.tp_profile_end() == 0
    assert L.tp_profile_label(0) == b""


def test_shard_range():
    assert tp.tp_shard_range(4096, 8, 3) == (1536, 512)
    assert tp.tp_shard_range(11008, 4, 3) == (8256, 2752)
    assert tp.tp_shard_range(32, 4, 0) == (0, 8)
    with pytest.raises(tp.TPError) as e:
        tp.tp_shard_range(11008, 3, 0)
    assert e.value.status == E_DIVIS and "divisible" in e.value.detail
    for args in ((0, 4, 0), (16, 0, 0), (16, 4, 4), (16, 4, -1)):
        with pytest.raises(tp.TPError) as e:
            tp.tp_shard_range(*args)
        assert e.value.status == E_DIM
    assert tp.lib().tp_shard_range(8, 2, 0, None, None) == E_NULL
