"""fastocr_create_static (the handle whose scratch lives in the library's
static device array; no device allocation) against fastocr_create: the same
decode, step for step, gives the same outputs and kept sets.  Two static
handles in a row, the second for a smaller input, each compared with an
ordinary handle of its configuration."""

import numpy as np
import pytest
import torch

import dynamic_kv_cache_amd as fo
from workload import get_workload

from gpu_harness import TOL, check_out, log, make_config, upload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decode_pair(up, steps):
    """Run the same decode on an ordinary and a static handle; compare every
    layer's output and the kept set after every layer."""
    wl = up.wl
    L, B, Hq, d = wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim
    cfg = make_config(up)
    ha = fo.fastocr_create(cfg)
    hs = fo.fastocr_create_static(cfg)
    ia, is_ = fo.fastocr_get_info(ha), fo.fastocr_get_info(hs)
    assert ia == is_, (ia, is_)
    assert 0 < is_["scratch_bytes"] <= fo.STATIC_SCRATCH_MIB << 20
    k_max = ia["k_max"]
    oa = torch.empty((B, Hq, d), dtype=up.io_dtype, device=DEV)
    os_ = torch.empty_like(oa)
    sa, ss = (torch.zeros((B, k_max), dtype=torch.int32, device=DEV) for _ in range(2))
    ca, cs = (torch.zeros((B,), dtype=torch.int32, device=DEV) for _ in range(2))
    worst = 0.0
    for t in range(steps):
        if t == wl.warmup_steps:
            assert fo.fastocr_profile_warmup(ha) == fo.fastocr_profile_warmup(hs)
        for l in range(L):
            fo.fastocr_attend(ha, l, up.Qd[l][t], up.Kd[l], up.Vd[l], up.lens[t], oa)
            fo.fastocr_attend(hs, l, up.Qd[l][t], up.Kd[l], up.Vd[l], up.lens[t], os_)
            fo.fastocr_get_selection(ha, sa, ca)
            fo.fastocr_get_selection(hs, ss, cs)
            torch.cuda.synchronize()
            a = oa.float().cpu().numpy().astype(np.float64)
            b = os_.float().cpu().numpy().astype(np.float64)
            worst = max(worst, check_out(b, a, wl.dtype, f"static vs ordinary t={t} l={l}"))
            assert torch.equal(ca, cs) and torch.equal(sa, ss), f"kept set t={t} l={l}"
    assert fo.fastocr_get_status(ha) == 0 and fo.fastocr_get_status(hs) == 0
    return ha, hs, worst


def test_static_handle_matches_ordinary_twice():
    # first: 7B-like shapes (8 layers, 4 focal); second, smaller: the tiny page
    big = upload(get_workload("7b-b1").with_overrides(num_layers=8, focal_band=(3, 5), num_focal=3,
                                                      warmup_steps=3), steps=9)
    ha, hs, worst1 = _decode_pair(big, 9)
    # a second static handle on this GPU while the first is live would share
    # its scratch: refused
    with pytest.raises(fo.FastOCRError) as err:
        fo.fastocr_create_static(make_config(big))
    assert err.value.code == fo.ERR_STATE
    fo.fastocr_destroy(hs)
    fo.fastocr_destroy(ha)
    small = upload(get_workload("tiny-fp32"), steps=10)
    ha2, hs2, worst2 = _decode_pair(small, 10)
    fo.fastocr_destroy(hs2)
    fo.fastocr_destroy(ha2)
    log(f"[static] worst |static - ordinary|: {worst1:.2e} (7B-like), {worst2:.2e} (tiny)")


def test_static_handle_rejects_oversize_config():
    # a configuration whose scratch exceeds the static array is refused with
    # its own status code, and leaves the array free
    cfg = fo.Config(num_layers=80, num_q_heads=64, num_kv_heads=8, head_dim=128, batch=64,
                    max_seq_len=15000, max_img_tokens=12800, tau=0.05, num_focal=8, warmup_steps=8)
    need = fo.fastocr_plan_launch(cfg)["scratch_bytes"]
    assert need > fo.STATIC_SCRATCH_MIB << 20
    with pytest.raises(fo.FastOCRError) as err:
        fo.fastocr_create_static(cfg)
    assert err.value.code == fo.ERR_SCRATCH
    h = fo.fastocr_create_static(fo.Config(num_layers=2, num_q_heads=4, num_kv_heads=2, head_dim=64, batch=1,
                                           max_seq_len=64, max_img_tokens=32, tau=0.5, num_focal=1,
                                           warmup_steps=1, dtype="f32"))
    fo.fastocr_destroy(h)
