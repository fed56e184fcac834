"""Host-side checks of the speed-up switch settings (no GPU): the eight
settings, their names, and the workloads the runner refuses before it
allocates anything."""

import pytest

from small_workloads import tiny_semi_ar, tiny_two_layer, gpu_small_d128, workload


def test_settings_cover_table6_and_the_dense_mdm():
    from masked_discrete_diffusion_amd.ablation import ALL_SWITCHES, TABLE6, Switches
    flags = {(s.cache_prompt, s.cache_res, s.truncate) for s in TABLE6}
    assert len(TABLE6) == 7 and len(flags) == 7 and (False, True, True) not in flags
    assert TABLE6[0].name == "none" and TABLE6[-1].name == "cache_prompt+cache_res+truncate"
    assert ALL_SWITCHES[-1].bidirectional and ALL_SWITCHES[-1].name == "dense_bidirectional"
    with pytest.raises(ValueError):
        Switches(True, False, False, bidirectional=True)


def test_runner_refuses_semi_ar_and_two_layers():
    from masked_discrete_diffusion_amd.ablation import AblationRunner, Switches
    for cfg in (tiny_semi_ar(), tiny_two_layer()):
        with pytest.raises(ValueError):
            AblationRunner(workload(cfg), Switches(), device="cpu")


def test_rewind_is_exported():
    from masked_discrete_diffusion_amd import _lib as L
    assert hasattr(L.load(), "mdm_cache_rewind")
    assert L.mdm_cache_len(None) == -1
