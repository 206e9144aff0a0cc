"""CPU checks of the GPU tests' helpers: the tabulated E5M2 write gives exactly the oracle's own
cache write (the full-size parity tests build their oracle pools with it)."""
import numpy as np

import oracle
from gpu_harness import e5m2_of_bf16, oracle_pools, oracle_pools_from_plan
from workloads import POISON_BITS, make_workload, write_plan


def test_table_is_the_oracle_encoder_on_special_patterns():
    tab = e5m2_of_bf16()
    pats = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x4770, 0x4760, 0x3780,
                     0x3700, 0x0001, 0x477F], np.uint16)
    assert np.array_equal(tab[pats], oracle.f64_to_e5m2(oracle.bf16_to_f64(pats)))


def test_pools_from_plan_equal_the_oracle_cache_write():
    for kv in ("e5m2", "bf16"):
        w = make_workload([1, 17, 40, 300, 0], num_q_heads=8, num_kv_heads=2, head_dim=64, q_dtype="bf16",
                          kv_dtype=kv, seed=5)
        pk, pv = oracle_pools_from_plan(w, write_plan(w, "all"))
        rk, rv = oracle_pools(w)
        assert np.array_equal(pk.view(np.uint8), rk.view(np.uint8)) and np.array_equal(pv.view(np.uint8), rv.view(np.uint8))
        assert (pk.view(np.uint8) == np.uint8(POISON_BITS["e5m2"])).any() if kv == "e5m2" else True
