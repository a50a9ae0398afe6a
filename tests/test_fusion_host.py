"""Shared-input fusion, host side: a fused tensor (q|k|v, gate|up) holds the same
weights as its projections stacked along N, and packing is row-local, so its
packed codes and scales are the projections' packings stacked."""
import numpy as np

from weight_only_bit_block_amd import inputs


def test_fused_workload_shapes():
    a, b = inputs.decode_step(1), inputs.decode_step(1, fused=True)
    assert len(a.tensors) == 197 and len(b.tensors) == 113
    assert a.weight_bytes == b.weight_bytes and a.flops == b.flops
    names = [t.name for t in b.tensors[:4]]
    assert names == ["L0.qkv", "L0.o", "L0.gateup", "L0.down"]
    assert [t.N for t in b.tensors[:4]] == [4096, 1024, 6144, 1024]
    m = inputs.decode_step(4, mixed=True, fused=True)
    assert [t.bits for t in m.tensors[:4]] == [8, 8, 4, 4] and m.tensors[-1].bits == 8


def test_fused_weights_are_stacked_projections():
    a, b = inputs.decode_step(1), inputs.decode_step(1, fused=True)
    by_name = {t.name: t for t in a.tensors}
    for t in b.tensors[4:8]:                       # layer 1
        parts = t.parts or (t.proj,)
        stacked = np.concatenate([a.weight(by_name[f"L{t.layer}.{p}"]) for p in parts])
        assert np.array_equal(b.weight(t), stacked), t.name
        assert b.x_for(t) is a.x_for(by_name[f"L{t.layer}.{parts[0]}"]) or \
            np.array_equal(b.x_for(t), a.x_for(by_name[f"L{t.layer}.{parts[0]}"]))


def test_packing_of_stack_is_stack_of_packings(oracle_mod):
    wl = inputs.decode_step(1, mixed=True, fused=True)
    for t in wl.tensors[:3]:                       # qkv int8, o int8, gateup int4
        w = wl.weight(t)[::64]                      # every 64th row keeps it quick
        q, s = oracle_mod.quantize(w, t.bits)
        half = w.shape[0] // 2
        q0, s0 = oracle_mod.quantize(w[:half], t.bits)
        q1, s1 = oracle_mod.quantize(w[half:], t.bits)
        assert np.array_equal(q, np.concatenate([q0, q1])) and np.array_equal(s, np.concatenate([s0, s1]))
