"""GPU checks of tiered expert residency (include/moe_tier.h): layer outputs
read through the tier table -- experts in HBM slots or in pinned host
memory read over PCIe, with promotions and evictions running on a copy
stream while forward calls are queued -- equal the all-HBM outputs bitwise
(both tiers hold the same bytes), and both equal the CPU oracle within the
usual bounds (rel-L2 <= 1e-3, max-abs <= 1e-2).  The tiers follow "GTX
1070向け35BパラメータMoEモデル推論エンジン公開", section "VRAMとシステムメモリで
重みを分割する設計"."""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_expert_02_amd as moe
from quantized_moe_expert_02_amd import synth
from helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(*a):
    print(*a, flush=True)


def _pinned_copy(packed: torch.Tensor) -> torch.Tensor:
    """Pinned host copy of packed experts [n][pb], 256-byte aligned."""
    n, pb = packed.shape
    buf = torch.empty(n * pb + 256, dtype=torch.uint8, pin_memory=True)
    off = (-buf.data_ptr()) % 256
    host = buf[off:off + n * pb].view(n, pb)
    host.copy_(packed.cpu())
    host._keep = buf  # the view keeps its storage alive anyway; explicit for clarity
    return host


class TieredModel:
    def __init__(self, dims, n_layers, slots_per_layer, seed, policy=moe.MOE_TIER_LRU):
        self.dims, self.L, self.C = dims, n_layers, slots_per_layer
        self.canon = [synth.make_layer(dims, ("tier", seed, l)) for l in range(n_layers)]
        self.layers = [moe.PackedLayer.from_layer(c) for c in self.canon]
        E = dims.n_experts
        self.host = [_pinned_copy(pl.packed[:E]) for pl in self.layers]
        ptrs = [h.data_ptr() + e * h.shape[1] for h in self.host for e in range(E)]
        pb = self.layers[0].packed.shape[1]
        self.slots = torch.empty(max(1, n_layers * slots_per_layer) * pb, dtype=torch.uint8, device=DEV)
        self.table = torch.zeros(n_layers * E, dtype=torch.int64, device=DEV)
        self.copy_stream = torch.cuda.Stream()
        self.tier = moe.Tier(dims, n_layers, ptrs, slots_per_layer, slots=self.slots if slots_per_layer else None,
                             table=self.table, copy_stream=self.copy_stream, policy=policy)

    def oracle_y(self, l, x):
        return oracle.forward(self.canon[l], x.cpu())

    def forward(self, l, x, y, ws, ti):
        pl = self.layers[l]
        w = self.tier.weights(l, pl.router_w, pl.router_b, pl.shared_ptr)
        import ctypes
        d = moe._dims(self.dims)
        rc = moe.lib().moe_w4a16_forward(ctypes.byref(d), ctypes.byref(w), moe._p(x), x.shape[0], moe._p(y),
                                         moe._p(ti), None, moe._p(ws), ws.numel(), moe._stream(None))
        assert rc == moe.MOE_OK, rc


def _step_inputs(dims, T, tag):
    return synth.make_tokens(dims, T, tag).to(DEV)


@pytest.mark.parametrize("wfmt", [synth.INT4_ROW, synth.E2M1_B16, synth.INT8_ROW, synth.INT2_ROW])
def test_all_experts_from_host_memory(wfmt):
    """slots_per_layer = 0: every routed expert is read over PCIe."""
    dims = synth.Dims(512, 256, 16, 4, 1, wfmt)
    _log("tier zero-copy", dims)
    m = TieredModel(dims, 1, 0, ("zc", wfmt))
    for T in (1, 5, 40):
        x = _step_inputs(dims, T, ("zc", wfmt, T))
        ws = moe.workspace(dims, T, DEV)
        y = torch.empty((T, dims.hidden), dtype=torch.float16, device=DEV)
        ti = torch.empty((T, dims.top_k), dtype=torch.int32, device=DEV)
        m.forward(0, x, y, ws, ti)
        y_ref = moe.moe_w4a16_forward(m.layers[0], x)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), T
        assert_close(y, m.oracle_y(0, x), f"tier zero-copy wfmt={wfmt} T={T}")
    assert m.tier.stats()["promotions"] == 0
    m.tier.close()


def test_lru_promotions_race_with_queued_forwards():
    """Two layers, three HBM slots each: every step promotes and evicts while
    the next forward calls are already queued; outputs stay bitwise equal to
    the all-HBM layer, and the LRU state follows the reported unions."""
    dims = synth.Dims(512, 256, 24, 4, 1, synth.INT4_ROW)
    _log("tier lru race", dims)
    L, C, E = 2, 3, dims.n_experts
    m = TieredModel(dims, L, C, "race")
    rng = np.random.default_rng(5)
    outs = []
    prev = {}  # layer -> routing of its previous step (device tensor)
    for step in range(10):
        for l in range(L):
            # the previous step's union of this layer is read first; it is
            # reported after this step's forward has been queued, so its
            # promotions and evictions race with that forward
            report = sorted(set(prev[l].cpu().numpy().ravel().tolist())) if l in prev else []
            T = int(rng.choice([1, 3, 8, 20]))
            x = _step_inputs(dims, T, ("race", step, l))
            ws = moe.workspace(dims, T, DEV)
            y = torch.empty((T, dims.hidden), dtype=torch.float16, device=DEV)
            ti = torch.empty((T, dims.top_k), dtype=torch.int32, device=DEV)
            m.forward(l, x, y, ws, ti)
            m.tier.use(l, report)
            if step % 3 == 2:
                m.tier.prefetch(l, rng.choice(E, size=2, replace=False).tolist())
            prev[l] = ti
            outs.append((l, x, y, ws))
    torch.cuda.synchronize()
    torch.cuda.current_stream().wait_stream(m.copy_stream)
    torch.cuda.synchronize()
    for l, x, y, ws in outs:
        y_ref = moe.moe_w4a16_forward(m.layers[l], x)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), l
        assert_close(y, m.oracle_y(l, x), f"tier lru layer={l} T={x.shape[0]}")
    st = m.tier.stats()
    _log("  stats", st)
    assert st["evictions"] > 0 and st["hits"] > 0 and st["misses"] > 0
    resident = [(l, e) for l in range(L) for e in range(E) if m.tier.slot(l, e) >= 0]
    assert len(resident) == L * C
    # the table points every resident expert at its slot, the others at host memory
    tab = m.table.cpu().numpy()
    pb = m.layers[0].packed.shape[1]
    for l in range(L):
        for e in range(E):
            s = m.tier.slot(l, e)
            want = (m.slots.data_ptr() + (l * C + s) * pb) if s >= 0 else None
            if want is not None:
                assert tab[l * E + e] == want
            else:
                assert tab[l * E + e] != 0 and not (m.slots.data_ptr() <= tab[l * E + e] < m.slots.data_ptr() + m.slots.numel())
    m.tier.close()


@pytest.mark.parametrize("policy", [moe.MOE_TIER_LRU, moe.MOE_TIER_HOT])
def test_load_before_use_and_hot_set(policy):
    """Each step routes first, reports its union, makes the compute stream
    wait for the promotions (moe_tier_sync) and then runs the layer: outputs
    equal the all-HBM layer bitwise; under LRU every reported expert is
    resident when the layer runs (nothing is read over PCIe)."""
    dims = synth.Dims(512, 256, 24, 4, 1, synth.INT4_ROW)
    _log("tier load-before-use", policy)
    C = 6
    m = TieredModel(dims, 1, C, ("lbu", policy), policy=policy)
    pl = m.layers[0]
    for step in range(8):
        T = 1 + step % 3
        x = _step_inputs(dims, T, ("lbu", policy, step))
        ws = moe.workspace(dims, T, DEV)
        r = moe.moe_route(pl, x, ws=ws)
        nu = int(r["n_unique"][0])
        union = r["uniq_ids"][:nu].cpu().tolist()
        m.tier.use(0, union)
        m.tier.sync()
        if policy == moe.MOE_TIER_LRU and len(union) <= C:
            assert all(m.tier.slot(0, e) >= 0 for e in union)
        y = torch.empty((T, dims.hidden), dtype=torch.float16, device=DEV)
        ti = torch.empty((T, dims.top_k), dtype=torch.int32, device=DEV)
        m.forward(0, x, y, ws, ti)
        y_ref = moe.moe_w4a16_forward(pl, x)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), step
        assert_close(y, m.oracle_y(0, x), f"tier load-before-use step={step}")
        assert sorted(set(ti.cpu().numpy().ravel().tolist())) == union
    st = m.tier.stats()
    _log("  stats", st)
    assert st["promotions"] > 0
    m.tier.close()
