"""CPU checks of the ResNet-50 trunk's launch schedule (no GPU): the hand-off between
two 64-channel blocks fused into one launch (the block's last 1x1 conv and the next
block's first), every launch's inputs produced by earlier launches, every conv run
once, and no fusion when it is switched off."""
import types

from integer_quantized_nn_amd import synth
from integer_quantized_nn_amd.resnet50 import QuantResNet50Trunk


def _units(fuse):
    tr = synth.resnet50_trunk(seed=0, batch=1)
    holder = types.SimpleNamespace(trunk=tr)
    return tr, QuantResNet50Trunk._launch_units(holder, fuse)


def test_fused_pairs_and_order():
    tr, units = _units(True)
    names = ["+".join(tr.layers[i].name for i in u) for u in units]
    assert len(units) == 50
    assert [n for n in names if "+" in n] == ["l1.0.c3+l1.1.c1", "l1.1.c3+l1.2.c1", "l1.2.c3+l2.0.c1"]
    # every conv exactly once
    assert sorted(i for u in units for i in u) == list(range(len(tr.layers)))
    # a launch reads only tensors written before it (the pooled stem output with the stem)
    ready = {"input"}
    for u in units:
        for i in u:
            layer = tr.layers[i]
            assert layer.src in ready, layer.name
            assert layer.res_src is None or layer.res_src in ready, layer.name
            ready.add(layer.out)
            if layer.name == "stem":
                ready.add("pool")
    # a pair's second conv reads the first's output
    for u in units:
        if len(u) == 2:
            assert tr.layers[u[1]].src == tr.layers[u[0]].out


def test_no_fusion():
    tr, units = _units(False)
    assert units == [(i,) for i in range(len(tr.layers))]
