"""GPU parity of the decode chain (qgemv_affine_chain_*): the linears of a
decode step in dependency stages, run in one launch, against the oracle's
composition of the same linears (every output stored in the activation dtype
before later stages read it; the chain's outputs are compared with the
oracle's fp64 values, each linear on its own inputs as the oracle stored
them)."""
import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import TORCH_DT, assert_float_bar, dev16, dev32, host_f64, require_gpu

pytestmark = pytest.mark.gpu

# the 1B decode set: (name, N, K)
LAYER = [("q", 2048, 2048), ("k", 512, 2048), ("v", 512, 2048), ("o", 2048, 2048),
         ("gate", 8192, 2048), ("up", 8192, 2048), ("down", 2048, 8192)]


def decoder_spec(layers):
    """Stages of a decoder without attention: q/k/v read h; o reads q (a
    stand-in for the attention output) plus the residual h; gate/up read o;
    down reads silu(gate) * up plus the residual o, and is the next h."""
    spec, h = [], "h0"
    for l in range(layers):
        n = lambda s: f"{s}{l}"
        st = 4 * l
        spec += [dict(name=n("q"), N=2048, K=2048, stage=st, x=h), dict(name=n("k"), N=512, K=2048, stage=st, x=h),
                 dict(name=n("v"), N=512, K=2048, stage=st, x=h),
                 dict(name=n("o"), N=2048, K=2048, stage=st + 1, x=n("q"), resid=h),
                 dict(name=n("gate"), N=8192, K=2048, stage=st + 2, x=n("o")),
                 dict(name=n("up"), N=8192, K=2048, stage=st + 2, x=n("o")),
                 dict(name=n("down"), N=2048, K=8192, stage=st + 3, x=n("up"), gate=n("gate"), resid=n("o"))]
        h = n("down")
    return spec, {"h0": 2048}


def run_chain(spec, inputs, G, dt, seed, scale_range=(0.002, 0.004), runs=1, inplace=()):
    """Weights and inputs seeded; the chain run `runs` times (outputs NaN
    first each time); every output checked against the oracle.  Scales of
    0.002-0.004 keep the activations near unit size through the decoder's
    stages (larger ones grow them about fourfold a layer, and the gated
    input silu(gate) * up must stay inside fp16)."""
    dev = require_gpu()
    host = {name: si.activations(1, n, seed=(*seed, 1, i), dtype=dt).reshape(n)
            for i, (name, n) in enumerate(sorted(inputs.items()))}
    bufs = {name: dev16(v, dt, dev) for name, v in host.items()}
    lins_h, lins_d = [], []
    for i, l in enumerate(spec):
        N, K = l["N"], l["K"]
        p, s, b = si.affine_weights(N, K, G, 4, seed=(*seed, 2, i), scale_range=scale_range, bias_mode="noise",
                                    sb_dtype=dt)
        lins_h.append(dict(name=l["name"], packed=p, scales=s, biases=b, N=N, K=K, x=l["x"], gate=l.get("gate"),
                           resid=l.get("resid")))
        if l["name"] in inplace:  # y is the residual's buffer: the in-place update
            y = bufs[l["resid"]]
        else:
            y = torch.empty(N, dtype=TORCH_DT[dt], device=dev)
        bufs[l["name"]] = y
        lins_d.append(dict(x=bufs[l["x"]], gate=bufs[l["gate"]] if l.get("gate") else None,
                           resid=bufs[l["resid"]] if l.get("resid") else None, w=dev32(p, dev), s=dev16(s, dt, dev),
                           b=dev16(b, dt, dev), y=y, stage=l["stage"]))
    print(f"[case] chain {len(spec)} linears, {spec[-1]['stage'] + 1} stages, G={G} {dt} seed={seed}", flush=True)
    chain = qa.GemvChain(lins_d, G)
    ref_bufs = dict(host)
    ref = oracle.qgemv_affine_chain(lins_h, ref_bufs, dt, G)
    # the in-place outputs replace their residual's stored value
    for l in spec:
        if l["name"] in inplace:
            ref_bufs[l["resid"]] = ref_bufs[l["name"]]
    for rep in range(runs):
        for l in spec:
            if l["name"] not in inplace:
                bufs[l["name"]].fill_(float("nan"))
        if inplace:  # the residuals they overwrite start from the inputs again
            for name, v in host.items():
                bufs[name].copy_(dev16(v, dt, dev))
        torch.cuda.synchronize()
        chain()
        torch.cuda.synchronize()
        for l in spec:
            assert_float_bar(host_f64(bufs[l["name"]]).reshape(1, -1), ref[l["name"]].reshape(1, -1),
                             f"{l['name']} run {rep}")
    assert not chain.timed_out()
    chain.close()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_decoder_layers(dt):
    spec, inputs = decoder_spec(2)
    run_chain(spec, inputs, 64, dt, seed=(80, int(dt == "f16")))


def test_repeated_runs_reset_the_counts():
    # the stage counts are back at zero after every run: three runs of one
    # plan, every output written afresh each time
    spec, inputs = decoder_spec(1)
    run_chain(spec, inputs, 128, "bf16", seed=(81,), runs=3)


@pytest.mark.parametrize("K", [12288, 16384, 32])
def test_long_and_short_rows(K):
    # K past 8192: each wave takes more than one 2048-code chunk (12288: the
    # last chunk on some waves only); K = 32: one group, most lanes idle
    spec = [dict(name="a", N=96, K=K, stage=0, x="x"), dict(name="b", N=37, K=96, stage=1, x="a"),
            dict(name="c", N=300, K=K, stage=1, x="x", resid="r")]
    run_chain(spec, {"x": K, "r": 300}, 32, "f16", seed=(82, K))


def test_inplace_residual():
    # y == resid: the residual update in place (the stage reads the value
    # before its own write)
    spec = [dict(name="a", N=256, K=512, stage=0, x="x"),
            dict(name="b", N=512, K=256, stage=1, x="a", resid="x"),
            dict(name="c", N=64, K=512, stage=2, x="b")]
    run_chain(spec, {"x": 512}, 64, "bf16", seed=(83,), inplace=("b",))


@pytest.mark.parametrize("i", range(16))
def test_random_chains(i):
    r = np.random.default_rng((84, i))
    dt = str(r.choice(["bf16", "f16"]))
    G = int(r.choice([32, 64, 128]))
    Ks = [k for k in (32, 64, 96, 128, 256, 384, 512, 1024, 2048, 4096, 8192) if k % G == 0]
    inputs, lengths, spec = {}, {}, []   # lengths: buffer name -> length

    def pick(n, p_new):
        have = [b for b, m in lengths.items() if m == n]
        if have and r.random() > p_new:
            return str(r.choice(have))
        name = f"in{len(inputs)}"
        inputs[name] = n
        lengths[name] = n
        return name

    stages = int(r.integers(1, 6))
    made = []
    for st in range(stages):
        new = {}
        for j in range(int(r.integers(1, 4))):
            K = int(r.choice(Ks + [m for m in lengths.values() if m % G == 0 and m % 32 == 0]))
            N = int(r.integers(1, 600)) if r.random() < 0.5 else int(r.choice(Ks))
            l = dict(name=f"s{st}l{j}", N=N, K=K, stage=st, x=pick(K, 0.3))
            if r.random() < 0.35:
                l["gate"] = pick(K, 0.4)
            if r.random() < 0.35:
                l["resid"] = pick(N, 0.4)
            spec.append(l)
            new[l["name"]] = N
        lengths.update(new)  # readable from the next stage on
    run_chain(spec, inputs, G, dt, seed=(85, i))
