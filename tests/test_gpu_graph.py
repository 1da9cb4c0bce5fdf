"""The decode step (cache write, absorption, split + combine; on one stream as
the bench runs it, or with the cache write on a side stream) captured in a
HIP graph: every replay, with eager work and synchronisations between
replays, gives the same bits as the eager step."""
import numpy as np
import pytest
import torch

from mla_latent_kv_22_amd import harness, inputs as I
from tests._util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("two_streams", [False, True], ids=["one_stream", "side_stream_write"])
def test_graph_replays_match_eager(two_streams):
    need_gpu()
    print(f"[case] graph replay v2lite dims two_streams={two_streams}", flush=True)
    cfg = I.scaled(I.V2LITE, batch=6, seq_len=700, min_seq_len=1, paged=True)
    inp = I.make(cfg, 5)
    st = harness.DecodeStep(cfg, inp)
    side = torch.cuda.Stream() if two_streams else None
    pool0 = st.pool.clone()
    st.step(pool=st.pool, side_stream=side)
    torch.cuda.synchronize()
    ref_out, ref_lse = st.out.clone(), st.lse.clone()
    ref_pool = st.pool.clone()

    work = st.pool.clone()
    work.copy_(pool0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step(pool=work, side_stream=side)
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: reset the pool, scribble over the outputs
        work.copy_(pool0)
        st.out.fill_(float("nan"))
        st.lse.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep}: out differs"
        assert torch.equal(st.lse, ref_lse), f"replay {rep}: lse differs"
        assert torch.equal(work.view(torch.int16), ref_pool.view(torch.int16)), f"replay {rep}: cache differs"
