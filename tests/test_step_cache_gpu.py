"""Graph-cached endpoint calls (etg_step_gather / etg_step_logits): every call,
eager first hit, capture on the second and replays after, is checked against the
oracle and bitwise against the plain entry points on the same inputs.  Replays
run with new inputs in the static buffers and with eager library work between
them, and the cache's counters show that graphs were captured and replayed."""
import numpy as np
import pytest
import torch

import embedding_table_gather_amd as etg
import oracle
import synth
from oracle import accept
from tests.gpu_util import bits, ids_dev, note, table, to_dev

pytestmark = pytest.mark.gpu

BF16 = etg.BF16


def test_step_gather_buckets_replay_bit_exact():
    V, d = 5003, 896
    host = synth.make_table(BF16, V, d, seed=301)
    t = table(host, BF16, V, d)
    sc = etg.StepCache(t, max_ids=700, max_batch=4, k=10, use_graphs=True)
    assert sc.rows.shape[0] == 704  # 700 ids take the bucket of 704 (a multiple of 64)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for n in (5, 64, 65, 628):
            for rep in range(8):  # id slots 0-3: first hits (eager), then second hits (captured)
                ids = synth.uniform_ids(n, V, seed=1000 * n + rep)
                note(f"step gather n={n} rep={rep}")
                rows = sc.gather(ids, scale="sqrt_d")
                # eager library work between the replays
                other = t.embed_gather(ids_dev(ids[::-1].copy()), scale="sqrt_d", check=False)
                s.synchronize()
                ref, _ = oracle.embed_gather(host, BF16, V, d, ids, scale=oracle.sqrt_d(d))
                assert np.array_equal(bits(rows), bits(ref)), (n, rep)
                assert np.array_equal(bits(other), bits(ref[::-1])), (n, rep)
    # a graph per (bucket, id slot): 5 -> 64 and 64 -> 64 share the bucket (4 graphs,
    # 12 launches), 65 -> 128 and 628 -> 640 (4 graphs and 4 launches each)
    assert sc.stats() == (12, 20)


def test_step_gather_bucket_sharing_and_null_stream():
    V, d = 3001, 256
    host = synth.make_table(etg.F32, V, d, seed=302)
    t = table(host, etg.F32, V, d)
    sc = etg.StepCache(t, max_ids=300, max_batch=1, k=1, use_graphs=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for i, n in enumerate((3, 64, 10, 60) * 3):  # one bucket (64): 4 slots eager, captured, replayed
            ids = synth.uniform_ids(n, V, seed=n + i)
            rows = sc.gather(ids)
            s.synchronize()
            ref, _ = oracle.embed_gather(host, etg.F32, V, d, ids)
            assert np.array_equal(bits(rows), bits(ref))
    assert sc.stats() == (4, 8)
    # graphs off: the same calls, all eager
    sc3 = etg.StepCache(t, max_ids=300, max_batch=1, k=1, use_graphs=False)
    with torch.cuda.stream(s):
        for i, n in enumerate((3, 64, 10, 60) * 3):
            ids = synth.uniform_ids(n, V, seed=n + i)
            rows = sc3.gather(ids)
            s.synchronize()
            ref, _ = oracle.embed_gather(host, etg.F32, V, d, ids)
            assert np.array_equal(bits(rows), bits(ref))
    assert sc3.stats() == (0, 0)
    # the null stream cannot be captured: every call there runs eagerly
    sc2 = etg.StepCache(t, max_ids=300, max_batch=1, k=1, use_graphs=True)
    for n in (7, 7, 7):
        ids = synth.uniform_ids(n, V, seed=99)
        rows = sc2.gather(ids)
        torch.cuda.synchronize()
        ref, _ = oracle.embed_gather(host, etg.F32, V, d, ids)
        assert np.array_equal(bits(rows), bits(ref))
    assert sc2.stats() == (0, 0)


@pytest.mark.parametrize("dtype,V,d", [(BF16, 20011, 896), (etg.F32, 4096, 256), (etg.Q8_0, 3001, 768)])
def test_step_logits_replays_match_eager_and_oracle(dtype, V, d):
    host = synth.make_table(dtype, V, d, seed=303)
    t = table(host, dtype, V, d)
    k = 10
    sc = etg.StepCache(t, max_ids=64, max_batch=24, k=k, use_graphs=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for B in (1, 4, 8, 20):
            for rep in range(4):
                R = synth.residuals(B, d, seed=7000 + 10 * B + rep)
                sc.residual[:B].copy_(to_dev(R))
                note(f"step logits dtype={dtype} B={B} rep={rep}")
                ev = sc.logits(B)
                wi, ws = t.logits_topk(to_dev(R), k)  # eager, between replays
                ev.synchronize()
                s.synchronize()
                gi, gs = sc.ids[:B].numpy().copy(), sc.scores[:B].numpy().copy()
                assert np.array_equal(gi, wi.cpu().numpy()), (B, rep)
                assert np.array_equal(gs.view(np.uint32), ws.cpu().numpy().view(np.uint32)), (B, rep)
                L, A = oracle.logits(host, dtype, V, d, R)
                oids, _ = oracle.topk(L, k)
                fails = accept.check_full(gi, gs, L, A, oids, accept.tol_coeff(dtype))
                assert not fails, fails[:3]
    graphs, replays = sc.stats()
    assert graphs == 4 and replays == 12


def test_step_gather_back_to_back_calls_keep_their_ids():
    # no synchronisation between calls: each call's ids must reach the device before
    # the next call rewrites the page-locked staging buffer
    V, d = 4099, 128
    host = synth.make_table(BF16, V, d, seed=305)
    t = table(host, BF16, V, d)
    sc = etg.StepCache(t, max_ids=64, max_batch=1, k=1, use_graphs=True)
    outs = [torch.empty((40, d), dtype=torch.float32, device="cuda") for _ in range(12)]
    s = torch.cuda.Stream()
    idss = [synth.uniform_ids(40, V, seed=500 + i) for i in range(12)]
    with torch.cuda.stream(s):
        for i in range(12):
            outs[i].copy_(sc.gather(idss[i]))
    s.synchronize()
    for i in range(12):
        ref, _ = oracle.embed_gather(host, BF16, V, d, idss[i])
        assert np.array_equal(bits(outs[i]), bits(ref)), i


def test_step_errors_refuse_before_enqueueing():
    V, d = 100, 64
    host = synth.make_table(BF16, V, d, seed=304)
    t = table(host, BF16, V, d)
    sc = etg.StepCache(t, max_ids=10, max_batch=2, k=3)
    with pytest.raises(etg.EtgError, match="bad token id"):
        sc.gather(np.array([1, 100, 2], np.int32))
    with pytest.raises(etg.EtgError, match="bad token id"):
        sc.gather(np.array([-1], np.int32))
    with pytest.raises(etg.EtgError, match="ESHAPE"):
        sc.gather(np.zeros(11, np.int32))
    with pytest.raises(etg.EtgError, match="ESHAPE"):
        sc.logits(3)
    assert sc.stats() == (0, 0)
