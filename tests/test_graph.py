"""Host-side tests (no GPU): the C ABI library loads and exports every declared
symbol; the library's task-graph planner (mk_plan_graph, pure host code) builds
exactly the graph the oracle's independent builder defines; the oracle builder
is pinned by a hand-derived fixture; every graph passes the structural checker
and runs to completion under random and adversarial interleavings of static and
dynamic queues."""
import os
import re
import subprocess

import numpy as np
import pytest

import persistent_megakernel_decode_cu_amd as mk
import synth
from oracle import taskgraph as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")
FIXTURE = os.path.join(ROOT, "tests", "golden", "tiny_graph.txt")
BATCH_FIXTURE = os.path.join(ROOT, "tests", "golden", "batch_graph.txt")
MOE_FIXTURE = os.path.join(ROOT, "tests", "golden", "moe_graph.txt")
OPS = {"QKV": tg.OP_QKV, "ATTN": tg.OP_ATTN, "OPROJ": tg.OP_OPROJ, "GATEUP": tg.OP_GATEUP, "DOWN": tg.OP_DOWN,
       "LMHEAD": tg.OP_LMHEAD, "ROUTE": tg.OP_ROUTE, "EGU": tg.OP_EGU, "EDOWN": tg.OP_EDOWN}
TOY = synth.configs.ModelConfig("toy-1layer", 1, 128, 1, 1, 128, 128, 64, True, 10000.0)
# the same attention shape with 4 experts of SwiGLU 128 and top-2 routing
TOY_MOE = synth.configs.ModelConfig("toy-moe-1layer", 1, 128, 1, 1, 128, 0, 64, True, 10000.0,
                                    n_experts=4, top_k=2, expert_ffn=128)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b(mk[bm]?_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 19, names
    lib = mk.load()
    for n in names:
        assert hasattr(lib, n), f"libmk.so does not export {n}"
    out = subprocess.run(["nm", "-D", "--defined-only", mk.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (\w+)", out.stdout))
    assert set(names) <= exported
    # nothing but the declared C entry points is exported with the mk prefix (no C++ mangling leaks)
    extra = {s for s in exported if re.match(r"mk[bm]?_", s)} - set(names)
    assert not extra, extra


def test_status_strings():
    lib = mk.load()
    for s in range(8):
        assert lib.mk_status_str(s)
    assert lib.mk_status_str(99) == b"unknown status"


class _Fake:
    """Stands in for a device tensor: planning reads shapes only, never the pointers."""

    def data_ptr(self):
        return 0x10000


def plan(cfg, W, B=1, C=2048, sched=0, policy=0, attn_splits=0):
    names = ["tok_embed", "final_norm"] + ([] if cfg.tied else ["lm_head"])
    for l in range(cfg.n_layers):
        ffn = ("router", "exp_gate", "exp_up", "exp_down") if cfg.n_experts else ("w_gate", "w_up", "w_down")
        names += [f"l{l}.{n}" for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm") + ffn]
    model = mk.Model(cfg, {n: _Fake() for n in names})
    opt = mk.options(sched=sched, policy=policy, attn_splits=attn_splits)
    return mk.parse_export(mk.mk_plan_graph(model.desc, B, C, opt, W))


def compare(ex, g, cfg, W, C, B=1):
    hd = ex["header"]
    t = g["tiling"]
    assert (hd["W"], hd["C"], hd["B"]) == (W, C, B)
    assert (hd["L"], hd["h"], hd["nq"], hd["nkv"], hd["d"], hd["f"], hd["V"]) == (
        cfg.n_layers, cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn, cfg.vocab)
    assert (hd["grp"], hd["qkv_pairs"], hd["attn_splits"], hd["o_rows"], hd["lm_rows"]) == (
        t["grp"], t["pairs"], t["S"], t["o_rows"], t["lm_rows"])
    if t["E"]:
        assert (hd["E"], hd["topk"], hd["fe"], hd["r_gu"], hd["r_dn"]) == (
            t["E"], t["topk"], t["fe"], t["r_gu"], t["r_dn"])
    else:
        assert (hd["g_rows"], hd["kd"], hd["d_rows"], hd["E"]) == (t["g_rows"], t["kd"], t["d_rows"], 0)
    assert hd["n_tasks"] == len(g["tasks"]) and hd["n_events"] == len(g["target"])
    rec = ex["tasks"]
    for name in rec.dtype.names:
        want = np.array([k[name] for k in g["tasks"]], dtype=rec.dtype[name])
        np.testing.assert_array_equal(rec[name], want, err_msg=f"task field {name}")
    np.testing.assert_array_equal(ex["target"], g["target"])
    np.testing.assert_array_equal(ex["nsub"], g["nsub"])
    np.testing.assert_array_equal(ex["order"], g["order"])
    qo = ex["queue_off"]
    for w in range(W):
        np.testing.assert_array_equal(ex["queue"][qo[w]:qo[w + 1]], g["queues"][w], err_msg=f"queue {w}")


def read_fixture(path=FIXTURE):
    rows, meta = [], {}
    for line in open(path):
        if line.startswith("#"):
            m = re.match(r"#\s*(targets|queue \d+):\s*(.*)", line)
            if m:
                meta[m.group(1)] = [int(x) for x in m.group(2).split()]
            continue
        if line.strip():
            f = line.split()
            num = lambda s: tg.NONE if s == "-" else int(s)
            rows.append(dict(id=int(f[0]), op=OPS[f[1]], layer=int(f[2]), part=int(f[3]), row0=int(f[4]),
                             nrows=int(f[5]), flags=int(f[6]), seq=int(f[7]), wait_ev=num(f[8]),
                             wait_target=int(f[9]), sig_ev=num(f[10]), wbytes=int(f[11]), wofs=int(f[12])))
    return rows, meta


def test_oracle_builder_matches_hand_derived_toy_graph():
    rows, meta = read_fixture()
    g = tg.build(TOY, 1, 64, 2)
    assert len(g["tasks"]) == len(rows) == 33
    for want, got in zip(rows, g["tasks"]):
        for k, v in want.items():
            assert got[k] == v, (want["id"], k, got[k], v)
    assert g["target"] == meta["targets"]
    assert g["queues"] == [meta["queue 0"], meta["queue 1"]]
    tg.check(g, TOY, 1)


def test_library_planner_matches_hand_derived_toy_graph():
    g = tg.build(TOY, 1, 64, 2)
    compare(plan(TOY, 2, C=64), g, TOY, 2, 64)


def _fixture_equals(path, g, n_tasks):
    rows, meta = read_fixture(path)
    assert len(g["tasks"]) == len(rows) == n_tasks
    for want, got in zip(rows, g["tasks"]):
        for k, v in want.items():
            assert got[k] == v, (want["id"], k, got[k], v)
    assert g["target"] == meta["targets"]
    assert g["queues"] == [meta["queue 0"], meta["queue 1"]]


def test_oracle_builder_matches_hand_derived_batch_graph():
    """Three sequences with four chunk slots each (dealt at run time): slot order 0, 1, 3, 2 outermost, then sequences;
    one event per KV group counting every slot task of every sequence (the O-projection waits for all of
    them, the run-time merge included); GEMV tiles of the single column group."""
    g = tg.build(TOY, 3, 64, 2, attn_splits=4)
    _fixture_equals(BATCH_FIXTURE, g, 44)
    tg.check(g, TOY, 3)


def test_library_planner_matches_hand_derived_batch_graph():
    g = tg.build(TOY, 3, 64, 2, attn_splits=4)
    _fixture_equals(BATCH_FIXTURE, g, 44)
    compare(plan(TOY, 2, B=3, C=64, attn_splits=4), g, TOY, 2, 64, B=3)


def test_oracle_builder_matches_hand_derived_moe_graph():
    """Four experts, top-2: one router tile raising every expert's event, each expert's gate/up tile raising
    its own, each expert's down tile waiting for its expert (two producers each) and feeding the layer's
    residual event (four producers)."""
    g = tg.build(TOY_MOE, 2, 64, 2)
    _fixture_equals(MOE_FIXTURE, g, 39)
    tg.check(g, TOY_MOE, 2)


def test_library_planner_matches_hand_derived_moe_graph():
    g = tg.build(TOY_MOE, 2, 64, 2)
    _fixture_equals(MOE_FIXTURE, g, 39)
    compare(plan(TOY_MOE, 2, B=2, C=64), g, TOY_MOE, 2, 64, B=2)


CASES = [
    (synth.configs.TINY, 1, 512, 0, 0, 0),
    (synth.configs.TINY, 4, 512, 0, 0, 0),
    (synth.configs.TINY, 37, 512, 1, 1, 0),
    (synth.configs.TINY.with_(tied=False), 256, 256, 0, 1, 3),
    (synth.configs.LLAMA_1B, 256, 2048, 0, 0, 0),
    (synth.configs.LLAMA_1B, 256, 2048, 1, 1, 0),
    (synth.configs.LLAMA_1B, 100, 8192, 0, 0, 0),
    (synth.configs.LLAMA_1B, 304, 4096, 0, 0, 5),
    (synth.configs.LLAMA_8B, 256, 4096, 0, 0, 0),
    (synth.configs.TINY, 4, 512, 2, 0, 0),
    (synth.configs.LLAMA_1B, 256, 2048, 2, 0, 0),
    (synth.configs.TINY, 4, 512, 3, 0, 0),
    (synth.configs.LLAMA_1B, 256, 2048, 3, 0, 0),
]


@pytest.mark.parametrize("cfg,W,C,sched,policy,splits", CASES,
                         ids=[f"{c[0].name}-W{c[1]}-C{c[2]}-s{c[3]}-p{c[4]}-a{c[5]}" for c in CASES])
def test_library_planner_equals_oracle_graph(cfg, W, C, sched, policy, splits):
    ex = plan(cfg, W, C=C, sched=sched, policy=policy, attn_splits=splits)
    g = tg.build(cfg, 1, C, W, policy=policy, attn_splits=splits, sched=sched)
    compare(ex, g, cfg, W, C)
    assert ex["header"]["sched"] == sched
    if cfg.n_layers <= 16:
        tg.check(g, cfg, 1)


BATCH_CASES = [
    (synth.configs.TINY, 3, 37, 512, 0),
    # batches whose row bound 1024 // B is not a power of two, with few workgroups
    # (tile heights then come from the bound)
    (synth.configs.TINY, 3, 4, 512, 0),
    (synth.configs.LLAMA_1B, 6, 32, 2048, 0),
    (synth.configs.TINY, 16, 256, 512, 1),
    (synth.configs.LLAMA_1B, 16, 256, 4352, 0),
    (synth.configs.LLAMA_1B, 4, 256, 2048, 1),
    (synth.configs.TINY, 20, 64, 512, 0),
    (synth.configs.LLAMA_1B, 32, 256, 4352, 0),
    (synth.configs.TINY_MOE, 5, 37, 512, 0),
    # one sequence with experts: the several-sequence path with a column group of one
    (synth.configs.TINY_MOE, 1, 16, 512, 0),
    (synth.configs.MOE_1B, 1, 256, 2048, 0),
    (synth.configs.TINY_MOE, 20, 64, 512, 1),
    (synth.configs.MOE_1B, 16, 256, 2048, 0),
    # three and four column groups of 16 sequences (the largest batch), with and without experts
    (synth.configs.TINY, 64, 64, 512, 0),
    (synth.configs.TINY_MOE, 37, 64, 512, 0),
    (synth.configs.TINY_MOE, 64, 128, 512, 1),
]


@pytest.mark.parametrize("cfg,B,W,C,policy", BATCH_CASES,
                         ids=[f"{c[0].name}-B{c[1]}-W{c[2]}-C{c[3]}-p{c[4]}" for c in BATCH_CASES])
def test_batched_planner_equals_oracle_graph(cfg, B, W, C, policy):
    """Batch > 1: attention tasks per sequence, tiles bounded by rows x sequences, GEMV tiles per column group,
    router and expert tasks for MoE; the library builds exactly the oracle's graph, which passes the checker
    and every simulated interleaving."""
    ex = plan(cfg, W, B=B, C=C, policy=policy)
    g = tg.build(cfg, B, C, W, policy=policy)
    compare(ex, g, cfg, W, C, B)
    tg.check(g, cfg, B)
    n = len(g["tasks"])
    assert tg.simulate(g, W, seed=B) == n
    assert tg.simulate(g, W, seed=B + 1, dynamic=True) == n
    assert tg.simulate(g, W, seed=B + 2, event=True) == n


def test_batched_checker_catches_an_oproj_that_skips_attention():
    cfg = synth.configs.TINY
    g = tg.build(cfg, 3, 512, 8)
    k = next(k for k in g["tasks"] if k["op"] == tg.OP_OPROJ and k["part"] == 1)
    k["wait_ev"] = next(t["sig_ev"] for t in g["tasks"] if t["op"] == tg.OP_QKV and t["part"] == 1)
    k["wait_target"] = g["target"][k["wait_ev"]]
    with pytest.raises(AssertionError):
        tg.check(g, cfg, 3)


def test_planner_rejects_what_it_does_not_implement():
    cfg = synth.configs.TINY
    with pytest.raises(mk.MkError):
        plan(cfg, 4, B=65)
    with pytest.raises(mk.MkError):
        plan(synth.configs.LLAMA_8B, 256, B=2)
    with pytest.raises(mk.MkError):
        plan(cfg.with_(head_dim=96), 4)
    with pytest.raises(mk.MkError):
        plan(cfg.with_(n_q=3), 4)
    with pytest.raises(mk.MkError):
        plan(cfg.with_(hidden=8192), 4)
    with pytest.raises(mk.MkError):
        plan(cfg.with_(hidden=64), 4)
    with pytest.raises(mk.MkError):  # the merges read at most 16 chunk partials
        plan(cfg, 16, B=3, attn_splits=17)
    assert plan(cfg, 16, B=3, attn_splits=16)["header"]["attn_splits"] == 16


def _plan_with(cfg, W, opt):
    names = ["tok_embed", "final_norm"] + ([] if cfg.tied else ["lm_head"])
    for l in range(cfg.n_layers):
        names += [f"l{l}.{n}" for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")]
    model = mk.Model(cfg, {n: _Fake() for n in names})
    return mk.mk_plan_graph(model.desc, 1, 512, opt, W)


def test_options_zero_filled_is_the_default_and_bad_values_are_refused():
    """A zero-filled mk_options is the default configuration (the same graph as NULL options); the page size
    is fixed at 16 KiB (0 or 16 accepted); poison is 0 or 1."""
    import ctypes
    cfg = synth.configs.TINY
    lib = mk.load()
    names = ["tok_embed", "final_norm"] + [f"l{l}.{n}" for l in range(cfg.n_layers)
                                           for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate",
                                                     "w_up", "w_down")]
    model = mk.Model(cfg, {n: _Fake() for n in names})
    need = ctypes.c_size_t(0)
    assert lib.mk_plan_graph(model.desc, 1, 512, None, 4, None, 0, ctypes.byref(need)) == mk.MK_E_INVALID
    buf = ctypes.create_string_buffer(need.value)
    assert lib.mk_plan_graph(model.desc, 1, 512, None, 4, buf, need.value, ctypes.byref(need)) == mk.MK_OK
    assert _plan_with(cfg, 4, mk.Options()) == buf.raw
    assert _plan_with(cfg, 4, mk.options(page_kib=16)) == buf.raw
    for bad in (mk.options(page_kib=8), mk.options(page_kib=32), mk.options(poison=2), mk.options(sched=4)):
        with pytest.raises(mk.MkError) as ei:
            _plan_with(cfg, 4, bad)
        assert ei.value.status == mk.MK_E_INVALID
    # the dropped-signal test hook: task n - 1 for a positive value, off for 0
    assert mk.options(drop_signal_of_task=0).debug_drop_signal == 1
    assert mk.options().debug_drop_signal == 0


@pytest.mark.parametrize("W", [1, 3, 16, 37])
@pytest.mark.parametrize("dynamic", [False, True])
def test_every_interleaving_completes(W, dynamic):
    cfg = synth.configs.TINY
    g = tg.build(cfg, 1, 512, W)
    n = len(g["tasks"])
    for seed in range(4):
        assert tg.simulate(g, W, seed=seed, dynamic=dynamic) == n
    # adversary: one workgroup moves only when nothing else can
    for slow in (0, W - 1):
        assert tg.simulate(g, W, seed=9, slow=slow, dynamic=dynamic) == n


def test_llama1b_graph_completes_under_random_interleaving():
    cfg = synth.configs.LLAMA_1B
    W = 256
    ex = tg.from_export(plan(cfg, W))
    n = len(ex["tasks"])
    assert tg.simulate(ex, W, seed=1) == n
    assert tg.simulate(ex, W, seed=2, dynamic=True, lookahead=2) == n


def test_checker_and_simulator_catch_planted_mistakes():
    """Mistakes planted in a copy of the oracle graph are caught (the checker is not vacuous)."""
    cfg = synth.configs.TINY
    W = 4
    base = tg.build(cfg, 1, 512, W)

    def planted(edit):
        g = tg.build(cfg, 1, 512, W)
        edit(g)
        return g

    def wrong_target(g):
        g["target"][3] -= 1

    def skip_wait(g):
        k = next(k for k in g["tasks"] if k["op"] == tg.OP_OPROJ and k["layer"] == 1)
        k["wait_ev"] = tg.NONE

    def wait_on_wrong_group(g):
        k = next(k for k in g["tasks"] if k["op"] == tg.OP_ATTN and k["part"] == 1)
        k["wait_ev"] -= 1

    def double_tile(g):
        a = next(k for k in g["tasks"] if k["op"] == tg.OP_GATEUP)
        a["row0"] += a["nrows"]

    def two_residuals(g):
        k = next(k for k in g["tasks"] if k["op"] == tg.OP_OPROJ and not k["flags"])
        k["flags"] = tg.TF_RESID

    def queue_out_of_order(g):
        q = g["queues"][1]
        q[2], q[3] = q[3], q[2]

    for edit in (wrong_target, skip_wait, wait_on_wrong_group, double_tile, two_residuals, queue_out_of_order):
        with pytest.raises(AssertionError):
            tg.check(planted(edit), cfg, 1)
    tg.check(base, cfg, 1)

    # a queue order that puts a consumer before its producer on the same workgroup deadlocks
    g = tg.build(cfg, 1, 512, 1)
    q = g["queues"][0]
    i = next(k["id"] for k in g["tasks"] if k["op"] == tg.OP_ATTN)
    q.remove(i)
    q.insert(0, i)
    assert tg.simulate(g, 1) < len(g["tasks"])


def test_checker_catches_planted_routing_mistakes():
    """Expert down tiles must follow every router tile: a router tile that raises only its first
    event (targets recounted to match) or a missing router row is caught."""
    cfg = synth.configs.TINY_MOE
    B, W = 5, 8

    def recount(g):
        g["target"] = [0] * len(g["target"])
        for k in g["tasks"]:
            for ev in tg.signals(k, cfg.n_experts):
                g["target"][ev] += 1
        for k in g["tasks"]:
            if k["wait_ev"] != tg.NONE:
                k["wait_target"] = g["target"][k["wait_ev"]]

    g = tg.build(cfg, B, 512, W)
    tg.check(g, cfg, B)
    k = next(k for k in g["tasks"] if k["op"] == tg.OP_ROUTE and k["layer"] == 1)
    k["flags"] &= ~tg.TF_SIGRANGE
    recount(g)
    with pytest.raises(AssertionError, match="before its producer"):
        tg.check(g, cfg, B)

    g = tg.build(cfg, B, 512, W)
    k = next(k for k in g["tasks"] if k["op"] == tg.OP_ROUTE)
    k["nrows"] -= 1
    with pytest.raises(AssertionError, match="router logits"):
        tg.check(g, cfg, B)


@pytest.mark.parametrize("cfg,B,W", [(synth.configs.TINY, 1, 1), (synth.configs.TINY, 1, 37),
                                     (synth.configs.TINY, 5, 8), (synth.configs.TINY_MOE, 5, 8)],
                         ids=["tiny-W1", "tiny-W37", "tiny-B5", "tiny-moe-B5"])
def test_event_driven_dispatch_completes(cfg, B, W):
    """Event-driven dispatch (tasks taken from a ready queue that each activated event extends with its
    dependents): every task is released exactly once, and random and adversarial interleavings finish."""
    g = tg.build(cfg, B, 512, W, sched=2)
    n = len(g["tasks"])
    released = sorted(g["init"] + [i for c in g["cons"] for i in c])
    assert released == list(range(n))
    assert all(n_ == 1 for n_ in g["nsub"])
    for seed in range(3):
        assert tg.simulate(g, W, seed=seed, event=True) == n
        # scheduler waves: events posted to scheduler ev % W, dispatched in id order
        assert tg.simulate(g, W, seed=seed, scheduler=True) == n
    assert tg.simulate(g, W, seed=7, event=True, slow=0) == n
    assert tg.simulate(g, W, seed=7, scheduler=True, slow=0) == n
    # an event whose count never completes (one producer's signal lost) stalls its dependents
    k = next(k for k in g["tasks"] if k["op"] == tg.OP_QKV and k["layer"] == 1)
    k["sig_ev"] = tg.NONE
    assert tg.simulate(g, W, seed=1, event=True) < n
