"""ORACLE — test infrastructure only.

Independent definition of the task graph the megakernel interprets: which tile
tasks exist, which event each one waits on and signals, how many producers
(targets) each event has, how the weight tiles are laid out, and how tasks are
placed on per-workgroup queues.  The C++ builder of the library must export
exactly this graph (bit for bit); the checker and the interleaving simulator
below verify the properties any such graph must have.

Vocabulary of the pages: tasks are the rectangles and events the circles of
MPK's task graph; a task's trigger edge goes to the event it completes, an
event's dependency edges go to the tasks it releases (MPK news page, part 1);
events are integer counters that a finishing task increments and a starting
task waits on until they reach their target (Hazy Research megakernel news
page, section 4, "synchronisation").  Static queues are per-workgroup lists
fixed before launch, the dynamic queue is one global list claimed by atomic
pops (koas-w.github.io notes, "static and dynamic scheduling").

The tiling rules (written from the design, not from the C++ code):
  * QKV tiles: 8 RoPE pairs (16 weight rows: 8 first halves then 8 second
    halves) of one head; heads ordered by KV group: the group's query heads,
    its key head, its value head; pair blocks in order.
  * the several-sequence rules below ("batch > 1") hold for every graph with
    experts too, at batch 1 as well: expert routing exists only on that path.
  * attention: attn_splits chunks per (sequence, KV group), default
    clamp(ceil(max_ctx / 256), 1, 16) at batch 1, clamp(pow2_floor(W /
    (B n_kv)), 1, 8) for batch 2 (and experts at batch 1) and clamp(pow2_floor(2 W /
    (B n_kv)), 1, 4) for batch > 2, at most max_ctx.  With several sequences the
    B S attention records of a KV group are slots (slot = seq S + chunk) that the
    device deals to the sequences at every step in proportion to their contexts
    (fake_device.py gives the rule); some slots may stay empty.  The last chunk
    task of a (sequence, KV group) to finish merges the chunks for the
    O-projection, which therefore waits on the same event as at batch 1.
  * O-proj tiles: (KV group g, row block) over columns g*grp*d .. +grp*d, with
    o_rows = min(h, R, max(16, pow2_floor(h * n_kv / W))), R = pow2_floor(1024 // min(B, 16)).
  * down tiles: (K block of kd = min(1024, f) columns, row block of
    d_rows = min(h, R, max(16, pow2_floor(h * (f / kd) / W))) rows).
  * gate/up tiles: g_rows gate rows then the same g_rows up rows, with
    g_rows = min(kd, R // 2, max(8, pow2_ceil(ceil(f / W)))).
  * LM head tiles: lm_rows = min(1024, ceil(V / W) rounded up to 16) rows, the
    last one shorter; its weight bytes are its rows rounded up to 16.  (With
    several sequences a workgroup takes an LM tile in chunks of
    (1024 // B) // 64 * 64 rows, so its row results stay within 1024 values.)
  * with more than 16 sequences every GEMV tile (QKV, O-proj, gate/up, down,
    LM head) is emitted once per column group of 16 sequences (task field seq =
    the group), group by group within each op, on the same weights.
  * per layer the events are created in the order qkv[g], attn[g], xb, m[kb],
    x_next; tasks in the order QKV, attention, O-proj, gate/up, down; then the
    LM-head tiles.  An event with more than 32 producers uses 8 sub-counters.
  * packed weights: gains ((2L+1) rows of h), embedding, LM-head tiles (always
    a copy of their own), then per layer QKV, O, gate/up, down regions, each
    region padded to 256 B, tiles inside a region in task order.
  * static queues: round-robin (task i -> workgroup i mod W) or least-loaded
    (cost = weight bytes + 8192, ties to the lowest workgroup); the dynamic
    queue is the task order itself.
"""
import math

import numpy as np

OP_QKV, OP_ATTN, OP_OPROJ, OP_GATEUP, OP_DOWN, OP_LMHEAD, OP_ROUTE, OP_EGU, OP_EDOWN = 1, 2, 3, 4, 5, 6, 7, 8, 9
NONE = 0xFFFFFFFF
TF_RESID = 1
TF_SIGRANGE = 2  # a router tile raises the events of all E experts, sig_ev .. sig_ev + E - 1


def signals(k, E):
    """The events task k raises when it finishes."""
    if k["sig_ev"] == NONE:
        return []
    return [k["sig_ev"] + i for i in range(E)] if k["flags"] & TF_SIGRANGE else [k["sig_ev"]]


def idle_units_in_last_wave(n_tasks, n_units):
    """Units left without work in the last wave when n_tasks equal tasks run in
    waves over n_units units (the tail effect of a one-kernel-per-op launch)."""
    rem = n_tasks % n_units
    return 0 if rem == 0 else n_units - rem


def _pow2_floor(x):
    p = 1
    while p * 2 <= x:
        p *= 2
    return p


def _pow2_ceil(x):
    p = 1
    while p < x:
        p *= 2
    return p


def _pad(x):
    return (x + 255) // 256 * 256


def _round16(x):
    return (x + 15) // 16 * 16


def tiling(cfg, B, C, W, attn_splits=0):
    h, nq, nkv, d, f, V = cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn, cfg.vocab
    grp = nq // nkv
    several = B > 1 or cfg.n_experts > 0
    if attn_splits > 0:
        S = attn_splits
    else:
        # batch 1: 256-position chunks; batch > 1: about one attention task per
        # workgroup and layer over all sequences and KV groups, at most 8 slots
        S = max(1, min(16, -(-C // 256))) if not several else (
            max(1, min(8, _pow2_floor(max(1, W // (B * nkv))))) if B <= 2 else
            max(1, min(4, _pow2_floor(max(1, 2 * W // (B * nkv))))))
    S = min(S, C)
    max_rows = _pow2_floor(1024 // min(B, 16))  # rows x sequences (of one column group) of a tile
    E = cfg.n_experts
    if E:  # mixture of experts: about one expert gate/up tile and one expert down tile per workgroup
        fe = cfg.expert_ffn
        return dict(grp=grp, pairs=8, S=S,
                    o_rows=min(h, max_rows, max(16, _pow2_floor(h * nkv // W))),
                    E=E, topk=cfg.top_k, fe=fe,
                    r_gu=min(fe, max(32, _pow2_floor(E * fe // W))),
                    r_dn=min(h, max(64, _pow2_floor(E * h // W))),
                    lm_rows=min(1024, _round16(-(-V // W))))
    kd = min(1024, f)
    return dict(grp=grp, pairs=8, S=S, E=0,
                o_rows=min(h, max_rows, max(16, _pow2_floor(h * nkv // W))),
                kd=kd, d_rows=min(h, max_rows, max(16, _pow2_floor(h * (f // kd) // W))),
                g_rows=min(kd, max_rows // 2, max(8, _pow2_ceil(-(-f // W)))),
                lm_rows=min(1024, _round16(-(-V // W))))


def layout(cfg, lm_rows, n_lm):
    h, L = cfg.hidden, cfg.n_layers
    at = 0
    lay = {"gains": at}
    at = _pad(at + (2 * L + 1) * h * 2)
    lay["embed"] = at
    at = _pad(at + cfg.vocab * h * 2)
    lay["lm"] = at  # own copy even when tied (tiles in GEMV page order)
    at = _pad(at + n_lm * lm_rows * h * 2)
    lay["layer0"] = at
    x = 0
    lay["qkv"] = x
    x = _pad(x + (cfg.n_q + 2 * cfg.n_kv) * cfg.head_dim * h * 2)
    lay["o"] = x
    x = _pad(x + h * cfg.n_q * cfg.head_dim * 2)
    if cfg.n_experts:
        E, fe = cfg.n_experts, cfg.expert_ffn
        lay["router"] = x  # E rows padded to 16
        x = _pad(x + _round16(E) * h * 2)
        lay["egu"] = x
        x = _pad(x + 2 * E * fe * h * 2)
        lay["edown"] = x
        x = _pad(x + E * h * fe * 2)
    else:
        lay["gu"] = x
        x = _pad(x + 2 * cfg.ffn * h * 2)
        lay["down"] = x
        x = _pad(x + h * cfg.ffn * 2)
    lay["layer_bytes"] = x
    return lay


def build(cfg, B, C, W, policy=0, attn_splits=0, sched=0):
    """The task graph as a list of task dicts plus event targets, sub-counter
    counts, static queues, the dynamic order and, for event-driven dispatch
    (sched 2), the dependents of every event and the tasks that wait on none."""
    t = tiling(cfg, B, C, W, attn_splits)
    n_lm = -(-cfg.vocab // t["lm_rows"])
    lay = layout(cfg, t["lm_rows"], n_lm)
    h, nq, nkv, d, f, L = cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn, cfg.n_layers
    grp, P, S = t["grp"], t["pairs"], t["S"]
    E = t["E"]
    n_kb = 0 if E else f // t["kd"]
    n_sg = -(-B // 16)  # column groups of 16 sequences
    tasks, target = [], []

    def event():
        target.append(0)
        return len(target) - 1

    def task(**k):
        rec = dict(op=0, flags=0, layer=0, part=0, row0=0, nrows=0, wait_ev=NONE, sig_ev=NONE, wbytes=0, wofs=0,
                   seq=0)
        rec.update(k)
        rec["id"] = len(tasks)
        for ev in signals(rec, E):
            target[ev] += 1
        tasks.append(rec)

    ev_x = NONE
    for l in range(L):
        base = lay["layer0"] + l * lay["layer_bytes"]
        ev_qkv = [event() for _ in range(nkv)]
        ev_attn = [event() for _ in range(nkv)]
        ev_xb = event()
        ev_m = [event() for _ in range(n_kb)]
        ev_me = [event() for _ in range(E)]
        ev_next = event()
        wb = 2 * P * h * 2
        for sg in range(n_sg):
            tile = 0
            for g in range(nkv):
                heads = [g * grp + s for s in range(grp)] + [nq + g, nq + nkv + g]
                for slot in heads:
                    for pb in range(d // 2 // P):
                        task(op=OP_QKV, layer=l, part=slot, row0=pb * P, nrows=P, seq=sg, wait_ev=ev_x,
                             sig_ev=ev_qkv[g], wbytes=wb, wofs=base + lay["qkv"] + tile * wb)
                        tile += 1
        # several sequences: chunk slots in the order 0, 1, .., S/2 - 1, S - 1, .., S/2 (outermost),
        # so that round-robin queues pair slot c with slot S - 1 - c; one sequence: per group
        if B > 1 or E:
            corder = list(range((S + 1) // 2)) + list(range(S - 1, (S + 1) // 2 - 1, -1))
            attn = [(b, g, c) for c in corder for b in range(B) for g in range(nkv)]
        else:
            attn = [(0, g, c) for g in range(nkv) for c in range(S)]
        for b, g, c in attn:
            task(op=OP_ATTN, layer=l, part=g, row0=c, nrows=grp, seq=b, wait_ev=ev_qkv[g], sig_ev=ev_attn[g])
        wb = t["o_rows"] * grp * d * 2
        for sg in range(n_sg):
            for g in range(nkv):
                for rb in range(h // t["o_rows"]):
                    task(op=OP_OPROJ, layer=l, part=g, row0=rb * t["o_rows"], nrows=t["o_rows"], seq=sg,
                         flags=TF_RESID if g == 0 else 0, wait_ev=ev_attn[g], sig_ev=ev_xb, wbytes=wb,
                         wofs=base + lay["o"] + (g * (h // t["o_rows"]) + rb) * wb)
        if E:
            # router tiles of 16 experts' logits, each raising every expert's event; every
            # expert's gate/up tiles (r_gu rows of m, gate and up interleaved by 32), which
            # need only the normalised residual; its down tiles, which apply the routing
            for sg in range(n_sg):
                for r0 in range(0, E, 16):
                    task(op=OP_ROUTE, layer=l, row0=r0, nrows=min(16, E - r0), seq=sg, flags=TF_SIGRANGE,
                         wait_ev=ev_xb, sig_ev=ev_me[0], wbytes=16 * h * 2, wofs=base + lay["router"] + r0 * h * 2)
            fe, rg, rd = t["fe"], t["r_gu"], t["r_dn"]
            wb = 2 * rg * h * 2
            for sg in range(n_sg):
                for e in range(E):
                    for i in range(fe // rg):
                        task(op=OP_EGU, layer=l, part=e, row0=i * rg, nrows=rg, seq=sg, wait_ev=ev_xb,
                             sig_ev=ev_me[e], wbytes=wb, wofs=base + lay["egu"] + (e * (fe // rg) + i) * wb)
            wb = rd * fe * 2
            for sg in range(n_sg):
                for e in range(E):
                    for rb in range(h // rd):
                        task(op=OP_EDOWN, layer=l, part=e, row0=rb * rd, nrows=rd, seq=sg,
                             wait_ev=ev_me[e], sig_ev=ev_next, wbytes=wb,
                             wofs=base + lay["edown"] + (e * (h // rd) + rb) * wb)
            ev_x = ev_next
            continue
        wb = 2 * t["g_rows"] * h * 2
        for sg in range(n_sg):
            for i in range(f // t["g_rows"]):
                task(op=OP_GATEUP, layer=l, row0=i * t["g_rows"], nrows=t["g_rows"], seq=sg, wait_ev=ev_xb,
                     sig_ev=ev_m[i * t["g_rows"] // t["kd"]], wbytes=wb, wofs=base + lay["gu"] + i * wb)
        wb = t["d_rows"] * t["kd"] * 2
        for sg in range(n_sg):
            for kb in range(n_kb):
                for rb in range(h // t["d_rows"]):
                    task(op=OP_DOWN, layer=l, part=kb, row0=rb * t["d_rows"], nrows=t["d_rows"], seq=sg,
                         flags=TF_RESID if kb == 0 else 0, wait_ev=ev_m[kb], sig_ev=ev_next, wbytes=wb,
                         wofs=base + lay["down"] + (kb * (h // t["d_rows"]) + rb) * wb)
        ev_x = ev_next
    for sg in range(n_sg):
        for i in range(n_lm):
            rows = min(t["lm_rows"], cfg.vocab - i * t["lm_rows"])
            task(op=OP_LMHEAD, layer=L, row0=i * t["lm_rows"], nrows=rows, seq=sg, wait_ev=ev_x,
                 wbytes=_round16(rows) * h * 2, wofs=lay["lm"] + i * t["lm_rows"] * h * 2)
    # events with more than 4 producers spread their counts over the device's counter words
    # (recorded as nsub 8), except under event-driven dispatch, where one counter per event
    # tells its last producer
    nsub = [8 if n > 4 and sched < 2 else 1 for n in target]
    for k in tasks:
        k["wait_target"] = target[k["wait_ev"]] if k["wait_ev"] != NONE else 0
        k["wait_nsub"] = nsub[k["wait_ev"]] if k["wait_ev"] != NONE else 1
        k["sig_nsub"] = nsub[k["sig_ev"]] if k["sig_ev"] != NONE else 1
    queues = [[] for _ in range(W)]
    if policy == 0:
        for i in range(len(tasks)):
            queues[i % W].append(i)
    else:
        load = [0] * W
        for i, k in enumerate(tasks):
            w = min(range(W), key=lambda j: (load[j], j))
            load[w] += k["wbytes"] + 8192
            queues[w].append(i)
    cons = [[] for _ in target]
    for k in tasks:
        if k["wait_ev"] != NONE:
            cons[k["wait_ev"]].append(k["id"])
    init = [k["id"] for k in tasks if k["wait_ev"] == NONE]
    return dict(tiling=t, layout=lay, tasks=tasks, target=target, nsub=nsub, queues=queues,
                order=list(range(len(tasks))), cons=cons, init=init)


# ---- checker (properties every valid graph has) -----------------------------------------

def check(g, cfg, B):
    """Checks coverage, targets, dependency soundness, queue validity; raises AssertionError."""
    tasks, target = g["tasks"], g["target"]
    consumers = {}
    for k in tasks:
        if k["wait_ev"] != NONE:
            consumers.setdefault(k["wait_ev"], []).append(k["id"])
    h, nq, nkv, d, f, L, V = cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim, cfg.ffn, cfg.n_layers, cfg.vocab
    grp = nq // nkv
    n_sg = -(-B // 16)
    E = g["tiling"]["E"]
    DOWN = OP_EDOWN if E else OP_DOWN  # the op that completes a layer
    # G2 targets = producers
    prod = [0] * len(target)
    for k in tasks:
        for ev in signals(k, E):
            prod[ev] += 1
    assert prod == list(target), "event targets differ from producer counts"
    for k in tasks:
        if k["wait_ev"] != NONE:
            assert k["wait_target"] == target[k["wait_ev"]]
    # G1 coverage
    for l in range(L):
        lt = [k for k in tasks if k["layer"] == l]
        # every GEMV output is produced exactly once per column group of 16 sequences
        cov = np.zeros((n_sg, nq + 2 * nkv, d // 2), int)
        for k in lt:
            if k["op"] == OP_QKV:
                cov[k["seq"], k["part"], k["row0"]:k["row0"] + k["nrows"]] += 1
        assert (cov == 1).all(), "QKV pairs not covered exactly once"
        o = np.zeros((n_sg, h, nkv), int)
        for k in lt:
            if k["op"] == OP_OPROJ:
                o[k["seq"], k["row0"]:k["row0"] + k["nrows"], k["part"]] += 1
        assert (o == 1).all(), "O-proj (row, group) not covered exactly once"
        if E:
            fe = g["tiling"]["fe"]
            rt = np.zeros((n_sg, E), int)
            egu = np.zeros((n_sg, E, fe), int)
            edn = np.zeros((n_sg, E, h), int)
            for k in lt:
                if k["op"] == OP_ROUTE:
                    rt[k["seq"], k["row0"]:k["row0"] + k["nrows"]] += 1
                if k["op"] == OP_EGU:
                    egu[k["seq"], k["part"], k["row0"]:k["row0"] + k["nrows"]] += 1
                if k["op"] == OP_EDOWN:
                    edn[k["seq"], k["part"], k["row0"]:k["row0"] + k["nrows"]] += 1
            assert (rt == 1).all(), "router logits not covered exactly once per column group"
            assert (egu == 1).all(), "expert gate/up rows not covered exactly once"
            assert (edn == 1).all(), "expert down rows not covered exactly once"
        else:
            gu = np.zeros((n_sg, f), int)
            for k in lt:
                if k["op"] == OP_GATEUP:
                    gu[k["seq"], k["row0"]:k["row0"] + k["nrows"]] += 1
            assert (gu == 1).all(), "gate/up rows not covered exactly once"
            kd = g["tiling"]["kd"]
            dn = np.zeros((n_sg, h, f // kd), int)
            for k in lt:
                if k["op"] == OP_DOWN:
                    dn[k["seq"], k["row0"]:k["row0"] + k["nrows"], k["part"]] += 1
            assert (dn == 1).all(), "down (row, K block) not covered exactly once"
        at = np.zeros((B, nkv, g["tiling"]["S"]), int)
        for k in lt:
            if k["op"] == OP_ATTN:
                at[k["seq"], k["part"], k["row0"]] += 1
        assert (at == 1).all(), "attention chunks not covered exactly once"
        # exactly one residual-adding tile per O-proj / down row
        r1 = np.zeros((n_sg, h), int)
        r2 = np.zeros((n_sg, h), int)
        for k in lt:
            if k["op"] == OP_OPROJ and k["flags"] & TF_RESID:
                r1[k["seq"], k["row0"]:k["row0"] + k["nrows"]] += 1
            if k["op"] == DOWN and k["flags"] & TF_RESID:
                r2[k["seq"], k["row0"]:k["row0"] + k["nrows"]] += 1
        # (with experts, the residual rides on each sequence's first-choice expert: no tile flag,
        # and every expert's down tiles cover every row, checked above)
        assert (r1 == 1).all() and (r2 == (0 if E else 1)).all(), "residual added more or less than once"
    lm = np.zeros((n_sg, V), int)
    for k in tasks:
        if k["op"] == OP_LMHEAD:
            lm[k["seq"], k["row0"]:k["row0"] + k["nrows"]] += 1
    assert (lm == 1).all(), "LM-head rows not covered exactly once"
    # G3 soundness: every reader starts after every writer of what it reads, through the event edges
    hb_sets = ancestor_sets(g)
    by = {}
    for k in tasks:
        by.setdefault((k["op"], k["layer"]), []).append(k)
    kd = g["tiling"].get("kd", 0)

    def ids(op, layer, pred=lambda w: True):
        return {w["id"] for w in by.get((op, layer), []) if pred(w)}

    def group_of_slot(s):
        return s // grp if s < nq else (s - nq) % nkv

    checked = set()
    for k in tasks:
        l, op = k["layer"], k["op"]
        key = (op, l, k["part"] if op in (OP_ATTN, OP_OPROJ, OP_DOWN, OP_EDOWN) else 0, k["wait_ev"])
        if key in checked:
            continue
        checked.add(key)
        need = set()
        prev = ids(DOWN, l - 1) if l > 0 else set()
        if op == OP_QKV:
            need = prev
        elif op == OP_ATTN:
            need = ids(OP_QKV, l, lambda w: group_of_slot(w["part"]) == k["part"])
        elif op == OP_OPROJ:
            # batch > 1: the last attention chunk of a (sequence, KV group) merges the
            # chunks into the O-projection's operands, so all of them precede it
            need = ids(OP_ATTN, l, lambda w: w["part"] == k["part"]) | prev
        elif op == OP_GATEUP:
            need = ids(OP_OPROJ, l)
        elif op == OP_DOWN:
            need = ids(OP_GATEUP, l, lambda w: w["row0"] // kd == k["part"]) | ids(OP_OPROJ, l)
        elif op == OP_ROUTE:
            need = ids(OP_OPROJ, l)
        elif op == OP_EGU:  # the normalised residual
            need = ids(OP_OPROJ, l)
        elif op == OP_EDOWN:  # its expert's m rows, every router logit (the routing) and the residual
            need = ids(OP_EGU, l, lambda w: w["part"] == k["part"]) | ids(OP_ROUTE, l) | ids(OP_OPROJ, l)
        elif op == OP_LMHEAD and L > 0:
            need = ids(DOWN, L - 1)
        anc = hb_sets(k["id"])
        missing = need - anc
        assert not missing, f"task {k['id']} may start before its producer(s) {sorted(missing)[:4]}"
    # buffers reused from one layer to the next (q/k/v, attention partials, m): every reader of
    # layer l happens before every writer of layer l+1
    for l in range(L - 1):
        for rop, wop in ((OP_ATTN, OP_QKV), (OP_ATTN if B > 1 else OP_OPROJ, OP_ATTN),
                         (OP_EDOWN, OP_EGU) if E else (OP_DOWN, OP_GATEUP)):
            rs = ids(rop, l)
            for w in by.get((wop, l + 1), []):
                missing = rs - hb_sets(w["id"])
                assert not missing, f"writer {w['id']} of layer {l + 1} may overtake readers {sorted(missing)[:4]}"
    # G4 queues: every task exactly once, each queue in increasing (topological) order
    seen = sorted(i for q in g["queues"] for i in q)
    assert seen == list(range(len(tasks))), "static queues do not hold every task exactly once"
    for q in g["queues"]:
        assert all(a < b for a, b in zip(q, q[1:])), "a static queue is not in task order"
    assert list(g["order"]) == list(range(len(tasks))), "the dynamic order is not the task order"
    for k in tasks:
        for ev in signals(k, E):
            for c in consumers.get(ev, []):
                assert k["id"] < c, "a producer comes after its consumer in the task order"
    # G5 weights: the tiles of each packed region cover it exactly, without overlap
    lay = g.get("layout")
    if lay is None:
        return
    # (the tiles of column groups past the first read the first group's tiles)
    first = {(k["op"], k["layer"], k["part"], k["row0"]): (k["wofs"], k["wbytes"]) for k in tasks if k["seq"] == 0}
    for k in tasks:
        if k["wbytes"] and k["op"] != OP_ATTN and k["seq"] > 0:
            assert first[(k["op"], k["layer"], k["part"], k["row0"])] == (k["wofs"], k["wbytes"]), \
                "a column group's tile reads other weights than the first group's"
    tasks = [k for k in tasks if k["op"] == OP_ATTN or k["seq"] == 0]
    spans = sorted((k["wofs"], k["wbytes"], k["op"]) for k in tasks if k["wbytes"] and k["op"] != OP_LMHEAD)
    pos = lay["layer0"]
    for ofs, nb, op in spans:
        assert ofs == pos or (ofs > pos and ofs - pos < 256), f"gap or overlap in packed weights at {ofs}"
        pos = ofs + nb
    assert pos <= lay["layer0"] + L * lay["layer_bytes"]
    lm = sorted((k["wofs"], k["wbytes"]) for k in tasks if k["op"] == OP_LMHEAD)
    pos = lay["lm"]
    for ofs, nb in lm:
        assert ofs == pos
        pos += nb
    assert pos == lay["lm"] + _round16(V) * h * 2


def ancestor_sets(g):
    """Returns anc(i): the set of tasks that finish before task i can start, through event edges."""
    tasks = g["tasks"]
    E = g["tiling"].get("E", 0)
    producers = {}
    for k in tasks:
        for ev in signals(k, E):
            producers.setdefault(ev, []).append(k["id"])
    memo = {}
    # events are created in topological order, so one forward pass fills the table
    for e in range(len(g["target"])):
        s = set()
        for p in producers.get(e, []):
            s.add(p)
            we = tasks[p]["wait_ev"]
            if we != NONE:
                assert we < e, "an event waits on a later event"
                s |= memo[we]
        memo[e] = frozenset(s)
    return lambda i: memo[tasks[i]["wait_ev"]] if tasks[i]["wait_ev"] != NONE else frozenset()


def simulate(g, W, seed=0, slow=None, dynamic=False, lookahead=2, event=False, scheduler=False):
    """Runs the graph on W virtual workgroups under a seeded random interleaving.

    scheduler (implies event): an activated event is not dispatched at once but
    posted to the queue of scheduler ev % W, which dispatches its events in id
    order, each once it has been activated (one more kind of move).

    Static: each workgroup runs its queue in order.  Dynamic: a workgroup claims
    the next task of the global order whenever it holds fewer than `lookahead`
    claimed tasks (the loader claims ahead of the compute waves), and runs its
    oldest claimed task.  Event-driven: the same claims, but of the next slot of a
    ready queue that starts with the tasks that wait on no event; when a task's count
    completes an event, the event's dependents are appended to the queue, and a
    claimed slot can run only once it is filled.  A task may run once its event
    counter has reached its target.  `slow`: a workgroup that only moves when no
    other one can.  Returns the number of tasks that ran (all of them unless the
    graph deadlocks).
    """
    rng = np.random.default_rng(seed)
    tasks = g["tasks"]
    E = g["tiling"].get("E", 0)
    ctr = [0] * len(g["target"])
    n = len(tasks)
    n_ev = len(g["target"])
    event = event or scheduler
    next_ev = list(range(W))  # each scheduler's next event: w, w + W, ...
    if event:
        dynamic = True
        rq = list(g["init"])  # the ready queue: filled slots
        if "cons" in g:
            cons = g["cons"]
        else:
            cons = [[] for _ in g["target"]]
            for k in tasks:
                if k["wait_ev"] != NONE:
                    cons[k["wait_ev"]].append(k["id"])
    if dynamic:
        order = list(g["order"])
        nxt = 0
        held = [[] for _ in range(W)]  # claimed slots (event) or task ids
    else:
        queues = [list(q) for q in g["queues"]]
        pos = [0] * W
    done = 0

    def head(w):
        if dynamic:
            if not held[w]:
                return None
            if event:
                s = held[w][0]
                return rq[s] if s < len(rq) else None
            return held[w][0]
        return queues[w][pos[w]] if pos[w] < len(queues[w]) else None

    while True:
        moves = []
        for w in range(W):
            i = head(w)
            if i is not None:
                k = tasks[i]
                if k["wait_ev"] == NONE or ctr[k["wait_ev"]] >= k["wait_target"]:
                    moves.append((w, "run"))
            if dynamic and len(held[w]) < lookahead and nxt < n:
                moves.append((w, "claim"))
            if scheduler and next_ev[w] < n_ev and ctr[next_ev[w]] >= g["target"][next_ev[w]]:
                moves.append((w, "dispatch"))
        if not moves:
            break
        if slow is not None:
            others = [m for m in moves if m[0] != slow]
            if others:
                moves = others
        w, what = moves[rng.integers(len(moves))]
        if what == "claim":
            held[w].append(nxt if event else order[nxt])
            nxt += 1
            continue
        if what == "dispatch":
            rq.extend(cons[next_ev[w]])
            next_ev[w] += W
            continue
        if dynamic:
            s = held[w].pop(0)
            i = rq[s] if event else s
        else:
            i = queues[w][pos[w]]
            pos[w] += 1
        k = tasks[i]
        for ev in signals(k, E):
            ctr[ev] += 1
            if event and not scheduler and ctr[ev] == g["target"][ev]:
                rq.extend(cons[ev])
        done += 1
    return done


def from_export(ex):
    """The library's exported graph in this module's dict form (for check and simulate)."""
    hd = ex["header"]
    names = ex["tasks"].dtype.names
    tasks = [{n: int(r[n]) for n in names} for r in ex["tasks"]]
    qo = ex["queue_off"]
    queues = [list(map(int, ex["queue"][qo[w]:qo[w + 1]])) for w in range(hd["W"])]
    return dict(tasks=tasks, target=list(map(int, ex["target"])), nsub=list(map(int, ex["nsub"])),
                queues=queues, order=list(map(int, ex["order"])),
                tiling=dict(kd=hd["kd"], S=hd["attn_splits"], E=hd["E"]), layout=None)
