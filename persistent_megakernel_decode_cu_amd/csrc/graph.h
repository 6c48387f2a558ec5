// Host task-graph builder (no GPU calls); see graph.cpp.
#pragma once
#include <string>
#include <vector>

#include "mk_internal.h"

namespace mk {

struct Dims {
    int L, h, nq, nkv, d, f, V, n_experts, top_k, fe;
};

struct PlanOptions {
    int attn_splits;
};

struct Graph {
    Tiling T;
    Layout lay;
    uint32_t sched = 0;
    std::vector<Task> tasks;        // topological order
    std::vector<uint32_t> target;   // producers per event (per step)
    std::vector<uint32_t> nsub;     // sub-counters per event
    std::vector<uint32_t> queue_off, queue;  // static per-workgroup queues
    std::vector<uint32_t> order;    // dynamic queue (topological order)
    // event-driven dispatch (sched 2): the tasks released by each event, in task order
    // (cons[cons_off[e] .. cons_off[e + 1]]), and the tasks that wait on no event
    std::vector<uint32_t> cons_off, cons, init;
    uint32_t new_event();
};

int plan_tiling(const Dims& dm, int B, int C, int W, const PlanOptions& o, Tiling* t, std::string* err);
void plan_layout(const Tiling& T, bool tied, Layout* out);
int build_graph(const Tiling& T, const Layout& Ly, int sched, int policy, Graph* g);
// sub-counters, each event's dependents and the queues of a graph whose tasks and targets are built
void finish_graph(Graph& g, int sched, int policy);
// the prompt graph (prefill_graph.cpp): T tokens of one sequence per launch (dense models, head_dim 64,
// hidden <= 2048);
// *unsupported tells a valid shape this graph does not implement from a bad argument
int plan_prefill_tiling(const Dims& dm, int T, int C, int W, Tiling* t, std::string* err, bool* unsupported);
int build_prefill_graph(const Tiling& T, const Layout& Ly, int sched, int policy, Graph* g);
size_t export_size(const Graph& g);
size_t export_graph(const Graph& g, void* buf, size_t cap);

}  // namespace mk
