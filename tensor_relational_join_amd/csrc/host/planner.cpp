// planner.cpp -- logical optimization ("Every Kernel Is a Join", section 4):
// choose one join-agg spec per abstract operator of a computation graph so as
// to minimize the communication-cost proxy of section 4.3, with the dynamic
// program over output tilings of section 4.2 and the graph cuts of section 4.5.
//
// A view (ja_graph_add_view) re-indexes a tensor by a reshape and a
// permutation of axes; it is realised by a repartition into whatever blocking
// each consumer asks for, so it frees the tilings on both sides and every
// edge out of it costs one full repartition.
//
// Candidate specs of an operator cut its shardable indices into near-equal
// intervals whose counts multiply to the processor count p (section 3.3 asks
// for one function spec per combination of intervals; section 4.3 for
// near-equal intervals).  A tiling of a tensor is then fixed by its interval
// count per dimension.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <map>
#include <queue>

#include "ja_host.h"

namespace ja {
namespace {

struct GTensor {
    std::vector<int64_t> shape;
    int producer = -1;                          // operator, or -1 for a computation input or a view
    int view_of = -1;                           // a view: the tensor it re-indexes
    std::vector<std::pair<int, int>> consumers;  // (operator, input slot)
    double numel() const {
        double n = 1;
        for (int64_t e : shape) n *= (double)e;
        return n;
    }
};

struct Cand {
    std::vector<int32_t> cnt;               // intervals per letter (letter order)
    std::vector<std::vector<int32_t>> in;  // tiling of each input: counts per dimension
    std::vector<int32_t> out;               // tiling of the output
    double join = 0, agg = 0;
    double dev_us = 0;                      // device-time model of the operator under this spec
};

struct GOp {
    ja_spec spec;
    std::vector<int> inputs;
    int out = -1;
    std::vector<int64_t> ext;  // letter order
    std::vector<Cand> cands;
    int chosen = -1;
};

}  // namespace
}  // namespace ja

struct ja_graph {
    std::vector<ja::GTensor> t;
    std::vector<ja::GOp> ops;
};

namespace ja {
namespace {

// Letters an operator may split (section 3.3): every index of a contraction
// and of an elementwise join ("any"); for attention the key-value batch and
// head letters and the two sequence letters (the query-head group letters and
// the head dimension are not directly shardable); for RMSNorm the row and the
// feature letter.
std::vector<bool> shardable(const ja_spec& s) {
    std::vector<bool> sh(s.letters.size(), true);
    if (s.kind == JA_OP_ATTENTION) {
        const std::string &q = s.ins[0], &k = s.ins[1];
        for (size_t i = 0; i < s.letters.size(); ++i) {
            const char c = s.letters[i];
            sh[i] = k.find(c) != std::string::npos || c == s.att_s;
        }
        sh[s.letter_index(q.back())] = false;
    }
    return sh;
}

void enum_counts(const std::vector<int64_t>& ext, const std::vector<bool>& sh, size_t i, int64_t left,
                 std::vector<int32_t>& cur, std::vector<std::vector<int32_t>>& out) {
    if (i == ext.size()) {
        if (left == 1) out.push_back(cur);
        return;
    }
    const int64_t hi = sh[i] ? std::min<int64_t>(ext[i], left) : 1;
    for (int64_t c = 1; c <= hi; ++c) {
        if (left % c) continue;
        cur[i] = (int32_t)c;
        enum_counts(ext, sh, i + 1, left / c, cur, out);
    }
}

std::vector<int32_t> tiling_of(const ja_spec& s, const std::string& letters, const std::vector<int32_t>& cnt) {
    std::vector<int32_t> t;
    for (char c : letters) t.push_back(cnt[s.letter_index(c)]);
    return t;
}

// Join and aggregation sub-costs (section 4.3) of one candidate: the kept
// cells of the interval grid are its function specifications.  Join: the
// elements of every input block of every function specification.
// Aggregation: for each distinct aggregated type, (copies - 1) times its
// elements -- the output blocks of a contraction or attention (copies = the
// cells sharing the output key), the per-row sums of squares of RMSNorm
// (copies = the feature intervals of a row interval); nothing for the 1:1
// joins.
void sub_costs(const GOp& op, Cand& c) {
    const ja_spec& s = op.spec;
    const int nl = (int)s.letters.size();
    std::vector<std::vector<int64_t>> sp(nl);
    for (int i = 0; i < nl; ++i) sp[i] = equal_splits(op.ext[i], c.cnt[i]);
    auto len = [&](int l, int64_t k) { return (double)(sp[l][k + 1] - sp[l][k]); };
    const int is = s.causal ? s.letter_index(s.causal_s) : -1, it = s.causal ? s.letter_index(s.causal_t) : -1;
    std::map<std::vector<int64_t>, std::pair<int64_t, double>> groups;  // key -> (copies, elements)
    std::vector<int64_t> idx(nl, 0);
    int64_t ncell = 1;
    for (int i = 0; i < nl; ++i) ncell *= c.cnt[i];
    c.join = c.agg = 0;
    for (int64_t cell = 0; cell < ncell; ++cell) {
        int64_t r = cell;
        for (int i = nl - 1; i >= 0; --i) {
            idx[i] = r % c.cnt[i];
            r /= c.cnt[i];
        }
        if (is >= 0 && sp[it][idx[it]] >= sp[is][idx[is] + 1]) continue;  // dropped by the causal predicate
        for (const std::string& in : s.ins) {
            double n = 1;
            for (char ch : in) n *= len(s.letter_index(ch), idx[s.letter_index(ch)]);
            c.join += n;
        }
        if (s.kind == JA_OP_CONTRACT || s.kind == JA_OP_ATTENTION || s.kind == JA_OP_RMSNORM) {
            const std::string agg = s.kind == JA_OP_RMSNORM ? s.out.substr(0, 1) : s.out;
            std::vector<int64_t> key;
            double n = 1;
            for (char ch : agg) {
                key.push_back(idx[s.letter_index(ch)]);
                n *= len(s.letter_index(ch), idx[s.letter_index(ch)]);
            }
            auto& g = groups[key];
            g.first += 1;
            g.second = n;
        }
    }
    for (auto& kv : groups) c.agg += (double)(kv.second.first - 1) * kv.second.second;
}

// ---- device-time model of this library's kernels on one MI355X -----------
// The pages' proxy ignores computation (section 4.3) and name computation
// awareness as future work (section 8).  On one GPU the join and the
// aggregation are fused into the kernels, so the time of a plan is its
// kernels' time plus its repartitions' copies.  Model: a contraction is
// 256 x 256 output tiles, each taking its segment's contracted extent at the
// measured per-CU rate of the fused bf16 contraction, placed longest first on
// the least loaded of 256 CUs; attention is 128-query-row tiles costed by the
// keys they see, at the measured attention rate; RMSNorm, SwiGLU, add and
// repartitions move their bytes at the measured copy rate; every launch adds
// a fixed latency.
constexpr int DEV_CUS = 256;
constexpr double DEV_GEMM_CU_FLOPS = 1213e12 / DEV_CUS;  // measured fused bf16 contraction, per CU
constexpr double DEV_ATTN_CU_FLOPS = 775e12 / DEV_CUS;   // measured causal attention, per CU
constexpr double DEV_COPY_BPS = 5.0e12;                  // measured plain device copy, bytes/s
constexpr double DEV_LAUNCH_US = 4.0;                    // per kernel launch
constexpr int DEV_GEMM_TILE = 256, DEV_ATTN_ROWS = 128;
constexpr double DEV_HALF_TILE = 0.66;  // measured: a half-height contraction tile's time over a full tile's

// Longest-processing-time-first placement of tile times on DEV_CUS CUs: the
// finishing time of the last CU.
double makespan(std::vector<double> t) {
    std::sort(t.begin(), t.end(), std::greater<double>());
    std::priority_queue<double, std::vector<double>, std::greater<double>> load;
    for (int i = 0; i < DEV_CUS; ++i) load.push(0.0);
    double end = 0;
    for (double x : t) {
        const double l = load.top() + x;
        load.pop();
        load.push(l);
        end = std::max(end, l);
    }
    return end;
}

// A contraction's tiles: a last round that would fill at most half the CUs
// runs, after the full rounds, as a second launch of twice as many
// half-height tiles (the shortest tiles form that round).
double contract_makespan(std::vector<double> t) {
    const size_t n = t.size(), r = n % DEV_CUS;
    if (n <= (size_t)DEV_CUS || r == 0 || 2 * r > (size_t)DEV_CUS) return makespan(t);
    std::sort(t.begin(), t.end(), std::greater<double>());
    std::vector<double> half;
    for (size_t i = n - r; i < n; ++i) {
        half.push_back(DEV_HALF_TILE * t[i]);
        half.push_back(DEV_HALF_TILE * t[i]);
    }
    t.resize(n - r);
    return makespan(t) + DEV_LAUNCH_US + makespan(half);
}

void device_time(const GOp& op, Cand& c) {
    const ja_spec& s = op.spec;
    const int nl = (int)s.letters.size();
    double numel_out = 1;
    for (char ch : s.out) numel_out *= (double)op.ext[s.letter_index(ch)];
    if (s.kind == JA_OP_RMSNORM || s.kind == JA_OP_SWIGLU || s.kind == JA_OP_ADD) {
        const double bytes = s.kind == JA_OP_RMSNORM ? 2.0 * (2.0 * numel_out + (double)op.ext[s.letter_index(s.ins[1][0])])
                                                     : 2.0 * 3.0 * numel_out;
        c.dev_us = DEV_LAUNCH_US + bytes / DEV_COPY_BPS * 1e6;
        return;
    }
    std::vector<std::vector<int64_t>> sp(nl);
    for (int i = 0; i < nl; ++i) sp[i] = equal_splits(op.ext[i], c.cnt[i]);
    const int is = s.causal ? s.letter_index(s.causal_s) : -1, it = s.causal ? s.letter_index(s.causal_t) : -1;
    // segments: kept cells grouped by output key
    std::map<std::vector<int64_t>, std::vector<std::vector<int64_t>>> seg;
    std::vector<int64_t> idx(nl, 0);
    int64_t ncell = 1;
    for (int i = 0; i < nl; ++i) ncell *= c.cnt[i];
    for (int64_t cell = 0; cell < ncell; ++cell) {
        int64_t r = cell;
        for (int i = nl - 1; i >= 0; --i) {
            idx[i] = r % c.cnt[i];
            r /= c.cnt[i];
        }
        if (is >= 0 && sp[it][idx[it]] >= sp[is][idx[is] + 1]) continue;
        std::vector<int64_t> key;
        for (char ch : s.out) key.push_back(idx[s.letter_index(ch)]);
        seg[key].push_back(idx);
    }
    auto len = [&](int l, int64_t k) { return sp[l][k + 1] - sp[l][k]; };
    std::vector<double> tiles;
    if (s.kind == JA_OP_CONTRACT) {
        const std::string &A = s.ins[0], &B = s.ins[1];
        for (auto& kv : seg) {
            const std::vector<int64_t>& first = kv.second[0];
            double nb = 1, M = 1, N = 1;
            for (char ch : s.out) {
                const int l = s.letter_index(ch);
                const bool inA = A.find(ch) != std::string::npos, inB = B.find(ch) != std::string::npos;
                (inA && inB ? nb : inA ? M : N) *= (double)len(l, first[l]);
            }
            double K = 0;
            for (auto& cell : kv.second) {
                double k = 1;
                for (int l = 0; l < nl; ++l)
                    if (s.out.find(s.letters[l]) == std::string::npos) k *= (double)len(l, cell[l]);
                K += k;
            }
            const double t = 2.0 * DEV_GEMM_TILE * DEV_GEMM_TILE * K / DEV_GEMM_CU_FLOPS * 1e6;
            const int64_t n = (int64_t)nb * (int64_t)std::ceil(M / DEV_GEMM_TILE) * (int64_t)std::ceil(N / DEV_GEMM_TILE);
            tiles.insert(tiles.end(), (size_t)n, t);
        }
    } else {  // attention
        const std::string& q = s.ins[0];
        const int ls = s.letter_index(s.att_s), ld = s.letter_index(q.back());
        const int lt = s.letter_index(s.att_t);
        const double D = (double)op.ext[ld];
        for (auto& kv : seg) {
            const std::vector<int64_t>& first = kv.second[0];
            double nbh = 1;
            for (size_t i = 0; i + 2 < q.size(); ++i) nbh *= (double)len(s.letter_index(q[i]), first[s.letter_index(q[i])]);
            const int64_t s_lo = sp[ls][first[ls]], S = len(ls, first[ls]);
            for (int64_t s0 = 0; s0 < S; s0 += DEV_ATTN_ROWS) {
                const int64_t last = s_lo + std::min<int64_t>(S, s0 + DEV_ATTN_ROWS) - 1;
                double keys = 0;
                for (auto& cell : kv.second) {
                    const int64_t t_lo = sp[lt][cell[lt]], t_hi = sp[lt][cell[lt] + 1];
                    keys += (double)std::max<int64_t>(0, (is >= 0 ? std::min(t_hi, last + 1) : t_hi) - t_lo);
                }
                const double t = 4.0 * DEV_ATTN_ROWS * D * keys / DEV_ATTN_CU_FLOPS * 1e6;
                tiles.insert(tiles.end(), (size_t)nbh, t);
            }
        }
    }
    c.dev_us = DEV_LAUNCH_US + (s.kind == JA_OP_CONTRACT ? contract_makespan(tiles) : makespan(tiles));
}

// A repartition in the device-time model: one launch copying the tensor once.
double rep_time(const ja_graph* g, int op, int slot, const std::vector<int32_t>& cons_tiling,
                const std::vector<int32_t>& prod_tiling);

uint64_t splitmix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

// Repartition sub-cost (section 4.3) of input `slot` of operator `op`: every
// element of the tensor when the tiling the consumer's spec asks for differs
// from the tiling its producer's spec leaves.
double rep_cost(const ja_graph* g, int op, int slot, const std::vector<int32_t>& cons_tiling,
                const std::vector<int32_t>& prod_tiling) {
    return cons_tiling == prod_tiling ? 0.0 : g->t[g->ops[op].inputs[slot]].numel();
}

double copy_time(double numel) { return DEV_LAUNCH_US + 2.0 * 2.0 * numel / DEV_COPY_BPS * 1e6; }

double rep_time(const ja_graph* g, int op, int slot, const std::vector<int32_t>& cons_tiling,
                const std::vector<int32_t>& prod_tiling) {
    if (cons_tiling == prod_tiling) return 0.0;
    return copy_time(g->t[g->ops[op].inputs[slot]].numel());
}

// An edge out of a view: the re-indexing is a repartition into whatever
// blocking the consumer asks for, so it costs all the view's elements (one
// copy launch in the device model) whatever the tilings on either side.
double view_edge(const ja_graph* g, int op, int slot, bool dev) {
    const double n = g->t[g->ops[op].inputs[slot]].numel();
    return dev ? copy_time(n) : n;
}

}  // namespace
}  // namespace ja

using namespace ja;

extern "C" {

ja_status ja_graph_create(ja_graph** out) {
    if (!out) return fail(JA_ERR_ARG, "out is NULL");
    *out = new ja_graph();
    return JA_OK;
}

void ja_graph_destroy(ja_graph* g) { delete g; }

ja_status ja_graph_add_input(ja_graph* g, int32_t rank, const int64_t* shape, int32_t* tensor) {
    if (!g || !shape || !tensor) return fail(JA_ERR_ARG, "NULL argument");
    if (rank < 1 || rank > JA_MAX_RANK) return fail(JA_ERR_ARG, "rank must be 1..8");
    GTensor t;
    for (int i = 0; i < rank; ++i) {
        if (shape[i] < 1) return fail(JA_ERR_SHAPE, "extents must be positive");
        t.shape.push_back(shape[i]);
    }
    g->t.push_back(t);
    *tensor = (int32_t)g->t.size() - 1;
    return JA_OK;
}

ja_status ja_graph_add_op(ja_graph* g, const ja_spec* spec, const int32_t* inputs, int32_t n_inputs, int32_t* tensor) {
    if (!g || !spec || !inputs || !tensor) return fail(JA_ERR_ARG, "NULL argument");
    if (n_inputs != (int32_t)spec->ins.size()) return fail(JA_ERR_ARG, "input count does not match the spec");
    if (!spec->packed.empty() || spec->packed_device)
        return fail(JA_ERR_UNSUPPORTED, "planning packed-sequence attention");
    if (spec->epilogue != JA_EPI_NONE) return fail(JA_ERR_UNSUPPORTED, "planning a contraction with an epilogue");
    GOp op;
    op.spec = *spec;
    op.ext.assign(spec->letters.size(), 0);
    for (int k = 0; k < n_inputs; ++k) {
        if (inputs[k] < 0 || inputs[k] >= (int32_t)g->t.size()) return fail(JA_ERR_ARG, "unknown input tensor");
        const GTensor& t = g->t[inputs[k]];
        const std::string& in = spec->ins[k];
        if (t.shape.size() != in.size()) return fail(JA_ERR_SHAPE, "input rank does not match the spec");
        for (size_t d = 0; d < in.size(); ++d) {
            int64_t& e = op.ext[spec->letter_index(in[d])];
            if (e && e != t.shape[d]) return fail(JA_ERR_SHAPE, std::string("letter ") + in[d] + " has two extents");
            e = t.shape[d];
        }
        op.inputs.push_back(inputs[k]);
    }
    for (size_t i = 0; i < op.ext.size(); ++i)
        if (!op.ext[i]) return fail(JA_ERR_SHAPE, std::string("letter ") + spec->letters[i] + " has no extent");
    GTensor o;
    for (char c : spec->out) o.shape.push_back(op.ext[spec->letter_index(c)]);
    o.producer = (int)g->ops.size();
    g->ops.push_back(op);
    g->t.push_back(o);
    const int id = (int)g->ops.size() - 1;
    g->ops[id].out = (int)g->t.size() - 1;
    for (int k = 0; k < n_inputs; ++k) g->t[inputs[k]].consumers.push_back({id, k});
    *tensor = (int32_t)g->t.size() - 1;
    return JA_OK;
}

ja_status ja_graph_add_view(ja_graph* g, int32_t tensor, const ja_view* view, int32_t rank, const int64_t* shape,
                            int32_t* out) {
    if (!g || !view || !shape || !out) return fail(JA_ERR_ARG, "NULL argument");
    if (tensor < 0 || tensor >= (int32_t)g->t.size()) return fail(JA_ERR_ARG, "unknown tensor");
    if (g->t[tensor].view_of >= 0) return fail(JA_ERR_UNSUPPORTED, "a view of a view");
    if (rank < 1 || rank > JA_MAX_RANK || view->rank < 1 || view->rank > JA_MAX_RANK)
        return fail(JA_ERR_ARG, "rank must be 1..8");
    double nv = 1, no = 1;
    std::vector<bool> seen(view->rank, false);
    for (int i = 0; i < view->rank; ++i) {
        if (view->shape[i] < 1) return fail(JA_ERR_SHAPE, "view extents must be positive");
        nv *= (double)view->shape[i];
        const int pm = view->perm[i];
        if (pm < 0 || pm >= view->rank || seen[pm]) return fail(JA_ERR_ARG, "view perm is not a permutation");
        seen[pm] = true;
    }
    GTensor o;
    for (int i = 0; i < rank; ++i) {
        if (shape[i] < 1) return fail(JA_ERR_SHAPE, "extents must be positive");
        no *= (double)shape[i];
        o.shape.push_back(shape[i]);
    }
    if (nv != g->t[tensor].numel() || no != nv) return fail(JA_ERR_SHAPE, "a view keeps the element count");
    o.view_of = tensor;
    g->t.push_back(o);
    *out = (int32_t)g->t.size() - 1;
    return JA_OK;
}

ja_status ja_graph_count(const ja_graph* g, int32_t* n_ops, int32_t* n_tensors) {
    if (!g) return fail(JA_ERR_ARG, "graph is NULL");
    if (n_ops) *n_ops = (int32_t)g->ops.size();
    if (n_tensors) *n_tensors = (int32_t)g->t.size();
    return JA_OK;
}

ja_status ja_graph_plan(ja_graph* g, int32_t p, int32_t mode, uint64_t seed, double* cost) {
    if (!g) return fail(JA_ERR_ARG, "graph is NULL");
    if (p < 1) return fail(JA_ERR_ARG, "processor count must be positive");
    if (mode < JA_PLAN_OPTIMAL || mode > JA_PLAN_DEVICE) return fail(JA_ERR_ARG, "unknown plan mode");
    if (g->ops.empty()) return fail(JA_ERR_ARG, "graph has no operator");
    const int nop = (int)g->ops.size();
    // candidate specs and their join / aggregation sub-costs
    for (int i = 0; i < nop; ++i) {
        GOp& op = g->ops[i];
        std::vector<std::vector<int32_t>> counts;
        std::vector<int32_t> cur(op.ext.size(), 1);
        enum_counts(op.ext, shardable(op.spec), 0, p, cur, counts);
        if (counts.empty())
            return fail(JA_ERR_UNSUPPORTED, "operator " + std::to_string(i) + " has no spec with " +
                                                std::to_string(p) + " function specifications");
        op.cands.clear();
        for (auto& cnt : counts) {
            Cand c;
            c.cnt = cnt;
            for (const std::string& in : op.spec.ins) c.in.push_back(tiling_of(op.spec, in, cnt));
            c.out = tiling_of(op.spec, op.spec.out, cnt);
            sub_costs(op, c);
            device_time(op, c);
            op.cands.push_back(c);
        }
        op.chosen = -1;
    }
    if (mode == JA_PLAN_RANDOM) {
        for (int i = 0; i < nop; ++i)
            g->ops[i].chosen = (int)(splitmix64(seed * 0x100000001B3ull + (uint64_t)i) % g->ops[i].cands.size());
    } else {
        const bool with_rep = mode != JA_PLAN_GREEDY;
        const bool dev = mode == JA_PLAN_DEVICE;
        auto edge = [&](int op, int slot, const std::vector<int32_t>& cons, const std::vector<int32_t>& prod) {
            return dev ? rep_time(g, op, slot, cons, prod) : rep_cost(g, op, slot, cons, prod);
        };
        // pieces (section 4.5): cut every edge out of a tensor with several consumers
        auto cut = [&](int tensor) { return g->t[tensor].consumers.size() > 1; };
        std::vector<int> piece(nop);
        for (int i = 0; i < nop; ++i) piece[i] = i;
        std::function<int(int)> find = [&](int x) { return piece[x] == x ? x : piece[x] = find(piece[x]); };
        for (int i = 0; i < nop; ++i)
            for (int in : g->ops[i].inputs)
                if (g->t[in].producer >= 0 && !cut(in)) piece[find(i)] = find(g->t[in].producer);
        std::map<int, std::vector<int>> members;
        for (int i = 0; i < nop; ++i) members[find(i)].push_back(i);
        std::vector<std::vector<int>> pieces;
        for (auto& kv : members) pieces.push_back(kv.second);
        auto root_of = [&](const std::vector<int>& ops) {
            for (int i : ops) {
                const GTensor& o = g->t[g->ops[i].out];
                if (o.consumers.size() != 1 || cut(g->ops[i].out)) return i;
            }
            return ops.back();
        };
        // larger pieces first; equal sizes in the order of their roots
        std::stable_sort(pieces.begin(), pieces.end(), [&](const std::vector<int>& a, const std::vector<int>& b) {
            if (a.size() != b.size()) return a.size() > b.size();
            return root_of(a) < root_of(b);
        });
        std::vector<bool> fixed(nop, false);
        for (const auto& pc : pieces) {
            const int root = root_of(pc);
            // Opt tables: per operator, per output tiling, the best cost and candidate;
            // per candidate, the producer tiling chosen for each in-piece input
            std::map<int, std::map<std::vector<int32_t>, std::pair<double, int>>> opt;
            std::map<int, std::vector<std::vector<std::vector<int32_t>>>> pick;
            for (int i : pc) {  // operator ids rise along every edge: a topological order
                GOp& op = g->ops[i];
                auto& tab = opt[i];
                auto& pk = pick[i];
                pk.assign(op.cands.size(), {});
                for (size_t ci = 0; ci < op.cands.size(); ++ci) {
                    const Cand& c = op.cands[ci];
                    double b = dev ? c.dev_us : c.join + c.agg;
                    pk[ci].assign(op.inputs.size(), {});
                    for (size_t k = 0; k < op.inputs.size(); ++k) {
                        const int tin = op.inputs[k], q = g->t[tin].producer;
                        if (g->t[tin].view_of >= 0) {  // a view: one repartition, any tiling
                            if (with_rep) b += view_edge(g, i, (int)k, dev);
                            continue;
                        }
                        if (q < 0) continue;  // a computation input: materialised in the blocks asked for
                        if (cut(tin)) {
                            // charged here if its producer is already fixed, else when it is planned
                            if (fixed[q] && with_rep) b += edge(i, (int)k, c.in[k], g->ops[q].cands[g->ops[q].chosen].out);
                            continue;
                        }
                        double best = 0;
                        bool first = true;
                        for (auto& kv : opt[q]) {
                            const double v = kv.second.first + (with_rep ? edge(i, (int)k, c.in[k], kv.first) : 0.0);
                            if (first || v < best) {
                                best = v;
                                pk[ci][k] = kv.first;
                                first = false;
                            }
                        }
                        b += best;
                    }
                    if (i == root && with_rep) {
                        // consumers of the root's output in pieces planned earlier
                        for (auto& cs : g->t[op.out].consumers)
                            if (fixed[cs.first])
                                b += edge(cs.first, cs.second,
                                              g->ops[cs.first].cands[g->ops[cs.first].chosen].in[cs.second], c.out);
                    }
                    auto it = tab.find(c.out);
                    if (it == tab.end() || b < it->second.first) tab[c.out] = {b, (int)ci};
                }
            }
            // trace back from the root's cheapest tiling
            std::vector<std::pair<int, std::vector<int32_t>>> stack;
            {
                auto& tab = opt[root];
                auto best = tab.begin();
                for (auto it = tab.begin(); it != tab.end(); ++it)
                    if (it->second.first < best->second.first) best = it;
                stack.push_back({root, best->first});
            }
            while (!stack.empty()) {
                auto [i, tiling] = stack.back();
                stack.pop_back();
                GOp& op = g->ops[i];
                const int ci = opt[i][tiling].second;
                op.chosen = ci;
                for (size_t k = 0; k < op.inputs.size(); ++k) {
                    const int tin = op.inputs[k], q = g->t[tin].producer;
                    if (q >= 0 && !cut(tin)) stack.push_back({q, pick[i][ci][k]});
                }
            }
            for (int i : pc) fixed[i] = true;
        }
    }
    if (cost) {
        if (mode == JA_PLAN_DEVICE) return ja_graph_device_time(g, nullptr, cost);
        double r, j, a;
        const ja_status st = ja_graph_cost(g, nullptr, &r, &j, &a);
        if (st) return st;
        *cost = r + j + a;
    }
    return JA_OK;
}

ja_status ja_graph_plan_intervals(const ja_graph* g, int32_t op, int32_t* intervals, int32_t cap) {
    if (!g || !intervals) return fail(JA_ERR_ARG, "NULL argument");
    if (op < 0 || op >= (int32_t)g->ops.size()) return fail(JA_ERR_ARG, "unknown operator");
    const GOp& o = g->ops[op];
    if (o.chosen < 0) return fail(JA_ERR_STATE, "graph has not been planned");
    if (cap < (int32_t)o.ext.size()) return fail(JA_ERR_WORKSPACE, "interval buffer too small");
    std::copy(o.cands[o.chosen].cnt.begin(), o.cands[o.chosen].cnt.end(), intervals);
    return JA_OK;
}

}  // extern "C"

namespace {
// The candidate of every operator: from `intervals`, or the planned one.
ja_status assignment(const ja_graph* g, const int32_t* const* intervals, std::vector<Cand>& pl) {
    const int nop = (int)g->ops.size();
    pl.assign(nop, Cand());
    for (int i = 0; i < nop; ++i) {
        const GOp& op = g->ops[i];
        if (intervals) {
            if (!intervals[i]) return fail(JA_ERR_ARG, "NULL interval list");
            Cand c;
            for (size_t l = 0; l < op.ext.size(); ++l) {
                if (intervals[i][l] < 1 || intervals[i][l] > op.ext[l])
                    return fail(JA_ERR_DECOMP, "interval count outside [1, extent]");
                c.cnt.push_back(intervals[i][l]);
            }
            for (const std::string& in : op.spec.ins) c.in.push_back(tiling_of(op.spec, in, c.cnt));
            c.out = tiling_of(op.spec, op.spec.out, c.cnt);
            sub_costs(op, c);
            device_time(op, c);
            pl[i] = c;
        } else {
            if (op.chosen < 0) return fail(JA_ERR_STATE, "graph has not been planned");
            pl[i] = op.cands[op.chosen];
        }
    }
    return JA_OK;
}
}  // namespace

extern "C" {

ja_status ja_graph_cost(const ja_graph* g, const int32_t* const* intervals, double* repart, double* join,
                        double* agg) {
    if (!g) return fail(JA_ERR_ARG, "graph is NULL");
    const int nop = (int)g->ops.size();
    std::vector<Cand> pl;
    ja_status st = assignment(g, intervals, pl);
    if (st) return st;
    double r = 0, j = 0, a = 0;
    for (int i = 0; i < nop; ++i) {
        const GOp& op = g->ops[i];
        j += pl[i].join;
        a += pl[i].agg;
        for (size_t k = 0; k < op.inputs.size(); ++k) {
            const int q = g->t[op.inputs[k]].producer;
            if (g->t[op.inputs[k]].view_of >= 0)
                r += view_edge(g, i, (int)k, false);
            else if (q >= 0)
                r += rep_cost(g, i, (int)k, pl[i].in[k], pl[q].out);
        }
    }
    if (repart) *repart = r;
    if (join) *join = j;
    if (agg) *agg = a;
    return JA_OK;
}

ja_status ja_graph_device_time(const ja_graph* g, const int32_t* const* intervals, double* us) {
    if (!g || !us) return fail(JA_ERR_ARG, "NULL argument");
    std::vector<Cand> pl;
    ja_status st = assignment(g, intervals, pl);
    if (st) return st;
    double t = 0;
    for (size_t i = 0; i < g->ops.size(); ++i) {
        const GOp& op = g->ops[i];
        t += pl[i].dev_us;
        for (size_t k = 0; k < op.inputs.size(); ++k) {
            const int q = g->t[op.inputs[k]].producer;
            if (g->t[op.inputs[k]].view_of >= 0)
                t += view_edge(g, (int)i, (int)k, true);
            else if (q >= 0)
                t += rep_time(g, (int)i, (int)k, pl[i].in[k], pl[q].out);
        }
    }
    *us = t;
    return JA_OK;
}

}  // extern "C"
