// core.cpp -- errors, relation descriptors, operator specs, decompositions and
// the join (tuple-list builder) of libja.
//
// Terms follow "Every Kernel Is a Join" (paperpeel full text): tensor types
// and tilings (section 3.1), projections, function specs and join-agg specs
// (section 3.2), shardable indices and interval requests (section 3.3).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "ja_host.h"

namespace ja {

static thread_local std::string g_last_error;

ja_status fail(ja_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}
void clear_error() { g_last_error.clear(); }

ja_status hip_fail(hipError_t e, const char* what) {
    std::string m = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
    return fail(JA_ERR_HIP, m);
}

size_t dtype_size(int32_t dtype) {
    switch (dtype) {
        case JA_F32: return 4;
        case JA_BF16: return 2;
        case JA_F16: return 2;
        default: return 0;
    }
}

std::vector<int64_t> equal_splits(int64_t n, int64_t q) {
    std::vector<int64_t> p(1, 0);
    int64_t base = n / q, extra = n % q;
    for (int64_t i = 0; i < q; ++i) p.push_back(p.back() + base + (i < extra ? 1 : 0));
    return p;
}

ja_status check_splits(const int64_t* pts, int64_t n, int64_t q, std::vector<int64_t>& out, const char* what) {
    if (q < 1 || q > n) return fail(JA_ERR_DECOMP, std::string(what) + ": interval count must be in [1, extent]");
    if (!pts) {
        out = equal_splits(n, q);
        return JA_OK;
    }
    out.assign(pts, pts + q + 1);
    if (out.front() != 0 || out.back() != n)
        return fail(JA_ERR_DECOMP, std::string(what) + ": split points must start at 0 and end at the extent");
    for (int64_t i = 0; i < q; ++i)
        if (out[i + 1] <= out[i]) return fail(JA_ERR_DECOMP, std::string(what) + ": split points must rise strictly");
    return JA_OK;
}

int64_t Rel::block_index(const int64_t* key) const {
    int64_t lin = 0;
    for (int d = 0; d < rank; ++d) lin = lin * nblk(d) + key[d];
    return lin;
}

int64_t Rel::find(int d, int64_t x) const {
    auto it = std::upper_bound(sp[d].begin(), sp[d].end(), x);
    return (int64_t)(it - sp[d].begin()) - 1;
}

ja_status rel_from_desc(const ja_relation_desc* desc, Rel& r) {
    if (!desc) return fail(JA_ERR_ARG, "relation descriptor is NULL");
    if (desc->rank < 1 || desc->rank > JA_MAX_RANK) return fail(JA_ERR_ARG, "relation rank must be 1..8");
    if (!dtype_size(desc->dtype)) return fail(JA_ERR_DTYPE, "unknown relation dtype");
    r = Rel();
    r.rank = desc->rank;
    r.dtype = desc->dtype;
    r.nblocks = 1;
    r.elems = 1;
    for (int d = 0; d < r.rank; ++d) {
        if (desc->shape[d] < 1) return fail(JA_ERR_SHAPE, "relation extents must be positive");
        r.shape[d] = desc->shape[d];
        ja_status st = check_splits(desc->splits[d], desc->shape[d], desc->nblk[d], r.sp[d], "relation blocking");
        if (st) return fail(JA_ERR_SHAPE, ja_last_error());
        r.nblocks *= desc->nblk[d];
        r.elems *= desc->shape[d];
    }
    if (r.nblocks > (int64_t)1 << 26) return fail(JA_ERR_UNSUPPORTED, "more than 2^26 blocks in one relation");
    // Blocks in lexicographic key order, each dense row-major over its box.
    r.blk_off.resize(r.nblocks);
    std::vector<int64_t> key(r.rank, 0);
    int64_t off = 0;
    for (int64_t b = 0; b < r.nblocks; ++b) {
        r.blk_off[b] = off;
        int64_t n = 1;
        for (int d = 0; d < r.rank; ++d) n *= r.ext(d, key[d]);
        off += n;
        for (int d = r.rank - 1; d >= 0; --d) {
            if (++key[d] < r.nblk(d)) break;
            key[d] = 0;
        }
    }
    return JA_OK;
}

// ---- operator specs -----------------------------------------------------------

static bool valid_letters(const std::string& s) {
    if (s.empty() || s.size() > 26) return false;
    bool seen[26] = {false};
    for (char c : s) {
        if (c < 'a' || c > 'z' || seen[c - 'a']) return false;
        seen[c - 'a'] = true;
    }
    return true;
}

static ja_status parse_params(const char* params, ja_spec* s) {
    if (!params) return JA_OK;
    std::string p(params);
    size_t pos = 0;
    while (pos < p.size()) {
        size_t end = p.find(';', pos);
        if (end == std::string::npos) end = p.size();
        std::string kv = p.substr(pos, end - pos);
        pos = end + 1;
        if (kv.empty()) continue;
        size_t eq = kv.find('=');
        if (eq == std::string::npos) return fail(JA_ERR_SPEC, "param without '=': " + kv);
        std::string k = kv.substr(0, eq), v = kv.substr(eq + 1);
        if (k == "scale" || k == "eps") {
            char* e = nullptr;
            double x = std::strtod(v.c_str(), &e);
            if (!e || *e || v.empty() || !std::isfinite(x)) return fail(JA_ERR_SPEC, "bad number for " + k);
            if (k == "scale") {
                if (!(x > 0)) return fail(JA_ERR_SPEC, "scale must be > 0");
                s->scale = x;
                s->has_scale = true;
            } else {
                if (x < 0) return fail(JA_ERR_SPEC, "eps must be >= 0");
                s->eps = x;
            }
        } else if (k == "packed" && v == "device") {
            // the sequence ends are the split points of the sequence letters
            s->packed.clear();
            s->packed_device = true;
        } else if (k == "packed") {
            // ascending positive sequence ends, comma separated
            s->packed.clear();
            s->packed_device = false;
            size_t q = 0;
            while (q <= v.size()) {
                size_t c = v.find(',', q);
                if (c == std::string::npos) c = v.size();
                const std::string num = v.substr(q, c - q);
                char* e = nullptr;
                const long long x = std::strtoll(num.c_str(), &e, 10);
                if (num.empty() || !e || *e || x <= 0 || (!s->packed.empty() && x <= s->packed.back()) ||
                    x > ((int64_t)1 << 31) - 1)
                    return fail(JA_ERR_SPEC, "packed expects ascending positive sequence ends");
                s->packed.push_back(x);
                q = c + 1;
            }
        } else if (k == "causal") {
            if (v.size() != 3 || v[1] != ',') return fail(JA_ERR_SPEC, "causal expects '<s>,<t>'");
            s->causal = true;
            s->causal_s = v[0];
            s->causal_t = v[2];
        } else {
            return fail(JA_ERR_SPEC, "unknown param " + k);
        }
    }
    return JA_OK;
}

static ja_status parse_spec(const char* einsum, const char* op, const char* params, ja_spec* s) {
    if (!einsum || !op) return fail(JA_ERR_ARG, "einsum and op must not be NULL");
    std::string e(einsum);
    size_t arrow = e.find("->");
    if (arrow == std::string::npos) return fail(JA_ERR_SPEC, "einsum needs '->'");
    s->out = e.substr(arrow + 2);
    std::string lhs = e.substr(0, arrow);
    s->ins.clear();
    size_t pos = 0;
    while (true) {
        size_t c = lhs.find(',', pos);
        s->ins.push_back(lhs.substr(pos, c == std::string::npos ? std::string::npos : c - pos));
        if (c == std::string::npos) break;
        pos = c + 1;
    }
    for (auto& x : s->ins)
        if (!valid_letters(x)) return fail(JA_ERR_SPEC, "operand '" + x + "' must be distinct letters a-z");
    if (!valid_letters(s->out)) return fail(JA_ERR_SPEC, "output must be distinct letters a-z");
    s->letters.clear();
    for (char c : e)
        if (c >= 'a' && c <= 'z' && s->letters.find(c) == std::string::npos) s->letters.push_back(c);
    for (char c : s->out) {
        bool found = false;
        for (auto& x : s->ins) found |= x.find(c) != std::string::npos;
        if (!found) return fail(JA_ERR_SPEC, std::string("output letter ") + c + " appears in no input");
    }
    ja_status st = parse_params(params, s);
    if (st) return st;

    std::string o(op);
    if (o == "contract" || o == "contract_add" || o == "contract_swiglu") {
        // contract_add: C = A B + R, the residual R joined 1:1 on the output
        // key; contract_swiglu: B's last letter indexes a (gate, up) pair and
        // C = silu(A B [gate]) * (A B [up]).  Both are applied to the
        // aggregated block before it is written.
        s->kind = JA_OP_CONTRACT;
        s->epilogue = o == "contract_add" ? JA_EPI_ADD : o == "contract_swiglu" ? JA_EPI_SWIGLU : JA_EPI_NONE;
        if (s->epilogue == JA_EPI_ADD) {
            if (s->ins.size() != 3 || s->ins[2] != s->out)
                return fail(JA_ERR_SPEC, "contract_add takes A, B and a residual with the output's letters");
        } else if (s->ins.size() != 2) {
            return fail(JA_ERR_SPEC, o + " takes two operands");
        }
        if (s->epilogue == JA_EPI_SWIGLU) {
            const char c = s->ins[1].empty() ? 0 : s->ins[1].back();
            if (!c || s->ins[0].find(c) != std::string::npos || s->out.find(c) != std::string::npos)
                return fail(JA_ERR_SPEC, "contract_swiglu needs B's last letter to index the (gate, up) pair, "
                                         "in neither A nor the output");
            s->pair = c;
        }
        for (char c : s->letters) {
            if (c == s->pair) continue;
            int n = (s->ins[0].find(c) != std::string::npos) + (s->ins[1].find(c) != std::string::npos) +
                    (s->out.find(c) != std::string::npos);
            if (n < 2) return fail(JA_ERR_SPEC, std::string("letter ") + c + " must appear in two of A, B, C");
        }
        s->group_by = s->out;
    } else if (o == "attention") {
        s->kind = JA_OP_ATTENTION;
        if (s->ins.size() != 3) return fail(JA_ERR_SPEC, "attention takes Q, K, V");
        // Q = O = [batch..., group..., s, d], K = V = [batch..., t, d]: the
        // optional group letters index the query heads that share one
        // key-value head (grouped-query attention).  Batch-head letters may
        // also follow the position letter (token-major relations, e.g.
        // bshd,bthd,bthd->bshd): with the position and head-dimension letters
        // removed, Q's letters must be K's followed by the group letters.
        const std::string &q = s->ins[0], &k = s->ins[1], &v = s->ins[2];
        if (q != s->out || k != v || k.size() < 2 || q.size() < k.size())
            return fail(JA_ERR_SPEC,
                        "attention needs Q = O = [batch..., group..., s, d] and K = V = [batch..., t, d]");
        const size_t r = q.size(), rk = k.size();
        if (q[r - 1] != k[rk - 1])
            return fail(JA_ERR_SPEC, "attention: Q and K must end in the same head-dimension letter");
        // the key position letter: the one letter of K that Q lacks
        char ct = 0;
        for (size_t i = 0; i + 1 < rk; ++i)
            if (q.find(k[i]) == std::string::npos) {
                if (ct) return fail(JA_ERR_SPEC, "attention: K has more than one letter that Q lacks");
                ct = k[i];
            }
        if (!ct) return fail(JA_ERR_SPEC, "attention: K needs a key position letter absent from Q");
        // the query position letter: Q's second to last when that letter is
        // absent from K and K's position letter is K's second to last (the
        // head-major form, so "bgsrd,bgtd" has position letter r and group
        // letter s), else the letter at the key position letter's place in K
        // (the letters before both the same: token-major)
        const size_t pt = k.find(ct);
        char cs = 0;
        if (k.find(q[r - 2]) == std::string::npos && k[rk - 2] == ct)
            cs = q[r - 2];
        else if (pt < r - 1 && q.substr(0, pt) == k.substr(0, pt) && k.find(q[pt]) == std::string::npos)
            cs = q[pt];
        if (!cs) return fail(JA_ERR_SPEC, "attention letters must be [batch..., s, batch..., d] and [batch..., t, batch..., d]");
        std::string lq, lk;  // batch-head letters in storage order
        for (char c : q.substr(0, r - 1))
            if (c != cs) lq += c;
        for (char c : k.substr(0, rk - 1))
            if (c != ct) lk += c;
        if (lq.compare(0, lk.size(), lk) != 0)
            return fail(JA_ERR_SPEC, "attention: Q's batch-head letters must be K's followed by the group letters");
        for (size_t i = lk.size(); i < lq.size(); ++i)
            if (k.find(lq[i]) != std::string::npos)
                return fail(JA_ERR_SPEC, "attention group letters must not index K and V");
        s->att_s = cs;
        s->att_t = ct;
        if (s->causal && (s->causal_s != cs || s->causal_t != ct))
            return fail(JA_ERR_SPEC, "causal pair must name the query and key position letters");
        s->group_by = s->out;
    } else if (o == "rmsnorm") {
        s->kind = JA_OP_RMSNORM;
        if (s->ins.size() != 2 || s->ins[0].size() != 2 || s->ins[1].size() != 1 || s->ins[1][0] != s->ins[0][1] ||
            s->out != s->ins[0])
            return fail(JA_ERR_SPEC, "rmsnorm expects 'rd,d->rd'");
        s->group_by = s->out.substr(0, 1);
    } else if (o == "swiglu" || o == "add") {
        s->kind = o == "swiglu" ? JA_OP_SWIGLU : JA_OP_ADD;
        if (s->ins.size() != 2 || s->ins[0] != s->ins[1] || s->ins[0] != s->out)
            return fail(JA_ERR_SPEC, o + " expects two operands with the output's letters");
        s->group_by = s->out;
    } else {
        return fail(JA_ERR_SPEC, "unknown op " + o);
    }
    if (s->kind != JA_OP_ATTENTION && (!s->packed.empty() || s->packed_device))
        return fail(JA_ERR_SPEC, "packed applies to attention only");
    if (!s->causal || s->kind == JA_OP_ATTENTION) return JA_OK;
    return fail(JA_ERR_SPEC, "causal applies to attention only");
}

// ---- join: enumerate the join-agg spec's function specs ------------------------

ja_status build_tuples(const ja_spec* s, const ja_decomp* d, ja_tuples& t) {
    const int nl = (int)s->letters.size();
    // iteration order: group-by letters first (their order), then the rest in letter order
    std::vector<int> order;
    for (char c : s->group_by) order.push_back(s->letter_index(c));
    for (int i = 0; i < nl; ++i)
        if (s->group_by.find(s->letters[i]) == std::string::npos) order.push_back(i);
    const int ng = (int)s->group_by.size();
    std::vector<int64_t> cnt(nl);
    int64_t total = 1;
    for (int i = 0; i < nl; ++i) {
        cnt[i] = (int64_t)d->sp[i].size() - 1;
        total *= cnt[i];
        if (total > ((int64_t)1 << 28)) return fail(JA_ERR_UNSUPPORTED, "more than 2^28 grid cells");
    }
    int is = -1, it = -1;
    if (s->causal) {
        is = s->letter_index(s->causal_s);
        it = s->letter_index(s->causal_t);
    }
    int ps = -1, pt = -1;  // packed sequences: the query and key position letters
    if (!s->packed.empty() || s->packed_device) {
        ps = s->letter_index(s->att_s);
        pt = s->letter_index(s->att_t);
    }
    t.nl = nl;
    t.rec.clear();
    t.seg.assign(1, 0);
    std::vector<int64_t> idx(nl, 0);
    std::vector<int64_t> prev_g(ng, -1);
    int64_t n = 0;
    for (int64_t c = 0; c < total; ++c) {
        bool keep = true;
        if (s->causal) {
            // drop the tuple when its first key comes after its last query
            if (d->sp[it][idx[it]] >= d->sp[is][idx[is] + 1]) keep = false;
        }
        if (keep && ps >= 0) {
            // drop the tuple when its query and key intervals share no sequence
            // (both are unions of whole sequences, so: when they do not overlap)
            const int64_t slo = d->sp[ps][idx[ps]], shi = d->sp[ps][idx[ps] + 1];
            const int64_t tlo = d->sp[pt][idx[pt]], thi = d->sp[pt][idx[pt] + 1];
            if (std::max(slo, tlo) >= std::min(shi, thi)) keep = false;
        }
        if (keep) {
            bool newseg = n > 0;
            bool same = true;
            for (int g = 0; g < ng; ++g) same &= prev_g[g] == idx[order[g]];
            if (n > 0 && !same) t.seg.push_back(n);
            (void)newseg;
            for (int g = 0; g < ng; ++g) prev_g[g] = idx[order[g]];
            for (int i = 0; i < nl; ++i) t.rec.push_back((int32_t)idx[i]);
            ++n;
        }
        for (int k = nl - 1; k >= 0; --k) {
            int l = order[k];
            if (++idx[l] < cnt[l]) break;
            idx[l] = 0;
        }
    }
    if (n > 0) t.seg.push_back(n);
    return JA_OK;
}

}  // namespace ja

using namespace ja;

extern "C" {

int32_t ja_abi_version(void) { return JA_ABI_VERSION; }

const char* ja_status_str(ja_status st) {
    switch (st) {
        case JA_OK: return "JA_OK";
        case JA_ERR_ARG: return "JA_ERR_ARG";
        case JA_ERR_SPEC: return "JA_ERR_SPEC";
        case JA_ERR_DECOMP: return "JA_ERR_DECOMP";
        case JA_ERR_SHAPE: return "JA_ERR_SHAPE";
        case JA_ERR_DTYPE: return "JA_ERR_DTYPE";
        case JA_ERR_WORKSPACE: return "JA_ERR_WORKSPACE";
        case JA_ERR_UNSUPPORTED: return "JA_ERR_UNSUPPORTED";
        case JA_ERR_HIP: return "JA_ERR_HIP";
        case JA_ERR_STATE: return "JA_ERR_STATE";
        default: return "JA_ERR_UNKNOWN";
    }
}

const char* ja_last_error(void) { return g_last_error.c_str(); }

ja_status ja_relation_bytes(const ja_relation_desc* desc, size_t* bytes) {
    if (!bytes) return fail(JA_ERR_ARG, "bytes is NULL");
    Rel r;
    ja_status st = rel_from_desc(desc, r);
    if (st) return st;
    *bytes = (size_t)r.elems * dtype_size(r.dtype);
    return JA_OK;
}

ja_status ja_relation_nblocks(const ja_relation_desc* desc, int64_t* nblocks) {
    if (!nblocks) return fail(JA_ERR_ARG, "nblocks is NULL");
    Rel r;
    ja_status st = rel_from_desc(desc, r);
    if (st) return st;
    *nblocks = r.nblocks;
    return JA_OK;
}

ja_status ja_relation_block(const ja_relation_desc* desc, const int64_t* key, int64_t* lo, int64_t* hi,
                            size_t* byte_off) {
    if (!key) return fail(JA_ERR_ARG, "key is NULL");
    Rel r;
    ja_status st = rel_from_desc(desc, r);
    if (st) return st;
    for (int d = 0; d < r.rank; ++d)
        if (key[d] < 0 || key[d] >= r.nblk(d)) return fail(JA_ERR_ARG, "block key out of range");
    for (int d = 0; d < r.rank; ++d) {
        if (lo) lo[d] = r.sp[d][key[d]];
        if (hi) hi[d] = r.sp[d][key[d] + 1];
    }
    if (byte_off) *byte_off = (size_t)r.blk_off[r.block_index(key)] * dtype_size(r.dtype);
    return JA_OK;
}

ja_status ja_spec_create(const char* einsum, const char* op, const char* params, ja_spec** out) {
    if (!out) return fail(JA_ERR_ARG, "out is NULL");
    *out = nullptr;
    ja_spec* s = new ja_spec();
    ja_status st = parse_spec(einsum, op, params, s);
    if (st) {
        delete s;
        return st;
    }
    *out = s;
    return JA_OK;
}

void ja_spec_destroy(ja_spec* s) { delete s; }

ja_status ja_spec_letters(const ja_spec* s, char* buf, size_t cap) {
    if (!s || !buf) return fail(JA_ERR_ARG, "NULL argument");
    if (cap < s->letters.size() + 1) return fail(JA_ERR_ARG, "buffer too small");
    std::memcpy(buf, s->letters.c_str(), s->letters.size() + 1);
    return JA_OK;
}

ja_status ja_decomp_create(const ja_spec* s, const int64_t* extents, const int32_t* intervals,
                           const int64_t* const* splits, ja_decomp** out) {
    if (!out) return fail(JA_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (!s || !extents || !intervals) return fail(JA_ERR_ARG, "NULL argument");
    ja_decomp* d = new ja_decomp();
    d->letters = s->letters;
    const int nl = (int)s->letters.size();
    d->ext.assign(extents, extents + nl);
    d->sp.resize(nl);
    for (int i = 0; i < nl; ++i) {
        if (extents[i] < 1) {
            delete d;
            return fail(JA_ERR_DECOMP, std::string("letter ") + s->letters[i] + ": extent must be positive");
        }
        ja_status st = check_splits(splits ? splits[i] : nullptr, extents[i], intervals[i], d->sp[i],
                                    (std::string("letter ") + s->letters[i]).c_str());
        if (st) {
            delete d;
            return st;
        }
    }
    if (s->kind == JA_OP_ATTENTION) {
        // the head dimension is joined on, never split
        int id = s->letter_index(s->ins[0].back());
        if (d->sp[id].size() != 2) {
            delete d;
            return fail(JA_ERR_DECOMP, "attention: the head-dimension letter cannot be split");
        }
        if (s->packed_device) {
            // sequence ends given by the cuts themselves: both sequence letters cut alike
            const std::string &q = s->ins[0], &k = s->ins[1];
            if (d->sp[s->letter_index(s->att_s)] != d->sp[s->letter_index(s->att_t)]) {
                delete d;
                return fail(JA_ERR_DECOMP, "attention: packed=device needs the same cuts on both sequence letters");
            }
        }
        if (!s->packed.empty()) {
            // packed sequences: the sequence letters span every sequence and may be
            // split only at sequence ends (section 3.3)
            const std::string &q = s->ins[0], &k = s->ins[1];
            for (char c : {s->att_s, s->att_t}) {
                const std::vector<int64_t>& sp = d->sp[s->letter_index(c)];
                bool ok = sp.back() == s->packed.back();
                for (size_t i = 1; ok && i + 1 < sp.size(); ++i)
                    ok = std::binary_search(s->packed.begin(), s->packed.end(), sp[i]);
                if (!ok) {
                    delete d;
                    return fail(JA_ERR_DECOMP, std::string("attention: letter ") + c +
                                                   " must end at the last sequence end and be split only at sequence ends");
                }
            }
        }
    }
    *out = d;
    return JA_OK;
}

void ja_decomp_destroy(ja_decomp* d) { delete d; }

ja_status ja_join(const ja_spec* s, const ja_decomp* d, ja_tuples** out) {
    if (!out) return fail(JA_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (!s || !d) return fail(JA_ERR_ARG, "NULL argument");
    if (d->letters != s->letters) return fail(JA_ERR_DECOMP, "decomposition was made for another spec");
    ja_tuples* t = new ja_tuples();
    ja_status st = build_tuples(s, d, *t);
    if (st) {
        delete t;
        return st;
    }
    *out = t;
    return JA_OK;
}

ja_status ja_tuples_count(const ja_tuples* t, int64_t* n_tuples, int64_t* n_segs, int32_t* n_letters) {
    if (!t) return fail(JA_ERR_ARG, "tuples is NULL");
    if (n_tuples) *n_tuples = t->count();
    if (n_segs) *n_segs = (int64_t)t->seg.size() - 1;
    if (n_letters) *n_letters = t->nl;
    return JA_OK;
}

ja_status ja_tuples_export(const ja_tuples* t, int32_t* rec, int64_t rec_cap, int64_t* seg_off, int64_t seg_cap) {
    if (!t) return fail(JA_ERR_ARG, "tuples is NULL");
    if (rec) {
        if (rec_cap < (int64_t)t->rec.size()) return fail(JA_ERR_WORKSPACE, "record buffer too small");
        std::copy(t->rec.begin(), t->rec.end(), rec);
    }
    if (seg_off) {
        if (seg_cap < (int64_t)t->seg.size()) return fail(JA_ERR_WORKSPACE, "segment buffer too small");
        std::copy(t->seg.begin(), t->seg.end(), seg_off);
    }
    return JA_OK;
}

void ja_tuples_destroy(ja_tuples* t) { delete t; }

}  // extern "C"
