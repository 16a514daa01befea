// repart.cpp -- re-blocking a relation between two decompositions.
//
// "Every Kernel Is a Join" (paperpeel full text), section 5.3: take every cut
// position of the source blocking and every cut position of the target
// blocking, dimension by dimension, and cut the tensor at all of them.  The
// resulting grid cells ("atoms") are small enough that each source block and
// each target block is made of whole atoms with no overlap.  Moving data
// between the two blockings then means slicing source blocks into atoms,
// shipping the atoms, and gluing them into target blocks.  On one GPU nothing
// is shipped, so the slicing and the gluing collapse into a single copy of
// every atom from its place in the source buffer to its place in the target
// buffer.
//
// A repartition may also re-index the tensor (read as another shape, permute
// axes, read as the destination's shape), e.g. token-major projections to
// head-major attention inputs.  To keep every atom a box on both sides, the
// planner works in the finest common factorisation of all the shapes involved
// ("sub-dimensions"), and refines the overlay so that every boundary of a
// block of a merged dimension splits the sub-dimensions it spans by their
// mixed-radix digits.
#include <algorithm>
#include <cstring>
#include <functional>
#include <set>

#include "ja_host.h"

using namespace ja;

struct ja_repart {
    std::vector<RepTask> tasks;
    int64_t n_atoms = 0;
    int32_t esize = 0;
    void* dev = nullptr;
};

namespace {

// Suffix products ("strides" of row-major dims), outermost first, plus the total.
std::vector<int64_t> strides_of(const std::vector<int64_t>& shape) {
    std::vector<int64_t> s(shape.size());
    int64_t acc = 1;
    for (int i = (int)shape.size() - 1; i >= 0; --i) {
        s[i] = acc;
        acc *= shape[i];
    }
    return s;
}

// Refine one dimension of extent n by two sets of local cut values (each a
// value u meaning "the inner part has extent u").  Returns the sub-extents
// from outer to inner, or an empty vector if the cuts do not nest.
std::vector<int64_t> refine(int64_t n, const std::set<int64_t>& cuts) {
    if (n == 1) return {1};  // a unit dimension is its own (single) sub-dimension
    std::vector<int64_t> c(cuts.begin(), cuts.end());  // ascending, includes 1 and n
    std::vector<int64_t> sub;
    for (size_t i = c.size() - 1; i > 0; --i) {
        if (c[i] % c[i - 1]) return {};
        sub.push_back(c[i] / c[i - 1]);
    }
    return sub;
}

struct Sub {
    int64_t ext;
    int vdim;        // parent view dimension
    int64_t vstride; // stride in the view's row-major order
    int64_t pstride; // stride in the permuted order
    int sdim;        // source logical dimension containing it
    int64_t sw;      // its weight inside that source dimension
    int ddim;        // destination logical dimension containing it
    int64_t dw;      // its weight inside that destination dimension
};

}  // namespace

static ja_status build_repart(const Rel& S, const Rel& Dr, const ja_view* view, ja_repart* rp) {
    std::vector<int64_t> sshape(S.shape, S.shape + S.rank), dshape(Dr.shape, Dr.shape + Dr.rank);
    std::vector<int64_t> vshape;
    std::vector<int> perm;
    if (!view) {
        if (sshape != dshape) return fail(JA_ERR_SHAPE, "without a view, source and destination shapes must match");
        vshape = sshape;
        for (int i = 0; i < S.rank; ++i) perm.push_back(i);
    } else {
        if (view->rank < 1 || view->rank > JA_MAX_RANK) return fail(JA_ERR_ARG, "view rank must be 1..8");
        std::vector<bool> seen(view->rank, false);
        for (int i = 0; i < view->rank; ++i) {
            if (view->shape[i] < 1) return fail(JA_ERR_SHAPE, "view extents must be positive");
            int pi = view->perm[i];
            if (pi < 0 || pi >= view->rank || seen[pi]) return fail(JA_ERR_ARG, "view perm is not a permutation");
            seen[pi] = true;
            vshape.push_back(view->shape[i]);
            perm.push_back(pi);
        }
        int64_t nv = 1;
        for (auto x : vshape) nv *= x;
        if (nv != S.elems || nv != Dr.elems) return fail(JA_ERR_SHAPE, "view element count differs from the relations'");
    }
    const int vr = (int)vshape.size();
    std::vector<int64_t> pshape(vr);
    for (int k = 0; k < vr; ++k) pshape[k] = vshape[perm[k]];
    std::vector<int> inv(vr);
    for (int k = 0; k < vr; ++k) inv[perm[k]] = k;

    // --- common factorisation -------------------------------------------------
    auto vst = strides_of(vshape), pst = strides_of(pshape), sst = strides_of(sshape), dst = strides_of(dshape);
    std::vector<std::set<int64_t>> cuts(vr);
    for (int v = 0; v < vr; ++v) {
        cuts[v].insert(1);
        cuts[v].insert(vshape[v]);
    }
    // source dims cut view dims (both row-major over the same linear order)
    for (int d = 0; d <= S.rank; ++d) {
        int64_t c = d < S.rank ? sst[d] * sshape[d] : 1;
        for (int v = 0; v < vr; ++v)
            if (c > vst[v] && c < vst[v] * vshape[v]) {
                if (c % vst[v]) return fail(JA_ERR_UNSUPPORTED, "view shape does not factor the source shape");
                cuts[v].insert(c / vst[v]);
            }
    }
    // destination dims cut permuted dims
    for (int d = 0; d <= Dr.rank; ++d) {
        int64_t c = d < Dr.rank ? dst[d] * dshape[d] : 1;
        for (int k = 0; k < vr; ++k)
            if (c > pst[k] && c < pst[k] * pshape[k]) {
                if (c % pst[k]) return fail(JA_ERR_UNSUPPORTED, "view shape does not factor the destination shape");
                cuts[perm[k]].insert(c / pst[k]);
            }
    }
    // sub-dimensions in view order
    std::vector<Sub> subs;
    std::vector<std::vector<int>> subs_of_v(vr);
    for (int v = 0; v < vr; ++v) {
        auto ext = refine(vshape[v], cuts[v]);
        if (ext.empty()) return fail(JA_ERR_UNSUPPORTED, "reshapes of the view do not factor into common sub-dimensions");
        int64_t inner = vshape[v];
        for (auto e : ext) {
            inner /= e;
            if (e == 1) continue;  // unit sub-dimensions index nothing
            Sub s{};
            s.ext = e;
            s.vdim = v;
            s.vstride = vst[v] * inner;
            s.pstride = pst[inv[v]] * inner;
            subs_of_v[v].push_back((int)subs.size());
            subs.push_back(s);
        }
    }
    const int ns = (int)subs.size();
    for (auto& s : subs) {
        s.sdim = s.ddim = -1;
        for (int d = 0; d < S.rank; ++d)
            if (s.vstride >= sst[d] && s.vstride < sst[d] * sshape[d]) {
                s.sdim = d;
                s.sw = s.vstride / sst[d];
            }
        for (int d = 0; d < Dr.rank; ++d)
            if (s.pstride >= dst[d] && s.pstride < dst[d] * dshape[d]) {
                s.ddim = d;
                s.dw = s.pstride / dst[d];
            }
        if (s.sdim < 0 || s.ddim < 0) return fail(JA_ERR_UNSUPPORTED, "internal: sub-dimension not placed");
    }

    // --- overlay grid with digit refinement --------------------------------------
    std::vector<std::set<int64_t>> pts(ns);
    for (int g = 0; g < ns; ++g) {
        pts[g].insert(0);
        pts[g].insert(subs[g].ext);
    }
    auto add_boundaries = [&](const Rel& R, bool is_src) {
        for (int d = 0; d < R.rank; ++d) {
            // sub-dims of this logical dim, outer to inner
            std::vector<int> grp;
            for (int g = 0; g < ns; ++g)
                if ((is_src ? subs[g].sdim : subs[g].ddim) == d) grp.push_back(g);
            std::sort(grp.begin(), grp.end(), [&](int a, int b) {
                return (is_src ? subs[a].sw : subs[a].dw) > (is_src ? subs[b].sw : subs[b].dw);
            });
            for (size_t bi = 1; bi + 1 < R.sp[d].size(); ++bi) {
                int64_t x = R.sp[d][bi];
                for (size_t k = 0; k < grp.size(); ++k) {
                    const Sub& s = subs[grp[k]];
                    int64_t w = is_src ? s.sw : s.dw;
                    int64_t digit = (x / w) % s.ext;
                    pts[grp[k]].insert(digit);
                    if (k + 1 < grp.size()) pts[grp[k]].insert(std::min(digit + 1, s.ext));
                }
            }
        }
    };
    add_boundaries(S, true);
    add_boundaries(Dr, false);
    std::vector<std::vector<int64_t>> grid(ns);
    int64_t natoms = 1;
    for (int g = 0; g < ns; ++g) {
        grid[g].assign(pts[g].begin(), pts[g].end());
        natoms *= (int64_t)grid[g].size() - 1;
        if (natoms > ((int64_t)1 << 24)) return fail(JA_ERR_UNSUPPORTED, "more than 2^24 atoms");
    }
    rp->n_atoms = natoms;

    // block strides (row-major inside a block) of a relation's block
    auto block_place = [](const Rel& R, const int64_t* x, int64_t* bstride, int64_t& base) {
        int64_t key[JA_MAX_RANK], lo[JA_MAX_RANK], ext[JA_MAX_RANK];
        for (int d = 0; d < R.rank; ++d) {
            key[d] = R.find(d, x[d]);
            lo[d] = R.sp[d][key[d]];
            ext[d] = R.ext(d, key[d]);
        }
        int64_t acc = 1;
        for (int d = R.rank - 1; d >= 0; --d) {
            bstride[d] = acc;
            acc *= ext[d];
        }
        base = R.blk_off[R.block_index(key)];
        for (int d = 0; d < R.rank; ++d) base += (x[d] - lo[d]) * bstride[d];
    };

    const int32_t es = (int32_t)rp->esize;
    std::vector<int64_t> cell(ns, 0);
    for (int64_t a = 0; a < natoms; ++a) {
        int64_t lo[64], n[64];
        for (int g = 0; g < ns; ++g) {
            lo[g] = grid[g][cell[g]];
            n[g] = grid[g][cell[g] + 1] - lo[g];
        }
        int64_t xs[JA_MAX_RANK] = {0}, xd[JA_MAX_RANK] = {0};
        for (int g = 0; g < ns; ++g) {
            xs[subs[g].sdim] += lo[g] * subs[g].sw;
            xd[subs[g].ddim] += lo[g] * subs[g].dw;
        }
        int64_t sbs[JA_MAX_RANK], dbs[JA_MAX_RANK], sbase, dbase;
        block_place(S, xs, sbs, sbase);
        block_place(Dr, xd, dbs, dbase);
        struct Dim {
            int64_t n, ss, ds;
        };
        std::vector<Dim> dims;
        for (int g = 0; g < ns; ++g)
            if (n[g] > 1) dims.push_back({n[g], subs[g].sw * sbs[subs[g].sdim], subs[g].dw * dbs[subs[g].ddim]});
        // destination-major order: the innermost loop walks the smallest destination stride
        std::sort(dims.begin(), dims.end(), [](const Dim& p, const Dim& q) { return p.ds > q.ds; });
        std::vector<Dim> m;
        for (auto& dd : dims) {
            if (!m.empty() && m.back().ss == dd.n * dd.ss && m.back().ds == dd.n * dd.ds) {
                m.back().n *= dd.n;
                m.back().ss = dd.ss;
                m.back().ds = dd.ds;
            } else {
                m.push_back(dd);
            }
        }
        if (m.empty()) m.push_back({1, 1, 1});
        // emit tasks of at most 4 loop levels; extra outer levels loop here
        std::function<void(size_t, int64_t, int64_t)> emit = [&](size_t first, int64_t so, int64_t dof) {
            if (m.size() - first > 4) {
                for (int64_t i = 0; i < m[first].n; ++i) emit(first + 1, so + i * m[first].ss, dof + i * m[first].ds);
                return;
            }
            RepTask t{};
            t.src_off = so;
            t.dst_off = dof;
            int pad = 4 - (int)(m.size() - first);
            for (int k = 0; k < 4; ++k) {
                if (k < pad) {
                    t.n[k] = 1;
                    t.ss[k] = t.ds[k] = 0;
                } else {
                    const Dim& dd = m[first + k - pad];
                    t.n[k] = (int32_t)dd.n;
                    t.ss[k] = dd.ss;
                    t.ds[k] = dd.ds;
                }
            }
            // cut big tasks into chunks of at most REP_CHUNK elements
            std::function<void(RepTask, int)> cut = [&](RepTask u, int lvl) {
                int64_t total = (int64_t)u.n[0] * u.n[1] * u.n[2] * u.n[3];
                if (total <= REP_CHUNK) {
                    rp->tasks.push_back(u);
                    return;
                }
                while (lvl < 3 && u.n[lvl] == 1) ++lvl;
                int64_t inner = 1;
                for (int k = lvl + 1; k < 4; ++k) inner *= u.n[k];
                if (lvl == 3 || inner <= REP_CHUNK) {
                    int64_t per = std::max<int64_t>(1, REP_CHUNK / inner);
                    for (int64_t i0 = 0; i0 < u.n[lvl]; i0 += per) {
                        RepTask v = u;
                        v.n[lvl] = (int32_t)std::min<int64_t>(per, u.n[lvl] - i0);
                        v.src_off = u.src_off + i0 * u.ss[lvl];
                        v.dst_off = u.dst_off + i0 * u.ds[lvl];
                        rp->tasks.push_back(v);
                    }
                } else {
                    for (int64_t i0 = 0; i0 < u.n[lvl]; ++i0) {
                        RepTask v = u;
                        v.n[lvl] = 1;
                        v.src_off = u.src_off + i0 * u.ss[lvl];
                        v.dst_off = u.dst_off + i0 * u.ds[lvl];
                        cut(v, lvl + 1);
                    }
                }
            };
            cut(t, 0);
        };
        emit(0, sbase, dbase);
        for (int g = ns - 1; g >= 0; --g) {
            if (++cell[g] < (int64_t)grid[g].size() - 1) break;
            cell[g] = 0;
        }
    }
    // Every task must stay inside both buffers and, together, the tasks must
    // write exactly as many elements as the destination holds; anything else
    // is a planner bug and is refused before a kernel could run it.
    int64_t covered = 0;
    for (const auto& t : rp->tasks) {
        int64_t smax = t.src_off, dmax = t.dst_off, cnt = 1;
        for (int k = 0; k < 4; ++k) {
            if (t.n[k] < 1 || t.ss[k] < 0 || t.ds[k] < 0) return fail(JA_ERR_UNSUPPORTED, "internal: bad copy task");
            smax += (int64_t)(t.n[k] - 1) * t.ss[k];
            dmax += (int64_t)(t.n[k] - 1) * t.ds[k];
            cnt *= t.n[k];
        }
        if (t.src_off < 0 || t.dst_off < 0 || smax >= S.elems || dmax >= Dr.elems || cnt > REP_CHUNK)
            return fail(JA_ERR_UNSUPPORTED, "internal: copy task out of bounds");
        covered += cnt;
    }
    if (covered != Dr.elems) return fail(JA_ERR_UNSUPPORTED, "internal: copy tasks do not cover the destination");
    // 16-byte vector copies are valid for a task when its innermost loop is
    // contiguous on both sides and every offset and stride is 16-byte aligned.
    const int64_t vec = 16 / es;
    for (auto& t : rp->tasks) {
        bool ok = t.ss[3] == 1 && t.ds[3] == 1 && t.n[3] % vec == 0 && t.src_off % vec == 0 && t.dst_off % vec == 0;
        for (int k = 0; k < 3 && ok; ++k) ok = (t.n[k] == 1) || (t.ss[k] % vec == 0 && t.ds[k] % vec == 0);
        t.flags = ok ? REP_VEC : 0;
    }
    return JA_OK;
}

extern "C" {

ja_status ja_repart_create(const ja_relation_desc* src, const ja_relation_desc* dst, const ja_view* view,
                           ja_repart** out) {
    if (!out) return fail(JA_ERR_ARG, "out is NULL");
    *out = nullptr;
    Rel S, D;
    ja_status st;
    if ((st = rel_from_desc(src, S)) || (st = rel_from_desc(dst, D))) return st;
    if (S.dtype != D.dtype) return fail(JA_ERR_DTYPE, "repartition keeps the dtype");
    ja_repart* rp = new ja_repart();
    rp->esize = (int32_t)dtype_size(S.dtype);
    st = build_repart(S, D, view, rp);
    if (st) {
        delete rp;
        return st;
    }
    *out = rp;
    return JA_OK;
}

ja_status ja_repart_count(const ja_repart* rp, int64_t* n_atoms, int64_t* n_tasks) {
    if (!rp) return fail(JA_ERR_ARG, "repart is NULL");
    if (n_atoms) *n_atoms = rp->n_atoms;
    if (n_tasks) *n_tasks = (int64_t)rp->tasks.size();
    return JA_OK;
}

ja_status ja_repart_device_bytes(const ja_repart* rp, size_t* bytes) {
    if (!rp || !bytes) return fail(JA_ERR_ARG, "NULL argument");
    *bytes = std::max<size_t>(16, rp->tasks.size() * sizeof(RepTask));
    return JA_OK;
}

ja_status ja_repart_upload(ja_repart* rp, void* dev_buf, size_t bytes, void* stream) {
    if (!rp || !dev_buf) return fail(JA_ERR_ARG, "NULL argument");
    size_t need = rp->tasks.size() * sizeof(RepTask);
    if (bytes < need) return fail(JA_ERR_WORKSPACE, "table buffer smaller than ja_repart_device_bytes");
    if ((uintptr_t)dev_buf & 15) return fail(JA_ERR_ARG, "table buffer must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    if (need) {
        JA_TRY_HIP(hipMemcpyAsync(dev_buf, rp->tasks.data(), need, hipMemcpyHostToDevice, st));
        JA_TRY_HIP(hipStreamSynchronize(st));
    }
    rp->dev = dev_buf;
    return JA_OK;
}

ja_status ja_repart_run(const ja_repart* rp, const void* src_ptr, void* dst_ptr, void* stream) {
    if (!rp || !src_ptr || !dst_ptr) return fail(JA_ERR_ARG, "NULL argument");
    if (!rp->dev) return fail(JA_ERR_STATE, "repartition tables are not uploaded");
    if (((uintptr_t)src_ptr & 15) || ((uintptr_t)dst_ptr & 15)) return fail(JA_ERR_ARG, "buffers must be 16-byte aligned");
    if (rp->tasks.empty()) return JA_OK;
    JA_TRY_HIP(launch_repart(rp->dev, (int64_t)rp->tasks.size(), src_ptr, dst_ptr, rp->esize, 1, (hipStream_t)stream));
    return JA_OK;
}

void ja_repart_destroy(ja_repart* rp) { delete rp; }

ja_status ja_repartition_workspace_bytes(const ja_relation_desc* src, const ja_relation_desc* dst,
                                         const ja_view* view, size_t* bytes) {
    if (!bytes) return fail(JA_ERR_ARG, "bytes is NULL");
    ja_repart* rp = nullptr;
    ja_status st = ja_repart_create(src, dst, view, &rp);
    if (st) return st;
    ja_repart_device_bytes(rp, bytes);
    ja_repart_destroy(rp);
    return JA_OK;
}

ja_status ja_repartition(const ja_relation_desc* src, const void* src_ptr, const ja_relation_desc* dst,
                         void* dst_ptr, const ja_view* view, void* dev_ws, size_t ws_bytes, void* stream) {
    ja_repart* rp = nullptr;
    ja_status st = ja_repart_create(src, dst, view, &rp);
    if (st) return st;
    st = ja_repart_upload(rp, dev_ws, ws_bytes, stream);
    if (!st) st = ja_repart_run(rp, src_ptr, dst_ptr, stream);
    ja_repart_destroy(rp);
    return st;
}

}  // extern "C"
