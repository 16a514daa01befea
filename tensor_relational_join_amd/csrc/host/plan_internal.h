// plan_internal.h -- the plan object and the table helpers shared by the
// planners of libja (plan.cpp: attention, RMSNorm, 1:1 joins and the ABI;
// plan_contract.cpp: contractions).
#pragma once
#include <algorithm>
#include <cstring>

#include "ja_host.h"

struct ja_plan {
    ja_op_kind kind;
    std::vector<uint8_t> table;
    void* dev = nullptr;
    int32_t n_in = 0;
    // contract
    int64_t tiles_off = 0, segs_off = 0, tuples_off = 0;
    int32_t ntiles = 0;
    int64_t utiles_off = 0, usegs_off = 0;
    int32_t nutiles = 0;
    int64_t atiles_off = 0, asegs_off = 0, apoff_off = 0;
    int32_t natiles = 0;
    int32_t in_dtype = 0, out_dtype = 0, a_layout = 0, b_layout = 0;
    int32_t epilogue = 0;  // JA_EPI_*: the 1:1 join applied to the aggregated tile on its way out
    int64_t partial_elems = 0;
    // attention
    float scale = 0.f;
    int32_t causal = 0;
    int32_t att_inner = 0;  // some block stores batch-heads inside a row (token-major)
    int64_t seq_off = 0;  // packed sequences: int32 sequence ends in the table
    int32_t nseq = 0;
    // rmsnorm
    int64_t rsplit_off = 0, nblk_off = 0;
    int32_t nrb = 0, ndb = 0, D = 0, norm_vec = 0, norm_w = 0;
    int64_t rows = 0;
    float eps = 0.f;
    // 1:1 joins
    int64_t n = 0;
};

namespace ja {

// Append a POD array to the table at a 16-byte aligned offset.
template <class T>
inline int64_t put(std::vector<uint8_t>& tab, const std::vector<T>& v) {
    size_t off = (tab.size() + 15) & ~(size_t)15;
    tab.resize(off + v.size() * sizeof(T));
    if (!v.empty()) std::memcpy(tab.data() + off, v.data(), v.size() * sizeof(T));
    return (int64_t)off;
}

// Check that relation `r` is the projection grid the decomposition asks for:
// one dimension per letter of `s`, extents and split points equal to the
// decomposition's for those letters.
inline ja_status match_rel(const Rel& r, const std::string& s, const ja_spec* sp, const ja_decomp* d, const char* what) {
    if (r.rank != (int)s.size())
        return fail(JA_ERR_SHAPE, std::string(what) + ": rank differs from its letters '" + s + "'");
    for (int k = 0; k < r.rank; ++k) {
        int l = sp->letter_index(s[k]);
        if (r.shape[k] != d->ext[l])
            return fail(JA_ERR_SHAPE, std::string(what) + ": extent of letter " + s[k] + " differs from the decomposition");
        if (r.sp[k] != d->sp[l])
            return fail(JA_ERR_SHAPE, std::string(what) + ": blocking of letter " + s[k] +
                                          " differs from the decomposition (repartition it first)");
    }
    return JA_OK;
}

// The same check for a relation that may be blocked coarser than the
// decomposition: each of its split points is one of the decomposition's, so
// every interval of the decomposition lies inside one of its blocks.
inline ja_status match_rel_coarse(const Rel& r, const std::string& s, const ja_spec* sp, const ja_decomp* d,
                                  const char* what) {
    if (r.rank != (int)s.size())
        return fail(JA_ERR_SHAPE, std::string(what) + ": rank differs from its letters '" + s + "'");
    for (int k = 0; k < r.rank; ++k) {
        int l = sp->letter_index(s[k]);
        if (r.shape[k] != d->ext[l])
            return fail(JA_ERR_SHAPE, std::string(what) + ": extent of letter " + s[k] + " differs from the decomposition");
        for (int64_t x : r.sp[k])
            if (!std::binary_search(d->sp[l].begin(), d->sp[l].end(), x))
                return fail(JA_ERR_SHAPE, std::string(what) + ": blocking of letter " + s[k] +
                                              " is neither the decomposition's nor coarser (repartition it first)");
    }
    return JA_OK;
}

// Interval index of letter c in tuple record `rec`.
inline int64_t coord(const ja_spec* s, const int32_t* rec, char c) { return rec[s->letter_index(c)]; }

inline int64_t block_of(const Rel& r, const std::string& letters, const ja_spec* s, const int32_t* rec) {
    int64_t key[JA_MAX_RANK];
    for (size_t k = 0; k < letters.size(); ++k) key[k] = coord(s, rec, letters[k]);
    return r.block_index(key);
}

inline int64_t extent_of(const ja_decomp* d, const ja_spec* s, const int32_t* rec, const std::string& letters) {
    int64_t n = 1;
    for (char c : letters) {
        int l = s->letter_index(c);
        n *= d->sp[l][rec[l] + 1] - d->sp[l][rec[l]];
    }
    return n;
}

ja_status plan_contract(ja_plan* p, const ja_spec* s, const ja_decomp* d, const ja_tuples& t,
                        const ja_relation_desc* const* in, const ja_relation_desc* out);
}  // namespace ja
