// djoin.cpp -- host side of the device-side join: the argument block, the
// static table (packed sequence ends), the workspace layout and the launch.
#include <algorithm>
#include <cstring>

#include "../ja_join.h"
#include "ja_host.h"

namespace ja {
hipError_t launch_djoin(const DJoinArgs& a, const int64_t* splits, const int64_t* ends, int32_t* rec,
                        int64_t* seg_off, int64_t* counts, uint32_t* ccnt, uint32_t* cbase, uint32_t* gcnt,
                        uint32_t* gbase, uint32_t* gpre, hipStream_t stream);

namespace {

DJDiv make_div(uint32_t d) {
    DJDiv f{d, 0, 0, 0};
    if (d > 1) {
        uint32_t l = 0;
        while (((uint64_t)1 << l) < d) ++l;  // ceil(log2 d)
        f.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
        f.s = l - 1;
    }
    return f;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace
}  // namespace ja

struct ja_djoin {
    ja::DJoinArgs a;
    std::vector<int64_t> ends;  // packed sequence ends (the table)
    size_t off_ccnt = 0, off_cbase = 0, off_gcnt = 0, off_gbase = 0, off_gpre = 0, ws_bytes = 0;
    void* dev = nullptr;
};

using namespace ja;

extern "C" {

ja_status ja_djoin_create(const ja_spec* s, const int64_t* extents, const int32_t* intervals, ja_djoin** out) {
    if (!out) return fail(JA_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (!s || !extents || !intervals) return fail(JA_ERR_ARG, "NULL argument");
    const int nl = (int)s->letters.size();
    if (nl < 1 || nl > DJ_MAX_LETTERS) return fail(JA_ERR_UNSUPPORTED, "device join: 1 to 26 letters");
    for (int i = 0; i < nl; ++i)
        if (extents[i] < 1 || intervals[i] < 1 || intervals[i] > extents[i])
            return fail(JA_ERR_DECOMP, std::string("letter ") + s->letters[i] +
                                           ": extent must be positive and the interval count in [1, extent]");
    if (s->kind == JA_OP_ATTENTION) {
        const std::string &q = s->ins[0], &k = s->ins[1];
        if (intervals[s->letter_index(q.back())] != 1)
            return fail(JA_ERR_DECOMP, "attention: the head-dimension letter cannot be split");
        if (s->packed_device) {
            const int ls = s->letter_index(s->att_s), lt = s->letter_index(s->att_t);
            if (extents[ls] != extents[lt] || intervals[ls] != intervals[lt])
                return fail(JA_ERR_DECOMP, "attention: packed=device needs the same cuts on both sequence letters");
        }
        if (!s->packed.empty())
            for (char c : {s->att_s, s->att_t}) {
                const int l = s->letter_index(c);
                if (extents[l] != s->packed.back() || intervals[l] > (int64_t)s->packed.size())
                    return fail(JA_ERR_DECOMP, std::string("attention: letter ") + c +
                                                   " must span every packed sequence, with at most one interval per sequence");
            }
    }
    ja_djoin* j = new ja_djoin();
    DJoinArgs& a = j->a;
    std::memset(&a, 0, sizeof(a));
    a.nl = nl;
    // iteration order: the group-by letters first, then the rest in letter order
    std::vector<int> order;
    for (char c : s->group_by) order.push_back(s->letter_index(c));
    for (int i = 0; i < nl; ++i)
        if (s->group_by.find(s->letters[i]) == std::string::npos) order.push_back(i);
    int64_t ncell = 1, ngroup = 1, nsplit = 0;
    for (int i = 0; i < nl; ++i) {
        a.cnt[i] = intervals[i];
        a.ext[i] = extents[i];
        a.sp_off[i] = (int32_t)nsplit;
        nsplit += a.cnt[i] + 1;
        ncell *= a.cnt[i];
        if (ncell > DJ_MAX_CELLS) {
            delete j;
            return fail(JA_ERR_UNSUPPORTED, "device join: more than 2^28 grid cells");
        }
    }
    int64_t stride = 1;
    for (int k = nl - 1; k >= 0; --k) {
        const int l = order[k];
        a.stride[l] = make_div((uint32_t)stride);
        a.count[l] = make_div((uint32_t)a.cnt[l]);
        stride *= a.cnt[l];
    }
    for (size_t g = 0; g < s->group_by.size(); ++g) ngroup *= a.cnt[order[g]];
    a.ncell = (uint32_t)ncell;
    a.ngroup = (uint32_t)ngroup;
    a.inner = make_div((uint32_t)(ncell / ngroup));
    a.nchunk = (uint32_t)((ncell + DJ_CHUNK - 1) / DJ_CHUNK);
    a.ngchunk = (uint32_t)((ngroup + DJ_CHUNK - 1) / DJ_CHUNK);
    a.nsplit = (uint32_t)nsplit;
    a.is = a.it = a.ps = a.pt = -1;
    if (s->causal) {
        a.is = s->letter_index(s->causal_s);
        a.it = s->letter_index(s->causal_t);
    }
    if (!s->packed.empty() || s->packed_device) {
        a.ps = s->letter_index(s->att_s);
        a.pt = s->letter_index(s->att_t);
        j->ends = s->packed;
        a.nends = s->packed_device ? -1 : (int32_t)s->packed.size();
    }
    if (j->ends.empty()) j->ends.assign(2, 0);  // a non-empty table
    size_t o = 0;
    j->off_ccnt = o;
    o = align256(o + 4 * (size_t)a.nchunk);
    j->off_cbase = o;
    o = align256(o + 4 * (size_t)a.nchunk);
    j->off_gcnt = o;
    o = align256(o + 4 * (size_t)a.ngchunk);
    j->off_gbase = o;
    o = align256(o + 4 * (size_t)a.ngchunk);
    j->off_gpre = o;
    o = align256(o + 4 * ((size_t)ngroup + 1));
    j->ws_bytes = o;
    *out = j;
    return JA_OK;
}

ja_status ja_djoin_device_bytes(const ja_djoin* j, size_t* table_bytes, size_t* workspace_bytes,
                                int64_t* max_tuples, int64_t* max_segs, int64_t* n_splits) {
    if (!j) return fail(JA_ERR_ARG, "device join is NULL");
    if (table_bytes) *table_bytes = j->ends.size() * sizeof(int64_t);
    if (workspace_bytes) *workspace_bytes = j->ws_bytes;
    if (max_tuples) *max_tuples = j->a.ncell;
    if (max_segs) *max_segs = j->a.ngroup;
    if (n_splits) *n_splits = j->a.nsplit;
    return JA_OK;
}

ja_status ja_djoin_upload(ja_djoin* j, void* dev_buf, size_t bytes, void* stream) {
    if (!j || !dev_buf) return fail(JA_ERR_ARG, "NULL argument");
    const size_t need = j->ends.size() * sizeof(int64_t);
    if (bytes < need) return fail(JA_ERR_WORKSPACE, "table buffer smaller than ja_djoin_device_bytes");
    if ((uintptr_t)dev_buf & 15) return fail(JA_ERR_ARG, "table buffer must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    JA_TRY_HIP(hipMemcpyAsync(dev_buf, j->ends.data(), need, hipMemcpyHostToDevice, st));
    JA_TRY_HIP(hipStreamSynchronize(st));
    j->dev = dev_buf;
    return JA_OK;
}

ja_status ja_djoin_run(const ja_djoin* j, const int64_t* splits_dev, int32_t* rec, int64_t* seg_off,
                       int64_t* counts, void* workspace, void* stream) {
    if (!j) return fail(JA_ERR_ARG, "device join is NULL");
    if (!j->dev) return fail(JA_ERR_STATE, "device join table is not uploaded");
    if (!splits_dev || !rec || !seg_off || !counts || !workspace) return fail(JA_ERR_ARG, "NULL buffer");
    if (((uintptr_t)splits_dev | (uintptr_t)seg_off | (uintptr_t)counts) & 7)
        return fail(JA_ERR_ARG, "split, segment and count buffers must be 8-byte aligned");
    if ((uintptr_t)rec & 3) return fail(JA_ERR_ARG, "record buffer must be 4-byte aligned");
    if ((uintptr_t)workspace & 255) return fail(JA_ERR_ARG, "workspace must be 256-byte aligned");
    uint8_t* ws = (uint8_t*)workspace;
    JA_TRY_HIP(launch_djoin(j->a, splits_dev, (const int64_t*)j->dev, rec, seg_off, counts,
                            (uint32_t*)(ws + j->off_ccnt), (uint32_t*)(ws + j->off_cbase),
                            (uint32_t*)(ws + j->off_gcnt), (uint32_t*)(ws + j->off_gbase),
                            (uint32_t*)(ws + j->off_gpre), (hipStream_t)stream));
    return JA_OK;
}

void ja_djoin_destroy(ja_djoin* j) { delete j; }

}  // extern "C"
