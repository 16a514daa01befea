// ja_host.h -- internal host-side structures of libja.
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../../include/ja.h"
#include "../ja_tables.h"

namespace ja {

// ---- errors --------------------------------------------------------------
ja_status fail(ja_status st, const std::string& msg);
void clear_error();
ja_status hip_fail(hipError_t e, const char* what);

#define JA_TRY_HIP(expr)                                        \
    do {                                                        \
        hipError_t _e = (expr);                                 \
        if (_e != hipSuccess) return ::ja::hip_fail(_e, #expr); \
    } while (0)

size_t dtype_size(int32_t dtype);

// ---- relations -------------------------------------------------------------
// A validated relation descriptor with its block offsets precomputed.
struct Rel {
    int rank = 0;
    int32_t dtype = 0;
    int64_t shape[JA_MAX_RANK] = {0};
    std::vector<int64_t> sp[JA_MAX_RANK];  // split points per dimension
    int64_t nblocks = 0;
    int64_t elems = 0;
    std::vector<int64_t> blk_off;  // element offset of each block, lexicographic key order

    int nblk(int d) const { return (int)sp[d].size() - 1; }
    // Linear block index of a key (lexicographic, first dimension slowest).
    int64_t block_index(const int64_t* key) const;
    // Block extents (hi - lo) of the block with the given key.
    int64_t ext(int d, int64_t k) const { return sp[d][k + 1] - sp[d][k]; }
    // Index of the interval of dimension d that contains x.
    int64_t find(int d, int64_t x) const;
};

ja_status rel_from_desc(const ja_relation_desc* desc, Rel& out);
// Near-equal split points (first n mod q intervals one longer).
std::vector<int64_t> equal_splits(int64_t n, int64_t q);
ja_status check_splits(const int64_t* pts, int64_t n, int64_t q, std::vector<int64_t>& out, const char* what);

}  // namespace ja

// ---- opaque handles ------------------------------------------------------------
enum ja_op_kind { JA_OP_CONTRACT = 0, JA_OP_ATTENTION, JA_OP_RMSNORM, JA_OP_SWIGLU, JA_OP_ADD };

struct ja_spec {
    ja_op_kind kind;
    std::vector<std::string> ins;
    std::string out;
    std::string letters;   // first-appearance order
    std::string group_by;  // letters of the aggregation key, in order
    double scale = 0.0;
    bool has_scale = false;
    bool causal = false;
    char causal_s = 0, causal_t = 0;
    // attention: the query and key position letters.  Q = O = [outer..., s,
    // inner..., d] and K = V = [outer..., t, inner..., d]: the letters other
    // than s (t) and d index batch-heads, those after s (t) stored inside a
    // row (token-major relations), those before it outside
    char att_s = 0, att_t = 0;
    std::vector<int64_t> packed;  // attention: ascending ends of sequences packed along the s and t letters
    bool packed_device = false;   // attention: the sequences end exactly at the cuts of the s and t letters
    int32_t epilogue = 0;         // contract: JA_EPI_NONE, JA_EPI_ADD (third operand R) or JA_EPI_SWIGLU
    char pair = 0;                // contract_swiglu: B's last letter, (gate, up) = (0, 1), absent from A and C
    double eps = 1e-6;
    int letter_index(char c) const {
        auto p = letters.find(c);
        return p == std::string::npos ? -1 : (int)p;
    }
};

struct ja_decomp {
    std::string letters;
    std::vector<int64_t> ext;
    std::vector<std::vector<int64_t>> sp;
};

struct ja_tuples {
    int32_t nl = 0;
    std::vector<int32_t> rec;     // n * nl interval indices, letter order
    std::vector<int64_t> seg;     // CSR offsets, nseg + 1
    int64_t count() const { return nl ? (int64_t)rec.size() / nl : 0; }
};

namespace ja {
ja_status build_tuples(const ja_spec* spec, const ja_decomp* d, ja_tuples& t);
}

// ---- kernel launchers (implemented in the .hip sources) --------------------
namespace ja {
hipError_t launch_gemm(const void* table, int64_t tiles_off, int32_t ntiles, int64_t segs_off, int64_t tuples_off,
                       const void* A, const void* B, void* C, const void* R, int32_t epi, int32_t in_dtype,
                       int32_t out_dtype, int32_t a_layout, int32_t b_layout, hipStream_t stream);
// seq_off / nseq: the packed sequences' int32 end positions in the table (nseq = 0: not packed)
// partial: write the per-tuple softmax triples instead of O; flags: bf16, 4
// words per tile for the range check (see attention.hip), unused for f16
hipError_t launch_attention(const void* table, int64_t tiles_off, int32_t ntiles, int64_t segs_off,
                            int64_t tuples_off, int64_t seq_off, int32_t nseq, const void* Q, const void* K,
                            const void* V, void* O, uint32_t* flags, float scale, int32_t causal, int32_t f16,
                            int32_t partial, hipStream_t stream);
hipError_t launch_smax_agg(const void* table, int64_t tiles_off, int32_t ntiles, int64_t segs_off, int64_t poff_off,
                           const float* partials, void* out, int32_t f16, hipStream_t stream);
hipError_t launch_rmsnorm(const void* table, int64_t rsplit_off, int32_t nrb, int64_t blocks_off, int32_t ndb,
                          int64_t rows, int32_t D, int32_t W, const void* x, const void* gain, void* y, float eps,
                          int32_t vec, int32_t f16, hipStream_t stream);
hipError_t launch_swiglu(const void* g, const void* u, void* h, int64_t n, int32_t f16, hipStream_t stream);
hipError_t launch_add(const void* a, const void* b, void* c, int64_t n, int32_t f16, hipStream_t stream);
hipError_t launch_agg(const void* table, int64_t tiles_off, int32_t ntiles, int64_t segs_off, int64_t poff_off,
                      const float* partials, void* out, int32_t out_dtype, int32_t op, hipStream_t stream);
hipError_t launch_repart(const void* table, int64_t ntasks, const void* src, void* dst, int32_t esize,
                         int32_t vec_ok, hipStream_t stream);
}  // namespace ja
