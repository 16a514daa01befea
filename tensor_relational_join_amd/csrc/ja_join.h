// ja_join.h -- the argument block of the device-side join, written by the
// host (host/djoin.cpp) and read by the join kernels (hip/join.hip).
//
// The join of "Every Kernel Is a Join" (section 3.2, step 1; section 3.3)
// enumerates the cells of the interval grid of a decomposition, keeps the
// cells the operator's join predicate allows, orders them by the group-by
// key and cuts equal keys into aggregation segments.  The grid is walked in
// "iteration order": the group-by letters first (in group-by order), then the
// other letters in letter order, the last one fastest; cell c of that walk
// has, for every letter, interval index (c / stride) mod count.  Kept cells in
// walk order are exactly the sorted tuple list, and the cells of group g are
// the contiguous run [g * ninner, (g + 1) * ninner).
#pragma once
#include <stdint.h>

namespace ja {

constexpr int DJ_MAX_LETTERS = 26;
constexpr int DJ_THREADS = 256;                   // threads per workgroup of the chunked kernels
constexpr int DJ_CPT = 16;                        // grid cells (or groups) per thread
constexpr int DJ_CHUNK = DJ_THREADS * DJ_CPT;     // cells (or groups) per workgroup
constexpr int DJ_SCAN_THREADS = 1024;             // the one-workgroup scan of chunk counts
constexpr int64_t DJ_MAX_CELLS = (int64_t)1 << 28;

// Unsigned 32-bit division by an invariant d >= 1 with a multiply-high
// (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", 1994, the round-up variant): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, t = mulhi(n, m) and
// q = (t + ((n - t) >> 1)) >> (l - 1) equals floor(n / d) for every 32-bit n.
struct DJDiv {
    uint32_t d, m, s, pad;
};

// Status bits the join writes into counts[2].
enum : int32_t {
    DJ_BAD_SPLITS = 1,  // split points do not start at 0, end at the extent and rise strictly
    DJ_BAD_PACKED = 2,  // a packed sequence letter cut away from a sequence end
    DJ_BAD_SEQS = 4,    // sequences given by the cuts: the two sequence letters cut differently
};

struct DJoinArgs {
    int32_t nl;           // letters
    int32_t is, it;       // causal query / key letters (-1: no causal predicate)
    int32_t ps, pt;       // packed-sequence query / key letters (-1: not packed)
    int32_t nends;        // packed sequence ends in the table (-1: the cuts are the ends)
    uint32_t ncell;       // grid cells (product of the interval counts)
    uint32_t ngroup;      // group-by keys (product of the group-by letters' counts)
    uint32_t nchunk;      // workgroups over cells
    uint32_t ngchunk;     // workgroups over groups
    uint32_t nsplit;      // split points in the device array (sum of counts + 1)
    uint32_t pad;
    int32_t sp_off[DJ_MAX_LETTERS];  // first split point of each letter in the device array
    int32_t cnt[DJ_MAX_LETTERS];     // intervals of each letter
    int64_t ext[DJ_MAX_LETTERS];     // extent of each letter
    DJDiv stride[DJ_MAX_LETTERS];    // cells between consecutive interval indices of the letter
    DJDiv count[DJ_MAX_LETTERS];     // the interval count as a divisor
    DJDiv inner;                     // cells per group
};

}  // namespace ja
