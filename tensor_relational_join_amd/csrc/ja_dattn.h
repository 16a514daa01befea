// ja_dattn.h -- the argument block of the device-side attention planner,
// written by the host (host/dattn.cpp) and read by the table-building kernels
// (hip/dattn.hip).
//
// Packed sequences whose ends are the cuts of the sequence letters
// ("packed=device"): the device-side join lists the (query block, key block)
// tuples, and these kernels turn its records into the attention kernel's
// tables (segments, tuples, 128-row tiles) without the host.  Q and O are
// stored blocked by the batch and group letters only ([batch..., group..., S,
// D], s and d whole), K and V by their batch letters only, so a block of a
// sequence is a run of rows inside its batch-head block and the layout does
// not depend on where the sequences end.
#pragma once
#include <stdint.h>

namespace ja {

constexpr int DA_MAX_LETTERS = 8;  // batch and group letters of Q (of K)
constexpr int DA_THREADS = 256;
constexpr int DA_SCAN_THREADS = 1024;

struct DAttnArgs {
    int32_t nl;              // letters of the spec
    int32_t ls, lt;          // the query and key sequence letters
    int32_t nq, nk;          // batch (+ group) letters of Q, batch letters of K
    int32_t qlet[DA_MAX_LETTERS], qcnt[DA_MAX_LETTERS];  // in Q's order: letter, intervals
    int32_t klet[DA_MAX_LETTERS], kcnt[DA_MAX_LETTERS];  // in K's order
    int32_t sp_s, sp_t;      // first split point of s and of t in the split array
    int32_t nseq;            // sequences (intervals of s and of t)
    int32_t D;               // head dimension
    int64_t S;               // extent of s and t
    uint32_t max_segs, max_tuples, max_tiles;
    uint32_t nbucket;        // 128-row tile positions inside a sequence: ceil(S / 128)
};

}  // namespace ja
