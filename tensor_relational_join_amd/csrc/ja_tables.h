// ja_tables.h -- plain-old-data records that the host planner writes into a
// plan's device table and the HIP kernels read.  Shared by the host core and
// the kernels of libja only.
#pragma once
#include <stdint.h>

namespace ja {

// ---------------------------------------------------------------- contract
// A GEMM-shaped view of one tuple: every operand block is a dense row-major
// box whose letters group into [batch..., rows..., cols...] runs, so a block
// is `nbatch` matrices.  Offsets and strides are in elements.

// One unit of workgroup work: an output tile of one segment.
struct GemmTile {
    int32_t seg;    // segment (= output block) index
    int32_t m0;     // first output row of the tile inside the block
    int32_t n0;     // first output column of the tile inside the block
    int32_t batch;  // batch index inside the block
};

// One aggregation segment: all tuples that write the same output block.
struct GemmSeg {
    int64_t c_off;      // output block offset
    int64_t c_bstride;  // output batch stride
    int32_t M, N, ldc;  // block rows, block columns, row pitch
    int32_t t_begin, t_end;  // tuple range [t_begin, t_end)
    int32_t nst;             // contracted stages of the tuples: the sum of ceil(K / GEMM_DMA_BK)
};

// One joined tuple: the A block and the B block it multiplies.
struct GemmTuple {
    int64_t a_off, b_off;
    int64_t a_bstride, b_bstride;
    int32_t K;         // contracted extent of the tuple
    int32_t lda, ldb;  // pitch of the A and B matrices
    int32_t pad;
};

// Layout of an operand matrix inside its block.
enum : int32_t {
    JA_A_MK = 0,  // A[m][k] at m*lda + k (k contiguous)
    JA_A_KM = 1,  // A[m][k] at k*lda + m (m contiguous)
    JA_B_KN = 0,  // B[k][n] at k*ldb + n (n contiguous)
    JA_B_NK = 1,  // B[k][n] at n*ldb + k (k contiguous)
};

// What the contraction kernel does with an aggregated output tile on its way
// out (a 1:1 join on the output key applied before the single write).
enum : int32_t {
    JA_EPI_NONE = 0,    // write the aggregated block
    JA_EPI_ADD = 1,     // add the residual relation's element at the same offset
    JA_EPI_SWIGLU = 2,  // columns come in (gate, up) pairs: write silu(gate) * up, one element per pair
};

// ---------------------------------------------------------------- attention
struct AttnTile {
    int32_t seg;  // segment = one (batch-heads, query interval) output block
    int32_t bh;   // batch-head index inside the block
    int32_t s0;   // first query row of the tile inside the block
    int32_t pad;
};

// A Q, K, V or O block is [outer batch-heads][rows][inner batch-heads][D]:
// the batch-head letters before the position letter index whole [rows][inner]
// [D] slabs, those after it (token-major relations) sit inside a row.  With
// hin inner batch-heads, batch-head bh's row r starts at element
//   (bh / hin) * bstride + (bh % hin) * D + r * hin * D.
struct AttnSeg {
    int64_t q_off, o_off;  // Q block and O block offsets (O has Q's letters)
    int64_t q_bstride;     // S * q_hin * D
    int32_t S;             // query rows in the block
    int32_t s_lo;          // global query index of the block's first row
    int32_t t_begin, t_end;
    int32_t rep;           // query batch-heads per key-value batch-head: K/V index = bh / rep
    int32_t q_hin;         // inner batch-heads of the Q and O blocks
    int32_t kv_hin;        // inner batch-heads of the segment's K and V blocks
    int32_t pad;
};

struct AttnTuple {
    int64_t k_off, v_off;
    int64_t kv_bstride;  // T * kv_hin * D
    int32_t T;           // keys in the block
    int32_t t_lo;        // global key index of the block's first key
};

// ---------------------------------------------------------------- rmsnorm
struct NormBlock {
    int64_t off;    // offset of the (row interval, column interval) block
    int32_t width;  // columns in the block
    int32_t d_lo;   // first column (= offset of the gain block)
};

// ---------------------------------------------------------------- aggregation
struct AggTile {
    int32_t seg;
    int32_t e0;  // first element of the chunk inside the output block
};

struct AggSeg {
    int64_t out_off;
    int32_t nelem;
    int32_t t_begin, t_end;
    int32_t pad;
};

// ---------------------------------------------------------------- repartition
// One copy task: a 4-deep strided loop nest (n[3] innermost) copying
// n[0]*n[1]*n[2]*n[3] elements from src_off + i.ss to dst_off + i.ds.
struct RepTask {
    int64_t src_off, dst_off;
    int64_t ss[4], ds[4];
    int32_t n[4];
    int32_t flags;  // REP_VEC
    int32_t pad;
};

}  // namespace ja

namespace ja {
// Tile shapes shared by the planner (which enumerates tiles) and the kernels.
constexpr int GEMM_BF16_TM = 256;  // output rows per workgroup tile, bf16 MFMA kernel
constexpr int GEMM_BF16_TN = 256;  // output columns per workgroup tile
constexpr int GEMM_GROUP_M = 4;    // row tiles per group in the tile order (L2 reuse)
constexpr int GEMM_DMA_STAGES = 4; // 32-wide stages in flight in the direct-to-LDS kernel
constexpr int GEMM_DMA_BK = 32;     // contracted elements per stage of the 16-bit kernels
constexpr int GEMM_F32_TM = 64;    // fp32 kernel tile
constexpr int GEMM_F32_TN = 64;
constexpr int ATTN_TQ = 128;       // query rows per attention workgroup
constexpr int ATTN_D = 128;        // head dimension the attention kernel is built for
constexpr int ATTN_PROW = 132;     // f32 per query row of an attention partial: m, l, 2 pad, acc[128]
constexpr int SMAX_ROWS = 8;       // query rows per softmax-aggregation workgroup
constexpr int AGG_CHUNK = 2048;    // output elements per aggregation workgroup
constexpr int REP_CHUNK = 16384;   // max elements per repartition task
constexpr int REP_VEC = 1;         // RepTask.flags bit: 16-byte vector copies are valid
}  // namespace ja
