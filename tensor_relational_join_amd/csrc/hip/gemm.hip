// gemm.hip -- the contraction join-agg: per-tuple block products with the SUM
// aggregation fused in.
//
// A matrix multiply is a join of A blocks and B blocks on the contracted
// index followed by a SUM over the contracted blocks ("Every Kernel Is a
// Join", paperpeel full text, section 1 and section 3.2, Examples 3.8 and
// 3.9).  Here one workgroup owns one output tile of one segment (all tuples
// that write one output block).  It walks the segment's tuples in ascending
// order and, inside each tuple, the contracted extent in BK-wide stages,
// accumulating in fp32 registers across tuple boundaries; the aggregated tile
// is written once.  So the SUM costs no extra memory traffic and needs no
// atomics (eager aggregation pushed into the kernel).
//
// bf16 path: v_mfma_f32_16x16x32_bf16 on CDNA4.  A workgroup of 8 wavefronts
// owns a 256 x 256 output tile (128 x 64 per wavefront), which keeps the
// operand traffic from L2 at 64 KiB per 8.4 MFLOP stage.  Operand tiles are
// staged through LDS as [row][k] (k contiguous) so that every MFMA operand
// fragment is one 16-byte LDS read; an operand whose k is not contiguous in
// memory is transposed in registers on its way to LDS (4 x 8 sub-blocks).
// LDS is double buffered (128 KiB of the 160 KiB per CU); the global loads of
// stage i+1 are in flight while stage i multiplies.  The host lists the tiles
// of a segment in groups of GEMM_GROUP_M row tiles, and xcd_remap hands each
// XCD a contiguous run of that list, so the tiles resident on one XCD share A
// and B panels in its L2.
#include <type_traits>

#include "dev_common.h"

namespace ja {

// ---------------------------------------------------------------- bf16 MFMA
// LDS operand tiles are [rows][BK] bf16 with no padding.  The 16-byte chunk c
// (8 consecutive k) of row r sits at chunk position c ^ swz(r), with
// swz(r) = (r ^ (r >> 3)) mod (BK / 8).  Both access patterns are then free
// of bank conflicts: an MFMA fragment read (16 consecutive rows, one logical
// chunk) touches 8 distinct chunk positions in every group of 8 rows, and the
// transposing writes (rows 8 apart, one logical chunk) spread over all of
// them as well.
template <int BK>
__device__ __forceinline__ int lds_chunk(int r, int c) {
    return r * BK + ((c ^ ((r ^ (r >> 3)) & (BK / 8 - 1))) << 3);
}

// Operand whose k is contiguous in memory: element (r, k) at p[r*ld + k].
// Each thread moves VPT 16-byte chunks; 8 consecutive lanes cover one row.
template <int R, int BK, int NT>
struct DirectStage {
    static constexpr int CPR = BK / 8;
    static constexpr int VPT = R * CPR / NT;
    static_assert(R * CPR % NT == 0, "staging must divide evenly");
    uint4 v[VPT];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ p, int64_t ld, int r0, int rext, int k0,
                                         int kext, int tid) {
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int vi = tid + j * NT, r = vi / CPR, c = vi % CPR;
            const int gr = r0 + r, gk = k0 + c * 8;
            v[j] = make_uint4(0, 0, 0, 0);
            if (gr < rext && gk < kext) v[j] = *reinterpret_cast<const uint4*>(p + (int64_t)gr * ld + gk);
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int vi = tid + j * NT;
            *reinterpret_cast<uint4*>(lds + lds_chunk<BK>(vi / CPR, vi % CPR)) = v[j];
        }
    }
};

// Operand whose rows are contiguous in memory: element (r, k) at p[k*ld + r].
// Each thread loads sub-blocks of 4 k x 8 rows (four 16-byte loads along the
// rows, 32 lanes cover 256 consecutive rows) and transposes them in
// registers into eight 8-byte runs of 4 consecutive k.
template <int R, int BK, int NT>
struct TransStage {
    static constexpr int RG = R / 8;
    static constexpr int SPT = (BK / 4) * RG / NT;
    static_assert((BK / 4) * RG % NT == 0, "staging must divide evenly");
    uint4 v[SPT * 4];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ p, int64_t ld, int r0, int rext, int k0,
                                         int kext, int tid) {
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int si = tid + j * NT, kg = si / RG, rg = si % RG;
            const int gr = r0 + rg * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int gk = k0 + kg * 4 + i;
                v[j * 4 + i] = make_uint4(0, 0, 0, 0);
                if (gr < rext && gk < kext) v[j * 4 + i] = *reinterpret_cast<const uint4*>(p + (int64_t)gk * ld + gr);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int si = tid + j * NT, kg = si / RG, rg = si % RG;
            const uint32_t* q0 = reinterpret_cast<const uint32_t*>(&v[j * 4 + 0]);
            const uint32_t* q1 = reinterpret_cast<const uint32_t*>(&v[j * 4 + 1]);
            const uint32_t* q2 = reinterpret_cast<const uint32_t*>(&v[j * 4 + 2]);
            const uint32_t* q3 = reinterpret_cast<const uint32_t*>(&v[j * 4 + 3]);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // rows 8rg + 2w (low halves) and 8rg + 2w + 1 (high halves), k = 4kg .. 4kg+3
                uint2 lo, hi;
                lo.x = (q0[w] & 0xffffu) | (q1[w] << 16);
                lo.y = (q2[w] & 0xffffu) | (q3[w] << 16);
                hi.x = (q0[w] >> 16) | (q1[w] & 0xffff0000u);
                hi.y = (q2[w] >> 16) | (q3[w] & 0xffff0000u);
                const int r = rg * 8 + 2 * w;
                *reinterpret_cast<uint2*>(lds + lds_chunk<BK>(r, kg >> 1) + (kg & 1) * 4) = lo;
                *reinterpret_cast<uint2*>(lds + lds_chunk<BK>(r + 1, kg >> 1) + (kg & 1) * 4) = hi;
            }
        }
    }
};

template <int R, int BK, int NT, bool TRANS>
using Stage = typename std::conditional<TRANS, TransStage<R, BK, NT>, DirectStage<R, BK, NT>>::type;

// One workgroup = one BM x BN output tile of one segment; WM x WN waves, each
// owning a (BM/WM) x (BN/WN) sub-tile of 16x16 fragments.  The MFMA is issued
// with the B fragment as its first operand, so each accumulator holds C^T:
// lane l owns C[m = l % 16][n = 4 (l / 16) .. +3], four adjacent columns that
// leave in one store.
template <int BM, int BN, int BK, int WM, int WN, int AL, int BL, int OUT_BF16>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(const GemmTile* __restrict__ tiles, int ntiles,
                                                                const GemmSeg* __restrict__ segs,
                                                                const GemmTuple* __restrict__ tuples,
                                                                const uint16_t* __restrict__ A,
                                                                const uint16_t* __restrict__ B, void* __restrict__ C) {
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    using SA = Stage<BM, BK, NT, AL == JA_A_KM>;
    using SB = Stage<BN, BK, NT, BL == JA_B_KN>;
    extern __shared__ __attribute__((aligned(16))) uint16_t gemm_lds[];
    // [A buffer 0][A buffer 1][B buffer 0][B buffer 1]
    auto As = [&](int b) { return gemm_lds + b * (BM * BK); };
    auto Bs = [&](int b) { return gemm_lds + 2 * BM * BK + b * (BN * BK); };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const GemmTile tl = tiles[xcd_remap(blockIdx.x, ntiles)];
    const GemmSeg sg = segs[tl.seg];
    const int m0 = tl.m0, n0 = tl.n0;

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    SA sa;
    SB sb;
    // stage cursor: tuple t, contracted offset k0 inside it
    int t = sg.t_begin, k0 = 0;
    auto load_stage = [&](int tt, int kk) {
        const GemmTuple tp = tuples[tt];
        const uint16_t* pa = A + tp.a_off + (int64_t)tl.batch * tp.a_bstride;
        const uint16_t* pb = B + tp.b_off + (int64_t)tl.batch * tp.b_bstride;
        sa.load(pa, tp.lda, m0, sg.M, kk, tp.K, tid);
        sb.load(pb, tp.ldb, n0, sg.N, kk, tp.K, tid);
    };
    auto advance = [&]() {
        k0 += BK;
        if (k0 >= tuples[t].K) {
            k0 = 0;
            ++t;
        }
    };
    if (t >= sg.t_end) return;  // a segment always has tuples; guard anyway
    load_stage(t, k0);
    sa.store(As(0), tid);
    sb.store(Bs(0), tid);
    advance();
    __syncthreads();
    int buf = 0;
    const int arow = wm * WTM + (lane & 15), brow = wn * WTN + (lane & 15);
    const int kc = lane >> 4;  // this lane's 8-k chunk inside a 32-k step
    while (true) {
        const bool more = t < sg.t_end;
        if (more) load_stage(t, k0);
        const uint16_t* as = As(buf);
        const uint16_t* bs = Bs(buf);
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            bf16x8_t af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t*>(as + lds_chunk<BK>(arow + i * 16, ks / 8 + kc));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(bs + lds_chunk<BK>(brow + j * 16, ks / 8 + kc));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
        }
        if (!more) break;
        sa.store(As(buf ^ 1), tid);
        sb.store(Bs(buf ^ 1), tid);
        advance();
        __syncthreads();
        buf ^= 1;
    }

    // epilogue: lane owns C[row][col .. col+3] of every fragment
    const int64_t cbase = sg.c_off + (int64_t)tl.batch * sg.c_bstride;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = m0 + wm * WTM + i * 16 + (lane & 15);
        if (row >= sg.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WTN + j * 16 + 4 * kc;
            const int64_t off = cbase + (int64_t)row * sg.ldc + col;
            const f32x4_t a = acc[i][j];
            if (col + 4 <= sg.N && (off & 3) == 0) {
                if (OUT_BF16)
                    *reinterpret_cast<uint2*>((uint16_t*)C + off) = make_uint2(pack_bf16x2(a[0], a[1]),
                                                                               pack_bf16x2(a[2], a[3]));
                else
                    *reinterpret_cast<float4*>((float*)C + off) = make_float4(a[0], a[1], a[2], a[3]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (col + r < sg.N) {
                        if (OUT_BF16)
                            ((uint16_t*)C)[off + r] = (uint16_t)f32_to_bf16(a[r]);
                        else
                            ((float*)C)[off + r] = a[r];
                    }
            }
        }
    }
}

// ---------------------------------------------------------------- fp32 path
// Plain LDS-tiled fp32 FMA kernel (64x64 tile, 4x4 outputs per thread) for
// fp32 relations.  Same segment / tuple walk as the bf16 kernel.
template <int AL, int BL>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmTile* __restrict__ tiles, int ntiles,
                                                       const GemmSeg* __restrict__ segs,
                                                       const GemmTuple* __restrict__ tuples,
                                                       const float* __restrict__ A, const float* __restrict__ B,
                                                       float* __restrict__ C) {
    constexpr int T = 64, TK = 16;
    __shared__ float As[TK][T + 1], Bs[TK][T + 1];
    const GemmTile tl = tiles[xcd_remap(blockIdx.x, ntiles)];
    const GemmSeg sg = segs[tl.seg];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int t = sg.t_begin; t < sg.t_end; ++t) {
        const GemmTuple tp = tuples[t];
        const float* pa = A + tp.a_off + (int64_t)tl.batch * tp.a_bstride;
        const float* pb = B + tp.b_off + (int64_t)tl.batch * tp.b_bstride;
        for (int k0 = 0; k0 < tp.K; k0 += TK) {
            for (int e = threadIdx.x; e < T * TK; e += 256) {
                int r = e / TK, k = e % TK;  // A element (m0 + r, k0 + k)
                int gm = tl.m0 + r, gk = k0 + k;
                float va = 0.f;
                if (gm < sg.M && gk < tp.K) va = AL == JA_A_MK ? pa[(int64_t)gm * tp.lda + gk] : pa[(int64_t)gk * tp.lda + gm];
                As[k][r] = va;
                int c = e % T, kb = e / T;  // B element (k0 + kb, n0 + c)
                int gn = tl.n0 + c, gkb = k0 + kb;
                float vb = 0.f;
                if (gn < sg.N && gkb < tp.K)
                    vb = BL == JA_B_KN ? pb[(int64_t)gkb * tp.ldb + gn] : pb[(int64_t)gn * tp.ldb + gkb];
                Bs[kb][c] = vb;
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TK; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(As[k][ty * 4 + i], Bs[k][tx * 4 + j], acc[i][j]);
            __syncthreads();
        }
    }
    const int64_t cbase = sg.c_off + (int64_t)tl.batch * sg.c_bstride;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int row = tl.m0 + ty * 4 + i, col = tl.n0 + tx * 4 + j;
            if (row < sg.M && col < sg.N) C[cbase + (int64_t)row * sg.ldc + col] = acc[i][j];
        }
}

// ---------------------------------------------------------------- dispatch
template <int AL, int BL, int OB>
static void launch_bf16(const GemmTile* tiles, int ntiles, const GemmSeg* segs, const GemmTuple* tuples, const void* A,
                        const void* B, void* C, hipStream_t s) {
    constexpr int BM = GEMM_BF16_TM, BN = GEMM_BF16_TN, BK = GEMM_BF16_TK, WM = 2, WN = 4;
    constexpr unsigned lds = 2u * (BM + BN) * BK * sizeof(uint16_t);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, WM, WN, AL, BL, OB>), dim3(ntiles), dim3(WM * WN * 64), lds, s,
                       tiles, ntiles, segs, tuples, (const uint16_t*)A, (const uint16_t*)B, C);
}

template <int AL, int BL>
static void launch_bf16_out(int out_bf16, const GemmTile* tiles, int ntiles, const GemmSeg* segs,
                            const GemmTuple* tuples, const void* A, const void* B, void* C, hipStream_t s) {
    if (out_bf16)
        launch_bf16<AL, BL, 1>(tiles, ntiles, segs, tuples, A, B, C, s);
    else
        launch_bf16<AL, BL, 0>(tiles, ntiles, segs, tuples, A, B, C, s);
}

hipError_t launch_gemm(const void* table, int64_t tiles_off, int32_t ntiles, int64_t segs_off, int64_t tuples_off,
                       const void* A, const void* B, void* C, int32_t in_dtype, int32_t out_dtype, int32_t a_layout,
                       int32_t b_layout, hipStream_t s) {
    const uint8_t* t = (const uint8_t*)table;
    const GemmTile* tiles = (const GemmTile*)(t + tiles_off);
    const GemmSeg* segs = (const GemmSeg*)(t + segs_off);
    const GemmTuple* tuples = (const GemmTuple*)(t + tuples_off);
    if (in_dtype == JA_BF16) {
        const int ob = out_dtype == JA_BF16;
        if (a_layout == JA_A_MK && b_layout == JA_B_KN)
            launch_bf16_out<JA_A_MK, JA_B_KN>(ob, tiles, ntiles, segs, tuples, A, B, C, s);
        else if (a_layout == JA_A_MK && b_layout == JA_B_NK)
            launch_bf16_out<JA_A_MK, JA_B_NK>(ob, tiles, ntiles, segs, tuples, A, B, C, s);
        else if (a_layout == JA_A_KM && b_layout == JA_B_KN)
            launch_bf16_out<JA_A_KM, JA_B_KN>(ob, tiles, ntiles, segs, tuples, A, B, C, s);
        else
            launch_bf16_out<JA_A_KM, JA_B_NK>(ob, tiles, ntiles, segs, tuples, A, B, C, s);
    } else {
#define JA_F32_CASE(al, bl)                                                                                       \
    hipLaunchKernelGGL((gemm_f32_kernel<al, bl>), dim3(ntiles), dim3(256), 0, s, tiles, ntiles, segs, tuples,     \
                       (const float*)A, (const float*)B, (float*)C)
        if (a_layout == JA_A_MK && b_layout == JA_B_KN)
            JA_F32_CASE(JA_A_MK, JA_B_KN);
        else if (a_layout == JA_A_MK && b_layout == JA_B_NK)
            JA_F32_CASE(JA_A_MK, JA_B_NK);
        else if (a_layout == JA_A_KM && b_layout == JA_B_KN)
            JA_F32_CASE(JA_A_KM, JA_B_KN);
        else
            JA_F32_CASE(JA_A_KM, JA_B_NK);
#undef JA_F32_CASE
    }
    return hipGetLastError();
}

}  // namespace ja
