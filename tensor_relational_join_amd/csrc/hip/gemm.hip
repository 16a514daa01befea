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
// bf16 path: v_mfma_f32_16x16x32_bf16 on CDNA4.  Operand tiles are staged
// through LDS as [row][k] (k contiguous) so that every MFMA operand fragment
// is one 16-byte LDS read; an operand whose k is not contiguous in memory is
// transposed in registers on its way to LDS (4x8 sub-blocks).  LDS is double
// buffered; the global loads of stage i+1 are in flight while stage i
// multiplies.
#include "dev_common.h"

namespace ja {

// ---------------------------------------------------------------- bf16 MFMA
template <int R, int BK, int NT, bool TRANS>
struct Stager {
    static_assert(BK % 8 == 0 && R % 8 == 0, "tile shape");
    static constexpr int LDK = BK + 8;  // padded LDS row pitch (elements)
    // direct: each thread moves VPT 16-byte vectors of a [R][BK] tile
    static constexpr int VPT = TRANS ? 1 : (R * BK / 8) / NT;
    // transposed: each thread moves SPT sub-blocks of 4 k-rows x 8 columns
    static constexpr int SPT = TRANS ? ((BK / 4) * (R / 8)) / NT : 1;
    static_assert(TRANS || (R * BK / 8) % NT == 0, "direct staging must divide evenly");
    static_assert(!TRANS || ((BK / 4) * (R / 8)) % NT == 0, "transposed staging must divide evenly");
    uint4 v[TRANS ? SPT * 4 : VPT];

    // Load the tile rows [r0, r0+R) x k [k0, k0+BK) of an operand whose element
    // (r, k) is at p[r*ld + k] (direct) or p[k*ld + r] (transposed).
    __device__ __forceinline__ void load(const uint16_t* __restrict__ p, int64_t ld, int r0, int rext, int k0,
                                         int kext, int tid) {
        if (!TRANS) {
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                int vi = tid + j * NT;
                int r = vi / (BK / 8), kv = vi % (BK / 8);
                int gr = r0 + r, gk = k0 + kv * 8;
                if (gr < rext && gk < kext)
                    v[j] = *reinterpret_cast<const uint4*>(p + (int64_t)gr * ld + gk);
                else
                    v[j] = make_uint4(0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                int si = tid + j * NT;
                int kg = si / (R / 8), rg = si % (R / 8);
                int gr = r0 + rg * 8;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int gk = k0 + kg * 4 + i;
                    if (gr < rext && gk < kext)
                        v[j * 4 + i] = *reinterpret_cast<const uint4*>(p + (int64_t)gk * ld + gr);
                    else
                        v[j * 4 + i] = make_uint4(0, 0, 0, 0);
                }
            }
        }
    }

    __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
        if (!TRANS) {
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                int vi = tid + j * NT;
                int r = vi / (BK / 8), kv = vi % (BK / 8);
                *reinterpret_cast<uint4*>(lds + r * LDK + kv * 8) = v[j];
            }
        } else {
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                int si = tid + j * NT;
                int kg = si / (R / 8), rg = si % (R / 8);
                const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&v[j * 4 + 0]);
                const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&v[j * 4 + 1]);
                const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&v[j * 4 + 2]);
                const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&v[j * 4 + 3]);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    // columns 2w (low halves) and 2w+1 (high halves): 4 consecutive k each
                    uint2 lo, hi;
                    lo.x = (r0[w] & 0xffffu) | (r1[w] << 16);
                    lo.y = (r2[w] & 0xffffu) | (r3[w] << 16);
                    hi.x = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
                    hi.y = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
                    *reinterpret_cast<uint2*>(lds + (rg * 8 + 2 * w) * LDK + kg * 4) = lo;
                    *reinterpret_cast<uint2*>(lds + (rg * 8 + 2 * w + 1) * LDK + kg * 4) = hi;
                }
            }
        }
    }
};

template <int BM, int BN, int BK, int WM, int WN, int AL, int BL, int OUT_BF16>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(const GemmTile* __restrict__ tiles, int ntiles,
                                                                const GemmSeg* __restrict__ segs,
                                                                const GemmTuple* __restrict__ tuples,
                                                                const uint16_t* __restrict__ A,
                                                                const uint16_t* __restrict__ B, void* __restrict__ C) {
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int LDK = BK + 8;
    using SA = Stager<BM, BK, NT, AL == JA_A_KM>;
    using SB = Stager<BN, BK, NT, BL == JA_B_KN>;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDK];

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
    sa.store(As[0], tid);
    sb.store(Bs[0], tid);
    advance();
    __syncthreads();
    int buf = 0;
    const int arow = wm * WTM + (lane & 15), brow = wn * WTN + (lane & 15);
    const int kq = (lane >> 4) * 8;
    while (true) {
        const bool more = t < sg.t_end;
        if (more) load_stage(t, k0);
        const uint16_t* as = As[buf];
        const uint16_t* bs = Bs[buf];
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            bf16x8_t af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t*>(as + (arow + i * 16) * LDK + ks + kq);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(bs + (brow + j * 16) * LDK + ks + kq);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (!more) break;
        sa.store(As[buf ^ 1], tid);
        sb.store(Bs[buf ^ 1], tid);
        advance();
        __syncthreads();
        buf ^= 1;
    }

    // epilogue: lane holds C[4*(lane/16) + r][lane%16] of every 16x16 fragment
    const int64_t cbase = sg.c_off + (int64_t)tl.batch * sg.c_bstride;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WTN + j * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * WTM + i * 16 + (lane >> 4) * 4 + r;
                if (row < sg.M && col < sg.N) {
                    if (OUT_BF16)
                        ((uint16_t*)C)[cbase + (int64_t)row * sg.ldc + col] = (uint16_t)f32_to_bf16(acc[i][j][r]);
                    else
                        ((float*)C)[cbase + (int64_t)row * sg.ldc + col] = acc[i][j][r];
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
    constexpr int BM = GEMM_BF16_TM, BN = GEMM_BF16_TN, BK = 64, WM = 2, WN = 2;
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, WM, WN, AL, BL, OB>), dim3(ntiles), dim3(WM * WN * 64), 0, s,
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
