// stream_ops.hip -- the HBM-bound kernels of libja: repartition copies,
// the 1:1 key joins (SwiGLU, residual add), RMSNorm, and the standalone
// segmented aggregation.
//
// All of them stream: coalesced 16-byte loads issued back to back before any
// use, arithmetic in fp32, one pass over the data.  Loads of data read once
// carry the non-temporal hint; stores do not, since the next operator reads
// them and finds them in the caches (non-temporal stores measured no faster
// alone and slowed the consumers down inside the block).
#include "dev_common.h"

namespace ja {

// ---------------------------------------------------------------- repartition
// One workgroup per copy task (at most REP_CHUNK elements).  Each thread
// issues all of its loads before its first store (lanes past the task's end
// copy the task's first vector, which the planner has checked to be in
// bounds, onto itself), so a pass keeps REP_MAXV loads in flight per
// thread.  A task whose outer loops are trivial is a plain rows x vectors
// copy and needs no index division; a power-of-two row length needs none at
// all.
constexpr int REP_THREADS = 256;
constexpr int REP_MAXV = 8;  // vectors per thread per pass

template <bool FLAT, bool POW2>
__device__ __forceinline__ void rep_vec_pass(const RepTask& t, const uint8_t* __restrict__ src,
                                             uint8_t* __restrict__ dst, int32_t esize, uint32_t vpe, uint32_t vpr,
                                             uint32_t lg, uint32_t total, uint32_t base) {
    const uint32_t n1 = t.n[1], n2 = t.n[2];
    uint4 v[REP_MAXV];
    int64_t doff[REP_MAXV];
#pragma unroll
    for (int j = 0; j < REP_MAXV; ++j) {
        const uint32_t i = base + threadIdx.x + j * REP_THREADS;
        const uint32_t ii = i < total ? i : 0u;
        const uint32_t r = POW2 ? ii >> lg : ii / vpr;
        const uint32_t c = ii - r * vpr;
        int64_t so, dof;
        if (FLAT) {
            so = t.src_off + (int64_t)r * t.ss[2] + (int64_t)c * vpe;
            dof = t.dst_off + (int64_t)r * t.ds[2] + (int64_t)c * vpe;
        } else {
            const uint32_t i2 = r % n2, r1 = r / n2;
            const uint32_t i1 = r1 % n1, i0 = r1 / n1;
            so = t.src_off + i0 * t.ss[0] + i1 * t.ss[1] + i2 * t.ss[2] + (int64_t)c * vpe;
            dof = t.dst_off + i0 * t.ds[0] + i1 * t.ds[1] + i2 * t.ds[2] + (int64_t)c * vpe;
        }
        // issued as asm so the compiler cannot sink each load to its store
        // and wait for it there; one explicit wait covers them all
        asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(v[j]) : "v"(src + so * esize) : "memory");
        doff[j] = dof;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // stores are unconditional (a lane past the end rewrites the task's first
    // vector with the bytes lane 0 writes there)
#pragma unroll
    for (int j = 0; j < REP_MAXV; ++j) *reinterpret_cast<uint4*>(dst + doff[j] * esize) = v[j];
}

__global__ __launch_bounds__(REP_THREADS) void repart_kernel(const RepTask* __restrict__ tasks,
                                                             const uint8_t* __restrict__ src,
                                                             uint8_t* __restrict__ dst, int32_t esize) {
    const RepTask t = tasks[blockIdx.x];
    const uint32_t n1 = t.n[1], n2 = t.n[2], n3 = t.n[3];
    const uint32_t rows = (uint32_t)t.n[0] * n1 * n2;
    if (t.flags & REP_VEC) {
        const uint32_t vpe = 16 / esize;  // elements per vector
        const uint32_t vpr = n3 / vpe;    // vectors per row
        const uint32_t total = rows * vpr;
        const bool flat = t.n[0] == 1 && n1 == 1;
        const bool pow2 = (vpr & (vpr - 1)) == 0;
        const uint32_t lg = __builtin_ctz(vpr);
        for (uint32_t base = 0; base < total; base += REP_THREADS * REP_MAXV) {
            if (flat && pow2)
                rep_vec_pass<true, true>(t, src, dst, esize, vpe, vpr, lg, total, base);
            else if (flat)
                rep_vec_pass<true, false>(t, src, dst, esize, vpe, vpr, lg, total, base);
            else
                rep_vec_pass<false, false>(t, src, dst, esize, vpe, vpr, lg, total, base);
        }
    } else {
        const uint32_t total = rows * n3;
        for (uint32_t i = threadIdx.x; i < total; i += REP_THREADS) {
            uint32_t r = i / n3, c = i - r * n3;
            uint32_t i2 = r % n2, r1 = r / n2;
            uint32_t i1 = r1 % n1, i0 = r1 / n1;
            int64_t so = t.src_off + i0 * t.ss[0] + i1 * t.ss[1] + i2 * t.ss[2] + (int64_t)c * t.ss[3];
            int64_t dof = t.dst_off + i0 * t.ds[0] + i1 * t.ds[1] + i2 * t.ds[2] + (int64_t)c * t.ds[3];
            if (esize == 2)
                *reinterpret_cast<uint16_t*>(dst + dof * 2) = *reinterpret_cast<const uint16_t*>(src + so * 2);
            else
                *reinterpret_cast<uint32_t*>(dst + dof * 4) = *reinterpret_cast<const uint32_t*>(src + so * 4);
        }
    }
}

hipError_t launch_repart(const void* table, int64_t ntasks, const void* src, void* dst, int32_t esize,
                         int32_t vec_ok, hipStream_t stream) {
    (void)vec_ok;
    const RepTask* tasks = (const RepTask*)table;
    for (int64_t first = 0; first < ntasks; first += 0x7fffffff) {
        int64_t n = ntasks - first < 0x7fffffff ? ntasks - first : 0x7fffffff;
        hipLaunchKernelGGL(repart_kernel, dim3((unsigned)n), dim3(REP_THREADS), 0, stream, tasks + first,
                           (const uint8_t*)src, (uint8_t*)dst, esize);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- 1:1 joins
// The three relations are identically blocked, so the join is a zip of the
// flat buffers.  Each thread handles ZIP_V vectors of 8 16-bit elements
// (bf16, or IEEE half with F16).
constexpr int ZIP_THREADS = 256;
constexpr int ZIP_V = 4;

template <int OP, bool F16>  // OP 0: swiglu, 1: add
__global__ __launch_bounds__(ZIP_THREADS) void zip_kernel(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                          uint4* __restrict__ c, int64_t nvec) {
    const int64_t base = (int64_t)blockIdx.x * ZIP_THREADS * ZIP_V + threadIdx.x;
    uint4 va[ZIP_V], vb[ZIP_V];
#pragma unroll
    for (int j = 0; j < ZIP_V; ++j) {
        int64_t i = base + j * ZIP_THREADS;
        if (i < nvec) {
            va[j] = ld_nt(a + i);
            vb[j] = ld_nt(b + i);
        }
    }
#pragma unroll
    for (int j = 0; j < ZIP_V; ++j) {
        int64_t i = base + j * ZIP_THREADS;
        if (i >= nvec) continue;
        uint32_t x[4] = {va[j].x, va[j].y, va[j].z, va[j].w};
        uint32_t y[4] = {vb[j].x, vb[j].y, vb[j].z, vb[j].w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float x0 = h16lo_to_f32<F16>(x[k]), x1 = h16hi_to_f32<F16>(x[k]);
            float y0 = h16lo_to_f32<F16>(y[k]), y1 = h16hi_to_f32<F16>(y[k]);
            float r0, r1;
            if (OP == 0) {
                r0 = silu_mul(x0, y0);
                r1 = silu_mul(x1, y1);
            } else {
                r0 = x0 + y0;
                r1 = x1 + y1;
            }
            o[k] = pack_h16x2<F16>(r0, r1);
        }
        c[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

template <int OP, bool F16>
__global__ void zip_tail_kernel(const uint16_t* a, const uint16_t* b, uint16_t* c, int64_t first, int64_t n) {
    int64_t i = first + threadIdx.x;
    if (i >= n) return;
    float x = h16_to_f32<F16>(a[i]), y = h16_to_f32<F16>(b[i]);
    float r = OP == 0 ? silu_mul(x, y) : x + y;
    c[i] = (uint16_t)f32_to_h16<F16>(r);
}

template <int OP, bool F16>
static hipError_t launch_zip(const void* a, const void* b, void* c, int64_t n, hipStream_t stream) {
    int64_t nvec = n / 8;
    if (nvec > 0) {
        int64_t per = (int64_t)ZIP_THREADS * ZIP_V;
        int64_t grid = (nvec + per - 1) / per;
        hipLaunchKernelGGL((zip_kernel<OP, F16>), dim3((unsigned)grid), dim3(ZIP_THREADS), 0, stream, (const uint4*)a,
                           (const uint4*)b, (uint4*)c, nvec);
    }
    if (n % 8)
        hipLaunchKernelGGL((zip_tail_kernel<OP, F16>), dim3(1), dim3(8), 0, stream, (const uint16_t*)a, (const uint16_t*)b,
                           (uint16_t*)c, nvec * 8, n);
    return hipGetLastError();
}

hipError_t launch_swiglu(const void* g, const void* u, void* h, int64_t n, int32_t f16, hipStream_t stream) {
    return f16 ? launch_zip<0, true>(g, u, h, n, stream) : launch_zip<0, false>(g, u, h, n, stream);
}
hipError_t launch_add(const void* a, const void* b, void* c, int64_t n, int32_t f16, hipStream_t stream) {
    return f16 ? launch_zip<1, true>(a, b, c, n, stream) : launch_zip<1, false>(a, b, c, n, stream);
}

// ---------------------------------------------------------------- RMSNorm
// One wavefront per row.  Pass 1 walks the row's pieces in every column block
// (the join of the row's tuples), stages them in LDS and SUM-aggregates the
// squares; pass 2 joins each piece 1:1 with the row statistic and the gain.
constexpr int NORM_WAVES = 4;

template <bool F16>
__global__ __launch_bounds__(NORM_WAVES * 64) void rmsnorm_kernel(const int64_t* __restrict__ rsplit, int32_t nrb,
                                                                  const NormBlock* __restrict__ blocks, int32_t ndb,
                                                                  int64_t rows, int32_t D,
                                                                  const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ gain,
                                                                  uint16_t* __restrict__ y, float eps, int32_t vec) {
    extern __shared__ uint16_t lds_row[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * NORM_WAVES + wave;
    if (r >= rows) return;
    uint16_t* row = lds_row + (size_t)wave * D;
    int rb = 0;
    while (rb + 1 < nrb && rsplit[rb + 1] <= r) ++rb;
    const int64_t rr = r - rsplit[rb];
    const NormBlock* bl = blocks + (int64_t)rb * ndb;
    float ss = 0.f;
    for (int db = 0; db < ndb; ++db) {
        const NormBlock b = bl[db];
        const uint16_t* src = x + b.off + rr * b.width;
        if (vec) {
            for (int e = lane * 8; e < b.width; e += 512) {
                uint4 v = ld_nt(src + e);
                *reinterpret_cast<uint4*>(row + b.d_lo + e) = v;
                uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float a0 = h16lo_to_f32<F16>(w[k]), a1 = h16hi_to_f32<F16>(w[k]);
                    ss += a0 * a0 + a1 * a1;
                }
            }
        } else {
            for (int e = lane; e < b.width; e += 64) {
                uint16_t h = src[e];
                row[b.d_lo + e] = h;
                float a = h16_to_f32<F16>(h);
                ss += a * a;
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float inv = rsqrtf(ss / (float)D + eps);
    for (int db = 0; db < ndb; ++db) {
        const NormBlock b = bl[db];
        uint16_t* dstp = y + b.off + rr * b.width;
        if (vec) {
            for (int e = lane * 8; e < b.width; e += 512) {
                uint4 v = *reinterpret_cast<const uint4*>(row + b.d_lo + e);
                uint4 g = *reinterpret_cast<const uint4*>(gain + b.d_lo + e);
                uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w}, o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    o[k] = pack_h16x2<F16>(h16lo_to_f32<F16>(w[k]) * inv * h16lo_to_f32<F16>(gw[k]),
                                       h16hi_to_f32<F16>(w[k]) * inv * h16hi_to_f32<F16>(gw[k]));
                *reinterpret_cast<uint4*>(dstp + e) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        } else {
            for (int e = lane; e < b.width; e += 64)
                dstp[e] = (uint16_t)f32_to_h16<F16>(h16_to_f32<F16>(row[b.d_lo + e]) * inv * h16_to_f32<F16>(gain[b.d_lo + e]));
        }
    }
}

// The same join with the whole row held in registers: one wavefront per
// row, lane l holding the 16-byte vectors at columns 512 k + 8 l.  Used when
// every column block is W wide with W a multiple of 512, so each vector lies
// in one block and its block index k * 512 / W is uniform; all NV loads of a
// row are in flight together, then one wavefront reduction, then the stores.
template <int NV, bool F16>
__global__ __launch_bounds__(NORM_WAVES * 64) void rmsnorm_rows_kernel(const int64_t* __restrict__ rsplit,
                                                                       int32_t nrb,
                                                                       const NormBlock* __restrict__ blocks,
                                                                       int32_t ndb, int64_t rows, int32_t W,
                                                                       const uint16_t* __restrict__ x,
                                                                       const uint16_t* __restrict__ gain,
                                                                       uint16_t* __restrict__ y, float eps) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * NORM_WAVES + wave;
    if (r >= rows) return;
    int rb = 0;
    while (rb + 1 < nrb && rsplit[rb + 1] <= r) ++rb;
    const int64_t rr = r - rsplit[rb];
    const NormBlock* bl = blocks + (int64_t)rb * ndb;
    uint4 v[NV];
    int64_t off[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int db = (k * 512) / W;
        off[k] = bl[db].off + rr * W + (k * 512 - db * W) + lane * 8;
        v[k] = ld_nt(x + off[k]);
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a0 = h16lo_to_f32<F16>(w[q]), a1 = h16hi_to_f32<F16>(w[q]);
            ss += a0 * a0 + a1 * a1;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float inv = rsqrtf(ss / (float)(NV * 512) + eps);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const uint4 g = *reinterpret_cast<const uint4*>(gain + k * 512 + lane * 8);
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w}, gw[4] = {g.x, g.y, g.z, g.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = pack_h16x2<F16>(h16lo_to_f32<F16>(w[q]) * inv * h16lo_to_f32<F16>(gw[q]),
                               h16hi_to_f32<F16>(w[q]) * inv * h16hi_to_f32<F16>(gw[q]));
        *reinterpret_cast<uint4*>(y + off[k]) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// vec: 0 scalar pieces, 1 16-byte pieces (both staged through LDS), 2 rows
// held in registers (D a multiple of 512 up to 8192, every block W wide with
// W a multiple of 512; the planner checks this)
template <bool F16>
static hipError_t launch_rmsnorm_t(const void* table, int64_t rsplit_off, int32_t nrb, int64_t blocks_off,
                                   int32_t ndb, int64_t rows, int32_t D, int32_t W, const void* x, const void* gain,
                                   void* y, float eps, int32_t vec, hipStream_t stream) {
    const uint8_t* t = (const uint8_t*)table;
    int64_t grid = (rows + NORM_WAVES - 1) / NORM_WAVES;
    if (vec == 2) {
        const int nv = D / 512;
#define JA_ROWS_CASE(N)                                                                                           \
    case N:                                                                                                       \
        hipLaunchKernelGGL((rmsnorm_rows_kernel<N, F16>), dim3((unsigned)grid), dim3(NORM_WAVES * 64), 0, stream,        \
                           (const int64_t*)(t + rsplit_off), nrb, (const NormBlock*)(t + blocks_off), ndb, rows, W, \
                           (const uint16_t*)x, (const uint16_t*)gain, (uint16_t*)y, eps);                        \
        break;
        switch (nv) {
            JA_ROWS_CASE(1)
            JA_ROWS_CASE(2)
            JA_ROWS_CASE(3)
            JA_ROWS_CASE(4)
            JA_ROWS_CASE(5)
            JA_ROWS_CASE(6)
            JA_ROWS_CASE(7)
            JA_ROWS_CASE(8)
            JA_ROWS_CASE(10)
            JA_ROWS_CASE(12)
            JA_ROWS_CASE(14)
            JA_ROWS_CASE(16)
            default: return hipErrorInvalidValue;
        }
#undef JA_ROWS_CASE
        return hipGetLastError();
    }
    hipLaunchKernelGGL(rmsnorm_kernel<F16>, dim3((unsigned)grid), dim3(NORM_WAVES * 64),
                       (unsigned)((size_t)NORM_WAVES * D * 2), stream, (const int64_t*)(t + rsplit_off), nrb,
                       (const NormBlock*)(t + blocks_off), ndb, rows, D, (const uint16_t*)x, (const uint16_t*)gain,
                       (uint16_t*)y, eps, vec);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const void* table, int64_t rsplit_off, int32_t nrb, int64_t blocks_off, int32_t ndb,
                          int64_t rows, int32_t D, int32_t W, const void* x, const void* gain, void* y, float eps,
                          int32_t vec, int32_t f16, hipStream_t stream) {
    return f16 ? launch_rmsnorm_t<true>(table, rsplit_off, nrb, blocks_off, ndb, rows, D, W, x, gain, y, eps, vec, stream)
               : launch_rmsnorm_t<false>(table, rsplit_off, nrb, blocks_off, ndb, rows, D, W, x, gain, y, eps, vec,
                                         stream);
}

// ---------------------------------------------------------------- aggregation
// One workgroup per (segment, chunk of AGG_CHUNK output elements); each
// thread folds its elements over the segment's tuples in ascending order and
// writes them once.  No atomics: every output element has one owner.  A
// thread owns PER consecutive elements: where every partial block of the
// segment and the output block start on a 16-byte boundary they move as
// 16-byte vectors (two loads per tuple, one store of 8 halves or two of 4
// floats), otherwise, and for the last elements of a block, one by one.
constexpr int AGG_THREADS = 256;

template <int OUT>  // 0: f32, 1: bf16, 2: IEEE half
__global__ __launch_bounds__(AGG_THREADS) void agg_kernel(const AggTile* __restrict__ tiles,
                                                          const AggSeg* __restrict__ segs,
                                                          const int64_t* __restrict__ poff,
                                                          const float* __restrict__ part, void* __restrict__ out,
                                                          int32_t op) {
    const AggTile tl = tiles[blockIdx.x];
    const AggSeg sg = segs[tl.seg];
    constexpr int PER = AGG_CHUNK / AGG_THREADS;
    static_assert(PER == 8, "a thread owns two 16-byte vectors of partials");
    const bool mx = op == JA_AGG_MAX;
    const int e0 = tl.e0 + threadIdx.x * PER;
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = mx ? -INFINITY : 0.f;
    bool vec = (sg.out_off & (OUT == 0 ? 3 : 7)) == 0;
    for (int t = sg.t_begin; t < sg.t_end; ++t) vec = vec && (poff[t] & 3) == 0;
    if (vec && e0 + PER <= sg.nelem) {
#pragma unroll 4
        for (int t = sg.t_begin; t < sg.t_end; ++t) {
            const float* p = part + poff[t] + e0;
            const float4 a = ld_nt_f4(p), b = ld_nt_f4(p + 4);
            const float v[PER] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < PER; ++j) acc[j] = mx ? fmaxf(acc[j], v[j]) : acc[j] + v[j];
        }
        if (OUT == 0) {
            float4* o = reinterpret_cast<float4*>((float*)out + sg.out_off + e0);
            o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        } else {
            uint32_t w[PER / 2];
#pragma unroll
            for (int j = 0; j < PER / 2; ++j)
                w[j] = OUT == 1 ? pack_bf16x2(acc[2 * j], acc[2 * j + 1]) : pack_f16x2(acc[2 * j], acc[2 * j + 1]);
            *reinterpret_cast<uint4*>((uint16_t*)out + sg.out_off + e0) = make_uint4(w[0], w[1], w[2], w[3]);
        }
        return;
    }
    for (int t = sg.t_begin; t < sg.t_end; ++t) {
        const float* p = part + poff[t];
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (e0 + j < sg.nelem) acc[j] = mx ? fmaxf(acc[j], p[e0 + j]) : acc[j] + p[e0 + j];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = e0 + j;
        if (e < sg.nelem) {
            if (OUT == 1)
                ((uint16_t*)out)[sg.out_off + e] = (uint16_t)f32_to_bf16(acc[j]);
            else if (OUT == 2)
                ((uint16_t*)out)[sg.out_off + e] = (uint16_t)f32_to_f16(acc[j]);
            else
                ((float*)out)[sg.out_off + e] = acc[j];
        }
    }
}

hipError_t launch_agg(const void* table, int64_t tiles_off, int32_t ntiles, int64_t segs_off, int64_t poff_off,
                      const float* partials, void* out, int32_t out_dtype, int32_t op, hipStream_t stream) {
    const uint8_t* t = (const uint8_t*)table;
    if (out_dtype == JA_BF16)
        hipLaunchKernelGGL(agg_kernel<1>, dim3(ntiles), dim3(AGG_THREADS), 0, stream, (const AggTile*)(t + tiles_off),
                           (const AggSeg*)(t + segs_off), (const int64_t*)(t + poff_off), partials, out, op);
    else if (out_dtype == JA_F16)
        hipLaunchKernelGGL(agg_kernel<2>, dim3(ntiles), dim3(AGG_THREADS), 0, stream, (const AggTile*)(t + tiles_off),
                           (const AggSeg*)(t + segs_off), (const int64_t*)(t + poff_off), partials, out, op);
    else
        hipLaunchKernelGGL(agg_kernel<0>, dim3(ntiles), dim3(AGG_THREADS), 0, stream, (const AggTile*)(t + tiles_off),
                           (const AggSeg*)(t + segs_off), (const int64_t*)(t + poff_off), partials, out, op);
    return hipGetLastError();
}

// ---------------------------------------------------------------- softmax aggregation
// The aggregation of attention's per-tuple triples (the operator need not be
// addition, "Every Kernel Is a Join", paperpeel full text, section 5.2): each
// query row's triples (m, l, acc) from the tuples of its segment, in tuple
// order, folded with m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m),
// acc = acc1 e^(m1-m) + acc2 e^(m2-m) from the identity (-inf, 0, 0); the
// row's output is acc / l.  A workgroup owns SMAX_ROWS rows of one segment,
// 32 lanes per row, 4 of the 128 values per lane; the partial row of tuple t
// starts at poff[t] + row ATTN_PROW (f32 [m, l, -, -, acc[128]]), the output
// row at out_off + row 128.  AggSeg.nelem counts the segment's rows.
template <bool F16>
__global__ __launch_bounds__(256) void smax_agg_kernel(const AggTile* __restrict__ tiles,
                                                       const AggSeg* __restrict__ segs,
                                                       const int64_t* __restrict__ poff,
                                                       const float* __restrict__ part, uint16_t* __restrict__ out) {
    static_assert(256 / 32 == SMAX_ROWS, "32 lanes per row");
    const AggTile tl = tiles[blockIdx.x];
    const AggSeg sg = segs[tl.seg];
    const int row = tl.e0 + (int)(threadIdx.x >> 5), c = (threadIdx.x & 31) * 4;
    if (row >= sg.nelem) return;
    float m = -INFINITY, l = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int t = sg.t_begin; t < sg.t_end; ++t) {
        const float* pr = part + poff[t] + (int64_t)row * ATTN_PROW;
        const float2 ml = *reinterpret_cast<const float2*>(pr);
        const float4 a = ld_nt_f4(pr + 4 + c);
        const float mn = fmaxf(m, ml.x);
        if (mn == -INFINITY) continue;  // identity folded with identity
        const float s1 = __expf(m - mn), s2 = __expf(ml.x - mn);  // exp(-inf) = 0
        l = l * s1 + ml.y * s2;
        acc.x = acc.x * s1 + a.x * s2;
        acc.y = acc.y * s1 + a.y * s2;
        acc.z = acc.z * s1 + a.z * s2;
        acc.w = acc.w * s1 + a.w * s2;
        m = mn;
    }
    const float inv = 1.0f / l;
    *reinterpret_cast<uint2*>(out + sg.out_off + (int64_t)row * ATTN_D + c) =
        make_uint2(pack_h16x2<F16>(acc.x * inv, acc.y * inv), pack_h16x2<F16>(acc.z * inv, acc.w * inv));
}

hipError_t launch_smax_agg(const void* table, int64_t tiles_off, int32_t ntiles, int64_t segs_off, int64_t poff_off,
                           const float* partials, void* out, int32_t f16, hipStream_t stream) {
    const uint8_t* t = (const uint8_t*)table;
    auto kernel = f16 ? smax_agg_kernel<true> : smax_agg_kernel<false>;
    hipLaunchKernelGGL(kernel, dim3(ntiles), dim3(256), 0, stream, (const AggTile*)(t + tiles_off),
                       (const AggSeg*)(t + segs_off), (const int64_t*)(t + poff_off), partials, (uint16_t*)out);
    return hipGetLastError();
}

}  // namespace ja
