// dattn.hip -- the attention kernel's tables built on the GPU from the
// device-side join's records ("Every Kernel Is a Join", section 3.2 step 1
// on the device; section 3.3 packed sequences whose ends are the cuts).
//
//   zero    clears the histogram and cursors
//   seg     per segment (one output block: a query batch-head block and one
//           sequence): its AttnSeg and its 128-row tile count; its batch-heads
//           are added to a histogram indexed by the segment's tiles per
//           batch-head (one atomic per segment); the int32 sequence ends the
//           kernel masks with
//   scan    one workgroup: tiles at position q = batch-heads of segments with
//           more than q tiles (a suffix sum of that histogram), then the first
//           slot of every position, later positions (tiles that see more keys)
//           first, and the tile count
//   tiles   per segment: its tiles (batch-head, first row), each in a slot of
//           its position taken with an atomic cursor, so the longest tiles
//           are launched first as the host planner orders them (the order
//           inside a position is free: every tile writes its own rows)
//   tuples  per tuple: its AttnTuple (key block rows inside the key batch-head
//           block)
// Every kernel reads the join's counts from device memory and leaves slots
// past them untouched; the attention kernel is then launched over the upper
// bound of tiles and its workgroups past the count return at once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../ja_dattn.h"
#include "../ja_tables.h"

namespace ja {

__device__ __forceinline__ uint32_t da_block(const int32_t* r, const int32_t* let, const int32_t* cnt, int n) {
    uint32_t b = 0;
    for (int m = 0; m < n; ++m) b = b * (uint32_t)cnt[m] + (uint32_t)r[let[m]];
    return b;
}

__global__ __launch_bounds__(DA_THREADS) void da_zero_kernel(uint32_t n, uint32_t* __restrict__ hist,
                                                             uint32_t* __restrict__ cursor) {
    const uint32_t i = blockIdx.x * DA_THREADS + threadIdx.x;
    if (i < n) {
        hist[i] = 0;
        cursor[i] = 0;
    }
}

__global__ __launch_bounds__(DA_THREADS) void da_seg_kernel(DAttnArgs a, const int64_t* __restrict__ sp,
                                                            const int32_t* __restrict__ rec,
                                                            const int64_t* __restrict__ seg_off,
                                                            const int64_t* __restrict__ counts,
                                                            const int64_t* __restrict__ qbase,
                                                            const int32_t* __restrict__ qn,
                                                            const int32_t* __restrict__ kn, AttnSeg* __restrict__ segs,
                                                            uint32_t* __restrict__ tcnt, uint32_t* __restrict__ hist,
                                                            int32_t* __restrict__ seq32) {
    const uint32_t k = blockIdx.x * DA_THREADS + threadIdx.x;
    if (k < (uint32_t)a.nseq) seq32[k] = (int32_t)sp[a.sp_s + k + 1];
    if (k >= a.max_segs) return;
    if ((int64_t)k >= counts[1]) {
        tcnt[k] = 0;
        return;
    }
    const int64_t t0 = seg_off[k], t1 = seg_off[k + 1];
    const int32_t* r = rec + t0 * a.nl;
    const uint32_t qi = da_block(r, a.qlet, a.qcnt, a.nq), ki = da_block(r, a.klet, a.kcnt, a.nk);
    const int64_t s_lo = sp[a.sp_s + r[a.ls]], s_hi = sp[a.sp_s + r[a.ls] + 1];
    AttnSeg g;
    g.q_off = qbase[qi] + s_lo * a.D;
    g.o_off = g.q_off;
    g.q_bstride = a.S * a.D;
    g.S = (int32_t)(s_hi - s_lo);
    g.s_lo = (int32_t)s_lo;
    g.t_begin = (int32_t)t0;
    g.t_end = (int32_t)t1;
    g.rep = qn[qi] / kn[ki];
    g.q_hin = 1;  // head-major blocks: every batch-head letter before the position letter
    g.kv_hin = 1;
    g.pad = 0;
    segs[k] = g;
    const int32_t ntq = (g.S + ATTN_TQ - 1) / ATTN_TQ;
    tcnt[k] = (uint32_t)qn[qi] * (uint32_t)ntq;
    atomicAdd(&hist[ntq - 1], (uint32_t)qn[qi]);  // segments with ntq tiles per batch-head
}

// Exclusive prefix sum over the one workgroup of DA_SCAN_THREADS threads.
__device__ __forceinline__ uint32_t da_block_scan(uint32_t v, uint32_t* lds, uint32_t& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) lds[w] = x;
    __syncthreads();
    uint32_t off = 0, tot = 0;
    for (int i = 0; i < DA_SCAN_THREADS / 64; ++i) {
        const uint32_t t = lds[i];
        off += i < w ? t : 0u;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return off + x - v;
}

// One workgroup.  hist[j] holds the batch-heads of segments with j + 1 tiles
// per batch-head; position q then holds pos[q] = sum of hist[j] over j >= q
// (a suffix sum), written over hist; base[q] = tiles at positions after q (a
// suffix sum of pos excluding q); the total goes to *ntiles.  Each thread
// owns a run of `per` consecutive entries counted from the end and touches
// no other thread's entries.
__global__ __launch_bounds__(DA_SCAN_THREADS) void da_scan_kernel(uint32_t* __restrict__ hist,
                                                                  uint32_t* __restrict__ base, uint32_t n,
                                                                  int32_t* __restrict__ ntiles) {
    __shared__ uint32_t lds[DA_SCAN_THREADS / 64];
    const uint32_t per = (n + DA_SCAN_THREADS - 1) / DA_SCAN_THREADS;
    const uint32_t i0 = threadIdx.x * per;  // i counts from the end: entry n - 1 - i
    uint32_t s = 0;
    for (uint32_t i = i0; i < i0 + per && i < n; ++i) s += hist[n - 1 - i];
    uint32_t tot;
    const uint32_t run0 = da_block_scan(s, lds, tot);  // hist of the entries after this thread's run
    uint32_t run = run0, psum = 0;
    for (uint32_t i = i0; i < i0 + per && i < n; ++i) {
        run += hist[n - 1 - i];
        psum += run;
    }
    uint32_t ptot;
    uint32_t prun = da_block_scan(psum, lds, ptot);
    run = run0;
    for (uint32_t i = i0; i < i0 + per && i < n; ++i) {
        run += hist[n - 1 - i];
        hist[n - 1 - i] = run;
        base[n - 1 - i] = prun;
        prun += run;
    }
    if (threadIdx.x == 0) *ntiles = (int32_t)ptot;
}

__global__ __launch_bounds__(DA_THREADS) void da_tile_kernel(const int64_t* __restrict__ counts,
                                                             const AttnSeg* __restrict__ segs,
                                                             const uint32_t* __restrict__ tcnt,
                                                             const uint32_t* __restrict__ base,
                                                             uint32_t* __restrict__ cursor,
                                                             AttnTile* __restrict__ tiles) {
    const uint32_t k = blockIdx.x;
    if ((int64_t)k >= counts[1]) return;
    const uint32_t ntq = (uint32_t)((segs[k].S + ATTN_TQ - 1) / ATTN_TQ);
    const uint32_t n = tcnt[k];
    for (uint32_t j = threadIdx.x; j < n; j += DA_THREADS) {
        const uint32_t q = j % ntq;
        AttnTile t;
        t.seg = (int32_t)k;
        t.bh = (int32_t)(j / ntq);
        t.s0 = (int32_t)q * ATTN_TQ;
        t.pad = 0;
        tiles[base[q] + atomicAdd(&cursor[q], 1u)] = t;
    }
}

__global__ __launch_bounds__(DA_THREADS) void da_tuple_kernel(DAttnArgs a, const int64_t* __restrict__ sp,
                                                              const int32_t* __restrict__ rec,
                                                              const int64_t* __restrict__ counts,
                                                              const int64_t* __restrict__ kbase,
                                                              AttnTuple* __restrict__ tuples) {
    const uint32_t i = blockIdx.x * DA_THREADS + threadIdx.x;
    if (i >= a.max_tuples || (int64_t)i >= counts[0]) return;
    const int32_t* r = rec + (int64_t)i * a.nl;
    const uint32_t ki = da_block(r, a.klet, a.kcnt, a.nk);
    const int64_t t_lo = sp[a.sp_t + r[a.lt]], t_hi = sp[a.sp_t + r[a.lt] + 1];
    AttnTuple t;
    t.k_off = kbase[ki] + t_lo * a.D;
    t.v_off = t.k_off;
    t.kv_bstride = a.S * a.D;
    t.T = (int32_t)(t_hi - t_lo);
    t.t_lo = (int32_t)t_lo;
    tuples[i] = t;
}

hipError_t launch_dattn_tables(const DAttnArgs& a, const int64_t* splits, const int32_t* rec, const int64_t* seg_off,
                               const int64_t* counts, const int64_t* qbase, const int32_t* qn, const int64_t* kbase,
                               const int32_t* kn, AttnSeg* segs, AttnTuple* tuples, AttnTile* tiles,
                               uint32_t* tcnt, uint32_t* hist, uint32_t* base, uint32_t* cursor, int32_t* ntiles,
                               int32_t* seq32, hipStream_t stream) {
    const uint32_t nseg_blocks = (a.max_segs > (uint32_t)a.nseq ? a.max_segs : (uint32_t)a.nseq);
    hipLaunchKernelGGL(da_zero_kernel, dim3((a.nbucket + DA_THREADS - 1) / DA_THREADS), dim3(DA_THREADS), 0, stream,
                       a.nbucket, hist, cursor);
    hipLaunchKernelGGL(da_seg_kernel, dim3((nseg_blocks + DA_THREADS - 1) / DA_THREADS), dim3(DA_THREADS), 0, stream,
                       a, splits, rec, seg_off, counts, qbase, qn, kn, segs, tcnt, hist, seq32);
    hipLaunchKernelGGL(da_scan_kernel, dim3(1), dim3(DA_SCAN_THREADS), 0, stream, hist, base, a.nbucket, ntiles);
    hipLaunchKernelGGL(da_tile_kernel, dim3(a.max_segs), dim3(DA_THREADS), 0, stream, counts, (const AttnSeg*)segs,
                       (const uint32_t*)tcnt, (const uint32_t*)base, cursor, tiles);
    hipLaunchKernelGGL(da_tuple_kernel, dim3((a.max_tuples + DA_THREADS - 1) / DA_THREADS), dim3(DA_THREADS), 0,
                       stream, a, splits, rec, counts, kbase, tuples);
    return hipGetLastError();
}

}  // namespace ja
