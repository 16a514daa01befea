// join.hip -- the join step on the GPU: enumerate the interval grid, keep the
// cells the join predicate allows, write them in group-by-key order and cut
// equal keys into CSR aggregation segments ("Every Kernel Is a Join",
// section 3.2 step 1, and section 3.3 for the causal and packed-sequence
// predicates).  The split positions are read from device memory, so a
// decomposition whose cuts come from device data needs no host round trip.
//
// Walking the grid in iteration order (ja_join.h) makes the sorted tuple
// list a stream compaction of the grid: a kept cell's record position is the
// number of kept cells before it.  Segments are the non-empty groups, so the
// segment offsets are a second compaction, over groups.  Each compaction is
// count per workgroup -> one-workgroup scan of the counts -> write, so the
// result is deterministic and needs no atomics on global memory.  Inside a
// workgroup, positions come from wavefront ballots, and a row of consecutive
// cells is spread over consecutive lanes and each wavefront stages its kept
// records in LDS, so that records are written as contiguous runs.  A grid of
// at most 8,192 cells, 8,191 groups and 2,048 split points runs as one
// workgroup in one launch (dj_small_kernel); larger grids take six:
//
//   cell_count    per chunk of DJ_CHUNK cells: kept cells
//   scan(cells)   checks the split points (status into counts[2]); chunk
//                 bases; total tuples into gpre[ngroup]
//   cell_write    records of kept cells; gpre[g] = tuples before group g
//   group_count   per chunk of groups: non-empty groups
//   scan(groups)  chunk bases; n_tuples, n_segs, seg_off[n_segs]
//   group_write   seg_off[k] = first tuple of the k-th non-empty group
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../ja_join.h"

namespace ja {

__device__ __forceinline__ uint32_t dj_div(uint32_t n, const DJDiv& f) {
    if (f.d == 1) return n;
    const uint32_t t = __umulhi(n, f.m);
    return (t + ((n - t) >> 1)) >> f.s;
}

// Interval index of letter l in grid cell c.
__device__ __forceinline__ uint32_t dj_index(uint32_t c, const DJoinArgs& a, int l) {
    const uint32_t q = dj_div(c, a.stride[l]);
    return q - dj_div(q, a.count[l]) * a.count[l].d;
}

// The join predicate of the operator, PRED bit 0: causal attention drops a
// cell whose key interval starts at or after the end of its query interval;
// PRED bit 1: packed sequences drop a cell whose query and key intervals
// (unions of whole sequences) do not overlap, i.e. share no sequence.
template <int PRED>
__device__ __forceinline__ bool dj_keep(uint32_t c, const DJoinArgs& a, const int64_t* __restrict__ sp) {
    bool keep = true;
    if (PRED & 1) {
        const int64_t t_lo = sp[a.sp_off[a.it] + dj_index(c, a, a.it)];
        const int64_t s_hi = sp[a.sp_off[a.is] + dj_index(c, a, a.is) + 1];
        keep = t_lo < s_hi;
    }
    if (PRED & 2) {
        const uint32_t si = dj_index(c, a, a.ps), ti = dj_index(c, a, a.pt);
        const int64_t s_lo = sp[a.sp_off[a.ps] + si], s_hi = sp[a.sp_off[a.ps] + si + 1];
        const int64_t t_lo = sp[a.sp_off[a.pt] + ti], t_hi = sp[a.sp_off[a.pt] + ti + 1];
        keep = keep && (s_lo > t_lo ? s_lo : t_lo) < (s_hi < t_hi ? s_hi : t_hi);
    }
    return keep;
}

// Exclusive prefix sum over a workgroup of NT threads (NT a multiple of 64);
// `total` receives the workgroup's sum.  lds holds NT / 64 words.
template <int NT>
__device__ __forceinline__ uint32_t dj_block_scan(uint32_t v, uint32_t* lds, uint32_t& total) {
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
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        const uint32_t t = lds[i];
        off += i < w ? t : 0u;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return off + x - v;
}

// Status bits of the split points (DJ_BAD_*), computed by one workgroup of
// NT threads (one split point per thread and pass) and returned to all of
// them.
template <int NT>
__device__ int32_t dj_validate_block(const DJoinArgs& a, const int64_t* __restrict__ sp,
                                     const int64_t* __restrict__ ends, int32_t* st) {
    if (threadIdx.x == 0) *st = 0;
    __syncthreads();
    int32_t bad = 0;
    for (uint32_t e = threadIdx.x; e < a.nsplit; e += NT) {
        int l = 0;
        int32_t n = a.cnt[0];
        int64_t ext = a.ext[0];
        for (int m = 1; m < a.nl; ++m)
            if ((uint32_t)a.sp_off[m] <= e) {
                l = m;
                n = a.cnt[m];
                ext = a.ext[m];
            }
        const int32_t j = (int32_t)e - a.sp_off[l];
        const int64_t x = sp[e];
        if (j == 0 ? x != 0 : x <= sp[e - 1]) bad |= DJ_BAD_SPLITS;
        if (j == n && x != ext) bad |= DJ_BAD_SPLITS;
        if (l == a.ps && a.nends < 0 && x != sp[a.sp_off[a.pt] + j]) bad |= DJ_BAD_SEQS;
        if ((l == a.ps || l == a.pt) && a.nends >= 0 && j > 0 && j < n) {
            // an interior cut must be a sequence end (binary search)
            int32_t lo = 0, hi = a.nends;
            while (lo < hi) {
                const int32_t mid = (lo + hi) >> 1;
                if (ends[mid] < x) lo = mid + 1;
                else hi = mid;
            }
            if (lo == a.nends || ends[lo] != x) bad |= DJ_BAD_PACKED;
        }
    }
    if (bad) atomicOr(st, bad);
    __syncthreads();
    return *st;
}

// A chunk of NT * DJ_CPT cells (or groups) is DJ_CPT rows of NT: item j of
// thread t is chunk0 + j * NT + t, so within a row consecutive lanes hold
// consecutive items and their outputs land side by side.  bal[j] is the
// wavefront's ballot of row j's kept items.  The predicates of 8 rows are
// evaluated before their ballots, so those rows' split-point loads are in
// flight together.
template <int NT, int PRED>
__device__ __forceinline__ void dj_cell_rows(const DJoinArgs& a, const int64_t* __restrict__ sp, uint32_t c0,
                                             bool ok, uint64_t* bal) {
    constexpr int BATCH = 8;
#pragma unroll
    for (int j0 = 0; j0 < DJ_CPT; j0 += BATCH) {
        bool k[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const uint32_t c = c0 + (j0 + j) * NT + threadIdx.x;
            const uint32_t cc = c < a.ncell ? c : 0u;  // past the grid: evaluate cell 0, drop the answer
            k[j] = dj_keep<PRED>(cc, a, sp) && ok && c < a.ncell;
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) bal[j0 + j] = __ballot(k[j]);
    }
}

template <int NT>
__device__ __forceinline__ void dj_group_rows(const uint32_t* gpre, uint32_t ngroup, uint32_t g0, uint64_t* bal) {
    bool k[DJ_CPT];
#pragma unroll
    for (int j = 0; j < DJ_CPT; ++j) {
        const uint32_t g = g0 + j * NT + threadIdx.x;
        const uint32_t gg = g < ngroup ? g : 0u;
        k[j] = gpre[gg + 1] > gpre[gg] && g < ngroup;
    }
#pragma unroll
    for (int j = 0; j < DJ_CPT; ++j) bal[j] = __ballot(k[j]);
}

__device__ __forceinline__ uint32_t dj_popc_all(const uint64_t* bal) {
    uint32_t n = 0;
#pragma unroll
    for (int j = 0; j < DJ_CPT; ++j) n += __popcll(bal[j]);
    return n;
}

// Output positions of one chunk, starting at `base`: the ballot counts of
// every (row, wavefront) go through LDS once; item (j, thread) lands at base +
// all kept items of earlier rows + those of earlier wavefronts in row j + the
// kept lanes below it.  Calls emit(item, pos, kept, valid, wpos, wcount) on
// every lane for every row (valid: item < limit; wpos, wcount: first position
// and number of the wavefront's kept items in the row, the same on every
// lane) and returns base + the chunk's kept count.
template <int NT, typename F>
__device__ __forceinline__ uint32_t dj_emit(const uint64_t* bal, uint32_t (*rows)[NT / 64], uint32_t c0,
                                            uint32_t limit, uint32_t base, F emit) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    __syncthreads();  // earlier readers of rows are done
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < DJ_CPT; ++j) rows[j][w] = __popcll(bal[j]);
    }
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1;
    uint32_t run = base;
#pragma unroll
    for (int j = 0; j < DJ_CPT; ++j) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int v = 0; v < NT / 64; ++v) {
            const uint32_t t = rows[j][v];
            before += v < w ? t : 0u;
            all += t;
        }
        const uint32_t c = c0 + j * NT + threadIdx.x;
        emit(c, run + before + (uint32_t)__popcll(bal[j] & below), (bal[j] >> lane) & 1, c < limit, run + before,
             (uint32_t)__popcll(bal[j]));
        run += all;
    }
    return run;
}

// LDS writes of this wavefront are complete and visible to its other lanes
// (the LDS serves one wavefront's requests in order; the wait and the
// barrier keep the compiler from moving accesses across).
__device__ __forceinline__ void dj_wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// The records of one wavefront's kept cells of a row, written side by side:
// each kept lane puts its record at its rank in the wavefront's LDS stage
// (64 * DJ_MAX_LETTERS words), then all lanes copy the wcount * nl words
// to rec + wpos * nl with consecutive lanes on consecutive words.
__device__ __forceinline__ void dj_stage_records(const DJoinArgs& a, int32_t* __restrict__ rec, int32_t* stage,
                                                 uint32_t c, uint32_t rank, bool kept, uint32_t wpos,
                                                 uint32_t wcount) {
    if (wcount == 0) return;
    if (kept)
        for (int l = 0; l < a.nl; ++l) stage[rank * a.nl + l] = (int32_t)dj_index(c, a, l);
    dj_wave_lds_sync();
    const uint32_t n = wcount * (uint32_t)a.nl;
    int32_t* dst = rec + (int64_t)wpos * a.nl;
    for (uint32_t f = threadIdx.x & 63; f < n; f += 64) dst[f] = stage[f];
    dj_wave_lds_sync();
}

// ---------------------------------------------------------------- small grids
// Up to DJ_SMALL_CELLS cells, DJ_SMALL_GROUPS groups and DJ_SMALL_SPLITS split
// points: the whole join in one workgroup of DJ_SMALL_THREADS and one launch,
// with the split points, the group prefix and the record stages in LDS.
constexpr int DJ_SMALL_THREADS = 512;
constexpr uint32_t DJ_SMALL_CELLS = 8192;
constexpr uint32_t DJ_SMALL_GROUPS = 8191;
constexpr uint32_t DJ_SMALL_SPLITS = 2048;

template <int PRED>
__global__ __launch_bounds__(DJ_SMALL_THREADS) void dj_small_kernel(DJoinArgs a, const int64_t* __restrict__ sp,
                                                                    const int64_t* __restrict__ ends,
                                                                    int32_t* __restrict__ rec,
                                                                    int64_t* __restrict__ seg_off,
                                                                    int64_t* __restrict__ counts) {
    constexpr int NT = DJ_SMALL_THREADS;
    __shared__ int64_t lsp[DJ_SMALL_SPLITS];
    __shared__ uint32_t gp[DJ_SMALL_GROUPS + 1];
    __shared__ uint32_t rows[DJ_CPT][NT / 64];
    __shared__ int32_t stage[NT / 64][64 * DJ_MAX_LETTERS];
    __shared__ int32_t st;
    for (uint32_t e = threadIdx.x; e < a.nsplit; e += NT) lsp[e] = sp[e];
    __syncthreads();
    const int32_t status = dj_validate_block<NT>(a, lsp, ends, &st);
    int32_t* wstage = stage[threadIdx.x >> 6];
    uint64_t bal[DJ_CPT];
    uint32_t ntup = 0;
    for (uint32_t c0 = 0; c0 < a.ncell; c0 += NT * DJ_CPT) {
        dj_cell_rows<NT, PRED>(a, lsp, c0, status == 0, bal);
        ntup = dj_emit<NT>(bal, rows, c0, a.ncell, ntup,
                           [&](uint32_t c, uint32_t pos, bool kept, bool valid, uint32_t wpos, uint32_t wcount) {
                               const uint32_t g = dj_div(c, a.inner);
                               if (valid && c == g * a.inner.d) gp[g] = pos;  // tuples before the group's first cell
                               dj_stage_records(a, rec, wstage, c, pos - wpos, kept, wpos, wcount);
                           });
    }
    if (threadIdx.x == 0) gp[a.ngroup] = ntup;
    __syncthreads();
    uint32_t nseg = 0;
    for (uint32_t g0 = 0; g0 < a.ngroup; g0 += NT * DJ_CPT) {
        dj_group_rows<NT>(gp, a.ngroup, g0, bal);
        nseg = dj_emit<NT>(bal, rows, g0, a.ngroup, nseg,
                           [&](uint32_t g, uint32_t k, bool nonempty, bool, uint32_t, uint32_t) {
                               if (nonempty) seg_off[k] = gp[g];
                           });
    }
    if (threadIdx.x == 0) {
        seg_off[nseg] = ntup;
        counts[0] = ntup;
        counts[1] = nseg;
        counts[2] = status;
    }
}

// ---------------------------------------------------------------- large grids
// Kept cells per chunk, whatever the split points' status (the scan that
// follows validates them and discards these counts when they are bad).  A
// cell's predicate reads only split points inside the array, valid or not.
template <int PRED>
__global__ __launch_bounds__(DJ_THREADS) void dj_cell_count_kernel(DJoinArgs a, const int64_t* __restrict__ sp,
                                                                   uint32_t* __restrict__ chunk_cnt) {
    __shared__ uint32_t lds[DJ_THREADS / 64];
    uint64_t bal[DJ_CPT];
    dj_cell_rows<DJ_THREADS, PRED>(a, sp, blockIdx.x * DJ_CHUNK, true, bal);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = dj_popc_all(bal);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int v = 0; v < DJ_THREADS / 64; ++v) t += lds[v];
        chunk_cnt[blockIdx.x] = t;
    }
}

// One workgroup: exclusive scan of n chunk counts into base[].  Cells pass
// (GROUPS = false): first the split points are validated (status into
// counts[2]; with a bad status every count is taken as zero, so no tuple is
// written), then the total number of tuples goes to gpre[ngroup].  Groups
// pass: the total number of segments closes seg_off, and counts[0..1] get the
// tuple and segment totals.
template <bool GROUPS>
__global__ __launch_bounds__(DJ_SCAN_THREADS) void dj_scan_kernel(DJoinArgs a, const int64_t* __restrict__ sp,
                                                                  const int64_t* __restrict__ ends,
                                                                  const uint32_t* __restrict__ cnt,
                                                                  uint32_t* __restrict__ base, uint32_t n,
                                                                  uint32_t* __restrict__ gpre,
                                                                  int64_t* __restrict__ seg_off,
                                                                  int64_t* __restrict__ counts) {
    __shared__ uint32_t lds[DJ_SCAN_THREADS / 64];
    __shared__ int32_t st;
    const uint32_t ngroup = a.ngroup;
    bool ok = true;
    if (!GROUPS) {
        const int32_t status = dj_validate_block<DJ_SCAN_THREADS>(a, sp, ends, &st);
        if (threadIdx.x == 0) counts[2] = status;
        ok = status == 0;
    }
    const uint32_t per = (n + DJ_SCAN_THREADS - 1) / DJ_SCAN_THREADS;
    const uint32_t i0 = threadIdx.x * per;
    uint32_t s = 0;
    for (uint32_t i = i0; i < i0 + per && i < n; ++i) s += ok ? cnt[i] : 0u;
    uint32_t tot;
    uint32_t run = dj_block_scan<DJ_SCAN_THREADS>(s, lds, tot);
    for (uint32_t i = i0; i < i0 + per && i < n; ++i) {
        base[i] = run;
        run += ok ? cnt[i] : 0u;
    }
    if (threadIdx.x == 0) {
        if (!GROUPS) {
            gpre[ngroup] = tot;
        } else {
            const uint32_t tuples = gpre[ngroup];
            seg_off[tot] = tuples;
            counts[0] = tuples;
            counts[1] = tot;
        }
    }
}

template <int PRED>
__global__ __launch_bounds__(DJ_THREADS) void dj_cell_write_kernel(DJoinArgs a, const int64_t* __restrict__ sp,
                                                                   const int64_t* __restrict__ counts,
                                                                   const uint32_t* __restrict__ chunk_base,
                                                                   int32_t* __restrict__ rec,
                                                                   uint32_t* __restrict__ gpre) {
    __shared__ uint32_t rows[DJ_CPT][DJ_THREADS / 64];
    __shared__ int32_t stage[DJ_THREADS / 64][64 * DJ_MAX_LETTERS];
    int32_t* wstage = stage[threadIdx.x >> 6];
    uint64_t bal[DJ_CPT];
    const uint32_t c0 = blockIdx.x * DJ_CHUNK;
    dj_cell_rows<DJ_THREADS, PRED>(a, sp, c0, counts[2] == 0, bal);
    dj_emit<DJ_THREADS>(bal, rows, c0, a.ncell, chunk_base[blockIdx.x],
                        [&](uint32_t c, uint32_t pos, bool kept, bool valid, uint32_t wpos, uint32_t wcount) {
                            const uint32_t g = dj_div(c, a.inner);
                            if (valid && c == g * a.inner.d) gpre[g] = pos;  // tuples before the group's first cell
                            dj_stage_records(a, rec, wstage, c, pos - wpos, kept, wpos, wcount);
                        });
}

__global__ __launch_bounds__(DJ_THREADS) void dj_group_count_kernel(uint32_t ngroup, const uint32_t* __restrict__ gpre,
                                                                    uint32_t* __restrict__ chunk_cnt) {
    __shared__ uint32_t lds[DJ_THREADS / 64];
    uint64_t bal[DJ_CPT];
    dj_group_rows<DJ_THREADS>(gpre, ngroup, blockIdx.x * DJ_CHUNK, bal);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = dj_popc_all(bal);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int v = 0; v < DJ_THREADS / 64; ++v) t += lds[v];
        chunk_cnt[blockIdx.x] = t;
    }
}

__global__ __launch_bounds__(DJ_THREADS) void dj_group_write_kernel(uint32_t ngroup, const uint32_t* __restrict__ gpre,
                                                                    const uint32_t* __restrict__ chunk_base,
                                                                    int64_t* __restrict__ seg_off) {
    __shared__ uint32_t rows[DJ_CPT][DJ_THREADS / 64];
    uint64_t bal[DJ_CPT];
    const uint32_t g0 = blockIdx.x * DJ_CHUNK;
    dj_group_rows<DJ_THREADS>(gpre, ngroup, g0, bal);
    dj_emit<DJ_THREADS>(bal, rows, g0, ngroup, chunk_base[blockIdx.x],
                        [&](uint32_t g, uint32_t k, bool nonempty, bool, uint32_t, uint32_t) {
                            if (nonempty) seg_off[k] = gpre[g];
                        });
}

template <int PRED>
static void launch_djoin_t(const DJoinArgs& a, const int64_t* splits, const int64_t* ends, int32_t* rec,
                           int64_t* seg_off, int64_t* counts, uint32_t* ccnt, uint32_t* cbase, uint32_t* gcnt,
                           uint32_t* gbase, uint32_t* gpre, hipStream_t stream) {
    if (a.ncell <= DJ_SMALL_CELLS && a.ngroup <= DJ_SMALL_GROUPS && a.nsplit <= DJ_SMALL_SPLITS) {
        hipLaunchKernelGGL(dj_small_kernel<PRED>, dim3(1), dim3(DJ_SMALL_THREADS), 0, stream, a, splits, ends, rec,
                           seg_off, counts);
        return;
    }
    hipLaunchKernelGGL(dj_cell_count_kernel<PRED>, dim3(a.nchunk), dim3(DJ_THREADS), 0, stream, a, splits, ccnt);
    hipLaunchKernelGGL(dj_scan_kernel<false>, dim3(1), dim3(DJ_SCAN_THREADS), 0, stream, a, splits, ends,
                       (const uint32_t*)ccnt, cbase, a.nchunk, gpre, seg_off, counts);
    hipLaunchKernelGGL(dj_cell_write_kernel<PRED>, dim3(a.nchunk), dim3(DJ_THREADS), 0, stream, a, splits,
                       (const int64_t*)counts, (const uint32_t*)cbase, rec, gpre);
    hipLaunchKernelGGL(dj_group_count_kernel, dim3(a.ngchunk), dim3(DJ_THREADS), 0, stream, a.ngroup,
                       (const uint32_t*)gpre, gcnt);
    hipLaunchKernelGGL(dj_scan_kernel<true>, dim3(1), dim3(DJ_SCAN_THREADS), 0, stream, a, splits, ends,
                       (const uint32_t*)gcnt, gbase, a.ngchunk, gpre, seg_off, counts);
    hipLaunchKernelGGL(dj_group_write_kernel, dim3(a.ngchunk), dim3(DJ_THREADS), 0, stream, a.ngroup,
                       (const uint32_t*)gpre, (const uint32_t*)gbase, seg_off);
}

// Small grids: one launch.  Otherwise six: the workspace holds four uint32
// arrays (cell chunk counts and bases, group chunk counts and bases) and gpre
// (ngroup + 1 entries), at the offsets the host computed.
hipError_t launch_djoin(const DJoinArgs& a, const int64_t* splits, const int64_t* ends, int32_t* rec,
                        int64_t* seg_off, int64_t* counts, uint32_t* ccnt, uint32_t* cbase, uint32_t* gcnt,
                        uint32_t* gbase, uint32_t* gpre, hipStream_t stream) {
    const int pred = (a.is >= 0 ? 1 : 0) | (a.ps >= 0 ? 2 : 0);
    auto go = pred == 0 ? launch_djoin_t<0> : pred == 1 ? launch_djoin_t<1> : pred == 2 ? launch_djoin_t<2>
                                                                                       : launch_djoin_t<3>;
    go(a, splits, ends, rec, seg_off, counts, ccnt, cbase, gcnt, gbase, gpre, stream);
    return hipGetLastError();
}

}  // namespace ja
