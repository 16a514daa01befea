// attention.hip -- causal attention as a join-agg.
//
// Each tuple joins a query block with one key block and its value block on
// the head dimension; the per-tuple result is the triple (row max m, row sum
// of exponentials l, exponential-weighted sum of values acc), and tuples of
// one query block are aggregated with the associative operator
//   m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m), acc = acc1 e^(m1-m) + acc2 e^(m2-m)
// ("Every Kernel Is a Join", paperpeel full text: attention modelled as a
// join followed by an aggregation, section 1; the aggregation operator need
// not be addition, section 5.2).  Fully masked (query block, key block) pairs
// never reach the kernel: the join drops them.

#include "dev_common.h"

namespace ja {

constexpr int AT_KT = 64;         // keys per step
constexpr int AT_THREADS = 256;   // 4 wavefronts x 32 queries
constexpr int AT_STAGE = AT_KT * ATTN_D * 2;  // elements per stage: K [64][128] bf16 + V^T [128][64] fp16

typedef int32_t at_i32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));

// LDS layouts (element offsets), chosen against bank-conflict counts measured
// on gfx950 so that every MFMA fragment read takes the minimum 4 LDS cycles:
// K tile [key][d] bf16, 16-byte chunk c of row `key` at c ^ kswz(key);
// V^T tile [d][key'] fp16 (key' = key with the middle quads of every 16 keys
// swapped, see below), chunk c of row d at c ^ vswz(d).  A V^T row is 128
// bytes, so rows of one parity share one half of the 64 banks.  An MFMA read
// covers 32 consecutive rows, inside which the last term of vswz is constant;
// the 8 rows of one parity that a staging write covers (rows 16 apart) get 8
// distinct swizzles, which spreads them over all chunk positions of their half.
__device__ __forceinline__ int kswz(int r) { return ((r & 1) << 1) ^ ((r >> 1) & 1) ^ (r & 4) ^ ((r >> 1) & 8); }
__device__ __forceinline__ int vswz(int d) {
    return (d & 6) ^ (((d >> 3) & 1) * 3) ^ (((d >> 4) & 1) * 7) ^ (((d >> 5) & 3) << 1);
}
__device__ __forceinline__ int at_koff(int key, int c) { return key * ATTN_D + ((c ^ kswz(key)) << 3); }
__device__ __forceinline__ int at_voff(int d, int c) { return d * AT_KT + ((c ^ vswz(d)) << 3); }

__device__ __forceinline__ at_i32x4_t at_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    at_i32x4_t r;
    r.x = (int32_t)(uint32_t)a;
    r.y = (int32_t)(uint32_t)(a >> 32);
    r.z = (int32_t)bytes;
    r.w = 0x00020000;
    return r;
}
// Buffer load of 16 bytes; offsets past the descriptor's extent read as zero,
// so masked loads need no branch (a branch around a load makes the compiler
// wait for it on the spot).
extern "C" __device__ at_i32x4_t at_buffer_load_x4(at_i32x4_t rsrc, int32_t voffset, int32_t soffset, int32_t aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");

// 16 bytes per lane, global -> LDS (lane l's bytes at lds_byte + 16 l); the
// compiler does not see the LDS write, the step loop waits on vmcnt itself.
__device__ __forceinline__ void at_dma16(at_i32x4_t rsrc, uint32_t lds_byte, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_byte), "v"(voff),
                 "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// One workgroup = 4 wavefronts = 128 query rows of one segment.  The
// segment's tuples are folded in ascending key order, 64 keys per step:
//   S^T[key][query] = K Q^T with v_mfma_f32_32x32x16_bf16 (Q fragments stay
//                     in registers; each lane then holds one query);
//   P = exp2(S * scale log2(e) - m), in fp32, rounded to fp16;
//   O^T[d][query] += V^T P^T with v_mfma_f32_32x32x16_f16.
// K and V are double buffered: while step i multiplies, K of step i + 1
// streams into LDS directly and V of step i + 1 waits in registers, to be
// converted to fp16 and transposed into LDS after the step's MFMAs; one
// barrier per step.  Masks are only evaluated on steps that cross the
// causal diagonal or the end of a key block, and O is rescaled only when
// some query's running maximum moved.
// With tables built on the device, the grid covers an upper bound of tiles and
// the count is read from ntiles_dev (NULL: the grid is exact).
//
// bf16 relations: V is rounded to fp16 for the P V product, whose exponent
// range is far narrower than bf16's.  Ordinary data passes as is; at the end
// of a tile every wave records in `flags` whether its accumulators look out of
// range -- a value that is not finite (V beyond fp16's range) or outputs
// averaging below 2^-12 (V perhaps below fp16's normal range).  A second,
// REDO launch over the same tiles returns at once except on flagged tiles,
// which take the largest exponent among the V rows the tile reads; when that lies outside [-8, 14]
// it computes the tile again with every staged V value multiplied by
// 2^-shift (shift = exponent - 14, so the largest magnitude lands in
// [2^14, 2^15)) and O multiplied by 2^shift on the way out.  Powers of two
// are exact in both formats, so any finite bf16 V is computed in range; data
// of ordinary magnitude pays a sum over the accumulators, a store per wave
// and a REDO launch whose workgroups find no flag and return.
//
// PARTIAL: every segment is one tuple and the tile writes, instead of O, the
// tuple's unnormalised triple per query row -- f32 [m, l, 0, 0, acc[128]]
// (ATTN_PROW floats) at element o_off + (bh S + row) ATTN_PROW, with m in
// units of the scaled scores (P = exp(scale q.k - m)) -- for ja_agg to fold.
template <bool PACKED, bool F16, bool PARTIAL, bool REDO>
__global__ __launch_bounds__(AT_THREADS, 2) void attention_kernel(const AttnTile* __restrict__ tiles,
                                                               const int32_t* __restrict__ ntiles_dev,
                                                               const AttnSeg* __restrict__ segs,
                                                               const AttnTuple* __restrict__ tuples,
                                                               const int32_t* __restrict__ seq_ends, int nseq,
                                                               const uint16_t* __restrict__ Q,
                                                               const uint16_t* __restrict__ K,
                                                               const uint16_t* __restrict__ V, void* __restrict__ O,
                                                               uint32_t* __restrict__ flags, float scale_log2,
                                                               int causal) {
    constexpr int D = ATTN_D;
    const int vt = blockIdx.x;
    if (ntiles_dev && vt >= *ntiles_dev) return;
    if constexpr (REDO) {
        // only the tiles a wave of the first launch flagged
        const uint4 f = *reinterpret_cast<const uint4*>(flags + 4 * vt);
        if ((f.x | f.y | f.z | f.w) == 0) return;
    }
    extern __shared__ __attribute__((aligned(16))) uint16_t at_lds[];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)at_lds;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, lq = lane & 31;
    const AttnTile tl = tiles[vt];
    const AttnSeg sg = segs[tl.seg];
    const int kvbh = tl.bh / sg.rep;  // key-value batch-head (query heads of a group share it)
    // element offsets of this batch-head's first row and the row strides
    // (inner batch-heads sit inside a row: token-major relations)
    const int64_t qbh = (int64_t)(tl.bh / sg.q_hin) * sg.q_bstride + (int64_t)(tl.bh % sg.q_hin) * D;
    const int32_t qrs = sg.q_hin * D, kvrs = sg.kv_hin * D;
    const int kvo = kvbh / sg.kv_hin, kvi = kvbh % sg.kv_hin;
    const int qrow = tl.s0 + wave * 32 + lq;  // query row inside the block
    const int qglob = sg.s_lo + qrow;         // global query index (causal mask)
    const int wave_qmin = sg.s_lo + tl.s0 + wave * 32;
    const int wave_qmax = sg.s_lo + min(tl.s0 + wave * 32 + 31, sg.S - 1);
    const int tile_qmax = sg.s_lo + min(tl.s0 + 127, sg.S - 1);
    // Packed sequences: [seq_lo, seq_hi) of a position's sequence.  A key is
    // visible to a query only inside the query's sequence; the bounds are
    // nondecreasing in the position, so the first and last rows of a
    // wavefront or tile bound its rows'.
    constexpr bool packed = PACKED;
    auto seq_of = [&](int pos, int& lo, int& hi) {
        int a = 0, b = nseq - 1;  // first sequence whose end lies past pos
        while (a < b) {
            const int m = (a + b) >> 1;
            if (seq_ends[m] > pos)
                b = m;
            else
                a = m + 1;
        }
        hi = seq_ends[a];
        lo = a > 0 ? seq_ends[a - 1] : 0;
    };
    int qs_lo = 0, qs_hi = 0x7fffffff, w_lo_min = 0, w_lo_max = 0, w_hi_min = 0x7fffffff, w_hi_max = 0x7fffffff;
    int t_lo_min = 0, t_hi_max = 0x7fffffff;
    if constexpr (PACKED) {
        int dummy;
        seq_of(min(qglob, sg.s_lo + sg.S - 1), qs_lo, qs_hi);
        seq_of(min(wave_qmin, wave_qmax), w_lo_min, w_hi_min);
        seq_of(wave_qmax, w_lo_max, w_hi_max);
        seq_of(sg.s_lo + tl.s0, t_lo_min, dummy);
        seq_of(tile_qmax, dummy, t_hi_max);
    }
    // a tuple's keys [first_key, end_key) that some query row of the tile can see
    auto first_key = [&](const AttnTuple& tp) { return packed ? max(0, (t_lo_min - tp.t_lo) / AT_KT * AT_KT) : 0; };
    auto end_key = [&](const AttnTuple& tp) {
        int e = tp.T;
        if (causal) e = min(e, tile_qmax - tp.t_lo + 1);
        if (packed) e = min(e, t_hi_max - tp.t_lo);
        return e;
    };
    auto tuple_steps = [&](const AttnTuple& tp) {
        const int f = first_key(tp), e = end_key(tp);
        return e > f ? (e - f + AT_KT - 1) / AT_KT : 0;
    };

    // Q^T fragments (B operand): lane holds Q[query lq][d = 16 st + 8 g .. +7]
    bf16x8_t qf[D / 16];
    {
        const at_i32x4_t rq = at_rsrc(Q + sg.q_off + qbh, (uint32_t)((sg.q_bstride - qbh % sg.q_bstride) * 2));
        const int32_t qo = qrow < sg.S ? (qrow * qrs + 8 * g) * 2 : (int32_t)0x80000000;
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
            qf[st] = __builtin_bit_cast(bf16x8_t, at_buffer_load_x4(rq, qo + (qrow < sg.S ? 32 * st : 0), 0, 0));
    }
    f32x16_t oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // steps: (tuple, 64-key offset) pairs some query of the tile can see
    int nsteps = 0;
    for (int t = sg.t_begin; t < sg.t_end; ++t) nsteps += tuple_steps(tuples[t]);
    // a cursor over the steps: enter the first tuple with steps at or after t
    // (without packing every tuple the walk reaches has steps)
    auto enter = [&](int& t, int& k) {
        if constexpr (PACKED) {
            while (t < sg.t_end && tuple_steps(tuples[t]) == 0) ++t;
            k = t < sg.t_end ? first_key(tuples[t]) : 0;
        } else {
            k = 0;
        }
    };
    auto advance = [&](int& t, int& k, const AttnTuple& tp) {  // tp = tuples[t]
        k += AT_KT;
        if (k >= end_key(tp)) {
            ++t;
            enter(t, k);
        }
    };

    // per-lane DMA slots of the K tile (4 per wavefront): key and chunk
    int kkey[4];
    uint32_t koffb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int s = (wave * 4 + j) * 64 + lane;  // 16-byte slot of the 16 KiB tile
        const int key = s >> 4, c = (s & 15) ^ kswz(key);
        kkey[j] = key;
        koffb[j] = (uint32_t)((key * kvrs + c * 8) * 2);
    }
    // V staging: keys 4 kg .. 4 kg + 3 of the step, d = 8 dj .. 8 dj + 7
    const int kg = tid >> 4, dj = tid & 15;
    const int32_t vlane = ((kg * 4) * kvrs + dj * 8) * 2;  // byte offset of this lane's first V row at key 0
    at_i32x4_t vr[4];

    // load cursor
    int lt = sg.t_begin, lkt = 0;
    enter(lt, lkt);
    auto load_step = [&](int buf) {
        const AttnTuple tp = tuples[lt];
        // the buffers' extents end at the block's end (within an outer slab)
        const int64_t kvb = (int64_t)kvo * tp.kv_bstride + (int64_t)kvi * D;
        const uint32_t ext = (uint32_t)((tp.kv_bstride - (int64_t)kvi * D) * 2);
        const uint16_t* kb = K + tp.k_off + kvb;
        const at_i32x4_t rs = at_rsrc(kb, ext);
        const uint32_t st = lds0 + (uint32_t)(buf * AT_STAGE * 2);
        const uint32_t soff = (uint32_t)(lkt * kvrs * 2);
        const at_i32x4_t rv = at_rsrc(V + tp.v_off + kvb, ext);
        if (lkt + AT_KT <= tp.T) {  // every key of the step is in the block
#pragma unroll
            for (int j = 0; j < 4; ++j) at_dma16(rs, st + (wave * 4 + j) * 1024, koffb[j], soff);
#pragma unroll
            for (int i = 0; i < 4; ++i) vr[i] = at_buffer_load_x4(rv, vlane + i * kvrs * 2, (int32_t)soff, 0);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // keys past the block read as zero: 0x80000000 stays past the
                // descriptor's extent with or without the scalar offset added
                const bool ok = lkt + kkey[j] < tp.T;
                at_dma16(rs, st + (wave * 4 + j) * 1024, ok ? koffb[j] : 0x80000000u, soff);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = lkt + kg * 4 + i;
                vr[i] = at_buffer_load_x4(rv, key < tp.T ? (key * kvrs + dj * 8) * 2 : (int32_t)0x80000000, 0, 0);
            }
        }
        advance(lt, lkt, tp);  // to the next visible step
    };
    // V^T[d][key'] <- vr, in fp16 (converted from bf16, moved as is from
    // fp16); key' swaps the middle quads of each 16 keys, matching the order
    // P^T takes from the S^T accumulators.  Word w of a key's 8 d values holds
    // rows 8 dj + 2 w (low half) and 8 dj + 2 w + 1 (high half); each write
    // instruction covers rows of both parities (both halves of the banks), so
    // lanes of odd dj write the odd row first.  Byte selectors (v_perm_b32)
    // pick each lane's first and second row out of the words directly.
    int vshift = 0;  // REDO: V staged as V 2^-vshift, O written as O 2^vshift
    auto cvt = [&](float x) -> _Float16 {
        if constexpr (REDO) x = __builtin_amdgcn_ldexpf(x, -vshift);
        return (_Float16)x;
    };
    const int par = dj & 1;
    // bf16 half of a word -> its float bits (the half in the top two bytes)
    const uint32_t sel_f1 = par ? 0x03020c0cu : 0x01000c0cu, sel_f2 = par ? 0x01000c0cu : 0x03020c0cu;
    // fp16: the same half of two words side by side (first word low)
    const uint32_t sel_h1 = par ? 0x07060302u : 0x05040100u, sel_h2 = par ? 0x05040100u : 0x07060302u;
    auto store_v = [&](int buf) {
        _Float16* vt = reinterpret_cast<_Float16*>(at_lds + buf * AT_STAGE + AT_KT * D);
        const int hgrp = kg >> 2, q = kg & 3;
        const int qpos = q == 1 ? 2 : (q == 2 ? 1 : q);
        const int c = 2 * hgrp + (qpos >> 1), half = qpos & 1;
        const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&vr[0]);
        const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&vr[1]);
        const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&vr[2]);
        const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&vr[3]);  // words of the 4 keys' 8 d values
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint2 first, second;  // the 4 keys' fp16 values of rows 8 dj + 2 w + par and 8 dj + 2 w + (1 - par)
            if constexpr (F16) {
                first = make_uint2(__builtin_amdgcn_perm(r1[w], r0[w], sel_h1), __builtin_amdgcn_perm(r3[w], r2[w], sel_h1));
                second = make_uint2(__builtin_amdgcn_perm(r1[w], r0[w], sel_h2), __builtin_amdgcn_perm(r3[w], r2[w], sel_h2));
            } else {
                typedef _Float16 h4 __attribute__((ext_vector_type(4)));
                auto f = [](uint32_t x, uint32_t sel) { return __uint_as_float(__builtin_amdgcn_perm(x, x, sel)); };
                const h4 a = {cvt(f(r0[w], sel_f1)), cvt(f(r1[w], sel_f1)), cvt(f(r2[w], sel_f1)), cvt(f(r3[w], sel_f1))};
                const h4 b = {cvt(f(r0[w], sel_f2)), cvt(f(r1[w], sel_f2)), cvt(f(r2[w], sel_f2)), cvt(f(r3[w], sel_f2))};
                first = __builtin_bit_cast(uint2, a);
                second = __builtin_bit_cast(uint2, b);
            }
            const int d0 = dj * 8 + 2 * w + par, d1 = dj * 8 + 2 * w + (par ^ 1);
            *reinterpret_cast<uint2*>(vt + at_voff(d0, c) + half * 4) = first;
            *reinterpret_cast<uint2*>(vt + at_voff(d1, c) + half * 4) = second;
        }
    };
    // V^T fragment reads: row 32 dt + lq, chunk (2 kq + g) ^ vswz(32 dt + lq)
    // = (g ^ vswz(lq)) ^ 2 (kq ^ dt), so four per-lane byte offsets (one per
    // kq ^ dt) and an immediate per dt address all sixteen reads of a step
    uint32_t vrd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) vrd[e] = (uint32_t)(lq * AT_KT * 2 + ((((g ^ vswz(lq)) ^ (2 * e)) & 7) << 4));
    auto sync_step = [&]() { asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    if constexpr (REDO) {
        // the largest exponent field among the V rows of the visible keys
        // (a superset of what the steps read), over the workgroup
        uint32_t em = 0;
        for (int t = sg.t_begin; t < sg.t_end; ++t) {
            const AttnTuple tp = tuples[t];
            const int f = first_key(tp), e = end_key(tp);
            if (e <= f) continue;
            const uint16_t* vb = V + tp.v_off + (int64_t)kvo * tp.kv_bstride + (int64_t)kvi * D;
            for (int c = tid; c < (e - f) * (D / 8); c += AT_THREADS) {
                const uint4 v = *reinterpret_cast<const uint4*>(vb + (int64_t)(f + c / (D / 8)) * kvrs + (c % (D / 8)) * 8);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) em = max(em, max((w[k] >> 7) & 0xffu, (w[k] >> 23) & 0xffu));
            }
        }
#pragma unroll
        for (int k = 1; k < 64; k <<= 1) em = max(em, (uint32_t)__shfl_xor((int)em, k));
        __shared__ uint32_t at_emax[AT_THREADS / 64];
        if (lane == 0) at_emax[wave] = em;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        em = at_emax[0];
#pragma unroll
        for (int w = 1; w < AT_THREADS / 64; ++w) em = max(em, at_emax[w]);
        const int e = (int)max(em, 1u) - 127;  // a field of 0 (zeros, subnormals) counts as 2^-126
        vshift = __builtin_amdgcn_readfirstlane((e >= 15 || e < -8) ? e - 14 : 0);
        // flagged by a false alarm: the first launch's result stands
        if (vshift == 0) return;
    }
    // compute cursor (same walk as the load cursor)
    int ct = sg.t_begin, ckt = 0;
    enter(ct, ckt);
    if (nsteps > 0) {
        load_step(0);
        store_v(0);
        sync_step();
    }
    for (int i = 0; i < nsteps; ++i) {
        const int buf = i & 1;
        const bool more = i + 1 < nsteps;
        if (more) load_step(buf ^ 1);
        const AttnTuple tp = tuples[ct];
        const int key0 = tp.t_lo + ckt;  // global index of the step's first key
        if ((!causal || key0 <= wave_qmax) && (!packed || (key0 + AT_KT > w_lo_min && key0 < w_hi_max))) {
            const uint16_t* ks = at_lds + buf * AT_STAGE;
            const _Float16* vt = reinterpret_cast<const _Float16*>(ks + AT_KT * D);
            // ---- S^T = K Q^T: two 32-key tiles
            f32x16_t s[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                // all eight fragments of the 32-key tile first, so LDS latency
                // overlaps the MFMA chain
                bf16x8_t kf[D / 16];
#pragma unroll
                for (int st = 0; st < D / 16; ++st)
                    kf[st] = *reinterpret_cast<const bf16x8_t*>(ks + at_koff(kt * 32 + lq, 2 * st + g));
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
                for (int st = 0; st < D / 16; ++st)
                    if constexpr (F16)
                        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8_t, kf[st]),
                                                                       __builtin_bit_cast(h8_t, qf[st]), s[kt], 0, 0, 0);
                    else
                        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s[kt], 0, 0, 0);
            }
            // ---- masks: only where the step crosses the diagonal or the key block's end
            const bool ragged = ckt + AT_KT > tp.T;
            const bool seqmask = packed && (key0 < w_lo_max || key0 + AT_KT > w_hi_min);
            if (ragged || seqmask) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        // acc index r -> key 8 (r / 4) + 4 g + r % 4 inside the 32-key tile
                        const int kk = kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                        const int key = key0 + kk;
                        const bool ok = ckt + kk < tp.T && (!causal || key <= qglob) &&
                                        (!packed || (key >= qs_lo && key < qs_hi));
                        s[kt][r] = ok ? s[kt][r] : -INFINITY;
                    }
            } else if (causal && key0 + AT_KT - 1 > wave_qmin) {
                const int lim = qglob - key0 - 4 * g;  // key kk visible iff kk - 4 g <= lim
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[kt][r] = kt * 32 + 8 * (r >> 2) + (r & 3) <= lim ? s[kt][r] : -INFINITY;
            }
            // ---- online softmax for query lq (this lane holds 32 of the 64
            // keys, the lane 32 away the other 32).  The maximum is taken on
            // raw scores, which the positive scale preserves.  The reference
            // maximum m_run only moves when a new score exceeds it by more
            // than 2^8 after scaling, so P stays in (0, 256] (exact in the
            // fp16 range) and O and l are rescaled rarely; the result
            // O = acc / l does not depend on the reference.
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
            {
                const auto sw =
                    __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const bool move = mx * scale_log2 > m_run * scale_log2 + 8.0f || (m_run == -INFINITY && mx != -INFINITY);
            if (__builtin_amdgcn_ballot_w64(move) != 0) {
                const float m_new = move ? mx : m_run;
                const float alpha = move ? __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2) : 1.0f;
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            }
            const float mc = m_run == -INFINITY ? 0.f : m_run * scale_log2;
            // P in fp16, two scores per conversion; the row sum is taken over
            // the rounded values the MFMA consumes (fp16 pairs dotted with 1)
            typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
            h8_t pf[4];
            float lsum = 0.f;
            const h2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], scale_log2, -mc));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r + 1], scale_log2, -mc));
                    const h2_t ph = {(_Float16)p0, (_Float16)p1};  // round to nearest even
                    lsum = __builtin_amdgcn_fdot2(ph, one2, lsum, false);
                    pf[kt * 2 + (r >> 3)][r & 7] = ph[0];
                    pf[kt * 2 + (r >> 3)][(r & 7) + 1] = ph[1];
                }
            l_run += lsum;
            // ---- O^T += V^T P^T : 4 k-steps of 16 keys
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                h8_t vf[D / 32];
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    vf[dt] = *reinterpret_cast<const h8_t*>(reinterpret_cast<const char*>(vt) + vrd[kq ^ dt] +
                                                            dt * 32 * AT_KT * 2);
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[dt], pf[kq], oacc[dt], 0, 0, 0);
            }
        }
        if (more) store_v(buf ^ 1);
        advance(ct, ckt, tp);  // the compute cursor
        sync_step();
    }
    // ---- finalize: O = acc / l ; lane holds O^T[d = 32 dt + 8 j + 4 g + r][query lq]
    float l_tot;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if constexpr (!F16 && !REDO) {
        // this wave's verdict for the REDO launch: its accumulators are not
        // finite (V beyond fp16's range), or its outputs average below 2^-12
        // (V perhaps below fp16's normal range; rows that saw no key are left
        // out)
        float sabs = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) sabs += fabsf(oacc[dt][r]);
        const bool odd = !(sabs < INFINITY) || (l_tot > 0.f && sabs < l_tot * 0x1p-6f);
        const uint32_t any = __builtin_amdgcn_ballot_w64(odd) != 0;
        if (lane == 0) flags[4 * vt + wave] = any;
    }
    auto unscale = [&](float x) {
        if constexpr (REDO) return __builtin_amdgcn_ldexpf(x, vshift);
        return x;
    };
    if constexpr (PARTIAL) {
        if (qrow < sg.S) {
            float* pp = (float*)O + sg.o_off + ((int64_t)tl.bh * sg.S + qrow) * ATTN_PROW;
            if (g == 0)
                *reinterpret_cast<float4*>(pp) = make_float4(
                    m_run == -INFINITY ? -INFINITY : m_run * (scale_log2 * 0.6931471805599453f), l_tot, 0.f, 0.f);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d = dt * 32 + 8 * j + 4 * g;
                    *reinterpret_cast<float4*>(pp + 4 + d) =
                        make_float4(unscale(oacc[dt][4 * j + 0]), unscale(oacc[dt][4 * j + 1]),
                                    unscale(oacc[dt][4 * j + 2]), unscale(oacc[dt][4 * j + 3]));
                }
        }
    } else {
        const float inv = 1.0f / l_tot;
        if (qrow < sg.S) {
            uint16_t* op = (uint16_t*)O + sg.o_off + qbh + (int64_t)qrow * qrs;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d = dt * 32 + 8 * j + 4 * g;
                    uint2 w;
                    w.x = pack_h16x2<F16>(unscale(oacc[dt][4 * j + 0] * inv), unscale(oacc[dt][4 * j + 1] * inv));
                    w.y = pack_h16x2<F16>(unscale(oacc[dt][4 * j + 2] * inv), unscale(oacc[dt][4 * j + 3] * inv));
                    *reinterpret_cast<uint2*>(op + d) = w;
                }
        }
    }
}

template <bool PACKED, bool F16, bool PARTIAL>
static void launch_pair(const AttnTile* tiles, int ntiles, const int32_t* ntiles_dev, const AttnSeg* segs,
                        const AttnTuple* tuples, const int32_t* seq_ends, int nseq, const void* Q, const void* K,
                        const void* V, void* O, uint32_t* flags, float scale_log2, int causal, hipStream_t stream) {
    const unsigned lds = 2u * AT_STAGE * sizeof(uint16_t);
    hipLaunchKernelGGL((attention_kernel<PACKED, F16, PARTIAL, false>), dim3(ntiles), dim3(AT_THREADS), lds, stream,
                       tiles, ntiles_dev, segs, tuples, seq_ends, nseq, (const uint16_t*)Q, (const uint16_t*)K,
                       (const uint16_t*)V, O, flags, scale_log2, causal);
    if constexpr (!F16)  // the flagged tiles again, V scaled (every other workgroup returns at once)
        hipLaunchKernelGGL((attention_kernel<PACKED, F16, PARTIAL, true>), dim3(ntiles), dim3(AT_THREADS), lds, stream,
                           tiles, ntiles_dev, segs, tuples, seq_ends, nseq, (const uint16_t*)Q, (const uint16_t*)K,
                           (const uint16_t*)V, O, flags, scale_log2, causal);
}

hipError_t launch_attention(const void* table, int64_t tiles_off, int32_t ntiles, int64_t segs_off,
                            int64_t tuples_off, int64_t seq_off, int32_t nseq, const void* Q, const void* K,
                            const void* V, void* O, uint32_t* flags, float scale, int32_t causal, int32_t f16,
                            int32_t partial, hipStream_t stream) {
    const uint8_t* t = (const uint8_t*)table;
    const float sl2 = scale * 1.4426950408889634f;
    const AttnTile* tl = (const AttnTile*)(t + tiles_off);
    const AttnSeg* sg = (const AttnSeg*)(t + segs_off);
    const AttnTuple* tp = (const AttnTuple*)(t + tuples_off);
    const int32_t* se = nseq ? (const int32_t*)(t + seq_off) : nullptr;
#define JA_ATT(P, H, R) launch_pair<P, H, R>(tl, ntiles, nullptr, sg, tp, se, nseq, Q, K, V, O, flags, sl2, causal, stream)
    if (partial) {
        if (nseq) {
            if (f16) JA_ATT(true, true, true); else JA_ATT(true, false, true);
        } else {
            if (f16) JA_ATT(false, true, true); else JA_ATT(false, false, true);
        }
    } else {
        if (nseq) {
            if (f16) JA_ATT(true, true, false); else JA_ATT(true, false, false);
        } else {
            if (f16) JA_ATT(false, true, false); else JA_ATT(false, false, false);
        }
    }
#undef JA_ATT
    return hipGetLastError();
}

hipError_t launch_attention_dev(const AttnTile* tiles, const int32_t* ntiles_dev, uint32_t max_tiles,
                                const AttnSeg* segs, const AttnTuple* tuples, const int32_t* seq_ends, int32_t nseq,
                                const void* Q, const void* K, const void* V, void* O, uint32_t* flags, float scale,
                                int32_t causal, int32_t f16, hipStream_t stream) {
    const float sl2 = scale * 1.4426950408889634f;
    if (f16)
        launch_pair<true, true, false>(tiles, (int)max_tiles, ntiles_dev, segs, tuples, seq_ends, nseq, Q, K, V, O,
                                       flags, sl2, causal, stream);
    else
        launch_pair<true, false, false>(tiles, (int)max_tiles, ntiles_dev, segs, tuples, seq_ends, nseq, Q, K, V, O,
                                        flags, sl2, causal, stream);
    return hipGetLastError();
}

}  // namespace ja
