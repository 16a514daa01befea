// gemm.hip -- the contraction join-agg: per-tuple block products with the SUM
// aggregation fused in.
//
// A matrix multiply is a join of A blocks and B blocks on the contracted
// index followed by a SUM over the contracted blocks ("Every Kernel Is a
// Join", paperpeel full text, section 1 and section 3.2, Examples 3.8 and
// 3.9).  Here a workgroup owns one output tile of one segment (all tuples
// that write one output block) at a time.  It walks the segment's tuples in
// ascending order and, inside each tuple, the contracted extent in BK-wide
// stages, accumulating in fp32 registers across tuple boundaries; the
// aggregated tile is written once.  So the SUM costs no extra memory traffic
// and needs no atomics (eager aggregation pushed into the kernel).
//
// bf16 / f16 path: v_mfma_f32_16x16x32_{bf16,f16} on CDNA4.  A workgroup of 8
// wavefronts owns a 256 x 256 output tile (128 x 64 per wavefront).  Operand
// tiles travel from global memory straight into LDS (buffer_load ... lds) in
// 32-wide stages, four stages in flight (128 KiB of the 160 KiB of LDS per
// CU).  The host lists the tiles of a segment in groups of GEMM_GROUP_M row
// tiles, and xcd_remap hands each XCD a contiguous run of that list, so the
// tiles resident on one XCD share A and B panels in its L2.  The kernel is
// persistent: one workgroup per compute unit walks its XCD's run, loading
// the next tile's first stage while the current tile's results are stored.
// Operand matrices are addressed with 32-bit buffer offsets, so the planner
// refuses an operand matrix of 2^30 elements or more.
#include <atomic>
#include <type_traits>

#include "dev_common.h"

namespace ja {

// ---------------------------------------------------------------- epilogue
// Write one lane's four adjacent outputs a[0..3]: columns col .. col + 3 of a
// segment block N columns wide, `off` the element offset of column col in the
// output as the contraction lays it out.  The epilogue `epi` is the 1:1 join
// applied on the way out: JA_EPI_ADD adds the residual R at the same offset
// (`r` holds its four elements when the store is vectorised, loaded earlier
// by residual4); with JA_EPI_SWIGLU the columns are (gate, up) pairs (N even,
// col a multiple of 4) and the pair at offset off writes silu(gate) * up to
// element off / 2 of the real output.
__device__ __forceinline__ bool vec_store(int64_t off, int col, int N) { return col + 4 <= N && (off & 3) == 0; }

// The residual's four elements at off when the store there is vectorised
// (all of a wavefront's loads are issued before its first store).
__device__ __forceinline__ uint2 residual4(const uint16_t* __restrict__ R, int epi, int64_t off, int col, int N) {
    if (epi == JA_EPI_ADD && vec_store(off, col, N)) return *reinterpret_cast<const uint2*>(R + off);
    return make_uint2(0u, 0u);
}

template <bool IN_F16, bool OUT16>
__device__ __forceinline__ void store_out4(void* __restrict__ C, const uint16_t* __restrict__ R, int epi, int64_t off,
                                           int col, int N, f32x4_t a, uint2 r) {
    if constexpr (OUT16) {
        uint16_t* c = (uint16_t*)C;
        if (epi == JA_EPI_SWIGLU) {
            const int64_t o = off >> 1;
            const float h0 = silu_mul(a[0], a[1]);
            const float h1 = silu_mul(a[2], a[3]);
            if (col + 4 <= N && (o & 1) == 0) {
                *reinterpret_cast<uint32_t*>(c + o) = pack_h16x2<IN_F16>(h0, h1);
            } else {
                if (col + 2 <= N) c[o] = (uint16_t)f32_to_h16<IN_F16>(h0);
                if (col + 4 <= N) c[o + 1] = (uint16_t)f32_to_h16<IN_F16>(h1);
            }
            return;
        }
        if (vec_store(off, col, N)) {
            if (epi == JA_EPI_ADD) {
                a[0] += h16lo_to_f32<IN_F16>(r.x);
                a[1] += h16hi_to_f32<IN_F16>(r.x);
                a[2] += h16lo_to_f32<IN_F16>(r.y);
                a[3] += h16hi_to_f32<IN_F16>(r.y);
            }
            *reinterpret_cast<uint2*>(c + off) =
                make_uint2(pack_h16x2<IN_F16>(a[0], a[1]), pack_h16x2<IN_F16>(a[2], a[3]));
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (col + r < N) {
                    float v = a[r];
                    if (epi == JA_EPI_ADD) v += h16_to_f32<IN_F16>(R[off + r]);
                    c[off + r] = (uint16_t)f32_to_h16<IN_F16>(v);
                }
        }
    } else {
        float* c = (float*)C;
        if (col + 4 <= N && (off & 3) == 0) {
            *reinterpret_cast<float4*>(c + off) = make_float4(a[0], a[1], a[2], a[3]);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (col + r < N) c[off + r] = a[r];
        }
    }
}

// ---------------------------------------------------------------- bf16 MFMA, direct-to-LDS pipeline
// The same tile and wavefront shape, but operand tiles travel from global
// memory straight into LDS (buffer_load ... lds, 16 bytes per lane) and NS
// stages of BK = 32 contracted elements are in flight at once, so a stage's
// loads have NS - 1 stages of MFMA work to arrive in.  No operand passes
// through registers on its way in; an operand whose rows are contiguous in
// memory (k strided) is stored as [k][rows] and read back transposed with
// ds_read_b64_tr_b16.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_p;
typedef __attribute__((address_space(3))) bf16x8_t* lds_bf16x8_p;

// GemmAsm<FM, KN, F16>::run / drain: the K loop in assembly (generated by gen_gemm_asm.py)
#include "gemm_asm.inc"

constexpr uint32_t DMA_OOB = 0x80000000u;  // a buffer offset past any valid extent: reads as zero

// Raw buffer descriptor over [base, base + bytes).
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4_t r;
    r.x = (int32_t)(uint32_t)a;
    r.y = (int32_t)(uint32_t)(a >> 32);  // stride 0
    r.z = (int32_t)bytes;
    r.w = 0x00020000;
    return r;
}

// 16 bytes per lane from global memory into LDS: lane l's bytes land at
// lds_byte + 16 l (lds_byte is wave-uniform); the global byte offset is
// voff + soff (soff is wave-uniform).  The compiler does not see the LDS
// write; the pipeline below waits on vmcnt itself before each barrier.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t lds_byte, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_byte), "v"(voff),
                 "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// LDS layouts of a 32-wide stage (element offsets).  K-contiguous tile
// [rows][32]: 16-byte chunk c of row r at c ^ ksw(r).  Row-contiguous tile
// [32][R]: chunk c (8 rows of the operand) of k-row k at c ^ msw(k).  Both
// were chosen against bank-conflict counts measured on gfx950 (64 banks of
// 4 bytes; a ds_read_b128 serves 16 lanes per cycle, not 16 consecutive
// lanes): an MFMA fragment read of either tile takes the minimum 4 (b128)
// or 2 (b64 transposed) LDS cycles.
__device__ __forceinline__ int ksw(int r) { return ((r >> 2) & 1) << 1; }
__device__ __forceinline__ int msw(int k) { return 2 * ((k & 3) | ((k >> 1) & 4)); }
__device__ __forceinline__ int koff(int r, int c) { return r * 32 + ((c ^ ksw(r)) << 3); }
template <int R>
__device__ __forceinline__ int moff(int k, int n) {
    return k * R + (((n >> 3) ^ msw(k)) << 3) + (n & 7);
}

// One operand tile of a stage: rows [r0, r0 + R) x k [k0, k0 + 32).  Each
// lane's byte offsets for k0 = 0 are computed once per tuple (rows past the
// block already folded into an out-of-range offset); a full stage then only
// adds the uniform k0 term as the instruction's scalar offset.
template <int R, int NT, bool MN>
struct DmaTile {
    static constexpr int SLOTS = R * 32 / 8;
    static constexpr int WAVES = NT / 64;
    static constexpr int PER_WAVE = SLOTS / 64 / WAVES;  // load instructions per wavefront per stage
    static_assert(SLOTS % (64 * WAVES) == 0, "tile must split evenly over the wavefronts");
    uint32_t off[PER_WAVE];  // byte offset of this lane's slot at k0 = 0

    // the slot's logical (row, k) inside the tile
    __device__ static void slot(int s, int& r, int& k) {
        if (MN) {
            k = s / (R / 8);
            r = ((s % (R / 8)) ^ msw(k)) * 8;
        } else {
            r = s / 4;
            k = ((s % 4) ^ ksw(r)) * 8;
        }
    }
    __device__ void setup(int ld, int r0, int rext, int wave, int lane) {
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            int r, k;
            slot((wave * PER_WAVE + j) * 64 + lane, r, k);
            const int gr = r0 + r;
            off[j] = gr < rext ? (uint32_t)((MN ? (int64_t)k * ld + gr : (int64_t)gr * ld + k) * 2) : DMA_OOB;
        }
    }
    // uniform byte offset of contracted position k0
    __device__ static uint32_t koffset(int ld, int k0) { return (uint32_t)((MN ? (int64_t)k0 * ld : (int64_t)k0) * 2); }

    // k of load instruction j's first element inside the stage (for ragged stages only)
    __device__ static int kin(int j, int wave, int lane) {
        int r, k;
        slot((wave * PER_WAVE + j) * 64 + lane, r, k);
        return k;
    }
    __device__ void issue(uint32_t lds_byte, i32x4_t rsrc, int ld, int k0, int kext, int wave, int lane) const {
        const uint32_t soff = koffset(ld, k0);
        if (k0 + 32 <= kext) {
#pragma unroll
            for (int j = 0; j < PER_WAVE; ++j) dma16(rsrc, lds_byte + (wave * PER_WAVE + j) * 1024, off[j], soff);
        } else {  // ragged last stage: slots past the contracted extent read zeros
#pragma unroll
            for (int j = 0; j < PER_WAVE; ++j)
                dma16(rsrc, lds_byte + (wave * PER_WAVE + j) * 1024,
                      (k0 + kin(j, wave, lane) < kext && off[j] != DMA_OOB) ? off[j] + soff : DMA_OOB, 0u);
        }
    }

    // The MFMA operand for fragment rows [rb, rb + 16): lane l gets row
    // rb + l % 16, k = 8 (l / 16) .. +7.
    __device__ static bf16x8_t frag(const uint16_t* tile, int rb, int lane) {
        if (MN) {
            const int g = lane >> 4, j = lane & 15;
            const int k = 8 * g + (j >> 2), n = rb + 4 * (j & 3);
            const uint16_t* p0 = tile + moff<R>(k, n);
            const uint16_t* p1 = tile + moff<R>(k + 4, n);
            i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)p0);
            i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)p1);
            typedef short i16x8_t __attribute__((ext_vector_type(8)));
            i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8_t, v);
        } else {
            const int r = rb + (lane & 15);
            return *reinterpret_cast<const bf16x8_t*>(tile + koff(r, lane >> 4));
        }
    }
};

// Wait until at most `left` of this wavefront's loads are in flight, then
// barrier.  `left` is a compile-time count.
template <int LEFT>
__device__ __forceinline__ void wait_loads_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(LEFT) : "memory");
}

template <int BM, int BN, int NS, int WM, int WN, int AL, int BL, bool IN_F16, bool OUT16>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_dma_kernel(const GemmTile* __restrict__ tiles, int ntiles,
                                                                    const GemmSeg* __restrict__ segs,
                                                                    const GemmTuple* __restrict__ tuples,
                                                                    const uint16_t* __restrict__ A,
                                                                    const uint16_t* __restrict__ B,
                                                                    void* __restrict__ C,
                                                                    const uint16_t* __restrict__ R, int epi) {
    constexpr int NT = WM * WN * 64;
    constexpr int BK = GEMM_DMA_BK;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    using TA = DmaTile<BM, NT, AL == JA_A_KM>;
    using TB = DmaTile<BN, NT, BL == JA_B_KN>;
    constexpr int PER_STAGE = TA::PER_WAVE + TB::PER_WAVE;
    // LDS: the A tiles of the NS stages, then their B tiles (so that every
    // fragment read of a stage is a base register plus a 16-bit offset)
    constexpr uint32_t A_STAGE = BM * BK * 2, B_STAGE = BN * BK * 2, B_REGION = NS * A_STAGE;
    static_assert(NS >= 2 && NS <= 4, "pipeline depth");
    static_assert((NS - 1) * PER_STAGE <= 63, "vmcnt range");
    extern __shared__ __attribute__((aligned(16))) uint16_t gemm_lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)gemm_lds;
    // The workgroup is persistent: it takes the tiles of the list at
    // positions blockIdx.x, blockIdx.x + gridDim.x, ... (after xcd_remap, so
    // every tile it takes is dealt to its own XCD, in the list's order).
    // A kernel whose tile height is below the list's (BM < GEMM_BF16_TM) runs
    // the tail of a list: virtual tile u = xcd_remap(v) is rows
    // [BM (u % 2), BM (u % 2 + 1)) of listed tile u / 2 (GEMM_BF16_TM = 2 BM).
    constexpr bool HALF = BM < GEMM_BF16_TM;
    static_assert(!HALF || 2 * BM == GEMM_BF16_TM, "a tail tile is half a listed tile");
    // (the virtual tiles of a tail launch are dealt through xcd_remap too, so
    // the two halves of a listed tile and its neighbours share one L2)
    auto tile_at = [&](int v) { return HALF ? tiles[xcd_remap(v, ntiles) >> 1] : tiles[xcd_remap(v, ntiles)]; };
    auto row0 = [&](int v, const GemmTile& t) { return HALF ? t.m0 + (xcd_remap(v, ntiles) & 1) * BM : t.m0; };
    int vt = blockIdx.x;
    GemmTile tl = tile_at(vt);
    GemmSeg sg = segs[tl.seg];
    int m0 = row0(vt, tl), n0 = tl.n0;
    auto count_stages = [&]() { return sg.nst; };  // planned on the host
    int nst = count_stages();

    f32x4_t acc[FM][FN];

    // load cursor: tuple lt, contracted offset lk inside it; the per-lane
    // offsets and buffer descriptors of tuple lt are cached (per tile: the
    // offsets depend on the tile's rows and columns)
    int lt = sg.t_begin, lk = 0, cached = -1;
    TA ta;
    TB tb;
    i32x4_t rsa, rsb;
    int lda = 0, ldb = 0, kext = 0;
    // (kernels with the assembly K loop issue here only between tiles, and
    // recompute the offsets each time rather than keep them live: kept, they
    // would be spilled, and a spill reload's wait also waits for the stage
    // loads in flight)
    constexpr bool RECOMPUTE = OUT16 && AL == JA_A_MK && NT == 512 && NS == 4 && BK == 32 && BN == 256 &&
                               (BM == 256 || BM == 128);
    auto use_tuple = [&]() {
        if (RECOMPUTE || cached != lt) {
            const GemmTuple tp = tuples[lt];
            const uint16_t* pa = A + tp.a_off + (int64_t)tl.batch * tp.a_bstride;
            const uint16_t* pb = B + tp.b_off + (int64_t)tl.batch * tp.b_bstride;
            rsa = buffer_rsrc(pa, (uint32_t)(tp.a_bstride * 2));
            rsb = buffer_rsrc(pb, (uint32_t)(tp.b_bstride * 2));
            lda = tp.lda;
            ldb = tp.ldb;
            kext = tp.K;
            // from an opaque copy of the lane index, so that the slot
            // arithmetic is not hoisted out of the tile loop and kept live
            int el = lane;
            asm volatile("" : "+v"(el));
            ta.setup(lda, m0, sg.M, wave, el);
            tb.setup(ldb, n0, sg.N, wave, el);
            cached = lt;
        }
    };
    auto issue = [&](int buf) {
        use_tuple();
        int el = lane;  // opaque, as in use_tuple
        asm volatile("" : "+v"(el));
        ta.issue(lds0 + buf * A_STAGE, rsa, lda, lk, kext, wave, el);
        tb.issue(lds0 + B_REGION + buf * B_STAGE, rsb, ldb, lk, kext, wave, el);
        lk += BK;
        if (lk >= kext) {
            lk = 0;
            ++lt;
        }
    };
    // Stage s lives in LDS buffer s % NS.  The fragments of stage it + 1 are
    // read into registers while the MFMAs of stage it run, so once a
    // wavefront passes the barrier of iteration it, nobody reads buffer
    // it % NS any more and it is refilled with stage it + NS.
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < nst) issue(s);

    const int arow = wm * WTM, brow = wn * WTN;
    bf16x8_t fa[2][FM], fb[2][FN];
    auto read_frags = [&](int buf, bf16x8_t* a, bf16x8_t* b) {
        const uint16_t* as = gemm_lds + buf * (A_STAGE / 2);
        const uint16_t* bs = gemm_lds + (B_REGION + buf * B_STAGE) / 2;
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = TA::frag(as, arow + i * 16, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = TB::frag(bs, brow + j * 16, lane);
    };
    // wait until stage `need` has landed: the stages issued after it may stay in flight
    auto wait_stage = [&](int need) {
        // issued so far: stages 0 .. NS - 1 up front, then one per step
        const int ahead = need == 0 ? min(NS - 1, nst - 1) : min(need + NS - 2, nst - 1) - need;
        if (ahead >= 3)
            wait_loads_barrier<(NS >= 4 ? 3 : 0) * PER_STAGE>();
        else if (ahead == 2)
            wait_loads_barrier<(NS >= 3 ? 2 : 0) * PER_STAGE>();
        else if (ahead == 1)
            wait_loads_barrier<PER_STAGE>();
        else
            wait_loads_barrier<0>();
    };
    // After the barrier a wavefront starts its MFMAs at once (their operands
    // were read one step earlier) and issues the refill of buffer it % NS
    // halfway through them, so the load issue hides behind matrix work.
    // Per step: barrier; the first quarter of the MFMAs (their operands were
    // read one step earlier and are complete, so any wait the compiler puts
    // before them is free); the fragment reads of the next stage; a quarter;
    // the refill of buffer it % NS; the last half.  The reads and the load
    // issue thus run in the shadow of matrix work.  The wait and the reads
    // also run on the last step (reading a buffer nobody refills any more)
    // so that every path has the same LDS reads in flight.
    auto mfma_rows = [&](int i0, int i1, const bf16x8_t* ca, const bf16x8_t* cb) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            if (i >= i0 && i < i1)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mfma16x16x32<IN_F16>(cb[j], ca[i], acc[i][j]);
    };
    auto step = [&](int it, bf16x8_t* ca, bf16x8_t* cb, bf16x8_t* na, bf16x8_t* nb) {
        wait_stage(it + 1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_rows(0, FM / 4, ca, cb);
        __builtin_amdgcn_sched_barrier(0);
        read_frags((it + 1) % NS, na, nb);
        __builtin_amdgcn_sched_barrier(0);
        mfma_rows(FM / 4, FM / 2, ca, cb);
        __builtin_amdgcn_sched_barrier(0);
        if (it + NS < nst) issue(it % NS);
        __builtin_amdgcn_sched_barrier(0);
        mfma_rows(FM / 2, FM, ca, cb);
    };
    // Row-major A and 16-bit outputs in the 8-wavefront kernels: the K loop is inline assembly
    // (GemmAsm, written out by gen_gemm_asm.py) that threads the next stage's
    // fragment reads and the refill loads between the MFMAs one at a time.
    // The C++ side walks a tile's steps in runs: steps whose refills are full
    // stages of one tuple, a single step whose refill is a ragged stage, and
    // the last steps, which refill nothing.  Each run starts from stage buffer
    // it % NS with the lane's fragment addresses offset to it.
    // (fp32 outputs, the unfused form's per-tuple partials, keep the compiler's
    // loop: their four-byte stores from AGPR accumulators measured 10% slower)
    constexpr bool ASM = RECOMPUTE;
    using GA = GemmAsm<FM, BL == JA_B_KN, IN_F16>;
    static_assert(!ASM || (GA::PA == TA::PER_WAVE && GA::PB == TB::PER_WAVE && FN == 4), "asm instance");
    // Between statements the compiler has only the registers the statement
    // leaves it (its fragments take 96 VGPRs, the accumulators 128 AGPRs), so
    // every per-lane value a statement needs is recomputed before it from an
    // opaque copy of the lane index instead of being kept across the loop.
    // head: 0, or the memory operations per fragment pair and lane (1: a
    // store, 2: a residual load and a store) of the previous tile's full-tile
    // epilogue, issued after this tile's first NS stages, which its first
    // steps need not wait for.  pbase: the stage buffer holding the tile's
    // stage 0.  pf: the tile's last NS steps refill the stage buffers with
    // the first NS stages of the workgroup's next tile (full stages of its
    // first tuple), so those load while this tile drains and stores.
    int scached = -1;
    auto k_loop_asm = [&](uint32_t head, int pbase, bool pf) {
        int it = 0;
        scached = -1;
        while (it < nst) {
            int el = lane;
            asm volatile("" : "+v"(el));
            const uint32_t ph = (uint32_t)((it + pbase) % NS);
            // the lane's fragment addresses in stage buffer ph (as TA::frag and TB::frag compute them)
            const uint32_t ra = lds0 + ph * A_STAGE + 2 * koff(arow + (el & 15), el >> 4);
            uint32_t rb[GA::NRB];
            if constexpr (BL == JA_B_KN) {
                const int jl = el & 15, k = 8 * (el >> 4) + (jl >> 2);
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = brow + j * 16 + 4 * (jl & 3);
                    rb[2 * j] = lds0 + B_REGION + ph * B_STAGE + 2 * moff<BN>(k, n);
                    rb[2 * j + 1] = lds0 + B_REGION + ph * B_STAGE + 2 * moff<BN>(k + 4, n);
                }
            } else {
                rb[0] = lds0 + B_REGION + ph * B_STAGE + 2 * koff(brow + (el & 15), el >> 4);
            }
            // n1 steps refilling a stage each (the refill of step it is stage
            // it + NS, at the load cursor), then n2 steps refilling nothing
            uint32_t va[GA::PA], vb[GA::PB], sa = 0, sb = 0, ia = 0, ib = 0;
            int n1 = 0;
            if (it + NS < nst) {
                if (scached != lt) {  // the tuple's scalars only: per-lane offsets are recomputed below
                    const GemmTuple tp = tuples[lt];
                    rsa = buffer_rsrc(A + tp.a_off + (int64_t)tl.batch * tp.a_bstride, (uint32_t)(tp.a_bstride * 2));
                    rsb = buffer_rsrc(B + tp.b_off + (int64_t)tl.batch * tp.b_bstride, (uint32_t)(tp.b_bstride * 2));
                    lda = tp.lda;
                    ldb = tp.ldb;
                    kext = tp.K;
                    scached = lt;
                    cached = -1;
                }
                // this run's load offsets, from the lane index (not kept from the tuple's set-up)
                TA xa_t;
                TB xb_t;
                xa_t.setup(lda, m0, sg.M, wave, el);
                xb_t.setup(ldb, n0, sg.N, wave, el);
                ia = TA::koffset(lda, BK);
                ib = TB::koffset(ldb, BK);
                n1 = 1;
                if (lk + BK <= kext) {
                    n1 = min((kext - lk) / BK, nst - NS - it);
#pragma unroll
                    for (int j = 0; j < GA::PA; ++j) va[j] = xa_t.off[j];
#pragma unroll
                    for (int j = 0; j < GA::PB; ++j) vb[j] = xb_t.off[j];
                    sa = TA::koffset(lda, lk);
                    sb = TB::koffset(ldb, lk);
                } else {  // ragged stage: slots past the contracted extent read zeros
                    const uint32_t xa = TA::koffset(lda, lk), xb = TB::koffset(ldb, lk);
#pragma unroll
                    for (int j = 0; j < GA::PA; ++j)
                        va[j] = (lk + TA::kin(j, wave, el) < kext && xa_t.off[j] != DMA_OOB) ? xa_t.off[j] + xa : DMA_OOB;
#pragma unroll
                    for (int j = 0; j < GA::PB; ++j)
                        vb[j] = (lk + TB::kin(j, wave, el) < kext && xb_t.off[j] != DMA_OOB) ? xb_t.off[j] + xb : DMA_OOB;
                }
                lk += n1 * BK;
                if (lk >= kext) {
                    lk = 0;
                    ++lt;
                }
            } else if (pf) {  // it == nst - NS: refill with the next tile's stages 0 .. NS - 1
                const int vn = vt + (int)gridDim.x;
                const GemmTile tn = tile_at(vn);
                const GemmSeg sn = segs[tn.seg];
                const GemmTuple tp = tuples[sn.t_begin];
                rsa = buffer_rsrc(A + tp.a_off + (int64_t)tn.batch * tp.a_bstride, (uint32_t)(tp.a_bstride * 2));
                rsb = buffer_rsrc(B + tp.b_off + (int64_t)tn.batch * tp.b_bstride, (uint32_t)(tp.b_bstride * 2));
                scached = -1;
                cached = -1;
                TA xa_t;
                TB xb_t;
                xa_t.setup(tp.lda, row0(vn, tn), sn.M, wave, el);
                xb_t.setup(tp.ldb, tn.n0, sn.N, wave, el);
                ia = TA::koffset(tp.lda, BK);
                ib = TB::koffset(tp.ldb, BK);
#pragma unroll
                for (int j = 0; j < GA::PA; ++j) va[j] = xa_t.off[j];
#pragma unroll
                for (int j = 0; j < GA::PB; ++j) vb[j] = xb_t.off[j];
                n1 = NS;
            } else {
#pragma unroll
                for (int j = 0; j < GA::PA; ++j) va[j] = DMA_OOB;
#pragma unroll
                for (int j = 0; j < GA::PB; ++j) vb[j] = DMA_OOB;
            }
            const int n2 = !pf && it + n1 + NS >= nst ? nst - it - n1 : 0;
            const uint32_t nh = __builtin_amdgcn_readfirstlane(it == 0 && n1 >= NS - 1 ? head : 0u);
            const uint32_t ma = lds0 + ph * A_STAGE + wave * TA::PER_WAVE * 1024;
            const uint32_t mb = lds0 + B_REGION + ph * B_STAGE + wave * TB::PER_WAVE * 1024;
            // (uniform values; read from lane 0 so that they stay scalar operands)
            sa = __builtin_amdgcn_readfirstlane(sa);
            sb = __builtin_amdgcn_readfirstlane(sb);
            ia = __builtin_amdgcn_readfirstlane(ia);
            ib = __builtin_amdgcn_readfirstlane(ib);
            GA::steps(acc, (uint32_t)n1, (uint32_t)n2, ph, ra, rb, rsa, rsb, va, vb, sa, sb, ia, ib, ma, mb, nh);
            it += n1 + n2;
        }
    };
    if (!ASM && nst > 0) {
        wait_stage(0);
        read_frags(0, fa[0], fb[0]);
    }
    // epilogue of one tile: lane owns C[row][col .. col+3] of every fragment
    // An accumulator fragment moved into VGPRs where it is used: with the
    // accumulators in AGPRs the compiler would otherwise copy them all out at
    // the start of the epilogue and spill what does not fit.
    auto accv = [&](int i, int j) {
        f32x4_t a = acc[i][j];
        if constexpr (ASM) asm volatile("" : "+v"(a));
        return a;
    };
    // a whole tile inside its block with 8-element aligned rows: the epilogue
    // stores it in fragment pairs, FM * FN / 2 stores per lane
    auto paired = [&](int64_t cbase, int ldc, int eM, int eN, int em0, int en0) {
        return OUT16 && FN % 2 == 0 && em0 + BM <= eM && en0 + BN <= eN && ((cbase | (int64_t)ldc) & 7) == 0;
    };
    auto epilogue = [&](int64_t cbase, int ldc, int eM, int eN, int em0, int en0) {
        // The lane's row and column offsets are recomputed here from an
        // opaque copy of the lane index: hoisted out of the tile loop they
        // would stay live through the K loop and push it into spills.
        int el = lane;
        asm volatile("" : "+v"(el));
        const int kc = el >> 4;
        // A whole tile inside its block with 4-element aligned rows (the
        // usual case): every store is a vector store, so the bounds and
        // alignment checks and the choice of epilogue are made once per tile.
        // Full tiles whose rows are 8-element aligned, in fragment pairs: one
        // v_permlane16_swap per accumulator register gives each lane eight
        // adjacent columns (lanes 0-15 and 32-47 columns 0-7 and 8-15 of the
        // first fragment, lanes 16-31 and 48-63 those of the second), so each
        // store writes 16 bytes per lane and 64 contiguous bytes per row:
        // half the store instructions of the plain layout and no 32-byte
        // pieces, which matters because every compute unit writes its tile at
        // the same moment.
        if (paired(cbase, ldc, eM, eN, em0, en0)) {
            uint16_t* c = (uint16_t*)C;
            const int64_t lbase =
                cbase + (int64_t)(em0 + arow + (el & 15)) * ldc + en0 + brow + (kc & 1) * 16 + (kc >> 1) * 8;
            // the lane's eight columns of fragment pair (i, 2 p), in order
            auto pair = [&](int i, int p, float* v) {
                const f32x4_t x = accv(i, 2 * p), y = accv(i, 2 * p + 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[r]), __float_as_uint(y[r]), false,
                                                                     false);
                    v[r] = __uint_as_float(sw[0]);
                    v[4 + r] = __uint_as_float(sw[1]);
                }
            };
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int64_t rbase = lbase + (int64_t)i * 16 * ldc;
                if (epi == JA_EPI_ADD) {
                    uint4 res[FN / 2];
#pragma unroll
                    for (int p = 0; p < FN / 2; ++p) res[p] = *reinterpret_cast<const uint4*>(R + rbase + 32 * p);
#pragma unroll
                    for (int p = 0; p < FN / 2; ++p) {
                        float v[8];
                        pair(i, p, v);
                        const uint32_t w[4] = {res[p].x, res[p].y, res[p].z, res[p].w};
                        uint32_t o[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            o[q] = pack_h16x2<IN_F16>(v[2 * q] + h16lo_to_f32<IN_F16>(w[q]),
                                                      v[2 * q + 1] + h16hi_to_f32<IN_F16>(w[q]));
                        *reinterpret_cast<uint4*>(c + rbase + 32 * p) = make_uint4(o[0], o[1], o[2], o[3]);
                    }
                } else {
#pragma unroll
                    for (int p = 0; p < FN / 2; ++p) {
                        float v[8];
                        pair(i, p, v);
                        if (epi == JA_EPI_SWIGLU)  // four (gate, up) pairs -> four adjacent outputs
                            *reinterpret_cast<uint2*>(c + ((rbase + 32 * p) >> 1)) =
                                make_uint2(pack_h16x2<IN_F16>(silu_mul(v[0], v[1]), silu_mul(v[2], v[3])),
                                           pack_h16x2<IN_F16>(silu_mul(v[4], v[5]), silu_mul(v[6], v[7])));
                        else
                            *reinterpret_cast<uint4*>(c + rbase + 32 * p) =
                                make_uint4(pack_h16x2<IN_F16>(v[0], v[1]), pack_h16x2<IN_F16>(v[2], v[3]),
                                           pack_h16x2<IN_F16>(v[4], v[5]), pack_h16x2<IN_F16>(v[6], v[7]));
                    }
                }
            }
            return;
        }
        if (OUT16 && em0 + BM <= eM && en0 + BN <= eN && ((cbase | (int64_t)ldc) & 3) == 0) {
            uint16_t* c = (uint16_t*)C;
            const int64_t lbase = cbase + (int64_t)(em0 + arow + (el & 15)) * ldc + en0 + brow + 4 * kc;
            if (epi == JA_EPI_SWIGLU) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int64_t o = (lbase + (int64_t)i * 16 * ldc + j * 16) >> 1;
                        const f32x4_t a = accv(i, j);
                        *reinterpret_cast<uint32_t*>(c + o) =
                            pack_h16x2<IN_F16>(silu_mul(a[0], a[1]), silu_mul(a[2], a[3]));
                    }
            } else if (epi == JA_EPI_ADD) {
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    uint2 res[FN];
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        res[j] = *reinterpret_cast<const uint2*>(R + lbase + (int64_t)i * 16 * ldc + j * 16);
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const f32x4_t a = accv(i, j);
                        *reinterpret_cast<uint2*>(c + lbase + (int64_t)i * 16 * ldc + j * 16) =
                            make_uint2(pack_h16x2<IN_F16>(a[0] + h16lo_to_f32<IN_F16>(res[j].x),
                                                          a[1] + h16hi_to_f32<IN_F16>(res[j].x)),
                                       pack_h16x2<IN_F16>(a[2] + h16lo_to_f32<IN_F16>(res[j].y),
                                                          a[3] + h16hi_to_f32<IN_F16>(res[j].y)));
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const f32x4_t a = accv(i, j);
                        *reinterpret_cast<uint2*>(c + lbase + (int64_t)i * 16 * ldc + j * 16) =
                            make_uint2(pack_h16x2<IN_F16>(a[0], a[1]), pack_h16x2<IN_F16>(a[2], a[3]));
                    }
            }
            return;
        }
        // one row of fragments at a time: its residual loads are all in
        // flight before the first of its stores
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = em0 + arow + i * 16 + (el & 15);
            uint2 res[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = en0 + brow + j * 16 + 4 * kc;
                res[j] = row < eM ? residual4(R, epi, cbase + (int64_t)row * ldc + col, col, eN) : make_uint2(0u, 0u);
            }
            if (row >= eM) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = en0 + brow + j * 16 + 4 * kc;
                store_out4<IN_F16, OUT16>(C, R, epi, cbase + (int64_t)row * ldc + col, col, eN, accv(i, j), res[j]);
            }
        }
    };

    // the previous tile's epilogue, if it stored in fragment pairs after this
    // tile's first NS stages had been issued: its memory operations per
    // fragment pair and lane (0: not so)
    uint32_t stored_after = 0;
    int pbase = 0;  // stage buffer of the tile's stage 0 (ASM)
    bool pf = false;
    while (true) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (ASM) {
            // Stage 0 is followed in issue order by stages 1 .. NS - 1 and
            // then the previous tile's epilogue (its stores, and with head 2
            // a residual load before each); vector memory operations
            // complete in issue order, so waiting for stage 0 leaves both in
            // flight.
            const uint32_t head = nst >= NS ? stored_after : 0u;
            if (head == 2)
                wait_loads_barrier<(NS - 1) * PER_STAGE + 2 * GA::STORES>();
            else if (head == 1)
                wait_loads_barrier<(NS - 1) * PER_STAGE + GA::STORES>();
            else if (nst > 0)
                wait_stage(0);
            // prefetch the next tile's first stages if this tile has a full
            // drain and the next one starts with NS full stages of one tuple
            pf = false;
            if (nst >= NS && vt + (int)gridDim.x < ntiles) {
                const GemmTile tn = tile_at(vt + (int)gridDim.x);
                const GemmSeg sn = segs[tn.seg];
                pf = sn.nst >= NS && tuples[sn.t_begin].K >= NS * BK;
            }
            k_loop_asm(head, pbase, pf);
        } else {
            if (nst > 0) {
                wait_stage(0);
                read_frags(0, fa[0], fb[0]);
            }
            for (int it = 0; it < nst; it += 2) {
                step(it, fa[0], fb[0], fa[1], fb[1]);
                if (it + 1 < nst) step(it + 1, fa[1], fb[1], fa[0], fb[0]);
            }
        }
        // Next tile: with pf its first NS stages were loaded during this
        // tile's last NS steps.  Otherwise they are loaded now, while this
        // tile's results leave (all of them, unless the epilogue loads a
        // residual: that load would wait behind them, so then only the first
        // stage goes early and the rest after the stores).  The barrier makes
        // sure that every wavefront's last fragment reads are complete before
        // LDS is refilled.
        const int64_t ecbase = sg.c_off + (int64_t)tl.batch * sg.c_bstride;
        const int eldc = sg.ldc, eM = sg.M, eN = sg.N, em0 = m0, en0 = n0;
        const int vnext = vt + (int)gridDim.x;
        const bool more = vnext < ntiles;
        const int nst_done = nst;
        if (more) {
            vt = vnext;
            tl = tile_at(vt);
            sg = segs[tl.seg];
            m0 = row0(vt, tl);
            n0 = tl.n0;
            nst = count_stages();
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // an epilogue that loads the residual would wait behind every stage
        // issued before it, so then only the first goes out early
        const int early = epi == JA_EPI_ADD ? 1 : NS;
        if (more) {
            lt = sg.t_begin;
            lk = 0;
            cached = -1;
            if (pf) {  // stages 0 .. NS - 1 are in flight, in the buffers after this tile's last
                pbase = (pbase + nst_done) % NS;
                lk = NS * BK;
                if (lk >= tuples[lt].K) {
                    lk = 0;
                    ++lt;
                }
            } else {
                pbase = 0;
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    if (s < early && s < nst) issue(s);
            }
        }
        stored_after = more && (pf || early == NS) && paired(ecbase, eldc, eM, eN, em0, en0)
                           ? (epi == JA_EPI_ADD ? 2u : 1u)
                           : 0u;
        epilogue(ecbase, eldc, eM, eN, em0, en0);
        if (!more) break;
        cached = -1;  // the load offsets are recomputed rather than kept through the epilogue
        if (!pf) {
#pragma unroll
            for (int s = 1; s < NS; ++s)
                if (s >= early && s < nst) issue(s);
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
// Compute units of the current device (one persistent contraction workgroup
// each); cached per device.
static int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 0;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int AL, int BL, bool F16, bool OUT16>
static void launch_bf16_dma(const GemmTile* tiles, int ntiles, const GemmSeg* segs, const GemmTuple* tuples,
                            const void* A, const void* B, void* C, const void* R, int epi, hipStream_t s) {
    constexpr int BM = GEMM_BF16_TM, BN = GEMM_BF16_TN, NS = GEMM_DMA_STAGES, WM = 2, WN = 4;
    constexpr unsigned lds = (unsigned)NS * (BM + BN) * 32 * sizeof(uint16_t);
    // one workgroup per compute unit (128 KiB of LDS each), walking the tile list
    const int cus = device_cus();
    // A last round that would fill at most half the compute units runs as
    // twice as many half-height tiles instead: 2r tiles of half the work each
    // finish sooner than r full tiles on r units.
    const int tail = cus > 0 && ntiles > cus && 2 * (ntiles % cus) <= cus ? ntiles % cus : 0;
    const int nmain = ntiles - tail;
    const int grid = cus > 0 && cus < nmain ? cus : nmain;
    hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, NS, WM, WN, AL, BL, F16, OUT16>), dim3(grid),
                       dim3(WM * WN * 64), lds, s, tiles, nmain, segs, tuples, (const uint16_t*)A,
                       (const uint16_t*)B, C, (const uint16_t*)R, epi);
    if (tail > 0) {
        constexpr int HM = BM / 2;
        constexpr unsigned hlds = (unsigned)NS * (HM + BN) * 32 * sizeof(uint16_t);
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<HM, BN, NS, WM, WN, AL, BL, F16, OUT16>), dim3(2 * tail),
                           dim3(WM * WN * 64), hlds, s, tiles + nmain, 2 * tail, segs, tuples, (const uint16_t*)A,
                           (const uint16_t*)B, C, (const uint16_t*)R, epi);
    }
}

// 16-bit inputs (bf16 or, with F16, IEEE half) into fp32 accumulators;
// out16 writes the output in the input's format, otherwise fp32.
template <int AL, int BL, bool F16>
static void launch_bf16_out(int out16, const GemmTile* tiles, int ntiles, const GemmSeg* segs,
                            const GemmTuple* tuples, const void* A, const void* B, void* C, const void* R, int epi,
                            hipStream_t s) {
    if (out16)
        launch_bf16_dma<AL, BL, F16, true>(tiles, ntiles, segs, tuples, A, B, C, R, epi, s);
    else
        launch_bf16_dma<AL, BL, F16, false>(tiles, ntiles, segs, tuples, A, B, C, R, epi, s);
}

template <bool F16>
static void launch_h16(int a_layout, int b_layout, int out16, const GemmTile* tiles, int ntiles,
                       const GemmSeg* segs, const GemmTuple* tuples, const void* A, const void* B, void* C,
                       const void* R, int epi, hipStream_t s) {
    if (a_layout == JA_A_MK && b_layout == JA_B_KN)
        launch_bf16_out<JA_A_MK, JA_B_KN, F16>(out16, tiles, ntiles, segs, tuples, A, B, C, R, epi, s);
    else if (a_layout == JA_A_MK && b_layout == JA_B_NK)
        launch_bf16_out<JA_A_MK, JA_B_NK, F16>(out16, tiles, ntiles, segs, tuples, A, B, C, R, epi, s);
    else if (a_layout == JA_A_KM && b_layout == JA_B_KN)
        launch_bf16_out<JA_A_KM, JA_B_KN, F16>(out16, tiles, ntiles, segs, tuples, A, B, C, R, epi, s);
    else
        launch_bf16_out<JA_A_KM, JA_B_NK, F16>(out16, tiles, ntiles, segs, tuples, A, B, C, R, epi, s);
}

hipError_t launch_gemm(const void* table, int64_t tiles_off, int32_t ntiles, int64_t segs_off, int64_t tuples_off,
                       const void* A, const void* B, void* C, const void* R, int32_t epi, int32_t in_dtype,
                       int32_t out_dtype, int32_t a_layout, int32_t b_layout, hipStream_t s) {
    const uint8_t* t = (const uint8_t*)table;
    const GemmTile* tiles = (const GemmTile*)(t + tiles_off);
    const GemmSeg* segs = (const GemmSeg*)(t + segs_off);
    const GemmTuple* tuples = (const GemmTuple*)(t + tuples_off);
    if (in_dtype == JA_BF16 || in_dtype == JA_F16) {
        const int out16 = out_dtype != JA_F32;
        if (in_dtype == JA_F16)
            launch_h16<true>(a_layout, b_layout, out16, tiles, ntiles, segs, tuples, A, B, C, R, epi, s);
        else
            launch_h16<false>(a_layout, b_layout, out16, tiles, ntiles, segs, tuples, A, B, C, R, epi, s);
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
