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
//
// One workgroup = 4 wavefronts = 128 query rows of one segment.  A segment's
// tuples are folded in ascending key order, 64 keys per step:
//   S^T[key][query] = K Q^T  with v_mfma_f32_32x32x16_bf16 (Q fragments stay
//                            in registers for the whole segment);
//   P = exp2(S * scale * log2(e) - m), fp32, then fp16;
//   O^T[d][query] += V^T P^T with v_mfma_f32_32x32x16_f16.
// Computing S transposed puts each lane on one query, so P leaves the first
// MFMA's accumulators already in the second MFMA's B-operand layout.  V is
// transposed (and converted to fp16) on its way to LDS, with the key order
// inside each 16-key group arranged to match those accumulators.
#include "dev_common.h"

namespace ja {

constexpr int AT_KT = 64;          // keys per step
constexpr int AT_KPITCH = 128 + 8; // K tile row pitch in LDS (elements)
constexpr int AT_VPITCH = AT_KT + 8;

__global__ __launch_bounds__(256) void attention_kernel(const AttnTile* __restrict__ tiles, int ntiles,
                                                        const AttnSeg* __restrict__ segs,
                                                        const AttnTuple* __restrict__ tuples,
                                                        const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                                        float scale_log2, int causal) {
    constexpr int D = ATTN_D;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[AT_KT * AT_KPITCH];
    __shared__ __attribute__((aligned(16))) _Float16 Vt[D * AT_VPITCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, lq = lane & 31;
    const AttnTile tl = tiles[blockIdx.x];
    const AttnSeg sg = segs[tl.seg];
    const int qrow = tl.s0 + wave * 32 + lq;  // query row inside the block
    const int qglob = sg.s_lo + qrow;         // global query index (causal mask)
    const int wave_qmax = sg.s_lo + min(tl.s0 + wave * 32 + 31, sg.S - 1);

    // Q^T fragments (B operand): lane holds Q[query lq][d = 16*step + 8*g .. +7]
    bf16x8_t qf[D / 16];
    {
        const uint16_t* qp = Q + sg.q_off + (int64_t)tl.bh * sg.q_bhstride + (int64_t)qrow * D + 8 * g;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qrow < sg.S) v = *reinterpret_cast<const uint4*>(qp + 16 * st);
            qf[st] = *reinterpret_cast<bf16x8_t*>(&v);
        }
    }
    f32x16_t oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int t = sg.t_begin; t < sg.t_end; ++t) {
        const AttnTuple tp = tuples[t];
        const uint16_t* kb = K + tp.k_off + (int64_t)tl.bh * tp.kv_bhstride;
        const uint16_t* vb = V + tp.v_off + (int64_t)tl.bh * tp.kv_bhstride;
        for (int kt0 = 0; kt0 < tp.T; kt0 += AT_KT) {
            const int key0 = tp.t_lo + kt0;  // global index of the step's first key
            // whole workgroup skips steps no query of the tile can see
            const int tile_qmax = sg.s_lo + min(tl.s0 + 127, sg.S - 1);
            if (causal && key0 > tile_qmax) break;
            // ---- stage K (direct) and V (transposed to [d][key], fp16) through registers
            uint4 kr[4], vr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int vi = tid + j * 256;
                int r = vi >> 4, c = (vi & 15) * 8;
                kr[j] = make_uint4(0, 0, 0, 0);
                if (kt0 + r < tp.T) kr[j] = *reinterpret_cast<const uint4*>(kb + (int64_t)(kt0 + r) * D + c);
            }
            // V: one sub-block of 4 keys x 8 d per thread (16 key quads x 16 d octets)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int key = kt0 + (tid >> 4) * 4 + i;
                vr[i] = make_uint4(0, 0, 0, 0);
                if (key < tp.T) vr[i] = *reinterpret_cast<const uint4*>(vb + (int64_t)key * D + (tid & 15) * 8);
            }
            __syncthreads();  // previous step's readers are done
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int vi = tid + j * 256;
                int r = vi >> 4, c = (vi & 15) * 8;
                *reinterpret_cast<uint4*>(Ks + r * AT_KPITCH + c) = kr[j];
            }
            {
                // thread: keys kg*4..+3, d = 8*(tid&15) .. +7
                int kg = tid >> 4, d0 = (tid & 15) * 8;
                int hgrp = kg >> 2, q = kg & 3;
                int qpos = q == 1 ? 2 : (q == 2 ? 1 : q);  // swap the middle quads of each 16-key group
                int col = hgrp * 16 + qpos * 4;
                const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&vr[0]);
                const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&vr[1]);
                const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&vr[2]);
                const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&vr[3]);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        float a0 = e ? bf16hi_to_f32(r0[w]) : bf16lo_to_f32(r0[w]);
                        float a1 = e ? bf16hi_to_f32(r1[w]) : bf16lo_to_f32(r1[w]);
                        float a2 = e ? bf16hi_to_f32(r2[w]) : bf16lo_to_f32(r2[w]);
                        float a3 = e ? bf16hi_to_f32(r3[w]) : bf16lo_to_f32(r3[w]);
                        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
                        h4 hv = {(_Float16)a0, (_Float16)a1, (_Float16)a2, (_Float16)a3};
                        *reinterpret_cast<h4*>(Vt + (d0 + 2 * w + e) * AT_VPITCH + col) = hv;
                    }
                }
            }
            __syncthreads();
            if (causal && key0 > wave_qmax) continue;  // nothing visible to this wave
            // ---- S^T = K Q^T : two 32-key tiles
            f32x16_t s[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
                for (int st = 0; st < D / 16; ++st) {
                    bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(Ks + (kt * 32 + lq) * AT_KPITCH + 16 * st + 8 * g);
                    s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s[kt], 0, 0, 0);
                }
            }
            // ---- online softmax for query lq (this lane holds 32 of the 64 keys)
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // acc index r -> key 8*(r/4) + 4*g + r%4 inside the 32-key tile
                    int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    float v = s[kt][r] * scale_log2;
                    bool ok = (kt0 + kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3)) < tp.T && (!causal || key <= qglob);
                    v = ok ? v : -INFINITY;
                    s[kt][r] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            m_run = m_new;
            float lsum = 0.f;
            typedef _Float16 h8 __attribute__((ext_vector_type(8)));
            h8 pf[4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = __builtin_amdgcn_exp2f(s[kt][r] - m_use);
                    lsum += p;
                    pf[kt * 2 + (r >> 3)][r & 7] = (_Float16)p;
                }
            l_run = l_run * alpha + lsum;
#pragma unroll
            for (int i = 0; i < D / 32; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
            // ---- O^T += V^T P^T : 4 k-steps of 16 keys
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    h8 vf = *reinterpret_cast<const h8*>(Vt + (dt * 32 + lq) * AT_VPITCH + ks * 16 + 8 * g);
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[ks], oacc[dt], 0, 0, 0);
                }
            }
        }
    }
    // ---- finalize: O = acc / l ; lane holds O^T[d = 32*dt + 8j + 4g + r][query lq]
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    if (qrow < sg.S) {
        uint16_t* op = O + sg.o_off + (int64_t)tl.bh * sg.q_bhstride + (int64_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int d = dt * 32 + 8 * j + 4 * g;
                uint2 w;
                w.x = pack_bf16x2(oacc[dt][4 * j + 0] * inv, oacc[dt][4 * j + 1] * inv);
                w.y = pack_bf16x2(oacc[dt][4 * j + 2] * inv, oacc[dt][4 * j + 3] * inv);
                *reinterpret_cast<uint2*>(op + d) = w;
            }
    }
}

hipError_t launch_attention(const void* table, int64_t tiles_off, int32_t ntiles, int64_t segs_off,
                            int64_t tuples_off, const void* Q, const void* K, const void* V, void* O, float scale,
                            int32_t causal, hipStream_t stream) {
    const uint8_t* t = (const uint8_t*)table;
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL(attention_kernel, dim3(ntiles), dim3(256), 0, stream, (const AttnTile*)(t + tiles_off), ntiles,
                       (const AttnSeg*)(t + segs_off), (const AttnTuple*)(t + tuples_off), (const uint16_t*)Q,
                       (const uint16_t*)K, (const uint16_t*)V, (uint16_t*)O, scale_log2, causal);
    return hipGetLastError();
}

}  // namespace ja
