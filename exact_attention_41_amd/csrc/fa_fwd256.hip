// Exact-attention forward for head dimension 256 on gfx950.
//
// The method is that of the d = 64 / 128 forward: key/value tiles streamed
// through LDS ("FlashAttention" page, systems-analysis.ru, section "Tiling"),
// per-row running maximum and exp-sum (section "Online softmax"), products,
// mask and softmax fused in one kernel (section "Fusing into one CUDA
// kernel"), the output normalised once at the end and each wave owning whole
// query rows ("FlashAttention-2" page, systems-analysis.info, sections
// "1. Reducing non-matrix operations" and "3. Improved work partitioning
// within the block"). Head size 256 is the extension that the "FlashAttention"
// page (section "FlashAttention-2 (2023)") names among FlashAttention-2's.
//
// The register plan differs. A 32-row block of O^T is 32 x 256 fp32, 128
// registers per lane, and the resident Q^T fragments take 64 more, which does
// not fit two waves per SIMD. So each SIMD runs one wave (four per
// workgroup, 32 query rows each), O^T and Q^T live in AGPRs (their products
// are inline assembly), and the wave overlaps its own vector and matrix work:
//
//   iteration t:  mask and row maximum of S(t), rare rescale of O
//                 S(t+1) = K(t+1) Q^T    32 MFMAs, each followed by one element
//                                        of P(t) = exp2(S(t) c - m c) and its sums
//                 O^T += V(t)^T P(t)^T   32 MFMAs, with the transposed LDS
//                                        writes of V(t+1) between them
//
// K tiles reach LDS by global_load_lds two tiles ahead (row-major,
// swizzled); V tiles go through registers into the transposed [d][64 keys]
// layout one tile ahead, so every MFMA operand is a plain 16-byte LDS read,
// issued four MFMAs ahead. One workgroup barrier per tile.
#include "fa_kernels.hpp"
#include "fa_device.hpp"

namespace fa {

constexpr int kW256Waves = 4;
#ifndef FA_W256_AHEAD
#define FA_W256_AHEAD 4
#endif
constexpr int kW256Ahead = FA_W256_AHEAD;   // LDS fragment reads in flight ahead of the MFMAs
// The P V product takes fp16 operands, as in the d = 64 / 128 forward: P as
// fp16(2^7 P) (P <= 2^8 by the rescale rule, so 2^7 P stays in range) and V
// as fp16(2^-8 V) (exact for 2^-6 <= |v| < 65504 * 2^8; below, an absolute
// error of at most 2^-17); the epilogue takes both factors out again. With
// bf16 P the output's rounding moves D = dO . O of the backward by a few
// 1e-3 of |dO| |V| on short causal rows, enough to take dK past 1e-2.
constexpr float kP256Shift = 7.f;
constexpr float kV256Scale = 1.f / 256.f;
constexpr float kO256Scale = 256.f;

template <bool CAUSAL>
__global__ void __launch_bounds__(kW256Waves * 64, 1)
fwd_d256_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                uint16_t* __restrict__ ORes, float* __restrict__ LSE, int BH, int G, int N,
                int Nk, float c, int nqb) {
    constexpr int D = 256, BC = 64, NW = kW256Waves, BR = NW * 32;
    constexpr int KS = D / 16;            // MFMA k-steps over d
    constexpr int NB = D / 32;            // 32-wide blocks of the output columns
    constexpr int TB = BC * D * 2;        // 32 KiB: one tile of K, or of V^T
    constexpr int KPW = TB / 1024 / NW;   // 1 KB K staging blocks per wave
    constexpr int OFF_K = 0, OFF_V = TB, BUF = 2 * TB;
    constexpr int LA = kW256Ahead;
    constexpr int DCH = D / 8;            // 16-byte chunks per row
    constexpr int VU = 16 * DCH / (NW * 64);   // 4-key x 8-column V micro-tiles per thread
    __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;

    // Longest query blocks first (causal), heads fastest, and the XCD-aware
    // head numbering of the d = 64 / 128 forward: with BH a multiple of 8,
    // XCD x (workgroup id mod 8) runs the contiguous heads [x BH/8, (x+1) BH/8).
    const int bid = blockIdx.x;
    const int hh = bid % BH;
    const int bh = (BH & 7) ? hh : (hh & 7) * (BH >> 3) + (hh >> 3);
    const int qb_rank = bid / BH;
    const int qb = CAUSAL ? (nqb - 1 - qb_rank) : qb_rank;

    const size_t head = (size_t)bh * (size_t)N * D;
    const size_t kvhead = (size_t)(bh / G) * (size_t)Nk * D;
    const uint16_t* Qh = Q + head;
    const uint16_t* Kh = K + kvhead;
    const uint16_t* Vh = V + kvhead;
    const int q0 = qb * BR;
    const int wq0 = q0 + wave * 32;
    const int qi = wq0 + l32;             // this lane's query row
    const int off = Nk - N;               // query row i sits at position i + off

    // Q^T fragments (the B operand of S^T = K Q^T), parked in AGPRs. Rows past
    // the end read row N-1 (finite data, never stored).
    u32x4_t qf[KS];
    {
        const int qr = min(qi, N - 1);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[s] = *(const u32x4_t*)(Qh + (size_t)qr * D + 16 * s + 8 * g);
            park_in_agprs(qf[s]);
        }
    }

    const int n_all = (Nk + BC - 1) / BC;
    const int q_last = min(q0 + BR, N) - 1 + off;
    const int n_tiles = CAUSAL ? min(n_all, max(q_last, 0) / BC + 1) : n_all;

    // V tile t through registers: micro-tile u = tid + 256 k covers keys
    // 4 (u / DCH) .. +3 and columns 8 (u % DCH) .. +7; rows past Nk read row
    // Nk-1 (their probabilities are zero). Written transposed: column n of the
    // four keys is one 8-byte slot of row n of the [d][64 keys] tile.
    u32x4_t vreg[VU][4];
    auto v_load_part = [&](int t, int k, int rr) {
        const int u = tid + NW * 64 * k;
        const int ch = u % DCH, rg = u / DCH;
        const int j = min(t * BC + 4 * rg + rr, Nk - 1);
        vreg[k][rr] = *(const u32x4_t*)(Vh + (size_t)j * D + ch * 8);
    };
    auto v_store_part = [&](lds_char* vt, int k, int e) {
        const int u = tid + NW * 64 * k;
        const int ch = u % DCH, rg = u / DCH;
        const int slot = tr_key_position(4 * rg) >> 2;
        const int w = e >> 1;
        // bf16 pair -> fp16 pair of 2^-8 v, once per word (its two elements)
        if ((e & 1) == 0) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) vreg[k][rr][w] = bf16x2_to_f16x2(vreg[k][rr][w], kV256Scale);
        }
        const uint32_t r0 = vreg[k][0][w], r1 = vreg[k][1][w];
        const uint32_t r2 = vreg[k][2][w], r3 = vreg[k][3][w];
        u32x2_t col;
        if (e & 1) {
            col[0] = (r0 >> 16) | (r1 & 0xffff0000u);
            col[1] = (r2 >> 16) | (r3 & 0xffff0000u);
        } else {
            col[0] = (r0 & 0xffffu) | (r1 << 16);
            col[1] = (r2 & 0xffffu) | (r3 << 16);
        }
        *(__attribute__((address_space(3))) u32x2_t*)(vt + tr_slot_offset(ch * 8 + e, slot)) = col;
    };

    // Lane-dependent LDS bases; the rest of every fragment address is an
    // immediate offset. kbp[k]: K row l32, logical chunk 2k + g (chunks 16..31
    // are 256 B further, rows 32..63 16 KiB further); it starts at the buffer
    // of K(1). vbp[2 t4 + p]: V^T row 32 p + l32, key slot 4 t4 + 2 g (rows
    // 64 m further are 8 KiB m further); it starts at the buffer of V(0).
    lds_char* const s0 = (lds_char*)smem;
    lds_char* kbp[8];
    lds_char* vbp[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        kbp[k] = s0 + BUF + OFF_K + row_chunk_offset<D>(l32, 2 * k + g);
        vbp[k] = s0 + OFF_V + tr_slot_offset(32 * (k & 1) + l32, 4 * (k >> 1) + 2 * g);
    }
    auto k_frag = [&](int o, int shift) -> u32x4_t {   // product o of S: step o/2, key half o&1
        const int s = o >> 1, jb = o & 1;
        return *(const lds_u32x4_t*)(kbp[s & 7] + shift + (s >> 3) * 256 + jb * 16384);
    };
    auto v_frag = [&](int w) -> u32x4_t {               // product w of P V
        const int t4 = w / NB, nb = w % NB;
        return *(const lds_u32x4_t*)(vbp[2 * t4 + (nb & 1)] + (nb - (nb & 1)) * 4096);
    };

    const float thresh = kRescaleLog2 / c;
    float m_ref = kNegInf, l_run = 0.f, l_rnd = 0.f;
    f32x16_t acc_o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[nb][r] = 0.f;

    // ---- prologue: K(0), K(1), V(0) into LDS, then S(0) ---------------------
    stage_tile_lds<D, KPW, NW, false>(Kh, s0 + OFF_K, 0, Nk, wave, lane);
    stage_tile_lds<D, KPW, NW, false>(Kh, s0 + BUF + OFF_K, BC, Nk, wave, lane);
#pragma unroll
    for (int k = 0; k < VU; ++k)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) v_load_part(0, k, rr);
#pragma unroll
    for (int k = 0; k < VU; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) v_store_part(s0 + OFF_V, k, e);
    __syncthreads();

    f32x16_t sa[2], sb[2];
    {
        u32x4_t fr[LA + 1];
#pragma unroll
        for (int o = 0; o < LA; ++o) fr[o] = k_frag(o, -BUF);
#pragma unroll
        for (int o = 0; o < 2 * KS; ++o) {
            if (o + LA < 2 * KS) fr[(o + LA) % (LA + 1)] = k_frag(o + LA, -BUF);
            const int s = o >> 1, jb = o & 1;
            const u32x4_t a = fr[o % (LA + 1)];
            if (s == 0) mfma_bf16_first(sa[jb], a, qf[s]);
            else if (s == KS - 1) mfma_bf16_last(sa[jb], a, qf[s]);
            else mfma_bf16_next(sa[jb], a, qf[s]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();                       // K(0)'s buffer is free for K(2)

    // Mask of S(t) in place (only tiles that cross Nk or reach past this
    // wave's first row; idempotent) and the row maximum.
    auto mask_max = [&](int t, f32x16_t (&sc)[2]) -> float {
        const int kv0 = t * BC;
        if (kv0 + BC > Nk || (CAUSAL && kv0 + BC - 1 > wq0 + off)) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = kv0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (j >= Nk || (CAUSAL && j > qi + off)) sc[jb][r] = kNegInf;
                }
        }
        float m = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, sc[jb][r]);
        return max_with_partner32(m);
    };
    // Move the reference maximum up to mt and rescale what has been
    // accumulated by exp2((m_old - m_new) c). The only vector-unit access to
    // the AGPR accumulator: it runs outside the tile loop, so that the loop
    // never copies the accumulator out of the AGPRs.
    auto rescale = [&](float mt) {
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = (m_ref == kNegInf) ? 0.f : fast_exp2((m_ref - m_new) * c);
        l_run *= alpha;
        l_rnd *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            agpr_settle(acc_o[nb]);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[nb][r] *= alpha;
        }
        m_ref = m_new;
    };

    // ---- the products and the softmax of one key tile -------------------------
    auto tile_body = [&](int t, f32x16_t (&sc)[2], f32x16_t (&sn)[2], auto next_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;   // S(t+1) and V(t+1) exist
        constexpr int NS = NEXT ? 2 * KS : 0;
        constexpr int NOPS = NS + 4 * NB;
        auto frag = [&](int o) -> u32x4_t { return o < NS ? k_frag(o, 0) : v_frag(o - NS); };
        u32x4_t fr[LA + 1];
#pragma unroll
        for (int o = 0; o < LA; ++o) fr[o] = frag(o);
        // exp2(s c - m_ref c + 7) = 2^7 P
        const float mc = ((m_ref == kNegInf) ? 0.f : m_ref * c) - kP256Shift;

        // Element e of P(t) (times 2^7): key half e/16, accumulator register e%16.
        float pv[16];
        u32x4_t pf[4];
        auto p_elem = [&](int e) {
            const int jb = e >> 4, r = e & 15;
            pv[r] = fast_exp2(__builtin_fmaf(sc[jb][r], c, -mc));
            l_run += pv[r];
            if ((r & 7) == 7) {
                const int t4 = e >> 3, rb = r - 7;
                pf[t4] = u32x4_t{pack_f16x2(pv[rb + 0], pv[rb + 1]), pack_f16x2(pv[rb + 2], pv[rb + 3]),
                                 pack_f16x2(pv[rb + 4], pv[rb + 5]), pack_f16x2(pv[rb + 6], pv[rb + 7])};
                // O is normalised by the sum of the fp16 probabilities that
                // multiply V (the rounding error of P then scales with
                // v_j - O); lse uses the fp32 sum.
#pragma unroll
                for (int w = 0; w < 4; ++w) l_rnd = add_f16x2(pf[t4][w], l_rnd);
                // The sums are used from the next tile on: keep their
                // computation between the products of this one.
                keep_here(l_run);
                keep_here(l_rnd);
            }
        };
        if (!NEXT) {
#pragma unroll
            for (int e = 0; e < 32; ++e) p_elem(e);
        }

        lds_char* const kdst = s0 + (t & 1) * BUF + OFF_K;         // K(t+2)
        lds_char* const vdst = s0 + ((t + 1) & 1) * BUF + OFF_V;   // V(t+1)
        const int k2 = (t + 2) * BC;
#pragma unroll
        for (int o = 0; o < NOPS; ++o) {
            if (o + LA < NOPS) fr[(o + LA) % (LA + 1)] = frag(o + LA);
            const u32x4_t a = fr[o % (LA + 1)];
            if (o < NS) {
                const int s = o >> 1, jb = o & 1;
                if (s == 0) mfma_bf16_first(sn[jb], a, qf[s]);
                else if (s == KS - 1) mfma_bf16_last(sn[jb], a, qf[s]);
                else mfma_bf16_next(sn[jb], a, qf[s]);
                p_elem(o);
                // K(t+2) into LDS (past the last tile: rows Nk-1, never read),
                // then V(t+1) into registers. The first transposed write of
                // V(t+1) waits for all of them, a whole S phase later.
                if (o < KPW) stage_tile_block<D>(Kh, kdst, k2, Nk, wave + NW * o, lane);
                else if (o < KPW + 4 * VU) v_load_part(t + 1, (o - KPW) >> 2, (o - KPW) & 3);
            } else {
                const int w = o - NS, t4 = w / NB, nb = w % NB;
                mfma_f16_agpr(acc_o[nb], a, pf[t4]);
                if (NEXT && (w & 1) == 0 && (w >> 1) < 8 * VU)
                    v_store_part(vdst, (w >> 1) >> 3, (w >> 1) & 7);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // Next tile: K(t+2) sits in the buffer K(t) left, V(t+1) in the other.
        const int kstep = (t & 1) ? BUF : -BUF;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            kbp[k] += kstep;
            vbp[k] -= kstep;
        }
        __syncthreads();   // loads landed, writes visible, every wave done with tile t
    };

    // Tiles 0 .. n_tiles-2, then the last. A row whose tile maximum exceeds
    // its reference by more than the threshold while it has no keys yet
    // (O = 0, l = 0) just takes the new reference. Should a row that holds a
    // sum need it, the rest of the tiles run in a second copy of the loop
    // that rescales O where needed; the first loop never touches O with the
    // vector unit, so O stays in the AGPRs there.
    int t = 0;
    bool rare = false;
    for (; t + 1 < n_tiles; ++t) {
        const float mt = mask_max(t, sa);
        const bool up = mt > m_ref + thresh;
        if (__any(up && m_ref != kNegInf)) {
            rare = true;
            break;
        }
        if (up) m_ref = mt;
        tile_body(t, sa, sb, BoolTag<true>{});
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) sa[jb] = sb[jb];
    }
    if (rare) {
        for (; t + 1 < n_tiles; ++t) {
            const float mt = mask_max(t, sa);
            if (__any(mt > m_ref + thresh)) rescale(mt);
            tile_body(t, sa, sb, BoolTag<true>{});
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) sa[jb] = sb[jb];
        }
    }
    {
        const float mt = mask_max(t, sa);
        if (__any(mt > m_ref + thresh)) rescale(mt);
        tile_body(t, sa, sb, BoolTag<false>{});
    }

    // ---- epilogue: deferred normalisation, logsumexp, bf16 store (and, when
    // ORes is given, the bf16 rounding residual of each stored value) --------
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) agpr_settle(acc_o[nb]);
    const float l = sum_with_partner32(l_run);
    const float lr = sum_with_partner32(l_rnd);
    const float inv = (lr > 0.f) ? kO256Scale / lr : 0.f;
    if (qi < N && g == 0) {
        const float mc = (m_ref == kNegInf) ? 0.f : m_ref * c;
        LSE[(size_t)bh * N + qi] = (l > 0.f) ? (mc + (fast_log2(l) - kP256Shift)) * kLn2 : kNegInf;
    }
    // O goes out through LDS: each wave writes its 32 rows (16 KiB) into its
    // quarter of the first 64 KiB (16-byte chunks of a row swizzled by the
    // row), then stores whole rows, consecutive lanes taking consecutive
    // 16-byte chunks. Every copy into the buffers (the last K staging reaches
    // past the final tile) has landed and every read of them is done first.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __syncthreads();
    constexpr int RB = D * 2;              // bytes per row
    constexpr int CH = RB / 16;            // 16-byte chunks per row
    lds_char* const region = s0 + wave * 32 * RB;
    auto put = [&](bool residual) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = acc_o[nb][4 * q4 + e] * inv;
                u32x2_t w;
                w[0] = pack_bf16x2(x[0], x[1]);
                w[1] = pack_bf16x2(x[2], x[3]);
                if (residual) {
                    w[0] = pack_bf16x2_residual(x[0], x[1], w[0]);
                    w[1] = pack_bf16x2_residual(x[2], x[3], w[1]);
                }
                const int ch = 4 * nb + q4;    // columns 32 nb + 8 q4 .. +7
                *(__attribute__((address_space(3))) u32x2_t*)(
                    region + l32 * RB + ((ch ^ (l32 & (CH - 1))) * 16) + 8 * g) = w;
            }
    };
    auto out = [&](uint16_t* __restrict__ dst) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
        for (int i = 0; i < 32 * CH / 64; ++i) {
            const int idx = i * 64 + lane, row = idx / CH, ch = idx % CH;
            const u32x4_t v = *(const __attribute__((address_space(3))) u32x4_t*)(
                region + row * RB + ((ch ^ (row & (CH - 1))) * 16));
            if (wq0 + row < N) *(u32x4_t*)(dst + head + (size_t)(wq0 + row) * D + 8 * ch) = v;
        }
    };
    put(false);
    out(O);
    if (ORes != nullptr) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        put(true);
        out(ORes);
    }
}

template <bool CAUSAL>
static hipError_t launch_fwd_d256_t(const FwdArgs& a) {
    constexpr int BR = kW256Waves * 32;
    const int BH = a.B * a.H;
    const int nqb = (a.N + BR - 1) / BR;
    hipLaunchKernelGGL((fwd_d256_kernel<CAUSAL>), dim3(nqb * BH), dim3(kW256Waves * 64), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.o, (uint16_t*)a.o_res, a.lse, BH, a.H / a.Hkv, a.N, a.Nk,
                       a.scale * kLog2e, nqb);
    return hipGetLastError();
}

hipError_t launch_fwd_d256(const FwdArgs& a) {
    return a.causal ? launch_fwd_d256_t<true>(a) : launch_fwd_d256_t<false>(a);
}

}  // namespace fa
