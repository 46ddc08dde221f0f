// Exact-attention forward with 8-bit floating-point operands (OCP e4m3) for
// gfx950, head dimension 128.
//
// The "FlashAttention" page (systems-analysis.ru, section "FlashAttention-2
// (2023)") and the "FlashAttention-2" page (systems-analysis.info, section
// "Comparison with later versions / FlashAttention-3") name FP8 arithmetic
// among the FlashAttention-3 changes. Here
// q, k and v are stored as e4m3 with one dequantisation factor per tensor
// (real value = descale * stored value); both products run on the fp8 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales, fp32
// accumulation), the softmax statistics stay fp32, the probabilities enter
// the P V product as e4m3, and O is written as bf16.
//
// Method and schedule are those of the bf16 forward: tiles streamed through
// LDS, online softmax with a lagging reference maximum, normalisation at the
// end, 8 waves of 32 query rows in two groups that alternate a matrix slot
// (S(t) = K(t) Q^T and O += V(t-1)^T P(t-1)) and a vector slot (mask, max,
// exp2, fp8 packing). Differences:
//   * one MFMA covers 64 contraction elements: S^T takes 2 key halves x 2
//     steps over d, O^T += V^T P^T one product per 32 output columns;
//   * every operand fragment is 32 bytes per lane (two 16-byte LDS reads);
//   * the probabilities are scaled by 2^kP8Shift with a rescale threshold of
//     2^kP8Threshold (their sum stays within e4m3's 448 and typical values
//     stay in its normal range);
//   * O is normalised by the sum of the e4m3 probabilities that multiplied V,
//     taken by one more MFMA per tile (an all-ones block times P^T) instead of
//     vector instructions; lse uses the fp32 sum of the unrounded ones.
#include "fa_kernels.hpp"
#include "fa_device.hpp"

namespace fa {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;

constexpr int kFp8Waves = 8;
constexpr float kP8Threshold = 4.f;   // log2 units
constexpr float kP8Shift = 4.f;       // probabilities carry 2^kP8Shift

// D(32x32,f32) += A(32x64,e4m3) * B(64x32,e4m3): lane l supplies row (A) or
// column (B) l % 32 and 32 consecutive-in-register contraction elements for
// lane group l / 32 (A and B use the same assignment); accumulator layout as
// for the bf16 product.
__device__ __forceinline__ f32x16_t mfma_fp8(const i32x8_t& a, const i32x8_t& b,
                                             const f32x16_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7f7f7f7f, 0,
                                                           0x7f7f7f7f);
}

// K tile in LDS: 64 keys x 128 bytes, the row-major layout (and swizzle) of a
// [64][64] bf16 tile, so the bf16 staging helpers fill it. A fragment is the
// 32 bytes [64 s + 32 g, +32) of row `row`: logical chunks 4 s + 2 g and +1.
__device__ __forceinline__ i32x8_t k_frag8(const lds_char* tile, int row, int s, int g) {
    const u32x4_t lo = *(const lds_u32x4_t*)(tile + row_chunk_offset<64>(row, 4 * s + 2 * g));
    const u32x4_t hi = *(const lds_u32x4_t*)(tile + row_chunk_offset<64>(row, 4 * s + 2 * g + 1));
    return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// V^T tile in LDS: row n (output column) holds the 64 keys of the tile as
// bytes, key 32 jb + 8 a + 4 g + c at position 32 g + 16 jb + 4 a + c, so
// that the 32 keys one lane group's probabilities cover (two S^T
// accumulators) are one 32-byte run; 16-byte chunks XORed with (n >> 2) & 3.
__device__ __forceinline__ int vt8_swizzle(int n) { return (n >> 2) & 3; }
__device__ __forceinline__ int vt8_offset(int n, int pos) {
    return n * 64 + (((pos >> 4) ^ vt8_swizzle(n)) << 4) + (pos & 15);
}
__device__ __forceinline__ i32x8_t vt_frag8(const lds_char* tile, int n, int g) {
    const u32x4_t lo = *(const lds_u32x4_t*)(tile + vt8_offset(n, 32 * g));
    const u32x4_t hi = *(const lds_u32x4_t*)(tile + vt8_offset(n, 32 * g + 16));
    return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Four floats -> four e4m3 bytes (round to nearest even), x0 in the low byte.
__device__ __forceinline__ int pack_fp8x4(float x0, float x1, float x2, float x3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

__device__ __forceinline__ void wg_barrier8() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <bool CAUSAL>
__global__ void __launch_bounds__(kFp8Waves * 64, 1)
fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
               const uint8_t* __restrict__ V, uint16_t* __restrict__ O,
               float* __restrict__ LSE, int BH, int G, int N, int Nk, float c, float o_scale,
               int nqb) {
    constexpr int D = 128;
    constexpr int BC = 64;                 // keys per tile
    constexpr int BR = kFp8Waves * 32;     // query rows per workgroup
    constexpr int KS = D / 64;             // MFMA steps over d
    constexpr int NB = D / 32;             // 32-wide blocks of the output columns
    constexpr int TILE = BC * D;           // bytes of a K or V^T tile (8 KiB)
    constexpr int BLOCKS = TILE / 1024;

    __shared__ __attribute__((aligned(16))) char kb0[TILE], kb1[TILE], vb0[TILE], vb1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;             // 0: group A, 1: group B
    const int g = lane >> 5;
    const int l32 = lane & 31;

    // Longest query blocks first (causal), heads fastest, XCD-aware head order
    // (as in the bf16 forward).
    const int bid = blockIdx.x;
    const int hh = bid % BH;
    const int bh = (BH & 7) ? hh : (hh & 7) * (BH >> 3) + (hh >> 3);
    const int qb_rank = bid / BH;
    const int qb = CAUSAL ? (nqb - 1 - qb_rank) : qb_rank;

    const size_t head = (size_t)bh * (size_t)N * D;
    const size_t kvhead = (size_t)(bh / G) * (size_t)Nk * D;
    const uint8_t* Qh = Q + head;
    const uint8_t* Kh = K + kvhead;
    const uint8_t* Vh = V + kvhead;
    const int q0 = qb * BR;
    const int wq0 = q0 + wave * 32;
    const int qi = wq0 + l32;
    const int off = Nk - N;                // query row i sits at position i + off

    // Q^T fragments: bytes [64 s + 32 g, +32) of this lane's row.
    i32x8_t qf[KS];
    {
        const int qr = min(qi, N - 1);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4_t lo = *(const u32x4_t*)(Qh + (size_t)qr * D + 64 * s + 32 * g);
            const u32x4_t hi = *(const u32x4_t*)(Qh + (size_t)qr * D + 64 * s + 32 * g + 16);
            qf[s] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    }

    const int n_all = (Nk + BC - 1) / BC;
    const int q_last = min(q0 + BR, N) - 1 + off;
    const int n_tiles = CAUSAL ? min(n_all, max(q_last, 0) / BC + 1) : n_all;

    auto Kb = [&](int i) { return i ? (lds_char*)kb1 : (lds_char*)kb0; };
    auto Vb = [&](int i) { return i ? (lds_char*)vb1 : (lds_char*)vb0; };

    const float thresh = kP8Threshold / c;
    float m_ref = kNegInf, l_run = 0.f;
    f32x16_t acc_o[NB], acc_l, acc_s[2];
    i32x8_t pf = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    const i32x8_t ones = i32x8_t{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                                 0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        acc_l[r] = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc_o[nb][r] = 0.f;
    }

    // V(t) through registers into the transposed tile: unit u (of 16 x 32)
    // is 4 keys (4 (u / 32) ..) x 4 columns (4 (u % 32) ..); each group moves
    // half of the units, loading them in its matrix slot and writing them in
    // its next vector slot. Rows past Nk read row Nk-1 (masked keys).
    uint32_t vreg[4];
    const int vu = grp * 256 + (wave & 3) * 64 + lane;
    const int v_cg = vu % 32, v_kg = vu / 32;
    auto v_load = [&](int t) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int j = min(t * BC + 4 * v_kg + rr, Nk - 1);
            vreg[rr] = *(const uint32_t*)(Vh + (size_t)j * D + 4 * v_cg);
        }
    };
    auto v_store = [&](int t) {
        lds_char* vl = Vb(t & 1);
        // position of key 4 v_kg = 32 jb + 8 a + 4 g': 32 g' + 16 jb + 4 a
        const int pos = 32 * (v_kg & 1) + 16 * (v_kg >> 3) + 4 * ((v_kg >> 1) & 3);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t w = ((vreg[0] >> (8 * b)) & 0xffu) |
                               (((vreg[1] >> (8 * b)) & 0xffu) << 8) |
                               (((vreg[2] >> (8 * b)) & 0xffu) << 16) |
                               (((vreg[3] >> (8 * b)) & 0xffu) << 24);
            *(__attribute__((address_space(3))) uint32_t*)(vl + vt8_offset(4 * v_cg + b, pos)) = w;
        }
    };

    // Matrix slot of tile t: S(t) = K(t) Q^T (4 products) and
    // O += V(t-1)^T P(t-1), l += 1 P(t-1) (5 products). In the first slot P = 0
    // and the V buffer holds zeros; in the last one S is discarded.
    auto matrix_slot = [&](int t) {
        __builtin_amdgcn_s_setprio(1);
        const lds_char* kt = Kb(t & 1);
        const lds_char* vt = Vb((t + 1) & 1);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_s[jb][r] = 0.f;
        constexpr int NS = 2 * KS, NP = NB + 1;
#pragma unroll
        for (int x = 0; x < (NS > NP ? NS : NP); ++x) {
            if (x < NS) {
                const int s = x >> 1, jb = x & 1;
                acc_s[jb] = mfma_fp8(k_frag8(kt, 32 * jb + l32, s, g), qf[s], acc_s[jb]);
            }
            if (x < NB) acc_o[x] = mfma_fp8(vt_frag8(vt, 32 * x + l32, g), pf, acc_o[x]);
            else if (x == NB) acc_l = mfma_fp8(ones, pf, acc_l);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    };

    // Vector slot of tile t: softmax of S(t) into P(t).
    auto vector_slot = [&](int t) {
        const int kv0 = t * BC;
        if ((kv0 + BC > Nk) || (CAUSAL && kv0 + BC - 1 > wq0 + off)) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = kv0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
                    if ((j >= Nk) || (CAUSAL && j > qi + off)) acc_s[jb][r] = kNegInf;
                }
        }
        float m = fmaxf(acc_s[0][0], acc_s[1][0]);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, acc_s[jb][r]);
        const float mt = max_with_partner32(m);
        if (__any(mt > m_ref + thresh)) {
            const float m_new = fmaxf(m_ref, mt);
            const float alpha = (m_ref == kNegInf) ? 0.f : fast_exp2((m_ref - m_new) * c);
            l_run *= alpha;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc_l[r] *= alpha;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc_o[nb][r] *= alpha;
            }
            m_ref = m_new;
        }
        // p = 2^shift exp2((s - m_ref) c) <= 2^(shift + threshold) = 256.
        const float mc = (m_ref == kNegInf) ? 0.f : m_ref * c - kP8Shift;
        // Byte e = 16 jb + r of this lane's 32 probabilities is accumulator
        // register r of key half jb (key 32 jb + 8 (r / 4) + 4 g + r % 4).
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p[e] = fast_exp2(__builtin_fmaf(acc_s[jb][4 * q4 + e], c, -mc));
                    l_run += p[e];
                }
                pf[4 * jb + q4] = pack_fp8x4(p[0], p[1], p[2], p[3]);
            }
    };

    // ---- prologue: K(0) into LDS, zeros into the V buffer of "tile -1" -----
    if (grp == 0)
        stage_tile_lds<64, BLOCKS / 4, 4, false>((const uint16_t*)Kh, Kb(0), 0, Nk, wave, lane);
    for (int i = tid; i < TILE / 16; i += kFp8Waves * 64)
        *(__attribute__((address_space(3))) u32x4_t*)(Vb(1) + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
    __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0)
    __syncthreads();
    if (grp == 1) {                        // group B runs one slot behind
        v_load(0);
        v_store(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        wg_barrier8();
    }

    // Slot 2t: A matrix(t), B vector(t-1); slot 2t+1: A vector(t), B matrix(t).
    for (int t = 0; t <= n_tiles; ++t) {
        matrix_slot(t);
        if (t < n_tiles) {
            if (grp == 0) {
                if (t + 1 < n_tiles)
                    stage_tile_lds<64, BLOCKS / 4, 4, false>((const uint16_t*)Kh, Kb((t + 1) & 1),
                                                             (t + 1) * BC, Nk, wave, lane);
                v_load(t);
            } else if (t + 1 < n_tiles) {
                v_load(t + 1);
            }
        }
        wg_barrier8();
        if (t < n_tiles) {
            vector_slot(t);
            if (grp == 0) v_store(t);
            else if (t + 1 < n_tiles) v_store(t + 1);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            // Group A's V(t) is read right after this barrier: its writes must
            // be complete (lgkmcnt(0)). Group B's V(t+1) is first read two
            // barriers on, after the LDS wait that ends B's next matrix slot.
            if (grp == 0) __builtin_amdgcn_s_waitcnt(0xC07F);
            wg_barrier8();
        }
    }
    if (grp == 0) wg_barrier8();           // same number of barriers in both groups

    // ---- epilogue: normalisation by the e4m3 weights, lse, bf16 store ------
    const float l = sum_with_partner32(l_run);
    const float lr = acc_l[0];             // every row of the ones product is the sum
    if (qi < N) {
        const float inv = (lr > 0.f) ? o_scale / lr : 0.f;
        const float mc = (m_ref == kNegInf) ? 0.f : m_ref * c - kP8Shift;
        if (g == 0)
            LSE[(size_t)bh * N + qi] = (l > 0.f) ? (mc + fast_log2(l)) * kLn2 : kNegInf;
        uint16_t* orow = O + (size_t)bh * N * D + (size_t)qi * D;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                u32x2_t w;
                w[0] = pack_bf16x2(acc_o[nb][4 * q4 + 0] * inv, acc_o[nb][4 * q4 + 1] * inv);
                w[1] = pack_bf16x2(acc_o[nb][4 * q4 + 2] * inv, acc_o[nb][4 * q4 + 3] * inv);
                *(u32x2_t*)(orow + 32 * nb + 8 * q4 + 4 * g) = w;
            }
    }
}

template <bool CAUSAL>
static hipError_t launch_fwd_fp8_t(const FwdArgs& a) {
    constexpr int BR = kFp8Waves * 32;
    const int BH = a.B * a.H;
    const int nqb = (a.N + BR - 1) / BR;
    const float c = a.scale * a.descale_q * a.descale_k * kLog2e;
    hipLaunchKernelGGL((fwd_fp8_kernel<CAUSAL>), dim3(nqb * BH), dim3(kFp8Waves * 64), 0,
                       a.stream, (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v,
                       (uint16_t*)a.o, a.lse, BH, a.H / a.Hkv, a.N, a.Nk, c, a.descale_v, nqb);
    return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdArgs& a) {
    return a.causal ? launch_fwd_fp8_t<true>(a) : launch_fwd_fp8_t<false>(a);
}

}  // namespace fa
