// Fused exact-attention forward kernels for gfx950.
//
// One workgroup owns a block of query rows of one (batch, head) and streams
// the keys and values through LDS tile by tile ("FlashAttention" page,
// systems-analysis.ru, section "Tiling"), keeping for every query row the
// running maximum and running sum of exponentials (section "Online softmax"),
// with the product Q K^T, the mask, the softmax and the product with V fused
// in one kernel (section "Fusing into one CUDA kernel"). The output is
// normalised once at the end instead of after every tile, and each wavefront
// owns whole query rows so that the row statistics never leave its registers
// ("FlashAttention-2" page, systems-analysis.info, sections "1. Reducing
// non-matrix operations" and "3. Improved work partitioning within the
// block"); the grid spreads the query blocks of one head over many compute
// units (section "2. Improved parallelism").
#include "fa_kernels.hpp"
#include "fa_device.hpp"

namespace fa {

// ---------------------------------------------------------------------------
// bf16 forward.
//
// Per wave: IB blocks of 32 query rows. Per iteration: a tile of 64 keys.
//   S^T (keys x queries) = K * Q^T      A = K tile from LDS, B = Q^T in VGPRs
//   P^T = exp2(S^T*c - m*c)             column i of S^T sits in one lane pair
//   O^T (d x queries)   += V^T * P^T    A = V^T from LDS, B = P^T from the
//                                        S^T accumulators, rounded to bf16
// Computing the transposed products puts one query row per lane (pair), so the
// row max, row sum and the rescaling of O need no cross-lane traffic except
// one v_permlane32_swap per row and tile.
// ---------------------------------------------------------------------------
template <int D, int IB, int NW, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64, 1)
fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                float* __restrict__ LSE, int BH, int N, float c, int nqb) {
    constexpr int BC = 64;                 // keys per tile
    constexpr int NT = NW * 64;            // threads per workgroup
    constexpr int BR = NW * IB * 32;       // query rows per workgroup
    constexpr int DCH = D / 8;             // 16-byte chunks per row
    constexpr int KS = D / 16;             // MFMA k-steps over d
    constexpr int NB = D / 32;             // 32-wide blocks of the output columns
    constexpr int KT_BYTES = BC * D * 2;
    constexpr int VT_BYTES = D * BC * 2;
    constexpr int BUF_BYTES = KT_BYTES + VT_BYTES;
    constexpr int K_LOADS = BC * DCH / NT;             // 16-byte K chunks per thread
    constexpr int V_UNITS = (BC / 4) * DCH;            // 4-key x 8-column V micro-tiles
    constexpr int V_LOADS = (V_UNITS + NT - 1) / NT;
    static_assert(BC * DCH % NT == 0, "K tile must split evenly over the threads");

    __shared__ __attribute__((aligned(16))) char smem[2 * BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 5;
    const int l32 = lane & 31;

    // Longest query blocks first (causal), heads fastest: consecutive
    // workgroup ids take different heads, so with the round-robin dispatch over
    // the eight XCDs every XCD keeps to a fixed subset of heads and their K/V
    // stays in that XCD's L2.
    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb_rank = bid / BH;
    const int qb = CAUSAL ? (nqb - 1 - qb_rank) : qb_rank;

    const size_t head = (size_t)bh * (size_t)N * D;
    const uint16_t* Qh = Q + head;
    const uint16_t* Kh = K + head;
    const uint16_t* Vh = V + head;
    const int q0 = qb * BR;
    const int wq0 = q0 + wave * IB * 32;

    // Q^T operand fragments, resident for the whole kernel.
    u32x4_t qf[IB][KS];
#pragma unroll
    for (int ib = 0; ib < IB; ++ib) {
        const int qi = wq0 + 32 * ib + l32;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (qi < N)
                qf[ib][s] = *(const u32x4_t*)(Qh + (size_t)qi * D + 16 * s + 8 * g);
            else
                qf[ib][s] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }

    const int n_all = (N + BC - 1) / BC;
    const int q_last = min(q0 + BR, N) - 1;
    const int n_tiles = CAUSAL ? min(n_all, q_last / BC + 1) : n_all;

    u32x4_t kreg[K_LOADS];
    u32x4_t vreg[V_LOADS][4];

    auto load_tile = [&](int kv0) {
#pragma unroll
        for (int it = 0; it < K_LOADS; ++it) {
            const int cidx = tid + it * NT;
            const int row = cidx / DCH, ch = cidx % DCH;
            const int j = kv0 + row;
            kreg[it] = (j < N) ? *(const u32x4_t*)(Kh + (size_t)j * D + ch * 8)
                               : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < V_LOADS; ++it) {
            const int u = tid + it * NT;
            if (V_UNITS % NT == 0 || u < V_UNITS) {
                const int ch = u % DCH, rg = u / DCH;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int j = kv0 + 4 * rg + rr;
                    vreg[it][rr] = (j < N) ? *(const u32x4_t*)(Vh + (size_t)j * D + ch * 8)
                                           : u32x4_t{0u, 0u, 0u, 0u};
                }
            }
        }
    };

    auto store_tile = [&](int buf) {
        char* kl = smem + buf * BUF_BYTES;
        char* vl = kl + KT_BYTES;
#pragma unroll
        for (int it = 0; it < K_LOADS; ++it) {
            const int cidx = tid + it * NT;
            const int row = cidx / DCH, ch = cidx % DCH;
            *(u32x4_t*)(kl + row_chunk_offset<D>(row, ch)) = kreg[it];
        }
#pragma unroll
        for (int it = 0; it < V_LOADS; ++it) {
            const int u = tid + it * NT;
            if (V_UNITS % NT == 0 || u < V_UNITS) {
                const int ch = u % DCH, rg = u / DCH;
                const int slot = tr_key_position(4 * rg) >> 2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int w = e >> 1;
                    const uint32_t r0 = vreg[it][0][w], r1 = vreg[it][1][w];
                    const uint32_t r2 = vreg[it][2][w], r3 = vreg[it][3][w];
                    u32x2_t col;
                    if (e & 1) {
                        col[0] = (r0 >> 16) | (r1 & 0xffff0000u);
                        col[1] = (r2 >> 16) | (r3 & 0xffff0000u);
                    } else {
                        col[0] = (r0 & 0xffffu) | (r1 << 16);
                        col[1] = (r2 & 0xffffu) | (r3 << 16);
                    }
                    *(u32x2_t*)(vl + tr_slot_offset(ch * 8 + e, slot)) = col;
                }
            }
        }
    };

    float m_run[IB], l_run[IB];
    f32x16_t acc_o[NB][IB];
#pragma unroll
    for (int ib = 0; ib < IB; ++ib) {
        m_run[ib] = kNegInf;
        l_run[ib] = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[nb][ib][r] = 0.f;
    }

    load_tile(0);
    store_tile(0);
    __syncthreads();

    const int wave_last = wq0 + IB * 32 - 1;
    for (int t = 0; t < n_tiles; ++t) {
        const int kv0 = t * BC;
        if (t + 1 < n_tiles) load_tile(kv0 + BC);
        const char* kl = smem + (t & 1) * BUF_BYTES;
        const char* vl = kl + KT_BYTES;

        if (!CAUSAL || kv0 <= wave_last) {
            // ---- S^T = K Q^T -------------------------------------------------
            f32x16_t acc_s[2][IB];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc_s[jb][ib][r] = 0.f;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const u32x4_t kf =
                        *(const u32x4_t*)(kl + row_chunk_offset<D>(32 * jb + l32, 2 * s + g));
#pragma unroll
                    for (int ib = 0; ib < IB; ++ib)
                        acc_s[jb][ib] = mfma_32x32x16(kf, qf[ib][s], acc_s[jb][ib]);
                }
            }

            // ---- mask: keys past the end, and keys after the query (causal) --
            const bool need_mask = (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > wq0);
            if (need_mask) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int ib = 0; ib < IB; ++ib) {
                        const int qi = wq0 + 32 * ib + l32;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int j = kv0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
                            const bool masked = (j >= N) || (CAUSAL && j > qi);
                            if (masked) acc_s[jb][ib][r] = kNegInf;
                        }
                    }
            }

            // ---- online softmax (one query row per lane pair) -----------------
            u32x4_t pf[IB][4];
#pragma unroll
            for (int ib = 0; ib < IB; ++ib) {
                float mt = acc_s[0][ib][0];
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, acc_s[jb][ib][r]);
                mt = max_with_partner32(mt);
                const float m_new = fmaxf(m_run[ib], mt);
                const float m_use = (m_new == kNegInf) ? 0.f : m_new;
                const float alpha =
                    (m_run[ib] == kNegInf) ? 0.f : fast_exp2((m_run[ib] - m_use) * c);
                const float mc = m_use * c;
                float ls = 0.f;
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = fast_exp2(__builtin_fmaf(acc_s[jb][ib][r], c, -mc));
                        acc_s[jb][ib][r] = p;
                        ls += p;
                    }
                l_run[ib] = l_run[ib] * alpha + ls;
                m_run[ib] = m_new;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc_o[nb][ib][r] *= alpha;
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) {
                    const int jb = t4 >> 1, rb = 8 * (t4 & 1);
                    pf[ib][t4] = u32x4_t{pack_bf16x2(acc_s[jb][ib][rb + 0], acc_s[jb][ib][rb + 1]),
                                         pack_bf16x2(acc_s[jb][ib][rb + 2], acc_s[jb][ib][rb + 3]),
                                         pack_bf16x2(acc_s[jb][ib][rb + 4], acc_s[jb][ib][rb + 5]),
                                         pack_bf16x2(acc_s[jb][ib][rb + 6], acc_s[jb][ib][rb + 7])};
                }
            }

            // ---- O^T += V^T P^T ----------------------------------------------
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const u32x4_t vf =
                        *(const u32x4_t*)(vl + tr_slot_offset(32 * nb + l32, 4 * t4 + 2 * g));
#pragma unroll
                    for (int ib = 0; ib < IB; ++ib)
                        acc_o[nb][ib] = mfma_32x32x16(vf, pf[ib][t4], acc_o[nb][ib]);
                }
            }
        }

        if (t + 1 < n_tiles) store_tile((t + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: deferred normalisation, logsumexp, bf16 store ------------
#pragma unroll
    for (int ib = 0; ib < IB; ++ib) {
        const float l = sum_with_partner32(l_run[ib]);
        const int qi = wq0 + 32 * ib + l32;
        if (qi < N) {
            const float inv = (l > 0.f) ? 1.f / l : 0.f;
            const float m_use = (m_run[ib] == kNegInf) ? 0.f : m_run[ib];
            if (g == 0)
                LSE[(size_t)bh * N + qi] = (l > 0.f) ? (m_use * c + fast_log2(l)) * kLn2 : kNegInf;
            uint16_t* orow = O + head + (size_t)qi * D;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    u32x2_t w;
                    w[0] = pack_bf16x2(acc_o[nb][ib][4 * q4 + 0] * inv, acc_o[nb][ib][4 * q4 + 1] * inv);
                    w[1] = pack_bf16x2(acc_o[nb][ib][4 * q4 + 2] * inv, acc_o[nb][ib][4 * q4 + 3] * inv);
                    *(u32x2_t*)(orow + 32 * nb + 8 * q4 + 4 * g) = w;
                }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 forward: fp32 operands and fp32 FMA arithmetic throughout.
// SPLIT = D/64 lanes share one query row, each holding 64 of its columns;
// a wave owns 64/SPLIT rows and walks the keys in tiles of 32 staged in LDS.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64, 1)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
               const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
               int BH, int N, float c, int nqb) {
    constexpr int SPLIT = D / 64;
    constexpr int RPW = 64 / SPLIT;      // query rows per wave
    constexpr int BCF = 32;              // keys per tile
    __shared__ __attribute__((aligned(16))) float ks[BCF][D];
    __shared__ __attribute__((aligned(16))) float vs[BCF][D];

    const int lane = threadIdx.x;
    const int row = lane % RPW;
    const int part = lane / RPW;
    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb = CAUSAL ? (nqb - 1 - bid / BH) : bid / BH;
    const size_t head = (size_t)bh * (size_t)N * D;
    const int q0 = qb * RPW;
    const int qi = q0 + row;

    float q[64], acc[64];
#pragma unroll
    for (int e = 0; e < 64; e += 4) {
        f32x4_t x = (qi < N) ? *(const f32x4_t*)(Q + head + (size_t)qi * D + 64 * part + e)
                             : f32x4_t{0.f, 0.f, 0.f, 0.f};
        q[e] = x[0]; q[e + 1] = x[1]; q[e + 2] = x[2]; q[e + 3] = x[3];
        acc[e] = acc[e + 1] = acc[e + 2] = acc[e + 3] = 0.f;
    }
    float m_run = kNegInf, l_run = 0.f;
    const int q_last = min(q0 + RPW, N) - 1;
    const int kv_end = CAUSAL ? q_last + 1 : N;

    for (int kv0 = 0; kv0 < kv_end; kv0 += BCF) {
        __syncthreads();
        for (int idx = lane; idx < BCF * D / 4; idx += 64) {
            const int r = idx / (D / 4), cc = (idx % (D / 4)) * 4;
            const int j = kv0 + r;
            f32x4_t kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
            if (j < N) {
                kx = *(const f32x4_t*)(K + head + (size_t)j * D + cc);
                vx = *(const f32x4_t*)(V + head + (size_t)j * D + cc);
            }
            *(f32x4_t*)&ks[r][cc] = kx;
            *(f32x4_t*)&vs[r][cc] = vx;
        }
        __syncthreads();

        float s[BCF];
#pragma unroll
        for (int jj = 0; jj < BCF; ++jj) {
            float partial = 0.f;
#pragma unroll
            for (int e = 0; e < 64; ++e) partial = __builtin_fmaf(q[e], ks[jj][64 * part + e], partial);
            if constexpr (SPLIT == 2) partial += partner32(partial);
            const int j = kv0 + jj;
            s[jj] = (j >= N || (CAUSAL && j > qi)) ? kNegInf : partial;
        }
        float mt = s[0];
#pragma unroll
        for (int jj = 1; jj < BCF; ++jj) mt = fmaxf(mt, s[jj]);
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_use) * c);
        const float mc = m_use * c;
        float ls = 0.f;
#pragma unroll
        for (int jj = 0; jj < BCF; ++jj) {
            s[jj] = fast_exp2(__builtin_fmaf(s[jj], c, -mc));
            ls += s[jj];
        }
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int e = 0; e < 64; ++e) {
            float a = acc[e] * alpha;
#pragma unroll
            for (int jj = 0; jj < BCF; ++jj) a = __builtin_fmaf(s[jj], vs[jj][64 * part + e], a);
            acc[e] = a;
        }
    }

    if (qi < N) {
        const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
        const float m_use = (m_run == kNegInf) ? 0.f : m_run;
        if (part == 0)
            LSE[(size_t)bh * N + qi] = (l_run > 0.f) ? (m_use * c + fast_log2(l_run)) * kLn2 : kNegInf;
#pragma unroll
        for (int e = 0; e < 64; e += 4) {
            f32x4_t x = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
            *(f32x4_t*)(O + head + (size_t)qi * D + 64 * part + e) = x;
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const FwdArgs& a) {
    constexpr int IB = FwdBf16Config<D>::IB;
    constexpr int NW = FwdBf16Config<D>::NW;
    constexpr int BR = NW * IB * 32;
    const int BH = a.B * a.H;
    const int nqb = (a.N + BR - 1) / BR;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, IB, NW, CAUSAL>), dim3(nqb * BH), dim3(NW * 64), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, BH, a.N, c, nqb);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
    if (a.d == 128) return a.causal ? launch_fwd_bf16_t<128, true>(a) : launch_fwd_bf16_t<128, false>(a);
    return a.causal ? launch_fwd_bf16_t<64, true>(a) : launch_fwd_bf16_t<64, false>(a);
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_f32_t(const FwdArgs& a) {
    constexpr int RPW = 64 / (D / 64);
    const int BH = a.B * a.H;
    const int nqb = (a.N + RPW - 1) / RPW;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(nqb * BH), dim3(64), 0, a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o,
                       a.lse, BH, a.N, c, nqb);
    return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs& a) {
    if (a.d == 128) return a.causal ? launch_fwd_f32_t<128, true>(a) : launch_fwd_f32_t<128, false>(a);
    return a.causal ? launch_fwd_f32_t<64, true>(a) : launch_fwd_f32_t<64, false>(a);
}

}  // namespace fa
