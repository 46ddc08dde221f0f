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
#include <type_traits>

#include "fa_kernels.hpp"
#include "fa_device.hpp"

namespace fa {

// ---------------------------------------------------------------------------
// bf16 forward.
//
// Workgroup: 8 waves, 32 query rows per wave, 256 rows in all; tiles of 64
// keys. Products (transposed, so that a query row lives in one lane pair):
//   S^T (keys x queries) = K * Q^T      A = K tile (LDS), B = Q^T (VGPRs)
//   P^T = exp2(S^T*c - m*c)             row max/sum: registers + one
//                                        v_permlane32_swap per row and tile
//   O^T (d x queries)   += V^T * P^T    A = V^T (LDS, transposed, fp16),
//                                        B = P^T from the S^T accumulators (fp16)
//
// The P V product takes fp16 operands (11-bit significand, against bf16's
// 8): with a sharp softmax the rounding of P in bf16 alone moves O by a few
// 1e-3. V enters as fp16(2^-8 V) (exact for 2^-6 <= |v| < 65504 * 2^8; below,
// an absolute error of at most 2^-17; at or above 65504 * 2^8 it overflows)
// and P as fp16(2^7 P) (P <= 2^8 by the rescale rule below, so 2^7 P stays
// in range and its small values keep their precision); the epilogue takes
// both factors out again.
//
// Schedule ("ping-pong"): waves 0-3 (group A) and 4-7 (group B) share the
// four SIMDs, one of each per SIMD. Time is cut into slots separated by
// workgroup barriers; in every slot one group runs its matrix slot
//     S(t) = K(t) Q^T  and  O += V(t-1)^T P(t-1)      (32 MFMAs, priority 1)
// while the other runs its vector slot
//     mask, row max, rare rescale, P(t) = exp2(...), fp16 packing, row sum,
// and the roles swap each slot (B runs one slot behind A). So the matrix cores
// of a SIMD work on one wave while the vector unit serves the other.
// K tiles go straight from global memory into LDS (buffer_load ... lds) and V
// tiles go through group A's registers into a transposed LDS layout, so every
// MFMA operand comes from a plain 16-byte LDS read; double buffered: in its
// matrix slot for tile t group A issues the loads of K(t+1) and V(t), in its
// vector slot it writes V(t) to LDS, and both are first read in slot 2t+2.
// ---------------------------------------------------------------------------

constexpr int kFwdWaves = 8;
// Powers of two on the fp16 operands of the P V product: P is formed as
// 2^kPShift P, V enters as 2^-kVShift V.
constexpr float kPShift = 7.f;
constexpr float kVScale = 1.f / 256.f;      // 2^-8
// O = 2^8 acc / sum(fp16 P): the P factor cancels in the ratio, V's does not.
constexpr float kOScale = 256.f;
#ifndef FA_FWD_AHEAD
#define FA_FWD_AHEAD 4
#endif
constexpr int kFwdAhead = FA_FWD_AHEAD;   // LDS fragment reads in flight ahead of the MFMAs

__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kFwdWaves * 64, 1)
fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                uint16_t* __restrict__ ORes, float* __restrict__ LSE, int BH, int G, int N,
                int Nk, float c, int nqb) {
    constexpr int BC = 64;                 // keys per tile
    constexpr int BR = kFwdWaves * 32;     // query rows per workgroup
    constexpr int KS = D / 16;             // MFMA k-steps over d
    constexpr int NB = D / 32;             // 32-wide blocks of the output columns
    constexpr int TILE = BC * D * 2;
    constexpr int BLOCKS = TILE / 1024;    // 1 KB staging blocks per tile

    __shared__ __attribute__((aligned(16))) char kb0[TILE], kb1[TILE], vb0[TILE], vb1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;             // 0: group A, 1: group B
    const int g = lane >> 5;
    const int l32 = lane & 31;

    // Longest query blocks first (causal), heads fastest. Workgroup ids are
    // dispatched round-robin over the eight XCDs, so id mod 8 picks the XCD;
    // when BH is a multiple of 8 the heads are renumbered so that XCD x runs
    // the contiguous heads [x BH/8, (x+1) BH/8): every XCD keeps to a fixed
    // set of heads, and the G query heads that share a K/V head (G dividing
    // BH/8) read it from the same L2.
    const int bid = blockIdx.x;
    const int hh = bid % BH;
    const int bh = (BH & 7) ? hh : (hh & 7) * (BH >> 3) + (hh >> 3);
    const int qb_rank = bid / BH;
    const int qb = CAUSAL ? (nqb - 1 - qb_rank) : qb_rank;

    const size_t head = (size_t)bh * (size_t)N * D;
    const size_t kvhead = (size_t)(bh / G) * (size_t)Nk * D;  // K/V head of this query head
    const uint16_t* Qh = Q + head;
    const uint16_t* Kh = K + kvhead;
    const uint16_t* Vh = V + kvhead;
    const int q0 = qb * BR;
    const int wq0 = q0 + wave * 32;
    const int qi = wq0 + l32;              // this lane's query row
    // Query row i sits at position i + off: with the causal mask it keeps the
    // keys j <= i + off (off = 0 for the square problem).
    const int off = Nk - N;

    // Q^T operand fragments, resident for the whole kernel. Rows past the end
    // read row N-1 (finite data, never stored).
    u32x4_t qf[KS];
    {
        const int qr = min(qi, N - 1);
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qf[s] = *(const u32x4_t*)(Qh + (size_t)qr * D + 16 * s + 8 * g);
    }

    const int n_all = (Nk + BC - 1) / BC;
    const int q_last = min(q0 + BR, N) - 1 + off;       // last position of the block
    const int n_tiles = CAUSAL ? min(n_all, max(q_last, 0) / BC + 1) : n_all;

    // Buffer i of K / V (selects, not an array: LDS addresses stay scalar).
    auto Kb = [&](int i) { return i ? (lds_char*)kb1 : (lds_char*)kb0; };
    auto Vb = [&](int i) { return i ? (lds_char*)vb1 : (lds_char*)vb0; };

    // m_ref: reference maximum (raw score units) of this lane's row; the
    // probabilities of a tile are exp2((s - m_ref) c) <= 2^kRescaleLog2, and
    // they are formed as 2^kPShift times that (the fp16 operand's factor).
    const float thresh = kRescaleLog2 / c;
    float m_ref = kNegInf, l_rnd = 0.f;
    f32x16_t acc_o[NB], acc_s[2];
    u32x4_t pf[4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[nb][r] = 0.f;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) pf[t4] = u32x4_t{0u, 0u, 0u, 0u};

    // K(t+1) goes straight into LDS (group A, global_load_lds). V(t) goes
    // through registers into a transposed layout ([d][64 keys], the permuted
    // key order of fa_device.hpp) so the matrix slot reads V^T fragments with
    // plain 16-byte LDS reads. The tile is cut into 512 micro-tiles of 4 keys
    // x CW = d/32 columns, 256 per group, so that every thread of a group
    // moves exactly one: it loads them in its matrix slot (4 rows of CW
    // values) and writes them in its next vector slot (one 8-byte slot of 4
    // keys per column). Rows past Nk read row Nk-1 (masked keys).
    constexpr int CW = D / 32;                         // columns per micro-tile
    constexpr int NCG = D / CW;                        // column groups (32)
    static_assert(16 * NCG == 2 * kFwdWaves * 32, "one micro-tile per thread");
    typedef __attribute__((ext_vector_type(CW / 2))) uint32_t vrow_t;   // CW bf16 values
    vrow_t vreg[4];
    const int vu = grp * 256 + (wave & 3) * 64 + lane;
    const int v_cg = vu % NCG, v_rg = vu / NCG;
    auto v_load = [&](int t) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int j = min(t * BC + 4 * v_rg + rr, Nk - 1);
            vreg[rr] = *(const vrow_t*)(Vh + (size_t)j * D + v_cg * CW);
        }
    };
    auto v_store = [&](int t) {
        lds_char* vl = Vb(t & 1);
        const int slot = tr_key_position(4 * v_rg) >> 2;
        // bf16 pairs -> fp16 pairs of 2^-8 v (same packing)
        vrow_t hreg[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int w = 0; w < CW / 2; ++w) hreg[rr][w] = bf16x2_to_f16x2(vreg[rr][w], kVScale);
#pragma unroll
        for (int e = 0; e < CW; ++e) {
            const int w = e >> 1;
            const uint32_t r0 = hreg[0][w], r1 = hreg[1][w], r2 = hreg[2][w], r3 = hreg[3][w];
            u32x2_t col;
            if (e & 1) {
                col[0] = (r0 >> 16) | (r1 & 0xffff0000u);
                col[1] = (r2 >> 16) | (r3 & 0xffff0000u);
            } else {
                col[0] = (r0 & 0xffffu) | (r1 << 16);
                col[1] = (r2 & 0xffffu) | (r3 << 16);
            }
            *(__attribute__((address_space(3))) u32x2_t*)(vl + tr_slot_offset(v_cg * CW + e, slot)) = col;
        }
    };

    // Matrix slot of tile t: S(t) = K(t) Q^T and O += V(t-1)^T P(t-1),
    // interleaved MFMA by MFMA, each MFMA's 16-byte LDS fragment read four
    // MFMAs ahead. In the first slot P = 0 and the V buffer holds zeros; in
    // the last one S reads a stale K buffer and is discarded.
    auto matrix_slot = [&](int t) {
        __builtin_amdgcn_s_setprio(1);
        const lds_char* kt = Kb(t & 1);
        const lds_char* vt = Vb((t + 1) & 1);      // V(t-1)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_s[jb][r] = 0.f;
        constexpr int NS = 2 * KS, NP = 4 * NB;       // MFMAs of S(t) and of P V
#pragma unroll
        for (int x = 0; x < (NS > NP ? NS : NP); ++x) {
            if (x < NS) {
                const int s = x >> 1, jb = x & 1;
                acc_s[jb] = mfma_32x32x16(lds_k_frag<D>(kt, 32 * jb + l32, 2 * s + g), qf[s],
                                          acc_s[jb]);
            }
            if (x < NP) {
                const int t4 = x / NB, nb = x % NB;
                const u32x4_t vf = *(const __attribute__((address_space(3))) u32x4_t*)(
                    vt + tr_slot_offset(32 * nb + l32, 4 * t4 + 2 * g));
                acc_o[nb] = mfma_32x32x16_f16(vf, pf[t4], acc_o[nb]);
            }
        }
        // One LDS read per MFMA: kFwdAhead reads ahead, then alternate.
        __builtin_amdgcn_sched_group_barrier(0x100, kFwdAhead, 0);
#pragma unroll
        for (int x = 0; x < NS + NP - kFwdAhead; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kFwdAhead, 0);
        __builtin_amdgcn_s_setprio(0);
        wait_lds();
    };

    // Vector slot of tile t: softmax of S(t) into P(t).
    auto vector_slot = [&](int t) {
        const int kv0 = t * BC;
        const bool need_mask = (kv0 + BC > Nk) || (CAUSAL && kv0 + BC - 1 > q0 + off);
        if (need_mask) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = kv0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
                    if ((j >= Nk) || (CAUSAL && j > qi + off)) acc_s[jb][r] = kNegInf;
                }
        }
        float m = fmaxf(acc_s[0][0], acc_s[0][1]);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, acc_s[jb][r]);
        const float mt = max_with_partner32(m);
        if (__any(mt > m_ref + thresh)) {
            // Rare: move the reference maximum up and rescale what has been
            // accumulated so far by exp2((m_old - m_new) c).
            const float m_new = fmaxf(m_ref, mt);
            const float alpha = (m_ref == kNegInf) ? 0.f : fast_exp2((m_ref - m_new) * c);
            l_rnd *= alpha;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_o[nb][r] *= alpha;
            m_ref = m_new;
        }
        // exp2(s c - m_ref c + kPShift) = 2^kPShift P
        const float mc = ((m_ref == kNegInf) ? 0.f : m_ref * c) - kPShift;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int jb = t4 >> 1, rb = 8 * (t4 & 1);
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(acc_s[jb][rb + e], c, -mc));
            pf[t4] = u32x4_t{pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]),
                             pack_f16x2(p[4], p[5]), pack_f16x2(p[6], p[7])};
            // Sum of the fp16 probabilities that multiply V (fp32
            // accumulation): normalising O by it makes the rounding error of
            // P scale with (v_j - O) instead of v_j (zero for a row dominated
            // by one key). lse takes the same sum: each term is within 2^-11
            // of 2^kPShift P (relative), so the sum is too, and lse within
            // ln(1 + 2^-11) < 5e-4 (the row's largest term is at least
            // 2^kPShift, so fp16 underflow of the smallest terms is far below
            // that).
#pragma unroll
            for (int w = 0; w < 4; ++w) l_rnd = add_f16x2(pf[t4][w], l_rnd);
        }
    };

    // ---- prologue: K(0) into LDS, zeros into the V buffer of "tile -1" -----
    if (grp == 0) stage_tile_lds<D, BLOCKS / 4, 4, false>(Kh, Kb(0), 0, Nk, wave, lane);
    for (int i = tid; i < TILE / 16; i += kFwdWaves * 64)
        *(__attribute__((address_space(3))) u32x4_t*)(Vb(1) + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
    wait_vmem();
    __syncthreads();
    if (grp == 1) {                        // group B runs one slot behind; it
        v_load(0);                         // writes its half of V(0) meanwhile
        v_store(0);
        wait_vmem();
        wg_barrier();
    }

    // Slot 2t: A matrix(t), B vector(t-1); slot 2t+1: A vector(t), B matrix(t).
    // V(t) is written in slots 2t+1 (A's half) and 2t (B's half, loaded in
    // slot 2t-1; V(0) in the prologue) into the buffer V(t-2) left; K(t+1) is
    // loaded by A in slot 2t. All of them are first read in slot 2t+2.
    for (int t = 0; t <= n_tiles; ++t) {
        matrix_slot(t);
        // Group A stages V(t), group B V(t+1). One call site for both: with
        // two, the compiler loads into different registers and joins them
        // with copies that wait for the loads before the barrier below.
        const int tv = min(t + grp, n_tiles - 1);
        if (t < n_tiles) {
            v_load(tv);
            if (grp == 0 && t + 1 < n_tiles)
                stage_tile_lds<D, BLOCKS / 4, 4, false>(Kh, Kb((t + 1) & 1), (t + 1) * BC, Nk,
                                                        wave, lane);
        }
        wg_barrier();
        if (t < n_tiles) {
            vector_slot(t);
            // The V writes wait for the loads: after the softmax, not in it.
            __builtin_amdgcn_sched_barrier(0);
            if (t + grp < n_tiles) v_store(tv);
            wait_vmem();
            // Group A's half of V(t) is read right after this barrier: its
            // writes must be complete. Group B's half, V(t+1), is first read
            // two barriers on, and the wait_lds at the end of B's next matrix
            // slot completes it before the second.
            if (grp == 0) wait_lds();
            wg_barrier();
        }
    }
    if (grp == 0) wg_barrier();            // same number of barriers in both groups

    // ---- epilogue: deferred normalisation, logsumexp, bf16 store (and, when
    // ORes is given, the bf16 rounding residual of each stored value) --------
    const float lr = sum_with_partner32(l_rnd);
    const float inv = (lr > 0.f) ? kOScale / lr : 0.f;
    if (qi < N && g == 0) {
        const float mc = (m_ref == kNegInf) ? 0.f : m_ref * c;
        LSE[(size_t)bh * N + qi] = (lr > 0.f) ? (mc + (fast_log2(lr) - kPShift)) * kLn2 : kNegInf;
    }
    // O goes out through LDS: each wave writes its 32 rows into a region of the
    // K/V buffers (16-byte chunks of a row swizzled by the row), then stores
    // whole rows, consecutive lanes taking consecutive 16-byte chunks. Every
    // copy into the buffers has landed and every read of them is done first.
    wait_vmem();
    wait_lds();
    __syncthreads();
    constexpr int RB = D * 2;              // bytes per row
    constexpr int CH = RB / 16;            // 16-byte chunks per row
    lds_char* region = ((wave >> 1) == 0 ? Kb(0) : (wave >> 1) == 1 ? Kb(1)
                        : (wave >> 1) == 2 ? Vb(0) : Vb(1)) + (wave & 1) * 32 * RB;
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
        wait_lds();
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
        wait_lds();
        put(true);
        out(ORes);
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
    constexpr int BR = kFwdWaves * 32;
    const int BH = a.B * a.H;
    const int nqb = (a.N + BR - 1) / BR;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(nqb * BH), dim3(kFwdWaves * 64), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, (uint16_t*)a.o_res, a.lse, BH, a.H / a.Hkv,
                       a.N, a.Nk,
                       c, nqb);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
    if (a.d == 256) return launch_fwd_d256(a);
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
