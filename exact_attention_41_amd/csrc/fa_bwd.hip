// Exact-attention backward kernels for gfx950 (bf16 storage, fp32 accumulate).
//
// The pages describe the forward only; the backward here is the exact
// gradient of L = sum(O * dO) with P recomputed from the forward's
// logsumexp instead of stored (the O(N) memory property of the "FlashAttention"
// page, systems-analysis.ru, section "Complexity and optimality"):
//   D_i  = sum_c dO_ic O_ic                       (preprocess kernel)
//   P_ij = exp(scale q_i.k_j - lse_i)             (recomputed, masked)
//   dV   = P^T dO,  dP = dO V^T,  dS = P * (dP - D)
//   dK   = scale dS^T Q                           (key-block kernel)
//   dQ   = scale dS K                             (query-block kernel)
// dK/dV and dQ are produced by two separate passes, so every output element
// is written by exactly one workgroup and no floating-point atomics are used:
// the result is bitwise reproducible ("FlashAttention-2" page,
// systems-analysis.info, section "Performance": exact and deterministic).
#include "fa_kernels.hpp"
#include "fa_device.hpp"

namespace fa {

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i, one fp32 value per query row.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
bwd_delta_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                 float* __restrict__ delta, long long rows) {
    constexpr int TPR = D / 8;        // threads per row, 16 bytes each
    constexpr int RPB = 256 / TPR;    // rows per block
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int ch = threadIdx.x % TPR;
    float acc = 0.f;
    if (row < rows) {
        const u32x4_t a = *(const u32x4_t*)(O + row * D + ch * 8);
        const u32x4_t b = *(const u32x4_t*)(dO + row * D + ch * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc = __builtin_fmaf(bf16_lo(a[w]), bf16_lo(b[w]), acc);
            acc = __builtin_fmaf(bf16_hi(a[w]), bf16_hi(b[w]), acc);
        }
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (ch == 0 && row < rows) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// Staging helpers: a 64-row bf16 tile [64][D] moved from global memory to LDS
// as 4-row x 8-column micro-tiles, written both row-major (swizzled 16-byte
// chunks) and/or transposed ([D][64] with the permuted key order and slot
// swizzle of fa_device.hpp). Rows at or past N are zero-filled.
// ---------------------------------------------------------------------------
template <int D, int NT>
struct Tile64 {
    static constexpr int DCH = D / 8;
    static constexpr int UNITS = 16 * DCH;                 // 4x8 micro-tiles
    static constexpr int LOADS = (UNITS + NT - 1) / NT;
    static constexpr int BYTES = 64 * D * 2;
    u32x4_t r[LOADS][4];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int row0, int N, int tid) {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int u = tid + it * NT;
            if (UNITS % NT == 0 || u < UNITS) {
                const int ch = u % DCH, rg = u / DCH;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int row = row0 + 4 * rg + rr;
                    r[it][rr] = (row < N) ? *(const u32x4_t*)(src + (size_t)row * D + ch * 8)
                                          : u32x4_t{0u, 0u, 0u, 0u};
                }
            }
        }
    }

    __device__ __forceinline__ void store_rowmajor(char* dst, int tid) const {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int u = tid + it * NT;
            if (UNITS % NT == 0 || u < UNITS) {
                const int ch = u % DCH, rg = u / DCH;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    *(u32x4_t*)(dst + row_chunk_offset<D>(4 * rg + rr, ch)) = r[it][rr];
            }
        }
    }

    __device__ __forceinline__ void store_transposed(char* dst, int tid) const {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int u = tid + it * NT;
            if (UNITS % NT == 0 || u < UNITS) {
                const int ch = u % DCH, rg = u / DCH;
                const int slot = tr_key_position(4 * rg) >> 2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int w = e >> 1;
                    const uint32_t r0 = r[it][0][w], r1 = r[it][1][w];
                    const uint32_t r2 = r[it][2][w], r3 = r[it][3][w];
                    u32x2_t col;
                    if (e & 1) {
                        col[0] = (r0 >> 16) | (r1 & 0xffff0000u);
                        col[1] = (r2 >> 16) | (r3 & 0xffff0000u);
                    } else {
                        col[0] = (r0 & 0xffffu) | (r1 << 16);
                        col[1] = (r2 & 0xffffu) | (r3 << 16);
                    }
                    *(u32x2_t*)(dst + tr_slot_offset(ch * 8 + e, slot)) = col;
                }
            }
        }
    }
};

// Row-major 16-byte fragment of a [64][D] swizzled tile: row `row`, chunk `ch`.
template <int D>
__device__ __forceinline__ u32x4_t lds_row_frag(const char* base, int row, int ch) {
    return *(const u32x4_t*)(base + row_chunk_offset<D>(row, ch));
}

// Transposed fragment: row n of a [D][64] tile, positions [8q, 8q+8).
__device__ __forceinline__ u32x4_t lds_tr_frag(const char* base, int n, int q) {
    return *(const u32x4_t*)(base + tr_slot_offset(n, 2 * q));
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per block of NW*32 keys; each wave owns 32 keys and
// walks the query tiles (64 rows each) that can see them.
// Products (lane = key column j, registers = query rows i):
//   S  = Q K^T        A = Q tile (LDS, row-major)   B = K^T (VGPRs)
//   dP = dO V^T       A = dO tile (LDS, row-major)  B = V^T (VGPRs)
//   dV^T += dO^T P    A = dO^T (LDS, transposed)    B = P  (registers)
//   dK^T += Q^T dS    A = Q^T (LDS, transposed)     B = dS (registers)
// ---------------------------------------------------------------------------
template <int D, int NW, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64, 1)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ LSE, const float* __restrict__ delta,
                uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                int BH, int N, float c, float scale) {
    constexpr int BQ = 64;
    constexpr int NT = NW * 64;
    constexpr int BKV = NW * 32;
    constexpr int KS = D / 16;
    constexpr int NB = D / 32;
    using TileT = Tile64<D, NT>;
    constexpr int TB = TileT::BYTES;
    constexpr int OFF_Q = 0, OFF_QT = TB, OFF_DO = 2 * TB, OFF_DOT = 3 * TB;
    constexpr int OFF_LSE = 4 * TB, OFF_DEL = 4 * TB + BQ * 4;
    constexpr int BUF = 4 * TB + 2 * BQ * 4;
    __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int kb = bid / BH;              // low key blocks see the most queries: first
    const size_t head = (size_t)bh * (size_t)N * D;
    const uint16_t* Qh = Q + head;
    const uint16_t* dOh = dO + head;
    const float* lse_h = LSE + (size_t)bh * N;
    const float* del_h = delta + (size_t)bh * N;

    const int k0 = kb * BKV;
    const int kw0 = k0 + wave * 32;
    const int kj = kw0 + l32;             // this lane's key

    u32x4_t kf[KS], vf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        if (kj < N) {
            kf[s] = *(const u32x4_t*)(K + head + (size_t)kj * D + 16 * s + 8 * g);
            vf[s] = *(const u32x4_t*)(V + head + (size_t)kj * D + 16 * s + 8 * g);
        } else {
            kf[s] = vf[s] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }

    f32x16_t acc_dk[NB], acc_dv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_dk[nb][r] = acc_dv[nb][r] = 0.f;

    const int n_tiles = (N + BQ - 1) / BQ;
    const int t0 = CAUSAL ? (k0 / BQ) : 0;

    TileT qt, dot;
    float stat = 0.f;   // lse*log2e (threads 0..63) or delta (64..127) of the next tile

    auto load = [&](int i0) {
        qt.load(Qh, i0, N, tid);
        dot.load(dOh, i0, N, tid);
        if (tid < 2 * BQ) {
            const int i = i0 + (tid & (BQ - 1));
            if (tid < BQ) stat = (i < N) ? lse_h[i] * kLog2e : __builtin_huge_valf();
            else stat = (i < N) ? del_h[i] : 0.f;
        }
    };
    auto store = [&](int buf) {
        char* b = smem + buf * BUF;
        qt.store_rowmajor(b + OFF_Q, tid);
        qt.store_transposed(b + OFF_QT, tid);
        dot.store_rowmajor(b + OFF_DO, tid);
        dot.store_transposed(b + OFF_DOT, tid);
        if (tid < 2 * BQ) ((float*)(b + OFF_LSE))[tid] = stat;
    };

    if (t0 < n_tiles) {
        load(t0 * BQ);
        store(0);
    }
    __syncthreads();

    for (int t = t0; t < n_tiles; ++t) {
        const int i0 = t * BQ;
        const int buf = (t - t0) & 1;
        if (t + 1 < n_tiles) load(i0 + BQ);
        const char* b = smem + buf * BUF;

        if (!CAUSAL || i0 + BQ - 1 >= kw0) {
            f32x16_t acc_s[2], acc_dp[2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_s[ib][r] = acc_dp[ib][r] = 0.f;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const u32x4_t qa = lds_row_frag<D>(b + OFF_Q, 32 * ib + l32, 2 * s + g);
                    acc_s[ib] = mfma_32x32x16(qa, kf[s], acc_s[ib]);
                    const u32x4_t da = lds_row_frag<D>(b + OFF_DO, 32 * ib + l32, 2 * s + g);
                    acc_dp[ib] = mfma_32x32x16(da, vf[s], acc_dp[ib]);
                }
            }

            const bool need_mask = CAUSAL && (i0 < kw0 + 31);
            const float* lse_t = (const float*)(b + OFF_LSE);
            const float* del_t = (const float*)(b + OFF_DEL);
            u32x4_t pp[4], dsp[4];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                float pv[16], dsv[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int ii = 32 * ib + 8 * q4 + 4 * g;
                    const f32x4_t l4 = *(const f32x4_t*)(lse_t + ii);
                    const f32x4_t d4 = *(const f32x4_t*)(del_t + ii);
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int r = 4 * q4 + r4;
                        float p = fast_exp2(__builtin_fmaf(acc_s[ib][r], c, -l4[r4]));
                        if (need_mask && kj > i0 + ii + r4) p = 0.f;
                        pv[r] = p;
                        dsv[r] = p * (acc_dp[ib][r] - d4[r4]);
                    }
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int rb = 8 * h;
                    pp[2 * ib + h] = u32x4_t{pack_bf16x2(pv[rb + 0], pv[rb + 1]), pack_bf16x2(pv[rb + 2], pv[rb + 3]),
                                             pack_bf16x2(pv[rb + 4], pv[rb + 5]), pack_bf16x2(pv[rb + 6], pv[rb + 7])};
                    dsp[2 * ib + h] = u32x4_t{pack_bf16x2(dsv[rb + 0], dsv[rb + 1]), pack_bf16x2(dsv[rb + 2], dsv[rb + 3]),
                                              pack_bf16x2(dsv[rb + 4], dsv[rb + 5]), pack_bf16x2(dsv[rb + 6], dsv[rb + 7])};
                }
            }

#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const u32x4_t a1 = lds_tr_frag(b + OFF_DOT, 32 * nb + l32, 2 * t4 + g);
                    acc_dv[nb] = mfma_32x32x16(a1, pp[t4], acc_dv[nb]);
                    const u32x4_t a2 = lds_tr_frag(b + OFF_QT, 32 * nb + l32, 2 * t4 + g);
                    acc_dk[nb] = mfma_32x32x16(a2, dsp[t4], acc_dk[nb]);
                }
            }
        }

        if (t + 1 < n_tiles) store(buf ^ 1);
        __syncthreads();
    }

    if (kj < N) {
        uint16_t* dkrow = dK + head + (size_t)kj * D;
        uint16_t* dvrow = dV + head + (size_t)kj * D;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                u32x2_t wk, wv;
                wk[0] = pack_bf16x2(acc_dk[nb][4 * q4 + 0] * scale, acc_dk[nb][4 * q4 + 1] * scale);
                wk[1] = pack_bf16x2(acc_dk[nb][4 * q4 + 2] * scale, acc_dk[nb][4 * q4 + 3] * scale);
                wv[0] = pack_bf16x2(acc_dv[nb][4 * q4 + 0], acc_dv[nb][4 * q4 + 1]);
                wv[1] = pack_bf16x2(acc_dv[nb][4 * q4 + 2], acc_dv[nb][4 * q4 + 3]);
                *(u32x2_t*)(dkrow + 32 * nb + 8 * q4 + 4 * g) = wk;
                *(u32x2_t*)(dvrow + 32 * nb + 8 * q4 + 4 * g) = wv;
            }
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per block of NW*32 queries; each wave owns 32 query rows
// and walks the key tiles (64 keys each) they can see.
// Products (lane = query column i, registers = key rows j):
//   S^T  = K Q^T       A = K tile (LDS, row-major)   B = Q^T (VGPRs)
//   dP^T = V dO^T      A = V tile (LDS, row-major)   B = dO^T (VGPRs)
//   dQ^T += K^T dS^T   A = K^T (LDS, transposed)     B = dS^T (registers)
// ---------------------------------------------------------------------------
template <int D, int NW, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64, 1)
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
              const float* __restrict__ LSE, const float* __restrict__ delta,
              uint16_t* __restrict__ dQ, int BH, int N, float c, float scale, int nqb) {
    constexpr int BC = 64;
    constexpr int NT = NW * 64;
    constexpr int BQ = NW * 32;
    constexpr int KS = D / 16;
    constexpr int NB = D / 32;
    using TileT = Tile64<D, NT>;
    constexpr int TB = TileT::BYTES;
    constexpr int OFF_K = 0, OFF_KT = TB, OFF_V = 2 * TB;
    constexpr int BUF = 3 * TB;
    __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb = CAUSAL ? (nqb - 1 - bid / BH) : bid / BH;
    const size_t head = (size_t)bh * (size_t)N * D;
    const uint16_t* Kh = K + head;
    const uint16_t* Vh = V + head;
    const int q0 = qb * BQ;
    const int wq0 = q0 + wave * 32;
    const int qi = wq0 + l32;             // this lane's query row

    u32x4_t qf[KS], of[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        if (qi < N) {
            qf[s] = *(const u32x4_t*)(Q + head + (size_t)qi * D + 16 * s + 8 * g);
            of[s] = *(const u32x4_t*)(dO + head + (size_t)qi * D + 16 * s + 8 * g);
        } else {
            qf[s] = of[s] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    const float lse2 = (qi < N) ? LSE[(size_t)bh * N + qi] * kLog2e : __builtin_huge_valf();
    const float dl = (qi < N) ? delta[(size_t)bh * N + qi] : 0.f;

    f32x16_t acc_dq[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_dq[nb][r] = 0.f;

    const int n_all = (N + BC - 1) / BC;
    const int q_last = min(q0 + BQ, N) - 1;
    const int n_tiles = CAUSAL ? min(n_all, q_last / BC + 1) : n_all;

    TileT kt, vt;
    auto load = [&](int j0) {
        kt.load(Kh, j0, N, tid);
        vt.load(Vh, j0, N, tid);
    };
    auto store = [&](int buf) {
        char* b = smem + buf * BUF;
        kt.store_rowmajor(b + OFF_K, tid);
        kt.store_transposed(b + OFF_KT, tid);
        vt.store_rowmajor(b + OFF_V, tid);
    };

    load(0);
    store(0);
    __syncthreads();

    const int wave_last = wq0 + 31;
    for (int t = 0; t < n_tiles; ++t) {
        const int j0 = t * BC;
        if (t + 1 < n_tiles) load(j0 + BC);
        const char* b = smem + (t & 1) * BUF;

        if (!CAUSAL || j0 <= wave_last) {
            f32x16_t acc_s[2], acc_dp[2];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_s[jb][r] = acc_dp[jb][r] = 0.f;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const u32x4_t ka = lds_row_frag<D>(b + OFF_K, 32 * jb + l32, 2 * s + g);
                    acc_s[jb] = mfma_32x32x16(ka, qf[s], acc_s[jb]);
                    const u32x4_t va = lds_row_frag<D>(b + OFF_V, 32 * jb + l32, 2 * s + g);
                    acc_dp[jb] = mfma_32x32x16(va, of[s], acc_dp[jb]);
                }
            }

            const bool need_mask = (j0 + BC > N) || (CAUSAL && j0 + BC - 1 > wq0);
            u32x4_t dsp[4];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                float dsv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = j0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
                    float p = fast_exp2(__builtin_fmaf(acc_s[jb][r], c, -lse2));
                    if (need_mask && (j >= N || (CAUSAL && j > qi))) p = 0.f;
                    dsv[r] = p * (acc_dp[jb][r] - dl);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int rb = 8 * h;
                    dsp[2 * jb + h] = u32x4_t{pack_bf16x2(dsv[rb + 0], dsv[rb + 1]), pack_bf16x2(dsv[rb + 2], dsv[rb + 3]),
                                              pack_bf16x2(dsv[rb + 4], dsv[rb + 5]), pack_bf16x2(dsv[rb + 6], dsv[rb + 7])};
                }
            }

#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const u32x4_t a = lds_tr_frag(b + OFF_KT, 32 * nb + l32, 2 * t4 + g);
                    acc_dq[nb] = mfma_32x32x16(a, dsp[t4], acc_dq[nb]);
                }
            }
        }

        if (t + 1 < n_tiles) store((t + 1) & 1);
        __syncthreads();
    }

    if (qi < N) {
        uint16_t* row = dQ + head + (size_t)qi * D;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                u32x2_t w;
                w[0] = pack_bf16x2(acc_dq[nb][4 * q4 + 0] * scale, acc_dq[nb][4 * q4 + 1] * scale);
                w[1] = pack_bf16x2(acc_dq[nb][4 * q4 + 2] * scale, acc_dq[nb][4 * q4 + 3] * scale);
                *(u32x2_t*)(row + 32 * nb + 8 * q4 + 4 * g) = w;
            }
    }
}

// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a) {
    constexpr int NW = 4;
    const int BH = a.B * a.H;
    const long long rows = (long long)BH * a.N;
    const float c = a.scale * kLog2e;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       a.stream, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.delta, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nkb = (a.N + NW * 32 - 1) / (NW * 32);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, CAUSAL>), dim3(nkb * BH), dim3(NW * 64), 0, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.delta, (uint16_t*)a.dk, (uint16_t*)a.dv,
                       BH, a.N, c, a.scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nqb = (a.N + NW * 32 - 1) / (NW * 32);
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, CAUSAL>), dim3(nqb * BH), dim3(NW * 64), 0, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.delta, (uint16_t*)a.dq, BH, a.N, c,
                       a.scale, nqb);
    return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdArgs& a) {
    if (a.d == 128) return a.causal ? launch_bwd_t<128, true>(a) : launch_bwd_t<128, false>(a);
    return a.causal ? launch_bwd_t<64, true>(a) : launch_bwd_t<64, false>(a);
}

}  // namespace fa
