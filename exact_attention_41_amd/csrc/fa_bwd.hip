// Exact-attention backward kernels for gfx950 (bf16 storage, fp32 accumulate).
//
// The pages describe the forward only; the backward here is the exact
// gradient of L = sum(O * dO), with P recomputed from the forward's
// logsumexp instead of stored (the O(N) memory property of the "FlashAttention"
// page, systems-analysis.ru, section "Complexity and optimality"):
//   P_ij = exp(scale q_i.k_j - lse_i)  (masked),   dP = dO V^T
//   D_i  = sum_j P_ij dP_ij,   dS = P * (dP - D)
//   dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K
//
// Three phases, all deterministic (each output element is written by exactly
// one workgroup, no floating-point atomics: the "FlashAttention-2" page,
// systems-analysis.info, section "Performance", calls the method exact and
// deterministic):
//   1. prepare: per head, the largest |x| of Q, K, V and dO, turned into
//      power-of-two factors so that every fp16 operand below (a bf16 input
//      scaled by a power of two) is in range, and exact for |x| down to
//      2^-17 of the head's largest (smaller values round, by at most 2^-24
//      of the largest: fp16's subnormal step); then fp16 copies of s_Q Q,
//      s_dO dO and s_K K, laid out for the pass that reads them: as rows
//      (read transposed with ds_read_b64_tr_b16 where a product needs them
//      so), or per 64-row tile exactly as a transposed LDS tile. The same
//      pass forms D_i = dO_i . O_i per row: from O plus the forward's
//      rounding residual of O when the caller has it (D itself), else from
//      the bf16 O alone (the rounding of O moves that too far: only a
//      centre D^ for step 2).
//   2. dQ pass: one workgroup per query block, over the key tiles. With D
//      known, dQ_i = scale * sum_j P_ij (dP_ij - D_i) K_j. Otherwise, with
//      E_ij = P_ij (dP_ij - D^_i), it uses
//          dQ_i = scale * (sum_j E_ij K_j - (D_i - D^_i) sum_j P_ij K_j)
//      and accumulates both sums and D_i - D^_i = sum_j E_ij in the same
//      pass; D is exact. Subtracting the centre before E is rounded keeps
//      its rounding error proportional to |dP - D| rather than |dP| (large
//      when V has a large mean). It leaves lse and D per query tile in the
//      workspace for the next pass.
//   3. dK/dV pass: one workgroup per key block, over the query tiles.
// S and dP are products of the inputs: the bf16 values themselves, or their
// fp16 copies scaled by powers of two (the same values in the range above).
// The probabilities and dS enter the gradient products as fp16 (11-bit
// significand) rather than bf16 (8-bit), against fp16 copies of Q, dO or K:
// this keeps dQ, dK and dV within 1e-2 of the exact gradients where bf16
// operands do not.
//
// Every tile reaches LDS by direct global-to-LDS loads (row-major tiles of
// the bf16 inputs or of their fp16 copies, with the chunk swizzle applied
// through the source addresses; transposed tiles as straight copies of
// their images), issued ahead into LDS buffers of their own, so that each
// pass needs one barrier per tile (per step in the 32-row passes) and its
// fragment reads run on through it; no tile passes through VGPRs.
#include "fa_kernels.hpp"
#include "fa_device.hpp"

namespace fa {

// LDS fragments are read this many products ahead of their use, in the dQ
// and the dK/dV pass. The ring of fragment registers (one more than this)
// runs on from step to step, so it must divide the products of every step.
#ifndef FA_BWD_DQ_FRAG_AHEAD
#define FA_BWD_DQ_FRAG_AHEAD 7
#endif
constexpr int kDqFragAhead = FA_BWD_DQ_FRAG_AHEAD;
#ifndef FA_BWD_DKDV_FRAG_AHEAD
#define FA_BWD_DKDV_FRAG_AHEAD 7
#endif
constexpr int kDkdvFragAhead = FA_BWD_DKDV_FRAG_AHEAD;
// The dK/dV pass with 16-row steps reads fp16 rows of s_Q Q and s_dO dO and
// takes the transposed operands of its dV, dK products from them
// (ds_read_b64_tr_b16); 0: bf16 rows plus transposed fp16 images.
#ifndef FA_DKDV_TR
#define FA_DKDV_TR 1
#endif
// The dQ pass with 16-row steps at d = 256 reads fp16 rows of s_K K and takes
// the transposed operand of its dQ product from them; at d <= 128 (and with
// 0) it reads bf16 K rows plus the transposed fp16 K image. (Same-box A/B:
// the rows at d = 256 causal 0.452 -> 0.432 ms, at d = 128 3% slower, at
// d = 64 32% slower.)
#ifndef FA_DQ_TR
#define FA_DQ_TR 1
#endif
constexpr bool dq16_tr(int D) { return FA_DQ_TR != 0 && D == 256; }
// The passes with 16-row steps form their fragment addresses once per tile
// (the dK/dV pass at every head size, the dQ pass at d <= 128 for its K image
// and at d = 128 and 256 for its rows).
// The dQ pass with 16-row steps writes the fp16 Q and dO rows of the dK/dV
// pass (when both passes have 16-row steps, at d = 128 and 256); 0: the image
// pass does.
#ifndef FA_ROWS_FROM_DQ
#define FA_ROWS_FROM_DQ 1
#endif
#ifndef FA_DKDV_PRE
#define FA_DKDV_PRE 1
#endif

// Vector-memory wait (the global-to-LDS copies) and a workgroup barrier that
// lets LDS reads stay in flight across it (__syncthreads waits for them). The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }     // lgkmcnt(0)
__device__ __forceinline__ void step_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Workspace layout (byte offsets; every block 256-byte aligned).
// ---------------------------------------------------------------------------
static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int bwd_scale_chunks(long long Nq, long long Nk, long long d) {
    const long long n = Nq > Nk ? Nq : Nk, rows = scale_chunk_rows(d);
    return (int)((n + rows - 1) / rows);
}

BwdWorkspace bwd_workspace_layout(long long B, long long H, long long Hkv, long long Nq,
                                  long long Nk, long long d) {
    BwdWorkspace w;
    const size_t bh = (size_t)(B * H), bhkv = (size_t)(B * Hkv);
    const size_t chunks = (size_t)bwd_scale_chunks(Nq, Nk, d);
    const size_t tq = (size_t)((Nq + 63) / 64), tk = (size_t)((Nk + 63) / 64);
    const size_t tile = 64 * (size_t)d * 2;             // one transposed 64-row tile
    w.scales = 0;
    w.partial = w.scales + align256(bh * 4 * 4);
    w.dhat = w.partial + align256((bh + bhkv) * chunks * 2 * 4);
    w.stats = w.dhat + align256(bh * (size_t)Nq * 4);
    w.qt = w.stats + align256(bh * tq * 128 * 4);
    w.ot = w.qt + align256(bh * tq * tile);
    w.kt = w.ot + align256(bh * tq * tile);
    w.total = w.kt + align256(bhkv * tk * tile);
    return w;
}

// ---------------------------------------------------------------------------
// Phase 1a: per (head, chunk of scale_chunk_rows(D) rows), the largest |x| of two
// tensors, as bf16 magnitude bits (for finite values the integer order of
// (bits & 0x7fff) is the order of |x|): Q and dO (Nq rows) for the BH query
// heads (rows r < BH of the grid), K and V (Nk rows) for the BHkv K/V heads
// (rows r >= BH). Chunks past a tensor's rows record 0. For the query heads
// it also forms D_i = dO_i . O_i (fp32) of every row of the chunk, with O the
// bf16 output, or that plus its bf16 rounding residual when ORes is given.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
bwd_absmax_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                  const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                  const uint16_t* __restrict__ O, const uint16_t* __restrict__ ORes,
                  uint32_t* __restrict__ partial,
                  float* __restrict__ dhat, int BH, int Nq, int Nk, int chunks) {
    constexpr int DCH = D / 8;
    const int bid = blockIdx.x;
    const int r = bid / chunks, ch = bid % chunks;
    const bool kv = r >= BH;
    const int N = kv ? Nk : Nq;
    constexpr int CR = scale_chunk_rows(D);
    const int row0 = ch * CR;
    const int nrows = min(CR, N - row0);
    const size_t base = ((size_t)(kv ? r - BH : r) * N + row0) * D;
    const uint16_t* src0 = (kv ? K : Q) + base;
    const uint16_t* src1 = (kv ? V : dO) + base;
    const bool with_d = !kv, with_res = !kv && ORes != nullptr;
    uint32_t m[2] = {0u, 0u};
    // Thread idx holds chunk idx % DCH of row idx / DCH (256 is a multiple
    // of DCH, so a row's DCH chunks sit in DCH consecutive lanes, all in or
    // all out of the loop together). Every load of an iteration is issued
    // before any is used, two iterations at a time.
#pragma unroll 2
    for (int idx = threadIdx.x; idx < nrows * DCH; idx += 256) {
        const size_t e = (size_t)idx * 8;
        const u32x4_t w0 = *(const u32x4_t*)(src0 + e);
        const u32x4_t w1 = *(const u32x4_t*)(src1 + e);
        u32x4_t ow = {0u, 0u, 0u, 0u}, rw = {0u, 0u, 0u, 0u};
        if (with_d) ow = *(const u32x4_t*)(O + base + e);
        if (with_res) rw = *(const u32x4_t*)(ORes + base + e);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            m[0] = max(m[0], max(w0[c] & 0x7fffu, (w0[c] >> 16) & 0x7fffu));
            m[1] = max(m[1], max(w1[c] & 0x7fffu, (w1[c] >> 16) & 0x7fffu));
        }
        if (with_d) {
            // D = dO . O with O = bf16(O) (+ its residual: the sum is exact in fp32)
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                s = __builtin_fmaf(bf16_lo(w1[c]), bf16_lo(ow[c]) + bf16_lo(rw[c]), s);
                s = __builtin_fmaf(bf16_hi(w1[c]), bf16_hi(ow[c]) + bf16_hi(rw[c]), s);
            }
#pragma unroll
            for (int off = DCH / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
            if (idx % DCH == 0) dhat[(size_t)r * Nq + row0 + idx / DCH] = s;
        }
    }
    __shared__ uint32_t red[4][2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m[t] = max(m[t], (uint32_t)__shfl_xor((int)m[t], off));
        if (lane == 0) red[wave][t] = m[t];
    }
    __syncthreads();
    if (threadIdx.x < 2) {
        const int t = threadIdx.x;
        const uint32_t v = max(max(red[0][t], red[1][t]), max(red[2][t], red[3][t]));
        partial[((size_t)r * chunks + ch) * 2 + t] = v;
    }
}

// Phase 1b: per query head, the power-of-two factor 2^-(e+1) for a largest
// magnitude in [2^e, 2^(e+1)), so the scaled tensor has |x| < 1 (1 for an
// all-zero tensor); factors are kept within [2^-60, 2^60]. Q and dO take the
// largest magnitude over the G query heads that share a K/V head, so one
// factor serves the whole group; K and V take their K/V head's.
__device__ __forceinline__ float pow2_factor(uint32_t m) {
    if (m == 0u) return 1.f;
    int e = (int)(m >> 7) - 127;          // floor(log2 max) (subnormals: -127)
    e = min(max(e + 1, -60), 60);
    return __uint_as_float((uint32_t)(127 - e) << 23);
}

__global__ void __launch_bounds__(64)
bwd_scale_kernel(const uint32_t* __restrict__ partial, float* __restrict__ scales, int BH,
                 int G, int chunks) {
    const int bh = blockIdx.x * 64 + threadIdx.x;
    if (bh >= BH) return;
    const int g0 = bh - bh % G, kvh = bh / G;
    uint32_t mq = 0u, mo = 0u, mk = 0u, mv = 0u;
    for (int h = g0; h < g0 + G; ++h)
        for (int c = 0; c < chunks; ++c) {
            mq = max(mq, partial[((size_t)h * chunks + c) * 2 + 0]);
            mo = max(mo, partial[((size_t)h * chunks + c) * 2 + 1]);
        }
    for (int c = 0; c < chunks; ++c) {
        mk = max(mk, partial[((size_t)(BH + kvh) * chunks + c) * 2 + 0]);
        mv = max(mv, partial[((size_t)(BH + kvh) * chunks + c) * 2 + 1]);
    }
    scales[(size_t)bh * 4 + 0] = pow2_factor(mq);
    scales[(size_t)bh * 4 + 1] = pow2_factor(mk);
    scales[(size_t)bh * 4 + 2] = pow2_factor(mv);
    scales[(size_t)bh * 4 + 3] = pow2_factor(mo);
}

// ---------------------------------------------------------------------------
// A 64-row, 16-bit tile [64][D] (source rows LD values apart) read as 4-row
// x 8-column micro-tiles and written transposed ([D][64], with the slot
// swizzle of fa_device.hpp; the rows in the permuted order of fa_device.hpp,
// or with NATURAL in their own order), to LDS or to a global image of that
// layout. With CVT the source is bf16 and the copy is fp16 of the value times
// a power of two. Rows at or past N repeat row N-1 (finite values that the
// consumers' masks multiply by zero).
// ---------------------------------------------------------------------------
template <int D, int NT, int LD = D>
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
                    const int row = min(row0 + 4 * rg + rr, N - 1);
                    r[it][rr] = *(const u32x4_t*)(src + (size_t)row * LD + ch * 8);
                }
            }
        }
    }

    // The tile as rows again (row r at dst + r * row_bytes), fp16 of the value
    // times s with CVT.
    template <bool CVT>
    __device__ __forceinline__ void store_rows(char* dst, int row_bytes, int tid, float s = 1.f) const {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int u = tid + it * NT;
            if (UNITS % NT == 0 || u < UNITS) {
                const int ch = u % DCH, rg = u / DCH;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    u32x4_t x;
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        x[w] = CVT ? bf16x2_to_f16x2(r[it][rr][w], s) : r[it][rr][w];
                    *(u32x4_t*)(dst + (size_t)(4 * rg + rr) * row_bytes + ch * 16) = x;
                }
            }
        }
    }

    template <bool CVT, bool NATURAL = false>
    __device__ __forceinline__ void store_transposed(char* dst, int tid, float s = 1.f) const {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int u = tid + it * NT;
            if (UNITS % NT == 0 || u < UNITS) {
                const int ch = u % DCH, rg = u / DCH;
                const int slot = NATURAL ? rg : (tr_key_position(4 * rg) >> 2);
                u32x4_t x[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        x[rr][w] = CVT ? bf16x2_to_f16x2(r[it][rr][w], s) : r[it][rr][w];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int w = e >> 1;
                    u32x2_t col;
                    if (e & 1) {
                        col[0] = (x[0][w] >> 16) | (x[1][w] & 0xffff0000u);
                        col[1] = (x[2][w] >> 16) | (x[3][w] & 0xffff0000u);
                    } else {
                        col[0] = (x[0][w] & 0xffffu) | (x[1][w] << 16);
                        col[1] = (x[2][w] & 0xffffu) | (x[3][w] << 16);
                    }
                    *(u32x2_t*)(dst + tr_slot_offset(ch * 8 + e, slot)) = col;
                }
            }
        }
    }
};

// The d = 256 images of Q and dO hold each 32-row half of a 64-row tile as a
// [256][32] block of its own (64-byte rows of four 16-byte chunks): chunk c of
// row n (rows 8c .. 8c+7 of the half) sits at chunk c ^ ((n >> 2) & 3), so
// that 16 consecutive rows reading one chunk cover every bank once.
__device__ __forceinline__ int img32_offset(int n, int c) { return 64 * n + 16 * (c ^ ((n >> 2) & 3)); }

// The K images of the dQ pass with 16-row steps at d <= 128, in step order:
// the 16-byte chunk c (keys 8c .. 8c+7 of the 64-key tile) of row n sits at
// (c/2) 32 D + 32 n + 16 (c%2 ^ bit 3 of n), i.e. the tile's four 16-key
// steps one after the other, each a [D][16] block of 32-byte rows whose two
// halves swap every eight rows. Sixteen consecutive rows reading one chunk
// then cover every bank once, and a fragment of step s or of row block 32 x
// lies a constant distance from that of step 0, row block 0.
template <int D>
__device__ __forceinline__ int kt_step_offset(int n, int c) {
    return (c >> 1) * (32 * D) + 32 * n + 16 * ((c & 1) ^ ((n >> 3) & 1));
}


// Phase 1c: fp16 transposed images. One workgroup per (head, 64-row tile,
// column part): the first BH*Tq tiles are the Q images of the query heads,
// the next BH*Tq the dO images, the last BHkv*Tk the K images of the K/V
// heads. A head size DT above 128 is cut into NP = DT/128 parts of 128
// columns, each imaged on its own ([tile][part] order), as the passes below
// stage them. Bit 0 of `natural` is set when the dK/dV pass is the one with
// 16-row steps (bwd_dkdv16_kernel), which reads eight consecutive query rows
// per lane: for head sizes up to 128 it keeps the rows of the Q and dO images
// in their own order, and at d = 256 it writes them as the [256][32] halves
// of img32_offset. Bit 1 does the same for the K images when the dQ pass is
// the one with 16-row steps (bwd_dq16_kernel), at d <= 128 in the step order
// of kt_step_offset. Every other image uses the permuted row order. The grid
// starts at tile bid0: 2 BH Tq for the K images alone (when the dQ pass
// writes the Q and dO rows).
template <int DT>
__global__ void __launch_bounds__(256)
bwd_image_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                 const uint16_t* __restrict__ dO, const float* __restrict__ scales,
                 char* __restrict__ qt, char* __restrict__ ot, char* __restrict__ kt, int BH,
                 int G, int Nq, int Nk, int Tq, int Tk, int natural, int bid0) {
    constexpr int D = DT > 128 ? 128 : DT;
    constexpr int NP = DT / D;
    using TileT = Tile64<D, 256, DT>;
    const int bid = bid0 + blockIdx.x / NP, part = blockIdx.x % NP;
    const int qblocks = BH * Tq;
    const int which = bid < qblocks ? 0 : (bid < 2 * qblocks ? 1 : 2);
    const int rel = bid - (which < 2 ? which * qblocks : 2 * qblocks);
    const int T = which < 2 ? Tq : Tk, N = which < 2 ? Nq : Nk;
    const int head = rel / T, tile = rel % T;  // query head (Q, dO) or K/V head (K)
    const uint16_t* src = which == 0 ? Q : (which == 1 ? dO : K);
    char* dst = which == 0 ? qt : (which == 1 ? ot : kt);
    const float s = which == 0 ? scales[head * 4 + 0]
                  : (which == 1 ? scales[head * 4 + 3] : scales[head * G * 4 + 1]);
    // Transposed into LDS first (8-byte writes spread over the tile), then
    // copied out in 16-byte chunks that consecutive threads take in order.
    __shared__ __attribute__((aligned(16))) char img[TileT::BYTES];
    TileT tl;
    tl.load(src + (size_t)head * N * DT + part * D, tile * 64, N, threadIdx.x);
    // Bit 2: Q and dO as fp16 rows ([Tq * 64][DT] per head, row-major), each
    // thread converting the 4 x 8 micro-tiles it loaded; bit 3: K as fp16
    // rows ([Tk * 64][DT] per K/V head).
    if (natural & (which < 2 ? 4 : 8)) {
        char* rows = dst + ((size_t)head * T + tile) * NP * TileT::BYTES;
        tl.template store_rows<true>(rows + part * D * 2, DT * 2, threadIdx.x, s);
        return;
    }
    // (d = 256: Q and dO in the half-tile layout of img32_offset)
    const bool halves = DT > 128 && (natural & (which < 2 ? 1 : 2));
    if (halves || (DT <= 128 && (natural & (which < 2 ? 1 : 2))))
        tl.template store_transposed<true, true>(img, threadIdx.x, s);
    else tl.template store_transposed<true, false>(img, threadIdx.x, s);
    __syncthreads();
    if (DT > 128 && halves) {
        // rows 128 part .. +127 of the tile's two [256][32] halves: 16-byte
        // chunk position cc of row n of half h holds chunk c = cc ^ ((n >> 2)
        // & 3), i.e. rows 32 h + 8 c .. +7 of the transposed part
        static_assert(DT <= 128 || TileT::BYTES == 16384, "two halves of 128 rows x 32 per part");
        char* out = dst + ((size_t)head * T + tile) * NP * TileT::BYTES;
#pragma unroll
        for (int i = threadIdx.x; i < TileT::BYTES / 16; i += 256) {
            const int h = i >> 9, n = (i >> 2) & 127, cc = i & 3;
            const int c = cc ^ ((n >> 2) & 3);
            *(u32x4_t*)(out + h * TileT::BYTES + img32_offset(128 * part + n, c)) =
                *(const u32x4_t*)(img + tr_slot_offset(n, 8 * h + 2 * c));
        }
        return;
    }
    char* out = dst + (((size_t)head * T + tile) * NP + part) * TileT::BYTES;
    if (DT <= 128 && which == 2 && (natural & 2)) {
        // the K image of the dQ pass with 16-row steps, in the step order of
        // kt_step_offset: chunk i holds step i / 2D, row (i % 2D) / 2, half
        // i % 2 (chunk c % 2 ^ bit 3 of the row)
#pragma unroll
        for (int i = threadIdx.x; i < TileT::BYTES / 16; i += 256) {
            const int st = i / (2 * D), n = (i % (2 * D)) >> 1;
            const int c = 2 * st + ((i & 1) ^ ((n >> 3) & 1));
            *(u32x4_t*)(out + 16 * i) = *(const u32x4_t*)(img + tr_slot_offset(n, 2 * c));
        }
        return;
    }
#pragma unroll
    for (int i = threadIdx.x; i < TileT::BYTES / 16; i += 256)
        *(u32x4_t*)(out + 16 * i) = *(const u32x4_t*)(img + 16 * i);
}

// ---------------------------------------------------------------------------
// Phase 2: dQ (and the per-tile lse and D for phase 3).
// One workgroup per block of NW*32 queries; each wave owns 32 query rows,
// one per lane pair. Products (lane = query column i, registers = key rows j):
//   S^T  = K Q^T               A = K tile (LDS, bf16)      B = Q^T (VGPRs)
//   dP~^T = V (sE dO)^T        A = V tile (LDS, bf16)      B = sE dO^T (VGPRs)
//   A~^T += K~^T (P*dP~)^T     A = (sK K)^T (LDS, fp16)    B = P*dP~ (fp16)
//   B~^T += K~^T P^T           A = (sK K)^T (LDS, fp16)    B = P (fp16)
// with sE = s_dO * s_V and the dP~ chain started from -sE D^ (so that the
// accumulator holds dP~ - sE D^); finally dQ = scale/(sK sE) (A~ - D~ B~),
// D~ = sE (D - D^) = sum_j P*dP~.
// With DK (the preprocess formed D itself, from O and its rounding residual)
// the chain starts from -sE D, there is no B~ sum and no D~, and
// dQ = scale/(sK sE) A~: three products per score instead of four.
// A head size DT above 128 runs as NC = DT/128 column parts: each key tile
// is staged as NC steps of 128 columns of K and V, S and dP accumulate over
// all of them, and each workgroup forms the dQ columns of one part (the
// grid holds NC workgroups per query block; the first writes lse and D).
// ---------------------------------------------------------------------------
template <int DT, int NW, bool CAUSAL, bool DK>
__global__ void __launch_bounds__(NW * 64, 1)
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
              const float* __restrict__ LSE, const float* __restrict__ scales,
              const float* __restrict__ dhat, const char* __restrict__ kt_img,
              float* __restrict__ stats,
              uint16_t* __restrict__ dQ, int BH, int G, int N, int Nk, int T, int Tk,
              float c, float scale, int nqb) {
    constexpr int D = DT > 128 ? 128 : DT;  // columns of one staged tile and of one dQ part
    constexpr int NC = DT / D;              // column steps per key tile = dQ parts
    // Above d = 128 the parked Q and dO fill the AGPR file with the sums:
    // products that read them carry the VALU-write wait states.
    constexpr bool WS = DT > 128;
    constexpr int BC = 64;
    constexpr int BQ = NW * 32;
    constexpr int KS = D / 16;              // S (or dP) products per step and 32-key half
    constexpr int KST = DT / 16;
    constexpr int NB = D / 32;
    constexpr int TB = 64 * D * 2;         // bytes of one 64-row tile
    constexpr int BLK = TB / 1024;         // its 1 KB staging blocks
    constexpr int OFF_K = 0, OFF_V = TB, OFF_KT = 2 * TB;
    constexpr int BUF = 3 * TB;
    // Three buffers: while step s is computed from buffer s % 3, step s + 1
    // is staged into the next one, and the last fragments of step s - 1 may
    // still be in flight from the third.
    constexpr int NBUF = 3;
    __shared__ __attribute__((aligned(16))) char smem[NBUF * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int part = (bid / BH) % NC;      // dQ columns [D part, D part + D)
    const int qbi = bid / (BH * NC);
    const int qb = CAUSAL ? (nqb - 1 - qbi) : qbi;
    const size_t head = (size_t)bh * (size_t)N * DT;
    const size_t kvhead = (size_t)(bh / G) * (size_t)Nk * DT;  // K/V head of this query head
    const uint16_t* Kh = K + kvhead;
    const uint16_t* Vh = V + kvhead;
    const char* kt_h = kt_img + (size_t)(bh / G) * Tk * NC * TB;
    const int q0 = qb * BQ;
    const int wq0 = q0 + wave * 32;
    const int qi = wq0 + l32;             // this lane's query row
    const int off = Nk - N;               // query row i sits at key position i + off

    const float sK = scales[bh * 4 + 1];
    const float sV = scales[bh * 4 + 2], sDO = scales[bh * 4 + 3];
    const float sE = sDO * sV;

    u32x4_t qf[KST], of[KST];
#pragma unroll
    for (int s = 0; s < KST; ++s) {
        if (qi < N) {
            const size_t off = head + (size_t)qi * DT + 16 * s + 8 * g;
            const u32x4_t qv = *(const u32x4_t*)(Q + off);
            const u32x4_t ov = *(const u32x4_t*)(dO + off);
#pragma unroll
            for (int w = 0; w < 4; ++w) of[s][w] = bf16x2_scale(ov[w], sE);
            qf[s] = qv;
        } else {
            qf[s] = of[s] = u32x4_t{0u, 0u, 0u, 0u};
        }
        park_in_agprs(qf[s]);
        park_in_agprs(of[s]);
    }
    // Rows past N, and rows that see no key (lse = -inf), take +inf: every
    // probability of theirs is then exactly 0.
    const float lse_i = (qi < N) ? LSE[(size_t)bh * N + qi] : kNegInf;
    const float lse2 = (lse_i == kNegInf) ? __builtin_huge_valf() : lse_i * kLog2e;
    // The centre sE D^ (or sE D) of this row's dP~ (0 past N), as the start
    // value of every dP~ chain.
    const float dhs = (qi < N) ? sE * dhat[(size_t)bh * N + qi] : 0.f;
    f32x16_t dinit;
#pragma unroll
    for (int r = 0; r < 16; ++r) dinit[r] = -dhs;

    f32x16_t acc_a[NB], acc_b[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_a[nb][r] = acc_b[nb][r] = 0.f;
    float dsum = 0.f;

    const int n_all = (Nk + BC - 1) / BC;
    const int q_last = min(q0 + BQ, N) - 1 + off;      // last key position of the block
    const int n_tiles = CAUSAL ? min(n_all, max(q_last, 0) / BC + 1) : n_all;

    // Column step cs of key tile t into buffer buf: K and V rows (bf16,
    // swizzled) and, for the last step, this part's (sK K)^T image, BLK 1 KB
    // blocks each, spread over the NW waves; part k of the step's parts is
    // one block of this wave. Past the last tile the buffer is filled from a
    // valid tile and never read.
    constexpr int PPT = BLK / NW;            // blocks per wave and tensor
    auto stage_part = [&](int t, int cs, int buf, int k) {
        lds_char* base = (lds_char*)(smem + buf * BUF);
        const int tensor = k / PPT, b = wave + NW * (k % PPT);
        if (tensor < 2)
            stage_tile_block_async<D, DT>((tensor == 0 ? Kh : Vh) + cs * D,
                                          base + (tensor == 0 ? OFF_K : OFF_V), t * BC, Nk, b,
                                          lane);
        else
            stage_image_block_full_async(kt_h + ((size_t)min(t, Tk - 1) * NC + part) * TB,
                                         base + OFF_KT, b, lane);
    };

    // Lane-dependent LDS bases of buffer 0: pb[k], k < 8, for the row-major
    // S/dP fragments (chunk step s; for d = 64 also the key half) and
    // pb[8 + 2 t4 + (nb & 1)] for the transposed dQ fragments; the rest of
    // each fragment address is an immediate offset.
    lds_char* const s0 = (lds_char*)smem;
    lds_char* pb[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int jb = (D == 64) ? k / KS : 0, st = (D == 64) ? k % KS : k;
        pb[k] = s0 + row_chunk_offset<D>(32 * jb + l32, 2 * st + g);
        pb[8 + k] = s0 + tr_slot_offset(32 * (k & 1) + l32, 2 * (2 * (k >> 1) + g));
    }

    // Fragment o of a step (o < 2 NSD: the S/dP fragments, in product
    // order; then the K~^T fragments of the dQ sums) in the buffer `delta`
    // bytes past the current bases.
    constexpr int NSD = 2 * KS;
    constexpr int LA = kDqFragAhead;
    auto frag = [&](int o, int delta) -> u32x4_t {
        if (o < 2 * NSD) {
            const int jb = o / NSD, w = o % NSD, st = w >> 1;
            const int k = (D == 64) ? jb * KS + st : st;
            const int off = ((w & 1) ? OFF_V : OFF_K) + ((D == 64) ? 0 : jb * 32 * D * 2);
            return *(const lds_u32x4_t*)(pb[k] + delta + off);
        }
        const int w = o - 2 * NSD, t4 = w / NB, nb = w % NB;
        const int off = OFF_KT + (nb - (nb & 1)) * 32 * 128;
        return *(const lds_u32x4_t*)(pb[8 + 2 * t4 + (nb & 1)] + delta + off);
    };

    {
        constexpr int NP0 = (NC == 1 ? 3 : 2) * PPT;
#pragma unroll
        for (int k = 0; k < NP0; ++k) stage_part(0, 0, 0, k);
    }
    // (the copies are not visible to the compiler: wait for them explicitly)
    wait_copies();
    __syncthreads();
    // The fragment ring, carried from step to step: product o of a step
    // takes fr[o % (LA + 1)], and the first LA fragments of the next step
    // are read during the last LA products of this one.
    u32x4_t fr[LA + 1];
#pragma unroll
    for (int o = 0; o < LA; ++o) fr[o] = frag(o, 0);

    // One key tile: NC column steps, each staging the next step (the next
    // column step of this tile, or the first of the next tile) into the next
    // buffer, running its products and moving the bases to that buffer.
    // Every wave waits at one barrier per step, LA products before the
    // step's end: by then its copies of the next step have landed, so after
    // it every wave may read the next step, and every wave has read all of
    // the previous step, whose buffer the step after the next one reuses.
    auto iteration = [&](int t, auto mask_tag) {
        const int j0 = t * BC;
        f32x16_t sa[2], da[2];

        // One column step as a software pipeline: S, dP of key half 0, then
        // of half 1; in the last step (S and dP complete) half 0 is
        // exponentiated under half 1's products, and the two dQ sums follow
        // in four 16-key steps (the first two while half 1 is
        // exponentiated); a dQ step's K~^T fragment feeds both sums.
        // Fragments are read LA steps ahead; sched_barrier keeps that order.
        // Only tiles that cross Nk or reach past a wave's first row take the
        // mask.
        auto step = [&](auto cs_tag, auto mask_tag) {
            constexpr int CS = decltype(cs_tag)::value;
            constexpr bool LAST = CS == NC - 1;
            constexpr bool MASK = decltype(mask_tag)::value;
            constexpr int NOPS = LAST ? 2 * NSD + 4 * NB : 2 * NSD;
            static_assert(NOPS % (LA + 1) == 0, "the fragment ring must wrap at a step's end");
            static_assert(LA < 2 * NSD, "the next step's first fragments are S/dP fragments");
            constexpr int EPO_A = 16 / NSD;
            constexpr int EPO_B = 16 / (2 * NB);
            // the step staged meanwhile and its parts
            constexpr int NCS = LAST ? 0 : CS + 1;
            constexpr int NPART = (NCS == NC - 1 ? 3 : 2) * PPT;
            static_assert(NPART <= NSD, "the copies go among the first S/dP products");
            const int nt = LAST ? t + 1 : t;
            const int sidx = t * NC + CS;
            const int cur = sidx % NBUF;
            const int nxt = (cur == NBUF - 1) ? -(NBUF - 1) * BUF : BUF;   // to the next buffer

            float pv[16], ev[16];
            u32x4_t pf[4], ef[4];
            auto softmax_elem = [&](int jb, int r) {
                const int j = j0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
                float p = fast_exp2(__builtin_fmaf(sa[jb][r], c, -lse2));
                if (MASK && (j >= Nk || (CAUSAL && j > qi + off))) p = 0.f;
                const float e = p * da[jb][r];
                if constexpr (!DK) dsum += e;
                pv[r] = p;
                ev[r] = e;
                if ((r & 7) == 7) {
                    const int h = r >> 3, rb = 8 * h;
                    if constexpr (!DK)
                        pf[2 * jb + h] = u32x4_t{pack_f16x2(pv[rb + 0], pv[rb + 1]), pack_f16x2(pv[rb + 2], pv[rb + 3]),
                                                 pack_f16x2(pv[rb + 4], pv[rb + 5]), pack_f16x2(pv[rb + 6], pv[rb + 7])};
                    ef[2 * jb + h] = u32x4_t{pack_f16x2(ev[rb + 0], ev[rb + 1]), pack_f16x2(ev[rb + 2], ev[rb + 3]),
                                             pack_f16x2(ev[rb + 4], ev[rb + 5]), pack_f16x2(ev[rb + 6], ev[rb + 7])};
                }
            };

#pragma unroll
            for (int o = 0; o < NOPS; ++o) {
                if (o == NOPS - LA) {
                    // this wave's copies of the next step have landed; after
                    // the barrier everyone's have
                    wait_copies();
                    step_barrier();
                }
                if (o + LA < NOPS) fr[(o + LA) % (LA + 1)] = frag(o + LA, 0);
                else fr[(o + LA) % (LA + 1)] = frag(o + LA - NOPS, nxt);
                const u32x4_t a = fr[o % (LA + 1)];
                if (o < 2 * NSD) {
                    const int jb = o / NSD, w = o % NSD, st = w >> 1;
                    f32x16_t& acc = (w & 1) ? da[jb] : sa[jb];
                    const u32x4_t& bop = (w & 1) ? of[CS * KS + st] : qf[CS * KS + st];
                    // A chain's last product of a step carries the wait
                    // states a VALU read of its result needs.
                    if (CS == 0 && st == 0) {
                        if (w & 1) mfma_bf16_first_c<WS>(acc, a, bop, dinit);
                        else mfma_bf16_first<WS>(acc, a, bop);
                    } else if (st == KS - 1) {
                        mfma_bf16_last<WS>(acc, a, bop);
                    } else {
                        mfma_bf16_next<WS>(acc, a, bop);
                    }
                    if (LAST && jb == 1) {
#pragma unroll
                        for (int e = 0; e < EPO_A; ++e) softmax_elem(0, w * EPO_A + e);
                    }
                } else {
                    const int w = o - 2 * NSD, t4 = w / NB, nb = w % NB;
                    mfma_f16_agpr(acc_a[nb], a, ef[t4]);
                    if constexpr (!DK) mfma_f16_agpr(acc_b[nb], a, pf[t4]);
                    if (t4 < 2) {
#pragma unroll
                        for (int e = 0; e < EPO_B; ++e) softmax_elem(1, w * EPO_B + e);
                    }
                }
                // The next step's copies, among the first S/dP products
                // (VALU-free in every step), well before the barrier.
#pragma unroll
                for (int k = 0; k < NPART; ++k)
                    if (o == k * NSD / NPART) stage_part(nt, NCS, (cur + 1) % NBUF, k);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the bases move to the next buffer
#pragma unroll
            for (int k = 0; k < 16; ++k) pb[k] += nxt;
        };
        step(IntTag<0>{}, mask_tag);
        if constexpr (NC > 1) step(IntTag<1>{}, mask_tag);
    };
    // Tiles from t_mask on cross Nk or reach past the key position of the
    // block's first row (a wave whose rows all precede such a tile computes
    // it fully masked).
    const int first_free = q0 + off + 1;       // keys below this are seen by every row
    const int t_mask = min(CAUSAL ? (first_free > 0 ? first_free / BC : 0) : n_tiles, Nk / BC);
    for (int t = 0; t < min(t_mask, n_tiles); ++t) iteration(t, BoolTag<false>{});
    for (int t = max(t_mask, 0); t < n_tiles; ++t) iteration(t, BoolTag<true>{});

#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        agpr_settle(acc_a[nb]);
        if constexpr (!DK) agpr_settle(acc_b[nb]);
    }
    const float dt = DK ? 0.f : sum_with_partner32(dsum);    // D~ = sE * (D - D^)
    if (part == 0 && g == 0 && qi < T * 64) {
        float* st = stats + ((size_t)bh * T + (qi >> 6)) * 128;
        st[qi & 63] = lse2;
        st[64 + (qi & 63)] = (qi < N) ? -(dhs + dt) : 0.f;   // -sE * D
    }
    if (qi < N) {
        const float f = scale / (sK * sE);
        uint16_t* row = dQ + head + (size_t)qi * DT + D * part;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float x[4];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int r = 4 * q4 + r4;
                    x[r4] = DK ? f * acc_a[nb][r] : f * __builtin_fmaf(-dt, acc_b[nb][r], acc_a[nb][r]);
                }
                u32x2_t w;
                w[0] = pack_bf16x2(x[0], x[1]);
                w[1] = pack_bf16x2(x[2], x[3]);
                *(u32x2_t*)(row + 32 * nb + 8 * q4 + 4 * g) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// Phase 3: dK, dV. One workgroup per block of NW*32 keys; each wave owns 32
// keys (one per lane pair) and walks the query tiles (64 rows) that see them.
// Products (lane = key column j, registers = query rows i):
//   S   = Q K^T              A = Q tile (LDS, bf16)         B = K^T (VGPRs)
//   dP  = dO V^T             A = dO tile (LDS, bf16)        B = V^T (VGPRs)
//   dV^T += dO~^T P          A = (s_dO dO)^T (LDS, fp16)    B = P (fp16)
//   dK^T += Q~^T dS~         A = (s_Q Q)^T (LDS, fp16)      B = dS~ = P (sE dP - sE D)
// A head size DT above 128 runs as NC = DT/128 column parts, as in the dQ
// pass: each query tile is staged as NC steps of 128 columns of Q and dO, S
// and dP accumulate over all of them, and each workgroup forms the dK and dV
// columns of one part.
// ---------------------------------------------------------------------------
template <int DT, int NW, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64, 1)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ scales, const float* __restrict__ stats,
                const char* __restrict__ qt_img, const char* __restrict__ ot_img,
                uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BHkv, int G, int N,
                int Nk, int T, float c, float scale) {
    constexpr int D = DT > 128 ? 128 : DT;  // columns of one staged tile and of one dK/dV part
    constexpr int NC = DT / D;
    // Above d = 128 the parked K and V fill the AGPR file with the sums: the
    // compiler then copies some of them into AGPRs just before their
    // products, which carry the VALU-write wait states.
    constexpr bool WS = DT > 128;
    constexpr int BQ = 64;
    constexpr int BKV = NW * 32;
    constexpr int KS = D / 16;
    constexpr int KST = DT / 16;
    constexpr int NB = D / 32;
    constexpr int TB = 64 * D * 2;
    constexpr int BLK = TB / 1024;
    // LDS: two buffers of row-major Q and dO tiles (read by the S and dP
    // products; one per column step), two of transposed images (read by the
    // dV and dK products; one per query tile) and three of statistics. The
    // row-major and image buffers turn over at different points of a step,
    // which is what lets one barrier per step, between the S/dP and the
    // gradient products, serve both (see the loop below).
    constexpr int OFF_Q = 0, OFF_DO = TB;        // within a row-major buffer
    constexpr int OFF_QT = 0, OFF_DOT = TB;      // within an image buffer
    // (A statistics copy fills 1 KB of LDS: 512 bytes of values, then the
    // lanes past them repeat the last chunk.)
    constexpr int RBUF = 2 * TB, IBUF = 2 * TB, TBUF = 1024;
    constexpr int OFF_R = 0, OFF_I = 2 * RBUF, OFF_T = 2 * RBUF + 2 * IBUF;
    __shared__ __attribute__((aligned(16))) char smem[OFF_T + 3 * TBUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int bid = blockIdx.x;
    const int bkv = bid % BHkv;           // K/V head
    const int part = (bid / BHkv) % NC;   // dK, dV columns [D part, D part + D)
    const int kb = bid / (BHkv * NC);     // low key blocks see the most queries: first
    const size_t head = (size_t)bkv * (size_t)Nk * DT;
    const int qh0 = bkv * G;              // its first query head; the group is qh0 .. qh0+G-1

    // One factor each for Q and dO serves the whole group of query heads.
    const float sQ = scales[qh0 * 4 + 0];
    const float sV = scales[qh0 * 4 + 2], sDO = scales[qh0 * 4 + 3];
    const float sE = sDO * sV;

    const int k0 = kb * BKV;
    const int kw0 = k0 + wave * 32;
    const int kj = kw0 + l32;             // this lane's key
    const int off = Nk - N;               // query row i sits at key position i + off
    const int kq = kj - off;              // causal: the first query row that sees key kj

    u32x4_t kf[KST], vf[KST];
#pragma unroll
    for (int s = 0; s < KST; ++s) {
        if (kj < Nk) {
            kf[s] = *(const u32x4_t*)(K + head + (size_t)kj * DT + 16 * s + 8 * g);
            vf[s] = *(const u32x4_t*)(V + head + (size_t)kj * DT + 16 * s + 8 * g);
        } else {
            kf[s] = vf[s] = u32x4_t{0u, 0u, 0u, 0u};
        }
        park_in_agprs(kf[s]);
        park_in_agprs(vf[s]);
    }

    f32x16_t acc_dk[NB], acc_dv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_dk[nb][r] = acc_dv[nb][r] = 0.f;

    const int n_tiles = (N + BQ - 1) / BQ;
    // Causal: query tiles before t0 see no key of this block (t0 may reach
    // n_tiles: then no query sees it and dK = dV = 0).
    const int t0 = CAUSAL ? min(max(k0 - off, 0) / BQ, n_tiles) : 0;

    // Column step cs of query tile t of group member gq (query head qh0 + gq):
    // stage_r puts its Q and dO rows (bf16, swizzled) into row-major buffer
    // rb, stage_i the tile's two transposed fp16 images (this part's columns)
    // into image buffer ib, BLK 1 KB blocks each spread over the NW waves
    // (part k is one block of this wave); stage_stats the tile's 128
    // statistics into statistics buffer sb (wave 0). Tiles past the last of
    // the last member are filled from a valid tile and never read.
    constexpr int PPT = BLK / NW;
    auto live_head = [&](int gq, int t) -> size_t {
        return (size_t)(qh0 + ((gq < G && t < n_tiles) ? gq : 0));
    };
    auto live_tile = [&](int gq, int t) -> size_t { return (size_t)((gq < G && t < n_tiles) ? t : 0); };
    auto stage_r = [&](int gq, int t, int cs, int rb, int k) {
        lds_char* base = (lds_char*)(smem + OFF_R + rb * RBUF);
        const int tensor = k / PPT, b = wave + NW * (k % PPT);
        const size_t qh = live_head(gq, t), ti = live_tile(gq, t);
        stage_tile_block_async<D, DT>((tensor == 0 ? Q : dO) + qh * N * DT + cs * D,
                                      base + (tensor == 0 ? OFF_Q : OFF_DO), (int)ti * BQ, N, b,
                                      lane);
    };
    auto stage_i = [&](int gq, int t, int ib, int k) {
        lds_char* base = (lds_char*)(smem + OFF_I + ib * IBUF);
        const int tensor = k / PPT, b = wave + NW * (k % PPT);
        const size_t qh = live_head(gq, t), ti = live_tile(gq, t);
        stage_image_block_full_async(
            (tensor == 0 ? qt_img : ot_img) + ((qh * T + ti) * NC + part) * TB,
            base + (tensor == 0 ? OFF_QT : OFF_DOT), b, lane);
    };
    auto stage_stats = [&](int gq, int t, int sb) {
        lds_char* base = (lds_char*)(smem + OFF_T + sb * TBUF);
        const size_t qh = live_head(gq, t), ti = live_tile(gq, t);
        if (wave == 0) stage_image_block_async(stats + (qh * T + ti) * 128, 512, base, 0, lane);
    };
    // The query tile after (gq, t): the member's next tile, else the next
    // member's first.
    auto next_tile = [&](int& gq, int& t) {
        if (t + 1 < n_tiles) {
            ++t;
        } else {
            ++gq;
            t = t0;
        }
    };

    // Lane-dependent LDS bases: pb[k], k < 8, for the row-major S/dP
    // fragments of row-major buffer 0 (chunk step s; for d = 64 also the
    // query half) and pb[8 + 2 t4 + (nb & 1)] for the transposed dV/dK
    // fragments of image buffer 0; everything else in a fragment address is
    // a compile-time offset, so each read is one ds_read with an immediate
    // offset from a base moved once per step (row-major) or per query tile
    // (images, statistics).
    lds_char* const s0 = (lds_char*)smem;
    lds_char* pb[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int ib = (D == 64) ? k / KS : 0, st = (D == 64) ? k % KS : k;
        pb[k] = s0 + OFF_R + row_chunk_offset<D>(32 * ib + l32, 2 * st + g);
        pb[8 + k] = s0 + OFF_I + tr_slot_offset(32 * (k & 1) + l32, 2 * (2 * (k >> 1) + g));
    }
    lds_char* pst = s0 + OFF_T + 16 * g;

    constexpr int NSD = 2 * KS;
    constexpr int NG = 2 * NB;
    constexpr int LA = kDkdvFragAhead;
    // Fragment o of a step (o < 2 NSD: S/dP fragments in product order, from
    // the row-major buffer `dr` bytes past the current one; then the dV/dK
    // fragments from the current image buffer).
    auto frag = [&](int o, int dr) -> u32x4_t {
        if (o < 2 * NSD) {
            const int ib = o / NSD, w = o % NSD, st = w >> 1;
            const int k = (D == 64) ? ib * KS + st : st;
            const int off = ((w & 1) ? OFF_DO : OFF_Q) + ((D == 64) ? 0 : ib * 32 * D * 2);
            return *(const lds_u32x4_t*)(pb[k] + dr + off);
        }
        const int w = o - 2 * NSD, t4 = w / NG, nb = (w % NG) >> 1;
        const int off = ((w & 1) ? OFF_QT : OFF_DOT) + (nb - (nb & 1)) * 32 * 128;
        return *(const lds_u32x4_t*)(pb[8 + 2 * t4 + (nb & 1)] + off);
    };

    // Prologue: the first two column steps' rows, the first tile's images
    // and statistics (and, with one step per tile, the second tile's
    // statistics): everything read before the first step's barrier or right
    // after it.
    {
        int g1 = 0, t1 = t0;
        next_tile(g1, t1);
#pragma unroll
        for (int k = 0; k < 2 * PPT; ++k) {
            stage_r(0, t0, 0, 0, k);
            if (NC == 1) stage_r(g1, t1, 0, 1, k);
            else stage_r(0, t0, 1, 1, k);
            stage_i(0, t0, 0, k);
        }
        stage_stats(0, t0, 0);
        if (NC == 1) stage_stats(g1, t1, 1);
    }
    // (the copies are not visible to the compiler: wait for them explicitly)
    wait_copies();
    __syncthreads();
    // The fragment ring, carried from step to step: product o of a step
    // takes fr[o % (LA + 1)], and the first LA fragments of the next step
    // are read during the last LA products of this one.
    u32x4_t fr[LA + 1];
#pragma unroll
    for (int o = 0; o < LA; ++o) fr[o] = frag(o, 0);

    // One query tile of group member gq: NC column steps. Step s (counting
    // column steps from the first) has one barrier, LA products before its
    // last S/dP product. Before it each wave waits for its own copies and
    // for its LDS reads of the row-major buffer; so after it the next step's
    // rows, this tile's images and the next tile's statistics have landed
    // for every wave, and no wave reads step s's rows any more. Then each
    // wave copies step s + 2's rows into step s's row-major buffer and, in
    // the last step of a tile, the next tile's images into the other image
    // buffer (the previous tile's, finished in the previous step) and the
    // statistics of the tile that step s + 2 belongs to into the third
    // statistics buffer. The fragment reads run on through the barrier (the
    // dV/dK fragments of this step) and into the next step.
    const int nt = n_tiles - t0;
    auto iteration = [&](int gq, int t, auto mask_tag) {
        const int i0 = t * BQ;
        const int L = gq * nt + t - t0;    // query tiles before this one
        int ga = gq, ta = t;               // the next tile
        next_tile(ga, ta);
        int gb = ga, tb = ta;              // the one after
        next_tile(gb, tb);
        f32x16_t sa[2], da[2];

        // One column step as a software pipeline: S, dP of query half 0, then
        // of half 1; in the last step (S and dP complete) half 0 is
        // exponentiated under half 1's products, then dV, dK run over four
        // 16-query steps (the first two while half 1 is exponentiated). Each
        // product's LDS fragment is read LA products ahead; sched_barrier
        // keeps that order. Only tiles that reach above a wave's first key
        // take the causal mask.
        auto step = [&](auto cs_tag, auto mask_tag) {
            constexpr int CS = decltype(cs_tag)::value;
            constexpr bool LAST = CS == NC - 1;
            constexpr bool MASK = decltype(mask_tag)::value;
            constexpr int NOPS = LAST ? 2 * NSD + 4 * NG : 2 * NSD;
            static_assert(NOPS % (LA + 1) == 0, "the fragment ring must wrap at a step's end");
            static_assert(LA < 2 * NSD, "the barrier falls among the S/dP products");
            constexpr int EPO_A = 16 / NSD;
            constexpr int EPO_B = 16 / (2 * NG);
            constexpr int OB = 2 * NSD - LA;      // the barrier, before product OB
            // Copies after the barrier: in the VALU-free dV/dK products of a
            // last step, else among the products left after the barrier.
            constexpr int O0 = LAST ? 2 * NSD + 2 * NG : OB;
            constexpr int NPR = 2 * PPT;          // row-major parts of a step
            constexpr int NPI = LAST ? 2 * PPT : 0;
            constexpr int NPART = NPR + NPI;
            const int sidx = L * NC + CS;
            const int rcur = sidx & 1;
            const int rnxt = rcur ? -RBUF : RBUF;  // to the other row-major buffer
            // Step s + 2: the same column step of the tile after the next
            // (one step per tile) or of the next tile.
            const int g2 = NC == 1 ? gb : ga, t2 = NC == 1 ? tb : ta;

            f32x4_t l4[4], d4[4];     // lse*log2e and -sE*D of the half being exponentiated
            float pv[16], dsv[16];
            u32x4_t pp[4], dsp[4];
            auto read_stats = [&](int ib, int q4) {
                l4[q4] = *(const lds_f32x4_t*)(pst + (32 * ib + 8 * q4) * 4);
                d4[q4] = *(const lds_f32x4_t*)(pst + 256 + (32 * ib + 8 * q4) * 4);
            };
            auto softmax_elem = [&](int ib, int r) {
                const int q4 = r >> 2, r4 = r & 3;
                float p = fast_exp2(__builtin_fmaf(sa[ib][r], c, -l4[q4][r4]));
                if (MASK && kq > i0 + 32 * ib + 8 * q4 + 4 * g + r4) p = 0.f;
                pv[r] = p;
                dsv[r] = p * __builtin_fmaf(da[ib][r], sE, d4[q4][r4]);
                if (ib == 0 && r4 == 3) read_stats(1, q4);
                if ((r & 7) == 7) {
                    const int h = r >> 3, rb = 8 * h;
                    pp[2 * ib + h] = u32x4_t{pack_f16x2(pv[rb + 0], pv[rb + 1]), pack_f16x2(pv[rb + 2], pv[rb + 3]),
                                             pack_f16x2(pv[rb + 4], pv[rb + 5]), pack_f16x2(pv[rb + 6], pv[rb + 7])};
                    dsp[2 * ib + h] = u32x4_t{pack_f16x2(dsv[rb + 0], dsv[rb + 1]), pack_f16x2(dsv[rb + 2], dsv[rb + 3]),
                                              pack_f16x2(dsv[rb + 4], dsv[rb + 5]), pack_f16x2(dsv[rb + 6], dsv[rb + 7])};
                }
            };

#pragma unroll
            for (int o = 0; o < NOPS; ++o) {
                if (o == OB) {
                    wait_copies();
                    wait_lds();
                    step_barrier();
                }
                if (o + LA < NOPS) fr[(o + LA) % (LA + 1)] = frag(o + LA, 0);
                else fr[(o + LA) % (LA + 1)] = frag(o + LA - NOPS, rnxt);
                const u32x4_t a = fr[o % (LA + 1)];
                if (LAST && o == 0) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) read_stats(0, q4);
                }
                if (o < 2 * NSD) {
                    const int ib = o / NSD, w = o % NSD, st = w >> 1;
                    f32x16_t& acc = (w & 1) ? da[ib] : sa[ib];
                    const u32x4_t& bop = (w & 1) ? vf[CS * KS + st] : kf[CS * KS + st];
                    // A chain's last product of a step carries the wait
                    // states a VALU read of its result needs.
                    if (CS == 0 && st == 0) mfma_bf16_first<WS>(acc, a, bop);
                    else if (st == KS - 1) mfma_bf16_last<WS>(acc, a, bop);
                    else mfma_bf16_next<WS>(acc, a, bop);
                    if (LAST && ib == 1) {
#pragma unroll
                        for (int e = 0; e < EPO_A; ++e) softmax_elem(0, w * EPO_A + e);
                    }
                } else {
                    const int w = o - 2 * NSD, t4 = w / NG, nb = (w % NG) >> 1;
                    if (w & 1) mfma_f16_agpr(acc_dk[nb], a, dsp[t4]);
                    else mfma_f16_agpr(acc_dv[nb], a, pp[t4]);
                    if (t4 < 2) {
#pragma unroll
                        for (int e = 0; e < EPO_B; ++e) softmax_elem(1, w * EPO_B + e);
                    }
                }
#pragma unroll
                for (int k = 0; k < NPART; ++k)
                    if (o == O0 + k * (NOPS - O0) / NPART) {
                        if (k < NPR) stage_r(g2, t2, CS, rcur, k);
                        else stage_i(ga, ta, (L + 1) & 1, k - NPR);
                    }
                if (LAST && o == O0 + 1) stage_stats(g2, t2, (L + (NC == 1 ? 2 : 1)) % 3);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the row-major bases move to the other buffer; after a tile's
            // last step the image and statistics bases move to the next tile's
#pragma unroll
            for (int k = 0; k < 8; ++k) pb[k] += rnxt;
            if constexpr (LAST) {
                const int inxt = (L & 1) ? -IBUF : IBUF;
#pragma unroll
                for (int k = 8; k < 16; ++k) pb[k] += inxt;
                pst += (L % 3 == 2) ? -2 * TBUF : TBUF;
            }
        };
        step(IntTag<0>{}, mask_tag);
        if constexpr (NC > 1) step(IntTag<1>{}, mask_tag);
    };
    // Causal: only tiles whose first row precedes the block's last key
    // position reach above some wave's keys (two tiles when Nq = Nk; a wave
    // whose keys all follow such a tile computes it fully masked).
    // dK and dV sum over the G query heads that share this K/V head.
    const int last_kq = k0 + BKV - 1 - off;
    const int t_free = CAUSAL ? min(max((max(last_kq, 0) + BQ - 1) / BQ, t0), n_tiles) : t0;
    for (int gq = 0; gq < G; ++gq) {
        for (int t = t0; t < t_free; ++t) iteration(gq, t, BoolTag<true>{});
        for (int t = t_free; t < n_tiles; ++t) iteration(gq, t, BoolTag<false>{});
    }

#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        agpr_settle(acc_dk[nb]);
        agpr_settle(acc_dv[nb]);
    }
    if (kj < Nk) {
        const float fk = scale / (sQ * sE), fv = 1.f / sDO;
        uint16_t* dkrow = dK + head + (size_t)kj * DT + D * part;
        uint16_t* dvrow = dV + head + (size_t)kj * DT + D * part;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                u32x2_t wk, wv;
                wk[0] = pack_bf16x2(acc_dk[nb][4 * q4 + 0] * fk, acc_dk[nb][4 * q4 + 1] * fk);
                wk[1] = pack_bf16x2(acc_dk[nb][4 * q4 + 2] * fk, acc_dk[nb][4 * q4 + 3] * fk);
                wv[0] = pack_bf16x2(acc_dv[nb][4 * q4 + 0] * fv, acc_dv[nb][4 * q4 + 1] * fv);
                wv[1] = pack_bf16x2(acc_dv[nb][4 * q4 + 2] * fv, acc_dv[nb][4 * q4 + 3] * fv);
                *(u32x2_t*)(dkrow + 32 * nb + 8 * q4 + 4 * g) = wk;
                *(u32x2_t*)(dvrow + 32 * nb + 8 * q4 + 4 * g) = wv;
            }
    }
}

// 16x16x32 product with bf16 operands, or fp16 with F16.
template <bool F16>
__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// A operand of a 32x32x16 product taken transposed from a row-major 16-bit
// tile (rows r, 16-byte chunks swizzled as tr_rows_swizzle): lane l gets
// column c0 + l%32 of rows r0 + 8 (l/32) .. +7, in row order; two
// ds_read_b64_tr_b16. Within a group of 16 lanes, ds_read_b64_tr_b16 returns
// to lane i element e of the 8 bytes addressed by lane 4e + i/4, at position
// i%4; so lane i addresses row base + i/4, columns cb + 4 (i%4) .. +3, with
// cb = c0 + 16 ((l/16) % 2) and base = r0 + 8 (l/32) (then + 4).
template <int D>
__device__ __forceinline__ int rows_tr_offset(int r0, int c0, int lane, int half) {
    const int i = lane & 15;
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
    return rows_offset<D, true>(r0 + (i >> 2) + 4 * half, col >> 3) + ((col & 7) << 1);
}
// The two reads at byte addresses p1, p2 of LDS.
__device__ __forceinline__ u32x4_t tr_frag_at(const lds_char* p1, const lds_char* p2) {
    const i16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p1);
    const i16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p2);
    const u32x2_t ux = __builtin_bit_cast(u32x2_t, x), uy = __builtin_bit_cast(u32x2_t, y);
    return u32x4_t{ux[0], ux[1], uy[0], uy[1]};
}
template <int D>
__device__ __forceinline__ u32x4_t rows_tr_frag(const lds_char* tile, int r0, int c0, int lane) {
    return tr_frag_at(tile + rows_tr_offset<D>(r0, c0, lane, 0), tile + rows_tr_offset<D>(r0, c0, lane, 1));
}

// Waves of the pass below: one per SIMD with 64 keys per wave or at d = 256,
// two per SIMD with 32 keys per wave at d <= 128.
constexpr int dkdv16_waves(int D, int KW) { return D == 256 ? 4 : 256 / KW; }

// ---------------------------------------------------------------------------
// Phase 3 with 16-row steps: dK, dV. For head sizes 64 and 128, KW = 64 keys
// per wave (4 waves, one per SIMD) or 32 (8 waves, two per SIMD), one
// workgroup per block of 256 keys, query tiles of 64 rows (four steps). At
// d = 256, 32 keys per wave (4 waves, one per SIMD: the dK and dV sums of all
// 256 columns take the 256 AGPRs, the resident K and V 128 VGPRs), one
// workgroup per block of 128 keys, query tiles of 32 rows (two steps, so that
// a tile's rows and images, 64 KiB, are double-buffered in LDS): S and dP are
// formed once for all 256 columns of dK and dV. Each workgroup walks the
// query tiles that see its keys in 16-row steps, so every LDS fragment feeds
// several products (the 32-key form above reads a fresh fragment for each):
//   S, dP (16 queries x KW keys): 16x16x32 products, A = a 16-row slice of
//     the Q (dO) rows from LDS, read once for the KW/16 key blocks; B = K^T
//     (V^T), resident in VGPRs. With TR the rows are the fp16 copies of s_Q Q
//     and s_dO dO and the products fp16 against fp16 s_K K and s_V V;
//     otherwise bf16. Accumulator lane l: key 16j + l%16, queries 4(l/16) ..
//     +3.
//   P and dS = P (sE dP - sE D) are formed there and packed to fp16 (dS as
//     the packed fp16 product of the fp16 P and the fp16 sE (dP - D): one
//     conversion and one v_pk_mul_f16 per pair of scores), and one
//     v_permlane16_swap per pair of registers brings each lane the eight
//     queries 8g .. 8g+7 (g = l/32) of key l%32 of a 32-key block: the B
//     operand layout of the 32x32x16 product.
//   dV^T += dO~^T P, dK^T += Q~^T dS~ (32 dims x 32 keys per product, fp16,
//     AGPR accumulators), A = the 16-query slice of dO~ (Q~) transposed: with
//     TR read from the fp16 rows by ds_read_b64_tr_b16, otherwise from a
//     transposed fp16 image staged beside the rows; read once for the wave's
//     32-key blocks.
// Step s's softmax runs between the products of step s-1's dV/dK. Every
// query tile is staged whole (double-buffered) with one barrier per tile.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int KW, bool TR>
__global__ void __launch_bounds__(dkdv16_waves(D, KW) * 64, 1)
bwd_dkdv16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                  const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                  const float* __restrict__ scales, const float* __restrict__ stats,
                  const char* __restrict__ qt_img, const char* __restrict__ ot_img,
                  uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BHkv, int G, int N,
                  int Nk, int T, float c, float scale) {
    static_assert(D == 64 || D == 128 || (D == 256 && KW == 32),
                  "the dK, dV sums and the resident K, V of a wave fit its registers");
    static_assert(KW == 64 || KW == 32, "keys per wave");
    constexpr int NW = dkdv16_waves(D, KW);   // 4 (one per SIMD) or 8 (two per SIMD)
    constexpr int NJ = KW / 16;          // 16-key blocks of a wave
    constexpr int NH = KW / 32;          // 32-key blocks of a wave
    constexpr int BQ = D == 256 ? 32 : 64;    // query rows per tile
    constexpr int NSTEP = BQ / 16;       // 16-row steps per tile
    constexpr int BKV = NW * KW;         // keys per workgroup
    constexpr int KC = D / 32;           // 32-wide contraction chunks of S and dP
    constexpr int NB = D / 32;           // 32-wide row blocks of dV^T and dK^T
    constexpr int TB = BQ * D * 2;       // bytes of one tile (rows or image)
    constexpr int BLK = TB / 1024;       // its 1 KB copy blocks
    constexpr int PPT = BLK / NW;        // blocks per wave and tensor
    // TR: the tile is the fp16 rows of s_Q Q and s_dO dO only, and the dV, dK
    // products read their transposed operands from them (ds_read_b64_tr_b16);
    // otherwise the bf16 rows of Q and dO, then their transposed fp16 images.
    constexpr int NT = TR ? 2 : 4;       // tensors per tile
    constexpr int OFF_Q = 0, OFF_DO = TB, OFF_QT = 2 * TB, OFF_DOT = 3 * TB;
    // Fragment addresses formed once per tile (below)
    constexpr bool PRE = TR && FA_DKDV_PRE != 0;
    constexpr int BUF = NT * TB;
    // A statistics copy fills 1 KB of LDS (512 bytes of values, then lanes
    // repeating the last chunk).
    constexpr int SBUF = 1024;
    constexpr int OFF_S = 2 * BUF;
    __shared__ __attribute__((aligned(16))) char smem[2 * BUF + 2 * SBUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;   // 16x16 products: key l16, query rows 4 q4 ..
    const int g = lane >> 5, l32 = lane & 31;    // 32x32 products
    const int bid = blockIdx.x;
    const int bkv = bid % BHkv;                  // K/V head
    const int kb = bid / BHkv;                   // low key blocks see the most queries: first
    const size_t head = (size_t)bkv * (size_t)Nk * D;
    const int qh0 = bkv * G;

    const float sQ = scales[qh0 * 4 + 0], sK = scales[qh0 * 4 + 1];
    const float sV = scales[qh0 * 4 + 2], sDO = scales[qh0 * 4 + 3];
    const float sE = sDO * sV;
    // TR: S is formed from s_Q Q and s_K K (powers of two), so the exponent
    // factor takes them out.
    const float cS = TR ? c / (sQ * sK) : c;

    const int k0 = kb * BKV;
    const int kw0 = k0 + wave * KW;
    const int off = Nk - N;                      // query row i sits at key position i + off

    // K^T and V^T operands of the 16x16x32 products: bf16 K and sE V (sE a
    // power of two, so sE V is exact), or with TR fp16 of s_K K and s_V V
    // (exact copies: the factors put the largest magnitude in [1/2, 1)). Keys
    // past Nk read key Nk-1, whose gradients are not stored.
    u32x4_t kr[KC][NJ], vr[KC][NJ];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const size_t row = (size_t)min(kw0 + 16 * j + l16, Nk - 1);
            const u32x4_t k = *(const u32x4_t*)(K + head + row * D + 32 * kc + 8 * q4);
            const u32x4_t v = *(const u32x4_t*)(V + head + row * D + 32 * kc + 8 * q4);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                kr[kc][j][w] = TR ? bf16x2_to_f16x2(k[w], sK) : k[w];
                vr[kc][j][w] = TR ? bf16x2_to_f16x2(v[w], sV) : bf16x2_scale(v[w], sE);
            }
        }

    // dV^T, dK^T of the wave's 32-key blocks (AGPRs)
    f32x16_t acc_dv[NH][NB], acc_dk[NH][NB];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_dv[h][nb][r] = acc_dk[h][nb][r] = 0.f;

    const int n_tiles = (N + BQ - 1) / BQ;
    const int t0 = CAUSAL ? min(max(k0 - off, 0) / BQ, n_tiles) : 0;

    auto live_head = [&](int gq, int t) -> size_t {
        return (size_t)(qh0 + ((gq < G && t < n_tiles) ? gq : 0));
    };
    auto live_tile = [&](int gq, int t) -> size_t { return (size_t)((gq < G && t < n_tiles) ? t : 0); };
    // Part k (< 4 PPT) of query tile (gq, t) into buffer b: Q rows, dO rows,
    // the Q~^T image, the dO~^T image, PPT 1 KB blocks each per wave. A tile
    // past the last is filled from a valid one and never read. (Copies that
    // the compiler does not see as LDS writes; the barrier at each tile's
    // start, after every wave has waited for its own copies and for its LDS
    // reads of the buffer's previous tile, orders them.)
    auto stage = [&](int gq, int t, int b, int k) {
        lds_char* base = (lds_char*)(smem + b * BUF);
        const int tensor = k / PPT, blk = wave + NW * (k % PPT);
        const size_t qh = live_head(gq, t), ti = live_tile(gq, t);
        if (TR)   // fp16 rows: [T * 64][D] per query head
            stage_tile_block_async<D, D, true>((const uint16_t*)(tensor == 0 ? qt_img : ot_img) +
                                             qh * (size_t)(T * 64) * D,
                                         base + (tensor == 0 ? OFF_Q : OFF_DO), (int)ti * BQ, N,
                                         blk, lane);
        else if (tensor < 2)
            stage_tile_block_async<D, D>((tensor == 0 ? Q : dO) + qh * N * D,
                                         base + (tensor == 0 ? OFF_Q : OFF_DO), (int)ti * BQ, N,
                                         blk, lane);
        else
            stage_image_block_full_async((tensor == 2 ? qt_img : ot_img) + (qh * (T * 64 / BQ) + ti) * TB,
                                         base + (tensor == 2 ? OFF_QT : OFF_DOT), blk, lane);
    };
    // (statistics are kept per 64-row tile: a 32-row tile takes half of one)
    auto stage_stats = [&](int gq, int t, int b) {
        const size_t qh = live_head(gq, t), ti = live_tile(gq, t);
        if (wave == 0)
            stage_image_block_async(stats + (qh * T + ti * BQ / 64) * 128, 512,
                                    (lds_char*)(smem + OFF_S + b * SBUF), 0, lane);
    };
    // Query tiles run from the last down: the workgroups of one K/V head
    // that run together (on one XCD) then read the same tile at about the
    // same time, whatever their first tile, and share it through L2.
    auto next_tile = [&](int& gq, int& t) {
        if (t > t0) {
            --t;
        } else {
            ++gq;
            t = n_tiles - 1;
        }
    };

    // Byte offset of 16-byte chunk c (rows 8c .. 8c+7 of the tile) of row n
    // of a transposed image.
    auto img_offset = [](int n, int c) -> int {
        return D == 256 ? img32_offset(n, c) : tr_slot_offset(n, 2 * c);
    };

    // One query tile of group member gq, buffer b, as one fully unrolled
    // sequence of fragment operations. Step s (16 query rows) has three
    // segments:
    //   A(s): S(s) = Q K^T, fragments Q(kc), four 16x16x32 products each;
    //         under it the swaps of step s-1 into the B operands.
    //   B(s): dP(s) - D = dO V~^T - D (V~ = sE V; the chain starts from
    //         -sE D), fragments dO(kc).
    //   C(s): dV and dK of step s-1, fragments dO~^T(nb), Q~^T(nb), two
    //         32x32x16 products each; under them P(s) = exp2(S c - lse)
    //         (written over S), dS(s) = P (dP - D) and the fp16 packing of
    //         P(s) and dS(s). (A 32x32x16 product leaves room for a few vector
    //         instructions; the 16x16x32 products of A and B hardly any.)
    // Step 0's C has no products (its vector work runs alone) and step 3's dV,
    // dK follow the last C. The swaps write the B operands only after the
    // products that read the previous ones have issued (a matrix product
    // reads A and B when it issues). Each fragment is read LA operations
    // ahead through a ring of registers that starts again at every tile.
    // Causal runs mask the tiles that reach above some of the block's keys,
    // on S at the end of each step's A segment, behind a uniform branch: two
    // copies of this code (masked and not) do not fit the registers together.
    constexpr int NS = KC, NGR = 2 * NB;
    constexpr int NOPS = NSTEP * (2 * NS) + NSTEP * NGR;
    // (look-ahead 3 at d = 256, where 128 keys per workgroup leave the
    // registers for it; 2 otherwise)
    constexpr int LA = D == 256 ? 3 : 2;
    // Operation o: kind (0 Q, 1 dO, 2 dO~^T, 3 Q~^T), step, chunk or block.
    struct Op { int kind, s, x; };
    auto op_of = [](int o) constexpr -> Op {
        // per step s < 3: A(s) NS, B(s) NS, then grad(s-1) NGR for s >= 1;
        // finally grad(3)
        int base = 0;
        for (int s = 0; s < NSTEP; ++s) {
            if (o < base + NS) return Op{0, s, o - base};
            base += NS;
            if (o < base + NS) return Op{1, s, o - base};
            base += NS;
            if (s >= 1) {
                if (o < base + NGR) return Op{2 + ((o - base) & 1), s - 1, (o - base) >> 1};
                base += NGR;
            }
        }
        return Op{2 + ((o - base) & 1), NSTEP - 1, (o - base) >> 1};
    };
    auto tile = [&](int gq, int t, int b, bool mask_tile) {
        const int i0 = t * BQ;
        // (the tile's rows within its 64-row statistics block)
        const lds_char* st = (lds_char*)smem + OFF_S + b * SBUF + 4 * ((t * BQ) & 63);
        int ga = gq, ta = t;
        next_tile(ga, ta);
        f32x4_t sa[NJ], da[NJ];         // S then P, and dP - D, of the current step
        u32x4_t pk[NH], dk2[NH];        // B operands (P, dS) of the 32-key blocks
        float lse4[4];
        f32x4_t dinit;                  // -sE D of the step's four rows
        uint32_t pp[NJ][2], dp[NJ][2];  // packed P, dS of the 16-key blocks
        // Causal: key kw0 + 16 j + l16 is above query row i0 + 16 s + 4 q4 + i
        // when dlt > 16 (s - j) + i.
        const int dlt = kw0 + l16 - i0 - 4 * q4 - off;

        // PRE: the lane's fragment addresses of step 0 and of the first (up
        // to) four 32-column blocks in this tile's buffer, once per tile. The
        // row swizzle depends on a row's four low bits only (and for rows of
        // 256 bytes or more acts on a chunk's four low bits), so a step's
        // rows lie a constant 16 rows further and column block x + 4 a
        // constant 256 bytes further: each read is one instruction with an
        // immediate offset. Pinned, so that they are kept rather than rebuilt
        // at every read.
        constexpr int NXS = NS < 4 ? NS : 4, NXB = NB < 4 ? NB : 4;
        int pr[PRE ? NXS : 1], pt[PRE ? NXB : 1][2];
        if constexpr (PRE) {
#pragma unroll
            for (int x = 0; x < NXS; ++x) {
                pr[x] = b * BUF + rows_offset<D, TR>(l16, 4 * x + q4);
                keep_here(pr[x]);
            }
#pragma unroll
            for (int x = 0; x < NXB; ++x)
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    pt[x][k] = b * BUF + rows_tr_offset<D>(8 * g, 32 * x, lane, k);
                    keep_here(pt[x][k]);
                }
        }
        auto frag = [&](int o) -> u32x4_t {
            const Op op = op_of(o);
            const lds_char* base = (lds_char*)smem + b * BUF;
            if constexpr (PRE) {
                const lds_char* s0 = (lds_char*)smem + 16 * op.s * (D * 2) + 256 * (op.x >> 2);
                if (op.kind < 2)
                    return *(const lds_u32x4_t*)(s0 + pr[op.x & 3] + (op.kind == 0 ? OFF_Q : OFF_DO));
                const int t0 = op.kind == 2 ? OFF_DO : OFF_Q;
                return tr_frag_at(s0 + pt[op.x & 3][0] + t0, s0 + pt[op.x & 3][1] + t0);
            }
            if (op.kind < 2)
                return *(const lds_u32x4_t*)(base + (op.kind == 0 ? OFF_Q : OFF_DO) +
                                             rows_offset<D, TR>(16 * op.s + l16, 4 * op.x + q4));
            if (TR)   // dims 32 x + l32, rows 16 s + 8 g .. +7, from the rows
                return rows_tr_frag<D>(base + (op.kind == 2 ? OFF_DO : OFF_Q), 16 * op.s + 8 * g,
                                       32 * op.x, lane);
            return *(const lds_u32x4_t*)(base + (op.kind == 2 ? OFF_DOT : OFF_QT) +
                                         img_offset(32 * op.x + l32, 2 * op.s + g));
        };
        auto load_stats = [&](int s) {
            const f32x4_t a = *(const lds_f32x4_t*)(st + 4 * (16 * s + 4 * q4));
            const f32x4_t d = *(const lds_f32x4_t*)(st + 4 * (64 + 16 * s + 4 * q4));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lse4[i] = a[i];
                dinit[i] = d[i];
            }
        };
        // P of step s, key block j, over S: element (j, i) is key kw0 + 16 j +
        // l16 and query row i0 + 16 s + 4 q4 + i.
        auto exp_block = [&](int j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sa[j][i] = fast_exp2(__builtin_fmaf(sa[j][i], cS, -lse4[i]));
        };
        // Causal tiles that reach above some of the keys: S of step s set to
        // -inf there (so that P = 0), all key blocks behind one uniform
        // branch. The empty assembly gives each step's comparisons an operand
        // of their own: equal thresholds of different steps would otherwise
        // be merged into comparisons ahead of the first branch, on the path
        // of the tiles that need no mask.
        auto mask_step = [&](int s) {
            if (CAUSAL && mask_tile) {
                int dl = dlt;
                asm volatile("" : "+v"(dl));
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (dl > 16 * (s - j) + i) sa[j][i] = kNegInf;
            }
        };
        // dS = P (dP - D) of key block j, and both packed to fp16
        auto ds_block = [&](int j) {
            pp[j][0] = pack_f16x2(sa[j][0], sa[j][1]);
            pp[j][1] = pack_f16x2(sa[j][2], sa[j][3]);
            // (from the fp16 P: one conversion and one packed product per
            // pair instead of two products and a conversion)
            dp[j][0] = mul_f16x2(pp[j][0], pack_f16x2(da[j][0], da[j][1]));
            dp[j][1] = mul_f16x2(pp[j][1], pack_f16x2(da[j][2], da[j][3]));
        };
        // Key blocks 2h, 2h+1 -> the 32-key block h in the 32x32 B layout.
        auto swap_block = [&](int h) {
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const auto rp = __builtin_amdgcn_permlane16_swap(pp[2 * h][w], pp[2 * h + 1][w],
                                                                 false, false);
                const auto rd = __builtin_amdgcn_permlane16_swap(dp[2 * h][w], dp[2 * h + 1][w],
                                                                 false, false);
                pk[h][w] = rp[0];
                pk[h][2 + w] = rp[1];
                dk2[h][w] = rd[0];
                dk2[h][2 + w] = rd[1];
            }
        };

        u32x4_t fr[LA + 1];
#pragma unroll
        for (int o = 0; o < LA; ++o) fr[o] = frag(o);
        load_stats(0);
#pragma unroll
        for (int o = 0; o < NOPS; ++o) {
            const Op op = op_of(o);
            if (o + LA < NOPS) fr[(o + LA) % (LA + 1)] = frag(o + LA);
            const u32x4_t a = fr[o % (LA + 1)];
            if (op.kind == 0) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (op.x == 0) sa[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    sa[j] = mfma16x16x32<TR>(a, kr[op.x][j], sa[j]);
                }
                // A(s): the swaps of step s-1
                if (op.s >= 1 && op.x == 0) swap_block(0);
                if (NH > 1 && op.s >= 1 && op.x == NS - 1) swap_block(NH - 1);
                if (op.x == NS - 1) mask_step(op.s);
            } else if (op.kind == 1) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (op.x == 0) da[j] = dinit;
                    da[j] = mfma16x16x32<TR>(a, vr[op.x][j], da[j]);
                }
                if (op.x == NS - 1 && op.s == 0) {
                    // C(0): no products to run under
#pragma unroll
                    for (int j = 0; j < NJ; ++j) exp_block(j);
#pragma unroll
                    for (int j = 0; j < NJ; ++j) ds_block(j);
                    load_stats(1);
                }
            } else {
                if (op.kind == 2) {
#pragma unroll
                    for (int h = 0; h < NH; ++h) mfma_f16_agpr(acc_dv[h][op.x], a, pk[h]);
                } else {
#pragma unroll
                    for (int h = 0; h < NH; ++h) mfma_f16_agpr(acc_dk[h][op.x], a, dk2[h]);
                }
                // C(s) = grad(s-1): P, dS and packing of step s = op.s + 1, one
                // key block's exponentials after each dO~^T operation's
                // products and its dS after the following Q~^T operation's
                if (op.s < NSTEP - 1) {
                    const int sn = op.s + 1;
#pragma unroll
                    for (int j = op.x * NJ / NB; j < (op.x + 1) * NJ / NB; ++j) {
                        if (op.kind == 2) exp_block(j);
                        else ds_block(j);
                    }
                    if (op.kind == 3 && op.x == NB - 1 && sn < NSTEP - 1) load_stats(sn + 1);
                }
                // before the last step's grad: its swaps (no S segment follows)
                if (op.s == NSTEP - 2 && op.kind == 3 && op.x == NB - 1) {
#pragma unroll
                    for (int h = 0; h < NH; ++h) swap_block(h);
                }
            }
            // the next tile's copies, one every third operation from the fourth on
#pragma unroll
            for (int k = 0; k < NT * PPT; ++k)
                if (o == 3 + 3 * k) stage(ga, ta, b ^ 1, k);
            if (o == 4) stage_stats(ga, ta, b ^ 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Causal: tiles whose first row precedes the block's last key position
    // reach above some of its keys.
    const int last_kq = k0 + BKV - 1 - off;
    const int t_free = CAUSAL ? min(max((max(last_kq, 0) + BQ - 1) / BQ, t0), n_tiles) : t0;
    if (t0 < n_tiles) {
#pragma unroll
        for (int k = 0; k < NT * PPT; ++k) stage(0, n_tiles - 1, 0, k);
        stage_stats(0, n_tiles - 1, 0);
        int L = 0;
        for (int gq = 0; gq < G; ++gq) {
            for (int t = n_tiles - 1; t >= t0; --t, ++L) {
                // this wave's copies of tile L have landed and its reads of
                // tile L-1 are done; after the barrier everyone's are
                wait_copies();
                wait_lds();
                step_barrier();
                tile(gq, t, L & 1, t < t_free);
            }
        }
        wait_copies();
    }

#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            agpr_settle(acc_dk[h][nb]);
            agpr_settle(acc_dv[h][nb]);
        }
    const float fk = scale / (sQ * sE), fv = 1.f / sDO;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int kj = kw0 + 32 * h + l32;
        if (kj < Nk) {
            uint16_t* dkrow = dK + head + (size_t)kj * D;
            uint16_t* dvrow = dV + head + (size_t)kj * D;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u32x2_t wk, wv;
                    wk[0] = pack_bf16x2(acc_dk[h][nb][4 * q + 0] * fk, acc_dk[h][nb][4 * q + 1] * fk);
                    wk[1] = pack_bf16x2(acc_dk[h][nb][4 * q + 2] * fk, acc_dk[h][nb][4 * q + 3] * fk);
                    wv[0] = pack_bf16x2(acc_dv[h][nb][4 * q + 0] * fv, acc_dv[h][nb][4 * q + 1] * fv);
                    wv[1] = pack_bf16x2(acc_dv[h][nb][4 * q + 2] * fv, acc_dv[h][nb][4 * q + 3] * fv);
                    *(u32x2_t*)(dkrow + 32 * nb + 8 * q + 4 * g) = wk;
                    *(u32x2_t*)(dvrow + 32 * nb + 8 * q + 4 * g) = wv;
                }
        }
    }
}

// Waves of the pass below: one per SIMD with 64 rows per wave or at d = 256,
// two per SIMD with 32 rows per wave at d <= 128.
constexpr int dq16_waves(int D, int QW) { return D == 256 ? 4 : 256 / QW; }

// ---------------------------------------------------------------------------
// Phase 2 with 16-row steps, when D is known before the pass (formed by the
// preprocess from O and its rounding residual): dQ, the dK/dV pass above with
// the roles of queries and keys exchanged. For head sizes 64 and 128, QW = 64
// query rows per wave (4 waves, one per SIMD) or 32 (8 waves, two per SIMD),
// one workgroup per block of 256 query rows, key tiles of 64 keys (four
// steps). At d = 256, 32 rows per wave (4 waves, one per SIMD), one workgroup
// per block of 128 rows, key tiles of 32 keys (two steps, so that a tile's K
// and V rows and its K~^T image, 48 KiB, are double-buffered in LDS): S and
// dP are formed once for all 256 columns of dQ. Each workgroup walks the key
// tiles its rows see in 16-key steps:
//   S, dP (16 keys x QW queries): v_mfma_f32_16x16x32_bf16, A = a 16-row
//     slice of the K (V) tile from LDS, read once for the QW/16 query blocks;
//     B = Q^T ((sE dO)^T), resident in VGPRs. Accumulator lane l: query
//     16j + l%16, keys 4(l/16) .. +3 of the step.
//   dS = P (sE dP - sE D) is formed there (the dP chain starts from -sE D),
//     packed to fp16, and one v_permlane16_swap per pair of registers brings
//     each lane the eight keys 8g .. 8g+7 (g = l/32) of query l%32 of a
//     32-query block: the B operand layout of the 32x32x16 product.
//   dQ^T += K~^T dS~ (32 dims x 32 queries per product, fp16, AGPR
//     accumulators), A = the 16-key slice of K~ transposed, read once for the
//     wave's 32-query blocks: at d <= 128 from the transposed K~ image (rows
//     in their own order), at d = 256 (TR) from the fp16 rows of s_K K by
//     ds_read_b64_tr_b16, the same rows that S then takes (fp16 products
//     against fp16 s_Q Q).
// lse and D belong to a lane's query columns and are loaded once. Step s's
// dS runs between the products of step s-1's dQ. Every key tile is staged
// whole (double-buffered) with one barrier per tile. The pass also leaves lse
// and D per query tile for the dK/dV pass.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int QW, bool TR>
__global__ void __launch_bounds__(dq16_waves(D, QW) * 64, 1)
bwd_dq16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ LSE, const float* __restrict__ scales,
                const float* __restrict__ dvals, const char* __restrict__ kt_img,
                float* __restrict__ stats, uint16_t* __restrict__ dQ,
                uint16_t* __restrict__ q_rows, uint16_t* __restrict__ do_rows, int BH, int G,
                int N, int Nk, int T, int Tk, float c, float scale, int nqb) {
    static_assert(D == 64 || D == 128 || (D == 256 && QW == 32),
                  "the dQ sums and the resident Q, dO of a wave fit its registers");
    static_assert(QW == 64 || QW == 32, "query rows per wave");
    constexpr int NW = dq16_waves(D, QW);     // 4 (one per SIMD) or 8 (two per SIMD)
    constexpr int NJ = QW / 16;          // 16-query blocks of a wave
    constexpr int NH = QW / 32;          // 32-query blocks of a wave
    constexpr int BC = D == 256 ? 32 : 64;    // keys per tile
    constexpr int NSTEP = BC / 16;       // 16-key steps per tile
    constexpr int BQ = NW * QW;          // query rows per workgroup
    constexpr int KC = D / 32;           // 32-wide contraction chunks of S and dP
    constexpr int NB = D / 32;           // 32-wide row blocks of dQ^T
    constexpr int TB = BC * D * 2;       // bytes of one tile (rows or image)
    constexpr int BLK = TB / 1024;       // its 1 KB copy blocks
    constexpr int PPT = BLK / NW;        // blocks per wave and tensor
    // TR: the tile is the fp16 rows of s_K K and the bf16 rows of V, and the
    // dQ product reads its transposed K operand from the first
    // (ds_read_b64_tr_b16); otherwise K and V rows, then the K~^T image.
    constexpr int NT = TR ? 2 : 3;       // tensors per tile
    constexpr int OFF_K = 0, OFF_V = TB, OFF_KT = 2 * TB;
    // Fragment addresses formed once per tile (below)
    constexpr bool PRE = TR && D == 256 && FA_DKDV_PRE != 0;
    constexpr bool PREI = !TR && D <= 128 && FA_DKDV_PRE != 0;
    constexpr int BUF = NT * TB;
    __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q4 = lane >> 4;   // 16x16 products: query l16, keys 4 q4 ..
    const int g = lane >> 5, l32 = lane & 31;    // 32x32 products
    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qbi = bid / BH;
    const int qb = CAUSAL ? (nqb - 1 - qbi) : qbi;   // causal: longest blocks first
    const size_t head = (size_t)bh * (size_t)N * D;
    const size_t kvhead = (size_t)(bh / G) * (size_t)Nk * D;  // K/V head of this query head
    const uint16_t* Kh = K + kvhead;
    const uint16_t* Vh = V + kvhead;
    // (TR: [Tk * 64][D] fp16 rows per K/V head; otherwise tile images)
    const char* kt_h = kt_img + (size_t)(bh / G) * (TR ? (size_t)Tk * 64 * D * 2 : (size_t)(Tk * 64 / BC) * TB);
    const int q0 = qb * BQ;
    const int qw0 = q0 + wave * QW;
    const int off = Nk - N;              // query row i sits at key position i + off

    const float sQ = scales[bh * 4 + 0], sK = scales[bh * 4 + 1];
    const float sV = scales[bh * 4 + 2], sDO = scales[bh * 4 + 3];
    const float sE = sDO * sV;
    // TR: S is formed from s_Q Q and s_K K (powers of two), so the exponent
    // factor takes them out.
    const float cS = TR ? c / (sQ * sK) : c;

    // Q^T and (sE dO)^T operands of the 16x16x32 products (rows past N read
    // row N-1: finite values whose probabilities are 0 and whose dQ is not
    // stored), and the statistics of the lane's four query columns. Rows
    // past N, and rows that see no key (lse = -inf), take +inf as lse log2 e:
    // each of their probabilities is then exactly 0.
    u32x4_t qr[KC][NJ], orr[KC][NJ];
    float lse2[NJ], dhs[NJ];
    f32x4_t dinit[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int qi = qw0 + 16 * j + l16;
        const size_t row = (size_t)min(qi, N - 1);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const u32x4_t qv = *(const u32x4_t*)(Q + head + row * D + 32 * kc + 8 * q4);
#pragma unroll
            for (int w = 0; w < 4; ++w) qr[kc][j][w] = TR ? bf16x2_to_f16x2(qv[w], sQ) : qv[w];
            const u32x4_t v = *(const u32x4_t*)(dO + head + row * D + 32 * kc + 8 * q4);
#pragma unroll
            for (int w = 0; w < 4; ++w) orr[kc][j][w] = bf16x2_scale(v[w], sE);
            // The fp16 rows of s_Q Q and s_dO dO for the dK/dV pass ([T * 64][D]
            // per head). (Not at d = 64: there the code takes registers that
            // two waves per SIMD need.)
            if (D >= 128 && q_rows != nullptr && qi < N) {
                const size_t at = ((size_t)bh * T * 64 + qi) * D + 32 * kc + 8 * q4;
                u32x4_t fq, fo;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    fq[w] = TR ? qr[kc][j][w] : bf16x2_to_f16x2(qv[w], sQ);
                    fo[w] = bf16x2_to_f16x2(v[w], sDO);
                }
                *(u32x4_t*)(q_rows + at) = fq;
                *(u32x4_t*)(do_rows + at) = fo;
            }
        }
        const float lse_i = (qi < N) ? LSE[(size_t)bh * N + qi] : kNegInf;
        lse2[j] = (lse_i == kNegInf) ? __builtin_huge_valf() : lse_i * kLog2e;
        dhs[j] = (qi < N) ? sE * dvals[(size_t)bh * N + qi] : 0.f;
        dinit[j] = f32x4_t{-dhs[j], -dhs[j], -dhs[j], -dhs[j]};
    }

    // dQ^T of the wave's 32-query blocks (AGPRs)
    f32x16_t acc[NH][NB];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[h][nb][r] = 0.f;

    const int n_all = (Nk + BC - 1) / BC;
    const int q_last = min(q0 + BQ, N) - 1 + off;      // last key position of the block
    const int n_tiles = CAUSAL ? min(n_all, max(q_last, 0) / BC + 1) : n_all;
    // Tiles from t_mask on cross Nk or reach past the key position of the
    // block's first row (a wave whose rows all precede such a tile computes
    // it fully masked).
    const int first_free = q0 + off + 1;       // keys below this are seen by every row
    const int t_mask = min(CAUSAL ? (first_free > 0 ? first_free / BC : 0) : n_tiles, Nk / BC);

    // Part k (< 3 PPT) of key tile t into buffer b: K rows, V rows, the K~^T
    // image, PPT 1 KB blocks each per wave. A tile past the last is filled
    // from tile 0 and never read. (Copies that the compiler does not see as
    // LDS writes; the barrier at each tile's start, after every wave has
    // waited for its own copies and for its LDS reads of the buffer's
    // previous tile, orders them.)
    auto stage = [&](int t, int b, int k) {
        lds_char* base = (lds_char*)(smem + b * BUF);
        const int tensor = k / PPT, blk = wave + NW * (k % PPT);
        const int ti = t < n_tiles ? t : 0;
        if (TR && tensor == 0)
            stage_tile_block_async<D, D, true>((const uint16_t*)kt_h, base + OFF_K, ti * BC, Nk, blk,
                                               lane);
        else if (tensor < 2)
            stage_tile_block_async<D, D>(tensor == 0 ? Kh : Vh, base + (tensor == 0 ? OFF_K : OFF_V),
                                         ti * BC, Nk, blk, lane);
        else
            stage_image_block_full_async(kt_h + (size_t)ti * TB, base + OFF_KT, blk, lane);
    };

    // One key tile in buffer b as one fully unrolled sequence of fragment
    // operations. Step s (16 keys) has three segments:
    //   A(s): S(s) = K Q^T, fragments K(kc), four 16x16x32 products each;
    //         under it the swaps of step s-1 into the B operands.
    //   B(s): dP(s) - D = V~ (sE dO)^T - sE D, fragments V(kc).
    //   C(s): dQ of step s-1, fragments K~^T(nb), two 32x32x16 products
    //         each; under them P(s) = exp2(S c - lse) and dS(s) = P (dP - D)
    //         with its fp16 packing, one 16-query block per operation (d =
    //         128) or two (d = 64).
    // Step 0's C has no products (its vector work runs alone) and step 3's dQ
    // follows the last C. Each fragment is read LA operations ahead through a
    // ring of registers that starts again at every tile. Tiles that need a
    // mask run it on S at the end of each step's A segment, behind a uniform
    // branch.
    constexpr int NS = KC, NGR = NB;
    constexpr int NOPS = NSTEP * (2 * NS) + NSTEP * NGR;
    constexpr int LA = 2;
    static_assert(3 + 3 * (NT * PPT - 1) < NOPS, "the next tile's copies fit in the operations");
    // Operation o: kind (0 K, 1 V, 2 K~^T), step, chunk or block.
    struct Op { int kind, s, x; };
    auto op_of = [](int o) constexpr -> Op {
        int base = 0;
        for (int s = 0; s < NSTEP; ++s) {
            if (o < base + NS) return Op{0, s, o - base};
            base += NS;
            if (o < base + NS) return Op{1, s, o - base};
            base += NS;
            if (s >= 1) {
                if (o < base + NGR) return Op{2, s - 1, o - base};
                base += NGR;
            }
        }
        return Op{2, NSTEP - 1, o - base};
    };
    // Byte offset of 16-byte chunk c (keys 8c .. 8c+7 of the tile) of row n of
    // the K~^T image.
    auto img_offset = [](int n, int c) -> int {
        return D == 256 ? img32_offset(n, c) : kt_step_offset<D>(n, c);
    };
    auto tile = [&](int t, int b, bool mask_tile) {
        const int j0 = t * BC;
        f32x4_t sa[NJ], da[NJ];         // S then P, and dP - D, of the current step
        u32x4_t ds2[NH];                // B operands (dS) of the 32-query blocks
        uint32_t dp[NJ][2];             // packed dS of the 16-query blocks
        // key j0 + 16 s + 4 q4 + i against query qw0 + 16 j + l16: masked when
        // past Nk, or (causal) when dlt + 16 (s - j) + i > 0
        const int dlt = j0 + 4 * q4 - qw0 - l16 - off;
        const int kq = j0 + 4 * q4;

        // PRE (d = 256): the lane's fragment addresses of step 0 and of the
        // first four 32-column blocks in this tile's buffer, once per tile,
        // as in the dK/dV pass (rows of 512 bytes: a step's rows lie 16 rows
        // further, column block x + 4 256 bytes further). Pinned.
        // PREI (d <= 128): the lane's K~^T image address of step 0, row
        // block 0 (kt_step_offset), and at d = 128 its K and V row addresses
        // of step 0 (the row swizzle of 256-byte rows acts on a row's four low
        // bits, so a step's rows lie 16 rows further). Pinned.
        int pr_[PREI && D == 128 ? 4 : 1], pim = 0;
        if constexpr (PREI) {
            pim = b * BUF + OFF_KT + kt_step_offset<D>(l32, g);
            keep_here(pim);
            if constexpr (D == 128) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    pr_[x] = b * BUF + row_chunk_offset<D>(l16, 4 * x + q4);
                    keep_here(pr_[x]);
                }
            }
        }
        int pk_[PRE ? 4 : 1], pv_[PRE ? 4 : 1], pt[PRE ? 4 : 1][2];
        if constexpr (PRE) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                pk_[x] = b * BUF + OFF_K + rows_offset<D, TR>(l16, 4 * x + q4);
                pv_[x] = b * BUF + OFF_V + row_chunk_offset<D>(l16, 4 * x + q4);
                keep_here(pk_[x]);
                keep_here(pv_[x]);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    pt[x][k] = b * BUF + OFF_K + rows_tr_offset<D>(8 * g, 32 * x, lane, k);
                    keep_here(pt[x][k]);
                }
            }
        }
        auto fragment = [&](int o) -> u32x4_t {
            const Op op = op_of(o);
            const lds_char* base = (lds_char*)smem + b * BUF;
            if constexpr (PRE) {
                const lds_char* s0 = (lds_char*)smem + 16 * op.s * (D * 2) + 256 * (op.x >> 2);
                if (op.kind == 0) return *(const lds_u32x4_t*)(s0 + pk_[op.x & 3]);
                if (op.kind == 1) return *(const lds_u32x4_t*)(s0 + pv_[op.x & 3]);
                return tr_frag_at(s0 + pt[op.x & 3][0], s0 + pt[op.x & 3][1]);
            }
            if constexpr (PREI) {
                if (op.kind == 2)
                    return *(const lds_u32x4_t*)((lds_char*)smem + pim + op.s * (32 * D) + op.x * 1024);
                if constexpr (D == 128)
                    return *(const lds_u32x4_t*)((lds_char*)smem + 16 * op.s * (D * 2) + pr_[op.x] +
                                                 (op.kind == 0 ? OFF_K : OFF_V));
            }
            if (op.kind == 0)
                return *(const lds_u32x4_t*)(base + OFF_K +
                                             rows_offset<D, TR>(16 * op.s + l16, 4 * op.x + q4));
            if (op.kind == 1)
                return *(const lds_u32x4_t*)(base + OFF_V +
                                             row_chunk_offset<D>(16 * op.s + l16, 4 * op.x + q4));
            if (TR)   // dims 32 x + l32, keys 16 s + 8 g .. +7, from the K rows
                return rows_tr_frag<D>(base + OFF_K, 16 * op.s + 8 * g, 32 * op.x, lane);
            return *(const lds_u32x4_t*)(base + OFF_KT + img_offset(32 * op.x + l32, 2 * op.s + g));
        };
        // P of query block j (over S), then dS = P (dP - D) packed
        auto ds_block = [&](int j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sa[j][i] = fast_exp2(__builtin_fmaf(sa[j][i], cS, -lse2[j]));
            dp[j][0] = pack_f16x2(sa[j][0] * da[j][0], sa[j][1] * da[j][1]);
            dp[j][1] = pack_f16x2(sa[j][2] * da[j][2], sa[j][3] * da[j][3]);
        };
        // Tiles that need a mask: S of step s set to -inf where masked (so
        // that P = 0), all query blocks behind one uniform branch. The empty
        // assembly gives each step's comparisons operands of their own:
        // equal thresholds of different steps would otherwise be merged into
        // comparisons ahead of the first branch, on the path of the tiles
        // that need no mask.
        auto mask_step = [&](int s) {
            if (mask_tile) {
                int kl = Nk - kq, dl = dlt;
                asm volatile("" : "+v"(kl), "+v"(dl));
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (16 * s + i >= kl || (CAUSAL && dl + 16 * (s - j) + i > 0)) sa[j][i] = kNegInf;
            }
        };
        // Query blocks 2h, 2h+1 -> the 32-query block h in the 32x32 B layout.
        auto swap_block = [&](int h) {
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const auto rd = __builtin_amdgcn_permlane16_swap(dp[2 * h][w], dp[2 * h + 1][w],
                                                                 false, false);
                ds2[h][w] = rd[0];
                ds2[h][2 + w] = rd[1];
            }
        };

        u32x4_t fr[LA + 1];
#pragma unroll
        for (int o = 0; o < LA; ++o) fr[o] = fragment(o);
#pragma unroll
        for (int o = 0; o < NOPS; ++o) {
            const Op op = op_of(o);
            if (o + LA < NOPS) fr[(o + LA) % (LA + 1)] = fragment(o + LA);
            const u32x4_t a = fr[o % (LA + 1)];
            if (op.kind == 0) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (op.x == 0) sa[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    sa[j] = mfma16x16x32<TR>(a, qr[op.x][j], sa[j]);
                }
                // A(s): the swaps of step s-1
                if (op.s >= 1 && op.x == 0) swap_block(0);
                if (NH > 1 && op.s >= 1 && op.x == NS - 1) swap_block(NH - 1);
                if (op.x == NS - 1) mask_step(op.s);
            } else if (op.kind == 1) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (op.x == 0) da[j] = dinit[j];
                    da[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, orr[op.x][j]),
                        da[j], 0, 0, 0);
                }
                if (op.x == NS - 1 && op.s == 0) {
                    // C(0): no products to run under
#pragma unroll
                    for (int j = 0; j < NJ; ++j) ds_block(j);
                }
            } else {
#pragma unroll
                for (int h = 0; h < NH; ++h) mfma_f16_agpr(acc[h][op.x], a, ds2[h]);
                // C(s) = dQ(s-1): dS of step s = op.s + 1
                if (op.s < NSTEP - 1) {
#pragma unroll
                    for (int j = op.x * NJ / NB; j < (op.x + 1) * NJ / NB; ++j) ds_block(j);
                }
                // before the last step's dQ: its swaps (no S segment follows)
                if (op.s == NSTEP - 2 && op.x == NB - 1) {
#pragma unroll
                    for (int h = 0; h < NH; ++h) swap_block(h);
                }
            }
            // the next tile's copies, one every third operation from the fourth on
#pragma unroll
            for (int k = 0; k < NT * PPT; ++k)
                if (o == 3 + 3 * k) stage(t + 1, b ^ 1, k);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

#pragma unroll
    for (int k = 0; k < NT * PPT; ++k) stage(0, 0, k);
    for (int t = 0; t < n_tiles; ++t) {
        // this wave's copies of tile t have landed and its reads of tile t-1
        // are done; after the barrier everyone's are
        wait_copies();
        wait_lds();
        step_barrier();
        tile(t, t & 1, t >= t_mask);
    }
    wait_copies();

#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) agpr_settle(acc[h][nb]);
    // lse log2 e and -sE D of the wave's rows, into their query tile
    const int tq = qw0 >> 6;
    if (q4 == 0 && tq < T) {
        float* st = stats + ((size_t)bh * T + tq) * 128 + (qw0 & 63);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            st[16 * j + l16] = lse2[j];
            st[64 + 16 * j + l16] = -dhs[j];
        }
    }
    const float f = scale / (sK * sE);
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int qi = qw0 + 32 * h + l32;
        if (qi < N) {
            uint16_t* row = dQ + head + (size_t)qi * D;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u32x2_t w;
                    w[0] = pack_bf16x2(acc[h][nb][4 * q + 0] * f, acc[h][nb][4 * q + 1] * f);
                    w[1] = pack_bf16x2(acc[h][nb][4 * q + 2] * f, acc[h][nb][4 * q + 3] * f);
                    *(u32x2_t*)(row + 32 * nb + 8 * q + 4 * g) = w;
                }
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers (arguments already validated by the C-ABI layer).
// ---------------------------------------------------------------------------
constexpr int kBwdWaves = 4;

static BwdWorkspace ws_of(const BwdArgs& a) {
    return bwd_workspace_layout(a.B, a.H, a.Hkv, a.N, a.Nk, a.d);
}

template <typename T>
static T* ws_ptr(const BwdArgs& a, size_t off) { return (T*)((char*)a.workspace + off); }

static int q_tiles64(const BwdArgs& a) { return (a.N + 63) / 64; }
// The dK/dV pass with 16-row steps (bwd_dkdv16_kernel): for head sizes up to
// 128 (256-key workgroups) when its grid still has two workgroups per compute
// unit of an MI355X, at d = 256 (128-key workgroups) when it has one;
// otherwise (few K/V heads or short sequences, where large key blocks leave
// the longest causal block alone at the end, or at d = 256 too few
// workgroups to fill the chip without the column parts) the 128-key pass.
// The preprocess lays the Q and dO images out for the pass chosen here.
static bool use_dkdv16(const BwdArgs& a) {
    if (a.d == 256) return (long long)((a.Nk + 127) / 128) * a.B * a.Hkv >= 256;
    return (long long)((a.Nk + 255) / 256) * a.B * a.Hkv >= 512;
}
// The dQ pass with 16-row steps (bwd_dq16_kernel): D known, and for head sizes
// up to 128 (256-row workgroups) at least 512 workgroups, at d = 256 (128-row
// workgroups) at least 256 (smaller grids keep more workgroups per compute
// unit with the 128-row pass, and at d = 256 its column parts).
static bool use_dq16(const BwdArgs& a) {
    if (!a.d_known) return false;
    if (a.d == 256) return (long long)((a.N + 127) / 128) * a.B * a.H >= 256;
    return (long long)((a.N + 255) / 256) * a.B * a.H >= 512;
}
static int k_tiles64(const BwdArgs& a) { return (a.Nk + 63) / 64; }
// The fp16 rows of s_Q Q and s_dO dO that the dK/dV pass with 16-row steps
// reads are written by the dQ pass with 16-row steps, which loads those rows
// anyway, when both passes run at d = 128 or 256 (otherwise by the image pass:
// at d = 64 the store code takes registers that two dQ waves per SIMD need).
static bool rows_from_dq(const BwdArgs& a) {
    return FA_ROWS_FROM_DQ != 0 && FA_DKDV_TR != 0 && a.d >= 128 && use_dq16(a) && use_dkdv16(a);
}
// Column parts of a head (128 columns each above d = 128).
static int col_parts(int d) { return d > 128 ? d / 128 : 1; }

template <int D>
static hipError_t launch_prepare_t(const BwdArgs& a) {
    const BwdWorkspace w = ws_of(a);
    const int BH = a.B * a.H, BHkv = a.B * a.Hkv, G = a.H / a.Hkv;
    const int chunks = bwd_scale_chunks(a.N, a.Nk, a.d);
    const int Tq = q_tiles64(a), Tk = k_tiles64(a);
    uint32_t* partial = ws_ptr<uint32_t>(a, w.partial);
    hipLaunchKernelGGL((bwd_absmax_kernel<D>), dim3((BH + BHkv) * chunks), dim3(256), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (const uint16_t*)a.dout, (const uint16_t*)a.o,
                       (const uint16_t*)a.o_res, partial, ws_ptr<float>(a, w.dhat), BH, a.N,
                       a.Nk, chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_scale_kernel, dim3((BH + 63) / 64), dim3(64), 0, a.stream,
                       (const uint32_t*)partial, ws_ptr<float>(a, w.scales), BH, G, chunks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // (the Q and dO rows come from the dQ pass when both passes have 16-row
    // steps: then only the K images are made here)
    const int first = rows_from_dq(a) ? 2 * BH * Tq : 0;
    hipLaunchKernelGGL((bwd_image_kernel<D>),
                       dim3((2 * BH * Tq + BHkv * Tk - first) * col_parts(D)), dim3(256), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.dout, ws_ptr<const float>(a, w.scales),
                       ws_ptr<char>(a, w.qt), ws_ptr<char>(a, w.ot), ws_ptr<char>(a, w.kt), BH,
                       G, a.N, a.Nk, Tq, Tk,
                       (use_dkdv16(a) ? (FA_DKDV_TR ? 4 : 1) : 0) |
                           (use_dq16(a) ? (dq16_tr(D) ? 8 : 2) : 0),
                       first);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dq_t(const BwdArgs& a) {
    constexpr int NW = kBwdWaves;
    const BwdWorkspace w = ws_of(a);
    const int BH = a.B * a.H;
    if (use_dq16(a)) {
        // d = 128: 32 rows per wave, two waves per SIMD (each wave's vector work
        // can run under the other's products); d = 64: 64 rows, one wave per
        // SIMD; d = 256: 32 rows, one wave per SIMD
        constexpr int QW = D == 64 ? 64 : 32;
        constexpr int NWQ = dq16_waves(D, QW);
        const int nqb = (a.N + NWQ * QW - 1) / (NWQ * QW);
        hipLaunchKernelGGL((bwd_dq16_kernel<D, CAUSAL, QW, dq16_tr(D)>), dim3(nqb * BH),
                           dim3(NWQ * 64), 0, a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                           (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse,
                           ws_ptr<const float>(a, w.scales), ws_ptr<const float>(a, w.dhat),
                           ws_ptr<const char>(a, w.kt), ws_ptr<float>(a, w.stats),
                           (uint16_t*)a.dq,
                           rows_from_dq(a) ? ws_ptr<uint16_t>(a, w.qt) : (uint16_t*)nullptr,
                           rows_from_dq(a) ? ws_ptr<uint16_t>(a, w.ot) : (uint16_t*)nullptr,
                           BH, a.H / a.Hkv, a.N, a.Nk, q_tiles64(a),
                           k_tiles64(a), a.scale * kLog2e, a.scale, nqb);
        return hipGetLastError();
    }
    const int nqb = (a.N + NW * 32 - 1) / (NW * 32);
    auto kernel = a.d_known ? bwd_dq_kernel<D, NW, CAUSAL, true>
                            : bwd_dq_kernel<D, NW, CAUSAL, false>;
    hipLaunchKernelGGL(kernel, dim3(nqb * BH * col_parts(D)), dim3(NW * 64), 0, a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse,
                       ws_ptr<const float>(a, w.scales), ws_ptr<const float>(a, w.dhat),
                       ws_ptr<const char>(a, w.kt),
                       ws_ptr<float>(a, w.stats), (uint16_t*)a.dq, BH, a.H / a.Hkv, a.N, a.Nk,
                       q_tiles64(a), k_tiles64(a), a.scale * kLog2e, a.scale, nqb);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dkdv_t(const BwdArgs& a) {
    const BwdWorkspace w = ws_of(a);
    const int BHkv = a.B * a.Hkv;
    if (use_dkdv16(a)) {
        // d <= 128: 256 keys per workgroup; d = 64: 32 keys per wave, two
        // waves per SIMD (each wave's vector work can run under the other's
        // products); d = 128: 64 keys, one wave per SIMD (the dK and dV sums
        // and the resident K and V of 32 keys, 192 registers, leave too few
        // for a second wave). d = 256: 32 keys per wave, one wave per SIMD,
        // 128 keys per workgroup, every column of dK and dV from one pass.
        constexpr int KW = D == 128 ? 64 : 32;
        constexpr int NW = dkdv16_waves(D, KW);
        const int nkb = (a.Nk + NW * KW - 1) / (NW * KW);
        hipLaunchKernelGGL((bwd_dkdv16_kernel<D, CAUSAL, KW, (FA_DKDV_TR != 0)>), dim3(nkb * BHkv),
                           dim3(NW * 64), 0,
                           a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                           (const uint16_t*)a.v, (const uint16_t*)a.dout,
                           ws_ptr<const float>(a, w.scales), ws_ptr<const float>(a, w.stats),
                           ws_ptr<const char>(a, w.qt), ws_ptr<const char>(a, w.ot),
                           (uint16_t*)a.dk, (uint16_t*)a.dv, BHkv, a.H / a.Hkv, a.N, a.Nk,
                           q_tiles64(a), a.scale * kLog2e, a.scale);
    } else {
        constexpr int NW = kBwdWaves;
        const int nkb = (a.Nk + NW * 32 - 1) / (NW * 32);
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, CAUSAL>), dim3(nkb * BHkv * col_parts(D)),
                           dim3(NW * 64), 0,
                           a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                           (const uint16_t*)a.v, (const uint16_t*)a.dout,
                           ws_ptr<const float>(a, w.scales), ws_ptr<const float>(a, w.stats),
                           ws_ptr<const char>(a, w.qt), ws_ptr<const char>(a, w.ot),
                           (uint16_t*)a.dk, (uint16_t*)a.dv, BHkv, a.H / a.Hkv, a.N, a.Nk,
                           q_tiles64(a), a.scale * kLog2e, a.scale);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_prepare(const BwdArgs& a) {
    if (a.d == 256) return launch_prepare_t<256>(a);
    return a.d == 128 ? launch_prepare_t<128>(a) : launch_prepare_t<64>(a);
}

hipError_t launch_bwd_dq(const BwdArgs& a) {
    if (a.d == 256) return a.causal ? launch_dq_t<256, true>(a) : launch_dq_t<256, false>(a);
    if (a.d == 128) return a.causal ? launch_dq_t<128, true>(a) : launch_dq_t<128, false>(a);
    return a.causal ? launch_dq_t<64, true>(a) : launch_dq_t<64, false>(a);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a) {
    if (a.d == 256) return a.causal ? launch_dkdv_t<256, true>(a) : launch_dkdv_t<256, false>(a);
    if (a.d == 128) return a.causal ? launch_dkdv_t<128, true>(a) : launch_dkdv_t<128, false>(a);
    return a.causal ? launch_dkdv_t<64, true>(a) : launch_dkdv_t<64, false>(a);
}

}  // namespace fa
