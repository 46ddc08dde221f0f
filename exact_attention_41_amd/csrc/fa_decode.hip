// Split-K/V decoding for gfx950: a few query rows per head (the last Nq
// positions of a sequence) against a long K/V sequence of Nk keys.
//
// The work is split over the keys, as the inference engines among the
// "FlashAttention-2" page's References (FlashDecoding++, FlashInfer) do, and
// the partial results are
// merged with the two statistics of the online softmax (the "FlashAttention"
// page, systems-analysis.ru, section "Online softmax"): a key range r gives
// the row maximum m_r, the exp-sum l_r and the unnormalised O_r, and
//   m = max_r m_r,  l = sum_r 2^(m_r - m) l_r,  O = sum_r 2^(m_r - m) O_r / l.
//
// Phase 1 (decode_split_kernel): every wave owns one key range of one K/V
// head and all G * Nq query rows that read that head (G query heads per K/V
// head, packed into one 32-row block: G * Nq <= 32). It walks the range in
// 32-key tiles, loading tile t+1 while it computes tile t: K straight from
// global memory into the registers of the MFMA A operand (its fragments are
// row-major 16-byte chunks), V by global-to-LDS loads into the wave's own two
// 8 KiB buffers (row-major, V-type swizzle). It computes S^T = K Q^T on bf16
// MFMA, the masked online softmax in fp32 and O^T += V^T P^T with V^T read
// by transposing LDS reads, and writes (m, l, O) of its range's real query
// rows to the workspace. Waves never wait for each other, and two
// workgroups fit on a compute unit.
// Phase 2 (decode_merge_kernel): one wave per output row merges the ranges
// and writes O (bf16) and the natural-log lse.
//
// The pass is bound by HBM (every K/V byte is read once); the MFMA work is a
// small fraction of its time even with padded query rows.
#include "fa_kernels.hpp"
#include "fa_device.hpp"

namespace fa {

constexpr int kDecWaves = 4;   // waves per workgroup, each with its own key range
constexpr int kDecRows = 32;   // packed query rows per K/V head
constexpr int kDecTile = 32;   // keys per tile

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Compute units of the current device (256 on an MI355X; also the value used
// when no device answers, e.g. for a size query on a host without a GPU).
static long long device_compute_units() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
        (void)hipGetLastError();   // leave no error of this query behind
        return 256;
    }
    return n;
}

DecodeWorkspace decode_workspace_layout(long long B, long long Hkv, long long Nk, long long d) {
    DecodeWorkspace w;
    const long long bhkv = B * Hkv;
    const long long tiles = (Nk + kDecTile - 1) / kDecTile;
    // One round of waves: as many ranges as the compute units hold at once
    // (16, 8 or 4 waves per unit at d = 64, 128, 256: the register and LDS
    // budgets of the split kernel), at least one tile per range. A second
    // round only adds a tail.
    const long long waves = device_compute_units() * (d <= 64 ? 16 : (d <= 128 ? 8 : 4));
    long long ns = (waves + bhkv - 1) / bhkv;
    ns = ns < 1 ? 1 : (ns > tiles ? tiles : ns);
    const long long per = (tiles + ns - 1) / ns;          // tiles per range
    w.split_len = (int)(per * kDecTile);
    w.nsplit = (int)((Nk + w.split_len - 1) / w.split_len);
    const size_t parts = (size_t)bhkv * (size_t)w.nsplit * kDecRows;
    w.part_o = 0;
    w.part_ml = align256(parts * (size_t)d * 4);
    w.total = w.part_ml + align256(parts * 2 * 4);
    return w;
}

// Two workgroups per compute unit for d <= 128; at d = 256 the V buffers
// (128 KiB per workgroup) and the 128-register output block allow one.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kDecWaves * 64, D > 128 ? 1 : 2)
decode_split_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                    const uint16_t* __restrict__ V, float* __restrict__ part_o,
                    float* __restrict__ part_ml, int G, int Nq, int Nk, int L, int nsplit,
                    float c) {
    constexpr int KS = D / 16;
    constexpr int NB = D / 32;
    constexpr int TB = kDecTile * D * 2;     // bytes of one 32-key tile of V
    constexpr int BLK = TB / 1024;           // its 1 KB staging blocks
    // vmcnt encoding of "all but the next tile's loads (KS + BLK) done".
    constexpr int NEXT = KS + BLK;
    constexpr int WAIT_NEXT = (NEXT & 15) | ((NEXT >> 4) << 14) | 0x0F70;
    static_assert(NEXT < 64, "vmcnt holds at most 63");
    __shared__ __attribute__((aligned(16))) char smem[kDecWaves * 2 * TB];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int sp = blockIdx.x * kDecWaves + wave;
    if (sp >= nsplit) return;              // the whole wave: no barrier follows
    const int bkv = blockIdx.y;            // K/V head (batch-major)
    const int M = G * Nq;                  // real query rows; the rest are padding
    const int r = l32;                     // this lane's packed query row
    const int qi = (r < M) ? r % Nq : 0;   // its position among the Nq queries
    const int last_key = Nk - Nq + qi;     // causal: keys j <= last_key are kept
    const uint16_t* Kh = K + (size_t)bkv * Nk * D;
    const uint16_t* Vh = V + (size_t)bkv * Nk * D;
    lds_char* vb0 = (lds_char*)smem + wave * 2 * TB;
    lds_char* vb1 = vb0 + TB;

    u32x4_t qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        if (r < M) {
            const size_t row = (size_t)(bkv * G + r / Nq) * Nq + qi;
            qf[s] = *(const u32x4_t*)(Q + row * D + 16 * s + 8 * g);
        } else {
            qf[s] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }

    f32x16_t acc_o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc_o[nb][e] = 0.f;
    float m_run = kNegInf, l_run = 0.f;    // m in scaled log2 units (score * c)

    const int k_begin = sp * L, k_end = min(k_begin + L, Nk);
    const int k_lim = CAUSAL ? min(k_end, last_key + 1) : k_end;   // keys below this are kept
    // Tile at key j0: V rows into an LDS buffer (rows at or past the range end
    // read the range's last row; they are masked), then K fragments of rows j0 + l32 (clamped into the
    // array; rows at or past the range end are masked) into registers.
    auto issue = [&](int j0, lds_char* vb, u32x4_t (&kf)[KS]) {
        stage_tile_lds<D, BLK, 1, true>(Vh, vb, j0, k_end, 0, lane);
        const size_t row = (size_t)min(j0 + l32, Nk - 1);
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[s] = *(const u32x4_t*)(Kh + row * D + 16 * s + 8 * g);
    };
    auto compute = [&](int j0, const lds_char* vt, const u32x4_t (&kf)[KS]) {
        f32x16_t sa;
#pragma unroll
        for (int e = 0; e < 16; ++e) sa[e] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) sa = mfma_32x32x16(kf[s], qf[s], sa);

        float mt = kNegInf;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = j0 + 8 * (e >> 2) + 4 * g + (e & 3);
            float x = sa[e] * c;
            if (j >= k_lim) x = kNegInf;
            sa[e] = x;
            mt = fmaxf(mt, x);
        }
        mt = max_with_partner32(mt);
        const float m_new = fmaxf(m_run, mt);
        const float mc = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - mc);      // 0 while nothing was kept
        l_run *= alpha;
        // O changes only where the maximum moved: skip the rescale when no
        // row of the wave needs it.
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc_o[nb][e] *= alpha;
        }
        m_run = m_new;

        u32x4_t pp[2];
        {
            float pv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                pv[e] = fast_exp2(sa[e] - mc);
                l_run += pv[e];
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int b = 8 * h;
                pp[h] = u32x4_t{pack_bf16x2(pv[b + 0], pv[b + 1]), pack_bf16x2(pv[b + 2], pv[b + 3]),
                                pack_bf16x2(pv[b + 4], pv[b + 5]), pack_bf16x2(pv[b + 6], pv[b + 7])};
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc_o[nb] = mfma_32x32x16(lds_vt_frag<D>(vt, 32 * nb, h, lane), pp[h], acc_o[nb]);
        // The products above consumed every LDS read of this tile, so its
        // buffer may be refilled.
    };
    // One step: issue the next tile (when there is one), wait for this one,
    // compute it. The loads return in order, so waiting until only the next
    // tile's NEXT loads are outstanding means this tile has landed.
    u32x4_t ka[KS], kb[KS];
    auto step = [&](int j0, lds_char* vcur, lds_char* vnext, const u32x4_t (&kcur)[KS],
                    u32x4_t (&knext)[KS]) {
        const bool more = j0 + kDecTile < k_end;
        if (more) issue(j0 + kDecTile, vnext, knext);
        __builtin_amdgcn_sched_barrier(0);
        if (more) __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_sched_barrier(0);
        compute(j0, vcur, kcur);
        __builtin_amdgcn_sched_barrier(0);
    };

    issue(k_begin, vb0, ka);
    for (int j0 = k_begin; j0 < k_end; j0 += 2 * kDecTile) {
        step(j0, vb0, vb1, ka, kb);
        if (j0 + kDecTile < k_end) step(j0 + kDecTile, vb1, vb0, kb, ka);
    }

    if (r < M) {
        const float l = sum_with_partner32(l_run);
        const size_t part = ((size_t)bkv * nsplit + sp) * kDecRows + r;
        if (g == 0) {
            part_ml[part * 2 + 0] = m_run;
            part_ml[part * 2 + 1] = l;
        }
        float* orow = part_o + part * D;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4_t x = {acc_o[nb][4 * q4 + 0], acc_o[nb][4 * q4 + 1],
                                   acc_o[nb][4 * q4 + 2], acc_o[nb][4 * q4 + 3]};
                *(f32x4_t*)(orow + 32 * nb + 8 * q4 + 4 * g) = x;
            }
    }
}

// One workgroup per output row (query head, position): the four waves take
// every fourth key range, then combine through LDS.
template <int D>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                    uint16_t* __restrict__ O, float* __restrict__ LSE, int G, int Nq,
                    int nsplit) {
    constexpr int PER = D / 64;            // output columns per lane
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int R = blockIdx.x;
    const int qh = R / Nq, qi = R % Nq;    // global query head, position
    const int bkv = qh / G;
    const int r = (qh % G) * Nq + qi;      // packed row in the split phase
    const size_t base = (size_t)bkv * nsplit * kDecRows + r;

    float m = kNegInf;
    for (int s = lane; s < nsplit; s += 64) m = fmaxf(m, part_ml[(base + (size_t)s * kDecRows) * 2]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float mc = (m == kNegInf) ? 0.f : m;

    float l = 0.f, o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
#pragma unroll 4
    for (int s = wave; s < nsplit; s += 4) {
        const size_t p = base + (size_t)s * kDecRows;
        const float w = fast_exp2(part_ml[p * 2] - mc);
        l += w * part_ml[p * 2 + 1];
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] += w * part_o[p * D + PER * lane + e];
    }
    __shared__ float so[4][D];
    __shared__ float sl[4];
#pragma unroll
    for (int e = 0; e < PER; ++e) so[wave][PER * lane + e] = o[e];
    if (lane == 0) sl[wave] = l;
    __syncthreads();
    if (wave == 0) {
        const float lt = sl[0] + sl[1] + sl[2] + sl[3];
        const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
        float x[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int col = PER * lane + e;
            x[e] = (so[0][col] + so[1][col] + so[2][col] + so[3][col]) * inv;
        }
        uint16_t* orow = O + (size_t)R * D;
        if constexpr (PER == 1) {
            orow[lane] = (uint16_t)(pack_bf16x2(x[0], 0.f) & 0xffffu);
        } else {
#pragma unroll
            for (int e = 0; e < PER; e += 2)
                *(uint32_t*)(orow + PER * lane + e) = pack_bf16x2(x[e], x[e + 1]);
        }
        if (lane == 0) LSE[R] = (lt > 0.f) ? (m + fast_log2(lt)) * kLn2 : kNegInf;
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_decode_t(const DecArgs& a) {
    const DecodeWorkspace w = decode_workspace_layout(a.B, a.Hkv, a.Nk, a.d);
    const int G = a.H / a.Hkv;
    float* part_o = (float*)((char*)a.workspace + w.part_o);
    float* part_ml = (float*)((char*)a.workspace + w.part_ml);
    const dim3 grid((w.nsplit + kDecWaves - 1) / kDecWaves, a.B * a.Hkv);
    hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL>), grid, dim3(kDecWaves * 64), 0, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, part_o,
                       part_ml, G, a.Nq, a.Nk, w.split_len, w.nsplit, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rows = a.B * a.H * a.Nq;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(rows), dim3(256), 0, a.stream,
                       (const float*)part_o, (const float*)part_ml, (uint16_t*)a.o, a.lse, G,
                       a.Nq, w.nsplit);
    return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a) {
    if (a.d == 256) return a.causal ? launch_decode_t<256, true>(a) : launch_decode_t<256, false>(a);
    if (a.d == 128) return a.causal ? launch_decode_t<128, true>(a) : launch_decode_t<128, false>(a);
    return a.causal ? launch_decode_t<64, true>(a) : launch_decode_t<64, false>(a);
}

}  // namespace fa
