// Internal interface between the C-ABI layer (fa_api.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// H query heads; K/V have Hkv heads (Hkv divides H), query head h using K/V
// head h / (H / Hkv). Hkv == H is ordinary multi-head attention. N query rows
// per head, Nk keys; query row i sits at position Nk - N + i (Nk == N: the
// square case).
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, Hkv, N, Nk, d;
    bool causal;
    float scale;
    hipStream_t stream;
    // fp8 forward only: the real values are descale_x times the stored ones.
    float descale_q = 1.f, descale_k = 1.f, descale_v = 1.f;
    // bf16 forwards only: where to store O - bf16(O) as bf16 (nullptr: not stored).
    void* o_res = nullptr;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;      // the forward's output (read by the preprocess only)
    const void* o_res;  // its rounding residual O - bf16(O), or nullptr (preprocess only)
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    void* workspace;
    int B, H, Hkv, N, Nk, d;   // N query rows, Nk keys (bottom-right causal alignment)
    bool causal;
    float scale;
    hipStream_t stream;
    // The preprocess formed D_i = dO_i . O_i from O and its residual (the dQ
    // pass then takes D from the workspace instead of forming it).
    bool d_known = false;
};

// Rows per chunk of the max-abs pre-pass of the backward: 256 up to d = 128,
// 128 at d = 256 (the same bytes per chunk, so the same number of workgroups
// per byte).
constexpr int kScaleRows = 256;
constexpr int scale_chunk_rows(long long d) { return d > 128 ? (int)(kScaleRows * 128 / d) : kScaleRows; }

// Byte offsets of the backward workspace blocks (Tq = ceil(Nq / 64) and
// Tk = ceil(Nk / 64) tiles of 64 rows per head; an image is the byte layout
// of one transposed LDS tile; BH = B*H query heads, BHkv = B*Hkv K/V heads;
// chunks = ceil(max(Nq, Nk) / kScaleRows)):
//   scales  fp32 [BH][4]             power-of-two factors for Q, K, V, dO as
//                                    seen by each query head (Q and dO common
//                                    to the query heads of one K/V head)
//   partial u32  [BH + BHkv][chunks][2] per-chunk largest |x| (bf16 magnitude
//                                    bits): (Q, dO) per query head, then (K, V)
//                                    per K/V head
//   dhat    fp32 [BH][Nq]            D_i = dO_i . O_i: from the bf16 O alone, the
//                                    centre the dQ pass subtracts from dP before
//                                    rounding (D itself is formed exactly there);
//                                    from O plus its residual, D itself
//   stats   fp32 [BH][Tq][128]       per query tile: lse*log2(e) of its 64 rows,
//                                    then -sE*D (sE = s_dO*s_V); from the dQ pass
//   qt      fp16 [BH][Tq][64*d]      images of (s_Q Q)^T, one per 64-row tile
//   ot      fp16 [BH][Tq][64*d]      images of (s_dO dO)^T
//   kt      fp16 [BHkv][Tk][64*d]    images of (s_K K)^T
// (at d = 256 a 64-row tile's image is either its two 128-column parts or,
// for the passes with 16-row steps, its two 32-row halves, each a [256][32]
// block; the preprocess writes the layout of the pass that reads it)
struct BwdWorkspace {
    size_t scales, partial, dhat, stats, qt, ot, kt, total;
};
BwdWorkspace bwd_workspace_layout(long long B, long long H, long long Hkv, long long Nq,
                                  long long Nk, long long d);
int bwd_scale_chunks(long long Nq, long long Nk, long long d);

// Decoding: Nq query rows per query head (the last Nq positions) against Nk
// keys; q, o [B][H][Nq][d], k, v [B][Hkv][Nk][d], lse [B][H][Nq].
struct DecArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    void* workspace;
    int B, H, Hkv, Nq, Nk, d;
    bool causal;
    float scale;
    hipStream_t stream;
};

// Decoding workspace: the key ranges and their partial results
// (fp32 O [B*Hkv][nsplit][32][d], then (m, l) [B*Hkv][nsplit][32][2]).
struct DecodeWorkspace {
    int nsplit, split_len;
    size_t part_o, part_ml, total;
};
DecodeWorkspace decode_workspace_layout(long long B, long long Hkv, long long Nk, long long d);

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_d256(const FwdArgs& a);   // bf16, d = 256 (one wave per SIMD)
hipError_t launch_fwd_fp8(const FwdArgs& a);    // fp8 e4m3 q, k, v; d = 128
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_prepare(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_decode(const DecArgs& a);

}  // namespace fa
