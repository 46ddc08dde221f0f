// Internal interface between the C-ABI layer (fa_api.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, N, d;
    bool causal;
    float scale;
    hipStream_t stream;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    void* workspace;
    int B, H, N, d;
    bool causal;
    float scale;
    hipStream_t stream;
};

// Rows per chunk of the max-abs pre-pass of the backward.
constexpr int kScaleRows = 256;

// Byte offsets of the backward workspace blocks (T = ceil(N / 64) tiles of
// 64 rows per head; an image is the byte layout of one transposed LDS tile):
//   scales  fp32 [B][H][4]           power-of-two factors for Q, K, V, dO
//   partial u32  [B][H][chunks][4]   per-chunk largest |x| (bf16 magnitude bits)
//   stats   fp32 [B][H][T][128]      per query tile: lse*log2(e) of its 64 rows,
//                                    then sE*D (sE = s_dO*s_V); from the dQ pass
//   qt      fp16 [B][H][T][64*d]     images of (s_Q Q)^T, one per 64-row tile
//   ot      fp16 [B][H][T][64*d]     images of (s_dO dO)^T
//   kt      fp16 [B][H][T][64*d]     images of (s_K K)^T
struct BwdWorkspace {
    size_t scales, partial, stats, qt, ot, kt, total;
};
BwdWorkspace bwd_workspace_layout(long long B, long long H, long long N, long long d);

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_prepare(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);

}  // namespace fa
