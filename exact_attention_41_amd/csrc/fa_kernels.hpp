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

// Byte offsets of the backward workspace blocks:
//   delta   fp32 [B][H][N]      D_i = sum_j P_ij dP_ij (written by the dQ pass)
//   scales  fp32 [B][H][4]      power-of-two factors for Q, K, V, dO
//   partial u32 [B][H][chunks][4] per-chunk largest |x| (bf16 magnitude bits)
//   q16     fp16 [B][H][N][d]   Q times its factor (written by the dQ pass)
//   do16    fp16 [B][H][N][d]   dO times its factor (written by the dQ pass)
struct BwdWorkspace {
    size_t delta, scales, partial, q16, do16, total;
};
BwdWorkspace bwd_workspace_layout(long long B, long long H, long long N, long long d);


hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_scales(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);

}  // namespace fa
