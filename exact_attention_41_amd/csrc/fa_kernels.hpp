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
    const void* o;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* delta;      // workspace: D_i = sum_c dO_ic O_ic, [B][H][N]
    int B, H, N, d;
    bool causal;
    float scale;
    hipStream_t stream;
};

// Tile shape of the bf16 forward: IB blocks of 32 query rows per wave,
// NW waves per workgroup.
template <int D> struct FwdBf16Config { static constexpr int IB = 2; static constexpr int NW = 4; };

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_bf16(const BwdArgs& a);

}  // namespace fa
