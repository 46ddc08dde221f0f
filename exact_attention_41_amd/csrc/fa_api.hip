// C-ABI entry points of libfa.so: argument validation, then kernel launch.
// Every check happens before anything is enqueued, so an error status means
// no work was launched.
#include <math.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "fa.h"
#include "fa_kernels.hpp"

namespace {

constexpr int kMaxN = 1 << 26;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Head sizes with kernels: 64 and 128 everywhere, 256 for everything but
// the fp32 and fp8 forwards.
bool head_dim_ok(int d, bool wide) { return d == 64 || d == 128 || (wide && d == 256); }

// Shared size/scale checks. Returns FA_OK and sets *empty when B*H*N == 0.
fa_status_t check_common(int B, int H, int N, int d, float scale, bool wide, bool* empty) {
    if (B < 0 || H < 0 || N < 0) return FA_ERR_INVALID_ARG;
    // scale > 0: the kernels mask a score by making it -inf before scaling,
    // which a zero scale would turn into NaN.
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!head_dim_ok(d, wide)) return FA_ERR_UNSUPPORTED;
    *empty = (B == 0 || H == 0 || N == 0);
    if (*empty) return FA_OK;
    if (N > kMaxN) return FA_ERR_UNSUPPORTED;
    // Grid = (query blocks of >= 32 rows) x B x H must fit a 32-bit grid.
    const long long bh = (long long)B * (long long)H;
    const long long blocks = bh * (((long long)N + 31) / 32);
    if (bh > (1LL << 30) || blocks > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// K/V head count: 1 <= Hkv, Hkv divides H (anything when H == 0).
fa_status_t check_heads(int H, int Hkv) {
    if (Hkv < 0) return FA_ERR_INVALID_ARG;
    if (H > 0 && (Hkv == 0 || H % Hkv != 0)) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

fa_status_t check_tensor(const void* p) {
    if (!p) return FA_ERR_INVALID_ARG;
    if (!aligned(p, 16)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa_status_t check_lse(const void* p) {
    if (!p) return FA_ERR_INVALID_ARG;
    if (!aligned(p, 4)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

#define FA_TRY(expr)                       \
    do {                                   \
        fa_status_t st_ = (expr);          \
        if (st_ != FA_OK) return st_;      \
    } while (0)

fa_status_t check_fwd(const void* q, const void* k, const void* v, const void* o,
                      const void* lse, int B, int H, int N, int d, float scale, bool wide,
                      bool* empty) {
    FA_TRY(check_common(B, H, N, d, scale, wide, empty));
    if (*empty) return FA_OK;
    // Null pointers are argument errors, checked before alignment.
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    FA_TRY(check_tensor(q));
    FA_TRY(check_tensor(k));
    FA_TRY(check_tensor(v));
    FA_TRY(check_tensor(o));
    FA_TRY(check_lse(lse));
    return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_str(fa_status_t status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
        case FA_ERR_HIP: return "FA_ERR_HIP";
    }
    return "FA_ERR_UNKNOWN";
}

}  // extern "C"

namespace {

// The bf16 forward of every entry point; o_res (the rounding residual of O)
// is stored when it is not null.
fa_status_t fwd_bf16(const void* q, const void* k, const void* v, void* o, void* o_res,
                     float* lse, int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                     float scale, hipStream_t stream) {
    bool empty = false;
    if (Nk < 0) return FA_ERR_INVALID_ARG;
    FA_TRY(check_fwd(q, k, v, o, lse, B, H, Nq, d, scale, true, &empty));
    FA_TRY(check_heads(H, Hkv));
    if (empty) return FA_OK;
    if (o_res) FA_TRY(check_tensor(o_res));
    if (Nk == 0) return FA_ERR_INVALID_ARG;      // query rows but no keys
    if (Nk > kMaxN) return FA_ERR_UNSUPPORTED;
    fa::FwdArgs a{q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal != 0, scale, stream};
    a.o_res = o_res;
    return fa::launch_fwd_bf16(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status_t fa_fwd_rect(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                        hipStream_t stream) {
    return fwd_bf16(q, k, v, o, nullptr, lse, B, H, Hkv, Nq, Nk, d, causal, scale, stream);
}

fa_status_t fa_fwd_train(const void* q, const void* k, const void* v, void* o, void* o_res,
                         float* lse, int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                         float scale, hipStream_t stream) {
    if (!o_res && B > 0 && H > 0 && Nq > 0) return FA_ERR_INVALID_ARG;
    return fwd_bf16(q, k, v, o, o_res, lse, B, H, Hkv, Nq, Nk, d, causal, scale, stream);
}

fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                       float descale_q, float descale_k, float descale_v, hipStream_t stream) {
    bool empty = false;
    if (Nk < 0) return FA_ERR_INVALID_ARG;
    for (float x : {descale_q, descale_k, descale_v})
        if (!isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID_ARG;
    FA_TRY(check_fwd(q, k, v, o, lse, B, H, Nq, d, scale, false, &empty));
    FA_TRY(check_heads(H, Hkv));
    if (d != 128) return FA_ERR_UNSUPPORTED;
    if (empty) return FA_OK;
    if (Nk == 0) return FA_ERR_INVALID_ARG;
    if (Nk > kMaxN) return FA_ERR_UNSUPPORTED;
    fa::FwdArgs a{q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal != 0, scale, stream,
                  descale_q, descale_k, descale_v};
    return fa::launch_fwd_fp8(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Hkv, int N, int d, int causal, float scale,
                       hipStream_t stream) {
    return fa_fwd_rect(q, k, v, o, lse, B, H, Hkv, N, N, d, causal, scale, stream);
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale, hipStream_t stream) {
    return fa_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, stream);
}

fa_status_t fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                       int B, int H, int N, int d, int causal, float scale, hipStream_t stream) {
    bool empty = false;
    FA_TRY(check_fwd(q, k, v, o, lse, B, H, N, d, scale, false, &empty));
    if (empty) return FA_OK;
    fa::FwdArgs a{q, k, v, o, lse, B, H, H, N, N, d, causal != 0, scale, stream};
    return fa::launch_fwd_f32(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_rect_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d) {
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || !head_dim_ok(d, true)) return 0;
    if (Hkv <= 0 || H % Hkv != 0) return 0;
    return fa::bwd_workspace_layout(B, H, Hkv, Nq, Nk, d).total;
}

size_t fa_bwd_gqa_workspace_size(int B, int H, int Hkv, int N, int d) {
    return fa_bwd_rect_workspace_size(B, H, Hkv, N, N, d);
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
    return fa_bwd_gqa_workspace_size(B, H, H, N, d);
}

}  // extern "C"

namespace {

// Checks shared by the backward entry points: null tensor pointers (or a null
// lse when `need_lse`) are argument errors, misaligned ones unsupported, and
// the workspace is checked last.
fa_status_t check_bwd(std::initializer_list<const void*> tensors, bool need_lse, const void* lse,
                      const void* workspace, size_t workspace_bytes, int B, int H, int Hkv,
                      int Nq, int Nk, int d, float scale, bool* empty) {
    if (Nk < 0) return FA_ERR_INVALID_ARG;
    FA_TRY(check_common(B, H, Nq, d, scale, true, empty));
    FA_TRY(check_heads(H, Hkv));
    if (*empty && (B == 0 || H == 0 || Nk == 0)) return FA_OK;
    // Rows without keys, or keys without rows (whose gradients are zero and
    // left to the caller), are argument errors.
    if (*empty || Nk == 0) return FA_ERR_INVALID_ARG;
    bool unused = false;
    FA_TRY(check_common(B, H, Nk, d, scale, true, &unused));
    for (const void* p : tensors)
        if (!p) return FA_ERR_INVALID_ARG;
    if (need_lse && !lse) return FA_ERR_INVALID_ARG;
    for (const void* p : tensors) FA_TRY(check_tensor(p));
    if (need_lse) FA_TRY(check_lse(lse));
    if (!workspace || !aligned(workspace, 256) ||
        workspace_bytes < fa_bwd_rect_workspace_size(B, H, Hkv, Nq, Nk, d))
        return FA_ERR_WORKSPACE;
    return FA_OK;
}

fa::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* o,
                     const void* o_res, const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, void* workspace, int B, int H, int Hkv, int Nq, int Nk, int d,
                     int causal, float scale, hipStream_t stream) {
    fa::BwdArgs a{q, k, v, o, o_res, dout, lse, dq, dk, dv, workspace,
                  B, H, Hkv, Nq, Nk, d, causal != 0, scale, stream};
    a.d_known = o_res != nullptr;
    return a;
}

}  // namespace

extern "C" {

fa_status_t fa_bwd_preprocess(const void* q, const void* k, const void* v, const void* o,
                              const void* o_res, const void* dout, void* workspace,
                              size_t workspace_bytes, int B, int H, int N, int d,
                              hipStream_t stream) {
    bool empty = false;
    FA_TRY(check_bwd({q, k, v, o, dout}, false, nullptr, workspace, workspace_bytes, B, H, H, N,
                     N, d, 1.f, &empty));
    if (empty) return FA_OK;
    if (o_res) FA_TRY(check_tensor(o_res));
    const fa::BwdArgs a = bwd_args(q, k, v, o, o_res, dout, nullptr, nullptr, nullptr, nullptr,
                                   workspace, B, H, H, N, N, d, 0, 1.f, stream);
    return fa::launch_bwd_prepare(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, void* workspace, size_t workspace_bytes, void* dq,
                      int B, int H, int N, int d, int causal, float scale, int d_ready,
                      hipStream_t stream) {
    bool empty = false;
    FA_TRY(check_bwd({q, k, v, dout, dq}, true, lse, workspace, workspace_bytes, B, H, H, N, N,
                     d, scale, &empty));
    if (empty) return FA_OK;
    fa::BwdArgs a = bwd_args(q, k, v, nullptr, nullptr, dout, lse, dq, nullptr, nullptr,
                             workspace, B, H, H, N, N, d, causal, scale, stream);
    a.d_known = d_ready != 0;
    return fa::launch_bwd_dq(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                        const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                        int B, int H, int N, int d, int causal, float scale, hipStream_t stream) {
    bool empty = false;
    FA_TRY(check_bwd({q, k, v, dout, dk, dv}, false, nullptr, workspace, workspace_bytes, B, H,
                     H, N, N, d, scale, &empty));
    if (empty) return FA_OK;
    const fa::BwdArgs a = bwd_args(q, k, v, nullptr, nullptr, dout, nullptr, nullptr, dk, dv,
                                   const_cast<void*>(workspace), B, H, H, N, N, d, causal, scale,
                                   stream);
    return fa::launch_bwd_dkdv(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"

namespace {

// The backward of every entry point; with o_res, D comes from O and its
// residual in the preprocess.
fa_status_t bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                     const void* o_res, const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, void* workspace, size_t workspace_bytes, int B, int H, int Hkv,
                     int Nq, int Nk, int d, int causal, float scale, hipStream_t stream) {
    bool empty = false;
    FA_TRY(check_bwd({q, k, v, o, dout, dq, dk, dv}, true, lse, workspace, workspace_bytes, B, H,
                     Hkv, Nq, Nk, d, scale, &empty));
    if (empty) return FA_OK;
    if (o_res) FA_TRY(check_tensor(o_res));
    const fa::BwdArgs a = bwd_args(q, k, v, o, o_res, dout, lse, dq, dk, dv, workspace, B, H,
                                   Hkv, Nq, Nk, d, causal, scale, stream);
    if (fa::launch_bwd_prepare(a) != hipSuccess) return FA_ERR_HIP;
    if (fa::launch_bwd_dq(a) != hipSuccess) return FA_ERR_HIP;
    if (fa::launch_bwd_dkdv(a) != hipSuccess) return FA_ERR_HIP;
    return FA_OK;
}

}  // namespace

extern "C" {

fa_status_t fa_bwd_rect(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int Nq,
                        int Nk, int d, int causal, float scale, hipStream_t stream) {
    return bwd_bf16(q, k, v, o, nullptr, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H,
                    Hkv, Nq, Nk, d, causal, scale, stream);
}

fa_status_t fa_bwd_train(const void* q, const void* k, const void* v, const void* o,
                         const void* o_res, const void* dout, const float* lse, void* dq,
                         void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
                         int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                         hipStream_t stream) {
    if (!o_res && B > 0 && H > 0 && (Nq > 0 || Nk > 0)) return FA_ERR_INVALID_ARG;
    return bwd_bf16(q, k, v, o, o_res, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H,
                    Hkv, Nq, Nk, d, causal, scale, stream);
}

fa_status_t fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N,
                       int d, int causal, float scale, hipStream_t stream) {
    return fa_bwd_rect(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, Hkv,
                       N, N, d, causal, scale, stream);
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                   int causal, float scale, hipStream_t stream) {
    return fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H, N,
                      d, causal, scale, stream);
}

size_t fa_decode_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d) {
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || !head_dim_ok(d, true)) return 0;
    if (Hkv <= 0 || H % Hkv != 0 || Nq > Nk || (H / Hkv) * Nq > 32) return 0;
    return fa::decode_workspace_layout(B, Hkv, Nk, d).total;
}

}  // extern "C"

namespace {

// Every check of fa_decode except the workspace's. Sets *empty when there is
// nothing to compute.
fa_status_t check_decode(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, int B, int H, int Hkv, int Nq, int Nk, int d,
                         float scale, bool* empty) {
    *empty = false;
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    FA_TRY(check_heads(H, Hkv));
    if (!head_dim_ok(d, true)) return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || Nq == 0) {
        *empty = true;
        return FA_OK;
    }
    if (Nq > Nk) return FA_ERR_INVALID_ARG;
    if (Nk > kMaxN || (H / Hkv) * Nq > 32) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H > (1LL << 30) || (long long)B * Hkv > 65535) return FA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    FA_TRY(check_tensor(q));
    FA_TRY(check_tensor(k));
    FA_TRY(check_tensor(v));
    FA_TRY(check_tensor(o));
    FA_TRY(check_lse(lse));
    return FA_OK;
}

// ---------------------------------------------------------------------------
// Fixed device scratch of fa_decode_noalloc: the split phase's partial
// results live here instead of in a caller's workspace. One copy per device
// (each GPU that runs the entry point holds it until the process ends); in
// host code `scratch` only names the symbol, so its device address is taken
// once per device with hipGetSymbolAddress and only that address is passed
// to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)40 << 20;   // 40 MiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch (looked up on its first use
// on that device, with that device current).
hipError_t current_device_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

fa_status_t fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int Nq,
                      int Nk, int d, int causal, float scale, hipStream_t stream) {
    bool empty = false;
    FA_TRY(check_decode(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, &empty));
    if (empty) return FA_OK;
    if (!workspace || !aligned(workspace, 256) ||
        workspace_bytes < fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d))
        return FA_ERR_WORKSPACE;
    const fa::DecArgs a{q, k, v, o, lse, workspace, B, H, Hkv, Nq, Nk, d, causal != 0, scale,
                        stream};
    return fa::launch_decode(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                              float scale, hipStream_t stream) {
    bool empty = false;
    FA_TRY(check_decode(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, &empty));
    if (empty) return FA_OK;
    if (fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d) > kNoAllocScratchBytes)
        return FA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (current_device_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
    const fa::DecArgs a{q, k, v, o, lse, ws, B, H, Hkv, Nq, Nk, d, causal != 0, scale, stream};
    return fa::launch_decode(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
