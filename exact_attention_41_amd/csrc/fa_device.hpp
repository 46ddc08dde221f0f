// Device-side building blocks shared by the forward and backward kernels:
// CDNA4 (gfx950) MFMA wrappers, bf16 packing, cross-lane helpers and the
// LDS swizzles. Everything here is wave64-specific.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Rescale threshold of the forward's online softmax, in log2 units: the
// reference maximum of a row is moved only when a tile's maximum exceeds it
// by more than this, so probabilities stay below 2^8 and the output
// accumulator is rescaled rarely. The result is the same function (every
// term and the normaliser carry the same factor); only the rounding differs.
constexpr float kRescaleLog2 = 8.f;

// D(32x32,f32) += A(32x16,bf16) * B(16x32,bf16).
// Operand layout used throughout: lane l supplies row (A) / column (B)
// l % 32 and eight consecutive-in-register values of the contraction index
// for lane group g = l / 32. A and B use the same (g, element) -> k mapping,
// so any consistent assignment of contraction indices to (g, element) is a
// valid product. Accumulator register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ f32x16_t mfma_32x32x16(const u32x4_t& a, const u32x4_t& b,
                                                  const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Same product with fp16 operands (same rate on gfx950, 3 more mantissa bits).
__device__ __forceinline__ f32x16_t mfma_32x32x16_f16(const u32x4_t& a, const u32x4_t& b,
                                                      const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Compile-time flag carried into a generic lambda.
template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// Compile-time integer carried into a generic lambda.
template <int I>
struct IntTag {
    static constexpr int value = I;
};

typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;

// fp16 product accumulated in place into an accumulator held in AGPRs.
// When one wave owns a SIMD's whole register file the compiler keeps every
// matrix result in AGPRs and copies operands and results between the two
// files around each product; written as inline assembly, the accumulator
// stays in AGPRs and the operands stay in VGPRs. The leading s_nop supplies
// the two wait states a matrix instruction needs after a VALU write of one
// of its sources; SrcC is vDst, which dependent products forward in
// hardware. Read the accumulator only after agpr_settle().
__device__ __forceinline__ void mfma_f16_agpr(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// bf16 product accumulated in place into an accumulator held in AGPRs, both
// operands in VGPRs (otherwise as mfma_f16_agpr).
__device__ __forceinline__ void mfma_bf16_agpr(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// bf16 product into a VGPR accumulator with the B operand held in AGPRs (a
// loop-invariant operand parked outside the VGPR file). A chain of products
// into one accumulator is mfma_bf16_first (SrcC = 0), mfma_bf16_next and
// mfma_bf16_last; SrcC = vDst within the chain, which dependent products
// forward in hardware, and the last one is followed by the wait states the
// VALU needs before it may read a matrix result (more than an 8-pass
// product requires). With WS set, each product is preceded by the two wait
// states a matrix instruction needs after a VALU write of a source: for
// kernels whose AGPR file is full, where the compiler may copy a parked
// operand into an AGPR just before the product (it does not see that the
// assembly is a matrix instruction, so it adds no wait states of its own).
template <bool WS = false>
__device__ __forceinline__ void mfma_bf16_first(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
    if constexpr (WS)
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
// The first product of a chain that starts from the accumulator value c
// instead of 0 (SrcC = c, a separate VGPR block).
template <bool WS = false>
__device__ __forceinline__ void mfma_bf16_first_c(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b,
                                                  const f32x16_t& c) {
    if constexpr (WS)
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(acc) : "v"(a), "a"(b), "v"(c));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(acc) : "v"(a), "a"(b), "v"(c));
}
template <bool WS = false>
__device__ __forceinline__ void mfma_bf16_next(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
    if constexpr (WS)
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
template <bool WS = false>
__device__ __forceinline__ void mfma_bf16_last(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
    if constexpr (WS)
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7"
            : "+v"(acc) : "v"(a), "a"(b));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7"
            : "+v"(acc) : "v"(a), "a"(b));
}

// Pins a value computed for a later tile at this point of the schedule: the
// compiler otherwise sinks its computation (and everything feeding it) to
// where it is used, past the barriers and products it was interleaved with.
__device__ __forceinline__ void keep_here(u32x4_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void keep_here(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void keep_here(int& x) { asm volatile("" : "+v"(x)); }

// Moves a loop-invariant matrix operand into AGPRs once, so that products
// taking it through an "a" operand read it there instead of copying it from
// VGPRs at every use.
__device__ __forceinline__ void park_in_agprs(u32x4_t& x) { asm("" : "+a"(x)); }

// Wait states between the last matrix write of an AGPR accumulator and any
// other read of it (more than the 8-pass product needs).
__device__ __forceinline__ void agpr_settle(f32x16_t& acc) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
}

// Two fp32 values -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2_t p = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// Product of two packed fp16 pairs, lane by lane (v_pk_mul_f16).
__device__ __forceinline__ uint32_t mul_f16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) * __builtin_bit_cast(f16x2_t, b));
}

// A packed bf16 pair times s (a power of two), as a packed fp16 pair.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, float s) {
    return pack_f16x2(__uint_as_float(w << 16) * s, __uint_as_float(w & 0xffff0000u) * s);
}

// A packed bf16 pair times s (a power of two), still bf16 (exact unless the
// result leaves the fp32 exponent range).
__device__ __forceinline__ uint32_t bf16x2_scale(uint32_t w, float s) {
    const uint32_t lo = __float_as_uint(__uint_as_float(w << 16) * s) >> 16;
    const uint32_t hi = __float_as_uint(__uint_as_float(w & 0xffff0000u) * s) & 0xffff0000u;
    return lo | hi;
}

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// The rounding residuals of a pair packed as w = pack_bf16x2(lo, hi), again as
// a bf16 pair: x - bf16(x) is exact in fp32, and bf16(x) + bf16(x - bf16(x))
// keeps about 16 significant bits of x.
__device__ __forceinline__ uint32_t pack_bf16x2_residual(float lo, float hi, uint32_t w) {
    return pack_bf16x2(lo - bf16_lo(w), hi - bf16_hi(w));
}

// Value of x held by the lane 32 positions away (l ^ 32), via v_permlane32_swap.
__device__ __forceinline__ float partner32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    // r[0]: lanes 0-31 keep x, lanes 32-63 receive x of lanes 0-31;
    // r[1]: lanes 0-31 receive x of lanes 32-63, lanes 32-63 keep x.
    const int lane = __lane_id();
    return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ float max_with_partner32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_partner32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16-byte-chunk XOR swizzle for a row-major [rows][D] bf16 tile in LDS.
// D = 128 or 256: rows are 256 or 512 B (16 or 32 chunks), and the low four
// bits of the chunk index are XORed with the row; D = 64: rows are 128 B
// (8 chunks). Sixteen consecutive rows reading the same logical chunk land on
// distinct 16-byte bank groups (and so do eight).
template <int D>
__device__ __forceinline__ int row_chunk_swizzle(int row) {
    if constexpr (D >= 128) return row & 15;
    else return (row ^ (row >> 3)) & 7;
}

template <int D>
__device__ __forceinline__ int row_chunk_offset(int row, int chunk) {
    return row * (D * 2) + ((chunk ^ row_chunk_swizzle<D>(row)) << 4);
}

// Row-major tiles that are also read transposed (ds_read_b64_tr_b16: 32
// lanes read four consecutive rows x 64 bytes). For 256- and 512-byte rows
// the XOR takes the row's two low bits into chunk bits 2-3 (and bits 2-3
// into bits 0-1): four consecutive rows then land in four different 64-byte
// bank ranges, and 16 consecutive rows reading one chunk still cover every
// bank once. 128-byte rows take row_chunk_swizzle's pattern of rows 0-15 for
// every group of 16 rows (the same banks within a group). In both, a row's
// XOR depends on its four low bits only, so a fragment 16 rows further lies
// a constant distance further.
template <int D>
__device__ __forceinline__ int tr_rows_swizzle(int row) {
    if constexpr (D >= 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (row & 7) ^ ((row >> 3) & 1);
}

// Byte offset of 16-byte chunk `chunk` of row `row`: row_chunk_offset, or with
// TRS the swizzle of tr_rows_swizzle.
template <int D, bool TRS>
__device__ __forceinline__ int rows_offset(int row, int chunk) {
    return row * (D * 2) +
           ((chunk ^ (TRS ? tr_rows_swizzle<D>(row) : row_chunk_swizzle<D>(row))) << 4);
}

// Transposed tile layout ("[n][key]"), 64 keys per row = 128 B = 16 slots of
// 8 B. Within every group of 16 keys the order is permuted so that the eight
// keys one MFMA lane group needs are contiguous (key 16t + 8a + 4g + c is
// stored at position 16t + 8g + 4a + c), and the 8-byte slot is XORed with an
// even, row-dependent value so 16-byte reads stay aligned and consecutive rows
// spread over the banks.
__device__ __forceinline__ int tr_slot_swizzle(int n) { return ((n ^ (n >> 3)) & 7) << 1; }

__device__ __forceinline__ int tr_key_position(int key) {
    const int t = key >> 4, a = (key >> 3) & 1, g = (key >> 2) & 1, c = key & 3;
    return (t << 4) | (g << 3) | (a << 2) | c;
}

// Byte offset of the 8-byte slot that holds positions [4s, 4s+4) of row n.
__device__ __forceinline__ int tr_slot_offset(int n, int slot) {
    return n * 128 + ((slot ^ tr_slot_swizzle(n)) << 3);
}

// ---------------------------------------------------------------------------
// Direct global -> LDS staging (global_load_lds_dwordx4) of a [64][D] bf16
// tile into a row-major LDS tile with XOR-swizzled 16-byte chunks. Each wave
// instruction fills 1 KB of LDS contiguously, lane l writing bytes
// [16l, 16l+16); the source is a per-lane address, so the swizzle is applied
// by choosing which global chunk each lane fetches. Rows at or past N read
// row N - 1 (N >= 1): finite data in rows that every caller masks. The
// compiler does not order these copies against LDS reads: wait on vmcnt (a
// barrier does) before reading what they wrote.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;

// A wave-uniform pointer, held in scalar registers: the compiler may
// otherwise fold a per-lane offset into it early and add the two with a
// 64-bit vector instruction before every copy.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
    const uint64_t u = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (const char*)(((uint64_t)hi << 32) | lo);
}

// 16 bytes per lane from global address base + voff (base wave-uniform, so
// the copy takes the scalar-base + 32-bit-offset form) into LDS bytes
// [16 l, 16 l + 16) after the wave-uniform address `dst`.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, lds_char* dst) {
    // An offset that is the same on every call (a loop invariant) would be
    // widened to 64 bits once, outside the loop, and the wide sum would then
    // miss the scalar-base form: the empty asm keeps it a 32-bit value here.
    asm volatile("" : "+v"(voff));
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(uniform_ptr(base) + voff),
        (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// The same copy as one inline-assembly block (M0 = the LDS destination, then
// the load). The compiler then does not see an LDS write: it would otherwise
// wait for every outstanding LDS read before each copy (it cannot prove that
// the copy's destination does not overlap them), which empties a kernel's
// ring of fragment reads at every copy. The caller orders the copies against
// LDS reads itself: each copy goes to a buffer that no wave reads until the
// next barrier, and each wave waits for its copies (vmcnt) before that
// barrier. No VGPR is written.
__device__ __forceinline__ void lds_dma16_async(const void* base, uint32_t voff, lds_char* dst) {
    const uint64_t b = (uint64_t)uniform_ptr(base);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(b), "s"(m0)
                 : "memory", "m0");
}

// K-type tiles: chunk c of row r is stored at chunk c ^ row_chunk_swizzle(r).
// V-type tiles: chunk c of row r is stored at chunk c ^ (2 * (r & 3)), which
// makes the transposed 8-byte reads below conflict-free.
__device__ __forceinline__ int v_chunk_swizzle(int row) { return (row & 3) << 1; }

// 1 KB block b of the [64][D] tile at row row0 of `src` (N >= 1 rows of D
// bf16 values, consecutive rows LD >= D values apart) into LDS: lane `lane`
// fetches the chunk whose swizzled place is bytes [16 lane, 16 lane + 16) of
// the block. Rows past N read row N - 1; a tile wholly past N reads row N - 1
// throughout.
template <int D, bool VTYPE, int LD = D>
__device__ __forceinline__ void stage_block(const uint16_t* __restrict__ src, lds_char* tile,
                                            int row0, int N, int b, int lane) {
    constexpr int DCH = D / 8;
    constexpr int RPK = 1024 / (2 * D);        // rows per 1 KB block
    const int row = b * RPK + lane / DCH;      // row within the tile
    const int phys = lane % DCH;
    const int logical = phys ^ (VTYPE ? v_chunk_swizzle(row) : row_chunk_swizzle<D>(row));
    const int rb = min(row0, N - 1);           // uniform
    const uint32_t voff = (uint32_t)(min(row, N - 1 - rb) * (2 * LD) + logical * 16);
    lds_dma16(src + (size_t)rb * LD, voff, tile + b * 1024);
}

// Stage blocks b = first, first + STRIDE, ... (< 64 * D * 2 / 1024) of the
// tile starting at row row0 of `src` (a [N][D] bf16 array).
template <int D, int COUNT, int STRIDE, bool VTYPE>
__device__ __forceinline__ void stage_tile_lds(const uint16_t* __restrict__ src, lds_char* tile,
                                               int row0, int N, int first, int lane) {
#pragma unroll
    for (int k = 0; k < COUNT; ++k) stage_block<D, VTYPE>(src, tile, row0, N, first + STRIDE * k, lane);
}

// Single-block forms, for spreading a tile's loads over a longer stretch of
// other work: 1 KB block b of a K-type tile, or of a tile image that is
// already laid out as the LDS tile (a byte-for-byte copy of the `bytes`
// bytes at `src`, a multiple of 16; lanes past them re-read its last chunk
// and fill LDS that no one reads).
template <int D, int LD = D>
__device__ __forceinline__ void stage_tile_block(const uint16_t* __restrict__ src, lds_char* tile,
                                                 int row0, int N, int b, int lane) {
    stage_block<D, false, LD>(src, tile, row0, N, b, lane);
}

template <int D, int LD = D, bool TRS = false>
__device__ __forceinline__ void stage_tile_block_async(const uint16_t* __restrict__ src,
                                                       lds_char* tile, int row0, int N, int b,
                                                       int lane) {
    constexpr int DCH = D / 8;
    constexpr int RPK = 1024 / (2 * D);
    const int row = b * RPK + lane / DCH;
    const int phys = lane % DCH;
    const int logical = phys ^ (TRS ? tr_rows_swizzle<D>(row) : row_chunk_swizzle<D>(row));
    const int rb = min(row0, N - 1);
    const uint32_t voff = (uint32_t)(min(row, N - 1 - rb) * (2 * LD) + logical * 16);
    lds_dma16_async(src + (size_t)rb * LD, voff, tile + b * 1024);
}

__device__ __forceinline__ void stage_image_block_full_async(const void* src, lds_char* tile,
                                                             int b, int lane) {
    lds_dma16_async((const char*)src + b * 1024, (uint32_t)(lane * 16), tile + b * 1024);
}

__device__ __forceinline__ void stage_image_block_async(const void* src, int bytes,
                                                        lds_char* tile, int b, int lane) {
    lds_dma16_async(src, (uint32_t)min(b * 1024 + lane * 16, bytes - 16), tile + b * 1024);
}

__device__ __forceinline__ void stage_image_block(const void* src, int bytes, lds_char* tile,
                                                  int b, int lane) {
    lds_dma16(src, (uint32_t)min(b * 1024 + lane * 16, bytes - 16), tile + b * 1024);
}

// The same for a block wholly inside the image (bytes >= 1024 (b + 1)): the
// block's start goes into the uniform base, each lane's offset is 16 lane.
__device__ __forceinline__ void stage_image_block_full(const void* src, lds_char* tile, int b,
                                                       int lane) {
    lds_dma16((const char*)src + b * 1024, (uint32_t)(lane * 16), tile + b * 1024);
}

// 16-byte A/B fragment of a K-type tile: row `row`, logical chunk `ch`.
template <int D>
__device__ __forceinline__ u32x4_t lds_k_frag(const lds_char* tile, int row, int ch) {
    return *(const __attribute__((address_space(3))) u32x4_t*)(tile + row_chunk_offset<D>(row, ch));
}

// Transposed MFMA A fragment from a V-type tile [64 keys][D]: lane l gets
// rows n = n0 + l%32 of V^T and the eight keys 16t + {4g..4g+3, 8+4g..8+4g+3}
// (g = l/32), in that element order; two ds_read_b64_tr_b16. Within a group of
// 16 lanes, ds_read_b64_tr_b16 returns to lane i element e of the 8 bytes
// addressed by lane 4e + i/4, at position i%4; so lane i addresses key row
// base + i/4, columns c0 + 4(i%4) .. +3.
template <int D>
__device__ __forceinline__ u32x4_t lds_vt_frag(const lds_char* tile, int n0, int t, int lane) {
    const int g = lane >> 5, half = (lane >> 4) & 1, i = lane & 15;
    const int col = n0 + 16 * half + 4 * (i & 3);
    const int r1 = 16 * t + 4 * g + (i >> 2), r2 = r1 + 8;
    const int o1 = r1 * (2 * D) + ((((col >> 3) ^ v_chunk_swizzle(r1))) << 4) + ((col & 7) << 1);
    const int o2 = r2 * (2 * D) + ((((col >> 3) ^ v_chunk_swizzle(r2))) << 4) + ((col & 7) << 1);
    const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(tile + o1));
    const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(tile + o2));
    const u32x2_t ua = __builtin_bit_cast(u32x2_t, a), ub = __builtin_bit_cast(u32x2_t, b);
    return u32x4_t{ua[0], ua[1], ub[0], ub[1]};
}

// Sum of a packed fp16 pair added to acc (v_dot2_f32_f16 with (1, 1)).
__device__ __forceinline__ float add_f16x2(uint32_t w, float acc) {
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), one, acc, false);
}

// Sum of a packed bf16 pair added to acc (v_dot2_f32_bf16 with (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

}  // namespace fa
