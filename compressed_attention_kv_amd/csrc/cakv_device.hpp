// cakv_device.hpp -- device helpers for the gfx950 (CDNA4) kernels of the
// compressed-attention library: storage conversions, the fp8 E4M3 encoder,
// rotary sin/cos from exact fractional turns, MFMA operand types and wave
// reductions.  Written for wave64 and the gfx950 MFMA / conversion units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cakv {

// Device-side checks of the kernels' own index invariants, compiled in only
// with -DCAKV_DEBUG (the debug build): a failed check prints its condition
// and traps.  In the regular build they cost nothing.
#ifdef CAKV_DEBUG
#define CAKV_DCHECK(cond)                                                                        \
    do {                                                                                         \
        if (!(cond)) {                                                                           \
            printf("CAKV_DCHECK failed: %s at %s:%d (block %d)\n", #cond, __FILE__, __LINE__,    \
                   (int)blockIdx.x);                                                             \
            __builtin_trap();                                                                    \
        }                                                                                        \
    } while (0)
#else
#define CAKV_DCHECK(cond) ((void)0)
#endif

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- storage types
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// two floats -> packed pair of f16 (round to nearest even, v_cvt_pk_f16_f32)
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short bf16x2_t __attribute__((ext_vector_type(2)));  // two bf16 bit patterns (v_dot2_f32_bf16)

// A 32-bit word as a bf16 pair.  Goes through a scalar copy: a bit cast
// applied directly to an element of an ext_vector inside an unrolled loop
// has been compiled as if it always named element 0.
__device__ __forceinline__ bf16x2_t word_as_bf16x2(uint32_t w) {
    bf16x2_t v;
    __builtin_memcpy(&v, &w, 4);
    return v;
}
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2v_t h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// two floats -> packed f16 pair (round to nearest even; one v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    const f16x2_t h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------- fp8 E4M3 (OCP)
// Round-to-nearest-even encode of a finite v with |v| <= 448 (values beyond
// saturate to the largest finite code).  Normal range: keep 3 mantissa bits of
// the fp32 pattern with an RNE bias and move the exponent from bias 127 to 7;
// subnormal range (|v| < 2^-6, step 2^-9): round |v| * 512 to an integer.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    float a = __builtin_fabsf(v);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        uint32_t b = __float_as_uint(a);
        b += 0x7ffffu + ((b >> 20) & 1u);
        code = (b >> 20) - (120u << 3);
        code = code > 0x7eu ? 0x7eu : code;
    }
    return code | sign;
}

// OCP E4M3 code -> its exact value (bias 7, three mantissa bits, exponent
// field 0 holds subnormals m * 2^-9; the NaN code is never produced by the
// encoder and decodes as the largest magnitude plus one step, 480)
__device__ __forceinline__ float e4m3_decode_f32(uint32_t c) {
    const int e = (c >> 3) & 15, m = c & 7;
    const float v = e == 0 ? __builtin_ldexpf((float)m, -9) : __builtin_ldexpf((float)(8 + m), e - 10);
    return (c & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------- rotary sin / cos
// sin and cos of 2*pi*x for a fraction of a turn x (any real, fp64).  The
// integer part is dropped exactly in fp64, the rest is folded to an octant
// |y| <= 1/8 turn and evaluated with Taylor polynomials (error < 2e-9 on
// |angle| <= pi/4, below fp32 rounding).
__device__ __forceinline__ void sincos_turns(double x, float* s_out, float* c_out) {
    double f = x - __builtin_floor(x);            // [0, 1)
    double qd = __builtin_rint(f * 4.0);          // quadrant 0..4
    float y = (float)(f - qd * 0.25);             // [-1/8, 1/8] turn, exact subtraction
    int q = ((int)qd) & 3;
    float a = y * 6.28318530717958647692f;
    float a2 = a * a;
    float s = a * (1.0f + a2 * (-1.0f / 6.0f + a2 * (1.0f / 120.0f + a2 * (-1.0f / 5040.0f + a2 * (1.0f / 362880.0f)))));
    float c = 1.0f + a2 * (-0.5f + a2 * (1.0f / 24.0f + a2 * (-1.0f / 720.0f + a2 * (1.0f / 40320.0f + a2 * (-1.0f / 3628800.0f)))));
    // quadrant q: (sin, cos) of q*pi/2 + a
    const float so = ((q & 1) ? c : s) * ((q & 2) ? -1.0f : 1.0f);
    const float co = ((q & 1) ? s : c) * (((q + 1) & 2) ? -1.0f : 1.0f);
    *s_out = so;
    *c_out = co;
}

// ---------------------------------------------------------------- wave helpers
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    // sum over aligned groups of W consecutive lanes (W a power of two <= 64)
#pragma unroll
    for (int o = 1; o < W; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// v + (v of the lane that DPP control CTRL selects), all lanes active
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// max(v, +0) on the bit pattern (negative floats are negative integers):
// one integer max, no NaN canonicalisation.  Through scalar copies, like
// word_as_bf16x2: a bit cast written directly on an ext_vector element has
// been compiled as if it named element 0.
__device__ __forceinline__ float relu_bits(float v) {
    int b;
    __builtin_memcpy(&b, &v, 4);
    b = b > 0 ? b : 0;
    float r;
    __builtin_memcpy(&r, &b, 4);
    return r;
}

// v of the neighbouring lane l ^ 1 (DPP quad_perm [1,0,3,2]), all lanes active
__device__ __forceinline__ float lane_swap1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xf, 0xf, true));
}

// Sum over each row of 16 lanes, returned in every lane of the row: four DPP
// butterfly steps (lane ^ 1, lane ^ 2, then the 8- and 16-lane mirrors, which
// pair each lane with one in the other half), no LDS round trip.
__device__ __forceinline__ float row16_sum(float v) {
    v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141>(v);  // row_half_mirror
    v = dpp_add<0x140>(v);  // row_mirror
    return v;
}

// Sum over each group of 8 lanes, returned in every lane of the group.
__device__ __forceinline__ float row8_sum(float v) {
    v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141>(v);  // row_half_mirror
    return v;
}

// max / sum of v over lanes l and l ^ 32 with v_permlane32_swap (a VALU
// exchange, no LDS round trip): swapping the upper half of a copy of v with
// the lower half of another copy leaves v[l % 32] in the first and
// v[l % 32 + 32] in the second, in every lane.  Written as asm (with the
// wait states the instruction needs after its operands are written; not
// volatile, so it does not pin the schedule around it):
// through the builtin, the compiler has folded the two results into one.
__device__ __forceinline__ void self_swap32(float v, float* lo, float* hi) {
    uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    *lo = __builtin_bit_cast(float, a);
    *hi = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float xor32_max(float v) {
    float lo, hi;
    self_swap32(v, &lo, &hi);
    return fmaxf(lo, hi);
}
__device__ __forceinline__ float xor32_sum(float v) {
    float lo, hi;
    self_swap32(v, &lo, &hi);
    return lo + hi;
}

__device__ __forceinline__ float lane_value(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over all 64 lanes as a wave-uniform (scalar) value.
__device__ __forceinline__ float wave_sum_uniform(float v) {
    v = row16_sum(v);
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// order-preserving image of an fp32 score: a > b  <=>  key(a) > key(b);
// -0 and +0 share one key.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t b = (s == 0.0f) ? 0u : __float_as_uint(s);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Asynchronous 16-byte-per-lane HBM -> LDS load (global_load_lds_dwordx4):
// lane i writes LDS bytes [lds_base + 16 i, +16).  Written as one asm block
// that saves and restores M0 around the load (M0 carries the LDS base; one
// wait state after writing it), so the compiler neither sees an LDS store
// it would have to wait for nor loses its own M0.  There is no register
// output; completion is awaited explicitly (vmcnt) before the data is read.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gptr), "s"(lds_base)
        : "memory");
}

// The same load without a memory clobber, for the fast tile step: there the
// destination buffer is not touched by any other access until the closing
// barrier (which waits for the load explicitly), so LDS reads of the other
// buffers may move across it.
__device__ __forceinline__ void lds_dma16_nc(const void* gptr, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gptr), "s"(lds_base));
}

// Asynchronous 4-byte-per-lane HBM -> LDS load (global_load_lds_dword):
// lane i writes LDS bytes [lds_base + 4 i, +4).  Same M0 handling as above.
__device__ __forceinline__ void lds_dma4(const void* gptr, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gptr), "s"(lds_base)
        : "memory");
}

// Wait until at most N of this wave's vector-memory operations (loads,
// stores and asynchronous LDS loads, which complete in issue order) are
// still outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);  // vmcnt(N), other counters untouched
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Barrier that waits for this wave's LDS traffic only: asynchronous
// HBM->LDS loads (and other vector-memory operations) stay in flight across
// it.  Signal fences keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace cakv
