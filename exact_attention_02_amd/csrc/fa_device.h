// Device helpers shared by the attention kernels for gfx950: MFMA wrappers,
// 16-bit packing, exact e4m3 widening, output stores, cross-half reductions,
// the swizzled LDS layout and buffer-resource (range-checked) copies.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int BC = 64;   // keys per K/V tile staged in LDS
constexpr float LN2 = 0.693147180559945309f;
constexpr float LOG2E = 1.44269504088896341f;

// Per input type: the MFMA used for S^T = K Q^T (always a 16-bit MFMA: e4m3
// inputs are widened exactly to bf16 for it, because the f8f6f4 MFMA sums its
// 64 products with fewer bits than fp32 and the scores feed the LSE), the MFMA
// used for O^T += V^T P^T, and the lazy-rescale threshold.
template <int IN> struct In;
template <> struct In<IN_BF16> {
    static constexpr int EB = 2;            // bytes per stored element
    static constexpr int QK = IN_BF16;      // score MFMA operand type
    static constexpr int PV_KSTEP = 16;     // keys per P.V MFMA
    static constexpr int PV_OPW = 4;        // dwords per P.V operand
    static constexpr float TAU = 8.f, PRESCALE = 1.f;
};
template <> struct In<IN_F16> {
    static constexpr int EB = 2;
    static constexpr int QK = IN_F16;
    static constexpr int PV_KSTEP = 16;
    static constexpr int PV_OPW = 4;
    static constexpr float TAU = 8.f, PRESCALE = 1.f;
};
// e4m3: P is stored as e4m3 of p * 2^6 with p <= 2^TAU = 4, so it stays below
// 256 < 448 (the format's largest value) while small weights keep most of the
// format's range above its smallest subnormal.
template <> struct In<IN_E4M3> {
    static constexpr int EB = 1;
    static constexpr int QK = IN_BF16;
    static constexpr int PV_KSTEP = 64;
    static constexpr int PV_OPW = 8;
    static constexpr float TAU = 2.f, PRESCALE = 64.f;
};

__device__ __forceinline__ f32x16 mfma16(int qk, const i32x4& a, const i32x4& b, const f32x16& c) {
    if (qk == IN_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    // operand format 0 = OCP E4M3 for both; block scales 0 = unscaled.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Two floats -> two 16-bit values (round to nearest even) in one dword.
template <int T> __device__ __forceinline__ int pack2(float a, float b);
template <> __device__ __forceinline__ int pack2<IN_BF16>(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(int, v);
}
template <> __device__ __forceinline__ int pack2<IN_F16>(float a, float b) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(int, v);
}
// Exact inverse of one half of pack2.
template <int T> __device__ __forceinline__ float unpack_lo(int w);
template <int T> __device__ __forceinline__ float unpack_hi(int w);
template <> __device__ __forceinline__ float unpack_lo<IN_BF16>(int w) { return __int_as_float(w << 16); }
template <> __device__ __forceinline__ float unpack_hi<IN_BF16>(int w) { return __int_as_float(w & 0xffff0000); }
template <> __device__ __forceinline__ float unpack_lo<IN_F16>(int w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffff));
}
template <> __device__ __forceinline__ float unpack_hi<IN_F16>(int w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)((unsigned)w >> 16));
}

// Four e4m3 values (one dword) -> four bf16 values (two dwords), exactly.
__device__ __forceinline__ i32x2 e4m3x4_to_bf16(int w) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return i32x2{__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
}

// Output conversion of four consecutive values of a row.
template <int OUT> struct Out;
template <> struct Out<OUT_F32> {
    static constexpr int EB = 4;
    __device__ static void store4(uint8_t* dst, float a, float b, float c, float d) {
        *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
    }
};
template <> struct Out<OUT_BF16> {
    static constexpr int EB = 2;
    __device__ static i32x2 pack4(float a, float b, float c, float d) {
        return i32x2{pack2<IN_BF16>(a, b), pack2<IN_BF16>(c, d)};
    }
    __device__ static void store4(uint8_t* dst, float a, float b, float c, float d) {
        *reinterpret_cast<i32x2*>(dst) = pack4(a, b, c, d);
    }
};
template <> struct Out<OUT_F16> {
    static constexpr int EB = 2;
    __device__ static i32x2 pack4(float a, float b, float c, float d) {
        return i32x2{pack2<IN_F16>(a, b), pack2<IN_F16>(c, d)};
    }
    __device__ static void store4(uint8_t* dst, float a, float b, float c, float d) {
        *reinterpret_cast<i32x2*>(dst) = pack4(a, b, c, d);
    }
};

// This lane's value combined with lane l^32's (the other half of the wave).
__device__ __forceinline__ float max_halves(float x) {
    auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// LDS layout of one K or V tile: BC rows of RB bytes; the 16-byte chunk c of
// row x sits at chunk position c ^ (x mod SW) with SW = min(chunks per row, 8),
// so lanes reading one chunk column of consecutive rows hit distinct banks.
template <int RB>
__device__ __forceinline__ int lds_off(int x, int chunk) {
    constexpr int SW = (RB / 16) < 8 ? (RB / 16) : 8;
    return x * RB + ((chunk ^ (x & (SW - 1))) << 4);
}

// For e4m3, V's rows are stored permuted so that each lane half's 32 keys --
// the keys its 32 P values belong to -- are 32 consecutive LDS rows, which is
// the row run ds_read_b64_tr_b8 reads (8 rows per read). Key x = 32*blk +
// 8*a + 4*h + b goes to LDS row 32*h + 16*blk + 4*a + b.
__device__ __forceinline__ int v8_row(int x) {
    const int blk = x >> 5, a = (x >> 3) & 3, h = (x >> 2) & 1, b = x & 3;
    return (h << 5) | (blk << 4) | (a << 2) | b;
}

__device__ __forceinline__ int v8_row_inv(int xv) {
    const int h = xv >> 5, blk = (xv >> 4) & 1, a = (xv >> 2) & 3, b = xv & 3;
    return (blk << 5) | (a << 3) | (h << 2) | b;
}

// Buffer resource over [base, base + bytes): loads beyond `bytes` return
// zeros (and write zeros to LDS), so tails need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// The same descriptor as four dwords (base, stride 0, byte count, raw format).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, unsigned bytes) {
    const unsigned long long a = (unsigned long long)base;
    return i32x4{(int)(a & 0xffffffffu), (int)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// LDS layout of a K or V tile: row x of RB bytes holds its 16-byte chunk c at
// position c ^ swz(x). LDS serves 256 bytes (64 banks of 4 bytes) per cycle:
// a 16-lane group of 16-byte score-operand reads covers 16 consecutive rows
// at one chunk, and a 32-lane half of the transposing V reads covers 4
// consecutive rows at 4 aligned chunks. swz spreads both over distinct
// banks: at 128-byte rows, two rows share a 256-byte bank cycle and
// swz = ((x >> 1) & 1) << 2 | (x >> 2) & 3 separates rows x, x + 2 into
// different groups of four chunks; at 256-byte rows, swz = (x & 3) << 2 |
// (x >> 2) & 3 does the same for four consecutive rows. It depends on x mod
// 16 only.
template <int RB>
__device__ __forceinline__ int swz16(int x) {
    if constexpr (RB == 128) return (((x >> 1) & 1) << 2) | ((x >> 2) & 3);
    else return ((x & 3) << 2) | ((x >> 2) & 3);
}
template <int RB>
__device__ __forceinline__ int lds_pos(int x, int c) {
    return x * RB + ((c ^ swz16<RB>(x)) << 4);
}

// HBM -> LDS copy of 16 bytes per lane: lane l's bytes land at LDS address
// lds_base + 16*l (lds_base wave-uniform). Issued from asm so that the
// compiler does not hold every later transposing LDS read until all such
// copies land; completion is awaited explicitly (vmcnt(0)) before the barrier
// that publishes the tile. The block writes no register, and m0 is set here:
// gfx950 does not use m0 for ordinary LDS access.
__device__ __forceinline__ void dma16(const i32x4& rsrc, unsigned lds_base, unsigned voff) {
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :
                 : "v"(voff), "s"(lds_base), "s"(rsrc)
                 : "memory", "m0");
}
// The same with a wave-uniform byte offset soff added to every lane's voff.
__device__ __forceinline__ void dma16(const i32x4& rsrc, unsigned lds_base, unsigned voff, unsigned soff) {
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
                 :
                 : "v"(voff), "s"(lds_base), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// ds_read_b64_tr_b16 at an LDS byte address: in each 16-lane group, lanes
// 4r..4r+3 name row r of a 4 x 16 block of 16-bit values (8 bytes each) and
// lane c receives column c of the 4 rows.
__device__ __forceinline__ i32x2 read_tr16(const lds_u8* addr) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)addr);
    return __builtin_bit_cast(i32x2, v);
}

// Softcap, s <- cap * tanh(x) with x = scale * s / cap, on small arguments:
// for |x| <= SC_POLY_X the Taylor polynomial x - x^3/3 + 2x^5/15 - 17x^7/315
// is within 62 |x|^9 / 2835 <= 1.2e-8 of tanh(x) (the series alternates with
// decreasing terms there). It costs six FMAs and multiplies where the closed
// form tanh|x| = 1 - 2 / (e^(2|x|) + 1) costs an exponential and a reciprocal.
// A lane takes it for its 16 scores of a block when all of them lie in range
// (softcap_poly_ok); a masked score (-inf) sends the lane to the closed form.
// tanh(kx * s) for |s| <= smax
__device__ __forceinline__ float softcap_tanh_poly(const SoftcapPoly& P, float s) {
    const float s2 = s * s;
    float q = fmaf(s2, P.d, P.c);
    q = fmaf(s2, q, P.b);
    const float sx = s * P.kx;
    return fmaf(sx * s2, q, sx);
}
// every one of the 16 scores within the polynomial's range
__device__ __forceinline__ bool softcap_poly_ok(const SoftcapPoly& P, const f32x16& S) {
    float am = fabsf(S[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) am = fmaxf(am, fabsf(S[r]));
    return am <= P.smax;
}

// Opt-in clock telemetry (fa_set_clock_telemetry in include/fa.h): the first
// lane of a workgroup writes the shader-clock counter (s_memtime) and the
// fixed 100 MHz counter (s_memrealtime) to record blockIdx.x mod clk_n, at the
// workgroup's start (half 0) and at its end (half 1). A kernel argument
// decides it, so with telemetry off the cost is one scalar branch each time.
__device__ __forceinline__ void clock_stamp(unsigned long long* clk, int clk_n, int half) {
    if (clk != nullptr && threadIdx.x == 0) {
        unsigned long long* o = clk + 4 * (size_t)(blockIdx.x % (unsigned)clk_n) + 2 * half;
        o[0] = (unsigned long long)__builtin_amdgcn_s_memtime();
        o[1] = (unsigned long long)__builtin_amdgcn_s_memrealtime();
    }
}

}  // namespace fa
