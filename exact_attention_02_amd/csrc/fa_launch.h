// Internal interface between the C-ABI entry points and the kernels.
#pragma once

#include <stdint.h>

namespace fa {

enum InKind { IN_F16 = 0, IN_BF16 = 1, IN_E4M3 = 2 };
enum OutKind { OUT_F32 = 0, OUT_F16 = 1, OUT_BF16 = 2 };

// KERNEL_TILE64: 64-key tiles, one softmax per tile (all input types).
// KERNEL_PIPE16: 16-bit inputs, scores of the next 32 keys formed during the
// softmax of the current 32 (fa_fwd16.hip).
enum ScoreMod { MOD_NONE = 0, MOD_SOFTCAP = 1, MOD_ALIBI = 2 };
// Softcap on small arguments: tanh(kx * s) by an odd polynomial for |s| <=
// smax (softcap_tanh_poly in fa_device.h). Filled on the host, so that the
// kernels read the constants from their arguments.
constexpr double SC_POLY_X = 0.2;   // largest |x| = |kx * s| on the polynomial
struct SoftcapPoly {
    float kx;       // scale / cap
    float b, c, d;  // -kx^2 / 3, 2 kx^4 / 15, -17 kx^6 / 315
    float smax;     // SC_POLY_X / kx
};
inline SoftcapPoly softcap_poly(double kx) {
    const double x2 = kx * kx;
    return {(float)kx, (float)(-x2 / 3), (float)(2 * x2 * x2 / 15), (float)(-17 * x2 * x2 * x2 / 315),
            (float)(SC_POLY_X / kx)};
}
// KERNEL_KSPLIT: 16-bit inputs at D = 64 on small grids, 32 query rows per
// workgroup whose waves split the keys (fa_fwd_ks.hip).
// KERNEL_SERIAL: 16-bit inputs, with or without a score modifier, one 32 x 32
// block at a time per wave, four waves per SIMD at D = 64 (fa_serial.h).
enum KernelKind { KERNEL_TILE64 = 0, KERNEL_PIPE16 = 1, KERNEL_KSPLIT = 2, KERNEL_SERIAL = 3 };

// Everything a workgroup needs; passed by value as the kernel argument.
struct Params {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    uint8_t* o;
    float* lse;
    int Nq, Nk;
    int wl, wr;     // row i sees keys [i' - wl, i' + wr], i' = i + Nk - Nq (clamped to Nq + Nk)
    int n_bh;       // B * H
    int H;          // heads (ALiBi: the head of bh is bh % H)
    int mod;        // MOD_NONE, MOD_SOFTCAP or MOD_ALIBI (16-bit kernel only)
    float mk1, mk2; // softcap constants: 2 * c / cap and cap * log2(e)
    SoftcapPoly scp;  // softcap on small arguments (fa_device.h)
    const float* slopes;  // ALiBi: [H] device array of per-head slopes
    // Split-KV: each head's key tiles are split into n_split contiguous ranges,
    // one workgroup each; a split writes its O (divided by its own sum) and its
    // LSE in fp32 to ws_o [n_bh, n_split, Nq, D] and ws_lse [n_bh, n_split, Nq].
    int n_split;    // 1: no split (O and LSE go to o and lse directly)
    float* ws_o;
    float* ws_lse;
    int n_qt;       // query tiles per head
    int hg;         // workgroup order (decode_wg): heads per group in phase 1,
    int tl;         // and the query tiles below tl that phase 2 interleaves
    float c;        // scale * descale_q * descale_k * log2(e): scores in base-2 units
    float out_mul;  // descale_v (1 unless e4m3)
    // fa_set_clock_telemetry: NULL, or clk_n records of four 64-bit counters
    // (shader clock and 100 MHz at a workgroup's start, then at its end)
    unsigned long long* clk;
    int clk_n;
};

// The backward's arguments (16-bit inputs, D = 64 or 128). ndvec and l2 are
// a workspace of 2 * n_bh * nqp floats: per row, -(dO . O) and the LSE in
// base-2 units (+inf for a row that sees no key), rows of a head padded to
// nqp, a multiple of 4.
struct BwdParams {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    const uint8_t* o;
    const uint8_t* dout;
    const float* lse;
    uint8_t* dq;
    uint8_t* dk;
    uint8_t* dv;
    float* ndvec;
    float* l2;
    int Nq, Nk;
    int wl, wr;     // as in Params
    int n_bh;
    int nqp;        // Nq rounded up to a multiple of 4
    int n_qt;       // 128-row query blocks per head (dQ kernel)
    int n_kt;       // 128-key blocks per head (dK/dV kernel)
    int hg;         // workgroup order (decode_wg): heads per group in phase 1,
    int tl;         // and the key blocks below tl that phase 2 interleaves
    float c;        // scale * log2(e)
    float scale;
    int H;          // heads (ALiBi: the head of bh is bh % H)
    int mod;        // MOD_NONE, MOD_SOFTCAP or MOD_ALIBI
    float mk1, mk2; // softcap constants: 2 * c / cap and cap * log2(e)
    SoftcapPoly scp;  // softcap on small arguments (fa_device.h)
    const float* slopes;  // ALiBi: [H] device array of per-head slopes
};

// Enqueues the three backward kernels on `stream`; returns hipGetLastError().
int launch_bwd(int in, int D, const BwdParams& p, void* stream);

// Tile shape a launch uses.
struct Plan {
    int in, out, D;
    int kernel;     // KERNEL_TILE64, KERNEL_PIPE16 or KERNEL_KSPLIT
    int nw;         // waves per workgroup
    int qb;         // 32-row query blocks per wave
    int br;         // query rows per workgroup (nw * 32 * qb)
    int bc;         // key rows per tile
    int n_qt;
    long long n_wg;
};

// The current value of a tuning override of fa_set_knob (include/fa.h), -1
// when unset.
int knob(int which);

// Waves (32 query rows each) per workgroup of the serial kernel. At D = 128
// eight waves (one workgroup per CU) halve the K/V staging per query row and
// run at a higher clock: causal B1 H32 N32768 +4%, with a 4096-key window
// +0.7%; they are used when the grid still gives every CU a workgroup. At
// D = 64 four waves (four workgroups per CU) are faster on causal problems.
#ifndef FA_SR_NW_D64
#define FA_SR_NW_D64 4
#endif
#ifndef FA_SR_NW_D128
#define FA_SR_NW_D128 8
#endif
// Keys per K/V tile of the serial kernel (64, or 128 with eight waves).
#ifndef FA_SR_TK_D64
#define FA_SR_TK_D64 64
#endif
#ifndef FA_SR_TK_D128
#define FA_SR_TK_D128 64
#endif
// e4m3 inputs at D = 128 with eight waves: keys per tile.
#ifndef FA_SR_TK_E4M3_D128
#define FA_SR_TK_E4M3_D128 128
#endif
// Keys per tile a serial-kernel plan takes for nw waves and tile size tk.
constexpr int serial_tile_keys(int nw, int tk) { return (nw == 8 && tk == 128) ? 128 : 64; }
// ... for input type in (InKind) at head size D.
constexpr int serial_tile_keys(int in, int D, int nw) {
    return serial_tile_keys(nw, in == IN_E4M3 && D == 128 ? FA_SR_TK_E4M3_D128
                                                                  : (D == 64 ? FA_SR_TK_D64 : FA_SR_TK_D128));
}

// Picks the tile shape for a problem. Pure host arithmetic.
// mod != MOD_NONE needs the serial or the pipelined kernel, the ones with
// score modifiers; splitkv (split-KV) runs on the serial, the pipelined or the
// key-split kernel.
Plan make_plan(int in, int out, int D, int B, int H, int Nq, int mod = MOD_NONE, bool splitkv = false);

// Enqueues the kernel chosen by `plan` on `stream`; returns the hipError_t
// value of hipGetLastError() after the launch (0 on success).
int launch(const Plan& plan, const Params& p, void* stream);
int launch16(const Plan& plan, const Params& p, void* stream);
int launch_ks(const Plan& plan, const Params& p, void* stream);
int launch_serial(const Plan& plan, const Params& p, void* stream);
// The serial kernel's launches for one input type and score modifier
// (fa_serial.h); each set is instantiated in an object of its own
// (fa_fwd_serial_inst.hip), launch_serial picks the set.
template <int IN, int MOD>
int launch_serial_in(const Plan& plan, const Params& p, void* stream);
// The merge of the splits (p.n_split > 1): O and LSE from ws_o and ws_lse.
int launch_combine(const Plan& plan, const Params& p, void* stream);

}  // namespace fa
