// C-ABI entry points of libfa.so (declared in include/fa.h).
//
// Every argument is validated before the first HIP call, so argument errors
// are reported (and testable) on a machine without a GPU. The library keeps
// no state besides a per-device cache of "is this a gfx950" and the tuning
// overrides of fa_set_knob (unset unless a caller sets them).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/fa.h"
#include "fa_launch.h"
#include "fa_sched.h"

namespace {

// fa_set_knob's overrides, indexed by FA_KNOB_*; -1: unset.
std::atomic<int> g_knob[6] = {-1, -1, -1, -1, -1, -1};
// fa_set_clock_telemetry's buffer (NULL: off) and its record count.
std::atomic<unsigned long long*> g_clk{nullptr};
std::atomic<int> g_clk_n{0};

}  // namespace

namespace fa {
int knob(int which) { return (which >= 1 && which <= 5) ? g_knob[which].load(std::memory_order_relaxed) : -1; }
}  // namespace fa

namespace {

struct DtypeInfo {
    int in, out;
};

// K and V bytes of the heads in flight across the chip that phase 1 of the
// workgroup order keeps within: half of the 8 XCDs' 4 MiB L2 caches. The
// serial kernel, four workgroups per CU, runs best with twice that (two
// heads of the causal B4 H12 N8192 D64 forward per XCD: +1.7% over one).
#ifndef FA_WG_KV_BUDGET_MB
#define FA_WG_KV_BUDGET_MB 16
#endif
#ifndef FA_WG_KV_BUDGET_MB_SERIAL
#define FA_WG_KV_BUDGET_MB_SERIAL 32
#endif

// Heads per group in phase 1 of the workgroup order (decode_wg), for heads of
// per_head_kv bytes of K and V. FA_KNOB_WG_GROUP forces it (tuning; clamped
// to the heads per XCD).
int head_group(long long n_bh, long long per_head_kv, bool serial = false) {
    if (const int f = fa::knob(FA_KNOB_WG_GROUP); f >= 1) return f;
    const long long mb = serial ? FA_WG_KV_BUDGET_MB_SERIAL : FA_WG_KV_BUDGET_MB;
    return fa::wg_head_group(n_bh, per_head_kv, mb << 20);
}

// Query tiles (of n_tiles per head) whose workgroups the order interleaves
// across heads at the end (decode_wg phase 2): the lightest 3/8. Fewer leave
// a tail; more add L2 misses for no gain (measured on the causal B4 H12
// N8192 forward and backward). FA_KNOB_WG_LIGHT forces it (tuning).
int light_tiles(int n_tiles) {
    if (const int f = fa::knob(FA_KNOB_WG_LIGHT); f >= 0) return f;
    return (int)((3LL * n_tiles) / 8);
}

bool dtype_info(int dtype, DtypeInfo* di) {
    switch (dtype) {
        case FA_F16: *di = {fa::IN_F16, fa::OUT_F16}; return true;
        case FA_BF16: *di = {fa::IN_BF16, fa::OUT_BF16}; return true;
        case FA_F16_F32OUT: *di = {fa::IN_F16, fa::OUT_F32}; return true;
        case FA_E4M3: *di = {fa::IN_E4M3, fa::OUT_BF16}; return true;
        case FA_BF16_F32OUT: *di = {fa::IN_BF16, fa::OUT_F32}; return true;
        default: return false;
    }
}

bool finite_positive(float x) { return std::isfinite(x) && x > 0.f; }

// Argument checks shared by the entry points and the plan introspection.
int check_shape(int B, int H, int Nq, int Nk, int D, int dtype, DtypeInfo* di) {
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
    if (D != 64 && D != 128) return FA_ERR_HEADDIM;
    if (!dtype_info(dtype, di)) return FA_ERR_DTYPE;
    // element counts must fit 63 bits; the grid must fit 2^31 - 1 workgroups
    const long long bh = (long long)B * H;
    if (bh > (1LL << 31)) return FA_ERR_SHAPE;
    const long long nmax = Nq > Nk ? Nq : Nk;
    if (nmax > 0 && bh > (1LL << 62) / ((long long)nmax * D * 4)) return FA_ERR_SHAPE;
    // one head's rows of any tensor must stay below 2^31 bytes (32-bit
    // buffer descriptors and offsets in the kernels)
    if (nmax * D * 4 >= (1LL << 31)) return FA_ERR_SHAPE;
    const fa::Plan pl = fa::make_plan(di->in, di->out, D, B, H, Nq);
    if (pl.n_wg > 0x7fffffffLL) return FA_ERR_SHAPE;
    return FA_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// The scratch of fa_fwd_splitkv_noalloc: one array per GPU, in the code
// object's device memory. In host code `scratch` names a host-side stand-in,
// not device memory: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[64];

// The current device's address of `scratch`, or NULL if it cannot be had.
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_scratch[dev].store(q, std::memory_order_release);
    return q;
}

std::atomic<int> g_dev_ok[64];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_DEVICE;
    if (dev < 64) {
        const int known = g_dev_ok[dev].load(std::memory_order_relaxed);
        if (known == 1) return FA_OK;
        if (known == 2) return FA_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? FA_OK : FA_ERR_DEVICE;
}

// fa_fwd's mask arguments: window >= 0, and a window needs causal.
bool causal_window_ok(int causal, int window) { return window >= 0 && (window == 0 || causal); }

// The interval extents of fa_fwd_window (-1: unbounded), clamped to Nq + Nk.
bool window_extents(int window_left, int window_right, int Nq, int Nk, int* wl, int* wr) {
    if (window_left < -1 || window_right < -1) return false;
    const int big = Nq + Nk;
    *wl = (window_left < 0 || window_left > big) ? big : window_left;
    *wr = (window_right < 0 || window_right > big) ? big : window_right;
    return true;
}

int run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int D,
        float scale, int wl, int wr, int dtype, void* stream, float dq, float dk, float dv,
        int mod = FA_MOD_NONE, float cap = 0.f, const float* slopes = nullptr, int n_split = 1,
        void* workspace = nullptr, bool check_only = false) {
    DtypeInfo di;
    const int st = check_shape(B, H, Nq, Nk, D, dtype, &di);
    if (st != FA_OK) return st;
    if (!finite_positive(scale) || !finite_positive(dq) || !finite_positive(dk) || !finite_positive(dv))
        return FA_ERR_SCALE;
    const long long rows = (long long)B * H * Nq;
    if (rows == 0) return FA_OK;  // empty problem: nothing to do
    if (!q || !o || !lse) return FA_ERR_NULL;
    if (Nk > 0 && (!k || !v)) return FA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    if (check_only) return FA_OK;
    const int dst = check_device();
    if (dst != FA_OK) return dst;

    const fa::Plan pl = fa::make_plan(di.in, di.out, D, B, H, Nq, mod, n_split > 1);
    fa::Params p;
    p.q = (const uint8_t*)q;
    p.k = (const uint8_t*)k;
    p.v = (const uint8_t*)v;
    p.o = (uint8_t*)o;
    p.lse = lse;
    p.Nq = Nq;
    p.Nk = Nk;
    p.wl = wl;
    p.wr = wr;
    p.n_bh = B * H;
    p.n_qt = pl.n_qt;
    p.hg = head_group(p.n_bh, 2LL * Nk * D * (di.in == fa::IN_E4M3 ? 1 : 2), pl.kernel == fa::KERNEL_SERIAL);
    p.tl = light_tiles(pl.n_qt);
    p.c = scale * dq * dk * 1.44269504088896341f;
    p.out_mul = dv;
    p.H = H;
    p.mod = mod;
    p.mk1 = (mod == FA_MOD_SOFTCAP) ? 2.f * p.c / cap : 0.f;
    p.mk2 = (mod == FA_MOD_SOFTCAP) ? cap * 1.44269504088896341f : 0.f;
    p.scp = (mod == FA_MOD_SOFTCAP) ? fa::softcap_poly((double)scale * dq * dk / cap) : fa::SoftcapPoly{};
    p.slopes = slopes;
    p.n_split = n_split;
    p.ws_o = (float*)workspace;
    p.ws_lse = workspace ? (float*)workspace + (size_t)B * H * n_split * Nq * D : nullptr;
    p.clk_n = g_clk_n.load(std::memory_order_acquire);
    p.clk = p.clk_n > 0 ? g_clk.load(std::memory_order_acquire) : nullptr;
    if (fa::knob(FA_KNOB_DEBUG) > 0)
        std::fprintf(stderr, "fa_fwd: in=%d out=%d D=%d kernel=%d nw=%d qb=%d br=%d bc=%d n_qt=%d n_wg=%lld\n",
                     pl.in, pl.out, pl.D, pl.kernel, pl.nw, pl.qb, pl.br, pl.bc, pl.n_qt, pl.n_wg);
    (void)hipGetLastError();  // clear a stale error left by the caller
    int err = fa::launch(pl, p, stream);
    if (err == 0 && n_split > 1) err = fa::launch_combine(pl, p, stream);
    return err == 0 ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int D,
           float scale, int causal, int window, int dtype, void* stream) {
    if (!causal_window_ok(causal, window)) {
        DtypeInfo di;
        const int st = check_shape(B, H, Nq, Nk, D, dtype, &di);
        return st != FA_OK ? st : FA_ERR_MASK;
    }
    int wl, wr;
    fa::mask_extents(causal, window, Nq, Nk, &wl, &wr);
    return run(q, k, v, o, lse, B, H, Nq, Nk, D, scale, wl, wr, dtype, stream, 1.f, 1.f, 1.f);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
               int D, float scale, int causal, int window, int dtype, void* stream, float descale_q,
               float descale_k, float descale_v) {
    if (dtype != FA_E4M3) return FA_ERR_DTYPE;
    if (!causal_window_ok(causal, window)) {
        DtypeInfo di;
        const int st = check_shape(B, H, Nq, Nk, D, dtype, &di);
        return st != FA_OK ? st : FA_ERR_MASK;
    }
    int wl, wr;
    fa::mask_extents(causal, window, Nq, Nk, &wl, &wr);
    return run(q, k, v, o, lse, B, H, Nq, Nk, D, scale, wl, wr, dtype, stream, descale_q, descale_k, descale_v);
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                  int D, float scale, int window_left, int window_right, int dtype, void* stream, float descale_q,
                  float descale_k, float descale_v) {
    DtypeInfo di;
    const int st = check_shape(B, H, Nq, Nk, D, dtype, &di);
    if (st != FA_OK) return st;
    int wl, wr;
    if (!window_extents(window_left, window_right, Nq, Nk, &wl, &wr)) return FA_ERR_MASK;
    if (dtype != FA_E4M3 && (descale_q != 1.f || descale_k != 1.f || descale_v != 1.f)) return FA_ERR_SCALE;
    return run(q, k, v, o, lse, B, H, Nq, Nk, D, scale, wl, wr, dtype, stream, descale_q, descale_k, descale_v);
}

int fa_fwd_mod(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
               int D, float scale, int window_left, int window_right, int dtype, void* stream, int score_mod,
               float softcap, const float* alibi_slopes) {
    DtypeInfo di;
    const int st = check_shape(B, H, Nq, Nk, D, dtype, &di);
    if (st != FA_OK) return st;
    int wl, wr;
    if (!window_extents(window_left, window_right, Nq, Nk, &wl, &wr)) return FA_ERR_MASK;
    if (score_mod != FA_MOD_NONE && score_mod != FA_MOD_SOFTCAP && score_mod != FA_MOD_ALIBI) return FA_ERR_MOD;
    if (score_mod != FA_MOD_NONE && di.in == fa::IN_E4M3) return FA_ERR_MOD;
    if (score_mod == FA_MOD_SOFTCAP && !finite_positive(softcap)) return FA_ERR_MOD;
    if (score_mod == FA_MOD_ALIBI && (long long)B * H * Nq > 0) {
        if (!alibi_slopes) return FA_ERR_NULL;
        if (!aligned(alibi_slopes, 4)) return FA_ERR_ALIGN;
    }
    return run(q, k, v, o, lse, B, H, Nq, Nk, D, scale, wl, wr, dtype, stream, 1.f, 1.f, 1.f, score_mod, softcap,
               alibi_slopes);
}

long long fa_splitkv_workspace_bytes(int B, int H, int Nq, int D, int num_splits) {
    if (B < 0 || H < 0 || Nq < 0 || D <= 0 || num_splits < 1) return -1;
    if (num_splits == 1) return 0;
    const long long rows = (long long)B * H * num_splits * Nq;
    return rows * D * 4 + rows * 4;
}

int fa_splitkv_num_splits(int B, int H, int Nq, int Nk, int D, int dtype) {
    DtypeInfo di;
    if (check_shape(B, H, Nq, Nk, D, dtype, &di) != FA_OK || di.in == fa::IN_E4M3) return 1;
    const fa::Plan pl = fa::make_plan(di.in, di.out, D, B, H, Nq, fa::MOD_NONE, true);
    const long long tiles = ((long long)Nk + pl.bc - 1) / pl.bc;
    // enough workgroups to fill every CU twice over, with at least 4 key tiles per split
    const long long want = 512;
    long long s = pl.n_wg >= want ? 1 : (want + pl.n_wg - 1) / pl.n_wg;
    if (s > tiles / 4) s = tiles / 4;
    if (s > 256) s = 256;
    return s < 1 ? 1 : (int)s;
}

}  // extern "C"

namespace {

// fa_fwd_splitkv; with scratch, the workspace is the library's static scratch
// array (fa_fwd_splitkv_noalloc) and every argument is checked before it is
// looked up.
int splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int D,
            float scale, int window_left, int window_right, int dtype, void* stream, int num_splits, void* workspace,
            long long workspace_bytes, bool use_scratch) {
    DtypeInfo di;
    const int st = check_shape(B, H, Nq, Nk, D, dtype, &di);
    if (st != FA_OK) return st;
    if (di.in == fa::IN_E4M3) return FA_ERR_DTYPE;
    int wl, wr;
    if (!window_extents(window_left, window_right, Nq, Nk, &wl, &wr)) return FA_ERR_MASK;
    if (num_splits < 1 || num_splits > 1024) return FA_ERR_SHAPE;
    const fa::Plan pl = fa::make_plan(di.in, di.out, D, B, H, Nq, fa::MOD_NONE, true);
    if (pl.n_wg * num_splits > 0x7fffffffLL) return FA_ERR_SHAPE;
    const long long need = fa_splitkv_workspace_bytes(B, H, Nq, D, num_splits);
    const bool needs_ws = (long long)B * H * Nq > 0 && num_splits > 1;
    if (use_scratch) {
        if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
        const int chk = run(q, k, v, o, lse, B, H, Nq, Nk, D, scale, wl, wr, dtype, stream, 1.f, 1.f, 1.f,
                            FA_MOD_NONE, 0.f, nullptr, num_splits, nullptr, true);
        if (chk != FA_OK) return chk;
        if (needs_ws) {
            const int dst = check_device();
            if (dst != FA_OK) return dst;
            workspace = scratch_ptr();
            if (!workspace) return FA_ERR_SCRATCH;
            workspace_bytes = FA_NOALLOC_SCRATCH_BYTES;
        }
    } else if (needs_ws) {
        if (!workspace) return FA_ERR_NULL;
        if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
        if (workspace_bytes < need) return FA_ERR_SHAPE;
    }
    return run(q, k, v, o, lse, B, H, Nq, Nk, D, scale, wl, wr, dtype, stream, 1.f, 1.f, 1.f, FA_MOD_NONE, 0.f,
               nullptr, num_splits, num_splits > 1 ? workspace : nullptr);
}

}  // namespace

extern "C" {

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                   int D, float scale, int window_left, int window_right, int dtype, void* stream, int num_splits,
                   void* workspace, long long workspace_bytes) {
    return splitkv(q, k, v, o, lse, B, H, Nq, Nk, D, scale, window_left, window_right, dtype, stream, num_splits,
                   workspace, workspace_bytes, false);
}

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                           int Nk, int D, float scale, int window_left, int window_right, int dtype, void* stream,
                           int num_splits) {
    return splitkv(q, k, v, o, lse, B, H, Nq, Nk, D, scale, window_left, window_right, dtype, stream, num_splits,
                   nullptr, 0, true);
}

long long fa_bwd_workspace_bytes(int B, int H, int Nq) {
    if (B < 0 || H < 0 || Nq < 0) return -1;
    const long long nqp = ((long long)Nq + 3) / 4 * 4;
    return 2 * (long long)B * H * nqp * 4;
}

}  // extern "C"

namespace {

int run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
            void* dk, void* dv, int B, int H, int Nq, int Nk, int D, float scale, int window_left, int window_right,
            int dtype, void* stream, void* workspace, long long workspace_bytes, int mod, float cap,
            const float* slopes) {
    DtypeInfo di;
    const int st = check_shape(B, H, Nq, Nk, D, dtype, &di);
    if (st != FA_OK) return st;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    int wl, wr;
    if (!window_extents(window_left, window_right, Nq, Nk, &wl, &wr)) return FA_ERR_MASK;
    if (!finite_positive(scale)) return FA_ERR_SCALE;
    if (mod != FA_MOD_NONE && mod != FA_MOD_SOFTCAP && mod != FA_MOD_ALIBI) return FA_ERR_MOD;
    if (mod == FA_MOD_SOFTCAP && !finite_positive(cap)) return FA_ERR_MOD;
    const long long n_bh = (long long)B * H;
    const long long n_qt = ((long long)Nq + 127) / 128, n_kt = ((long long)Nk + 127) / 128;
    if (n_bh * n_qt > 0x7fffffffLL || n_bh * n_kt > 0x7fffffffLL) return FA_ERR_SHAPE;
    const long long nqp = ((long long)Nq + 3) / 4 * 4;
    if ((n_bh * nqp + 255) / 256 > 0x7fffffffLL) return FA_ERR_SHAPE;
    if (n_bh == 0 || (Nq == 0 && Nk == 0)) return FA_OK;  // nothing to write
    if (Nq > 0 && (!q || !o || !dout || !lse || !dq || !workspace)) return FA_ERR_NULL;
    if (Nk > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULL;
    if (mod == FA_MOD_ALIBI && !slopes) return FA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 16) || !aligned(lse, 4) ||
        !aligned(slopes, 4))
        return FA_ERR_ALIGN;
    if (Nq > 0 && workspace_bytes < fa_bwd_workspace_bytes(B, H, Nq)) return FA_ERR_SHAPE;
    const int dst = check_device();
    if (dst != FA_OK) return dst;

    fa::BwdParams p;
    p.q = (const uint8_t*)q;
    p.k = (const uint8_t*)k;
    p.v = (const uint8_t*)v;
    p.o = (const uint8_t*)o;
    p.dout = (const uint8_t*)dout;
    p.lse = lse;
    p.dq = (uint8_t*)dq;
    p.dk = (uint8_t*)dk;
    p.dv = (uint8_t*)dv;
    p.nqp = (int)nqp;
    p.ndvec = (float*)workspace;
    p.l2 = workspace ? (float*)workspace + n_bh * nqp : nullptr;
    p.Nq = Nq;
    p.Nk = Nk;
    p.wl = wl;
    p.wr = wr;
    p.n_bh = (int)n_bh;
    p.n_qt = (int)n_qt;
    p.n_kt = (int)n_kt;
    // the dQ kernel streams K and V, the dK/dV kernel Q and dO
    p.hg = head_group(n_bh, 4LL * (Nq > Nk ? Nq : Nk) * D);
    p.tl = light_tiles((int)(n_qt > n_kt ? n_qt : n_kt));
    p.c = scale * 1.44269504088896341f;
    p.scale = scale;
    p.H = H;
    p.mod = mod;
    p.mk1 = (mod == FA_MOD_SOFTCAP) ? 2.f * p.c / cap : 0.f;
    p.mk2 = (mod == FA_MOD_SOFTCAP) ? cap * 1.44269504088896341f : 0.f;
    p.scp = (mod == FA_MOD_SOFTCAP) ? fa::softcap_poly((double)scale / cap) : fa::SoftcapPoly{};
    p.slopes = slopes;
    (void)hipGetLastError();
    return fa::launch_bwd(di.in, D, p, stream) == 0 ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
           void* dk, void* dv, int B, int H, int Nq, int Nk, int D, float scale, int window_left, int window_right,
           int dtype, void* stream, void* workspace, long long workspace_bytes) {
    return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, D, scale, window_left, window_right, dtype,
                   stream, workspace, workspace_bytes, FA_MOD_NONE, 0.f, nullptr);
}

int fa_bwd_mod(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int D, float scale, int window_left,
               int window_right, int dtype, void* stream, void* workspace, long long workspace_bytes, int score_mod,
               float softcap, const float* alibi_slopes) {
    return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, D, scale, window_left, window_right, dtype,
                   stream, workspace, workspace_bytes, score_mod, softcap, alibi_slopes);
}

const char* fa_status_str(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "invalid or too large sizes";
        case FA_ERR_HEADDIM: return "head dimension must be 64 or 128";
        case FA_ERR_DTYPE: return "unsupported dtype";
        case FA_ERR_MASK: return "window must be >= 0 and needs causal; window extents must be >= -1";
        case FA_ERR_SCALE: return "scale and descales must be finite and positive";
        case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
        case FA_ERR_DEVICE: return "no gfx950 HIP device is current";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_MOD: return "unknown score modifier, a bad modifier parameter, or a modifier with e4m3 inputs";
        case FA_ERR_SCRATCH: return "the problem needs more than the library's static scratch, or it is unavailable";
        default: return "unknown status";
    }
}

int fa_plan_grid(int B, int H, int Nq, int Nk, int D, int causal, int window, int dtype, long long* n_wg, int* br,
                 int* qw, int* bc) {
    DtypeInfo di;
    const int st = check_shape(B, H, Nq, Nk, D, dtype, &di);
    if (st != FA_OK) return st;
    if (!causal_window_ok(causal, window)) return FA_ERR_MASK;
    if (!n_wg || !br || !qw || !bc) return FA_ERR_NULL;
    const fa::Plan pl = fa::make_plan(di.in, di.out, D, B, H, Nq);
    *n_wg = pl.n_wg;
    *br = pl.br;
    *qw = 32 * pl.qb;
    *bc = pl.bc;
    return FA_OK;
}

int fa_plan_tile(int B, int H, int Nq, int Nk, int D, int causal, int window, int dtype, long long wg, int* bh,
                 int* qtile, int* kv_lo, int* kv_hi) {
    DtypeInfo di;
    const int st = check_shape(B, H, Nq, Nk, D, dtype, &di);
    if (st != FA_OK) return st;
    if (!causal_window_ok(causal, window)) return FA_ERR_MASK;
    if (!bh || !qtile || !kv_lo || !kv_hi) return FA_ERR_NULL;
    const fa::Plan pl = fa::make_plan(di.in, di.out, D, B, H, Nq);
    if (wg < 0 || wg >= pl.n_wg) return FA_ERR_SHAPE;
    fa::decode_wg(wg, B * H, pl.n_qt,
                  head_group((long long)B * H, 2LL * Nk * D * (di.in == fa::IN_E4M3 ? 1 : 2),
                             pl.kernel == fa::KERNEL_SERIAL),
                  light_tiles(pl.n_qt), bh, qtile);
    const int r0 = *qtile * pl.br;
    const int r1 = (r0 + pl.br < Nq) ? r0 + pl.br : Nq;
    int wl, wr;
    fa::mask_extents(causal, window, Nq, Nk, &wl, &wr);
    fa::kv_range(r0, r1, Nq, Nk, wl, wr, kv_lo, kv_hi);
    return FA_OK;
}

int fa_plan_block_class(int w0, int w1, int c0, int c1, int Nq, int Nk, int causal, int window) {
    int wl, wr;
    fa::mask_extents(causal, window, Nq, Nk, &wl, &wr);
    return fa::tile_class(w0, w1, c0, c1, Nq, Nk, wl, wr);
}

int fa_plan_window_range(int r0, int r1, int Nq, int Nk, int window_left, int window_right, int* kv_lo,
                         int* kv_hi) {
    int wl, wr;
    if (!window_extents(window_left, window_right, Nq, Nk, &wl, &wr)) return FA_ERR_MASK;
    if (r0 < 0 || r1 <= r0 || r1 > Nq || Nk < 0) return FA_ERR_SHAPE;
    if (!kv_lo || !kv_hi) return FA_ERR_NULL;
    fa::kv_range(r0, r1, Nq, Nk, wl, wr, kv_lo, kv_hi);
    return FA_OK;
}

int fa_plan_block_class_window(int w0, int w1, int c0, int c1, int Nq, int Nk, int window_left, int window_right) {
    int wl, wr;
    if (!window_extents(window_left, window_right, Nq, Nk, &wl, &wr)) return -1;
    return fa::tile_class(w0, w1, c0, c1, Nq, Nk, wl, wr);
}

int fa_set_knob(int knob, int value) {
    if (knob < 1 || knob > 5 || value < -1) return FA_ERR_SHAPE;
    g_knob[knob].store(value, std::memory_order_relaxed);
    return FA_OK;
}

int fa_plan_kernel(int B, int H, int Nq, int Nk, int D, int dtype, int score_mod, int splitkv) {
    DtypeInfo di;
    const int st = check_shape(B, H, Nq, Nk, D, dtype, &di);
    if (st != FA_OK) return -st;
    if (score_mod != FA_MOD_NONE && score_mod != FA_MOD_SOFTCAP && score_mod != FA_MOD_ALIBI) return -FA_ERR_MOD;
    if (score_mod != FA_MOD_NONE && di.in == fa::IN_E4M3) return -FA_ERR_MOD;
    if (splitkv && (score_mod != FA_MOD_NONE || di.in == fa::IN_E4M3)) return -FA_ERR_DTYPE;
    return fa::make_plan(di.in, di.out, D, B, H, Nq, score_mod, splitkv != 0).kernel;
}

int fa_set_clock_telemetry(unsigned long long* buf, int n) {
    if ((buf == nullptr) != (n == 0) || n < 0) return buf == nullptr ? FA_ERR_NULL : FA_ERR_SHAPE;
    if (buf && !aligned(buf, 8)) return FA_ERR_ALIGN;
    // off first, so that a concurrent launch never pairs the new count with the old buffer
    g_clk_n.store(0, std::memory_order_release);
    g_clk.store(buf, std::memory_order_release);
    g_clk_n.store(n, std::memory_order_release);
    return FA_OK;
}

}  // extern "C"
