/*
 * fa.h -- C ABI of the MI355X (gfx950) fused exact-attention forward library.
 *
 * The operation is scaled dot-product attention,
 *     O = softmax(scale * Q K^T) V,
 * (aiinarabic.com "flash-attention" page, equation (1), with scale = 1/sqrt(d_k)
 * there), computed tile by tile with an online softmax so the Nq x Nk score
 * matrix is never written to device memory (same page, the kernel-fusion
 * discussion and Figure 4; inskillml course module 9, "FlashAttention: compute
 * without writing the weights"). Besides O the call writes each row's
 * log-sum-exp, the softmax normaliser the pages say the forward keeps for the
 * backward pass (aiinarabic.com page, the recomputation paragraph).
 *
 * Tensor layout follows the SDPA call in inskillml module 9: (batch, heads,
 * sequence, head_dim), contiguous and row-major:
 *     q   [B, H, Nq, D]      k, v [B, H, Nk, D]
 *     o   [B, H, Nq, D]      lse  [B, H, Nq]  (float32)
 * All of q, k, v, o, lse are device pointers; q, k, v, o 16-byte aligned and
 * lse 4-byte aligned. The caller allocates and owns every buffer; the library
 * allocates nothing, frees nothing and keeps no pointer after the call.
 *
 * Masks (is_causal in the SDPA call; sliding windows in module 9's "Sparse
 * patterns" section):
 *     causal != 0 : query row i sees keys j <= i + (Nk - Nq)
 *                   (rows aligned at the bottom right when Nq != Nk).
 *     window  > 0 : additionally j > i + (Nk - Nq) - window, i.e. the `window`
 *                   most recent keys including the diagonal. Needs causal.
 *     window == 0 : no window.
 * fa_fwd_window takes the mask as one key interval per row instead: row i
 * sees the keys j with
 *     i' - window_left <= j <= i' + window_right,   i' = i + (Nk - Nq),
 * where -1 leaves that side unbounded. (-1, 0) is the causal mask, (w-1, 0)
 * the causal window above, (w, w) the sliding window |i - j| <= w of module
 * 9's sparse-attention-patterns section (w keys on each side of the token),
 * and (-1, -1) no mask.
 * A row that sees no key gets O = 0 and LSE = -inf.
 *
 * Streams: work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 * the default stream) and the call returns without synchronising. Faults inside
 * the kernel surface at the caller's next synchronisation, as usual in HIP.
 *
 * Errors: every argument is checked before any HIP call; on an argument error
 * the outputs are untouched and nothing is enqueued. No C++ exception or abort
 * crosses this boundary. The functions are re-entrant and thread-safe.
 */
#ifndef FA_H_
#define FA_H_

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtypes: inputs -> output. LSE is always float32. */
enum {
    FA_F16 = 1,          /* q, k, v float16  -> o float16  */
    FA_BF16 = 2,         /* q, k, v bfloat16 -> o bfloat16 */
    FA_F16_F32OUT = 3,   /* q, k, v float16  -> o float32  */
    FA_E4M3 = 4,         /* q, k, v OCP E4M3FN (8-bit, bias 7, max 448) -> o bfloat16 */
    FA_BF16_F32OUT = 5   /* q, k, v bfloat16 -> o float32  */
};

/* Status codes. */
enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,     /* a negative size, sizes whose products overflow, or
                             max(Nq, Nk) * D * 4 >= 2^31 (one head's rows) */
    FA_ERR_HEADDIM = 3,   /* D is not 64 or 128 */
    FA_ERR_DTYPE = 4,     /* unknown dtype, or fa_fwd_fp8 with a non-e4m3 dtype */
    FA_ERR_MASK = 5,      /* window < 0, or window > 0 without causal; or a
                             window extent below -1 (fa_fwd_window) */
    FA_ERR_SCALE = 6,     /* scale or a descale is not finite and positive */
    FA_ERR_ALIGN = 7,     /* q/k/v/o not 16-byte aligned, or lse not 4-byte aligned */
    FA_ERR_DEVICE = 8,    /* no HIP device, or the current device is not gfx950 */
    FA_ERR_LAUNCH = 9,    /* the kernel launch failed (hipGetLastError) */
    FA_ERR_MOD = 10,      /* fa_fwd_mod: unknown score modifier, softcap not finite
                             and positive, or a modifier with FA_E4M3 inputs */
    FA_ERR_SCRATCH = 11   /* fa_fwd_splitkv_noalloc: the problem needs more than the
                             library's static scratch (FA_NOALLOC_SCRATCH_BYTES), or
                             the scratch's device address could not be obtained */
};

/* Score modifiers of fa_fwd_mod. */
enum {
    FA_MOD_NONE = 0,
    FA_MOD_SOFTCAP = 1,   /* s <- softcap * tanh(s / softcap) */
    FA_MOD_ALIBI = 2      /* s <- s + alibi_slopes[h] * (j - i'), i' = i + Nk - Nq */
};

/*
 * fa_fwd: attention forward, O and LSE.
 *   q, k, v : inputs in the layout above, in `dtype`'s input type.
 *   o       : output [B,H,Nq,D] in `dtype`'s output type.
 *   lse     : output [B,H,Nq] float32, natural-log log-sum-exp of the scaled
 *             scores over the visible keys: ln sum_j exp(scale * q_i . k_j).
 *   B, H, Nq, Nk, D : sizes; any of B, H, Nq equal to 0 is an empty problem
 *             (FA_OK, nothing enqueued); Nk = 0 gives O = 0, LSE = -inf.
 *   scale   : multiplier of the dot products (1/sqrt(D) in the pages).
 *   causal, window : the masks above.
 *   dtype   : one of the FA_* dtypes; FA_E4M3 behaves as fa_fwd_fp8 with all
 *             descales 1.
 *   stream  : hipStream_t or NULL.
 * Returns FA_OK or an FA_ERR_* code.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Nq, int Nk, int D, float scale,
           int causal, int window, int dtype, void* stream);

/*
 * fa_fwd_fp8: as fa_fwd for FA_E4M3 inputs that were quantised per tensor.
 * The real values are q8 * descale_q, k8 * descale_k and v8 * descale_v, so
 * the scores are scale * descale_q * descale_k * (q8 . k8) and the output is
 * descale_v * softmax(...) v8. FP8 inputs are the low-precision path of
 * FlashAttention-3 (news.hamidun.com FlashAttention-3 item, "How the speedup
 * works", third point). dtype must be FA_E4M3.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Nq, int Nk, int D, float scale,
               int causal, int window, int dtype, void* stream,
               float descale_q, float descale_k, float descale_v);

/*
 * fa_fwd_window: as fa_fwd, with the mask given as the key interval
 * [i' - window_left, i' + window_right] of each row (see the header comment;
 * -1 leaves a side unbounded, larger extents than Nq + Nk act as unbounded).
 * descale_q, descale_k, descale_v apply to FA_E4M3 inputs as in fa_fwd_fp8 and
 * must be 1 for the other dtypes (FA_ERR_SCALE otherwise). Errors as fa_fwd;
 * an extent below -1 is FA_ERR_MASK.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Nq, int Nk, int D, float scale,
                  int window_left, int window_right, int dtype, void* stream,
                  float descale_q, float descale_k, float descale_v);

/*
 * fa_fwd_mod: as fa_fwd_window, with a modifier applied to every visible
 * scaled score s = scale * q_i . k_j before the softmax -- the score_mod
 * variants FLASHLIGHT generates kernels for (gist.science summary of
 * FLASHLIGHT, Results: ALiBi and Softcap among the variants):
 *   FA_MOD_NONE    : none (the same results as fa_fwd_window);
 *   FA_MOD_SOFTCAP : s <- softcap * tanh(s / softcap); softcap finite, > 0;
 *   FA_MOD_ALIBI   : s <- s + alibi_slopes[h] * (j - i'), i' = i + (Nk - Nq),
 *                    h the head; alibi_slopes is a device array of H float32
 *                    (4-byte aligned) the caller owns.
 * The LSE output is the log-sum-exp of the modified scores.
 * fp16 and bf16 inputs only (FA_ERR_MOD for FA_E4M3 with a modifier).
 * Errors as fa_fwd_window, plus FA_ERR_MOD, and FA_ERR_NULL for a NULL
 * alibi_slopes with FA_MOD_ALIBI on a non-empty problem.
 */
int fa_fwd_mod(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Nq, int Nk, int D, float scale,
               int window_left, int window_right, int dtype, void* stream,
               int score_mod, float softcap, const float* alibi_slopes);

/*
 * Split-KV (decode-shaped problems, Nq << Nk): fa_fwd_splitkv splits the key
 * range of every (batch, head, query tile) into num_splits contiguous parts,
 * one workgroup each, so that a few long rows still spread over the whole
 * chip. Each part writes its partial O (normalised by its own sum) and its
 * LSE in fp32 to `workspace`; a second kernel on the same stream merges them
 * with the online-softmax identity (gist.science summary of FLASHLIGHT,
 * Methodology item 3):
 *     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) * O_s.
 * The result is the same attention as fa_fwd_window up to rounding.
 *
 * fa_splitkv_workspace_bytes: bytes of workspace fa_fwd_splitkv needs
 *   (B*H*num_splits*Nq*(D+1)*4; 0 for num_splits == 1), or -1 for bad sizes.
 * fa_splitkv_num_splits: a split count that gives about 512 workgroups,
 *   with at least 4 key tiles of 64 per split (1 when splitting does not pay
 *   or the arguments are invalid).
 * fa_fwd_splitkv: as fa_fwd_window for fp16/bf16 inputs (FA_ERR_DTYPE for
 *   FA_E4M3). workspace: device memory of at least workspace_bytes >=
 *   fa_splitkv_workspace_bytes(...), 16-byte aligned, owned by the caller,
 *   overwritten by the call; it must not be shared by calls that may run
 *   concurrently. num_splits in [1, 1024] (FA_ERR_SHAPE otherwise, or when the
 *   workspace is too small); num_splits == 1 needs no workspace.
 */
long long fa_splitkv_workspace_bytes(int B, int H, int Nq, int D, int num_splits);
int fa_splitkv_num_splits(int B, int H, int Nq, int Nk, int D, int dtype);
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int D, float scale,
                   int window_left, int window_right, int dtype, void* stream,
                   int num_splits, void* workspace, long long workspace_bytes);

/*
 * fa_fwd_splitkv_noalloc: fa_fwd_splitkv for callers that cannot allocate
 * device memory around the call -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. The split results go to a
 * scratch array the library holds in device memory (FA_NOALLOC_SCRATCH_BYTES
 * on each GPU it runs on, kept until the process ends) instead of a caller's
 * workspace; the call allocates and frees nothing. Arguments, results and
 * errors as fa_fwd_splitkv without (workspace, workspace_bytes), plus
 * FA_ERR_SCRATCH when fa_splitkv_workspace_bytes(B, H, Nq, D, num_splits)
 * exceeds FA_NOALLOC_SCRATCH_BYTES (checked before any device work). Every
 * split writes its whole slice of the scratch before the merge reads it, so
 * nothing is cleared between calls. All calls on one GPU share its array:
 * calls that may overlap on that GPU (on several streams, or from several
 * threads) race on it and must be serialised by the caller.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32LL << 20)
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int D, float scale,
                           int window_left, int window_right, int dtype, void* stream,
                           int num_splits);

/*
 * Backward pass: the gradients dQ, dK, dV of O = softmax(scale Q K^T) V
 * (with the mask of fa_fwd_window) contracted with an upstream gradient dO.
 * The softmax weights are formed again from Q, K and the forward's LSE
 * rather than read from memory (aiinarabic.com flash-attention page, the
 * paragraph on recomputation: only the softmax normaliser is kept from the
 * forward pass). With P = exp(scale S - LSE) and D_i = dO_i . O_i:
 *     dV = P^T dO,  dS = P o (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *
 * q, o, dout, dq: [B, H, Nq, D]; k, v, dk, dv: [B, H, Nk, D]; all
 *   contiguous, of `dtype` (FA_F16 or FA_BF16; FA_ERR_DTYPE otherwise),
 *   16-byte aligned device memory. o and lse are the forward's outputs for
 *   the same q, k, v, scale and extents (lse: [B, H, Nq] float32, -inf for a
 *   row that sees no key; such rows get dQ = 0 and add nothing to dK, dV).
 * dq, dk, dv: outputs, overwritten (keys that no row sees get dK = dV = 0).
 * window_left, window_right: the extents of fa_fwd_window.
 * workspace: device memory of at least fa_bwd_workspace_bytes(B, H, Nq)
 *   bytes, 16-byte aligned, owned by the caller and overwritten; calls that
 *   may run concurrently must not share it (FA_ERR_SHAPE when too small,
 *   FA_ERR_NULL when NULL and Nq > 0).
 * Every kernel is enqueued on `stream`; the call does not synchronise.
 * Errors as fa_fwd_window (scale must be finite and positive).
 *
 * fa_bwd_workspace_bytes: 8 * B * H * (Nq rounded up to a multiple of 4),
 *   or -1 for negative sizes.
 */
long long fa_bwd_workspace_bytes(int B, int H, int Nq);
/*
 * fa_bwd_mod: fa_bwd for the attention of fa_fwd_mod, whose scores pass
 * through a modifier f before the softmax (score_mod, softcap and
 * alibi_slopes as in fa_fwd_mod; o and lse must come from fa_fwd_mod with the
 * same modifier). P is the softmax of the modified scores and dS picks up
 * f'(s) by the chain rule: 1 - tanh(s / cap)^2 for FA_MOD_SOFTCAP, 1 for
 * FA_MOD_ALIBI. Errors as fa_bwd, plus FA_ERR_MOD for an unknown modifier or
 * a softcap that is not finite and positive, FA_ERR_NULL for a NULL
 * alibi_slopes with FA_MOD_ALIBI, FA_ERR_ALIGN if it is not 4-byte aligned.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int Nq, int Nk, int D, float scale,
           int window_left, int window_right, int dtype, void* stream,
           void* workspace, long long workspace_bytes);
int fa_bwd_mod(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv,
               int B, int H, int Nq, int Nk, int D, float scale,
               int window_left, int window_right, int dtype, void* stream,
               void* workspace, long long workspace_bytes,
               int score_mod, float softcap, const float* alibi_slopes);

/* Static, human-readable text for a status code (never NULL). */
const char* fa_status_str(int status);

/*
 * Launch-plan introspection (host only; no HIP call, usable without a GPU).
 * These expose the logical-grid scheduler the kernel uses, so its coverage and
 * bijection properties can be tested on the CPU.
 *
 * fa_plan_grid: for a problem, the workgroup count, the query rows per
 *   workgroup (br), the query rows per wave (qw) and the key rows per tile (bc)
 *   that fa_fwd would launch with. Returns FA_OK or an argument error code.
 */
int fa_plan_grid(int B, int H, int Nq, int Nk, int D, int causal, int window, int dtype,
                 long long* n_wg, int* br, int* qw, int* bc);

/*
 * fa_plan_tile: for workgroup `wg` of that plan, its (batch*head) index, its
 *   query tile, and the key range [kv_lo, kv_hi) it visits.
 */
int fa_plan_tile(int B, int H, int Nq, int Nk, int D, int causal, int window, int dtype,
                 long long wg, int* bh, int* qtile, int* kv_lo, int* kv_hi);

/*
 * fa_plan_block_class: the class the kernel gives a block of query rows
 *   [w0, w1) against keys [c0, c1): 0 skipped (no visible pair), 1 computed
 *   without a mask (every pair visible), 2 computed with the mask.
 */
int fa_plan_block_class(int w0, int w1, int c0, int c1, int Nq, int Nk, int causal, int window);

/*
 * fa_plan_window_range: the keys [*kv_lo, *kv_hi) visible to at least one row
 * of [r0, r1) under fa_fwd_window's mask -- the key range a workgroup owning
 * those rows visits. Returns FA_OK, FA_ERR_MASK for an extent below -1,
 * FA_ERR_SHAPE unless 0 <= r0 < r1 <= Nq and Nk >= 0, FA_ERR_NULL for a NULL
 * output pointer.
 */
int fa_plan_window_range(int r0, int r1, int Nq, int Nk, int window_left, int window_right,
                         int* kv_lo, int* kv_hi);

/*
 * fa_plan_block_class_window: as fa_plan_block_class under fa_fwd_window's
 * mask; -1 for an extent below -1.
 */
int fa_plan_block_class_window(int w0, int w1, int c0, int c1, int Nq, int Nk,
                               int window_left, int window_right);

/*
 * fa_plan_kernel: which forward kernel a call would launch (host only):
 *   0  the 64-key-tile kernel     (e4m3 inputs split by fa_fwd_splitkv,
 *                                  which rejects them; else only when forced)
 *   1  the pipelined kernel       (only when forced)
 *   2  the key-split kernel       (16-bit inputs at D = 64 with no score
 *                                  modifier on small grids)
 *   3  the serial kernel          (every other call: 16-bit inputs with or
 *                                  without a score modifier, e4m3 inputs)
 * score_mod != 0 plans fa_fwd_mod, splitkv != 0 fa_fwd_splitkv (which also
 * launches the merge kernel when its split count exceeds 1), else fa_fwd and
 * fa_fwd_window. Returns the kind, or minus an argument error code.
 */
int fa_plan_kernel(int B, int H, int Nq, int Nk, int D, int dtype, int score_mod, int splitkv);

/*
 * Tuning and test overrides of the launch planning, process-wide and off by
 * default: the library reads no environment variable. fa_set_knob sets one
 * (value -1 restores the planner's own choice) and returns FA_OK, or
 * FA_ERR_SHAPE for an unknown knob or a value below -1. Results stay within
 * the parity bounds under every setting; the tests use these to run each
 * kernel and tile shape on every case.
 *   FA_KNOB_KERNEL    force a kernel kind of fa_plan_kernel where it applies
 *                     (0 any input without a score modifier; 1 16-bit
 *                     inputs; 2 16-bit inputs at D = 64 with no score
 *                     modifier; 3 any input, e4m3 without a modifier or a
 *                     split)
 *   FA_KNOB_TILE_QB   query blocks of 32 rows per wave (1 or 2; D = 64) for
 *                     the 64-key-tile and pipelined kernels
 *   FA_KNOB_WG_GROUP  heads per group in phase 1 of the workgroup order
 *   FA_KNOB_WG_LIGHT  query tiles per head interleaved in its phase 2
 *   FA_KNOB_DEBUG     nonzero: print each launch plan to stderr
 * Setting a knob while another thread launches gives that launch either
 * value; the outputs are valid under both.
 */
enum { FA_KNOB_KERNEL = 1, FA_KNOB_TILE_QB = 2, FA_KNOB_WG_GROUP = 3, FA_KNOB_WG_LIGHT = 4, FA_KNOB_DEBUG = 5 };
int fa_set_knob(int knob, int value);

/*
 * fa_set_clock_telemetry: a measurement aid, off by default. With buf a
 * caller-owned device buffer of 4 * n 64-bit values (8-byte aligned), every
 * forward launch after the call has the first lane of each workgroup w write
 * the shader-clock counter (s_memtime) and the fixed 100 MHz counter
 * (s_memrealtime) when w starts, to buf[4 * (w mod n)] and the next value, and
 * both again when w ends, to the two values after. Summed over the workgroups
 * of one launch, the shader counter's advance over the 100 MHz counter's,
 * times 100 MHz, is the mean shader clock the kernel ran at. fa_set_clock_
 * telemetry(NULL, 0) turns it off. The setting is process-wide; launches on
 * several streams while it is on write the same records. Returns FA_OK,
 * FA_ERR_NULL (NULL with n > 0), FA_ERR_SHAPE (a buffer with n <= 0) or
 * FA_ERR_ALIGN. The buffer must stay valid until the launches that use it end.
 */
int fa_set_clock_telemetry(unsigned long long* buf, int n);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
