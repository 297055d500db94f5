/*
 * kivi.h -- C ABI of libkivi, the MI355X (gfx950) KIVI KV-cache
 * quantization hot path.
 *
 * Sources, cited by page title and section:
 *   [Metal post]  blog post "A 5.65x Metal Kernel That Made My LLM Exactly
 *                 0% Faster" (VeloxQuant-MLX)
 *   [Benchmarks]  VeloxQuant-MLX "Benchmarks" page
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees, copies between host and device or
 *    synchronizes; each call validates its arguments on the host, enqueues
 *    its kernels on `stream` and returns.
 *  - Validation happens before anything is enqueued: a negative return
 *    means nothing was launched.  A zero-sized call (S == 0, n_tokens == 0,
 *    B == 0) succeeds without launching.
 *  - fp16 tensors are passed as `uint16_t*` holding IEEE binary16 bits (the
 *    _bf16 calls take bfloat16 bits instead).
 *  - Strides are in elements of the array they index.  Token rows inside a
 *    bh slab are contiguous (row stride = head_dim).
 *  - Inputs must not alias outputs.  Calls on different streams may run
 *    concurrently if their outputs do not overlap.
 *  - Faults inside a kernel surface at the caller's next synchronization.
 *  - Supported parameters: bits in {2, 4}; head_dim 128 with group_size
 *    32, 64 or 128, or any other multiple of 16 from 16 to 256 with
 *    group_size 32 (when 32 does not divide head_dim, a token's last value
 *    group holds the remaining 16 channels: [Metal post] "Kernel B" cuts a
 *    row's last group at the row's end).  The attend takes every store
 *    geometry with binary32 scale/zero (binary16 ones: head_dim 128); its
 *    key and value stores share head_dim and group size, and q, the
 *    residual and out have head_dim channels.  Every head_dim runs on the
 *    MFMA kernels: 64, 128 and 256 on their own channel geometry, the others
 *    on that of the next of them, with the extra channels computed as zeros
 *    and never stored.  Anything else returns KIVI_ERR_UNSUPPORTED.
 *
 * Packed store layout (the pages fix none; [Metal post] "So why does the
 * kernel ship?" asks for packed storage of the codes):
 *   codes  uint32 [BH][cap][head_dim*bits/32]  token-major; the code of
 *          channel d of token t sits in word (t, d / (32/bits)) at bit
 *          offset bits * (d % (32/bits)), least significant first.
 *   keys   scale, zero [BH][cap/G][head_dim]   one pair per
 *          (token group, channel): per-channel quantization.
 *   values scale, zero [BH][cap][ceil(head_dim/G)]   one pair per
 *          (token, channel group): per-token quantization.
 *   zero is the group minimum (a float offset, not an integer zero point).
 *   scale and zero are binary32 (meta_format KIVI_META_F32, the default)
 *   or binary16 (KIVI_META_F16).  The pages leave this precision open;
 *   [Benchmarks] "KV-Cache Kernel Roofline" reports KV-compression ratios,
 *   which depend on it.  A binary16 store holds the binary32 scale and zero
 *   rounded to nearest even, and its codes and reconstructions are taken
 *   with those stored values (so a reader of the store reproduces them
 *   exactly); a scale that rounds to 0 codes its group as constant, and a
 *   code past 2^bits - 1 is clipped.  It halves the metadata bytes (4-bit,
 *   groups of 32: 5 bits per element instead of 6) and is supported for
 *   fp16 caches at head_dim 128, by the flush, dequantize and attend calls.
 */
#ifndef KIVI_H
#define KIVI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's own stream handle type (identical typedef to hip_runtime_api.h). */
typedef struct ihipStream_t* hipStream_t;

enum {
    KIVI_OK = 0,
    KIVI_ERR_NULL = -1,        /* a required pointer is NULL                  */
    KIVI_ERR_SHAPE = -2,       /* negative size, window outside the store,
                                  misaligned key offset, Hq % Hkv != 0, ...   */
    KIVI_ERR_UNSUPPORTED = -3, /* bits, group_size, head_dim or kind unsupported */
    KIVI_ERR_ALIGN = -4,       /* pointer not 16-byte aligned or stride not a
                                  multiple of 16 bytes                         */
    KIVI_ERR_WORKSPACE = -5,   /* attend workspace NULL or too small          */
    KIVI_ERR_HIP = -6          /* a HIP launch failed; see kivi_last_hip_error */
};

enum { KIVI_KEYS = 0, KIVI_VALUES = 1 };
enum { KIVI_META_F32 = 0, KIVI_META_F16 = 1 };
/* flags of kivi_decode_attend_workspace_bytes: which attend call it sizes */
enum { KIVI_ATTEND_BF16 = 1, KIVI_ATTEND_VARLEN = 2 };

/* A packed store (see the layout above).  The struct itself lives in host
 * memory and is only read during the call; the arrays are device memory. */
typedef struct kivi_store {
    uint32_t* codes;           /* [BH][cap][head_dim*bits/32]                 */
    void*     scale;           /* keys [BH][cap/G][D]; values [BH][cap][ceil(D/G)];
                                  float, or binary16 bits (meta_format)       */
    void*     zero;            /* same shape and format as scale              */
    int64_t   codes_bh_stride; /* uint32 words between bh slabs (>= cap*row) */
    int64_t   meta_bh_stride;  /* scale elements between bh slabs             */
    int64_t   cap;             /* token capacity of each slab                 */
    int32_t   bits;            /* 2 or 4                                      */
    int32_t   group_size;      /* 32, 64 or 128                               */
    int32_t   head_dim;        /* a multiple of 16 from 16 to 256             */
    int32_t   kind;            /* KIVI_KEYS or KIVI_VALUES                    */
    int32_t   meta_format;     /* KIVI_META_F32 or KIVI_META_F16              */
} kivi_store;

/*
 * Per-channel key flush.  [Metal post] "What we're actually optimizing":
 * keys get one scale per channel computed across a group of tokens, with
 * zero = min, scale = (max - min) / (2^bits - 1), q = round((x - zero) /
 * scale) clipped to [0, 2^bits - 1]; "Kernel A": the group of channel d is
 * tokens [g*G, min(g*G + G, S)) of that channel; "Three ways to be off by
 * one bit": ties round to even, q*scale and +zero are rounded separately,
 * a ragged last group behaves as if padded with its last real token.
 * Arithmetic is IEEE binary32 (IEEE division, no contraction), bit-exact
 * with the documented reading.  A group with max == min gets scale 0 and
 * code 0.
 *
 *   x              fp16 [BH][S][head_dim], slab bh at x + bh*x_bh_stride
 *   dst            key store (kind KIVI_KEYS); tokens [dst_token,
 *                  dst_token + S) of every slab are written, nothing else
 *   dst_token      multiple of group_size; dst_token + S <= dst->cap
 *   recon          optional (NULL for none): fp16 [BH][S][head_dim]
 *                  reconstruction q*scale + zero of every input element
 *   recon_bh_stride  elements between recon slabs
 * Returns KIVI_OK or a negative KIVI_ERR_* code.
 */
int kivi_quantize_keys(const uint16_t* x, int64_t BH, int64_t S, int64_t x_bh_stride,
                       const kivi_store* dst, int64_t dst_token,
                       uint16_t* recon, int64_t recon_bh_stride, hipStream_t stream);

/*
 * Per-token value flush.  [Metal post] "What we're actually optimizing":
 * values get one scale per token computed across a group of channels;
 * "Kernel B": the group of token s is channels [j*G, j*G + G) of that
 * token.  Same element rule, arguments and write window as
 * kivi_quantize_keys, except that dst_token may be any offset and dst has
 * kind KIVI_VALUES.
 */
int kivi_quantize_values(const uint16_t* x, int64_t BH, int64_t S, int64_t x_bh_stride,
                         const kivi_store* dst, int64_t dst_token,
                         uint16_t* recon, int64_t recon_bh_stride, hipStream_t stream);

/*
 * The same flushes for bfloat16 caches: x (and recon, if given) hold
 * bfloat16 bit patterns, widened exactly to fp32 (bfloat16 is binary32 with
 * the low 16 fraction bits dropped); every later step is the same fp32
 * arithmetic, and the reconstruction is rounded to bfloat16 (nearest even).
 * The packed store is identical to the one the fp16 calls write.  Inputs
 * must be finite with a finite max - min in every group.  A store with
 * binary16 scale/zero returns KIVI_ERR_UNSUPPORTED (a bfloat16 minimum need
 * not be a binary16 value).
 */
int kivi_quantize_keys_bf16(const uint16_t* x, int64_t BH, int64_t S, int64_t x_bh_stride,
                            const kivi_store* dst, int64_t dst_token,
                            uint16_t* recon, int64_t recon_bh_stride, hipStream_t stream);
int kivi_quantize_values_bf16(const uint16_t* x, int64_t BH, int64_t S, int64_t x_bh_stride,
                              const kivi_store* dst, int64_t dst_token,
                              uint16_t* recon, int64_t recon_bh_stride, hipStream_t stream);

/*
 * Dequantize tokens [token_begin, token_begin + n_tokens) of every slab of
 * a key or value store to fp16: out = fp16_rne(fl(fl(q*scale) + zero))
 * ([Metal post] "Three ways to be off by one bit", item 1: no fused
 * multiply-add; "So why does the kernel ship?": KIVI as shipped expands the
 * store back to fp16).  Bit-exact with the reconstruction the flush writes.
 *
 *   src        store; src->kind selects the key or value metadata layout
 *   BH         number of slabs to read (<= what the store holds)
 *   out        fp16 [BH][n_tokens][head_dim], slab bh at out + bh*out_bh_stride
 */
int kivi_dequantize(const kivi_store* src, int64_t BH, int64_t token_begin, int64_t n_tokens,
                    uint16_t* out, int64_t out_bh_stride, hipStream_t stream);

/* kivi_dequantize with a bfloat16 output: out = bf16_rne(fl(fl(q*scale) +
 * zero)), bit-exact with the reconstruction the bfloat16 flushes write.
 * Stores with binary32 scale/zero only (KIVI_ERR_UNSUPPORTED otherwise). */
int kivi_dequantize_bf16(const kivi_store* src, int64_t BH, int64_t token_begin, int64_t n_tokens,
                         uint16_t* out, int64_t out_bh_stride, hipStream_t stream);

/*
 * Fused dequantize + attend for one new query token per sequence
 * ([Benchmarks] "KV-Cache Kernel Roofline: What Actually Limits Decode":
 * a decode+attend kernel that reads the packed state directly, measured
 * against dequantize + SDPA on the same compressed state; [Metal post]
 * "What we're actually optimizing": the newest residual_length tokens stay
 * fp16).  For every sequence b and query head h (kv head h / (Hq/Hkv)):
 *   out[b][h] = softmax(q[b][h] . K^T * softmax_scale) V
 * over K, V = [store tokens 0..n_quant-1 dequantized ; residual tokens
 * 0..n_res-1], accumulated in fp32 (the result is within 2e-3 max-abs of
 * the float64 definition, not bit-exact).
 *
 *   q          fp16 [B][Hq][head_dim]
 *   k, v       key and value stores whose slab b*Hkv + kv holds sequence b,
 *              kv head kv (same bits, same cap >= n_quant)
 *   k_res, v_res  fp16 residual windows [B*Hkv][..][head_dim], slab stride
 *              res_bh_stride; may be NULL when n_res == 0
 *   out        fp32 [B][Hq][head_dim]
 *   workspace  device scratch of at least
 *              kivi_decode_attend_workspace_bytes(B, Hq, Hkv, n_quant, n_res,
 *              head_dim, 0) bytes, 256-byte aligned, owned by the caller; its
 *              contents on entry do not matter.  It holds the per-split
 *              partials between the call's two kernels, so calls that may
 *              overlap in time need separate workspaces.
 * n_quant + n_res must be > 0, n_quant and n_res below 2^24, Hq/Hkv one of
 * 1, 2, 4, 8, B * Hkv at most 65535, and softmax_scale finite and > 0
 * (KIVI_ERR_SHAPE otherwise).
 */
int kivi_decode_attend(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                       const kivi_store* k, const kivi_store* v, int64_t n_quant,
                       const uint16_t* k_res, const uint16_t* v_res, int64_t res_bh_stride,
                       int64_t n_res, float softmax_scale, float* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kivi_decode_attend without a workspace argument, for callers that cannot
 * allocate device memory: code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The split partials go to a 32 MiB device
 * array the library owns (part of its code object: each GPU the library runs
 * on holds one copy, from load until the process ends); the call allocates
 * nothing.  A shape whose partials exceed it
 * (kivi_decode_attend_workspace_bytes(B, Hq, Hkv, n_quant, n_res, head_dim,
 * 0) > 32 MiB) returns KIVI_ERR_WORKSPACE with nothing launched.  All calls
 * on one GPU share its array: calls that may overlap in time on one GPU
 * (several streams or host threads) race, and the caller must keep them
 * apart.  The first call on each device looks the array's address up
 * (hipGetSymbolAddress) and must not be made during stream capture.
 * Everything else (arguments, result, errors) is as for kivi_decode_attend.
 */
int kivi_decode_attend_noalloc(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                               const kivi_store* k, const kivi_store* v, int64_t n_quant,
                               const uint16_t* k_res, const uint16_t* v_res, int64_t res_bh_stride,
                               int64_t n_res, float softmax_scale, float* out, hipStream_t stream);

/*
 * kivi_decode_attend over a batch of sequences of different lengths, in one
 * launch ([Benchmarks] "KV-Cache Kernel Roofline: What Actually Limits
 * Decode": several concurrent requests routed through one fused decode
 * kernel, the way to fill the GPU at decode).  Sequence b attends over store
 * tokens [0, n_quant[b]) then residual tokens [0, n_res[b]) of its own slabs
 * b*Hkv + kv, exactly as kivi_decode_attend does for a batch of one.
 *
 *   n_quant, n_res  DEVICE int32 [B], 4-byte aligned, read by the kernel
 *              (so the lengths can change between replays of a captured
 *              graph).  A value is clamped to [0, max_n_quant] /
 *              [0, max_n_res]; the host cannot see them, so the clamp is what
 *              keeps every load inside the store and residual bounds below.
 *   max_n_quant, max_n_res  host bounds on the lengths: the grid, the
 *              workspace (kivi_decode_attend_workspace_bytes(B, Hq, Hkv,
 *              max_n_quant, max_n_res, head_dim, KIVI_ATTEND_VARLEN)) and the
 *              store/residual validation use them.  max_n_quant + max_n_res
 *              must be > 0.
 * A sequence whose clamped lengths are both 0 gets an all-zero output row.
 * Every other argument and every error is as for kivi_decode_attend.
 */
int kivi_decode_attend_varlen(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                              const kivi_store* k, const kivi_store* v,
                              const int32_t* n_quant, int64_t max_n_quant,
                              const uint16_t* k_res, const uint16_t* v_res, int64_t res_bh_stride,
                              const int32_t* n_res, int64_t max_n_res, float softmax_scale,
                              float* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * The same two attends for bfloat16 caches: q, k_res and v_res hold
 * bfloat16 bit patterns, and the stores (written by the _bf16 flushes, with
 * binary32 scale/zero) are reconstructed to bfloat16 in registers, as
 * kivi_dequantize_bf16 would.  QK^T and PV run on bfloat16 MFMA operands
 * with fp32 accumulation; the softmax probabilities enter PV as a bfloat16
 * pair (a truncated high part and the rounded remainder, 2^-16 relative),
 * so the result is within 2e-3 max-abs of the float64 definition over the
 * bfloat16 reconstruction for values of order 1.  A store with binary16
 * scale/zero returns KIVI_ERR_UNSUPPORTED; everything else is as for
 * kivi_decode_attend and kivi_decode_attend_varlen (workspace sized with
 * KIVI_ATTEND_BF16 in the flags).
 */
int kivi_decode_attend_bf16(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                            const kivi_store* k, const kivi_store* v, int64_t n_quant,
                            const uint16_t* k_res, const uint16_t* v_res, int64_t res_bh_stride,
                            int64_t n_res, float softmax_scale, float* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
int kivi_decode_attend_varlen_bf16(const uint16_t* q, int64_t B, int32_t Hq, int32_t Hkv,
                                   const kivi_store* k, const kivi_store* v,
                                   const int32_t* n_quant, int64_t max_n_quant,
                                   const uint16_t* k_res, const uint16_t* v_res,
                                   int64_t res_bh_stride, const int32_t* n_res, int64_t max_n_res,
                                   float softmax_scale, float* out, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of one attend call: B, Hq, Hkv, n_quant and n_res as the
 * call passes them (the _varlen calls: their max_n_quant and max_n_res),
 * head_dim of its stores, and flags KIVI_ATTEND_BF16 for the _bf16 calls
 * plus KIVI_ATTEND_VARLEN for the _varlen ones.  Exactly what that call
 * checks for; 0 for arguments no call accepts. */
size_t kivi_decode_attend_workspace_bytes(int64_t B, int32_t Hq, int32_t Hkv, int64_t n_quant,
                                          int64_t n_res, int32_t head_dim, int32_t flags);

/* Static description of a status code. */
const char* kivi_status_string(int status);

/* hipError_t of the last KIVI_ERR_HIP returned on this host thread. */
int kivi_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_H */
