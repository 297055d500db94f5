/*
 * kivi_cache.h -- a KIVI KV cache for a decode loop, on top of the calls in
 * kivi.h: every layer's packed key/value stores and fp16 residual windows in
 * one caller-allocated device buffer, the flush rule, per-step append and
 * attend, and one deferred flush launch per tensor for all layers.
 *
 * Sources, cited by page title and section:
 *   [Metal post]  blog post "A 5.65x Metal Kernel That Made My LLM Exactly
 *                 0% Faster", "What we're actually optimizing": the newest
 *                 residual_length tokens stay fp16, older tokens are
 *                 quantized (keys per channel in groups of tokens, values per
 *                 token); "The full end-to-end record": the tokens flushed
 *                 per layer are whole groups older than the residual window.
 *   [Qwen3 post]  blog post "A Kernel That Wasn't There": decode flushes are
 *                 small and a prefill flush must be large to amortize
 *                 dispatch.
 *   [Benchmarks]  VeloxQuant-MLX "Benchmarks" page, "KV-Cache Kernel
 *                 Roofline": cross-layer batched dispatch of the kernels.
 *
 * Token accounting (R = residual_length, F = flush_tokens, G = group_size):
 * a sequence of S tokens holds its oldest Q(S) = max(0, floor((S - R) / F) * F)
 * tokens quantized and the other S - Q(S) (between R and R + F - 1 once
 * S >= R) in fp16.  With F = G this is "every whole group older than the
 * newest R tokens".  A decode step appends one token per sequence to every
 * layer; the step's attention sees it in fp16, and the flush that the new
 * length calls for runs after the step's last layer (kivi_cache_end_step),
 * as one launch per tensor over all layers.  All sequences of the batch have
 * the same length.
 *
 * The residual window of a slab is a ring of R + F token rows: flushes take
 * the oldest F rows and advance the ring's head by F, so no row is ever
 * moved.  Attention is a sum over tokens, so it reads the ring in ring order.
 *
 * Device layout (kivi_cache_device_bytes bytes at `device`, 256-byte aligned
 * sections, slab s = (layer * batch + b) * kv_heads + h):
 *   key store, value store   as in kivi.h with cap = store_capacity tokens
 *                            and the configuration's scale/zero format
 *   key ring, value ring     16-bit [slabs][R + F][head_dim] (fp16, or
 *                            bfloat16 for a bfloat16 cache)
 *   key, value staging       the same shape as the rings
 *
 * The library never allocates: the caller allocates the device buffer and
 * the kivi_cache struct.  Every call validates on the host before it enqueues
 * anything (negative return = nothing launched, cache state unchanged) and
 * enqueues on `stream`.  A cache must be used from one stream at a time.
 */
#ifndef KIVI_CACHE_H
#define KIVI_CACHE_H

#include <stddef.h>
#include <stdint.h>

#include "kivi.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { KIVI_CACHE_MAX_LAYERS = 256 };

typedef struct kivi_cache_config {
    int32_t layers;           /* 1 .. KIVI_CACHE_MAX_LAYERS                    */
    int32_t batch;            /* sequences B >= 1                              */
    int32_t kv_heads;         /* Hkv >= 1                                      */
    int32_t bits;             /* 2 or 4                                        */
    int32_t head_dim;         /* 128, or a multiple of 16 from 16 to 256       */
    int32_t group_size;       /* 32, 64 or 128 at head_dim 128; else 32        */
    int32_t residual_length;  /* R >= 0, a multiple of flush_tokens            */
    int32_t flush_tokens;     /* F > 0, a multiple of group_size               */
    int64_t store_capacity;   /* quantized tokens per sequence, a multiple of F */
    int32_t meta_format;      /* scale/zero of the stores: KIVI_META_F32 (0) or
                                 KIVI_META_F16 (1), as in kivi.h                */
    int32_t bf16;             /* 0: fp16 cache; 1: bfloat16 cache (prompt, new
                                 rows, rings and queries in bfloat16, the _bf16
                                 flushes and attend; binary32 scale/zero)     */
} kivi_cache_config;

/* Host-side state of a cache.  Filled by kivi_cache_init; the fields are
 * readable (the stores and rings can be inspected or handed to kivi.h calls)
 * but only the kivi_cache_* calls may change them. */
typedef struct kivi_cache {
    kivi_cache_config cfg;
    kivi_store k_store;       /* all layers' slabs (BH = layers*batch*kv_heads) */
    kivi_store v_store;
    uint16_t* k_ring;         /* 16-bit [slabs][ring][head_dim]                */
    uint16_t* v_ring;
    uint16_t* k_stage;        /* 16-bit [slabs][ring][head_dim]: a prompt      */
    uint16_t* v_stage;        /* chunk's first flush groups are assembled here */
    int64_t ring;             /* R + F rows per slab                           */
    int64_t length;           /* tokens per sequence so far                    */
    int64_t n_quant;          /* of which quantized (in the stores)            */
    int64_t n_res;            /* of which fp16, rows head .. head+n_res-1 (mod ring) */
    int64_t head;             /* ring row of the oldest fp16 token             */
    uint64_t appended[KIVI_CACHE_MAX_LAYERS / 64]; /* layers appended this step */
} kivi_cache;

/* Device bytes a cache of this configuration needs; 0 if the configuration
 * is invalid. */
size_t kivi_cache_device_bytes(const kivi_cache_config* cfg);

/* Lays the cache out in `device` (device memory, 256-byte aligned, at least
 * kivi_cache_device_bytes bytes) and sets it empty.  Host-only: launches
 * nothing and does not touch the device memory. */
int kivi_cache_init(kivi_cache* cache, const kivi_cache_config* cfg, void* device, size_t bytes);

/* A chunk of S prompt tokens for every layer and sequence at once, appended
 * to the cache (empty, or holding earlier chunks and decode steps; not in
 * the middle of a step).  k, v: 16-bit (the cache's format)
 * [layers*batch*kv_heads][S][head_dim] with slab stride x_bh_stride (slab
 * order as in the device layout).  After the call the cache holds L + S
 * tokens of which Q(L + S) are quantized, exactly as if the whole prompt had
 * arrived at once: the newly flushed tokens [Q(L), Q(L + S)) go into the
 * stores, the ones whose key groups begin among the fp16 tokens already in
 * the rings through the staging rows (one gather launch, then one flush
 * launch per tensor over all layers), the rest straight from k and v (one
 * flush launch per tensor); the chunk's tokens that stay fp16 are copied
 * into the rings (one launch).  Long prompts can so be fed in pieces (the
 * pages' runtime prefills 2048-token chunks: [Metal post] "Four benchmarks
 * that lied", Lie #1).  Q(L + S) must fit the store capacity. */
int kivi_cache_prefill(kivi_cache* cache, const uint16_t* k, const uint16_t* v,
                       int64_t x_bh_stride, int64_t S, hipStream_t stream);

/* Step: append this step's token of every sequence to layer `layer`.
 * k_new, v_new: 16-bit [batch*kv_heads][head_dim], contiguous.  Once per layer
 * per step, before that layer's kivi_cache_attend. */
int kivi_cache_append(kivi_cache* cache, int32_t layer, const uint16_t* k_new,
                      const uint16_t* v_new, hipStream_t stream);

/* Step: decode attention of layer `layer` after its append: one query token
 * per sequence (q 16-bit [batch][Hq][head_dim]) over the layer's quantized
 * tokens and its fp16 tokens including this step's, as kivi_decode_attend
 * (out fp32 [batch][Hq][head_dim]; workspace of at least
 * kivi_cache_attend_workspace_bytes(cache, Hq) bytes). */
int kivi_cache_attend(const kivi_cache* cache, int32_t layer, const uint16_t* q, int32_t Hq,
                      float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Step, fused: kivi_cache_append then kivi_cache_attend of layer `layer` in
 * one kernel launch pair instead of three launches.  The attend reads this
 * step's token from k_new / v_new directly, and the wave that holds it also
 * writes it into the layer's rings, so the cache afterwards is as if both
 * calls had run; out is bit-identical to theirs.  Arguments, workspace and
 * errors as the two calls (the layer must not have appended this step;
 * nothing is launched and the layer stays un-appended on error).  k_new and
 * v_new are read during the launch only. */
int kivi_cache_append_attend(kivi_cache* cache, int32_t layer, const uint16_t* k_new,
                             const uint16_t* v_new, const uint16_t* q, int32_t Hq,
                             float softmax_scale, float* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes that serve kivi_cache_attend at every length the cache can
 * reach (so one allocation, or one captured graph, covers the whole loop). */
size_t kivi_cache_attend_workspace_bytes(const kivi_cache* cache, int32_t Hq);

/* Ends a step in which every layer appended once: the length grows by one
 * and, when the fp16 tokens reach R + F, the oldest F of every slab are
 * flushed into the stores in one launch per tensor over all layers.
 * Returns the number of kernel launches it made (0 or 2), or a negative
 * KIVI_ERR_* code (KIVI_ERR_SHAPE: a layer did not append, or the stores
 * are full). */
int kivi_cache_end_step(kivi_cache* cache, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_CACHE_H */
