/*
 * libkvarn -- KVarN 2-bit KV-cache quantizer for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes only. Device pointers are HIP device memory
 * owned by the caller; `stream` is a hipStream_t passed as void*. The library
 * never allocates or frees, enqueues all work on the caller's stream, and synchronizes
 * that stream only in kvarn_cache_init and kvarn_cache_flags. Its only global mutable
 * state is the device array behind kvarn_attn_decode_noalloc (below).
 *
 * Method (KVarN pages): each K/V token is rotated along head_dim by a randomized
 * Hadamard matrix H with H H^T = I (ai-paper-analysis page, section 3.1); VarN then
 * alternates a token-axis and a channel-axis variance normalization 2-3 times,
 * Sinkhorn-Knopp style, with grouped scales that dequantization undoes (section
 * 3.2); the result is quantized uniformly to 2 bits (4 levels). Decode attention
 * reads the cache with Q rotated by the same H so that Q K^T is unchanged
 * (section 3.1).
 *
 * Conventions fixed by this library where the pages are silent:
 *   H_D = diag(sigma) H_syl / sqrt(D), H_syl[i][j] = (-1)^popcount(i & j), sigma in {+1,-1}^D;
 *   inputs are taken as given (bf16) and kept so in the tail; a value beyond +-2^16
 *   saturates at +-2^16 (KVARN_FLAG_SATURATED), a NaN becomes +0 (KVARN_FLAG_NAN);
 *   "variance" is the mean square; a tile is G consecutive tokens x D channels of
 *   one (batch, kv head, stream); r (per token) and c (per channel) are stored as
 *   fp16 clamped to [2^-14, 65504]; the 2-bit grid is per channel over the tile's
 *   G tokens, asymmetric min/max, levels z + s*{0,1,2,3}, s and z fp16;
 *   codes round half to even and clamp to [0, 3] (3- and 4-bit codes: 2^bits levels,
 *   s = (max - min)/(2^bits - 1), clamp to [0, 2^bits - 1]).
 *
 * Cache buffer, format v3 (one caller-owned buffer per layer, 256-B aligned regions):
 *   header  align256(512 + 8*B*Hkv) bytes:
 *           u32 magic 0x4E52564B, u32 version 3, i32 geom[7] (batch, num_kv_heads,
 *           head_dim, capacity, group, varn_iters, bits), u32 flags (sticky) at byte 36,
 *           u32 variant at byte 40, i32 num_pages at byte 44, i8 sigma[D] at byte 64,
 *           u32 sign words[D/2] at byte 192 (word d: bit 15 set iff sigma[2d] = -1,
 *           bit 31 set iff sigma[2d+1] = -1, the sign bits of a packed pair of 16-bit
 *           floats), i32 len[B][Hkv][2] at byte 512;
 *   tiles   [B][Hkv][capacity/G][2 (K,V)][TR] tile records, region padded to 256 B;
 *           paged caches (num_pages > 0) instead hold a pool of num_pages pages,
 *           [num_pages][Hkv][2][TR] (one page = one group of G tokens of one sequence,
 *           every kv head, K and V), and the header grows by a page map int32
 *           [B][capacity/G] at byte 512 + 8*B*Hkv naming each tile's page (-1 = none,
 *           the state after kvarn_cache_init): header = align256(512 + 8*B*Hkv +
 *           4*B*capacity/G). A tile whose map entry is not a valid page is dropped by
 *           writers (KVARN_FLAG_UNMAPPED) and skipped by readers (attention leaves its
 *           tokens out, dequantization writes zeros).
 *   tail    [B][Hkv][2][G][D] bf16, unrotated tokens of the group being filled,
 *           slot = token index mod G.
 *   Tile record TR = G*D*bits/8 + 2G + 6D bytes (2 bits: 1856 at G=32, 2944 at G=64):
 *     codes  G*D*bits/8 B. 2-bit codes: four per byte, slot k of a byte at bits 2k..2k+1:
 *            K: token t owns the D/4 bytes from t*D/4 on, read as D/16 little-endian
 *               32-bit words; channel j = 16m + 2w + d (m < 8, d < 2) sits in word w
 *               at slot 4(m/2) + m%2 + 2d, i.e. byte t*D/4 + 4w + m/2, bits
 *               2(m%2 + 2d): each byte holds the channel pairs (2i, 2i+1) of two
 *               channel blocks of 16;
 *            V: code(t,j) in byte j*G/4 + t/4, bits 2*(t%4) (tokens fastest);
 *            3- and 4-bit codes q = qA + 4 qB: plane A (qA = bits 0..1) in the 2-bit
 *            layout above, then plane B. 4-bit: qB (bits 2..3) in the 2-bit layout.
 *            3-bit: qB (bit 2) one bit per code, 32-bit words: K: channel j of token
 *            t, in word w slot k of the 2-bit layout, at word 4t + w/2, bit
 *            4(k/2) + k%2 + 2(w%2); V: code (t = 8o + 2n + par, j = 16 blk + c with
 *            blk = i + 4hh, i = 2ip + ii) at word (16 ip + c) G/8 + o, bit
 *            4(n + 4hh) + par + 2ii. The grid has 2^bits levels.
 *     r fp16[G], c fp16[D], s fp16[D], z fp16[D].
 *   A tile token dequantizes as x_hat = (r_t c_j (z_j + s_j q_tj))_j H_D^T.
 *   Format history: v1 stored K and V codes alike (channel order, four per byte) and had
 *   no sign words, variant, num_pages or page map; v2 is the layout above (K channel-pair
 *   slots, V tokens fastest, sign words at 192, variant at 40, num_pages at 44, page map)
 *   with the tail in fp16 (inputs rounded to fp16); v3 keeps the tail in bf16.
 *
 * Errors: every argument check runs on the host before any HIP call; on error
 * nothing is enqueued and the cache is untouched. A failed launch returns
 * KVARN_ERR_DEVICE. Device-side conditions set sticky header flags.
 * One cache must not be written from two streams at once; reads may overlap.
 */
#ifndef KVARN_H
#define KVARN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define KVARN_API __attribute__((visibility("default")))
#else
#define KVARN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVARN_OK = 0,
    KVARN_ERR_NULL = 1,         /* a required pointer is NULL                              */
    KVARN_ERR_ALIGN = 2,        /* a device pointer is not 16-byte aligned                 */
    KVARN_ERR_GEOM = 3,         /* inconsistent geometry or sizes                          */
    KVARN_ERR_UNSUPPORTED = 4,  /* valid request outside what the library implements       */
    KVARN_ERR_RANGE = 5,        /* token count, head count or buffer size out of range     */
    KVARN_ERR_DEVICE = 6        /* the HIP runtime reported an error                       */
} kvarn_status;

/* Geometry of one layer cache: the pages' statement of the problem (K/V as [tokens,
 * kv_heads, head_dim] with a leading batch, the group of 32 or 64 sharing a scale and
 * the VarN iterations: ai-paper-analysis page, section 3.2; the 2-bit width:
 * researchpapers page). This library supports head_dim = 128, group in {32, 64},
 * bits in {2, 3, 4}, 0 <= varn_iters <= 8, capacity a positive multiple of group.
 * A caller that fills these seven fields gets the method as defined, with each
 * sequence's records stored contiguously. */
typedef struct {
    int32_t batch;          /* B   sequences                                   */
    int32_t num_kv_heads;   /* Hkv                                             */
    int32_t head_dim;       /* D                                               */
    int32_t capacity;       /* max tokens per sequence                         */
    int32_t group;          /* G   tokens per tile (the pages' 32 or 64)       */
    int32_t varn_iters;     /* VarN iterations (token pass + channel pass)     */
    int32_t bits;           /* code width: 2 (the pages'), 3 or 4; may carry KVARN_GEOM_EXT */
} kvarn_geom;

/* Extended geometry, for the ablation variants and paged caches. Every entry point
 * takes const kvarn_geom*; a caller that needs these fields passes the address of a
 * kvarn_geom_ext, whose first member is the kvarn_geom, with KVARN_GEOM_EXT ORed into
 * base.bits and size = sizeof(kvarn_geom_ext). Without the bit the library reads only
 * the seven fields above and takes variant = 0, num_pages = 0. A size other than
 * sizeof(kvarn_geom_ext) is refused with KVARN_ERR_GEOM. */
#define KVARN_GEOM_EXT 0x10000
typedef struct {
    kvarn_geom base;        /* base.bits = code width | KVARN_GEOM_EXT         */
    uint32_t size;          /* sizeof(kvarn_geom_ext)                          */
    int32_t variant;        /* ablation bits (KVARN_VARIANT_*), 0 for KVarN    */
    int32_t num_pages;      /* 0: records stored per sequence; > 0: paged      */
} kvarn_geom_ext;

/* Ablation variants (ai-paper-analysis page, section 5: Hadamard only = varn_iters 0,
 * VarN only, VarN along one axis only). The variant is written into the header at
 * byte 40 by kvarn_cache_init; every call on a cache must pass the geometry it was
 * initialized with. A cache with KVARN_VARIANT_NO_ROTATION uses the identity in
 * place of H_D everywhere (quantization, dequantization and attention; sigma is
 * stored but unused, and KVARN_Q_PREROTATED changes nothing). */
enum { KVARN_VARIANT_NO_ROTATION = 1u,      /* H_D = I: "VarN only"                            */
       KVARN_VARIANT_NO_CHANNEL_PASS = 2u,  /* VarN keeps the token-axis passes only: c = 1     */
       KVARN_VARIANT_NO_TOKEN_PASS = 4u,    /* VarN keeps the channel-axis passes only: r = 1   */
       KVARN_VARIANT_CENTERED = 8u          /* "variance" about the mean, not the mean square   */ };

enum { KVARN_OUT_F32 = 0, KVARN_OUT_BF16 = 1 };            /* dequantize output dtype     */
enum { KVARN_Q_PREROTATED = 1u };                          /* attention: q is already q H_D */
enum { KVARN_FLAG_CAPACITY = 1u,      /* an append found a full sequence; token dropped      */
       KVARN_FLAG_SATURATED = 2u,     /* an input had |x| > 2^16 and was saturated           */
       KVARN_FLAG_SCALE_CLAMPED = 4u, /* r or c hit [2^-14, 65504], or s/z saturated        */
       KVARN_FLAG_UNMAPPED = 8u,      /* a paged cache had no page for a tile being written  */
       KVARN_FLAG_NAN = 16u           /* an input was NaN; it was stored as 0                */ };

/* Format version of the cache buffer (3). */
KVARN_API int kvarn_format_version(void);

/* Size in bytes of a cache buffer for geometry *g. Host only. */
KVARN_API kvarn_status kvarn_cache_bytes(const kvarn_geom* g, size_t* bytes);

/* Write the header (magic, version, geometry, variant, num_pages, sigma and its sign words),
 * zero len[] and flags, and clear the page map of a paged cache to -1.
 * signs_host: host int8[head_dim], each +1 or -1: the random signs of H_D
 * (ai-paper-analysis page, section 3.1: randomized Hadamard matrix).
 * Synchronizes `stream`: the cache is ready when the call returns. */
KVARN_API kvarn_status kvarn_cache_init(const kvarn_geom* g, void* cache, const int8_t* signs_host, void* stream);

/* Reset the cache to hold tokens [0, num_tokens) of k and v.
 * k_bf16, v_bf16: device bf16 [B][num_tokens][Hkv][D], contiguous.
 * Full groups of G tokens are rotated, VarN-normalized and quantized into tile
 * records (ai-paper-analysis page, sections 3.1-3.2); the last num_tokens mod G
 * tokens go to the bf16 tail. Sets len = num_tokens. 0 <= num_tokens <= capacity. */
KVARN_API kvarn_status kvarn_quantize_prefill(const kvarn_geom* g, void* cache, const void* k_bf16,
                                    const void* v_bf16, int32_t num_tokens, void* stream);

/* kvarn_quantize_prefill for n_layers caches of one geometry and token count at once,
 * e.g. every layer of a model after its prefill forward pass: caches[i], k_bf16[i] and
 * v_bf16[i] are layer i's cache and inputs, with the layouts and the result of
 * kvarn_quantize_prefill(g, caches[i], k_bf16[i], v_bf16[i], num_tokens, stream) for each
 * i (bit-identical, flags included); each cache keeps its own sigma. The three pointer
 * arrays are host memory, read during the call; the caches must be distinct (two entries
 * naming one cache: KVARN_ERR_GEOM). 1 <= n_layers <= KVARN_MAX_PREFILL_LAYERS. The layers
 * run in one launch per 64, so the launch's ramp and tail are paid once for all of them.
 * (ai-paper-analysis page, sections 3.1-3.2.) */
#define KVARN_MAX_PREFILL_LAYERS 1024
KVARN_API kvarn_status kvarn_quantize_prefill_layers(const kvarn_geom* g, int32_t n_layers, void* const* caches,
                                           const void* const* k_bf16, const void* const* v_bf16,
                                           int32_t num_tokens, void* stream);

/* Append one token to every (batch, kv head): k_bf16, v_bf16 device bf16 [B][Hkv][D].
 * The token enters the bf16 tail; when the group of G fills it is quantized into
 * the next tile record (ai-paper-analysis page, section 3.2: the current group's
 * statistics are computed as tokens are written). A full sequence drops the token
 * and sets KVARN_FLAG_CAPACITY. */
KVARN_API kvarn_status kvarn_append_decode(const kvarn_geom* g, void* cache, const void* k_bf16,
                                 const void* v_bf16, void* stream);

/* Append counts[b] tokens to sequence b after its stored ones: k_bf16, v_bf16 device
 * bf16 [B][num_tokens][Hkv][D] (sequence b's tokens are its first counts[b] rows);
 * counts: device int32[B], each clamped to [0, num_tokens], or NULL for num_tokens
 * everywhere. The result is that of counts[b] single-token appends in order (and so,
 * from an empty sequence, of a prefill): a chunk of a prefill into a non-empty cache,
 * a ragged batch, or a per-sequence append mask (counts 0 or 1). Tokens past the
 * capacity are dropped (KVARN_FLAG_CAPACITY). 0 <= num_tokens <= capacity. Two launches.
 * (ai-paper-analysis page, section 3.2: a group is quantized once it is complete.) */
KVARN_API kvarn_status kvarn_append_tokens(const kvarn_geom* g, void* cache, const void* k_bf16,
                                 const void* v_bf16, int32_t num_tokens, const int32_t* counts,
                                 void* stream);

/* Paged caches only (num_pages > 0): tiles [tile_first, tile_first + num_tiles) of every
 * sequence take the pages in pages (device int32 [B][num_tiles]); an entry outside
 * [0, num_pages) unmaps the tile. The caller owns the pool: two tiles written into one
 * page overwrite each other. Layout of the map: see the cache format above. */
KVARN_API kvarn_status kvarn_cache_set_pages(const kvarn_geom* g, void* cache, const int32_t* pages,
                                   int32_t tile_first, int32_t num_tiles, void* stream);

/* Dequantize into k_out, v_out: device [B][max_tokens][Hkv][D], f32 or bf16 per
 * out_dtype. Tile tokens undo grid and scales and rotate back by H_D^T
 * (ai-paper-analysis page, section 3.2: the scaling is restored at
 * dequantization); tail tokens are copied; rows at or past len are zero.
 * 0 <= max_tokens <= capacity, else KVARN_ERR_RANGE; 0 is a no-op. */
KVARN_API kvarn_status kvarn_dequantize(const kvarn_geom* g, const void* cache, void* k_out, void* v_out,
                              int32_t max_tokens, int32_t out_dtype, void* stream);

/* Workspace bytes kvarn_attn_decode and kvarn_append_attn_decode need for num_q_heads
 * query heads. Host only. The workspace holds one f32 partial (m, l, 2 pad, o[D]) per
 * (batch, query head, span), followed by one i32 per (batch, kv head) (padded to 16
 * bytes). The span count depends on the geometry alone (about 2048 work-groups of 4
 * waves, each wave taking 2 to 16 tiles of a full sequence); a call cuts each
 * sequence's full tiles into that many spans of equal size, or fewer for a short one. */
KVARN_API kvarn_status kvarn_attn_workspace_bytes(const kvarn_geom* g, int32_t num_q_heads, size_t* bytes);

/* Single-query decode attention over every cached token:
 *   out[b][g] = sum_t softmax_t(scale * q[b][g] . k_hat_t) v_hat_t,
 * KV head of query head g = g / (num_q_heads / num_kv_heads).
 * q_bf16: device bf16 [B][Hq][D] in original space, rotated in-kernel by H_D
 * (ai-paper-analysis page, section 3.1: Q takes the same rotation so Q K^T is
 * unchanged), or already rotated when flags has KVARN_Q_PREROTATED.
 * softmax_scale <= 0 selects 1/sqrt(D). Tiles are read in rotated space with the
 * dequantization folded into the dot products (on the f16 MFMA, codes exact, the
 * per-tile factors split into f16 hi + lo parts); tail tokens in original space.
 * Two launches on `stream`: the tile pass, then the merge over spans and the tail.
 * workspace: device, >= kvarn_attn_workspace_bytes; out: device f32 [B][Hq][D],
 * original space. An empty sequence gives 0. num_q_heads must be a multiple of
 * num_kv_heads. */
KVARN_API kvarn_status kvarn_attn_decode(const kvarn_geom* g, const void* cache, const void* q_bf16,
                               int32_t num_q_heads, float softmax_scale, uint32_t flags,
                               void* workspace, size_t workspace_bytes, float* out, void* stream);

/* kvarn_attn_decode without a caller-supplied workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The span partials go to a workspace the library keeps as a file-scope device
 * array of 32 MiB on every GPU it runs on, held until the process ends; a geometry whose
 * kvarn_attn_workspace_bytes exceeds 32 MiB is refused with KVARN_ERR_RANGE before any HIP
 * call. The call allocates and frees nothing; its first call on a device looks up that
 * device's array address (the current device must be the stream's). Every call on one GPU
 * shares the array: two calls that overlap in time on one GPU (other streams, other host
 * threads) race on it, so the caller must order them. Results equal kvarn_attn_decode's. */
KVARN_API kvarn_status kvarn_attn_decode_noalloc(const kvarn_geom* g, const void* cache, const void* q_bf16,
                                       int32_t num_q_heads, float softmax_scale, uint32_t flags, float* out,
                                       void* stream);

/* One decode step of a layer: append k, v (as kvarn_append_decode) and attend with q
 * over the cache including the new token (as kvarn_attn_decode), in the two launches of
 * the attention: the append runs inside the merge launch. Same arguments and layouts as
 * those two calls. The result equals kvarn_append_decode followed by kvarn_attn_decode,
 * except on a step whose token completes a group of G: the attention then reads that
 * group as the bf16 values it is quantized from (the tile is written for later steps).
 * A full sequence drops the token (KVARN_FLAG_CAPACITY) and attends without it.
 * (ai-paper-analysis page, section 3.2: the group being filled is kept until complete;
 * section 3.1: the query is rotated like the keys.) */
KVARN_API kvarn_status kvarn_append_attn_decode(const kvarn_geom* g, void* cache, const void* k_bf16,
                                      const void* v_bf16, const void* q_bf16, int32_t num_q_heads,
                                      float softmax_scale, uint32_t flags, void* workspace,
                                      size_t workspace_bytes, float* out, void* stream);

/* Read the sticky flags into *flags_host. Synchronizes `stream`. */
KVARN_API kvarn_status kvarn_cache_flags(const void* cache, void* stream, uint32_t* flags_host);

/* Static string for a status code. */
KVARN_API const char* kvarn_status_str(kvarn_status s);

/* Test hook: kvarn_quantize_prefill plus the fp32 intermediates of the full tiles:
 * w = rotated tokens, y = normalized tokens W / (r16 c16), each device f32
 * [B][T_full][Hkv][D], T_full = G * floor(num_tokens / G). Any of w_*, y_* may be NULL. */
KVARN_API kvarn_status kvarn_debug_prefill(const kvarn_geom* g, void* cache, const void* k_bf16,
                                 const void* v_bf16, int32_t num_tokens, float* w_k, float* w_v,
                                 float* y_k, float* y_v, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_H */
