/* A plain C99 caller of libkvarn: compiles against include/kvarn.h alone and exercises
 * the calls that need no device (sizes, status strings, argument checks). Every entry
 * point is referenced through a function-pointer table, so linking fails if the library
 * does not export one of them. Prints one "name value" line per result. */
#include <stdio.h>
#include <string.h>

#include "kvarn.h"

typedef void (*entry_fn)(void);
static const entry_fn every_entry_point[] = {
    (entry_fn)kvarn_format_version,   (entry_fn)kvarn_cache_bytes,        (entry_fn)kvarn_cache_init,
    (entry_fn)kvarn_quantize_prefill, (entry_fn)kvarn_append_decode,      (entry_fn)kvarn_append_tokens,
    (entry_fn)kvarn_cache_set_pages,  (entry_fn)kvarn_dequantize,         (entry_fn)kvarn_attn_workspace_bytes,
    (entry_fn)kvarn_attn_decode,      (entry_fn)kvarn_append_attn_decode, (entry_fn)kvarn_cache_flags,
    (entry_fn)kvarn_status_str,       (entry_fn)kvarn_debug_prefill,      (entry_fn)kvarn_attn_decode_noalloc,
    (entry_fn)kvarn_quantize_prefill_layers,
};

/* A seven-field geometry followed in memory by values that would select an ablation
 * variant and a paged layout if the library read past the struct. */
struct boxed {
    kvarn_geom g;
    int32_t after[4];
};

int main(void) {
    kvarn_geom g;
    struct boxed bx;
    kvarn_geom_ext ext;
    size_t bytes = 0, ws = 0;
    kvarn_status st;
    int i;
    for (i = 0; i < (int)(sizeof every_entry_point / sizeof every_entry_point[0]); ++i)
        if (!every_entry_point[i]) return 2;
    printf("entry_points %d\n", i);
    printf("format_version %d\n", kvarn_format_version());

    memset(&g, 0, sizeof g);  /* the Phi-4-14B-shaped decode layer */
    g.batch = 32; g.num_kv_heads = 10; g.head_dim = 128; g.capacity = 17408;
    g.group = 32; g.varn_iters = 3; g.bits = 2;
    st = kvarn_cache_bytes(&g, &bytes);
    printf("cache_bytes_status %d\ncache_bytes %zu\n", (int)st, bytes);
    st = kvarn_attn_workspace_bytes(&g, 40, &ws);
    printf("workspace_status %d\nworkspace_bytes %zu\n", (int)st, ws);

    g.bits = 5;  /* outside 2..4 */
    printf("bits5_status %d\n", (int)kvarn_cache_bytes(&g, &bytes));
    g.bits = 2; g.group = 48;
    printf("group48_status %d\n", (int)kvarn_cache_bytes(&g, &bytes));
    g.group = 32;
    printf("null_geom_status %d\n", (int)kvarn_cache_bytes(NULL, &bytes));
    printf("null_out_status %d\n", (int)kvarn_cache_bytes(&g, NULL));
    printf("gqa_not_multiple_status %d\n", (int)kvarn_attn_workspace_bytes(&g, 15, &ws));
    /* a device call with a NULL cache is refused on the host, before any HIP call */
    printf("prefill_null_cache_status %d\n", (int)kvarn_quantize_prefill(&g, NULL, NULL, NULL, 0, NULL));
    {
        /* the multi-layer entry: host arrays of device pointers; two entries naming one cache */
        void* caches[2];
        const void* ins[2];
        caches[0] = (void*)(size_t)0x10000;
        caches[1] = (void*)(size_t)0x10000;
        ins[0] = (const void*)(size_t)0x20000;
        ins[1] = (const void*)(size_t)0x20000;
        printf("layers_null_status %d\n", (int)kvarn_quantize_prefill_layers(&g, 2, NULL, ins, ins, 0, NULL));
        printf("layers_duplicate_status %d\n", (int)kvarn_quantize_prefill_layers(&g, 2, caches, ins, ins, 0, NULL));
        printf("layers_count_status %d\n", (int)kvarn_quantize_prefill_layers(&g, 0, caches, ins, ins, 0, NULL));
    }
    printf("sizeof_geom %d\nsizeof_geom_ext %d\n", (int)sizeof(kvarn_geom), (int)sizeof(kvarn_geom_ext));
    bx.g = g;
    bx.after[0] = 40; bx.after[1] = 8; bx.after[2] = 100; bx.after[3] = -1;
    bytes = 0;
    st = kvarn_cache_bytes(&bx.g, &bytes);
    printf("boxed_status %d\nboxed_bytes %zu\n", (int)st, bytes);
    memset(&ext, 0, sizeof ext);
    ext.base = g;
    ext.base.bits = 2 | KVARN_GEOM_EXT;
    ext.size = (uint32_t)sizeof ext;
    ext.num_pages = 100;
    bytes = 0;
    st = kvarn_cache_bytes(&ext.base, &bytes);
    printf("ext_status %d\next_bytes %zu\n", (int)st, bytes);
    ext.size = 36;
    printf("ext_badsize_status %d\n", (int)kvarn_cache_bytes(&ext.base, &bytes));
    printf("status_str_ok %s\n", kvarn_status_str(KVARN_OK));
    printf("status_str_geom %s\n", kvarn_status_str(KVARN_ERR_GEOM));
    return 0;
}
