/*
 * A plain C99 client of include/zs.h: builds one rank's layout from the
 * command line and prints its tables, one record per line.  It exists to
 * show that the boundary is a C interface usable without C++ or Python;
 * tests/test_abi_c_client.py compiles it with gcc and compares its output
 * with the oracle's layout.  Host calls only: it needs no GPU.
 *
 * usage: abi_client flat|tensors WORLD RANK CAP_BYTES ALIGN_BYTES N...
 *        (CAP_BYTES is ignored in the tensors mode)
 * output:
 *   info FLAT SHARD N_BUCKETS N_CHUNKS N_TILES WORLD RANK
 *   tensor T FLAT_OFF
 *   bucket FLAT_OFF NUMEL SLICE SHARD_OFF TILE_OFF
 *   chunk TENSOR BUCKET TENSOR_OFF NUMEL SHARD_OFF
 *   owner T RANK SHARD_OFF                     (tensors mode)
 * or, when the build fails:
 *   error CODE STRERROR | LAST_ERROR
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zs.h"

static int fail(int rc, const char* what)
{
    printf("error %d %s | %s: %s\n", rc, zs_strerror(rc), what,
           zs_last_error());
    return 0;
}

int main(int argc, char** argv)
{
    if (argc < 6) {
        fprintf(stderr, "usage: %s flat|tensors WORLD RANK CAP ALIGN N...\n",
                argv[0]);
        return 2;
    }
    const int tensors = strcmp(argv[1], "tensors") == 0;
    const int32_t world = (int32_t)atol(argv[2]);
    const int32_t rank = (int32_t)atol(argv[3]);
    const int64_t cap = atoll(argv[4]);
    const int32_t align = (int32_t)atol(argv[5]);
    const int32_t nt = argc - 6;
    int64_t* numel = malloc(sizeof(int64_t) * (size_t)(nt > 0 ? nt : 1));
    if (!numel) return 2;
    for (int32_t i = 0; i < nt; ++i) numel[i] = atoll(argv[6 + i]);

    zs_layout* L = NULL;
    int rc = tensors
                 ? zs_layout_build_tensors(numel, nt, world, rank, align, &L)
                 : zs_layout_build(numel, nt, world, rank, cap, align, &L);
    if (rc != ZS_OK) {
        free(numel);
        return fail(rc, "build");
    }

    int64_t flat = 0, shard = 0, tiles = 0;
    int32_t nb = 0, nc = 0, w = 0, r = 0;
    if ((rc = zs_layout_info(L, &flat, &shard, &nb, &nc)) != ZS_OK)
        return fail(rc, "info");
    if ((rc = zs_layout_tiles(L, &tiles)) != ZS_OK)
        return fail(rc, "tiles");
    if ((rc = zs_layout_rank(L, &w, &r)) != ZS_OK)
        return fail(rc, "rank");
    printf("info %lld %lld %d %d %lld %d %d\n", (long long)flat,
           (long long)shard, nb, nc, (long long)tiles, w, r);

    int64_t* toff = malloc(sizeof(int64_t) * (size_t)(nt > 0 ? nt : 1));
    zs_bucket* b = malloc(sizeof(zs_bucket) * (size_t)(nb > 0 ? nb : 1));
    zs_chunk* c = malloc(sizeof(zs_chunk) * (size_t)(nc > 0 ? nc : 1));
    int32_t* own = malloc(sizeof(int32_t) * (size_t)(nt > 0 ? nt : 1));
    int64_t* own_off = malloc(sizeof(int64_t) * (size_t)(nt > 0 ? nt : 1));
    if (!toff || !b || !c || !own || !own_off) return 2;

    if ((rc = zs_layout_tensor_offsets(L, toff, nt)) < 0)
        return fail(rc, "tensor offsets");
    for (int32_t i = 0; i < rc; ++i)
        printf("tensor %d %lld\n", i, (long long)toff[i]);
    if ((rc = zs_layout_buckets(L, b, nb)) < 0)
        return fail(rc, "buckets");
    for (int32_t i = 0; i < rc; ++i)
        printf("bucket %lld %lld %lld %lld %lld\n", (long long)b[i].flat_off,
               (long long)b[i].numel, (long long)b[i].slice_numel,
               (long long)b[i].shard_off, (long long)b[i].tile_off);
    if ((rc = zs_layout_chunks(L, c, nc)) < 0)
        return fail(rc, "chunks");
    for (int32_t i = 0; i < rc; ++i)
        printf("chunk %d %d %lld %lld %lld\n", c[i].tensor_id, c[i].bucket_id,
               (long long)c[i].tensor_off, (long long)c[i].numel,
               (long long)c[i].shard_off);
    if (tensors) {
        if ((rc = zs_layout_owners(L, own, own_off, nt)) < 0)
            return fail(rc, "owners");
        for (int32_t i = 0; i < rc; ++i)
            printf("owner %d %d %lld\n", i, own[i], (long long)own_off[i]);
    }

    zs_layout_free(L);
    free(numel);
    free(toff);
    free(b);
    free(c);
    free(own);
    free(own_off);
    return 0;
}
