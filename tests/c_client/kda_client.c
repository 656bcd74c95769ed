/*
 * A plain C client of libkda (test infrastructure): it includes only include/libkda.h
 * and the HIP runtime API, and links libkda.so.
 *
 *   kda_client errors
 *       host-checkable error paths; calls nothing that needs a GPU.
 *   kda_client fwd DIR T B H dk dv slots dtype gate bound scale
 *       reads DIR/{q,k,v,raw,beta,alog,dtb,cu,pool,idx}.bin, runs kda_chunk_fwd on the
 *       device and writes DIR/out.bin and DIR/pool_out.bin (dtype 0 = f32, 1 = bf16).
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "libkda.h"

static int fail(const char *what) {
    fprintf(stderr, "kda_client: %s\n", what);
    return 1;
}

static kda_desc make_desc(long long T, int B, int H, int dk, int dv, int slots, int dtype, int gate, float bound,
                          float scale) {
    kda_desc d;
    memset(&d, 0, sizeof(d));
    d.total_tokens = T;
    d.batch = B;
    d.num_heads = H;
    d.dk = dk;
    d.dv = dv;
    d.max_slots = slots;
    d.qkv_dtype = dtype;
    d.out_dtype = dtype;
    d.gate_mode = gate;
    d.gate_lower_bound = bound;
    d.beta_mode = KDA_BETA_LOGITS;
    d.state_layout = KDA_STATE_K_FIRST;
    d.scale = scale;
    d.num_key_heads = 0;
    return d;
}

static int errors(void) {
    static float dummy[4];
    void *p = dummy;
    kda_desc d = make_desc(128, 2, 4, 128, 128, 4, KDA_BF16, KDA_GATE_SAFE, -5.f, 0.088f);
    if (kda_chunk_fwd(NULL, p, p, p, dummy, dummy, dummy, dummy, (const int32_t *)p, dummy, (const int32_t *)p, p,
                      NULL) != KDA_ERR_NULL)
        return fail("NULL descriptor not refused");
    if (kda_chunk_fwd(&d, NULL, p, p, dummy, dummy, dummy, dummy, (const int32_t *)p, dummy, (const int32_t *)p, p,
                      NULL) != KDA_ERR_NULL)
        return fail("NULL q not refused");
    d.dk = 96;
    d.dv = 96;
    if (kda_chunk_fwd(&d, p, p, p, dummy, dummy, dummy, dummy, (const int32_t *)p, dummy, (const int32_t *)p, p,
                      NULL) != KDA_ERR_UNSUPPORTED)
        return fail("dk = 96 not refused");
    d.dk = d.dv = 128;
    d.num_key_heads = 3;
    if (kda_chunk_fwd(&d, p, p, p, dummy, dummy, dummy, dummy, (const int32_t *)p, dummy, (const int32_t *)p, p,
                      NULL) != KDA_ERR_SHAPE)
        return fail("3 key heads for 4 value heads not refused");
    d.num_key_heads = 0;
    d.batch = 0;  /* nothing to do: returns before any launch */
    if (kda_chunk_fwd(&d, p, p, p, dummy, dummy, dummy, dummy, (const int32_t *)p, dummy, (const int32_t *)p, p,
                      NULL) != KDA_OK)
        return fail("empty batch not accepted");
    if (kda_affine_exclusive_scan(0, 2, 16, 16, dummy, dummy, dummy, dummy, dummy, dummy, NULL) != KDA_ERR_SHAPE)
        return fail("zero segments not refused");
    if (strcmp(kda_status_string(KDA_OK), "ok") != 0) return fail("status string");
    printf("errors ok\n");
    return 0;
}

static void *read_file(const char *dir, const char *name, size_t *n) {
    char path[4096];
    snprintf(path, sizeof(path), "%s/%s.bin", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) return NULL;
    fseek(f, 0, SEEK_END);
    *n = (size_t)ftell(f);
    fseek(f, 0, SEEK_SET);
    void *buf = malloc(*n ? *n : 1);
    if (buf && fread(buf, 1, *n, f) != *n) {
        free(buf);
        buf = NULL;
    }
    fclose(f);
    return buf;
}

static int write_file(const char *dir, const char *name, const void *buf, size_t n) {
    char path[4096];
    snprintf(path, sizeof(path), "%s/%s.bin", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f) return 1;
    const size_t w = fwrite(buf, 1, n, f);
    fclose(f);
    return w != n;
}

/* host file -> new device buffer */
static void *to_device(const char *dir, const char *name, size_t *n) {
    void *h = read_file(dir, name, n);
    if (!h) return NULL;
    void *d = NULL;
    if (hipMalloc(&d, *n ? *n : 1) != hipSuccess || hipMemcpy(d, h, *n, hipMemcpyHostToDevice) != hipSuccess) d = NULL;
    free(h);
    return d;
}

static int fwd(int argc, char **argv) {
    if (argc != 13) return fail("fwd: expected DIR T B H dk dv slots dtype gate bound scale");
    const char *dir = argv[2];
    kda_desc d = make_desc(atoll(argv[3]), atoi(argv[4]), atoi(argv[5]), atoi(argv[6]), atoi(argv[7]), atoi(argv[8]),
                           atoi(argv[9]), atoi(argv[10]), (float)atof(argv[11]), (float)atof(argv[12]));
    const char *names[10] = {"q", "k", "v", "raw", "beta", "alog", "dtb", "cu", "pool", "idx"};
    void *dev[10];
    size_t sz[10];
    for (int i = 0; i < 10; ++i)
        if (!(dev[i] = to_device(dir, names[i], &sz[i]))) return fail(names[i]);
    const size_t e = d.qkv_dtype == KDA_BF16 ? 2 : 4;
    const size_t out_bytes = (size_t)d.total_tokens * d.num_heads * d.dv * e;
    void *out = NULL;
    if (hipMalloc(&out, out_bytes ? out_bytes : 1) != hipSuccess) return fail("hipMalloc out");
    const kda_status st = kda_chunk_fwd(&d, dev[0], dev[1], dev[2], (const float *)dev[3], (const float *)dev[4],
                                        (const float *)dev[5], (const float *)dev[6], (const int32_t *)dev[7],
                                        (float *)dev[8], (const int32_t *)dev[9], out, NULL);
    if (st != KDA_OK) {
        fprintf(stderr, "kda_chunk_fwd: %s\n", kda_status_string(st));
        return 1;
    }
    if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize");
    void *h_out = malloc(out_bytes ? out_bytes : 1), *h_pool = malloc(sz[8]);
    if (hipMemcpy(h_out, out, out_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(h_pool, dev[8], sz[8], hipMemcpyDeviceToHost) != hipSuccess)
        return fail("copy back");
    if (write_file(dir, "out", h_out, out_bytes) || write_file(dir, "pool_out", h_pool, sz[8])) return fail("write");
    for (int i = 0; i < 10; ++i) (void)hipFree(dev[i]);
    (void)hipFree(out);
    free(h_out);
    free(h_pool);
    printf("fwd ok\n");
    return 0;
}

int main(int argc, char **argv) {
    if (argc >= 2 && strcmp(argv[1], "errors") == 0) return errors();
    if (argc >= 2 && strcmp(argv[1], "fwd") == 0) return fwd(argc, argv);
    return fail("usage: kda_client errors | kda_client fwd DIR T B H dk dv slots dtype gate bound scale");
}
