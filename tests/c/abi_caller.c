/*
 * A C caller of the scan's five entry points and three helpers written
 * against the contract's own prototypes: each library function is assigned
 * to a pointer of the contract's type, so a signature that differs fails to
 * compile (-Werror).  At run time it makes only calls that the host-side
 * checks reject or that have nothing to do, so it needs no GPU.
 */
#include "bdssm.h"

#include <stdio.h>

typedef int (*prefill_t)(const bdssm_shape *, int64_t, const void *, const void *, const void *,
                         const void *, const float *, const float *, const float *, float *, void *,
                         void *, size_t, hipStream_t);
typedef int (*block_step_t)(const bdssm_shape *, const float *, const void *, const void *,
                            const void *, const void *, const float *, const float *, void *,
                            hipStream_t);
typedef int (*commit_t)(const bdssm_shape *, float *, const void *, const void *, const void *,
                        const void *, const float *, const float *, void *, hipStream_t);
typedef int (*train_scan_t)(const bdssm_shape *, int64_t, const void *, const void *, const void *,
                            const void *, const float *, const float *, const float *, void *,
                            float *, void *, size_t, hipStream_t);
typedef int (*full_scan_t)(const bdssm_shape *, int64_t, const void *, const void *, const void *,
                           const void *, const float *, const float *, void *, void *, size_t,
                           hipStream_t);
typedef size_t (*workspace_t)(const bdssm_shape *, int64_t);
typedef const char *(*status_str_t)(int);
typedef int (*version_t)(void);

int main(void) {
    const prefill_t prefill = bdssm_prefill;
    const block_step_t block_step = bdssm_block_step;
    const commit_t commit = bdssm_commit;
    const train_scan_t train_scan = bdssm_train_scan;
    const full_scan_t full_scan = bdssm_full_scan;
    const workspace_t workspace = bdssm_workspace_bytes;
    const status_str_t status_str = bdssm_status_str;
    const version_t version = bdssm_version;

    const bdssm_shape s = {8, 1536, 16, 16, BDSSM_BF16};
    const bdssm_shape bad = {8, 1536, 6, 16, BDSSM_BF16};    /* d_state 6: unsupported */
    const bdssm_shape empty = {0, 1536, 16, 16, BDSSM_F32};  /* batch 0: nothing to do */
    hipStream_t st = NULL;
    /* one line per result: name value */
    printf("version %d\n", version());
    printf("workspace_65536 %zu\n", workspace(&s, 65536));
    printf("workspace_bad %d\n", workspace(&bad, 65536) == (size_t)-1);
    printf("prefill_null %d\n", prefill(NULL, 16, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, st));
    printf("prefill_shape %d\n", prefill(&bad, 16, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, st));
    printf("block_step_null %d\n", block_step(NULL, 0, 0, 0, 0, 0, 0, 0, 0, st));
    printf("commit_shape %d\n", commit(&bad, 0, 0, 0, 0, 0, 0, 0, 0, st));
    printf("train_scan_shape %d\n", train_scan(&s, 24, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, st));
    printf("full_scan_empty %d\n", full_scan(&empty, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, st));
    printf("status_ok %s\n", status_str(BDSSM_OK));
    return 0;
}
