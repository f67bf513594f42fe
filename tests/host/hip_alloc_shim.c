/* Host-only stand-ins for three HIP allocation calls, preloaded into a test
 * process (no GPU is touched): device allocations come from malloc, every
 * pinned-host allocation fails with hipErrorOutOfMemory (2).  shim_counts()
 * reports the calls so that the test can check nothing leaked. */
#include <stddef.h>
#include <stdlib.h>

static int n_malloc, n_free, n_host;

int hipMalloc(void **p, size_t n)
{
    *p = malloc(n ? n : 1);
    if (!*p) return 2;
    ++n_malloc;
    return 0;
}

int hipFree(void *p)
{
    if (p) {
        free(p);
        ++n_free;
    }
    return 0;
}

int hipHostMalloc(void **p, size_t n, unsigned int flags)
{
    (void)n;
    (void)flags;
    *p = NULL;
    ++n_host;
    return 2;
}

void shim_counts(int *out)
{
    out[0] = n_malloc;
    out[1] = n_free;
    out[2] = n_host;
}
