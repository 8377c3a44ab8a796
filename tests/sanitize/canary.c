/* Sanitizer canary (test infrastructure): proves that a toolchain's
 * AddressSanitizer and UndefinedBehaviorSanitizer are live.  Run with "heap"
 * it reads one element past a heap block; with "overflow" it overflows a
 * signed int; with no argument it does neither and exits 0. */
#include <limits.h>
#include <stdlib.h>
#include <string.h>

int main(int argc, char **argv) {
    volatile int *p = (volatile int *)malloc(4 * sizeof(int));
    int r = 0;
    for (int i = 0; i < 4; ++i) p[i] = i;
    if (argc > 1 && strcmp(argv[1], "heap") == 0) r = p[4];
    if (argc > 1 && strcmp(argv[1], "overflow") == 0) {
        volatile int a = INT_MAX;
        r = a + argc;
    }
    free((void *)p);
    return r & 1;
}
