/* Line-driven caller of the C ABI in include/fa.h, for running the host-side
 * argument checks under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Built (by tests/test_abi_sanitized.py) as one executable together with the
 * library's host code compiled with both sanitizers and no device code. Each
 * line on stdin names one entry point and its arguments, separated by
 * spaces: pointers and 64-bit integers in decimal (0 is NULL), int and size_t
 * in decimal, floats as C99 hexadecimal or nan / inf / -inf. The driver calls
 * the function and prints its result on one line (fa_strerror prints the
 * string). Streams are always NULL. An unknown name or a wrong argument count
 * prints "error: ..." and exits with status 2.
 *
 * The driver is written in C on purpose: it also checks that fa.h compiles as
 * a C header. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa.h"

#define MAX_ARGS 32

static char* tok[MAX_ARGS + 1];
static int ntok;

static void* P(int i) { return (void*)(uintptr_t)strtoull(tok[i], NULL, 10); }
static int I(int i) { return (int)strtol(tok[i], NULL, 10); }
static size_t Z(int i) { return (size_t)strtoull(tok[i], NULL, 10); }
static float F(int i) { return strtof(tok[i], NULL); }
static uint64_t U(int i) { return (uint64_t)strtoull(tok[i], NULL, 10); }

static int need(int n) {
  if (ntok - 1 != n) {
    printf("error: %s takes %d arguments, got %d\n", tok[0], n, ntok - 1);
    exit(2);
  }
  return 1;
}

static void call(void) {
  const char* f = tok[0];
  if (!strcmp(f, "fa_version") && need(0)) {
    printf("%d\n", fa_version());
  } else if (!strcmp(f, "fa_strerror") && need(1)) {
    printf("%s\n", fa_strerror(I(1)));
  } else if (!strcmp(f, "fa_fwd_workspace_size") && need(7)) {
    printf("%zu\n", fa_fwd_workspace_size(I(1), I(2), I(3), I(4), I(5), I(6), (fa_dtype)I(7)));
  } else if (!strcmp(f, "fa_bwd_workspace_size") && need(7)) {
    printf("%zu\n", fa_bwd_workspace_size(I(1), I(2), I(3), I(4), I(5), I(6), (fa_dtype)I(7)));
  } else if (!strcmp(f, "fa_fwd_paged_workspace_size") && need(7)) {
    printf("%zu\n",
           fa_fwd_paged_workspace_size(I(1), I(2), I(3), I(4), I(5), I(6), (fa_dtype)I(7)));
  } else if (!strcmp(f, "fa_fwd") && need(17)) {
    printf("%d\n", fa_fwd(P(1), P(2), P(3), P(4), (float*)P(5), P(6), Z(7), I(8), I(9), I(10),
                          I(11), I(12), I(13), F(14), I(15), (fa_dtype)I(16), (hipStream_t)P(17)));
  } else if (!strcmp(f, "fa_bwd") && need(21)) {
    printf("%d\n", fa_bwd(P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8), P(9),
                          P(10), Z(11), I(12), I(13), I(14), I(15), I(16), I(17), F(18), I(19),
                          (fa_dtype)I(20), (hipStream_t)P(21)));
  } else if (!strcmp(f, "fa_bwd_stage") && need(22)) {
    printf("%d\n", fa_bwd_stage(I(1), P(2), P(3), P(4), P(5), (const float*)P(6), P(7), P(8),
                                P(9), P(10), P(11), Z(12), I(13), I(14), I(15), I(16), I(17),
                                I(18), F(19), I(20), (fa_dtype)I(21), (hipStream_t)P(22)));
  } else if (!strcmp(f, "fa_bwd_noalloc") && need(19)) {
    printf("%d\n", fa_bwd_noalloc(P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8),
                                  P(9), I(10), I(11), I(12), I(13), I(14), I(15), F(16), I(17),
                                  (fa_dtype)I(18), (hipStream_t)P(19)));
  } else if (!strcmp(f, "fa_fwd_paged") && need(19)) {
    printf("%d\n", fa_fwd_paged(P(1), P(2), P(3), (const int*)P(4), (const int*)P(5), P(6),
                                (float*)P(7), P(8), Z(9), I(10), I(11), I(12), I(13), I(14), I(15),
                                I(16), F(17), (fa_dtype)I(18), (hipStream_t)P(19)));
  } else if (!strcmp(f, "fa_fwd_dropout") && need(20)) {
    printf("%d\n", fa_fwd_dropout(P(1), P(2), P(3), P(4), (float*)P(5), P(6), Z(7), I(8), I(9),
                                  I(10), I(11), I(12), I(13), F(14), I(15), F(16), U(17), U(18),
                                  (fa_dtype)I(19), (hipStream_t)P(20)));
  } else if (!strcmp(f, "fa_bwd_dropout") && need(24)) {
    printf("%d\n", fa_bwd_dropout(P(1), P(2), P(3), P(4), (const float*)P(5), P(6), P(7), P(8),
                                  P(9), P(10), Z(11), I(12), I(13), I(14), I(15), I(16), I(17),
                                  F(18), I(19), F(20), U(21), U(22), (fa_dtype)I(23),
                                  (hipStream_t)P(24)));
  } else if (!strcmp(f, "fa_dropout_mask") && need(9)) {
    printf("%d\n", fa_dropout_mask((unsigned char*)P(1), I(2), I(3), I(4), I(5), F(6), U(7), U(8),
                                   (hipStream_t)P(9)));
  } else if (!strcmp(f, "fa_fwd_fp8") && need(17)) {
    printf("%d\n", fa_fwd_fp8(P(1), P(2), P(3), P(4), (float*)P(5), I(6), I(7), I(8), I(9), I(10),
                              I(11), F(12), I(13), F(14), F(15), F(16), (hipStream_t)P(17)));
  } else {
    printf("error: unknown entry point %s\n", f);
    exit(2);
  }
}

int main(void) {
  char line[4096];
  while (fgets(line, sizeof line, stdin)) {
    ntok = 0;
    for (char* t = strtok(line, " \t\r\n"); t && ntok <= MAX_ARGS; t = strtok(NULL, " \t\r\n"))
      tok[ntok++] = t;
    if (ntok == 0) continue;
    call();
    fflush(stdout);
  }
  return 0;
}
