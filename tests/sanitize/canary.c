/* A heap overflow the sanitizer must report: proves that the sanitizer test harness
 * (compiler flags, preloaded runtime, exit status) detects an error at all. */
#include <stdio.h>
#include <stdlib.h>

int main(int argc, char **argv) {
  (void)argv;
  int *a = malloc(8 * sizeof(int));
  for (int i = 0; i < 8; ++i) a[i] = i;
  const int v = a[8 + argc - 1];   /* one past the end */
  printf("%d\n", v);
  free(a);
  return 0;
}
