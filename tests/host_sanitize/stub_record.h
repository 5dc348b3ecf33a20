// The last launch the stand-in launchers were asked for.
#ifndef STUB_RECORD_H
#define STUB_RECORD_H
#include <stdint.h>

struct stub_call {
  const char *what;
  const void *a, *b;
  void *out;
  int64_t n0, n1, n2, n3;
  int i0;
  int64_t n4;
  const void *lse = nullptr;  // log-sum-exp pairs buffer
  int64_t lse_cap = 0;
  const void *shard_lse = nullptr;
};
extern stub_call g_last;

#endif
