// Queries of the host-memory HIP stand-in (hip_stub.cpp) for the host check.
#pragma once
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  char name[160];
  unsigned grid[3], block[3];
  size_t shmem;
} StubLaunch;

size_t stub_live_allocations(void);             /* hipMalloc blocks not yet freed      */
size_t stub_allocation_size(const void* p);     /* bytes of a live block, else 0       */
size_t stub_launch_count(void);
StubLaunch stub_launch(size_t i);
void stub_clear_launches(void);
void stub_fail_malloc_after(int n);             /* the n-th next hipMalloc fails (0: the next) */
/* Keep a copy of the first `bytes` bytes of the first kernel argument of every
 * launch whose kernel name contains `name_part` (at most 4 such rules). */
void stub_capture_first_arg(const char* name_part, size_t bytes);
/* The copy kept for launch i: its size (0 when none was kept), copied to out
 * when out is not null and max is at least that size. */
size_t stub_launch_first_arg(size_t i, void* out, size_t max);

#ifdef __cplusplus
}
#endif
