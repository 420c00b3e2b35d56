// Stand-in for the HIP runtime header in host-only test builds (never part of the library):
// the quantiser's host build needs nothing from it; the C-ABI validation build needs the
// error and stream types and hipGetErrorString, whose host stubs live in the test driver.
#pragma once
#ifdef NVFP4_HOST_ABI_TEST
typedef int hipError_t;
typedef struct ihipStream_t *hipStream_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
const char *hipGetErrorString(hipError_t e);
#endif
