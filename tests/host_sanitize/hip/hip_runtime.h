/* Host-only stand-in for the HIP runtime header, for the sanitizer build of
 * the C-ABI layer (api.cpp): the few types and codes that layer and
 * kernels.h name.  The kernels are not compiled in that build; stubs stand
 * in for their launchers. */
#pragma once
#include <stdint.h>

typedef struct ihipStream_t* hipStream_t;
typedef enum hipError_t { hipSuccess = 0, hipErrorInvalidValue = 1 } hipError_t;
