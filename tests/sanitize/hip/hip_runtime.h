/* Host-only stand-in for <hip/hip_runtime.h>, used only to build libcpattn's
 * C-ABI layer (cpattn.cpp) with the host compiler under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  It declares just what that file and
 * cpa_internal.h use; the device-side pieces become plain host objects. */
#pragma once
#include <cstddef>
#include <cstdint>

typedef int hipError_t;
typedef struct ihipStream_t* hipStream_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorInvalidDevice = 101 };

#define __device__
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) (&(x))

const char* hipGetErrorString(hipError_t e);
hipError_t hipGetDevice(int* dev);
hipError_t hipSetDevice(int dev);
hipError_t hipStreamGetDevice(hipStream_t s, int* dev);
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol);
