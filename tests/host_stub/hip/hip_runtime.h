/* Host-only stand-in for the few HIP runtime names the C-ABI host code uses, so that
 * abi.cpp and validate.cpp build with plain g++ (and its sanitizers) for the host
 * tests.  Nothing here touches a GPU. */
#pragma once
#include <stddef.h>
#include <stdint.h>

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorLaunchFailure = 719 };
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

const char* hipGetErrorString(hipError_t e);
hipError_t hipEventRecord(hipEvent_t ev, hipStream_t st);
