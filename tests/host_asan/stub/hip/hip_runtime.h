// Host-only stand-in for the HIP runtime API, for building the library's host
// bookkeeping (pool.hip) with the host compiler under AddressSanitizer.
// "Device" memory is host memory; every call is defined by the test driver,
// which records what the library asks for and can make a call fail.
#pragma once

#include <cstddef>
#include <cstdint>

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorOutOfMemory = 2,
  hipErrorInvalidDevice = 101,
  hipErrorLaunchFailure = 719,
  hipErrorNotSupported = 801
} hipError_t;

typedef struct ihipStream_t* hipStream_t;

typedef enum hipMemcpyKind {
  hipMemcpyHostToHost = 0,
  hipMemcpyHostToDevice = 1,
  hipMemcpyDeviceToHost = 2,
  hipMemcpyDeviceToDevice = 3,
  hipMemcpyDefault = 4
} hipMemcpyKind;

#define hipHostMallocDefault 0u
#define __device__
#define __host__
#define __global__
#define __forceinline__ inline
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) (reinterpret_cast<const void*>(&(x)))

inline unsigned int __umulhi(unsigned int a, unsigned int b) {
  return static_cast<unsigned int>((static_cast<unsigned long long>(a) * b) >> 32);
}

const char* hipGetErrorString(hipError_t e);
hipError_t hipGetDevice(int* device);
hipError_t hipSetDevice(int device);
hipError_t hipDeviceSynchronize(void);
hipError_t hipStreamSynchronize(hipStream_t stream);
hipError_t hipMalloc(void** ptr, size_t bytes);
hipError_t hipFree(void* ptr);
hipError_t hipHostMalloc(void** ptr, size_t bytes, unsigned int flags);
hipError_t hipHostFree(void* ptr);
hipError_t hipMemset(void* dst, int value, size_t bytes);
hipError_t hipMemsetAsync(void* dst, int value, size_t bytes, hipStream_t stream);
hipError_t hipMemcpy(void* dst, const void* src, size_t bytes, hipMemcpyKind kind);
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t stream);
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol);
