// Host stand-in for <hip/hip_runtime.h>, used only to build the library's
// kernel sources for the CPU SIMT emulator (tests/native/emu/emu.cpp).
//
// Kernel code compiles as ordinary C++: every work-item runs as a fiber,
// threadIdx / blockIdx name the running work-item, __shared__ data is
// per-OS-thread (one workgroup runs at a time on each thread), and every
// operation that exchanges data between work-items (barriers, cross-lane
// builtins, MFMA, transposing LDS reads, LDS-DMA copies) is a call into the
// emulator, which runs the wave's or workgroup's lanes up to that call and
// then performs the operation for all of them at once.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ thread_local
#define __align__(n) __attribute__((aligned(n)))

struct alignas(16) uint4 { unsigned int x, y, z, w; };
struct alignas(8) uint2 { unsigned int x, y; };
struct alignas(16) int4 { int x, y, z, w; };
struct alignas(16) float4 { float x, y, z, w; };
struct alignas(8) float2 { float x, y; };
inline uint4 make_uint4(unsigned a, unsigned b, unsigned c, unsigned d) { return uint4{a, b, c, d}; }
inline uint2 make_uint2(unsigned a, unsigned b) { return uint2{a, b}; }
inline float4 make_float4(float a, float b, float c, float d) { return float4{a, b, c, d}; }
inline float2 make_float2(float a, float b) { return float2{a, b}; }

struct dim3 {
  unsigned x, y, z;
  constexpr dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};

inline float __uint_as_float(unsigned u) { float f; memcpy(&f, &u, 4); return f; }
inline unsigned __float_as_uint(float f) { unsigned u; memcpy(&u, &f, 4); return u; }

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorInvalidConfiguration = 9, hipErrorLaunchFailure = 719 };
typedef struct ihipStream_t* hipStream_t;
enum { hipFuncAttributeMaxDynamicSharedMemorySize = 8 };
inline hipError_t hipFuncSetAttribute(const void*, int, int) { return hipSuccess; }

namespace emu {

struct Idx { unsigned x, y, z; };
extern thread_local Idx tid, bid, bdim, gdim;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// the launch: runs fn() once per work-item of every workgroup
void launch_impl(void (*thunk)(const void*), const void* fn, dim3 grid, dim3 block, size_t shmem, const char* name);
template <class F>
void thunk_of(const void* f) { (*static_cast<const F*>(f))(); }
template <class F>
void launch(const F& f, dim3 grid, dim3 block, size_t shmem, const char* name) {
  launch_impl(&thunk_of<F>, &f, grid, block, shmem, name);
}
hipError_t last_error();

// workgroup and wave operations (called by every active work-item)
void syncthreads();
int readfirstlane(int v);
uint64_t ballot(bool pred);
unsigned shfl_xor_u32(unsigned v, int lane_mask, int width);
u32x2 permlane32_swap(unsigned old, unsigned src, bool fi, bool bc);
f32x16 mfma_32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c, int cbsz, int abid, int blgp);
s16x4 ds_read_tr16_b64(const void* lds);
// LDS-DMA copy of 16 bytes per lane from base + voff to LDS offset m0 + 16 lane
void dma16(uint64_t base, uint32_t voff, uint32_t m0);
void wait_vmem0();
// the dynamic LDS of the running workgroup, and an LDS pointer's offset in it
unsigned char* lds_dynamic();
uint32_t lds_offset(const void* p);

// per-lane arithmetic builtins
float exp2f_(float x);
float fdot2_bf16(bf16x2 a, bf16x2 b, float c, bool clamp);
unsigned perm_b32(unsigned s0, unsigned s1, unsigned sel);

}  // namespace emu

#define threadIdx (::emu::tid)
#define blockIdx (::emu::bid)
#define blockDim (::emu::bdim)
#define gridDim (::emu::gdim)
#define __syncthreads() ::emu::syncthreads()

template <class T>
inline T __shfl_xor(T v, int lane_mask, int width = 64) {
  static_assert(sizeof(T) == 4, "32-bit shuffles only");
  unsigned u;
  memcpy(&u, &v, 4);
  u = ::emu::shfl_xor_u32(u, lane_mask, width);
  T r;
  memcpy(&r, &u, 4);
  return r;
}

#define __builtin_amdgcn_readfirstlane(x) ::emu::readfirstlane(x)
#define __builtin_amdgcn_ballot_w64(x) ::emu::ballot(x)
#define __builtin_amdgcn_sched_barrier(x) ((void)0)
#define __builtin_amdgcn_exp2f(x) ::emu::exp2f_(x)
#define __builtin_amdgcn_fdot2_f32_bf16(a, b, c, cl) ::emu::fdot2_bf16(a, b, c, cl)
#define __builtin_amdgcn_perm(a, b, s) ::emu::perm_b32(a, b, s)
#define __builtin_amdgcn_permlane32_swap(a, b, fi, bc) ::emu::permlane32_swap(a, b, fi, bc)
#define __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, x, y, z) ::emu::mfma_32x32x16_bf16(a, b, c, x, y, z)
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(p) ::emu::ds_read_tr16_b64((const void*)(p))

#define hipLaunchKernelGGL(kernel, grid, block, shmem, stream, ...) \
  ::emu::launch([=]() { kernel(__VA_ARGS__); }, dim3(grid), dim3(block), (size_t)(shmem), #kernel)
inline hipError_t hipGetLastError() { return ::emu::last_error(); }
