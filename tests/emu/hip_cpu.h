// CPU stand-in for <hip/hip_runtime.h>, used only to run the library's HIP sources on the host
// under AddressSanitizer (test infrastructure; the product is built by hipcc for gfx950).
//
// Execution model: every GPU thread of a workgroup is a fiber; workgroups run one after the
// other; __syncthreads() waits for every live thread of the workgroup; wave intrinsics
// (ballot, readlane, shuffles, DPP moves, lane swaps, MFMA) are 64-lane exchanges that need
// every lane of the wave to arrive, so a wave operation under a partial execution mask stops
// the run with a message instead of giving a silently wrong answer.  __shared__ variables
// become function-local statics (one workgroup is live at a time), atomics are plain
// read-modify-writes (fibers never interleave inside one) and "device" pointers are host
// pointers.
#pragma once
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <tuple>
#include <utility>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __shared__ static
#define __launch_bounds__(...)
#define amdgpu_waves_per_eu(...)              // occupancy attributes mean nothing on the host
#define amdgpu_flat_work_group_size(...)
#define __align__(n) __attribute__((aligned(n)))

struct dim3 {
  uint32_t x, y, z;
  constexpr dim3(uint32_t a = 1, uint32_t b = 1, uint32_t c = 1) : x(a), y(b), z(c) {}
};
// HIP's vector types are aligned to their size; so are these, so that the alignment check of
// the emulation build sees a misaligned 16-byte access as the GPU would
struct __attribute__((aligned(16))) int4 { int x, y, z, w; };
struct __attribute__((aligned(16))) uint4 { unsigned x, y, z, w; };
struct __attribute__((aligned(16))) float4 { float x, y, z, w; };
struct __attribute__((aligned(8))) int2 { int x, y; };

typedef int v8i_emu __attribute__((ext_vector_type(8)));
typedef float v4f_emu __attribute__((ext_vector_type(4)));
typedef unsigned int v2u_emu __attribute__((ext_vector_type(2)));

namespace emu {
struct Ctx { dim3 tid, bid, bdim, gdim; int lane, wave; };
Ctx *ctx();
void barrier();
// wave exchange: every live lane of the current wave deposits `in`; `fn` runs once on all
// deposits and fills every lane's output.
void wave_op(const void *in, size_t in_bytes, void *out, size_t out_bytes,
             void (*fn)(const unsigned char *in, unsigned char *out, size_t ib, size_t ob, const void *arg),
             const void *arg);
void launch(dim3 grid, dim3 block, std::function<void()> body);
void lds_register(void *p, size_t n);
}  // namespace emu

#define threadIdx (emu::ctx()->tid)
#define blockIdx (emu::ctx()->bid)
#define blockDim (emu::ctx()->bdim)
#define gridDim (emu::ctx()->gdim)
inline void __syncthreads() { emu::barrier(); }
inline int __lane_id() { return emu::ctx()->lane; }

inline float __int_as_float(int x) { float f; memcpy(&f, &x, 4); return f; }
inline float __uint_as_float(unsigned x) { float f; memcpy(&f, &x, 4); return f; }
inline int __float_as_int(float f) { int x; memcpy(&x, &f, 4); return x; }
inline unsigned __float_as_uint(float f) { unsigned x; memcpy(&x, &f, 4); return x; }
inline int __ffsll(unsigned long long x) { return x ? __builtin_ctzll(x) + 1 : 0; }
inline int __ffsll(long long x) { return __ffsll(static_cast<unsigned long long>(x)); }
inline int __popcll(unsigned long long x) { return __builtin_popcountll(x); }
inline int __popc(unsigned x) { return __builtin_popcount(x); }
inline int __ffs(unsigned x) { return x ? __builtin_ctz(x) + 1 : 0; }
inline int __ffs(int x) { return __ffs(static_cast<unsigned>(x)); }
inline int __clzll(long long x) { return x ? __builtin_clzll(static_cast<unsigned long long>(x)) : 64; }

using std::max;
using std::min;
inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }
inline unsigned min(unsigned a, unsigned b) { return a < b ? a : b; }
inline unsigned max(unsigned a, unsigned b) { return a > b ? a : b; }
inline long long min(long long a, long long b) { return a < b ? a : b; }
inline long long max(long long a, long long b) { return a > b ? a : b; }
inline long min(long a, long b) { return a < b ? a : b; }
inline long max(long a, long b) { return a > b ? a : b; }

// atomics: relaxed read-modify-writes (device-scope relaxed atomics on the GPU), visible as
// atomics to ThreadSanitizer
template <typename T> inline T atomicAdd(T *p, T v) { return __atomic_fetch_add(p, v, __ATOMIC_RELAXED); }
template <typename T> inline T atomicSub(T *p, T v) { return __atomic_fetch_sub(p, v, __ATOMIC_RELAXED); }
template <typename T> inline T atomicOr(T *p, T v) { return __atomic_fetch_or(p, v, __ATOMIC_RELAXED); }
inline unsigned atomicAdd(unsigned *p, int v) { return atomicAdd<unsigned>(p, static_cast<unsigned>(v)); }
inline int atomicAdd(int *p, unsigned v) { return atomicAdd<int>(p, static_cast<int>(v)); }
inline unsigned atomicSub(unsigned *p, int v) { return atomicSub<unsigned>(p, static_cast<unsigned>(v)); }
inline int atomicSub(int *p, unsigned v) { return atomicSub<int>(p, static_cast<int>(v)); }
inline int atomicOr(int *p, unsigned v) { return atomicOr<int>(p, static_cast<int>(v)); }
// compare-and-swap: returns the old value; stores v when it equalled expected
template <typename T> inline T atomicCAS(T *p, T expected, T v) {
  __atomic_compare_exchange_n(p, &expected, v, false, __ATOMIC_RELAXED, __ATOMIC_RELAXED);
  return expected;
}

template <typename T> inline T emu_nontemporal_load(const T *p) { return *p; }

// ---- wave intrinsics
unsigned long long __ballot(bool pred);
inline unsigned long long __ballot(int pred) { return __ballot(pred != 0); }
int emu_readlane_i(int v, int lane);
void emu_amdgcn_wave_barrier();                                  // lanes of the wave meet
inline int emu_amdgcn_readlane(int v, int lane) { return emu_readlane_i(v, lane); }
inline int emu_amdgcn_readfirstlane(int v) { return emu_readlane_i(v, 0); }   // full waves only
inline void emu_amdgcn_sched_group_barrier(int, int, int) {}                 // scheduling hint
inline void emu_amdgcn_sched_barrier(int) {}                                  // scheduling hint
float __shfl_xor(float v, int mask, int width = 64);
int __shfl_xor(int v, int mask, int width = 64);
unsigned __shfl_xor(unsigned v, int mask, int width = 64);
float __shfl(float v, int lane, int width = 64);
int __shfl(int v, int lane, int width = 64);
unsigned __shfl(unsigned v, int lane, int width = 64);
int emu_amdgcn_update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask, bool bound_ctrl);
v2u_emu emu_amdgcn_permlane16_swap(unsigned a, unsigned b, bool fi, bool bc);
v2u_emu emu_amdgcn_permlane32_swap(unsigned a, unsigned b, bool fi, bool bc);
v4f_emu emu_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(v8i_emu a, v8i_emu b, v4f_emu c, int, int, int, int, int, int);
inline unsigned long long emu_amdgcn_s_memrealtime() { return 0; }

// ---- host runtime
typedef int hipError_t;
typedef struct emu_stream *hipStream_t;
typedef struct emu_graph *hipGraph_t;
typedef struct emu_graph *hipGraphExec_t;
typedef struct emu_event *hipEvent_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
enum { hipMemcpyHostToDevice = 1, hipMemcpyDeviceToHost = 2, hipMemcpyDeviceToDevice = 3, hipMemcpyDefault = 4 };
enum { hipStreamCaptureModeGlobal = 0, hipStreamCaptureModeThreadLocal = 1 };
enum { hipHostMallocDefault = 0, hipHostMallocMapped = 2, hipHostMallocCoherent = 0x40000000, hipHostMallocNonCoherent = 0x80000000 };
enum { hipEventDisableTiming = 2 };
hipError_t hipGetLastError();
const char *hipGetErrorString(hipError_t);
hipError_t hipMemcpy(void *d, const void *s, size_t n, int kind);
hipError_t hipMemcpyAsync(void *d, const void *s, size_t n, int kind, hipStream_t st);
hipError_t hipStreamSynchronize(hipStream_t);
hipError_t hipStreamBeginCapture(hipStream_t, int mode);
hipError_t hipStreamEndCapture(hipStream_t, hipGraph_t *g);
hipError_t hipGraphInstantiate(hipGraphExec_t *e, hipGraph_t g, void *, void *, size_t);
hipError_t hipGraphLaunch(hipGraphExec_t e, hipStream_t st);
hipError_t hipGraphDestroy(hipGraph_t g);
hipError_t hipGraphExecDestroy(hipGraphExec_t e);
hipError_t hipHostMalloc(void **p, size_t n, unsigned flags);
hipError_t hipHostGetDevicePointer(void **d, void *h, unsigned flags);
hipError_t hipHostFree(void *p);
hipError_t hipGetDevice(int *d);
hipError_t hipGetSymbolAddress(void **p, const void *sym);
// A __device__ variable's bytes are poisoned the first time its address is taken, since GPU code
// must not rely on the loader's zero fill of memory it later reuses.
namespace emu { const void *device_symbol(const void *p, size_t n); }
#define HIP_SYMBOL(x) (emu::device_symbol(&(x), sizeof(x)))

namespace emu {
template <typename F, typename... A>
inline void launch_kernel(dim3 g, dim3 b, F f, A... args) {
  auto tup = std::make_tuple(args...);
  launch(g, b, [f, tup]() { std::apply(f, tup); });
}
}  // namespace emu
#define EMU_LAUNCH(kernel, grid, block, ...) emu::launch_kernel(dim3(grid), dim3(block), &kernel, __VA_ARGS__)
