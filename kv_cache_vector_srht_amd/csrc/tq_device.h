// Device helpers shared by the HIP translation units of libtq (gfx950, wave64).
#ifndef TQ_DEVICE_H_
#define TQ_DEVICE_H_

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include "tq_internal.h"

namespace tq {
namespace dev {

constexpr int D = TQ_HEAD_DIM;
constexpr int PT = TQ_PAGE_TOKENS;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSqrtHalfPi = 1.2533141373155003f;  // sqrt(pi / 2)
constexpr float kHalfPi = 1.5707963267948966f;       // pi / 2
constexpr int kEncodeRowBytes = 144;                 // LDS row of 128 code bytes + pad

// ------------------------------------------------------------ checked builds
// A build with TQ_DEVICE_CHECKS=1 verifies the kernels' index invariants as
// they run: an index outside its array sets its check's bit in this
// translation unit's check word (tq_device_checks reads them) and is clamped
// into the array, so the access stays in bounds.  A release build compiles the
// checks out (checked() returns its index).
#ifndef TQ_DEVICE_CHECKS
#define TQ_DEVICE_CHECKS 0
#endif
enum : uint32_t {
  kCheckEncodeGrid = 1u,      // the encoder's lookup grid
  kCheckEncodeStream = 2u,    // stream dwords and code-byte rows of a page part
  kCheckQjlLds = 4u,          // the QJL key encoder's LDS (S' tiles, tables, rows)
  kCheckDecodeTable = 8u,     // decode's codebook tables and weight rows
  kCheckDecodeIndex = 16u,    // decode's descriptor slots and partial slots
  kCheckCombine = 32u,        // the combine's partial lists
  kCheckPages = 64u,          // the append and re-tier kernels
};
#if TQ_DEVICE_CHECKS
static __device__ uint32_t g_check_word;
#endif
__device__ __forceinline__ int checked(int i, int n, uint32_t bit) {
#if TQ_DEVICE_CHECKS
  if ((unsigned)i >= (unsigned)n) {
    atomicOr(&g_check_word, bit);
    return i < 0 ? 0 : n - 1;
  }
#else
  (void)n;
  (void)bit;
#endif
  return i;
}

// ----------------------------------------------------------------- helpers
__device__ __forceinline__ size_t page_size_dev(int kb, int vb, bool qjl) {
  return kb == 0 ? (size_t)2 * PT * D * 2 : (size_t)1024 * (kb + vb) + 512 + (qjl ? 1280 : 0);
}

// A page descriptor as the kernels read it: a pending page is an fp16 page.
struct PageDesc {
  uint64_t off;
  int kb, vb;
  bool qjl, present;
};

__device__ __forceinline__ PageDesc read_desc(uint64_t d) {
  PageDesc p;
  p.off = d & TQ_PAGE_OFFSET_MASK;
  p.present = (d & TQ_PAGE_PRESENT) != 0;
  const bool pending = (d & TQ_PAGE_PENDING) != 0;
  p.kb = pending ? 0 : (int)((d >> 48) & 15);
  p.vb = pending ? 0 : (int)((d >> 52) & 15);
  p.qjl = !pending && (d & TQ_PAGE_QJL) != 0;
  return p;
}

__device__ __forceinline__ float flip_if(float x, uint32_t neg) {
  return __uint_as_float(__float_as_uint(x) ^ (neg << 31));
}

__device__ __forceinline__ uint32_t dsign(const uint32_t (&m)[4], int j) {
  return (m[j >> 5] >> (j & 31)) & 1u;
}

// In-register Walsh-Hadamard transform (Sylvester order, unnormalised).
__device__ __forceinline__ void fwht128(float (&x)[D]) {
#pragma clang loop unroll(full)
  for (int h = 1; h < D; h <<= 1) {
#pragma clang loop unroll(full)
    for (int i = 0; i < D; i += 2 * h) {
#pragma clang loop unroll(full)
      for (int j = i; j < i + h; ++j) {
        const float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
    }
  }
}

// `w` (<= 16) bits starting at bit `pos` of a little-endian dword array; with
// the caller's loops unrolled, pos is a constant and this folds to one or two
// instructions.
template <int N>
__device__ __forceinline__ uint32_t bits_at(const uint32_t (&s)[N], int pos, int w) {
  const int wi = pos >> 5, sh = pos & 31;
  uint32_t v = s[wi] >> sh;
  if (sh + w > 32) v |= s[wi + 1] << (32 - sh);
  return v & ((1u << w) - 1u);
}

// Coordinate k (0 or 1) of V stream s of a packed page: stream s = n + 32 P
// (n < 32) holds, for every token t, the codes of the coordinate pair c0, c0 + 1
// at stream positions 2t and 2t + 1, with
// c0 = 64 bit2(n) + 32 P + 8 (n >> 3) + 2 (n & 3).  Each stream is one
// coordinate pair over the page's 64 tokens (a PolarQuant pair too), the pair
// the decode's matrix-core value sums give a lane.
__device__ __forceinline__ int v_stream_coord(int s, int k) {
  const int n = s & 31;
  return 64 * ((n >> 2) & 1) + 32 * (s >> 5) + 8 * (n >> 3) + 2 * (n & 3) + k;
}

// Wavefront reductions (every lane active).  Inside each 16-lane row the
// partner values come through DPP (quad permutations xor 1 and xor 2, then the
// half-row and row mirrors), which keeps them in the VALU pipeline; the four
// row results are then read as scalars.  Every lane returns the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror: the other quad of the 8
  v = fmaxf(v, dpp_f<0x140>(v));   // row_mirror: the other 8 of the row
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Orders this wave's LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float load_elem(const void* p, int dtype, size_t i) {
  return dtype == TQ_DTYPE_F16 ? __half2float(reinterpret_cast<const __half*>(p)[i])
                               : reinterpret_cast<const float*>(p)[i];
}


// Host helpers of the entry points.
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// OR-s this translation unit's check word into *out and zeroes it when reset
// (synchronous copies; a release build has no word and leaves *out alone).
static inline int read_check_word(uint32_t* out, bool reset) {
#if TQ_DEVICE_CHECKS
  uint32_t v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_check_word), sizeof v) != hipSuccess) return TQ_ERR_DEVICE;
  *out |= v;
  if (reset) {
    const uint32_t z = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_check_word), &z, sizeof z) != hipSuccess) return TQ_ERR_DEVICE;
  }
#else
  (void)out;
  (void)reset;
#endif
  return TQ_OK;
}

inline int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace dev
}  // namespace tq

#endif  // TQ_DEVICE_H_
