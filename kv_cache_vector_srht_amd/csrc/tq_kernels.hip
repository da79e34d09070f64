// HIP kernels of libtq for gfx950 (CDNA4, wave64) and their C-ABI entry points.
//
// Encode ("TurboQuant-MLX v2.0", How It Works > Pipeline; "TurboMOQ",
// Architecture): one wavefront per (page, KV head, session, K|V); lane = token.
// Each lane holds its 128-value head vector in registers, computes the norm,
// applies D, the 128-point Walsh-Hadamard butterfly (7 stages, in registers),
// D and 1/norm, quantises against the boundaries staged in LDS and packs its
// codes.  Key streams are written straight from the lane that owns the token;
// value streams are transposed through LDS first.  QJL keys also get
// r = x - xhat (one more in-register butterfly) and the 128 signs of S r.
//
// Decode attention: (1) query prep rotates each query head (R q, and S q for
// QJL), pre-scaled for exp2; (2) split-K: a 4-wave workgroup per (session,
// KV head, page range); per page, lane = token for the key scores of the G
// query heads of the KV head (codes looked up two at a time in LDS tables,
// query coordinates read as wave-uniform scalars), an online softmax with
// wavefront reductions, then lane = (token quarter, 8 coordinates) for the
// value accumulation in the rotated domain; (3) combine: log-sum-exp merge of
// the splits and one inverse rotation per query head (the Walsh-Hadamard
// transform factored out of the value sum, as the MLX TurboQuant skill page
// reports for its Metal kernels, Path A > Optimisations Metal).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int D = TQ_HEAD_DIM;
constexpr int PT = TQ_PAGE_TOKENS;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSqrtHalfPi = 1.2533141373155003f;  // sqrt(pi / 2)
constexpr int kEncodeRowBytes = 144;                 // LDS row of 128 code bytes + pad

// ----------------------------------------------------------------- helpers
__device__ __forceinline__ size_t page_size_dev(int kb, int vb, bool qjl) {
  return kb == 0 ? (size_t)2 * PT * D * 2 : (size_t)1024 * (kb + vb) + 512 + (qjl ? 1280 : 0);
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

__device__ __forceinline__ float wave_max(float v) {
#pragma clang loop unroll(full)
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma clang loop unroll(full)
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
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

// ------------------------------------------------------------------ encode
struct EncodeArgs {
  const void* k;
  const void* v;
  int dtype;
  int tok0, ntok, page0;
  int64_t sb, sh, st;
  int32_t* err;
  const uint64_t* pages;
  int n_kv_heads, max_pages;
  char* pool;
  uint64_t pool_bytes;
  const uint32_t* sign_mask;
  const float* k_table;
  const float* v_table;
  const float* qjl_s;
};

__device__ __forceinline__ void raise_flag(int32_t* err, int bit) {
  if (err) atomicOr(err, bit);
}

// Loads one head vector (128 values) as float.
__device__ __forceinline__ void load_row(const void* base, int dtype, size_t elem_off, float (&x)[D]) {
  if (dtype == TQ_DTYPE_F16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(base) + elem_off);
#pragma clang loop unroll(full)
    for (int c = 0; c < D / 8; ++c) {
      uint4 w = p[c];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma clang loop unroll(full)
      for (int e = 0; e < 4; ++e) {
        __half2 h2 = *reinterpret_cast<const __half2*>(&ww[e]);
        float2 f = __half22float2(h2);
        x[8 * c + 2 * e] = f.x;
        x[8 * c + 2 * e + 1] = f.y;
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem_off);
#pragma clang loop unroll(full)
    for (int c = 0; c < D / 4; ++c) {
      float4 f = p[c];
      x[4 * c] = f.x;
      x[4 * c + 1] = f.y;
      x[4 * c + 2] = f.z;
      x[4 * c + 3] = f.w;
    }
  }
}

// Walsh-Hadamard transform of each 64-value half (stages 1..32); the last
// stage (pairs j, j+64) is left to the caller so that it can consume outputs
// as they are produced.
__device__ __forceinline__ void fwht_halves(float (&x)[D]) {
#pragma clang loop unroll(full)
  for (int h = 1; h < D / 2; h <<= 1) {
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

template <int B>
__device__ __forceinline__ uint32_t quantize(float u, const float* thr) {
  uint32_t c = 0;
#pragma clang loop unroll(full)
  for (int s = 1 << (B - 1); s >= 1; s >>= 1) c += (u >= thr[c + s - 1]) ? (uint32_t)s : 0u;
  return c;
}

// Norm, rotation and quantisation of one vector held by this lane:
// u = D H D x / ||x||, code_j = #{k : t_k <= u_j} (binary search over the
// boundaries in LDS).  Codes go to `emit(j, code)`; on return x holds the
// rotated-domain residual u - c[code] (used by QJL).
template <int B, class Emit>
__device__ __forceinline__ float rotate_quantize(float (&x)[D], const uint32_t (&m)[4],
                                                 const float* thr, const float* cent, Emit emit) {
  float ss = 0.f;
#pragma clang loop unroll(full)
  for (int j = 0; j < D; ++j) ss = fmaf(x[j], x[j], ss);
  const float n = sqrtf(ss);
#pragma clang loop unroll(full)
  for (int j = 0; j < D; ++j) x[j] = flip_if(x[j], dsign(m, j));
  fwht_halves(x);
  const float inv = n > 0.f ? 1.0f / n : 0.f;
#pragma clang loop unroll(full)
  for (int j = 0; j < D / 2; ++j) {
    const float a = x[j], b = x[j + D / 2];
    const float u0 = flip_if(a + b, dsign(m, j)) * inv;
    const float u1 = flip_if(a - b, dsign(m, j + D / 2)) * inv;
    const uint32_t c0 = quantize<B>(u0, thr);
    const uint32_t c1 = quantize<B>(u1, thr);
    emit(j, c0);
    emit(j + D / 2, c1);
    x[j] = u0 - cent[c0];
    x[j + D / 2] = u1 - cent[c1];
  }
  return n;
}

template <int PART, int B>
__device__ __forceinline__ void encode_packed(const float* __restrict__ qjl_s, char* page, bool qjl, int lane,
                              float (&x)[D], const uint32_t (&m)[4], float* lds_thr,
                              float* lds_cent, uint32_t* lds_rows) {
  constexpr int kb = B;
  if constexpr (PART == 0) {
    uint32_t sw[4 * B];
#pragma clang loop unroll(full)
    for (int i = 0; i < 4 * B; ++i) sw[i] = 0;
    const float n = rotate_quantize<B>(x, m, lds_thr, lds_cent, [&](int j, uint32_t c) {
      const int pos = j * B, wi = pos >> 5, sh = pos & 31;
      sw[wi] |= c << sh;
      if (sh + B > 32) sw[wi + 1] |= c >> (32 - sh);
    });
    uint4* dst = reinterpret_cast<uint4*>(page);
#pragma clang loop unroll(full)
    for (int w = 0; w < B; ++w)
      dst[w * 64 + lane] = make_uint4(sw[4 * w], sw[4 * w + 1], sw[4 * w + 2], sw[4 * w + 3]);
    reinterpret_cast<float*>(page + 1024 * kb)[lane] = n;
    if (qjl) {
      // r = x - xhat = (n / d) D H D (u - c): one more butterfly in registers.
      float e2 = 0.f;
#pragma clang loop unroll(full)
      for (int j = 0; j < D; ++j) {
        e2 = fmaf(x[j], x[j], e2);
        x[j] = flip_if(x[j], dsign(m, j));
      }
      fwht128(x);
      const float sc = n * (1.0f / D);
#pragma clang loop unroll(full)
      for (int j = 0; j < D; ++j) x[j] = flip_if(x[j], dsign(m, j)) * sc;
      const float gamma = n * sqrtf(e2) * 0.08838834764831845f;  // n ||u - c|| / sqrt(d)
      uint32_t zw[4];
#pragma clang loop unroll(full)
      for (int w = 0; w < 4; ++w) {
        uint32_t bitsw = 0;
        for (int ii = 0; ii < 32; ++ii) {
          const float* srow = qjl_s + (size_t)(32 * w + ii) * D;
          float p = 0.f;
#pragma clang loop unroll(full)
          for (int j = 0; j < D; ++j) p = fmaf(srow[j], x[j], p);
          bitsw |= (p >= 0.f ? 1u : 0u) << ii;
        }
        zw[w] = bitsw;
      }
      char* qbase = page + 1024 * kb + 256;
      reinterpret_cast<uint4*>(qbase)[lane] = make_uint4(zw[0], zw[1], zw[2], zw[3]);
      reinterpret_cast<float*>(qbase + 1024)[lane] = gamma;
    }
  } else {
    // Codes as bytes into this lane's LDS row, then transpose into V streams.
    uint32_t cb[D / 4];
#pragma clang loop unroll(full)
    for (int i = 0; i < D / 4; ++i) cb[i] = 0;
    const float n = rotate_quantize<B>(x, m, lds_thr, lds_cent, [&](int j, uint32_t c) {
      cb[j >> 2] |= c << (8 * (j & 3));
    });
    uint4* row = reinterpret_cast<uint4*>(reinterpret_cast<char*>(lds_rows) + lane * kEncodeRowBytes);
#pragma clang loop unroll(full)
    for (int i = 0; i < D / 16; ++i) row[i] = make_uint4(cb[4 * i], cb[4 * i + 1], cb[4 * i + 2], cb[4 * i + 3]);
    __syncthreads();
    const int q = lane >> 4, ii = lane & 15;
    uint32_t sw[4 * B];
#pragma clang loop unroll(full)
    for (int i = 0; i < 4 * B; ++i) sw[i] = 0;
#pragma clang loop unroll(full)
    for (int k = 0; k < 16; ++k) {
      const uint2 b8 = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(lds_rows) +
                                                        (4 * k + q) * kEncodeRowBytes + 8 * ii);
#pragma clang loop unroll(full)
      for (int e = 0; e < 8; ++e) {
        const uint32_t c = ((e < 4 ? b8.x : b8.y) >> (8 * (e & 3))) & 0xffu;
        const int pos = (8 * k + e) * B, wi = pos >> 5, sh = pos & 31;
        sw[wi] |= c << sh;
        if (sh + B > 32) sw[wi + 1] |= c >> (32 - sh);
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(page);
#pragma clang loop unroll(full)
    for (int w = 0; w < B; ++w)
      dst[w * 64 + lane] = make_uint4(sw[4 * w], sw[4 * w + 1], sw[4 * w + 2], sw[4 * w + 3]);
    reinterpret_cast<float*>(page + 1024 * B)[lane] = n;
  }
}

// One wavefront per (page, KV head, session); PART 0 encodes keys, 1 values.
template <int PART>
__global__ __launch_bounds__(64) void encode_kernel(EncodeArgs a, const uint64_t* __restrict__ pages,
                                                    const float* __restrict__ qjl_s) {
  __shared__ float lds_thr[256];
  __shared__ float lds_cent[256];
  __shared__ uint32_t lds_rows[PT * kEncodeRowBytes / 4];
  const int lane = threadIdx.x;
  const int pg = a.page0 + blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  constexpr int part = PART;
  const uint64_t desc = pages[((size_t)b * a.n_kv_heads + h) * a.max_pages + pg];
  if (!(desc & TQ_PAGE_PRESENT)) {
    if (lane == 0) raise_flag(a.err, 2);
    return;
  }
  const int kb = (int)((desc >> 48) & 15), vb = (int)((desc >> 52) & 15);
  const bool qjl = (desc & TQ_PAGE_QJL) != 0;
  const uint64_t off = desc & TQ_PAGE_OFFSET_MASK;
  const bool bad_fmt = kb == 0 ? (vb != 0 || qjl) : (kb > 8 || vb < 1 || vb > 8);
  if (bad_fmt || off + page_size_dev(kb, vb, qjl) > a.pool_bytes) {
    if (lane == 0) raise_flag(a.err, 4);
    return;
  }
  char* page = a.pool + off;
  const int t_first = pg * PT;
  const int lo = max(t_first, a.tok0), hi = min(t_first + PT, a.tok0 + a.ntok);
  const void* src = part == 0 ? a.k : a.v;
  const size_t base = (size_t)b * a.sb + (size_t)h * a.sh;

  if (kb == 0) {
    // fp16 page: copy the covered rows of this part, 4 rows per pass.
    __half* dst = reinterpret_cast<__half*>(page + part * PT * D * 2);
    const int r = lane >> 4, c8 = (lane & 15) * 8;
    for (int t = lo + r; t < hi; t += 4) {
      const size_t e = base + (size_t)(t - a.tok0) * a.st + c8;
      uint4 out;
      if (a.dtype == TQ_DTYPE_F16) {
        out = *reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(src) + e);
      } else {
        const float4 f0 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + e);
        const float4 f1 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + e + 4);
        __half2 h0 = __floats2half2_rn(f0.x, f0.y), h1 = __floats2half2_rn(f0.z, f0.w);
        __half2 h2 = __floats2half2_rn(f1.x, f1.y), h3 = __floats2half2_rn(f1.z, f1.w);
        out = make_uint4(*reinterpret_cast<uint32_t*>(&h0), *reinterpret_cast<uint32_t*>(&h1),
                         *reinterpret_cast<uint32_t*>(&h2), *reinterpret_cast<uint32_t*>(&h3));
      }
      *reinterpret_cast<uint4*>(dst + (size_t)(t - t_first) * D + c8) = out;
    }
    return;
  }
  if (lo != t_first || hi != t_first + PT) {
    if (lane == 0) raise_flag(a.err, 1);
    return;
  }
  if (part == 0 && qjl && a.qjl_s == nullptr) {
    if (lane == 0) raise_flag(a.err, 8);
    return;
  }
  if (part == 0 && !qjl) return;   // non-QJL key pages are written by encode_pages_kernel
  const int B = part == 0 ? kb : vb;
  const float* table = part == 0 ? a.k_table : a.v_table;
  const int L = 1 << B;
  for (int i = lane; i < L; i += 64) {
    lds_cent[i] = table[centroid_offset(B) + i];
    if (i < L - 1) lds_thr[i] = table[boundary_offset(B) + i];
  }
  uint32_t m[4];
#pragma clang loop unroll(full)
  for (int w = 0; w < 4; ++w) m[w] = a.sign_mask[w];
  float x[D];
  load_row(src, a.dtype, base + (size_t)(t_first + lane - a.tok0) * a.st, x);
  __syncthreads();
  char* part_base = part == 0 ? page : page + 1024 * kb + 256 + (qjl ? 1280 : 0);
  switch (B) {
    case 1: encode_packed<PART, 1>(qjl_s, part_base, qjl, lane, x, m, lds_thr, lds_cent, lds_rows); break;
    case 2: encode_packed<PART, 2>(qjl_s, part_base, qjl, lane, x, m, lds_thr, lds_cent, lds_rows); break;
    case 3: encode_packed<PART, 3>(qjl_s, part_base, qjl, lane, x, m, lds_thr, lds_cent, lds_rows); break;
    case 4: encode_packed<PART, 4>(qjl_s, part_base, qjl, lane, x, m, lds_thr, lds_cent, lds_rows); break;
    case 5: encode_packed<PART, 5>(qjl_s, part_base, qjl, lane, x, m, lds_thr, lds_cent, lds_rows); break;
    case 6: encode_packed<PART, 6>(qjl_s, part_base, qjl, lane, x, m, lds_thr, lds_cent, lds_rows); break;
    case 7: encode_packed<PART, 7>(qjl_s, part_base, qjl, lane, x, m, lds_thr, lds_cent, lds_rows); break;
    default: encode_packed<PART, 8>(qjl_s, part_base, qjl, lane, x, m, lds_thr, lds_cent, lds_rows); break;
  }
}

// ------------------------------------------------------- encode (quad lanes)
// One 256-thread block per (range of pages, KV head, session), keys and values.
// A lane quad holds one token's vector, 32 values per lane: lane e of the quad
// owns coordinates 32c + 8e + k (c = 0..3, k = 0..7), loaded as four 16-byte
// chunks so that a wave's loads cover whole 64-byte row segments.  The
// Walsh-Hadamard transform runs over coordinate bits {0,1,2,5,6} inside the
// lane and over bits {3,4} across the quad (DPP quad permutations).
//
// Codes of u = H D x / ||x|| come from the width's lookup grid in LDS
// (code = count below the bin + [u >= the bin's boundary]), so one code path
// serves every width.  The outer D is applied afterwards as a code flip:
// exact, because the float32 boundary sets are symmetric
// (code(-u) = L-1-code(u) except at exact ties, which lie inside the boundary
// allowance).  Codes go to an LDS byte matrix [token][coordinate]; each lane
// then packs 32 consecutive codes of one stream (exactly b dwords) with a
// streaming accumulator whose flush points are uniform.
constexpr int kRowStride = 144;            // LDS byte-matrix row: 128 codes + pad
constexpr int kEncodeBlock = 256;
constexpr int kEncodePagesPerBlock = 8;

__device__ __forceinline__ float quad_swap(float v, int m) {
  // partner lane = lane ^ m inside the quad; m is a compile-time 1 or 2 after unrolling
  return m == 1 ? __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false))
                : __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

struct Lut {
  float S, O;
  int nb;
};

struct EncodeLane {
  uint32_t hmask[16];   // D sign bits of the lane's value pairs, placed for an fp16x2 xor
  uint32_t fmask[8];    // per code byte: 0xff when the outer D flips that coordinate
  uint32_t dl;          // D bits of the lane's 32 slots
};

// Encodes this lane's quarter of one token into code bytes of its LDS matrix
// row; returns the vector norm (the same in the four lanes of the quad).
template <int DT>
__device__ __forceinline__ float encode_quarter(const void* src, size_t row_off, int e,
                                                const EncodeLane& el, int B, const Lut& lut,
                                                const uint2* ent, uint32_t* mat_row) {
  float x[32];
  if constexpr (DT == TQ_DTYPE_F16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(src) + row_off);
#pragma clang loop unroll(full)
    for (int c = 0; c < 4; ++c) {
      const uint4 w = p[4 * c + e];
      const uint32_t ww[4] = {w.x ^ el.hmask[4 * c], w.y ^ el.hmask[4 * c + 1],
                              w.z ^ el.hmask[4 * c + 2], w.w ^ el.hmask[4 * c + 3]};
#pragma clang loop unroll(full)
      for (int kk = 0; kk < 4; ++kk) {
        const float2 f = __half22float2(*reinterpret_cast<const __half2*>(&ww[kk]));
        x[8 * c + 2 * kk] = f.x;
        x[8 * c + 2 * kk + 1] = f.y;
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + row_off);
#pragma clang loop unroll(full)
    for (int c = 0; c < 4; ++c) {
      const float4 f0 = p[2 * (4 * c + e)], f1 = p[2 * (4 * c + e) + 1];
      const float v[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma clang loop unroll(full)
      for (int k = 0; k < 8; ++k) x[8 * c + k] = flip_if(v[k], (el.dl >> (8 * c + k)) & 1u);
    }
  }
  float ss = 0.f;
#pragma clang loop unroll(full)
  for (int s = 0; s < 32; ++s) ss = fmaf(x[s], x[s], ss);
  ss += quad_swap(ss, 1);
  ss += quad_swap(ss, 2);
  // in-lane butterflies over slot bits 0..4 (coordinate bits 0,1,2,5,6)
#pragma clang loop unroll(full)
  for (int h = 1; h < 32; h <<= 1)
#pragma clang loop unroll(full)
    for (int s = 0; s < 32; ++s)
      if (!(s & h)) {
        const float a0 = x[s], b0 = x[s + h];
        x[s] = a0 + b0;
        x[s + h] = a0 - b0;
      }
  // across the quad: coordinate bits 3 (lane bit 0) and 4 (lane bit 1)
#pragma clang loop unroll(full)
  for (int m = 1; m <= 2; m <<= 1) {
    const float sg = (e & m) ? -1.f : 1.f;
#pragma clang loop unroll(full)
    for (int s = 0; s < 32; ++s) x[s] = fmaf(x[s], sg, quad_swap(x[s], m));
  }
  const float n = sqrtf(ss);
  const float inv = n > 0.f ? 1.0f / n : 0.f;
  uint32_t cb[8];
#pragma clang loop unroll(full)
  for (int i = 0; i < 8; ++i) cb[i] = 0;
#pragma clang loop unroll(full)
  for (int s = 0; s < 32; ++s) {
    const float u = x[s] * inv;
    const int bin = min(max((int)fmaf(u, lut.S, lut.O), 0), lut.nb - 1);
    const uint2 en = ent[bin];
    const uint32_t c = en.x + (u >= __uint_as_float(en.y) ? 1u : 0u);
    cb[s >> 2] |= c << (8 * (s & 3));
  }
  const uint32_t flip = ((1u << B) - 1u) * 0x01010101u;
  // chunk c holds coordinates 32c + 8e .. +7: row bytes 32c + 8e
#pragma clang loop unroll(full)
  for (int c = 0; c < 4; ++c) {
    const uint2 v = make_uint2(cb[2 * c] ^ (el.fmask[2 * c] & flip), cb[2 * c + 1] ^ (el.fmask[2 * c + 1] & flip));
    *reinterpret_cast<uint2*>(reinterpret_cast<char*>(mat_row) + 32 * c + 8 * e) = v;
  }
  return n;
}

// Writes dwords [e*B, e*B + B) of stream s of a code block from its codes
// 32e..32e+31 (bytes of c8), LSB-first.
__device__ __forceinline__ void store_stream_part(int B, char* blk, int s, int e, const uint32_t (&c8)[8]) {
  uint64_t acc = 0;
  int nb = 0, d = e * B;
#pragma clang loop unroll(full)
  for (int n = 0; n < 32; ++n) {
    acc |= (uint64_t)((c8[n >> 2] >> (8 * (n & 3))) & 0xffu) << nb;
    nb += B;
    if (nb >= 32) {
      reinterpret_cast<uint32_t*>(blk + ((d >> 2) * 64 + s) * 16)[d & 3] = (uint32_t)acc;
      acc >>= 32;
      nb -= 32;
      ++d;
    }
  }
}

template <int DT>
__global__ __launch_bounds__(kEncodeBlock) void encode_pages_kernel(EncodeArgs a,
                                                                    const uint64_t* __restrict__ pages) {
  __shared__ uint2 entk[kLutMaxBins], entv[kLutMaxBins];
  __shared__ uint32_t matk[PT * kRowStride / 4], matv[PT * kRowStride / 4];
  __shared__ float normk[PT], normv[PT];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = lane & 3, t = wave * 16 + (lane >> 2);
  const int h = blockIdx.y, b = blockIdx.z;
  const int pg0 = a.page0 + blockIdx.x * kEncodePagesPerBlock;
  const int pg_last = (a.tok0 + a.ntok - 1) / PT;

  EncodeLane el;
  {
    uint32_t m[4];
#pragma clang loop unroll(full)
    for (int w = 0; w < 4; ++w) m[w] = a.sign_mask[w];
    el.dl = 0;
#pragma clang loop unroll(full)
    for (int c = 0; c < 4; ++c) el.dl |= ((m[c] >> (8 * e)) & 0xffu) << (8 * c);
#pragma clang loop unroll(full)
    for (int i = 0; i < 16; ++i)
      el.hmask[i] = (((el.dl >> (2 * i)) & 1u) << 15) | (((el.dl >> (2 * i + 1)) & 1u) << 31);
#pragma clang loop unroll(full)
    for (int i = 0; i < 8; ++i) {
      uint32_t f = 0;
#pragma clang loop unroll(full)
      for (int k = 0; k < 4; ++k) f |= ((el.dl >> (4 * i + k)) & 1u) ? (0xffu << (8 * k)) : 0u;
      el.fmask[i] = f;
    }
  }
  int cur_kb = -1, cur_vb = -1;
  Lut lk{0.f, 0.f, 1}, lv{0.f, 0.f, 1};
  const size_t base = (size_t)b * a.sb + (size_t)h * a.sh;
  const uint64_t* prow = pages + ((size_t)b * a.n_kv_heads + h) * a.max_pages;

  for (int pg = pg0; pg < pg0 + kEncodePagesPerBlock && pg <= pg_last; ++pg) {
    const uint64_t desc = prow[pg];
    if (!(desc & TQ_PAGE_PRESENT)) {
      if (tid == 0) raise_flag(a.err, 2);
      continue;
    }
    const int kb = (int)((desc >> 48) & 15), vb = (int)((desc >> 52) & 15);
    const bool qjl = (desc & TQ_PAGE_QJL) != 0;
    const uint64_t off = desc & TQ_PAGE_OFFSET_MASK;
    const bool bad_fmt = kb == 0 ? (vb != 0 || qjl) : (kb > 8 || vb < 1 || vb > 8);
    if (bad_fmt || off + page_size_dev(kb, vb, qjl) > a.pool_bytes) {
      if (tid == 0) raise_flag(a.err, 4);
      continue;
    }
    char* page = a.pool + off;
    const int t_first = pg * PT;
    const int lo = max(t_first, a.tok0), hi = min(t_first + PT, a.tok0 + a.ntok);
    if (kb == 0) {
      // fp16 page: copy the covered rows of K then V, 16 bytes per thread and pass
      for (int idx = tid; idx < 2 * PT * 16; idx += kEncodeBlock) {
        const int part = idx >> 10, r = (idx >> 4) & 63, c8 = (idx & 15) * 8;
        const int tok = t_first + r;
        if (tok < lo || tok >= hi) continue;
        const void* src = part == 0 ? a.k : a.v;
        const size_t ee = base + (size_t)(tok - a.tok0) * a.st + c8;
        uint4 out;
        if constexpr (DT == TQ_DTYPE_F16) {
          out = *reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(src) + ee);
        } else {
          const float4 f0 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + ee);
          const float4 f1 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + ee + 4);
          __half2 h0 = __floats2half2_rn(f0.x, f0.y), h1 = __floats2half2_rn(f0.z, f0.w);
          __half2 h2 = __floats2half2_rn(f1.x, f1.y), h3 = __floats2half2_rn(f1.z, f1.w);
          out = make_uint4(*reinterpret_cast<uint32_t*>(&h0), *reinterpret_cast<uint32_t*>(&h1),
                           *reinterpret_cast<uint32_t*>(&h2), *reinterpret_cast<uint32_t*>(&h3));
        }
        *reinterpret_cast<uint4*>(page + part * PT * D * 2 + ((size_t)r * D + c8) * 2) = out;
      }
      continue;
    }
    if (lo != t_first || hi != t_first + PT) {
      if (tid == 0) raise_flag(a.err, 1);
      continue;
    }
    // stage the lookup grids when the widths change (uniform branch)
    if (kb != cur_kb || vb != cur_vb) {
      __syncthreads();
      const float* hk = a.k_table + kLutHeaderOffset + 4 * (kb - 1);
      const float* hv = a.v_table + kLutHeaderOffset + 4 * (vb - 1);
      lk = Lut{hk[0], hk[1], min((int)__float_as_uint(hk[2]), kLutMaxBins)};
      lv = Lut{hv[0], hv[1], min((int)__float_as_uint(hv[2]), kLutMaxBins)};
      const uint2* sk = reinterpret_cast<const uint2*>(a.k_table + __float_as_uint(hk[3]));
      const uint2* sv = reinterpret_cast<const uint2*>(a.v_table + __float_as_uint(hv[3]));
      for (int i = tid; i < lk.nb; i += kEncodeBlock) entk[i] = sk[i];
      for (int i = tid; i < lv.nb; i += kEncodeBlock) entv[i] = sv[i];
      cur_kb = kb;
      cur_vb = vb;
      __syncthreads();
    }
    const size_t row_off = base + (size_t)(t_first + t - a.tok0) * a.st;
    uint32_t* rowk = matk + t * (kRowStride / 4);
    uint32_t* rowv = matv + t * (kRowStride / 4);
    // QJL key pages are written by the per-token kernel (codes + sketch)
    const float nk = qjl ? 0.f : encode_quarter<DT>(a.k, row_off, e, el, kb, lk, entk, rowk);
    const float nv = encode_quarter<DT>(a.v, row_off, e, el, vb, lv, entv, rowv);
    if (e == 0) {
      normk[t] = nk;
      normv[t] = nv;
    }
    __syncthreads();
    // pack: lane (stream s, part e) writes dwords [e*B, e*B+B) of stream s
    char* vblk = page + 1024 * kb + 256 + (qjl ? 1280 : 0);
    const int s = t;
    if (!qjl) {
      // K stream s = token s: codes 32e..32e+31 are bytes 32e.. of row s
      const char* r = reinterpret_cast<const char*>(matk + s * (kRowStride / 4)) + 32 * e;
      const uint4 c0 = *reinterpret_cast<const uint4*>(r);
      const uint4 c1 = *reinterpret_cast<const uint4*>(r + 16);
      const uint32_t c8[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      store_stream_part(kb, page, s, e, c8);
    }
    {
      // V stream s = 16q + i: positions 8k + j (k = 4e..4e+3) = token 4k+q, coordinate 8i+j
      const int q = s >> 4, i = s & 15;
      uint32_t c8[8];
#pragma clang loop unroll(full)
      for (int kk = 0; kk < 4; ++kk) {
        const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(matv) +
                                                        (4 * (4 * e + kk) + q) * kRowStride + 8 * i);
        c8[2 * kk] = v.x;
        c8[2 * kk + 1] = v.y;
      }
      store_stream_part(vb, vblk, s, e, c8);
    }
    if (e == 0) {
      if (!qjl) reinterpret_cast<float*>(page + 1024 * kb)[s] = normk[s];
      reinterpret_cast<float*>(vblk + 1024 * vb)[s] = normv[s];
    }
    __syncthreads();
  }
}

// -------------------------------------------------------------- dequantize
struct DequantArgs {
  const uint64_t* pages;
  int n_kv_heads, max_pages;
  const char* pool;
  uint64_t pool_bytes;
  const uint32_t* sign_mask;
  const float* table;
  const float* qjl_s;
  int which, add_qjl, tok0, ntok, page0;
  float* out;
};

// Code n of stream s of a block staged in LDS (word-interleaved layout).
__device__ __forceinline__ uint32_t stream_code(const uint32_t* blk, int b, int s, int n) {
  const int pos = n * b, dw = pos >> 5, sh = pos & 31;
  auto dword = [&](int d) { return blk[((d >> 2) * 64 + s) * 4 + (d & 3)]; };
  uint32_t v = dword(dw) >> sh;
  if (sh + b > 32) v |= dword(dw + 1) << (32 - sh);
  return v & ((1u << b) - 1u);
}

__global__ __launch_bounds__(64) void dequant_kernel(DequantArgs a, const float* __restrict__ qjl_s) {
  __shared__ uint32_t blk[2048];  // up to an 8-bit block (8 KB)
  __shared__ float cent[256];
  const int lane = threadIdx.x;
  const int pg = a.page0 + blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const uint64_t desc = a.pages[((size_t)b * a.n_kv_heads + h) * a.max_pages + pg];
  const int t = pg * PT + lane;
  const bool in_range = t >= a.tok0 && t < a.tok0 + a.ntok;
  float* dst = a.out + (((size_t)b * a.n_kv_heads + h) * a.ntok + (size_t)(t - a.tok0)) * D;
  const int kb = (int)((desc >> 48) & 15), vb = (int)((desc >> 52) & 15);
  const bool qjl = (desc & TQ_PAGE_QJL) != 0;
  const uint64_t off = desc & TQ_PAGE_OFFSET_MASK;
  const bool bad = !(desc & TQ_PAGE_PRESENT) || off + page_size_dev(kb, vb, qjl) > a.pool_bytes ||
                   (kb == 0 && (vb != 0 || qjl)) || kb > 8 || (kb > 0 && (vb < 1 || vb > 8));
  if (bad) {
    if (in_range)
      for (int j = 0; j < D; ++j) dst[j] = __builtin_nanf("");
    return;
  }
  const char* page = a.pool + off;
  if (kb == 0) {
    if (!in_range) return;
    const __half* row = reinterpret_cast<const __half*>(page + a.which * PT * D * 2) + (size_t)lane * D;
    for (int j = 0; j < D; ++j) dst[j] = __half2float(row[j]);
    return;
  }
  const int B = a.which == 0 ? kb : vb;
  const char* blk_src = a.which == 0 ? page : page + 1024 * kb + 256 + (qjl ? 1280 : 0);
  const float norm = reinterpret_cast<const float*>(blk_src + 1024 * B)[lane];
  for (int i = lane; i < 256 * B; i += 64) blk[i] = reinterpret_cast<const uint32_t*>(blk_src)[i];
  for (int i = lane; i < (1 << B); i += 64) cent[i] = a.table[centroid_offset(B) + i];
  __syncthreads();
  if (!in_range) return;
  uint32_t m[4];
  for (int w = 0; w < 4; ++w) m[w] = a.sign_mask[w];
  float x[D];
  if (a.which == 0) {
#pragma clang loop unroll(full)
    for (int j = 0; j < D; ++j) x[j] = cent[stream_code(blk, B, lane, j)];
  } else {
    const int q = lane & 3, k = lane >> 2;
#pragma clang loop unroll(full)
    for (int j = 0; j < D; ++j) x[j] = cent[stream_code(blk, B, 16 * q + (j >> 3), 8 * k + (j & 7))];
  }
  // xhat = (n / sqrt(d)) R c = (n / d) D H D c
#pragma clang loop unroll(full)
  for (int j = 0; j < D; ++j) x[j] = flip_if(x[j], dsign(m, j));
  fwht128(x);
  const float sc = norm * (1.0f / D);
#pragma clang loop unroll(full)
  for (int j = 0; j < D; ++j) x[j] = flip_if(x[j], dsign(m, j)) * sc;
  if (a.which == 0 && qjl && a.add_qjl && qjl_s) {
    const char* qb = page + 1024 * kb + 256;
    const uint4 zw4 = reinterpret_cast<const uint4*>(qb)[lane];
    const uint32_t zw[4] = {zw4.x, zw4.y, zw4.z, zw4.w};
    const float gamma = reinterpret_cast<const float*>(qb + 1024)[lane];
    const float coef = kSqrtHalfPi / TQ_JL_DIM * gamma;
    for (int i = 0; i < TQ_JL_DIM; ++i) {
      const float zi = ((zw[i >> 5] >> (i & 31)) & 1u) ? coef : -coef;
      const float* srow = qjl_s + (size_t)i * D;
#pragma clang loop unroll(full)
      for (int j = 0; j < D; ++j) x[j] = fmaf(zi, srow[j], x[j]);
    }
  }
  float4* d4 = reinterpret_cast<float4*>(dst);
#pragma clang loop unroll(full)
  for (int c = 0; c < D / 4; ++c) d4[c] = make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
}

// ------------------------------------------------------------------ decode
struct DecodeArgs {
  const void* q;
  int q_dtype;
  int64_t q_sb, q_sh;
  int n_q_heads, group;
  float scale2;  // softmax scale * log2(e)
  const int32_t* n_tokens;
  int n_sessions, n_kv_heads, max_pages;
  const char* pool;
  uint64_t pool_bytes;
  const uint32_t* sign_mask;
  const float* k_table;
  const float* v_table;
  const float* qjl_s;
  int n_splits, pages_per_split;
  float* wsq;   // [B][H_q][384]: rotated q, plain q, S q (pre-scaled)
  float* wsp;   // [B][H_q][n_splits][kPartialFloats]: m, l, -, -, acc[128]
  float* out;
};

// (1) query prep: one 128-thread block per (session, query head).
__global__ __launch_bounds__(128) void qprep_kernel(DecodeArgs a) {
  __shared__ float buf[D];
  __shared__ float qs[D];
  const int j = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / a.n_q_heads, h = row - b * a.n_q_heads;
  const float qj = load_elem(a.q, a.q_dtype, (size_t)b * a.q_sb + (size_t)h * a.q_sh + j);
  const uint32_t neg = (a.sign_mask[j >> 5] >> (j & 31)) & 1u;
  qs[j] = qj;
  buf[j] = flip_if(qj, neg);
  __syncthreads();
#pragma clang loop unroll(full)
  for (int hh = 1; hh < D; hh <<= 1) {
    const float mine = buf[j], other = buf[j ^ hh];
    __syncthreads();
    buf[j] = (j & hh) ? other - mine : mine + other;
    __syncthreads();
  }
  // Layout per (session, KV head): three sections of 128 x G floats (rotated q,
  // plain q, S q), each ordered [coordinate / 4][query head in group][coordinate % 4]
  // so that one 16-dword scalar load brings 4 coordinates of 4 heads.
  const int G = a.group, g = h / G, hg = h - g * G;
  float* w = a.wsq + ((size_t)b * a.n_kv_heads + g) * kQPrepFloats * G;
  const size_t slot = ((size_t)(j >> 2) * G + hg) * 4 + (j & 3);
  // R q = D H D q / sqrt(d); packed-page scores use (R q) * scale2 / sqrt(d).
  w[slot] = flip_if(buf[j], neg) * (a.scale2 * (1.0f / D));
  w[D * G + slot] = qj * a.scale2;
  if (a.qjl_s) {
    const float* srow = a.qjl_s + (size_t)j * D;
    float p = 0.f;
    for (int i = 0; i < D; ++i) p = fmaf(srow[i], qs[i], p);
    w[2 * D * G + slot] = p * (a.scale2 * kSqrtHalfPi / TQ_JL_DIM);
  } else {
    w[2 * D * G + slot] = 0.f;
  }
}

// Per-workgroup LDS of the split kernel.
template <int G>
struct SplitLds {
  float2 kpair[340];          // pair tables for bits 1..4 (4 + 16 + 64 + 256 entries)
  float2 vpair[340];
  float kcent[512];           // centroid lists for every bit width (table layout)
  float vcent[512];
  float w[kDecodeWaves][PT * G];           // softmax weights of the current page
  float red[kDecodeWaves][G * D];          // workgroup reduction
  float stat[kDecodeWaves][2][G];          // m, l per wave
};

__device__ __forceinline__ int pair_offset(int b) {
  return b == 1 ? 0 : b == 2 ? 4 : b == 3 ? 20 : 84;
}

// Key scores of one packed page, lane = token: s[h] = sum_j qr[h][j] c[code_j].
// Query values are wave-uniform scalar loads; they share the LGKM counter with
// the LDS codebook lookups and return out of order, so the loop is pipelined by
// hand: for chunk n the first FMA waits for chunk n's data only, then chunk
// n+1's scalar loads and lookups are issued, then the rest of chunk n runs.
template <int B, int G>
__device__ __forceinline__ void key_scores(const char* blk, int lane, const float* __restrict__ qr,
                                           const float2* pair, const float* cent, float (&s)[G]) {
  constexpr int CH = 4;                       // coordinates per chunk
  uint32_t sw[4 * B];
  const uint4* src = reinterpret_cast<const uint4*>(blk);
#pragma clang loop unroll(full)
  for (int w = 0; w < B; ++w) {
    const uint4 v = src[w * 64 + lane];
    sw[4 * w] = v.x; sw[4 * w + 1] = v.y; sw[4 * w + 2] = v.z; sw[4 * w + 3] = v.w;
  }
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) s[h] = 0.f;
  float qa[G][CH], qb[G][CH], ca[CH], cb[CH];
  auto fetch = [&](int n, float (&qd)[G][CH], float (&cd)[CH]) {
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h)
#pragma clang loop unroll(full)
      for (int e = 0; e < CH; ++e) qd[h][e] = qr[(n * G + h) * CH + e];
    if constexpr (B <= 4) {
      const float2* pt = pair + pair_offset(B);
#pragma clang loop unroll(full)
      for (int e = 0; e < CH; e += 2) {
        const float2 c = pt[bits_at(sw, (n * CH + e) * B, 2 * B)];
        cd[e] = c.x;
        cd[e + 1] = c.y;
      }
    } else {
      const float* ct = cent + centroid_offset(B);
#pragma clang loop unroll(full)
      for (int e = 0; e < CH; ++e) cd[e] = ct[bits_at(sw, (n * CH + e) * B, B)];
    }
  };
  auto fmas = [&](const float (&qd)[G][CH], const float (&cd)[CH], int e0, int e1) {
#pragma clang loop unroll(full)
    for (int e = e0; e < e1; ++e)
#pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h) s[h] = fmaf(qd[h][e], cd[e], s[h]);
  };
  fetch(0, qa, ca);
#pragma clang loop unroll(full)
  for (int n = 0; n < D / CH; n += 2) {
    fmas(qa, ca, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
    fetch(n + 1, qb, cb);
    __builtin_amdgcn_sched_barrier(0);
    fmas(qa, ca, 1, CH);
    fmas(qb, cb, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (n + 2 < D / CH) fetch(n + 2, qa, ca);
    __builtin_amdgcn_sched_barrier(0);
    fmas(qb, cb, 1, CH);
  }
}

// Key scores of an fp16 page, lane = token, with the unrotated query.
template <int G>
__device__ __forceinline__ void key_scores_fp16(const char* page, int lane, const float* __restrict__ qo,
                                                float (&s)[G]) {
  const __half* krow = reinterpret_cast<const __half*>(page) + (size_t)lane * D;
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma clang loop unroll(full)
  for (int c = 0; c < D / 8; ++c) {
    const uint4 kv = reinterpret_cast<const uint4*>(krow)[c];
    const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma clang loop unroll(full)
    for (int e = 0; e < 4; ++e) {
      const float2 f = __half22float2(*reinterpret_cast<const __half2*>(&kw[e]));
      const int j = 8 * c + 2 * e;
#pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h) {
        s[h] = fmaf(qo[((j >> 2) * G + h) * 4 + (j & 3)], f.x, s[h]);
        s[h] = fmaf(qo[((j >> 2) * G + h) * 4 + (j & 3) + 1], f.y, s[h]);
      }
    }
  }
}

// QJL term: sum_i qs[h][i] (2 z_i - 1) for lane = token.
template <int G>
__device__ __forceinline__ void qjl_scores(const char* qb, int lane, const float* __restrict__ qsv,
                                           float (&t)[G]) {
  const uint4 z4 = reinterpret_cast<const uint4*>(qb)[lane];
  const uint32_t zw[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) t[h] = 0.f;
#pragma clang loop unroll(full)
  for (int i = 0; i < TQ_JL_DIM; ++i) {
    const float z = ((zw[i >> 5] >> (i & 31)) & 1u) ? 1.f : -1.f;
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h) t[h] = fmaf(qsv[((i >> 2) * G + h) * 4 + (i & 3)], z, t[h]);
  }
}

// Value accumulation of one packed page: lane (q, i) owns coordinates
// 8i..8i+7 of tokens 4k+q; acc[h][e] += w[token][h] c[code].
template <int B, int G>
__device__ __forceinline__ void value_accum(const char* blk, int lane, const float* wv,
                                            const float2* pair, const float* cent, float (&acc)[G][8]) {
  uint32_t sw[4 * B];
  const uint4* src = reinterpret_cast<const uint4*>(blk);
#pragma clang loop unroll(full)
  for (int w = 0; w < B; ++w) {
    const uint4 v = src[w * 64 + lane];
    sw[4 * w] = v.x; sw[4 * w + 1] = v.y; sw[4 * w + 2] = v.z; sw[4 * w + 3] = v.w;
  }
  const int q = lane >> 4;
#pragma clang loop unroll(full)
  for (int k = 0; k < 16; ++k) {
    float wt[G];
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h) wt[h] = wv[(4 * k + q) * G + h];
    if constexpr (B <= 4) {
      const float2* pt = pair + pair_offset(B);
#pragma clang loop unroll(full)
      for (int e = 0; e < 8; e += 2) {
        const float2 c = pt[bits_at(sw, (8 * k + e) * B, 2 * B)];
#pragma clang loop unroll(full)
        for (int h = 0; h < G; ++h) {
          acc[h][e] = fmaf(wt[h], c.x, acc[h][e]);
          acc[h][e + 1] = fmaf(wt[h], c.y, acc[h][e + 1]);
        }
      }
    } else {
      const float* ct = cent + centroid_offset(B);
#pragma clang loop unroll(full)
      for (int e = 0; e < 8; ++e) {
        const float c = ct[bits_at(sw, (8 * k + e) * B, B)];
#pragma clang loop unroll(full)
        for (int h = 0; h < G; ++h) acc[h][e] = fmaf(wt[h], c, acc[h][e]);
      }
    }
  }
}

// Value accumulation of an fp16 page into the rotated-domain sums: each token's
// row is rotated with the unnormalised D H D (the 16 lanes of a quarter hold
// its 128 values, 8 each), so that D H D acc / d at the end returns sum p v.
template <int G>
__device__ __forceinline__ void value_accum_fp16(const char* page, int lane, const float* wv,
                                                 const uint32_t (&dm)[8], float (&acc)[G][8]) {
  const __half* vbase = reinterpret_cast<const __half*>(page + PT * D * 2);
  const int q = lane >> 4, i = lane & 15;
  for (int k = 0; k < 16; ++k) {
    const int t = 4 * k + q;
    const uint4 vv = reinterpret_cast<const uint4*>(vbase + (size_t)t * D + 8 * i)[0];
    const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
    float x[8];
#pragma clang loop unroll(full)
    for (int e = 0; e < 4; ++e) {
      const float2 f = __half22float2(*reinterpret_cast<const __half2*>(&vw[e]));
      x[2 * e] = flip_if(f.x, dm[2 * e]);
      x[2 * e + 1] = flip_if(f.y, dm[2 * e + 1]);
    }
    // coordinate bits 0..2: within the lane
#pragma clang loop unroll(full)
    for (int hh = 1; hh < 8; hh <<= 1)
#pragma clang loop unroll(full)
      for (int e = 0; e < 8; ++e)
        if (!(e & hh)) {
          const float a0 = x[e], b0 = x[e + hh];
          x[e] = a0 + b0;
          x[e + hh] = a0 - b0;
        }
    // coordinate bits 3..6: across the 16 lanes of the quarter
#pragma clang loop unroll(full)
    for (int m = 1; m < 16; m <<= 1) {
      const float sg = (i & m) ? -1.f : 1.f;
#pragma clang loop unroll(full)
      for (int e = 0; e < 8; ++e) {
        const float other = __shfl_xor(x[e], m, 64);
        x[e] = fmaf(sg, x[e], other);
      }
    }
    float wt[G];
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h) wt[h] = wv[t * G + h];
#pragma clang loop unroll(full)
    for (int e = 0; e < 8; ++e) {
      const float y = flip_if(x[e], dm[e]);
#pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h) acc[h][e] = fmaf(wt[h], y, acc[h][e]);
    }
  }
}

// Online-softmax update of one page for G heads.  s: log2-domain scores of
// this lane's token (-inf when masked); on return s holds p = 2^(s - m) and
// alpha the rescale of the running sums.
template <int G>
__device__ __forceinline__ void softmax_update(float (&s)[G], float (&m)[G], float (&l)[G],
                                               float (&alpha)[G]) {
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) {
    const float mx = wave_max(s[h]);
    const float mn = fmaxf(m[h], mx);
    if (mn == -INFINITY) {
      alpha[h] = 1.f;
      s[h] = 0.f;
    } else {
      alpha[h] = exp2f(m[h] - mn);
      s[h] = exp2f(s[h] - mn);
    }
    m[h] = mn;
    l[h] = fmaf(l[h], alpha[h], s[h]);
  }
}

template <int G>
__global__ __launch_bounds__(64 * kDecodeWaves) void split_kernel(DecodeArgs a,
                                                                  const float* __restrict__ wsq,
                                                                  const uint64_t* __restrict__ pages,
                                                                  float* __restrict__ wsp) {
  __shared__ SplitLds<G> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;

  // Stage codebooks: pair tables for 1..4 bits and all centroid lists.
  for (int i = tid; i < 510; i += blockDim.x) {
    sm.kcent[i] = a.k_table[i];
    sm.vcent[i] = a.v_table[i];
  }
  __syncthreads();
  for (int i = tid; i < 340; i += blockDim.x) {
    const int bb = i < 4 ? 1 : i < 20 ? 2 : i < 84 ? 3 : 4;
    const int idx = i - pair_offset(bb), L = 1 << bb;
    const int lo = idx & (L - 1), hi = idx >> bb;
    sm.kpair[i] = make_float2(sm.kcent[centroid_offset(bb) + lo], sm.kcent[centroid_offset(bb) + hi]);
    sm.vpair[i] = make_float2(sm.vcent[centroid_offset(bb) + lo], sm.vcent[centroid_offset(bb) + hi]);
  }
  __syncthreads();

  const int ntok = max(0, a.n_tokens[b]);
  const int npages = min(a.max_pages, (ntok + PT - 1) / PT);   // never past the table row
  const int p_begin = split * a.pages_per_split;
  const int p_end = min(npages, p_begin + a.pages_per_split);
  const uint64_t* ptab = pages + ((size_t)b * a.n_kv_heads + hkv) * a.max_pages;
  const int hq0 = hkv * G;
  const float* __restrict__ qrow = wsq + ((size_t)b * a.n_kv_heads + hkv) * kQPrepFloats * G;

  float m[G], l[G], acc[G][8];
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma clang loop unroll(full)
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  float* wv = sm.w[wave];
  const int q4 = lane >> 4, i16 = lane & 15;

  for (int p = p_begin + wave; p < p_end; p += kDecodeWaves) {
    const uint64_t desc = ptab[p];
    const int kb = (int)((desc >> 48) & 15), vb = (int)((desc >> 52) & 15);
    const bool qjl = (desc & TQ_PAGE_QJL) != 0;
    const uint64_t off = desc & TQ_PAGE_OFFSET_MASK;
    if (!(desc & TQ_PAGE_PRESENT) || off + page_size_dev(kb, vb, qjl) > a.pool_bytes) continue;
    if (kb == 0 ? (vb != 0 || qjl) : (kb > 8 || vb < 1 || vb > 8)) continue;
    if (qjl && a.qjl_s == nullptr) continue;
    const char* page = a.pool + off;
    const int valid = min(PT, ntok - p * PT);
    float s[G], alpha[G];
    const char* vblk = page + 1024 * kb + 256;
    float nv = 1.f;
    if (kb == 0) {
      key_scores_fp16<G>(page, lane, qrow + D * G, s);
    } else {
      switch (kb) {
        case 1: key_scores<1, G>(page, lane, qrow, sm.kpair, sm.kcent, s); break;
        case 2: key_scores<2, G>(page, lane, qrow, sm.kpair, sm.kcent, s); break;
        case 3: key_scores<3, G>(page, lane, qrow, sm.kpair, sm.kcent, s); break;
        case 4: key_scores<4, G>(page, lane, qrow, sm.kpair, sm.kcent, s); break;
        case 5: key_scores<5, G>(page, lane, qrow, sm.kpair, sm.kcent, s); break;
        case 6: key_scores<6, G>(page, lane, qrow, sm.kpair, sm.kcent, s); break;
        case 7: key_scores<7, G>(page, lane, qrow, sm.kpair, sm.kcent, s); break;
        default: key_scores<8, G>(page, lane, qrow, sm.kpair, sm.kcent, s); break;
      }
      const float nk = reinterpret_cast<const float*>(page + 1024 * kb)[lane];
#pragma clang loop unroll(full)
      for (int h = 0; h < G; ++h) s[h] *= nk;
      if (qjl) {
        float t[G];
        qjl_scores<G>(vblk, lane, qrow + 2 * D * G, t);
        const float gamma = reinterpret_cast<const float*>(vblk + 1024)[lane];
#pragma clang loop unroll(full)
        for (int h = 0; h < G; ++h) s[h] = fmaf(gamma, t[h], s[h]);
        vblk += 1280;
      }
      nv = reinterpret_cast<const float*>(vblk + 1024 * vb)[lane];
    }
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h)
      if (lane >= valid) s[h] = -INFINITY;
    softmax_update<G>(s, m, l, alpha);
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h) {
#pragma clang loop unroll(full)
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha[h];
      wv[lane * G + h] = s[h] * nv;
    }
    wave_lds_sync();
    if (kb == 0) {
      uint32_t dm[8];
      const uint32_t dword = a.sign_mask[i16 >> 2];
#pragma clang loop unroll(full)
      for (int e = 0; e < 8; ++e) dm[e] = (dword >> (8 * (i16 & 3) + e)) & 1u;
      value_accum_fp16<G>(page, lane, wv, dm, acc);
    } else {
      switch (vb) {
        case 1: value_accum<1, G>(vblk, lane, wv, sm.vpair, sm.vcent, acc); break;
        case 2: value_accum<2, G>(vblk, lane, wv, sm.vpair, sm.vcent, acc); break;
        case 3: value_accum<3, G>(vblk, lane, wv, sm.vpair, sm.vcent, acc); break;
        case 4: value_accum<4, G>(vblk, lane, wv, sm.vpair, sm.vcent, acc); break;
        case 5: value_accum<5, G>(vblk, lane, wv, sm.vpair, sm.vcent, acc); break;
        case 6: value_accum<6, G>(vblk, lane, wv, sm.vpair, sm.vcent, acc); break;
        case 7: value_accum<7, G>(vblk, lane, wv, sm.vpair, sm.vcent, acc); break;
        default: value_accum<8, G>(vblk, lane, wv, sm.vpair, sm.vcent, acc); break;
      }
    }
    wave_lds_sync();
  }

  // ---- workgroup reduction: waves, then token quarters.
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) l[h] = wave_sum(l[h]);
  if (lane == 0) {
#pragma clang loop unroll(full)
    for (int h = 0; h < G; ++h) {
      sm.stat[wave][0][h] = m[h];
      sm.stat[wave][1][h] = l[h];
    }
  }
  __syncthreads();
  float M[G];
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) {
    M[h] = -INFINITY;
    for (int w = 0; w < kDecodeWaves; ++w) M[h] = fmaxf(M[h], sm.stat[w][0][h]);
  }
  float* part = wsp + (((size_t)b * a.n_q_heads + hq0) * a.n_splits + split) * kPartialFloats;
  const size_t head_stride = (size_t)a.n_splits * kPartialFloats;
  if (tid < G) {
    const int h = tid;
    float lsum = 0.f;
    for (int w = 0; w < kDecodeWaves; ++w)
      if (sm.stat[w][0][h] != -INFINITY) lsum += sm.stat[w][1][h] * exp2f(sm.stat[w][0][h] - M[h]);
    float* ph = part + h * head_stride;
    ph[0] = M[h];
    ph[1] = lsum;
  }
#pragma clang loop unroll(full)
  for (int h = 0; h < G; ++h) {
    const float f = m[h] == -INFINITY ? 0.f : exp2f(m[h] - M[h]);
#pragma clang loop unroll(full)
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e] * f;
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (q4 == 0) sm.red[wave][h * D + 8 * i16 + e] = v;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += blockDim.x) {
    float v = 0.f;
#pragma clang loop unroll(full)
    for (int w = 0; w < kDecodeWaves; ++w) v += sm.red[w][idx];
    const int h = idx / D, j = idx - h * D;
    part[h * head_stride + 4 + j] = v;
  }
}

// (3) combine: one 128-thread block per (session, query head).  The split
// weights 2^(m_s - M) are computed once into LDS; the value sums then stream
// with independent loads.
__global__ __launch_bounds__(128) void combine_kernel(DecodeArgs a) {
  __shared__ float buf[D];
  __shared__ float wgt[1024];
  __shared__ float red[2];
  const int j = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / a.n_q_heads;
  const int ns = a.n_splits;
  const float* part = a.wsp + (size_t)row * ns * kPartialFloats;
  float* o = a.out + (size_t)row * D;
  // global max over splits
  float mloc = -INFINITY;
  for (int s = j; s < ns; s += D) mloc = fmaxf(mloc, part[(size_t)s * kPartialFloats]);
  mloc = wave_max(mloc);
  if ((j & 63) == 0) red[j >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  __syncthreads();
  if (M == -INFINITY || a.n_tokens[b] <= 0) {
    o[j] = 0.f;
    return;
  }
  float lloc = 0.f;
  for (int s = j; s < ns; s += D) {
    const float ms = part[(size_t)s * kPartialFloats];
    const float f = ms == -INFINITY ? 0.f : exp2f(ms - M);
    wgt[s] = f;
    lloc = fmaf(part[(size_t)s * kPartialFloats + 1], f, lloc);
  }
  lloc = wave_sum(lloc);
  if ((j & 63) == 0) red[j >> 6] = lloc;
  __syncthreads();
  const float L = red[0] + red[1];
  float ar0 = 0.f, ar1 = 0.f, ar2 = 0.f, ar3 = 0.f;
  int s = 0;
  for (; s + 4 <= ns; s += 4) {
    ar0 = fmaf(part[(size_t)s * kPartialFloats + 4 + j], wgt[s], ar0);
    ar1 = fmaf(part[(size_t)(s + 1) * kPartialFloats + 4 + j], wgt[s + 1], ar1);
    ar2 = fmaf(part[(size_t)(s + 2) * kPartialFloats + 4 + j], wgt[s + 2], ar2);
    ar3 = fmaf(part[(size_t)(s + 3) * kPartialFloats + 4 + j], wgt[s + 3], ar3);
  }
  for (; s < ns; ++s) ar0 = fmaf(part[(size_t)s * kPartialFloats + 4 + j], wgt[s], ar0);
  const float ar = (ar0 + ar1) + (ar2 + ar3);
  const uint32_t neg = (a.sign_mask[j >> 5] >> (j & 31)) & 1u;
  buf[j] = flip_if(ar, neg);
  __syncthreads();
#pragma clang loop unroll(full)
  for (int hh = 1; hh < D; hh <<= 1) {
    const float mine = buf[j], other = buf[j ^ hh];
    __syncthreads();
    buf[j] = (j & hh) ? other - mine : mine + other;
    __syncthreads();
  }
  // o = D H D acc / d / L
  o[j] = flip_if(buf[j], neg) * (1.0f / D) / L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace
}  // namespace tq

using namespace tq;

extern "C" {

int tq_encode_kv(const tq_layer* layer, const tq_cache* cache, const tq_kv_input* in, void* stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (!in || !in->k || !in->v) return fail(TQ_ERR_INVALID_ARG, "null input");
  if (in->dtype != TQ_DTYPE_F16 && in->dtype != TQ_DTYPE_F32)
    return fail(TQ_ERR_INVALID_ARG, "unknown input dtype %d", in->dtype);
  if (in->ntok < 1 || in->tok0 < 0) return fail(TQ_ERR_INVALID_ARG, "bad token range");
  if (in->tok0 % TQ_PAGE_TOKENS) return fail(TQ_ERR_INVALID_ARG, "tok0 must be a multiple of 64");
  if ((int64_t)in->tok0 + in->ntok > (int64_t)cache->max_pages * TQ_PAGE_TOKENS)
    return fail(TQ_ERR_INVALID_ARG, "token range past the page table");
  if (in->stride_b < 0 || in->stride_h < 0 || in->stride_t < 0)
    return fail(TQ_ERR_INVALID_ARG, "negative stride");
  const int esz = in->dtype == TQ_DTYPE_F16 ? 2 : 4;
  if (!aligned16(in->k) || !aligned16(in->v) || (in->stride_b * esz) % 16 ||
      (in->stride_h * esz) % 16 || (in->stride_t * esz) % 16)
    return fail(TQ_ERR_ALIGNMENT, "input rows must be 16-byte aligned");
  if (((uintptr_t)in->error_flags & 3) != 0) return fail(TQ_ERR_ALIGNMENT, "error_flags misaligned");
  EncodeArgs a;
  a.k = in->k;
  a.v = in->v;
  a.dtype = in->dtype;
  a.tok0 = in->tok0;
  a.ntok = in->ntok;
  a.page0 = in->tok0 / TQ_PAGE_TOKENS;
  a.sb = in->stride_b;
  a.sh = in->stride_h;
  a.st = in->stride_t;
  a.err = in->error_flags;
  a.pages = cache->pages;
  a.n_kv_heads = cache->n_kv_heads;
  a.max_pages = cache->max_pages;
  a.pool = reinterpret_cast<char*>(cache->pool);
  a.pool_bytes = cache->pool_bytes;
  a.sign_mask = layer->sign_mask;
  a.k_table = layer->k_table;
  a.v_table = layer->v_table;
  a.qjl_s = layer->qjl_s;
  const int last_page = (in->tok0 + in->ntok - 1) / TQ_PAGE_TOKENS;
  const int n_pages = last_page - a.page0 + 1;
  dim3 grid((n_pages + kEncodePagesPerBlock - 1) / kEncodePagesPerBlock, cache->n_kv_heads,
            cache->n_sessions);
  if (a.dtype == TQ_DTYPE_F16)
    hipLaunchKernelGGL(encode_pages_kernel<TQ_DTYPE_F16>, grid, dim3(kEncodeBlock), 0,
                       (hipStream_t)stream, a, cache->pages);
  else
    hipLaunchKernelGGL(encode_pages_kernel<TQ_DTYPE_F32>, grid, dim3(kEncodeBlock), 0,
                       (hipStream_t)stream, a, cache->pages);
  int st2 = launch_status("encode");
  if (st2) return st2;
  if (layer->qjl_s) {
    // keys of QJL pages: codes, norm and sign sketch, one wavefront per page
    dim3 qgrid(n_pages, cache->n_kv_heads, cache->n_sessions);
    hipLaunchKernelGGL(encode_kernel<0>, qgrid, dim3(64), 0, (hipStream_t)stream, a, cache->pages,
                       layer->qjl_s);
    st2 = launch_status("encode QJL keys");
  }
  return st2;
}

int tq_dequantize(const tq_layer* layer, const tq_cache* cache, int which, int add_qjl, int tok0,
                  int ntok, float* out, void* stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (which != 0 && which != 1) return fail(TQ_ERR_INVALID_ARG, "which must be 0 (K) or 1 (V)");
  if (!out) return fail(TQ_ERR_INVALID_ARG, "null output");
  if (!aligned16(out)) return fail(TQ_ERR_ALIGNMENT, "output must be 16-byte aligned");
  if (tok0 < 0 || ntok < 1 || (int64_t)tok0 + ntok > (int64_t)cache->max_pages * TQ_PAGE_TOKENS)
    return fail(TQ_ERR_INVALID_ARG, "bad token range");
  DequantArgs a;
  a.pages = cache->pages;
  a.n_kv_heads = cache->n_kv_heads;
  a.max_pages = cache->max_pages;
  a.pool = reinterpret_cast<const char*>(cache->pool);
  a.pool_bytes = cache->pool_bytes;
  a.sign_mask = layer->sign_mask;
  a.table = which == 0 ? layer->k_table : layer->v_table;
  a.qjl_s = layer->qjl_s;
  a.which = which;
  a.add_qjl = add_qjl;
  a.tok0 = tok0;
  a.ntok = ntok;
  a.page0 = tok0 / TQ_PAGE_TOKENS;
  a.out = out;
  const int last_page = (tok0 + ntok - 1) / TQ_PAGE_TOKENS;
  dim3 grid(last_page - a.page0 + 1, cache->n_kv_heads, cache->n_sessions);
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(64), 0, (hipStream_t)stream, a, layer->qjl_s);
  return launch_status("dequantize");
}

int tq_decode_attention(const tq_layer* layer, const tq_cache* cache, const tq_query* query,
                        float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_layer(layer);
  if (st) return st;
  if ((st = check_cache(cache))) return st;
  if (!query || !query->q) return fail(TQ_ERR_INVALID_ARG, "null query");
  if (query->dtype != TQ_DTYPE_F16 && query->dtype != TQ_DTYPE_F32)
    return fail(TQ_ERR_INVALID_ARG, "unknown query dtype %d", query->dtype);
  if (query->n_q_heads <= 0 || query->n_q_heads % cache->n_kv_heads)
    return fail(TQ_ERR_INVALID_ARG, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)",
                query->n_q_heads, cache->n_kv_heads);
  const int G = query->n_q_heads / cache->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(TQ_ERR_UNSUPPORTED, "GQA group %d not in {1, 2, 4, 8}", G);
  if (query->stride_b < 0 || query->stride_h < 0) return fail(TQ_ERR_INVALID_ARG, "negative stride");
  if (!out || !workspace) return fail(TQ_ERR_INVALID_ARG, "null output or workspace");
  if (!aligned16(out) || !aligned16(workspace)) return fail(TQ_ERR_ALIGNMENT, "out/workspace misaligned");
  if (!(query->softmax_scale >= 0.f) || isinf(query->softmax_scale))
    return fail(TQ_ERR_INVALID_ARG, "bad softmax scale");
  const SplitPlan sp = split_plan(cache->n_sessions, cache->n_kv_heads, cache->max_pages);
  if (sp.n_splits > 1024) return fail(TQ_ERR_UNSUPPORTED, "%d splits exceed 1024", sp.n_splits);
  const size_t need = decode_workspace_bytes(cache->n_sessions, query->n_q_heads, sp.n_splits);
  if (workspace_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  DecodeArgs a;
  a.q = query->q;
  a.q_dtype = query->dtype;
  a.q_sb = query->stride_b;
  a.q_sh = query->stride_h;
  a.n_q_heads = query->n_q_heads;
  a.group = G;
  const float scale = query->softmax_scale > 0.f ? query->softmax_scale : 0.08838834764831845f;
  a.scale2 = scale * kLog2e;
  a.n_tokens = cache->n_tokens;
  a.n_sessions = cache->n_sessions;
  a.n_kv_heads = cache->n_kv_heads;
  a.max_pages = cache->max_pages;
  a.pool = reinterpret_cast<const char*>(cache->pool);
  a.pool_bytes = cache->pool_bytes;
  a.sign_mask = layer->sign_mask;
  a.k_table = layer->k_table;
  a.v_table = layer->v_table;
  a.qjl_s = layer->qjl_s;
  a.n_splits = sp.n_splits;
  a.pages_per_split = sp.pages_per_split;
  a.wsq = reinterpret_cast<float*>(workspace);
  a.wsp = a.wsq + (size_t)cache->n_sessions * query->n_q_heads * kQPrepFloats;
  a.out = out;
  hipStream_t s = (hipStream_t)stream;
  const int rows = cache->n_sessions * query->n_q_heads;
  hipLaunchKernelGGL(qprep_kernel, dim3(rows), dim3(128), 0, s, a);
  if ((st = launch_status("query prep"))) return st;
  dim3 grid(sp.n_splits, cache->n_kv_heads, cache->n_sessions);
  switch (G) {
    case 1: hipLaunchKernelGGL(split_kernel<1>, grid, dim3(64 * kDecodeWaves), 0, s, a, a.wsq, cache->pages, a.wsp); break;
    case 2: hipLaunchKernelGGL(split_kernel<2>, grid, dim3(64 * kDecodeWaves), 0, s, a, a.wsq, cache->pages, a.wsp); break;
    case 4: hipLaunchKernelGGL(split_kernel<4>, grid, dim3(64 * kDecodeWaves), 0, s, a, a.wsq, cache->pages, a.wsp); break;
    default: hipLaunchKernelGGL(split_kernel<8>, grid, dim3(64 * kDecodeWaves), 0, s, a, a.wsq, cache->pages, a.wsp); break;
  }
  if ((st = launch_status("split"))) return st;
  hipLaunchKernelGGL(combine_kernel, dim3(rows), dim3(128), 0, s, a);
  return launch_status("combine");
}

}  // extern "C"
