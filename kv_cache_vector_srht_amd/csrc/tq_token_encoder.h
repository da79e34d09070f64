// The per-token encoder of libtq's device code (one lane per head vector):
// rotation, norm, scalar quantisation and packing of one page part, plus the
// QJL sign sketch of keys ("TurboMOQ", QJL residual correction).  Used by the
// QJL key encoder, the decode-loop packing of a full tail page and the
// re-tiering of fp16 pages.
#ifndef TQ_TOKEN_ENCODER_H_
#define TQ_TOKEN_ENCODER_H_

#include "tq_device.h"

namespace tq {
namespace dev {

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

// PolarQuant tables carry their angle shift t in the last entry; a page of
// width bw has a pair table (bw <= 4) and a split (radius bw - t and angle
// bw + t bits in 1..8) only for some shifts.
__device__ __forceinline__ int polar_shift_of(const float* table) { return (int)table[kPolarShiftSlot]; }
__device__ __forceinline__ bool polar_width_ok(int bw, int t) {
  return bw >= 1 && bw <= 4 && bw - t >= 1 && bw + t >= 1 && bw + t <= 8;
}
// Stage, for encode_packed, the quantiser of width B of `table` (PolarQuant:
// the radius boundaries of B - shift bits, padded with +inf to 255 entries so
// that the radius search takes a fixed number of steps, and the pair table of
// width B).  lds_thr holds 256 floats.
__device__ __forceinline__ void stage_token_tables(const float* table, int B, bool polar, int shift, int lane,
                                                   int nthreads, float* lds_thr, float* lds_cent,
                                                   float2* lds_pair) {
  const int W = polar ? B - shift : B, L = 1 << W;
  for (int i = lane; i < L; i += nthreads) {
    lds_cent[i] = table[centroid_offset(W) + i];
    if (i < L - 1) lds_thr[i] = table[boundary_offset(W) + i];
  }
  if (polar) {
    for (int i = L - 1 + lane; i < 255; i += nthreads) lds_thr[i] = __builtin_inff();
    const float2* pt = reinterpret_cast<const float2*>(table + kPairOffset) + pair_offset_host(B);
    for (int i = lane; i < (1 << (2 * B)); i += nthreads) lds_pair[i] = pt[i];
  }
}

// PolarQuant of one vector held by this lane: u as above, then for each
// coordinate pair i the radius r = |(u_2i, u_2i+1)| against the 2^RB - 1
// radius boundaries in `thr` (RB = B - shift bits) and the angle sector
// floor((atan2(u_2i+1, u_2i) + pi) 2^AB / (2 pi)) mod 2^AB (AB = B + shift
// bits); the pair field F = radius | angle << RB goes to emit(2i, F's low B
// bits) and emit(2i+1, its high B bits).  On return x holds u minus the
// pair's reconstruction pair[F].
// The pair field of one coordinate pair u = (u0, u1) at page width B and
// angle shift `shift`: F = radius | angle << (B - shift) as above, the radius
// boundaries in `thr` padded with +inf to 255 entries.
template <int B>
__device__ __forceinline__ uint32_t polar_pair_field(float u0, float u1, const float* thr, int shift) {
  const int RB = B - shift, L = 1 << (B + shift);
  constexpr int kMaxRB = B + 3 < 8 ? B + 3 : 8;   // the radius width at shift -3
  constexpr float kPi = 3.14159265358979323846f;
  const float kSectors = (float)L / (2.0f * 3.14159265358979323846f);
  const float r = sqrtf(fmaf(u0, u0, u1 * u1));
  // a zero pair takes the angle atan2(+0, +0) = 0, whatever its zeros' signs
  const float th = (u0 == 0.f && u1 == 0.f) ? 0.f : atan2f(u1, u0);
  // #{boundaries <= r}: a binary search of kMaxRB steps over the 2^RB - 1 of
  // them and the +inf padding behind them (the same steps at every shift, so
  // that the pair loop unrolls and x stays in registers); the clamp keeps an
  // r of +inf at the top level
  uint32_t rc = 0;
#pragma clang loop unroll(full)
  for (int st = 1 << (kMaxRB - 1); st >= 1; st >>= 1) rc += (r >= thr[rc + st - 1]) ? (uint32_t)st : 0u;
  rc = min(rc, (uint32_t)((1 << RB) - 1));
  const uint32_t tc = (uint32_t)(int)floorf((th + kPi) * kSectors) & (uint32_t)(L - 1);
  return rc | (tc << RB);
}

template <int B, class Emit>
__device__ __forceinline__ float rotate_quantize_polar(float (&x)[D], const uint32_t (&m)[4],
                                                       const float* thr, const float2* pair, Emit emit,
                                                       int shift) {
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
    x[j] = flip_if(a + b, dsign(m, j)) * inv;
    x[j + D / 2] = flip_if(a - b, dsign(m, j + D / 2)) * inv;
  }
#pragma clang loop unroll(full)
  for (int i = 0; i < D / 2; ++i) {
    const float u0 = x[2 * i], u1 = x[2 * i + 1];
    const uint32_t F = polar_pair_field<B>(u0, u1, thr, shift);
    emit(2 * i, F & ((1u << B) - 1u));
    emit(2 * i + 1, F >> B);
    const float2 p = pair[F];
    x[2 * i] = u0 - p.x;
    x[2 * i + 1] = u1 - p.y;
  }
  return n;
}

// One part (PART 0 keys, 1 values) of a page: this lane's vector encoded at
// width B, scalar or (polar, B <= 4) PolarQuant with the pair table in LDS
// and, in lds_thr, the radius boundaries of B - polar_shift bits.
// Returns the vector's norm; for keys x is left holding the rotated-domain
// residual u - c[code] (qjl_sketch's input).
template <int PART, int B>
__device__ __forceinline__ float encode_packed(char* page, int lane, float (&x)[D], const uint32_t (&m)[4],
                                               float* lds_thr, float* lds_cent, uint32_t* lds_rows,
                                               bool polar = false, const float2* lds_pair = nullptr,
                                               int polar_shift = 0) {
  constexpr int kb = B;
  if constexpr (PART == 0) {
    uint32_t sw[4 * B];
#pragma clang loop unroll(full)
    for (int i = 0; i < 4 * B; ++i) sw[i] = 0;
    auto emit = [&](int j, uint32_t c) {
      const int pos = j * B, wi = pos >> 5, sh = pos & 31;
      sw[wi] |= c << sh;
      if (sh + B > 32) sw[wi + 1] |= c >> (32 - sh);
    };
    float n;
    if constexpr (B <= 4) {
      n = polar ? rotate_quantize_polar<B>(x, m, lds_thr, lds_pair, emit, polar_shift)
                : rotate_quantize<B>(x, m, lds_thr, lds_cent, emit);
    } else {
      n = rotate_quantize<B>(x, m, lds_thr, lds_cent, emit);
    }
    uint4* dst = reinterpret_cast<uint4*>(page);
#pragma clang loop unroll(full)
    for (int w = 0; w < B; ++w)
      dst[w * 64 + lane] = make_uint4(sw[4 * w], sw[4 * w + 1], sw[4 * w + 2], sw[4 * w + 3]);
    reinterpret_cast<float*>(page + 1024 * kb)[lane] = n;
    return n;
  } else {
    // Codes as bytes into this lane's LDS row, then transpose into V streams.
    uint32_t cb[D / 4];
#pragma clang loop unroll(full)
    for (int i = 0; i < D / 4; ++i) cb[i] = 0;
    auto emit = [&](int j, uint32_t c) { cb[j >> 2] |= c << (8 * (j & 3)); };
    float n;
    if constexpr (B <= 4) {
      n = polar ? rotate_quantize_polar<B>(x, m, lds_thr, lds_pair, emit, polar_shift)
                : rotate_quantize<B>(x, m, lds_thr, lds_cent, emit);
    } else {
      n = rotate_quantize<B>(x, m, lds_thr, lds_cent, emit);
    }
    uint4* row = reinterpret_cast<uint4*>(reinterpret_cast<char*>(lds_rows) + lane * kEncodeRowBytes);
#pragma clang loop unroll(full)
    for (int i = 0; i < D / 16; ++i) row[i] = make_uint4(cb[4 * i], cb[4 * i + 1], cb[4 * i + 2], cb[4 * i + 3]);
    __syncthreads();
    // stream `lane`: positions 2t, 2t + 1 = token t at its two coordinates
    const uint8_t* rows = reinterpret_cast<const uint8_t*>(lds_rows);
    const int c0 = v_stream_coord(lane, 0), c1 = v_stream_coord(lane, 1);
    uint32_t sw[4 * B];
#pragma clang loop unroll(full)
    for (int i = 0; i < 4 * B; ++i) sw[i] = 0;
#pragma clang loop unroll(full)
    for (int t = 0; t < PT; ++t) {
#pragma clang loop unroll(full)
      for (int k = 0; k < 2; ++k) {
        const uint32_t c = rows[t * kEncodeRowBytes + (k ? c1 : c0)];
        const int pos = (2 * t + k) * B, wi = pos >> 5, sh = pos & 31;
        sw[wi] |= c << sh;
        if (sh + B > 32) sw[wi + 1] |= c >> (32 - sh);
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(page);
#pragma clang loop unroll(full)
    for (int w = 0; w < B; ++w)
      dst[w * 64 + lane] = make_uint4(sw[4 * w], sw[4 * w + 1], sw[4 * w + 2], sw[4 * w + 3]);
    reinterpret_cast<float*>(page + 1024 * B)[lane] = n;
    return n;
  }
}

// The residual of a QJL key ("TurboMOQ", QJL residual correction) from the
// rotated-domain residual u - c that encode_packed leaves in x: on return x
// holds r = x - xhat = (n / d) D H D (u - c) (one more butterfly in
// registers); returns gamma = ||r||.
__device__ __forceinline__ float qjl_residual(float (&x)[D], const uint32_t (&m)[4], float n) {
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
  return n * sqrtf(e2) * 0.08838834764831845f;  // n ||u - c|| / sqrt(d)
}

// The QJL sign sketch of one key, lane = token: z = sign(S r) (bit i of the
// lane's 128-bit word) and gamma, stored at qbase (64 x 16 B signs) and
// qbase + 1024 (64 x float32).  One copy serves every width; the bulk encode
// computes the same sketch a page at a time on the matrix cores.
__device__ __forceinline__ void qjl_sketch(const float* __restrict__ qjl_s, char* qbase, int lane,
                                           float (&x)[D], const uint32_t (&m)[4], float n) {
  const float gamma = qjl_residual(x, m, n);
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
  reinterpret_cast<uint4*>(qbase)[lane] = make_uint4(zw[0], zw[1], zw[2], zw[3]);
  reinterpret_cast<float*>(qbase + 1024)[lane] = gamma;
}

}  // namespace dev
}  // namespace tq

#endif  // TQ_TOKEN_ENCODER_H_
