// Encode kernels of libtq for gfx950 (CDNA4, wave64) and tq_encode_kv.
//
// Encode ("TurboQuant-MLX v2.0", How It Works > Pipeline; "TurboMOQ",
// Architecture): every 128-value head vector x is rotated by D H D, its norm is
// stored, and each coordinate of u = D H D x / ||x|| is quantised and packed.
// encode_pages_kernel (four lanes per vector, below) writes fp16 pages and the
// packed keys and values of every page without a QJL residual.
// The keys of QJL pages (codes, norm, and the signs of S r for r = x - xhat,
// "TurboMOQ", QJL residual correction, the sketch on the matrix cores) come
// from qjl_quad_kernel (four lanes per vector).
#include <algorithm>
#include <atomic>

#include "tq_device.h"
#include "tq_token_encoder.h"

namespace tq {
namespace dev {
namespace {

// ------------------------------------------------------------------ encode
struct EncodeArgs {
  const void* k;
  const void* v;
  int dtype;
  int tok0, ntok, page0;
  int64_t sb, sh, st;
  int32_t* err;
  const uint64_t* pages;
  int n_sessions, n_kv_heads, max_pages;
  char* pool;
  uint64_t pool_bytes;
  const uint32_t* sign_mask;
  const float* k_table;
  const float* v_table;
  const float* qjl_s;
  int k_polar, v_polar;   // PolarQuant parts (at most 4 bits wide)
  int pages_per_block;    // encode_pages_kernel: pages per workgroup
};

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
// serves every width.  The outer D (times the lane's sign, below) is applied
// to u before the lookup, so exact ties round up on every coordinate.  Codes
// go to an LDS byte matrix [token][coordinate]; each lane
// then packs 32 consecutive codes of one stream (exactly b dwords) with a
// streaming accumulator whose flush points are uniform.
constexpr int kRowStride = 144;            // LDS byte-matrix row: 128 codes + pad
constexpr int kEncodeBlock = 256;
constexpr int kEncodePagesPerBlock = 4;   // the default launch shape
constexpr int kEncodeMaxPagesPerBlock = 16;

__device__ __forceinline__ float quad_swap(float v, int m) {
  // partner lane = lane ^ m inside the quad; m is a compile-time 1 or 2 after unrolling
  return m == 1 ? __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false))
                : __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// x[s] += sg * x[s] of the partner lane (quad permutation CTRL), for the 32
// values, as v_fmac_f32 with a DPP source; the compiler does not fuse a DPP
// move into a multiply-accumulate, so it is written out.  Each group opens with
// two wait states (s_nop 1), which covers the DPP read-after-VALU-write hazard
// for every register it reads.
template <int CTRL>
__device__ __forceinline__ void quad_butterfly(float (&x)[32], float sg) {
  static_assert(CTRL == 0xB1 || CTRL == 0x4E, "quad permutations [1,0,3,2] and [2,3,0,1]");
#define TQ_FMAC_DPP(PERM)                                                                          \
  asm volatile("s_nop 1\n"                                                                        \
               "v_fmac_f32_dpp %0, %0, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                  \
               "v_fmac_f32_dpp %1, %1, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                  \
               "v_fmac_f32_dpp %2, %2, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                  \
               "v_fmac_f32_dpp %3, %3, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                  \
               "v_fmac_f32_dpp %4, %4, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                  \
               "v_fmac_f32_dpp %5, %5, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                  \
               "v_fmac_f32_dpp %6, %6, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                  \
               "v_fmac_f32_dpp %7, %7, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                  \
               "v_fmac_f32_dpp %8, %8, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                  \
               "v_fmac_f32_dpp %9, %9, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                  \
               "v_fmac_f32_dpp %10, %10, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %11, %11, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %12, %12, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %13, %13, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %14, %14, %16 " PERM " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %15, %15, %16 " PERM " row_mask:0xf bank_mask:0xf"                   \
               : "+v"(x[g + 0]), "+v"(x[g + 1]), "+v"(x[g + 2]), "+v"(x[g + 3]), "+v"(x[g + 4]),        \
                 "+v"(x[g + 5]), "+v"(x[g + 6]), "+v"(x[g + 7]), "+v"(x[g + 8]), "+v"(x[g + 9]),        \
                 "+v"(x[g + 10]), "+v"(x[g + 11]), "+v"(x[g + 12]), "+v"(x[g + 13]), "+v"(x[g + 14]),   \
                 "+v"(x[g + 15])                                                                   \
               : "v"(sg))
#pragma clang loop unroll(full)
  for (int g = 0; g < 32; g += 16) {
    if constexpr (CTRL == 0xB1) {
      TQ_FMAC_DPP("quad_perm:[1,0,3,2]");
    } else {
      TQ_FMAC_DPP("quad_perm:[2,3,0,1]");
    }
  }
#undef TQ_FMAC_DPP
}

// The rest of the 128-point transform of a quad's vector once slot bit 0's
// butterflies are done: in-lane butterflies over slot bits 1..4 (coordinate
// bits 1,2,5,6), then across the quad coordinate bits 3 (lane bit 0) and 4
// (lane bit 1).  Each lane computes mine + sg * partner (one multiply-add with
// the partner read through DPP), so an upper lane keeps the negated butterfly
// output; afterwards lane e holds rho_e times the transform, rho_e = -1 for
// e = 1, 2, which the sign applied before quantising undoes (EncodeLane::fl
// carries it).
__device__ __forceinline__ void quarter_butterflies(float (&x)[32], int e) {
#pragma clang loop unroll(full)
  for (int h = 2; h < 32; h <<= 1)
#pragma clang loop unroll(full)
    for (int s = 0; s < 32; ++s)
      if (!(s & h)) {
        const float a0 = x[s], b0 = x[s + h];
        x[s] = a0 + b0;
        x[s + h] = a0 - b0;
      }
  quad_butterfly<0xB1>(x, (e & 1) ? -1.f : 1.f);
  quad_butterfly<0x4E>(x, (e & 2) ? -1.f : 1.f);
}

struct Lut {
  float S, O;
  int nb;
  float fmax;   // nb - 1 as a float
};

struct EncodeLane {
  uint32_t hmask[16];   // D sign bits of the lane's value pairs, placed for an fp16x2 xor
  uint32_t fl;          // bit s: slot s's transform is negated (outer D times the lane's sign)
  uint32_t dl;          // D bits of the lane's 32 slots
};

// Quad lane e's sign words: the D signs of its coordinates 32c + 8e + k.
__device__ __forceinline__ EncodeLane encode_lane(const uint32_t* sign_mask, int e) {
  EncodeLane el;
  uint32_t m[4];
#pragma clang loop unroll(full)
  for (int w = 0; w < 4; ++w) m[w] = sign_mask[w];
  el.dl = 0;
#pragma clang loop unroll(full)
  for (int c = 0; c < 4; ++c) el.dl |= ((m[c] >> (8 * e)) & 0xffu) << (8 * c);
#pragma clang loop unroll(full)
  for (int i = 0; i < 16; ++i)
    el.hmask[i] = (((el.dl >> (2 * i)) & 1u) << 15) | (((el.dl >> (2 * i + 1)) & 1u) << 31);
  // lanes 1 and 2 of the quad hold the negated transform (quarter_butterflies)
  el.fl = (e == 1 || e == 2) ? ~el.dl : el.dl;
  return el;
}

// Encodes this lane's quarter of one token into code bytes of its LDS matrix
// row; returns the vector norm (the same in the four lanes of the quad).
// This lane's quarter of one token as loaded: chunk c (coordinates
// 32c + 8e .. + 7) is w[c] in fp16, w[2c], w[2c + 1] in float32.
template <int DT>
struct Quarter {
  uint4 w[DT == TQ_DTYPE_F16 ? 4 : 8];
};

template <int DT>
__device__ __forceinline__ void load_quarter(Quarter<DT>& qv, const void* src, size_t row_off, int e) {
  if constexpr (DT == TQ_DTYPE_F16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(src) + row_off);
#pragma clang loop unroll(full)
    for (int c = 0; c < 4; ++c) qv.w[c] = p[4 * c + e];
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(src) + row_off);
#pragma clang loop unroll(full)
    for (int c = 0; c < 4; ++c) {
      qv.w[2 * c] = p[2 * (4 * c + e)];
      qv.w[2 * c + 1] = p[2 * (4 * c + e) + 1];
    }
  }
}

// Leaves in x this lane's share of rho_e H D x (slot 8c + k = coordinate
// 32c + 8e + k) for the loaded quarter; returns ||x|| (the same in the four
// lanes of the quad).
template <int DT>
__device__ __forceinline__ float rotate_loaded(const Quarter<DT>& qv, int e, const EncodeLane& el, float (&x)[32]) {
  float ss = 0.f;
  if constexpr (DT == TQ_DTYPE_F16) {
    // slots 2i, 2i+1 are the two halves of one fp16 pair: the first butterfly
    // (slot bit 0) reads them straight from the pair with mixed-precision
    // multiply-adds (lo + 1.0 * hi, lo - 1.0 * hi), so no conversion is issued;
    // the pair's two squares enter the norm as one fp16 dot product with a
    // float32 accumulator (fp16 products are exact in float32)
#pragma clang loop unroll(full)
    for (int c = 0; c < 4; ++c) {
      const uint4 w = qv.w[c];
      const uint32_t ww[4] = {w.x ^ el.hmask[4 * c], w.y ^ el.hmask[4 * c + 1],
                              w.z ^ el.hmask[4 * c + 2], w.w ^ el.hmask[4 * c + 3]};
#pragma clang loop unroll(full)
      for (int kk = 0; kk < 4; ++kk) {
        typedef _Float16 h2v __attribute__((ext_vector_type(2)));
        const h2v hv = __builtin_bit_cast(h2v, ww[kk]);
        ss = __builtin_amdgcn_fdot2(hv, hv, ss, false);
        float sum, dif;
        asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(sum) : "v"(ww[kk]));
        asm("v_fma_mix_f32 %0, %1, 1.0, -%1 op_sel:[0,0,1] op_sel_hi:[1,0,1]"
            : "=v"(dif) : "v"(ww[kk]));
        x[8 * c + 2 * kk] = sum;
        x[8 * c + 2 * kk + 1] = dif;
      }
    }
  } else {
#pragma clang loop unroll(full)
    for (int c = 0; c < 4; ++c) {
      const uint4 f0 = qv.w[2 * c], f1 = qv.w[2 * c + 1];
      const float v[8] = {__uint_as_float(f0.x), __uint_as_float(f0.y), __uint_as_float(f0.z), __uint_as_float(f0.w),
                          __uint_as_float(f1.x), __uint_as_float(f1.y), __uint_as_float(f1.z), __uint_as_float(f1.w)};
#pragma clang loop unroll(full)
      for (int k = 0; k < 8; ++k) x[8 * c + k] = flip_if(v[k], (el.dl >> (8 * c + k)) & 1u);
    }
#pragma clang loop unroll(full)
    for (int s = 0; s < 32; ++s) ss = fmaf(x[s], x[s], ss);
#pragma clang loop unroll(full)
    for (int s = 0; s < 32; s += 2) {
      const float a0 = x[s], b0 = x[s + 1];
      x[s] = a0 + b0;
      x[s + 1] = a0 - b0;
    }
  }
  ss += quad_swap(ss, 1);
  ss += quad_swap(ss, 2);
  quarter_butterflies(x, e);
  return sqrtf(ss);
}

template <int DT>
__device__ __forceinline__ float rotate_quarter(const void* src, size_t row_off, int e, const EncodeLane& el,
                                                float (&x)[32]) {
  Quarter<DT> qv;
  load_quarter<DT>(qv, src, row_off, e);
  return rotate_loaded<DT>(qv, e, el, x);
}

template <int DT, bool POLAR = false>
__device__ __forceinline__ float encode_quarter(const void* src, size_t row_off, int e,
                                                const EncodeLane& el, int B, const Lut& lut,
                                                const uint2* ent, uint32_t* mat_row, int shift = 0) {
  float x[32];
  const float n = rotate_quarter<DT>(src, row_off, e, el, x);
  const float inv = n > 0.f ? 1.0f / n : 0.f;
  uint32_t cb[8];
#pragma clang loop unroll(full)
  for (int i = 0; i < 8; ++i) cb[i] = 0;
  if constexpr (POLAR) {
    // PolarQuant: slots 2m, 2m+1 are a coordinate pair.  Undo the outer D and
    // the lane's sign to get u, then the radius code from the lookup grid
    // (built on the radius boundaries of B - shift bits) and the angle sector
    // floor((theta + pi) L / (2 pi)) mod L, L = 2^(B + shift), without an
    // arctangent up to 16 sectors: the signs give the quadrant (sectors of
    // L/4 each from -pi), and inside it the angle psi from the quadrant's
    // start has tan psi = a / b with (a, b) = (|u1|, |u0|) in quadrants 0 and
    // 2, (|u0|, |u1|) in 1 and 3, so the sector's offset counts the edges
    // 2 pi j / L with a >= tan(2 pi j / L) b (finer grids take psi from an
    // arctangent).  The pair field F = radius | angle << (B - shift) goes to
    // the two slots, low B bits first.  The codes are final: no flip below.
    const uint32_t lsign = (e == 1 || e == 2) ? 1u : 0u;
    const int L = 1 << (B + shift), RB = B - shift;
#pragma clang loop unroll(full)
    for (int m = 0; m < 16; ++m) {
      const int s0 = 2 * m, s1 = 2 * m + 1;
      const float u0 = flip_if(x[s0], ((el.dl >> s0) & 1u) ^ lsign) * inv;
      const float u1 = flip_if(x[s1], ((el.dl >> s1) & 1u) ^ lsign) * inv;
      const float r = sqrtf(fmaf(u0, u0, u1 * u1));
      // the radius in the grid's coordinate, compared there with the boundary
      const float tr = fmaf(r, lut.S, lut.O);
      uint32_t bin;
      if (lut.nb == kLutByteBins)
        bin = __builtin_amdgcn_cvt_pk_u8_f32(tr, 0, 0u);
      else
        bin = (uint32_t)(int)__builtin_amdgcn_fmed3f(tr, 0.f, lut.fmax);
      const uint2 en = ent[checked((int)bin, lut.nb, kCheckEncodeGrid)];
      const uint32_t rc = en.x + (tr >= __uint_as_float(en.y) ? 1u : 0u);
      uint32_t tc;
      if (L == 2) {
        tc = u1 >= 0.f ? 1u : 0u;
      } else {
        const bool n0 = u0 < 0.f, n1 = u1 < 0.f;
        const uint32_t qd = n1 ? (n0 ? 0u : 1u) : (n0 ? 3u : 2u);
        const float a0 = fabsf(u0), a1 = fabsf(u1);
        const float pa = (qd & 1u) ? a0 : a1, pb = (qd & 1u) ? a1 : a0;
        uint32_t sub = 0;
        if (L == 8) {
          sub = pa >= pb ? 1u : 0u;                                   // tan(pi/4)
        } else if (L == 16) {
          sub = (pa >= 0.41421356237309503f * pb ? 1u : 0u) +        // tan(pi/8)
                (pa >= pb ? 1u : 0u) +                                // tan(pi/4)
                (pa >= 2.41421356237309503f * pb ? 1u : 0u);          // tan(3 pi/8)
        } else if (L > 16) {
          sub = min((uint32_t)(atan2f(pa, pb) * ((float)L / 6.28318530717958648f)), (uint32_t)(L / 4 - 1));
        }
        // a zero pair takes the angle atan2(+0, +0) = 0 (quadrant 2, no edge
        // passed), whatever the signs of its zeros; pa = 0 < pb gives 0 anyway
        if (pa == 0.f) sub = 0;
        tc = qd * (uint32_t)(L >> 2) + sub;
      }
      const uint32_t F = rc | (tc << RB);
      cb[s0 >> 2] |= (F & ((1u << B) - 1u)) << (8 * (s0 & 3));
      cb[s1 >> 2] |= (F >> B) << (8 * (s1 & 3));
    }
#pragma clang loop unroll(full)
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<uint2*>(reinterpret_cast<char*>(mat_row) + 32 * c + 8 * e) =
          make_uint2(cb[2 * c], cb[2 * c + 1]);
    return n;
  }
  // u carries its sign (outer D times the lane's sign) before the lookup, so
  // that an exact tie u = t_k counts t_k on every coordinate (#{t_k <= u}),
  // as for unflipped ones: a code flip after quantising would count it on
  // flipped coordinates only (L - 1 - #{t_k <= -u} = #{t_k < u}).  The value
  // goes to the grid's coordinate g = u S + O as one fma of the signed slot
  // with S / ||x||, and the grid's boundaries are stored in that coordinate;
  // a zero row (every g = O) ties with the boundary 0 exactly.
  const float sinv = lut.S * inv;
  if (lut.nb == kLutByteBins) {
    // 256-bin grid: the bin is g (O carries the -1/2) rounded and saturated
    // to a byte by one conversion
#pragma clang loop unroll(full)
    for (int s = 0; s < 32; ++s) {
      const float g = fmaf(flip_if(x[s], (el.fl >> s) & 1u), sinv, lut.O);
      const uint32_t bin = __builtin_amdgcn_cvt_pk_u8_f32(g, 0, 0u);
      const uint2 en = ent[checked((int)bin, lut.nb, kCheckEncodeGrid)];
      const uint32_t c = en.x + (g >= __uint_as_float(en.y) ? 1u : 0u);
      cb[s >> 2] |= c << (8 * (s & 3));
    }
  } else {
#pragma clang loop unroll(full)
    for (int s = 0; s < 32; ++s) {
      const float g = fmaf(flip_if(x[s], (el.fl >> s) & 1u), sinv, lut.O);
      // bin = clamp(floor(g), 0, nb - 1), clamped in float (one med3)
      const int bin = (int)__builtin_amdgcn_fmed3f(g, 0.f, lut.fmax);
      const uint2 en = ent[checked(bin, lut.nb, kCheckEncodeGrid)];
      const uint32_t c = en.x + (g >= __uint_as_float(en.y) ? 1u : 0u);
      cb[s >> 2] |= c << (8 * (s & 3));
    }
  }
  // chunk c holds coordinates 32c + 8e .. +7: row bytes 32c + 8e
#pragma clang loop unroll(full)
  for (int c = 0; c < 4; ++c)
    *reinterpret_cast<uint2*>(reinterpret_cast<char*>(mat_row) + 32 * c + 8 * e) = make_uint2(cb[2 * c], cb[2 * c + 1]);
  return n;
}

// Writes dwords [e*B, e*B + B) of stream s of a code block from its codes
// 32e..32e+31 (one per byte of c8, each below 2^B), LSB-first: code n at bit
// n B.  Up to 4 bits the width is a template argument, so every shift is a
// constant: each dword of four codes is folded in two shift-or-mask steps
// (pairs, then a 4B-bit quad) and the eight quads are placed at bit 4B k.
template <int B>
__device__ __forceinline__ void store_stream_part_w(char* blk, int s, int e, const uint32_t (&c8)[8]) {
  uint32_t out[B];
#pragma clang loop unroll(full)
  for (int i = 0; i < B; ++i) out[i] = 0;
  static_assert(B >= 1 && B <= 4, "narrow widths");
  {
    constexpr uint32_t m2 = ((1u << (2 * B)) - 1u) * 0x00010001u, m4 = (1u << (4 * B)) - 1u;
#pragma clang loop unroll(full)
    for (int k = 0; k < 8; ++k) {
      const uint32_t w = c8[k];
      const uint32_t pr = (w | (w >> (8 - B))) & m2;             // c0 | c1 << B, c2 | c3 << B
      const uint32_t qd = (pr | (pr >> (16 - 2 * B))) & m4;      // c0 | c1 << B | c2 << 2B | c3 << 3B
      constexpr int kw = 4 * B;
      const int bit = kw * k, d = bit >> 5, sh = bit & 31;
      out[d] |= qd << sh;
      if (sh + kw > 32) out[d + 1] |= qd >> (32 - sh);
    }
  }
  uint32_t* const base = reinterpret_cast<uint32_t*>(blk + s * 16);   // dword d: base[(d >> 2) * 256 + (d & 3)]
#pragma clang loop unroll(full)
  for (int i = 0; i < B; ++i) {
    const int dd = checked(e * B + i, 4 * B, kCheckEncodeStream);   // dwords e B .. e B + B - 1, e < 4
    base[(dd >> 2) * 256 + (dd & 3)] = out[i];
  }
}

__device__ __forceinline__ void store_stream_part(int B, char* blk, int s, int e, const uint32_t (&c8)[8]) {
  switch (B) {
    case 1: store_stream_part_w<1>(blk, s, e, c8); break;
    case 2: store_stream_part_w<2>(blk, s, e, c8); break;
    case 3: store_stream_part_w<3>(blk, s, e, c8); break;
    case 4: store_stream_part_w<4>(blk, s, e, c8); break;
    default: {
      // 5-8 bits (a few important heads): code by code at run-time offsets
      uint32_t* const base = reinterpret_cast<uint32_t*>(blk + s * 16);
      int d = e * B;
      uint64_t acc = 0;
      int nb = 0;
      for (int n = 0; n < 32; ++n) {
        acc |= (uint64_t)((c8[n >> 2] >> (8 * (n & 3))) & 0xffu) << nb;
        nb += B;
        if (nb >= 32) {
          const int dd = checked(d, 4 * B, kCheckEncodeStream);
          base[(dd >> 2) * 256 + (dd & 3)] = (uint32_t)acc;
          ++d;
          acc >>= 32;
          nb -= 32;
        }
      }
    }
  }
}

// POLAR: the instantiation for layers with PolarQuant parts (K and/or V, as
// a.k_polar / a.v_polar say); the plain one has no polar code at all.
template <int DT, bool POLAR>
__global__ __launch_bounds__(kEncodeBlock) void encode_pages_kernel(EncodeArgs a,
                                                                    const uint64_t* __restrict__ pages) {
  __shared__ uint2 entk[kLutMaxBins], entv[kLutMaxBins];
  __shared__ uint32_t matk[PT * kRowStride / 4], matv[PT * kRowStride / 4];
  __shared__ float normk[PT], normv[PT];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = lane & 3, t = wave * 16 + (lane >> 2);
  const int h = blockIdx.y, b = blockIdx.z;
  const int pg0 = a.page0 + blockIdx.x * a.pages_per_block;
  const int pg_last = (a.tok0 + a.ntok - 1) / PT;

  const EncodeLane el = encode_lane(a.sign_mask, e);
  int cur_kb = -1, cur_vb = -1;
  Lut lk{0.f, 0.f, 1, 0.f}, lv{0.f, 0.f, 1, 0.f};
  // PolarQuant parts: the angle shift (radius width = page width - shift)
  const int tk = POLAR && a.k_polar ? polar_shift_of(a.k_table) : 0;
  const int tv = POLAR && a.v_polar ? polar_shift_of(a.v_table) : 0;

  const size_t base = (size_t)b * a.sb + (size_t)h * a.sh;
  const uint64_t* prow = pages + ((size_t)b * a.n_kv_heads + h) * a.max_pages;

  for (int pg = pg0; pg < pg0 + a.pages_per_block && pg <= pg_last; ++pg) {
    const uint64_t desc = prow[pg];
    if (!(desc & TQ_PAGE_PRESENT)) {
      if (tid == 0) raise_flag(a.err, 2);
      continue;
    }
    const PageDesc pd = read_desc(desc);
    const int kb = pd.kb, vb = pd.vb;
    const bool qjl = pd.qjl;
    const uint64_t off = pd.off;
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
      // a polar part quantises the radius at its own width (clamped into the
      // table for widths it refuses below)
      const int rk = POLAR && a.k_polar ? min(8, max(1, kb - tk)) : kb;
      const int rv = POLAR && a.v_polar ? min(8, max(1, vb - tv)) : vb;
      const float* hk = a.k_table + kLutHeaderOffset + 4 * (rk - 1);
      const float* hv = a.v_table + kLutHeaderOffset + 4 * (rv - 1);
      const int nbk = min((int)__float_as_uint(hk[2]), kLutMaxBins);
      const int nbv = min((int)__float_as_uint(hv[2]), kLutMaxBins);
      lk = Lut{hk[0], hk[1], nbk, (float)(nbk - 1)};
      lv = Lut{hv[0], hv[1], nbv, (float)(nbv - 1)};
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
    // QJL key pages are written by the per-token kernel (codes + sketch), as
    // are PolarQuant parts it refuses
    const bool kp = POLAR && a.k_polar, vp = POLAR && a.v_polar;
    const bool k_bad = kp && !polar_width_ok(kb, tk), v_bad = vp && !polar_width_ok(vb, tv);
    const bool skip_k = qjl || k_bad, skip_v = v_bad;
    // a PolarQuant part wider than 4 bits has no pair table, and one whose
    // width cannot carry the angle shift has no split: refused, untouched
    if (tid == 0 && (k_bad || v_bad)) raise_flag(a.err, 4);
    float nk = 0.f, nv = 0.f;
    if (!skip_k)
      nk = kp ? encode_quarter<DT, POLAR>(a.k, row_off, e, el, kb, lk, entk, rowk, tk)
              : encode_quarter<DT>(a.k, row_off, e, el, kb, lk, entk, rowk);
    if (!skip_v)
      nv = vp ? encode_quarter<DT, POLAR>(a.v, row_off, e, el, vb, lv, entv, rowv, tv)
              : encode_quarter<DT>(a.v, row_off, e, el, vb, lv, entv, rowv);
    if (e == 0) {
      normk[t] = nk;
      normv[t] = nv;
    }
    __syncthreads();
    // pack: lane (stream s, part e) writes dwords [e*B, e*B+B) of stream s
    char* vblk = page + 1024 * kb + 256 + (qjl ? 1280 : 0);
    const int s = t;
    if (!skip_k) {
      // K stream s = token s: codes 32e..32e+31 are bytes 32e.. of row s
      const char* r = reinterpret_cast<const char*>(matk + s * (kRowStride / 4)) + 32 * e;
      const uint4 c0 = *reinterpret_cast<const uint4*>(r);
      const uint4 c1 = *reinterpret_cast<const uint4*>(r + 16);
      const uint32_t c8[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      store_stream_part(kb, page, s, e, c8);
    }
    if (!skip_v) {
      // V stream s: positions 2t, 2t + 1 (t = 16e .. 16e + 15) = token t at
      // coordinates v_stream_coord(s, 0) and v_stream_coord(s, 1)
      const uint8_t* mv = reinterpret_cast<const uint8_t*>(matv);
      const int c0 = v_stream_coord(s, 0), c1 = v_stream_coord(s, 1);
      uint32_t c8[8];
#pragma clang loop unroll(full)
      for (int kk = 0; kk < 8; ++kk) {
        const int t0 = 16 * e + 2 * kk;
        const int r0 = checked(t0 * kRowStride, (PT - 1) * kRowStride, kCheckEncodeStream);
        c8[kk] = (uint32_t)mv[r0 + c0] | ((uint32_t)mv[r0 + c1] << 8) |
                 ((uint32_t)mv[r0 + kRowStride + c0] << 16) | ((uint32_t)mv[r0 + kRowStride + c1] << 24);
      }
      store_stream_part(vb, vblk, s, e, c8);
    }
    if (e == 0) {
      if (!skip_k) reinterpret_cast<float*>(page + 1024 * kb)[s] = normk[s];
      if (!skip_v) reinterpret_cast<float*>(vblk + 1024 * vb)[s] = normv[s];
    }
    __syncthreads();
  }
}


// ------------------------------------------------- QJL keys (quad lanes)
// Keys of QJL pages: the four-lanes-per-vector encoder of encode_pages_kernel
// (16 tokens per wave and pass, four passes per page; PolarQuant keys in their
// own instantiation), and the sign sketch in the rotated domain on the matrix
// cores.  The
// residual r = x - xhat = (||x|| / d) D H D (u - c) ("TurboMOQ", QJL residual
// correction), so S r = (||x|| / d) S' (u - c) with S' = S D H D: the signs
// of S r are those of S' v for v = f (u - c), any f > 0, when ||x|| > 0, and
// all + for a zero row (r = 0).  f scales each token's v to norm sqrt(d), and
// each row of S' is scaled to a largest magnitude of 8 (neither changes a
// sign), which keeps both operands well inside float16's range.
//
// The products run as float16 pairs: every float32 operand y is hi + lo with
// hi = fp16(y) and lo = fp16(y - hi) (both rounded to nearest), and
// S' v = S'hi vhi + S'hi vlo + S'lo vhi on v_mfma_f32_16x16x32_f16 (fp16
// products are exact in the float32 accumulator).  The dropped S'lo vlo and
// the rounding of the lo parts leave at most 2^-21 |S'_ij v_j| per term, far
// inside the rounding band of a QJL sign (1e-5 ||S'_i|| ||v||), where float32
// evaluation already decides nothing.
//
// Each pass multiplies the 16 tokens' v by S'^T, [16 x 128] . [128 x 128]:
// 8 column blocks x 4 K steps x 3 products.  MFMA lane l = 16 kq + i holds
// A row i (token) and K elements 8 kq .. 8 kq + 7 of a 32-wide step t; K
// element (t, kq, j) is coordinate 32 t + 8 kq + j, which quad lane kq of
// token i holds in slot 8 t + j, so the A operands are one lane permutation of
// the encoder's registers.  B lane l holds sketch row 16 nb + l % 16 at the
// same 8 K elements; D lane l, register v: token 4 (l / 16) + v.  S' is built
// once per workgroup in LDS (each row rotated by a quad, as a token is), hi
// and lo as 16-byte lane vectors:
//   S'[n][32 t + 8 kq + j] at vector ((n / 16) 4 + t) 64 + 16 kq + n % 16, half j.
// One 8-wave workgroup per CU (S' takes 64 KiB of LDS), persistent over the
// call's pages.
constexpr int kQjlQuadWaves = 8;
typedef float mfma_acc4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// u = the lane's slots, outer D and lane sign applied, times inv; code =
// #{t_k <= u} (binary search over the width's boundaries), into cb's bytes;
// x[s] <- u - c[code]; e2 += the squares of those residuals.
template <int B>
__device__ __forceinline__ void quantize_residual(float (&x)[32], float inv, uint32_t fl, const float* thr,
                                                  const float* cent, uint32_t (&cb)[8], float& e2) {
#pragma clang loop unroll(full)
  for (int s = 0; s < 32; ++s) {
    const float u = flip_if(x[s] * inv, (fl >> s) & 1u);
    const uint32_t c = quantize<B>(u, thr);
    cb[s >> 2] |= c << (8 * (s & 3));
    const float r = u - cent[checked((int)c, 1 << B, kCheckQjlLds)];
    e2 = fmaf(r, r, e2);
    x[s] = r;
  }
}

// PolarQuant (B <= 4): slots 2m, 2m + 1 hold a coordinate pair; its pair field
// F (polar_pair_field) goes to the two code bytes, low B bits first, and x
// keeps u minus the pair's reconstruction pair[F].
template <int B>
__device__ __forceinline__ void quantize_residual_polar(float (&x)[32], float inv, uint32_t fl, const float* thr,
                                                        const float2* pair, int shift, uint32_t (&cb)[8],
                                                        float& e2) {
#pragma clang loop unroll(full)
  for (int m = 0; m < 16; ++m) {
    const int s0 = 2 * m, s1 = 2 * m + 1;
    const float u0 = flip_if(x[s0] * inv, (fl >> s0) & 1u), u1 = flip_if(x[s1] * inv, (fl >> s1) & 1u);
    const uint32_t F = polar_pair_field<B>(u0, u1, thr, shift);
    cb[s0 >> 2] |= (F & ((1u << B) - 1u)) << (8 * (s0 & 3));
    cb[s1 >> 2] |= (F >> B) << (8 * (s1 & 3));
    const float2 p = pair[checked((int)F, 1 << (2 * B), kCheckQjlLds)];
    const float r0 = u0 - p.x, r1 = u1 - p.y;
    e2 = fmaf(r0, r0, e2);
    e2 = fmaf(r1, r1, e2);
    x[s0] = r0;
    x[s1] = r1;
  }
}

// y = hi + lo in float16 (both rounded to nearest); two values per dword,
// the lower slot in the low half.
__device__ __forceinline__ void split_pair(float y0, float y1, uint32_t& hi, uint32_t& lo) {
  const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1;
  const _Float16 l0 = (_Float16)(y0 - (float)h0), l1 = (_Float16)(y1 - (float)h1);
  hi = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  lo = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
}

__device__ __forceinline__ half8 as_half8(uint4 v) { return __builtin_bit_cast(half8, v); }

// POLAR: the instantiation for PolarQuant keys (widths up to 4 bits, the pair
// table in LDS as well).
template <int DT, bool POLAR>
__global__ __launch_bounds__(64 * kQjlQuadWaves) void qjl_quad_kernel(EncodeArgs a, const uint64_t* __restrict__ pages,
                                                                      int n_pages) {
  __shared__ uint4 sph[D * D / 8];
  __shared__ uint4 spl[D * D / 8];
  __shared__ uint32_t rows[kQjlQuadWaves][16 * kRowStride / 4];
  __shared__ float lds_thr[kQjlQuadWaves][256];
  __shared__ float lds_cent[kQjlQuadWaves][256];
  __shared__ float2 lds_pair[kQjlQuadWaves][POLAR ? 256 : 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, e = lane & 3, mq = lane >> 2;
  const EncodeLane el = encode_lane(a.sign_mask, e);
  // S' rows: quad i / 4 rotates row i of S (all four lanes of a quad take the
  // same trip count, as the DPP butterflies need)
  for (int i = tid >> 2; i < D; i += blockDim.x >> 2) {
    const float* srow = a.qjl_s + (size_t)i * D;
    float x[32];
#pragma clang loop unroll(full)
    for (int c = 0; c < 4; ++c)
#pragma clang loop unroll(full)
      for (int k = 0; k < 8; ++k) x[8 * c + k] = flip_if(srow[32 * c + 8 * e + k], (el.dl >> (8 * c + k)) & 1u);
#pragma clang loop unroll(full)
    for (int s = 0; s < 32; s += 2) {
      const float a0 = x[s], b0 = x[s + 1];
      x[s] = a0 + b0;
      x[s + 1] = a0 - b0;
    }
    quarter_butterflies(x, e);
    float mx = 0.f;
#pragma clang loop unroll(full)
    for (int s = 0; s < 32; ++s) mx = fmaxf(mx, fabsf(x[s]));
    mx = fmaxf(mx, quad_swap(mx, 1));
    mx = fmaxf(mx, quad_swap(mx, 2));
    const float g = mx > 0.f ? 8.0f / mx : 0.f;
#pragma clang loop unroll(full)
    for (int c = 0; c < 4; ++c) {
      uint32_t hi[4], lo[4];
#pragma clang loop unroll(full)
      for (int m = 0; m < 4; ++m) {
        const int s0 = 8 * c + 2 * m;
        split_pair(flip_if(x[s0] * g, (el.fl >> s0) & 1u), flip_if(x[s0 + 1] * g, (el.fl >> (s0 + 1)) & 1u), hi[m],
                   lo[m]);
      }
      const int at = checked(((i >> 4) * 4 + c) * 64 + 16 * e + (i & 15), D * D / 8, kCheckQjlLds);
      sph[at] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      spl[at] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  }
  __syncthreads();

  float* thr = lds_thr[wave];
  float* cent = lds_cent[wave];
  float2* pair = lds_pair[wave];
  uint32_t* rw = rows[wave];
  const int shift = POLAR ? polar_shift_of(a.k_table) : 0;
  const int src = 4 * (lane & 15) + (lane >> 4);     // the encoder lane of this lane's A operands
  const int vsel = lane & 3, gsh = 16 * ((lane >> 2) & 3);   // lanes 0-15: token = 4 (gsh / 16) + vsel
  int cur_kb = -1;
  const int total = n_pages * a.n_kv_heads * a.n_sessions;
  for (int item = blockIdx.x * kQjlQuadWaves + wave; item < total; item += gridDim.x * kQjlQuadWaves) {
    const int pgi = item % n_pages, rest = item / n_pages;
    const int h = rest % a.n_kv_heads, b = rest / a.n_kv_heads;
    const int pg = a.page0 + pgi;
    const uint64_t desc = pages[((size_t)b * a.n_kv_heads + h) * a.max_pages + pg];
    if (!(desc & TQ_PAGE_PRESENT)) continue;    // flagged by encode_pages_kernel
    const PageDesc pd = read_desc(desc);
    const int kb = pd.kb, vb = pd.vb;
    const bool bad_fmt = kb == 0 ? (vb != 0 || pd.qjl) : (kb > 8 || vb < 1 || vb > 8);
    if (!pd.qjl || bad_fmt || pd.off + page_size_dev(kb, vb, true) > a.pool_bytes) continue;
    const int t_first = pg * PT;
    if (max(t_first, a.tok0) != t_first || min(t_first + PT, a.tok0 + a.ntok) != t_first + PT) continue;
    if (POLAR && !polar_width_ok(kb, shift)) continue;   // refused (and flagged) by encode_pages_kernel
    if (kb != cur_kb) {
      wave_lds_sync();
      stage_token_tables(a.k_table, kb, POLAR, shift, lane, 64, thr, cent, POLAR ? pair : nullptr);
      wave_lds_sync();
      cur_kb = kb;
    }
    char* page = a.pool + pd.off;
    char* qbase = page + 1024 * kb + 256;
    const size_t base = (size_t)b * a.sb + (size_t)h * a.sh;
    const size_t row0 = base + (size_t)(t_first + mq - a.tok0) * a.st;
    Quarter<DT> qv;
    load_quarter<DT>(qv, a.k, row0, e);
#pragma clang loop unroll(disable)
    for (int q = 0; q < 4; ++q) {
      const int tok = 16 * q + mq;
      float x[32];
      const float n = rotate_loaded<DT>(qv, e, el, x);
      // the next pass's rows load during this pass's quantiser and products
      if (q < 3) load_quarter<DT>(qv, a.k, row0 + (size_t)(16 * (q + 1)) * a.st, e);
      const float inv = n > 0.f ? 1.0f / n : 0.f;
      uint32_t cb[8];
#pragma clang loop unroll(full)
      for (int i = 0; i < 8; ++i) cb[i] = 0;
      float e2 = 0.f;
      if constexpr (POLAR) {
        switch (kb) {
          case 1: quantize_residual_polar<1>(x, inv, el.fl, thr, pair, shift, cb, e2); break;
          case 2: quantize_residual_polar<2>(x, inv, el.fl, thr, pair, shift, cb, e2); break;
          case 3: quantize_residual_polar<3>(x, inv, el.fl, thr, pair, shift, cb, e2); break;
          default: quantize_residual_polar<4>(x, inv, el.fl, thr, pair, shift, cb, e2); break;
        }
      } else {
        switch (kb) {
          case 1: quantize_residual<1>(x, inv, el.fl, thr, cent, cb, e2); break;
          case 2: quantize_residual<2>(x, inv, el.fl, thr, cent, cb, e2); break;
          case 3: quantize_residual<3>(x, inv, el.fl, thr, cent, cb, e2); break;
          case 4: quantize_residual<4>(x, inv, el.fl, thr, cent, cb, e2); break;
          case 5: quantize_residual<5>(x, inv, el.fl, thr, cent, cb, e2); break;
          case 6: quantize_residual<6>(x, inv, el.fl, thr, cent, cb, e2); break;
          case 7: quantize_residual<7>(x, inv, el.fl, thr, cent, cb, e2); break;
          default: quantize_residual<8>(x, inv, el.fl, thr, cent, cb, e2); break;
        }
      }
      e2 += quad_swap(e2, 1);
      e2 += quad_swap(e2, 2);
      // codes: row mq holds token tok's 128 code bytes (coordinate order)
      char* row = reinterpret_cast<char*>(rw + mq * (kRowStride / 4));
#pragma clang loop unroll(full)
      for (int c = 0; c < 4; ++c) *reinterpret_cast<uint2*>(row + 32 * c + 8 * e) = make_uint2(cb[2 * c], cb[2 * c + 1]);
      // A operands: v = f (u - c) as float16 hi + lo; slots 8t .. 8t + 7 of
      // quad lane kq of token i go to lane 16 kq + i as step t's
      const float f = e2 > 0.f ? 11.313708498984761f * __builtin_amdgcn_rsqf(fmaxf(e2, 1e-30f)) : 0.f;
      uint4 ah[4], al[4];
#pragma clang loop unroll(full)
      for (int t = 0; t < 4; ++t) {
        uint32_t hi[4], lo[4];
#pragma clang loop unroll(full)
        for (int m = 0; m < 4; ++m) split_pair(x[8 * t + 2 * m] * f, x[8 * t + 2 * m + 1] * f, hi[m], lo[m]);
        ah[t] = make_uint4(__shfl(hi[0], src), __shfl(hi[1], src), __shfl(hi[2], src), __shfl(hi[3], src));
        al[t] = make_uint4(__shfl(lo[0], src), __shfl(lo[1], src), __shfl(lo[2], src), __shfl(lo[3], src));
      }
      const float ntok = __shfl(n, 4 * (lane & 15));
      wave_lds_sync();
      {
        // K stream tok: quad lane e packs codes 32e .. 32e + 31
        const uint4 c0 = *reinterpret_cast<const uint4*>(row + 32 * e);
        const uint4 c1 = *reinterpret_cast<const uint4*>(row + 32 * e + 16);
        const uint32_t c8[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        store_stream_part(kb, page, tok, e, c8);
      }
      if (e == 0) {
        reinterpret_cast<float*>(page + 1024 * kb)[tok] = n;
        reinterpret_cast<float*>(qbase + 1024)[tok] = n * sqrtf(e2) * 0.08838834764831845f;   // n ||u - c|| / sqrt(d)
      }
      // sketch dword c of the 16 tokens: sketch rows 32c .. 32c + 31 as the
      // column blocks 2c (low half) and 2c + 1
      uint32_t w[4];
#pragma clang loop unroll(full)
      for (int c = 0; c < 4; ++c) {
        mfma_acc4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma clang loop unroll(full)
        for (int t = 0; t < 4; ++t) {
          const int b0 = checked(((2 * c) * 4 + t) * 64 + lane, D * D / 8, kCheckQjlLds);
          const int b1 = checked(((2 * c + 1) * 4 + t) * 64 + lane, D * D / 8, kCheckQjlLds);
          const half8 h0 = as_half8(sph[b0]), l0 = as_half8(spl[b0]);
          const half8 h1 = as_half8(sph[b1]), l1 = as_half8(spl[b1]);
          const half8 xa = as_half8(ah[t]), xl = as_half8(al[t]);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, h0, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, h1, acc1, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, l0, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, l1, acc1, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, h0, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, h1, acc1, 0, 0, 0);
        }
        // ballot bit l of register v: token 4 (l / 16) + v, sketch row 16 nb + l % 16
        uint64_t l0 = 0, l1 = 0;
#pragma clang loop unroll(full)
        for (int v = 0; v < 4; ++v) {
          const uint64_t p0 = __ballot(acc0[v] >= 0.f), p1 = __ballot(acc1[v] >= 0.f);
          if (vsel == v) {
            l0 = p0;
            l1 = p1;
          }
        }
        w[c] = (uint32_t)((l0 >> gsh) & 0xffffu) | ((uint32_t)((l1 >> gsh) & 0xffffu) << 16);
      }
      if (lane < 16)
        reinterpret_cast<uint4*>(qbase)[16 * q + lane] =
            ntok > 0.f ? make_uint4(w[0], w[1], w[2], w[3]) : make_uint4(~0u, ~0u, ~0u, ~0u);
      wave_lds_sync();   // the next pass rewrites the rows
    }
  }
}
}  // namespace
}  // namespace dev
}  // namespace tq

using namespace tq;
using namespace tq::dev;

int tq::check_word_encode(uint32_t* out, bool reset) { return read_check_word(out, reset); }

namespace {

// Compute units of device `dev`, queried once per device and cached in an
// atomic (calls from several host threads may race to store the same value).
int compute_units(int dev) {
  static std::atomic<int> cached[64];
  if (dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n >= 1) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

extern "C" {

int tq_encode_kv(const tq_layer* layer, const tq_cache* cache, const tq_kv_input* in, void* stream) {
  return tq_encode_kv_shaped(layer, cache, in, 0, 0, stream);
}

int tq_encode_kv_shaped(const tq_layer* layer, const tq_cache* cache, const tq_kv_input* in,
                        int pages_per_block, int qjl_workgroups, void* stream) {
  if (pages_per_block < 0 || pages_per_block > kEncodeMaxPagesPerBlock)
    return fail(TQ_ERR_INVALID_ARG, "pages_per_block %d outside 0..%d", pages_per_block, kEncodeMaxPagesPerBlock);
  if (qjl_workgroups < 0) return fail(TQ_ERR_INVALID_ARG, "negative qjl_workgroups");
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
  a.n_sessions = cache->n_sessions;
  a.n_kv_heads = cache->n_kv_heads;
  a.max_pages = cache->max_pages;
  a.pool = reinterpret_cast<char*>(cache->pool);
  a.pool_bytes = cache->pool_bytes;
  a.sign_mask = layer->sign_mask;
  a.k_table = layer->k_table;
  a.v_table = layer->v_table;
  a.qjl_s = layer->qjl_s;
  a.k_polar = layer->k_codebook == TQ_CODEBOOK_POLAR;
  a.v_polar = layer->v_codebook == TQ_CODEBOOK_POLAR;
  a.pages_per_block = pages_per_block > 0 ? pages_per_block : kEncodePagesPerBlock;
  const int last_page = (in->tok0 + in->ntok - 1) / TQ_PAGE_TOKENS;
  const int n_pages = last_page - a.page0 + 1;
  dim3 grid((n_pages + a.pages_per_block - 1) / a.pages_per_block, cache->n_kv_heads,
            cache->n_sessions);
  const bool polar = a.k_polar || a.v_polar;
  if (a.dtype == TQ_DTYPE_F16) {
    if (polar)
      hipLaunchKernelGGL((encode_pages_kernel<TQ_DTYPE_F16, true>), grid, dim3(kEncodeBlock), 0,
                         (hipStream_t)stream, a, cache->pages);
    else
      hipLaunchKernelGGL((encode_pages_kernel<TQ_DTYPE_F16, false>), grid, dim3(kEncodeBlock), 0,
                         (hipStream_t)stream, a, cache->pages);
  } else {
    if (polar)
      hipLaunchKernelGGL((encode_pages_kernel<TQ_DTYPE_F32, true>), grid, dim3(kEncodeBlock), 0,
                         (hipStream_t)stream, a, cache->pages);
    else
      hipLaunchKernelGGL((encode_pages_kernel<TQ_DTYPE_F32, false>), grid, dim3(kEncodeBlock), 0,
                         (hipStream_t)stream, a, cache->pages);
  }
  int st2 = launch_status("encode");
  if (st2) return st2;
  if (layer->qjl_s) {
    // keys of QJL pages: codes, norm and sign sketch, a page per wave on
    // persistent workgroups (as many as the items need, one 8-wave workgroup
    // per CU)
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) cus = compute_units(dev);
    const int64_t items = (int64_t)n_pages * cache->n_kv_heads * cache->n_sessions;
    const int64_t want = (items + kQjlQuadWaves - 1) / kQjlQuadWaves;
    const int64_t cap = qjl_workgroups > 0 ? qjl_workgroups : cus;
    const dim3 grid_q((unsigned)std::max<int64_t>(1, std::min<int64_t>(want, cap))), block_q(64 * kQjlQuadWaves);
    const hipStream_t sq = (hipStream_t)stream;
    if (a.dtype == TQ_DTYPE_F16) {
      if (a.k_polar)
        hipLaunchKernelGGL((qjl_quad_kernel<TQ_DTYPE_F16, true>), grid_q, block_q, 0, sq, a, cache->pages, n_pages);
      else
        hipLaunchKernelGGL((qjl_quad_kernel<TQ_DTYPE_F16, false>), grid_q, block_q, 0, sq, a, cache->pages, n_pages);
    } else {
      if (a.k_polar)
        hipLaunchKernelGGL((qjl_quad_kernel<TQ_DTYPE_F32, true>), grid_q, block_q, 0, sq, a, cache->pages, n_pages);
      else
        hipLaunchKernelGGL((qjl_quad_kernel<TQ_DTYPE_F32, false>), grid_q, block_q, 0, sq, a, cache->pages, n_pages);
    }
    st2 = launch_status("encode QJL keys");
  }
  return st2;
}

}  // extern "C"
